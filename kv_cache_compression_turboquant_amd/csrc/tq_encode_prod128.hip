// TurboQuant_prod encode at d = 128, rows layout ([TQ] TurboQuant_prod section: a (b-1)-bit
// TurboQuant_mse stage, then the 1-bit QJL sign sketch of the residual and the residual norm).
//
// One wave takes tiles of 32 vectors on the 32 x 32 x 16 bf16 matrix cores:
//   y^T = R x^T    A = rotation fragments (LDS), B = x straight from HBM (exact in bf16), two
//                  passes (R hi, R lo); fp32 x adds a pass with x's low part;
//   z^T = S' r^T   A = fragments of S' = S R^T (LDS), B = the rotated-domain residual
//                  r = y / ||x|| - C[idx] in bf16 hi + lo, three passes (S'hi rhi, S'hi rlo,
//                  S'lo rhi), so z carries fp32-level accuracy into its sign.
// Lane (i, j) (i = lane % 32, j = lane / 32) holds vector i of the tile and, in both products, its
// 64 consecutive coordinates 64 j .. 64 j + 63: the B operand of instruction s is coordinates
// 64 j + 8 s .. + 7 and output block ob, register r is coordinate 64 j + 16 ob + r (the host lays
// the A rows out so).  So the residual the quantizer leaves in a lane's registers is exactly that
// lane's B operand for the second product, and each lane writes whole words of the packed row:
// 2 * BITS index words and 2 sign words.
// Order of work per tile: the rotation's output blocks run ob = 3 .. 0; block ob + 1 is quantized
// while block ob's MFMAs run.  The S' product starts with the instructions that read blocks 3 .. 1
// before block 0 is quantized.  Loads of the tile after next are issued once x is dead.
#include <hip/hip_ext.h>

#include "tq_device.h"

namespace tq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProdWaves = 8;
constexpr int kFrag32U4 = 2048;   // u32x4 per pass: 4 output blocks x 8 instructions x 64 lanes

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// w = 2 w + (this lane's bit of `lanes`): one v_addc with the lane mask as carry-in.
__device__ __forceinline__ uint32_t shift_in(uint32_t w, uint64_t lanes) {
  uint32_t r;
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(lanes));
  return r;
}

// A lane's 64 input coordinates of one vector.
template <bool BF16IN>
struct XRaw;
template <>
struct XRaw<true> {
  u32x4 v[8];
};
template <>
struct XRaw<false> {
  f32x4 v[16];
};

template <bool BF16IN>
__device__ __forceinline__ void load_x(const void* x, int64_t n, int64_t tile, int lane, XRaw<BF16IN>& r) {
  const int64_t row0 = tile * 32 + (lane & 31);
  const int64_t row = row0 < n ? row0 : n - 1;    // past the end: the last row (never stored)
  const int half = lane >> 5;
  if constexpr (BF16IN) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + row * 128 + 64 * half);
#pragma unroll
    for (int s = 0; s < 8; ++s) r.v[s] = src[s];
  } else {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + row * 128 + 64 * half);
#pragma unroll
    for (int s = 0; s < 16; ++s) r.v[s] = src[s];
  }
}

// Compile-time loop C, C - 1, .., 0 (bit offsets must be constants).
template <int C>
struct Ci {
  static constexpr int value = C;
};
template <int C, typename F>
__device__ __forceinline__ void down_from(F&& f) {
  if constexpr (C >= 0) {
    f(Ci<C>{});
    down_from<C - 1>(f);
  }
}

// Per-vector quantizer state: thresholds t_p * ||x|| / post_scale against the raw product, the
// non-negative centroids, and the raw-product -> unit-coordinate scale.
template <int BITS>
struct QState {
  static constexpr int H = 1 << (BITS - 1);
  float thr[H > 1 ? H - 1 : 1];
  float mag[H];
  float scale;
};

// Quantize one coordinate (lane-local index LI, raw product v): push its BITS index bits (top
// first) into the lane's words and return the unit-scale residual v * scale - C[idx].
// idx = (m ^ sgn) + H with m = #{p : |v| >= thr_p}: top bit [v >= 0], low bits those of m XNOR
// [v >= 0].  m's bits come from a binary search over the sorted thresholds.
template <int BITS, int LI>
__device__ __forceinline__ float quant_coord(float v, const QState<BITS>& q, uint32_t (&w)[2 * BITS]) {
  constexpr int P = BITS * LI;
  const bool nonneg = v >= 0.f;
  const uint64_t pos = __builtin_amdgcn_ballot_w64(nonneg);
  w[(P + BITS - 1) >> 5] = shift_in(w[(P + BITS - 1) >> 5], pos);
  const float a = fabsf(v);
  float mag;
  if constexpr (BITS == 1) {
    mag = q.mag[0];
  } else if constexpr (BITS == 2) {
    const bool ge = a >= q.thr[0];
    w[P >> 5] = shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(ge) ^ pos));
    mag = ge ? q.mag[1] : q.mag[0];
  } else {
    const bool hi = a >= q.thr[1];
    w[(P + 1) >> 5] = shift_in(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(hi) ^ pos));
    const bool lo = a >= (hi ? q.thr[2] : q.thr[0]);
    w[P >> 5] = shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(lo) ^ pos));
    mag = hi ? (lo ? q.mag[3] : q.mag[2]) : (lo ? q.mag[1] : q.mag[0]);
  }
  return fmaf(v, q.scale, nonneg ? -mag : mag);
}

// Quantize output block OB (coordinates 16 OB + 15 .. 16 OB, descending) and leave its residual
// as bf16 hi / lo pairs in rh / rl (instruction s = 2 OB + (r >> 3), dword (r & 7) / 2).
template <int BITS, int OB>
__device__ __forceinline__ void quant_block(const f32x16& y, const QState<BITS>& q, uint32_t (&w)[2 * BITS],
                                            u32x4 (&rh)[8], u32x4 (&rl)[8], float& rs) {
  float res[16];
  down_from<15>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    res[r] = quant_coord<BITS, 16 * OB + r>(y[r], q, w);
  });
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    rs = fmaf(res[r], res[r], rs);
    rs = fmaf(res[r + 1], res[r + 1], rs);
    const f32x2 pr = {res[r], res[r + 1]};
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
    const f32x2 rem = {res[r] - __uint_as_float(h << 16), res[r + 1] - __uint_as_float(h & 0xffff0000u)};
    const int s = 2 * OB + (r >> 3);
    rh[s][(r & 7) >> 1] = h;
    rl[s][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
  }
}

// Sign bits of S' output block OB (sign index 16 OB + r of the lane's 64): pushed in descending
// order into the lane's two sign words.
template <int OB>
__device__ __forceinline__ void push_signs(const f32x16& z, uint32_t (&qw)[2]) {
#pragma unroll
  for (int r = 15; r >= 0; --r) qw[OB >> 1] = shift_in(qw[OB >> 1], __builtin_amdgcn_ballot_w64(z[r] >= 0.f));
}

template <int BITS, bool BF16IN, int RP>
__global__ __launch_bounds__(kProdWaves * 64, 1) void k_encode_prod_d128(
    const void* __restrict__ x, int64_t n, const u32x4* __restrict__ frag_r, const u32x4* __restrict__ frag_s,
    float post_scale, CodebookArgs cb, uint32_t* __restrict__ idx_out, float* __restrict__ norms_out,
    uint32_t* __restrict__ qjl_out, float* __restrict__ rnorm_out) {
  constexpr int H = 1 << (BITS - 1);
  constexpr int kThreads = kProdWaves * 64;
  constexpr int kTotal = (RP + 2) * kFrag32U4;
  constexpr int kStage = kTotal / kThreads;
  static_assert(kTotal % kThreads == 0, "staging split");
  // rotation passes 0 .. RP-1, then S' hi, S' lo; each [ob][s][lane]
  __shared__ u32x4 lds[kTotal];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int64_t ntiles = (n + 31) >> 5;
  const int64_t stride = (int64_t)gridDim.x * kProdWaves;
  int64_t tw = (int64_t)blockIdx.x * kProdWaves + wave;

  // Fragment loads first, then the first tile's, so the tile stays in flight across the staging.
  // Blocks start at different slices: every block reads the same fragments.
  {
    u32x4 stage[kStage];
    const int rot0 = (int)(blockIdx.x % kStage);
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int i = threadIdx.x + ((k + rot0) % kStage) * kThreads;
      stage[k] = i < RP * kFrag32U4 ? frag_r[i] : frag_s[i - RP * kFrag32U4];
    }
#pragma unroll
    for (int k = 0; k < kStage; ++k) lds[threadIdx.x + ((k + rot0) % kStage) * kThreads] = stage[k];
  }
  // bf16 input: two register sets in turn, so a tile's loads go out a whole tile before it is
  // needed (fp32 input has one set: its raw tile is twice the size).
  constexpr int NB = BF16IN ? 2 : 1;
  XRaw<BF16IN> xa, xb;
  load_x<BF16IN>(x, n, tw, lane, xa);
  if constexpr (NB == 2) load_x<BF16IN>(x, n, tw + stride, lane, xb);
  __syncthreads();

  const float inv_post = 1.0f / post_scale;
  const u32x4* lds_s = lds + RP * kFrag32U4;
  auto step = [&](XRaw<BF16IN>& xr, const int64_t tw) {
    // ---- B operands of the rotation and the norm
    u32x4 bx[8], bxl[BF16IN ? 1 : 8];
    float ss = 0.f;
    if constexpr (BF16IN) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bx[s] = xr.v[s];
        uint32_t wv[4];
        __builtin_memcpy(wv, &xr.v[s], sizeof(wv));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x2 p = __builtin_bit_cast(bf16x2, wv[k]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f32x4 a = xr.v[2 * s], b = xr.v[2 * s + 1];
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x2 pr = {v[2 * k], v[2 * k + 1]};
          const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
          const f32x2 rem = {v[2 * k] - __uint_as_float(h << 16), v[2 * k + 1] - __uint_as_float(h & 0xffff0000u)};
          bx[s][k] = h;
          bxl[s][k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
          ss = fmaf(v[2 * k], v[2 * k], ss);
          ss = fmaf(v[2 * k + 1], v[2 * k + 1], ss);
        }
      }
    }
    ss += __shfl_xor(ss, 32);
    const float nrm = sqrtf(ss);
    const bool live = nrm > 0.f;
    QState<BITS> qs;
    {
      const float tsc = nrm * inv_post;
#pragma unroll
      for (int p = 0; p < H - 1; ++p) qs.thr[p] = live ? __int_as_float(cb.tpos[p]) * tsc : INFINITY;
#pragma unroll
      for (int p = 0; p < H; ++p) qs.mag[p] = live ? cb.cpos[p] : 0.f;
      qs.scale = live ? post_scale / nrm : 0.f;
    }

    // ---- y^T = R x^T, block by block (ob = 3 .. 0), the previous block quantized meanwhile
    uint32_t w[2 * BITS];
#pragma unroll
    for (int k = 0; k < 2 * BITS; ++k) w[k] = 0;
    u32x4 rh[8], rl[8];
    float rs = 0.f;
    f32x16 prev = zero16();
    down_from<3>([&](auto obc) {
      constexpr int ob = decltype(obc)::value;
      f32x16 acc = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 a0 = lds[(ob * 8 + s) * 64 + lane];
        acc = mfma32(a0, bx[s], acc);
        if constexpr (!BF16IN) acc = mfma32(a0, bxl[s], acc);
        if constexpr (RP == 2) acc = mfma32(lds[kFrag32U4 + (ob * 8 + s) * 64 + lane], bx[s], acc);
      }
      if constexpr (ob < 3) quant_block<BITS, ob + 1>(prev, qs, w, rh, rl, rs);
      prev = acc;
      __builtin_amdgcn_sched_barrier(0);
    });

    // x is dead: the next tile's loads go out now and arrive during the second product
    const int64_t tn = tw + NB * stride;
    if (tn < ntiles) load_x<BF16IN>(x, n, tn, lane, xr);

    // ---- z^T = S' r^T.  Block 3's instructions that read residual blocks 3 .. 1 (s = 7 .. 2)
    // first, then block 0 is quantized, then the rest.
    uint32_t qw[2] = {0u, 0u};
    f32x16 zprev = zero16();
    {
      f32x16 z = zero16();
#pragma unroll
      for (int s = 7; s >= 2; --s) {
        const u32x4 sh = lds_s[(3 * 8 + s) * 64 + lane];
        const u32x4 sl = lds_s[kFrag32U4 + (3 * 8 + s) * 64 + lane];
        z = mfma32(sh, rh[s], z);
        z = mfma32(sh, rl[s], z);
        z = mfma32(sl, rh[s], z);
      }
      quant_block<BITS, 0>(prev, qs, w, rh, rl, rs);
#pragma unroll
      for (int s = 1; s >= 0; --s) {
        const u32x4 sh = lds_s[(3 * 8 + s) * 64 + lane];
        const u32x4 sl = lds_s[kFrag32U4 + (3 * 8 + s) * 64 + lane];
        z = mfma32(sh, rh[s], z);
        z = mfma32(sh, rl[s], z);
        z = mfma32(sl, rh[s], z);
      }
      zprev = z;
      __builtin_amdgcn_sched_barrier(0);
    }
    down_from<2>([&](auto obc) {
      constexpr int ob = decltype(obc)::value;
      f32x16 z = zero16();
#pragma unroll
      for (int s = 7; s >= 0; --s) {
        const u32x4 sh = lds_s[(ob * 8 + s) * 64 + lane];
        const u32x4 sl = lds_s[kFrag32U4 + (ob * 8 + s) * 64 + lane];
        z = mfma32(sh, rh[s], z);
        z = mfma32(sh, rl[s], z);
        z = mfma32(sl, rh[s], z);
      }
      push_signs<ob + 1>(zprev, qw);
      zprev = z;
      __builtin_amdgcn_sched_barrier(0);
    });
    push_signs<0>(zprev, qw);

    // ---- stores
    rs += __shfl_xor(rs, 32);
    const int64_t row = tw * 32 + (lane & 31);
    if (row < n) {
      uint32_t* dst = idx_out + row * (4 * BITS) + 2 * BITS * half;
#pragma unroll
      for (int k = 0; k < 2 * BITS; ++k) dst[k] = w[k];
      *reinterpret_cast<u32x2*>(qjl_out + row * 4 + 2 * half) = u32x2{qw[0], qw[1]};
      if (half == 0) {
        norms_out[row] = nrm;
        rnorm_out[row] = nrm * sqrtf(rs);
      }
    }
  };
  // Entered unconditionally: a wave without a tile of its own (last block only) makes one pass
  // over clamped rows and stores nothing.
  for (;;) {
    step(xa, tw);
    if constexpr (NB == 2) {
      if (tw + stride >= ntiles) break;
      step(xb, tw + stride);
    }
    tw += NB * stride;
    if (tw >= ntiles) break;
  }
}

template <int BITS, bool BF16IN, int RP>
hipError_t prod_launch(const void* x, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl, const CodebookArgs& cb,
                       uint32_t* idx, float* norms, uint32_t* qbits, float* rnorms, hipStream_t st) {
  const int64_t ntiles = (n + 31) / 32;
  int64_t blocks = (ntiles + kProdWaves - 1) / kProdWaves;
  const int64_t cap = (int64_t)num_cus();
  if (blocks > cap) blocks = cap;
  const u32x4* fr = reinterpret_cast<const u32x4*>(rot->frag32_dev);
  const u32x4* fs = reinterpret_cast<const u32x4*>(qjl->frag32_dev);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (take_armed_timer(&ev0, &ev1)) {
    hipExtLaunchKernelGGL((k_encode_prod_d128<BITS, BF16IN, RP>), dim3((unsigned)blocks), dim3(kProdWaves * 64), 0,
                          st, ev0, ev1, 0, x, n, fr, fs, rot->post_scale, cb, idx, norms, qbits, rnorms);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_encode_prod_d128<BITS, BF16IN, RP>), dim3((unsigned)blocks), dim3(kProdWaves * 64), 0, st, x,
                     n, fr, fs, rot->post_scale, cb, idx, norms, qbits, rnorms);
  return hipGetLastError();
}

template <int BITS>
hipError_t prod_dispatch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                         const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits, float* rnorms,
                         hipStream_t st) {
  if (bf16)
    return rot->passes == 1 ? prod_launch<BITS, true, 1>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                            : prod_launch<BITS, true, 2>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
  return rot->passes == 1 ? prod_launch<BITS, false, 1>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                          : prod_launch<BITS, false, 2>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
}

}  // namespace

hipError_t launch_encode_prod_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                   const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                   uint32_t* qjl_bits, float* rnorms, hipStream_t st) {
  if (!rot->frag32_dev || !qjl->frag32_dev) return hipErrorInvalidValue;
  switch (cb.bits) {
    case 1: return prod_dispatch<1>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, st);
    case 2: return prod_dispatch<2>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, st);
    case 3: return prod_dispatch<3>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
