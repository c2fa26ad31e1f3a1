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
// while block 0 is quantized.  Loads of the tile after next are issued once x is dead.  Every
// MFMA's A fragment is read from LDS a few instructions ahead.
#include <hip/hip_ext.h>

#include "tq_device.h"

namespace tq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProdWaves = 8;
// Tuning switch (build-time define): TQ_PROD_PRIO = 1 (default) raises a wave's issue priority while it runs
// the S' product (MFMA-heavy), so the other wave's quantizer (VALU-heavy) issues in its shadow.
#ifndef TQ_PROD_PRIO
#define TQ_PROD_PRIO 1
#endif

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

// w = (w << 1) | (sign bit of z): one v_alignbit.
__device__ __forceinline__ uint32_t sign_in(uint32_t w, float z) {
  return (w << 1) | (__float_as_uint(z) >> 31);
}

// Sum of v over lanes l and l ^ 32 (a register swap of the wave's halves, no LDS).
__device__ __forceinline__ float add_halves(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Raw buffer resource over `bytes` bytes at p (loads past the end read zeros, stores past the end
// are dropped, by the range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
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

// Loads of tile `tile` through a buffer resource bounded by the tile's rows that exist: rows past
// the end read zeros (never stored).  A buffer load may alias the kernel's buffer stores for all
// the compiler knows, so it is not sunk past them to its use in the next tile (an ordinary load
// from a restrict pointer would be, exposing the memory latency there).
template <bool BF16IN>
__device__ __forceinline__ void load_x(const void* x, int64_t n, int64_t tile, int lane, XRaw<BF16IN>& r) {
  constexpr uint32_t kRow = BF16IN ? 256u : 512u;
  const int64_t row0 = tile * 32;
  const int64_t left = n - row0;
  const uint32_t rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
  const __amdgpu_buffer_rsrc_t rx =
      store_rsrc(static_cast<const char*>(x) + (row0 < n ? row0 : 0) * kRow, rows * kRow);
  const uint32_t off = (uint32_t)(lane & 31) * kRow + (uint32_t)(lane >> 5) * (kRow / 2);
  if constexpr (BF16IN) {
#pragma unroll
    for (int s = 0; s < 8; ++s) r.v[s] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u * s, 0, 0);
  } else {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      r.v[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u * s, 0, 0));
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
// Named members rather than arrays: a select tree over an array's elements is otherwise turned
// into a per-lane indexed load from LDS (with bank conflicts), slower than three selects.
template <int BITS>
struct QState {
  float t0, t1, t2;          // positive thresholds (BITS = 2: t0; BITS = 3: t0 < t1 < t2)
  float m0, m1, m2, m3;      // non-negative centroids (BITS = 1: m0; 2: m0, m1; 3: m0 .. m3)
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
    mag = q.m0;
  } else if constexpr (BITS == 2) {
    const bool ge = a >= q.t0;
    w[P >> 5] = shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(ge) ^ pos));
    mag = ge ? q.m1 : q.m0;
  } else {
    const bool hi = a >= q.t1;
    w[(P + 1) >> 5] = shift_in(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(hi) ^ pos));
    const bool lo = a >= (hi ? q.t2 : q.t0);
    w[P >> 5] = shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(lo) ^ pos));
    const float m_lo = lo ? q.m1 : q.m0;
    const float m_hi = lo ? q.m3 : q.m2;
    mag = hi ? m_hi : m_lo;
  }
  return fmaf(v, q.scale, nonneg ? -mag : mag);
}

// Quantize the pair of coordinates (R, R + 1) of output block OB (R even; R + 1 first, so a
// lane's coordinates go in descending order), accumulate their squared residuals into rs and
// leave the residuals as one bf16 hi / lo dword each in rh / rl (instruction s = 2 OB + (R >> 3),
// dword (R & 7) / 2 of the second product's B operand).
template <int BITS, int OB, int R>
__device__ __forceinline__ void quant_pair(const f32x16& y, const QState<BITS>& q, uint32_t (&w)[2 * BITS],
                                           u32x4 (&rh)[8], u32x4 (&rl)[8], float& rs) {
  const float r1 = quant_coord<BITS, 16 * OB + R + 1>(y[R + 1], q, w);
  const float r0 = quant_coord<BITS, 16 * OB + R>(y[R], q, w);
  rs = fmaf(r0, r0, rs);
  rs = fmaf(r1, r1, rs);
  const f32x2 pr = {r0, r1};
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
  const f32x2 rem = {r0 - __uint_as_float(h << 16), r1 - __uint_as_float(h & 0xffff0000u)};
  constexpr int s = 2 * OB + (R >> 3);
  rh[s][(R & 7) >> 1] = h;
  rl[s][(R & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
}

// Sign bits of registers R and R - 1 of S' output block OB (sign index 16 OB + r of the lane's 64),
// pushed in descending order into the lane's two sign words: w = (w << 1) | (z >> 31), one
// v_alignbit each.  The words collect [z < 0] and are inverted once at the end, so a bit is
// [z >= 0] for every z but -0 (which the product does not produce: its accumulator starts at +0).
template <int OB, int R>
__device__ __forceinline__ void push_sign_pair(const f32x16& z, uint32_t (&qw)[2]) {
  qw[OB >> 1] = sign_in(qw[OB >> 1], z[R]);
  qw[OB >> 1] = sign_in(qw[OB >> 1], z[R - 1]);
  // pin the pushes here: shifts are free to sink to the stores, which would keep all 64 z live
  asm volatile("" : "+v"(qw[OB >> 1]));
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Ci<B>{});
    static_for<B + 1, E>(f);
  }
}

// The matrix products of one tile as one flat sequence of 64 steps, each step's A fragments read
// from LDS kRing steps ahead into a ring of registers (an LDS read waited on right before its MFMA
// would expose the LDS latency at every instruction).  Steps 0 .. 31: the rotation, output block
// ob = 3 - k / 8, instruction s = k % 8 (RP fragments).  Steps 32 .. 63: S', output block
// ob = 3 - (k - 32) / 8, instruction s = 7 - (k - 32) % 8 (S' hi and lo).  The sequence repeats
// from tile to tile, so the ring runs on across tiles.
constexpr int kRing = 4;   // divides the 64 steps, so step k of every tile uses slot k % kRing

template <int RP, int K>
__device__ __forceinline__ void load_step(const u32x4* lds, int lane, u32x4 (&slot)[2]) {
  if constexpr (K < 32) {
    constexpr int ob = 3 - (K >> 3), s = K & 7;
    slot[0] = lds[(ob * 8 + s) * 64 + lane];
    if constexpr (RP == 2) slot[1] = lds[kFrag32U4 + (ob * 8 + s) * 64 + lane];
  } else {
    constexpr int ob = 3 - ((K - 32) >> 3), s = 7 - ((K - 32) & 7);
    slot[0] = lds[RP * kFrag32U4 + (ob * 8 + s) * 64 + lane];
    slot[1] = lds[(RP + 1) * kFrag32U4 + (ob * 8 + s) * 64 + lane];
  }
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: tile bases in SGPRs
  const int half = lane >> 5;
  const int64_t ntiles = (n + 31) >> 5;
  const int64_t stride = (int64_t)gridDim.x * kProdWaves;
  int64_t tw = (int64_t)blockIdx.x * kProdWaves + wave;

  // Fragment loads first, then the first tiles', so the tiles stay in flight across the staging.
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
  // The tile loads are unconditional (rows past the end read the last row, never stored): a
  // conditional load would leave the number of loads in flight unknown to the compiler, which then
  // waits for all of them.
  XRaw<BF16IN> xr;
  load_x<BF16IN>(x, n, tw, lane, xr);
  __syncthreads();

  u32x4 ring[kRing][2];
  static_for<0, kRing>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    load_step<RP, k>(lds, lane, ring[k]);
  });

  const float inv_post = 1.0f / post_scale;
  // State a tile's rotation phase hands to its S' phase.
  QState<BITS> qs;
  uint32_t w[2 * BITS];
  u32x4 rh[8], rl[8];
  float rs, nrm;
  f32x16 prev;

  // ---- rotation phase of tile tw: steps 0 .. 31, then the loads of tile tw + stride
  auto rphase = [&](const int64_t tw) {
    // ---- B operands of the rotation
    u32x4 bx[8], bxl[BF16IN ? 1 : 8];
    float ss = 0.f;
    if constexpr (BF16IN) {
#pragma unroll
      for (int s = 0; s < 8; ++s) bx[s] = xr.v[s];
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
#pragma unroll
    for (int k = 0; k < 2 * BITS; ++k) w[k] = 0;
    rs = 0.f;
    f32x16 acc = zero16();
    prev = zero16();

    // ---- steps 0 .. 31: y^T = R x^T; block ob + 1 is quantized (two coordinates per step)
    // during block ob's instructions; the norm is formed during block 3's.
    static_for<0, 32>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ob = 3 - (k >> 3), s = k & 7;
      if constexpr (s == 0) acc = zero16();
      acc = mfma32(ring[k % kRing][0], bx[s], acc);
      if constexpr (!BF16IN) acc = mfma32(ring[k % kRing][0], bxl[s], acc);
      if constexpr (RP == 2) acc = mfma32(ring[k % kRing][1], bx[s], acc);
      load_step<RP, (k + kRing) % 64>(lds, lane, ring[k % kRing]);
      if constexpr (ob == 3) {
        if constexpr (BF16IN) {
          uint32_t wv[4];
          __builtin_memcpy(wv, &bx[s], sizeof(wv));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 p2 = __builtin_bit_cast(bf16x2, wv[e]);
            ss = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss, false);
          }
        }
        if constexpr (s == 7) {
          ss = add_halves(ss);
          nrm = sqrtf(ss);
          const bool live = nrm > 0.f;
          const float tsc = nrm * inv_post;
          auto thr = [&](int p) { return p < H - 1 ? (live ? __int_as_float(cb.tpos[p]) * tsc : INFINITY) : INFINITY; };
          auto mag = [&](int p) { return p < H ? (live ? cb.cpos[p] : 0.f) : 0.f; };
          qs.t0 = thr(0);
          qs.t1 = thr(1);
          qs.t2 = thr(2);
          qs.m0 = mag(0);
          qs.m1 = mag(1);
          qs.m2 = mag(2);
          qs.m3 = mag(3);
          qs.scale = live ? post_scale / nrm : 0.f;
        }
      } else {
        quant_pair<BITS, ob + 1, 14 - 2 * s>(prev, qs, w, rh, rl, rs);
      }
      if constexpr (s == 7) prev = acc;
      __builtin_amdgcn_sched_barrier(0);
    });

    // x is dead: the next tile's loads go out now, to arrive during this tile's S' phase
    load_x<BF16IN>(x, n, tw + stride, lane, xr);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- S' phase of tile tw, then its stores
  auto sphase = [&](const int64_t tw) {
    // ---- steps 32 .. 63: z^T = S' r^T.  Block 3 runs s = 7 .. 0, so its first six steps read
    // only residual blocks 3 .. 1 while block 0 is quantized (16 coordinates over those six steps);
    // each later block pushes the previous block's 16 signs (two per step).
    uint32_t qw[2] = {0u, 0u};
    f32x16 z = zero16(), zprev = zero16();
    if constexpr (TQ_PROD_PRIO) __builtin_amdgcn_s_setprio(2);
    static_for<32, 64>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ob = 3 - ((k - 32) >> 3), s = 7 - ((k - 32) & 7), i = (k - 32) & 7;
      if constexpr (i == 0) z = zero16();
      z = mfma32(ring[k % kRing][0], rh[s], z);
      z = mfma32(ring[k % kRing][0], rl[s], z);
      z = mfma32(ring[k % kRing][1], rh[s], z);
      load_step<RP, (k + kRing) % 64>(lds, lane, ring[k % kRing]);
      if constexpr (ob == 3) {
        // block 0's pairs (14, 15), (12, 13), .. (0, 1) over steps i = 0 .. 5
        if constexpr (i < 6) {
          constexpr int p0 = (i * 8) / 6, p1 = ((i + 1) * 8) / 6;   // pairs [p0, p1) of 8
          static_for<p0, p1>([&](auto pc) { quant_pair<BITS, 0, 14 - 2 * decltype(pc)::value>(prev, qs, w, rh, rl, rs); });
        }
      } else {
        push_sign_pair<ob + 1, 15 - 2 * i>(zprev, qw);
      }
      if constexpr (i == 7) zprev = z;
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, 8>([&](auto ic) { push_sign_pair<0, 15 - 2 * decltype(ic)::value>(zprev, qw); });
    qw[0] = ~qw[0];
    qw[1] = ~qw[1];
    if constexpr (TQ_PROD_PRIO) __builtin_amdgcn_s_setprio(0);

    // ---- stores, through buffer resources bounded by the tile's rows that exist: a row past the
    // end is dropped by the range check.  Every store is unconditional, so the compiler keeps
    // exact count of the memory operations in flight (a store under a branch makes it wait for
    // all of them, the next tile's loads included, before the next tile starts).  Both halves of a
    // vector hold the same norm and residual norm and both store them.
    rs = add_halves(rs);
    const int64_t row0 = tw * 32;
    const int64_t left = n - row0;
    const uint32_t live_rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
    const int i = lane & 31;
    const __amdgpu_buffer_rsrc_t ridx = store_rsrc(idx_out + (row0 < n ? row0 : 0) * (4 * BITS), live_rows * (16u * BITS));
    const __amdgpu_buffer_rsrc_t rq = store_rsrc(qjl_out + (row0 < n ? row0 : 0) * 4, live_rows * 16u);
    const __amdgpu_buffer_rsrc_t rn = store_rsrc(norms_out + (row0 < n ? row0 : 0), live_rows * 4u);
    const __amdgpu_buffer_rsrc_t rr = store_rsrc(rnorm_out + (row0 < n ? row0 : 0), live_rows * 4u);
#pragma unroll
    for (int k = 0; k < BITS; ++k)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[2 * k], w[2 * k + 1]}, ridx,
                                            (uint32_t)(i * (16 * BITS) + 8 * BITS * half + 8 * k), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{qw[0], qw[1]}, rq, (uint32_t)(i * 16 + 8 * half), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nrm), rn, (uint32_t)(i * 4), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nrm * sqrtf(rs)), rr, (uint32_t)(i * 4), 0, 0);
  };
  // The loop is rotated so that it starts at an S' phase: on every path into its first
  // instruction the latest memory operations are the same eight tile loads, so the compiler's
  // wait counts there are exact (with the rotation phase first, the first entry, which has no
  // stores behind the loads, would force a wait for every store of the previous tile).
  // Entered unconditionally: a wave without a tile of its own (last block only) makes one pass
  // over clamped rows and stores nothing.
  rphase(tw);
  for (;;) {
    sphase(tw);
    tw += stride;
    if (tw >= ntiles) break;
    rphase(tw);
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
