// TurboQuant_mse encode at head dim 64 on the 32 x 32 x 16 bf16 matrix cores ([TQ] TurboQuant_mse
// section: the norm, the rotation, the nearest centroid of each coordinate, the packed indices;
// "Sub-byte KV cache quantization with TurboQuant", deployment checklist: the codebook's d is the
// model's head_dim, 64 in several common models).
//
// One wave takes tiles of 32 vectors and computes y^T = R x^T:
//   A = fragments of R, held in registers for the whole kernel (2 output blocks x 4 instructions x
//       2 passes, R as bf16 hi + lo: 16 u32x4 per lane), built once per block from the fp32 R;
//   B = x straight from HBM: bf16 input is exact, fp32 input is split into bf16 hi + lo (a third
//       pass, R hi times x lo).
// Lane (i, j) (i = lane % 32 the tile's vector, j = lane / 32) reads its vector's coordinates
// 32 j .. 32 j + 31 (instruction s: 32 j + 8 s .. + 7, the same contraction slots in A), and
// register r of output block ob holds y coordinate 32 j + 16 ob + r: the fragment rows are laid
// out so.  The lane therefore owns 32 consecutive coordinates of one vector and writes the BITS
// whole words of the packed row that hold them.
// Quantizer and packing as in the d = 128 encode: decisions on the raw product against
// t_p * ||x|| (sign-magnitude form of the antisymmetric codebook; a zero vector has every threshold
// at +inf and gets index K/2), bits shifted into the words from the bottom, coordinates in
// descending order.
#include <hip/hip_ext.h>

#include <type_traits>

#include "tq_device.h"

namespace tq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kE64Waves = 4;
constexpr int kE64Stride = 68;   // LDS row stride of the staged R (floats; 16-byte aligned rows)

__device__ __forceinline__ f32x16 mfma32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// w = 2 w + (this lane's bit of `lanes`): one v_addc with the lane mask as carry-in.
__device__ __forceinline__ uint32_t shift_in64(uint32_t w, uint64_t lanes) {
  uint32_t r;
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(lanes));
  return r;
}

// Buffer resource over `bytes` bytes at p: loads past the end read zeros, stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc64(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// bf16 hi / lo pair of two fp32 values (hi rounded to nearest even, lo = bf16 of the remainder).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2 pr = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
  const f32x2 rem = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
}

template <bool BF16IN>
struct X64;
template <>
struct X64<true> {
  u32x4 v[4];
};
template <>
struct X64<false> {
  f32x4 v[8];
};

// The lane's 32 coordinates of vector i of tile `tile` (rows past n read zeros, never stored).
template <bool BF16IN>
__device__ __forceinline__ void load_x64(const void* x, int64_t n, int64_t tile, int lane, X64<BF16IN>& r) {
  constexpr uint32_t kRow = BF16IN ? 128u : 256u;
  const int64_t row0 = tile * 32;
  const int64_t left = n - row0;
  const uint32_t rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
  const __amdgpu_buffer_rsrc_t rx = rsrc64(static_cast<const char*>(x) + (row0 < n ? row0 : 0) * kRow, rows * kRow);
  const uint32_t off = (uint32_t)(lane & 31) * kRow + (uint32_t)(lane >> 5) * (kRow / 2);
  if constexpr (BF16IN) {
#pragma unroll
    for (int s = 0; s < 4; ++s) r.v[s] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u * s, 0, 0);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      r.v[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u * s, 0, 0));
  }
}

// Push the BITS index bits of lane-local coordinate LI (top bit first).  idx = (m ^ sgn) + K/2,
// m = #{p : |v| >= t_p}: the top bit is [v >= 0], the low bits are m's bits XNOR [v >= 0]; m's
// bits come from a binary search over the sorted positive thresholds, top first.
template <int BITS, int LI>
__device__ __forceinline__ void push_coord64(float v, const float (&t)[7], uint32_t (&w)[BITS]) {
  constexpr int P = BITS * LI;
  const uint64_t pos = __builtin_amdgcn_ballot_w64(v >= 0.f);
  w[(P + BITS - 1) >> 5] = shift_in64(w[(P + BITS - 1) >> 5], pos);
  const float a = fabsf(v);
  if constexpr (BITS == 2) {
    w[P >> 5] = shift_in64(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= t[0]) ^ pos));
  } else if constexpr (BITS == 3) {
    const bool hi = a >= t[1];
    w[(P + 1) >> 5] = shift_in64(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(hi) ^ pos));
    w[P >> 5] = shift_in64(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= (hi ? t[2] : t[0])) ^ pos));
  } else if constexpr (BITS == 4) {
    const bool h2 = a >= t[3];
    w[(P + 2) >> 5] = shift_in64(w[(P + 2) >> 5], ~(__builtin_amdgcn_ballot_w64(h2) ^ pos));
    const bool h1 = a >= (h2 ? t[5] : t[1]);
    w[(P + 1) >> 5] = shift_in64(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(h1) ^ pos));
    const float t0 = h1 ? (h2 ? t[6] : t[2]) : (h2 ? t[4] : t[0]);
    w[P >> 5] = shift_in64(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= t0) ^ pos));
  }
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for64(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for64<B + 1, E>(f);
  }
}

template <int BITS, bool BF16IN, int RP>
__global__ __launch_bounds__(kE64Waves * 64, 2) void k_encode_mse_d64(const void* __restrict__ x, int64_t n,
                                                                     const float* __restrict__ r32, CodebookArgs cb,
                                                                     uint32_t* __restrict__ idx_out,
                                                                     float* __restrict__ norms_out) {
  constexpr int H = 1 << (BITS - 1);
  __shared__ float rs[64 * kE64Stride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 31, j = lane >> 5;
  const int64_t ntiles = (n + 31) >> 5;
  const int64_t stride = (int64_t)gridDim.x * kE64Waves;
  int64_t tw = (int64_t)blockIdx.x * kE64Waves + wave;

  // R into LDS (coalesced), the first tile's loads in flight meanwhile.
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(r32);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = threadIdx.x + k * kE64Waves * 64;   // float4 index, 1024 of them
      const f32x4 v = src[q];
      *reinterpret_cast<f32x4*>(&rs[(q >> 4) * kE64Stride + 4 * (q & 15)]) = v;
    }
  }
  X64<BF16IN> xr;
  load_x64<BF16IN>(x, n, tw, lane, xr);
  __syncthreads();

  // A fragments: lane (i, j), output block ob, instruction s: R[o][32 j + 8 s + e], e = 0..7, with
  // o the y coordinate that D row i of block ob carries (rows 8 (r / 4) + 4 j' + r % 4 of a block
  // belong to lane half j' and register r).
  u32x4 fa[RP][2][4];
#pragma unroll
  for (int ob = 0; ob < 2; ++ob) {
    const int o = 32 * ((i >> 2) & 1) + 16 * ob + 4 * (i >> 3) + (i & 3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* row = &rs[o * kE64Stride + 32 * j + 8 * s];
      const f32x4 a = *reinterpret_cast<const f32x4*>(row);
      const f32x4 b = *reinterpret_cast<const f32x4*>(row + 4);
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t hi, lo;
        split2(v[2 * k], v[2 * k + 1], hi, lo);
        fa[0][ob][s][k] = hi;
        if constexpr (RP == 2) fa[1][ob][s][k] = lo;
      }
    }
  }

  for (;;) {
    const X64<BF16IN> cur = xr;
    load_x64<BF16IN>(x, n, tw + stride, lane, xr);

    // B operands and the norm
    u32x4 bx[4], bxl[BF16IN ? 1 : 4];
    float ss = 0.f;
    if constexpr (BF16IN) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bx[s] = cur.v[s];
        uint32_t wv[4];
        __builtin_memcpy(wv, &cur.v[s], sizeof(wv));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 p2 = __builtin_bit_cast(bf16x2, wv[e]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss, false);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f32x4 a = cur.v[2 * s], b = cur.v[2 * s + 1];
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t hi, lo;
          split2(v[2 * k], v[2 * k + 1], hi, lo);
          bx[s][k] = hi;
          bxl[s][k] = lo;
          ss = fmaf(v[2 * k], v[2 * k], ss);
          ss = fmaf(v[2 * k + 1], v[2 * k + 1], ss);
        }
      }
    }

    // y^T = R x^T, block 1 first (its coordinates are packed first); each accumulator's MFMAs
    // back to back.
    f32x16 acc[2];
    static_for64<0, 2>([&](auto oc) {
      constexpr int ob = 1 - decltype(oc)::value;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ob][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc[ob] = mfma32x16(fa[0][ob][s], bx[s], acc[ob]);
        if constexpr (!BF16IN) acc[ob] = mfma32x16(fa[0][ob][s], bxl[s], acc[ob]);
        if constexpr (RP == 2) acc[ob] = mfma32x16(fa[1][ob][s], bx[s], acc[ob]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });

    ss += __shfl_xor(ss, 32);
    const float nrm = sqrtf(ss);
    const bool live = nrm > 0.f;
    float t[7];
#pragma unroll
    for (int p = 0; p < 7; ++p) t[p] = (p < H - 1 && live) ? __int_as_float(cb.tpos[p]) * nrm : INFINITY;

    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = 0u;
    static_for64<0, 32>([&](auto lc) {
      constexpr int li = 31 - decltype(lc)::value;   // descending
      push_coord64<BITS, li>(acc[li >> 4][li & 15], t, w);
    });

    // stores through buffer resources bounded by the tile's rows that exist
    const int64_t row0 = tw * 32;
    const int64_t left = n - row0;
    const uint32_t live_rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
    const __amdgpu_buffer_rsrc_t ridx =
        rsrc64(idx_out + (row0 < n ? row0 : 0) * (2 * BITS), live_rows * (8u * BITS));
    const __amdgpu_buffer_rsrc_t rn = rsrc64(norms_out + (row0 < n ? row0 : 0), live_rows * 4u);
    const uint32_t wo = (uint32_t)(i * (8 * BITS) + 4 * BITS * j);
    if constexpr (BITS == 1) {
      __builtin_amdgcn_raw_buffer_store_b32(w[0], ridx, wo, 0, 0);
    } else if constexpr (BITS == 2) {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, ridx, wo, 0, 0);
    } else if constexpr (BITS == 3) {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, ridx, wo, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(w[2], ridx, wo + 8u, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, ridx, wo, 0, 0);
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nrm), rn, (uint32_t)(i * 4), 0, 0);

    tw += stride;
    if (tw >= ntiles) break;
  }
}

// ---------------------------------------------------------------------------------------
// TurboQuant_prod at d = 64 ([TQ] TurboQuant_prod section): the (b-1)-bit MSE stage as above, then
// the residual in the rotated domain, r = y / ||x|| - C[idx], and the 1-bit sketch sign(S' r) with
// S' = S R^T, and gamma = ||x|| ||r||.  The residual the quantizer leaves in a lane's registers
// (coordinates 32 j .. 32 j + 31 of vector i) is that lane's B operand of the second product in
// bf16 hi + lo (coordinate 32 j + 8 s + e in instruction s); S' is split once per block into
// hi / lo A fragments kept in LDS; three passes (S'hi rhi, S'hi rlo, S'lo rhi) carry fp32-level
// accuracy into the signs.  The lane's 32 signs are word j of the vector's sketch.
// ---------------------------------------------------------------------------------------
template <int BITS>
struct PQ64 {
  float t0, t1, t2;        // positive thresholds on the raw product (t_p ||x||)
  float m0, m1, m2, m3;    // non-negative centroids
  float scale;             // raw product -> unit coordinate (1 / ||x||; 0 for a zero vector)
};

// Quantize lane-local coordinate LI (raw product v): push its BITS index bits, return the
// unit-scale residual v / ||x|| - C[idx].
template <int BITS, int LI>
__device__ __forceinline__ float pq64_coord(float v, const PQ64<BITS>& q, uint32_t (&w)[BITS]) {
  constexpr int P = BITS * LI;
  const bool nonneg = v >= 0.f;
  const uint64_t pos = __builtin_amdgcn_ballot_w64(nonneg);
  w[(P + BITS - 1) >> 5] = shift_in64(w[(P + BITS - 1) >> 5], pos);
  const float a = fabsf(v);
  float mag;
  if constexpr (BITS == 1) {
    mag = q.m0;
  } else if constexpr (BITS == 2) {
    const bool ge = a >= q.t0;
    w[P >> 5] = shift_in64(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(ge) ^ pos));
    mag = ge ? q.m1 : q.m0;
  } else {
    const bool hi = a >= q.t1;
    w[(P + 1) >> 5] = shift_in64(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(hi) ^ pos));
    const bool lo = a >= (hi ? q.t2 : q.t0);
    w[P >> 5] = shift_in64(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(lo) ^ pos));
    const float m_lo = lo ? q.m1 : q.m0;
    const float m_hi = lo ? q.m3 : q.m2;
    mag = hi ? m_hi : m_lo;
  }
  return fmaf(v, q.scale, nonneg ? -mag : mag);
}

// Sum of v over lanes l and l ^ 32 (a register swap of the wave's halves).
__device__ __forceinline__ float add_halves64(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int BITS, bool BF16IN>
__global__ __launch_bounds__(kE64Waves * 64, 2) void k_encode_prod_d64(
    const void* __restrict__ x, int64_t n, const float* __restrict__ r32, const float* __restrict__ sp32,
    CodebookArgs cb, uint32_t* __restrict__ idx_out, float* __restrict__ norms_out, uint32_t* __restrict__ qjl_out,
    float* __restrict__ rnorm_out) {
  constexpr int H = 1 << (BITS - 1);
  __shared__ float rs[64 * kE64Stride];
  __shared__ u32x4 sfr[2][2][4][64];   // S' fragments [pass][output block][instruction][lane]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 31, j = lane >> 5;
  const int64_t ntiles = (n + 31) >> 5;
  const int64_t stride = (int64_t)gridDim.x * kE64Waves;
  int64_t tw = (int64_t)blockIdx.x * kE64Waves + wave;

  auto stage = [&](const float* m) {
    const f32x4* src = reinterpret_cast<const f32x4*>(m);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = threadIdx.x + k * kE64Waves * 64;
      *reinterpret_cast<f32x4*>(&rs[(q >> 4) * kE64Stride + 4 * (q & 15)]) = src[q];
    }
  };
  // lane (i, j), block ob, instruction s: row o of the matrix staged in rs, columns 32 j + 8 s ..
  auto frag = [&](int ob, int s, uint32_t (&hi)[4], uint32_t (&lo)[4]) {
    const int o = 32 * ((i >> 2) & 1) + 16 * ob + 4 * (i >> 3) + (i & 3);
    const float* row = &rs[o * kE64Stride + 32 * j + 8 * s];
    const f32x4 a = *reinterpret_cast<const f32x4*>(row);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + 4);
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) split2(v[2 * k], v[2 * k + 1], hi[k], lo[k]);
  };

  stage(r32);
  X64<BF16IN> xr;
  load_x64<BF16IN>(x, n, tw, lane, xr);
  __syncthreads();
  u32x4 fa[2][2][4];   // R fragments [pass][block][instruction]
#pragma unroll
  for (int ob = 0; ob < 2; ++ob)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t hi[4], lo[4];
      frag(ob, s, hi, lo);
      fa[0][ob][s] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      fa[1][ob][s] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  __syncthreads();
  stage(sp32);
  __syncthreads();
  // every wave writes the same S' fragments (its lanes' own slots)
#pragma unroll
  for (int ob = 0; ob < 2; ++ob)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t hi[4], lo[4];
      frag(ob, s, hi, lo);
      sfr[0][ob][s][lane] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      sfr[1][ob][s][lane] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  __syncthreads();

  for (;;) {
    const X64<BF16IN> cur = xr;
    load_x64<BF16IN>(x, n, tw + stride, lane, xr);

    u32x4 bx[4], bxl[BF16IN ? 1 : 4];
    float ss = 0.f;
    if constexpr (BF16IN) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bx[s] = cur.v[s];
        uint32_t wv[4];
        __builtin_memcpy(wv, &cur.v[s], sizeof(wv));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 p2 = __builtin_bit_cast(bf16x2, wv[e]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss, false);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f32x4 a = cur.v[2 * s], b = cur.v[2 * s + 1];
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t hi, lo;
          split2(v[2 * k], v[2 * k + 1], hi, lo);
          bx[s][k] = hi;
          bxl[s][k] = lo;
          ss = fmaf(v[2 * k], v[2 * k], ss);
          ss = fmaf(v[2 * k + 1], v[2 * k + 1], ss);
        }
      }
    }

    // y^T = R x^T
    f32x16 acc[2];
    static_for64<0, 2>([&](auto oc) {
      constexpr int ob = 1 - decltype(oc)::value;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ob][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc[ob] = mfma32x16(fa[0][ob][s], bx[s], acc[ob]);
        if constexpr (!BF16IN) acc[ob] = mfma32x16(fa[0][ob][s], bxl[s], acc[ob]);
        acc[ob] = mfma32x16(fa[1][ob][s], bx[s], acc[ob]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });

    ss = add_halves64(ss);
    const float nrm = sqrtf(ss);
    const bool live = nrm > 0.f;
    PQ64<BITS> q;
    auto thr = [&](int p) { return p < H - 1 ? (live ? __int_as_float(cb.tpos[p]) * nrm : INFINITY) : INFINITY; };
    auto mag = [&](int p) { return p < H ? (live ? cb.cpos[p] : 0.f) : 0.f; };
    q.t0 = thr(0);
    q.t1 = thr(1);
    q.t2 = thr(2);
    q.m0 = mag(0);
    q.m1 = mag(1);
    q.m2 = mag(2);
    q.m3 = mag(3);
    q.scale = live ? 1.f / nrm : 0.f;

    // indices (descending coordinates) and the residual as the second product's B operand
    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = 0u;
    float rsum = 0.f;
    u32x4 rh[4], rl[4];
    static_for64<0, 16>([&](auto pc) {
      constexpr int li1 = 31 - 2 * decltype(pc)::value, li0 = li1 - 1;   // pair (li0, li1)
      const float r1 = pq64_coord<BITS, li1>(acc[li1 >> 4][li1 & 15], q, w);
      const float r0 = pq64_coord<BITS, li0>(acc[li0 >> 4][li0 & 15], q, w);
      rsum = fmaf(r0, r0, rsum);
      rsum = fmaf(r1, r1, rsum);
      uint32_t hi, lo;
      split2(r0, r1, hi, lo);
      rh[li0 >> 3][(li0 & 7) >> 1] = hi;
      rl[li0 >> 3][(li0 & 7) >> 1] = lo;
    });

    // z^T = S' r^T: three passes per instruction
    f32x16 z[2];
    static_for64<0, 2>([&](auto oc) {
      constexpr int ob = 1 - decltype(oc)::value;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[ob][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 ah = sfr[0][ob][s][lane], al = sfr[1][ob][s][lane];
        z[ob] = mfma32x16(ah, rh[s], z[ob]);
        z[ob] = mfma32x16(ah, rl[s], z[ob]);
        z[ob] = mfma32x16(al, rh[s], z[ob]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // the lane's 32 signs [z >= 0], descending, into one word
    uint32_t qw = 0u;
    static_for64<0, 32>([&](auto lc) {
      constexpr int li = 31 - decltype(lc)::value;
      qw = shift_in64(qw, __builtin_amdgcn_ballot_w64(z[li >> 4][li & 15] >= 0.f));
    });
    rsum = add_halves64(rsum);

    const int64_t row0 = tw * 32;
    const int64_t left = n - row0;
    const uint32_t live_rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
    const int64_t rb = row0 < n ? row0 : 0;
    const __amdgpu_buffer_rsrc_t ridx = rsrc64(idx_out + rb * (2 * BITS), live_rows * (8u * BITS));
    const __amdgpu_buffer_rsrc_t rq = rsrc64(qjl_out + rb * 2, live_rows * 8u);
    const __amdgpu_buffer_rsrc_t rn = rsrc64(norms_out + rb, live_rows * 4u);
    const __amdgpu_buffer_rsrc_t rr = rsrc64(rnorm_out + rb, live_rows * 4u);
    const uint32_t wo = (uint32_t)(i * (8 * BITS) + 4 * BITS * j);
    if constexpr (BITS == 1) {
      __builtin_amdgcn_raw_buffer_store_b32(w[0], ridx, wo, 0, 0);
    } else if constexpr (BITS == 2) {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, ridx, wo, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, ridx, wo, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(w[2], ridx, wo + 8u, 0, 0);
    }
    __builtin_amdgcn_raw_buffer_store_b32(qw, rq, (uint32_t)(i * 8 + 4 * j), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nrm), rn, (uint32_t)(i * 4), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nrm * sqrtf(rsum)), rr, (uint32_t)(i * 4), 0, 0);

    tw += stride;
    if (tw >= ntiles) break;
  }
}

template <int BITS, bool BF16IN>
hipError_t prod64_launch(const void* x, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                         const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits, float* rnorms,
                         hipStream_t st) {
  const int64_t ntiles = (n + 31) / 32;
  int64_t blocks = (ntiles + kE64Waves - 1) / kE64Waves;
  const int64_t cap = (int64_t)num_cus() * 2;   // the resident blocks (two waves per SIMD)
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((k_encode_prod_d64<BITS, BF16IN>), dim3((unsigned)blocks), dim3(kE64Waves * 64), 0, st, x, n,
                     rot->r32_dev, qjl->sp32_dev, cb, idx, norms, qbits, rnorms);
  return hipGetLastError();
}

template <int BITS, bool BF16IN>
hipError_t mse64_launch(const void* x, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb, uint32_t* idx,
                        float* norms, hipStream_t st) {
  const int64_t ntiles = (n + 31) / 32;
  int64_t blocks = (ntiles + kE64Waves - 1) / kE64Waves;
  const int64_t cap = (int64_t)num_cus() * (BF16IN ? 3 : 2);   // the resident blocks (3 or 2 waves per SIMD)
  if (blocks > cap) blocks = cap;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (take_armed_timer(&ev0, &ev1)) {
    hipExtLaunchKernelGGL((k_encode_mse_d64<BITS, BF16IN, 2>), dim3((unsigned)blocks), dim3(kE64Waves * 64), 0, st,
                          ev0, ev1, 0, x, n, rot->r32_dev, cb, idx, norms);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_encode_mse_d64<BITS, BF16IN, 2>), dim3((unsigned)blocks), dim3(kE64Waves * 64), 0, st, x, n,
                     rot->r32_dev, cb, idx, norms);
  return hipGetLastError();
}

template <int BITS>
hipError_t mse64_dispatch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                          uint32_t* idx, float* norms, hipStream_t st) {
  return bf16 ? mse64_launch<BITS, true>(x, n, rot, cb, idx, norms, st)
              : mse64_launch<BITS, false>(x, n, rot, cb, idx, norms, st);
}

}  // namespace

hipError_t launch_encode_prod_d64(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                  const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                  uint32_t* qbits, float* rnorms, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (rot->d != 64 || !rot->r32_dev || !qjl || !qjl->sp32_dev) return hipErrorInvalidValue;
  switch (cb.bits) {
    case 1: return bf16 ? prod64_launch<1, true>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : prod64_launch<1, false>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
    case 2: return bf16 ? prod64_launch<2, true>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : prod64_launch<2, false>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
    case 3: return bf16 ? prod64_launch<3, true>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : prod64_launch<3, false>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_encode_mse_d64(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                 const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (rot->d != 64 || !rot->r32_dev) return hipErrorInvalidValue;
  switch (cb.bits) {
    case 1: return mse64_dispatch<1>(x, bf16, n, rot, cb, idx, norms, st);
    case 2: return mse64_dispatch<2>(x, bf16, n, rot, cb, idx, norms, st);
    case 3: return mse64_dispatch<3>(x, bf16, n, rot, cb, idx, norms, st);
    case 4: return mse64_dispatch<4>(x, bf16, n, rot, cb, idx, norms, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
