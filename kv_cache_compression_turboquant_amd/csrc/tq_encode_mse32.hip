// TurboQuant_mse encode at d = 128 (rows layout) with a dense rotation, on the 32 x 32 x 16 bf16
// matrix cores ([TQ] TurboQuant_mse section: the norm, the rotation, the nearest centroid of each
// coordinate, the packed indices).
//
// One wave takes tiles of 32 vectors: y^T = R x^T with A = fragments of R (bf16 hi and lo, LDS) and
// B = x straight from HBM (bf16 exact; fp32 split into hi + lo, one more pass).  Lane (i, j)
// (i = lane % 32 the vector, j = lane / 32) holds coordinates 64 j .. 64 j + 63 of vector i in both
// operands, and output block ob, register r is coordinate 64 j + 16 ob + r (the host lays the
// fragment rows out so).  The blocks run ob = 3 .. 0; block ob + 1 is quantized while block ob's
// MFMAs run, two coordinates per step, and block 0 after the last one.  Each lane pushes the index
// bits of its 64 coordinates (descending) into the 2 BITS words of the row it owns, from the wave's
// decision masks (one v_addc per bit), as the other encodes do.  Fragments stream through a ring
// of registers a few steps ahead of their MFMA; the next tile's loads go out once x is dead.
#include <hip/hip_ext.h>

#include <type_traits>

#include "tq_device.h"

namespace tq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef TQ_MSE32_WAVES
#define TQ_MSE32_WAVES 8
#endif
#ifndef TQ_MSE32_BLOCKS
#define TQ_MSE32_BLOCKS 2
#endif
#ifndef TQ_MSE32_WPE
#define TQ_MSE32_WPE 4
#endif
constexpr int kM32Waves = TQ_MSE32_WAVES;   // waves per block
constexpr int kM32Blocks = TQ_MSE32_BLOCKS; // resident blocks per CU (64 KB of fragments each)
constexpr int kM32Wpe = TQ_MSE32_WPE;       // waves per SIMD the registers are sized for
constexpr int kM32FragU4 = 2048;   // u32x4 per pass: 4 output blocks x 8 instructions x 64 lanes
#ifndef TQ_MSE32_RING
#define TQ_MSE32_RING 2
#endif
constexpr int kM32Ring = TQ_MSE32_RING;  // fragment ring; divides the 32 steps of a tile

__device__ __forceinline__ f32x16 m32_mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// w = 2 w + (this lane's bit of `lanes`): one v_addc with the lane mask as carry-in.
__device__ __forceinline__ uint32_t m32_shift_in(uint32_t w, uint64_t lanes) {
  uint32_t r;
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(lanes));
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t m32_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int B, int E, typename F>
__device__ __forceinline__ void m32_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    m32_for<B + 1, E>(f);
  }
}

template <bool BF16IN>
struct M32X;
template <>
struct M32X<true> {
  u32x4 v[8];
};
template <>
struct M32X<false> {
  f32x4 v[16];
};

// The lane's 64 coordinates of vector i of tile `tile` (rows past n read zeros, never stored).
template <bool BF16IN>
__device__ __forceinline__ void m32_load(const void* x, int64_t n, int64_t tile, int lane, M32X<BF16IN>& r) {
  constexpr uint32_t kRow = BF16IN ? 256u : 512u;
  const int64_t row0 = tile * 32;
  const int64_t left = n - row0;
  const uint32_t rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
  const __amdgpu_buffer_rsrc_t rx = m32_rsrc(static_cast<const char*>(x) + (row0 < n ? row0 : 0) * kRow, rows * kRow);
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

// Step K (0 .. 31) of a tile: output block 3 - K / 8, instruction K % 8; its RP fragments.
template <int RP, int K>
__device__ __forceinline__ void m32_frag(const u32x4* lds, u32x4 (&slot)[2]) {
  constexpr int ob = 3 - (K >> 3), s = K & 7;
  slot[0] = lds[(ob * 8 + s) * 64];
  if constexpr (RP == 2) slot[1] = lds[kM32FragU4 + (ob * 8 + s) * 64];
}

// Push the BITS index bits of lane-local coordinate LI (raw product v; thresholds t on it).
template <int BITS, int LI>
__device__ __forceinline__ void m32_push(float v, const float (&t)[7], uint32_t (&w)[2 * BITS]) {
  constexpr int P = BITS * LI;
  const uint64_t pos = __builtin_amdgcn_ballot_w64(v >= 0.f);
  w[(P + BITS - 1) >> 5] = m32_shift_in(w[(P + BITS - 1) >> 5], pos);
  const float a = fabsf(v);
  if constexpr (BITS == 2) {
    w[P >> 5] = m32_shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= t[0]) ^ pos));
  } else if constexpr (BITS == 3) {
    const bool hi = a >= t[1];
    w[(P + 1) >> 5] = m32_shift_in(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(hi) ^ pos));
    w[P >> 5] = m32_shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= (hi ? t[2] : t[0])) ^ pos));
  } else if constexpr (BITS == 4) {
    const bool h2 = a >= t[3];
    w[(P + 2) >> 5] = m32_shift_in(w[(P + 2) >> 5], ~(__builtin_amdgcn_ballot_w64(h2) ^ pos));
    const bool h1 = a >= (h2 ? t[5] : t[1]);
    w[(P + 1) >> 5] = m32_shift_in(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(h1) ^ pos));
    const float t0 = h1 ? (h2 ? t[6] : t[2]) : (h2 ? t[4] : t[0]);
    w[P >> 5] = m32_shift_in(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= t0) ^ pos));
  }
}

template <int BITS, bool BF16IN, int RP>
__global__ __launch_bounds__(kM32Waves * 64, kM32Wpe) void k_encode_mse32_d128(
    const void* __restrict__ x, int64_t n, const u32x4* __restrict__ frag_r, float post_scale, CodebookArgs cb,
    uint32_t* __restrict__ idx_out, float* __restrict__ norms_out) {
  constexpr int H = 1 << (BITS - 1);
  constexpr int kThreads = kM32Waves * 64;
  constexpr int kTotal = RP * kM32FragU4;
  __shared__ u32x4 lds[kTotal];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 31, j = lane >> 5;
  const int64_t ntiles = (n + 31) >> 5;
  const int64_t stride = (int64_t)gridDim.x * kM32Waves;
  int64_t tw = (int64_t)blockIdx.x * kM32Waves + wave;

  // fragments into LDS, the first tile's loads meanwhile
  for (int k = threadIdx.x; k < kTotal; k += kThreads) lds[k] = frag_r[k];
  M32X<BF16IN> xr;
  m32_load<BF16IN>(x, n, tw, lane, xr);
  __syncthreads();
  const u32x4* const ldl = lds + lane;
  u32x4 ring[kM32Ring][2];
  m32_for<0, kM32Ring>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    m32_frag<RP, k>(ldl, ring[k]);
  });
  const float inv_post = 1.0f / post_scale;

  for (;;) {
    // B operands (and the fp32 input's low part)
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
    uint32_t w[2 * BITS];
#pragma unroll
    for (int k = 0; k < 2 * BITS; ++k) w[k] = 0u;
    float t[7];
    f32x16 acc = {}, prev = {};
    float nrm = 0.f;

    m32_for<0, 32>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ob = 3 - (k >> 3), s = k & 7;
      if constexpr (s == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      }
      acc = m32_mfma(ring[k % kM32Ring][0], bx[s], acc);
      if constexpr (!BF16IN) acc = m32_mfma(ring[k % kM32Ring][0], bxl[s], acc);
      if constexpr (RP == 2) acc = m32_mfma(ring[k % kM32Ring][1], bx[s], acc);
      if constexpr (k + kM32Ring < 32) m32_frag<RP, k + kM32Ring>(ldl, ring[k % kM32Ring]);
      if constexpr (ob == 3) {
        // the norm during block 3 (bf16: one dot2 per pair), the thresholds at its end
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
          const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
          nrm = sqrtf(__uint_as_float(p[0]) + __uint_as_float(p[1]));
          // decisions on the raw product against t_p * ||x|| / post_scale; a zero vector keeps every
          // threshold at +inf (index K/2)
          const bool live = nrm > 0.f;
          const float tsc = nrm * inv_post;
#pragma unroll
          for (int q = 0; q < 7; ++q) t[q] = (q < H - 1 && live) ? __int_as_float(cb.tpos[q]) * tsc : INFINITY;
        }
      } else {
        // block ob + 1: coordinates 16 (ob + 1) + 15 - 2 s and 16 (ob + 1) + 14 - 2 s
        constexpr int r1 = 15 - 2 * s, r0 = r1 - 1;
        m32_push<BITS, 16 * (ob + 1) + r1>(prev[r1], t, w);
        m32_push<BITS, 16 * (ob + 1) + r0>(prev[r0], t, w);
      }
      if constexpr (s == 7) prev = acc;
      __builtin_amdgcn_sched_barrier(0);
    });
    // x is dead: the next tile's loads go out, then block 0 is quantized
    m32_load<BF16IN>(x, n, tw + stride, lane, xr);
    m32_for<0, kM32Ring>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      m32_frag<RP, k>(ldl, ring[k]);
    });
    m32_for<0, 8>([&](auto pc) {
      constexpr int r1 = 15 - 2 * decltype(pc)::value, r0 = r1 - 1;
      m32_push<BITS, r1>(prev[r1], t, w);
      m32_push<BITS, r0>(prev[r0], t, w);
    });

    // stores, bounded by the tile's rows that exist
    const int64_t row0 = tw * 32;
    const int64_t left = n - row0;
    const uint32_t live_rows = left >= 32 ? 32u : (left > 0 ? (uint32_t)left : 0u);
    const int64_t rb = row0 < n ? row0 : 0;
    const __amdgpu_buffer_rsrc_t ridx = m32_rsrc(idx_out + rb * (4 * BITS), live_rows * (16u * BITS));
    const __amdgpu_buffer_rsrc_t rn = m32_rsrc(norms_out + rb, live_rows * 4u);
    const uint32_t wo = (uint32_t)(i * (16 * BITS) + 8 * BITS * j);
#pragma unroll
    for (int k = 0; k < BITS; ++k)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[2 * k], w[2 * k + 1]}, ridx, wo + 8u * k, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nrm), rn, (uint32_t)(i * 4), 0, 0);

    tw += stride;
    if (tw >= ntiles) break;
  }
}

template <int BITS, bool BF16IN, int RP>
hipError_t mse32_launch(const void* x, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb, uint32_t* idx,
                        float* norms, hipStream_t st) {
  const int64_t ntiles = (n + 31) / 32;
  int64_t blocks = (ntiles + kM32Waves - 1) / kM32Waves;
  const int64_t cap = (int64_t)num_cus() * kM32Blocks;
  if (blocks > cap) blocks = cap;
  const u32x4* fr = reinterpret_cast<const u32x4*>(rot->frag32_dev);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (take_armed_timer(&ev0, &ev1)) {
    hipExtLaunchKernelGGL((k_encode_mse32_d128<BITS, BF16IN, RP>), dim3((unsigned)blocks), dim3(kM32Waves * 64), 0,
                          st, ev0, ev1, 0, x, n, fr, rot->post_scale, cb, idx, norms);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_encode_mse32_d128<BITS, BF16IN, RP>), dim3((unsigned)blocks), dim3(kM32Waves * 64), 0, st,
                     x, n, fr, rot->post_scale, cb, idx, norms);
  return hipGetLastError();
}

template <int BITS>
hipError_t mse32_dispatch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                          uint32_t* idx, float* norms, hipStream_t st) {
  if (bf16)
    return rot->passes == 1 ? mse32_launch<BITS, true, 1>(x, n, rot, cb, idx, norms, st)
                            : mse32_launch<BITS, true, 2>(x, n, rot, cb, idx, norms, st);
  return rot->passes == 1 ? mse32_launch<BITS, false, 1>(x, n, rot, cb, idx, norms, st)
                          : mse32_launch<BITS, false, 2>(x, n, rot, cb, idx, norms, st);
}

}  // namespace

hipError_t launch_encode_mse32_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                    const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (!rot->frag32_dev) return hipErrorInvalidValue;
  switch (cb.bits) {
    case 1: return mse32_dispatch<1>(x, bf16, n, rot, cb, idx, norms, st);
    case 2: return mse32_dispatch<2>(x, bf16, n, rot, cb, idx, norms, st);
    case 3: return mse32_dispatch<3>(x, bf16, n, rot, cb, idx, norms, st);
    case 4: return mse32_dispatch<4>(x, bf16, n, rot, cb, idx, norms, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
