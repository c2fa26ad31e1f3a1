// Measurement kernels: the achievable ceilings that the roofline fractions are read against.
// A streaming read and a streaming copy of a caller buffer (HBM), and a loop of independent
// MFMA chains (matrix-core issue rate).  Not part of the method; nothing here is on the hot path.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef unsigned int pk_u32x4 __attribute__((ext_vector_type(4)));
typedef float pk_f32x4 __attribute__((ext_vector_type(4)));
typedef float pk_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 pk_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 pk_f16x8 __attribute__((ext_vector_type(8)));

constexpr int kPeakThreads = 256;
constexpr int kPeakUnroll = 4;   // 16-byte loads in flight per thread and iteration

// Grid-stride read of n16 16-byte words, kPeakUnroll loads issued before any is used.  The XOR of
// everything read is stored only when `flag` is set (the host passes 0), which keeps the loads live.
__global__ __launch_bounds__(kPeakThreads) void k_peak_read(const pk_u32x4* __restrict__ src, int64_t n16, int flag,
                                                            uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kPeakThreads;
  int64_t i = (int64_t)blockIdx.x * kPeakThreads + threadIdx.x;
  pk_u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kPeakUnroll - 1) * stride < n16; i += kPeakUnroll * stride) {
    pk_u32x4 v[kPeakUnroll];
#pragma unroll
    for (int u = 0; u < kPeakUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kPeakUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  if (flag) sink[(int64_t)blockIdx.x * kPeakThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(kPeakThreads) void k_peak_copy(pk_u32x4* __restrict__ dst, const pk_u32x4* __restrict__ src,
                                                            int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kPeakThreads;
  int64_t i = (int64_t)blockIdx.x * kPeakThreads + threadIdx.x;
  for (; i + (kPeakUnroll - 1) * stride < n16; i += kPeakUnroll * stride) {
    pk_u32x4 v[kPeakUnroll];
#pragma unroll
    for (int u = 0; u < kPeakUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kPeakUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// CHAINS independent accumulators per wave, each advanced `iters` times.  Operands come from the
// thread index, so nothing folds; every lane stores the sum of its accumulators.
template <int KIND>
__global__ __launch_bounds__(kPeakThreads) void k_peak_mfma(int iters, float* __restrict__ out) {
  const uint32_t seed = 0x3f803f80u ^ (threadIdx.x * 0x00010001u);
  const pk_u32x4 ab = {seed, seed ^ 0x00400040u, seed ^ 0x00200020u, seed ^ 0x00100010u};
  float total = 0.f;
  if constexpr (KIND == 0 || KIND == 2) {   // 16 x 16 x 32
    constexpr int CHAINS = 8;
    pk_f32x4 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = pk_f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) {
        if constexpr (KIND == 0)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pk_bf16x8, ab),
                                                           __builtin_bit_cast(pk_bf16x8, ab), acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(pk_f16x8, ab),
                                                          __builtin_bit_cast(pk_f16x8, ab), acc[c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) total += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {                                  // 32 x 32 x 16
    constexpr int CHAINS = 4;
    pk_f32x16 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) {
        if constexpr (KIND == 1)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pk_bf16x8, ab),
                                                           __builtin_bit_cast(pk_bf16x8, ab), acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(pk_f16x8, ab),
                                                          __builtin_bit_cast(pk_f16x8, ab), acc[c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += acc[c][r];
  }
  out[(int64_t)blockIdx.x * kPeakThreads + threadIdx.x] = total;
}

}  // namespace

hipError_t launch_peak_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_peak_read, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st,
                     static_cast<const pk_u32x4*>(src), bytes / 16, 0, sink);
  return hipGetLastError();
}

hipError_t launch_peak_copy(void* dst, const void* src, int64_t bytes, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(k_peak_copy, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st, static_cast<pk_u32x4*>(dst),
                     static_cast<const pk_u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(int kind, int iters, int blocks, float* out, hipStream_t st) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_peak_mfma<0>, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st, iters, out); break;
    case 1: hipLaunchKernelGGL(k_peak_mfma<1>, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st, iters, out); break;
    case 2: hipLaunchKernelGGL(k_peak_mfma<2>, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st, iters, out); break;
    case 3: hipLaunchKernelGGL(k_peak_mfma<3>, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st, iters, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
