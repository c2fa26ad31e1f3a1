// Device-side helpers shared by the HIP kernels for gfx950 (MI355X): vector types, MFMA
// wrappers, bf16 / fp16 bit conversions, the bucketize and pack primitives, and the small
// LDS tables that decode packed indices into fp16 centroid operands.
//
// MFMA conventions (v_mfma_f32_16x16x32_{bf16,f16}): lane l = n + 16 g (n = l % 16,
// g = l / 16) holds A row n, B column n and D column n.  Within one instruction, element e of
// lane group g covers contraction slot 8 g + e for both A and B, and register r of D holds row
// 4 g + r.  Every contraction here is over vector coordinates, and the kernels assign
// coordinate 32 g + 8 s + e to element e of lane group g in instruction s (s = 0..3 for
// d = 128), identically for both operands, so each lane streams 32 consecutive coordinates.
#ifndef TQ_DEVICE_H_
#define TQ_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kQjl = 1.2533141373155002512f;  // sqrt(pi / 2)

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// idx = #{k : y >= t_k} over the 2^BITS - 1 thresholds (ties go to the upper index).
template <int BITS>
__device__ __forceinline__ uint32_t bucketize(float y, const CodebookArgs& cb) {
  uint32_t idx = 0;
#pragma unroll
  for (int k = 0; k < (1 << BITS) - 1; ++k) idx += (y >= cb.t[k]) ? 1u : 0u;
  return idx;
}

// Pack 32 BITS-bit indices (local order) into BITS words, LSB-first stream.
template <int BITS>
__device__ __forceinline__ void pack32(const uint32_t (&idx)[32], uint32_t (&w)[BITS]) {
#pragma unroll
  for (int j = 0; j < BITS; ++j) w[j] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int p = BITS * i, wi = p >> 5, sh = p & 31;
    w[wi] |= idx[i] << sh;
    if (sh + BITS > 32) w[wi + 1] |= idx[i] >> (32 - sh);
  }
}


constexpr int kFragU4 = kFragElems * 2 / 16;  // u32x4 per pass = 2048

// The four instructions' A (or B) fragments of 32-coordinate block c, for each pass.
template <int P>
__device__ __forceinline__ void load_frags(const u32x4* lds, int c, int lane, u32x4 (&a)[P][4]) {
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int s = 0; s < 4; ++s) a[p][s] = lds[p * kFragU4 + (c * 4 + s) * 64 + lane];
}

// Raw input of one 16-vector tile held by a lane: 32 consecutive coordinates of one vector.
template <bool BF16IN>
struct RawTile;
template <>
struct RawTile<true> {
  u32x4 v[4];
};
template <>
struct RawTile<false> {
  f32x4 v[8];
};

template <bool BF16IN>
__device__ __forceinline__ void load_tile(const void* x, int64_t n, int64_t tile, int nl, int g,
                                          RawTile<BF16IN>& r) {
  const int64_t row = tile * 16 + nl;
  const int64_t lrow = row < n ? row : n - 1;
  if constexpr (BF16IN) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + lrow * 128 + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) r.v[s] = src[s];
  } else {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + lrow * 128 + 32 * g);
#pragma unroll
    for (int s = 0; s < 8; ++s) r.v[s] = src[s];
  }
}

}  // namespace
}  // namespace tq

#endif  // TQ_DEVICE_H_
