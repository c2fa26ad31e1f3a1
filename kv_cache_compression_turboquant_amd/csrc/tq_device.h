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

// Decode tables in LDS: a field of F packed bits (F = 6 for 3-bit indices, else 8) maps to the
// fp16 centroids of its F / BITS coordinates (SPLIT: followed by their fp16 remainders
// c - fp16(c)).  The table is stored COPIES times, interleaved entry by entry, and lane l reads
// copy l % COPIES: with COPIES = 128 / entry bytes, the lanes that one LDS cycle serves (128
// bytes) hit distinct banks whatever their fields.  Fewer copies trade conflicts for space.
template <int BITS, bool SPLIT, int COPIES>
struct DecodeTable {
  static constexpr int F = BITS == 3 ? 6 : 8;
  static constexpr int PER = F / BITS;                    // coordinates per field
  static constexpr int ENTRIES = 1 << F;
  static constexpr int EB = PER * 2 * (SPLIT ? 2 : 1);    // bytes per entry
  static constexpr int STRIDE = EB * COPIES;              // bytes between consecutive fields
  static constexpr int BYTES = ENTRIES * STRIDE;
  static constexpr int FIELDS = 8 / PER;                  // fields per instruction (8 coordinates)
  __device__ static const uint8_t* lane_base(const uint8_t* tab, int lane) { return tab + (lane % COPIES) * EB; }
};

// Copies of a table within an LDS budget: conflict-free (128 / entry bytes) if it fits.
template <int BITS, bool SPLIT, int BUDGET>
constexpr int table_copies() {
  constexpr int F = BITS == 3 ? 6 : 8;
  constexpr int EB = (F / BITS) * 2 * (SPLIT ? 2 : 1);
  constexpr int full = 128 / EB;
  constexpr int fit = BUDGET / ((1 << F) * EB);
  return full < fit ? full : (fit > 0 ? fit : 1);
}

// Bits [off, off + width) of a little-endian word array (off, width compile-time after unrolling).
template <int N>
__device__ __forceinline__ uint32_t get_bits(const uint32_t (&w)[N], int off, int width) {
  const int lo = off >> 5, sh = off & 31;
  uint32_t v = w[lo] >> sh;
  if (sh + width > 32 && lo + 1 < N) v |= w[lo + 1] << (32 - sh);
  return width == 32 ? v : (v & ((1u << width) - 1u));
}

// Eight consecutive BITS-bit indices starting at stream bit `off`, decoded to 8 fp16 values
// (one MFMA operand) through the lane's copy of the table (tabl = DecodeTable::lane_base).
template <int BITS, int COPIES, int N>
__device__ __forceinline__ u32x4 decode8(const uint32_t (&w)[N], int off, const uint8_t* tabl) {
  constexpr int S = DecodeTable<BITS, false, COPIES>::STRIDE;
  u32x4 out;
  if constexpr (BITS == 1) {
    out = *reinterpret_cast<const u32x4*>(tabl + get_bits(w, off, 8) * S);
  } else if constexpr (BITS == 2) {
    const uint32_t f = get_bits(w, off, 16);
    const u32x2 a = *reinterpret_cast<const u32x2*>(tabl + (f & 0xffu) * S);
    const u32x2 b = *reinterpret_cast<const u32x2*>(tabl + (f >> 8) * S);
    out = u32x4{a[0], a[1], b[0], b[1]};
  } else if constexpr (BITS == 3) {
    const uint32_t f = get_bits(w, off, 24);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(tabl + ((f >> (6 * j)) & 63u) * S);
  } else {
    const uint32_t f = get_bits(w, off, 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(tabl + ((f >> (8 * j)) & 0xffu) * S);
  }
  return out;
}

// Split-precision table: each entry holds the PER fp16 centroids followed by the PER fp16
// remainders c - fp16(c), so one read yields both B operands (hi, lo).
template <int BITS, int COPIES>
__device__ __forceinline__ void build_table2(uint8_t* tab, const float* cent32) {
  using DT = DecodeTable<BITS, true, COPIES>;
  for (int i = threadIdx.x; i < DT::ENTRIES * COPIES; i += blockDim.x) {
    const int e = i / COPIES;
    uint16_t* dst = reinterpret_cast<uint16_t*>(tab + i * DT::EB);
#pragma unroll
    for (int j = 0; j < DT::PER; ++j) {
      const float c = cent32[(e >> (BITS * j)) & ((1 << BITS) - 1)];
      const _Float16 hi = (_Float16)c;
      const _Float16 lo = (_Float16)(c - (float)hi);
      dst[j] = __builtin_bit_cast(uint16_t, hi);
      dst[DT::PER + j] = __builtin_bit_cast(uint16_t, lo);
    }
  }
}

// (hi and lo are read separately, each straight into its operand registers: reading an entry
// whole and splitting it costs register moves.)
template <int BITS, int COPIES, int N>
__device__ __forceinline__ void decode8_2(const uint32_t (&w)[N], int off, const uint8_t* tabl, u32x4& hi, u32x4& lo) {
  constexpr int S = DecodeTable<BITS, true, COPIES>::STRIDE;
  constexpr int H = DecodeTable<BITS, true, COPIES>::PER * 2;  // bytes of an entry's hi part
  if constexpr (BITS == 1) {
    const uint8_t* e = tabl + get_bits(w, off, 8) * S;
    hi = *reinterpret_cast<const u32x4*>(e);
    lo = *reinterpret_cast<const u32x4*>(e + H);
  } else if constexpr (BITS == 2) {
    const uint32_t f = get_bits(w, off, 16);
    const uint8_t* ea = tabl + (f & 0xffu) * S;
    const uint8_t* eb = tabl + (f >> 8) * S;
    const u32x2 ha = *reinterpret_cast<const u32x2*>(ea);
    const u32x2 hb = *reinterpret_cast<const u32x2*>(eb);
    const u32x2 la = *reinterpret_cast<const u32x2*>(ea + H);
    const u32x2 lb = *reinterpret_cast<const u32x2*>(eb + H);
    hi = u32x4{ha[0], ha[1], hb[0], hb[1]};
    lo = u32x4{la[0], la[1], lb[0], lb[1]};
  } else {
    const uint32_t f = get_bits(w, off, BITS == 3 ? 24 : 32);
    constexpr int FW = BITS == 3 ? 6 : 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* e = tabl + ((f >> (FW * j)) & ((1u << FW) - 1u)) * S;
      hi[j] = *reinterpret_cast<const uint32_t*>(e);
      lo[j] = *reinterpret_cast<const uint32_t*>(e + H);
    }
  }
}

// Keys: instruction s covers local coordinates 8 s .. 8 s + 7 of the lane's 32.
template <int BITS, int COPIES>
__device__ __forceinline__ u32x4 decode_keys(const uint32_t (&w)[BITS], int s, const uint8_t* tabl) {
  return decode8<BITS, COPIES>(w, 8 * BITS * s, tabl);
}

// Builds the replicated fp16 decode table of a codebook in LDS (cent: 16 fp16 centroids in LDS).
template <int BITS, int COPIES>
__device__ __forceinline__ void build_table(uint8_t* tab, const _Float16* cent) {
  using DT = DecodeTable<BITS, false, COPIES>;
  for (int i = threadIdx.x; i < DT::ENTRIES * COPIES; i += blockDim.x) {
    const int e = i / COPIES;
    uint16_t* dst = reinterpret_cast<uint16_t*>(tab + i * DT::EB);
#pragma unroll
    for (int j = 0; j < DT::PER; ++j)
      dst[j] = __builtin_bit_cast(uint16_t, cent[(e >> (BITS * j)) & ((1 << BITS) - 1)]);
  }
}


// Transpose-reduce of a 16 x 16 MFMA result whose rows are 4 parts x 4 heads: lane (n, g) holds
// row 4 g + r = (part g, head r) of column n in v[r].  Returns, in lane (n, g), the sum over the
// four parts of head g for column n.  The lane swaps exchange halves of the wave in registers
// (permlane32: lanes l and l ^ 32; permlane16: rows 2k and 2k + 1); each returns the pair
// {own, partner} ordered so that adding the two results needs no per-lane select.
__device__ __forceinline__ float reduce_parts(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  // g < 2: parts g and g + 2 of heads 0 / 1; g >= 2: parts g - 2 and g of heads 2 / 3
  const float k0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float k1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
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
