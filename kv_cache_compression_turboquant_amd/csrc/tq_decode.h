// Decode-side helpers shared by the score, attention and search kernels: replicated LDS tables
// that turn packed indices into fp16 MFMA operands, and the transpose-reduce of 4-part results.
#ifndef TQ_DECODE_H_
#define TQ_DECODE_H_

#include "tq_device.h"

namespace tq {
namespace {

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
// remainders c - fp16(c) (read whole by decode_split_slot).
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

// Split-table operand with each entry's hi and lo values side by side in the contraction: the
// lane's decoded stream lists, field after field, the PER fp16 centroids of the field's
// coordinates, then their PER remainders; instruction j takes stream positions 8 j .. 8 j + 7,
// which are whole entries (PER <= 4) or half an entry (PER = 8), so the LDS reads land in the
// operand registers as they are.  SplitSlot gives the coordinate and half of a position; the
// other operand must follow the same order.
template <int BITS>
struct SplitSlot {
  static constexpr int PER = (BITS == 3 ? 6 : 8) / BITS;
  // local coordinate (0..31) and half (0: centroid, 1: remainder) of stream position p (0..63)
  __host__ __device__ static constexpr int coord(int p) { return (p / (2 * PER)) * PER + p % PER; }
  __host__ __device__ static constexpr int half(int p) { return (p / PER) & 1; }
};

template <int BITS, int COPIES, int N>
__device__ __forceinline__ u32x4 decode_split_slot(const uint32_t (&w)[N], int j, const uint8_t* tabl) {
  using DT = DecodeTable<BITS, true, COPIES>;
  constexpr int S = DT::STRIDE, F = DT::F, PER = DT::PER;
  if constexpr (PER == 4) {
    return *reinterpret_cast<const u32x4*>(tabl + get_bits(w, F * j, F) * S);
  } else if constexpr (PER == 2) {
    const uint32_t f = get_bits(w, 2 * F * j, 2 * F);
    const u32x2 a = *reinterpret_cast<const u32x2*>(tabl + (f & ((1u << F) - 1u)) * S);
    const u32x2 c = *reinterpret_cast<const u32x2*>(tabl + (f >> F) * S);
    return u32x4{a[0], a[1], c[0], c[1]};
  } else {
    return *reinterpret_cast<const u32x4*>(tabl + get_bits(w, F * (j >> 1), F) * S + 16 * (j & 1));
  }
}

// Keys: instruction s covers local coordinates 8 s .. 8 s + 7 of the lane's 32.
template <int BITS, int COPIES>
__device__ __forceinline__ u32x4 decode_keys(const uint32_t (&w)[BITS], int s, const uint8_t* tabl) {
  return decode8<BITS, COPIES>(w, 8 * BITS * s, tabl);
}

// decode_keys with the table's own base and the lane's copy offset laneoff = (lane % COPIES) *
// entry bytes kept apart: when the field stride is a power of two above laneoff, each address is
// base + (field * stride | laneoff), one shift and one and-or per lookup, with the base folded
// into the LDS instruction's offset.
template <int BITS, int COPIES>
__device__ __forceinline__ u32x4 decode_keys_or(const uint32_t (&w)[BITS], int s, const uint8_t* tab,
                                                uint32_t laneoff) {
  using DT = DecodeTable<BITS, false, COPIES>;
  constexpr uint32_t S = DT::STRIDE;
  if constexpr ((S & (S - 1)) != 0) {
    return decode8<BITS, COPIES>(w, 8 * BITS * s, tab + laneoff);
  } else {
    auto at = [&](uint32_t field) { return tab + ((field * S) | laneoff); };
    const int off = 8 * BITS * s;
    u32x4 out;
    if constexpr (BITS == 1) {
      out = *reinterpret_cast<const u32x4*>(at(get_bits(w, off, 8)));
    } else if constexpr (BITS == 2) {
      const uint32_t f = get_bits(w, off, 16);
      const u32x2 a = *reinterpret_cast<const u32x2*>(at(f & 0xffu));
      const u32x2 b = *reinterpret_cast<const u32x2*>(at(f >> 8));
      out = u32x4{a[0], a[1], b[0], b[1]};
    } else if constexpr (BITS == 3) {
      const uint32_t f = get_bits(w, off, 24);
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(at((f >> (6 * j)) & 63u));
    } else {
      const uint32_t f = get_bits(w, off, 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(at((f >> (8 * j)) & 0xffu));
    }
    return out;
  }
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

// Raw buffer resource over n bytes at p (untyped dword loads; the hardware range check returns
// zero for any load at or past n bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

template <int W>
__device__ __forceinline__ void buffer_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[W]) {
  if constexpr (W == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (W == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (W == 3) {
    typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else if constexpr (W == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    // wider runs in pieces of at most four words
    static_assert(W <= 8, "at most eight words");
    uint32_t lo[4], hi[W - 4];
    buffer_words<4>(r, off, lo);
    buffer_words<W - 4>(r, off + 16u, hi);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = lo[j];
#pragma unroll
    for (int j = 0; j < W - 4; ++j) w[4 + j] = hi[j];
  }
}

}  // namespace
}  // namespace tq

#endif  // TQ_DECODE_H_
