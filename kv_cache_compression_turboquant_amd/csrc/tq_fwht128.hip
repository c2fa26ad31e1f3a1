// TurboQuant_mse encode at d = 128 with the randomized Hadamard rotation done as a fast
// Walsh-Hadamard transform in registers ("TurboQuant 和 RotorQuant 的真相", chapter 3, the
// custom WHT kernel; "Sub-byte KV cache quantization with TurboQuant", engineering path: the
// transform as an O(d log d) butterfly rather than a d x d product).
//
// R = H diag(sigma) / sqrt(d) (or, for the block rotation, blockdiag(H_32) diag(sigma) / sqrt(32)),
// so y = R x takes a sign flip and the butterflies of H.  Four consecutive lanes hold one vector,
// lane u of the quad coordinates 32 u .. 32 u + 31:
//   * the sign flip is an XOR of the fp32 sign bits with the lane's 32 bits of sigma;
//   * butterfly stages over coordinate bits 0..4 run inside the lane's registers;
//   * stages over bits 5 and 6 (the full transform only) exchange registers with the partner
//     lane u ^ 1, then u ^ 2, through DPP quad permutes, the butterfly being one fma with +-1;
//   * the norm is the lane's sum of squares reduced over the quad the same way.
// The Hadamard output keeps the input's index order, so each lane then owns the rotated
// coordinates 32 u .. 32 u + 31: it quantizes them (sign-magnitude thresholds scaled by the norm,
// bits pushed into its words from the wave's decision masks, as the MFMA encode) and writes its
// BITS words of the packed row itself.  No LDS, no MFMA.
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kFwhtThreads = 256;  // 64 vectors per block

// Partner value in lane ^ 1 (CTRL 0xB1) or lane ^ 2 (CTRL 0x4E) of the quad.
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// w = 2 w + (this lane's bit of `lanes`): one v_addc with the lane mask as carry-in.
__device__ __forceinline__ uint32_t shift_in_w(uint32_t w, uint64_t lanes) {
  uint32_t r;
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(lanes));
  return r;
}

// v[i .. i + 7] += s * (the same registers of the partner lane u ^ 1 (STAGE 0) or u ^ 2 (STAGE 1)):
// one v_fmac_f32 with a DPP quad permute of its first operand each.  The s_nop gives the two wait
// states a DPP read of a VGPR needs after the VALU instruction that wrote it (the compiler does not
// see into the asm); inside the block each instruction reads registers written at least 8
// instructions earlier or before the block.
template <int STAGE>
__device__ __forceinline__ void pair_stage8(float (&v)[32], int i, float s) {
  if constexpr (STAGE == 0) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]), "+v"(v[i + 4]), "+v"(v[i + 5]),
          "+v"(v[i + 6]), "+v"(v[i + 7])
        : "v"(s));
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]), "+v"(v[i + 4]), "+v"(v[i + 5]),
          "+v"(v[i + 6]), "+v"(v[i + 7])
        : "v"(s));
  }
}

template <int BITS, bool BF16IN, bool FULL>
__global__ __launch_bounds__(kFwhtThreads) void k_encode_fwht_d128(const void* __restrict__ x, int64_t n,
                                                                   uint4 sigma, float rscale, CodebookArgs cb,
                                                                   uint32_t* __restrict__ idx_out,
                                                                   float* __restrict__ norms) {
  constexpr int H = 1 << (BITS - 1);
  const int lane = threadIdx.x & 63;
  const int u = lane & 3;
  const int64_t row = ((int64_t)blockIdx.x * kFwhtThreads + threadIdx.x) >> 2;
  const int64_t r = row < n ? row : n - 1;

  // the lane's 32 input coordinates
  float v[32];
  if constexpr (BF16IN) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + r * 128 + 32 * u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
  } else {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + r * 128 + 32 * u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 w = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = w[j];
    }
  }

  // norm over the quad
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) ss = fmaf(v[i], v[i], ss);
  ss += quad_swap<0xB1>(ss);
  ss += quad_swap<0x4E>(ss);
  const float nrm = sqrtf(ss);

  // sign flip: bit i of the lane's sigma word is 1 where sigma = -1
  const uint32_t sw = u == 0 ? sigma.x : u == 1 ? sigma.y : u == 2 ? sigma.z : sigma.w;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((sw >> i) & 1u) << 31));

  // butterflies over coordinate bits 0..4, inside the lane
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  if constexpr (FULL) {
    // bits 5 and 6: the partner lane holds the other half of each pair.  Each lane forms
    // own + s * partner (s = -1 in the upper lane of the pair: one fma whose DPP operand is the
    // partner), which is the upper output negated; the stage at bit 6 pairs lanes of equal sign,
    // so lanes u = 1 and 2 end with every coordinate negated and u = 0 and 3 with none.  Their
    // magnitudes are exact; the sign decision below undoes the negation.
    const float s1 = (u & 1) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 32; i += 8) pair_stage8<0>(v, i, s1);
    const float s2 = (u & 2) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 32; i += 8) pair_stage8<1>(v, i, s2);
  }
  // lanes whose coordinates are negated (FULL: u = 1, 2 of each quad), among the live vectors'
  // lanes: a zero vector's +-0 coordinates must all count as non-negative
  const uint64_t neg = FULL ? (0x6666666666666666ull & __builtin_amdgcn_ballot_w64(nrm > 0.f)) : 0ull;

  // Sign-magnitude decisions against the thresholds t_p * ||x|| / rscale (v is sqrt(g) times the
  // unit coordinate's scale): idx = (m ^ sgn) + K/2, m = #{p : |v| >= t_p}, so the top bit is
  // [v >= 0] and the low bits are m's bits XNOR [v >= 0]; m's bits come from a binary search over
  // the sorted thresholds, top first.  Each bit enters its word from the bottom (one v_addc with
  // the wave's decision mask as carry-in), coordinates in descending order.  A zero vector has
  // every threshold at +inf and its coordinates (+-0) count as non-negative: index K/2.
  const bool live = nrm > 0.f;
  const float tsc = nrm * rscale;
  float thr[H > 1 ? H - 1 : 1];
#pragma unroll
  for (int p = 0; p < H - 1; ++p) thr[p] = live ? __int_as_float(cb.tpos[p]) * tsc : INFINITY;
  uint32_t w[BITS];
#pragma unroll
  for (int b = 0; b < BITS; ++b) w[b] = 0u;
#pragma unroll
  for (int ii = 0; ii < 32; ++ii) {
    const int i = 31 - ii;
    const int P = BITS * i;
    const float y = v[i];
    const uint64_t pos = __builtin_amdgcn_ballot_w64(y >= 0.f) ^ neg;
    w[(P + BITS - 1) >> 5] = shift_in_w(w[(P + BITS - 1) >> 5], pos);
    const float a = fabsf(y);
    if constexpr (BITS == 2) {
      w[P >> 5] = shift_in_w(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= thr[0]) ^ pos));
    } else if constexpr (BITS == 3) {
      const bool hi = a >= thr[1];
      w[(P + 1) >> 5] = shift_in_w(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(hi) ^ pos));
      w[P >> 5] = shift_in_w(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= (hi ? thr[2] : thr[0])) ^ pos));
    } else if constexpr (BITS == 4) {
      const bool b2 = a >= thr[3];
      w[(P + 2) >> 5] = shift_in_w(w[(P + 2) >> 5], ~(__builtin_amdgcn_ballot_w64(b2) ^ pos));
      const bool b1 = a >= (b2 ? thr[5] : thr[1]);
      w[(P + 1) >> 5] = shift_in_w(w[(P + 1) >> 5], ~(__builtin_amdgcn_ballot_w64(b1) ^ pos));
      const float t0 = b2 ? (b1 ? thr[6] : thr[4]) : (b1 ? thr[2] : thr[0]);
      w[P >> 5] = shift_in_w(w[P >> 5], ~(__builtin_amdgcn_ballot_w64(a >= t0) ^ pos));
    }
  }
  if (row < n) {
    uint32_t* dst = idx_out + row * (4 * BITS) + BITS * u;
#pragma unroll
    for (int b = 0; b < BITS; ++b) dst[b] = w[b];
    if (u == 0) norms[row] = nrm;
  }
}

template <int BITS, bool BF16IN>
hipError_t fwht_launch(const void* x, int64_t n, bool full, uint4 sigma, float rscale, const CodebookArgs& cb,
                       uint32_t* idx, float* norms, hipStream_t st) {
  const int64_t blocks = (n * 4 + kFwhtThreads - 1) / kFwhtThreads;
  if (full)
    hipLaunchKernelGGL((k_encode_fwht_d128<BITS, BF16IN, true>), dim3((unsigned)blocks), dim3(kFwhtThreads), 0, st,
                       x, n, sigma, rscale, cb, idx, norms);
  else
    hipLaunchKernelGGL((k_encode_fwht_d128<BITS, BF16IN, false>), dim3((unsigned)blocks), dim3(kFwhtThreads), 0,
                       st, x, n, sigma, rscale, cb, idx, norms);
  return hipGetLastError();
}

template <int BITS>
hipError_t fwht_dispatch(const void* x, bool bf16, int64_t n, bool full, uint4 sigma, float rscale,
                         const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st) {
  return bf16 ? fwht_launch<BITS, true>(x, n, full, sigma, rscale, cb, idx, norms, st)
              : fwht_launch<BITS, false>(x, n, full, sigma, rscale, cb, idx, norms, st);
}

}  // namespace

hipError_t launch_encode_fwht_d128(const void* x, bool bf16, int64_t n, bool full, const uint32_t sigma_bits[4],
                                   float rscale, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                   hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n > ((int64_t)1 << 40)) return hipErrorInvalidValue;
  const uint4 sigma = make_uint4(sigma_bits[0], sigma_bits[1], sigma_bits[2], sigma_bits[3]);
  switch (cb.bits) {
    case 1: return fwht_dispatch<1>(x, bf16, n, full, sigma, rscale, cb, idx, norms, st);
    case 2: return fwht_dispatch<2>(x, bf16, n, full, sigma, rscale, cb, idx, norms, st);
    case 3: return fwht_dispatch<3>(x, bf16, n, full, sigma, rscale, cb, idx, norms, st);
    case 4: return fwht_dispatch<4>(x, bf16, n, full, sigma, rscale, cb, idx, norms, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
