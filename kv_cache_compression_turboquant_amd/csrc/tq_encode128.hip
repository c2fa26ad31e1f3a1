// Fused TurboQuant encode at d = 128 (rows layout): norm, rotation on MFMA, bucketize, pack,
// and for TurboQuant_prod the QJL sign sketch of the residual with its norm.
#include "tq_device.h"

namespace tq {
namespace {

// ---------------------------------------------------------------------------------------
// Fused encode, d = 128.  One wave computes y^T = R x^T for NT tiles of 16 vectors:
// A = rotation fragments (LDS), B = x (registers, straight from HBM), D = y^T.  Lane (n, G)
// ends with coordinates 32 G .. 32 G + 31 of vector n, bucketizes them and writes BITS packed
// words (its aligned share of the row).  PROD runs a second product Z^T = S' R_res^T on the
// rotated-domain residual, whose B operand is exactly the lane's own registers.
// The fused path compares |y| against the positive thresholds (sign-magnitude form of the
// antisymmetric codebook); a value exactly on a threshold may go either way there, which the
// boundary-band rule allows.  The exact tie rule lives in k_quantize_rotated.
// The fragment loops are software pipelined: block c + 1's fragments are read from LDS while
// block c's MFMAs run; scheduling barriers keep the compiler from hoisting every read.
// ---------------------------------------------------------------------------------------

// MSE: 4 waves per block, two blocks per CU (<= 64 KB LDS each).  PROD keeps R and S' in LDS
// (up to 128 KB, one block per CU) and runs 8 waves per block instead.
template <bool PROD>
struct EncShape {
  static constexpr int kWaves = PROD ? 8 : 4;
  static constexpr int kBlocksPerCU = PROD ? 1 : 2;
};


template <int BITS, bool PROD, bool BF16IN, bool STORE_Y, int PASSES, int NT>
__global__ __launch_bounds__(EncShape<PROD>::kWaves * 64, EncShape<PROD>::kBlocksPerCU) void k_encode_d128(
    const void* __restrict__ x, int64_t n, const u32x4* __restrict__ frag_r,
    const u32x4* __restrict__ frag_s, float post_scale, CodebookArgs cb,
    uint32_t* __restrict__ idx_out, float* __restrict__ norms_out, uint32_t* __restrict__ qjl_out,
    float* __restrict__ rnorm_out, float* __restrict__ y_out) {
  constexpr int RP = PASSES;              // rotation passes held in LDS
  constexpr int SP = PROD ? 2 : 0;        // S' passes
  constexpr int kWaves = EncShape<PROD>::kWaves;
  constexpr int H = 1 << (BITS - 1);      // centroids per sign
  __shared__ u32x4 lds[(RP + SP) * kFragU4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int64_t ntiles = (n + 15) >> 4;
  const int64_t stride = (int64_t)gridDim.x * kWaves * NT;
  int64_t tw = ((int64_t)blockIdx.x * kWaves + wave) * NT;

  // Two tile groups in flight per wave, in two register sets used alternately (no copies, so
  // each wait covers exactly the group about to be used).  The first loads are issued before
  // the fragments are staged into LDS so that both latencies overlap.
  // (Loads past the end read the clamped last row: unconditional loads keep the register sets
  // fixed across iterations, where conditional ones would make the compiler copy them.)
  RawTile<BF16IN> bufA[NT], bufB[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, tw + t, nl, g, bufA[t]);
#pragma unroll
  for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, tw + stride + t, nl, g, bufB[t]);
  for (int i = threadIdx.x; i < RP * kFragU4; i += blockDim.x) lds[i] = frag_r[i];
  if constexpr (PROD) {
    for (int i = threadIdx.x; i < SP * kFragU4; i += blockDim.x) lds[RP * kFragU4 + i] = frag_s[i];
  }
  __syncthreads();
  if (tw >= ntiles) return;  // no barrier follows

  const float inv_post = 1.0f / post_scale;
  auto step = [&](RawTile<BF16IN> (&cur)[NT], const int64_t t0) {

    u32x4 bx[NT][4];      // bf16 x (or its hi part) for the 4 instructions
    u32x4 bxl[NT][4];     // bf16 low part of fp32 x
    float ss[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float acc2 = 0.f;
      if constexpr (BF16IN) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bx[t][s] = cur[t].v[s];
          // Copy to a plain array first: bit-casting an ext-vector element straight into the
          // dot2 operand miscompiles (every j reads element 0) with this compiler.
          uint32_t wv[4];
          __builtin_memcpy(wv, &cur[t].v[s], sizeof(wv));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x2 p = __builtin_bit_cast(bf16x2, wv[j]);
            acc2 = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc2, false);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x4 a = cur[t].v[2 * s], b = cur[t].v[2 * s + 1];
          const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
          u32x4 hi, lo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x2 pr = {v[2 * j], v[2 * j + 1]};
            const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
            const f32x2 rem = {v[2 * j] - __uint_as_float(h << 16), v[2 * j + 1] - __uint_as_float(h & 0xffff0000u)};
            hi[j] = h;
            lo[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
            acc2 = fmaf(v[2 * j], v[2 * j], acc2);
            acc2 = fmaf(v[2 * j + 1], v[2 * j + 1], acc2);
          }
          bx[t][s] = hi;
          bxl[t][s] = lo;
        }
      }
      ss[t] = acc2;
    }
    // the raw registers are free again: fetch the group two strides ahead into them
#pragma unroll
    for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, t0 + 2 * stride + t, nl, g, cur[t]);

    // y^T blocks: acc[t][c] holds rows 32 G + 4 c + r of tile t
    f32x4 acc[NT][8];
    {
      u32x4 cf[RP][4], nf[RP][4];
      load_frags<RP>(lds, 0, lane, cf);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + 1 < 8) load_frags<RP>(lds, c + 1, lane, nf);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            a = mfma_bf16(cf[0][s], bx[t][s], a);
            if constexpr (!BF16IN) a = mfma_bf16(cf[0][s], bxl[t][s], a);
            if constexpr (RP == 2) a = mfma_bf16(cf[1][s], bx[t][s], a);
          }
          acc[t][c] = a;
        }
        if (c + 1 < 8) {
#pragma unroll
          for (int p = 0; p < RP; ++p)
#pragma unroll
            for (int s = 0; s < 4; ++s) cf[p][s] = nf[p][s];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float sq = ss[t];
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      const float nrm = sqrtf(sq);
      const bool live = nrm > 0.f;
      const float scale = live ? post_scale / nrm : 0.f;   // raw product -> unit coordinate
      const int64_t row = (t0 + t) * 16 + nl;
      const bool valid = row < n;
      if (valid && g == 0 && norms_out) norms_out[row] = nrm;
      if constexpr (STORE_Y) {
        if (valid) {
          f32x4* dst = reinterpret_cast<f32x4*>(y_out + row * 128 + 32 * g);
#pragma unroll
          for (int c = 0; c < 8; ++c) dst[c] = acc[t][c] * scale;
        }
      } else {
        // Decisions on the raw product against per-vector thresholds t_p * ||x|| / post_scale
        // (the sign-magnitude form of the antisymmetric codebook): idx = (m ^ sign) + K/2 with
        // m = #{p : |y| >= t_p}.  A zero vector keeps every threshold at +inf (idx K/2).
        float thr[H > 1 ? H - 1 : 1];
        float mags[H];
        const float tsc = nrm * inv_post;
#pragma unroll
        for (int p = 0; p < H - 1; ++p) thr[p] = live ? __int_as_float(cb.tpos[p]) * tsc : INFINITY;
#pragma unroll
        for (int p = 0; p < H; ++p) mags[p] = live ? cb.cpos[p] : 0.f;
        uint32_t w[BITS];
#pragma unroll
        for (int j = 0; j < BITS; ++j) w[j] = 0;
        u32x4 rh[4], rl[4];
        float rs = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int rp = 0; rp < 2; ++rp) {
            float res[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float yv = acc[t][c][2 * rp + q];
              const float ay = fabsf(yv);
              uint32_t m = 0;
              float mag = mags[0];
#pragma unroll
              for (int p = 0; p < H - 1; ++p) {
                const bool ge = ay >= thr[p];
                m += ge ? 1u : 0u;
                if constexpr (PROD) mag = ge ? mags[p + 1] : mag;
              }
              const uint32_t sgn = (uint32_t)(__float_as_int(yv) >> 31);
              const uint32_t id = (m ^ sgn) + (uint32_t)H;
              if constexpr (PROD) {
                const float cv = __uint_as_float((__float_as_uint(mag) & 0x7fffffffu) | (__float_as_uint(yv) & 0x80000000u));
                res[q] = fmaf(yv, scale, -cv);
                rs = fmaf(res[q], res[q], rs);
              }
              const int li = 4 * c + 2 * rp + q;
              const int p = BITS * li, wi = p >> 5, sh = p & 31;
              w[wi] |= id << sh;
              if (sh + BITS > 32) w[wi + 1] |= id >> (32 - sh);
            }
            if constexpr (PROD) {
              const f32x2 pr = {res[0], res[1]};
              const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
              const f32x2 rem = {res[0] - __uint_as_float(h << 16), res[1] - __uint_as_float(h & 0xffff0000u)};
              rh[c >> 1][2 * (c & 1) + rp] = h;
              rl[c >> 1][2 * (c & 1) + rp] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
            }
          }
        if (valid) {
          uint32_t* dst = idx_out + row * (4 * BITS) + BITS * g;
#pragma unroll
          for (int j = 0; j < BITS; ++j) dst[j] = w[j];
        }
        if constexpr (PROD) {
          uint32_t bits = 0;
          const u32x4* sl = lds + RP * kFragU4;
          u32x4 cf[2][4], nf[2][4];
          load_frags<2>(sl, 0, lane, cf);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            if (c + 1 < 8) load_frags<2>(sl, c + 1, lane, nf);
            f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              z = mfma_bf16(cf[0][s], rh[s], z);
              z = mfma_bf16(cf[0][s], rl[s], z);
              z = mfma_bf16(cf[1][s], rh[s], z);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) bits |= (z[r] >= 0.f ? 1u : 0u) << (4 * c + r);
            if (c + 1 < 8) {
#pragma unroll
              for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int s = 0; s < 4; ++s) cf[p][s] = nf[p][s];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          rs += __shfl_xor(rs, 16);
          rs += __shfl_xor(rs, 32);
          if (valid) {
            qjl_out[row * 4 + g] = bits;
            if (g == 0) rnorm_out[row] = nrm * sqrtf(rs);
          }
        }
      }
    }
  };
  for (; tw < ntiles; tw += 2 * stride) {
    step(bufA, tw);
    if (tw + stride >= ntiles) break;
    step(bufB, tw + stride);
  }
}


template <int BITS, bool PROD, bool BF16IN, bool STORE_Y, int PASSES>
hipError_t enc_launch(const void* x, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                      const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits,
                      float* rnorms, float* y, hipStream_t st) {
  constexpr int NT = (PROD || !BF16IN) ? 1 : 2;
  constexpr int kWaves = EncShape<PROD>::kWaves;
  const int64_t ntiles = (n + 15) / 16;
  const int64_t per_block = (int64_t)kWaves * NT;
  int64_t blocks = (ntiles + per_block - 1) / per_block;
  const int64_t cap = (int64_t)num_cus() * EncShape<PROD>::kBlocksPerCU;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((k_encode_d128<BITS, PROD, BF16IN, STORE_Y, PASSES, NT>), dim3((unsigned)blocks),
                     dim3(kWaves * 64), 0, st, x, n,
                     reinterpret_cast<const u32x4*>(rot->frag_dev),
                     reinterpret_cast<const u32x4*>(qjl ? qjl->frag_dev : nullptr), rot->post_scale, cb, idx,
                     norms, qbits, rnorms, y);
  return hipGetLastError();
}

template <int BITS, bool PROD, bool STORE_Y>
hipError_t enc_dispatch_in(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                           const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                           uint32_t* qbits, float* rnorms, float* y, hipStream_t st) {
  if (bf16) {
    if (rot->passes == 1)
      return enc_launch<BITS, PROD, true, STORE_Y, 1>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, y, st);
    return enc_launch<BITS, PROD, true, STORE_Y, 2>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, y, st);
  }
  if (rot->passes == 1)
    return enc_launch<BITS, PROD, false, STORE_Y, 1>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, y, st);
  return enc_launch<BITS, PROD, false, STORE_Y, 2>(x, n, rot, qjl, cb, idx, norms, qbits, rnorms, y, st);
}

}  // namespace

hipError_t launch_encode_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                              const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx,
                              float* norms, uint32_t* qjl_bits, float* rnorms, float* y_out,
                              hipStream_t st) {
  if (y_out) return enc_dispatch_in<1, false, true>(x, bf16, n, rot, nullptr, cb, nullptr, norms, nullptr, nullptr, y_out, st);
  const bool prod = qjl != nullptr;
  switch (cb.bits) {
    case 1:
      return prod ? enc_dispatch_in<1, true, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st)
                  : enc_dispatch_in<1, false, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st);
    case 2:
      return prod ? enc_dispatch_in<2, true, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st)
                  : enc_dispatch_in<2, false, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st);
    case 3:
      return prod ? enc_dispatch_in<3, true, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st)
                  : enc_dispatch_in<3, false, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st);
    case 4:
      return prod ? enc_dispatch_in<4, true, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st)
                  : enc_dispatch_in<4, false, false>(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, nullptr, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
