// HIP kernels for gfx950 (MI355X): fused TurboQuant encode at d = 128, the reference
// quantizer, decode, the query prologue and the compressed-key score kernel.
//
// MFMA conventions (v_mfma_f32_16x16x32_{bf16,f16}): lane l = n + 16 g (n = l % 16,
// g = l / 16) holds A row n, B column n and D column n.  Within one instruction, element e of
// lane group g covers contraction slot 8 g + e for both A and B, and register r of D holds row
// 4 g + r.  Every contraction here is over vector coordinates, and the kernels assign
// coordinate 32 g + 8 s + e to element e of lane group g in instruction s (s = 0..3 for
// d = 128), identically for both operands, so each lane streams 32 consecutive coordinates.
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
constexpr int kFragU4 = kFragElems * 2 / 16;  // u32x4 per pass = 2048

// MSE: 4 waves per block, two blocks per CU (<= 64 KB LDS each).  PROD keeps R and S' in LDS
// (up to 128 KB, one block per CU) and runs 8 waves per block instead.
template <bool PROD>
struct EncShape {
  static constexpr int kWaves = PROD ? 8 : 4;
  static constexpr int kBlocksPerCU = PROD ? 1 : 2;
};

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
  for (int i = threadIdx.x; i < RP * kFragU4; i += blockDim.x) lds[i] = frag_r[i];
  if constexpr (PROD) {
    for (int i = threadIdx.x; i < SP * kFragU4; i += blockDim.x) lds[RP * kFragU4 + i] = frag_s[i];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int64_t ntiles = (n + 15) >> 4;
  const int64_t stride = (int64_t)gridDim.x * kWaves * NT;
  int64_t t0 = ((int64_t)blockIdx.x * kWaves + wave) * NT;
  if (t0 >= ntiles) return;  // no barrier follows

  const float inv_post = 1.0f / post_scale;
  RawTile<BF16IN> nxt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, t0 + t, nl, g, nxt[t]);

  for (; t0 < ntiles; t0 += stride) {
    RawTile<BF16IN> cur[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) cur[t] = nxt[t];
    if (t0 + stride < ntiles) {
#pragma unroll
      for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, t0 + stride + t, nl, g, nxt[t]);
    }

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
  }
}

int g_num_cus[64] = {0};

int num_cus() {
  int dev = 0;
  hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) return 256;
  if (!g_num_cus[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_num_cus[dev] = v;
  }
  return g_num_cus[dev];
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

// ---------------------------------------------------------------------------------------
// Reference quantizer: bucketize + pack fp32 rotated coordinates, one thread per
// (row, 32-coordinate group).
// ---------------------------------------------------------------------------------------
template <int BITS>
__global__ void k_quantize_rotated(const float* __restrict__ y, int64_t n, int d, CodebookArgs cb,
                                   uint32_t* __restrict__ out) {
  const int groups = d / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * groups) return;
  const int64_t row = i / groups;
  const int grp = (int)(i % groups);
  const f32x4* src = reinterpret_cast<const f32x4*>(y + row * d + 32 * grp);
  uint32_t idx[32];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f32x4 v = src[k];
#pragma unroll
    for (int j = 0; j < 4; ++j) idx[4 * k + j] = bucketize<BITS>(v[j], cb);
  }
  uint32_t w[BITS];
  pack32<BITS>(idx, w);
  uint32_t* dst = out + row * ((int64_t)d * BITS / 32) + BITS * grp;
#pragma unroll
  for (int j = 0; j < BITS; ++j) dst[j] = w[j];
}

// ---------------------------------------------------------------------------------------
// Decode: x_hat = s R^T C[idx] (+ gamma sqrt(pi/2)/d S^T z).  One block per row.
// ---------------------------------------------------------------------------------------
__global__ void k_decode(const uint32_t* __restrict__ idx, const float* __restrict__ norms,
                         const uint32_t* __restrict__ qbits, const float* __restrict__ rnorms, int d,
                         int bits, int blocked, CodebookArgs cb, const float* __restrict__ r32,
                         const float* __restrict__ s32, float* __restrict__ out) {
  extern __shared__ float sh[];  // [d] centroid values, [d] signs
  const int64_t row = blockIdx.x;
  const int words = d * bits / 32;
  const uint32_t* w = blocked ? idx + (row >> 5) * (int64_t)d * bits : idx + row * words;
  const int e32 = (int)(row & 31);
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    // stream bit of coordinate j: rows layout b*j; blocked: chunk (octet, j), row e within it
    const int p = blocked ? ((e32 >> 3) * d + j) * 8 * bits + bits * (e32 & 7) : j * bits;
    uint64_t win = w[p >> 5];
    if ((p & 31) + bits > 32) win |= (uint64_t)w[(p >> 5) + 1] << 32;
    const uint32_t id = (uint32_t)(win >> (p & 31)) & ((1u << bits) - 1u);
    sh[j] = cb.c[id];
    if (s32) sh[d + j] = ((qbits[row * (d / 32) + (j >> 5)] >> (j & 31)) & 1u) ? 1.f : -1.f;
  }
  __syncthreads();
  const float s = norms[row];
  const float gc = s32 ? rnorms[row] * kQjl / (float)d : 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float a = 0.f, b = 0.f;
    for (int j = 0; j < d; ++j) a += r32[(int64_t)j * d + i] * sh[j];
    if (s32)
      for (int j = 0; j < d; ++j) b += s32[(int64_t)j * d + i] * sh[d + j];
    out[row * d + i] = s * a + gc * b;
  }
}

// ---------------------------------------------------------------------------------------
// QJL sign bits as an fp16 MFMA operand without a table.  A lane's 32 sign bits z (coordinates
// 32 g + j at bit j) become 16 dwords: dword d holds the bits of coordinates d and 16 + d, taken
// in place at bit positions m and m + 16 of (d < 8 ? z << 8 : z), m = (d < 8 ? d + 8 : d), and
// OR-ed into a base pattern so that each half is the fp16 value alpha_m + beta_m * bit.  The
// query side carries q_s / beta_m in the same slot order, and the per-head constant
// K = sum_i q_s,i (1 + 2 alpha_i / beta_i) turns the product D into <q_s, 2 z - 1> = 2 D - K.
// ---------------------------------------------------------------------------------------
__device__ __constant__ float kSignAlpha[8] = {1.f, 1.f, 0.5f, 0.25f, 0.0625f, 0.00390625f, 0.f, 1.f};
__device__ __constant__ float kSignBeta[8] = {0.25f, 0.5f, 0.5f, 0.75f, 0.9375f, 0.99609375f, 2.f, -2.f};
__device__ __constant__ uint32_t kSignBase[8] = {0x3c003c00u, 0x3c003c00u, 0x38003800u, 0x34003400u,
                                                 0x2c002c00u, 0x1c001c00u, 0x00000000u, 0x3c003c00u};

// Slot order of the sign operand: element e of instruction s <-> local coordinate.
__host__ __device__ __forceinline__ int sign_slot_coord(int s, int e) { return (4 * s + (e >> 1)) + 16 * (e & 1); }
// Mask position index (m - 8) of dword d.
__host__ __device__ __forceinline__ int sign_slot_mpos(int d) { return d < 8 ? d : d - 8; }

__device__ __forceinline__ void sign_operand(uint32_t z, u32x4 (&bz)[4]) {
  const uint32_t zl = z << 8;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    const int m = d < 8 ? d + 8 : d;
    const uint32_t src = d < 8 ? zl : z;
    const uint32_t bases[8] = {0x3c003c00u, 0x3c003c00u, 0x38003800u, 0x34003400u,
                               0x2c002c00u, 0x1c001c00u, 0x00000000u, 0x3c003c00u};
    bz[d >> 2][d & 3] = (src & ((1u << m) | (1u << (m + 16)))) | bases[m - 8];
  }
}

// ---------------------------------------------------------------------------------------
// Query prologue, d = 128: for each (batch, kv head) block, q_rot = R q and q_s = S q of the
// heads sharing the kv head, written as fp16 hi/lo pairs: ws[(b*Hq + h)][part][128], part = 0
// rot hi, 1 rot lo, 2 sketch hi, 3 sketch lo.  Reads R^T / S^T so that thread j's loads of
// column j are coalesced.  The 128 contraction steps are split over eight thread groups of 16
// steps each, fully unrolled, so every load a thread needs is in flight at once (the kernel is
// latency-bound, not bandwidth-bound); the partial sums meet in LDS.
// ---------------------------------------------------------------------------------------
constexpr int kQprepParts = 8;
constexpr int kQprepThreads = 128 * kQprepParts;

__global__ __launch_bounds__(kQprepThreads) void k_qprep128(const float* __restrict__ q, int Hq, int ratio,
                                                            const float* __restrict__ rt,
                                                            const float* __restrict__ st,
                                                            uint16_t* __restrict__ ws,
                                                            float* __restrict__ kconst) {
  __shared__ float qs[4][128];
  __shared__ float part[2][kQprepParts][4][128];
  __shared__ float sum[2][4][128];
  const int Hkv = Hq / ratio;
  const int bg = blockIdx.x;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int h0 = kvh * ratio;
  const int j = threadIdx.x & 127, p = threadIdx.x >> 7;
  const int nmat = st ? 2 : 1;
  for (int hc = 0; hc < ratio; hc += 4) {
    const int nh = ratio - hc < 4 ? ratio - hc : 4;
    __syncthreads();
    if (threadIdx.x < 512) {
      const int hh = threadIdx.x >> 7;
      qs[hh][j] = hh < nh ? q[((int64_t)b * Hq + h0 + hc + hh) * 128 + j] : 0.f;
    }
    __syncthreads();
    const int k0 = p * (128 / kQprepParts);
    float rv[128 / kQprepParts], sv[128 / kQprepParts];
#pragma unroll
    for (int k = 0; k < 128 / kQprepParts; ++k) rv[k] = rt[(k0 + k) * 128 + j];
    if (st) {
#pragma unroll
      for (int k = 0; k < 128 / kQprepParts; ++k) sv[k] = st[(k0 + k) * 128 + j];
    }
    float ar[4] = {0.f, 0.f, 0.f, 0.f}, as[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 128 / kQprepParts; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = fmaf(rv[k], qs[i][k0 + k], ar[i]);
    if (st) {
#pragma unroll
      for (int k = 0; k < 128 / kQprepParts; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) as[i] = fmaf(sv[k], qs[i][k0 + k], as[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part[0][p][i][j] = ar[i];
      part[1][p][i][j] = as[i];
    }
    __syncthreads();
    // threads (m, j), m < nmat: the full sum of matrix m for the four heads
    if (threadIdx.x < 128 * nmat) {
      const int m = threadIdx.x >> 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = 0.f;
#pragma unroll
        for (int pp = 0; pp < kQprepParts; ++pp) a += part[m][pp][i][j];
        sum[m][i][j] = a;
      }
    }
    __syncthreads();
    if (threadIdx.x < 128 * nmat) {
      const int m = threadIdx.x >> 7;
      for (int i = 0; i < nh; ++i) {
        uint16_t* o = ws + ((int64_t)b * Hq + h0 + hc + i) * 4 * 128;
        float v;
        int mp = 0;
        if (m == 0) {
          v = sum[0][i][j];
        } else {
          // sketch in sign-slot order: output slot j = 32 G + 8 s + e  <-  coordinate
          // 32 G + c(s, e), scaled by 1 / beta
          const int G = j >> 5, s8 = (j & 31) >> 3, e = j & 7;
          const int c = 32 * G + sign_slot_coord(s8, e);
          mp = sign_slot_mpos(4 * s8 + (e >> 1));
          v = sum[1][i][c] / kSignBeta[mp];
        }
        const _Float16 vh = (_Float16)v;
        const _Float16 vl = (_Float16)(v - (float)vh);
        o[256 * m + j] = __builtin_bit_cast(uint16_t, vh);
        o[256 * m + 128 + j] = __builtin_bit_cast(uint16_t, vl);
      }
    }
    if (st && threadIdx.x < 64 * nh) {
      // per-head constant K = sum_i q_s,i (1 + 2 alpha_i / beta_i); wave i reduces head i
      const int i = threadIdx.x >> 6, l = threadIdx.x & 63;
      float acc = 0.f;
      for (int c = l; c < 128; c += 64) {
        const int jl = c & 31;                     // local coordinate within its group
        const int d = jl < 16 ? jl : jl - 16;      // dword holding it
        const int mp = sign_slot_mpos(d);
        acc += sum[1][i][c] * (1.f + 2.f * kSignAlpha[mp] / kSignBeta[mp]);
      }
      for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
      if (l == 0) kconst[(int64_t)b * Hq + h0 + hc + i] = acc;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Compressed-key score, d = 128.  Grid (key chunk, b * Hkv).  D = A B with A = query slots
// (16 rows: rot hi / rot lo / sketch hi / sketch lo for 4 heads), B = decoded keys (columns =
// 16 keys), so lane (n, G) receives the four partial sums of key n for slot group G.  Keys are
// decoded from whole packed words through small LDS tables that map a field of F bits to
// F / BITS fp16 centroids (F = 6 for 3 bits, else 8), built by each block in one pass.
// ---------------------------------------------------------------------------------------
constexpr int kScoreWaves = 4;
constexpr int kScoreBatch = 8;

template <int BITS>
struct DecodeTable {
  static constexpr int F = BITS == 3 ? 6 : 8;
  static constexpr int PER = F / BITS;             // coordinates per field
  static constexpr int ENTRIES = 1 << F;
  static constexpr int BYTES = ENTRIES * PER * 2;  // fp16 entries
  static constexpr int FIELDS = 8 / PER;           // fields per instruction (8 coordinates)
};

// Bits [off, off + width) of a little-endian word array (off, width compile-time after unrolling).
template <int N>
__device__ __forceinline__ uint32_t get_bits(const uint32_t (&w)[N], int off, int width) {
  const int lo = off >> 5, sh = off & 31;
  uint32_t v = w[lo] >> sh;
  if (sh + width > 32 && lo + 1 < N) v |= w[lo + 1] << (32 - sh);
  return width == 32 ? v : (v & ((1u << width) - 1u));
}

// Eight consecutive BITS-bit indices starting at stream bit `off`, decoded to 8 fp16 values
// (one MFMA operand) through the LDS table.
template <int BITS, int N>
__device__ __forceinline__ u32x4 decode8(const uint32_t (&w)[N], int off, const uint8_t* tab) {
  u32x4 out;
  if constexpr (BITS == 1) {
    out = *reinterpret_cast<const u32x4*>(tab + get_bits(w, off, 8) * 16);
  } else if constexpr (BITS == 2) {
    const uint32_t f = get_bits(w, off, 16);
    const u32x2 a = *reinterpret_cast<const u32x2*>(tab + (f & 0xffu) * 8);
    const u32x2 b = *reinterpret_cast<const u32x2*>(tab + (f >> 8) * 8);
    out = u32x4{a[0], a[1], b[0], b[1]};
  } else if constexpr (BITS == 3) {
    const uint32_t f = get_bits(w, off, 24);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(tab + ((f >> (6 * j)) & 63u) * 4);
  } else {
    const uint32_t f = get_bits(w, off, 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(tab + ((f >> (8 * j)) & 0xffu) * 4);
  }
  return out;
}

// Split-precision table: each entry holds the PER fp16 centroids followed by the PER fp16
// remainders c - fp16(c), so one read yields both B operands (hi, lo).
template <int BITS>
__device__ __forceinline__ void build_table2(uint8_t* tab, const float* cent32) {
  using DT = DecodeTable<BITS>;
  for (int e = threadIdx.x; e < DT::ENTRIES; e += blockDim.x) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(tab + e * DT::PER * 4);
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

template <int BITS, int N>
__device__ __forceinline__ void decode8_2(const uint32_t (&w)[N], int off, const uint8_t* tab, u32x4& hi, u32x4& lo) {
  if constexpr (BITS == 1) {
    const uint8_t* e = tab + get_bits(w, off, 8) * 32;
    hi = *reinterpret_cast<const u32x4*>(e);
    lo = *reinterpret_cast<const u32x4*>(e + 16);
  } else if constexpr (BITS == 2) {
    const uint32_t f = get_bits(w, off, 16);
    const u32x4 a = *reinterpret_cast<const u32x4*>(tab + (f & 0xffu) * 16);
    const u32x4 b = *reinterpret_cast<const u32x4*>(tab + (f >> 8) * 16);
    hi = u32x4{a[0], a[1], b[0], b[1]};
    lo = u32x4{a[2], a[3], b[2], b[3]};
  } else {
    const uint32_t f = get_bits(w, off, BITS == 3 ? 24 : 32);
    constexpr int FW = BITS == 3 ? 6 : 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2 e = *reinterpret_cast<const u32x2*>(tab + ((f >> (FW * j)) & ((1u << FW) - 1u)) * 8);
      hi[j] = e[0];
      lo[j] = e[1];
    }
  }
}

// Keys: instruction s covers local coordinates 8 s .. 8 s + 7 of the lane's 32.
template <int BITS>
__device__ __forceinline__ u32x4 decode_keys(const uint32_t (&w)[BITS], int s, const uint8_t* tab) {
  return decode8<BITS>(w, 8 * BITS * s, tab);
}

// Builds the fp16 decode table of a codebook in LDS (cent: 16 fp16 centroids in LDS).
template <int BITS>
__device__ __forceinline__ void build_table(uint8_t* tab, const _Float16* cent) {
  using DT = DecodeTable<BITS>;
  for (int e = threadIdx.x; e < DT::ENTRIES; e += blockDim.x) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(tab + e * DT::PER * 2);
#pragma unroll
    for (int j = 0; j < DT::PER; ++j)
      dst[j] = __builtin_bit_cast(uint16_t, cent[(e >> (BITS * j)) & ((1 << BITS) - 1)]);
  }
}

template <int BITS, bool PROD>
struct KeyTile {
  uint32_t w[BITS];
  float nrm;
  uint32_t zw;
  float gam;
};

// Lane (n, g) share of key tile `tile` of one sequence: its BITS words (coordinates 32 g ..),
// norm, and for prod its sign word and scaled residual norm.  Rows past T are clamped.
template <int BITS, bool PROD>
__device__ __forceinline__ void load_key_tile(const uint32_t* __restrict__ idx, const float* __restrict__ norms,
                                              const uint32_t* __restrict__ qbits, const float* __restrict__ rnorms,
                                              int64_t base_row, int64_t T, int64_t tile, int nl, int g,
                                              KeyTile<BITS, PROD>& k) {
  int64_t t = tile * 16 + nl;
  t = t < T ? t : T - 1;
  const int64_t row = base_row + t;
  const uint32_t* src = idx + row * (4 * BITS) + BITS * g;
#pragma unroll
  for (int j = 0; j < BITS; ++j) k.w[j] = src[j];
  k.nrm = norms[row];
  if constexpr (PROD) {
    k.zw = qbits[row * 4 + g];
    k.gam = rnorms[row] * (kQjl / 128.0f);
  } else {
    k.zw = 0;
    k.gam = 0.f;
  }
}

template <int BITS, bool PROD>
__global__ __launch_bounds__(kScoreWaves * 64) void k_scores_d128(
    const uint16_t* __restrict__ qws, const float* __restrict__ kconst, int Hq, int Hkv, int64_t T, int tiles_per_wave,
    const uint32_t* __restrict__ idx, const float* __restrict__ norms,
    const uint32_t* __restrict__ qbits, const float* __restrict__ rnorms, CodebookArgs cb,
    float* __restrict__ scores) {
  using DT = DecodeTable<BITS>;
  __shared__ __attribute__((aligned(16))) uint8_t tab[DT::BYTES];
  __shared__ _Float16 cent[16];
  if (threadIdx.x < 16) cent[threadIdx.x] = (_Float16)cb.c[threadIdx.x];
  __syncthreads();
  build_table<BITS>(tab, cent);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int ratio = Hq / Hkv;
  const int groups = (ratio + 3) / 4;
  const int64_t base_row = (int64_t)bg * T;
  const int64_t tile0 = ((int64_t)blockIdx.x * kScoreWaves + wave) * tiles_per_wave;
  const int64_t ntiles_seq = (T + 15) / 16;

  // A operands for head group 0 (kept in registers).
  auto load_a = [&](int hg, u32x4 (&am)[4], u32x4 (&aq)[4]) {
    const int slot = nl;             // A row
    const int hl = slot & 3;         // head within the group
    const int part = slot >> 2;      // 0 rot hi, 1 rot lo, 2 sketch hi, 3 sketch lo
    const int h = 4 * hg + hl;
    const bool live = h < ratio;
    const uint16_t* src = qws + (((int64_t)b * Hq + kvh * ratio + (live ? h : 0)) * 4 + part) * 128 + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(src + 8 * s);
      if (!live) v = u32x4{0u, 0u, 0u, 0u};
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      am[s] = part < 2 ? v : z;
      aq[s] = (PROD && part >= 2) ? v : z;
    }
  };
  u32x4 am0[4], aq0[4];
  load_a(0, am0, aq0);
  // sketch constant K of the lane's head (4 hg + g) after the reduction
  auto load_kc = [&](int hg) -> float {
    const int h = 4 * hg + g;
    return (PROD && h < ratio) ? kconst[(int64_t)b * Hq + kvh * ratio + h] : 0.f;
  };
  const float kc0 = load_kc(0);

  // Ping-pong over two tile buffers (no register copies), so the next tile's loads stay in flight
  // while the current one is scored and the wait before scoring counts only the older loads.
  auto score_tile = [&](const KeyTile<BITS, PROD>& cur, int64_t ti) {
    const int64_t tile = tile0 + ti;
    const int64_t t = tile * 16 + nl;
    const bool valid = t < T;
    const float nrm = cur.nrm;
    const float gam = cur.gam;
    u32x4 bk[4], bz[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) bk[s] = decode_keys<BITS>(cur.w, s, tab);
    if constexpr (PROD) sign_operand(cur.zw, bz);
    for (int hg = 0; hg < groups; ++hg) {
      u32x4 am[4], aq[4];
      if (hg == 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) { am[s] = am0[s]; aq[s] = aq0[s]; }
      } else {
        load_a(hg, am, aq);
      }
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc = mfma_f16(am[s], bk[s], acc);
        if constexpr (PROD) acc = mfma_f16(aq[s], bz[s], acc);
      }
      const float sc = g < 2 ? nrm : 2.f * gam;
      const float v0 = acc[0] * sc, v1 = acc[1] * sc, v2 = acc[2] * sc, v3 = acc[3] * sc;
      const bool lowg = g < 2;
      float k0 = lowg ? v0 : v2, k1 = lowg ? v1 : v3;
      const float s0 = lowg ? v2 : v0, s1 = lowg ? v3 : v1;
      k0 += __shfl_xor(s0, 32);
      k1 += __shfl_xor(s1, 32);
      const bool odd = g & 1;
      float mine = odd ? k1 : k0;
      const float other = odd ? k0 : k1;
      mine += __shfl_xor(other, 16);
      const int h = 4 * hg + g;
      if constexpr (PROD) mine -= gam * (hg == 0 ? kc0 : load_kc(hg));
      if (valid && h < ratio) scores[((int64_t)b * Hq + kvh * ratio + h) * T + t] = mine;
    }
  };
  // Batches of kScoreBatch tiles: every load of a batch is issued before any tile of it is
  // scored (straight-line code, so the waits are exact), and the batch's latency is paid once.
  int64_t last = tiles_per_wave;
  if (ntiles_seq - tile0 < last) last = ntiles_seq - tile0;
  for (int64_t tb = 0; tb < last; tb += kScoreBatch) {
    KeyTile<BITS, PROD> kt[kScoreBatch];
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u)
      load_key_tile<BITS, PROD>(idx, norms, qbits, rnorms, base_row, T, tile0 + tb + u, nl, g, kt[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u)
      if (tb + u < last) score_tile(kt[u], tb + u);
  }
}

template <int BITS, bool PROD>
hipError_t scores_launch(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                         const CodebookArgs& cb, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                         float* scores, void* ws, hipStream_t st) {
  const int ratio = Hq / Hkv;
  uint16_t* qws = static_cast<uint16_t*>(ws);
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  float* kconst = reinterpret_cast<float*>(static_cast<char*>(ws) + qbytes);
  hipLaunchKernelGGL(k_qprep128, dim3(B * Hkv), dim3(kQprepThreads), 0, st, q, Hq, ratio, rot->rt32_dev,
                     PROD ? qjl->st32_dev : nullptr, qws, kconst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = (T + 15) / 16;
  // enough blocks to fill the device about four times over
  const int64_t target = (int64_t)num_cus() * 4;
  const int64_t seqs = (int64_t)B * Hkv;
  int64_t tpw = (tiles * seqs + target * kScoreWaves - 1) / (target * kScoreWaves);
  tpw = (tpw + kScoreBatch - 1) / kScoreBatch * kScoreBatch;
  if (tpw < kScoreBatch) tpw = kScoreBatch;
  if (tpw > 64) tpw = 64;
  const int64_t chunks = (tiles + tpw * kScoreWaves - 1) / (tpw * kScoreWaves);
  hipLaunchKernelGGL((k_scores_d128<BITS, PROD>), dim3((unsigned)chunks, (unsigned)seqs), dim3(kScoreWaves * 64),
                     0, st, qws, kconst, Hq, Hkv, T, (int)tpw, K->idx, K->norms, PROD ? K->qjl : nullptr,
                     PROD ? K->rnorms : nullptr, cb, scores);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Token-blocked encode (the value-cache layout), d = 128, MSE.  The product is formed the
// other way round, D[token][coordinate] = x R^T (A = x, straight from HBM; B = R^T fragments in
// LDS), so lane (n, G) holds tokens 4 G .. 4 G + 3 of a 16-token tile at coordinates
// 8 n .. 8 n + 7.  Two tiles make one 32-token block; a chunk (8 tokens at one coordinate) is
// the lane's 4-token piece joined with the piece of lane (n, G ^ 1) after one exchange.
// ---------------------------------------------------------------------------------------
template <int BITS, bool BF16IN, int PASSES>
__global__ __launch_bounds__(256, 2) void k_encode_vblock_d128(
    const void* __restrict__ x, int64_t n, const u32x4* __restrict__ fragt, float post_scale,
    CodebookArgs cb, uint32_t* __restrict__ idx_out, float* __restrict__ norms_out) {
  constexpr int RP = PASSES;
  constexpr int H = 1 << (BITS - 1);
  constexpr int PB = 4 * BITS;              // bits of a 4-token piece
  __shared__ u32x4 lds[RP * kFragU4];
  for (int i = threadIdx.x; i < RP * kFragU4; i += blockDim.x) lds[i] = fragt[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int h = g & 1;
  const int64_t nblk = (n + 31) >> 5;
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t blk = (int64_t)blockIdx.x * 4 + wave;
  if (blk >= nblk) return;  // no barrier follows
  const float inv_post = 1.0f / post_scale;

  RawTile<BF16IN> nxt[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) load_tile<BF16IN>(x, n, 2 * blk + t, nl, g, nxt[t]);

  for (; blk < nblk; blk += stride) {
    RawTile<BF16IN> cur[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) cur[t] = nxt[t];
    if (blk + stride < nblk) {
#pragma unroll
      for (int t = 0; t < 2; ++t) load_tile<BF16IN>(x, n, 2 * (blk + stride) + t, nl, g, nxt[t]);
    }
    u32x4 ax[2][4], axl[2][4];
    float srow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float acc2 = 0.f;
      if constexpr (BF16IN) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ax[t][s] = cur[t].v[s];
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
            const uint32_t hh = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
            const f32x2 rem = {v[2 * j] - __uint_as_float(hh << 16), v[2 * j + 1] - __uint_as_float(hh & 0xffff0000u)};
            hi[j] = hh;
            lo[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
            acc2 = fmaf(v[2 * j], v[2 * j], acc2);
            acc2 = fmaf(v[2 * j + 1], v[2 * j + 1], acc2);
          }
          ax[t][s] = hi;
          axl[t][s] = lo;
        }
      }
      acc2 += __shfl_xor(acc2, 16);
      acc2 += __shfl_xor(acc2, 32);
      srow[t] = sqrtf(acc2);
      const int64_t row = (2 * blk + t) * 16 + nl;
      if (g == 0 && row < n) norms_out[row] = srow[t];
    }

    f32x4 acc[2][8];
    {
      u32x4 cf[RP][4], nf[RP][4];
      load_frags<RP>(lds, 0, lane, cf);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + 1 < 8) load_frags<RP>(lds, c + 1, lane, nf);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            a = mfma_bf16(ax[t][s], cf[0][s], a);
            if constexpr (!BF16IN) a = mfma_bf16(axl[t][s], cf[0][s], a);
            if constexpr (RP == 2) a = mfma_bf16(ax[t][s], cf[1][s], a);
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
    for (int t = 0; t < 2; ++t) {
      // per-token thresholds for the lane's tokens 4 G + r
      float thr[4][H > 1 ? H - 1 : 1];
      bool tok_ok[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sr = __shfl(srow[t], 4 * g + r);
        const bool live = sr > 0.f;
        tok_ok[r] = (2 * blk + t) * 16 + 4 * g + r < n;
#pragma unroll
        for (int p = 0; p < H - 1; ++p) thr[r][p] = live ? __int_as_float(cb.tpos[p]) * (sr * inv_post) : INFINITY;
      }
      uint32_t P[BITS];
#pragma unroll
      for (int j = 0; j < BITS; ++j) P[j] = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float yv = acc[t][c][r];
          const float ay = fabsf(yv);
          uint32_t m = 0;
#pragma unroll
          for (int p = 0; p < H - 1; ++p) m += (ay >= thr[r][p]) ? 1u : 0u;
          const uint32_t sgn = (uint32_t)(__float_as_int(yv) >> 31);
          const uint32_t id = tok_ok[r] ? (m ^ sgn) + (uint32_t)H : 0u;
          const int pos = PB * c + BITS * r, wi = pos >> 5, sh = pos & 31;
          P[wi] |= id << sh;
          if (sh + BITS > 32) P[wi + 1] |= id >> (32 - sh);
        }
      uint32_t Q[BITS];
#pragma unroll
      for (int j = 0; j < BITS; ++j) Q[j] = __shfl_xor(P[j], 16);
      uint32_t O[BITS];
#pragma unroll
      for (int j = 0; j < BITS; ++j) O[j] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // chunk for coordinate 8 n + 4 h + i: even-lane piece (tokens 0..3) | odd-lane piece << PB
        const uint32_t pe0 = get_bits(P, PB * i, PB), pe1 = get_bits(P, PB * (4 + i), PB);
        const uint32_t qe0 = get_bits(Q, PB * i, PB), qe1 = get_bits(Q, PB * (4 + i), PB);
        const uint32_t even = h ? qe1 : pe0;
        const uint32_t odd = h ? pe1 : qe0;
        const uint64_t chunk = (uint64_t)even | ((uint64_t)odd << PB);
        const int pos = 8 * BITS * i, wi = pos >> 5, sh = pos & 31;
        O[wi] |= (uint32_t)(chunk << sh);
        if (sh + 8 * BITS > 32) O[wi + 1] |= (uint32_t)(chunk >> (32 - sh));
      }
      const int o = 2 * t + (g >> 1);
      uint32_t* dst = idx_out + blk * (128 * BITS) + 32 * o * BITS + (2 * nl + h) * BITS;
#pragma unroll
      for (int j = 0; j < BITS; ++j) dst[j] = O[j];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Fused decode attention, d = 128.  Grid (split, b * Hkv), 4 waves per block.  Each wave walks
// 32-token steps (aligned to the value cache's 32-row blocks): keys are scored like the score
// kernel (lane (n, G) ends with head G's logit for key n), an online softmax keeps the running
// max and sum per head, the weights (times the value norms) go through a wave-private LDS strip
// to become the A operand (head rows, hi/lo fp16), and the value chunks decode straight into B
// fragments (8 tokens of one coordinate), so P V accumulates on MFMA in V's rotated domain.
// The block merges its waves and writes (max, sum, acc[128]) per head; k_attn_combine merges the
// splits and applies R_V^T.
// ---------------------------------------------------------------------------------------
constexpr int kAttnStepsPerBlock = 64;
constexpr int kAttnPart = 130;  // max, sum, 128 accumulators

// One 32-token step of a wave: the lane's key words and norms for both 16-token tiles, the
// value norms, and the value chunks of octet g at coordinates 8 n .. 8 n + 7.
template <int KB, int VB>
struct AttnStep {
  uint32_t kw[2][KB];
  float kn[2];
  float vn[2];
  uint32_t vw[2 * VB];
};

template <int KB, int VB>
__device__ __forceinline__ void load_attn_step(const uint32_t* __restrict__ kidx, const float* __restrict__ knorm,
                                               const uint32_t* __restrict__ vidx, const float* __restrict__ vnorm,
                                               int64_t nrows, int64_t blk, int nl, int g, AttnStep<KB, VB>& st) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int64_t r = blk * 32 + tt * 16 + nl;
    const int64_t rl = r < nrows ? r : nrows - 1;
    const uint32_t* src = kidx + rl * (4 * KB) + KB * g;
#pragma unroll
    for (int j = 0; j < KB; ++j) st.kw[tt][j] = src[j];
    st.kn[tt] = knorm[rl];
    st.vn[tt] = vnorm[rl];
  }
  const uint32_t* vs = vidx + blk * (128 * VB) + 32 * g * VB + 2 * nl * VB;
#pragma unroll
  for (int j = 0; j < 2 * VB; ++j) st.vw[j] = vs[j];
}

template <int KB, int VB>
__global__ __launch_bounds__(256) void k_attn_d128(
    const uint16_t* __restrict__ qws, int Hq, int Hkv, int64_t T, int nsplit,
    const uint32_t* __restrict__ kidx, const float* __restrict__ knorm,
    const uint32_t* __restrict__ vidx, const float* __restrict__ vnorm, int64_t nrows,
    CodebookArgs cbk, CodebookArgs cbv, float scale, float* __restrict__ part) {
  using DK = DecodeTable<KB>;
  using DV = DecodeTable<VB>;
  __shared__ __attribute__((aligned(16))) uint8_t ktab[2 * DK::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vtab[DV::BYTES];
  __shared__ float kcent[16];
  __shared__ _Float16 vcent[16];
  __shared__ __attribute__((aligned(16))) float wl[4][4][32];
  __shared__ float mm[4][4], ll[4][4];
  __shared__ float accs[4][4][128];
  if (threadIdx.x < 16) {
    kcent[threadIdx.x] = cbk.c[threadIdx.x];
    vcent[threadIdx.x] = (_Float16)cbv.c[threadIdx.x];
  }
  __syncthreads();
  build_table2<KB>(ktab, kcent);
  build_table<VB>(vtab, vcent);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int ratio = Hq / Hkv;
  const int64_t row0 = (int64_t)bh * T, rowE = row0 + T;
  const int64_t blk_first = row0 >> 5, blk_end = ((rowE - 1) >> 5) + 1;
  const int64_t bb = blk_first + (int64_t)blockIdx.x * kAttnStepsPerBlock;
  const int64_t be = bb + kAttnStepsPerBlock < blk_end ? bb + kAttnStepsPerBlock : blk_end;
  const int64_t cnt = be > bb ? be - bb : 0;
  const int64_t per = (cnt + 3) / 4;
  const int64_t wb = bb + wave * per;
  const int64_t we = wb + per < be ? wb + per : be;

  // query slots against the centroids' fp16 part (am): rows 0-3 rotated-query hi (heads),
  // 4-7 lo; against the centroid remainders (am2): rows 8-11 hi.  Other rows zero.
  u32x4 am[4], am2[4];
  {
    const int hl = nl & 3, prt = nl >> 2;
    const bool live = hl < ratio && prt < 3;
    const int src_part = prt == 1 ? 1 : 0;
    const uint16_t* src = qws + (((int64_t)b * Hq + kvh * ratio + (hl < ratio ? hl : 0)) * 4 + src_part) * 128 + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + 8 * s);
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      am[s] = (live && prt < 2) ? v : z;
      am2[s] = (live && prt == 2) ? v : z;
    }
  }

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads of the next 32-token step are issued before the current step is consumed.
  AttnStep<KB, VB> cur, nxt;
  if (wb < we) load_attn_step<KB, VB>(kidx, knorm, vidx, vnorm, nrows, wb, nl, g, cur);
  for (int64_t blk = wb; blk < we; ++blk) {
    if (blk + 1 < we) load_attn_step<KB, VB>(kidx, knorm, vidx, vnorm, nrows, blk + 1, nl, g, nxt);
    float lg[2], svv[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t r = blk * 32 + tt * 16 + nl;
      const bool valid = r >= row0 && r < rowE;
      const float sk = cur.kn[tt];
      svv[tt] = cur.vn[tt];
      f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 khi, klo;
        decode8_2<KB>(cur.kw[tt], 8 * KB * s, ktab, khi, klo);
        d = mfma_f16(am[s], khi, d);
        d = mfma_f16(am2[s], klo, d);
      }
      const float sc = sk;
      const float v0 = d[0] * sc, v1 = d[1] * sc, v2 = d[2] * sc, v3 = d[3] * sc;
      const bool lowg = g < 2;
      float k0 = lowg ? v0 : v2, k1 = lowg ? v1 : v3;
      const float s0 = lowg ? v2 : v0, s1 = lowg ? v3 : v1;
      k0 += __shfl_xor(s0, 32);
      k1 += __shfl_xor(s1, 32);
      const bool odd = g & 1;
      float mine = odd ? k1 : k0;
      mine += __shfl_xor(odd ? k0 : k1, 16);
      lg[tt] = (valid && g < ratio) ? mine * scale : -INFINITY;
    }
    // online softmax for head g
    float mx = fmaxf(lg[0], lg[1]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
    const float w0 = lg[0] == -INFINITY ? 0.f : __expf(lg[0] - m_new);
    const float w1 = lg[1] == -INFINITY ? 0.f : __expf(lg[1] - m_new);
    l_part = fmaf(l_part, alpha, w0 + w1);
    m_run = m_new;
    wl[wave][g][nl] = w0 * svv[0];
    wl[wave][g][16 + nl] = w1 * svv[1];
    if (__any(alpha < 1.f)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 16 * r);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c][r] *= ar;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // A operand: rows 0-3 weight hi per head, 4-7 weight lo, 8-15 zero; tokens 8 g .. 8 g + 7
    u32x4 aw;
    {
      const int hm = nl & 3, prt = nl >> 2;
      const f32x4 a = *reinterpret_cast<const f32x4*>(&wl[wave][hm][8 * g]);
      const f32x4 c2 = *reinterpret_cast<const f32x4*>(&wl[wave][hm][8 * g + 4]);
      const float v[8] = {a[0], a[1], a[2], a[3], c2[0], c2[1], c2[2], c2[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 h0 = (_Float16)v[2 * j], h1 = (_Float16)v[2 * j + 1];
        const _Float16 l0 = (_Float16)(v[2 * j] - (float)h0), l1 = (_Float16)(v[2 * j + 1] - (float)h1);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        aw[j] = prt == 0 ? hi : (prt == 1 ? lo : 0u);
      }
    }
    // B operand: the value chunks of octet g at coordinates 8 n .. 8 n + 7
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = mfma_f16(aw, decode8<VB>(cur.vw, 8 * VB * c, vtab), acc[c]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
  }

  // wave totals: sum over the 16 keys lanes; hi + lo accumulator rows
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) l_part += __shfl_xor(l_part, o);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[c][r] + __shfl_xor(acc[c][r], 16);
      if (g == 0) accs[wave][r][8 * nl + c] = v;
    }
  if (nl == 0) {
    mm[wave][g] = m_run;
    ll[wave][g] = l_part;
  }
  __syncthreads();
  float* out = part + ((int64_t)bh * nsplit + blockIdx.x) * 4 * kAttnPart;
  for (int i = threadIdx.x; i < 4 * 128; i += blockDim.x) {
    const int hh = i >> 7, c = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, mm[wv][hh]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        if (mm[wv][hh] == -INFINITY) continue;
        const float e = __expf(mm[wv][hh] - M);
        L = fmaf(ll[wv][hh], e, L);
        A = fmaf(accs[wv][hh][c], e, A);
      }
    }
    out[hh * kAttnPart + 2 + c] = A;
    if (c == 0) {
      out[hh * kAttnPart] = M;
      out[hh * kAttnPart + 1] = L;
    }
  }
}

// Merges the splits of one query head and maps back from V's rotated domain: out = R_V^T acc / L.
// 512 threads = 4 groups of 128 columns; the groups take every fourth split, then every fourth
// quarter of the R_V^T product, so each thread's loads are independent and issued together.
constexpr int kCombineThreads = 512;

__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(const float* __restrict__ part, int Hq, int Hkv,
                                                                  int nsplit, const float* __restrict__ r32v,
                                                                  float* __restrict__ out) {
  __shared__ float red[4][128];
  __shared__ float lred[4];
  __shared__ float wmax[kCombineThreads / 64];
  __shared__ float o[128];
  const int hg = blockIdx.x;
  const int b = hg / Hq, h = hg % Hq;
  const int ratio = Hq / Hkv;
  const int bh = b * Hkv + h / ratio, hl = h % ratio;
  const int t = threadIdx.x, c = t & 127, pp = t >> 7;
  const int64_t xs = 4 * kAttnPart;  // floats between consecutive splits of one head
  const float* p = part + (int64_t)bh * nsplit * xs + hl * kAttnPart;
  float M = -INFINITY;
  for (int x = t; x < nsplit; x += kCombineThreads) M = fmaxf(M, p[x * xs]);
  for (int s = 32; s > 0; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  if ((t & 63) == 0) wmax[t >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) M = fmaxf(M, wmax[w]);
  float L = 0.f, A = 0.f;
#pragma unroll 4
  for (int x = pp; x < nsplit; x += 4) {
    const float mx = p[x * xs];
    const float l = p[x * xs + 1];
    const float a = p[x * xs + 2 + c];
    if (mx != -INFINITY) {
      const float e = __expf(mx - M);
      L = fmaf(l, e, L);
      A = fmaf(a, e, A);
    }
  }
  red[pp][c] = A;
  if (c == 0) lred[pp] = L;
  __syncthreads();
  if (t < 128) {
    const float a = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
    const float l = (lred[0] + lred[1]) + (lred[2] + lred[3]);
    o[t] = l > 0.f ? a / l : 0.f;
  }
  __syncthreads();
  float y = 0.f;
#pragma unroll
  for (int j = 32 * pp; j < 32 * pp + 32; ++j) y = fmaf(r32v[j * 128 + c], o[j], y);
  red[pp][c] = y;
  __syncthreads();
  if (t < 128) out[(int64_t)hg * 128 + t] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
}

template <int KB, int VB>
hipError_t attn_launch(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                       const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                       const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale, float* out,
                       void* ws, hipStream_t st) {
  const int ratio = Hq / Hkv;
  uint16_t* qws = static_cast<uint16_t*>(ws);
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + qbytes);
  hipLaunchKernelGGL(k_qprep128, dim3(B * Hkv), dim3(kQprepThreads), 0, st, q, Hq, ratio, rot_k->rt32_dev, nullptr, qws,
                     nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t steps = T / 32 + 2;
  const int nsplit = (int)((steps + kAttnStepsPerBlock - 1) / kAttnStepsPerBlock);
  hipLaunchKernelGGL((k_attn_d128<KB, VB>), dim3(nsplit, B * Hkv), dim3(256), 0, st, qws, Hq, Hkv, T, nsplit,
                     K->idx, K->norms, V->idx, V->norms, K->n, cbk, cbv, scale, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(B * Hq), dim3(kCombineThreads), 0, st, part, Hq, Hkv, nsplit, rot_v->r32_dev, out);
  return hipGetLastError();
}

template <int BITS, bool BF16IN, int PASSES>
hipError_t vblock_launch(const void* x, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                         uint32_t* idx, float* norms, hipStream_t st) {
  const int64_t nblk = (n + 31) / 32;
  int64_t blocks = (nblk + 3) / 4;
  const int64_t cap = (int64_t)num_cus() * 2;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((k_encode_vblock_d128<BITS, BF16IN, PASSES>), dim3((unsigned)blocks), dim3(256), 0, st, x, n,
                     reinterpret_cast<const u32x4*>(rot->fragt_dev), rot->post_scale, cb, idx, norms);
  return hipGetLastError();
}

template <int BITS>
hipError_t vblock_dispatch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                           const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st) {
  if (bf16) return rot->passes == 1 ? vblock_launch<BITS, true, 1>(x, n, rot, cb, idx, norms, st)
                                    : vblock_launch<BITS, true, 2>(x, n, rot, cb, idx, norms, st);
  return rot->passes == 1 ? vblock_launch<BITS, false, 1>(x, n, rot, cb, idx, norms, st)
                          : vblock_launch<BITS, false, 2>(x, n, rot, cb, idx, norms, st);
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

hipError_t launch_quantize_rotated(const float* y, int64_t n, int d, const CodebookArgs& cb,
                                   uint32_t* idx, hipStream_t st) {
  const int64_t work = n * (d / 32);
  const int threads = 256;
  const dim3 grid((unsigned)((work + threads - 1) / threads));
  switch (cb.bits) {
    case 1: hipLaunchKernelGGL(k_quantize_rotated<1>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    case 2: hipLaunchKernelGGL(k_quantize_rotated<2>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    case 3: hipLaunchKernelGGL(k_quantize_rotated<3>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    case 4: hipLaunchKernelGGL(k_quantize_rotated<4>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const tq_packed* p, const CodebookArgs& cb, const tq_rotation_s* rot,
                         const tq_qjl_s* qjl, float* xhat, hipStream_t st) {
  const int d = p->d;
  const int threads = d < 256 ? d : 256;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)p->n), dim3(threads), 2 * d * sizeof(float), st, p->idx, p->norms,
                     qjl ? p->qjl : nullptr, qjl ? p->rnorms : nullptr, d, p->bits,
                     p->layout == TQ_LAYOUT_TOKEN_BLOCKED ? 1 : 0, cb, rot->r32_dev,
                     qjl ? qjl->s32_dev : nullptr, xhat);
  return hipGetLastError();
}

hipError_t launch_encode_vblock_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                     const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st) {
  switch (cb.bits) {
    case 1: return vblock_dispatch<1>(x, bf16, n, rot, cb, idx, norms, st);
    case 2: return vblock_dispatch<2>(x, bf16, n, rot, cb, idx, norms, st);
    case 3: return vblock_dispatch<3>(x, bf16, n, rot, cb, idx, norms, st);
    case 4: return vblock_dispatch<4>(x, bf16, n, rot, cb, idx, norms, st);
  }
  return hipErrorInvalidValue;
}

size_t decode_attn_workspace_bytes(int B, int Hq, int Hkv, int64_t T, int d) {
  (void)d;
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  const int64_t steps = T / 32 + 2;
  const int64_t nsplit = (steps + kAttnStepsPerBlock - 1) / kAttnStepsPerBlock;
  return qbytes + (size_t)B * Hkv * nsplit * 4 * kAttnPart * sizeof(float);
}

hipError_t launch_decode_attn(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                              const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                              const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale,
                              float* out, void* ws, hipStream_t st) {
#define TQ_ATTN(KB, VB) \
  if (cbk.bits == KB && cbv.bits == VB) return attn_launch<KB, VB>(q, B, Hq, Hkv, T, K, V, cbk, cbv, rot_k, rot_v, scale, out, ws, st);
  TQ_ATTN(2, 2) TQ_ATTN(4, 4) TQ_ATTN(3, 3) TQ_ATTN(4, 2) TQ_ATTN(2, 4) TQ_ATTN(3, 2) TQ_ATTN(4, 3)
  TQ_ATTN(1, 1) TQ_ATTN(2, 3) TQ_ATTN(3, 4)
#undef TQ_ATTN
  return hipErrorInvalidValue;
}

size_t scores_workspace_bytes(int B, int Hq, int d) {
  (void)d;
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  return qbytes + (size_t)B * Hq * sizeof(float);
}

hipError_t launch_scores(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                         const CodebookArgs& cb, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                         float* scores, void* ws, hipStream_t st) {
  const bool prod = K->mode == TQ_MODE_PROD;
  switch (cb.bits) {
    case 1: return prod ? scores_launch<1, true>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st)
                        : scores_launch<1, false>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st);
    case 2: return prod ? scores_launch<2, true>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st)
                        : scores_launch<2, false>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st);
    case 3: return prod ? scores_launch<3, true>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st)
                        : scores_launch<3, false>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st);
    case 4: return prod ? scores_launch<4, true>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st)
                        : scores_launch<4, false>(q, B, Hq, Hkv, T, K, cb, rot, qjl, scores, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
