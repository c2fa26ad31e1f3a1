// Fused TurboQuant encode at d = 128 (rows layout): norm, rotation on MFMA, bucketize, pack,
// and for TurboQuant_prod the QJL sign sketch of the residual with its norm.
#include <hip/hip_ext.h>

#include <type_traits>

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
    float* __restrict__ rnorm_out, float* __restrict__ y_out, int y_raw) {
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
  // each wait covers exactly the group about to be used).  (Loads past the end read the
  // clamped last row: unconditional loads keep the register sets fixed across iterations, where
  // conditional ones would make the compiler copy them.)
  // All fragment loads are issued first, then the first tile loads, so the fragments' waits do
  // not cover the tiles, which stay in flight while the fragments are written to LDS.  (A
  // load-wait-store loop would wait out one memory latency per fragment, behind the tiles.)
  constexpr int kThreads = kWaves * 64;
  constexpr int kTotal = (RP + SP) * kFragU4;
  constexpr int kStage = (kTotal + kThreads - 1) / kThreads;
  u32x4 stage[kStage];
  // Blocks start at different slices (rotated by block index): every block reads the same
  // fragments, and in lockstep they would all queue on one L2 channel at a time.
  const int rot0 = (int)(blockIdx.x % kStage);
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int jr = j + rot0 < kStage ? j + rot0 : j + rot0 - kStage;
    const int i = threadIdx.x + jr * kThreads;
    if (kTotal % kThreads == 0 || i < kTotal) stage[j] = i < RP * kFragU4 ? frag_r[i] : frag_s[i - RP * kFragU4];
  }
  RawTile<BF16IN> bufA[NT], bufB[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, tw + t, nl, g, bufA[t]);
#pragma unroll
  for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, tw + stride + t, nl, g, bufB[t]);
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int jr = j + rot0 < kStage ? j + rot0 : j + rot0 - kStage;
    const int i = threadIdx.x + jr * kThreads;
    if (kTotal % kThreads == 0 || i < kTotal) lds[i] = stage[j];
  }
  __syncthreads();

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
        // y_raw: the product itself (R x), else the unit-scale coordinates (R x / ||x||)
        const float ys = y_raw ? post_scale : scale;
        if (valid) {
          f32x4* dst = reinterpret_cast<f32x4*>(y_out + row * 128 + 32 * g);
#pragma unroll
          for (int c = 0; c < 8; ++c) dst[c] = acc[t][c] * ys;
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
  // The loop is entered unconditionally: an early exit here would let the compiler sink the tile
  // loads above past the barrier.  A wave without a tile of its own (only in the last block)
  // makes one pass over clamped rows and stores nothing, since every store checks its row.
  for (;;) {
    step(bufA, tw);
    if (tw + stride >= ntiles) break;
    step(bufB, tw + stride);
    tw += 2 * stride;
    if (tw >= ntiles) break;
  }
}


// ---------------------------------------------------------------------------------------
// MSE encode, d = 128, with the quantizer interleaved into the rotation.  Block c's MFMAs give
// each lane 4 coordinates of each of its vectors (rows 32 G + 4 c + r); those are bucketized and
// packed while the next block's MFMAs run, so only two blocks of results are live at a time.
//
// Packing by shift-in: the blocks run from c = 7 down to 0, so the lane's coordinates come in
// descending order and so do their stream bits (bit j of coordinate i is stream bit b i + j).
// Each bit then enters its word from the bottom, w = 2 w + bit, which is one v_addc with the
// bit as a lane mask: no shifts, selects or ORs per field.
// The index of y is (m ^ sgn) + K/2 with m = #{p : |y| >= t_p} (the sign-magnitude form of the
// antisymmetric codebook), so its top bit is [y >= 0] and its low bits are the bits of m, each
// XNOR-ed with [y >= 0] (a scalar op on the lane masks).  m comes from a binary search over the
// sorted positive thresholds: its bits are produced top first, exactly in push order.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t push_bit(uint32_t w, uint64_t lanes) {
  uint32_t r;
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(lanes));
  return r;
}

template <int BITS>
struct Thr {
  float t[BITS > 1 ? (1 << (BITS - 1)) - 1 : 1];
};

// Push the BITS index bits of lane-local coordinate LI (top bit first) for every tile.  Each
// step is issued for all tiles before the next one, so that the dependent steps of one tile
// (compare -> lane-mask op -> push) are separated by the independent work of the others.
template <int BITS, int LI, int NT>
__device__ __forceinline__ void push_index(const f32x4 (&v)[NT], const Thr<BITS> (&th)[NT], uint32_t (&w)[NT][BITS]) {
  constexpr int P = BITS * LI;  // stream bit of the index's bit 0
  constexpr int R = LI & 3;     // register of the block holding coordinate LI
  float a[NT];
  uint64_t pos[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    a[t] = fabsf(v[t][R]);
    pos[t] = __builtin_amdgcn_ballot_w64(v[t][R] >= 0.f);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) w[t][(P + BITS - 1) >> 5] = push_bit(w[t][(P + BITS - 1) >> 5], pos[t]);
  if constexpr (BITS == 2) {
    uint64_t b0[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) b0[t] = __builtin_amdgcn_ballot_w64(a[t] >= th[t].t[0]);
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t][P >> 5] = push_bit(w[t][P >> 5], ~(b0[t] ^ pos[t]));
  } else if constexpr (BITS == 3) {
    bool hi[NT];
    uint64_t b1[NT], b0[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      hi[t] = a[t] >= th[t].t[1];
      b1[t] = __builtin_amdgcn_ballot_w64(hi[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t][(P + 1) >> 5] = push_bit(w[t][(P + 1) >> 5], ~(b1[t] ^ pos[t]));
#pragma unroll
    for (int t = 0; t < NT; ++t) b0[t] = __builtin_amdgcn_ballot_w64(a[t] >= (hi[t] ? th[t].t[2] : th[t].t[0]));
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t][P >> 5] = push_bit(w[t][P >> 5], ~(b0[t] ^ pos[t]));
  } else if constexpr (BITS == 4) {
    bool h2[NT], h1[NT];
    uint64_t b2[NT], b1[NT], b0[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      h2[t] = a[t] >= th[t].t[3];
      b2[t] = __builtin_amdgcn_ballot_w64(h2[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t][(P + 2) >> 5] = push_bit(w[t][(P + 2) >> 5], ~(b2[t] ^ pos[t]));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      h1[t] = a[t] >= (h2[t] ? th[t].t[5] : th[t].t[1]);
      b1[t] = __builtin_amdgcn_ballot_w64(h1[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t][(P + 1) >> 5] = push_bit(w[t][(P + 1) >> 5], ~(b1[t] ^ pos[t]));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float t0 = h1[t] ? (h2[t] ? th[t].t[6] : th[t].t[2]) : (h2[t] ? th[t].t[4] : th[t].t[0]);
      b0[t] = __builtin_amdgcn_ballot_w64(a[t] >= t0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t][P >> 5] = push_bit(w[t][P >> 5], ~(b0[t] ^ pos[t]));
  }
}

// Coordinates 4 C + 3 .. 4 C of every tile, in descending order.
template <int BITS, int C, int NT>
__device__ __forceinline__ void push_block(const f32x4 (&v)[NT], const Thr<BITS> (&th)[NT], uint32_t (&w)[NT][BITS]) {
  push_index<BITS, 4 * C + 3, NT>(v, th, w);
  push_index<BITS, 4 * C + 2, NT>(v, th, w);
  push_index<BITS, 4 * C + 1, NT>(v, th, w);
  push_index<BITS, 4 * C, NT>(v, th, w);
}

// Compile-time loop C = HI, HI - 1, .., 0 (the block index must be a constant for the bit offsets;
// a plain loop of this size is not always unrolled).
template <int C>
struct BlockIdx {
  static constexpr int value = C;
};
template <int C, typename F>
__device__ __forceinline__ void for_blocks_down(F&& f) {
  if constexpr (C >= 0) {
    f(BlockIdx<C>{});
    for_blocks_down<C - 1>(f);
  }
}

constexpr int kMseWaves = 4;

// ---------------------------------------------------------------------------------------
// Outlier-8 keys: the rest channels go through the MSE encode below with the outlier channels
// zeroed, and the outlier channels become symmetric 8-bit integers with one absmax scale per
// key.  Lane (n, G) holds channels 32 G .. 32 G + 31 of its row, so it takes bits of word G of
// the head's rest mask, and slots NO/4 G .. NO/4 G + NO/4 - 1 of the head's outlier list, which
// it gathers from x (the row was just read, so these loads hit in cache).
// ---------------------------------------------------------------------------------------
struct OTile {
  uint32_t m;   // rest-mask word of the lane's channels
  uint32_t c;   // the word of the outlier list holding the lane's slots
};

template <int NO>
__device__ __forceinline__ void load_otile(const OutlierArgs& oa, int64_t n, int64_t tile, int nl, int g, OTile& o) {
  if constexpr (NO > 0) {
    const int64_t row = tile * 16 + nl;
    const uint32_t lrow = (uint32_t)(row < n ? row : n - 1);   // the host bounds n below 2^31
    const uint32_t h = (lrow / oa.T) % oa.H;
    o.m = oa.mask[h * 4 + g];
    o.c = oa.chan[h * 4 + ((g * (NO / 4)) >> 2)];
  }
}

__device__ __forceinline__ uint32_t bit_ext(uint32_t m, int p) {   // 0 or 0xffffffff
  return (uint32_t)((int32_t)(m << (31 - p)) >> 31);
}

template <bool BF16IN>
__device__ __forceinline__ void apply_rest_mask(RawTile<BF16IN>& r, uint32_t m) {
  if constexpr (BF16IN) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = 8 * s + 2 * j;
        // bytes 0-1 from the low channel's mask, bytes 2-3 from the high one's
        r.v[s][j] &= __builtin_amdgcn_perm(bit_ext(m, p + 1), bit_ext(m, p), 0x07060100u);
      }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        r.v[s][k] = __uint_as_float(__float_as_uint(r.v[s][k]) & bit_ext(m, 4 * s + k));
  }
}

template <int NO>
struct OVals {
  float v[NO > 0 ? NO / 4 : 1];
};

// The lane's outlier values of tile `tile` (rows past the end read the last row).
template <int NO, bool BF16IN>
__device__ __forceinline__ void gather_outliers(const void* x, int64_t n, int64_t tile, int nl, int g, const OTile& o,
                                                OVals<NO>& ov) {
  if constexpr (NO > 0) {
    constexpr int NS = NO / 4;
    const int64_t row = tile * 16 + nl;
    const int64_t lrow = row < n ? row : n - 1;
    const int b0 = (g * NS) & 3;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint32_t c = (o.c >> (8 * (b0 + i))) & 0xffu;
      if constexpr (BF16IN) {
        const uint16_t u = static_cast<const uint16_t*>(x)[lrow * 128 + c];
        ov.v[i] = __uint_as_float((uint32_t)u << 16);
      } else {
        ov.v[i] = static_cast<const float*>(x)[lrow * 128 + c];
      }
    }
  }
}

// scale = max |x_c| / 127 over the row's outlier channels (the four lanes of the row meet by
// shuffles), q_c = x_c / scale rounded to nearest even; stores the lane's NO/4 bytes and, from
// lane group 0, the scale.
template <int NO>
__device__ __forceinline__ void store_outliers(const OutlierArgs& oa, int64_t n, int64_t tile, int nl, int g,
                                               const OVals<NO>& ov) {
  if constexpr (NO > 0) {
    constexpr int NS = NO / 4;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) a = fmaxf(a, fabsf(ov.v[i]));
    a = fmaxf(a, __shfl_xor(a, 16));
    a = fmaxf(a, __shfl_xor(a, 32));
    const float sc = a / 127.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float qv = sc > 0.f ? rintf(ov.v[i] / sc) : 0.f;
      qv = fminf(fmaxf(qv, -127.f), 127.f);
      packed |= ((uint32_t)(int32_t)qv & 0xffu) << (8 * i);
    }
    const int64_t row = tile * 16 + nl;
    if (row < n) {
      int8_t* dst = oa.q8 + row * NO + NS * g;
      if constexpr (NS == 4) {
        *reinterpret_cast<uint32_t*>(dst) = packed;
      } else if constexpr (NS == 2) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
      } else {
        *dst = (int8_t)packed;
      }
      if (g == 0) oa.scale[row] = sc;
    }
  }
}

// NO > 0: outlier-8 keys (NO outlier channels per head, described by oa).
template <int BITS, bool BF16IN, int RP, int NT, int NO>
__global__ __launch_bounds__(kMseWaves * 64, 2) void k_encode_mse_d128(
    const void* __restrict__ x, int64_t n, const u32x4* __restrict__ frag_r, float post_scale,
    CodebookArgs cb, uint32_t* __restrict__ idx_out, float* __restrict__ norms_out, OutlierArgs oa) {
  constexpr int H = 1 << (BITS - 1);
  constexpr int kThreads = kMseWaves * 64;
  constexpr int kStage = RP * kFragU4 / kThreads;
  static_assert(RP * kFragU4 % kThreads == 0, "staging split");
  __shared__ u32x4 lds[RP * kFragU4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int64_t ntiles = (n + 15) >> 4;
  const int64_t stride = (int64_t)gridDim.x * kMseWaves * NT;
  int64_t tw = ((int64_t)blockIdx.x * kMseWaves + wave) * NT;

  // Fragment loads first, then the first tile group only.  The next group's loads are spread
  // over the MFMA blocks of the current step: a wave that issued several groups up front would
  // stall on the issue of its loads (the memory pipeline accepts a bounded number) and reach
  // the barrier, and its first MFMA, only once most of the device's requests had drained.
  u32x4 stage[kStage];
  const int rot0 = (int)(blockIdx.x % kStage);   // staggered start, as in k_encode_d128
#pragma unroll
  for (int j = 0; j < kStage; ++j) stage[j] = frag_r[threadIdx.x + ((j + rot0) % kStage) * kThreads];
  RawTile<BF16IN> bufA[NT], bufB[NT];
  OTile oA[NT], oB[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_tile<BF16IN>(x, n, tw + t, nl, g, bufA[t]);
#pragma unroll
  for (int t = 0; t < NT; ++t) load_otile<NO>(oa, n, tw + t, nl, g, oA[t]);
#pragma unroll
  for (int j = 0; j < kStage; ++j) lds[threadIdx.x + ((j + rot0) % kStage) * kThreads] = stage[j];
  __syncthreads();

  const float inv_post = 1.0f / post_scale;
  // Loads of the next group: NV vector loads per tile, LPB of them issued per MFMA block.
  constexpr int NV = BF16IN ? 4 : 8;
  constexpr int LPB = (NT * NV + 7) / 8;
  using Elem = typename std::conditional<BF16IN, u32x4, f32x4>::type;
  auto step = [&](RawTile<BF16IN> (&cur)[NT], RawTile<BF16IN> (&nxt)[NT], const OTile (&ocur)[NT], OTile (&onxt)[NT],
                  const int64_t t0) {
    const Elem* nsrc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = (t0 + stride + t) * 16 + nl;
      const int64_t lrow = row < n ? row : n - 1;   // clamped: past the end reads the last row
      nsrc[t] = reinterpret_cast<const Elem*>(static_cast<const char*>(x) + (lrow * 128 + 32 * g) * (BF16IN ? 2 : 4));
    }
    OVals<NO> ov[NT];
    if constexpr (NO > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        apply_rest_mask<BF16IN>(cur[t], ocur[t].m);
        gather_outliers<NO, BF16IN>(x, n, t0 + t, nl, g, ocur[t], ov[t]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) load_otile<NO>(oa, n, t0 + stride + t, nl, g, onxt[t]);
    }
    // B operands: bf16 input is used in place; fp32 input is split into bf16 hi + lo.
    u32x4 bxh[BF16IN ? 1 : NT][4], bxl[BF16IN ? 1 : NT][4];
    Thr<BITS> thr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float acc2 = 0.f;
      if constexpr (BF16IN) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
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
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x2 pr = {v[2 * j], v[2 * j + 1]};
            const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
            const f32x2 rem = {v[2 * j] - __uint_as_float(h << 16), v[2 * j + 1] - __uint_as_float(h & 0xffff0000u)};
            bxh[t][s][j] = h;
            bxl[t][s][j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
            acc2 = fmaf(v[2 * j], v[2 * j], acc2);
            acc2 = fmaf(v[2 * j + 1], v[2 * j + 1], acc2);
          }
        }
      }
      acc2 += __shfl_xor(acc2, 16);
      acc2 += __shfl_xor(acc2, 32);
      const float nrm = sqrtf(acc2);
      const bool live = nrm > 0.f;
      const int64_t row = (t0 + t) * 16 + nl;
      if (row < n && g == 0) norms_out[row] = nrm;
      // Decisions on the raw product against t_p * ||x|| / post_scale; a zero vector keeps every
      // threshold at +inf (index K/2 everywhere).
      const float tsc = nrm * inv_post;
      if constexpr (H > 1) {
#pragma unroll
        for (int p = 0; p < H - 1; ++p) thr[t].t[p] = live ? __int_as_float(cb.tpos[p]) * tsc : INFINITY;
      }
    }

    uint32_t w[NT][BITS];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < BITS; ++j) w[t][j] = 0;
    // One fragment set only: each pass's fragments for the next block are read into the
    // registers of the current one as soon as that pass's MFMAs have issued, and arrive during
    // the other pass and the quantizer work.  Blocks run c = 7 .. 0 (push order).
    f32x4 prev[NT];
    u32x4 cf[RP][4];
    load_frags<RP>(lds, 7, lane, cf);
    for_blocks_down<7>([&](auto ci) {
      constexpr int c = decltype(ci)::value;
      f32x4 now[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) now[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < RP; ++p) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if constexpr (BF16IN) {
              now[t] = mfma_bf16(cf[p][s], cur[t].v[s], now[t]);
            } else {
              now[t] = mfma_bf16(cf[p][s], bxh[t][s], now[t]);
              if (p == 0) now[t] = mfma_bf16(cf[p][s], bxl[t][s], now[t]);
            }
          }
        if constexpr (c > 0) {
#pragma unroll
          for (int s = 0; s < 4; ++s) cf[p][s] = lds[p * kFragU4 + ((c - 1) * 4 + s) * 64 + lane];
        }
      }
#pragma unroll
      for (int k = 0; k < LPB; ++k) {
        constexpr int q0 = (7 - c) * LPB;
        const int q = q0 + k;
        if (q < NT * NV) nxt[q / NV].v[q % NV] = nsrc[q / NV][q % NV];
      }
      if constexpr (c < 7) push_block<BITS, c + 1, NT>(prev, thr, w);
#pragma unroll
      for (int t = 0; t < NT; ++t) prev[t] = now[t];
      __builtin_amdgcn_sched_barrier(0);
    });
    push_block<BITS, 0, NT>(prev, thr, w);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = (t0 + t) * 16 + nl;
      if (row < n) {
        uint32_t* dst = idx_out + row * (4 * BITS) + BITS * g;
#pragma unroll
        for (int j = 0; j < BITS; ++j) dst[j] = w[t][j];
      }
    }
    if constexpr (NO > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) store_outliers<NO>(oa, n, t0 + t, nl, g, ov[t]);
    }
  };
  // Entered unconditionally (an early exit would let the compiler sink the tile loads past the
  // barrier); a wave without a tile of its own stores nothing, since every store checks its row.
  for (;;) {
    step(bufA, bufB, oA, oB, tw);
    if (tw + stride >= ntiles) break;
    step(bufB, bufA, oB, oA, tw + stride);
    tw += 2 * stride;
    if (tw >= ntiles) break;
  }
}

template <int BITS, bool BF16IN, int RP, int NO = 0>
hipError_t mse_launch(const void* x, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                      uint32_t* idx, float* norms, hipStream_t st, const OutlierArgs& oa = OutlierArgs{}) {
  constexpr int NT = BF16IN ? 2 : 1;
  const int64_t ntiles = (n + 15) / 16;
  const int64_t per_block = (int64_t)kMseWaves * NT;
  int64_t blocks = (ntiles + per_block - 1) / per_block;
  const int64_t cap = (int64_t)num_cus() * 2;
  if (blocks > cap) blocks = cap;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (take_armed_timer(&ev0, &ev1)) {
    // events attached to the dispatch itself: they bracket the kernel's execution alone
    hipExtLaunchKernelGGL((k_encode_mse_d128<BITS, BF16IN, RP, NT, NO>), dim3((unsigned)blocks), dim3(kMseWaves * 64),
                          0, st, ev0, ev1, 0, x, n, reinterpret_cast<const u32x4*>(rot->frag_dev), rot->post_scale, cb,
                          idx, norms, oa);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_encode_mse_d128<BITS, BF16IN, RP, NT, NO>), dim3((unsigned)blocks), dim3(kMseWaves * 64), 0,
                     st, x, n, reinterpret_cast<const u32x4*>(rot->frag_dev), rot->post_scale, cb, idx, norms, oa);
  return hipGetLastError();
}

template <int BITS, int NO>
hipError_t outlier8_dispatch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                             const OutlierArgs& oa, uint32_t* idx, float* norms, hipStream_t st) {
  if (bf16)
    return rot->passes == 1 ? mse_launch<BITS, true, 1, NO>(x, n, rot, cb, idx, norms, st, oa)
                            : mse_launch<BITS, true, 2, NO>(x, n, rot, cb, idx, norms, st, oa);
  return rot->passes == 1 ? mse_launch<BITS, false, 1, NO>(x, n, rot, cb, idx, norms, st, oa)
                          : mse_launch<BITS, false, 2, NO>(x, n, rot, cb, idx, norms, st, oa);
}

template <int NO>
hipError_t outlier8_bits(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                         const OutlierArgs& oa, uint32_t* idx, float* norms, hipStream_t st) {
  switch (cb.bits) {
    case 1: return outlier8_dispatch<1, NO>(x, bf16, n, rot, cb, oa, idx, norms, st);
    case 2: return outlier8_dispatch<2, NO>(x, bf16, n, rot, cb, oa, idx, norms, st);
    case 3: return outlier8_dispatch<3, NO>(x, bf16, n, rot, cb, oa, idx, norms, st);
    case 4: return outlier8_dispatch<4, NO>(x, bf16, n, rot, cb, oa, idx, norms, st);
  }
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t mse_dispatch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                        uint32_t* idx, float* norms, hipStream_t st) {
  if (bf16)
    return rot->passes == 1 ? mse_launch<BITS, true, 1>(x, n, rot, cb, idx, norms, st)
                            : mse_launch<BITS, true, 2>(x, n, rot, cb, idx, norms, st);
  return rot->passes == 1 ? mse_launch<BITS, false, 1>(x, n, rot, cb, idx, norms, st)
                          : mse_launch<BITS, false, 2>(x, n, rot, cb, idx, norms, st);
}


template <int BITS, bool PROD, bool BF16IN, bool STORE_Y, int PASSES>
hipError_t enc_launch(const void* x, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                      const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits,
                      float* rnorms, float* y, hipStream_t st, const uint16_t* frag = nullptr, int y_raw = 0) {
  constexpr int NT = (PROD || !BF16IN) ? 1 : 2;
  constexpr int kWaves = EncShape<PROD>::kWaves;
  const int64_t ntiles = (n + 15) / 16;
  const int64_t per_block = (int64_t)kWaves * NT;
  int64_t blocks = (ntiles + per_block - 1) / per_block;
  const int64_t cap = (int64_t)num_cus() * EncShape<PROD>::kBlocksPerCU;
  if (blocks > cap) blocks = cap;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (take_armed_timer(&ev0, &ev1)) {
    hipExtLaunchKernelGGL((k_encode_d128<BITS, PROD, BF16IN, STORE_Y, PASSES, NT>), dim3((unsigned)blocks),
                          dim3(kWaves * 64), 0, st, ev0, ev1, 0, x, n,
                          reinterpret_cast<const u32x4*>(frag ? frag : rot->frag_dev),
                          reinterpret_cast<const u32x4*>(qjl ? qjl->frag_dev : nullptr), rot->post_scale, cb, idx,
                          norms, qbits, rnorms, y, y_raw);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_encode_d128<BITS, PROD, BF16IN, STORE_Y, PASSES, NT>), dim3((unsigned)blocks),
                     dim3(kWaves * 64), 0, st, x, n,
                     reinterpret_cast<const u32x4*>(frag ? frag : rot->frag_dev),
                     reinterpret_cast<const u32x4*>(qjl ? qjl->frag_dev : nullptr), rot->post_scale, cb, idx,
                     norms, qbits, rnorms, y, y_raw);
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

hipError_t launch_rotate_raw_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, bool transpose,
                                  float* y, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const uint16_t* frag = transpose ? rot->fragT_dev : rot->frag_dev;
  if (!frag) return hipErrorInvalidValue;
  CodebookArgs none{};
  none.bits = 1;
  if (bf16)
    return rot->passes == 1
               ? enc_launch<1, false, true, true, 1>(x, n, rot, nullptr, none, nullptr, nullptr, nullptr, nullptr, y, st, frag, 1)
               : enc_launch<1, false, true, true, 2>(x, n, rot, nullptr, none, nullptr, nullptr, nullptr, nullptr, y, st, frag, 1);
  return rot->passes == 1
             ? enc_launch<1, false, false, true, 1>(x, n, rot, nullptr, none, nullptr, nullptr, nullptr, nullptr, y, st, frag, 1)
             : enc_launch<1, false, false, true, 2>(x, n, rot, nullptr, none, nullptr, nullptr, nullptr, nullptr, y, st, frag, 1);
}

hipError_t launch_encode_outlier8(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                                  const OutlierArgs& oa, uint32_t* idx, float* norms, hipStream_t st) {
  switch (oa.no) {
    case 4: return outlier8_bits<4>(x, bf16, n, rot, cb, oa, idx, norms, st);
    case 8: return outlier8_bits<8>(x, bf16, n, rot, cb, oa, idx, norms, st);
    case 16: return outlier8_bits<16>(x, bf16, n, rot, cb, oa, idx, norms, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_encode_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                              const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx,
                              float* norms, uint32_t* qjl_bits, float* rnorms, float* y_out,
                              hipStream_t st) {
  if (y_out) return enc_dispatch_in<1, false, true>(x, bf16, n, rot, nullptr, cb, nullptr, norms, nullptr, nullptr, y_out, st);
  const bool prod = qjl != nullptr;
  if (!prod) {
    switch (cb.bits) {
      case 1: return mse_dispatch<1>(x, bf16, n, rot, cb, idx, norms, st);
      case 2: return mse_dispatch<2>(x, bf16, n, rot, cb, idx, norms, st);
      case 3: return mse_dispatch<3>(x, bf16, n, rot, cb, idx, norms, st);
      case 4: return mse_dispatch<4>(x, bf16, n, rot, cb, idx, norms, st);
    }
    return hipErrorInvalidValue;
  }
  if (prod && cb.bits <= 3) return launch_encode_prod_d128(x, bf16, n, rot, qjl, cb, idx, norms, qjl_bits, rnorms, st);
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
