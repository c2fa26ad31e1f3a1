// Query prologue (q_rot = R q, q_s = S q once per query head) and the compressed-key score
// kernel at d = 128, MSE and TurboQuant_prod, with GQA sharing.
#include <hip/hip_ext.h>

#include "tq_cache.h"
#include "tq_decode.h"

namespace tq {
namespace {

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

// (src & mask) | base in one instruction.  The compiler splits it in two when both constants
// are literals (one scalar operand per instruction on this architecture): here the mask comes in
// a VGPR that stays loop-invariant and the base is the scalar operand.
__device__ __forceinline__ uint32_t and_or_vs(uint32_t src, uint32_t vmask, uint32_t sbase) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(src), "v"(vmask), "s"(sbase));
  return r;
}

__device__ __forceinline__ void sign_operand(uint32_t z, u32x4 (&bz)[4]) {
  const uint32_t zl = z << 8;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    const int m = d < 8 ? d + 8 : d;
    const uint32_t src = d < 8 ? zl : z;
    constexpr uint32_t bases[8] = {0x3c003c00u, 0x3c003c00u, 0x38003800u, 0x34003400u,
                                   0x2c002c00u, 0x1c001c00u, 0x00000000u, 0x3c003c00u};
    bz[d >> 2][d & 3] = and_or_vs(src, (1u << m) | (1u << (m + 16)), bases[m - 8]);
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
#ifndef TQ_QPREP_HEADS
#define TQ_QPREP_HEADS 2
#endif
constexpr int kQprepHeads = TQ_QPREP_HEADS;  // query heads per block pass (bounds the live LDS operands per thread)

__global__ __launch_bounds__(kQprepThreads) void k_qprep128(const float* __restrict__ q, int Hq, int ratio,
                                                            const float* __restrict__ rt,
                                                            const float* __restrict__ st,
                                                            uint16_t* __restrict__ ws,
                                                            float* __restrict__ kconst,
                                                            const uint32_t* __restrict__ omask,
                                                            const uint32_t* __restrict__ ochan, int no,
                                                            float* __restrict__ qo) {
  constexpr int HG = kQprepHeads;
  constexpr int KP = 128 / kQprepParts;
  __shared__ float qs[HG][128];
  __shared__ float part[2][kQprepParts][HG][128];
  __shared__ float sum[2][HG][128];
  const int Hkv = Hq / ratio;
  const int bg = blockIdx.x;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int h0 = kvh * ratio;
  const int j = threadIdx.x & 127, p = threadIdx.x >> 7;
  const int nmat = st ? 2 : 1;
  // The thread's slice of R^T and S^T column j does not depend on the queries: its loads are
  // issued before the queries are staged, so the two memory latencies overlap.
  const int k0 = p * KP;
  float rv[KP], sv[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) rv[k] = rt[(k0 + k) * 128 + j];
  if (st) {
#pragma unroll
    for (int k = 0; k < KP; ++k) sv[k] = st[(k0 + k) * 128 + j];
  }
  // blockIdx.y takes every gridDim.y-th group of HG heads (one group per block at launch)
  for (int hc = HG * blockIdx.y; hc < ratio; hc += HG * gridDim.y) {
    const int nh = ratio - hc < HG ? ratio - hc : HG;
    __syncthreads();
    if (threadIdx.x < HG * 128) {
      const int hh = threadIdx.x >> 7;
      float v = hh < nh ? q[((int64_t)b * Hq + h0 + hc + hh) * 128 + j] : 0.f;
      // outlier-8 keys: the rotated query sees only the rest channels of the KV head
      if (omask && !((omask[kvh * 4 + (j >> 5)] >> (j & 31)) & 1u)) v = 0.f;
      qs[hh][j] = v;
    } else if (omask && threadIdx.x < HG * 128 + HG * kOutlierMaxChannels) {
      // ... and the outlier components go to qo in the head's channel order
      const int u = threadIdx.x - HG * 128;
      const int hh = u / kOutlierMaxChannels, k = u % kOutlierMaxChannels;
      if (hh < nh && k < no) {
        const int c = (int)((ochan[kvh * 4 + (k >> 2)] >> (8 * (k & 3))) & 0xffu);
        const int64_t hrow = (int64_t)b * Hq + h0 + hc + hh;
        qo[hrow * kOutlierMaxChannels + k] = q[hrow * 128 + c];
      }
    }
    __syncthreads();
    float ar[HG], as[HG];
#pragma unroll
    for (int i = 0; i < HG; ++i) ar[i] = as[i] = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k)
#pragma unroll
      for (int i = 0; i < HG; ++i) ar[i] = fmaf(rv[k], qs[i][k0 + k], ar[i]);
    if (st) {
#pragma unroll
      for (int k = 0; k < KP; ++k)
#pragma unroll
        for (int i = 0; i < HG; ++i) as[i] = fmaf(sv[k], qs[i][k0 + k], as[i]);
    }
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      part[0][p][i][j] = ar[i];
      part[1][p][i][j] = as[i];
    }
    __syncthreads();
    // threads (m, j), m < nmat: the full sum of matrix m for the heads of this pass
    if (threadIdx.x < 128 * nmat) {
      const int m = threadIdx.x >> 7;
#pragma unroll
      for (int i = 0; i < HG; ++i) {
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
        if (m == 0) {
          v = sum[0][i][j];
        } else {
          // sketch in sign-slot order: output slot j = 32 G + 8 s + e  <-  coordinate
          // 32 G + c(s, e), scaled by 1 / beta
          const int G = j >> 5, s8 = (j & 31) >> 3, e = j & 7;
          const int c = 32 * G + sign_slot_coord(s8, e);
          const int mp = sign_slot_mpos(4 * s8 + (e >> 1));
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
// F / BITS fp16 centroids (F = 6 for 3 bits, else 8), built by each block in one pass and
// replicated so that the lanes of one LDS cycle read distinct banks.
// ---------------------------------------------------------------------------------------
// Launch shape (tuning defaults; overridable at build time).
#ifndef TQ_SCORE_BATCH
#define TQ_SCORE_BATCH 8
#endif
#ifndef TQ_SCORE_ROUNDS
#define TQ_SCORE_ROUNDS 1
#endif
#ifndef TQ_SCORE_PIPE
#define TQ_SCORE_PIPE 1
#endif
#ifndef TQ_SCORE_SHARE
#define TQ_SCORE_SHARE 1
#endif
#ifndef TQ_SCORE_MINB
#define TQ_SCORE_MINB 3   // resident blocks per CU the register budget is sized for
#endif
constexpr int kScoreWaves = 4;
constexpr int kScoreBatch = TQ_SCORE_BATCH;   // key tiles loaded before any of them is scored
constexpr int kScoreRounds = TQ_SCORE_ROUNDS; // target grid = this many rounds of resident blocks

template <int BITS, bool PROD, int NO = 0>
struct KeyTile {
  uint32_t w[BITS];
  float nrm;
  uint32_t zw;
  float gam;
  uint32_t o8[NO > 0 ? NO / 4 : 1];   // outlier-8 keys: the key's NO int8 values
  float osc;                          // and their scale
};

// The sequence's packed keys as buffer resources: each load is the resource plus one 32-bit
// per-lane offset, and tokens past T read as zero (their scores are never stored).
template <bool PROD>
struct KeyBufs {
  __amdgpu_buffer_rsrc_t idx, norms, qbits, rnorms, q8, osc;
};

// Lane (n, g) share of key tile `tile` of one sequence: its BITS words (coordinates 32 g ..),
// norm, and for prod its sign word and scaled residual norm.
// PERKEY false: the per-key scalars (norm, residual norm, outlier scale) are left out; the
// caller loads them for several tiles at once (see load_half).
template <int BITS, bool PROD, int NO, bool PERKEY = true>
__device__ __forceinline__ void load_key_tile(const KeyBufs<PROD>& kb, int tile, int nl, int g,
                                              KeyTile<BITS, PROD, NO>& k) {
  const uint32_t t = (uint32_t)tile * 16u + (uint32_t)nl;
  if constexpr (NO > 0) {
    buffer_words<NO / 4>(kb.q8, t * (uint32_t)NO, k.o8);
    if constexpr (PERKEY)
      k.osc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kb.osc, t * 4u, 0, 0));
  }
  buffer_words<BITS>(kb.idx, t * (16u * BITS) + (uint32_t)(4 * BITS * g), k.w);
  if constexpr (PERKEY) k.nrm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kb.norms, t * 4u, 0, 0));
  if constexpr (PROD) {
    k.zw = __builtin_amdgcn_raw_buffer_load_b32(kb.qbits, t * 16u + 4u * (uint32_t)g, 0, 0);
    if constexpr (PERKEY)
      k.gam = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kb.rnorms, t * 4u, 0, 0)) *
              (kQjl / 128.0f);
  } else {
    k.zw = 0;
    k.gam = 0.f;
  }
}

// MULTI: GQA ratio above 4, so each key is scored for several groups of 4 heads; otherwise the
// kernel carries only the single-group path.  NO > 0: outlier-8 keys, whose score adds
// scale * <q_O, q8> (fp32, on the vector ALUs) to the rest channels' term; qo holds q_O.
template <int BITS, bool PROD, bool MULTI, int NO>
__global__ __launch_bounds__(kScoreWaves * 64, TQ_SCORE_MINB) void k_scores_d128(
    const uint16_t* __restrict__ qws, const float* __restrict__ kconst, int Hq, int Hkv, int64_t T, int64_t seq_stride,
    int tiles_per_wave,
    const uint32_t* __restrict__ idx, const float* __restrict__ norms,
    const uint32_t* __restrict__ qbits, const float* __restrict__ rnorms, CodebookArgs cb,
    float* __restrict__ scores, const int8_t* __restrict__ q8, const float* __restrict__ oscale,
    const float* __restrict__ qo) {
  constexpr int TC = table_copies<BITS, false, 32768>();
  using DT = DecodeTable<BITS, false, TC>;
  __shared__ __attribute__((aligned(16))) uint8_t tab[DT::BYTES];
  __shared__ _Float16 cent[16];
  if (threadIdx.x < 16) cent[threadIdx.x] = (_Float16)cb.c[threadIdx.x];
  __syncthreads();
  build_table<BITS, TC>(tab, cent);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const uint32_t laneoff = (uint32_t)(lane % TC) * DT::EB;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int ratio = Hq / Hkv;
  const int groups = MULTI ? (ratio + 3) / 4 : 1;
  // sequence bg: rows [bg * seq_stride, bg * seq_stride + T) (seq_stride = T, or a cache's capacity)
  const int64_t base_row = (int64_t)bg * seq_stride;
  // the host bounds T so that a sequence's packed words stay below 4 GB (32-bit offsets)
  // this (batch, kv head)'s score rows, ratio x T floats (the host bounds ratio * T * 4 < 4 GB)
  const __amdgpu_buffer_rsrc_t sbuf =
      buffer_rsrc(scores + ((int64_t)b * Hq + kvh * ratio) * T, (uint32_t)ratio * (uint32_t)T * 4u);
  KeyBufs<PROD> kb;
  kb.idx = buffer_rsrc(idx + base_row * (4 * BITS), (uint32_t)T * (16u * BITS));
  kb.norms = buffer_rsrc(norms + base_row, (uint32_t)T * 4u);
  if constexpr (PROD) {
    kb.qbits = buffer_rsrc(qbits + base_row * 4, (uint32_t)T * 16u);
    kb.rnorms = buffer_rsrc(rnorms + base_row, (uint32_t)T * 4u);
  }
  if constexpr (NO > 0) {
    kb.q8 = buffer_rsrc(q8 + base_row * NO, (uint32_t)T * (uint32_t)NO);
    kb.osc = buffer_rsrc(oscale + base_row, (uint32_t)T * 4u);
  }
  const int64_t tile0 = ((int64_t)blockIdx.x * kScoreWaves + wave) * tiles_per_wave;
  const int64_t ntiles_seq = (T + 15) / 16;

  // A operand for head group 0 (kept in registers): lane (n, g) holds row n = 4 part + head
  // (part 0 rot hi, 1 rot lo, 2 sketch hi, 3 sketch lo), contraction slots 8 g .. 8 g + 7.  One
  // register set feeds both products: in the key product rows 8-15 (sketch) meet the centroids,
  // and in the sign product rows 0-7 (rotated query) meet the signs; those result rows are
  // discarded, since each lane keeps the rows of its own half (g < 2: rows 0-7 of the key
  // product; g >= 2: rows 8-15 of the sign product).  MSE zeroes the sketch rows.
  auto load_a = [&](int hg, u32x4 (&a)[4]) {
    const int hl = nl & 3;           // head within the group
    const int part = nl >> 2;
    const int h = 4 * hg + hl;
    const bool live = h < ratio && (PROD || part < 2);
    const uint16_t* src = qws + (((int64_t)b * Hq + kvh * ratio + (h < ratio ? h : 0)) * 4 + part) * 128 + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + 8 * s);
      a[s] = live ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 a0[4];
  load_a(0, a0);
  // Prod keys with one head group: the key product reads the rotated-query rows (0-7) and the
  // sign product the sketch rows (8-15) of two copies of the operand with the other rows zeroed,
  // so both products accumulate into one result whose rows are already the ones each lane
  // keeps (lanes of groups 0-1 hold rows 0-7, groups 2-3 rows 8-15): no per-lane select.  The
  // zero rows add exact zeros, so every kept row sums the same terms in the same order.
  constexpr bool kOneAcc = PROD && !MULTI;
  u32x4 a0k[kOneAcc ? 4 : 1], a0z[kOneAcc ? 4 : 1];
  if constexpr (kOneAcc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a0k[s] = nl < 8 ? a0[s] : u32x4{0u, 0u, 0u, 0u};
      a0z[s] = nl < 8 ? u32x4{0u, 0u, 0u, 0u} : a0[s];
    }
  }
  // sketch constant K of the lane's head (4 hg + g) after the reduction
  auto load_kc = [&](int hg) -> float {
    const int h = 4 * hg + g;
    return (PROD && h < ratio) ? kconst[(int64_t)b * Hq + kvh * ratio + h] : 0.f;
  };
  const float kc0 = load_kc(0);
  // q_O of the lane's head (4 hg + g), outlier-8 keys only
  auto load_qo = [&](int hg, float (&v)[NO > 0 ? NO : 1]) {
    const int h = 4 * hg + g;
    const float* src = qo + ((int64_t)b * Hq + kvh * ratio + (h < ratio ? h : 0)) * kOutlierMaxChannels;
#pragma unroll
    for (int k = 0; k < (NO > 0 ? NO : 1); ++k) v[k] = NO > 0 ? src[k] : 0.f;
  };
  // (kept in registers for a single head group only: with several groups the registers of a
  // batch of key tiles are needed for the keys)
  float qo0[NO > 0 && !MULTI ? NO : 1];
  if constexpr (NO > 0 && !MULTI) load_qo(0, qo0);

  // Ping-pong over two tile buffers (no register copies), so the next tile's loads stay in flight
  // while the current one is scored and the wait before scoring counts only the older loads.
  auto score_tile = [&](const KeyTile<BITS, PROD, NO>& cur, int64_t ti) {
    // token of the lane's key (below 2^25 + 16: the host bounds T, and ti stays below `last`)
    const uint32_t t = (uint32_t)(tile0 + ti) * 16u + (uint32_t)nl;
    const bool valid = t < (uint32_t)T;
    const float nrm = cur.nrm;
    const float gam = cur.gam;
    u32x4 bk[4], bz[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) bk[s] = decode_keys_or<BITS, TC>(cur.w, s, tab, laneoff);
    if constexpr (PROD) sign_operand(cur.zw, bz);
    float o8f[NO > 0 ? NO : 1];
    if constexpr (NO > 0) {
#pragma unroll
      for (int k = 0; k < NO; ++k) o8f[k] = (float)((int32_t)(cur.o8[k >> 2] << (24 - 8 * (k & 3))) >> 24);
    }
    for (int hg = 0; hg < groups; ++hg) {
      u32x4 a[4];
      if (!MULTI || hg == 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = a0[s];
      } else {
        load_a(hg, a);
      }
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kOneAcc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc = mfma_f16(a0k[s], bk[s], acc);
          acc = mfma_f16(a0z[s], bz[s], acc);
        }
      } else {
        f32x4 accz = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc = mfma_f16(a[s], bk[s], acc);
          if constexpr (PROD) accz = mfma_f16(a[s], bz[s], accz);
        }
        if constexpr (PROD) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = g < 2 ? acc[r] : accz[r];
        }
      }
      const float sc = g < 2 ? nrm : 2.f * gam;
      float mine = reduce_parts(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc);
      const int h = 4 * hg + g;
      if constexpr (PROD) mine -= gam * (hg == 0 ? kc0 : load_kc(hg));
      if constexpr (NO > 0) {
        float qv[NO];
        if constexpr (!MULTI) {
#pragma unroll
          for (int k = 0; k < NO; ++k) qv[k] = qo0[k];
        } else {
          load_qo(hg, qv);
        }
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < NO; ++k) o = fmaf(o8f[k], qv[k], o);
        mine = fmaf(cur.osc, o, mine);
      }
      if (valid && h < ratio)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mine), sbuf,
                                              ((uint32_t)h * (uint32_t)T + t) * 4u, 0, 0);
    }
  };
  int64_t last = tiles_per_wave;
  if (ntiles_seq - tile0 < last) last = ntiles_seq - tile0;
#if TQ_SCORE_PIPE
  // Two half-batches A and B of kScoreBatch / 2 tiles in ping-pong: the loads of one half are in
  // flight while the other half is scored, so a wave never waits for a whole batch's latency
  // with nothing to do.  Loads past the sequence read zeros (buffer range), so they are issued
  // unconditionally and every wait stays exact.
  // Each half's loads go through resources based at its first key (scalar arithmetic only), so
  // that every load address is a loop-invariant lane offset plus an immediate: no vector register
  // is written to form an address, and none can collide with the sources of a store still in
  // flight (a wait for such a store would also wait for every load issued before it).
  // With TQ_SCORE_SHARE the per-key scalars of a half (up to 64 keys) come in one load per
  // array, lane l holding key l of the half, and reach the lanes of tile u by a cross-lane
  // permute: a third of the vector memory instructions of a tile, whose address queue limits
  // the issue rate here.
  constexpr int HB = kScoreBatch / 2;
  constexpr bool kShare = TQ_SCORE_SHARE && HB <= 4;
  struct HalfScalars {
    float nrm, gam, osc;
  };
  KeyTile<BITS, PROD, NO> ka[HB], kbt[HB];
  HalfScalars sa, sb;
  auto load_half = [&](KeyTile<BITS, PROD, NO> (&kt)[HB], HalfScalars& hs, int64_t tb) {
    // the half's keys that lie inside both the sequence and the wave's own tiles: the loop's last
    // prefetch runs past the wave's tiles, and those loads must neither read the next wave's keys
    // nor cost traffic, so the range ends there (out-of-range loads read zero without memory access)
    const int64_t first = (tile0 + tb) * 16;
    int64_t rem = T - first;
    if ((last - tb) * 16 < rem) rem = (last - tb) * 16;
    const uint32_t nk = rem > 0 ? (uint32_t)rem : 0u;
    const int64_t row = base_row + first;
    KeyBufs<PROD> h;
    h.idx = buffer_rsrc(idx + row * (4 * BITS), nk * (16u * BITS));
    h.norms = buffer_rsrc(norms + row, nk * 4u);
    if constexpr (PROD) {
      h.qbits = buffer_rsrc(qbits + row * 4, nk * 16u);
      h.rnorms = buffer_rsrc(rnorms + row, nk * 4u);
    }
    if constexpr (NO > 0) {
      h.q8 = buffer_rsrc(q8 + row * NO, nk * (uint32_t)NO);
      h.osc = buffer_rsrc(oscale + row, nk * 4u);
    }
#pragma unroll
    for (int u = 0; u < HB; ++u) load_key_tile<BITS, PROD, NO, !kShare>(h, u, nl, g, kt[u]);
    if constexpr (kShare) {
      const uint32_t off = (uint32_t)lane * 4u;
      hs.nrm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(h.norms, off, 0, 0));
      if constexpr (PROD)
        hs.gam = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(h.rnorms, off, 0, 0)) *
                 (kQjl / 128.0f);
      if constexpr (NO > 0) hs.osc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(h.osc, off, 0, 0));
    }
  };
  auto score_half = [&](const KeyTile<BITS, PROD, NO> (&kt)[HB], const HalfScalars& hs, int64_t tb) {
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      if (tb + u < last) {
        if constexpr (kShare) {
          KeyTile<BITS, PROD, NO> k = kt[u];
          const int src = (nl + 16 * u) << 2;
          k.nrm = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(hs.nrm)));
          if constexpr (PROD) k.gam = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(hs.gam)));
          if constexpr (NO > 0) k.osc = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(hs.osc)));
          score_tile(k, tb + u);
        } else {
          score_tile(kt[u], tb + u);
        }
      }
    }
  };
  load_half(ka, sa, 0);
  for (int64_t tb = 0; tb < last; tb += 2 * HB) {
    load_half(kbt, sb, tb + HB);
    __builtin_amdgcn_sched_barrier(0);
    score_half(ka, sa, tb);
    if (tb + HB >= last) break;
    load_half(ka, sa, tb + 2 * HB);
    __builtin_amdgcn_sched_barrier(0);
    score_half(kbt, sb, tb + HB);
  }
#else
  // Batches of kScoreBatch tiles: every load of a batch is issued before any tile of it is
  // scored (straight-line code, so the waits are exact), and the batch's latency is paid once.
  for (int64_t tb = 0; tb < last; tb += kScoreBatch) {
    KeyTile<BITS, PROD, NO> kt[kScoreBatch];
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u)
      load_key_tile<BITS, PROD, NO>(kb, (int)(tile0 + tb + u), nl, g, kt[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u)
      if (tb + u < last) score_tile(kt[u], tb + u);
  }
#endif
}

template <int BITS, bool PROD, bool MULTI, int NO = 0>
hipError_t scores_launch_m(int B, int Hq, int Hkv, int64_t T, int64_t seq_stride, const tq_packed* K, const CodebookArgs& cb,
                         float* scores, const void* ws, hipStream_t st, const int8_t* q8 = nullptr,
                         const float* oscale = nullptr, const float* qo = nullptr) {
  const int ratio = Hq / Hkv;
  const uint16_t* qws = static_cast<const uint16_t*>(ws);
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  const float* kconst = reinterpret_cast<const float*>(static_cast<const char*>(ws) + qbytes);
  const int64_t tiles = (T + 15) / 16;
  // Size the grid as a whole number of rounds of resident blocks (a partial last round would
  // leave most of the device idle): blocks resident per CU come from the occupancy calculator.
  static int per_cu = 0;
  if (per_cu == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_scores_d128<BITS, PROD, MULTI, NO>, kScoreWaves * 64, 0) != hipSuccess ||
        v <= 0)
      v = 2;
    per_cu = v;
  }
  const int64_t target = (int64_t)num_cus() * per_cu * kScoreRounds;
  const int64_t seqs = (int64_t)B * Hkv;
  int64_t tpw = (tiles * seqs + target * kScoreWaves - 1) / (target * kScoreWaves);
  tpw = (tpw + kScoreBatch - 1) / kScoreBatch * kScoreBatch;
  if (tpw < kScoreBatch) tpw = kScoreBatch;
  if (tpw > 256) tpw = 256;
  const int64_t chunks = (tiles + tpw * kScoreWaves - 1) / (tpw * kScoreWaves);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (take_armed_timer(TQ_TIMED_SCORES, &ev0, &ev1)) {
    // events attached to the dispatch itself: they bracket the kernel's execution alone
    hipExtLaunchKernelGGL((k_scores_d128<BITS, PROD, MULTI, NO>), dim3((unsigned)chunks, (unsigned)seqs),
                          dim3(kScoreWaves * 64), 0, st, ev0, ev1, 0, qws, kconst, Hq, Hkv, T, seq_stride, (int)tpw,
                          K->idx, K->norms, PROD ? K->qjl : nullptr, PROD ? K->rnorms : nullptr, cb, scores, q8,
                          oscale, qo);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_scores_d128<BITS, PROD, MULTI, NO>), dim3((unsigned)chunks, (unsigned)seqs),
                     dim3(kScoreWaves * 64), 0, st, qws, kconst, Hq, Hkv, T, seq_stride, (int)tpw, K->idx, K->norms,
                     PROD ? K->qjl : nullptr, PROD ? K->rnorms : nullptr, cb, scores, q8, oscale, qo);
  return hipGetLastError();
}

template <int BITS, bool PROD>
hipError_t scores_launch(int B, int Hq, int Hkv, int64_t T, int64_t S, const tq_packed* K, const CodebookArgs& cb,
                         float* scores, const void* ws, hipStream_t st) {
  return Hq / Hkv > 4 ? scores_launch_m<BITS, PROD, true>(B, Hq, Hkv, T, S, K, cb, scores, ws, st)
                      : scores_launch_m<BITS, PROD, false>(B, Hq, Hkv, T, S, K, cb, scores, ws, st);
}

template <int BITS, int NO>
hipError_t outlier8_scores_launch(int B, int Hq, int Hkv, int64_t T, int64_t S, const tq_packed* K,
                                  const CodebookArgs& cb, float* scores, const void* ws, hipStream_t st,
                                  const int8_t* q8, const float* oscale, const float* qo) {
  return Hq / Hkv > 4 ? scores_launch_m<BITS, false, true, NO>(B, Hq, Hkv, T, S, K, cb, scores, ws, st, q8, oscale, qo)
                      : scores_launch_m<BITS, false, false, NO>(B, Hq, Hkv, T, S, K, cb, scores, ws, st, q8, oscale, qo);
}

template <int NO>
hipError_t outlier8_scores_bits(int B, int Hq, int Hkv, int64_t T, int64_t S, const tq_packed* K,
                                const CodebookArgs& cb, float* scores, const void* ws, hipStream_t st,
                                const int8_t* q8, const float* oscale, const float* qo) {
  switch (cb.bits) {
    case 1: return outlier8_scores_launch<1, NO>(B, Hq, Hkv, T, S, K, cb, scores, ws, st, q8, oscale, qo);
    case 2: return outlier8_scores_launch<2, NO>(B, Hq, Hkv, T, S, K, cb, scores, ws, st, q8, oscale, qo);
    case 3: return outlier8_scores_launch<3, NO>(B, Hq, Hkv, T, S, K, cb, scores, ws, st, q8, oscale, qo);
    case 4: return outlier8_scores_launch<4, NO>(B, Hq, Hkv, T, S, K, cb, scores, ws, st, q8, oscale, qo);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qprep128(const float* q, int B, int Hq, int Hkv, const float* rt, const float* st_mat,
                           uint16_t* qws, float* kconst, hipStream_t st, const OutlierArgs* oa, float* qo) {
  const int groups = (Hq / Hkv + kQprepHeads - 1) / kQprepHeads;
  hipLaunchKernelGGL(k_qprep128, dim3(B * Hkv, groups), dim3(kQprepThreads), 0, st, q, Hq, Hq / Hkv, rt, st_mat,
                     qws, kconst, oa ? oa->mask : nullptr, oa ? oa->chan : nullptr, oa ? oa->no : 0, qo);
  return hipGetLastError();
}

size_t scores_outlier8_workspace_bytes(int B, int Hq) {
  const size_t base = (scores_workspace_bytes(B, Hq, 128) + 255) & ~(size_t)255;
  return base + (size_t)B * Hq * kOutlierMaxChannels * sizeof(float);
}

hipError_t launch_scores_outlier8(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride,
                                  const tq_packed* K, const int8_t* q8, const float* oscale, const CodebookArgs& cb,
                                  const tq_rotation_s* rot, const OutlierArgs& oa, float* scores, void* ws,
                                  hipStream_t st) {
  uint16_t* qws = static_cast<uint16_t*>(ws);
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  float* kconst = reinterpret_cast<float*>(static_cast<char*>(ws) + qbytes);
  float* qo = reinterpret_cast<float*>(static_cast<char*>(ws) + ((scores_workspace_bytes(B, Hq, 128) + 255) &
                                                                 ~(size_t)255));
  hipError_t e = launch_qprep128(q, B, Hq, Hkv, rot->rt32_dev, nullptr, qws, kconst, st, &oa, qo);
  if (e != hipSuccess) return e;
  switch (oa.no) {
    case 4: return outlier8_scores_bits<4>(B, Hq, Hkv, T, seq_stride, K, cb, scores, ws, st, q8, oscale, qo);
    case 8: return outlier8_scores_bits<8>(B, Hq, Hkv, T, seq_stride, K, cb, scores, ws, st, q8, oscale, qo);
    case 16: return outlier8_scores_bits<16>(B, Hq, Hkv, T, seq_stride, K, cb, scores, ws, st, q8, oscale, qo);
  }
  return hipErrorInvalidValue;
}

size_t scores_workspace_bytes(int B, int Hq, int d) {
  (void)d;
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  return qbytes + (size_t)B * Hq * sizeof(float);
}

hipError_t launch_prepare_queries(const float* q, int B, int Hq, int Hkv, const tq_rotation_s* rot,
                                  const tq_qjl_s* qjl, void* ws, hipStream_t st) {
  uint16_t* qws = static_cast<uint16_t*>(ws);
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  float* kconst = reinterpret_cast<float*>(static_cast<char*>(ws) + qbytes);
  return launch_qprep128(q, B, Hq, Hkv, rot->rt32_dev, qjl ? qjl->st32_dev : nullptr, qws, kconst, st);
}

hipError_t launch_scores_strided(int B, int Hq, int Hkv, int64_t T, int64_t S, const tq_packed* K,
                                 const CodebookArgs& cb, float* scores, const void* ws, hipStream_t st) {
  const bool prod = K->mode == TQ_MODE_PROD;
  switch (cb.bits) {
    case 1: return prod ? scores_launch<1, true>(B, Hq, Hkv, T, S, K, cb, scores, ws, st)
                        : scores_launch<1, false>(B, Hq, Hkv, T, S, K, cb, scores, ws, st);
    case 2: return prod ? scores_launch<2, true>(B, Hq, Hkv, T, S, K, cb, scores, ws, st)
                        : scores_launch<2, false>(B, Hq, Hkv, T, S, K, cb, scores, ws, st);
    case 3: return prod ? scores_launch<3, true>(B, Hq, Hkv, T, S, K, cb, scores, ws, st)
                        : scores_launch<3, false>(B, Hq, Hkv, T, S, K, cb, scores, ws, st);
    case 4: return prod ? scores_launch<4, true>(B, Hq, Hkv, T, S, K, cb, scores, ws, st)
                        : scores_launch<4, false>(B, Hq, Hkv, T, S, K, cb, scores, ws, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scores_prepared(int B, int Hq, int Hkv, int64_t T, const tq_packed* K, const CodebookArgs& cb,
                                  float* scores, const void* ws, hipStream_t st) {
  return launch_scores_strided(B, Hq, Hkv, T, T, K, cb, scores, ws, st);
}

hipError_t launch_scores(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                         const CodebookArgs& cb, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                         float* scores, void* ws, hipStream_t st) {
  hipError_t e = launch_prepare_queries(q, B, Hq, Hkv, rot, K->mode == TQ_MODE_PROD ? qjl : nullptr, ws, st);
  if (e != hipSuccess) return e;
  return launch_scores_prepared(B, Hq, Hkv, T, K, cb, scores, ws, st);
}

}  // namespace tq
