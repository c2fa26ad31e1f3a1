// Value-cache encode in the token-blocked layout and the fused decode attention at d = 128:
// scores from packed K, online softmax, P V on MFMA in V's rotated domain, split merge and
// the inverse rotation.
#include "tq_cache.h"
#include "tq_decode.h"
#include "tq_split.h"

namespace tq {
namespace {

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
  {
    // All loads first (one wait), each block starting at a different slice so that blocks
    // reading the same fragments in lockstep do not all queue on one L2 channel.
    constexpr int kStage = RP * kFragU4 / 256;
    const int rot0 = (int)(blockIdx.x % kStage);
    u32x4 stage[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) stage[j] = fragt[threadIdx.x + ((j + rot0) % kStage) * 256];
#pragma unroll
    for (int j = 0; j < kStage; ++j) lds[threadIdx.x + ((j + rot0) % kStage) * 256] = stage[j];
  }
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
// Launch shape: each block takes `spb` 32-token steps of one (batch, kv head); spb is chosen at
// launch so the grid is a whole number of rounds of resident blocks, and never below
// kAttnMinSteps (which bounds the number of splits, hence the workspace).
#ifndef TQ_ATTN_ROUNDS
#define TQ_ATTN_ROUNDS 1
#endif
#ifndef TQ_ATTN_BATCH
#define TQ_ATTN_BATCH 1
#endif
// LDS budgets of the replicated K (split) and V decode tables, and the blocks per CU the kernel is
// built for: full replication of both tables needs 64 KB, which fits two blocks per CU, not three.
#ifndef TQ_ATTN_KBUDGET
#define TQ_ATTN_KBUDGET 32768
#endif
#ifndef TQ_ATTN_VBUDGET
#define TQ_ATTN_VBUDGET 16384
#endif
#ifndef TQ_ATTN_BLOCKS
#define TQ_ATTN_BLOCKS 3
#endif
constexpr int kAttnMinSteps = 16;
constexpr int kAttnBatch = TQ_ATTN_BATCH;  // 32-token steps loaded together
constexpr int kAttnRounds = TQ_ATTN_ROUNDS;
constexpr int kAttnPart = 130;

// The value held by a partner lane within the lane's row of 16, through DPP (no LDS): steps
// 0..3 pair lanes by xor 1, xor 2, mirror within 8, mirror within 16, so four max-steps leave
// every lane of a row with the row's maximum.
__device__ __forceinline__ float row16_partner(float v, int step) {
  const int x = __float_as_int(v);
  int y;
  switch (step) {
    case 0: y = __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return __int_as_float(y);
}  // max, sum, 128 accumulators

// One 32-token step of a wave: the lane's key words and norms for both 16-token tiles, the
// value norms, and the value chunks of octet g at coordinates 8 n .. 8 n + 7.
template <int KB, int VB, int NO = 0>
struct AttnStep {
  uint32_t kw[2][KB];
  float kn[2];
  float vn[2];
  uint32_t vw[2 * VB];
  uint32_t o8[2][NO > 0 ? NO / 4 : 1];   // outlier-8 keys: each key's NO int8 values
  float osc[2];                          // and their scale
  uint32_t kwr[2][2];                    // split keys: the lane's two-word window of the rest half
  float knr[2];                          // and the rest half's norm (kw / kn: the outlier half)
};

// One sequence's keys, key norms, value norms (from its first row) and value blocks (from its
// first 32-row block) as buffer resources: each load is the resource plus one 32-bit per-lane
// offset, and rows outside the sequence read as zero (the kernel masks them).
struct AttnBufs {
  __amdgpu_buffer_rsrc_t k, kn, vn, v, q8, osc, kr, knr;
};

// Split keys: lane group g takes coordinates 16 g .. 16 g + 15 of each half (64 coordinates of B
// bits, 2B words per row).  The lane reads a two-word window from split_word on (never past the
// row) and shifts it right by split_shift, which leaves its 16 indices at bit 0.
template <int B>
__device__ __forceinline__ uint32_t split_word(int g) {
  const uint32_t w = (uint32_t)(16 * g * B) >> 5;
  return w < 2u * B - 2u ? w : 2u * B - 2u;
}
template <int B>
__device__ __forceinline__ uint32_t split_shift(int g) {
  return (uint32_t)(16 * g * B) - 32u * split_word<B>(g);
}

template <int KB, int VB, int NO, int BR>
__device__ __forceinline__ void load_attn_step(const AttnBufs& ab, int64_t row0, int64_t T, int64_t blk_first,
                                               int64_t blk, int nl, int g, AttnStep<KB, VB, NO>& st) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    // Rows before the sequence (the first block of a sequence that starts mid-block) take row T,
    // the first row past the resources' ends, so they read zero (the kernel masks them).  A
    // wrapped negative offset would not do: the compiler may form the second tile's offset as the
    // first tile's plus an immediate, and the range check then rejects the second tile's valid
    // rows of lanes whose first-tile row lies before the sequence.
    const int32_t rs = (int32_t)(blk * 32 - row0) + tt * 16 + nl;   // in [-31, T + 31]: T < 2^25
    const uint32_t r = rs < 0 ? (uint32_t)T : (uint32_t)rs;
    if constexpr (BR > 0) {
      const u32x2 o = __builtin_amdgcn_raw_buffer_load_b64(ab.k, (r * (2u * KB) + split_word<KB>(g)) * 4u, 0, 0);
      const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(ab.kr, (r * (2u * BR) + split_word<BR>(g)) * 4u, 0, 0);
      st.kw[tt][0] = o[0];
      st.kw[tt][1] = o[1];
      st.kwr[tt][0] = q[0];
      st.kwr[tt][1] = q[1];
      st.knr[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ab.knr, r * 4u, 0, 0));
    } else {
      buffer_words<KB>(ab.k, r * (16u * KB) + (uint32_t)(4 * KB * g), st.kw[tt]);
    }
    if constexpr (NO > 0) {
      buffer_words<NO / 4>(ab.q8, r * (uint32_t)NO, st.o8[tt]);
      st.osc[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ab.osc, r * 4u, 0, 0));
    }
    st.kn[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ab.kn, r * 4u, 0, 0));
    st.vn[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ab.vn, r * 4u, 0, 0));
  }
  const uint32_t vb = (uint32_t)(blk - blk_first);
  buffer_words<2 * VB>(ab.v, (vb * (128u * VB) + (uint32_t)(32 * g * VB + 2 * nl * VB)) * 4u, st.vw);
}

// NO > 0: outlier-8 keys (the rest channels' code in kidx / knorm, the outlier channels' int8
// values in q8 and scales in oscale); the logit adds scale * <q_O, q8> in fp32, q_O from qo.
//
// BR > 0: split keys (the outlier halves at KB bits in kidx / knorm, the rest halves at BR bits in
// kidx_r / knorm_r, each half 64 coordinates in its own rotated domain); qws then holds the fp32
// rotated queries [B * Hq][128] of the split prologue (R_o q_O, then R_r q_R).  Lane group g
// takes coordinates 16 g .. 16 g + 15 of each half, the two halves accumulate apart and are
// scaled by their own norms before the parts are reduced.
template <int KB, int VB, int NO, int BR>
__global__ __launch_bounds__(256, TQ_ATTN_BLOCKS) void k_attn_d128(
    const uint16_t* __restrict__ qws, int Hq, int Hkv, int64_t T, int nsplit, int spb,
    const uint32_t* __restrict__ kidx, const float* __restrict__ knorm,
    const uint32_t* __restrict__ vidx, const float* __restrict__ vnorm, int64_t seq_stride,
    CodebookArgs cbk, CodebookArgs cbv, float scale, float* __restrict__ part, const int8_t* __restrict__ q8,
    const float* __restrict__ oscale, const float* __restrict__ qo, const uint32_t* __restrict__ kidx_r,
    const float* __restrict__ knorm_r, CodebookArgs cbr) {
  constexpr bool SPLIT = BR > 0;
  static_assert(!SPLIT || (KB >= 2 && NO == 0), "split keys: outlier half of 2 to 4 bits, no int8 outliers");
  // replicated decode tables (K up to 32 KB, split keys two of up to 16 KB, V up to 16 KB) so that
  // three blocks fit a CU
  constexpr int KC = table_copies<KB, true, SPLIT ? TQ_ATTN_KBUDGET / 2 : TQ_ATTN_KBUDGET>();
  constexpr int RC = table_copies<SPLIT ? BR : 1, true, TQ_ATTN_KBUDGET / 2>();
  constexpr int VC = table_copies<VB, false, TQ_ATTN_VBUDGET>();
  using DK = DecodeTable<KB, true, KC>;
  using DR = DecodeTable<SPLIT ? BR : 1, true, RC>;
  using DV = DecodeTable<VB, false, VC>;
  // the K tables' storage is reused for the block's merge buffer once every wave has finished
  constexpr int kMergeBytes = 4 * 4 * 128 * (int)sizeof(float);
  constexpr int kKTabBytes = DK::BYTES + (SPLIT ? DR::BYTES : 0);
  __shared__ __attribute__((aligned(16))) uint8_t ktab[kKTabBytes > kMergeBytes ? kKTabBytes : kMergeBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vtab[DV::BYTES];
  __shared__ float kcent[2][16];
  __shared__ _Float16 vcent[16];
  // Weights strip of each wave in fp16: part 0 the weights rounded to fp16, part 1 their
  // remainders, part 2 zeros (the operand rows that carry nothing); a row per head, 32 tokens
  // padded to 40 halves (80 bytes), so the 16-byte reads of different rows fall in distinct banks.
  constexpr int kWRow = 40;
  __shared__ __attribute__((aligned(16))) uint16_t wh[4][3][4][kWRow];
  __shared__ float mm[4][4], ll[4][4];
  if (threadIdx.x < 16) {
    kcent[0][threadIdx.x] = cbk.c[threadIdx.x];
    kcent[1][threadIdx.x] = cbr.c[threadIdx.x];
    vcent[threadIdx.x] = (_Float16)cbv.c[threadIdx.x];
  }
  __syncthreads();
  build_table2<KB, KC>(ktab, kcent[0]);
  if constexpr (SPLIT) build_table2<BR, RC>(ktab + DK::BYTES, kcent[1]);
  build_table<VB, VC>(vtab, vcent);
  for (int i = threadIdx.x; i < 4 * 4 * kWRow; i += blockDim.x) wh[i / (4 * kWRow)][2][(i / kWRow) % 4][i % kWRow] = 0;
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const uint8_t* ktabl = DK::lane_base(ktab, lane);
  const uint8_t* rtabl = DR::lane_base(ktab + DK::BYTES, lane);
  const uint8_t* vtabl = DV::lane_base(vtab, lane);
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int ratio = Hq / Hkv;
  // sequence bh: rows [bh * seq_stride, bh * seq_stride + T) (seq_stride = T, or a cache's capacity)
  const int64_t row0 = (int64_t)bh * seq_stride, rowE = row0 + T;
  const int64_t blk_first = row0 >> 5, blk_end = ((rowE - 1) >> 5) + 1;
  const int64_t bb = blk_first + (int64_t)blockIdx.x * spb;
  const int64_t be = bb + spb < blk_end ? bb + spb : blk_end;
  const int64_t cnt = be > bb ? be - bb : 0;
  const int64_t per = (cnt + 3) / 4;
  const int64_t wb = bb + wave * per;
  const int64_t we = wb + per < be ? wb + per : be;
  // (the host bounds T so that a sequence's words stay below 2 GB: 32-bit offsets)
  AttnBufs ab;
  ab.k = buffer_rsrc(kidx + row0 * (4 * KB), (uint32_t)T * (16u * KB));
  ab.kn = buffer_rsrc(knorm + row0, (uint32_t)T * 4u);
  ab.vn = buffer_rsrc(vnorm + row0, (uint32_t)T * 4u);
  ab.v = buffer_rsrc(vidx + blk_first * (128 * VB), (uint32_t)(blk_end - blk_first) * (512u * VB));
  if constexpr (SPLIT) {
    // half rows of 2 KB and 2 BR words
    ab.k = buffer_rsrc(kidx + row0 * (2 * KB), (uint32_t)T * (8u * KB));
    ab.kr = buffer_rsrc(kidx_r + row0 * (2 * BR), (uint32_t)T * (8u * BR));
    ab.knr = buffer_rsrc(knorm_r + row0, (uint32_t)T * 4u);
  }
  // q_O of the block's query heads, read from LDS when a logit needs it (held in registers it
  // would push the kernel past its register budget); lanes of heads past the ratio read head 0
  // and compute a logit that is discarded
  __shared__ __attribute__((aligned(16))) float qos[4][NO > 0 ? NO : 4];
  if constexpr (NO > 0) {
    ab.q8 = buffer_rsrc(q8 + row0 * NO, (uint32_t)T * (uint32_t)NO);
    ab.osc = buffer_rsrc(oscale + row0, (uint32_t)T * 4u);
    if (threadIdx.x < 4 * NO) {
      const int hh = threadIdx.x / NO, k = threadIdx.x % NO;
      qos[hh][k] = qo[((int64_t)b * Hq + kvh * ratio + (hh < ratio ? hh : 0)) * kOutlierMaxChannels + k];
    }
    __syncthreads();
  }

  // A operand of the key product, in the split-slot order of decode_split_slot (each table
  // entry's centroids and remainders side by side): rows 0-3 (heads) carry the rotated query's
  // fp16 hi part against both halves, rows 4-7 its lo part against the centroids only (the lo x
  // remainder term is below fp32 rounding); other rows zero.
  using KS = SplitSlot<KB>;
  u32x4 ak[8];
  if constexpr (SPLIT) {
    // instructions 0-3 the outlier half, 4-7 the rest half; lane group g holds the half's
    // coordinates 16 g .. 16 g + 15 in the split-slot order of that half's bit width
    using KR = SplitSlot<BR>;
    const int hl = nl & 3, prt = nl >> 2;
    const bool live = hl < ratio && prt < 2;
    const float* qf = reinterpret_cast<const float*>(qws) + ((int64_t)b * Hq + kvh * ratio + (hl < ratio ? hl : 0)) * 128;
    auto qpart = [&](int c) -> uint32_t {   // fp16 hi (prt 0) or lo (prt 1) of query coordinate c
      const float v = live ? qf[c] : 0.f;
      const _Float16 hi = (_Float16)v;
      const _Float16 out = prt == 0 ? hi : (_Float16)(v - (float)hi);
      return __builtin_bit_cast(uint16_t, out);
    };
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int half = j >> 2;
        const int p0 = 8 * (j & 3) + 2 * k, p1 = p0 + 1;
        const int c0 = half ? KR::coord(p0) : KS::coord(p0), c1 = half ? KR::coord(p1) : KS::coord(p1);
        const int h0 = half ? KR::half(p0) : KS::half(p0), h1 = half ? KR::half(p1) : KS::half(p1);
        const uint32_t lo = (h0 == 0 || prt == 0) ? qpart(64 * half + 16 * g + c0) : 0u;
        const uint32_t hi = (h1 == 0 || prt == 0) ? qpart(64 * half + 16 * g + c1) : 0u;
        ak[j][k] = lo | (hi << 16);
      }
  } else {
    const int hl = nl & 3, prt = nl >> 2;
    const bool live = hl < ratio && prt < 2;
    const uint16_t* src = qws + (((int64_t)b * Hq + kvh * ratio + (hl < ratio ? hl : 0)) * 4 + (prt == 1 ? 1 : 0)) * 128 + 32 * g;
    uint32_t qw[16];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + 8 * s);
#pragma unroll
      for (int k = 0; k < 4; ++k) qw[4 * s + k] = live ? v[k] : 0u;
    }
    auto qhalf = [&](int c) -> uint32_t { return (qw[c >> 1] >> (16 * (c & 1))) & 0xffffu; };
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p0 = 8 * j + 2 * k, p1 = p0 + 1;
        const uint32_t lo = (KS::half(p0) == 0 || prt == 0) ? qhalf(KS::coord(p0)) : 0u;
        const uint32_t hi = (KS::half(p1) == 0 || prt == 0) ? qhalf(KS::coord(p1)) : 0u;
        ak[j][k] = lo | (hi << 16);
      }
  }

  const uint16_t* wrow = &wh[wave][(nl >> 2) < 2 ? (nl >> 2) : 2][nl & 3][8 * g];
  float m_run = -INFINITY, l_part = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const AttnStep<KB, VB, NO>& cur, const int64_t blk) {
    float lg[2], svv[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t r = blk * 32 + tt * 16 + nl;
      const bool valid = r >= row0 && r < rowE;
      const float sk = cur.kn[tt];
      svv[tt] = cur.vn[tt];
      float mine;
      if constexpr (SPLIT) {
        const uint64_t wo = ((uint64_t)cur.kw[tt][1] << 32 | cur.kw[tt][0]) >> split_shift<KB>(g);
        const uint64_t wr = ((uint64_t)cur.kwr[tt][1] << 32 | cur.kwr[tt][0]) >> split_shift<BR>(g);
        const uint32_t wo2[2] = {(uint32_t)wo, (uint32_t)(wo >> 32)};
        const uint32_t wr2[2] = {(uint32_t)wr, (uint32_t)(wr >> 32)};
        f32x4 dout = f32x4{0.f, 0.f, 0.f, 0.f}, drest = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dout = mfma_f16(ak[j], decode_split_slot<KB, KC>(wo2, j, ktabl), dout);
          drest = mfma_f16(ak[4 + j], decode_split_slot<BR, RC>(wr2, j, rtabl), drest);
        }
        const float sr = cur.knr[tt];
        mine = reduce_parts(fmaf(dout[0], sk, drest[0] * sr), fmaf(dout[1], sk, drest[1] * sr),
                            fmaf(dout[2], sk, drest[2] * sr), fmaf(dout[3], sk, drest[3] * sr));
      } else {
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) d = mfma_f16(ak[j], decode_split_slot<KB, KC>(cur.kw[tt], j, ktabl), d);
        mine = reduce_parts(d[0] * sk, d[1] * sk, d[2] * sk, d[3] * sk);
      }
      if constexpr (NO > 0) {
        float o = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < NO / 4; ++k4) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(&qos[g][4 * k4]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            o = fmaf((float)((int32_t)(cur.o8[tt][k4] << (24 - 8 * k)) >> 24), qv[k], o);
        }
        mine = fmaf(cur.osc[tt], o, mine);
      }
      lg[tt] = (valid && g < ratio) ? mine * scale : -INFINITY;
    }
    // online softmax for head g
    float mx = fmaxf(lg[0], lg[1]);
#pragma unroll
    for (int o = 0; o < 4; ++o) mx = fmaxf(mx, row16_partner(mx, o));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
    const float w0 = lg[0] == -INFINITY ? 0.f : __expf(lg[0] - m_new);
    const float w1 = lg[1] == -INFINITY ? 0.f : __expf(lg[1] - m_new);
    l_part = fmaf(l_part, alpha, w0 + w1);
    m_run = m_new;
    {
      // the P V operand in fp16 hi + lo (round to nearest), formed once by the lane that owns the
      // weight: token nl and 16 + nl of head g
      const float p0 = w0 * svv[0], p1 = w1 * svv[1];
      const _Float16 h0 = (_Float16)p0, h1 = (_Float16)p1;
      const _Float16 r0 = (_Float16)(p0 - (float)h0), r1 = (_Float16)(p1 - (float)h1);
      wh[wave][0][g][nl] = __builtin_bit_cast(uint16_t, h0);
      wh[wave][0][g][16 + nl] = __builtin_bit_cast(uint16_t, h1);
      wh[wave][1][g][nl] = __builtin_bit_cast(uint16_t, r0);
      wh[wave][1][g][16 + nl] = __builtin_bit_cast(uint16_t, r1);
    }
    if (__any(alpha < 1.f)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 16 * r));
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c][r] *= ar;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // A operand: rows 0-3 the weights' fp16 part per head, 4-7 their remainders, 8-15 zero;
    // tokens 8 g .. 8 g + 7, one read from the lane's fixed row of the strip
    const u32x4 aw = *reinterpret_cast<const u32x4*>(wrow);
    // B operand: the value chunks of octet g at coordinates 8 n .. 8 n + 7
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = mfma_f16(aw, decode8<VB, VC>(cur.vw, 8 * VB * c, vtabl), acc[c]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  // Batches of kAttnBatch steps: all their loads are issued before the first step is consumed
  // (straight-line code, so each wait is exact and no registers are copied between steps).
  for (int64_t b0 = wb; b0 < we; b0 += kAttnBatch) {
    AttnStep<KB, VB, NO> st[kAttnBatch];
#pragma unroll
    for (int u = 0; u < kAttnBatch; ++u)
      if (b0 + u < we) load_attn_step<KB, VB, NO, BR>(ab, row0, T, blk_first, b0 + u, nl, g, st[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kAttnBatch; ++u)
      if (b0 + u < we) step(st[u], b0 + u);
  }

  // wave totals: sum over the 16 keys lanes; hi + lo accumulator rows
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) l_part += __shfl_xor(l_part, o);
  __syncthreads();  // every wave is done with the K table: its storage becomes the merge buffer
  float (*accs)[4][128] = reinterpret_cast<float (*)[4][128]>(ktab);
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

// The outlier-8 query components follow the split partials in the workspace.
size_t attn_partials_bytes(int B, int Hkv, int64_t T) {
  const int64_t steps = T / 32 + 2;
  const int64_t nsplit = (steps + kAttnMinSteps - 1) / kAttnMinSteps;  // the most splits a launch uses
  return ((size_t)B * Hkv * nsplit * 4 * kAttnPart * sizeof(float) + 255) & ~(size_t)255;
}

// Split keys for attn_launch: the rest halves' packed set and codebook, and the split prologue's
// inputs (channel order and the halves' R^T).
struct SplitAttnArgs {
  const tq_packed* Kr = nullptr;
  CodebookArgs cbr{};
  const int32_t* order = nullptr;
  const float* rto = nullptr;
  const float* rtr = nullptr;
};

template <int KB, int VB, int NO = 0, int BR = 0>
hipError_t attn_launch(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride, const tq_packed* K,
                       const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                       const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale, float* out,
                       void* ws, hipStream_t st, const OutlierArgs* oa = nullptr, const int8_t* q8 = nullptr,
                       const float* oscale = nullptr, const SplitAttnArgs* sa = nullptr) {
  uint16_t* qws = static_cast<uint16_t*>(ws);
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + qbytes);
  float* qo = NO > 0 ? reinterpret_cast<float*>(static_cast<char*>(ws) + qbytes + attn_partials_bytes(B, Hkv, T))
                     : nullptr;
  hipError_t e;
  if constexpr (BR > 0)   // fp32 [B * Hq][128] rotated split queries (the first half of the query region)
    e = launch_qprep_split(q, B, Hq, Hkv, sa->order, sa->rto, sa->rtr, reinterpret_cast<float*>(qws), st);
  else
    e = launch_qprep128(q, B, Hq, Hkv, rot_k->rt32_dev, nullptr, qws, nullptr, st, NO > 0 ? oa : nullptr, qo);
  if (e != hipSuccess) return e;
  static int per_cu = 0;
  if (per_cu == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_attn_d128<KB, VB, NO, BR>, 256, 0) != hipSuccess || v <= 0)
      v = 2;
    per_cu = v;
  }
  const int64_t seqs = (int64_t)B * Hkv;
  const int64_t steps = T / 32 + 2;
  const int64_t target = (int64_t)num_cus() * per_cu * kAttnRounds;
  const int64_t want = target / seqs > 0 ? target / seqs : 1;
  int64_t spb = (steps + want - 1) / want;
  spb = (spb + 3) / 4 * 4;
  if (spb < kAttnMinSteps) spb = kAttnMinSteps;
  const int nsplit = (int)((steps + spb - 1) / spb);
  hipLaunchKernelGGL((k_attn_d128<KB, VB, NO, BR>), dim3(nsplit, B * Hkv), dim3(256), 0, st, qws, Hq, Hkv, T, nsplit,
                     (int)spb, K->idx, K->norms, V->idx, V->norms, seq_stride, cbk, cbv, scale, part, q8, oscale, qo,
                     BR > 0 ? sa->Kr->idx : nullptr, BR > 0 ? sa->Kr->norms : nullptr, BR > 0 ? sa->cbr : cbk);
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
  const int64_t nsplit = (steps + kAttnMinSteps - 1) / kAttnMinSteps;  // the most splits a launch uses
  return qbytes + (size_t)B * Hkv * nsplit * 4 * kAttnPart * sizeof(float);
}

size_t decode_attn_outlier8_workspace_bytes(int B, int Hq, int Hkv, int64_t T) {
  const size_t qbytes = ((size_t)B * Hq * 4 * 128 * sizeof(uint16_t) + 255) & ~(size_t)255;
  return qbytes + attn_partials_bytes(B, Hkv, T) + (size_t)B * Hq * kOutlierMaxChannels * sizeof(float);
}

hipError_t launch_decode_attn_split(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* Ko,
                                    const tq_packed* Kr, const tq_packed* V, const CodebookArgs& cbo,
                                    const CodebookArgs& cbr, const CodebookArgs& cbv, const int32_t* order,
                                    const float* rto, const float* rtr, const tq_rotation_s* rot_v, float scale,
                                    float* out, void* ws, hipStream_t st) {
  SplitAttnArgs sa;
  sa.Kr = Kr;
  sa.cbr = cbr;
  sa.order = order;
  sa.rto = rto;
  sa.rtr = rtr;
#define TQ_ATTN_SPLIT(BO, BR, VB)                                                                                   \
  if (cbo.bits == BO && cbr.bits == BR && cbv.bits == VB)                                                        \
    return attn_launch<BO, VB, 0, BR>(q, B, Hq, Hkv, T, T, Ko, V, cbo, cbv, nullptr, rot_v, scale, out, ws, st,   \
                                      nullptr, nullptr, nullptr, &sa);
  TQ_ATTN_SPLIT(3, 2, 2) TQ_ATTN_SPLIT(3, 2, 3) TQ_ATTN_SPLIT(3, 2, 4)
  TQ_ATTN_SPLIT(4, 3, 2) TQ_ATTN_SPLIT(4, 3, 3) TQ_ATTN_SPLIT(4, 3, 4)
#undef TQ_ATTN_SPLIT
  return hipErrorInvalidValue;
}

hipError_t launch_decode_attn_outlier8(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride,
                                       const tq_packed* K, const int8_t* q8, const float* oscale, const tq_packed* V,
                                       const CodebookArgs& cbk, const CodebookArgs& cbv, const tq_rotation_s* rot_k,
                                       const tq_rotation_s* rot_v, const OutlierArgs& oa, float scale, float* out,
                                       void* ws, hipStream_t st) {
#define TQ_ATTN_O8(KB, VB, NO)                                                                                     \
  if (cbk.bits == KB && cbv.bits == VB && oa.no == NO)                                                            \
    return attn_launch<KB, VB, NO>(q, B, Hq, Hkv, T, seq_stride, K, V, cbk, cbv, rot_k, rot_v, scale, out, ws, st, \
                                   &oa, q8, oscale);
#define TQ_ATTN_O8_ALL(KB, VB) TQ_ATTN_O8(KB, VB, 4) TQ_ATTN_O8(KB, VB, 8) TQ_ATTN_O8(KB, VB, 16)
  TQ_ATTN_O8_ALL(3, 2) TQ_ATTN_O8_ALL(3, 3) TQ_ATTN_O8_ALL(2, 2) TQ_ATTN_O8_ALL(4, 2) TQ_ATTN_O8_ALL(4, 4)
  TQ_ATTN_O8_ALL(2, 4) TQ_ATTN_O8_ALL(4, 3) TQ_ATTN_O8_ALL(1, 1) TQ_ATTN_O8_ALL(2, 3) TQ_ATTN_O8_ALL(3, 4)
#undef TQ_ATTN_O8_ALL
#undef TQ_ATTN_O8
  return hipErrorInvalidValue;
}

hipError_t launch_decode_attn_strided(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride,
                                      const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk,
                                      const CodebookArgs& cbv, const tq_rotation_s* rot_k, const tq_rotation_s* rot_v,
                                      float scale, float* out, void* ws, hipStream_t st) {
#define TQ_ATTN(KB, VB) \
  if (cbk.bits == KB && cbv.bits == VB) \
    return attn_launch<KB, VB>(q, B, Hq, Hkv, T, seq_stride, K, V, cbk, cbv, rot_k, rot_v, scale, out, ws, st);
  TQ_ATTN(2, 2) TQ_ATTN(4, 4) TQ_ATTN(3, 3) TQ_ATTN(4, 2) TQ_ATTN(2, 4) TQ_ATTN(3, 2) TQ_ATTN(4, 3)
  TQ_ATTN(1, 1) TQ_ATTN(2, 3) TQ_ATTN(3, 4)
#undef TQ_ATTN
  return hipErrorInvalidValue;
}

hipError_t launch_decode_attn(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                              const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                              const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale,
                              float* out, void* ws, hipStream_t st) {
  return launch_decode_attn_strided(q, B, Hq, Hkv, T, T, K, V, cbk, cbv, rot_k, rot_v, scale, out, ws, st);
}

}  // namespace tq
