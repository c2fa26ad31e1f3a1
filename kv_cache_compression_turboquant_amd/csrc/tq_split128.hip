// Outlier-channel mixed precision at d = 128 ("TurboQuant 和 RotorQuant 的真相", the asymmetric
// needs of K and V: outlier channels at more bits than the rest; "TurboQuant 详解", the
// engineering data points at 2.5 and 3.5 bits per channel).  Every key vector is two
// TurboQuant_mse codes: its 64 outlier channels (listed per KV head) at BO bits and its other
// 64 channels at BR bits, each half with its own norm, its own 64 x 64 rotation and the
// codebook of dimension 64.  A query's score is the sum of the two halves' scores, each
// s <R q_half, C[idx]> in its own rotated domain.
#include <type_traits>

#include "tq_decode.h"
#include "tq_split.h"

namespace tq {
namespace {

template <int V>
using IC = std::integral_constant<int, V>;

// ---------------------------------------------------------------------------------------
// Encode.  A block of 8 waves takes 512 consecutive tokens of one sequence in eight rounds of 64
// (the next round's keys load into registers while the current one computes).
// Each round stages its 64 vectors in LDS in channel order (outlier channels first), so each
// half is a contiguous 64-vector.  Waves 0..3 rotate the outlier halves of vector groups
// 0..3 (16 vectors each) and waves 4..7 the other halves, so a wave's bit width is uniform.
// The rotation is Y = R X on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with fp32 sums:
// R as bf16 hi + lo (two passes, about 16 significant bits, as in the single-code encode), x as
// bf16 (exact for bf16 keys; fp32 keys add a third pass with the low part of x).  A = 16
// rotation rows x 32 contraction terms, B = 32 terms x the group's 16 vectors, 4 output blocks x
// 2 steps per half.  Lane l = n + 16 g supplies A row n, B column n and terms 8 g .. 8 g + 7 of
// each step and ends with coordinates 16 mb + 4 g + r of vector n.  The A fragments are built
// once per block in LDS (lane-major, so the reads are conflict-free).  bf16 keys are staged as
// they are (rows of 136 halves), so one 16-byte read is the B operand; fp32 keys are staged as
// fp32 (rows of 132 floats) and split into hi and lo when read.  Both paddings put the 16 rows a
// read touches in distinct banks.
// Quantization compares the unnormalized product against s * t_k (s the half's norm), the
// tie going up; a zero half (s = 0, product 0) compares 0 against the unscaled thresholds, so
// it takes the index of y = 0.  Indices are ORed into per-vector words in LDS and stored after a
// barrier.
// Rows past T are staged as zeros and never stored.
// ---------------------------------------------------------------------------------------
constexpr int kEncWaves = 8;
constexpr int kGroupRows = 16;                        // vectors per wave group per round
constexpr int kRoundRows = 4 * kGroupRows;            // 64
constexpr int kEncRounds = 8;
constexpr int kEncBlockRows = kRoundRows * kEncRounds;  // 512
constexpr int kXS = 132;
constexpr int kXH = 136;

// acc[mb][r] = unnormalized coordinate 16 mb + 4 g + r of vector v (this lane's), s = its norm.
template <int B, int OFF, int WT>
__device__ __forceinline__ void quantize_pack(const f32x4 (&acc)[4], float s, const CodebookArgs& cb,
                                              uint32_t* __restrict__ words, int g) {
  constexpr int K = 1 << B;
  float thr[K - 1];
#pragma unroll
  for (int q = 0; q < K - 1; ++q) thr[q] = s > 0.f ? s * cb.t[q] : cb.t[q];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    // coordinates 16 mb + 4 g .. + 3 are consecutive: one 4 B-bit field, ORed in with at most two
    // LDS atomics (the other three lanes of the vector fill the rest of the block's bits)
    uint32_t f = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t idx = 0;
#pragma unroll
      for (int q = 0; q < K - 1; ++q) idx += acc[mb][r] >= thr[q] ? 1u : 0u;
      f |= idx << (r * B);
    }
    const int p = (16 * mb + 4 * g) * B, w = p >> 5, sh = p & 31;
    atomicOr(&words[OFF + w], f << sh);
    if (sh + 4 * B > 32) atomicOr(&words[OFF + w + 1], f >> (32 - sh));
  }
}

template <int BO, int BR, bool BF16IN>
__global__ __launch_bounds__(kEncWaves * 64) void k_encode_split_d128(
    const void* __restrict__ x, int64_t T, int64_t out_stride, int64_t out_pos, int H, const int32_t* __restrict__ order,
    const float* __restrict__ ro,
    const float* __restrict__ rr, CodebookArgs cbo, CodebookArgs cbr, uint32_t* __restrict__ idx_o,
    float* __restrict__ norm_o, uint32_t* __restrict__ idx_r, float* __restrict__ norm_r) {
  constexpr int WO = 2 * BO, WR = 2 * BR, WT = WO + WR;
  __shared__ u32x4 afr[2][2][4][2][64];   // [half][hi, lo][out block][step][lane]: bf16 A fragments
  // staged vectors: fp32 rows of kXS floats, or for bf16 keys the bf16 values as they are, rows of
  // kXH halves (both padded so that the 16 rows a 16-byte read touches fall in distinct banks)
  __shared__ __align__(16) float xs[4][kGroupRows][kXS];
  uint16_t (*xh)[kGroupRows][kXH] = reinterpret_cast<uint16_t (*)[kGroupRows][kXH]>(&xs[0][0][0]);
  __shared__ int inv[kSplitD];
  __shared__ float nrm[2][kRoundRows];
  __shared__ uint32_t wbuf[kRoundRows][WT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = wave >> 2, grp = wave & 3;
  const int64_t seq = blockIdx.y;
  const int h = (int)(seq % H);
  const int64_t tblk = (int64_t)blockIdx.x * kEncBlockRows;

  // A fragments: lane l = n + 16 g of (half p, block mb, step st) holds R[16 mb + n][32 st + 8 g + e],
  // e = 0..7, as bf16 hi (round to nearest) and lo (the remainder, rounded)
  for (int e = tid; e < 2 * 4 * 2 * 64; e += kEncWaves * 64) {
    const int l = e & 63, st = (e >> 6) & 1, mb = (e >> 7) & 3, p = e >> 9;
    const float* src = (p ? rr : ro) + (16 * mb + (l & 15)) * 64 + 32 * st + 8 * (l >> 4);
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
    const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    u32x4 hi, lo;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t h0 = bf16_bits(f[2 * w]), h1 = bf16_bits(f[2 * w + 1]);
      hi[w] = h0 | (h1 << 16);
      lo[w] = bf16_bits(f[2 * w] - bf16_val(h0)) | (bf16_bits(f[2 * w + 1] - bf16_val(h1)) << 16);
    }
    afr[p][0][mb][st][l] = hi;
    afr[p][1][mb][st][l] = lo;
  }
  if (tid < kSplitD) inv[order[(int64_t)h * kSplitD + tid]] = tid;
  __syncthreads();

  const int ln = lane & 15, lg = lane >> 4;
  // staging: thread tid loads channels c8 .. c8 + 7 of round vectors (tid >> 4) + 32 k, k = 0, 1,
  // and writes each to its position in the staged vector (outlier half first)
  const int c8 = (tid & 15) * 8, vs = tid >> 4;
  int pos[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pos[i] = inv[c8 + i];

  // The next round's keys are loaded into registers while the current round computes.
  constexpr int NR = BF16IN ? 1 : 2;   // 16-byte loads per 8 channels
  u32x4 raw[2][NR];
  auto load_round = [&](int64_t tr) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t t = tr + vs + 32 * k;
      if (t < T) {
        const int64_t src = (seq * T + t) * kSplitD + c8;
#pragma unroll
        for (int j = 0; j < NR; ++j)
          raw[k][j] = BF16IN ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + src)
                             : *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + src + 4 * j);
      } else {
#pragma unroll
        for (int j = 0; j < NR; ++j) raw[k][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  load_round(tblk);

  for (int round = 0; round < kEncRounds; ++round) {
    const int64_t tr = tblk + (int64_t)round * kRoundRows;
    if (tr >= T) break;   // the block's remaining rounds are past the end (the same for every thread)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int v = vs + 32 * k;
      if constexpr (BF16IN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xh[v >> 4][v & 15][pos[2 * i]] = (uint16_t)(raw[k][0][i] & 0xffffu);
          xh[v >> 4][v & 15][pos[2 * i + 1]] = (uint16_t)(raw[k][0][i] >> 16);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xs[v >> 4][v & 15][pos[i]] = __uint_as_float(raw[k][0][i]);
          xs[v >> 4][v & 15][pos[4 + i]] = __uint_as_float(raw[k][NR - 1][i]);
        }
      }
    }
    for (int e = tid; e < kRoundRows * WT; e += kEncWaves * 64) (&wbuf[0][0])[e] = 0u;
    __syncthreads();
    if (round + 1 < kEncRounds && tr + kRoundRows < T) load_round(tr + kRoundRows);

    // The half's squared norm of vector (lane & 15): four partial sums of 16 squares, then
    // summed across the four lane quarters.
    float s2 = 0.f;
    {
      if constexpr (BF16IN) {
        const uint16_t* row = &xh[grp][lane & 15][part * 64 + (lane >> 4) * 16];
#pragma unroll
        for (int i = 0; i < 16; i += 8) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(row + i);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float lo = bf16_val(a[w] & 0xffffu), hi = bf16_val(a[w] >> 16);
            s2 = fmaf(lo, lo, s2);
            s2 = fmaf(hi, hi, s2);
          }
        }
      } else {
        const float* row = &xs[grp][lane & 15][part * 64 + (lane >> 4) * 16];
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(row + i);
          s2 = fmaf(a.x, a.x, s2);
          s2 = fmaf(a.y, a.y, s2);
          s2 = fmaf(a.z, a.z, s2);
          s2 = fmaf(a.w, a.w, s2);
        }
      }
      s2 += __shfl_xor(s2, 16);
      s2 += __shfl_xor(s2, 32);
    }
    const float s = sqrtf(s2);   // the half's norm of vector ln (every lane quarter holds it)
    if (lane < kGroupRows) nrm[part][grp * kGroupRows + lane] = s;

    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 bh, bl;
      if constexpr (BF16IN) {
        bh = *reinterpret_cast<const u32x4*>(&xh[grp][ln][part * 64 + 32 * st + 8 * lg]);
        bl = u32x4{0u, 0u, 0u, 0u};
      } else {
        const float* xb = &xs[grp][ln][part * 64 + 32 * st + 8 * lg];
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(xb);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(xb + 4);
        const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t h0 = bf16_bits(f[2 * w]), h1 = bf16_bits(f[2 * w + 1]);
          bh[w] = h0 | (h1 << 16);
          bl[w] = bf16_bits(f[2 * w] - bf16_val(h0)) | (bf16_bits(f[2 * w + 1] - bf16_val(h1)) << 16);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const u32x4 ah = afr[part][0][mb][st][lane], al = afr[part][1][mb][st][lane];
        acc[mb] = mfma_bf16(ah, bh, acc[mb]);
        acc[mb] = mfma_bf16(al, bh, acc[mb]);
        if (!BF16IN) acc[mb] = mfma_bf16(ah, bl, acc[mb]);
      }
    }
    uint32_t* words = wbuf[grp * kGroupRows + ln];
    if (part == 0)
      quantize_pack<BO, 0, WT>(acc, s, cbo, words, lg);
    else
      quantize_pack<BR, WO, WT>(acc, s, cbr, words, lg);
    __syncthreads();

    for (int e = tid; e < kRoundRows * WT; e += kEncWaves * 64) {
      const int v = e / WT, w = e - v * WT;
      const int64_t t = tr + v;
      if (t < T) {
        const int64_t row = seq * out_stride + out_pos + t;
        if (w < WO)
          idx_o[row * WO + w] = wbuf[v][w];
        else
          idx_r[row * WR + (w - WO)] = wbuf[v][w];
      }
    }
    if (tid < 2 * kRoundRows) {
      const int v = tid & (kRoundRows - 1);
      const int64_t t = tr + v;
      if (t < T) (tid < kRoundRows ? norm_o : norm_r)[seq * out_stride + out_pos + t] = nrm[tid / kRoundRows][v];
    }
    __syncthreads();  // the next round overwrites xs, wbuf and nrm
  }
}

// ---------------------------------------------------------------------------------------
// Short appends (a decode step's token): one block of 128 threads per (token, sequence).  Thread
// p gathers channel order[p] of its key, so wave 0 holds the outlier half and wave 1 the rest;
// each wave takes its half's norm with xor-shuffles, forms coordinate p & 63 of R x_half in fp32
// (R^T read coalesced), bucketizes it against the thresholds scaled by the norm and ORs its field
// into the key's words in LDS.
// ---------------------------------------------------------------------------------------
constexpr int64_t kSplitTokenMax = 32;   // appends of at most this many tokens per sequence

template <int BO, int BR, bool BF16IN>
__global__ __launch_bounds__(128) void k_append_split_token(
    const void* __restrict__ x, int64_t T, int64_t out_stride, int64_t out_pos, int H,
    const int32_t* __restrict__ order, const float* __restrict__ rto, const float* __restrict__ rtr, CodebookArgs cbo,
    CodebookArgs cbr, uint32_t* __restrict__ idx_o, float* __restrict__ norm_o, uint32_t* __restrict__ idx_r,
    float* __restrict__ norm_r) {
  constexpr int WO = 2 * BO, WR = 2 * BR;
  __shared__ float xs[kSplitD];
  __shared__ uint32_t words[WO + WR];
  const int p = threadIdx.x, lane = p & 63, half = p >> 6;
  const int64_t seq = blockIdx.y, t = blockIdx.x;
  const int h = (int)(seq % H);
  const int64_t src = (seq * T + t) * kSplitD + order[(int64_t)h * kSplitD + p];
  const float v = BF16IN ? bf16_val(static_cast<const uint16_t*>(x)[src]) : static_cast<const float*>(x)[src];
  xs[p] = v;
  if (p < WO + WR) words[p] = 0u;
  float s2 = v * v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s2 += __shfl_xor(s2, o);
  const float s = sqrtf(s2);
  __syncthreads();
  const float* rt = half ? rtr : rto;
  const float* xh = xs + half * 64;
  float y = 0.f;
#pragma unroll 16
  for (int i = 0; i < 64; ++i) y = fmaf(rt[i * 64 + lane], xh[i], y);
  const int64_t row = seq * out_stride + out_pos + t;
  auto quantize = [&](const CodebookArgs& cb, auto bits, int off) {
    constexpr int B = decltype(bits)::value;
    uint32_t idx = 0;
#pragma unroll
    for (int q = 0; q < (1 << B) - 1; ++q) idx += y >= (s > 0.f ? s * cb.t[q] : cb.t[q]) ? 1u : 0u;
    const int pb = lane * B, w = pb >> 5, sh = pb & 31;
    atomicOr(&words[off + w], idx << sh);
    if (sh + B > 32) atomicOr(&words[off + w + 1], idx >> (32 - sh));
  };
  if (half == 0)
    quantize(cbo, IC<BO>{}, 0);
  else
    quantize(cbr, IC<BR>{}, WO);
  __syncthreads();
  if (p < WO)
    idx_o[row * WO + p] = words[p];
  else if (p < WO + WR)
    idx_r[row * WR + (p - WO)] = words[p];
  if (lane == 0) (half ? norm_r : norm_o)[row] = s;
}

// ---------------------------------------------------------------------------------------
// Query prologue: one block of 512 threads per query head.  The query is gathered into the
// channel order of its KV head; thread (j, quarter) then sums 16 of the 64 terms of coordinate
// j & 63 of R_o q_O (j < 64) or of R_r q_R, reading R^T row-major so that the threads' loads are
// consecutive, and the four partial sums are added in LDS (short dependent chains: the kernel
// is all latency).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_qprep_split(const float* __restrict__ q, int Hq, int Hkv,
                                                     const int32_t* __restrict__ order, const float* __restrict__ rto,
                                                     const float* __restrict__ rtr, float* __restrict__ qws) {
  __shared__ float qs[kSplitD];
  __shared__ float part_sum[4][kSplitD];
  const int tid = threadIdx.x, j = tid & (kSplitD - 1), quarter = tid >> 7;
  const int64_t bh = blockIdx.x;
  const int hq = (int)(bh % Hq), hk = hq / (Hq / Hkv);
  if (tid < kSplitD) qs[j] = q[bh * kSplitD + order[(int64_t)hk * kSplitD + j]];
  __syncthreads();
  const int half = j >> 6, jj = j & 63;
  const float* rt = half ? rtr : rto;
  float a = 0.f;
#pragma unroll
  for (int i = 16 * quarter; i < 16 * quarter + 16; ++i) a = fmaf(rt[i * 64 + jj], qs[half * 64 + i], a);
  part_sum[quarter][j] = a;
  __syncthreads();
  if (tid < kSplitD) qws[bh * kSplitD + j] = (part_sum[0][j] + part_sum[1][j]) + (part_sum[2][j] + part_sum[3][j]);
}

// ---------------------------------------------------------------------------------------
// Scores: one thread per key (a block holds 256 consecutive tokens of one KV head).  The block
// first stages the rotated queries of the KV head's query heads in LDS as [chunk][coordinate][4]
// (4 heads per chunk, absent heads as zeros), so that one broadcast 16-byte read gives a
// coordinate's 4 query values.  The thread loads its key's 2 BO + 2 BR words and two norms,
// decodes each coordinate with a centroid table in LDS (at most 16 entries in distinct banks,
// so lookups never conflict) and accumulates 4 heads per pass over the key.
// Score = s_o <R_o q_O, C_o[idx_o]> + s_r <R_r q_R, C_r[idx_r]>.
// ---------------------------------------------------------------------------------------
constexpr int kScoreThreads = 256;
constexpr int kMaxChunks = kSplitMaxRatio / 4;

// 8 coordinates at a time.  The group's (at most two) packed words and its LDS offsets pass
// through an empty asm that depends on the previous group's sums, so the optimizer cannot
// compute every field and issue every LDS read of the pass at its top (which needs a register
// per value and spills); each group decodes from its own copy of the words.
template <int B, int NW>
__device__ __forceinline__ void half_dot(const uint32_t (&w)[NW], const float* ctab, const float (*qs)[4],
                                         f32x4& acc) {
#pragma unroll
  for (int i0 = 0; i0 < 64; i0 += 8) {
    constexpr int kSpan = 8 * B;
    const int wlo = (i0 * B) >> 5, whi = (i0 * B + kSpan - 1) >> 5;
    uint32_t lo = w[wlo], hi = w[whi];
    int base = i0, cbase = 0;
    asm volatile("" : "+v"(lo), "+v"(hi), "+v"(base), "+v"(cbase), "+v"(acc.x), "+v"(acc.y), "+v"(acc.z), "+v"(acc.w));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = (i0 + k) * B - 32 * wlo;   // bit offset of the field from word wlo
      uint32_t f;
      if (p + B <= 32)
        f = lo >> p;
      else if (p >= 32)
        f = hi >> (p - 32);
      else
        f = (lo >> p) | (hi << (32 - p));
      const float c = ctab[cbase + (int)(f & ((1u << B) - 1u))];
      const f32x4 qv = *reinterpret_cast<const f32x4*>(qs[base + k]);
      acc.x = fmaf(qv.x, c, acc.x);
      acc.y = fmaf(qv.y, c, acc.y);
      acc.z = fmaf(qv.z, c, acc.z);
      acc.w = fmaf(qv.w, c, acc.w);
    }
  }
}

template <int BO, int BR>
__global__ __launch_bounds__(kScoreThreads) void k_scores_split_d128(
    const float* __restrict__ qws, int Hq, int Hkv, int64_t T, int64_t seq_stride, CodebookArgs cbo, CodebookArgs cbr,
    const uint32_t* __restrict__ idx_o, const float* __restrict__ norm_o, const uint32_t* __restrict__ idx_r,
    const float* __restrict__ norm_r, float* __restrict__ scores) {
  constexpr int WO = 2 * BO, WR = 2 * BR;
  __shared__ float ctab[2][kMaxCentroids];
  __shared__ __align__(16) float qs[kMaxChunks][kSplitD][4];
  const int tid = threadIdx.x;
  const int64_t seq = blockIdx.y;
  const int b = (int)(seq / Hkv), hk = (int)(seq % Hkv);
  const int ratio = Hq / Hkv;
  const int nchunks = (ratio + 3) >> 2;
  const int64_t hq_first = (int64_t)b * Hq + (int64_t)hk * ratio;
  if (tid < kMaxCentroids)
    ctab[0][tid] = cbo.c[tid];
  else if (tid < 2 * kMaxCentroids)
    ctab[1][tid - kMaxCentroids] = cbr.c[tid - kMaxCentroids];
  for (int e = tid; e < nchunks * kSplitD * 4; e += kScoreThreads) {
    const int g = e & 3, i = (e >> 2) & (kSplitD - 1), c = e >> 9;
    const int head = 4 * c + g;
    qs[c][i][g] = head < ratio ? qws[(hq_first + head) * kSplitD + i] : 0.f;
  }
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kScoreThreads + tid;
  const bool live = t < T;
  const int64_t row = seq * seq_stride + (live ? t : T - 1);
  uint32_t wo[WO], wr[WR];
#pragma unroll
  for (int i = 0; i < WO; i += 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(idx_o + row * WO + i);
    wo[i] = v.x;
    wo[i + 1] = v.y;
  }
#pragma unroll
  for (int i = 0; i < WR; i += 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(idx_r + row * WR + i);
    wr[i] = v.x;
    wr[i + 1] = v.y;
  }
  const float so = norm_o[row], sr = norm_r[row];
  for (int c = 0; c < nchunks; ++c) {
    // The words are opaque to the optimizer here, so it decodes them again in every pass rather
    // than hoisting all 128 decoded centroids out of the loop into registers.
#pragma unroll
    for (int k = 0; k < WO; ++k) asm volatile("" : "+v"(wo[k]));
#pragma unroll
    for (int k = 0; k < WR; ++k) asm volatile("" : "+v"(wr[k]));
    f32x4 ao = {0.f, 0.f, 0.f, 0.f}, ar = {0.f, 0.f, 0.f, 0.f};
    half_dot<BO>(wo, ctab[0], &qs[c][0], ao);
    half_dot<BR>(wr, ctab[1], &qs[c][64], ar);
    const float r[4] = {so * ao.x + sr * ar.x, so * ao.y + sr * ar.y, so * ao.z + sr * ar.z, so * ao.w + sr * ar.w};
    if (live) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (4 * c + g < ratio) scores[(hq_first + 4 * c + g) * T + t] = r[g];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Split scores on the fp16 matrix cores.  Grid (key chunk, b * Hkv), 4 waves; a wave scores
// tiles of 16 keys.  D = A B per 16-key tile with A = 16 query slots (rows 0-3: the rotated
// query's fp16 hi part of 4 heads, rows 4-7 its lo part, rows 8-15 zero) and B = the 16 keys'
// decoded centroids.  Each half's 64 coordinates are two 32-term instructions; lane (n, g) of
// instruction s supplies coordinates 32 s + 8 g .. 32 s + 8 g + 7 of the half for key n: one
// run of 8 B-bit indices, cut from two adjacent words by one funnel shift and decoded through the
// half's replicated LDS table, so every lane decodes the same widths (no divergence between the
// halves).  The two halves accumulate apart (their norms differ); s_o D_o + s_r D_r is then
// reduced over the parts with the lane swaps of the single-code kernel, which leaves head g's
// score of key n in lane (n, g).  Keys are read once for every query head of their KV head:
// MULTI (more than 4 query heads per KV head) keeps the query operands of all groups of 4 heads
// in LDS and runs the groups on the decoded keys.
// ---------------------------------------------------------------------------------------
constexpr int kSplitScoreWaves = 4;
constexpr int kSplitTileBatch = 4;        // tiles loaded before any of them is scored
constexpr int kSplitTableBudget = 16384;  // LDS bytes per half's decode table

// Run s of lane group g in a half of B bits starts at bit (32 s + 8 g) B of the half's 2B-word
// row.  The lane loads the two words from run_word on (never past the row: the last run lies in
// the row's last word, so it is read as the high word of a pair) and shifts the pair right by
// run_shift.
template <int B>
__device__ __forceinline__ uint32_t run_word(int s, int g) {
  const uint32_t w = (uint32_t)((32 * s + 8 * g) * B) >> 5;
  return w < 2u * B - 2u ? w : 2u * B - 2u;
}
template <int B>
__device__ __forceinline__ uint32_t run_shift(int s, int g) {
  return (uint32_t)((32 * s + 8 * g) * B) - 32u * run_word<B>(s, g);
}
__device__ __forceinline__ uint32_t pair_bits(uint32_t lo, uint32_t hi, uint32_t sh) {
  return (uint32_t)((((uint64_t)hi << 32) | lo) >> sh);
}

// 8 indices of B bits in the low 8B bits of f, decoded into 8 fp16 centroids (one operand)
// through the lane's copy of the table (addresses base + (field * stride | laneoff)).
template <int B, int COPIES>
__device__ __forceinline__ u32x4 decode_run(uint32_t f, const uint8_t* tab, uint32_t laneoff) {
  using DT = DecodeTable<B, false, COPIES>;
  constexpr uint32_t S = DT::STRIDE;
  static_assert((S & (S - 1)) == 0, "field stride must be a power of two");
  auto at = [&](uint32_t field) { return tab + ((field * S) | laneoff); };
  u32x4 out;
  if constexpr (B == 1) {
    out = *reinterpret_cast<const u32x4*>(at(f & 0xffu));
  } else if constexpr (B == 2) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(at(f & 0xffu));
    const u32x2 b = *reinterpret_cast<const u32x2*>(at((f >> 8) & 0xffu));
    out = u32x4{a[0], a[1], b[0], b[1]};
  } else if constexpr (B == 3) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(at((f >> (6 * j)) & 63u));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const uint32_t*>(at((f >> (8 * j)) & 0xffu));
  }
  return out;
}

// A key tile's share for lane (n, g): for each half and run the two words holding the run, and
// the key's two norms.
struct SplitTile {
  uint32_t w[2][2][2];   // [half][run][lo, hi word]
  float so, sr;
};

template <int BO, int BR, bool MULTI>
__global__ __launch_bounds__(kSplitScoreWaves * 64, 2) void k_scores_split_mfma(
    const float* __restrict__ qws, int Hq, int Hkv, int64_t T, int64_t seq_stride, int tiles_per_wave,
    CodebookArgs cbo, CodebookArgs cbr, const uint32_t* __restrict__ idx_o, const float* __restrict__ norm_o,
    const uint32_t* __restrict__ idx_r, const float* __restrict__ norm_r, float* __restrict__ scores) {
  constexpr int TCO = table_copies<BO, false, kSplitTableBudget>();
  constexpr int TCR = table_copies<BR, false, kSplitTableBudget>();
  using DO = DecodeTable<BO, false, TCO>;
  using DR = DecodeTable<BR, false, TCR>;
  constexpr int WO = 2 * BO, WR = 2 * BR;   // words per half row
  __shared__ __attribute__((aligned(16))) uint8_t tabo[DO::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tabr[DR::BYTES];
  __shared__ _Float16 cent[2][16];
  // MULTI: the query operands of every head of the KV head, [head][part][instruction][lane group]
  __shared__ u32x4 qa[MULTI ? kSplitMaxRatio : 1][2][4][4];
  const int ratio = Hq / Hkv;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int64_t hq_first = (int64_t)b * Hq + (int64_t)kvh * ratio;
  if (threadIdx.x < 16) cent[0][threadIdx.x] = (_Float16)cbo.c[threadIdx.x];
  else if (threadIdx.x < 32) cent[1][threadIdx.x - 16] = (_Float16)cbr.c[threadIdx.x - 16];
  // The query operand of (head, part p, instruction i = 2 half + s, lane group g): coordinates
  // 64 half + 32 s + 8 g .. + 7 of the head's rotated query, fp16 hi (p = 0) or lo (p = 1).
  auto qfrag = [&](int head, int p, int i, int g) -> u32x4 {
    const float* src = qws + (hq_first + head) * kSplitD + 64 * (i >> 1) + 32 * (i & 1) + 8 * g;
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = src[2 * k], x1 = src[2 * k + 1];
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      const _Float16 e0 = p ? (_Float16)(x0 - (float)h0) : h0;
      const _Float16 e1 = p ? (_Float16)(x1 - (float)h1) : h1;
      v[k] = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
    }
    return v;
  };
  if constexpr (MULTI) {
    for (int e = threadIdx.x; e < ratio * 32; e += blockDim.x) {
      const int head = e >> 5, p = (e >> 4) & 1, i = (e >> 2) & 3, g = e & 3;
      qa[head][p][i][g] = qfrag(head, p, i, g);
    }
  }
  __syncthreads();
  build_table<BO, TCO>(tabo, cent[0]);
  build_table<BR, TCR>(tabr, cent[1]);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t lofo = (uint32_t)(lane % TCO) * DO::EB, lofr = (uint32_t)(lane % TCR) * DR::EB;
  const int64_t base_row = (int64_t)bg * seq_stride;
  const int64_t ntiles_seq = (T + 15) / 16;
  const int64_t tile0 = ((int64_t)blockIdx.x * kSplitScoreWaves + wave) * tiles_per_wave;
  int64_t last = tiles_per_wave;
  if (ntiles_seq - tile0 < last) last = ntiles_seq - tile0;
  // this (batch, kv head)'s score rows, ratio x T floats (the host bounds Hq * T * 4 < 4 GB)
  const __amdgpu_buffer_rsrc_t sbuf = buffer_rsrc(scores + hq_first * T, (uint32_t)ratio * (uint32_t)T * 4u);

  // query operands of head group 0 in registers (single group) -- row n = 4 part + head
  const int hl = nl & 3, part = nl >> 2;
  u32x4 a0[4];
  if constexpr (!MULTI) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a0[i] = (part < 2 && hl < ratio) ? qfrag(hl, part, i, g) : u32x4{0u, 0u, 0u, 0u};
  }
  // the lane's word offsets within a key's half row, per run
  const uint32_t wio0 = run_word<BO>(0, g), wio1 = run_word<BO>(1, g);
  const uint32_t wir0 = run_word<BR>(0, g), wir1 = run_word<BR>(1, g);
  const uint32_t sho0 = run_shift<BO>(0, g), sho1 = run_shift<BO>(1, g);
  const uint32_t shr0 = run_shift<BR>(0, g), shr1 = run_shift<BR>(1, g);

  for (int64_t tb = 0; tb < last; tb += kSplitTileBatch) {
    // resources based at the batch's first key and ending at the wave's last tile (or the
    // sequence's end): loads past them read zero without touching memory
    const int64_t first = (tile0 + tb) * 16;
    int64_t rem = T - first;
    if ((last - tb) * 16 < rem) rem = (last - tb) * 16;
    const uint32_t nk = rem > 0 ? (uint32_t)rem : 0u;
    const int64_t row = base_row + first;
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(idx_o + row * WO, nk * (4u * WO));
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(idx_r + row * WR, nk * (4u * WR));
    const __amdgpu_buffer_rsrc_t no = buffer_rsrc(norm_o + row, nk * 4u);
    const __amdgpu_buffer_rsrc_t nr = buffer_rsrc(norm_r + row, nk * 4u);
    SplitTile kt[kSplitTileBatch];
#pragma unroll
    for (int u = 0; u < kSplitTileBatch; ++u) {
      const uint32_t k = (uint32_t)(16 * u + nl);
      const u32x2 o0 = __builtin_amdgcn_raw_buffer_load_b64(ro, (k * WO + wio0) * 4u, 0, 0);
      const u32x2 o1 = __builtin_amdgcn_raw_buffer_load_b64(ro, (k * WO + wio1) * 4u, 0, 0);
      const u32x2 r0 = __builtin_amdgcn_raw_buffer_load_b64(rr, (k * WR + wir0) * 4u, 0, 0);
      const u32x2 r1 = __builtin_amdgcn_raw_buffer_load_b64(rr, (k * WR + wir1) * 4u, 0, 0);
      kt[u].w[0][0][0] = o0[0]; kt[u].w[0][0][1] = o0[1];
      kt[u].w[0][1][0] = o1[0]; kt[u].w[0][1][1] = o1[1];
      kt[u].w[1][0][0] = r0[0]; kt[u].w[1][0][1] = r0[1];
      kt[u].w[1][1][0] = r1[0]; kt[u].w[1][1][1] = r1[1];
      kt[u].so = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(no, k * 4u, 0, 0));
      kt[u].sr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(nr, k * 4u, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kSplitTileBatch; ++u) {
      if (tb + u >= last) break;
      const SplitTile& c = kt[u];
      u32x4 bo[2], br[2];
      bo[0] = decode_run<BO, TCO>(pair_bits(c.w[0][0][0], c.w[0][0][1], sho0), tabo, lofo);
      bo[1] = decode_run<BO, TCO>(pair_bits(c.w[0][1][0], c.w[0][1][1], sho1), tabo, lofo);
      br[0] = decode_run<BR, TCR>(pair_bits(c.w[1][0][0], c.w[1][0][1], shr0), tabr, lofr);
      br[1] = decode_run<BR, TCR>(pair_bits(c.w[1][1][0], c.w[1][1][1], shr1), tabr, lofr);
      const uint32_t t = (uint32_t)(tile0 + tb + u) * 16u + (uint32_t)nl;
      const bool valid = t < (uint32_t)T;
      const int groups = MULTI ? (ratio + 3) / 4 : 1;
      for (int hg = 0; hg < groups; ++hg) {
        u32x4 a[4];
        if constexpr (MULTI) {
          const int head = 4 * hg + hl;
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = (part < 2 && head < ratio) ? qa[head][part][i][g] : u32x4{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = a0[i];
        }
        f32x4 ao = f32x4{0.f, 0.f, 0.f, 0.f}, ar = f32x4{0.f, 0.f, 0.f, 0.f};
        ao = mfma_f16(a[0], bo[0], ao);
        ao = mfma_f16(a[1], bo[1], ao);
        ar = mfma_f16(a[2], br[0], ar);
        ar = mfma_f16(a[3], br[1], ar);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(c.so, ao[r], c.sr * ar[r]);
        const float mine = reduce_parts(v[0], v[1], v[2], v[3]);
        const int h = 4 * hg + g;
        if (valid && h < ratio)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mine), sbuf,
                                                ((uint32_t)h * (uint32_t)T + t) * 4u, 0, 0);
      }
    }
  }
}

// Calls f(IC<BO>, IC<BR>) for bit widths 1..4 each.
template <int BO, typename F>
hipError_t with_br(int br, F&& f) {
  switch (br) {
    case 1: return f(IC<BO>{}, IC<1>{});
    case 2: return f(IC<BO>{}, IC<2>{});
    case 3: return f(IC<BO>{}, IC<3>{});
    case 4: return f(IC<BO>{}, IC<4>{});
  }
  return hipErrorInvalidValue;
}

template <typename F>
hipError_t with_bits(int bo, int br, F&& f) {
  switch (bo) {
    case 1: return with_br<1>(br, f);
    case 2: return with_br<2>(br, f);
    case 3: return with_br<3>(br, f);
    case 4: return with_br<4>(br, f);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode_split(const void* x, bool bf16, int64_t n_seq, int H, int64_t T, int64_t out_stride,
                               int64_t pos, const int32_t* order, const float* ro, const float* rr, const float* rto,
                               const float* rtr, const CodebookArgs& cbo, const CodebookArgs& cbr, uint32_t* idx_o,
                               float* norm_o, uint32_t* idx_r, float* norm_r, hipStream_t st) {
  if (n_seq <= 0 || T <= 0) return hipSuccess;
  if (T <= kSplitTokenMax) {
    const dim3 tgrid((unsigned)T, (unsigned)n_seq);
    return with_bits(cbo.bits, cbr.bits, [&](auto bo, auto br) -> hipError_t {
      constexpr int BO = decltype(bo)::value, BR = decltype(br)::value;
      if (bf16)
        hipLaunchKernelGGL((k_append_split_token<BO, BR, true>), tgrid, dim3(128), 0, st, x, T, out_stride, pos, H,
                           order, rto, rtr, cbo, cbr, idx_o, norm_o, idx_r, norm_r);
      else
        hipLaunchKernelGGL((k_append_split_token<BO, BR, false>), tgrid, dim3(128), 0, st, x, T, out_stride, pos, H,
                           order, rto, rtr, cbo, cbr, idx_o, norm_o, idx_r, norm_r);
      return hipGetLastError();
    });
  }
  const dim3 grid((unsigned)((T + kEncBlockRows - 1) / kEncBlockRows), (unsigned)n_seq);
  return with_bits(cbo.bits, cbr.bits, [&](auto bo, auto br) -> hipError_t {
    constexpr int BO = decltype(bo)::value, BR = decltype(br)::value;
    if (bf16)
      hipLaunchKernelGGL((k_encode_split_d128<BO, BR, true>), grid, dim3(kEncWaves * 64), 0, st, x, T, out_stride, pos,
                         H, order, ro, rr, cbo, cbr, idx_o, norm_o, idx_r, norm_r);
    else
      hipLaunchKernelGGL((k_encode_split_d128<BO, BR, false>), grid, dim3(kEncWaves * 64), 0, st, x, T, out_stride, pos,
                         H, order, ro, rr, cbo, cbr, idx_o, norm_o, idx_r, norm_r);
    return hipGetLastError();
  });
}

hipError_t launch_qprep_split(const float* q, int B, int Hq, int Hkv, const int32_t* order, const float* rto,
                              const float* rtr, float* qws, hipStream_t st) {
  if ((int64_t)B * Hq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_qprep_split, dim3((unsigned)((int64_t)B * Hq)), dim3(512), 0, st, q, Hq, Hkv, order, rto, rtr,
                     qws);
  return hipGetLastError();
}

#ifndef TQ_SPLIT_SCORE_MFMA
#define TQ_SPLIT_SCORE_MFMA 1
#endif
#ifndef TQ_SPLIT_BLOCKS_PER_CU
#define TQ_SPLIT_BLOCKS_PER_CU 4
#endif

hipError_t launch_scores_split(const float* qws, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride, int bo, int br,
                               const CodebookArgs& cbo, const CodebookArgs& cbr, const uint32_t* idx_o,
                               const float* norm_o, const uint32_t* idx_r, const float* norm_r, float* scores,
                               hipStream_t st) {
  if ((int64_t)B * Hkv == 0 || T <= 0) return hipSuccess;
  if (!TQ_SPLIT_SCORE_MFMA) {
    const dim3 grid((unsigned)((T + kScoreThreads - 1) / kScoreThreads), (unsigned)((int64_t)B * Hkv));
    return with_bits(bo, br, [&](auto o, auto r) -> hipError_t {
      hipLaunchKernelGGL((k_scores_split_d128<decltype(o)::value, decltype(r)::value>), grid, dim3(kScoreThreads), 0,
                         st, qws, Hq, Hkv, T, seq_stride, cbo, cbr, idx_o, norm_o, idx_r, norm_r, scores);
      return hipGetLastError();
    });
  }
  // grid: TQ_SPLIT_BLOCKS_PER_CU blocks per CU over all sequences, whole batches of tiles per
  // wave (each block builds two decode tables first, so a block wants tiles enough to amortise them)
  const int64_t tiles = (T + 15) / 16;
  const int64_t seqs = (int64_t)B * Hkv;
  const int64_t target = (int64_t)num_cus() * TQ_SPLIT_BLOCKS_PER_CU;
  int64_t tpw = (tiles * seqs + target * kSplitScoreWaves - 1) / (target * kSplitScoreWaves);
  tpw = (tpw + kSplitTileBatch - 1) / kSplitTileBatch * kSplitTileBatch;
  if (tpw < kSplitTileBatch) tpw = kSplitTileBatch;
  if (tpw > 256) tpw = 256;
  const int64_t chunks = (tiles + tpw * kSplitScoreWaves - 1) / (tpw * kSplitScoreWaves);
  const dim3 grid((unsigned)chunks, (unsigned)seqs);
  const bool multi = Hq / Hkv > 4;
  return with_bits(bo, br, [&](auto o, auto r) -> hipError_t {
    constexpr int BO = decltype(o)::value, BR = decltype(r)::value;
    if (multi)
      hipLaunchKernelGGL((k_scores_split_mfma<BO, BR, true>), grid, dim3(kSplitScoreWaves * 64), 0, st, qws, Hq, Hkv, T,
                         seq_stride, (int)tpw, cbo, cbr, idx_o, norm_o, idx_r, norm_r, scores);
    else
      hipLaunchKernelGGL((k_scores_split_mfma<BO, BR, false>), grid, dim3(kSplitScoreWaves * 64), 0, st, qws, Hq, Hkv,
                         T, seq_stride, (int)tpw, cbo, cbr, idx_o, norm_o, idx_r, norm_r, scores);
    return hipGetLastError();
  });
}

}  // namespace tq
