// Prefill attention fused with the compressed cache, d = 128 ("TurboQuant 详解", KV-cache
// example: the prompt's keys and values are compressed as they are written; decode section, second
// route: the cache is unpacked and looked up inside the attention, never materialised;
// "TurboQuant 和 RotorQuant 的真相", Flash Attention fusion section).  A chunk of n_new tokens has
// already been appended to the key cache (rows layout) and the value cache (token-blocked layout)
// at positions pos ..; the query of chunk token i attends causally to cached tokens 0 .. pos + i.
//
// Flash-attention shape on the fp16 matrix cores, everything in the caches' rotated domains:
//   scores^T = K_hat Q^T   A = 16 keys decoded from their packed rows (fp16 centroid hi, and the
//                          remainder lo), B = 16 query tokens' R_K q (fp16 hi and lo);
//                          three products (Khi Qhi + Klo Qhi + Khi Qlo) per 32 coordinates.
//   O^T += V_hat^T P^T     A = value chunks (8 tokens of one coordinate) decoded from the staged
//                          value block, B = the softmax weights times the value norms in fp16
//                          hi and lo (two products).
// With 16-key tile t's A rows laid out as keys 8 (i / 4) + 4 t + i % 4, the scores of a lane
// (query n, lane group g) over a 32-key step are keys 8 g .. 8 g + 7: exactly the B operand the
// P V product needs, so the weights never leave the lane's registers, and each query's softmax
// reductions are across the four lane groups only.
// A block is four waves of one (batch, kv head); each wave takes one (pair of query heads of the
// kv head, 16-token tile) item: the two heads see the same keys, values and causal mask, so each
// decoded key and value operand feeds both heads' products.  The block's 32-key steps of packed
// keys, values and norms are staged in LDS (double buffered) and shared by its waves.  The output stays in V's rotated domain; k_prefill_unrotate
// applies R_V^T row by row.
#include <hip/hip_runtime.h>

#include "tq_cache.h"
#include "tq_decode.h"

namespace tq {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTok = 16;          // query tokens of a wave's item
// LDS budgets of the three decode tables (K centroid hi, K remainder lo, V).
constexpr int kPfTableBudget = 12288;

template <int KB, int VB>
__global__ __launch_bounds__(kPfWaves * 64, 2) void k_prefill_attn(
    float* qo, int Hq, int Hkv, int64_t n_new, int64_t pos,
    int64_t t_cap, const uint32_t* __restrict__ kidx, const float* __restrict__ knorm,
    const uint32_t* __restrict__ vidx, const float* __restrict__ vnorm, CodebookArgs cbk, CodebookArgs cbv,
    float scale) {
  constexpr int KC = table_copies<KB, false, kPfTableBudget>();
  constexpr int VC = table_copies<VB, false, kPfTableBudget>();
  using DK = DecodeTable<KB, false, KC>;
  using DV = DecodeTable<VB, false, VC>;
  constexpr int KW = 32 * 4 * KB;        // words of a step's 32 key rows
  constexpr int VW = 128 * VB;           // words of a step's value block
  __shared__ __attribute__((aligned(16))) uint8_t ktab_h[DK::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ktab_l[DK::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vtab[DV::BYTES];
  __shared__ _Float16 cent[3][16];
  // staging, double buffered: key rows, value block (one word of padding for the last chunk's
  // two-word read), key norms, value norms
  __shared__ __attribute__((aligned(16))) uint32_t kst[2][KW];
  __shared__ __attribute__((aligned(16))) uint32_t vst[2][VW + 4];
  __shared__ float knst[2][32], vnst[2][32];

  if (threadIdx.x < 16) {
    const float ck = cbk.c[threadIdx.x];
    const _Float16 hk = (_Float16)ck;
    cent[0][threadIdx.x] = hk;
    cent[1][threadIdx.x] = (_Float16)(ck - (float)hk);
    cent[2][threadIdx.x] = (_Float16)cbv.c[threadIdx.x];
  }
  if (threadIdx.x < 8) {
    vst[0][VW + (threadIdx.x & 3)] = 0u;
    vst[1][VW + (threadIdx.x & 3)] = 0u;
  }
  __syncthreads();
  build_table<KB, KC>(ktab_h, cent[0]);
  build_table<KB, KC>(ktab_l, cent[1]);
  build_table<VB, VC>(vtab, cent[2]);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const uint8_t* kth = DK::lane_base(ktab_h, lane);
  const uint8_t* ktl = DK::lane_base(ktab_l, lane);
  const uint8_t* vtl = DV::lane_base(vtab, lane);
  const int bh = blockIdx.y;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int ratio = Hq / Hkv;
  const int hp = (ratio + 1) / 2;                    // head pairs per kv head
  const int64_t ntile = (n_new + kPfTok - 1) / kPfTok;
  // this wave's item: (16-token tile tau, heads 2 pr and 2 pr + 1 of the kv head), tau-major
  const int64_t item = (int64_t)blockIdx.x * kPfWaves + wave;
  const int64_t tau = item / hp;
  const int pr = (int)(item % hp);
  const bool live = tau < ntile;
  const bool live1 = live && 2 * pr + 1 < ratio;     // an odd ratio leaves the last pair one head
  const int hjs[2] = {2 * pr, live1 ? 2 * pr + 1 : 2 * pr};
  const int64_t tok0 = tau * kPfTok;
  // the block's last live tile bounds the keys it needs: tokens 0 .. pos + (its last token)
  int64_t tau_max = ((int64_t)blockIdx.x * kPfWaves + kPfWaves - 1) / hp;
  if (tau_max > ntile - 1) tau_max = ntile - 1;
  const int64_t last_tok = (tau_max + 1) * kPfTok < n_new ? (tau_max + 1) * kPfTok - 1 : n_new - 1;
  const int64_t kend = pos + last_tok + 1;            // keys [0, kend)
  const int64_t nsteps = (kend + 31) >> 5;
  // keys this wave needs: [0, pos + tok0 + 16)
  const int64_t wave_keys = pos + tok0 + kPfTok;
  const int64_t row0 = (int64_t)bh * t_cap;

  // B operands of the key product: R_K q of query token tok0 + n of each head (qo, fp32), coordinates
  // 32 g + 8 s .. + 7, as fp16 hi and lo.  Only this wave reads or writes these rows of qo.
  u32x4 bqh[2][4], bql[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int64_t tq = tok0 + nl < n_new ? tok0 + nl : n_new - 1;
    const int64_t qrow = (((int64_t)b * Hq + kvh * ratio + hjs[hh]) * n_new + (live ? tq : 0));
    const f32x4* src = reinterpret_cast<const f32x4*>(qo + qrow * 128 + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 v0 = src[2 * s], v1 = src[2 * s + 1];
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const _Float16 h0 = (_Float16)v[2 * k], h1 = (_Float16)v[2 * k + 1];
        const _Float16 l0 = (_Float16)(v[2 * k] - (float)h0), l1 = (_Float16)(v[2 * k + 1] - (float)h1);
        bqh[hh][s][k] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        bql[hh][s][k] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
    }
  }
  const int64_t my_tok = pos + tok0 + nl;             // absolute position of the lane's query
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 o[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[hh][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // cooperative staging of step st: u32x4 units 0 .. KW/4 - 1 keys, then VW/4 value words, then
  // 8 + 8 units of norms
  constexpr int kUK = KW / 4, kUV = VW / 4, kUnits = kUK + kUV + 16;
  constexpr int kPer = (kUnits + kPfWaves * 64 - 1) / (kPfWaves * 64);
  u32x4 stg[kPer];
  auto fetch = [&](int64_t st) {
    const int64_t key0 = st * 32;
    const u32x4* ksrc = reinterpret_cast<const u32x4*>(kidx + (row0 + key0) * (4 * KB));
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(vidx + ((row0 + key0) >> 5) * (128 * VB));
    const u32x4* knsrc = reinterpret_cast<const u32x4*>(knorm + row0 + key0);
    const u32x4* vnsrc = reinterpret_cast<const u32x4*>(vnorm + row0 + key0);
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = threadIdx.x + p * kPfWaves * 64;
      if (u < kUK) stg[p] = ksrc[u];
      else if (u < kUK + kUV) stg[p] = vsrc[u - kUK];
      else if (u < kUK + kUV + 8) stg[p] = knsrc[u - kUK - kUV];
      else if (u < kUnits) stg[p] = vnsrc[u - kUK - kUV - 8];
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = threadIdx.x + p * kPfWaves * 64;
      if (u < kUK) reinterpret_cast<u32x4*>(kst[buf])[u] = stg[p];
      else if (u < kUK + kUV) reinterpret_cast<u32x4*>(vst[buf])[u - kUK] = stg[p];
      else if (u < kUK + kUV + 8) reinterpret_cast<u32x4*>(knst[buf])[u - kUK - kUV] = stg[p];
      else if (u < kUnits) reinterpret_cast<u32x4*>(vnst[buf])[u - kUK - kUV - 8] = stg[p];
    }
  };

  if (nsteps > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int64_t st = 0; st < nsteps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nsteps) fetch(st + 1);
    const int64_t key0 = st * 32;
    if (live && key0 < wave_keys) {
      // ---- scores^T for the step's 32 keys, both heads: tile t, lane (query nl, group g), register
      // r is key 8 g + 4 t + r
      float s[2][8];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kl = 8 * (nl >> 2) + 4 * t + (nl & 3);     // this lane's A row (key) of tile t
        uint32_t kw[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) kw[j] = kst[buf][kl * (4 * KB) + KB * g + j];
        f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x4 ah = decode_keys<KB, KC>(kw, q4, kth);
          const u32x4 al = decode_keys<KB, KC>(kw, q4, ktl);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            d[hh] = mfma_f16(ah, bqh[hh][q4], d[hh]);
            d[hh] = mfma_f16(al, bqh[hh][q4], d[hh]);
            d[hh] = mfma_f16(ah, bql[hh][q4], d[hh]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = 8 * g + 4 * t + r;
          const int64_t key = key0 + k;
          const bool vis = key <= my_tok;
          const float kn = knst[buf][k] * scale;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) s[hh][4 * t + r] = vis ? d[hh][r] * kn : -INFINITY;
        }
      }
      // ---- online softmax of query nl per head (its 32 keys are spread over the four lane groups)
      u32x4 bph[2], bpl[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float mx = s[hh][0];
#pragma unroll
        for (int k = 1; k < 8; ++k) mx = fmaxf(mx, s[hh][k]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[hh], mx);
        const float alpha = m_new == -INFINITY ? 1.f : __expf(m_run[hh] - m_new);
        float psum = 0.f;
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const float p0 = s[hh][k] == -INFINITY ? 0.f : __expf(s[hh][k] - m_new);
          const float p1 = s[hh][k + 1] == -INFINITY ? 0.f : __expf(s[hh][k + 1] - m_new);
          psum += p0 + p1;
          // masked keys give exactly 0 (rows past the written prefix may hold any bits, NaN norms too)
          const float w0 = s[hh][k] == -INFINITY ? 0.f : p0 * vnst[buf][8 * g + k];
          const float w1 = s[hh][k + 1] == -INFINITY ? 0.f : p1 * vnst[buf][8 * g + k + 1];
          const _Float16 h0 = (_Float16)w0, h1 = (_Float16)w1;
          const _Float16 r0 = (_Float16)(w0 - (float)h0), r1 = (_Float16)(w1 - (float)h1);
          ph[k >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          pl[k >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16);
        }
        l_run[hh] = fmaf(l_run[hh], alpha, psum);
        m_run[hh] = m_new;
        if (alpha < 1.f) {
#pragma unroll
          for (int c = 0; c < 8; ++c) o[hh][c] *= alpha;
        }
        bph[hh] = u32x4{ph[0], ph[1], ph[2], ph[3]};
        bpl[hh] = u32x4{pl[0], pl[1], pl[2], pl[3]};
      }
      // ---- O^T += V_hat^T P^T: A row m of block c is coordinate 16 c + m; lane (m, g) holds
      // the chunk of octet g (keys 8 g .. 8 g + 7) at that coordinate; one decode, both heads
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int off = ((g * 128 + 16 * c + nl) * 8 * VB);
        const uint32_t w2[2] = {vst[buf][off >> 5], vst[buf][(off >> 5) + 1]};
        const u32x4 av = decode8<VB, VC>(w2, off & 31, vtl);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          o[hh][c] = mfma_f16(av, bph[hh], o[hh][c]);
          o[hh][c] = mfma_f16(av, bpl[hh], o[hh][c]);
        }
      }
    }
    if (st + 1 < nsteps) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- the lane's query nl of each head: its sum over the four lane groups; coordinates
  // 16 c + 4 g + r
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float l = l_run[hh];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (live && (hh == 0 || live1) && tok0 + nl < n_new) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* dst = qo + ((((int64_t)b * Hq + kvh * ratio + hjs[hh]) * n_new) + tok0 + nl) * 128;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[16 * c + 4 * g + r] = o[hh][c][r] * inv;
    }
  }
}

template <int KB, int VB>
hipError_t prefill_launch(int B, int Hq, int Hkv, int64_t n_new, int64_t pos, int64_t t_cap, const tq_packed* K,
                          const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv, float scale,
                          float* qo, hipStream_t st) {
  const int ratio = Hq / Hkv;
  const int64_t items = (n_new + kPfTok - 1) / kPfTok * ((ratio + 1) / 2);
  const int64_t blocks = (items + kPfWaves - 1) / kPfWaves;
  hipLaunchKernelGGL((k_prefill_attn<KB, VB>), dim3((unsigned)blocks, (unsigned)(B * Hkv)), dim3(kPfWaves * 64), 0, st,
                     qo, Hq, Hkv, n_new, pos, t_cap, K->idx, K->norms, V->idx, V->norms, cbk, cbv, scale);
  return hipGetLastError();
}

}  // namespace

size_t prefill_attn_workspace_bytes(int B, int Hq, int64_t n_new) {
  // R_K q in fp32 for every query row (later the output in V's rotated domain)
  const size_t rows = (size_t)B * Hq * (size_t)n_new;
  return (rows * 128 * sizeof(float) + 255) & ~(size_t)255;
}

hipError_t launch_prefill_attn(const float* q, int B, int Hq, int Hkv, int64_t n_new, int64_t pos, int64_t t_cap,
                               const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk,
                               const CodebookArgs& cbv, const tq_rotation_s* rot_k, const tq_rotation_s* rot_v,
                               float scale, float* out, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)B * Hq * n_new;
  float* qo = static_cast<float*>(ws);   // R_K q, then the attention output in V's rotated domain
  hipError_t e = launch_rotate_raw_d128(q, false, rows, rot_k, false, qo, st);
  if (e != hipSuccess) return e;
#define TQ_PF(KB, VB) \
  if (cbk.bits == KB && cbv.bits == VB) \
    e = prefill_launch<KB, VB>(B, Hq, Hkv, n_new, pos, t_cap, K, V, cbk, cbv, scale, qo, st); else
  TQ_PF(2, 2) TQ_PF(4, 4) TQ_PF(3, 3) TQ_PF(4, 2) TQ_PF(2, 4) TQ_PF(3, 2) TQ_PF(4, 3) TQ_PF(1, 1) TQ_PF(2, 3)
  TQ_PF(3, 4) return hipErrorInvalidValue;
#undef TQ_PF
  if (e != hipSuccess) return e;
  return launch_rotate_raw_d128(qo, false, rows, rot_v, true, out, st);
}

}  // namespace tq
