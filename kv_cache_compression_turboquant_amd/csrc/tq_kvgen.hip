// KV-side kernels for head dims other than 128 (d = 64 and d = 256): the query prologue, the
// compressed-key scores and decode attention, and the d = 64 encode.  The d = 128 path has its
// own tuned kernels; these follow the same formulas with a simpler thread layout.
//
// Scores ([TQ] TurboQuant_mse / TurboQuant_prod inner products; [FP] inner-product bias and the
// QJL fix): <q, k~> = s <R q, C[idx]> (+ gamma sqrt(pi/2)/d <S q, z> for prod keys), with R q and
// S q formed once per query head in fp32.  A thread takes one key: its packed words stay in
// registers while the block's query heads (staged in LDS, eight at a time) are multiplied.
//
// Decode attention ("TurboQuant 和 RotorQuant 的真相", the attention formula; "TurboQuant 详解",
// decode with dequantization inside the kernel): softmax(scale q K^T) V over packed K and V in the
// rows layout.  A block takes a range of one sequence in tiles of 256 keys: logits thread by key,
// an online softmax per query head, then P V in V's rotated domain with each thread owning one
// coordinate (and a phase of the tile's keys) over the tile's value words staged in LDS.  Partials
// per range are merged by a second kernel, which also rotates back by R_V^T.
//
// Encode at d = 64 ([TQ] official steps 1-5 and TurboQuant_prod): one wave per vector, lane i
// owning coordinate i; y = R x, the residual's R^T and the sketch S are matrix-vector products
// with the matrices in LDS (64 x 64 fp32 each).
#include <type_traits>

#include "tq_device.h"

namespace tq {
namespace {

// Compile-time loop B, B + 1, .., E - 1 (the body gets std::integral_constant indices).
template <int B, int E, typename F>
__device__ __forceinline__ void gen_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    gen_for<B + 1, E>(f);
  }
}

constexpr int kGenThreads = 256;
constexpr int kGenHeadGroup = 8;   // query heads staged at once
constexpr int kGenAttnTiles = 4;   // 256-key tiles per attention range

// ---------------------------------------------------------------------------------------
// Query prologue: ws[h] = {R q_h (d floats), S q_h (d floats)}; one block of d threads per head.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void k_qprep_gen(const float* __restrict__ q, const float* __restrict__ rt32,
                                                 const float* __restrict__ st32, float* __restrict__ ws) {
  __shared__ float qs[D];
  const int64_t h = blockIdx.x;
  const int i = threadIdx.x;
  qs[i] = q[h * D + i];
  __syncthreads();
  float a = 0.f, c = 0.f;
  // rt32[j][i] = R[i][j] and st32[j][i] = S[i][j]: thread i reads consecutive columns
  for (int j = 0; j < D; ++j) a = fmaf(rt32[(size_t)j * D + i], qs[j], a);
  if (st32)
    for (int j = 0; j < D; ++j) c = fmaf(st32[(size_t)j * D + i], qs[j], c);
  ws[h * 2 * D + i] = a;
  ws[h * 2 * D + D + i] = c;
}

// BITS-bit field of coordinate I (compile-time) of a packed row held in registers.
template <int BITS, int I, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int p = BITS * I, wi = p >> 5, sh = p & 31;
  uint32_t v = w[wi] >> sh;
  if constexpr (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

// One key: its packed row (indices; signs for prod), its norm and its residual norm.
template <int D, int BITS, bool PROD>
struct GenKey {
  static constexpr int W = D * BITS / 32;  // index words per key (BITS per 32-coordinate chunk)
  static constexpr int WZ = D / 32;        // sign words per key (one per chunk)
  const uint32_t* w;                       // the key's index words
  const uint32_t* z;                       // the key's sign words (prod)
  float s, g;
};

template <int D, int BITS, bool PROD>
__device__ __forceinline__ void load_gen_key(const uint32_t* __restrict__ idx, const float* __restrict__ norms,
                                             const uint32_t* __restrict__ qjl, const float* __restrict__ rnorms,
                                             int64_t row, bool valid, GenKey<D, BITS, PROD>& k) {
  using K = GenKey<D, BITS, PROD>;
  // an invalid key reads row 0's words (in bounds) and gets norm 0, so it scores 0
  const int64_t r = valid ? row : 0;
  k.w = idx + r * K::W;
  k.z = PROD ? qjl + r * K::WZ : nullptr;
  k.s = valid ? norms[r] : 0.f;
  k.g = (PROD && valid) ? rnorms[r] : 0.f;
}

// Raw scores of one key against NH heads whose R q (qr) and S q (qz) rows sit in LDS:
// out[k] = s <qr_k, C[idx]> + gamma sqrt(pi/2)/D <qz_k, z>.  C: centroids in LDS.  The key's words
// are read chunk by chunk (32 coordinates: BITS index words and one sign word).
template <int D, int BITS, bool PROD, int NH>
__device__ __forceinline__ void gen_key_scores(const GenKey<D, BITS, PROD>& key, const float* qr, const float* qz,
                                               const float* cent, int nh, float (&out)[NH]) {
  float acc[NH], accz[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    acc[k] = 0.f;
    accz[k] = 0.f;
  }
#pragma unroll 1
  for (int c = 0; c < D / 32; ++c) {
    uint32_t wc[BITS];
#pragma unroll
    for (int b = 0; b < BITS; ++b) wc[b] = key.w[c * BITS + b];
    const uint32_t zw = PROD ? key.z[c] : 0u;
    float cv[32];
    gen_for<0, 32>([&](auto ee) {
      constexpr int e = decltype(ee)::value;
      cv[e] = cent[field<BITS, e>(wc)];
    });
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      if (k < nh) {
        const f32x4* qr4 = reinterpret_cast<const f32x4*>(qr + k * 2 * D + 32 * c);
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4) {
          const f32x4 qv = qr4[e4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[k] = fmaf(qv[e], cv[4 * e4 + e], acc[k]);
        }
        if constexpr (PROD) {
          const f32x4* qz4 = reinterpret_cast<const f32x4*>(qz + k * 2 * D + 32 * c);
#pragma unroll
          for (int e4 = 0; e4 < 8; ++e4) {
            const f32x4 qv = qz4[e4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int bit = 4 * e4 + e;
              // z = +1 where the bit is set, -1 otherwise
              accz[k] += __uint_as_float(__float_as_uint(qv[e]) ^ (((~zw >> bit) & 1u) << 31));
            }
          }
        }
      }
    }
  }
  constexpr float kRootHalfPi = 1.2533141373155002512f;
#pragma unroll
  for (int k = 0; k < NH; ++k) out[k] = key.s * acc[k] + (PROD ? key.g * (kRootHalfPi / (float)D) * accz[k] : 0.f);
}

// Stages the R q / S q rows of heads h0 .. h0 + nh - 1 of `ws` into LDS (2 D floats per head).
template <int D>
__device__ __forceinline__ void stage_heads(const float* __restrict__ ws, int64_t h0, int nh, float* dst) {
  for (int i = threadIdx.x; i < nh * 2 * D; i += blockDim.x) dst[i] = ws[h0 * 2 * D + i];
}

// ---------------------------------------------------------------------------------------
// Scores: grid (key tiles of 256, B * Hkv); keys of sequence (b, g) at rows (b Hkv + g) rows + t.
// ---------------------------------------------------------------------------------------
template <int D, int BITS, bool PROD>
__global__ __launch_bounds__(kGenThreads) void k_scores_gen(const float* __restrict__ ws, int Hq, int Hkv, int64_t T,
                                                           int64_t rows, const uint32_t* __restrict__ idx,
                                                           const float* __restrict__ norms,
                                                           const uint32_t* __restrict__ qjl,
                                                           const float* __restrict__ rnorms, CodebookArgs cb,
                                                           float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) float qh[kGenHeadGroup * 2 * D];
  __shared__ float cent[16];
  if (threadIdx.x < 16) cent[threadIdx.x] = cb.c[threadIdx.x];
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int ratio = Hq / Hkv;
  const int64_t t = (int64_t)blockIdx.x * kGenThreads + threadIdx.x;
  const bool valid = t < T;
  GenKey<D, BITS, PROD> key;
  load_gen_key<D, BITS, PROD>(idx, norms, qjl, rnorms, (int64_t)bg * rows + t, valid, key);
  for (int k0 = 0; k0 < ratio; k0 += kGenHeadGroup) {
    const int nh = ratio - k0 < kGenHeadGroup ? ratio - k0 : kGenHeadGroup;
    const int64_t h0 = (int64_t)b * Hq + (int64_t)g * ratio + k0;
    __syncthreads();
    stage_heads<D>(ws, h0, nh, qh);
    __syncthreads();
    float out[kGenHeadGroup];
    gen_key_scores<D, BITS, PROD, kGenHeadGroup>(key, qh, qh + D, cent, nh, out);
    if (valid) {
#pragma unroll
      for (int k = 0; k < kGenHeadGroup; ++k)
        if (k < nh) scores[(h0 + k) * T + t] = out[k];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Decode attention, one range of kGenAttnTiles tiles of one sequence per block; the GQA ratio
// (<= 8) heads of the sequence's kv head at once.  Per tile of 256 keys:
//   1. thread t stages key t's index words, its value's words and norms in LDS (one round of
//      loads per tile);
//   2. thread t forms key t's logits from the staged words (32 coordinates at a time);
//   3. online softmax per head (block reductions); p * s_v per (head, key) into LDS;
//   4. P V: thread (g4, kp) owns coordinates 4 g4 .. 4 g4 + 3 and the keys kp, kp + KP, ... of
//      the tile, so one value word read serves its four coordinates.
// Partials per (sequence, range, head): m, l, then D accumulators.
// ---------------------------------------------------------------------------------------
template <int D>
constexpr int attn_gen_part() { return D + 2; }

// Logits of one key whose index words sit in LDS (row kw, BITS words per 32 coordinates).
template <int D, int BITS, int NH>
__device__ __forceinline__ void gen_key_logits_lds(const uint32_t* kw, float s, const float* qh, const float* cent,
                                                   int nh, float (&out)[NH]) {
  float acc[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) acc[k] = 0.f;
#pragma unroll 1
  for (int c = 0; c < D / 32; ++c) {
    uint32_t wc[BITS];
#pragma unroll
    for (int b = 0; b < BITS; ++b) wc[b] = kw[c * BITS + b];
    float cv[32];
    gen_for<0, 32>([&](auto ee) {
      constexpr int e = decltype(ee)::value;
      cv[e] = cent[field<BITS, e>(wc)];
    });
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      if (k < nh) {
        const f32x4* qr4 = reinterpret_cast<const f32x4*>(qh + k * 2 * D + 32 * c);
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4) {
          const f32x4 qv = qr4[e4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[k] = fmaf(qv[e], cv[4 * e4 + e], acc[k]);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NH; ++k) out[k] = s * acc[k];
}

template <int D, int KB, int VB>
struct AttnGenLds {
  static constexpr int WK = D * KB / 32, WV = D * VB / 32;
  static constexpr int SK = WK + 1, SV = WV + 1;  // odd row strides: a thread's row reads hit distinct banks
  static constexpr int KP = kGenThreads / (D / 4);  // key phases of the P V step
  static constexpr int TILE_WORDS = kGenThreads * (SK + SV);
  static constexpr int RED_WORDS = (KP - 1) * kGenHeadGroup * D;  // phase partials, after the last tile
  static constexpr int REGION = TILE_WORDS > RED_WORDS ? TILE_WORDS : RED_WORDS;
};

template <int D, int KB, int VB>
__global__ __launch_bounds__(kGenThreads) void k_attn_gen(const float* __restrict__ ws, int Hq, int Hkv, int64_t T,
                                                         int64_t rows, int nsplit, float scale,
                                                         const uint32_t* __restrict__ kidx,
                                                         const float* __restrict__ knorm,
                                                         const uint32_t* __restrict__ vidx,
                                                         const float* __restrict__ vnorm, CodebookArgs cbk,
                                                         CodebookArgs cbv, float* __restrict__ parts) {
  using L = AttnGenLds<D, KB, VB>;
  constexpr int P = attn_gen_part<D>();
  constexpr int KP = L::KP;
  __shared__ __attribute__((aligned(16))) float qh[kGenHeadGroup * 2 * D];
  __shared__ float centk[16], centv[16];
  __shared__ float pv[kGenHeadGroup][kGenThreads];   // p * s_v
  __shared__ float ksn[kGenThreads];
  __shared__ float red[kGenHeadGroup][kGenThreads / 64];
  __shared__ uint32_t region[L::REGION];
  uint32_t* const kws = region;                         // [256][SK]
  uint32_t* const vws = region + kGenThreads * L::SK;   // [256][SV]
  float* const accred = reinterpret_cast<float*>(region);
  if (threadIdx.x < 16) {
    centk[threadIdx.x] = cbk.c[threadIdx.x];
    centv[threadIdx.x] = cbv.c[threadIdx.x];
  }
  const int bg = blockIdx.y, split = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int nh = Hq / Hkv;
  const int64_t h0 = (int64_t)b * Hq + (int64_t)g * nh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = threadIdx.x % (D / 4), kp = threadIdx.x / (D / 4);
  stage_heads<D>(ws, h0, nh, qh);
  float m[kGenHeadGroup], l[kGenHeadGroup], acc[kGenHeadGroup][4];
#pragma unroll
  for (int k = 0; k < kGenHeadGroup; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[k][e] = 0.f;
  }
  const int64_t tile0 = (int64_t)split * kGenAttnTiles;
  const int64_t ntiles = (T + kGenThreads - 1) / kGenThreads;
  const int64_t tile1 = tile0 + kGenAttnTiles < ntiles ? tile0 + kGenAttnTiles : ntiles;
  for (int64_t tile = tile0; tile < tile1; ++tile) {
    const int64_t t = tile * kGenThreads + threadIdx.x;
    const bool valid = t < T;
    const int64_t row = (int64_t)bg * rows + (valid ? t : 0);
    __syncthreads();  // the previous tile's LDS reads are done (and qh is staged)
    // 1. stage this thread's key and value words
    {
      const uint32_t* ks = kidx + row * L::WK;
      const uint32_t* vs = vidx + row * L::WV;
#pragma unroll
      for (int i = 0; i < L::WK; ++i) kws[threadIdx.x * L::SK + i] = ks[i];
#pragma unroll
      for (int i = 0; i < L::WV; ++i) vws[threadIdx.x * L::SV + i] = vs[i];
      ksn[threadIdx.x] = valid ? knorm[row] : 0.f;
    }
    const float vsn = valid ? vnorm[row] : 0.f;
    // 2. logits (a thread reads only its own staged row here)
    float lg[kGenHeadGroup];
    gen_key_logits_lds<D, KB, kGenHeadGroup>(kws + threadIdx.x * L::SK, ksn[threadIdx.x], qh, centk, nh, lg);
    // 3. online softmax per head
#pragma unroll
    for (int k = 0; k < kGenHeadGroup; ++k) {
      lg[k] = valid ? lg[k] * scale : -INFINITY;
      float mx = lg[k];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (lane == 0) red[k][wave] = mx;
    }
    __syncthreads();
    float pk[kGenHeadGroup];  // this thread's key's probabilities (for l)
#pragma unroll
    for (int k = 0; k < kGenHeadGroup; ++k) {
      float mx = red[k][0];
#pragma unroll
      for (int w = 1; w < kGenThreads / 64; ++w) mx = fmaxf(mx, red[k][w]);
      const float mn = fmaxf(m[k], mx);
      const float alpha = mn == -INFINITY ? 1.f : __expf(m[k] - mn);
      const float p = mn == -INFINITY ? 0.f : __expf(lg[k] - mn);
      pv[k][threadIdx.x] = p * vsn;
      pk[k] = p;
      m[k] = mn;
      l[k] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[k][e] *= alpha;
    }
    __syncthreads();  // pv and the staged value words are visible; red is free
    // 4. P V over coordinates 4 g4 .. 4 g4 + 3
    {
      const int bitpos = 4 * VB * g4;
      const int wi = bitpos >> 5, sh = bitpos & 31;
#pragma unroll 4
      for (int tt = kp; tt < kGenThreads; tt += KP) {
        uint32_t f = vws[tt * L::SV + wi] >> sh;
        if (sh + 4 * VB > 32) f |= vws[tt * L::SV + wi + 1] << (32 - sh);
        float cv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) cv[e] = centv[(f >> (VB * e)) & ((1u << VB) - 1u)];
#pragma unroll
        for (int k = 0; k < kGenHeadGroup; ++k) {
          if (k < nh) {
            const float p = pv[k][tt];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k][e] = fmaf(p, cv[e], acc[k][e]);
          }
        }
      }
    }
    // l: the tile's probabilities summed over the block
#pragma unroll
    for (int k = 0; k < kGenHeadGroup; ++k) {
      float sm = pk[k];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
      if (lane == 0) red[k][wave] = sm;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kGenHeadGroup; ++k) {
      float sm = 0.f;
#pragma unroll
      for (int w = 0; w < kGenThreads / 64; ++w) sm += red[k][w];
      l[k] += sm;
    }
  }
  // merge the key phases through LDS (the tile region is free now) and write the partials
  __syncthreads();
  if (kp > 0) {
#pragma unroll
    for (int k = 0; k < kGenHeadGroup; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) accred[((kp - 1) * kGenHeadGroup + k) * D + 4 * g4 + e] = acc[k][e];
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll 1
    for (int p = 0; p < KP - 1; ++p)
#pragma unroll
      for (int k = 0; k < kGenHeadGroup; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] += accred[(p * kGenHeadGroup + k) * D + 4 * g4 + e];
    float* dst = parts + ((int64_t)bg * nsplit + split) * kGenHeadGroup * P;
#pragma unroll
    for (int k = 0; k < kGenHeadGroup; ++k) {
      if (k < nh) {
        if (g4 == 0) {
          dst[k * P] = m[k];
          dst[k * P + 1] = l[k];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[k * P + 2 + 4 * g4 + e] = acc[k][e];
      }
    }
  }
}

// out[b, h] = R_V^T (sum_s e^{m_s - M} acc_s) / (sum_s e^{m_s - M} l_s); one block of D threads per
// query head.  The splits are taken D at a time: thread t forms split s0 + t's weight once, and
// the accumulation over the chunk then reads the weights from LDS while its loads of acc_s (one
// per split, independent) stay in flight together.
template <int D>
__device__ __forceinline__ float block_reduce_gen(float v, float* red, bool is_max) {
  constexpr int NW = D / 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if constexpr (NW > 1) {
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = is_max ? fmaxf(v, red[w]) : v + red[w];
  }
  return v;
}

template <int D>
__global__ __launch_bounds__(D) void k_attn_gen_combine(const float* __restrict__ parts, int Hq, int Hkv, int nsplit,
                                                        const float* __restrict__ r32v, float* __restrict__ out) {
  constexpr int P = attn_gen_part<D>();
  __shared__ float a[D];
  __shared__ float wsh[D];
  __shared__ float red[D / 64];
  const int64_t h = blockIdx.x;
  const int b = (int)(h / Hq), hq = (int)(h % Hq);
  const int ratio = Hq / Hkv;
  const int g = hq / ratio, k = hq % ratio;
  const int64_t sstride = (int64_t)kGenHeadGroup * P;
  const float* src = parts + ((int64_t)(b * Hkv + g) * nsplit) * sstride + k * P;
  const int i = threadIdx.x;
  float m = -INFINITY;
  for (int s = i; s < nsplit; s += D) m = fmaxf(m, src[s * sstride]);
  const float M = block_reduce_gen<D>(m, red, true);
  float lsum = 0.f, A = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += D) {
    const int s = s0 + i;
    float w = 0.f;
    if (s < nsplit) {
      const float ms = src[s * sstride];
      w = ms == -INFINITY ? 0.f : __expf(ms - M);
      lsum = fmaf(w, src[s * sstride + 1], lsum);
    }
    wsh[i] = w;
    __syncthreads();
    const int cnt = nsplit - s0 < D ? nsplit - s0 : D;
    const float* ps = src + (int64_t)s0 * sstride + 2 + i;
#pragma unroll 8
    for (int t = 0; t < cnt; ++t) A = fmaf(wsh[t], ps[t * sstride], A);
    __syncthreads();
  }
  const float L = block_reduce_gen<D>(lsum, red, false);
  a[i] = L > 0.f ? A / L : 0.f;
  __syncthreads();
  // R_V^T a: (R^T a)_i = sum_j R[j][i] a_j, R row-major: thread i reads consecutive columns
  float o = 0.f;
#pragma unroll 8
  for (int j = 0; j < D; ++j) o = fmaf(r32v[(size_t)j * D + i], a[j], o);
  out[h * D + i] = o;
}

// ---------------------------------------------------------------------------------------
// Encode at d = 64: one wave per vector, lane i = coordinate i; the block's waves stride over
// the vectors.  LDS: A[j][i] = R[i][j] (y = R x), and for prod B[j][i] = R[j][i] (R^T r) and
// Cs[j][i] = S[i][j] (S (R^T r)).
// ---------------------------------------------------------------------------------------
template <int BITS, bool PROD, bool BF16IN>
__global__ __launch_bounds__(kGenThreads) void k_encode_d64(const void* __restrict__ x, int64_t n,
                                                           const float* __restrict__ rt32,
                                                           const float* __restrict__ r32,
                                                           const float* __restrict__ st32, CodebookArgs cb,
                                                           uint32_t* __restrict__ idx_out, float* __restrict__ norms,
                                                           uint32_t* __restrict__ qjl_out, float* __restrict__ rnorms) {
  constexpr int D = 64, K = 1 << BITS, W = D * BITS / 32;
  constexpr int NW = kGenThreads / 64;
  __shared__ float A[D * D];
  __shared__ float Bm[PROD ? D * D : 1];
  __shared__ float Cs[PROD ? D * D : 1];
  __shared__ float xv[NW][D];
  __shared__ uint8_t ib[NW][D];
  for (int e = threadIdx.x; e < D * D; e += kGenThreads) {
    A[e] = rt32[e];
    if constexpr (PROD) {
      Bm[e] = r32[e];
      Cs[e] = st32[e];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * NW;
  // every wave of the block runs the same number of iterations (the barrier-free loop below only
  // uses wave-local LDS)
  for (int64_t v = (int64_t)blockIdx.x * NW + wave; v < n; v += nwaves) {
    float xi;
    if constexpr (BF16IN) {
      xi = __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[v * D + lane] << 16);
    } else {
      xi = static_cast<const float*>(x)[v * D + lane];
    }
    float ss = xi * xi;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    const float s = sqrtf(ss);
    xv[wave][lane] = xi;
    __builtin_amdgcn_wave_barrier();
    float y = 0.f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) y = fmaf(A[j * D + lane], xv[wave][j], y);
    // idx = #{k : y / s >= t_k} (ties to the upper index), decided as y >= t_k s; zero vector: K/2
    uint32_t id = 0;
    if (s > 0.f) {
#pragma unroll
      for (int k = 0; k < K - 1; ++k) id += y >= cb.t[k] * s ? 1u : 0u;
    } else {
      id = K / 2;
    }
    ib[wave][lane] = (uint8_t)id;
    __builtin_amdgcn_wave_barrier();
    if (lane < W) {
      uint32_t word = 0;
      for (int p = 0; p < 32; ++p) {
        const int bit = 32 * lane + p;
        word |= ((uint32_t)(ib[wave][bit / BITS] >> (bit % BITS)) & 1u) << p;
      }
      idx_out[v * W + lane] = word;
    }
    if (lane == 0) norms[v] = s;
    if constexpr (PROD) {
      // unit-scale residual in the rotated domain, gamma = s ||r||, signs of S (R^T r)
      const float r = s > 0.f ? y / s - cb.c[id] : 0.f;
      float rr = r * r;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) rr += __shfl_xor(rr, off);
      __builtin_amdgcn_wave_barrier();
      xv[wave][lane] = r;
      __builtin_amdgcn_wave_barrier();
      float o = 0.f;
#pragma unroll 8
      for (int j = 0; j < D; ++j) o = fmaf(Bm[j * D + lane], xv[wave][j], o);
      __builtin_amdgcn_wave_barrier();
      xv[wave][lane] = o;
      __builtin_amdgcn_wave_barrier();
      float z = 0.f;
#pragma unroll 8
      for (int j = 0; j < D; ++j) z = fmaf(Cs[j * D + lane], xv[wave][j], z);
      const uint64_t bits = __ballot(z >= 0.f);
      if (lane < 2) qjl_out[v * 2 + lane] = (uint32_t)(bits >> (32 * lane));
      if (lane == 0) rnorms[v] = s * sqrtf(rr);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int D, int BITS, bool PROD>
hipError_t scores_gen_launch(const float* ws, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                             const CodebookArgs& cb, float* scores, hipStream_t st) {
  const dim3 grid((unsigned)((T + kGenThreads - 1) / kGenThreads), (unsigned)(B * Hkv));
  hipLaunchKernelGGL((k_scores_gen<D, BITS, PROD>), grid, dim3(kGenThreads), 0, st, ws, Hq, Hkv, T, rows, K->idx,
                     K->norms, K->qjl, K->rnorms, cb, scores);
  return hipGetLastError();
}

template <int D, bool PROD>
hipError_t scores_gen_bits(const float* ws, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                           const CodebookArgs& cb, float* scores, hipStream_t st) {
  switch (cb.bits) {
    case 1: return scores_gen_launch<D, 1, PROD>(ws, B, Hq, Hkv, T, rows, K, cb, scores, st);
    case 2: return scores_gen_launch<D, 2, PROD>(ws, B, Hq, Hkv, T, rows, K, cb, scores, st);
    case 3: return scores_gen_launch<D, 3, PROD>(ws, B, Hq, Hkv, T, rows, K, cb, scores, st);
    case 4: return scores_gen_launch<D, 4, PROD>(ws, B, Hq, Hkv, T, rows, K, cb, scores, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t qprep_gen_launch(const float* q, int64_t heads, const tq_rotation_s* rot, const tq_qjl_s* qjl, float* ws,
                            hipStream_t st) {
  hipLaunchKernelGGL((k_qprep_gen<D>), dim3((unsigned)heads), dim3(D), 0, st, q, rot->rt32_dev,
                     qjl ? qjl->st32_dev : nullptr, ws);
  return hipGetLastError();
}

int attn_gen_splits(int64_t T) {
  const int64_t ntiles = (T + kGenThreads - 1) / kGenThreads;
  const int64_t s = (ntiles + kGenAttnTiles - 1) / kGenAttnTiles;
  return (int)(s > 0 ? s : 1);
}

template <int D, int KB, int VB>
hipError_t attn_gen_launch(const float* ws, int B, int Hq, int Hkv, int64_t T, int64_t rows, int nsplit, float scale,
                           const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                           float* parts, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_gen<D, KB, VB>), dim3((unsigned)nsplit, (unsigned)(B * Hkv)), dim3(kGenThreads), 0, st,
                     ws, Hq, Hkv, T, rows, nsplit, scale, K->idx, K->norms, V->idx, V->norms, cbk, cbv, parts);
  return hipGetLastError();
}

template <int D, int KB>
hipError_t attn_gen_vbits(const float* ws, int B, int Hq, int Hkv, int64_t T, int64_t rows, int nsplit, float scale,
                          const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                          float* parts, hipStream_t st) {
  switch (cbv.bits) {
    case 1: return attn_gen_launch<D, KB, 1>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
    case 2: return attn_gen_launch<D, KB, 2>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
    case 3: return attn_gen_launch<D, KB, 3>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
    case 4: return attn_gen_launch<D, KB, 4>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t attn_gen_kbits(const float* ws, int B, int Hq, int Hkv, int64_t T, int64_t rows, int nsplit, float scale,
                          const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                          float* parts, hipStream_t st) {
  switch (cbk.bits) {
    case 1: return attn_gen_vbits<D, 1>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
    case 2: return attn_gen_vbits<D, 2>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
    case 3: return attn_gen_vbits<D, 3>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
    case 4: return attn_gen_vbits<D, 4>(ws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
  }
  return hipErrorInvalidValue;
}

template <int BITS, bool PROD>
hipError_t encode_d64_launch(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                             const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits, float* rn,
                             hipStream_t st) {
  const int64_t waves = (n + 7) / 8;  // about eight vectors per wave
  int64_t blocks = (waves + kGenThreads / 64 - 1) / (kGenThreads / 64);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const float* st32 = qjl ? qjl->st32_dev : nullptr;
  if (bf16)
    hipLaunchKernelGGL((k_encode_d64<BITS, PROD, true>), dim3((unsigned)blocks), dim3(kGenThreads), 0, st, x, n,
                       rot->rt32_dev, rot->r32_dev, st32, cb, idx, norms, qbits, rn);
  else
    hipLaunchKernelGGL((k_encode_d64<BITS, PROD, false>), dim3((unsigned)blocks), dim3(kGenThreads), 0, st, x, n,
                       rot->rt32_dev, rot->r32_dev, st32, cb, idx, norms, qbits, rn);
  return hipGetLastError();
}

}  // namespace

size_t kv_gen_query_bytes(int B, int Hq, int d) {
  return (((size_t)B * Hq * 2 * d * sizeof(float)) + 255) & ~(size_t)255;
}

size_t attn_gen_workspace_bytes(int B, int Hq, int Hkv, int64_t T, int d) {
  const int nsplit = attn_gen_splits(T);
  return kv_gen_query_bytes(B, Hq, d) + (size_t)B * Hkv * nsplit * kGenHeadGroup * (d + 2) * sizeof(float);
}

hipError_t launch_scores_gen(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                             const CodebookArgs& cb, const tq_rotation_s* rot, const tq_qjl_s* qjl, float* scores,
                             void* ws, hipStream_t st) {
  const int d = rot->d;
  float* qws = static_cast<float*>(ws);
  const bool prod = K->mode == TQ_MODE_PROD;
  const int64_t heads = (int64_t)B * Hq;
  hipError_t e = d == 64 ? qprep_gen_launch<64>(q, heads, rot, prod ? qjl : nullptr, qws, st)
                         : qprep_gen_launch<256>(q, heads, rot, prod ? qjl : nullptr, qws, st);
  if (e != hipSuccess) return e;
  if (d == 64)
    return prod ? scores_gen_bits<64, true>(qws, B, Hq, Hkv, T, rows, K, cb, scores, st)
                : scores_gen_bits<64, false>(qws, B, Hq, Hkv, T, rows, K, cb, scores, st);
  return prod ? scores_gen_bits<256, true>(qws, B, Hq, Hkv, T, rows, K, cb, scores, st)
              : scores_gen_bits<256, false>(qws, B, Hq, Hkv, T, rows, K, cb, scores, st);
}

hipError_t launch_decode_attn_gen(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                                  const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                                  const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale, float* out,
                                  void* ws, hipStream_t st) {
  const int d = rot_k->d;
  float* qws = static_cast<float*>(ws);
  float* parts = reinterpret_cast<float*>(static_cast<char*>(ws) + kv_gen_query_bytes(B, Hq, d));
  const int64_t heads = (int64_t)B * Hq;
  const int nsplit = attn_gen_splits(T);
  hipError_t e = d == 64 ? qprep_gen_launch<64>(q, heads, rot_k, nullptr, qws, st)
                         : qprep_gen_launch<256>(q, heads, rot_k, nullptr, qws, st);
  if (e != hipSuccess) return e;
  e = d == 64 ? attn_gen_kbits<64>(qws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st)
              : attn_gen_kbits<256>(qws, B, Hq, Hkv, T, rows, nsplit, scale, K, V, cbk, cbv, parts, st);
  if (e != hipSuccess) return e;
  if (d == 64)
    hipLaunchKernelGGL((k_attn_gen_combine<64>), dim3((unsigned)heads), dim3(64), 0, st, parts, Hq, Hkv, nsplit,
                       rot_v->r32_dev, out);
  else
    hipLaunchKernelGGL((k_attn_gen_combine<256>), dim3((unsigned)heads), dim3(256), 0, st, parts, Hq, Hkv, nsplit,
                       rot_v->r32_dev, out);
  return hipGetLastError();
}

hipError_t launch_encode_d64(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                             const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits, float* rnorms,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const bool prod = qjl != nullptr;
  switch (cb.bits) {
    case 1: return prod ? encode_d64_launch<1, true>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : encode_d64_launch<1, false>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
    case 2: return prod ? encode_d64_launch<2, true>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : encode_d64_launch<2, false>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
    case 3: return prod ? encode_d64_launch<3, true>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : encode_d64_launch<3, false>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
    case 4: return prod ? encode_d64_launch<4, true>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st)
                        : encode_d64_launch<4, false>(x, bf16, n, rot, qjl, cb, idx, norms, qbits, rnorms, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
