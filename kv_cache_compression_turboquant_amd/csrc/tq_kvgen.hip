// KV-side kernels for head dims other than 128 (d = 64 and d = 256): the query prologue, the
// compressed-key scores and decode attention, and the d = 64 encode.  The d = 128 path has its
// own tuned kernels; these follow the same formulas with a simpler thread layout.
//
// Scores ([TQ] TurboQuant_mse / TurboQuant_prod inner products; [FP] inner-product bias and the
// QJL fix): <q, k~> = s <R q, C[idx]> (+ gamma sqrt(pi/2)/d <S q, z> for prod keys), with R q and
// S q formed once per query head in fp32, on the matrix cores: tiles of 16 keys (centroids decoded
// to fp16 through LDS tables) against up to 16 query heads (fp16 hi + lo).
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
#include <algorithm>
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
#ifndef TQ_GEN_ATTN_TILES
#define TQ_GEN_ATTN_TILES 4
#endif
constexpr int kGenAttnTiles = TQ_GEN_ATTN_TILES;   // 256-key tiles per attention range

// ---------------------------------------------------------------------------------------
// Query prologue: ws[h] = {R q_h (d floats), S q_h (d floats)}; one block of 256 threads per head.
// Thread (i4, jg) forms outputs 4 i4 .. 4 i4 + 3 over the rows j of its group jg (a float4 of
// R^T per row), and the groups are summed through LDS: short dependent load chains.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_qprep_gen(const float* __restrict__ q, const float* __restrict__ rt32,
                                                  const float* __restrict__ st32, float* __restrict__ ws) {
  constexpr int NI = D / 4;            // threads per row group
  constexpr int JG = 256 / NI;         // row groups
  constexpr int JN = D / JG;           // rows per group
  __shared__ float qs[D];
  __shared__ f32x4 part[2][JG][NI];
  const int64_t h = blockIdx.x;
  const int i4 = threadIdx.x % NI, jg = threadIdx.x / NI;
  if (threadIdx.x < D) qs[threadIdx.x] = q[h * D + threadIdx.x];
  __syncthreads();
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
  // rt32[j][i] = R[i][j] and st32[j][i] = S[i][j]
#pragma unroll 16
  for (int jj = 0; jj < JN; ++jj) {
    const int j = jg * JN + jj;
    const f32x4 r = *reinterpret_cast<const f32x4*>(rt32 + (size_t)j * D + 4 * i4);
    a += r * qs[j];
  }
  if (st32) {
#pragma unroll 16
    for (int jj = 0; jj < JN; ++jj) {
      const int j = jg * JN + jj;
      const f32x4 r = *reinterpret_cast<const f32x4*>(st32 + (size_t)j * D + 4 * i4);
      c += r * qs[j];
    }
  }
  part[0][jg][i4] = a;
  part[1][jg][i4] = c;
  __syncthreads();
  if (threadIdx.x < 2 * NI) {
    const int which = threadIdx.x / NI, k = threadIdx.x % NI;
    f32x4 t = part[which][0][k];
#pragma unroll
    for (int g2 = 1; g2 < JG; ++g2) t += part[which][g2][k];
    *reinterpret_cast<f32x4*>(ws + h * 2 * D + which * D + 4 * k) = t;
  }
}

// BITS-bit field of coordinate I (compile-time) of a packed row held in registers.
template <int BITS, int I, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int p = BITS * I, wi = p >> 5, sh = p & 31;
  uint32_t v = w[wi] >> sh;
  if constexpr (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

// ---------------------------------------------------------------------------------------
// Decode attention, one range of kGenAttnTiles tiles of one sequence per block; the GQA ratio
// (<= 8) heads of the sequence's kv head at once.  Per tile of 256 keys:
//   1. thread t stages key t's index words and its value's words in LDS (one round of loads per
//      tile; the norms stay in registers);
//   2. thread t forms key t's logits from its staged row, 32 coordinates at a time, with the
//      queries read by scalar loads (uniform across the wave, no LDS traffic);
//   3. online softmax per head (block reductions); p * s_v per (head, key) into LDS;
//   4. P V: thread (g4, kp) owns coordinates 4 g4 .. 4 g4 + 3 and the keys kp, kp + KP, ... of
//      the tile, so one value word read serves its four coordinates.
// Partials per (sequence, range, head): m, l, then D accumulators.
// ---------------------------------------------------------------------------------------
template <int D>
constexpr int attn_gen_part() { return D + 2; }

// Logits of one key whose index words sit in LDS (row kw, BITS words per 32 coordinates).  The
// rotated queries are read from global memory at wave-uniform addresses (scalar loads), 2 D floats
// per head.  (Rows held in registers instead measured slower at d = 64: fewer resident waves.)
template <int D, int BITS, int NH>
__device__ __forceinline__ void gen_key_logits_lds(const uint32_t* kw, float s, const float* __restrict__ qg,
                                                   const f32x2* pair, int nh, float (&out)[NH]) {
  float acc[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) acc[k] = 0.f;
#pragma unroll 1
  for (int c = 0; c < D / 32; ++c) {
    uint32_t wc[BITS];
#pragma unroll
    for (int b = 0; b < BITS; ++b) wc[b] = kw[c * BITS + b];
    float cv[32];
    // two coordinates per lookup: entry f of the pair table holds the centroids of the low and
    // the high BITS bits of the 2 BITS-bit field f
    gen_for<0, 16>([&](auto pp) {
      constexpr int e2 = decltype(pp)::value;
      const f32x2 c2 = pair[field<2 * BITS, e2>(wc)];
      cv[2 * e2] = c2[0];
      cv[2 * e2 + 1] = c2[1];
    });
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      if (k < nh) {
        const f32x4* qr4 = reinterpret_cast<const f32x4*>(qg + k * 2 * D + 32 * c);
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

template <int D, int KB, int VB, int NH>
struct AttnGenLds {
  static constexpr int WK = D * KB / 32, WV = D * VB / 32;
  static constexpr int SK = WK + 1, SV = WV + 1;  // odd row strides: a thread's row reads hit distinct banks
  static constexpr int KP = kGenThreads / (D / 4);  // key phases of the P V step
  static constexpr int TILE_WORDS = kGenThreads * (SK + SV);
  static constexpr int RED_WORDS = (KP - 1) * NH * D;  // phase partials, after the last tile
  static constexpr int REGION = TILE_WORDS > RED_WORDS ? TILE_WORDS : RED_WORDS;
};

template <int D, int KB, int VB, int NH, bool EXACT>
__global__ __launch_bounds__(kGenThreads) void k_attn_gen(const float* __restrict__ ws, int Hq, int Hkv, int64_t T,
                                                         int64_t rows, int nsplit, float scale,
                                                         const uint32_t* __restrict__ kidx,
                                                         const float* __restrict__ knorm,
                                                         const uint32_t* __restrict__ vidx,
                                                         const float* __restrict__ vnorm, CodebookArgs cbk,
                                                         CodebookArgs cbv, float* __restrict__ parts) {
  using L = AttnGenLds<D, KB, VB, NH>;
  constexpr int P = attn_gen_part<D>();
  constexpr int KP = L::KP;
  constexpr int VQ = VB <= 2 ? 1 << (4 * VB) : 1;   // value quad table: 4 coordinates per lookup
  __shared__ float centv[16];
  __shared__ __attribute__((aligned(16))) f32x2 kpair[1 << (2 * KB)];
  __shared__ __attribute__((aligned(16))) f32x4 vquad[VQ];
  __shared__ __attribute__((aligned(16))) float pv[kGenThreads][NH];   // p * s_v, a key's heads together
  __shared__ float red[NH][kGenThreads / 64];
  __shared__ uint32_t region[L::REGION];
  uint32_t* const kws = region;                         // [256][SK]
  uint32_t* const vws = region + kGenThreads * L::SK;   // [256][SV]
  float* const accred = reinterpret_cast<float*>(region);
  if (threadIdx.x < 16) centv[threadIdx.x] = cbv.c[threadIdx.x];
  for (int i = threadIdx.x; i < (1 << (2 * KB)); i += kGenThreads)
    kpair[i] = f32x2{cbk.c[i & ((1 << KB) - 1)], cbk.c[i >> KB]};
  if constexpr (VB <= 2) {
    constexpr uint32_t vm = (1u << VB) - 1u;
    for (int i = threadIdx.x; i < VQ; i += kGenThreads)
      vquad[i] = f32x4{cbv.c[i & vm], cbv.c[(i >> VB) & vm], cbv.c[(i >> (2 * VB)) & vm], cbv.c[(i >> (3 * VB)) & vm]};
  }
  const int bg = blockIdx.y, split = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int nh = EXACT ? NH : Hq / Hkv;  // EXACT: the GQA ratio is NH
  const int64_t h0 = (int64_t)b * Hq + (int64_t)g * nh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = threadIdx.x % (D / 4), kp = threadIdx.x / (D / 4);
  const float* const qg = ws + h0 * 2 * D;
  float m[NH], l[NH], acc[NH][4];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
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
    __syncthreads();  // the previous tile's LDS reads are done
    // 1. stage this thread's key and value words
    {
      const uint32_t* ks = kidx + row * L::WK;
      const uint32_t* vs = vidx + row * L::WV;
#pragma unroll
      for (int i = 0; i < L::WK; ++i) kws[threadIdx.x * L::SK + i] = ks[i];
#pragma unroll
      for (int i = 0; i < L::WV; ++i) vws[threadIdx.x * L::SV + i] = vs[i];
    }
    const float ksn = valid ? knorm[row] : 0.f;
    const float vsn = valid ? vnorm[row] : 0.f;
    // 2. logits (a thread reads only its own key row)
    float lg[NH];
    gen_key_logits_lds<D, KB, NH>(kws + threadIdx.x * L::SK, ksn, qg, kpair, nh, lg);
    // 3. online softmax per head
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      lg[k] = valid ? lg[k] * scale : -INFINITY;
      float mx = lg[k];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (lane == 0) red[k][wave] = mx;
    }
    __syncthreads();
    float pk[NH];  // this thread's key's probabilities (for l)
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      float mx = red[k][0];
#pragma unroll
      for (int w = 1; w < kGenThreads / 64; ++w) mx = fmaxf(mx, red[k][w]);
      const float mn = fmaxf(m[k], mx);
      const float alpha = mn == -INFINITY ? 1.f : __expf(m[k] - mn);
      const float p = mn == -INFINITY ? 0.f : __expf(lg[k] - mn);
      pv[threadIdx.x][k] = p * vsn;
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
        if constexpr (VB <= 2) {
          const f32x4 c4 = vquad[f & (uint32_t)(VQ - 1)];
#pragma unroll
          for (int e = 0; e < 4; ++e) cv[e] = c4[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) cv[e] = centv[(f >> (VB * e)) & ((1u << VB) - 1u)];
        }
        // all NH heads' probabilities in NH / 4 reads (heads past the ratio carry finite values
        // that are never stored)
#pragma unroll
        for (int k4 = 0; k4 < NH / 4; ++k4) {
          const f32x4 p4 = reinterpret_cast<const f32x4*>(pv[tt])[k4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * k4 + kk][e] = fmaf(p4[kk], cv[e], acc[4 * k4 + kk][e]);
        }
      }
    }
    // l: the tile's probabilities summed over the block
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      float sm = pk[k];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
      if (lane == 0) red[k][wave] = sm;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NH; ++k) {
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
    for (int k = 0; k < NH; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) accred[((kp - 1) * NH + k) * D + 4 * g4 + e] = acc[k][e];
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll 1
    for (int p = 0; p < KP - 1; ++p)
#pragma unroll
      for (int k = 0; k < NH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] += accred[(p * NH + k) * D + 4 * g4 + e];
    float* dst = parts + ((int64_t)bg * nsplit + split) * kGenHeadGroup * P;
#pragma unroll
    for (int k = 0; k < NH; ++k) {
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
// per split, independent) stay in flight together, 32 at a time, as do the loads of R's columns
// (the kernel is bound by these round trips to L2, not by its arithmetic).
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
#pragma unroll 32
    for (int t = 0; t < cnt; ++t) A = fmaf(wsh[t], ps[t * sstride], A);
    __syncthreads();
  }
  const float L = block_reduce_gen<D>(lsum, red, false);
  a[i] = L > 0.f ? A / L : 0.f;
  __syncthreads();
  // R_V^T a: (R^T a)_i = sum_j R[j][i] a_j, R row-major: thread i reads consecutive columns
  float o = 0.f;
#pragma unroll 32
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

// ---------------------------------------------------------------------------------------
// Scores on the matrix cores (v_mfma_f32_16x16x32_f16).  A wave takes tiles of 16 keys of one
// sequence against up to 16 of its query heads:
//   A = the keys' centroids: lane (n, g) holds key n of the tile at coordinates
//       (D/4) g + 8 s + e in instruction s (each lane a contiguous quarter of the key's row),
//       decoded from the packed words through LDS tables that map a byte (6 bits at 3 bits per
//       index) to the fp16 centroids of the indices it holds;
//   B = R q of the heads in fp16 hi + lo (two instructions per slice), and for prod keys S q
//       likewise against the +-1 sign operand (a byte of signs -> eight fp16 +-1, from a table);
//   D row 4 g + r, column n: key 4 g + r of the tile, head n.
// A block's four waves take gm_tiles<D>() consecutive tiles each, whose loads are all issued
// first; grid (key ranges, sequences, groups of 16 query heads).  (Longer-lived blocks that
// stream several such groups with the next one's loads in flight measured slower.)
// ---------------------------------------------------------------------------------------
#ifndef TQ_GM_TILES64
#define TQ_GM_TILES64 8
#endif
#ifndef TQ_GM_TILES256
#define TQ_GM_TILES256 4
#endif
// tiles of 16 keys per wave (registers); a block of four waves takes 64 gm_tiles<D>() keys
template <int D>
constexpr int gm_tiles() { return D == 64 ? TQ_GM_TILES64 : TQ_GM_TILES256; }

template <int BITS>
struct GmTab;
template <>
struct GmTab<1> {
  using E = u32x4;
  static constexpr int N = 256;
};
template <>
struct GmTab<2> {
  using E = u32x2;
  static constexpr int N = 256;
};
template <>
struct GmTab<3> {
  using E = uint32_t;
  static constexpr int N = 64;
};
template <>
struct GmTab<4> {
  using E = uint32_t;
  static constexpr int N = 256;
};

__device__ __forceinline__ uint32_t f16pair(float lo, float hi) { return f16_bits(lo) | (f16_bits(hi) << 16); }

// Table entry v: the fp16 centroids of the indices packed in v, first index in the low half.
template <int BITS>
__device__ __forceinline__ typename GmTab<BITS>::E gm_entry(uint32_t v, const float* c) {
  constexpr uint32_t M = (1u << BITS) - 1u;
  if constexpr (BITS == 4 || BITS == 3) {
    return f16pair(c[v & M], c[(v >> BITS) & M]);
  } else if constexpr (BITS == 2) {
    return u32x2{f16pair(c[v & 3u], c[(v >> 2) & 3u]), f16pair(c[(v >> 4) & 3u], c[(v >> 6) & 3u])};
  } else {
    u32x4 e;
#pragma unroll
    for (int k = 0; k < 4; ++k) e[k] = f16pair(c[(v >> (2 * k)) & 1u], c[(v >> (2 * k + 1)) & 1u]);
    return e;
  }
}

// A lane's quarter of a key row: BPL bits, loaded as NW words from the word holding its first
// bit and shifted down when that bit is not word-aligned (d = 64 at odd bit widths).
template <int D, int BITS>
struct GmSlice {
  static constexpr int BPL = D / 4 * BITS;
  static constexpr bool ALIGNED = BPL % 32 == 0;
  static constexpr int NW = ALIGNED ? BPL / 32 : (BPL + 16 + 31) / 32;
  static constexpr int NV = (BPL + 31) / 32;
};

// The A operand of instruction S from the lane's aligned slice words.
template <int BITS, int S, int NV>
__device__ __forceinline__ u32x4 gm_decode(const uint32_t (&sl)[NV], const typename GmTab<BITS>::E* tab) {
  u32x4 a;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = tab[(sl[S] >> (8 * k)) & 0xffu];
  } else if constexpr (BITS == 2) {
    constexpr int w = S >> 1, b0 = 2 * (S & 1);
    const u32x2 lo = tab[(sl[w] >> (8 * b0)) & 0xffu];
    const u32x2 hi = tab[(sl[w] >> (8 * b0 + 8)) & 0xffu];
    a = u32x4{lo[0], lo[1], hi[0], hi[1]};
  } else if constexpr (BITS == 1) {
    a = tab[(sl[S >> 2] >> (8 * (S & 3))) & 0xffu];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = 24 * S + 6 * k;   // a constant once unrolled
      const int wi = p >> 5, sh = p & 31;
      uint32_t v = sl[wi] >> sh;
      if (sh > 26) v |= sl[wi + 1] << (32 - sh);
      a[k] = tab[v & 63u];
    }
  }
  return a;
}

// Eight signs (a byte of the slice's sign bits) as fp16 +-1 from the sign table.
template <int D, int S>
__device__ __forceinline__ u32x4 gm_signs(uint32_t z0, uint32_t z1, const u32x4* tabz) {
  if constexpr (D == 256) {
    return tabz[(((S < 4) ? z0 : z1) >> (8 * (S & 3))) & 0xffu];
  } else {
    return tabz[(z0 >> (8 * S)) & 0xffu];
  }
}

// One tile's loads (16 keys from row t0 of the sequence; rows past T read zeros): the lane's slice words and sign words of key n, and the norms of
// the keys 4 g .. 4 g + 3 that the lane's results belong to.
template <int D, int BITS, bool PROD>
struct GmTile {
  uint32_t w[GmSlice<D, BITS>::NW];
  uint32_t z0, z1;
  float sn[4], gm[4];
};

template <int D, int BITS, bool PROD>
__device__ __forceinline__ void gm_load(GmTile<D, BITS, PROD>& tl, const uint32_t* idx, const float* norms,
                                        const uint32_t* qjl, const float* rnorms, int64_t rowb, int64_t t0,
                                        int64_t tlim, int n, int g, uint32_t wstart) {
  constexpr int W = D * BITS / 32, WZ = D / 32;
  const int64_t left = tlim - t0;
  const uint32_t nv = left >= 16 ? 16u : (left > 0 ? (uint32_t)left : 0u);
  const int64_t r0 = rowb + (left > 0 ? t0 : 0);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(idx + r0 * W), (short)0, (int)(nv * W * 4u), 0x00020000);
#pragma unroll
  for (int i = 0; i < GmSlice<D, BITS>::NW; ++i)
    tl.w[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, ((uint32_t)n * W + wstart + i) * 4u, 0, 0);
  tl.z0 = tl.z1 = 0u;
  if constexpr (PROD) {
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qjl + r0 * WZ), (short)0,
                                                                       (int)(nv * WZ * 4u), 0x00020000);
    if constexpr (D == 256) {
      tl.z0 = __builtin_amdgcn_raw_buffer_load_b32(rz, ((uint32_t)n * WZ + 2u * g) * 4u, 0, 0);
      tl.z1 = __builtin_amdgcn_raw_buffer_load_b32(rz, ((uint32_t)n * WZ + 2u * g + 1u) * 4u, 0, 0);
    } else {
      tl.z0 = __builtin_amdgcn_raw_buffer_load_b32(rz, ((uint32_t)n * WZ + (g >> 1)) * 4u, 0, 0);
    }
  }
  const __amdgpu_buffer_rsrc_t rn =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(norms + r0), (short)0, (int)(nv * 4u), 0x00020000);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    tl.sn[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, (uint32_t)(4 * g + r) * 4u, 0, 0));
  if constexpr (PROD) {
    const __amdgpu_buffer_rsrc_t rg =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rnorms + r0), (short)0, (int)(nv * 4u), 0x00020000);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tl.gm[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(4 * g + r) * 4u, 0, 0));
  }
}

// Workgroup barrier that waits only for the wave's LDS operations: a __syncthreads() would also
// wait for every global load in flight (the tile loads issued before the tables are built).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int BITS, bool PROD>
__global__ __launch_bounds__(256) void k_scores_gm(const float* __restrict__ ws, int Hq, int Hkv, int64_t T,
                                                   int64_t rows, const uint32_t* __restrict__ idx,
                                                   const float* __restrict__ norms, const uint32_t* __restrict__ qjl,
                                                   const float* __restrict__ rnorms, CodebookArgs cb,
                                                   float* __restrict__ scores) {
  using Tab = GmTab<BITS>;
  using SL = GmSlice<D, BITS>;
  using Tile = GmTile<D, BITS, PROD>;
  constexpr int NS = D / 32;                 // instructions per key slice
  constexpr int NT = gm_tiles<D>();          // tiles per wave
  __shared__ typename Tab::E tab[Tab::N];
  __shared__ u32x4 tabz[PROD ? 256 : 1];
  __shared__ float cent[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: tile bases in SGPRs
  const int n = lane & 15, g = lane >> 4;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int ratio = Hq / Hkv;
  const int k0 = blockIdx.z * 16;
  const int nh = ratio - k0 < 16 ? ratio - k0 : 16;
  const int64_t h0 = (int64_t)b * Hq + (int64_t)kvh * ratio + k0;
  const int64_t rowb = (int64_t)bg * rows;
  const int start_bit = SL::BPL * g;
  const uint32_t wstart = (uint32_t)(start_bit >> 5), wsh = (uint32_t)(start_bit & 31);
  constexpr float kQ = 1.2533141373155002512f / (float)D;
  const int64_t kg = (int64_t)blockIdx.x * NT * 64 + (int64_t)wave * NT * 16;   // the wave's first key

  // Head n's R q (and S q) at the lane's coordinates, loaded ahead of the tiles so that waiting
  // for them leaves the tile loads in flight (loads complete in order).
  const bool live = n < nh;
  f32x4 qv[PROD ? 2 : 1][NS][2];
  {
    const float* qr = ws + (h0 + (live ? n : 0)) * 2 * D + (D / 4) * g;
#pragma unroll
    for (int part = 0; part < (PROD ? 2 : 1); ++part)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qv[part][s][0] = *reinterpret_cast<const f32x4*>(qr + part * D + 8 * s);
        qv[part][s][1] = *reinterpret_cast<const f32x4*>(qr + part * D + 8 * s + 4);
      }
  }
  __builtin_amdgcn_sched_barrier(0);   // keep these loads ahead of the tile loads

  Tile ta[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) gm_load<D, BITS, PROD>(ta[tt], idx, norms, qjl, rnorms, rowb, kg + 16 * tt, T, n, g, wstart);

  if (threadIdx.x == 0) {
    // written by one lane from the (uniform) argument: an indexed read of the argument would be
    // a global load, and waiting for it would wait for the tile loads too
#pragma unroll
    for (int k = 0; k < 16; ++k) cent[k] = cb.c[k];
  }
  lds_barrier();
  if (threadIdx.x < Tab::N) tab[threadIdx.x] = gm_entry<BITS>(threadIdx.x, cent);
  if constexpr (PROD) {
    u32x4 e;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      e[k] = (((threadIdx.x >> (2 * k)) & 1u) ? 0x3C00u : 0xBC00u) |
             ((((threadIdx.x >> (2 * k + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
    tabz[threadIdx.x] = e;
  }

  // B operands: fp16 hi + lo of the loaded R q (and S q), zero past nh
  u32x4 qh[NS], ql[NS], zh[PROD ? NS : 1], zl[PROD ? NS : 1];
#pragma unroll
  for (int part = 0; part < (PROD ? 2 : 1); ++part)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 v0 = qv[part][s][0], v1 = qv[part][s][1];
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      u32x4 hi, lo;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a0 = live ? v[2 * k] : 0.f, a1 = live ? v[2 * k + 1] : 0.f;
        const _Float16 h0f = (_Float16)a0, h1f = (_Float16)a1;
        hi[k] = (uint32_t)__builtin_bit_cast(uint16_t, h0f) | ((uint32_t)__builtin_bit_cast(uint16_t, h1f) << 16);
        lo[k] = f16pair(a0 - (float)h0f, a1 - (float)h1f);
      }
      if (part == 0) {
        qh[s] = hi;
        ql[s] = lo;
      } else if constexpr (PROD) {
        zh[s] = hi;
        zl[s] = lo;
      }
    }
  lds_barrier();   // tables ready (the tile loads stay in flight)

  float* const out0 = scores + (h0 + n) * T;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int64_t t0 = kg + 16 * tt;
    if (t0 >= T) break;
    const int64_t left = T - t0;
    const uint32_t nv = left >= 16 ? 16u : (uint32_t)left;
    uint32_t sl[SL::NV];
#pragma unroll
    for (int i = 0; i < SL::NV; ++i)
      sl[i] = SL::ALIGNED ? ta[tt].w[i] : __builtin_amdgcn_alignbit(i + 1 < SL::NW ? ta[tt].w[i + 1] : 0u, ta[tt].w[i], wsh);
    const uint32_t za = (PROD && D == 64) ? ta[tt].z0 >> (16 * (g & 1)) : ta[tt].z0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accz = {0.f, 0.f, 0.f, 0.f};
    gen_for<0, NS>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      const u32x4 a = gm_decode<BITS, S, SL::NV>(sl, tab);
      acc = mfma_f16(a, qh[S], acc);
      acc = mfma_f16(a, ql[S], acc);
      if constexpr (PROD) {
        const u32x4 zs = gm_signs<D, S>(za, ta[tt].z1, tabz);
        accz = mfma_f16(zs, zh[S], accz);
        accz = mfma_f16(zs, zl[S], accz);
      }
    });
    // plain stores under the lane's own condition (a buffer resource would have to be uniform,
    // and each head's row has its own base)
    if (live) {
      float* dst = out0 + t0 + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = ta[tt].sn[r] * acc[r] + (PROD ? ta[tt].gm[r] * kQ * accz[r] : 0.f);
        if ((uint32_t)(4 * g + r) < nv) dst[r] = v;
      }
    }
  }
}

template <int D, int BITS, bool PROD>
hipError_t scores_gen_launch(const float* ws, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                             const CodebookArgs& cb, float* scores, hipStream_t st) {
  const int ratio = Hq / Hkv;
  constexpr int keys = 64 * gm_tiles<D>();
  const dim3 grid((unsigned)((T + keys - 1) / keys), (unsigned)(B * Hkv), (unsigned)((ratio + 15) / 16));
  hipLaunchKernelGGL((k_scores_gm<D, BITS, PROD>), grid, dim3(256), 0, st, ws, Hq, Hkv, T, rows, K->idx, K->norms,
                     K->qjl, K->rnorms, cb, scores);
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
  hipLaunchKernelGGL((k_qprep_gen<D>), dim3((unsigned)heads), dim3(256), 0, st, q, rot->rt32_dev,
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
  if (Hq / Hkv == 4)
    hipLaunchKernelGGL((k_attn_gen<D, KB, VB, 4, true>), dim3((unsigned)nsplit, (unsigned)(B * Hkv)), dim3(kGenThreads), 0,
                       st, ws, Hq, Hkv, T, rows, nsplit, scale, K->idx, K->norms, V->idx, V->norms, cbk, cbv, parts);
  else
    hipLaunchKernelGGL((k_attn_gen<D, KB, VB, kGenHeadGroup, false>), dim3((unsigned)nsplit, (unsigned)(B * Hkv)),
                       dim3(kGenThreads), 0, st, ws, Hq, Hkv, T, rows, nsplit, scale, K->idx, K->norms, V->idx,
                       V->norms, cbk, cbv, parts);
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
