// General-d TurboQuant encode (d a multiple of 128, 256 <= d <= 4096) and the top-k maximum
// inner-product search over a TurboQuant_prod database.
//
// Encode ([TQ] official steps 1-4 and TurboQuant_prod): the rotation is a tiled GEMM,
// y^T = R x^T, on bf16 MFMA.  A block owns 128 vectors x one 128-coordinate output block ob
// and loops over the contraction in halves of 64 coordinates; each half's pre-swizzled R
// fragments stream into one of two LDS buffers (direct-to-LDS loads) and are shared by the four
// waves, while each wave streams its 32 vectors from HBM as the B operand, one half ahead.
// With the fragment row order of the d = 128 kernel, lane
// (n, G) ends with coordinates 128 ob + 32 G .. + 31 of its vector, so the epilogue bucketizes
// and packs whole words in registers.  The norm is accumulated from the B operand, so no
// separate pass reads x.  Prod runs twice: the first GEMM also writes the rotated-domain
// residual (fp32, unit scale) and per-block partial squared norms to a workspace, and the second
// multiplies the residual by S' = S R^T, keeps the signs and forms gamma.
//
// Search ([FP] inner-product bias and QJL fix): the queries are rotated and sketched by the same
// GEMM kernel, converted once into fp16 MFMA fragments, and the scores are a second GEMM whose B
// operand is decoded from the packed database on the fly (centroids through an LDS table; QJL
// signs as +-(gamma / s) sqrt(pi/2) / d, so one accumulator holds both terms).  The database is
// scored in chunks; the scores of a chunk that can still enter a query's top-k go to the
// workspace, and a per-query kernel merges them into the running top-k.
#include "tq_decode.h"

namespace tq {
namespace {

constexpr int kGWaves = 4;
constexpr int kGTiles = 2;  // 16-vector tiles per wave
static_assert(kGWaves * kGTiles * 16 == kGenVectors, "a block covers kGenVectors vectors");

enum GenEpi { kEpiY = 0, kEpiMse = 1, kEpiRes = 2, kEpiSign = 3, kEpiRaw = 4 };

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at wave_dst + l, wave_dst being
// the same for the whole wave.
__device__ __forceinline__ void lds_dma16(const u32x4* src, u32x4* wave_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)wave_dst, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// A lane's input coordinates of one half chunk: for lane group g, coordinates 64 h + 8 g .. + 7 and
// 64 h + 32 + 8 g .. + 7 of the chunk (the B operand of instructions 2 h and 2 h + 1, in the
// column order of the general-d fragments).
template <bool BF16IN>
struct RawHalf;
template <>
struct RawHalf<true> {
  u32x4 v[2];
};
template <>
struct RawHalf<false> {
  f32x4 v[4];
};

template <bool BF16IN>
__device__ __forceinline__ void load_gen_half(const void* __restrict__ x, int64_t n, int d, int64_t row0, int kc,
                                              int h, int nl, int g, RawHalf<BF16IN>& t) {
  int64_t r = row0 + nl;
  if (r >= n) r = n - 1;
  const int64_t off = r * d + 128 * kc + 64 * h + 8 * g;
  if constexpr (BF16IN) {
    const uint16_t* src = static_cast<const uint16_t*>(x) + off;
    t.v[0] = *reinterpret_cast<const u32x4*>(src);
    t.v[1] = *reinterpret_cast<const u32x4*>(src + 32);
  } else {
    const float* src = static_cast<const float*>(x) + off;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      t.v[2 * i] = *reinterpret_cast<const f32x4*>(src + 32 * i);
      t.v[2 * i + 1] = *reinterpret_cast<const f32x4*>(src + 32 * i + 4);
    }
  }
}

// bf16 B operands (hi, and lo for fp32 input) of the half's two instructions; optional sum of
// squares of the coordinates.
template <bool BF16IN, bool NORM>
__device__ __forceinline__ void half_operand(const RawHalf<BF16IN>& t, u32x4 (&hi)[2], u32x4 (&lo)[2], float& ss) {
  if constexpr (BF16IN) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      hi[s] = t.v[s];
      if constexpr (NORM) {
        // plain-array copy before the bit cast (see the d = 128 encode)
        uint32_t wv[4];
        __builtin_memcpy(wv, &t.v[s], sizeof(wv));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 p = __builtin_bit_cast(bf16x2, wv[j]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
        }
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 a = t.v[2 * s], b = t.v[2 * s + 1];
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      u32x4 h4, l4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x2 pr = {v[2 * j], v[2 * j + 1]};
        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        const f32x2 rem = {v[2 * j] - __uint_as_float(hb << 16), v[2 * j + 1] - __uint_as_float(hb & 0xffff0000u)};
        h4[j] = hb;
        l4[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf16x2));
        if constexpr (NORM) {
          ss = fmaf(v[2 * j], v[2 * j], ss);
          ss = fmaf(v[2 * j + 1], v[2 * j + 1], ss);
        }
      }
      hi[s] = h4;
      lo[s] = l4;
    }
  }
}

// ---------------------------------------------------------------------------------------
// The general-d GEMM.  Grid: (vector tile of 128) x (output block ob), ob fastest.
//   kEpiY    : y_out = unit rotated coordinates, norms (block ob == 0)
//   kEpiRaw  : y_out = post_scale * product (no normalisation)
//   kEpiMse  : packed indices, norms
//   kEpiRes  : as kEpiMse plus res_out = y_unit - C[idx] and rpart[row][ob] = sum of squares
//   kEpiSign : x = residual rows; qjl_out = sign bits; block ob == 0 forms
//              rnorm_out = norms * sqrt(sum_ob rpart)
// ---------------------------------------------------------------------------------------
template <int EPI, bool BF16IN, int APASS, int BITS>
__global__ __launch_bounds__(kGWaves * 64, 2) void k_encode_gen(
    const void* __restrict__ x, int64_t n, int d, const u32x4* __restrict__ frag, float post_scale,
    CodebookArgs cb, float* __restrict__ norms, uint32_t* __restrict__ idx_out, float* __restrict__ y_out,
    float* __restrict__ res_out, float* __restrict__ rpart, uint32_t* __restrict__ qjl_out,
    float* __restrict__ rnorm_out, int og) {
  constexpr bool NORM = EPI != kEpiSign && EPI != kEpiRaw;
  constexpr bool SPLIT = !BF16IN;
  constexpr int H = 1 << (BITS - 1);
  // the fragments of one half chunk (64 coordinates): APASS x 8 output tiles x 2 instructions
  constexpr int HALF = APASS * 1024;
  __shared__ u32x4 lds[2][HALF];
  const int nb = d >> 7;
  int64_t vt = (int64_t)blockIdx.x / nb;
  int ob = (int)((int64_t)blockIdx.x % nb);
  if (og > 0) {
    // Blocks go to the eight XCDs in turn (block L to XCD L % 8).  XCD x takes the output blocks
    // of group x % og (whose R fragments stay in its L2) for every (8 / og)-th vector tile, and
    // takes a tile's output blocks one after the other, so that they run together and read the
    // tile's input rows from L2 once.  (The host sets og only where this is a bijection.)
    const int64_t L = blockIdx.x, slot = L / 8;
    const int xcd = (int)(L % 8), per = nb / og;
    ob = (xcd % og) * per + (int)(slot % per);
    vt = (slot / per) * (8 / og) + xcd / og;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t row0 = vt * kGenVectors + wave * (kGTiles * 16);

  f32x4 acc[kGTiles][8];
#pragma unroll
  for (int j = 0; j < kGTiles; ++j)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[kGTiles];
#pragma unroll
  for (int j = 0; j < kGTiles; ++j) ss[j] = 0.f;

  // The contraction runs in half chunks of 64 coordinates (instructions 2 h, 2 h + 1 of chunk
  // kc).  While half q is multiplied, its successor's fragments stream into the other LDS buffer
  // (direct-to-LDS loads, element e = p x 1024 + t x 128 + 64 i + lane) and each wave's next
  // input coordinates into the registers half q has just converted, so every load has a whole
  // half of MFMAs to arrive.
  const u32x4* fsrc = frag + (size_t)ob * nb * 2 * kFragU4;
  auto issue_frags = [&](int q) {
    const u32x4* src = fsrc + (size_t)(q >> 1) * 2 * kFragU4 + (q & 1) * 128;
    u32x4* dst = lds[q & 1];
#pragma unroll
    for (int u = 0; u < HALF / (kGWaves * 64); ++u) {
      const int e = u * (kGWaves * 64) + threadIdx.x;
      lds_dma16(src + (e >> 10) * kFragU4 + ((e >> 7) & 7) * 256 + (e & 127), dst + u * (kGWaves * 64) + wave * 64);
    }
  };
  const int nq = 2 * nb;
  RawHalf<BF16IN> raw[kGTiles];
  issue_frags(0);
#pragma unroll
  for (int j = 0; j < kGTiles; ++j) load_gen_half<BF16IN>(x, n, d, row0 + 16 * j, 0, 0, nl, g, raw[j]);
  wait_vm_all();
  __syncthreads();
  for (int q = 0; q < nq; ++q) {
    u32x4 bx[kGTiles][2], bxl[kGTiles][2];
#pragma unroll
    for (int j = 0; j < kGTiles; ++j) half_operand<BF16IN, NORM>(raw[j], bx[j], bxl[j], ss[j]);
    if (q + 1 < nq) {
      issue_frags(q + 1);
#pragma unroll
      for (int j = 0; j < kGTiles; ++j)
        load_gen_half<BF16IN>(x, n, d, row0 + 16 * j, (q + 1) >> 1, (q + 1) & 1, nl, g, raw[j]);
    }
    const u32x4* lq = lds[q & 1];
    u32x4 cf[APASS][2], nf[APASS][2];
#pragma unroll
    for (int p = 0; p < APASS; ++p)
#pragma unroll
      for (int i = 0; i < 2; ++i) cf[p][i] = lq[p * 1024 + i * 64 + lane];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t + 1 < 8) {
#pragma unroll
        for (int p = 0; p < APASS; ++p)
#pragma unroll
          for (int i = 0; i < 2; ++i) nf[p][i] = lq[p * 1024 + (t + 1) * 128 + i * 64 + lane];
      }
#pragma unroll
      for (int j = 0; j < kGTiles; ++j) {
        f32x4 a = acc[j][t];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a = mfma_bf16(cf[0][i], bx[j][i], a);
          if constexpr (SPLIT) a = mfma_bf16(cf[0][i], bxl[j][i], a);
          if constexpr (APASS == 2) a = mfma_bf16(cf[1][i], bx[j][i], a);
        }
        acc[j][t] = a;
        __builtin_amdgcn_sched_barrier(0);  // one accumulator's MFMAs back to back
      }
      if (t + 1 < 8) {
#pragma unroll
        for (int p = 0; p < APASS; ++p)
#pragma unroll
          for (int i = 0; i < 2; ++i) cf[p][i] = nf[p][i];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_all();   // the next half's fragments (in LDS) and input coordinates
    __syncthreads();  // every wave is done with lds[q & 1] and sees lds[(q + 1) & 1]
  }

  const float inv_post = 1.0f / post_scale;
#pragma unroll
  for (int j = 0; j < kGTiles; ++j) {
    const int64_t row = row0 + 16 * j + nl;
    const bool valid = row < n;
    if constexpr (EPI == kEpiSign) {
      uint32_t bits = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) bits |= (acc[j][t][r] >= 0.f ? 1u : 0u) << (4 * t + r);
      if (valid) {
        qjl_out[row * (d >> 5) + 4 * ob + g] = bits;
        if (ob == 0 && g == 0) {
          float sum = 0.f;
          for (int o = 0; o < nb; ++o) sum += rpart[row * nb + o];
          rnorm_out[row] = norms[row] * sqrtf(sum);
        }
      }
    } else if constexpr (EPI == kEpiRaw) {
      if (valid) {
        f32x4* dst = reinterpret_cast<f32x4*>(y_out + row * d + 128 * ob + 32 * g);
#pragma unroll
        for (int t = 0; t < 8; ++t) dst[t] = acc[j][t] * post_scale;
      }
    } else {
      float sq = ss[j];
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      const float nrm = sqrtf(sq);
      const bool live = nrm > 0.f;
      const float scale = live ? post_scale / nrm : 0.f;  // raw product -> unit coordinate
      if (valid && ob == 0 && g == 0) norms[row] = nrm;
      if constexpr (EPI == kEpiY) {
        if (valid) {
          f32x4* dst = reinterpret_cast<f32x4*>(y_out + row * d + 128 * ob + 32 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) dst[t] = acc[j][t] * scale;
        }
      } else {
        // sign-magnitude decisions against per-vector thresholds t_p * ||x|| / post_scale, as in
        // the d = 128 encode: idx = (m ^ sign) + K/2, m = #{p : |y| >= t_p}
        float thr[H > 1 ? H - 1 : 1];
        float mags[H];
        const float tsc = nrm * inv_post;
#pragma unroll
        for (int p = 0; p < H - 1; ++p) thr[p] = live ? __int_as_float(cb.tpos[p]) * tsc : INFINITY;
#pragma unroll
        for (int p = 0; p < H; ++p) mags[p] = live ? cb.cpos[p] : 0.f;
        uint32_t w[BITS];
#pragma unroll
        for (int b = 0; b < BITS; ++b) w[b] = 0;
        float rs = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          f32x4 resv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float yv = acc[j][t][r];
            const float ay = fabsf(yv);
            uint32_t m = 0;
            float mag = mags[0];
#pragma unroll
            for (int p = 0; p < H - 1; ++p) {
              const bool ge = ay >= thr[p];
              m += ge ? 1u : 0u;
              if constexpr (EPI == kEpiRes) mag = ge ? mags[p + 1] : mag;
            }
            const uint32_t sgn = (uint32_t)(__float_as_int(yv) >> 31);
            const uint32_t id = (m ^ sgn) + (uint32_t)H;
            if constexpr (EPI == kEpiRes) {
              const float cv =
                  __uint_as_float((__float_as_uint(mag) & 0x7fffffffu) | (__float_as_uint(yv) & 0x80000000u));
              const float res = fmaf(yv, scale, -cv);
              resv[r] = res;
              rs = fmaf(res, res, rs);
            }
            const int p = BITS * (4 * t + r), wi = p >> 5, sh = p & 31;
            w[wi] |= id << sh;
            if (sh + BITS > 32) w[wi + 1] |= id >> (32 - sh);
          }
          if constexpr (EPI == kEpiRes) {
            if (valid) reinterpret_cast<f32x4*>(res_out + row * d + 128 * ob + 32 * g)[t] = resv;
          }
        }
        if (valid) {
          uint32_t* dst = idx_out + row * ((int64_t)d * BITS / 32) + 4 * BITS * ob + BITS * g;
#pragma unroll
          for (int b = 0; b < BITS; ++b) dst[b] = w[b];
        }
        if constexpr (EPI == kEpiRes) {
          rs += __shfl_xor(rs, 16);
          rs += __shfl_xor(rs, 32);
          if (valid && g == 0) rpart[row * nb + ob] = rs;
        }
      }
    }
  }
}

template <int EPI, bool BF16IN, int APASS, int BITS>
hipError_t gen_launch(const void* x, int64_t n, int d, const uint16_t* frag, float post, const CodebookArgs& cb,
                      float* norms, uint32_t* idx, float* y, float* res, float* rpart, uint32_t* qbits, float* rn,
                      hipStream_t st) {
  const int64_t nvt = (n + kGenVectors - 1) / kGenVectors;
  const int nb = d / 128;
  const int64_t blocks = nvt * nb;
  // output-block groups per XCD mapping: the fewest groups (most output blocks per XCD) whose R
  // fragments fit a share of an XCD's 4 MB L2; 0 keeps the plain order
  int og = 0;
  for (int c : {1, 2, 4, 8}) {
    const size_t rbytes = (size_t)(nb / c) * 128 * d * 2 * APASS;
    if (nb % c == 0 && nvt % (8 / c) == 0 && rbytes <= (size_t)5 << 19) {
      og = c;
      break;
    }
  }
  hipLaunchKernelGGL((k_encode_gen<EPI, BF16IN, APASS, BITS>), dim3((unsigned)blocks), dim3(kGWaves * 64), 0, st,
                     x, n, d, reinterpret_cast<const u32x4*>(frag), post, cb, norms, idx, y, res, rpart, qbits, rn, og);
  return hipGetLastError();
}

template <int EPI, int BITS>
hipError_t gen_dispatch(const void* x, bool bf16, int64_t n, int d, const uint16_t* frag, int passes, float post,
                        const CodebookArgs& cb, float* norms, uint32_t* idx, float* y, float* res, float* rpart,
                        hipStream_t st) {
  if (bf16)
    return passes == 1
               ? gen_launch<EPI, true, 1, BITS>(x, n, d, frag, post, cb, norms, idx, y, res, rpart, nullptr, nullptr, st)
               : gen_launch<EPI, true, 2, BITS>(x, n, d, frag, post, cb, norms, idx, y, res, rpart, nullptr, nullptr, st);
  return passes == 1
             ? gen_launch<EPI, false, 1, BITS>(x, n, d, frag, post, cb, norms, idx, y, res, rpart, nullptr, nullptr, st)
             : gen_launch<EPI, false, 2, BITS>(x, n, d, frag, post, cb, norms, idx, y, res, rpart, nullptr, nullptr, st);
}

template <int EPI>
hipError_t gen_dispatch_bits(const void* x, bool bf16, int64_t n, int d, const tq_rotation_s* rot,
                             const CodebookArgs& cb, float* norms, uint32_t* idx, float* res, float* rpart,
                             hipStream_t st) {
  switch (cb.bits) {
    case 1: return gen_dispatch<EPI, 1>(x, bf16, n, d, rot->gfrag_dev, rot->passes, rot->post_scale, cb, norms, idx, nullptr, res, rpart, st);
    case 2: return gen_dispatch<EPI, 2>(x, bf16, n, d, rot->gfrag_dev, rot->passes, rot->post_scale, cb, norms, idx, nullptr, res, rpart, st);
    case 3: return gen_dispatch<EPI, 3>(x, bf16, n, d, rot->gfrag_dev, rot->passes, rot->post_scale, cb, norms, idx, nullptr, res, rpart, st);
    case 4: return gen_dispatch<EPI, 4>(x, bf16, n, d, rot->gfrag_dev, rot->passes, rot->post_scale, cb, norms, idx, nullptr, res, rpart, st);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------
// Search.
// ---------------------------------------------------------------------------------------
constexpr int kSearchKeys = 512;           // database vectors per score block (64 per wave)
constexpr int64_t kSearchChunk = 65536;    // database vectors per score chunk
// The first chunk keeps every score (there is no running k-th result yet) and its merge inserts
// often, so it is kept short; the chunks after it keep only what beats the running k-th result.
constexpr int64_t kSearchFirstChunk = 4096;
constexpr float kSketchScale = 1.0f / 1024.0f;  // query sketch scale; the key side carries 1024

// Query operands in fp16 MFMA fragment order: block (qb, kc) = 4096 u32x4 laid out
// [op][qt][s][lane]; element e of lane (m, g) = Q_op[128 qb + 16 qt + m][128 kc + 32 g + 8 s + e],
// op 0 = unit rotated query, op 1 = its sketch times kSketchScale; rows past nq are zero.
__global__ __launch_bounds__(256) void k_search_qfrag(const float* __restrict__ qr, const float* __restrict__ qs,
                                                       int64_t nq, int d, u32x4* __restrict__ qf) {
  const int nb = d >> 7;
  const int64_t qb = (int64_t)blockIdx.x / nb;
  const int kc = (int)((int64_t)blockIdx.x % nb);
  u32x4* dst = qf + ((size_t)qb * nb + kc) * 4096;
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) {
    const int lane = i & 63, s = (i >> 6) & 3, qt = (i >> 8) & 7, op = i >> 11;
    const int m = lane & 15, g = lane >> 4;
    const int64_t row = qb * 128 + 16 * qt + m;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < nq) {
      const float* src = (op ? qs : qr) + row * d + 128 * kc + 32 * g + 8 * s;
      const float sc = op ? kSketchScale : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(src[2 * j] * sc));
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(src[2 * j + 1] * sc));
        v[j] = lo | (hi << 16);
      }
    }
    dst[i] = v;
  }
}

// Sign operands of the lane's 32 coordinates of a contraction chunk (sign bits z, bit c for
// coordinate c): the fp16 pair {+-mag, +-mag} of coordinates 2 i, 2 i + 1, negative where the
// bit is 0.  sign_pairs arranges the inverted bits once per chunk so that one shift puts both bits
// of a pair on the fp16 sign positions 15 and 31: zp[0] holds coordinates 0..15 (coordinate 2 i
// at bit 2 i, 2 i + 1 at bit 2 i + 16), zp[1] coordinates 16..31 the same way.
__device__ __forceinline__ void sign_pairs(uint32_t z, uint32_t (&zp)[2]) {
  const uint32_t nz = ~z;
  zp[0] = (nz & 0x5555u) | ((nz << 15) & 0x55550000u);
  zp[1] = ((nz >> 16) & 0x5555u) | ((nz >> 1) & 0x55550000u);
}

// The operand of instruction s (coordinates 8 s .. 8 s + 7).
__device__ __forceinline__ u32x4 sign8(const uint32_t (&zp)[2], int s, uint32_t magpair) {
  const uint32_t w = zp[s >> 1];
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * (s & 1) + j;  // pair within the 16-coordinate half
    v[j] = ((w << (15 - 2 * i)) & 0x80008000u) | magpair;
  }
  return v;
}

// Scores of 128 queries against 512 database vectors of one chunk, one block per (query block,
// key block) tile: out[q][j] = ||q|| s_j (<q_rot, C[idx_j]> + (gamma_j / s_j) sqrt(pi/2)/d <q_s, z_j>)
// with unit q.  Eight waves, two per SIMD; wave w decodes its own 64 vectors once per contraction
// slice and multiplies them against all 128 queries (8 query tiles x 4 key tiles = 32 accumulator
// tiles), so each decoded operand feeds 16 MFMAs.  The query operands of contraction chunk kc + 1
// stream from memory straight into the second LDS buffer (2 x 64 KB), and the key words of kc + 1
// into registers, while chunk kc's MFMAs run.
//
// Only scores that can still enter a query's top-k are kept: with kth (the running k-th score of
// every query, from the chunks before) a score is written only if it is strictly larger (an equal
// score loses to the earlier, smaller index), and masks[q][64-vector group] gets one bit per
// written score; without kth (the first chunk) every score of a vector below m is written.
constexpr int kSearchWaves = 8;
constexpr int kSearchThreads = kSearchWaves * 64;
static_assert(kSearchKeys == kSearchWaves * 64, "one 64-vector group per wave");
static_assert(kSearchChunk % kSearchKeys == 0 && kSearchFirstChunk % kSearchKeys == 0, "chunks hold whole key blocks");

// The lane's key words of contraction chunk kc: for key tile j, the BITS index words of its 32
// coordinates (byte offset krow[j] * wb + gi in the index resource) and its sign word (krow[j] * zb
// + gz in the sign resource); the chunk's offset goes in the scalar offset.
template <int BITS>
__device__ __forceinline__ void search_key_words(__amdgpu_buffer_rsrc_t ri, __amdgpu_buffer_rsrc_t rz,
                                                 const uint32_t (&krow)[4], uint32_t wb, uint32_t zb, uint32_t gi,
                                                 uint32_t gz, int kc, uint32_t (&kw)[4][BITS], uint32_t (&zw)[4]) {
  typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t oi = krow[j] * wb + gi, si = 16u * BITS * (uint32_t)kc;
    if constexpr (BITS == 1) {
      kw[j][0] = __builtin_amdgcn_raw_buffer_load_b32(ri, oi, si, 0);
    } else if constexpr (BITS == 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ri, oi, si, 0);
      kw[j][0] = v[0]; kw[j][1] = v[1];
    } else if constexpr (BITS == 3) {
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(ri, oi, si, 0);
      kw[j][0] = v[0]; kw[j][1] = v[1]; kw[j][2] = v[2];
    } else {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ri, oi, si, 0);
      kw[j][0] = v[0]; kw[j][1] = v[1]; kw[j][2] = v[2]; kw[j][3] = v[3];
    }
    zw[j] = __builtin_amdgcn_raw_buffer_load_b32(rz, krow[j] * zb + gz, 16u * (uint32_t)kc, 0);
  }
}

template <int BITS>
__global__ __launch_bounds__(kSearchThreads, 1) void k_search_scores(
    const u32x4* __restrict__ qf, const float* __restrict__ qnorm, int64_t nq, int d,
    const uint32_t* __restrict__ idx, const float* __restrict__ norms, const uint32_t* __restrict__ qbits,
    const float* __restrict__ rnorms, int64_t m, CodebookArgs cb, const float* __restrict__ kth, int k,
    float* __restrict__ out, int64_t ldo, uint64_t* __restrict__ masks, int64_t ldm) {
  // the query operands take 128 KB of LDS: the decode table gets at most 8 KB
  constexpr int TC = table_copies<BITS, false, 8192>();
  using DT = DecodeTable<BITS, false, TC>;
  constexpr int PER = 4096 / kSearchThreads;  // query-operand loads per thread per chunk
  // one LDS array: the decode table first (at address 0, so that its lookups add no base), then
  // the two query-operand buffers, then the fp16 centroids
  // the two query-operand buffers, then the fp16 centroids and the block's query norms and kept-
  // score bounds (the epilogue reads them from here rather than waiting on memory per query)
  __shared__ __attribute__((aligned(16))) uint8_t smem[DT::BYTES + 2 * 4096 * 16 + 32 + 2 * 128 * 4];
  uint8_t* const tab = smem;
  u32x4 (*const lds)[4096] = reinterpret_cast<u32x4 (*)[4096]>(smem + DT::BYTES);
  _Float16* const cent = reinterpret_cast<_Float16*>(smem + DT::BYTES + 2 * 4096 * 16);
  float* const qn_s = reinterpret_cast<float*>(smem + DT::BYTES + 2 * 4096 * 16 + 32);
  float* const th_s = qn_s + 128;
  if (threadIdx.x < 16) cent[threadIdx.x] = (_Float16)cb.c[threadIdx.x];
  // Tile of this block.  Blocks go to the eight XCDs in turn (block L to XCD L % 8); when the
  // grid divides evenly, the tiles are dealt so that each XCD holds consecutive ones, and the
  // query blocks of one key block, which read the same database words, share an L2.
  const unsigned nqb = (unsigned)((nq + 127) / 128);
  unsigned tile = blockIdx.x;
  if (gridDim.x % 8 == 0) tile = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const unsigned qb = tile % nqb, kb = tile / nqb;
  const int nb = d >> 7;
  const int W = d * BITS / 32, dz = d >> 5;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t key0 = (int64_t)kb * kSearchKeys + wave * 64;
  const float kz = 1.2533141373155002512f / (float)d / kSketchScale;  // sqrt(pi/2) / d, rescaled

  const u32x4* qsrc = qf + (size_t)qb * nb * 4096;
  u32x4* const wdst0 = &lds[0][wave * 64];
  u32x4* const wdst1 = &lds[1][wave * 64];
#pragma unroll
  for (int i = 0; i < PER; ++i) lds_dma16(qsrc + i * kSearchThreads + threadIdx.x, wdst0 + i * kSearchThreads);

  float sk[4];
  uint32_t magp[4];
  uint32_t krow[4];  // row of each key tile's vector within the chunk (a chunk holds < 2^32 words)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t r = key0 + 16 * j + nl;
    if (r >= m) r = m - 1;
    krow[j] = (uint32_t)r;
    const float s = norms[r];
    sk[j] = s;
    const float zf = s > 0.f ? rnorms[r] / s * kz : 0.f;
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)zf);
    magp[j] = h | (h << 16);
  }
  if (threadIdx.x < 128) {
    // query norm, and the bound a kept score must beat: the running k-th score (+inf past nq)
    const int64_t q = (int64_t)qb * 128 + threadIdx.x;
    const bool vq = q < nq;
    qn_s[threadIdx.x] = vq ? qnorm[q] : 0.f;
    th_s[threadIdx.x] = !vq ? INFINITY : (kth != nullptr ? kth[q * k + k - 1] : -INFINITY);
  }
  // key words through buffer resources over the chunk (m * W and m * d / 32 words, < 2^32 bytes)
  const __amdgpu_buffer_rsrc_t ri = buffer_rsrc(idx, (uint32_t)(m * W * 4));
  const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(qbits, (uint32_t)(m * dz * 4));
  const uint32_t wb = 4u * W, zb = 4u * dz, gi = 4u * BITS * g, gz = 4u * g;
  uint32_t kw[4][BITS], zw[4];
  search_key_words<BITS>(ri, rz, krow, wb, zb, gi, gz, 0, kw, zw);
  __syncthreads();  // centroids
  build_table<BITS, TC>(tab, cent);
  wait_vm_all();
  __syncthreads();  // table and the first query operands
  const uint32_t laneoff = (uint32_t)(lane % TC) * DT::EB;

  f32x4 acc[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < nb; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nb;
    uint32_t nkw[4][BITS], nzw[4];
    if (more) {
      search_key_words<BITS>(ri, rz, krow, wb, zb, gi, gz, kc + 1, nkw, nzw);
      const u32x4* src = qsrc + (size_t)(kc + 1) * 4096 + threadIdx.x;
      u32x4* dst = cur ? wdst0 : wdst1;
#pragma unroll
      for (int i = 0; i < PER; ++i) lds_dma16(src + i * kSearchThreads, dst + i * kSearchThreads);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int b = 0; b < BITS; ++b) nkw[j][b] = 0u;
        nzw[j] = 0u;
      }
    }
    const u32x4* lq = lds[cur];
    uint32_t zp[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) sign_pairs(zw[j], zp[j]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 bm[4], bz[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bm[j] = decode_keys_or<BITS, TC>(kw[j], s, tab, laneoff);
        bz[j] = sign8(zp[j], s, magp[j]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 ar = lq[(t * 4 + s) * 64 + lane];
        const u32x4 az = lq[((8 + t) * 4 + s) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = mfma_f16(ar, bm[j], acc[t][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = mfma_f16(az, bz[j], acc[t][j]);
      }
      // one contraction slice at a time (the other wave on the SIMD covers the latencies)
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_all();     // next chunk's query operands (in LDS) and key words
    __syncthreads();   // every wave is done with lds[cur] and sees lds[cur ^ 1]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < BITS; ++b) kw[j][b] = nkw[j][b];
      zw[j] = nzw[j];
    }
  }

  // Epilogue: lane (nl, g) holds query 16 t + 4 g + r against vector 16 j + nl of the wave's group.
  // A wave past the chunk's last vector writes nothing (its group is no column of masks).
  if (key0 >= m) return;
  const int64_t gcol = (int64_t)kb * kSearchWaves + wave;
  bool kok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kok[j] = key0 + 16 * j + nl < m;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const f32x4 qn4 = *reinterpret_cast<const f32x4*>(qn_s + 16 * t + 4 * g);
    const f32x4 th4 = *reinterpret_cast<const f32x4*>(th_s + 16 * t + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t q = (int64_t)qb * 128 + 16 * t + 4 * g + r;
      float v[4];
      bool pass[4], any = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = qn4[r] * sk[j] * acc[t][j][r];
        pass[j] = kok[j] && v[j] > th4[r];  // th4 is +inf past nq
        any = any || pass[j];
      }
      uint64_t bits = 0;
      if (__ballot(any) != 0ull) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (pass[j]) out[q * ldo + key0 + 16 * j + nl] = v[j];
          const uint64_t b = __ballot(pass[j]);
          bits |= ((b >> (16 * g)) & 0xffffull) << (16 * j);
        }
      }
      if (nl == 0 && q < nq) masks[q * ldm + gcol] = bits;
    }
  }
}

// (score, index) order of the results: larger score first, then the smaller index.
__device__ __forceinline__ bool better(float a, int64_t ia, float b, int64_t ib) {
  return a > b || (a == b && ia < ib);
}

// Merges the kept scores of one chunk (see k_search_scores) of query blockIdx.x into its running
// top-k (top_s / top_i, sorted; ignored when `first`).  Thread i owns the 64-vector groups i,
// i + 256, ...: it loads all their masks at once, and for a group with bits set it reads the
// float4 batches of the group that hold kept scores.  When no score of the chunk was kept for
// the query, the running top-k stands and the block returns after the masks.  Every thread
// filters what it reads against the running k-th result and keeps a sorted list of KMAX entries;
// k rounds of a block-wide argmax then pick the results.
template <int KMAX>
__global__ __launch_bounds__(256) void k_search_topk(const float* __restrict__ sc, int64_t ldo,
                                                     const uint64_t* __restrict__ masks, int64_t ldm, int64_t ngroups,
                                                     int64_t base, int k, int first, float* __restrict__ top_s,
                                                     int64_t* __restrict__ top_i) {
  constexpr int G = 4;  // groups per thread per pass (a full chunk has 1024)
  __shared__ float red_s[4];
  __shared__ int64_t red_i[4];
  __shared__ int red_t[4];
  __shared__ int winner;
  const int64_t q = blockIdx.x;
  const float* row = sc + q * ldo;
  float ls[KMAX];
  int64_t li[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    ls[i] = -INFINITY;
    li[i] = -1;
  }
  auto insert = [&](float v, int64_t id) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k && better(v, id, ls[i], li[i])) {
        const float ts = ls[i];
        const int64_t ti = li[i];
        ls[i] = v;
        li[i] = id;
        v = ts;
        id = ti;
      }
    }
  };
  // this thread's groups (a chunk has at most 256 G) and their masks
  static_assert(kSearchChunk / 64 <= 256 * G, "one pass over the groups");
  const uint64_t* mrow = masks + q * ldm;
  uint64_t mk[G];
  int any = 0;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int64_t gi = threadIdx.x + (int64_t)u * blockDim.x;
    mk[u] = gi < ngroups ? mrow[gi] : 0ull;
    any |= mk[u] != 0ull;
  }
  // nothing of this chunk beat the running k-th result: the running top-k stands
  if (!__syncthreads_or(any) && !first) return;
  // the bound an element must beat: the running k-th result, then the thread's own k-th entry
  float ks = -INFINITY;
  int64_t ki = -1;
  if (!first) {
    ks = top_s[q * k + k - 1];
    ki = top_i[q * k + k - 1];
    if (threadIdx.x == 0)
      for (int i = 0; i < k; ++i) insert(top_s[q * k + i], top_i[q * k + i]);
  }
  auto consider = [&](float v, int64_t id) {
    if (better(v, id, ks, ki)) {
      insert(v, id);
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i == k - 1 && better(ls[i], li[i], ks, ki)) {
          ks = ls[i];
          ki = li[i];
        }
    }
  };
  const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (mk[u] == 0ull) continue;
    const int64_t gi = threadIdx.x + (int64_t)u * blockDim.x;
    // four batches of four float4 loads (16 scores each)
#pragma unroll 1
    for (int c0 = 0; c0 < 16; c0 += 4) {
      const uint32_t bits = (uint32_t)(mk[u] >> (4 * c0)) & 0xffffu;
      if (bits == 0) continue;
      f32x4 v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        v[c] = (bits >> (4 * c)) & 15u ? row4[gi * 16 + c0 + c] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((bits >> (4 * c + e)) & 1u) consider(v[c][e], base + gi * 64 + 4 * (c0 + c) + e);
    }
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < k; ++r) {
    float bs = ls[0];
    int64_t bi = li[0];
    int bt = threadIdx.x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float os = __shfl_xor(bs, off);
      const int64_t oi = __shfl_xor(bi, off);
      const int ot = __shfl_xor(bt, off);
      if (better(os, oi, bs, bi) || (os == bs && oi == bi && ot < bt)) {
        bs = os;
        bi = oi;
        bt = ot;
      }
    }
    if (lane == 0) {
      red_s[wave] = bs;
      red_i[wave] = bi;
      red_t[wave] = bt;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float s0 = red_s[0];
      int64_t i0 = red_i[0];
      int t0 = red_t[0];
      for (int w = 1; w < 4; ++w)
        if (better(red_s[w], red_i[w], s0, i0) || (red_s[w] == s0 && red_i[w] == i0 && red_t[w] < t0)) {
          s0 = red_s[w];
          i0 = red_i[w];
          t0 = red_t[w];
        }
      winner = t0;
      top_s[q * k + r] = s0;
      top_i[q * k + r] = i0;
    }
    __syncthreads();
    if (threadIdx.x == winner) {
#pragma unroll
      for (int i = 0; i + 1 < KMAX; ++i) {
        ls[i] = ls[i + 1];
        li[i] = li[i + 1];
      }
      ls[KMAX - 1] = -INFINITY;
      li[KMAX - 1] = -1;
    }
  }
}

template <int BITS>
hipError_t search_scores_launch(const u32x4* qf, const float* qnorm, int64_t nq, int d, const tq_packed* db,
                                int64_t base, int64_t m, const CodebookArgs& cb, const float* kth, int k, float* out,
                                int64_t ldo, uint64_t* masks, int64_t ldm, hipStream_t st) {
  const int W = d * BITS / 32;
  const int64_t blocks = (nq + 127) / 128 * ((m + kSearchKeys - 1) / kSearchKeys);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_search_scores<BITS>), dim3((unsigned)blocks), dim3(kSearchThreads), 0, st, qf, qnorm, nq, d,
                     db->idx + base * W, db->norms + base, db->qjl + base * (d / 32), db->rnorms + base, m, cb, kth, k,
                     out, ldo, masks, ldm);
  return hipGetLastError();
}

struct SearchLayout {
  size_t qr, qs, qn, qf, sc, mk, total;
  int64_t chunk;  // database vectors per score chunk
  int64_t ldo;    // score row stride (a multiple of 64 floats)
  int64_t ldm;    // mask row stride: 64-vector groups per chunk
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

SearchLayout search_layout(int64_t nq, int64_t n, int d) {
  SearchLayout l;
  const int64_t nqp = (nq + 127) / 128 * 128;
  l.chunk = n < kSearchChunk ? (n > 0 ? n : 1) : kSearchChunk;
  l.ldo = (l.chunk + 63) / 64 * 64;
  l.qr = 0;
  l.qs = l.qr + align256((size_t)nqp * d * 4);
  l.qn = l.qs + align256((size_t)nqp * d * 4);
  l.qf = l.qn + align256((size_t)nqp * 4);
  l.ldm = l.ldo / 64;
  l.sc = l.qf + align256((size_t)(nqp / 128) * (d / 128) * 4096 * 16);
  l.mk = l.sc + align256((size_t)nq * l.ldo * 4);
  l.total = l.mk + align256((size_t)nq * l.ldm * 8);
  return l;
}

}  // namespace

size_t encode_general_ws_per_vector(int d) { return (size_t)d * 4 + (size_t)(d / 128) * 4; }

hipError_t launch_encode_general(const void* x, bool bf16, int64_t n, int d, const tq_rotation_s* rot,
                                 const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                 uint32_t* qjl_bits, float* rnorms, float* y_out, void* ws, size_t ws_bytes,
                                 hipStream_t st) {
  if (y_out)
    return gen_dispatch<kEpiY, 1>(x, bf16, n, d, rot->gfrag_dev, rot->passes, rot->post_scale, cb, norms, nullptr,
                                  y_out, nullptr, nullptr, st);
  if (!qjl) return gen_dispatch_bits<kEpiMse>(x, bf16, n, d, rot, cb, norms, idx, nullptr, nullptr, st);
  const size_t per = encode_general_ws_per_vector(d);
  const int64_t cap = (int64_t)(ws_bytes / per);
  const int64_t chunk = cap >= n ? n : cap / kGenVectors * kGenVectors;
  if (chunk <= 0) return hipErrorInvalidValue;
  float* res = static_cast<float*>(ws);
  float* rpart = res + (size_t)chunk * d;
  const int W = d * cb.bits / 32;
  const size_t esz = bf16 ? 2 : 4;
  for (int64_t base = 0; base < n; base += chunk) {
    const int64_t m = n - base < chunk ? n - base : chunk;
    const void* xb = static_cast<const char*>(x) + (size_t)base * d * esz;
    hipError_t e = gen_dispatch_bits<kEpiRes>(xb, bf16, m, d, rot, cb, norms + base, idx + base * W, res, rpart, st);
    if (e != hipSuccess) return e;
    e = gen_launch<kEpiSign, false, 2, 1>(res, m, d, qjl->gfrag_dev, 1.0f, cb, norms + base, nullptr, nullptr, nullptr,
                                          rpart, qjl_bits + base * (d / 32), rnorms + base, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t search_workspace_bytes(int64_t nq, int64_t n, int d, int k) {
  (void)k;
  return search_layout(nq, n, d).total;
}

hipError_t launch_search_topk(const float* q, int64_t nq, const tq_packed* db, const CodebookArgs& cb,
                              const tq_rotation_s* rot, const tq_qjl_s* qjl, int k, float* top_s,
                              int64_t* top_i, void* ws, hipStream_t st) {
  const int d = db->d;
  const SearchLayout l = search_layout(nq, db->n, d);
  char* w = static_cast<char*>(ws);
  float* qr = reinterpret_cast<float*>(w + l.qr);
  float* qs = reinterpret_cast<float*>(w + l.qs);
  float* qn = reinterpret_cast<float*>(w + l.qn);
  u32x4* qf = reinterpret_cast<u32x4*>(w + l.qf);
  float* sc = reinterpret_cast<float*>(w + l.sc);
  uint64_t* mk = reinterpret_cast<uint64_t*>(w + l.mk);
  // query prologue: unit rotated queries and norms, then the sketch S q / ||q|| = S' (R q / ||q||)
  const uint16_t* rfrag = rot->gfrag_dev;
  const uint16_t* sfrag = qjl->gfrag_dev;
  hipError_t e = gen_dispatch<kEpiY, 1>(q, false, nq, d, rfrag, rot->passes, rot->post_scale, cb, qn, nullptr, qr,
                                        nullptr, nullptr, st);
  if (e != hipSuccess) return e;
  e = gen_launch<kEpiRaw, false, 2, 1>(qr, nq, d, sfrag, 1.0f, cb, nullptr, nullptr, qs, nullptr, nullptr, nullptr,
                                       nullptr, st);
  if (e != hipSuccess) return e;
  const int64_t nqb = (nq + 127) / 128;
  hipLaunchKernelGGL(k_search_qfrag, dim3((unsigned)(nqb * (d / 128))), dim3(256), 0, st, qr, qs, nq, d, qf);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = db->n;
  int64_t base = 0;
  do {
    const int64_t cap = base == 0 ? kSearchFirstChunk : l.chunk;
    const int64_t m = n - base < cap ? n - base : cap;
    // after the first chunk the running k-th scores decide which scores are kept
    const float* kth = base == 0 ? nullptr : top_s;
    if (m > 0) {
      switch (cb.bits) {
        case 1: e = search_scores_launch<1>(qf, qn, nq, d, db, base, m, cb, kth, k, sc, l.ldo, mk, l.ldm, st); break;
        case 2: e = search_scores_launch<2>(qf, qn, nq, d, db, base, m, cb, kth, k, sc, l.ldo, mk, l.ldm, st); break;
        case 3: e = search_scores_launch<3>(qf, qn, nq, d, db, base, m, cb, kth, k, sc, l.ldo, mk, l.ldm, st); break;
        case 4: e = search_scores_launch<4>(qf, qn, nq, d, db, base, m, cb, kth, k, sc, l.ldo, mk, l.ldm, st); break;
        default: return hipErrorInvalidValue;
      }
      if (e != hipSuccess) return e;
    }
    const int64_t groups = (m + 63) / 64;
    if (k <= 16)
      hipLaunchKernelGGL(k_search_topk<16>, dim3((unsigned)nq), dim3(256), 0, st, sc, l.ldo, mk, l.ldm, groups, base, k,
                         base == 0 ? 1 : 0, top_s, top_i);
    else
      hipLaunchKernelGGL(k_search_topk<kSearchMaxK>, dim3((unsigned)nq), dim3(256), 0, st, sc, l.ldo, mk, l.ldm, groups,
                         base, k, base == 0 ? 1 : 0, top_s, top_i);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    base += m;
  } while (base < n);
  return hipSuccess;
}

}  // namespace tq
