// Host side of the TurboQuant library: seeded generator, Householder QR, Lloyd-Max codebook,
// handle lifetime, argument validation and the C ABI entry points.
//
// Host arithmetic is compiled without floating-point contraction so that every fp64 step
// rounds once, as written.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "tq_cache.h"
#include "tq_internal.h"
#include "tq_split.h"

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

tq_status ok() { return TQ_OK; }

tq_status hip_fail(hipError_t e, const char* what) {
  return fail(TQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

std::atomic<uint64_t> g_next_id{1};

// ---- SplitMix64 (Steele, Lea, Flood 2014), counter form --------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline uint64_t draw(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * kGamma); }

inline double uniform53(uint64_t z) { return (double)(z >> 11) * 0x1.0p-53; }

// Box-Muller, cosine branch, draws 2e and 2e+1.
void gaussian_fill(uint64_t seed, int64_t n, double* out) {
  const double two_pi = 6.283185307179586476925;
  for (int64_t e = 0; e < n; ++e) {
    double u1 = uniform53(draw(seed, 2 * (uint64_t)e));
    double u2 = uniform53(draw(seed, 2 * (uint64_t)e + 1));
    out[e] = std::sqrt(-2.0 * std::log(1.0 - u1)) * std::cos(two_pi * u2);
  }
}

// ---- parallel helper ------------------------------------------------------------------
template <class F>
void parallel_for(int64_t begin, int64_t end, int64_t grain, F&& f) {
  int64_t n = end - begin;
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  int64_t nthreads = std::min<int64_t>(std::min<int64_t>(hw, 16), (n + grain - 1) / std::max<int64_t>(grain, 1));
  if (nthreads <= 1) {
    for (int64_t i = begin; i < end; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(nthreads);
  int64_t chunk = (n + nthreads - 1) / nthreads;
  for (int64_t t = 0; t < nthreads; ++t) {
    int64_t lo = begin + t * chunk, hi = std::min(end, lo + chunk);
    if (lo >= hi) break;
    th.emplace_back([lo, hi, &f]() {
      for (int64_t i = lo; i < hi; ++i) f(i);
    });
  }
  for (auto& t : th) t.join();
}

// ---- Householder QR with the non-negative-diagonal convention ----------------------------
// g: d x d row-major.  Returns R = Q D (row-major) where G = Q T, T upper triangular, and D
// flips the columns of Q whose diagonal entry of T is negative (sign(0) = +1), so that the
// factorisation G = (Q D)(D T) has a non-negative diagonal and is unique.
void qr_rotation(int d, const double* g, double* r_out) {
  // column-major working copy: a[j*d + i] = G[i][j]
  std::vector<double> a((size_t)d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) a[(size_t)j * d + i] = g[(size_t)i * d + j];
  std::vector<double> vs((size_t)d * d, 0.0);  // Householder vectors, column k from row k
  std::vector<double> diag(d, 0.0);
  std::vector<double> beta(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double* col = &a[(size_t)k * d];
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += col[i] * col[i];
    double norm = std::sqrt(norm2);
    double* v = &vs[(size_t)k * d];
    if (norm == 0.0) {
      diag[k] = 0.0;
      beta[k] = 0.0;
      continue;
    }
    double alpha = col[k] >= 0.0 ? -norm : norm;
    for (int i = k; i < d; ++i) v[i] = col[i];
    v[k] -= alpha;
    double vnorm2 = 0.0;
    for (int i = k; i < d; ++i) vnorm2 += v[i] * v[i];
    beta[k] = vnorm2 > 0.0 ? 2.0 / vnorm2 : 0.0;
    diag[k] = alpha;
    const double bk = beta[k];
    // apply H = I - beta v v^T to the trailing columns
    parallel_for(k + 1, d, 64, [&](int64_t j) {
      double* cj = &a[(size_t)j * d];
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * cj[i];
      double f = bk * dot;
      for (int i = k; i < d; ++i) cj[i] -= f * v[i];
    });
  }
  // Q = H_0 H_1 ... H_{d-1}: accumulate backwards on the identity (column-major q)
  std::vector<double> q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    if (beta[k] == 0.0) continue;
    const double* v = &vs[(size_t)k * d];
    const double bk = beta[k];
    parallel_for(k, d, 64, [&](int64_t j) {
      double* cj = &q[(size_t)j * d];
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * cj[i];
      double f = bk * dot;
      for (int i = k; i < d; ++i) cj[i] -= f * v[i];
    });
  }
  for (int j = 0; j < d; ++j) {
    double sgn = diag[j] >= 0.0 ? 1.0 : -1.0;
    for (int i = 0; i < d; ++i) r_out[(size_t)i * d + j] = sgn * q[(size_t)j * d + i];
  }
}

bool is_pow2(int d) { return d > 0 && (d & (d - 1)) == 0; }

// Group size of the block Hadamard rotation (TQ_ROT_BLOCK_WHT).
constexpr int kBlockWhtGroup = 32;

void hadamard_rotation(int d, uint64_t seed, double* r_out) {
  const double inv = 1.0 / std::sqrt((double)d);
  for (int j = 0; j < d; ++j) {
    double sigma = (draw(seed, (uint64_t)j) >> 63) ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) {
      int par = __builtin_popcount((unsigned)(i & j)) & 1;
      r_out[(size_t)i * d + j] = (par ? -1.0 : 1.0) * sigma * inv;
    }
  }
}

// Block randomized Hadamard: (1/sqrt(g)) blockdiag(H_g, ...) diag(sigma), the signs drawn as for
// the full transform; d a multiple of g.
void block_hadamard_rotation(int d, int g, uint64_t seed, double* r_out) {
  const double inv = 1.0 / std::sqrt((double)g);
  for (int j = 0; j < d; ++j) {
    double sigma = (draw(seed, (uint64_t)j) >> 63) ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) {
      double v = 0.0;
      if (i / g == j / g) {
        int par = __builtin_popcount((unsigned)((i % g) & (j % g))) & 1;
        v = (par ? -1.0 : 1.0) * sigma * inv;
      }
      r_out[(size_t)i * d + j] = v;
    }
  }
}

// ---- Lloyd-Max on the rotated-coordinate density, grid recipe ---------------------------
constexpr int kGridPoints = 50000;
constexpr int kIterations = 300;

void lloyd_codebook(int d, int b, int density, double* c_out, double* t_out) {
  const double sigma = 1.0 / std::sqrt((double)d);
  const double lo = std::max(-6.0 * sigma, -1.0);
  const double hi = std::min(6.0 * sigma, 1.0);
  const int n = kGridPoints;
  std::vector<double> x(n), w(n), wx(n);
  const double step = (hi - lo) / (double)(n - 1);
  for (int j = 0; j < n; ++j) x[j] = (double)j * step + lo;
  x[n - 1] = hi;
  const double expo = 0.5 * (double)(d - 3);
  for (int j = 0; j < n; ++j) {
    double xx = x[j] * x[j];
    if (density == TQ_DENSITY_BETA) {
      double one_minus = 1.0 - xx;
      w[j] = one_minus > 0.0 ? std::exp(expo * std::log1p(-xx)) : 0.0;
    } else {
      w[j] = std::exp(-0.5 * (double)d * x[j] * x[j]);
    }
    wx[j] = w[j] * x[j];
  }
  const int k = 1 << b;
  const double m = std::min(3.0 * sigma, 1.0);
  double c[tq::kMaxCentroids], t[tq::kMaxCentroids];
  for (int i = 0; i < k; ++i) c[i] = m * (-1.0 + (2.0 * (double)i + 1.0) / (double)k);
  for (int it = 0; it < kIterations; ++it) {
    for (int i = 0; i + 1 < k; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
    double mass[tq::kMaxCentroids] = {0}, mom[tq::kMaxCentroids] = {0};
    int cell = 0;  // grid is increasing: the cell index only grows
    for (int j = 0; j < n; ++j) {
      while (cell < k - 1 && x[j] >= t[cell]) ++cell;
      mass[cell] += w[j];
      mom[cell] += wx[j];
    }
    for (int i = 0; i < k; ++i)
      if (mass[i] > 0.0) c[i] = mom[i] / mass[i];
  }
  double cm[tq::kMaxCentroids];
  for (int i = 0; i < k; ++i) cm[i] = 0.5 * (c[i] - c[k - 1 - i]);
  for (int i = 0; i < k; ++i) c_out[i] = cm[i];
  for (int i = 0; i + 1 < k; ++i) t_out[i] = 0.5 * (cm[i] + cm[i + 1]);
}

void fill_args(tq_codebook_s* cb) {
  const int k = 1 << cb->b;
  for (int i = 0; i < tq::kMaxCentroids; ++i) {
    cb->args.c[i] = i < k ? (float)cb->c[i] : 0.0f;
    cb->args.t[i] = i + 1 < k ? (float)cb->t[i] : INFINITY;
  }
  cb->args.bits = cb->b;
  bool sym = cb->args.t[k / 2 - 1] == 0.0f;
  for (int i = 0; i < k && sym; ++i) sym = cb->args.c[k - 1 - i] == -cb->args.c[i];
  for (int i = 0; i + 1 < k && sym; ++i) sym = cb->args.t[k - 2 - i] == -cb->args.t[i];
  cb->args.sym = sym ? 1 : 0;
  for (int p = 0; p < tq::kMaxCentroids / 2; ++p) {
    cb->args.cpos[p] = p < k / 2 ? cb->args.c[k / 2 + p] : 0.0f;
    float tp = p < k / 2 - 1 ? cb->args.t[k / 2 + p] : INFINITY;
    int bitsv;
    std::memcpy(&bitsv, &tp, 4);
    cb->args.tpos[p] = bitsv;
  }
}

// ---- bf16 split fragments ------------------------------------------------------------
inline uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // NaN
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

inline float bf16_to_f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// B-operand fragments of M^T for the token-row product (x M^T): lane (n, g), instruction s,
// element e holds M[8 n + cb][32 g + 8 s + e].
void build_fragments_t(const double* m, double scale, std::vector<uint16_t>& out) {
  out.assign(2 * (size_t)tq::kFragElems, 0);
  for (int cb = 0; cb < 8; ++cb)
    for (int s = 0; s < 4; ++s)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          int nn = lane % 16, g = lane / 16;
          int row = 8 * nn + cb;
          int col = 32 * g + 8 * s + e;
          float v = (float)(m[(size_t)row * 128 + col] * scale);
          uint16_t hi = bf16_rne(v);
          uint16_t lo = bf16_rne(v - bf16_to_f(hi));
          size_t idx = (((size_t)cb * 4 + s) * 64 + lane) * 8 + e;
          out[idx] = hi;
          out[(size_t)tq::kFragElems + idx] = lo;
        }
}

// Fragments of the d = 128 matrix m (row-major fp64) scaled by `scale`.
void build_fragments(const double* m, double scale, std::vector<uint16_t>& out) {
  out.assign(2 * (size_t)tq::kFragElems, 0);
  for (int cb = 0; cb < 8; ++cb)
    for (int s = 0; s < 4; ++s)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          int mm = lane % 16, g = lane / 16;
          int row = 32 * (mm / 4) + 4 * cb + (mm % 4);
          int col = 32 * g + 8 * s + e;
          float v = (float)(m[(size_t)row * 128 + col] * scale);
          uint16_t hi = bf16_rne(v);
          float rem = v - bf16_to_f(hi);
          uint16_t lo = bf16_rne(rem);
          size_t idx = (((size_t)cb * 4 + s) * 64 + lane) * 8 + e;
          out[idx] = hi;
          out[(size_t)tq::kFragElems + idx] = lo;
        }
}

// Fragments of the d = 128 matrix m scaled by `scale` for v_mfma_f32_32x32x16_bf16 (A operand):
// [pass][ob][s][lane][e] = M[o][c], i = lane % 32, j = lane / 32,
// o = 64 ((i >> 2) & 1) + 16 ob + 4 (i >> 3) + (i & 3), c = 64 j + 8 s + e.  With this row order,
// output block ob's register r in lane (i, j) is coordinate 64 j + 16 ob + r.
void build_fragments32(const double* m, double scale, std::vector<uint16_t>& out) {
  out.assign(2 * (size_t)tq::kFragElems, 0);
  for (int ob = 0; ob < 4; ++ob)
    for (int s = 0; s < 8; ++s)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          const int i = lane % 32, j = lane / 32;
          const int row = 64 * ((i >> 2) & 1) + 16 * ob + 4 * (i >> 3) + (i & 3);
          const int col = 64 * j + 8 * s + e;
          const float v = (float)(m[(size_t)row * 128 + col] * scale);
          const uint16_t hi = bf16_rne(v);
          const uint16_t lo = bf16_rne(v - bf16_to_f(hi));
          const size_t idx = (((size_t)ob * 8 + s) * 64 + lane) * 8 + e;
          out[idx] = hi;
          out[(size_t)tq::kFragElems + idx] = lo;
        }
}

// Chunked fragments of a d x d matrix (d a multiple of 128) for the general-d GEMM kernels:
// chunk (ob, kc) is the 128 x 128 block M[128 ob .., 128 kc ..] with build_fragments' row order,
// but instruction s of lane group g takes columns 32 s + 8 g .. + 7 of the chunk, so that
// instructions 2 h and 2 h + 1 span the contiguous columns 64 h .. 64 h + 63 (the GEMM streams its
// input in such halves); chunks follow each other as [ob][kc][pass].
void build_fragments_g(const double* m, int d, double scale, std::vector<uint16_t>& out) {
  const int nb = d / 128;
  out.assign((size_t)nb * nb * 2 * tq::kFragElems, 0);
  parallel_for(0, (int64_t)nb * nb, 1, [&](int64_t blk) {
    const int ob = (int)(blk / nb), kc = (int)(blk % nb);
    const size_t base = (size_t)blk * 2 * tq::kFragElems;
    for (int t = 0; t < 8; ++t)
      for (int s = 0; s < 4; ++s)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const int mm = lane % 16, g = lane / 16;
            const int row = 128 * ob + 32 * (mm / 4) + 4 * t + (mm % 4);
            const int col = 128 * kc + 32 * s + 8 * g + e;
            const float v = (float)(m[(size_t)row * d + col] * scale);
            const uint16_t hi = bf16_rne(v);
            const uint16_t lo = bf16_rne(v - bf16_to_f(hi));
            const size_t idx = (((size_t)t * 4 + s) * 64 + lane) * 8 + e;
            out[base + idx] = hi;
            out[base + tq::kFragElems + idx] = lo;
          }
  });
}

inline bool general_d(int d) { return d % 128 == 0 && d >= 256 && d <= 4096; }

template <class T>
tq_status upload(const std::vector<T>& host, T** dev, const char* what) {
  hipError_t e = hipMalloc((void**)dev, host.size() * sizeof(T));
  if (e != hipSuccess) return hip_fail(e, what);
  e = hipMemcpy(*dev, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    hipFree(*dev);
    *dev = nullptr;
    return hip_fail(e, what);
  }
  return TQ_OK;
}

void free_rotation(tq_rotation_s* r) {
  if (!r) return;
  if (r->r32_dev) hipFree(r->r32_dev);
  if (r->rt32_dev) hipFree(r->rt32_dev);
  if (r->frag_dev) hipFree(r->frag_dev);
  if (r->fragt_dev) hipFree(r->fragt_dev);
  if (r->fragT_dev) hipFree(r->fragT_dev);
  if (r->frag32_dev) hipFree(r->frag32_dev);
  if (r->gfrag_dev) hipFree(r->gfrag_dev);
  delete r;
}

void free_qjl(tq_qjl_s* q) {
  if (!q) return;
  if (q->s32_dev) hipFree(q->s32_dev);
  if (q->st32_dev) hipFree(q->st32_dev);
  if (q->frag_dev) hipFree(q->frag_dev);
  if (q->frag32_dev) hipFree(q->frag32_dev);
  if (q->gfrag_dev) hipFree(q->gfrag_dev);
  if (q->sp32_dev) hipFree(q->sp32_dev);
  delete q;
}

tq_status finish_rotation(tq_rotation_s* r) {
  const int d = r->d;
  std::vector<float> r32((size_t)d * d), rt32((size_t)d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      r32[(size_t)i * d + j] = (float)r->r[(size_t)i * d + j];
      rt32[(size_t)j * d + i] = (float)r->r[(size_t)i * d + j];
    }
  tq_status st = upload(r32, &r->r32_dev, "upload rotation");
  if (st != TQ_OK) return st;
  st = upload(rt32, &r->rt32_dev, "upload rotation transpose");
  if (st != TQ_OK) return st;
  if (d == tq::kFragD) {
    std::vector<uint16_t> frag, fragt, frag32;
    if (r->kind == TQ_ROT_WHT || r->kind == TQ_ROT_BLOCK_WHT) {
      // sqrt(g) R = H diag(sigma) (block diagonal for BLOCK_WHT, g = its group; g = d otherwise)
      // has entries 0 and +-1: exact in bf16, one pass, scale after.
      const double g = std::sqrt((double)(r->kind == TQ_ROT_WHT ? d : kBlockWhtGroup));
      build_fragments(r->r.data(), g, frag);
      build_fragments_t(r->r.data(), g, fragt);
      build_fragments32(r->r.data(), g, frag32);
      r->passes = 1;
      r->post_scale = (float)(1.0 / g);
    } else {
      build_fragments(r->r.data(), 1.0, frag);
      build_fragments_t(r->r.data(), 1.0, fragt);
      build_fragments32(r->r.data(), 1.0, frag32);
      r->passes = 2;
      r->post_scale = 1.0f;
    }
    st = upload(frag, &r->frag_dev, "upload rotation fragments");
    if (st != TQ_OK) return st;
    st = upload(fragt, &r->fragt_dev, "upload rotation fragments");
    if (st != TQ_OK) return st;
    st = upload(frag32, &r->frag32_dev, "upload rotation fragments");
    if (st != TQ_OK) return st;
    {
      // fragments of R^T in the same layout (for y = R^T x); a (block) Hadamard R^T has the same
      // entries up to order, so the same scale and pass count hold
      std::vector<double> rtr((size_t)d * d);
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) rtr[(size_t)j * d + i] = r->r[(size_t)i * d + j];
      const bool wht_t = r->kind == TQ_ROT_WHT || r->kind == TQ_ROT_BLOCK_WHT;
      std::vector<uint16_t> fragT;
      build_fragments(rtr.data(), wht_t ? std::sqrt((double)(r->kind == TQ_ROT_WHT ? d : kBlockWhtGroup)) : 1.0,
                      fragT);
      st = upload(fragT, &r->fragT_dev, "upload rotation fragments");
      if (st != TQ_OK) return st;
    }
    // the general-d layout too: the search's query prologue runs the general-d GEMM at any d
    const bool wht = r->kind == TQ_ROT_WHT || r->kind == TQ_ROT_BLOCK_WHT;
    build_fragments_g(r->r.data(), d, wht ? std::sqrt((double)(r->kind == TQ_ROT_WHT ? d : kBlockWhtGroup)) : 1.0,
                      frag);
    st = upload(frag, &r->gfrag_dev, "upload rotation fragments");
    if (st != TQ_OK) return st;
  } else if (general_d(d)) {
    std::vector<uint16_t> frag;
    const bool wht = r->kind == TQ_ROT_WHT || r->kind == TQ_ROT_BLOCK_WHT;
    // (block) WHT: sqrt(g) R has entries 0 and +-1, exact in bf16: one pass, scaled after the product.
    const double g = std::sqrt((double)(r->kind == TQ_ROT_WHT ? d : kBlockWhtGroup));
    build_fragments_g(r->r.data(), d, wht ? g : 1.0, frag);
    r->passes = wht ? 1 : 2;
    r->post_scale = wht ? (float)(1.0 / g) : 1.0f;
    st = upload(frag, &r->gfrag_dev, "upload rotation fragments");
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

tq_status make_qjl(int d, std::vector<double>&& s, tq_rotation_t rot, tq_qjl_t* out) {
  auto* q = new (std::nothrow) tq_qjl_s();
  if (!q) return fail(TQ_ENOMEM, "host allocation failed");
  q->d = d;
  q->rot_id = rot->id;
  q->s = std::move(s);
  hipGetDevice(&q->device);
  std::vector<float> s32((size_t)d * d), st32((size_t)d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      s32[(size_t)i * d + j] = (float)q->s[(size_t)i * d + j];
      st32[(size_t)j * d + i] = (float)q->s[(size_t)i * d + j];
    }
  tq_status st = upload(s32, &q->s32_dev, "upload qjl");
  if (st == TQ_OK) st = upload(st32, &q->st32_dev, "upload qjl transpose");
  if (st == TQ_OK && (d == tq::kFragD || general_d(d) || d == 64)) {
    // S' = S R^T in fp64
    std::vector<double> sp((size_t)d * d, 0.0);
    const double* sm = q->s.data();
    const double* rm = rot->r.data();
    parallel_for(0, d, 8, [&](int64_t i) {
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += sm[(size_t)i * d + k] * rm[(size_t)j * d + k];
        sp[(size_t)i * d + j] = acc;
      }
    });
    std::vector<uint16_t> frag;
    if (d == tq::kFragD) {
      build_fragments(sp.data(), 1.0, frag);
      st = upload(frag, &q->frag_dev, "upload qjl fragments");
      if (st == TQ_OK) {
        build_fragments32(sp.data(), 1.0, frag);
        st = upload(frag, &q->frag32_dev, "upload qjl fragments");
      }
      if (st == TQ_OK) {
        // the general-d layout too, for the search's query prologue
        build_fragments_g(sp.data(), d, 1.0, frag);
        st = upload(frag, &q->gfrag_dev, "upload qjl fragments");
      }
    } else if (d == 64) {
      // the d = 64 prod encode splits S' into its own fragments in the kernel
      std::vector<float> sp32(sp.begin(), sp.end());
      st = upload(sp32, &q->sp32_dev, "upload qjl S'");
    } else {
      build_fragments_g(sp.data(), d, 1.0, frag);
      st = upload(frag, &q->gfrag_dev, "upload qjl fragments");
    }
  }
  if (st != TQ_OK) {
    free_qjl(q);
    return st;
  }
  *out = q;
  return ok();
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

tq_status check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  return TQ_OK;
}

// Kernel timers: event pairs created on first use, handed to one launch each.
struct Timer {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false, launched = false;
};
std::mutex g_timer_mu;
Timer g_timers[TQ_MAX_TIMERS];
constexpr int kTimedKinds = 2;
thread_local int g_armed_timer[kTimedKinds] = {-1, -1};

}  // namespace

bool tq::take_armed_timer(int which, hipEvent_t* start, hipEvent_t* stop) {
  if (which < 0 || which >= kTimedKinds) return false;
  const int id = g_armed_timer[which];
  if (id < 0) return false;
  g_armed_timer[which] = -1;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  *start = g_timers[id].start;
  *stop = g_timers[id].stop;
  g_timers[id].launched = true;
  return true;
}

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

int tq_timer_arm(void) { return tq_timer_arm_kernel(TQ_TIMED_ENCODE); }

int tq_timer_arm_kernel(tq_timed_kernel which) {
  if ((int)which < 0 || (int)which >= kTimedKinds) {
    fail(TQ_EINVAL, "tq_timer_arm_kernel: unknown kernel kind %d", (int)which);
    return -1;
  }
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (g_armed_timer[which] >= 0) {           // re-arming a kind replaces its armed timer
    g_timers[g_armed_timer[which]].used = false;
    g_armed_timer[which] = -1;
  }
  for (int i = 0; i < TQ_MAX_TIMERS; ++i) {
    Timer& t = g_timers[i];
    if (t.used) continue;
    if (!t.start && (hipEventCreate(&t.start) != hipSuccess || hipEventCreate(&t.stop) != hipSuccess)) {
      if (t.start) (void)hipEventDestroy(t.start);
      t.start = t.stop = nullptr;
      fail(TQ_EDEVICE, "tq_timer_arm: cannot create HIP events");
      return -1;
    }
    t.used = true;
    t.launched = false;
    g_armed_timer[which] = i;
    return i;
  }
  fail(TQ_ENOMEM, "tq_timer_arm: all %d timers in use", TQ_MAX_TIMERS);
  return -1;
}

tq_status tq_timer_read(int id, float* ms) {
  if (!ms || id < 0 || id >= TQ_MAX_TIMERS) return fail(TQ_EINVAL, "tq_timer_read: bad arguments");
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_timer_mu);
    if (!g_timers[id].used || !g_timers[id].launched)
      return fail(TQ_EINVAL, "tq_timer_read: timer %d was not armed and launched", id);
    a = g_timers[id].start;
    b = g_timers[id].stop;
  }
  hipError_t e = hipEventSynchronize(b);
  if (e != hipSuccess) return hip_fail(e, "tq_timer_read");
  e = hipEventElapsedTime(ms, a, b);
  if (e != hipSuccess) return hip_fail(e, "tq_timer_read");
  return ok();
}

void tq_timer_reset(void) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (Timer& t : g_timers) t.used = t.launched = false;
  for (int& a : g_armed_timer) a = -1;
}

tq_status tq_peak_read(const void* src_dev, size_t bytes, int blocks, uint32_t* sink_dev, void* stream) {
  const char* fn = "tq_peak_read";
  if (!src_dev || bytes == 0 || bytes % 16 != 0 || blocks < 1) return fail(TQ_EINVAL, "%s: bad arguments", fn);
  return check_launch(tq::launch_peak_read(src_dev, (int64_t)bytes, blocks, sink_dev, as_stream(stream)), fn);
}

tq_status tq_peak_copy(void* dst_dev, const void* src_dev, size_t bytes, int blocks, void* stream) {
  const char* fn = "tq_peak_copy";
  if (!src_dev || !dst_dev || bytes == 0 || bytes % 16 != 0 || blocks < 1) return fail(TQ_EINVAL, "%s: bad arguments", fn);
  return check_launch(tq::launch_peak_copy(dst_dev, src_dev, (int64_t)bytes, blocks, as_stream(stream)), fn);
}

tq_status tq_peak_mfma(int kind, int iters, int blocks, float* out_dev, void* stream) {
  const char* fn = "tq_peak_mfma";
  if (!out_dev || kind < 0 || kind > 3 || iters < 1 || blocks < 1) return fail(TQ_EINVAL, "%s: bad arguments", fn);
  return check_launch(tq::launch_peak_mfma(kind, iters, blocks, out_dev, as_stream(stream)), fn);
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

tq_status tq_host_splitmix64(uint64_t seed, uint64_t offset, int64_t n, uint64_t* out_host) {
  if (n < 0 || (n > 0 && !out_host)) return fail(TQ_EINVAL, "tq_host_splitmix64: bad arguments");
  for (int64_t i = 0; i < n; ++i) out_host[i] = draw(seed, offset + (uint64_t)i);
  return ok();
}

tq_status tq_host_gaussian(uint64_t seed, int64_t n, double* out_host) {
  if (n < 0 || (n > 0 && !out_host)) return fail(TQ_EINVAL, "tq_host_gaussian: bad arguments");
  gaussian_fill(seed, n, out_host);
  return ok();
}

tq_status tq_host_codebook(int d, int b, tq_density dens, double* c_host, double* t_host) {
  if (d < 2 || b < 1 || b > tq::kMaxBits || !c_host || !t_host ||
      (dens != TQ_DENSITY_BETA && dens != TQ_DENSITY_GAUSS))
    return fail(TQ_EINVAL, "tq_host_codebook: need d >= 2, 1 <= b <= 4, valid density, outputs");
  lloyd_codebook(d, b, dens, c_host, t_host);
  return ok();
}

tq_status tq_host_rotation(int d, uint64_t seed, tq_rot_kind kind, double* r_host) {
  if (d < 2 || !r_host) return fail(TQ_EINVAL, "tq_host_rotation: need d >= 2 and an output");
  if (kind == TQ_ROT_WHT) {
    if (!is_pow2(d)) return fail(TQ_EUNSUPPORTED, "tq_host_rotation: Hadamard needs d = 2^k (d=%d)", d);
    hadamard_rotation(d, seed, r_host);
    return ok();
  }
  if (kind == TQ_ROT_BLOCK_WHT) {
    if (d % kBlockWhtGroup != 0)
      return fail(TQ_EUNSUPPORTED, "tq_host_rotation: block Hadamard needs d a multiple of %d (d=%d)", kBlockWhtGroup, d);
    block_hadamard_rotation(d, kBlockWhtGroup, seed, r_host);
    return ok();
  }
  if (kind != TQ_ROT_DENSE) return fail(TQ_EINVAL, "tq_host_rotation: bad kind");
  std::vector<double> g((size_t)d * d);
  gaussian_fill(seed, (int64_t)d * d, g.data());
  qr_rotation(d, g.data(), r_host);
  return ok();
}

tq_status tq_host_qjl_matrix(int d, uint64_t seed, double* s_host) {
  if (d < 2 || !s_host) return fail(TQ_EINVAL, "tq_host_qjl_matrix: need d >= 2 and an output");
  gaussian_fill(seed, (int64_t)d * d, s_host);
  return ok();
}

tq_status tq_codebook(int d, int b, tq_density dens, tq_codebook_t* out) {
  if (!out) return fail(TQ_EINVAL, "tq_codebook: null output");
  auto* cb = new (std::nothrow) tq_codebook_s();
  if (!cb) return fail(TQ_ENOMEM, "host allocation failed");
  tq_status st = tq_host_codebook(d, b, dens, cb->c, cb->t);
  if (st != TQ_OK) {
    delete cb;
    return st;
  }
  cb->d = d;
  cb->b = b;
  fill_args(cb);
  *out = cb;
  return ok();
}

tq_status tq_codebook_from_values(int d, int b, const double* c_host, tq_codebook_t* out) {
  if (!out || !c_host || b < 1 || b > tq::kMaxBits || d < 1)
    return fail(TQ_EINVAL, "tq_codebook_from_values: bad arguments");
  const int k = 1 << b;
  for (int i = 0; i + 1 < k; ++i)
    if (!(c_host[i] < c_host[i + 1])) return fail(TQ_EINVAL, "centroids must be strictly increasing");
  auto* cb = new (std::nothrow) tq_codebook_s();
  if (!cb) return fail(TQ_ENOMEM, "host allocation failed");
  cb->d = d;
  cb->b = b;
  for (int i = 0; i < k; ++i) cb->c[i] = c_host[i];
  for (int i = 0; i + 1 < k; ++i) cb->t[i] = 0.5 * (c_host[i] + c_host[i + 1]);
  fill_args(cb);
  *out = cb;
  return ok();
}

tq_status tq_codebook_values(tq_codebook_t cb, double* c_host, double* t_host) {
  if (!cb || !c_host || !t_host) return fail(TQ_EINVAL, "tq_codebook_values: bad arguments");
  const int k = 1 << cb->b;
  for (int i = 0; i < k; ++i) c_host[i] = cb->c[i];
  for (int i = 0; i + 1 < k; ++i) t_host[i] = cb->t[i];
  return ok();
}

void tq_codebook_free(tq_codebook_t cb) { delete cb; }

tq_status tq_make_rotation(int d, uint64_t seed, tq_rot_kind kind, tq_rotation_t* out) {
  if (!out) return fail(TQ_EINVAL, "tq_make_rotation: null output");
  if (d < 2 || d > 8192) return fail(TQ_EUNSUPPORTED, "tq_make_rotation: d=%d out of range", d);
  auto* r = new (std::nothrow) tq_rotation_s();
  if (!r) return fail(TQ_ENOMEM, "host allocation failed");
  r->d = d;
  r->kind = kind;
  r->id = g_next_id++;
  hipGetDevice(&r->device);
  r->r.resize((size_t)d * d);
  tq_status st = tq_host_rotation(d, seed, kind, r->r.data());
  if (st == TQ_OK) st = finish_rotation(r);
  if (st != TQ_OK) {
    free_rotation(r);
    return st;
  }
  *out = r;
  return ok();
}

tq_status tq_rotation_from_matrix(int d, const double* r_host, tq_rotation_t* out) {
  if (!out || !r_host || d < 1) return fail(TQ_EINVAL, "tq_rotation_from_matrix: bad arguments");
  auto* r = new (std::nothrow) tq_rotation_s();
  if (!r) return fail(TQ_ENOMEM, "host allocation failed");
  r->d = d;
  r->kind = TQ_ROT_DENSE;
  r->id = g_next_id++;
  hipGetDevice(&r->device);
  r->r.assign(r_host, r_host + (size_t)d * d);
  tq_status st = finish_rotation(r);
  if (st != TQ_OK) {
    free_rotation(r);
    return st;
  }
  *out = r;
  return ok();
}

tq_status tq_rotation_export(tq_rotation_t rot, double* r_host) {
  if (!rot || !r_host) return fail(TQ_EINVAL, "tq_rotation_export: bad arguments");
  std::memcpy(r_host, rot->r.data(), rot->r.size() * sizeof(double));
  return ok();
}

void tq_rotation_free(tq_rotation_t rot) { free_rotation(rot); }

tq_status tq_make_qjl(int d, uint64_t seed, tq_rotation_t rot, tq_qjl_t* out) {
  if (!out || !rot) return fail(TQ_EINVAL, "tq_make_qjl: bad arguments");
  if (rot->d != d) return fail(TQ_ESHAPE, "tq_make_qjl: d=%d but rotation has d=%d", d, rot->d);
  std::vector<double> s((size_t)d * d);
  gaussian_fill(seed, (int64_t)d * d, s.data());
  return make_qjl(d, std::move(s), rot, out);
}

tq_status tq_qjl_from_matrix(int d, const double* s_host, tq_rotation_t rot, tq_qjl_t* out) {
  if (!out || !rot || !s_host) return fail(TQ_EINVAL, "tq_qjl_from_matrix: bad arguments");
  if (rot->d != d) return fail(TQ_ESHAPE, "tq_qjl_from_matrix: d=%d but rotation has d=%d", d, rot->d);
  std::vector<double> s(s_host, s_host + (size_t)d * d);
  return make_qjl(d, std::move(s), rot, out);
}

void tq_qjl_free(tq_qjl_t qjl) { free_qjl(qjl); }

size_t tq_packed_words(int d, int bits) {
  if (d <= 0 || bits <= 0 || ((int64_t)d * bits) % 32 != 0) return 0;
  return (size_t)d * bits / 32;
}

size_t tq_packed_idx_words(int64_t n, int d, int bits, tq_layout layout) {
  if (n < 0 || d <= 0 || bits <= 0 || ((int64_t)d * bits) % 32 != 0) return 0;
  if (layout == TQ_LAYOUT_ROWS) return (size_t)n * d * bits / 32;
  if (layout == TQ_LAYOUT_TOKEN_BLOCKED) return (size_t)((n + 31) / 32) * d * bits;
  return 0;
}

static tq_status check_packed(const tq_packed* p, int d, int bits, int mode, const char* fn) {
  if (!p) return fail(TQ_EINVAL, "%s: null packed descriptor", fn);
  if (p->d != d) return fail(TQ_ESHAPE, "%s: packed d=%d, expected %d", fn, p->d, d);
  if (p->bits != bits) return fail(TQ_ESHAPE, "%s: packed bits=%d, codebook has %d", fn, p->bits, bits);
  if (p->mode != mode) return fail(TQ_EINVAL, "%s: packed mode mismatch", fn);
  if (p->layout != TQ_LAYOUT_ROWS && p->layout != TQ_LAYOUT_TOKEN_BLOCKED)
    return fail(TQ_EINVAL, "%s: bad layout", fn);
  if (p->layout == TQ_LAYOUT_TOKEN_BLOCKED && mode != TQ_MODE_MSE)
    return fail(TQ_EUNSUPPORTED, "%s: the token-blocked layout holds MSE data only", fn);
  if (p->n < 0) return fail(TQ_EINVAL, "%s: negative n", fn);
  if (p->n > 0 && (!p->idx || !p->norms)) return fail(TQ_EINVAL, "%s: null idx/norms", fn);
  if (mode == TQ_MODE_PROD && p->n > 0 && (!p->qjl || !p->rnorms))
    return fail(TQ_EINVAL, "%s: prod needs qjl and rnorms buffers", fn);
  return TQ_OK;
}

tq_status tq_encode(const void* x_dev, tq_dtype dt, int64_t n, int d, int b, tq_mode mode,
                    tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, tq_packed* out, void* ws_dev,
                    size_t ws_bytes, void* stream) {
  static const char* fn = "tq_encode";
  if (!cb || !rot || !out) return fail(TQ_EINVAL, "%s: null handle or output", fn);
  if (n < 0) return fail(TQ_EINVAL, "%s: negative n", fn);
  if (n > 0 && !x_dev) return fail(TQ_EINVAL, "%s: null input", fn);
  if (dt != TQ_F32 && dt != TQ_BF16) return fail(TQ_EUNSUPPORTED, "%s: dtype must be f32 or bf16", fn);
  if (mode != TQ_MODE_MSE && mode != TQ_MODE_PROD) return fail(TQ_EINVAL, "%s: bad mode", fn);
  const int stage = mode == TQ_MODE_PROD ? b - 1 : b;
  if (stage < 1 || stage > tq::kMaxBits) return fail(TQ_EINVAL, "%s: bits b=%d invalid for this mode", fn, b);
  if (cb->b != stage) return fail(TQ_ESHAPE, "%s: codebook has %d bits, mode needs %d", fn, cb->b, stage);
  if (cb->d != d || rot->d != d) return fail(TQ_ESHAPE, "%s: d=%d, codebook d=%d, rotation d=%d", fn, d, cb->d, rot->d);
  if (((int64_t)d * stage) % 32 != 0) return fail(TQ_ESHAPE, "%s: d*bits must be a multiple of 32", fn);
  if (mode == TQ_MODE_PROD) {
    if (!qjl) return fail(TQ_EINVAL, "%s: prod mode needs a qjl handle", fn);
    if (qjl->d != d) return fail(TQ_ESHAPE, "%s: qjl d=%d", fn, qjl->d);
    if (qjl->rot_id != rot->id) return fail(TQ_EINVAL, "%s: qjl handle is bound to another rotation", fn);
  } else if (qjl) {
    return fail(TQ_EINVAL, "%s: qjl handle given for MSE mode", fn);
  }
  if (d != tq::kFragD && d != 64 && !general_d(d))
    return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d = 64, 128, or a multiple of 128 in [256, 4096])", fn, d);
  if (!cb->args.sym) return fail(TQ_EUNSUPPORTED, "%s: the encode kernels need an antisymmetric codebook", fn);
  tq_status st = check_packed(out, d, stage, mode, fn);
  if (st != TQ_OK) return st;
  if (out->n != n) return fail(TQ_ESHAPE, "%s: out->n=%lld, n=%lld", fn, (long long)out->n, (long long)n);
  if (d != tq::kFragD && out->layout != TQ_LAYOUT_ROWS)
    return fail(TQ_EUNSUPPORTED, "%s: the token-blocked layout needs d = 128", fn);
  if (general_d(d) && mode == TQ_MODE_PROD && n > 0) {
    const size_t per = tq::encode_general_ws_per_vector(d);
    if (!ws_dev) return fail(TQ_EINVAL, "%s: prod at d=%d needs a workspace", fn, d);
    if (ws_bytes < per * (size_t)std::min<int64_t>(n, tq::kGenVectors))
      return fail(TQ_ENOMEM, "%s: workspace of %zu bytes holds fewer than %d vectors (%zu bytes each)", fn,
                  ws_bytes, tq::kGenVectors, per);
  }
  if (n == 0) return ok();
  const bool prod = mode == TQ_MODE_PROD;
  if (d == 64 && !prod)
    return check_launch(tq::launch_encode_mse_d64(x_dev, dt == TQ_BF16, n, rot, cb->args, out->idx, out->norms,
                                                  as_stream(stream)),
                        fn);
  if (d == 64 && qjl->sp32_dev && cb->args.bits <= 3)
    return check_launch(tq::launch_encode_prod_d64(x_dev, dt == TQ_BF16, n, rot, qjl, cb->args, out->idx,
                                                   out->norms, out->qjl, out->rnorms, as_stream(stream)),
                        fn);
  if (d == 64)
    return check_launch(tq::launch_encode_d64(x_dev, dt == TQ_BF16, n, rot, prod ? qjl : nullptr, cb->args, out->idx,
                                              out->norms, prod ? out->qjl : nullptr, prod ? out->rnorms : nullptr,
                                              as_stream(stream)),
                        fn);
  if (d != tq::kFragD)
    return check_launch(tq::launch_encode_general(x_dev, dt == TQ_BF16, n, d, rot, prod ? qjl : nullptr, cb->args,
                                                  out->idx, out->norms, prod ? out->qjl : nullptr,
                                                  prod ? out->rnorms : nullptr, nullptr, ws_dev, ws_bytes,
                                                  as_stream(stream)),
                        fn);
  if (out->layout == TQ_LAYOUT_TOKEN_BLOCKED)
    return check_launch(tq::launch_encode_vblock_d128(x_dev, dt == TQ_BF16, n, rot, cb->args, out->idx,
                                                      out->norms, as_stream(stream)),
                        fn);
  if (!prod && (rot->kind == TQ_ROT_WHT || rot->kind == TQ_ROT_BLOCK_WHT) && cb->args.sym) {
    // randomized Hadamard: the butterfly transform in registers.  R = H_g-blocks diag(sigma) / sqrt(g)
    // and the first row of each Hadamard block is all ones, so sigma_j is the sign of R's entry in
    // the first row of j's block.
    const bool full = rot->kind == TQ_ROT_WHT;
    const int g = full ? tq::kFragD : kBlockWhtGroup;
    uint32_t sigma[4] = {0, 0, 0, 0};
    for (int j = 0; j < tq::kFragD; ++j)
      if (rot->r[(size_t)(j / g * g) * tq::kFragD + j] < 0.0) sigma[j >> 5] |= 1u << (j & 31);
    return check_launch(tq::launch_encode_fwht_d128(x_dev, dt == TQ_BF16, n, full, sigma, (float)std::sqrt((double)g),
                                                    cb->args, out->idx, out->norms, as_stream(stream)),
                        fn);
  }
  if (!prod && rot->frag32_dev)
    return check_launch(tq::launch_encode_mse32_d128(x_dev, dt == TQ_BF16, n, rot, cb->args, out->idx, out->norms,
                                                     as_stream(stream)),
                        fn);
  return check_launch(tq::launch_encode_d128(x_dev, dt == TQ_BF16, n, rot, prod ? qjl : nullptr, cb->args,
                                             out->idx, out->norms, prod ? out->qjl : nullptr,
                                             prod ? out->rnorms : nullptr, nullptr, as_stream(stream)),
                      fn);
}

size_t tq_encode_workspace(int64_t n, int d, int b, tq_mode mode) {
  (void)b;
  if (n <= 0 || mode != TQ_MODE_PROD || d == tq::kFragD || !general_d(d)) return 0;
  return tq::encode_general_ws_per_vector(d) * (size_t)std::min<int64_t>(n, tq::kEncodeChunk);
}

tq_status tq_rotate(const void* x_dev, tq_dtype dt, int64_t n, int d, tq_rotation_t rot,
                    float* y_dev, float* norms_dev, void* stream) {
  static const char* fn = "tq_rotate";
  if (!rot) return fail(TQ_EINVAL, "%s: null rotation", fn);
  if (n < 0) return fail(TQ_EINVAL, "%s: negative n", fn);
  if (n > 0 && (!x_dev || !y_dev || !norms_dev)) return fail(TQ_EINVAL, "%s: null buffer", fn);
  if (dt != TQ_F32 && dt != TQ_BF16) return fail(TQ_EUNSUPPORTED, "%s: dtype must be f32 or bf16", fn);
  if (rot->d != d) return fail(TQ_ESHAPE, "%s: rotation d=%d, d=%d", fn, rot->d, d);
  if (d != tq::kFragD && !general_d(d)) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported", fn, d);
  if (n == 0) return ok();
  tq::CodebookArgs none{};
  none.bits = 1;
  if (d != tq::kFragD)
    return check_launch(tq::launch_encode_general(x_dev, dt == TQ_BF16, n, d, rot, nullptr, none, nullptr,
                                                  norms_dev, nullptr, nullptr, y_dev, nullptr, 0,
                                                  as_stream(stream)),
                        fn);
  return check_launch(tq::launch_encode_d128(x_dev, dt == TQ_BF16, n, rot, nullptr, none, nullptr, norms_dev,
                                             nullptr, nullptr, y_dev, as_stream(stream)),
                      fn);
}

tq_status tq_quantize_rotated(const float* y_dev, int64_t n, int d, tq_codebook_t cb,
                              uint32_t* idx_dev, void* stream) {
  static const char* fn = "tq_quantize_rotated";
  if (!cb) return fail(TQ_EINVAL, "%s: null codebook", fn);
  if (n < 0) return fail(TQ_EINVAL, "%s: negative n", fn);
  if (n > 0 && (!y_dev || !idx_dev)) return fail(TQ_EINVAL, "%s: null buffer", fn);
  if (cb->d != d) return fail(TQ_ESHAPE, "%s: codebook d=%d, d=%d", fn, cb->d, d);
  if (d % 32 != 0) return fail(TQ_ESHAPE, "%s: d must be a multiple of 32", fn);
  if (n == 0) return ok();
  return check_launch(tq::launch_quantize_rotated(y_dev, n, d, cb->args, idx_dev, as_stream(stream)), fn);
}

tq_status tq_decode(const tq_packed* p, tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl,
                    float* xhat_dev, void* stream) {
  static const char* fn = "tq_decode";
  if (!p || !cb || !rot) return fail(TQ_EINVAL, "%s: null argument", fn);
  tq_status st = check_packed(p, rot->d, cb->b, p->mode, fn);
  if (st != TQ_OK) return st;
  if (p->mode != TQ_MODE_MSE && p->mode != TQ_MODE_PROD) return fail(TQ_EINVAL, "%s: bad mode", fn);
  if (cb->d != p->d) return fail(TQ_ESHAPE, "%s: codebook d=%d, packed d=%d", fn, cb->d, p->d);
  if (((int64_t)p->d * p->bits) % 32 != 0 || p->d % 32 != 0) return fail(TQ_ESHAPE, "%s: d*bits must be a multiple of 32", fn);
  if (qjl) {
    if (p->mode != TQ_MODE_PROD) return fail(TQ_EINVAL, "%s: qjl given for MSE data", fn);
    if (qjl->d != p->d) return fail(TQ_ESHAPE, "%s: qjl d=%d", fn, qjl->d);
  }
  if (p->n > 0 && !xhat_dev) return fail(TQ_EINVAL, "%s: null output", fn);
  if (p->n == 0) return ok();
  return check_launch(tq::launch_decode(p, cb->args, rot, qjl, xhat_dev, as_stream(stream)), fn);
}

// Head dims with the KV-side kernels of csrc/tq_kvgen.hip (d = 128 has its own).
static bool kv_generic_d(int d) { return d == 64 || d == 256; }

size_t tq_scores_workspace(int B, int Hq, int d) {
  if (B < 0 || Hq < 0 || d <= 0) return 0;
  return kv_generic_d(d) ? tq::kv_gen_query_bytes(B, Hq, d) : tq::scores_workspace_bytes(B, Hq, d);
}

// Shape rules shared by the score entry points.
static tq_status check_score_heads(int B, int Hq, int Hkv, const char* fn) {
  if (B < 0 || Hq < 0 || Hkv < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return fail(TQ_ESHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  const int ratio = Hq / Hkv;
  if (ratio > 4 && ratio % 4 != 0) return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d must be <= 4 or a multiple of 4", fn, ratio);
  if (ratio > 64) return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d above 64", fn, ratio);
  if ((int64_t)B * Hkv > 65535) return fail(TQ_EUNSUPPORTED, "%s: B*Hkv=%lld above 65535", fn, (long long)B * Hkv);
  return TQ_OK;
}

// Longest sequence the score and attention kernels take: their per-tile token offsets are
// 32-bit (at most 64 bytes of packed words per token).
constexpr int64_t kMaxSeqTokens = int64_t(1) << 25;

// rows: rows per sequence in K (T for a packed [B, Hkv, T] set, the capacity for a cache).
static tq_status check_score_keys(int B, int Hkv, int64_t T, int64_t rows, const tq_packed* K, tq_codebook_t cb,
                                  int d, const char* fn) {
  if (T < 0) return fail(TQ_EINVAL, "%s: negative T", fn);
  if (rows < T) return fail(TQ_EINVAL, "%s: T=%lld exceeds the capacity %lld", fn, (long long)T, (long long)rows);
  if (T > kMaxSeqTokens)
    return fail(TQ_EUNSUPPORTED, "%s: T=%lld exceeds %lld tokens per sequence", fn, (long long)T,
                (long long)kMaxSeqTokens);
  tq_status st = check_packed(K, d, cb->b, K->mode, fn);
  if (st != TQ_OK) return st;
  if (K->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: keys must use the ROWS layout", fn);
  if (cb->d != d) return fail(TQ_ESHAPE, "%s: codebook d=%d, keys d=%d", fn, cb->d, d);
  if (K->n != (int64_t)B * Hkv * rows)
    return fail(TQ_ESHAPE, "%s: K->n=%lld but B*Hkv*%lld=%lld", fn, (long long)K->n, (long long)rows,
                (long long)B * Hkv * rows);
  if (K->mode != TQ_MODE_PROD && K->mode != TQ_MODE_MSE) return fail(TQ_EINVAL, "%s: bad mode", fn);
  if (d != tq::kFragD && !kv_generic_d(d)) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (64, 128, 256)", fn, d);
  return TQ_OK;
}

tq_status tq_prepare_queries(const float* q_dev, int B, int Hq, int Hkv, tq_rotation_t rot, tq_qjl_t qjl,
                             void* ws_dev, size_t ws_bytes, void* stream) {
  static const char* fn = "tq_prepare_queries";
  if (!rot) return fail(TQ_EINVAL, "%s: null rotation", fn);
  tq_status st = check_score_heads(B, Hq, Hkv, fn);
  if (st != TQ_OK) return st;
  const int d = rot->d;
  if (d != tq::kFragD) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d=128)", fn, d);
  if (qjl && qjl->d != d) return fail(TQ_ESHAPE, "%s: qjl d=%d", fn, qjl->d);
  if ((int64_t)B * Hq == 0) return ok();
  if (!q_dev) return fail(TQ_EINVAL, "%s: null q", fn);
  const size_t need = tq::scores_workspace_bytes(B, Hq, d);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  return check_launch(tq::launch_prepare_queries(q_dev, B, Hq, Hkv, rot, qjl, ws_dev, as_stream(stream)), fn);
}

tq_status tq_scores_prepared(const void* ws_dev, size_t ws_bytes, int B, int Hq, int Hkv, int64_t T,
                             const tq_packed* K, tq_codebook_t cb, float* scores_dev, void* stream) {
  static const char* fn = "tq_scores_prepared";
  if (!K || !cb) return fail(TQ_EINVAL, "%s: null argument", fn);
  tq_status st = check_score_heads(B, Hq, Hkv, fn);
  if (st != TQ_OK) return st;
  st = check_score_keys(B, Hkv, T, T, K, cb, K->d, fn);
  if (st != TQ_OK) return st;
  if (K->d != tq::kFragD) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d=128)", fn, K->d);
  if ((int64_t)(Hq / Hkv) * T >= (int64_t(1) << 30))
    return fail(TQ_EUNSUPPORTED, "%s: (Hq/Hkv)*T=%lld: a kv head's score rows must stay below 4 GB", fn,
                (long long)(Hq / Hkv) * T);
  if ((int64_t)B * Hq * T == 0) return ok();
  if (!scores_dev) return fail(TQ_EINVAL, "%s: null scores", fn);
  const size_t need = tq::scores_workspace_bytes(B, Hq, K->d);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  return check_launch(tq::launch_scores_prepared(B, Hq, Hkv, T, K, cb->args, scores_dev, ws_dev, as_stream(stream)),
                      fn);
}

// use_scratch: the workspace is the library's static scratch (ws_dev / ws_bytes ignored).
static tq_status scores_impl(const char* fn, const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t rows,
                             const tq_packed* K, tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, float* scores_dev,
                             void* ws_dev, size_t ws_bytes, void* stream, bool use_scratch = false) {
  if (!K || !cb || !rot) return fail(TQ_EINVAL, "%s: null argument", fn);
  tq_status st = check_score_heads(B, Hq, Hkv, fn);
  if (st != TQ_OK) return st;
  const int d = rot->d;
  st = check_score_keys(B, Hkv, T, rows, K, cb, d, fn);
  if (st != TQ_OK) return st;
  if (rows > kMaxSeqTokens)
    return fail(TQ_EUNSUPPORTED, "%s: capacity %lld exceeds %lld tokens per sequence", fn, (long long)rows,
                (long long)kMaxSeqTokens);
  if ((int64_t)(Hq / Hkv) * T >= (int64_t(1) << 30))
    return fail(TQ_EUNSUPPORTED, "%s: (Hq/Hkv)*T=%lld: a kv head's score rows must stay below 4 GB", fn,
                (long long)(Hq / Hkv) * T);
  if (K->mode == TQ_MODE_PROD) {
    if (!qjl) return fail(TQ_EINVAL, "%s: prod keys need the qjl handle", fn);
    if (qjl->d != d) return fail(TQ_ESHAPE, "%s: qjl d=%d", fn, qjl->d);
  } else if (qjl) {
    return fail(TQ_EINVAL, "%s: qjl handle given for MSE keys", fn);
  }
  if ((int64_t)B * Hq * T == 0) return ok();
  if (!q_dev || !scores_dev) return fail(TQ_EINVAL, "%s: null q or scores", fn);
  const bool gen = d != tq::kFragD;
  size_t need = gen ? tq::kv_gen_query_bytes(B, Hq, d) : tq::scores_workspace_bytes(B, Hq, d);
  if (use_scratch && gen) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d=128)", fn, d);
  if (use_scratch) {
    if (need > tq::noalloc_scratch_bytes())
      return fail(TQ_ENOMEM, "%s: B*Hq=%lld query heads need %zu bytes of scratch, above the static %zu bytes",
                  fn, (long long)B * Hq, need, tq::noalloc_scratch_bytes());
    hipError_t se = tq::noalloc_scratch(&ws_dev);
    if (se != hipSuccess) return hip_fail(se, fn);
    ws_bytes = tq::noalloc_scratch_bytes();
  }
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  hipStream_t hs = as_stream(stream);
  if (gen)
    return check_launch(tq::launch_scores_gen(q_dev, B, Hq, Hkv, T, rows, K, cb->args, rot,
                                              K->mode == TQ_MODE_PROD ? qjl : nullptr, scores_dev, ws_dev, hs),
                        fn);
  hipError_t e = tq::launch_prepare_queries(q_dev, B, Hq, Hkv, rot, K->mode == TQ_MODE_PROD ? qjl : nullptr, ws_dev, hs);
  if (e == hipSuccess) e = tq::launch_scores_strided(B, Hq, Hkv, T, rows, K, cb->args, scores_dev, ws_dev, hs);
  return check_launch(e, fn);
}

tq_status tq_scores(const float* q_dev, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                    tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, float* scores_dev,
                    void* ws_dev, size_t ws_bytes, void* stream) {
  return scores_impl("tq_scores", q_dev, B, Hq, Hkv, T, T, K, cb, rot, qjl, scores_dev, ws_dev, ws_bytes, stream);
}

tq_status tq_scores_noalloc(const float* q_dev, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                            tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, float* scores_dev, void* stream) {
  return scores_impl("tq_scores_noalloc", q_dev, B, Hq, Hkv, T, T, K, cb, rot, qjl, scores_dev, nullptr, 0, stream,
                     true);
}

size_t tq_scores_noalloc_max_bytes(void) { return tq::noalloc_scratch_bytes(); }

tq_status tq_scores_cache(const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t T_cap, const tq_packed* K,
                          tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, float* scores_dev, void* ws_dev,
                          size_t ws_bytes, void* stream) {
  return scores_impl("tq_scores_cache", q_dev, B, Hq, Hkv, T, T_cap, K, cb, rot, qjl, scores_dev, ws_dev, ws_bytes,
                     stream);
}

size_t tq_decode_attn_workspace(int B, int Hq, int Hkv, int64_t T, int d) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || T < 0 || d <= 0) return 0;
  return kv_generic_d(d) ? tq::attn_gen_workspace_bytes(B, Hq, Hkv, T, d)
                         : tq::decode_attn_workspace_bytes(B, Hq, Hkv, T, d);
}

// rows: rows per sequence in K and V (T for packed [B, Hkv, T] sets, the capacity for a cache,
// which must then be a multiple of 32 so that every sequence owns whole value blocks).
static tq_status decode_attn_impl(const char* fn, const float* q_dev, int B, int Hq, int Hkv, int64_t T,
                                  int64_t rows, bool cache, const tq_packed* K, const tq_packed* V,
                                  tq_codebook_t cb_k, tq_codebook_t cb_v, tq_rotation_t rot_k, tq_rotation_t rot_v,
                                  float scale, float* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!K || !V || !cb_k || !cb_v || !rot_k || !rot_v) return fail(TQ_EINVAL, "%s: null argument", fn);
  if (B < 0 || Hq < 0 || Hkv < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (T < 1) return fail(TQ_EINVAL, "%s: attention over an empty cache (T=%lld)", fn, (long long)T);
  if (T > rows) return fail(TQ_EINVAL, "%s: T=%lld exceeds the capacity %lld", fn, (long long)T, (long long)rows);
  if (cache && rows % 32 != 0)
    return fail(TQ_ESHAPE, "%s: capacity %lld is not a multiple of 32 (value blocks)", fn, (long long)rows);
  if (rows > kMaxSeqTokens)
    return fail(TQ_EUNSUPPORTED, "%s: %lld tokens per sequence exceed %lld", fn, (long long)rows,
                (long long)kMaxSeqTokens);
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return fail(TQ_ESHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  const int ratio = Hq / Hkv;
  const int d = rot_k->d;
  const bool gen = kv_generic_d(d);
  if (gen ? ratio > 8 : (ratio != 1 && ratio != 2 && ratio != 4))
    return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d not supported at d=%d (%s)", fn, ratio, d,
                gen ? "at most 8" : "1, 2 or 4");
  if (rot_v->d != d || cb_k->d != d || cb_v->d != d) return fail(TQ_ESHAPE, "%s: d mismatch between handles", fn);
  tq_status st = check_packed(K, d, cb_k->b, TQ_MODE_MSE, fn);
  if (st != TQ_OK) return st;
  st = check_packed(V, d, cb_v->b, TQ_MODE_MSE, fn);
  if (st != TQ_OK) return st;
  if (K->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: K must use the ROWS layout", fn);
  if (!gen && V->layout != TQ_LAYOUT_TOKEN_BLOCKED)
    return fail(TQ_EUNSUPPORTED, "%s: V must use the TOKEN_BLOCKED layout at d=128", fn);
  if (gen && V->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: V must use the ROWS layout at d=%d", fn, d);
  const int64_t n = (int64_t)B * Hkv * rows;
  if (K->n != n || V->n != n)
    return fail(TQ_ESHAPE, "%s: K->n=%lld, V->n=%lld, B*Hkv*%lld=%lld", fn, (long long)K->n, (long long)V->n,
                (long long)rows, (long long)n);
  if (d != tq::kFragD && !gen) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (64, 128, 256)", fn, d);
  if ((int64_t)B * Hkv > 65535) return fail(TQ_EUNSUPPORTED, "%s: B*Hkv above 65535", fn);
  if ((int64_t)B * Hq == 0) return ok();
  if (!q_dev || !out_dev) return fail(TQ_EINVAL, "%s: null q or out", fn);
  size_t need = gen ? tq::attn_gen_workspace_bytes(B, Hq, Hkv, T, d) : tq::decode_attn_workspace_bytes(B, Hq, Hkv, T, d);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (gen)
    return check_launch(tq::launch_decode_attn_gen(q_dev, B, Hq, Hkv, T, rows, K, V, cb_k->args, cb_v->args, rot_k,
                                                   rot_v, scale, out_dev, ws_dev, as_stream(stream)),
                        fn);
  return check_launch(tq::launch_decode_attn_strided(q_dev, B, Hq, Hkv, T, rows, K, V, cb_k->args, cb_v->args, rot_k,
                                                     rot_v, scale, out_dev, ws_dev, as_stream(stream)),
                      fn);
}

tq_status tq_decode_attn(const float* q_dev, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                         const tq_packed* V, tq_codebook_t cb_k, tq_codebook_t cb_v,
                         tq_rotation_t rot_k, tq_rotation_t rot_v, float scale, float* out_dev,
                         void* ws_dev, size_t ws_bytes, void* stream) {
  return decode_attn_impl("tq_decode_attn", q_dev, B, Hq, Hkv, T, T, false, K, V, cb_k, cb_v, rot_k, rot_v, scale,
                          out_dev, ws_dev, ws_bytes, stream);
}

tq_status tq_decode_attn_cache(const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t T_cap,
                               const tq_packed* K, const tq_packed* V, tq_codebook_t cb_k, tq_codebook_t cb_v,
                               tq_rotation_t rot_k, tq_rotation_t rot_v, float scale, float* out_dev, void* ws_dev,
                               size_t ws_bytes, void* stream) {
  return decode_attn_impl("tq_decode_attn_cache", q_dev, B, Hq, Hkv, T, T_cap, true, K, V, cb_k, cb_v, rot_k, rot_v,
                          scale, out_dev, ws_dev, ws_bytes, stream);
}

// Argument checks of an append into one cache (shared by tq_cache_append and tq_kv_append).
static tq_status check_cache_append(const char* fn, tq_dtype dt, int B, int H, int64_t n_new, int64_t pos,
                                    int64_t T_cap, int b, tq_mode mode, tq_codebook_t cb, tq_rotation_t rot,
                                    tq_qjl_t qjl, const tq_packed* cache) {
  if (!cb || !rot || !cache) return fail(TQ_EINVAL, "%s: null handle or cache", fn);
  if (B < 0 || H < 0 || n_new < 0 || pos < 0 || T_cap < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (pos > T_cap - n_new)
    return fail(TQ_EINVAL, "%s: %lld tokens at position %lld overflow the capacity %lld", fn, (long long)n_new,
                (long long)pos, (long long)T_cap);
  if (dt != TQ_F32 && dt != TQ_BF16) return fail(TQ_EUNSUPPORTED, "%s: dtype must be f32 or bf16", fn);
  if (mode != TQ_MODE_MSE && mode != TQ_MODE_PROD) return fail(TQ_EINVAL, "%s: bad mode", fn);
  const int stage = mode == TQ_MODE_PROD ? b - 1 : b;
  if (stage < 1 || stage > tq::kMaxBits) return fail(TQ_EINVAL, "%s: bits b=%d invalid for this mode", fn, b);
  if (cb->b != stage) return fail(TQ_ESHAPE, "%s: codebook has %d bits, mode needs %d", fn, cb->b, stage);
  const int d = rot->d;
  if (cb->d != d) return fail(TQ_ESHAPE, "%s: codebook d=%d, rotation d=%d", fn, cb->d, d);
  if (d != tq::kFragD) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d=128)", fn, d);
  if (mode == TQ_MODE_PROD) {
    if (!qjl) return fail(TQ_EINVAL, "%s: prod mode needs a qjl handle", fn);
    if (qjl->d != d) return fail(TQ_ESHAPE, "%s: qjl d=%d", fn, qjl->d);
    if (qjl->rot_id != rot->id) return fail(TQ_EINVAL, "%s: qjl handle is bound to another rotation", fn);
  } else if (qjl) {
    return fail(TQ_EINVAL, "%s: qjl handle given for MSE mode", fn);
  }
  if (!cb->args.sym) return fail(TQ_EUNSUPPORTED, "%s: the encode kernels need an antisymmetric codebook", fn);
  tq_status st = check_packed(cache, d, stage, mode, fn);
  if (st != TQ_OK) return st;
  if (cache->n != (int64_t)B * H * T_cap)
    return fail(TQ_ESHAPE, "%s: cache->n=%lld but B*H*T_cap=%lld", fn, (long long)cache->n, (long long)B * H * T_cap);
  if (cache->layout == TQ_LAYOUT_TOKEN_BLOCKED && T_cap % 32 != 0)
    return fail(TQ_ESHAPE, "%s: a token-blocked cache needs T_cap a multiple of 32 (T_cap=%lld)", fn,
                (long long)T_cap);
  if ((int64_t)B * H > 65535) return fail(TQ_EUNSUPPORTED, "%s: B*H=%lld above 65535", fn, (long long)B * H);
  if (n_new > INT32_MAX) return fail(TQ_EUNSUPPORTED, "%s: n_new above 2^31 - 1", fn);
  return TQ_OK;
}

tq_status tq_cache_append(const void* x_dev, tq_dtype dt, int B, int H, int64_t n_new, int64_t pos, int64_t T_cap,
                          int b, tq_mode mode, tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, tq_packed* cache,
                          void* stream) {
  static const char* fn = "tq_cache_append";
  tq_status st = check_cache_append(fn, dt, B, H, n_new, pos, T_cap, b, mode, cb, rot, qjl, cache);
  if (st != TQ_OK) return st;
  if ((int64_t)B * H * n_new == 0) return ok();
  if (!x_dev) return fail(TQ_EINVAL, "%s: null input", fn);
  return check_launch(tq::launch_cache_append(x_dev, dt == TQ_BF16, (int64_t)B * H, n_new, pos, T_cap, rot,
                                              mode == TQ_MODE_PROD ? qjl : nullptr, cb->args, cache,
                                              as_stream(stream)),
                      fn);
}

tq_status tq_kv_append(const void* k_dev, const void* v_dev, tq_dtype dt, int B, int H, int64_t n_new, int64_t pos,
                       int64_t T_cap, int b_k, int b_v, tq_codebook_t cb_k, tq_codebook_t cb_v, tq_rotation_t rot_k,
                       tq_rotation_t rot_v, tq_packed* K, tq_packed* V, void* stream) {
  static const char* fn = "tq_kv_append";
  tq_status st = check_cache_append(fn, dt, B, H, n_new, pos, T_cap, b_k, TQ_MODE_MSE, cb_k, rot_k, nullptr, K);
  if (st != TQ_OK) return st;
  st = check_cache_append(fn, dt, B, H, n_new, pos, T_cap, b_v, TQ_MODE_MSE, cb_v, rot_v, nullptr, V);
  if (st != TQ_OK) return st;
  if (K->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: the key cache must use the ROWS layout", fn);
  if (V->layout != TQ_LAYOUT_TOKEN_BLOCKED)
    return fail(TQ_EUNSUPPORTED, "%s: the value cache must use the TOKEN_BLOCKED layout", fn);
  if ((int64_t)B * H * n_new == 0) return ok();
  if (!k_dev || !v_dev) return fail(TQ_EINVAL, "%s: null input", fn);
  return check_launch(tq::launch_kv_append(k_dev, v_dev, dt == TQ_BF16, (int64_t)B * H, n_new, pos, T_cap, rot_k,
                                           rot_v, cb_k->args, cb_v->args, K, V, as_stream(stream)),
                      fn);
}

size_t tq_prefill_attn_workspace(int B, int Hq, int64_t n_new, int d) {
  if (B < 0 || Hq < 0 || n_new < 0 || d != tq::kFragD) return 0;
  return tq::prefill_attn_workspace_bytes(B, Hq, n_new);
}

tq_status tq_prefill_attn(const float* q_dev, const void* k_dev, const void* v_dev, tq_dtype dt, int B, int Hq,
                          int Hkv, int64_t n_new, int64_t pos, int64_t T_cap, tq_codebook_t cb_k, tq_codebook_t cb_v,
                          tq_rotation_t rot_k, tq_rotation_t rot_v, tq_packed* K, tq_packed* V, float scale,
                          float* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  static const char* fn = "tq_prefill_attn";
  if (!cb_k || !cb_v || !rot_k || !rot_v || !K || !V) return fail(TQ_EINVAL, "%s: null argument", fn);
  if (B < 0 || Hq < 0 || Hkv < 0 || n_new < 0 || pos < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return fail(TQ_ESHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  if (Hq / Hkv > 64) return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d above 64", fn, Hq / Hkv);
  // the append's own checks (bits, layouts, capacity, d, dtype) on both caches
  tq_status st = check_cache_append(fn, dt, B, Hkv, n_new, pos, T_cap, cb_k->b, TQ_MODE_MSE, cb_k, rot_k, nullptr, K);
  if (st != TQ_OK) return st;
  st = check_cache_append(fn, dt, B, Hkv, n_new, pos, T_cap, cb_v->b, TQ_MODE_MSE, cb_v, rot_v, nullptr, V);
  if (st != TQ_OK) return st;
  if (K->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: the key cache must use the ROWS layout", fn);
  if (V->layout != TQ_LAYOUT_TOKEN_BLOCKED)
    return fail(TQ_EUNSUPPORTED, "%s: the value cache must use the TOKEN_BLOCKED layout", fn);
  if (T_cap % 32 != 0) return fail(TQ_ESHAPE, "%s: capacity %lld is not a multiple of 32", fn, (long long)T_cap);
  if (T_cap > kMaxSeqTokens) return fail(TQ_EUNSUPPORTED, "%s: capacity above %lld tokens", fn, (long long)kMaxSeqTokens);
  if ((int64_t)B * Hkv * n_new == 0) return ok();
  if ((int64_t)B * Hq * n_new >= (int64_t(1) << 31))
    return fail(TQ_EUNSUPPORTED, "%s: B*Hq*n_new above 2^31 - 1 query rows", fn);
  if (!q_dev || !k_dev || !v_dev || !out_dev) return fail(TQ_EINVAL, "%s: null q, k, v or out", fn);
  const size_t need = tq::prefill_attn_workspace_bytes(B, Hq, n_new);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  hipStream_t hs = as_stream(stream);
  hipError_t e = tq::launch_kv_append(k_dev, v_dev, dt == TQ_BF16, (int64_t)B * Hkv, n_new, pos, T_cap, rot_k, rot_v,
                                      cb_k->args, cb_v->args, K, V, hs);
  if (e == hipSuccess)
    e = tq::launch_prefill_attn(q_dev, B, Hq, Hkv, n_new, pos, T_cap, K, V, cb_k->args, cb_v->args, rot_k, rot_v, scale,
                                out_dev, ws_dev, hs);
  return check_launch(e, fn);
}

}  // extern "C"

// ---- outlier-channel split codes (d = 128) ------------------------------------------------

struct tq_split_s {
  int H;
  int device;
  std::vector<int32_t> order;     // [H, 128]: outlier channels as listed, then the rest ascending
  int32_t* order_dev = nullptr;
};

tq_status tq_make_split(int H, int d, const int32_t* outliers_host, tq_split_t* out) {
  static const char* fn = "tq_make_split";
  if (!out || !outliers_host || H < 1) return fail(TQ_EINVAL, "%s: bad arguments", fn);
  if (d != tq::kSplitD) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d=128)", fn, d);
  std::vector<int32_t> order((size_t)H * tq::kSplitD);
  for (int h = 0; h < H; ++h) {
    bool seen[tq::kSplitD] = {};
    const int32_t* o = outliers_host + (size_t)h * tq::kSplitHalf;
    for (int i = 0; i < tq::kSplitHalf; ++i) {
      if (o[i] < 0 || o[i] >= tq::kSplitD || seen[o[i]])
        return fail(TQ_EINVAL, "%s: head %d: channel %d repeated or outside [0, 128)", fn, h, (int)o[i]);
      seen[o[i]] = true;
      order[(size_t)h * tq::kSplitD + i] = o[i];
    }
    int k = tq::kSplitHalf;
    for (int c = 0; c < tq::kSplitD; ++c)
      if (!seen[c]) order[(size_t)h * tq::kSplitD + k++] = c;
  }
  auto* sp = new (std::nothrow) tq_split_s();
  if (!sp) return fail(TQ_ENOMEM, "host allocation failed");
  sp->H = H;
  hipGetDevice(&sp->device);
  sp->order = std::move(order);
  tq_status st = upload(sp->order, &sp->order_dev, "upload channel order");
  if (st != TQ_OK) {
    delete sp;
    return st;
  }
  *out = sp;
  return ok();
}

void tq_split_free(tq_split_t sp) {
  if (!sp) return;
  if (sp->order_dev) hipFree(sp->order_dev);
  delete sp;
}

// Handles and both halves' packed sets of split-coded keys: B * H sequences of `rows` rows each
// (rows = T for a packed set, the capacity for a cache).
static tq_status check_split_keys(int B, int H, int64_t rows, tq_split_t sp, tq_codebook_t cb_o, tq_codebook_t cb_r,
                                  tq_rotation_t rot_o, tq_rotation_t rot_r, const tq_packed* K_o,
                                  const tq_packed* K_r, const char* fn) {
  if (!sp || !cb_o || !cb_r || !rot_o || !rot_r || !K_o || !K_r) return fail(TQ_EINVAL, "%s: null argument", fn);
  if (B < 0 || H < 0 || rows < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (sp->H != H) return fail(TQ_ESHAPE, "%s: split has %d heads, keys have %d", fn, sp->H, H);
  if ((int64_t)B * H > 65535) return fail(TQ_EUNSUPPORTED, "%s: B*H=%lld above 65535", fn, (long long)B * H);
  if (rows > kMaxSeqTokens)
    return fail(TQ_EUNSUPPORTED, "%s: %lld rows per sequence above %lld", fn, (long long)rows, (long long)kMaxSeqTokens);
  const int m = tq::kSplitHalf;
  if (cb_o->d != m || cb_r->d != m) return fail(TQ_ESHAPE, "%s: codebooks need d=64", fn);
  if (rot_o->d != m || rot_r->d != m) return fail(TQ_ESHAPE, "%s: rotations need d=64", fn);
  tq_status st = check_packed(K_o, m, cb_o->b, TQ_MODE_MSE, fn);
  if (st == TQ_OK) st = check_packed(K_r, m, cb_r->b, TQ_MODE_MSE, fn);
  if (st != TQ_OK) return st;
  if (K_o->layout != TQ_LAYOUT_ROWS || K_r->layout != TQ_LAYOUT_ROWS)
    return fail(TQ_EUNSUPPORTED, "%s: split codes use the ROWS layout", fn);
  const int64_t n = (int64_t)B * H * rows;
  if (K_o->n != n || K_r->n != n)
    return fail(TQ_ESHAPE, "%s: packed n=%lld/%lld but B*H*%lld=%lld", fn, (long long)K_o->n, (long long)K_r->n,
                (long long)rows, (long long)n);
  return TQ_OK;
}

// Encode of x [B, H, n_new, 128] into rows pos .. pos + n_new - 1 of every sequence of split codes
// with `rows` rows per sequence.
static tq_status encode_split_impl(const char* fn, const void* x_dev, tq_dtype dt, int B, int H, int64_t n_new,
                                   int64_t pos, int64_t rows, tq_split_t split, tq_codebook_t cb_o, tq_codebook_t cb_r,
                                   tq_rotation_t rot_o, tq_rotation_t rot_r, tq_packed* out_o, tq_packed* out_r,
                                   void* stream) {
  tq_status st = check_split_keys(B, H, rows, split, cb_o, cb_r, rot_o, rot_r, out_o, out_r, fn);
  if (st != TQ_OK) return st;
  if (n_new < 0 || pos < 0 || pos + n_new > rows)
    return fail(TQ_EINVAL, "%s: rows %lld .. %lld outside the %lld rows per sequence", fn, (long long)pos,
                (long long)(pos + n_new), (long long)rows);
  if (dt != TQ_BF16 && dt != TQ_F32) return fail(TQ_EUNSUPPORTED, "%s: dtype %d", fn, (int)dt);
  if ((int64_t)B * H * n_new == 0) return ok();
  if (!x_dev) return fail(TQ_EINVAL, "%s: null x", fn);
  if (reinterpret_cast<uintptr_t>(x_dev) % 16 != 0) return fail(TQ_EINVAL, "%s: x must be 16-byte aligned", fn);
  return check_launch(tq::launch_encode_split(x_dev, dt == TQ_BF16, (int64_t)B * H, H, n_new, rows, pos,
                                              split->order_dev, rot_o->r32_dev, rot_r->r32_dev, rot_o->rt32_dev,
                                              rot_r->rt32_dev, cb_o->args, cb_r->args,
                                              out_o->idx, out_o->norms, out_r->idx, out_r->norms, as_stream(stream)),
                      fn);
}

tq_status tq_encode_split(const void* x_dev, tq_dtype dt, int B, int H, int64_t T, tq_split_t split,
                          tq_codebook_t cb_o, tq_codebook_t cb_r, tq_rotation_t rot_o, tq_rotation_t rot_r,
                          tq_packed* out_o, tq_packed* out_r, void* stream) {
  return encode_split_impl("tq_encode_split", x_dev, dt, B, H, T, 0, T, split, cb_o, cb_r, rot_o, rot_r, out_o, out_r,
                           stream);
}

tq_status tq_cache_append_split(const void* x_dev, tq_dtype dt, int B, int H, int64_t n_new, int64_t pos,
                                int64_t T_cap, tq_split_t split, tq_codebook_t cb_o, tq_codebook_t cb_r,
                                tq_rotation_t rot_o, tq_rotation_t rot_r, tq_packed* K_o, tq_packed* K_r,
                                void* stream) {
  return encode_split_impl("tq_cache_append_split", x_dev, dt, B, H, n_new, pos, T_cap, split, cb_o, cb_r, rot_o,
                           rot_r, K_o, K_r, stream);
}

size_t tq_scores_split_workspace(int B, int Hq) {
  if (B < 0 || Hq < 0) return 0;
  return (size_t)B * Hq * tq::kSplitD * sizeof(float);
}

// Scores over the first T rows of every sequence of split codes with `rows` rows per sequence.
static tq_status scores_split_impl(const char* fn, const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t rows,
                                   tq_split_t split, const tq_packed* K_o, const tq_packed* K_r, tq_codebook_t cb_o,
                                   tq_codebook_t cb_r, tq_rotation_t rot_o, tq_rotation_t rot_r, float* scores_dev,
                                   void* ws_dev, size_t ws_bytes, void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || T < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0)
    return fail(TQ_ESHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  if (Hq / Hkv > tq::kSplitMaxRatio)
    return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d above %d", fn, Hq / Hkv, tq::kSplitMaxRatio);
  tq_status st = check_split_keys(B, Hkv, rows, split, cb_o, cb_r, rot_o, rot_r, K_o, K_r, fn);
  if (st != TQ_OK) return st;
  if (T > rows) return fail(TQ_EINVAL, "%s: T=%lld exceeds the %lld rows per sequence", fn, (long long)T, (long long)rows);
  if ((int64_t)Hq * T >= (int64_t(1) << 30))
    return fail(TQ_EUNSUPPORTED, "%s: Hq*T=%lld: a batch's score rows must stay below 4 GB", fn, (long long)Hq * T);
  if ((int64_t)B * Hq * T == 0) return ok();
  if (!q_dev || !scores_dev) return fail(TQ_EINVAL, "%s: null q or scores", fn);
  const size_t need = tq_scores_split_workspace(B, Hq);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  hipStream_t hs = as_stream(stream);
  float* qws = static_cast<float*>(ws_dev);
  hipError_t e = tq::launch_qprep_split(q_dev, B, Hq, Hkv, split->order_dev, rot_o->rt32_dev, rot_r->rt32_dev, qws, hs);
  if (e == hipSuccess)
    e = tq::launch_scores_split(qws, B, Hq, Hkv, T, rows, cb_o->b, cb_r->b, cb_o->args, cb_r->args, K_o->idx,
                                K_o->norms, K_r->idx, K_r->norms, scores_dev, hs);
  return check_launch(e, fn);
}

tq_status tq_scores_split(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_split_t split,
                          const tq_packed* K_o, const tq_packed* K_r, tq_codebook_t cb_o, tq_codebook_t cb_r,
                          tq_rotation_t rot_o, tq_rotation_t rot_r, float* scores_dev, void* ws_dev,
                          size_t ws_bytes, void* stream) {
  return scores_split_impl("tq_scores_split", q_dev, B, Hq, Hkv, T, T, split, K_o, K_r, cb_o, cb_r, rot_o, rot_r,
                           scores_dev, ws_dev, ws_bytes, stream);
}

tq_status tq_scores_split_cache(const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t T_cap, tq_split_t split,
                                const tq_packed* K_o, const tq_packed* K_r, tq_codebook_t cb_o, tq_codebook_t cb_r,
                                tq_rotation_t rot_o, tq_rotation_t rot_r, float* scores_dev, void* ws_dev,
                                size_t ws_bytes, void* stream) {
  return scores_split_impl("tq_scores_split_cache", q_dev, B, Hq, Hkv, T, T_cap, split, K_o, K_r, cb_o, cb_r, rot_o,
                           rot_r, scores_dev, ws_dev, ws_bytes, stream);
}

size_t tq_search_workspace(int64_t nq, int64_t n, int d, int k) {
  if (nq <= 0 || n < 0 || d <= 0 || d % 128 != 0 || k < 1 || k > tq::kSearchMaxK) return 0;
  return tq::search_workspace_bytes(nq, n, d, k);
}

tq_status tq_search_topk(const float* q_dev, int64_t nq, const tq_packed* db, tq_codebook_t cb,
                         tq_rotation_t rot, tq_qjl_t qjl, int k, float* top_s_dev, int64_t* top_i_dev,
                         void* ws_dev, size_t ws_bytes, void* stream) {
  static const char* fn = "tq_search_topk";
  if (!db || !cb || !rot || !qjl) return fail(TQ_EINVAL, "%s: null handle or database", fn);
  if (nq < 0) return fail(TQ_EINVAL, "%s: negative nq", fn);
  if (k < 1 || k > tq::kSearchMaxK) return fail(TQ_EINVAL, "%s: k=%d outside [1, %d]", fn, k, tq::kSearchMaxK);
  const int d = db->d;
  if (db->mode != TQ_MODE_PROD) return fail(TQ_EUNSUPPORTED, "%s: the database must be prod mode", fn);
  if (db->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: the database must use the rows layout", fn);
  if (d != tq::kFragD && !general_d(d)) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported", fn, d);
  if (cb->d != d || rot->d != d || qjl->d != d)
    return fail(TQ_ESHAPE, "%s: d=%d, codebook d=%d, rotation d=%d, qjl d=%d", fn, d, cb->d, rot->d, qjl->d);
  if (cb->b != db->bits) return fail(TQ_ESHAPE, "%s: codebook has %d bits, database %d", fn, cb->b, db->bits);
  if (qjl->rot_id != rot->id) return fail(TQ_EINVAL, "%s: qjl handle is bound to another rotation", fn);
  tq_status st = check_packed(db, d, db->bits, TQ_MODE_PROD, fn);
  if (st != TQ_OK) return st;
  if (nq == 0) return ok();
  if (!q_dev || !top_s_dev || !top_i_dev || !ws_dev) return fail(TQ_EINVAL, "%s: null buffer", fn);
  const size_t need = tq::search_workspace_bytes(nq, db->n, d, k);
  if (ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  return check_launch(tq::launch_search_topk(q_dev, nq, db, cb->args, rot, qjl, k, top_s_dev, top_i_dev, ws_dev,
                                             as_stream(stream)),
                      fn);
}

// ---- outlier channels at 8 bits (d = 128) -------------------------------------------------

struct tq_outlier8_s {
  int H;
  int no;
  int device;
  std::vector<uint32_t> table;    // [H][8]: rest-mask words 0..3, then the sorted channels as bytes
  uint32_t* table_dev = nullptr;  // mask at [H][4], channels at H * 4 + [H][4]
};

tq_status tq_make_outlier8(int H, int d, int n_o, const int32_t* outliers_host, tq_outlier8_t* out) {
  static const char* fn = "tq_make_outlier8";
  if (!out || !outliers_host || H < 1) return fail(TQ_EINVAL, "%s: bad arguments", fn);
  if (d != tq::kFragD) return fail(TQ_EUNSUPPORTED, "%s: d=%d not supported (d=128)", fn, d);
  if (n_o != 4 && n_o != 8 && n_o != 16) return fail(TQ_EUNSUPPORTED, "%s: n_o=%d (4, 8 or 16)", fn, n_o);
  std::vector<uint32_t> table((size_t)H * 8, 0u);
  for (int h = 0; h < H; ++h) {
    bool seen[tq::kFragD] = {};
    for (int i = 0; i < n_o; ++i) {
      const int32_t c = outliers_host[(size_t)h * n_o + i];
      if (c < 0 || c >= tq::kFragD || seen[c])
        return fail(TQ_EINVAL, "%s: head %d: channel %d repeated or outside [0, 128)", fn, h, (int)c);
      seen[c] = true;
    }
    uint32_t* mask = &table[(size_t)h * 4];
    uint32_t* chan = &table[(size_t)H * 4 + (size_t)h * 4];
    int k = 0;
    for (int c = 0; c < tq::kFragD; ++c) {
      if (seen[c]) {
        chan[k >> 2] |= (uint32_t)c << (8 * (k & 3));
        ++k;
      } else {
        mask[c >> 5] |= 1u << (c & 31);
      }
    }
  }
  auto* o = new (std::nothrow) tq_outlier8_s();
  if (!o) return fail(TQ_ENOMEM, "host allocation failed");
  o->H = H;
  o->no = n_o;
  hipGetDevice(&o->device);
  o->table = std::move(table);
  tq_status st = upload(o->table, &o->table_dev, "upload outlier sets");
  if (st != TQ_OK) {
    delete o;
    return st;
  }
  *out = o;
  return ok();
}

void tq_outlier8_free(tq_outlier8_t o) {
  if (!o) return;
  if (o->table_dev) hipFree(o->table_dev);
  delete o;
}

static tq::OutlierArgs outlier8_args(tq_outlier8_t o, int64_t rows_per_seq) {
  tq::OutlierArgs a;
  a.mask = o->table_dev;
  a.chan = o->table_dev + (size_t)o->H * 4;
  a.T = (uint32_t)rows_per_seq;
  a.H = (uint32_t)o->H;
  a.no = o->no;
  return a;
}

// Handles and the packed rest code of outlier-8 keys: B * H sequences of `rows` rows each.
static tq_status check_outlier8_keys(int B, int H, int64_t rows, tq_outlier8_t o, tq_codebook_t cb,
                                     tq_rotation_t rot, const tq_packed* rest, const char* fn) {
  if (!o || !cb || !rot || !rest) return fail(TQ_EINVAL, "%s: null argument", fn);
  if (B < 0 || H < 0 || rows < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (o->H != H) return fail(TQ_ESHAPE, "%s: outlier sets of %d heads, keys have %d", fn, o->H, H);
  if (cb->d != tq::kFragD || rot->d != tq::kFragD) return fail(TQ_ESHAPE, "%s: codebook and rotation need d=128", fn);
  tq_status st = check_packed(rest, tq::kFragD, cb->b, TQ_MODE_MSE, fn);
  if (st != TQ_OK) return st;
  if (rest->layout != TQ_LAYOUT_ROWS) return fail(TQ_EUNSUPPORTED, "%s: the rest code uses the ROWS layout", fn);
  const int64_t n = (int64_t)B * H * rows;
  if (n >= (int64_t(1) << 31)) return fail(TQ_EUNSUPPORTED, "%s: %lld keys, at most 2^31 - 1", fn, (long long)n);
  if (rest->n != n)
    return fail(TQ_ESHAPE, "%s: rest n=%lld but B*H*%lld=%lld", fn, (long long)rest->n, (long long)rows, (long long)n);
  return TQ_OK;
}

tq_status tq_encode_outlier8(const void* x_dev, tq_dtype dt, int B, int H, int64_t T, tq_outlier8_t o,
                             tq_codebook_t cb, tq_rotation_t rot, tq_packed* rest, int8_t* q8_dev, float* scale_dev,
                             void* stream) {
  static const char* fn = "tq_encode_outlier8";
  tq_status st = check_outlier8_keys(B, H, T, o, cb, rot, rest, fn);
  if (st != TQ_OK) return st;
  if (dt != TQ_BF16 && dt != TQ_F32) return fail(TQ_EUNSUPPORTED, "%s: dtype %d", fn, (int)dt);
  if (!cb->args.sym) return fail(TQ_EUNSUPPORTED, "%s: the encode kernels need an antisymmetric codebook", fn);
  const int64_t n = (int64_t)B * H * T;
  if (n == 0) return ok();
  if (!x_dev || !q8_dev || !scale_dev) return fail(TQ_EINVAL, "%s: null x, q8 or scale", fn);
  if (reinterpret_cast<uintptr_t>(x_dev) % 16 != 0 || reinterpret_cast<uintptr_t>(q8_dev) % 16 != 0)
    return fail(TQ_EINVAL, "%s: x and q8 must be 16-byte aligned", fn);
  tq::OutlierArgs a = outlier8_args(o, T);
  a.q8 = q8_dev;
  a.scale = scale_dev;
  return check_launch(tq::launch_encode_outlier8(x_dev, dt == TQ_BF16, n, rot, cb->args, a, rest->idx, rest->norms,
                                                 as_stream(stream)),
                      fn);
}

size_t tq_scores_outlier8_workspace(int B, int Hq) {
  if (B < 0 || Hq < 0) return 0;
  return tq::scores_outlier8_workspace_bytes(B, Hq);
}

tq_status tq_scores_outlier8(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_outlier8_t o,
                             const tq_packed* rest, const int8_t* q8_dev, const float* scale_dev, tq_codebook_t cb,
                             tq_rotation_t rot, float* scores_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  static const char* fn = "tq_scores_outlier8";
  tq_status st = check_score_heads(B, Hq, Hkv, fn);
  if (st != TQ_OK) return st;
  st = check_outlier8_keys(B, Hkv, T, o, cb, rot, rest, fn);
  if (st != TQ_OK) return st;
  if (T > kMaxSeqTokens)
    return fail(TQ_EUNSUPPORTED, "%s: T=%lld exceeds %lld tokens per sequence", fn, (long long)T,
                (long long)kMaxSeqTokens);
  if ((int64_t)(Hq / Hkv) * T >= (int64_t(1) << 30))
    return fail(TQ_EUNSUPPORTED, "%s: (Hq/Hkv)*T=%lld: a kv head's score rows must stay below 4 GB", fn,
                (long long)(Hq / Hkv) * T);
  if ((int64_t)B * Hq * T == 0) return ok();
  if (!q_dev || !scores_dev || !q8_dev || !scale_dev) return fail(TQ_EINVAL, "%s: null q, scores, q8 or scale", fn);
  if (reinterpret_cast<uintptr_t>(q8_dev) % 16 != 0) return fail(TQ_EINVAL, "%s: q8 must be 16-byte aligned", fn);
  const size_t need = tq::scores_outlier8_workspace_bytes(B, Hq);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  return check_launch(tq::launch_scores_outlier8(q_dev, B, Hq, Hkv, T, T, rest, q8_dev, scale_dev, cb->args, rot,
                                                 outlier8_args(o, T), scores_dev, ws_dev, as_stream(stream)),
                      fn);
}

size_t tq_decode_attn_outlier8_workspace(int B, int Hq, int Hkv, int64_t T) {
  if (B < 0 || Hq < 0 || Hkv < 1 || T < 0) return 0;
  return tq::decode_attn_outlier8_workspace_bytes(B, Hq, Hkv, T);
}

tq_status tq_decode_attn_outlier8(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_outlier8_t o,
                                  const tq_packed* K, const int8_t* q8_dev, const float* scale_dev, const tq_packed* V,
                                  tq_codebook_t cb_k, tq_codebook_t cb_v, tq_rotation_t rot_k, tq_rotation_t rot_v,
                                  float scale, float* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  static const char* fn = "tq_decode_attn_outlier8";
  if (!V || !cb_v || !rot_v) return fail(TQ_EINVAL, "%s: null argument", fn);
  if (B < 0 || Hq < 0 || Hkv < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (T < 1) return fail(TQ_EINVAL, "%s: attention over an empty cache (T=%lld)", fn, (long long)T);
  if (T > kMaxSeqTokens)
    return fail(TQ_EUNSUPPORTED, "%s: %lld tokens per sequence exceed %lld", fn, (long long)T, (long long)kMaxSeqTokens);
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0)
    return fail(TQ_ESHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  const int ratio = Hq / Hkv;
  if (ratio != 1 && ratio != 2 && ratio != 4) return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d not in {1, 2, 4}", fn, ratio);
  tq_status st = check_outlier8_keys(B, Hkv, T, o, cb_k, rot_k, K, fn);
  if (st != TQ_OK) return st;
  if (rot_v->d != tq::kFragD || cb_v->d != tq::kFragD) return fail(TQ_ESHAPE, "%s: V handles need d=128", fn);
  st = check_packed(V, tq::kFragD, cb_v->b, TQ_MODE_MSE, fn);
  if (st != TQ_OK) return st;
  if (V->layout != TQ_LAYOUT_TOKEN_BLOCKED) return fail(TQ_EUNSUPPORTED, "%s: V must use the TOKEN_BLOCKED layout", fn);
  if (V->n != (int64_t)B * Hkv * T)
    return fail(TQ_ESHAPE, "%s: V->n=%lld, B*Hkv*T=%lld", fn, (long long)V->n, (long long)B * Hkv * T);
  if ((int64_t)B * Hkv > 65535) return fail(TQ_EUNSUPPORTED, "%s: B*Hkv above 65535", fn);
  if ((int64_t)B * Hq == 0) return ok();
  if (!q_dev || !out_dev || !q8_dev || !scale_dev) return fail(TQ_EINVAL, "%s: null q, out, q8 or scale", fn);
  if (reinterpret_cast<uintptr_t>(q8_dev) % 16 != 0) return fail(TQ_EINVAL, "%s: q8 must be 16-byte aligned", fn);
  const size_t need = tq::decode_attn_outlier8_workspace_bytes(B, Hq, Hkv, T);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  return check_launch(tq::launch_decode_attn_outlier8(q_dev, B, Hq, Hkv, T, T, K, q8_dev, scale_dev, V, cb_k->args,
                                                      cb_v->args, rot_k, rot_v, outlier8_args(o, T), scale, out_dev,
                                                      ws_dev, as_stream(stream)),
                      fn);
}

size_t tq_decode_attn_split_workspace(int B, int Hq, int Hkv, int64_t T) {
  if (B < 0 || Hq < 0 || Hkv < 1 || T < 0) return 0;
  return tq::decode_attn_workspace_bytes(B, Hq, Hkv, T, tq::kSplitD);
}

tq_status tq_decode_attn_split(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_split_t split,
                               const tq_packed* K_o, const tq_packed* K_r, const tq_packed* V, tq_codebook_t cb_o,
                               tq_codebook_t cb_r, tq_codebook_t cb_v, tq_rotation_t rot_o, tq_rotation_t rot_r,
                               tq_rotation_t rot_v, float scale, float* out_dev, void* ws_dev, size_t ws_bytes,
                               void* stream) {
  static const char* fn = "tq_decode_attn_split";
  if (!V || !cb_v || !rot_v) return fail(TQ_EINVAL, "%s: null argument", fn);
  if (B < 0 || Hq < 0 || Hkv < 0) return fail(TQ_EINVAL, "%s: negative size", fn);
  if (T < 1) return fail(TQ_EINVAL, "%s: attention over an empty cache (T=%lld)", fn, (long long)T);
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0)
    return fail(TQ_ESHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  const int ratio = Hq / Hkv;
  if (ratio != 1 && ratio != 2 && ratio != 4) return fail(TQ_EUNSUPPORTED, "%s: GQA ratio %d not in {1, 2, 4}", fn, ratio);
  tq_status st = check_split_keys(B, Hkv, T, split, cb_o, cb_r, rot_o, rot_r, K_o, K_r, fn);
  if (st != TQ_OK) return st;
  if (rot_v->d != tq::kSplitD || cb_v->d != tq::kSplitD) return fail(TQ_ESHAPE, "%s: V handles need d=128", fn);
  st = check_packed(V, tq::kSplitD, cb_v->b, TQ_MODE_MSE, fn);
  if (st != TQ_OK) return st;
  if (V->layout != TQ_LAYOUT_TOKEN_BLOCKED) return fail(TQ_EUNSUPPORTED, "%s: V must use the TOKEN_BLOCKED layout", fn);
  if (V->n != (int64_t)B * Hkv * T)
    return fail(TQ_ESHAPE, "%s: V->n=%lld, B*Hkv*T=%lld", fn, (long long)V->n, (long long)B * Hkv * T);
  const bool pair_ok = (cb_o->b == 3 && cb_r->b == 2) || (cb_o->b == 4 && cb_r->b == 3);
  if (!pair_ok || cb_v->b < 2)
    return fail(TQ_EUNSUPPORTED, "%s: (b_o, b_r, b_v) = (%d, %d, %d): needs (3, 2) or (4, 3) and b_v in 2..4", fn,
                cb_o->b, cb_r->b, cb_v->b);
  if ((int64_t)B * Hq == 0) return ok();
  if (!q_dev || !out_dev) return fail(TQ_EINVAL, "%s: null q or out", fn);
  const size_t need = tq::decode_attn_workspace_bytes(B, Hq, Hkv, T, tq::kSplitD);
  if (!ws_dev || ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  return check_launch(tq::launch_decode_attn_split(q_dev, B, Hq, Hkv, T, K_o, K_r, V, cb_o->args, cb_r->args,
                                                   cb_v->args, split->order_dev, rot_o->rt32_dev, rot_r->rt32_dev,
                                                   rot_v, scale, out_dev, ws_dev, as_stream(stream)),
                      fn);
}
