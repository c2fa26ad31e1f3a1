/*
 * tq.h -- C ABI of the TurboQuant encode / compressed-key score library for MI355X (gfx950).
 *
 * The library implements the data-parallel hot path of TurboQuant:
 *   encode : s = ||x||, y = R (x / s), per-coordinate Lloyd-Max index, b-bit packing, and for
 *            TurboQuant_prod a 1-bit QJL sign sketch of the residual plus its norm;
 *   score  : <q, x_hat> from packed keys with the query rotated once, optional QJL term,
 *            GQA sharing, and fused decode attention softmax(q K_hat^T * scale) V_hat.
 * Source pages (cited by title and section):
 *   [TQ]  "TurboQuant 详解" (wnma3mz blog): quantizer definition, TurboQuant_mse official steps,
 *         TurboQuant_prod section, KV prefill/decode flow.
 *   [FP]  "TurboQuant first-principles walkthrough" (blog.hotdry.top): rotation, codebook,
 *         distortion bound, QJL constant, fixed seed.
 *   [RQ]  "TurboQuant 和 RotorQuant 的真相" (zhichai.net): attention formula, word-wise unpack.
 *   [SB]  "Sub-byte KV cache quantization with TurboQuant" (blog2.hotdry.top): codebook
 *         recipe, fused score kernel with a pre-rotated query, GQA mapping, checklist.
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev are device pointers (HIP global memory of the current device);
 *    pointers named *_host are host pointers.  The caller owns every buffer it passes; the
 *    library never frees or retains caller memory.  Handles (codebook, rotation, qjl) are
 *    owned by the library until the matching *_free call; they are immutable after creation
 *    and may be shared across streams and threads.
 *  - Device work is enqueued on the given stream (NULL = the default stream) and is
 *    asynchronous; nothing synchronises the stream.  No entry point that takes a stream
 *    allocates device memory.
 *  - Return value: TQ_OK, or an error code.  Arguments are validated before any launch; on
 *    error nothing is enqueued, outputs are untouched, and tq_last_error() returns a
 *    thread-local message.  Asynchronous device faults surface at the caller's next
 *    synchronisation.  Non-finite inputs give unspecified (but in-bounds) results.
 *  - Sizes: 1 <= b <= 4 bits per index stage; d * b must be a multiple of 32.  Vector length
 *    d: the fused kernels cover d = 128, the head dimension of the KV workloads.  tq_encode,
 *    tq_decode, tq_rotate and tq_search_topk also take d a multiple of 128 in [256, 4096] (the
 *    embedding workloads, d = 1536 among them) on the general-d kernels.  Head dims 64 and 256
 *    ("Sub-byte KV cache quantization with TurboQuant", deployment checklist: the codebook d is
 *    the model's head_dim): tq_encode (rows layout; d = 64 on its own kernel), tq_scores,
 *    tq_scores_cache and tq_decode_attn (V in the rows layout) take them on the kernels of
 *    csrc/tq_kvgen.hip.  The prepared and static-scratch scores, the cache appends, prefill, split
 *    and outlier-8 entry points take d = 128 only.  Any other d returns TQ_EUNSUPPORTED.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 7

typedef enum tq_status {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* null pointer, bits out of range, negative size, bad enum */
  TQ_ESHAPE = 2,        /* d mismatch between codebook / rotation / tensors ([SB] checklist:
                           the codebook dimension must equal head_dim); Hq % Hkv != 0;
                           d * b not a multiple of 32 */
  TQ_EUNSUPPORTED = 3,  /* Hadamard rotation with d not a power of two; d outside the
                           supported range for this entry point; unsupported dtype */
  TQ_ENOMEM = 4,        /* caller workspace too small, or host allocation failed */
  TQ_EDEVICE = 5        /* a HIP runtime error (text in tq_last_error) */
} tq_status;

typedef enum tq_density { TQ_DENSITY_BETA = 0, TQ_DENSITY_GAUSS = 1 } tq_density;
/* Rotation kinds: DENSE = Q of the QR of a seeded Gaussian matrix; WHT = (1/sqrt(d)) H_d diag(sigma)
 * (d a power of two); BLOCK_WHT = (1/sqrt(32)) blockdiag(H_32, ..., H_32) diag(sigma), d a multiple
 * of 32 ([RQ] chapter 3: the 128 coordinates split into 4 groups of 32, each rotated on its own;
 * chapter 5: small orthogonal blocks instead of a full-rank transform). */
typedef enum tq_rot_kind { TQ_ROT_DENSE = 0, TQ_ROT_WHT = 1, TQ_ROT_BLOCK_WHT = 2 } tq_rot_kind;
typedef enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;
typedef enum tq_mode { TQ_MODE_MSE = 0, TQ_MODE_PROD = 1 } tq_mode;
/* Storage layout of packed indices.  ROWS: row r is the LSB-first stream of vector r's d
 * indices (d*bits/32 words per row).  TOKEN_BLOCKED (MSE only; the value-cache layout read by
 * tq_decode_attn): rows are grouped in blocks of 32 (rows past n hold index 0); inside block B,
 * chunk (o, c) for octet o = 0..3 and coordinate c = 0..d-1 sits at chunk position o*d + c and
 * holds the indices of rows 32B + 8o + e, e = 0..7, at coordinate c, LSB-first (row e at chunk
 * bits [bits*e, bits*e + bits)); the 8*bits-bit chunks are concatenated LSB-first, d*bits words
 * per block, ceil(n/32) blocks.  The pages fix no layout; both are this library's choice. */
typedef enum tq_layout { TQ_LAYOUT_ROWS = 0, TQ_LAYOUT_TOKEN_BLOCKED = 1 } tq_layout;

typedef struct tq_codebook_s* tq_codebook_t;
typedef struct tq_rotation_s* tq_rotation_t;
typedef struct tq_qjl_s* tq_qjl_t;
typedef struct tq_split_s* tq_split_t;
typedef struct tq_outlier8_s* tq_outlier8_t;

/* A packed set of n encoded vectors, all buffers device memory owned by the caller.
 * Row r of idx holds the d indices of vector r as one LSB-first bit stream: coordinate i
 * occupies stream bits [i*bits, i*bits + bits), stream bit p is bit (p % 32) of word p / 32
 * ([TQ] KV prefill example, step 5: a compact bit stream).  Row r of qjl holds bit i = 1 iff
 * (S r)_i >= 0 ([TQ] TurboQuant_prod: sign(0) = +1).  norms are fp32 ||x||, rnorms fp32
 * residual norms gamma = ||x - x_hat_mse||. */
typedef struct tq_packed {
  int32_t d;          /* vector length */
  int32_t bits;       /* bits per index: b for MSE, b - 1 for prod */
  int32_t mode;       /* tq_mode */
  int32_t layout;     /* tq_layout of idx */
  int64_t n;          /* number of vectors (rows) */
  uint32_t* idx;      /* ROWS: [n, d*bits/32]; TOKEN_BLOCKED: [ceil(n/32), d*bits] */
  float* norms;       /* [n] */
  uint32_t* qjl;      /* [n, d/32] for prod, else NULL */
  float* rnorms;      /* [n] for prod, else NULL */
} tq_packed;

/* ---- housekeeping ------------------------------------------------------------------- */
int tq_abi_version(void);
/* Thread-local text of the last error on this thread ("" if none).  Never NULL. */
const char* tq_last_error(void);

/* ---- host-only math (no GPU needed; deterministic; caller-owned host outputs) -------- */

/* Draws offset .. offset+n-1 of the SplitMix64 stream of `seed` (Steele, Lea, Flood 2014):
 * mix(seed + (i+1) * 0x9E3779B97F4A7C15).  The pages fix only "a fixed seed" ([FP] deployment
 * parameters); this generator is the library's reading. */
tq_status tq_host_splitmix64(uint64_t seed, uint64_t offset, int64_t n, uint64_t* out_host);
/* n standard normals of stream `seed`: Box-Muller cosine branch, draws 2e and 2e+1. */
tq_status tq_host_gaussian(uint64_t seed, int64_t n, double* out_host);
/* The (d, b) Lloyd-Max codebook on a 50000-point grid over +-6/sqrt(d) (clipped to [-1, 1]),
 * 300 iterations ([SB] engineering path, first layer; density [TQ] key insight), made
 * antisymmetric.  centroids_host: 2^b values; thresholds_host: 2^b - 1 midpoints.
 * Errors: TQ_EINVAL for b outside 1..4, d < 2 or bad density. */
tq_status tq_host_codebook(int d, int b, tq_density dens, double* centroids_host,
                           double* thresholds_host);
/* Rotation matrix R (d x d, row-major, y = R u): DENSE = Q of the QR of the seeded Gaussian
 * matrix with a non-negative triangular diagonal ([TQ] official step 1; [FP] rotation);
 * WHT = (1/sqrt(d)) H_d diag(sigma), Sylvester H, Rademacher sigma ([RQ] chapter 3);
 * BLOCK_WHT = the same with H_32 blocks on the diagonal and 1/sqrt(32).
 * Errors: TQ_EUNSUPPORTED for WHT with d not a power of two or BLOCK_WHT with d not a multiple
 * of 32; TQ_EINVAL for d < 2 or a bad kind. */
tq_status tq_host_rotation(int d, uint64_t seed, tq_rot_kind kind, double* r_host);
/* QJL matrix S (d x d, row-major, i.i.d. N(0,1) from stream `seed`). */
tq_status tq_host_qjl_matrix(int d, uint64_t seed, double* s_host);

/* ---- handles (created on the current device; uploads are synchronous) ---------------- */

/* Codebook handle for (d, b) by the recipe of tq_host_codebook. */
tq_status tq_codebook(int d, int b, tq_density dens, tq_codebook_t* out);
/* Codebook handle from caller centroids (2^b strictly increasing values, host). */
tq_status tq_codebook_from_values(int d, int b, const double* centroids_host, tq_codebook_t* out);
/* Reads back the fp64 centroids (2^b) and thresholds (2^b - 1) of a handle. */
tq_status tq_codebook_values(tq_codebook_t cb, double* centroids_host, double* thresholds_host);
void tq_codebook_free(tq_codebook_t cb);

/* Rotation handle: R generated once from `seed` and kept ([FP]: generated at init, shared by
 * all vectors).  The device copies include MFMA fragments for the fused kernels (d = 128) or
 * the general-d kernels (d a multiple of 128 in [256, 4096]); WHT needs d a power of two. */
tq_status tq_make_rotation(int d, uint64_t seed, tq_rot_kind kind, tq_rotation_t* out);
/* Rotation handle from a caller matrix (row-major d x d host fp64; treated as DENSE). */
tq_status tq_rotation_from_matrix(int d, const double* r_host, tq_rotation_t* out);
/* Copies the fp64 matrix of a rotation handle to r_host (d*d). */
tq_status tq_rotation_export(tq_rotation_t rot, double* r_host);
void tq_rotation_free(tq_rotation_t rot);

/* QJL handle for TurboQuant_prod ([TQ] TurboQuant_prod; [FP] QJL paragraph): S from `seed`,
 * bound to `rot` (the library keeps S' = S R^T so the sketch is taken of the rotated-domain
 * residual: sign(S r) = sign(S' (y - y_hat))).  rot must outlive nothing: S' is copied. */
tq_status tq_make_qjl(int d, uint64_t seed, tq_rotation_t rot, tq_qjl_t* out);
tq_status tq_qjl_from_matrix(int d, const double* s_host, tq_rotation_t rot, tq_qjl_t* out);
void tq_qjl_free(tq_qjl_t qjl);

/* ---- hot path ------------------------------------------------------------------------ */

/* Words per packed row: d * bits / 32. */
size_t tq_packed_words(int d, int bits);
/* Words of the idx buffer for n vectors in the given layout (0 on invalid arguments). */
size_t tq_packed_idx_words(int64_t n, int d, int bits, tq_layout layout);

/* Encode n vectors x_dev [n, d] (dtype dt, row-major) into *out ([TQ] official steps 1-4 and
 * KV prefill steps 1-6; prod: [TQ] TurboQuant_prod, (b-1)-bit stage + 1-bit QJL).
 * out->layout selects ROWS or TOKEN_BLOCKED (MSE only).
 * b is the total bit budget per coordinate; cb must have b bits (MSE) or b - 1 bits (prod);
 * qjl must be non-NULL exactly for prod and bound to `rot`.  out->d, out->bits, out->mode,
 * out->n must describe the call; out->idx/norms (and qjl/rnorms for prod) are written.
 * A zero vector encodes to norm 0 and the indices of y = 0.
 * Supported d: 128 (one fused kernel; rows or token-blocked layout; the randomized Hadamard
 * rotations in MSE mode as a butterfly transform in registers), 64 (rows layout; one wave per
 * vector, the rotation and the QJL sketch as fp32 matrix-vector products), or a multiple of 128 in
 * [256, 4096] (rows layout; rotation as a tiled MFMA GEMM whose epilogue quantizes and packs;
 * prod adds a second GEMM with S' on the residual, staged through ws_dev in chunks of vectors).
 * ws_dev / ws_bytes: caller device workspace, at least tq_encode_workspace(n, d, b, mode) bytes
 * is the size that needs a single chunk; any size that holds 128 vectors' residuals works
 * (more launches).  It may be NULL when tq_encode_workspace returns 0.
 * Errors: TQ_EINVAL, TQ_ESHAPE, TQ_EUNSUPPORTED as above; TQ_ENOMEM if ws_bytes is too small. */
tq_status tq_encode(const void* x_dev, tq_dtype dt, int64_t n, int d, int b, tq_mode mode,
                    tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, tq_packed* out,
                    void* ws_dev, size_t ws_bytes, void* stream);
/* Workspace bytes for tq_encode of n vectors: 0 for MSE and for d = 128; for prod at other d,
 * min(n, 131072) vectors x (d + d/128) fp32 values (residual rows and per-block partial norms). */
size_t tq_encode_workspace(int64_t n, int d, int b, tq_mode mode);

/* Rotated unit coordinates y = R x / ||x|| (fp32 [n, d]) and norms (fp32 [n]) exactly as the
 * encode kernel forms them before quantizing (same kernel, stores instead of packing).
 * For parity checks of the rotation.  d = 128, or a multiple of 128 in [256, 4096]. */
tq_status tq_rotate(const void* x_dev, tq_dtype dt, int64_t n, int d, tq_rotation_t rot,
                    float* y_dev, float* norms_dev, void* stream);

/* Bucketize + pack given fp32 rotated unit coordinates y_dev [n, d] against the fp32
 * thresholds of cb ([TQ] official step 3, nearest centroid; ties to the upper index);
 * writes idx_dev [n, d*b/32].  Bit-exact reference entry for the quantizer. */
tq_status tq_quantize_rotated(const float* y_dev, int64_t n, int d, tq_codebook_t cb,
                              uint32_t* idx_dev, void* stream);

/* Reconstruct x_hat_dev [n, d] fp32 = s R^T C[idx] ([TQ] official step 5), plus
 * gamma sqrt(pi/2)/d S^T z when qjl is non-NULL and p->mode is prod. */
tq_status tq_decode(const tq_packed* p, tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl,
                    float* xhat_dev, void* stream);

/* Workspace bytes tq_scores needs for B*Hq query heads of length d. */
size_t tq_scores_workspace(int B, int Hq, int d);
/* Raw scores <q, k_hat> (no 1/sqrt(d)) of q_dev [B, Hq, d] fp32 against packed keys K laid out
 * [B, Hkv, T] (K->n == B*Hkv*T), into scores_dev [B, Hq, T] fp32.  The query is rotated once
 * ([SB] third layer); query head h reads kv head h / (Hq / Hkv) ([SB] GQA mapping).
 * MSE: s <R q, C[idx]>;  prod: plus gamma sqrt(pi/2)/d <S q, z> ([TQ] TurboQuant_prod;
 * [FP] QJL constant).  The GQA ratio Hq / Hkv must be 1, 2, 3 or 4, or a multiple of 4 up to 64
 * (TQ_EUNSUPPORTED otherwise); d = 128, 64 or 256 (the last two: R q and S q in fp32, one thread
 * per key). */
tq_status tq_scores(const float* q_dev, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                    tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, float* scores_dev,
                    void* ws_dev, size_t ws_bytes, void* stream);

/* tq_scores for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same kernels and results, with the query
 * workspace taken from a static device array inside the library (tq_scores_noalloc_max_bytes()
 * bytes, 4 MiB: up to 4080 query heads B*Hq) instead of a caller buffer.  Each GPU holds its own
 * copy of that array until the process ends; its address is looked up on the first call on each
 * device.  Nothing is allocated: no hipMalloc, no hipFree, no allocating library call.  Every call
 * on one GPU uses the same array, so calls whose work overlaps on one GPU (other streams, other
 * threads) race and may return wrong scores: serialise them.  Errors as for tq_scores, plus
 * TQ_ENOMEM when tq_scores_workspace(B, Hq, d) exceeds the static size; d = 128 only. */
tq_status tq_scores_noalloc(const float* q_dev, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                            tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl, float* scores_dev, void* stream);
size_t tq_scores_noalloc_max_bytes(void);

/* The two stages of tq_scores, for callers that overlap the query prologue with other work (for
 * instance the encode of the keys being appended) on another stream.
 * tq_prepare_queries: q_rot = R q (fp16 hi/lo) and, when qjl is non-NULL, the QJL sketch S q
 * with its per-head constants, for q_dev [B, Hq, d] fp32, written into ws_dev (at least
 * tq_scores_workspace(B, Hq, d) bytes) ([SB] third layer: the query is rotated once).
 * tq_scores_prepared: the scores of tq_scores from such a workspace.  The workspace must have been
 * prepared with the same B, Hq, Hkv and rotation as the keys, and with the keys' qjl handle when K
 * is prod mode (the device contents are not checked).  Errors as for tq_scores; d = 128 only. */
tq_status tq_prepare_queries(const float* q_dev, int B, int Hq, int Hkv, tq_rotation_t rot, tq_qjl_t qjl,
                             void* ws_dev, size_t ws_bytes, void* stream);
tq_status tq_scores_prepared(const void* ws_dev, size_t ws_bytes, int B, int Hq, int Hkv, int64_t T,
                             const tq_packed* K, tq_codebook_t cb, float* scores_dev, void* stream);

/* Workspace bytes tq_decode_attn needs (query prologue plus per-split softmax partials). */
size_t tq_decode_attn_workspace(int B, int Hq, int Hkv, int64_t T, int d);
/* Fused decode attention over compressed K and V ([RQ] chapter 1: softmax(q K^T / sqrt(d)) V;
 * [TQ] decode section, second route: unpack, look up, scale and accumulate inside the kernel,
 * never materialising K_hat or V_hat; K and V stored TurboQuant_mse per [SB]).
 * out[b, h] = sum_t softmax_t(scale * <q[b,h], k_hat[b,g,t]>) v_hat[b,g,t], g = h / (Hq/Hkv),
 * k_hat = s_k R_K^T C_K[idx], v_hat = s_v R_V^T C_V[idx].  q_dev [B, Hq, d] fp32; K: ROWS
 * layout, MSE, n = B*Hkv*T; V: MSE, n = B*Hkv*T, TOKEN_BLOCKED layout at d = 128 and ROWS layout
 * at d = 64 or 256; out_dev [B, Hq, d] fp32.  The value sum is accumulated in V's rotated domain
 * and R_V^T is applied once per head.  Requires T >= 1 and d = 128 with Hq/Hkv in {1, 2, 4}, or
 * d = 64 or 256 with Hq/Hkv <= 8.  Errors as for tq_scores; TQ_EINVAL for T < 1. */
tq_status tq_decode_attn(const float* q_dev, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                         const tq_packed* V, tq_codebook_t cb_k, tq_codebook_t cb_v,
                         tq_rotation_t rot_k, tq_rotation_t rot_v, float scale, float* out_dev,
                         void* ws_dev, size_t ws_bytes, void* stream);

/* ---- streaming KV cache ---------------------------------------------------------------
 * [TQ] KV-cache example (prefill and decode): prefill writes the prompt's compressed keys and
 * values into the persistent cache; every decode step appends the new token's key and value to
 * the end of the cache at once, then attends over everything cached.  The section after it:
 * no online fitting is needed, so a token is quantized and written as soon as it exists.
 * A cache holds B*H sequences of capacity T_cap tokens each: sequence s = b*H + h owns rows
 * [s*T_cap, (s+1)*T_cap) of its packed buffers (cache->n == B*H*T_cap), all allocated once by
 * the caller, whose initial contents do not matter.  Keys: ROWS layout, MSE or prod.  Values:
 * TOKEN_BLOCKED layout, MSE, with T_cap a multiple of 32 so that every sequence owns whole
 * blocks.  Only d = 128. */

/* Encodes x_dev [B, H, n_new, d] (dtype dt, row-major) into rows pos .. pos+n_new-1 of every
 * sequence of *cache, with the rules of tq_encode for b, mode, cb, rot and qjl.  Every other
 * stored bit of the cache is left as it was, including the fields of other tokens that share a
 * value block (those fields are cleared and set with atomic operations on disjoint bits), so
 * appends to disjoint rows may run concurrently.  Appends of fewer than 64 tokens (decode
 * steps) run one fp32 block per token; longer ones (prefill) run the fused MFMA encode kernels
 * on whole rows, or on whole value blocks with the partial blocks at either end done per token.
 * Errors: TQ_EINVAL (null pointers, negative sizes, pos + n_new > T_cap, bits, mode, qjl
 * handle as for tq_encode); TQ_ESHAPE (cache->n != B*H*T_cap, codebook bits or d, TOKEN_BLOCKED
 * with T_cap % 32 != 0); TQ_EUNSUPPORTED (d != 128, dtype, B*H > 65535, n_new >= 2^31). */
tq_status tq_cache_append(const void* x_dev, tq_dtype dt, int B, int H, int64_t n_new, int64_t pos,
                          int64_t T_cap, int b, tq_mode mode, tq_codebook_t cb, tq_rotation_t rot,
                          tq_qjl_t qjl, tq_packed* cache, void* stream);

/* A decode step's appends to both caches in one call: keys k_dev and values v_dev [B, H, n_new, d]
 * (dtype dt) into rows pos .. pos+n_new-1 of a key cache K (ROWS layout, MSE, b_k bits, cb_k,
 * rot_k) and a value cache V (TOKEN_BLOCKED layout, MSE, b_v bits, cb_v, rot_v) of the same
 * geometry, with the results of two tq_cache_append calls.  Appends of fewer than 64 tokens run
 * both caches in one launch (for the (b_k, b_v) pairs tq_decode_attn takes; others in two).
 * Errors: those of tq_cache_append for either cache; TQ_EUNSUPPORTED for the wrong layouts. */
tq_status tq_kv_append(const void* k_dev, const void* v_dev, tq_dtype dt, int B, int H, int64_t n_new,
                       int64_t pos, int64_t T_cap, int b_k, int b_v, tq_codebook_t cb_k,
                       tq_codebook_t cb_v, tq_rotation_t rot_k, tq_rotation_t rot_v, tq_packed* K,
                       tq_packed* V, void* stream);

/* tq_scores over the first T rows (0 <= T <= T_cap) of every sequence of a key cache of capacity
 * T_cap (K->n == B*Hkv*T_cap): scores_dev [B, Hq, T].  Otherwise as tq_scores, with
 * TQ_EINVAL for T > T_cap. */
tq_status tq_scores_cache(const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t T_cap,
                          const tq_packed* K, tq_codebook_t cb, tq_rotation_t rot, tq_qjl_t qjl,
                          float* scores_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* tq_decode_attn over the first T rows (1 <= T <= T_cap) of every sequence of a key cache and a
 * value cache of capacity T_cap (a multiple of 32; K->n == V->n == B*Hkv*T_cap).  Workspace:
 * tq_decode_attn_workspace(B, Hq, Hkv, T, d) bytes (grows with T: size it with T_cap once to
 * cover every decode step).  Errors as for tq_decode_attn; TQ_EINVAL for T > T_cap; TQ_ESHAPE
 * for T_cap % 32 != 0. */
tq_status tq_decode_attn_cache(const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t T_cap,
                               const tq_packed* K, const tq_packed* V, tq_codebook_t cb_k,
                               tq_codebook_t cb_v, tq_rotation_t rot_k, tq_rotation_t rot_v,
                               float scale, float* out_dev, void* ws_dev, size_t ws_bytes,
                               void* stream);

/* Workspace bytes of tq_prefill_attn for a chunk of n_new tokens (the rotated queries, fp16 hi and
 * lo): 512 bytes per query row B*Hq*n_new.  0 for d != 128. */
size_t tq_prefill_attn_workspace(int B, int Hq, int64_t n_new, int d);
/* Prefill of a chunk fused with attention over the compressed cache ([TQ] KV-cache example,
 * prefill: the prompt's keys and values are compressed as they are written; decode section, second
 * route: unpack, look up and scale inside the attention, never materialising K_hat or V_hat;
 * [RQ] Flash Attention fusion section).  Appends keys k_dev and values v_dev [B, Hkv, n_new, d]
 * (dtype dt) at rows pos .. pos + n_new - 1 of every sequence of the key cache K (ROWS, MSE, cb_k's
 * bits) and the value cache V (TOKEN_BLOCKED, MSE, cb_v's bits) of capacity T_cap, exactly as
 * tq_kv_append does, then writes out_dev[b, h, i] (fp32 [B, Hq, n_new, d]) =
 *   sum_{t <= pos + i} softmax_t(scale <q[b,h,i], k_hat[b,g,t]>) v_hat[b,g,t],  g = h / (Hq/Hkv),
 * for queries q_dev fp32 [B, Hq, n_new, d]: chunk token i sits at position pos + i and attends
 * causally to every cached token up to itself (earlier chunks included).  Keys and values are read
 * back from the packed caches inside the kernel (k_hat = s R_K^T C_K[idx], v_hat = s R_V^T C_V[idx]);
 * the value sum runs in V's rotated domain and R_V^T is applied once per output row.
 * d = 128; T_cap a multiple of 32; GQA ratio up to 64; (b_k, b_v) in {(1,1), (2,2), (3,3), (4,4),
 * (2,3), (2,4), (3,2), (3,4), (4,2), (4,3)}.  ws_dev: tq_prefill_attn_workspace bytes.
 * Errors: those of tq_kv_append for either cache; TQ_ESHAPE (Hq % Hkv, T_cap % 32); TQ_EUNSUPPORTED
 * (ratio, bit pair, more than 2^31 - 1 query rows); TQ_ENOMEM (workspace); TQ_EINVAL (null pointers). */
tq_status tq_prefill_attn(const float* q_dev, const void* k_dev, const void* v_dev, tq_dtype dt, int B, int Hq,
                          int Hkv, int64_t n_new, int64_t pos, int64_t T_cap, tq_codebook_t cb_k, tq_codebook_t cb_v,
                          tq_rotation_t rot_k, tq_rotation_t rot_v, tq_packed* K, tq_packed* V, float scale,
                          float* out_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* ---- outlier-channel mixed precision (d = 128) ----------------------------------------
 * [RQ] the asymmetric needs of K and V: keys need more bits, e.g. mixed precision with the
 * outlier channels at more bits than the rest; [TQ] engineering data points: 2.5 and 3.5 bits
 * per channel.  The pages fix no mechanism; this library's reading: per KV head, the caller
 * names 64 outlier channels of the 128; each key vector becomes two TurboQuant_mse codes, its
 * outlier half (channels in the listed order) at b_o bits and its other half (ascending channel
 * order) at b_r bits, each half with its own norm, its own 64 x 64 rotation and the codebook of
 * dimension 64: (b_o + b_r) / 2 bits per channel, 2.5 at (3, 2) and 3.5 at (4, 3). */

/* Channel split of H KV heads: outliers_host [H, 64] int32, each row 64 distinct channels in
 * [0, 128).  The handle keeps the per-head channel order (outliers as listed, then the rest
 * ascending) on the current device.  d must be 128.  Errors: TQ_EINVAL (null pointers, H < 1,
 * a repeated or out-of-range channel), TQ_EUNSUPPORTED (d != 128), TQ_EDEVICE. */
tq_status tq_make_split(int H, int d, const int32_t* outliers_host, tq_split_t* out);
void tq_split_free(tq_split_t split);

/* Split encode of keys x_dev [B, H, T, 128] (dtype dt): out_o receives the outlier halves and
 * out_r the other halves, each a ROWS-layout MSE packed set with d = 64 and n = B*H*T (bits =
 * cb_o->b resp. cb_r->b; idx [n, 2*bits] words, norms [n] = the half's ||x_half||).  cb_o, cb_r:
 * codebooks with d = 64; rot_o, rot_r: rotations with d = 64 (any kind).  Index decisions follow
 * tq_encode's rule (ties to the upper index) on the half's rotation, formed in fp32 for up to
 * 32 tokens per sequence and otherwise like tq_encode's (R as bf16 hi + lo operands, fp32 sums).
 * x_dev must be 16-byte aligned.  Errors: TQ_EINVAL
 * (null pointers, negative sizes, misaligned x), TQ_ESHAPE (split->H != H, a handle or packed
 * set with d != 64, n or bits mismatch), TQ_EUNSUPPORTED (dtype, layout, B*H > 65535,
 * T > 2^25). */
tq_status tq_encode_split(const void* x_dev, tq_dtype dt, int B, int H, int64_t T, tq_split_t split,
                          tq_codebook_t cb_o, tq_codebook_t cb_r, tq_rotation_t rot_o,
                          tq_rotation_t rot_r, tq_packed* out_o, tq_packed* out_r, void* stream);

/* Workspace bytes of tq_scores_split: the rotated queries, B*Hq*128 fp32. */
size_t tq_scores_split_workspace(int B, int Hq);
/* Raw scores <q, x_hat> of queries q_dev [B, Hq, 128] fp32 against split-coded keys K_o, K_r
 * (as written by tq_encode_split for [B, Hkv, T]) into scores_dev [B, Hq, T] fp32: the sum over
 * the two halves of s_half <R_half q_half, C_half[idx]>, q_half gathered through the channel
 * order of the query head's KV head h // (Hq / Hkv).  Errors: as tq_encode_split for the keys and
 * handles; TQ_ESHAPE (Hq not a positive multiple of Hkv); TQ_EUNSUPPORTED (Hq / Hkv above 64);
 * TQ_ENOMEM (workspace). */
tq_status tq_scores_split(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_split_t split,
                          const tq_packed* K_o, const tq_packed* K_r, tq_codebook_t cb_o,
                          tq_codebook_t cb_r, tq_rotation_t rot_o, tq_rotation_t rot_r,
                          float* scores_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* Split codes as a streaming key cache ([TQ] KV-cache example: each decode step appends the new
 * token's key to the end of the cache; prefill writes the prompt's keys): keys x_dev
 * [B, H, n_new, 128] (dtype dt) into rows pos .. pos + n_new - 1 of every sequence of split
 * codes K_o, K_r of capacity T_cap (K_o->n == K_r->n == B*H*T_cap, sequence s owning rows
 * [s*T_cap, (s+1)*T_cap)).  Every other row is left unchanged.  Otherwise as tq_encode_split,
 * with TQ_EINVAL for pos + n_new > T_cap or negative n_new / pos. */
tq_status tq_cache_append_split(const void* x_dev, tq_dtype dt, int B, int H, int64_t n_new, int64_t pos,
                                int64_t T_cap, tq_split_t split, tq_codebook_t cb_o, tq_codebook_t cb_r,
                                tq_rotation_t rot_o, tq_rotation_t rot_r, tq_packed* K_o, tq_packed* K_r,
                                void* stream);
/* tq_scores_split over the first T rows (0 <= T <= T_cap) of every sequence of such a cache:
 * scores_dev [B, Hq, T].  Otherwise as tq_scores_split, with TQ_EINVAL for T > T_cap. */
tq_status tq_scores_split_cache(const float* q_dev, int B, int Hq, int Hkv, int64_t T, int64_t T_cap,
                                tq_split_t split, const tq_packed* K_o, const tq_packed* K_r,
                                tq_codebook_t cb_o, tq_codebook_t cb_r, tq_rotation_t rot_o,
                                tq_rotation_t rot_r, float* scores_dev, void* ws_dev, size_t ws_bytes,
                                void* stream);

/* Workspace bytes of tq_decode_attn_split (as tq_decode_attn's at d = 128). */
size_t tq_decode_attn_split_workspace(int B, int Hq, int Hkv, int64_t T);
/* Fused decode attention with split-coded keys ([RQ] chapter 1 formula and the asymmetric K/V
 * needs): as tq_decode_attn, with the logit of key t for query head h equal to scale * (the sum
 * over the two halves of s_half <R_half q_half, C_half[idx_half]>), q_half gathered through the
 * channel order of h's KV head.  K_o, K_r: split keys of [B, Hkv, T] as written by
 * tq_encode_split; V: TOKEN_BLOCKED MSE values of [B, Hkv, T] with d = 128; out_dev [B, Hq, 128]
 * fp32.  (b_o, b_r) must be (3, 2) or (4, 3) (2.5 and 3.5 bits per channel) and b_v 2, 3 or 4;
 * GQA ratio 1, 2 or 4; T >= 1.  Errors: as tq_scores_split for the keys and handles, as
 * tq_decode_attn otherwise; TQ_EUNSUPPORTED for other bit widths. */
tq_status tq_decode_attn_split(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_split_t split,
                               const tq_packed* K_o, const tq_packed* K_r, const tq_packed* V,
                               tq_codebook_t cb_o, tq_codebook_t cb_r, tq_codebook_t cb_v,
                               tq_rotation_t rot_o, tq_rotation_t rot_r, tq_rotation_t rot_v, float scale,
                               float* out_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* ---- outlier channels at 8 bits (d = 128) --------------------------------------------
 * [RQ] the asymmetric needs of K and V: one practice keeps a key's outlier channels at 8 bits
 * and codes the other channels at 3.  The page fixes neither the outlier set nor the 8-bit
 * format; this library's reading: per KV head the caller names n_o outlier channels (4, 8 or
 * 16); a key's outlier channels become symmetric 8-bit integers with one scale per key,
 * scale = max |x_c| / 127 over them and q_c = x_c / scale rounded to nearest even (fp32
 * arithmetic; an all-zero outlier part gives scale 0 and q 0); the key with its outlier channels
 * set to zero is coded by TurboQuant_mse at d = 128 exactly as tq_encode codes a whole key.  The
 * reconstruction takes the rest channels from that code and x_c = scale * q_c on the outlier
 * channels; 3 rest bits with 8 outliers is 3.5 bits per channel plus 64 bits of norms and scale. */

/* Outlier sets of H KV heads: outliers_host [H, n_o] int32, each row n_o distinct channels in
 * [0, 128), in any order.  The handle keeps, on the current device, each head's rest mask and
 * its outlier channels in ascending order: slot k of a key's 8-bit part is the head's k-th
 * smallest outlier channel.  d must be 128.  Errors: TQ_EINVAL (null pointers, H < 1, a repeated
 * or out-of-range channel), TQ_EUNSUPPORTED (d != 128, n_o not 4, 8 or 16), TQ_EDEVICE. */
tq_status tq_make_outlier8(int H, int d, int n_o, const int32_t* outliers_host, tq_outlier8_t* out);
void tq_outlier8_free(tq_outlier8_t o);

/* Encode of keys x_dev [B, H, T, 128] (dtype dt, 16-byte aligned) with the outlier sets `o`:
 * rest receives the TurboQuant_mse code of every key with its outlier channels zeroed (ROWS
 * layout, d = 128, bits = cb->b, n = B*H*T; norms = ||x_rest||), q8_dev [n, n_o] int8 the
 * outlier values in slot order and scale_dev [n] fp32 their scales.  The rest code's index
 * decisions follow tq_encode's.  Errors: TQ_EINVAL (null pointers, negative sizes, misaligned
 * x), TQ_ESHAPE (o's head count != H, cb / rot / rest with d != 128, n or bits mismatch, rest in
 * prod mode), TQ_EUNSUPPORTED (dtype, layout, n >= 2^31), TQ_EDEVICE. */
tq_status tq_encode_outlier8(const void* x_dev, tq_dtype dt, int B, int H, int64_t T, tq_outlier8_t o,
                             tq_codebook_t cb, tq_rotation_t rot, tq_packed* rest, int8_t* q8_dev,
                             float* scale_dev, void* stream);

/* Workspace bytes of tq_scores_outlier8: the score prologue of tq_scores plus the queries'
 * outlier components, B*Hq*16 fp32. */
size_t tq_scores_outlier8_workspace(int B, int Hq);
/* Raw scores <q, x_hat> of queries q_dev [B, Hq, 128] fp32 against outlier-8 keys (rest, q8_dev,
 * scale_dev as written by tq_encode_outlier8 for [B, Hkv, T]) into scores_dev [B, Hq, T] fp32:
 * s <R q_rest, C[idx]> + scale <q_O, q8>, with q_rest the query restricted to the rest channels
 * and q_O its outlier components, both taken through the outlier set of the query head's KV head
 * h // (Hq / Hkv) ([SB] fused score kernel and GQA mapping).  The first term runs on the same
 * fp16 matrix-core path as tq_scores, the second in fp32.  Errors: as tq_encode_outlier8 for the
 * keys and handles; TQ_ESHAPE (Hq not a positive multiple of Hkv); TQ_EUNSUPPORTED (GQA ratio as
 * tq_scores); TQ_ENOMEM (workspace). */
tq_status tq_scores_outlier8(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_outlier8_t o,
                             const tq_packed* rest, const int8_t* q8_dev, const float* scale_dev,
                             tq_codebook_t cb, tq_rotation_t rot, float* scores_dev, void* ws_dev,
                             size_t ws_bytes, void* stream);

/* Workspace bytes of tq_decode_attn_outlier8: tq_decode_attn's plus the queries' outlier
 * components (B*Hq*16 fp32). */
size_t tq_decode_attn_outlier8_workspace(int B, int Hq, int Hkv, int64_t T);
/* Fused decode attention with outlier-8 keys ([RQ] chapter 1: softmax(q K^T / sqrt(d)) V, and the
 * asymmetric K/V needs: K with outlier channels at 8 bits, V at fewer bits): as tq_decode_attn,
 * with the logit of key t for query head h equal to scale * (s_t <R q_rest, C_K[idx_t]> +
 * scale_t <q_O, q8_t>), q_rest and q_O taken through the outlier set of h's KV head.  K, q8_dev,
 * scale_dev: outlier-8 keys of [B, Hkv, T] as written by tq_encode_outlier8 (K: ROWS, MSE, d = 128,
 * bits = cb_k->b); V: TOKEN_BLOCKED MSE values of [B, Hkv, T]; out_dev [B, Hq, 128] fp32.
 * (K bits, V bits) must be one of tq_decode_attn's pairs; GQA ratio 1, 2 or 4; T >= 1.  Errors:
 * as tq_encode_outlier8 for the keys and handles, as tq_decode_attn otherwise; TQ_ENOMEM
 * (workspace); TQ_EDEVICE for a bit pair without a kernel. */
tq_status tq_decode_attn_outlier8(const float* q_dev, int B, int Hq, int Hkv, int64_t T, tq_outlier8_t o,
                                  const tq_packed* K, const int8_t* q8_dev, const float* scale_dev,
                                  const tq_packed* V, tq_codebook_t cb_k, tq_codebook_t cb_v,
                                  tq_rotation_t rot_k, tq_rotation_t rot_v, float scale, float* out_dev,
                                  void* ws_dev, size_t ws_bytes, void* stream);

/* Workspace bytes tq_search_topk needs for nq queries against n database vectors of length d
 * with k results per query (query operands, one chunk of scores, the running top-k). */
size_t tq_search_workspace(int64_t nq, int64_t n, int d, int k);
/* Maximum inner-product search over a TurboQuant_prod database ([FP] inner-product bias and the
 * QJL fix; [TQ] TurboQuant_prod estimator; [FP] deployment: vector retrieval with the encoder
 * as one matmul and a lookup).  For each query q_dev[i] (fp32 [nq, d]) the score of database
 * vector j is s_j <R q, C[idx_j]> + gamma_j sqrt(pi/2)/d <S q, z_j>, and the k largest scores
 * are written in descending order to top_s_dev [nq, k] fp32 with their indices to
 * top_i_dev [nq, k] int64; equal scores order by the smaller index.  If n < k the tail holds
 * -inf and index -1.  db: ROWS layout, prod mode, d a multiple of 128 in [128, 4096];
 * 1 <= k <= 32.  ws_dev: at least tq_search_workspace(nq, n, d, k) bytes.
 * Errors: TQ_EINVAL (null pointers, k out of range), TQ_ESHAPE (d mismatch), TQ_EUNSUPPORTED
 * (layout, mode or d), TQ_ENOMEM (workspace). */
tq_status tq_search_topk(const float* q_dev, int64_t nq, const tq_packed* db, tq_codebook_t cb,
                         tq_rotation_t rot, tq_qjl_t qjl, int k, float* top_s_dev,
                         int64_t* top_i_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* Kernel timers, for measurement tools (not part of the method).  tq_timer_arm makes the next
 * launch of the d = 128 rows-layout encode kernel on the calling thread (by tq_encode, or
 * tq_rotate at d = 128) attach a pair of HIP events to the kernel's dispatch, so that the
 * interval covers that kernel's execution alone (not the queue's own dispatch latency); other
 * calls leave the timer armed.  Returns a timer
 * id in [0, TQ_MAX_TIMERS), or -1 (TQ_ENOMEM in tq_last_error when every timer is in use,
 * TQ_EDEVICE when no events can be created).  tq_timer_read waits for that kernel and writes
 * its duration in milliseconds to *ms; TQ_EINVAL for an id that was not armed and launched.
 * tq_timer_reset releases every timer (the events are kept for reuse). */
#define TQ_MAX_TIMERS 256
int tq_timer_arm(void);
tq_status tq_timer_read(int id, float* ms);
void tq_timer_reset(void);
/* Kernels a timer can be attached to.  ENCODE: the d = 128 rows-layout encode kernel (what
 * tq_timer_arm arms).  SCORES: the d = 128 score kernel launched by tq_scores, tq_scores_prepared or
 * tq_scores_cache (not the query prologue before it).  One timer per kind can be armed at a time
 * on a thread; arming a kind again replaces the armed timer of that kind.  Returns as tq_timer_arm;
 * TQ_EINVAL in tq_last_error (and -1) for an unknown kind. */
typedef enum tq_timed_kernel { TQ_TIMED_ENCODE = 0, TQ_TIMED_SCORES = 1 } tq_timed_kernel;
int tq_timer_arm_kernel(tq_timed_kernel which);

/* ---- measurement ceilings (not part of the method) -----------------------------------
 * Kernels that give the achievable rates the roofline fractions are read against.
 * tq_peak_read: a streaming read of `bytes` (a multiple of 16) from src_dev by `blocks` blocks of
 *   256 threads (grid-stride, four 16-byte loads in flight per thread); nothing is written
 *   (sink_dev may be NULL: the kernel takes it but never stores to it).
 * tq_peak_copy: the same pattern copying src_dev to dst_dev (`bytes` read and written).
 * tq_peak_mfma: `blocks` blocks of 4 waves; each wave advances independent MFMA accumulator chains
 *   `iters` times (8 chains of v_mfma_f32_16x16x32 or 4 chains of v_mfma_f32_32x32x16): kind 0 =
 *   16x16x32 bf16, 1 = 32x32x16 bf16, 2 = 16x16x32 f16, 3 = 32x32x16 f16.  Every instruction is
 *   16384 (16x16x32) or 32768 (32x32x16) flops; out_dev receives blocks * 256 floats.
 * Errors: TQ_EINVAL (null buffers, bytes not a positive multiple of 16, blocks or iters < 1, bad
 * kind), TQ_EDEVICE. */
tq_status tq_peak_read(const void* src_dev, size_t bytes, int blocks, uint32_t* sink_dev, void* stream);
tq_status tq_peak_copy(void* dst_dev, const void* src_dev, size_t bytes, int blocks, void* stream);
tq_status tq_peak_mfma(int kind, int iters, int blocks, float* out_dev, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H_ */
