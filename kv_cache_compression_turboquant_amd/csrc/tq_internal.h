// Internal definitions shared by the host setup code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxBits = 4;
constexpr int kMaxCentroids = 1 << kMaxBits;
constexpr double kQjlConst = 1.2533141373155002512;  // sqrt(pi / 2)

// Codebook values handed to kernels by value (they live in the kernel argument segment).
struct CodebookArgs {
  float c[kMaxCentroids];  // centroids, fp32 rounded to nearest from fp64
  float t[kMaxCentroids];  // thresholds t[0 .. K-2]; t[K-1 ..] = +inf padding
  int bits;
  int sym;                 // 1 when exactly antisymmetric in fp32 (c[K-1-k] = -c[k], middle t = 0)
  // Sign-magnitude form used by the fused encode when sym: the K/2 - 1 positive thresholds as
  // their fp32 bit patterns and the K/2 non-negative centroids.
  int tpos[kMaxCentroids / 2];
  float cpos[kMaxCentroids / 2];
};

// MFMA A-operand fragments of a d x d matrix for the fused d = 128 kernels, bf16 bits.
// Element [pass][cb][s][lane][e] = M[32*(m/4) + 4*cb + (m%4)][32*g + 8*s + e],
// m = lane % 16, g = lane / 16; pass 0 = round-to-nearest bf16 of M, pass 1 = bf16 of the
// remainder.  Output block cb, lane group G and register r of the product then hold output
// coordinate 32*G + 4*cb + r (so one lane holds 32 consecutive output coordinates).
constexpr int kFragD = 128;
constexpr int kFragElems = 8 * 4 * 64 * 8;  // per pass, = 128 * 128

}  // namespace tq

struct tq_codebook_s {
  int d;
  int b;
  double c[tq::kMaxCentroids];
  double t[tq::kMaxCentroids];
  tq::CodebookArgs args;
};

struct tq_rotation_s {
  int d;
  int kind;                 // tq_rot_kind
  int device;
  uint64_t id;
  std::vector<double> r;    // fp64 R, row-major
  float* r32_dev = nullptr;       // fp32 R, row-major [d, d]
  float* rt32_dev = nullptr;      // fp32 R^T, row-major [d, d] (coalesced query rotation)
  uint16_t* frag_dev = nullptr;   // bf16 fragments [2][kFragElems] (d = 128 only)
  uint16_t* fragt_dev = nullptr;  // bf16 B-operand fragments of R^T [2][kFragElems] (d = 128):
                                  // [pass][cb][s][lane][e] = R[8*(lane%16) + cb][32*(lane/16) + 8s + e]
  uint16_t* gfrag_dev = nullptr;  // general-d GEMM (any d, d = 128 included): A fragments of R, one
                                  // (128 x 128) chunk per (output block ob, contraction block kc):
                                  // [ob][kc][pass 0..1][kFragElems], rows as in frag_dev, columns
                                  // 32 s + 8 g + e for instruction s of lane group g
  uint16_t* fragT_dev = nullptr;  // d = 128: A fragments of R^T, laid out as frag_dev (y = R^T x)
  uint16_t* frag32_dev = nullptr; // d = 128: A fragments for v_mfma_f32_32x32x16_bf16 [2][kFragElems]:
                                  // [pass][ob][s][lane][e] = R[o][c], i = lane % 32, j = lane / 32,
                                  // o = 64 ((i >> 2) & 1) + 16 ob + 4 (i >> 3) + (i & 3), c = 64 j + 8 s + e
  int passes = 2;                 // 1 when R is exactly representable after scaling
  float post_scale = 1.0f;        // y = post_scale * (fragments . x)
};

struct tq_qjl_s {
  int d;
  int device;
  uint64_t rot_id;
  std::vector<double> s;    // fp64 S, row-major
  float* s32_dev = nullptr;       // fp32 S, row-major [d, d]
  float* st32_dev = nullptr;      // fp32 S^T, row-major [d, d]
  uint16_t* frag_dev = nullptr;   // bf16 fragments of S' = S R^T [2][kFragElems] (d = 128)
  uint16_t* frag32_dev = nullptr; // S' as 32 x 32 x 16 fragments, laid out as tq_rotation_s::frag32_dev
  uint16_t* gfrag_dev = nullptr;  // general d: chunked A fragments of S', as tq_rotation_s::gfrag_dev
  float* sp32_dev = nullptr;      // d = 64: S' = S R^T in fp32, row-major [d, d]
};

namespace tq {

// Compute units of the current device (cached per device).
int num_cus();

// The event pair armed on this thread for kernel kind `which` (tq_timed_kernel), if any, handed
// to the next launch of that kind (and disarmed); false when none is armed.
bool take_armed_timer(int which, hipEvent_t* start, hipEvent_t* stop);
inline bool take_armed_timer(hipEvent_t* start, hipEvent_t* stop) {
  return take_armed_timer(TQ_TIMED_ENCODE, start, stop);
}

// Prefill attention over the caches after a chunk's append (tq_prefill128.hip): q [B, Hq, n_new,
// 128] fp32 -> out [B, Hq, n_new, 128] fp32; ws holds the rotated queries.
size_t prefill_attn_workspace_bytes(int B, int Hq, int64_t n_new);
hipError_t launch_prefill_attn(const float* q, int B, int Hq, int Hkv, int64_t n_new, int64_t pos, int64_t t_cap,
                               const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk,
                               const CodebookArgs& cbv, const tq_rotation_s* rot_k, const tq_rotation_s* rot_v,
                               float scale, float* out, void* ws, hipStream_t st);

// The static scratch of the allocation-free entry points (tq_noalloc.hip): its size, and the
// current device's address of it (looked up on the first call on each device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

// Measurement ceilings (tq_peaks.hip).
hipError_t launch_peak_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st);
hipError_t launch_peak_copy(void* dst, const void* src, int64_t bytes, int blocks, hipStream_t st);
hipError_t launch_peak_mfma(int kind, int iters, int blocks, float* out, hipStream_t st);

// Launchers (tq_encode128.hip, tq_misc.hip, tq_score128.hip, tq_attn128.hip).  All return the
// HIP error of the launch.
hipError_t launch_encode_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                              const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx,
                              float* norms, uint32_t* qjl_bits, float* rnorms, float* y_out,
                              hipStream_t st);
// TurboQuant_prod encode at d = 128 on the 32 x 32 x 16 matrix cores (tq_encode_prod128.hip).
hipError_t launch_encode_prod_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                   const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                   uint32_t* qjl_bits, float* rnorms, hipStream_t st);
// TurboQuant_mse encode at d = 128, rows layout, dense rotation, on the 32 x 32 x 16 matrix cores
// (tq_encode_mse32.hip).
hipError_t launch_encode_mse32_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                    const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st);
hipError_t launch_quantize_rotated(const float* y, int64_t n, int d, const CodebookArgs& cb,
                                   uint32_t* idx, hipStream_t st);
hipError_t launch_decode(const tq_packed* p, const CodebookArgs& cb, const tq_rotation_s* rot,
                         const tq_qjl_s* qjl, float* xhat, hipStream_t st);
// Head dims 64 and 256 on the KV side (rows layout throughout): scores of queries q [B, Hq, d] over
// packed keys at rows (b Hkv + g) rows + t; decode attention over packed K and V (MSE, rows layout,
// GQA ratio <= 8); the d = 64 encode (MSE, or prod with qjl).  Workspaces: kv_gen_query_bytes for
// the scores, attn_gen_workspace_bytes for the attention.
size_t kv_gen_query_bytes(int B, int Hq, int d);
size_t attn_gen_workspace_bytes(int B, int Hq, int Hkv, int64_t T, int d);
hipError_t launch_scores_gen(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                             const CodebookArgs& cb, const tq_rotation_s* rot, const tq_qjl_s* qjl, float* scores,
                             void* ws, hipStream_t st);
hipError_t launch_decode_attn_gen(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t rows, const tq_packed* K,
                                  const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                                  const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale, float* out,
                                  void* ws, hipStream_t st);
hipError_t launch_encode_d64(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                             const CodebookArgs& cb, uint32_t* idx, float* norms, uint32_t* qbits, float* rnorms,
                             hipStream_t st);
// y = R x (transpose: y = R^T x) for n rows of 128 at fp32 level (bf16 hi / lo passes), the product
// itself rather than unit coordinates; x fp32 or bf16, y fp32 [n, 128].
hipError_t launch_rotate_raw_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, bool transpose,
                                  float* y, hipStream_t st);

// TurboQuant_mse encode at d = 64 (rows layout) on the 32 x 32 x 16 matrix cores, R from rot->r32_dev.
hipError_t launch_encode_mse_d64(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                 const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st);
// TurboQuant_prod encode at d = 64 on the same matrix cores (cb: the (b-1)-bit stage), S' from
// qjl->sp32_dev.
hipError_t launch_encode_prod_d64(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                  const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                  uint32_t* qbits, float* rnorms, hipStream_t st);

// TurboQuant_mse encode at d = 128 (rows layout) for the randomized Hadamard rotations, as a
// fast Walsh-Hadamard transform in registers: full = true for H diag(sigma) / sqrt(128), false for
// blockdiag(H_32) diag(sigma) / sqrt(32); sigma_bits bit j set where sigma_j = -1; rscale = sqrt
// of the Hadamard size.  Needs a symmetric codebook (cb.sym).
hipError_t launch_encode_fwht_d128(const void* x, bool bf16, int64_t n, bool full, const uint32_t sigma_bits[4],
                                   float rscale, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                   hipStream_t st);
hipError_t launch_encode_vblock_d128(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot,
                                     const CodebookArgs& cb, uint32_t* idx, float* norms, hipStream_t st);
hipError_t launch_decode_attn(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                              const tq_packed* V, const CodebookArgs& cbk, const CodebookArgs& cbv,
                              const tq_rotation_s* rot_k, const tq_rotation_s* rot_v, float scale,
                              float* out, void* ws, hipStream_t st);
size_t decode_attn_workspace_bytes(int B, int Hq, int Hkv, int64_t T, int d);
hipError_t launch_scores(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* K,
                         const CodebookArgs& cb, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                         float* scores, void* ws, hipStream_t st);
size_t scores_workspace_bytes(int B, int Hq, int d);
// The two stages of launch_scores: the query prologue into ws, then the score kernel from ws.
hipError_t launch_prepare_queries(const float* q, int B, int Hq, int Hkv, const tq_rotation_s* rot,
                                  const tq_qjl_s* qjl, void* ws, hipStream_t st);
hipError_t launch_scores_prepared(int B, int Hq, int Hkv, int64_t T, const tq_packed* K, const CodebookArgs& cb,
                                  float* scores, const void* ws, hipStream_t st);
// General d (multiple of 128 in [256, 4096]), rows layout.  y_out set: rotated unit
// coordinates and norms only.  Prod (qjl set) stages the residual through ws in chunks.
hipError_t launch_encode_general(const void* x, bool bf16, int64_t n, int d, const tq_rotation_s* rot,
                                 const tq_qjl_s* qjl, const CodebookArgs& cb, uint32_t* idx, float* norms,
                                 uint32_t* qjl_bits, float* rnorms, float* y_out, void* ws, size_t ws_bytes,
                                 hipStream_t st);
size_t encode_general_ws_per_vector(int d);
constexpr int64_t kEncodeChunk = 131072;  // vectors per prod chunk at the default workspace size
constexpr int kGenVectors = 128;          // vectors per block of the general-d GEMM kernels

// Top-k inner-product search over a prod database (rows layout, d a multiple of 128).
size_t search_workspace_bytes(int64_t nq, int64_t n, int d, int k);
hipError_t launch_search_topk(const float* q, int64_t nq, const tq_packed* db, const CodebookArgs& cb,
                              const tq_rotation_s* rot, const tq_qjl_s* qjl, int k, float* top_s,
                              int64_t* top_i, void* ws, hipStream_t st);
constexpr int kSearchMaxK = 32;

// Keys whose outlier channels are kept as 8-bit integers (d = 128): per KV head a rest mask (bit
// c % 32 of word c / 32 set for a channel coded by TurboQuant_mse) and the head's NO outlier
// channels in ascending order, one per byte (word k holds channels 4 k .. 4 k + 3).
struct OutlierArgs {
  const uint32_t* mask = nullptr;   // [H][4]
  const uint32_t* chan = nullptr;   // [H][4]
  int8_t* q8 = nullptr;             // [n][NO] encode output
  float* scale = nullptr;           // [n] encode output
  uint32_t T = 1;                   // rows per sequence: row r belongs to KV head (r / T) % H
  uint32_t H = 1;
  int no = 0;                       // outlier channels per head: 4, 8 or 16
};
constexpr int kOutlierMaxChannels = 16;

// q_rot (and, with st_mat, the QJL sketch in sign-slot order plus the per-head constant) of
// every query head, d = 128, into the score workspace layout.  With oa.mask set, the query is
// restricted to the rest channels of its KV head first, and its outlier components (fp32, in
// the head's channel order) go to qo [B * Hq][16].
hipError_t launch_qprep128(const float* q, int B, int Hq, int Hkv, const float* rt, const float* st_mat,
                           uint16_t* qws, float* kconst, hipStream_t st, const OutlierArgs* oa = nullptr,
                           float* qo = nullptr);

// Outlier-8 keys (tq_encode128.hip, tq_score128.hip): x [n, 128] with n = sequences * oa.T, the
// rest channels TurboQuant_mse at cb.bits into idx / norms, the outlier channels into oa.q8 /
// oa.scale.  Scores: the score workspace followed by qo.
hipError_t launch_encode_outlier8(const void* x, bool bf16, int64_t n, const tq_rotation_s* rot, const CodebookArgs& cb,
                                  const OutlierArgs& oa, uint32_t* idx, float* norms, hipStream_t st);
size_t scores_outlier8_workspace_bytes(int B, int Hq);
// Decode attention with outlier-8 keys (tq_attn128.hip): the workspace of launch_decode_attn
// followed by qo.
size_t decode_attn_outlier8_workspace_bytes(int B, int Hq, int Hkv, int64_t T);
// Decode attention with split keys (tq_attn128.hip): the workspace of launch_decode_attn (its
// query region holds the fp32 rotated split queries).  (b_o, b_r) in {(3, 2), (4, 3)}.
hipError_t launch_decode_attn_split(const float* q, int B, int Hq, int Hkv, int64_t T, const tq_packed* Ko,
                                    const tq_packed* Kr, const tq_packed* V, const CodebookArgs& cbo,
                                    const CodebookArgs& cbr, const CodebookArgs& cbv, const int32_t* order,
                                    const float* rto, const float* rtr, const tq_rotation_s* rot_v, float scale,
                                    float* out, void* ws, hipStream_t st);
hipError_t launch_decode_attn_outlier8(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride,
                                       const tq_packed* K, const int8_t* q8, const float* oscale, const tq_packed* V,
                                       const CodebookArgs& cbk, const CodebookArgs& cbv, const tq_rotation_s* rot_k,
                                       const tq_rotation_s* rot_v, const OutlierArgs& oa, float scale, float* out,
                                       void* ws, hipStream_t st);
hipError_t launch_scores_outlier8(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride,
                                  const tq_packed* K, const int8_t* q8, const float* oscale, const CodebookArgs& cb,
                                  const tq_rotation_s* rot, const OutlierArgs& oa, float* scores, void* ws,
                                  hipStream_t st);

}  // namespace tq
