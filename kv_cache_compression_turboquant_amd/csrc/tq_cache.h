// Launchers of the streaming KV cache (tq_cache128.hip) and the capacity-strided forms of the
// score and decode-attention launchers (tq_score128.hip, tq_attn128.hip).
#pragma once

#include "tq_internal.h"

namespace tq {

// Appends of n_new tokens per sequence shorter than this go through the per-token kernel alone;
// longer ones (prefill) run the fused MFMA encode kernels on their whole blocks.
constexpr int64_t kAppendFusedMin = 64;

// Encodes x [n_seq, n_new, 128] (bf16 or fp32) into rows pos .. pos + n_new - 1 of every sequence
// of a cache whose sequence s owns rows [s t_cap, (s + 1) t_cap).  qjl set: prod (rows layout).
hipError_t launch_cache_append(const void* x, bool bf16, int64_t n_seq, int64_t n_new, int64_t pos, int64_t t_cap,
                               const tq_rotation_s* rot, const tq_qjl_s* qjl, const CodebookArgs& cb,
                               const tq_packed* cache, hipStream_t st);

// One decode step's (or any append's) keys xk and values xv [n_seq, n_new, 128] into a key cache
// (rows layout, MSE) and a value cache (token-blocked, MSE) of the same geometry; short appends
// run both caches in one launch.
hipError_t launch_kv_append(const void* xk, const void* xv, bool bf16, int64_t n_seq, int64_t n_new, int64_t pos,
                            int64_t t_cap, const tq_rotation_s* rk, const tq_rotation_s* rv, const CodebookArgs& cbk,
                            const CodebookArgs& cbv, const tq_packed* K, const tq_packed* V, hipStream_t st);

// Scores and decode attention over the first T rows of every sequence, sequences seq_stride rows
// apart (seq_stride = T for a packed [B, Hkv, T] set; the capacity for a cache).
hipError_t launch_scores_strided(int B, int Hq, int Hkv, int64_t T, int64_t seq_stride, const tq_packed* K,
                                 const CodebookArgs& cb, float* scores, const void* ws, hipStream_t st);
hipError_t launch_decode_attn_strided(const float* q, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride,
                                      const tq_packed* K, const tq_packed* V, const CodebookArgs& cbk,
                                      const CodebookArgs& cbv, const tq_rotation_s* rot_k, const tq_rotation_s* rot_v,
                                      float scale, float* out, void* ws, hipStream_t st);

}  // namespace tq
