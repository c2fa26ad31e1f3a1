// Launchers of the outlier-channel split codes at d = 128 (tq_split128.hip): every key vector
// is two TurboQuant_mse codes of 64 channels each, the outlier channels at BO bits and the rest
// at BR bits, each with its own norm and its own 64 x 64 rotation.
#pragma once

#include "tq_internal.h"

namespace tq {

constexpr int kSplitD = 128;
constexpr int kSplitHalf = 64;
constexpr int kSplitMaxRatio = 64;   // query heads per KV head the score kernel takes

// order [H, 128] int32 on the device: per head, the outlier channels first, then the rest.
// x [B * H, T, 128] bf16 or fp32 (T tokens per sequence); the codes of token t of sequence s go
// to row s * out_stride + pos + t (out_stride = T, pos = 0 for a packed set; the capacity and the
// append position for a cache).  ro / rr: fp32 row-major 64 x 64 rotations, rto / rtr their
// transposes.  Up to 32 tokens per sequence run one fp32 block per token; more run the MFMA
// kernel on blocks of 512 tokens.
hipError_t launch_encode_split(const void* x, bool bf16, int64_t n_seq, int H, int64_t T, int64_t out_stride,
                               int64_t pos, const int32_t* order, const float* ro, const float* rr, const float* rto,
                               const float* rtr, const CodebookArgs& cbo, const CodebookArgs& cbr, uint32_t* idx_o,
                               float* norm_o, uint32_t* idx_r, float* norm_r, hipStream_t st);

// Rotated queries: qws [B * Hq, 128] fp32 with entries 0..63 = R_o q_O and 64..127 = R_r q_R,
// q_O and q_R gathered through the channel order of the query head's KV head.
hipError_t launch_qprep_split(const float* q, int B, int Hq, int Hkv, const int32_t* order, const float* rto,
                              const float* rtr, float* qws, hipStream_t st);

// Scores [B, Hq, T] from the rotated queries and the two codes of keys [B, Hkv, T], sequences
// seq_stride rows apart (T for a packed set, the capacity for a cache).
hipError_t launch_scores_split(const float* qws, int B, int Hq, int Hkv, int64_t T, int64_t seq_stride, int bo, int br,
                               const CodebookArgs& cbo, const CodebookArgs& cbr, const uint32_t* idx_o,
                               const float* norm_o, const uint32_t* idx_r, const float* norm_r, float* scores,
                               hipStream_t st);

}  // namespace tq
