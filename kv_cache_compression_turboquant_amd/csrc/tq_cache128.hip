// Streaming compressed KV cache at d = 128: append the keys and values of new tokens to a
// preallocated packed cache ("TurboQuant 详解", the KV-cache example: each decode step appends
// the new token's K/V to the end of the cache at once; prefill writes the prompt's compressed
// K/V; the following section: no online fitting, only rotation, lookup and packing).
#include <algorithm>

#include "tq_cache.h"
#include "tq_device.h"

namespace tq {
namespace {

// ---------------------------------------------------------------------------------------
// Per-token append: one block of 128 threads per (token, sequence), thread j owning coordinate
// j.  s = ||x|| and y_j = (R x)_j / s in fp32 (R^T read coalesced, x from LDS), idx_j = #{k :
// y_j >= t_k}.  Rows layout: the row's words are assembled in LDS and stored whole.  Token-
// blocked layout: the token shares its words with the other 31 tokens of its block, so each
// field is cleared and set with two atomic operations on disjoint bits, which leaves every other
// field intact whatever else runs concurrently.  Prod (rows only): r = s (y - C[idx]) is the
// residual in the rotated domain, gamma = ||r||, and z = sign(S R^T r), again from fp32 matrices
// read coalesced (the transposed ones where the sum runs over rows).
// ---------------------------------------------------------------------------------------
template <int BITS, bool PROD, bool BLOCKED, bool BF16IN>
__device__ __forceinline__ void append_token(
    const void* __restrict__ x, int64_t x_tokens, int64_t x_first, int64_t pos, int64_t t_cap,
    const float* __restrict__ rt32, const float* __restrict__ r32, const float* __restrict__ st32, const CodebookArgs& cb,
    uint32_t* __restrict__ idx, float* __restrict__ norms, uint32_t* __restrict__ qbits, float* __restrict__ rnorms) {
  constexpr int W = 4 * BITS;  // words per row
  __shared__ float va[128], vb[128];
  __shared__ float red[2][2];
  __shared__ uint32_t words[W];
  const int j = threadIdx.x;
  const int lane = j & 63, wave = j >> 6;
  const int64_t seq = blockIdx.y;
  const int64_t t = blockIdx.x;
  const int64_t src = (seq * x_tokens + x_first + t) * 128 + j;
  const int64_t row = seq * t_cap + pos + t;
  const float xv = BF16IN ? bf16_val(static_cast<const uint16_t*>(x)[src]) : static_cast<const float*>(x)[src];
  // sum over the block; slot selects the reduction buffer so consecutive sums need no extra barrier
  auto block_sum = [&](float v, int slot) -> float {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[slot][wave] = v;
    __syncthreads();
    return red[slot][0] + red[slot][1];
  };
  // (m v)_j with m read column-wise (m[i * 128 + j]) and v in LDS: the thread's 128 loads are all
  // issued before the first product, so the sum waits out one memory latency, not one per batch.
  auto column_dot = [&](const float* __restrict__ m, const float* v) -> float {
    float c[128];
#pragma unroll
    for (int i = 0; i < 128; ++i) c[i] = m[i * 128 + j];
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 128; ++i) a = fmaf(c[i], v[i], a);
    return a;
  };
  va[j] = xv;
  if (!BLOCKED && j < W) words[j] = 0u;
  const float s = sqrtf(block_sum(xv * xv, 0));  // (its barrier also publishes va and words)
  const float acc = column_dot(rt32, va);
  const float y = s > 0.f ? acc / s : 0.f;
  const uint32_t k = bucketize<BITS>(y, cb);

  if constexpr (BLOCKED) {
    // chunk (octet o, coordinate j) at chunk position o * 128 + j, 8 * BITS bits per chunk,
    // token e of the octet at chunk bits [BITS e, BITS e + BITS)
    const int within = (int)(row & 31);
    const int p = (((within >> 3) * 128 + j) * 8 + (within & 7)) * BITS;
    uint32_t* blk = idx + (row >> 5) * (128 * BITS);
    const int w = p >> 5, sh = p & 31;
    const uint32_t m = (1u << BITS) - 1u;
    atomicAnd(&blk[w], ~(m << sh));
    atomicOr(&blk[w], k << sh);
    if (sh + BITS > 32) {
      atomicAnd(&blk[w + 1], ~(m >> (32 - sh)));
      atomicOr(&blk[w + 1], k >> (32 - sh));
    }
  } else {
    const int p = j * BITS, w = p >> 5, sh = p & 31;
    atomicOr(&words[w], k << sh);
    if (sh + BITS > 32) atomicOr(&words[w + 1], k >> (32 - sh));
  }
  if (j == 0) norms[row] = s;

  if constexpr (PROD) {
    const float r = s * (y - cb.c[k]);
    vb[j] = r;
    const float gamma = sqrtf(block_sum(r * r, 1));  // (publishes vb)
    const float ro = column_dot(r32, vb);  // (R^T r)_j: the residual in the original domain
    va[j] = ro;      // every thread finished reading va in the rotation (barrier above)
    __syncthreads();
    const float pr = column_dot(st32, va);  // (S r)_j
    const uint64_t z = __ballot(pr >= 0.f);
    if (lane == 0) {
      qbits[row * 4 + 2 * wave] = (uint32_t)z;
      qbits[row * 4 + 2 * wave + 1] = (uint32_t)(z >> 32);
    }
    if (j == 0) rnorms[row] = gamma;
  }
  if constexpr (!BLOCKED) {
    __syncthreads();
    if (j < W) idx[row * W + j] = words[j];
  }
}

template <int BITS, bool PROD, bool BLOCKED, bool BF16IN>
__global__ __launch_bounds__(128) void k_cache_append_d128(
    const void* __restrict__ x, int64_t x_tokens, int64_t x_first, int64_t pos, int64_t t_cap,
    const float* __restrict__ rt32, const float* __restrict__ r32, const float* __restrict__ st32, CodebookArgs cb,
    uint32_t* __restrict__ idx, float* __restrict__ norms, uint32_t* __restrict__ qbits, float* __restrict__ rnorms) {
  append_token<BITS, PROD, BLOCKED, BF16IN>(x, x_tokens, x_first, pos, t_cap, rt32, r32, st32, cb, idx, norms, qbits,
                                            rnorms);
}

// One decode step's key and value appends in one launch: blockIdx.z = 0 appends to the key cache
// (rows layout, MSE), 1 to the value cache (token-blocked, MSE); the two halves run side by side.
template <int KB, int VB, bool BF16IN>
__global__ __launch_bounds__(128) void k_kv_append_d128(
    const void* __restrict__ xk, const void* __restrict__ xv, int64_t x_tokens, int64_t pos, int64_t t_cap,
    const float* __restrict__ rtk, const float* __restrict__ rtv, CodebookArgs cbk, CodebookArgs cbv,
    uint32_t* __restrict__ kidx, float* __restrict__ knorms, uint32_t* __restrict__ vidx, float* __restrict__ vnorms) {
  if (blockIdx.z == 0)
    append_token<KB, false, false, BF16IN>(xk, x_tokens, 0, pos, t_cap, rtk, nullptr, nullptr, cbk, kidx, knorms,
                                           nullptr, nullptr);
  else
    append_token<VB, false, true, BF16IN>(xv, x_tokens, 0, pos, t_cap, rtv, nullptr, nullptr, cbv, vidx, vnorms,
                                          nullptr, nullptr);
}

template <int KB, int VB>
hipError_t kv_append_small(const void* xk, const void* xv, bool bf16, int64_t n_seq, int64_t n_new, int64_t pos,
                           int64_t t_cap, const tq_rotation_s* rk, const tq_rotation_s* rv, const CodebookArgs& cbk,
                           const CodebookArgs& cbv, const tq_packed* K, const tq_packed* V, hipStream_t st) {
  const dim3 grid((unsigned)n_new, (unsigned)n_seq, 2);
  if (bf16)
    hipLaunchKernelGGL((k_kv_append_d128<KB, VB, true>), grid, dim3(128), 0, st, xk, xv, n_new, pos, t_cap,
                       rk->rt32_dev, rv->rt32_dev, cbk, cbv, K->idx, K->norms, V->idx, V->norms);
  else
    hipLaunchKernelGGL((k_kv_append_d128<KB, VB, false>), grid, dim3(128), 0, st, xk, xv, n_new, pos, t_cap,
                       rk->rt32_dev, rv->rt32_dev, cbk, cbv, K->idx, K->norms, V->idx, V->norms);
  return hipGetLastError();
}

template <int BITS, bool PROD, bool BLOCKED>
hipError_t append_small(const void* x, bool bf16, int64_t n_seq, int64_t x_tokens, int64_t x_first, int64_t count,
                        int64_t pos, int64_t t_cap, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                        const CodebookArgs& cb, const tq_packed* c, hipStream_t st) {
  const dim3 grid((unsigned)count, (unsigned)n_seq);
  const float* st32 = PROD ? qjl->st32_dev : nullptr;
  uint32_t* qb = PROD ? c->qjl : nullptr;
  float* rn = PROD ? c->rnorms : nullptr;
  if (bf16)
    hipLaunchKernelGGL((k_cache_append_d128<BITS, PROD, BLOCKED, true>), grid, dim3(128), 0, st, x, x_tokens, x_first,
                       pos, t_cap, rot->rt32_dev, rot->r32_dev, st32, cb, c->idx, c->norms, qb, rn);
  else
    hipLaunchKernelGGL((k_cache_append_d128<BITS, PROD, BLOCKED, false>), grid, dim3(128), 0, st, x, x_tokens, x_first,
                       pos, t_cap, rot->rt32_dev, rot->r32_dev, st32, cb, c->idx, c->norms, qb, rn);
  return hipGetLastError();
}

template <int BITS>
hipError_t append_small_dispatch(const void* x, bool bf16, int64_t n_seq, int64_t x_tokens, int64_t x_first,
                                 int64_t count, int64_t pos, int64_t t_cap, const tq_rotation_s* rot,
                                 const tq_qjl_s* qjl, const CodebookArgs& cb, const tq_packed* c, hipStream_t st) {
  if (c->layout == TQ_LAYOUT_TOKEN_BLOCKED)
    return append_small<BITS, false, true>(x, bf16, n_seq, x_tokens, x_first, count, pos, t_cap, rot, qjl, cb, c, st);
  if (qjl)
    return append_small<BITS, true, false>(x, bf16, n_seq, x_tokens, x_first, count, pos, t_cap, rot, qjl, cb, c, st);
  return append_small<BITS, false, false>(x, bf16, n_seq, x_tokens, x_first, count, pos, t_cap, rot, qjl, cb, c, st);
}

// Tokens [x_first, x_first + count) of every sequence of x into cache positions pos + x_first ...
hipError_t append_range(const void* x, bool bf16, int64_t n_seq, int64_t n_new, int64_t x_first, int64_t count,
                        int64_t pos, int64_t t_cap, const tq_rotation_s* rot, const tq_qjl_s* qjl,
                        const CodebookArgs& cb, const tq_packed* c, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const int64_t p = pos + x_first;
  switch (cb.bits) {
    case 1: return append_small_dispatch<1>(x, bf16, n_seq, n_new, x_first, count, p, t_cap, rot, qjl, cb, c, st);
    case 2: return append_small_dispatch<2>(x, bf16, n_seq, n_new, x_first, count, p, t_cap, rot, qjl, cb, c, st);
    case 3: return append_small_dispatch<3>(x, bf16, n_seq, n_new, x_first, count, p, t_cap, rot, qjl, cb, c, st);
    case 4: return append_small_dispatch<4>(x, bf16, n_seq, n_new, x_first, count, p, t_cap, rot, qjl, cb, c, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kv_append(const void* xk, const void* xv, bool bf16, int64_t n_seq, int64_t n_new, int64_t pos,
                            int64_t t_cap, const tq_rotation_s* rk, const tq_rotation_s* rv, const CodebookArgs& cbk,
                            const CodebookArgs& cbv, const tq_packed* K, const tq_packed* V, hipStream_t st) {
  if (n_new >= kAppendFusedMin) {
    // long appends: each cache on its own (fused encode kernels on whole rows and blocks)
    hipError_t e = launch_cache_append(xk, bf16, n_seq, n_new, pos, t_cap, rk, nullptr, cbk, K, st);
    if (e != hipSuccess) return e;
    return launch_cache_append(xv, bf16, n_seq, n_new, pos, t_cap, rv, nullptr, cbv, V, st);
  }
#define TQ_KVA(KB_, VB_) \
  if (cbk.bits == KB_ && cbv.bits == VB_) \
    return kv_append_small<KB_, VB_>(xk, xv, bf16, n_seq, n_new, pos, t_cap, rk, rv, cbk, cbv, K, V, st);
  TQ_KVA(2, 2) TQ_KVA(4, 4) TQ_KVA(3, 3) TQ_KVA(4, 2) TQ_KVA(2, 4) TQ_KVA(3, 2) TQ_KVA(4, 3)
  TQ_KVA(1, 1) TQ_KVA(2, 3) TQ_KVA(3, 4)
#undef TQ_KVA
  // other bit pairs: one launch per cache
  hipError_t e = launch_cache_append(xk, bf16, n_seq, n_new, pos, t_cap, rk, nullptr, cbk, K, st);
  if (e != hipSuccess) return e;
  return launch_cache_append(xv, bf16, n_seq, n_new, pos, t_cap, rv, nullptr, cbv, V, st);
}

hipError_t launch_cache_append(const void* x, bool bf16, int64_t n_seq, int64_t n_new, int64_t pos, int64_t t_cap,
                               const tq_rotation_s* rot, const tq_qjl_s* qjl, const CodebookArgs& cb,
                               const tq_packed* c, hipStream_t st) {
  const bool blocked = c->layout == TQ_LAYOUT_TOKEN_BLOCKED;
  const size_t esize = bf16 ? 2 : 4;
  // Long appends: the fused encode kernels write whole rows (rows layout) or whole token blocks
  // (token-blocked layout; the partial blocks at either end go through the per-token kernel, so
  // that the other tokens sharing them keep their fields).
  int64_t head = n_new, mid = 0;
  if (n_new >= kAppendFusedMin) {
    head = blocked ? std::min<int64_t>((32 - pos % 32) % 32, n_new) : 0;
    mid = blocked ? (n_new - head) / 32 * 32 : n_new;
  }
  hipError_t e = append_range(x, bf16, n_seq, n_new, 0, head, pos, t_cap, rot, qjl, cb, c, st);
  if (e != hipSuccess) return e;
  if (mid > 0) {
    const int W = 4 * cb.bits;
    for (int64_t s = 0; s < n_seq; ++s) {
      const void* xs = static_cast<const char*>(x) + (size_t)((s * n_new + head) * 128) * esize;
      const int64_t row = s * t_cap + pos + head;
      if (blocked)
        e = launch_encode_vblock_d128(xs, bf16, mid, rot, cb, c->idx + (row / 32) * (int64_t)(128 * cb.bits),
                                      c->norms + row, st);
      else
        e = launch_encode_d128(xs, bf16, mid, rot, qjl, cb, c->idx + row * W, c->norms + row,
                               qjl ? c->qjl + row * 4 : nullptr, qjl ? c->rnorms + row : nullptr, nullptr, st);
      if (e != hipSuccess) return e;
    }
  }
  return append_range(x, bf16, n_seq, n_new, head + mid, n_new - head - mid, pos, t_cap, rot, qjl, cb, c, st);
}

}  // namespace tq
