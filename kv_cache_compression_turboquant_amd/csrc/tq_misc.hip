// Reference quantizer (bucketize + pack of given rotated coordinates) and the decoder
// x_hat = s R^T C[idx] (+ the QJL term), any d.
#include "tq_device.h"

namespace tq {
namespace {

// ---------------------------------------------------------------------------------------
// Reference quantizer: bucketize + pack fp32 rotated coordinates, one thread per
// (row, 32-coordinate group).
// ---------------------------------------------------------------------------------------
template <int BITS>
__global__ void k_quantize_rotated(const float* __restrict__ y, int64_t n, int d, CodebookArgs cb,
                                   uint32_t* __restrict__ out) {
  const int groups = d / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * groups) return;
  const int64_t row = i / groups;
  const int grp = (int)(i % groups);
  const f32x4* src = reinterpret_cast<const f32x4*>(y + row * d + 32 * grp);
  uint32_t idx[32];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f32x4 v = src[k];
#pragma unroll
    for (int j = 0; j < 4; ++j) idx[4 * k + j] = bucketize<BITS>(v[j], cb);
  }
  uint32_t w[BITS];
  pack32<BITS>(idx, w);
  uint32_t* dst = out + row * ((int64_t)d * BITS / 32) + BITS * grp;
#pragma unroll
  for (int j = 0; j < BITS; ++j) dst[j] = w[j];
}

// ---------------------------------------------------------------------------------------
// Decode: x_hat = s R^T C[idx] (+ gamma sqrt(pi/2)/d S^T z).  One block per row.
// ---------------------------------------------------------------------------------------
__global__ void k_decode(const uint32_t* __restrict__ idx, const float* __restrict__ norms,
                         const uint32_t* __restrict__ qbits, const float* __restrict__ rnorms, int d,
                         int bits, int blocked, CodebookArgs cb, const float* __restrict__ r32,
                         const float* __restrict__ s32, float* __restrict__ out) {
  extern __shared__ float sh[];  // [d] centroid values, [d] signs
  const int64_t row = blockIdx.x;
  const int words = d * bits / 32;
  const uint32_t* w = blocked ? idx + (row >> 5) * (int64_t)d * bits : idx + row * words;
  const int e32 = (int)(row & 31);
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    // stream bit of coordinate j: rows layout b*j; blocked: chunk (octet, j), row e within it
    const int p = blocked ? ((e32 >> 3) * d + j) * 8 * bits + bits * (e32 & 7) : j * bits;
    uint64_t win = w[p >> 5];
    if ((p & 31) + bits > 32) win |= (uint64_t)w[(p >> 5) + 1] << 32;
    const uint32_t id = (uint32_t)(win >> (p & 31)) & ((1u << bits) - 1u);
    sh[j] = cb.c[id];
    if (s32) sh[d + j] = ((qbits[row * (d / 32) + (j >> 5)] >> (j & 31)) & 1u) ? 1.f : -1.f;
  }
  __syncthreads();
  const float s = norms[row];
  const float gc = s32 ? rnorms[row] * kQjl / (float)d : 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float a = 0.f, b = 0.f;
    for (int j = 0; j < d; ++j) a += r32[(int64_t)j * d + i] * sh[j];
    if (s32)
      for (int j = 0; j < d; ++j) b += s32[(int64_t)j * d + i] * sh[d + j];
    out[row * d + i] = s * a + gc * b;
  }
}

}  // namespace

// Compute units of the current device, cached per device.
static int g_num_cus[64] = {0};

int num_cus() {
  int dev = 0;
  hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) return 256;
  if (!g_num_cus[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_num_cus[dev] = v;
  }
  return g_num_cus[dev];
}

hipError_t launch_quantize_rotated(const float* y, int64_t n, int d, const CodebookArgs& cb,
                                   uint32_t* idx, hipStream_t st) {
  const int64_t work = n * (d / 32);
  const int threads = 256;
  const dim3 grid((unsigned)((work + threads - 1) / threads));
  switch (cb.bits) {
    case 1: hipLaunchKernelGGL(k_quantize_rotated<1>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    case 2: hipLaunchKernelGGL(k_quantize_rotated<2>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    case 3: hipLaunchKernelGGL(k_quantize_rotated<3>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    case 4: hipLaunchKernelGGL(k_quantize_rotated<4>, grid, dim3(threads), 0, st, y, n, d, cb, idx); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const tq_packed* p, const CodebookArgs& cb, const tq_rotation_s* rot,
                         const tq_qjl_s* qjl, float* xhat, hipStream_t st) {
  const int d = p->d;
  const int threads = d < 256 ? d : 256;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)p->n), dim3(threads), 2 * d * sizeof(float), st, p->idx, p->norms,
                     qjl ? p->qjl : nullptr, qjl ? p->rnorms : nullptr, d, p->bits,
                     p->layout == TQ_LAYOUT_TOKEN_BLOCKED ? 1 : 0, cb, rot->r32_dev,
                     qjl ? qjl->s32_dev : nullptr, xhat);
  return hipGetLastError();
}

}  // namespace tq
