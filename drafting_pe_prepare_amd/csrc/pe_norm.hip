// RMSNorm: y = x / sqrt(mean(x^2) + eps) * gain, fp32 arithmetic, one
// workgroup per output row, 16-byte loads.  The drafter is a pre-norm
// Transformer ("P-EAGLE: parallel speculative decoding in vLLM", Architecture
// and mechanism: N-layer Transformer, then the LM head); the final norm runs
// only on the draft rows that feed the LM head.
#include "pe_common.h"
#include "pe_internal.h"

namespace pe {

// The row's chunks and the gain's stay in registers between the two passes
// (NCH per thread; a row of more than 256 * NCH chunks takes the loop again).
// expand_k > 0: row i is compact row i of a MASK-deduplicated first layer,
// and its raw chunks are also written to its slots of the full layout in
// x_full (one slot, or the request's K-1 MASK slots for its last compact row).
template <typename T, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_kernel(int d, const T* __restrict__ x,
                                                      const T* __restrict__ gain,
                                                      T* __restrict__ out,
                                                      const int32_t* __restrict__ rows_idx,
                                                      int rows_bound, float eps,
                                                      T* __restrict__ x_full = nullptr, int expand_k = 0,
                                                      bool scatter = false) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
  const int i = blockIdx.x;
  int src = rows_idx ? rows_idx[i] : i;
  if (src < 0 || src >= rows_bound) {
    if (scatter) return;  // no row to write
    src = 0;
  }
  const T* xr = x + (long long)src * d;
  T* yr = out + (long long)(scatter ? src : i) * d;
  const int nc = d / V;
  uint4 xs[NCH], gs[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    // unconditional loads (past the row's end: its last chunk, unused), so
    // that all of them are in flight together
    const int c = min(threadIdx.x + j * 256, nc - 1);
    xs[j] = ld16(xr + c * V);
    gs[j] = ld16(gain + c * V);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c < nc) {
      const T* e = reinterpret_cast<const T*>(&xs[j]);
#pragma unroll
      for (int q = 0; q < V; ++q) { float v = Elt<T>::ld(e + q); ss += v * v; }
    }
  }
  for (int c = threadIdx.x + NCH * 256; c < nc; c += 256) {
    uint4 raw = ld16(xr + c * V);
    const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int q = 0; q < V; ++q) { float v = Elt<T>::ld(e + q); ss += v * v; }
  }
  if (expand_k > 0) {
    const int K = expand_k, r = i / (K + 2), j = i - r * (K + 2);
    const int s0 = r * 2 * K + j, ns = j == K + 1 ? K - 1 : 1;
    for (int t = 0; t < ns; ++t) {
      T* xf = x_full + (long long)(s0 + t) * d;
#pragma unroll
      for (int jj = 0; jj < NCH; ++jj) {
        const int c = threadIdx.x + jj * 256;
        if (c < nc) *reinterpret_cast<uint4*>(xf + c * V) = xs[jj];
      }
      for (int c = threadIdx.x + NCH * 256; c < nc; c += 256) *reinterpret_cast<uint4*>(xf + c * V) = ld16(xr + c * V);
    }
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float rs = rsqrtf(tot / float(d) + eps);
  auto emit = [&](int c, const uint4& raw, const uint4& gr) {
    uint4 o;
    const T* e = reinterpret_cast<const T*>(&raw);
    const T* g = reinterpret_cast<const T*>(&gr);
    T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int q = 0; q < V; ++q) Elt<T>::st(oe + q, Elt<T>::ld(e + q) * rs * Elt<T>::ld(g + q));
    *reinterpret_cast<uint4*>(yr + c * V) = o;
  };
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c < nc) emit(c, xs[j], gs[j]);
  }
  for (int c = threadIdx.x + NCH * 256; c < nc; c += 256) emit(c, ld16(xr + c * V), ld16(gain + c * V));
}

hipError_t launch_rmsnorm(int dtype, int rows, int d, const void* x, const void* gain, void* out,
                          const int32_t* rows_idx, int rows_bound, float eps, hipStream_t st, bool scatter) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((rmsnorm_kernel<uint16_t, 2>), dim3(rows), dim3(256), 0, st, d,
                       (const uint16_t*)x, (const uint16_t*)gain, (uint16_t*)out, rows_idx,
                       rows_bound, eps, (uint16_t*)nullptr, 0, scatter);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<float, 2>), dim3(rows), dim3(256), 0, st, d, (const float*)x,
                       (const float*)gain, (float*)out, rows_idx, rows_bound, eps, (float*)nullptr, 0, scatter);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_expand(int rows, int d, const void* x, const void* gain, void* out, void* x_full,
                                 int K, float eps, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (K < 2 || rows % (K + 2)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rmsnorm_kernel<uint16_t, 2>), dim3(rows), dim3(256), 0, st, d, (const uint16_t*)x,
                     (const uint16_t*)gain, (uint16_t*)out, nullptr, rows, eps, (uint16_t*)x_full, K);
  return hipGetLastError();
}

}  // namespace pe
