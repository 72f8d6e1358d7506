// Verification by rejection sampling ("vLLM Speculators: parallel drafting for
// speculative decoding", Production integration: verification by rejection
// sampling keeps the verifier's output distribution).  With p_j =
// softmax(y_j / T) the verifier's rows and q_j = softmax(z_j / T) the
// drafter's, draft t_j is kept while U_j < min(1, p_j(t_j) / q_j(t_j)); at the
// first rejection j the emitted token is a draw from max(0, p_j - q_j)
// (normalised), after K kept drafts a draw from p_K.  Draws are Gumbel-max:
// argmax_v(log w(v) + G_v), G = -log(-log U), U from Philox4x32-10 (pe_common.h).
//
// gfx950 design: the step is bound by reading the fp32 logit rows (B (2K+1)
// rows of V floats).  Four launches: (1) one workgroup per row computes
// log-sum-exp of logit / T with 16-byte loads and a fixed reduction order;
// (2) one lane per request runs the sequential acceptance test (2 logits per
// draft); (3) kSampleParts workgroups per request score their slice of the
// emitting row and keep the best (value, index) key; (4) one wave per request
// reduces the keys.
#include <cmath>

#include "pe_common.h"
#include "pe_internal.h"

namespace pe {

// row rho < B*K: drafter row rho; else verifier row rho - B*K
__global__ __launch_bounds__(256) void lse_rows_kernel(int BK, int V, float inv_temp,
                                                       const float* __restrict__ zq,
                                                       const float* __restrict__ zp,
                                                       float* __restrict__ lse) {
  const int rho = blockIdx.x;
  const float* row = rho < BK ? zq + (long long)rho * V : zp + (long long)(rho - BK) * V;
  float m = -INFINITY, s = 0.f;
  auto add = [&](float x) {
    x *= inv_temp;
    if (x == -INFINITY) return;
    if (x > m) {
      s = s * expf(m - x) + 1.f;
      m = x;
    } else {
      s += expf(x - m);
    }
  };
  const int n4 = V >> 2;
  for (int c = threadIdx.x; c < n4; c += blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(row)[c];
    add(v.x); add(v.y); add(v.z); add(v.w);
  }
  for (int c = (n4 << 2) + threadIdx.x; c < V; c += blockDim.x) add(row[c]);
  // (m, s) pairs: wave, then workgroup, in a fixed order
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    const float mn = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
    m = mn;
  }
  __shared__ float sm[4], ss[4];
  if ((threadIdx.x & 63) == 0) { sm[threadIdx.x >> 6] = m; ss[threadIdx.x >> 6] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int w = 1; w < int(blockDim.x >> 6); ++w) {
      const float mn = fmaxf(M, sm[w]);
      S = (M == -INFINITY ? 0.f : S * expf(M - mn)) + (sm[w] == -INFINITY ? 0.f : ss[w] * expf(sm[w] - mn));
      M = mn;
    }
    lse[rho] = M + logf(S);
  }
}

// one lane per request: the first rejected draft (K when every draft is kept)
__global__ __launch_bounds__(64) void accept_kernel(int B, int K, int V, float inv_temp,
                                                    const int32_t* __restrict__ tokens,
                                                    const float* __restrict__ zq,
                                                    const float* __restrict__ zp,
                                                    const float* __restrict__ lse,
                                                    const uint64_t* __restrict__ seedp,
                                                    int32_t* __restrict__ accepted) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B) return;
  const uint64_t seed = *seedp;
  int a = K;
  for (int j = 0; j < K; ++j) {
    const int t = tokens[(long long)r * K + j];
    if (t < 0 || t >= V) { a = j; break; }  // a padded request's drafts (-1) are never kept
    const long long qi = (long long)r * K + j, pi = (long long)r * (K + 1) + j;
    const float lq = zq[qi * V + t] * inv_temp - lse[qi];
    const float lp = zp[pi * V + t] * inv_temp - lse[(long long)B * K + pi];
    const float ratio = expf(lp - lq);
    const float u = philox_uniform(uint32_t(j), uint32_t(r), RNG_ACCEPT, seed);
    if (!(u < fminf(1.f, ratio))) { a = j; break; }
  }
  accepted[r] = a;
}

// workgroup (part, r): best Gumbel-perturbed score over its slice of the row
// request r emits from
__global__ __launch_bounds__(256) void emit_scores_kernel(int B, int K, int V, float inv_temp,
                                                          const float* __restrict__ zq,
                                                          const float* __restrict__ zp,
                                                          const float* __restrict__ lse,
                                                          const int32_t* __restrict__ accepted,
                                                          const uint64_t* __restrict__ seedp,
                                                          uint64_t* __restrict__ keys) {
  const int part = blockIdx.x, r = blockIdx.y;
  const uint64_t seed = *seedp;
  const int a = accepted[r];
  const long long pi = (long long)r * (K + 1) + a, qi = (long long)r * K + a;
  const float* yp = zp + pi * V;
  const float lsp = lse[(long long)B * K + pi];
  const bool residual = a < K;
  const float* yq = residual ? zq + qi * V : yp;
  const float lsq = residual ? lse[qi] : 0.f;
  const int v0 = int((long long)V * part / gridDim.x), v1 = int((long long)V * (part + 1) / gridDim.x);
  uint64_t best = 0ull;
  for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
    const float lp = yp[v] * inv_temp - lsp;
    float score;
    if (residual) {
      const float w = expf(lp) - expf(yq[v] * inv_temp - lsq);
      score = w > 0.f ? logf(w) : -INFINITY;
    } else {
      score = lp;
    }
    score += gumbel_noise(philox_uniform(uint32_t(v), uint32_t(r), RNG_RESIDUAL, seed));
    const uint64_t k = argmax_key(score, v);
    best = k > best ? k : best;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t k = (uint64_t(__shfl_xor(uint32_t(best >> 32), o, 64)) << 32) |
                       uint64_t(__shfl_xor(uint32_t(best), o, 64));
    best = k > best ? k : best;
  }
  __shared__ uint64_t sb[4];
  if ((threadIdx.x & 63) == 0) sb[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x >> 6); ++w) best = sb[w] > best ? sb[w] : best;
    best = sb[0] > best ? sb[0] : best;
    keys[(long long)r * gridDim.x + part] = best;
  }
}

__global__ __launch_bounds__(64) void emit_pick_kernel(int P, const uint64_t* __restrict__ keys,
                                                       int32_t* __restrict__ next_tokens) {
  const int r = blockIdx.x, l = threadIdx.x;
  uint64_t best = 0ull;
  for (int p = l; p < P; p += 64) best = keys[(long long)r * P + p] > best ? keys[(long long)r * P + p] : best;
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t k = (uint64_t(__shfl_xor(uint32_t(best >> 32), o, 64)) << 32) |
                       uint64_t(__shfl_xor(uint32_t(best), o, 64));
    best = k > best ? k : best;
  }
  if (l == 0) next_tokens[r] = argmax_key_index(best);
}

hipError_t launch_verify_sampled(int B, int K, int V, float inv_temp, const int32_t* draft_tokens,
                                 const float* draft_logits, const float* target_logits,
                                 const uint64_t* seed, float* lse, uint64_t* keys,
                                 int32_t* accepted, int32_t* next_tokens, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(lse_rows_kernel, dim3(unsigned(B * (2 * K + 1))), dim3(256), 0, st, B * K, V, inv_temp,
                     draft_logits, target_logits, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3(unsigned((B + 63) / 64)), dim3(64), 0, st, B, K, V, inv_temp,
                     draft_tokens, draft_logits, target_logits, lse, seed, accepted);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_scores_kernel, dim3(unsigned(kSampleParts), unsigned(B)), dim3(256), 0, st, B, K, V,
                     inv_temp, draft_logits, target_logits, lse, accepted, seed, keys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_pick_kernel, dim3(unsigned(B)), dim3(64), 0, st, kSampleParts, keys, next_tokens);
  return hipGetLastError();
}

}  // namespace pe
