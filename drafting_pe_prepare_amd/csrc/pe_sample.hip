// Stochastic drafting and verification by rejection sampling ("vLLM
// Speculators: parallel drafting for speculative decoding", Production
// integration: verification by rejection sampling keeps the verifier's output
// distribution).  With p_j = softmax(y_j / T) the verifier's rows and q_j =
// softmax(z_j / T) the drafter's, draft t_j is kept while
// U_j < min(1, p_j(t_j) / q_j(t_j)); at the first rejection j the emitted
// token is a draw from max(0, p_j - q_j) (normalised), after K kept drafts a
// draw from p_K.  Draws are Gumbel-max, argmax_v(log w(v) + G_v) with
// G = -log(-log U), U from Philox4x32-10 (pe_common.h).
//
// Drafts are drawn the same way from the logit rows the LM head wrote (its
// fused greedy argmax stays untouched): up to kSampleParts workgroups per row keep
// their slice's best Gumbel-perturbed key, one wave per row picks the winner.
//
// gfx950 design: everything here is bound by reading fp32 logit rows.  Every
// thread takes groups of 4 consecutive tokens: one 16-byte load per row and
// one Philox block (4 words) per group.  Verification: (1) up to kLseParts
// workgroups per row reduce (max, sum exp) of a slice, (2) one thread per row
// combines them in a fixed order, (3) one wave per request runs the K
// acceptance tests at once (the first failing one decides), (4) up to kSampleParts
// workgroups per request score their slice of the emitting row, (5) one wave
// per request reduces the keys.
#include <cmath>

#include "pe_common.h"
#include "pe_internal.h"

namespace pe {

__device__ __forceinline__ uint64_t shfl_xor_key(uint64_t v, int o) {
  return (uint64_t(__shfl_xor(uint32_t(v >> 32), o, 64)) << 32) | uint64_t(__shfl_xor(uint32_t(v), o, 64));
}

// best key of a 256-thread workgroup -> keys[slot]
__device__ __forceinline__ void block_best_key(uint64_t best, uint64_t* keys, long long slot) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t k = shfl_xor_key(best, o);
    best = k > best ? k : best;
  }
  __shared__ uint64_t sb[4];
  if ((threadIdx.x & 63) == 0) sb[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x >> 6); ++w) best = sb[w] > best ? sb[w] : best;
    best = sb[0] > best ? sb[0] : best;
    keys[slot] = best;
  }
}

// token groups [g0, g1) of slice `part` of P over V/4 groups
__device__ __forceinline__ void slice_groups(int V, int part, int P, int& g0, int& g1) {
  const int ng = V >> 2;
  g0 = int((long long)ng * part / P);
  g1 = int((long long)ng * (part + 1) / P);
}

// ---------------------------------------------------------------------------
// drafting: workgroup (part, row) keeps the best perturbed logit / T
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void draft_scores_kernel(int V, int ldl, float inv_temp,
                                                           const float* __restrict__ logits,
                                                           const uint64_t* __restrict__ seedp,
                                                           uint64_t* __restrict__ keys) {
  const int part = blockIdx.x, row = blockIdx.y;
  const uint64_t seed = *seedp;
  const float* z = logits + (long long)row * ldl;
  int g0, g1;
  slice_groups(V, part, gridDim.x, g0, g1);
  uint64_t best = 0ull;
#pragma unroll 4
  for (int g = g0 + threadIdx.x; g < g1; g += blockDim.x) {
    const float4 zv = *reinterpret_cast<const float4*>(z + 4 * g);
    const Words4 x = philox4(uint32_t(g), uint32_t(row), RNG_DRAFT, seed);
    const float zz[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float score = zz[e] * inv_temp + gumbel_noise(word_uniform(x.w[e]));
      const uint64_t k = argmax_key(score, 4 * g + e);
      best = k > best ? k : best;
    }
  }
  block_best_key(best, keys, (long long)row * gridDim.x + part);
}

__global__ __launch_bounds__(64) void pick_kernel(int P, int Kd, const uint64_t* __restrict__ keys,
                                                  int32_t* __restrict__ tokens, int tstride,
                                                  const int32_t* __restrict__ seq_lens) {
  const int row = blockIdx.x, l = threadIdx.x;
  uint64_t best = 0ull;
  for (int p = l; p < P; p += 64) best = keys[(long long)row * P + p] > best ? keys[(long long)row * P + p] : best;
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t k = shfl_xor_key(best, o);
    best = k > best ? k : best;
  }
  if (l == 0) tokens[(long long)row * tstride] = (seq_lens && seq_lens[row / Kd] == 0) ? -1 : argmax_key_index(best);
}

// slices per row: about 2048 workgroups per launch, between lo and hi
static int parts_for(int rows, int lo, int hi) {
  const int p = 2048 / (rows > 0 ? rows : 1);
  return p < lo ? lo : (p > hi ? hi : p);
}

hipError_t launch_sample_drafts(int M, int Kd, int V, int ldl, float inv_temp, const float* logits,
                                const uint64_t* seed, uint64_t* keys, int32_t* tokens, int tstride,
                                const int32_t* seq_lens, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (V % 4 || ldl % 4) return hipErrorInvalidValue;
  const int P = parts_for(M, 4, kSampleParts);
  hipLaunchKernelGGL(draft_scores_kernel, dim3(unsigned(P), unsigned(M)), dim3(256), 0, st, V, ldl, inv_temp,
                     logits, seed, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pick_kernel, dim3(unsigned(M)), dim3(64), 0, st, P, Kd, keys, tokens, tstride, seq_lens);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// verification
// ---------------------------------------------------------------------------
// (max, sum exp) of logit / T over slice `part` of row rho (rho < BK: drafter
// row rho, else verifier row rho - BK) -> part_ms[(rho * kLseParts + part) * 2]
__global__ __launch_bounds__(256) void lse_parts_kernel(int BK, int V, float inv_temp,
                                                        const float* __restrict__ zq,
                                                        const float* __restrict__ zp,
                                                        float* __restrict__ part_ms) {
  const int part = blockIdx.x, rho = blockIdx.y;
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
  auto merge = [&](float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = (m == -INFINITY ? 0.f : s * expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
    m = mn;
  };
  int g0, g1;
  slice_groups(V, part, gridDim.x, g0, g1);
#pragma unroll 4
  for (int g = g0 + threadIdx.x; g < g1; g += blockDim.x) {
    const float4 v = *reinterpret_cast<const float4*>(row + 4 * g);
    add(v.x); add(v.y); add(v.z); add(v.w);
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    merge(m2, s2);
  }
  __shared__ float sm[4], ss[4];
  if ((threadIdx.x & 63) == 0) { sm[threadIdx.x >> 6] = m; ss[threadIdx.x >> 6] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0]; s = ss[0];
    for (int w = 1; w < int(blockDim.x >> 6); ++w) merge(sm[w], ss[w]);
    part_ms[((long long)rho * kLseParts + part) * 2] = m;
    part_ms[((long long)rho * kLseParts + part) * 2 + 1] = s;
  }
}

__device__ __forceinline__ float row_lse(const float* __restrict__ part_ms, long long rho, int P) {
  float m = -INFINITY, s = 0.f;
  for (int p = 0; p < P; ++p) {
    const float m2 = part_ms[(rho * kLseParts + p) * 2], s2 = part_ms[(rho * kLseParts + p) * 2 + 1];
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) continue;
    s = (m == -INFINITY ? 0.f : s * expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mn));
    m = mn;
  }
  return m + logf(s);
}

// one thread per row: the slices' (max, sum exp) combined in a fixed order
__global__ __launch_bounds__(256) void lse_combine_kernel(int rows, int P, const float* __restrict__ part_ms,
                                                          float* __restrict__ lse) {
  const int rho = blockIdx.x * blockDim.x + threadIdx.x;
  if (rho < rows) lse[rho] = row_lse(part_ms, rho, P);
}

// one wave per request, lane j < K tests draft j (all tests at once; the
// first failing one decides): the first rejected draft, K when every draft is
// kept
__global__ __launch_bounds__(64) void accept_kernel(int B, int K, int V, float inv_temp,
                                                    const int32_t* __restrict__ tokens,
                                                    const float* __restrict__ zq,
                                                    const float* __restrict__ zp,
                                                    const float* __restrict__ lse,
                                                    const uint64_t* __restrict__ seedp,
                                                    int32_t* __restrict__ accepted) {
  const int r = blockIdx.x, j = threadIdx.x;
  const long long BK = (long long)B * K;
  bool reject = false;
  if (j < K) {
    const uint64_t seed = *seedp;
    const int t = tokens[(long long)r * K + j];
    if (t < 0 || t >= V) {
      reject = true;  // a padded request's drafts (-1) are never kept
    } else {
      const long long qi = (long long)r * K + j, pi = (long long)r * (K + 1) + j;
      const float lq = zq[qi * V + t] * inv_temp - lse[qi];
      const float lp = zp[pi * V + t] * inv_temp - lse[BK + pi];
      const float ratio = expf(lp - lq);
      const float u = word_uniform(philox4(uint32_t(j), uint32_t(r), RNG_ACCEPT, seed).w[0]);
      reject = !(u < fminf(1.f, ratio));
    }
  }
  const unsigned long long m = __ballot(reject);
  if (j == 0) accepted[r] = m ? (__ffsll((long long)m) - 1) : K;
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
  int g0, g1;
  slice_groups(V, part, gridDim.x, g0, g1);
  uint64_t best = 0ull;
#pragma unroll 4
  for (int g = g0 + threadIdx.x; g < g1; g += blockDim.x) {
    const float4 pv = *reinterpret_cast<const float4*>(yp + 4 * g);
    const float4 qv = *reinterpret_cast<const float4*>(yq + 4 * g);
    const float pp[4] = {pv.x, pv.y, pv.z, pv.w}, qq[4] = {qv.x, qv.y, qv.z, qv.w};
    const Words4 x = philox4(uint32_t(g), uint32_t(r), RNG_RESIDUAL, seed);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lp = pp[e] * inv_temp - lsp;
      float score;
      if (residual) {
        const float w = expf(lp) - expf(qq[e] * inv_temp - lsq);
        score = w > 0.f ? logf(w) : -INFINITY;
      } else {
        score = lp;
      }
      score += gumbel_noise(word_uniform(x.w[e]));
      const uint64_t k = argmax_key(score, 4 * g + e);
      best = k > best ? k : best;
    }
  }
  block_best_key(best, keys, (long long)r * gridDim.x + part);
}

hipError_t launch_verify_sampled(int B, int K, int V, float inv_temp, const int32_t* draft_tokens,
                                 const float* draft_logits, const float* target_logits,
                                 const uint64_t* seed, float* lse, float* part_ms, uint64_t* keys,
                                 int32_t* accepted, int32_t* next_tokens, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (V % 4) return hipErrorInvalidValue;
  const int rows = B * (2 * K + 1), PL = parts_for(rows, 2, kLseParts), PE = parts_for(B, 4, kSampleParts);
  hipLaunchKernelGGL(lse_parts_kernel, dim3(unsigned(PL), unsigned(rows)), dim3(256), 0, st, B * K, V, inv_temp,
                     draft_logits, target_logits, part_ms);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lse_combine_kernel, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st, rows, PL, part_ms,
                     lse);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3(unsigned(B)), dim3(64), 0, st, B, K, V, inv_temp, draft_tokens,
                     draft_logits, target_logits, lse, seed, accepted);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_scores_kernel, dim3(unsigned(PE), unsigned(B)), dim3(256), 0, st, B, K, V, inv_temp,
                     draft_logits, target_logits, lse, accepted, seed, keys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pick_kernel, dim3(unsigned(B)), dim3(64), 0, st, PE, 1, keys, next_tokens, 1, nullptr);
  return hipGetLastError();
}

}  // namespace pe
