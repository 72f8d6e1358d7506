// Attention of the draft batch over the paged KV cache.
//
// Every non-rejected slot at position q attends to positions [0, q] of its
// request: the cached prefix plus the slots written in this pass (all KV writes
// of a layer land before this kernel runs).  "P-EAGLE: parallel speculative
// decoding in vLLM", Architecture and mechanism, Step 2 (all positions go
// through the Transformer together) and vLLM implementation details, KV cache
// (rejected slots never wrote, so they are never read as their own slot).
//
// gfx950 design (bf16, head_dim 64)
//  * Work item = (request, KV chunk, KV head).  All S*G queries of one KV head
//    (S slots x G query heads of the group) share every K/V tile, so the item
//    streams its chunk once; chunk size is chosen on the device from the
//    batch's total context so that about `target_items` items exist
//    (split-KV), and a merge kernel combines the fp32 partials.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16:
//    a lane then holds 8 consecutive positions of one query, which is exactly
//    the B operand of O^T = V^T P^T, so the softmax stays in registers with no
//    LDS round trip.  The V cache is stored d-major inside each block
//    ([block][kv head][d][block_size]), so V^T fragments are plain 16-byte
//    loads as well.  K rows of a 16-position tile are permuted (row 4a+i of
//    tile t holds position 8a+4t+i) so that the two score tiles of a 32-position
//    step give each lane its 8 consecutive positions.
//  * Online softmax in base 2 with the scale folded in; P is rounded to bf16
//    for the PV product, the row sum uses the same rounded values.
#include "pe_common.h"
#include "pe_internal.h"

namespace pe {

constexpr int kMaxB = 1024;

// Orders this wave's LDS writes before its later LDS reads (and the reverse)
// without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Split-KV plan shared by the partial and merge kernels: total context ->
// chunk size CH (multiple of 32, >= 64); off[r] = first chunk of request r.
__device__ void attn_plan(const int32_t* seq_lens, int B, int Hkv, int target, int* off,
                          int& CH) {
  __shared__ long long s_tot[4];
  __shared__ int s_part[256];
  const int tid = threadIdx.x, nt = blockDim.x;  // nt == 256
  long long tot = 0;
  for (int r = tid; r < B; r += nt) tot += max(seq_lens[r], 0);
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
  if ((tid & 63) == 0) s_tot[tid >> 6] = tot;
  __syncthreads();
  tot = s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
  long long ch = (tot * Hkv + target - 1) / (target > 0 ? target : 1);
  ch = (ch + 31) / 32 * 32;
  if (ch < 64) ch = 64;
  if (ch > (1 << 30)) ch = 1 << 30;
  CH = int(ch);
  const int per = (B + nt - 1) / nt;
  const int r0 = tid * per;
  int sum = 0;
  for (int r = r0; r < min(B, r0 + per); ++r) sum += (max(seq_lens[r], 0) + CH - 1) / CH;
  s_part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < nt; o <<= 1) {
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int run = s_part[tid] - sum;
  for (int r = r0; r < min(B, r0 + per); ++r) {
    off[r] = run;
    run += (max(seq_lens[r], 0) + CH - 1) / CH;
  }
  if (tid == nt - 1) off[B] = s_part[nt - 1];
  __syncthreads();
}

long long attn_max_items(int B, int Hkv, int target_items) {
  return (long long)target_items + (long long)(B + 1) * Hkv;
}

__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  __shared__ int s_off[kMaxB + 1];
  __shared__ float s_ot[4][64][17];
  int CH;
  attn_plan(a.seq_lens, a.B, a.Hkv, a.target_items, s_off, CH);
  const int G = a.Hq / a.Hkv, QN = a.S * G, QT = (QN + 15) >> 4;
  const int total = s_off[a.B] * a.Hkv;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
  const float sl2 = a.scale * 1.4426950408889634f;
  const uint16_t* Q = (const uint16_t*)a.q;
  const uint16_t* Kc = (const uint16_t*)a.kcache;
  const uint16_t* Vc = (const uint16_t*)a.vcache;
  const int bs = a.block_size;
  const uint4 zero = {0u, 0u, 0u, 0u};

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int rc = item / a.Hkv, g = item - rc * a.Hkv;
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= rc) lo = mid; else hi = mid;
    }
    const int r = lo, chunk = rc - s_off[r];
    const int L = a.seq_lens[r];
    const int pb = chunk * CH, pe = min(L, pb + CH);
    const int32_t* btr = a.bt + (long long)r * a.max_blocks;

    for (int t = w; t < QT; t += 4) {
      const int q = t * 16 + c;
      bool qv = q < QN;
      const int s = qv ? q / G : 0, hh = qv ? q % G : 0, row = r * a.S + s;
      qv = qv && !a.rej[row];
      const int qpos = qv ? a.positions[row] : -1;
      uint4 qf[2];
      const uint16_t* qp = Q + ((long long)row * a.Hq + g * G + hh) * 64 + gq * 8;
      qf[0] = qv ? ld16(qp) : zero;
      qf[1] = qv ? ld16(qp + 32) : zero;
      float m = -INFINITY, lsum = 0.f;
      f32x4 o[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

      for (int p = pb; p < pe; p += 32) {
        uint4 kf[2][2];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          int pp = p + 8 * (c >> 2) + 4 * pt + (c & 3);
          pp = pp < L ? pp : L - 1;
          const long long slot = (long long)btr[pp / bs] * bs + pp % bs;
          const uint16_t* kp = Kc + (slot * a.Hkv + g) * 64 + gq * 8;
          kf[pt][0] = ld16(kp);
          kf[pt][1] = ld16(kp + 32);
        }
        const int pv0 = p + 8 * gq;
        const int pvc = pv0 < L ? pv0 : ((L - 1) & ~7);
        const long long blk = btr[pvc / bs];
        const uint16_t* vb = Vc + ((blk * a.Hkv + g) * 64) * bs + (pvc % bs);
        uint4 vf[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vf[dt] = ld16(vb + (long long)(c + 16 * dt) * bs);

        f32x4 st[2];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          st[pt] = mfma16(kf[pt][0], qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
          st[pt] = mfma16(kf[pt][1], qf[1], st[pt]);
        }
        // lane (gq, c): st[pt][i] is the score of position p + 8gq + 4pt + i for query c
        float v[8];
        float mloc = -INFINITY;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = pv0 + 4 * pt + i;
            const bool ok = qv && pos < pe && pos <= qpos;
            const float x = ok ? st[pt][i] * sl2 : -INFINITY;
            v[4 * pt + i] = x;
            mloc = fmaxf(mloc, x);
          }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float mnew = fmaxf(m, mloc);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2f(m - mref);
        uint32_t pk[4];
        float ps = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint16_t b0 = f2bf(exp2f(v[2 * jj] - mref));
          const uint16_t b1 = f2bf(exp2f(v[2 * jj + 1] - mref));
          ps += bf2f(b0) + bf2f(b1);
          pk[jj] = uint32_t(b0) | (uint32_t(b1) << 16);
        }
        lsum = lsum * alpha + ps;
        m = mnew;
        const uint4 pf = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          o[dt] = o[dt] * alpha;
          o[dt] = mfma16(vf[dt], pf, o[dt]);
        }
      }
      lsum += __shfl_xor(lsum, 16, 64);
      lsum += __shfl_xor(lsum, 32, 64);

      // O^T lane (gq, c): o[dt][i] = O[q = c][d = 16dt + 4gq + i]; transpose via LDS
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_ot[w][16 * dt + 4 * gq + i][c] = o[dt][i];
      wave_lds_sync();  // s_ot[w] is private to this wave; waves run different tile counts
      {
        const int qq = l >> 2, d0 = (l & 3) * 16;
        const int qg = t * 16 + qq;
        if (qg < QN) {
          float* dst = a.part_o + ((long long)item * QN + qg) * 64 + d0;
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            float4 f;
            f.x = s_ot[w][d0 + 4 * v4 + 0][qq];
            f.y = s_ot[w][d0 + 4 * v4 + 1][qq];
            f.z = s_ot[w][d0 + 4 * v4 + 2][qq];
            f.w = s_ot[w][d0 + 4 * v4 + 3][qq];
            *reinterpret_cast<float4*>(dst + 4 * v4) = f;
          }
        }
        if (gq == 0 && q < QN) {
          a.part_ml[((long long)item * QN + q) * 2 + 0] = m;
          a.part_ml[((long long)item * QN + q) * 2 + 1] = lsum;
        }
      }
      wave_lds_sync();
    }
  }
}

__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  __shared__ int s_off[kMaxB + 1];
  int CH;
  attn_plan(a.seq_lens, a.B, a.Hkv, a.target_items, s_off, CH);
  const int G = a.Hq / a.Hkv, QN = a.S * G;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const long long total = (long long)a.B * a.S * a.Hq;
  uint16_t* out = (uint16_t*)a.out;
  for (long long x = (long long)blockIdx.x * 4 + w; x < total; x += (long long)gridDim.x * 4) {
    const int row = int(x / a.Hq), h = int(x % a.Hq);
    const int r = row / a.S, s = row % a.S, g = h / G, q = s * G + (h % G);
    uint16_t* dst = out + (long long)row * a.Hq * 64 + h * 64 + l;
    if (a.rej[row] || a.seq_lens[r] <= 0) { *dst = 0; continue; }
    const int c0 = s_off[r], nc = s_off[r + 1] - c0;
    float M = -INFINITY;
    for (int ch = 0; ch < nc; ++ch)
      M = fmaxf(M, a.part_ml[((long long)((c0 + ch) * a.Hkv + g) * QN + q) * 2]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY)
      for (int ch = 0; ch < nc; ++ch) {
        const long long it = (long long)(c0 + ch) * a.Hkv + g;
        const float mc = a.part_ml[(it * QN + q) * 2];
        const float wgt = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
        Lsum += wgt * a.part_ml[(it * QN + q) * 2 + 1];
        O += wgt * a.part_o[(it * QN + q) * 64 + l];
      }
    *dst = f2bf(Lsum > 0.f ? O / Lsum : 0.f);
  }
}

// fp32, any head_dim <= 128: one 64-thread workgroup per (slot, query head),
// threads stride over positions with their own online softmax, then combine.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int MAXD = 128;
  __shared__ float s_q[MAXD];
  __shared__ float s_m[64], s_l[64];
  __shared__ float s_o[64][MAXD + 1];
  const int row = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq, tid = threadIdx.x;
  const int r = row / a.S, G = a.Hq / a.Hkv, g = h / G, hd = a.hd;
  float* dst = (float*)a.out + (long long)row * a.Hq * hd + h * hd;
  const int L = a.seq_lens[r];
  if (a.rej[row] || L <= 0) {
    for (int d = tid; d < hd; d += 64) dst[d] = 0.f;
    return;
  }
  const int qpos = min(a.positions[row], L - 1);
  const float* Qr = (const float*)a.q + ((long long)row * a.Hq + h) * hd;
  for (int d = tid; d < hd; d += 64) s_q[d] = Qr[d];
  __syncthreads();
  const float* Kc = (const float*)a.kcache;
  const float* Vc = (const float*)a.vcache;
  const int32_t* btr = a.bt + (long long)r * a.max_blocks;
  const int bs = a.block_size;
  float m = -INFINITY, lsum = 0.f, o[MAXD];
  for (int d = 0; d < hd; ++d) o[d] = 0.f;
  for (int p = tid; p <= qpos; p += 64) {
    const long long blk = btr[p / bs], off = p % bs, slot = blk * bs + off;
    const float* kp = Kc + (slot * a.Hkv + g) * hd;
    float sc = 0.f;
    for (int d = 0; d < hd; ++d) sc = fmaf(s_q[d], kp[d], sc);
    sc *= a.scale;
    const float mn = fmaxf(m, sc);
    const float al = expf(m - mn), pw = expf(sc - mn);
    lsum = lsum * al + pw;
    const float* vp = Vc + ((blk * a.Hkv + g) * hd) * bs + off;
    for (int d = 0; d < hd; ++d) o[d] = o[d] * al + pw * vp[(long long)d * bs];
    m = mn;
  }
  s_m[tid] = m;
  s_l[tid] = lsum;
  for (int d = 0; d < hd; ++d) s_o[tid][d] = o[d];
  __syncthreads();
  float M = -INFINITY;
  for (int t = 0; t < 64; ++t) M = fmaxf(M, s_m[t]);
  for (int d = tid; d < hd; d += 64) {
    float Ls = 0.f, O = 0.f;
    for (int t = 0; t < 64; ++t) {
      const float wgt = (s_m[t] == -INFINITY) ? 0.f : expf(s_m[t] - M);
      Ls += wgt * s_l[t];
      O += wgt * s_o[t][d];
    }
    dst[d] = O / Ls;
  }
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (dtype == 0) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.B * a.S * a.Hq), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(attn_partial_kernel, dim3(a.grid), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  long long waves = (long long)a.B * a.S * a.Hq;
  long long blocks = (waves + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pe
