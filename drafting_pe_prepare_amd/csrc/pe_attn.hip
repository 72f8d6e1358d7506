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
//  * Stream = (request, KV head): all S*G queries of one KV head (S slots x G
//    query heads of the group) share every K/V tile, so a stream is read
//    once.  The streams' 64-position steps are laid end to end and cut into
//    equal contiguous ranges, one per workgroup (split-KV); a workgroup runs
//    each stream piece of its range and writes fp32 partials, and a merge
//    kernel combines a stream's pieces.  Equal ranges keep every workgroup
//    equally busy whatever the mix of context lengths.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16:
//    a lane then holds 8 consecutive positions of one query, which is exactly
//    the B operand of O^T = V^T P^T, so the softmax stays in registers with no
//    LDS round trip.  The V cache is stored d-major inside each block
//    ([block][kv head][d][block_size]), so V^T fragments are plain 16-byte
//    loads as well.  K rows of a 16-position tile are permuted (row 4a+i of
//    tile t holds position 8a+4t+i) so that the two score tiles of a 32-position
//    step give each lane its 8 consecutive positions.
//  * Online softmax in base 2 with the scale folded in.  The PV product takes
//    P as the sum of two bf16 values (hi, and the rounded remainder) on two
//    MFMAs, so P enters with ~16 significant bits; a single bf16 rounding of
//    P alone moves the logits by up to ~2% of their RMS on small drafters.
//    The row sum adds the fp32 values.
#include "pe_common.h"
#include "pe_internal.h"

#ifndef PE_ATTN_MIN_STEPS
#define PE_ATTN_MIN_STEPS 2  // shortest range per workgroup (64-position steps)
#endif
#ifndef PE_ATTN_LAZY
#define PE_ATTN_LAZY 1
#endif

namespace pe {

constexpr int kMaxB = kAttnMaxB;
// Largest excess (base 2) of a score over the running max that leaves the
// max in place as the exponent's reference (p up to 2^8).
constexpr float kLazyMax = 8.f;

// Orders this wave's LDS writes before its later LDS reads (and the reverse)
// without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Steps of one stream of a request with context L: 64-position steps,
// rounded up to a multiple of PE_ATTN_MIN_STEPS so that short ranges start
// on stream boundaries (a range that straddled two streams would pay the
// fixed cost of a piece twice); a padded step past L is empty.
__device__ __forceinline__ int attn_steps(int L) {
  const int n = (max(L, 0) + 63) >> 6;
  return (n + PE_ATTN_MIN_STEPS - 1) / PE_ATTN_MIN_STEPS * PE_ATTN_MIN_STEPS;
}

// Step plan: off[r] = steps of the requests before r (one KV head), off[B] =
// the total.  Any blockDim that is a multiple of 64 and <= 512.
__device__ void attn_plan(const int32_t* seq_lens, int B, int* off) {
  __shared__ int s_wsum[8];
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wid = tid >> 6;
  // thread tid owns requests [r0, r1)
  const int per = (B + nt - 1) / nt, r0 = min(B, tid * per), r1 = min(B, r0 + per);
  int sum = 0;
  for (int r = r0; r < r1; ++r) sum += attn_steps(seq_lens[r]);
  // block-wide exclusive prefix of the step counts: a shuffle scan inside
  // each wave, then the totals of the waves before it
  int inc = sum;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_wsum[wid] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += s_wsum[w];
  int run = base + inc - sum;
  for (int r = r0; r < r1; ++r) {
    off[r] = run;
    run += attn_steps(seq_lens[r]);
  }
  if (tid == nt - 1) off[B] = base + inc;
  __syncthreads();
}

// Workgroups that get a range: all of the grid, but no range shorter than
// PE_ATTN_MIN_STEPS steps (each piece pays a fixed cost: queries, block ids,
// DMA ramp-up), and never more than the steps (so every workgroup's range is
// non-empty and a stream's pieces are consecutive workgroups).
__device__ __forceinline__ int attn_ranges(long long P, int grid) {
  const long long g = P / PE_ATTN_MIN_STEPS;
  return int(g < 1 ? 1 : (g < grid ? g : grid));
}

// Stream s = r*Hkv + g covers global steps [Hkv*off[r] + g*n_r, ... + n_r),
// n_r = off[r+1] - off[r]; workgroup w of Gw covers [ceil(w P / Gw),
// ceil((w+1) P / Gw)), so step x lies in workgroup floor(x Gw / P).  The
// piece of stream s in workgroup w has partial index s + w, so a stream's
// pieces are consecutive and at most B*Hkv + Gw partials exist.
long long attn_max_items(int B, int Hkv, int grid) { return (long long)B * Hkv + grid; }

// LDS tiles of one 32-position step for one KV head.
//  K: 32 positions x 128 B; chunk c (16 B, 8 dims) of position p sits at
//     p*128 + (c ^ kswz(p))*16.  kswz makes the 8 rows a score fragment read
//     together (positions 8(r/4) + 4t + r%4, r = 0..7) land in 8 distinct
//     16-byte bank groups.
//  V: 64 dims x 64 B (d-major: 32 positions x 2 B per dim row), laid out with
//     the same pair-of-rows swizzle as the GEMM tiles (vswz).
__device__ __forceinline__ int kswz(int p) { return (p & 3) | (((p >> 3) & 1) << 2); }
__device__ __forceinline__ int vswz(int row, int c) {
  const int q = row >> 1;
  return q * 128 + ((((row & 1) << 2) | c) ^ (q & 3)) * 16;
}

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Persistent workgroups of 8 waves, each over its equal range of steps (one
// or more stream pieces).  A step covers 64 positions (two 32-position
// halves).  Every step each wave issues two 1 KB LDS DMAs three steps ahead:
// K rows 8(w%4).. of half w/4 and V lines 8(w%4).. of half w/4, so up to
// three 16 KB steps are in flight per workgroup.  Then each wave runs its QPW
// query tiles of 16 (S*G queries = S slots x G heads of the group) against
// the shared tiles.
template <int QPW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(QPW == 1 ? 4 : 1, QPW == 1 ? 4 : 2)))
void attn_partial_kernel(AttnArgs a) {
  __shared__ int s_off[kMaxB + 1];
  constexpr int HALF = 4096;                // one 32-position half of a K or V tile
  __shared__ __attribute__((aligned(16))) unsigned char k0[2 * HALF], k1[2 * HALF], k2[2 * HALF], k3[2 * HALF];
  __shared__ __attribute__((aligned(16))) unsigned char v0[2 * HALF], v1[2 * HALF], v2[2 * HALF], v3[2 * HALF];
  constexpr int WIN = 8192;                 // positions per block-id window
  __shared__ int s_bt[WIN / 16 + 2];        // block ids of the window (block_size >= 16)
  attn_plan(a.seq_lens, a.B, s_off);
  const long long P = (long long)s_off[a.B] * a.Hkv;
  const int Gw = attn_ranges(P, gridDim.x);
  if (blockIdx.x == 0) {  // the merge kernel reads the plan instead of recomputing it
    for (int r = threadIdx.x; r <= a.B; r += blockDim.x) a.plan_off[r] = s_off[r];
    if (threadIdx.x == 0) a.plan_off[a.B + 1] = Gw;
  }
  if ((int)blockIdx.x >= Gw) return;
  const int G = a.Hq / a.Hkv, QN = a.S * G, QT = (QN + 15) >> 4;
  const long long x1 = ((long long)(blockIdx.x + 1) * P + Gw - 1) / Gw;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
  const float sl2 = a.scale * 1.4426950408889634f;
  const uint16_t* Q = (const uint16_t*)a.q;
  const uint16_t* Kc = (const uint16_t*)a.kcache;
  const uint16_t* Vc = (const uint16_t*)a.vcache;
  const int bs = a.block_size, bsl = __builtin_ctz(bs);  // power of two (checked on the host)
  const uint4 zero = {0u, 0u, 0u, 0u};
  const uint4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
  // fragment offsets inside a 32-position half
  int koff[2][2], voff[4];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int p = 8 * (c >> 2) + 4 * pt + (c & 3);
      koff[pt][ks] = p * 128 + (((gq + 4 * ks)) ^ kswz(p)) * 16;
    }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) voff[dt] = vswz(c + 16 * dt, gq);
  // this wave's DMA lanes: half dh of the step; K row kpos (in the half) and
  // chunk kch; V line of dims vd, chunk vch
  const int dh = w >> 2, ww = w & 3;
  const int kpos = 8 * ww + (l >> 3), kch = (l & 7) ^ kswz(kpos);
  const int vline = 8 * ww + (l >> 3), vx = (l & 7) ^ (vline & 3);
  const int vd = 2 * vline + (vx >> 2), vch = vx & 3;
  // each wave's partial-output transpose buffer reuses one stage object once
  // an item's positions are done (64 x 17 floats per wave)
  unsigned char* const sto = w == 0 ? k0 : w == 1 ? k1 : w == 2 ? k2 : w == 3 ? k3
                           : w == 4 ? v0 : w == 5 ? v1 : w == 6 ? v2 : v3;
  float* const s_ot = reinterpret_cast<float*>(sto);

  for (long long x = ((long long)blockIdx.x * P + Gw - 1) / Gw; x < x1;) {
    // the stream piece starting at global step x: request r is the last one
    // whose streams start at or before x (it has steps, since the next
    // request's streams start after x)
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long long)s_off[mid] * a.Hkv <= x) lo = mid; else hi = mid;
    }
    const int r = lo, nr = s_off[r + 1] - s_off[r];
    const int within = int(x - (long long)s_off[r] * a.Hkv);
    const int g = within / nr, st0 = within - g * nr;
    const int st1 = int(min((long long)nr, st0 + (x1 - x)));
    x += st1 - st0;
    const long long item = (long long)r * a.Hkv + g + blockIdx.x;  // partial index
    const int L = a.seq_lens[r];
    const int cb = st0 * 64, ce = min(L, st1 * 64);  // empty (cb >= ce) for a padded step: the partial is zero
    const int32_t* btr = a.bt + (long long)(r / a.vpr) * a.max_blocks;

    // query tiles of this wave
    uint4 qf[QPW][2];
    float m[QPW];
    int qpos[QPW], qmin[QPW];
    bool qv[QPW], qany[QPW];
    f32x4 o[QPW][4];
    f32x4 osum[QPW];  // row sums of P: the PV product with an all-ones "V" tile
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
      const int q = (w + 8 * qq) * 16 + c;
      bool v = q < QN;
      const int s = v ? q / G : 0, hh = v ? q % G : 0, row = r * a.S + s;
      v = v && !a.rej[row];
      qv[qq] = v;
      qpos[qq] = v ? a.positions[row] : -1;
      const uint16_t* qp = Q + ((long long)row * a.Hq + g * G + hh) * 64 + gq * 8;
      qf[qq][0] = v ? ld16(qp) : zero;
      qf[qq][1] = v ? ld16(qp + 32) : zero;
      m[qq] = -INFINITY;
      osum[qq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[qq][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // lowest position among the tile's valid queries (wave-uniform): steps
      // that end at or before it need no causal mask
      int mn = v ? qpos[qq] : 0x7FFFFFFF;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mn = min(mn, __shfl_xor(mn, off, 64));
      qmin[qq] = mn;
      qany[qq] = __ballot(v) != 0;  // a tile whose slots are all rejected is skipped
    }

    // positions [cb, ce) in windows of WIN; the block ids of a window are
    // staged in LDS first, so no global load sits between the DMAs (vmcnt
    // retires in order: a block-table load would wait for every DMA before it)
    for (int pb = cb; pb < ce; pb += WIN) {
    const int pe = min(ce, pb + WIN);
    const int nsteps = (pe - pb + 63) >> 6;
    const int wb0 = pb >> bsl, wb1 = (pe - 1) >> bsl;
    for (int i = threadIdx.x; i <= wb1 - wb0; i += blockDim.x) s_bt[i] = btr[wb0 + i];
    __syncthreads();
    // the step position this lane fetches, clamped to the window: past its end
    // the scores are masked, but the block id must be a staged one.  Its block
    // id is read from LDS before the step's fragment reads, so waiting for it
    // does not wait for them.
    auto kpp = [&](int step) { return min(pb + step * 64 + 32 * dh + kpos, pe - 1); };
    auto vpp = [&](int step) {
      const int pp = pb + step * 64 + 32 * dh + (vch >> 1) * 16;
      return pp < pe ? pp : ((pe - 1) & ~15);
    };
    auto issue = [&](unsigned char* __restrict__ kst, unsigned char* __restrict__ vst, int kp, int kb,
                     int vp, int vb) {
      const long long slot = ((long long)kb << bsl) + (kp & (bs - 1));
      __builtin_amdgcn_global_load_lds(
          (__attribute__((address_space(1))) void*)(Kc + (slot * a.Hkv + g) * 64 + kch * 8),
          (__attribute__((address_space(3))) void*)(kst + dh * HALF + ww * 1024), 16, 0, 0);
      const int off = (vp & (bs - 1)) + (vch & 1) * 8;
      __builtin_amdgcn_global_load_lds(
          (__attribute__((address_space(1))) void*)(Vc + ((((long long)vb * a.Hkv + g) * 64 + vd) << bsl) + off),
          (__attribute__((address_space(3))) void*)(vst + dh * HALF + ww * 1024), 16, 0, 0);
    };
    auto issue_step = [&](unsigned char* __restrict__ kst, unsigned char* __restrict__ vst, int step) {
      const int kp = kpp(step), vp = vpp(step);
      issue(kst, vst, kp, s_bt[(kp >> bsl) - wb0], vp, s_bt[(vp >> bsl) - wb0]);
    };

    if (0 < nsteps) issue_step(k0, v0, 0);
    if (1 < nsteps) issue_step(k1, v1, 1);
    if (2 < nsteps) issue_step(k2, v2, 2);
    auto step = [&](const unsigned char* __restrict__ kcur, const unsigned char* __restrict__ vcur,
                    unsigned char* __restrict__ kref, unsigned char* __restrict__ vref, int st) {
      // two DMA instructions per wave per step
      const int later = min(2, nsteps - 1 - st);
      if (later >= 2) attn_wait_vmcnt<4>();
      else if (later == 1) attn_wait_vmcnt<2>();
      else attn_wait_vmcnt<0>();
      asm volatile("s_barrier" ::: "memory");  // see the GEMM: no fence, DMA stays in flight
      const bool refill = st + 3 < nsteps;
      int kp = 0, kb = 0, vp = 0, vb = 0;
      if (refill) {
        kp = kpp(st + 3);
        vp = vpp(st + 3);
        kb = s_bt[(kp >> bsl) - wb0];
        vb = s_bt[(vp >> bsl) - wb0];
      }
      // the two 32-position halves of the step, one after the other (each with
      // its own online-softmax update) so only one half's fragments are live
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 kf[2][2], vf[4];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            kf[pt][ks] = *reinterpret_cast<const uint4*>(kcur + h * HALF + koff[pt][ks]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vf[dt] = *reinterpret_cast<const uint4*>(vcur + h * HALF + voff[dt]);
        if (h == 0 && refill) issue(kref, vref, kp, kb, vp, vb);
        const int ph0 = pb + st * 64 + 32 * h, pv0 = ph0 + 8 * gq;
#pragma unroll
        for (int qq = 0; qq < QPW; ++qq) {
          if (w + 8 * qq >= QT) break;
          if (!qany[qq]) continue;  // every slot of this tile was rejected
          f32x4 sc[2];
#pragma unroll
          for (int pt = 0; pt < 2; ++pt) {
            sc[pt] = mfma16(kf[pt][0], qf[qq][0], f32x4{0.f, 0.f, 0.f, 0.f});
            sc[pt] = mfma16(kf[pt][1], qf[qq][1], sc[pt]);
          }
          // lane (gq, c): sc[pt][i] scores position pv0 + 4pt + i for query c.
          // The max is taken over raw scores (the scale is positive) and the
          // scale enters inside the exponent's FMA.
          float v[8];
          float mloc = -INFINITY;
          if (ph0 + 31 < pe && ph0 + 31 <= qmin[qq]) {
            // the whole half lies inside the window and before every valid
            // query of the tile: no mask (invalid queries' results are unused)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              v[t] = sc[t >> 2][t & 3];
              mloc = fmaxf(mloc, v[t]);
            }
          } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int pos = pv0 + t;
              const bool ok = qv[qq] && pos < pe && pos <= qpos[qq];
              v[t] = ok ? sc[t >> 2][t & 3] : -INFINITY;
              mloc = fmaxf(mloc, v[t]);
            }
          }
          float mref;
#if PE_ATTN_LAZY
          // (not with four query tiles per wave: the extra live values spill)
          if (QPW <= 2 && !__ballot(mloc * sl2 > m[qq] + kLazyMax)) {
            // no score of the half exceeds the running max by more than
            // kLazyMax (base 2): it stays the exponent's reference, so p <=
            // 2^kLazyMax, and neither the maximum across the query's lanes
            // nor a rescale is needed (a lane whose scores are all masked so
            // far keeps -inf and a reference of 0, its p being 0)
            mref = m[qq] == -INFINITY ? 0.f : m[qq];
          } else
#endif
          {
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            const float mnew = fmaxf(m[qq], mloc * sl2);
            mref = (mnew == -INFINITY) ? 0.f : mnew;
            if (__ballot(mnew != m[qq])) {  // some query's running max moved: rescale
              const float alpha = __builtin_amdgcn_exp2f(m[qq] - mref);
              osum[qq] = osum[qq] * alpha;
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) o[qq][dt] = o[qq][dt] * alpha;
            }
            m[qq] = mnew;
          }
          // P = hi + lo, both bf16: the PV product sees P to ~16 bits, and so
          // does the row sum, taken by the same MFMAs on an all-ones tile.
          // exp2 of a non-positive argument: v_exp_f32 flushes results below
          // 2^-126 to 0.
          uint32_t ph[4], pl[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(v[2 * jj], sl2, -mref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(v[2 * jj + 1], sl2, -mref));
            ph[jj] = f2bf2(p0, p1);
            pl[jj] = f2bf2(p0 - __uint_as_float(ph[jj] << 16), p1 - __uint_as_float(ph[jj] & 0xFFFF0000u));
          }
          const uint4 pfh = {ph[0], ph[1], ph[2], ph[3]};
          const uint4 pfl = {pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            o[qq][dt] = mfma16(vf[dt], pfh, o[qq][dt]);
            o[qq][dt] = mfma16(vf[dt], pfl, o[qq][dt]);
          }
          osum[qq] = mfma16(ones, pfh, osum[qq]);
          osum[qq] = mfma16(ones, pfl, osum[qq]);
        }
      }
    };
    for (int st = 0; st < nsteps; st += 4) {
      step(k0, v0, k3, v3, st);
      if (st + 1 < nsteps) step(k1, v1, k0, v0, st + 1);
      if (st + 2 < nsteps) step(k2, v2, k1, v1, st + 2);
      if (st + 3 < nsteps) step(k3, v3, k2, v2, st + 3);
    }
    __syncthreads();  // stages and s_bt are reused by the next window (or the transpose below)
    }  // windows

    // partials: O (un-normalised), running max m (base 2) and sum l per query
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
      const int t = w + 8 * qq;
      if (t >= QT) break;
      const float ls = osum[qq][0];  // every row of the ones tile holds query c's sum
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_ot[(16 * dt + 4 * gq + i) * 17 + c] = o[qq][dt][i];
      wave_lds_sync();
      const int qi = l >> 2, d0 = (l & 3) * 16, qg = t * 16 + qi;
      if (qg < QN) {
        float* dst = a.part_o + ((long long)item * QN + qg) * 64 + d0;
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          float4 f;
          f.x = s_ot[(d0 + 4 * v4 + 0) * 17 + qi];
          f.y = s_ot[(d0 + 4 * v4 + 1) * 17 + qi];
          f.z = s_ot[(d0 + 4 * v4 + 2) * 17 + qi];
          f.w = s_ot[(d0 + 4 * v4 + 3) * 17 + qi];
          *reinterpret_cast<float4*>(dst + 4 * v4) = f;
        }
      }
      const int q = t * 16 + c;
      if (gq == 0 && q < QN) {
        a.part_ml[((long long)item * QN + q) * 2 + 0] = m[qq];
        a.part_ml[((long long)item * QN + q) * 2 + 1] = ls;
      }
      wave_lds_sync();
    }
    __syncthreads();  // the stages are reused by the next item
  }
}

// The partials of stream (r, g): first index and count (0 when the request
// has no context).  Workgroup w holds the piece of every stream its range
// meets, at index s + w.
__device__ __forceinline__ int attn_pieces(const int32_t* off, int B, int Hkv, int r, int g,
                                           long long& first) {
  const int nr = off[r + 1] - off[r];
  if (nr <= 0) return 0;
  const long long P = (long long)off[B] * Hkv;
  const int Gw = off[B + 1];
  const long long x0 = (long long)off[r] * Hkv + (long long)g * nr, xe = x0 + nr - 1;
  const int wlo = int(x0 * Gw / P), whi = int(xe * Gw / P);
  first = (long long)r * Hkv + g + wlo;
  return whi - wlo + 1;
}

// One wave per (slot, query head): lane = dim.  Lanes first share out the
// chunks to find the max, then every chunk's weight is broadcast and the
// weighted partial rows are summed with independent loads.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int32_t* s_off = a.plan_off;  // written by the partial kernel
  const int G = a.Hq / a.Hkv, QN = a.S * G;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const long long total = (long long)a.B * a.S * a.Hq;
  uint16_t* out = (uint16_t*)a.out;
  for (long long x = (long long)blockIdx.x * 4 + w; x < total; x += (long long)gridDim.x * 4) {
    const int row = int(x / a.Hq), h = int(x % a.Hq);
    const int r = row / a.S, s = row % a.S, g = h / G, q = s * G + (h % G);
    uint16_t* dst = out + (long long)row * a.Hq * 64 + h * 64 + l;
    long long i0 = 0;
    const int nc = a.rej[row] ? 0 : attn_pieces(s_off, a.B, a.Hkv, r, g, i0);
    if (nc == 0) { *dst = 0; continue; }
    auto ml = [&](int ch) { return a.part_ml + ((i0 + ch) * QN + q) * 2; };
    float M = -INFINITY;
    for (int ch = l; ch < nc; ch += 64) M = fmaxf(M, ml(ch)[0]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int base = 0; base < nc; base += 64) {
        const int ch = base + l;
        float wl = 0.f, lc = 0.f;
        if (ch < nc) {
          const float mc = ml(ch)[0];
          wl = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
          lc = ml(ch)[1];
        }
        Lsum += wl * lc;
        const int n = min(64, nc - base);
#pragma unroll 4
        for (int j = 0; j < n; ++j) {
          const float wj = __shfl(wl, j, 64);
          const long long it = i0 + base + j;
          O += wj * a.part_o[(it * QN + q) * 64 + l];
        }
      }
      for (int o = 32; o > 0; o >>= 1) Lsum += __shfl_xor(Lsum, o, 64);
    }
    *dst = f2bf(Lsum > 0.f ? O / Lsum : 0.f);
  }
}

// One wave per (slot, KV head): lane l combines query head (l G)/64 of the
// group, dims (l G) % 64 .. +G.  A chunk's partials for the G heads of a slot
// are one contiguous block of G x 64 floats, so every lane reads G consecutive
// floats per chunk and the chunks' loads are independent.  G is a power of
// two <= 16 (attn_merge_kernel serves other groupings).
template <int G>
__global__ __launch_bounds__(256) void attn_merge_group_kernel(AttnArgs a) {
  const int32_t* s_off = a.plan_off;  // written by the partial kernel
  const int QN = a.S * G;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int hl = (l * G) >> 6, d0 = (l * G) & 63;
  const long long total = (long long)a.B * a.S * a.Hkv;
  uint16_t* out = (uint16_t*)a.out;
  for (long long x = (long long)blockIdx.x * 4 + w; x < total; x += (long long)gridDim.x * 4) {
    const int row = int(x / a.Hkv), g = int(x % a.Hkv);
    const int r = row / a.S, s = row % a.S, q = s * G + hl;
    uint16_t* dst = out + ((long long)row * a.Hq + g * G + hl) * 64 + d0;
    float O[G];
#pragma unroll
    for (int j = 0; j < G; ++j) O[j] = 0.f;
    float L = 0.f;
    long long i0 = 0;
    const int nc = a.rej[row] ? 0 : attn_pieces(s_off, a.B, a.Hkv, r, g, i0);
    if (nc > 0) {
      auto item = [&](int ch) { return i0 + ch; };
      // unrolled so that the chunks' loads are in flight together
      float M = -INFINITY;
#pragma unroll 8
      for (int ch = 0; ch < nc; ++ch) M = fmaxf(M, a.part_ml[(item(ch) * QN + q) * 2]);
      if (M != -INFINITY) {
#pragma unroll 8
        for (int ch = 0; ch < nc; ++ch) {
          const long long it = item(ch);
          const float mc = a.part_ml[(it * QN + q) * 2], lc = a.part_ml[(it * QN + q) * 2 + 1];
          const float wgt = (mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mc - M);
          L += wgt * lc;
          const float* po = a.part_o + (it * QN + q) * 64 + d0;
          if constexpr (G % 4 == 0) {
#pragma unroll
            for (int j = 0; j < G; j += 4) {
              const float4 v = *reinterpret_cast<const float4*>(po + j);
              O[j] += wgt * v.x; O[j + 1] += wgt * v.y; O[j + 2] += wgt * v.z; O[j + 3] += wgt * v.w;
            }
          } else {
#pragma unroll
            for (int j = 0; j < G; ++j) O[j] += wgt * po[j];
          }
        }
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if constexpr (G == 1) {
      dst[0] = f2bf(O[0] * inv);
    } else {
#pragma unroll
      for (int j = 0; j < G; j += 2) *reinterpret_cast<uint32_t*>(dst + j) = f2bf2(O[j] * inv, O[j + 1] * inv);
    }
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
  const int32_t* btr = a.bt + (long long)(r / a.vpr) * a.max_blocks;
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

// Groups of Sv consecutive slots as requests of their own (a prefill batch's
// slots in query blocks that fit one workgroup): one wave per group.
__global__ __launch_bounds__(256) void attn_group_lens_kernel(int Bv, int Sv, int vpr,
                                                              const int32_t* __restrict__ positions,
                                                              const uint8_t* __restrict__ rej,
                                                              const int32_t* __restrict__ seq_lens,
                                                              int32_t* __restrict__ out) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (v >= Bv) return;
  const long long base = (long long)v * Sv;
  int hi = -1;
  for (int s = l; s < Sv; s += 64)
    if (!rej[base + s]) hi = max(hi, positions[base + s]);
  for (int o = 32; o > 0; o >>= 1) hi = max(hi, __shfl_xor(hi, o, 64));
  if (l == 0) {
    const int L = seq_lens[v / vpr];
    out[v] = (L <= 0 || hi < 0) ? 0 : min(L, hi + 1);
  }
}

hipError_t launch_attn_group_lens(int Bv, int Sv, int vpr, const int32_t* positions, const uint8_t* rej,
                                  const int32_t* seq_lens, int32_t* out, hipStream_t st) {
  if (Bv <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_group_lens_kernel, dim3(unsigned((Bv + 3) / 4)), dim3(256), 0, st, Bv, Sv, vpr,
                     positions, rej, seq_lens, out);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (a.vpr < 1 || a.B > kMaxB) return hipErrorInvalidValue;
  if (dtype == 0) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.B * a.S * a.Hq), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  const int QT = (a.S * (a.Hq / a.Hkv) + 15) / 16;
  if (QT <= 8)
    hipLaunchKernelGGL(attn_partial_kernel<1>, dim3(a.grid), dim3(512), 0, st, a);
  else if (QT <= 16)
    hipLaunchKernelGGL(attn_partial_kernel<2>, dim3(a.grid), dim3(512), 0, st, a);
  else if (QT <= 32)
    hipLaunchKernelGGL(attn_partial_kernel<4>, dim3(a.grid), dim3(512), 0, st, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  const long long waves = (long long)a.B * a.S * (G <= 16 && (G & (G - 1)) == 0 ? a.Hkv : a.Hq);
  long long blocks = (waves + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  const dim3 mg((unsigned)blocks), mb(256);
  switch (G) {
    case 1: hipLaunchKernelGGL(attn_merge_group_kernel<1>, mg, mb, 0, st, a); break;
    case 2: hipLaunchKernelGGL(attn_merge_group_kernel<2>, mg, mb, 0, st, a); break;
    case 4: hipLaunchKernelGGL(attn_merge_group_kernel<4>, mg, mb, 0, st, a); break;
    case 8: hipLaunchKernelGGL(attn_merge_group_kernel<8>, mg, mb, 0, st, a); break;
    case 16: hipLaunchKernelGGL(attn_merge_group_kernel<16>, mg, mb, 0, st, a); break;
    default: hipLaunchKernelGGL(attn_merge_kernel, mg, mb, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace pe
