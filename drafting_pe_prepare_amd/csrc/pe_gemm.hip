// Dense contractions of the drafter: out[m, n] = sum_k A[m, k] W[n, k] with a
// fused epilogue.  "P-EAGLE: parallel speculative decoding in vLLM",
// Architecture and mechanism, Step 2: an fc over concat(emb, h), an N-layer
// Transformer and the LM head, over all K positions in one pass.  These are the
// dense parts of that pass: fc, QKV (+ RoPE + KV write), O (+ residual),
// gate/up (+ SiLU-and-mul), down (+ residual), LM head (+ row argmax).
//
// gfx950 design
//  * bf16 operands, fp32 accumulation on v_mfma_f32_16x16x32_bf16.  Both
//    operands are K-contiguous, so every lane feeds the MFMA straight from one
//    16-byte load (A row l%16 / W row l%16, k chunk l/16).
//  * M <= 64 (a draft batch of a few requests): the weights are the whole
//    traffic.  gemm_skinny splits K across the 16 waves of a workgroup, streams
//    W with non-temporal 16-byte loads, and reduces the wave partials through
//    LDS in a fixed order (deterministic), then runs the epilogue.
//  * LM head with M <= 16 rows: lmhead_wide keeps the rows in LDS, gives every
//    wave whole 16-column tiles over the full K, and keeps a running argmax key
//    per row in registers -- logits never reach memory unless asked for.
//  * 65..256 rows: gemm_tiled, 128x128x64 LDS-tiled, double-buffered, 4 waves
//    of 64x64; workgroups that share a weight tile are placed on one XCD (one
//    L2) back to back.  More rows run on pe_mm.hip.
//  * Epilogues run on an fp32 tile staged in LDS, so every variant shares them.
//    Column pairs that an epilogue needs together (RoPE rotate-half partners,
//    gate/up partners) are placed 16 logical columns apart inside one 32-column
//    block by the weight-row mapping (B_QKV, B_GATEUP).
//  * fp32 storage: gemm_f32, plain FMA, for the small fp32 workload only.
#include <algorithm>

#include "pe_common.h"
#include "pe_internal.h"

#ifndef PE_SPLITK_WG_PER_CU
#define PE_SPLITK_WG_PER_CU 2  // workgroups per CU that a split-K GEMM aims for
#endif
#ifndef PE_SPLITK_MIN_KTILES
#define PE_SPLITK_MIN_KTILES 8  // fewest 64-wide k-tiles per split
#endif
#ifndef PE_TAIL_MIN_KTILES
#define PE_TAIL_MIN_KTILES 4  // fewest 64-wide k-tiles per piece of a split LM-head tail
#endif
#ifndef PE_SKINNY_NTW_GU
#define PE_SKINNY_NTW_GU 4  // 16-column tiles per gate/up workgroup of up to 16 rows
#endif
#ifndef PE_SKINNY_U_NARROW
#define PE_SKINNY_U_NARROW 8  // k-steps of loads in flight per wave, one tile of up to 16 rows
#endif
#ifndef PE_SKINNY_U_WIDE
#define PE_SKINNY_U_WIDE 4  // the same, wider workgroups
#endif

namespace pe {

// ---------------------------------------------------------------------------
// operand addressing
// ---------------------------------------------------------------------------
// Rotate-half partner layout: inside each head of hd dims, logical 16-column
// group s maps to dims (s%2)*hd/2 + (s/2)*16 + [0,16), so groups 2j and 2j+1
// hold dims i and i + hd/2 for the same i.
__device__ __forceinline__ int rope_phys(int j, int hd) {
  const int jb = j % hd, s = jb >> 4, c = jb & 15;
  return (j - jb) + (s & 1) * (hd >> 1) + (s >> 1) * 16 + c;
}

template <typename T, int BMAP>
__device__ __forceinline__ const T* weight_row(const GemmArgs& g, int n) {
  const long long K = g.K;
  if (BMAP == B_GATEUP) {
    const int t = n >> 5, r = n & 31;
    return (r < 16 ? (const T*)g.W0 : (const T*)g.W1) + (long long)(t * 16 + (r & 15)) * K;
  } else if (BMAP == B_QKV) {
    if (n >= g.nq + g.nk) return (const T*)g.W2 + (long long)(n - g.nq - g.nk) * K;
    if (n < g.nq) return (const T*)g.W0 + (long long)rope_phys(n, g.hd) * K;
    return (const T*)g.W1 + (long long)rope_phys(n - g.nq, g.hd) * K;
  }
  return (const T*)g.W0 + (long long)n * K;
}

// A row m: `lo` serves k < d (or every k for A_PLAIN), `hi` serves k >= d.
template <typename T, int AL>
struct ARow {
  const T* lo;
  const T* hi;
  __device__ __forceinline__ void init(const GemmArgs& g, int m) {
    if (AL == A_FC) {
      int id = g.ids[m];
      id = id < 0 ? 0 : (id >= g.vocab ? g.vocab - 1 : id);
      lo = (const T*)g.embed + (long long)id * g.d;
      hi = (const T*)g.hid + (long long)m * g.d - g.d;
    } else {
      lo = (const T*)g.A + (long long)m * g.lda;
      hi = lo;
    }
  }
  __device__ __forceinline__ const T* at(int k, int d) const {
    return (AL == A_FC && k >= d) ? hi + k : lo + k;
  }
};

// ---------------------------------------------------------------------------
// epilogues on an fp32 tile in LDS: tile[i*ldt + c] = out[m0+i, n0+c] (logical)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_sincos(const GemmArgs& g, int pos, int i, float& cs, float& sn) {
  // angle pos * theta^(-2i/hd) in turns: the fp64 product minus its nearest
  // integer is the exact fraction of a turn for any position; v_sin_f32 and
  // v_cos_f32 take turns (max abs error 1.3e-7 on [-1/2, 1/2], measured)
  const double t = double(pos) * g.rope_turns[i];
  const float x = float(t - rint(t));
  sn = __builtin_amdgcn_sinf(x);
  cs = __builtin_amdgcn_cosf(x);
}

// Per-element epilogues.  epi_one: one logical column n of row m (E_STORE,
// E_RESID).  epi_pair: a 32-column logical block starting at nb, column c in
// [0,16) paired with c+16 (E_SILU: gate, up; E_QKV: RoPE partners or two V dims).
template <typename T, int EPI>
__device__ __forceinline__ void epi_one(const GemmArgs& g, int m, int n, float v) {
  const long long o = (long long)m * g.ldo + n;
  if (EPI == E_RESID) v += Elt<T>::ld((const T*)g.resid + o);
  Elt<T>::st((T*)g.out + o, v);
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_pair(const GemmArgs& g, int m, int nb, int c, float lo, float hi) {
  if (EPI == E_SILU) {
    const float v = lo / (1.0f + expf(-lo)) * hi;
    Elt<T>::st((T*)g.out + (long long)m * g.ldo + (nb >> 1) + c, v);
  } else if (EPI == E_QKV) {
    // bf16 storage implies head_dim 64 (checked at context creation)
    const int hd = sizeof(T) == 2 ? 64 : g.hd;
    if (nb < g.nq + g.nk) {
      const bool isq = nb < g.nq;
      const int j = isq ? nb : nb - g.nq;
      const int head = j / hd, s = (j % hd) >> 4;
      const int dlo = (s >> 1) * 16 + c, dhi = dlo + (hd >> 1);
      float cs, sn;
      rope_sincos(g, g.positions[m], dlo, cs, sn);
      const float olo = lo * cs - hi * sn, ohi = hi * cs + lo * sn;
      if (isq) {
        T* q = (T*)g.qout + ((long long)m * (g.nq / hd) + head) * hd;
        Elt<T>::st(q + dlo, olo);
        Elt<T>::st(q + dhi, ohi);
      } else {
        const long long slot = g.slots[m];
        if (slot >= 0 && slot < g.num_slots) {
          T* kp = (T*)g.kcache + (slot * g.Hkv + head) * hd;
          Elt<T>::st(kp + dlo, olo);
          Elt<T>::st(kp + dhi, ohi);
        }
      }
    } else {
      const long long slot = g.slots[m];
      if (slot >= 0 && slot < g.num_slots) {
        const int j = nb - g.nq - g.nk;
        const int head = j / hd, jb = j % hd;
        const int bsl = __builtin_ctz(g.block_size);  // a power of two (checked at context creation)
        const long long blk = slot >> bsl, off = slot & (g.block_size - 1);
        T* vp = (T*)g.vcache + (((blk * g.Hkv + head) * hd) << bsl) + off;
        Elt<T>::st(vp + ((long long)(jb + c) << bsl), lo);
        Elt<T>::st(vp + ((long long)(jb + 16 + c) << bsl), hi);
      }
    }
  }
}

// The same epilogues over an fp32 tile staged in LDS: tile[i*ldt + c] holds
// out[m0+i, n0+c] (logical columns).
template <typename T, int EPI>
__device__ void epilogue(const GemmArgs& g, const float* tile, int ldt, int m0, int TM, int n0,
                         int TN) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int mrows = min(TM, g.M - m0);
  const int ncols = min(TN, g.N - n0);
  if (mrows <= 0 || ncols <= 0) return;
  if (EPI == E_STORE || EPI == E_RESID) {
    for (int e = tid; e < mrows * ncols; e += nt) {
      const int i = e / ncols, c = e - i * ncols;
      epi_one<T, EPI>(g, m0 + i, n0 + c, tile[i * ldt + c]);
    }
  } else {
    const int np = ncols >> 1;
    for (int e = tid; e < mrows * np; e += nt) {
      const int i = e / np, p = e - i * np, b = p >> 4, c = p & 15;
      epi_pair<T, EPI>(g, m0 + i, n0 + b * 32, c, tile[i * ldt + b * 32 + c],
                       tile[i * ldt + b * 32 + 16 + c]);
    }
  }
}

// Row argmax of a tile: one wave per row, lanes over columns, 64-bit keys.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor(uint32_t(v), o, 64), hi = __shfl_xor(uint32_t(v >> 32), o, 64);
  return (uint64_t(hi) << 32) | lo;
}

// Row argmax of a staged tile: one wave per row, lanes over columns.  The
// best 64-bit key of the tile is stored at keys[row * parts + part]; every
// (row, part) is written by exactly one workgroup, so no atomics are needed and
// the keys need no clearing between launches.
__device__ void epilogue_argmax(const GemmArgs& g, const float* tile, int ldt, int m0, int TM,
                                int n0, int TN, int part) {
  const int mrows = min(TM, g.M - m0), ncols = min(TN, g.N - n0);
  if (mrows <= 0 || ncols <= 0) return;
  if (g.logits)
    for (int e = threadIdx.x; e < mrows * ncols; e += blockDim.x) {
      const int i = e / ncols, c = e - i * ncols;
      g.logits[(long long)(m0 + i) * g.ldl + n0 + c] = tile[i * ldt + c];
    }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int i = w; i < mrows; i += nw) {
    uint64_t best = 0;
    for (int c = l; c < ncols; c += 64) {
      const uint64_t k = argmax_key(tile[i * ldt + c], n0 + c);
      best = k > best ? k : best;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t k = shfl_xor_u64(best, o);
      best = k > best ? k : best;
    }
    if (l == 0) g.keys[(long long)(m0 + i) * g.parts + part] = best;
  }
}

// Argmax of the draft rows and greedy verification in one launch, for the step
// graph: one workgroup per request; wave w reduces draft rows w, w + waves, ...
// of the request (the same fixed reduction as argmax_tokens_kernel), then wave
// 0 finds the first draft that differs from the target's token (a' = K when
// none does) and takes the target's token there as the bonus.
// Max of this lane's keys kr[l], kr[l + stride], ... below `parts`: 8 loads
// in flight at a time (indices past the end re-read the last key, which
// leaves the max unchanged).
__device__ __forceinline__ uint64_t max_keys(const uint64_t* __restrict__ kr, int parts, int l, int stride) {
  uint64_t best = 0;
  for (int p0 = l; p0 < parts; p0 += 8 * stride) {
    uint64_t k[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = kr[min(p0 + i * stride, parts - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) best = k[i] > best ? k[i] : best;
  }
  return best;
}

__global__ __launch_bounds__(1024) void argmax_verify_kernel(int K, int parts,
                                                             const uint64_t* __restrict__ keys,
                                                             int32_t* __restrict__ tokens,
                                                             const int32_t* __restrict__ seq_lens,
                                                             const int32_t* __restrict__ target,
                                                             int32_t* __restrict__ acc,
                                                             int32_t* __restrict__ bonus,
                                                             const int32_t* __restrict__ nact) {
  __shared__ int32_t s_tok[64];
  const int r = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  if (nact && r >= nact[0]) {  // an inactive request: no keys were written for its rows
    if (w == 0) {
      if (l < K) tokens[(long long)r * K + l] = -1;
      if (l == 0) {
        acc[r] = 0;
        bonus[r] = 0;  // PE_PAD_TOKEN
      }
    }
    return;
  }
  const bool padded = seq_lens[r] == 0;
  for (int i = w; i < K; i += nw) {
    const long long row = (long long)r * K + i;
    const uint64_t* kr = keys + row * parts;
    uint64_t best = max_keys(kr, parts, l, 64);
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t k = shfl_xor_u64(best, o);
      best = k > best ? k : best;
    }
    if (l == 0) {
      const int tok = padded ? -1 : argmax_key_index(best);
      tokens[row] = tok;
      s_tok[i] = tok;
    }
  }
  __syncthreads();
  if (w == 0) {
    const int32_t* g = target + (long long)r * (K + 1);
    const bool miss = l < K && s_tok[l] != g[l];
    const unsigned long long m = __ballot(miss);
    const int a = m ? (__ffsll((long long)m) - 1) : K;
    if (l == 0) {
      acc[r] = a;
      bonus[r] = g[a];
    }
  }
}

// Argmax partial keys -> tokens, run as its own small kernel after the LM head
// (the kernel boundary orders the GEMM's stores before these reads).  One
// workgroup per draft row reduces that row's `parts` keys.
__global__ __launch_bounds__(256) void argmax_tokens_kernel(int M, int Kd, int parts,
                                                            const uint64_t* __restrict__ keys,
                                                            int32_t* __restrict__ tokens, int tstride,
                                                            const int32_t* __restrict__ seq_lens) {
  __shared__ uint64_t red[4];
  const int row = blockIdx.x;
  const uint64_t* kr = keys + (long long)row * parts;
  uint64_t best = max_keys(kr, parts, threadIdx.x, blockDim.x);
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t k = shfl_xor_u64(best, o);
    best = k > best ? k : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x >> 6); ++w) best = red[w] > best ? red[w] : best;
    best = red[0] > best ? red[0] : best;
    int tok = argmax_key_index(best);
    if (seq_lens && seq_lens[row / Kd] == 0) tok = -1;
    tokens[(long long)row * tstride] = tok;
  }
}

// ---------------------------------------------------------------------------
// bf16, M <= 64: split-K across the waves of a workgroup
// ---------------------------------------------------------------------------
// NRM (one row tile, A_PLAIN): the A rows are x and the operand is their
// RMSNorm, bf16((x * rs) * gain).  rs comes from the producer's per-tile sums
// of squares (GemmArgs::ssq_in): LDS DMAs issued ahead of the first batch of
// weights stage them (from byte 0, read only before every wave's first
// batch ends) and the norm's gain (past the wave-partial and tile buffers,
// which early waves fill while later ones still read the gain), and once
// that batch has landed each row's partials are summed in a fixed order.
// Kept in LDS, the gain takes no registers beside the batch.
template <int EPI, int AL, int BMAP, int MT, int NTW, int U, int NRM>
__global__ __launch_bounds__(1024) void gemm_skinny_kernel(GemmArgs g) {
  extern __shared__ float smem[];
  const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int col = l & 15, kg = l >> 4;
  const int n0 = blockIdx.x * (NTW * 16);
  const int ksteps = g.K >> 5;
  const int ks0 = (ksteps * w) / nw, ks1 = (ksteps * (w + 1)) / nw;

  // weight fragment of (tile t, k-step ks) for this lane: from the
  // fragment-order copy (one contiguous 1 KB per wave load) when there is one
  const uint16_t* wp[NTW];
  long long wstep;  // elements between consecutive k-steps
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    int n = n0 + t * 16 + col;
    n = n < g.N ? n : g.N - 1;
    if (g.Wp) wp[t] = (const uint16_t*)g.Wp + (long long)(n0 / 16 + t) * ksteps * 512 + l * 8;
    else wp[t] = weight_row<uint16_t, BMAP>(g, n) + kg * 8;
  }
  wstep = g.Wp ? 512 : 32;
  ARow<uint16_t, AL> ar[MT];
  bool av[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col;
    av[mt] = m < g.M;
    ar[mt].init(g, av[mt] ? m : 0);
  }
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // NRM: the 16 x ssq_n partial sums and the K gains go to LDS first (wave
  // w's lanes move bytes [1 KB w, 1 KB (w + 1)) of each; 16 ssq_n <= 256 nw
  // and 2 K <= 1 KB nw, checked on the host)
  constexpr int PER = MT * NTW * 256;  // floats of one wave's partial tile
  constexpr int LDT = NTW * 16 + 4;    // row stride of the staged output tile
  const int kGainOff = (nw * PER + MT * 16 * LDT + 3) & ~3;  // floats: past both
  // two DMAs per wave, unconditional so that every wave's vmcnt counts them
  // (a lane past the end re-reads the last chunk into its own, unused slot);
  // issued inside the first batch, after its A chunks and before its weights
  auto stage_norm = [&]() {
    const int e = (w * 64 + l) * 4;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform: the DMA's LDS base goes to m0
    dma16(g.ssq_in + min(e, 16 * g.ssq_n - 4), lds_addr((const unsigned char*)(smem + wu * 256)));
    dma16((const uint16_t*)g.norm_gain + 2 * min(e, g.K / 2 - 4),
          lds_addr((const unsigned char*)(smem + kGainOff + wu * 256)));
  };
  float rs = 1.f;
  const uint16_t* gain = reinterpret_cast<const uint16_t*>(smem + kGainOff) + kg * 8;

  const uint4 zero = {0u, 0u, 0u, 0u};
  // U k-steps of loads in flight per batch, then their MFMAs
  for (int ks = ks0; ks < ks1; ks += U) {
    const int n = min(U, ks1 - ks);
    uint4 b[U][NTW], a[U][MT];
    if constexpr (NRM) {
      // the batch's A chunks, then its weights, every load unconditional (a
      // step past the wave's range re-reads its last one; no MFMA uses it),
      // so that waiting for the A chunks leaves exactly U*NTW loads in flight
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = ks + min(u, n - 1);
        a[u][0] = ld16(ar[0].at(kk * 32 + kg * 8, g.d));  // row 0 stands in for rows past M
      }
      if (ks == ks0) stage_norm();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = ks + min(u, n - 1);
#pragma unroll
        for (int t = 0; t < NTW; ++t) b[u][t] = ld16(wp[t] + kk * wstep);
      }
      wait_vmcnt<U * NTW>();  // A chunks landed (and, first time, the DMAs); weights in flight
      if (ks == ks0) {  // every wave's first batch: the rows' rs
        const float* sq = smem;  // free until the wave partials are reduced below
        __shared__ float s_rs[16];
        asm volatile("s_barrier" ::: "memory");  // no fence: the weights stay in flight
        for (int i = w; i < 16; i += nw) {
          float sacc = 0.f;
          for (int p = l; p < g.ssq_n; p += 64) sacc += sq[i * g.ssq_n + p];
          sacc = wave_sum(sacc);
          // rows past M were never written by the producer: any rs (their A is zero)
          if (l == 0) s_rs[i] = i < g.M ? rsqrtf(sacc / float(g.K) + g.norm_eps) : 1.f;
        }
        wait_lgkm0();
        asm volatile("s_barrier" ::: "memory");
        rs = s_rs[col];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u < n) {
          const uint4 gv = *reinterpret_cast<const uint4*>(gain + (ks + u) * 32);
          const uint16_t* e = reinterpret_cast<const uint16_t*>(&a[u][0]);
          const uint16_t* ge = reinterpret_cast<const uint16_t*>(&gv);
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = f2bf2(bf2f(e[2 * q]) * rs * bf2f(ge[2 * q]), bf2f(e[2 * q + 1]) * rs * bf2f(ge[2 * q + 1]));
          a[u][0] = av[0] ? uint4{o[0], o[1], o[2], o[3]} : zero;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u < n) {
          const int k = (ks + u) * 32;
#pragma unroll
          for (int t = 0; t < NTW; ++t) b[u][t] = ld16(wp[t] + (ks + u) * wstep);  // plain: stays cache-resident
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) a[u][mt] = av[mt] ? ld16(ar[mt].at(k + kg * 8, g.d)) : zero;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < n) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < NTW; ++t) acc[mt][t] = mfma16(a[u][mt], b[u][t], acc[mt][t]);
      }
    }
  }

  // fixed-order reduction of the wave partials
  float* red = smem;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w * PER + ((mt * NTW + t) * 4 + i) * 64 + l] = acc[mt][t][i];
  __syncthreads();
  float* tile = smem + nw * PER;
  for (int e = threadIdx.x; e < PER; e += blockDim.x) {
    float s = 0.f;
    for (int ww = 0; ww < nw; ++ww) s += red[ww * PER + e];
    const int lane = e & 63, i = (e >> 6) & 3, mtt = e >> 8;
    const int t = mtt % NTW, mt = mtt / NTW;
    tile[(mt * 16 + (lane >> 4) * 4 + i) * LDT + t * 16 + (lane & 15)] = s;
  }
  __syncthreads();
  if constexpr (EPI == E_ARGMAX) {
    epilogue_argmax(g, tile, LDT, 0, MT * 16, n0, NTW * 16, blockIdx.x);
  } else if constexpr ((EPI == E_STORE || EPI == E_RESID) && MT == 1 && NTW == 1) {
    if (g.ssq_out) {
      // store, keep the stored (rounded) values, then each row's sum of squares
      const int mrows = min(16, g.M), ncols = min(16, g.N - n0);
      for (int e = threadIdx.x; e < mrows * ncols; e += blockDim.x) {
        const int i = e / ncols, c = e - i * ncols;
        const long long o = (long long)i * g.ldo + n0 + c;
        float v = tile[i * LDT + c];
        if (EPI == E_RESID) v += bf2f(((const uint16_t*)g.resid)[o]);
        const uint16_t h = f2bf(v);
        ((uint16_t*)g.out)[o] = h;
        tile[i * LDT + c] = bf2f(h);
      }
      __syncthreads();
      if ((int)threadIdx.x < mrows) {
        float sacc = 0.f;
        for (int c = 0; c < ncols; ++c) {
          const float v = tile[threadIdx.x * LDT + c];
          sacc += v * v;
        }
        g.ssq_out[(long long)threadIdx.x * g.ssq_n + blockIdx.x] = sacc;
      }
    } else {
      epilogue<uint16_t, EPI>(g, tile, LDT, 0, MT * 16, n0, NTW * 16);
    }
  } else {
    epilogue<uint16_t, EPI>(g, tile, LDT, 0, MT * 16, n0, NTW * 16);
  }
}

// ---------------------------------------------------------------------------
// bf16 LM head, M <= 16 rows: rows in LDS, whole tiles per wave, argmax in
// registers
// ---------------------------------------------------------------------------
// One workgroup per CU over a contiguous, tile-aligned range of 16-column
// tiles.  The range is cut into units of U k-steps (tile-major) and every wave
// takes an equal run of units, so all waves finish together.  A tile cut
// between waves leaves partial sums in LDS; after the barrier the wave that
// holds the tile's first unit adds them up and folds the tile into its argmax.
template <int U>
__global__ __launch_bounds__(512) void lmhead_wide_kernel(GemmArgs g) {
  extern __shared__ uint4 xs[];
  constexpr int MAXW = 8;
  __shared__ float part[MAXW][2][4][64];   // [wave][head/tail][i][lane]
  __shared__ int part_tile[MAXW][2];
  __shared__ uint64_t s_best[MAXW][16];
  const int K = g.K, kc = K >> 3, ldx = kc + 1;
  for (int c = threadIdx.x; c < g.M * kc; c += blockDim.x) {
    const int m = c / kc, j = c - m * kc;
    xs[m * ldx + j] = ld16((const uint16_t*)g.A + (long long)m * g.lda + j * 8);
  }
  const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int col = l & 15, kg = l >> 4;
  if (l < 2) part_tile[w][l] = -1;
  __syncthreads();
  const int ntiles = g.N >> 4;
  const int T0 = int((long long)ntiles * blockIdx.x / gridDim.x);
  const int T1 = int((long long)ntiles * (blockIdx.x + 1) / gridDim.x);
  const int cpt = (K >> 5) / U;  // units per tile
  const int nunits = (T1 - T0) * cpt;
  const int u0 = int((long long)nunits * w / nw), u1 = int((long long)nunits * (w + 1) / nw);
  const bool arow = col < g.M;
  const uint4 zero = {0u, 0u, 0u, 0u};
  const uint4* xrow = xs + col * ldx + kg;
  // fragment-order copy (contiguous 1 KB per k-step) when the context made one
  const int ksteps = K >> 5;
  const uint16_t* wbase = g.Wp ? (const uint16_t*)g.Wp + l * 8
                               : (const uint16_t*)g.W0 + (long long)col * K + kg * 8;
  uint64_t best[4] = {0ull, 0ull, 0ull, 0ull};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  auto fold = [&](int tile) {  // full 16x16 sums of `tile` are in acc
    const int n = tile * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = kg * 4 + i;
      if (row < g.M) {
        if (g.logits) g.logits[(long long)row * g.ldl + n] = acc[i];
        const uint64_t key = argmax_key(acc[i], n);
        best[i] = key > best[i] ? key : best[i];
      }
    }
  };
  auto issue = [&](uint4 (&b)[U], int u) {
    const int tile = T0 + u / cpt, s0 = (u % cpt) * U;
    if (g.Wp) {
      const uint16_t* wp = wbase + ((long long)tile * ksteps + s0) * 512;
#pragma unroll
      for (int j = 0; j < U; ++j) b[j] = ld_stream(wp + j * 512);
    } else {
      const uint16_t* wp = wbase + (long long)tile * 16 * K + s0 * 32;
#pragma unroll
      for (int j = 0; j < U; ++j) b[j] = ld_stream(wp + j * 32);
    }
  };
  auto consume = [&](uint4 (&b)[U], int u) {
    const int c = u % cpt, tile = T0 + u / cpt;
    const uint4* xr = xrow + c * U * 4;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint4 a = arow ? xr[j * 4] : zero;
      acc = mfma16(a, b[j], acc);
    }
    if (c == cpt - 1 || u == u1 - 1) {
      const bool head = (u - c < u0);      // the tile began before this wave's range
      const bool tail = (c != cpt - 1);    // the tile continues after it
      if (!head && !tail) {
        fold(tile);
      } else {
        const int slot = head ? 0 : 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) part[w][slot][i][l] = acc[i];
        if (l == 0) part_tile[w][slot] = tile;
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  uint4 b0[U], b1[U];
  if (u0 < u1) issue(b0, u0);
  for (int u = u0; u < u1; u += 2) {
    if (u + 1 < u1) issue(b1, u + 1);
    consume(b0, u);
    if (u + 1 < u1) {
      if (u + 2 < u1) issue(b0, u + 2);
      consume(b1, u + 1);
    }
  }
  __syncthreads();
  // tiles cut between waves: the wave holding the tile's first unit (its tail
  // slot) adds the head slots of the following waves that hold the same tile.
  // Waves with an empty run (fewer units than waves) hold nothing and are
  // passed over: the tile's later pieces can lie beyond them.
  const int tt = part_tile[w][1];
  if (tt >= 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = part[w][1][i][l];
    for (int v = w + 1; v < nw; ++v) {
      if (int((long long)nunits * v / nw) == int((long long)nunits * (v + 1) / nw)) continue;
      if (part_tile[v][0] != tt) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += part[v][0][i][l];
      if (part_tile[v][1] == tt) break;  // cannot happen: a run longer than a tile
    }
    fold(tt);
  }
  // row maxima: 16 lanes per row group, then across waves, one atomic per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    best[i] = row16_max_key(best[i]);
    if (col == 0) s_best[w][kg * 4 + i] = best[i];
  }
  __syncthreads();
  if (threadIdx.x < g.M) {
    uint64_t b = 0ull;
    for (int v = 0; v < nw; ++v) b = s_best[v][threadIdx.x] > b ? s_best[v][threadIdx.x] : b;
    g.keys[(long long)threadIdx.x * g.parts + blockIdx.x] = b;
  }
}

// ---------------------------------------------------------------------------
// bf16, M > 16: BM x BN tiles over k-tiles of 64 in an S-stage LDS ring filled
// by global_load_lds_dwordx4 (global -> LDS with no staging registers).
// S = 3 prefetches one k-tile further; the 64-row tiles that use it still fit
// two workgroups per CU.
//
// One DMA instruction moves 8 whole tile rows: 128 bytes (64 bf16 of k) per
// row, 16 bytes per lane.  Rows split into half lines (32-wide k-tiles) stream
// ~1.4x slower through this path (measured on a loads-only copy of the loop).
// LDS: tile row r takes 128 bytes and its 16-byte chunk c sits at slot
// c ^ ((r >> 1) & 7).  gfx950 serves a 16-byte LDS read 16 lanes per clock
// over 64 banks (256 bytes); the 16 lanes of a fragment read take rows
// r0 .. r0+15 at one chunk, and under this key those fall on 16 distinct
// 16-byte bank groups (with c ^ (r & 7), rows r and r + 8 shared one: a
// two-way conflict on every read).  Fragment rows r0 + 16i share (r >> 1) & 7,
// so fragment i is one base offset plus i * 2 KB.
//
// A k-tile feeds two 32-wide MFMA substeps; the fragments of the next substep
// are read while the MFMAs of the current one run, and there is one barrier
// per k-tile.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz64(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Split of a dense tiled product with a row map, chosen on the device from the
// rows it computes (the map's count is known only there): the T = row tiles x
// column tiles (in whole groups of 8, see the block mapping) run as
// ks = floor(slots / T) copies over k when T < slots, each of at least
// PE_SPLITK_MIN_KTILES k-tiles and within `cap` copies of the partial buffer.
struct TilePlan { int mt, per, ks; };
__host__ __device__ inline TilePlan tile_plan(int rows, int BM, int ntiles, int nk, int slots, int cap) {
  TilePlan p;
  p.mt = (rows + BM - 1) / BM;
  p.per = p.mt * ((ntiles + 7) / 8) * 8;
  p.ks = 1;
  if (slots > 0 && p.per > 0 && p.per < slots) {
    int ks = slots / p.per;
    const int kmax = nk / PE_SPLITK_MIN_KTILES;
    ks = ks < kmax ? ks : kmax;
    ks = ks < cap ? ks : cap;
    p.ks = ks > 1 ? ks : 1;
  }
  return p;
}


template <int EPI, int AL, int BMAP, int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tiled_kernel(GemmArgs g, int mtiles, int ntiles, int tail0, int dslots, int dcap) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int TI = BM / WM / 16, TJ = BN / WN / 16;   // MFMA tiles per wave
  // DMA instructions per wave per k-tile; A's row groups may not split evenly
  // (224-row tiles: 28 groups over 8 waves), then the last one is predicated
  constexpr int LA = (BM / 8 + NW - 1) / NW, LB = BN / 8 / NW;
  constexpr bool LA_EVEN = LA * 8 * NW == BM;
  static_assert(LB * 8 * NW == BN, "tile columns must split over the waves");
  static_assert(LA_EVEN || S == 2, "uneven A rows only with two stages (the step waits drain every DMA)");
  static_assert((BN / WN) % 32 == 0, "a wave's columns must be whole 32-column blocks");
  constexpr int STAGE = (BM + BN) * 128;                // bytes per stage
  static_assert(S == 2 || S == 3, "two or three stages");
  // distinct LDS objects, so the compiler sees that the DMA into one stage and
  // the fragment reads of another do not alias
  __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE], st1[STAGE], st2[S == 3 ? STAGE : 16];

  // split-K (E_PART): the grid holds ksplit copies of the tile grid, copy ks
  // summing k-tiles [ks nk / ksplit, (ks + 1) nk / ksplit); the copies are
  // multiples of 8 workgroups, so the XCD of a workgroup is unchanged
  int bid = blockIdx.x, ks = 0, kbase = 0, nk = g.K / 64, mt, nt;
  // rows computed: those of active requests (occupancy below the captured
  // batch skips the rest) and, with a row map, the compact rows, compact row
  // m standing for row rmap[m] of A and of the output; tiles past them exit
  int rows = active_rows(g.nact, g.rpr, g.M);
  if (g.rmap) rows = min(rows, *g.rcount);
  int mtg = mtiles;        // row tiles of the block mapping
  bool part = EPI == E_PART;  // write fp32 partials instead of the epilogue
  if constexpr (EPI == E_PART) {
    const int per = mtiles * ((ntiles + 7) / 8) * 8;
    ks = bid / per;
    bid -= ks * per;
    kbase = ks * nk / g.ksplit;
    nk = (ks + 1) * nk / g.ksplit - kbase;
  } else if constexpr (EPI != E_ARGMAX) {
    if (dslots > 0) {  // the split is planned here, from the rows computed
      const TilePlan p = tile_plan(rows, BM, ntiles, nk, dslots, dcap);
      if (bid >= p.per * p.ks) return;
      mtg = p.mt;
      if (p.ks > 1) {
        part = true;
        ks = bid / p.per;
        bid -= ks * p.per;
        kbase = ks * nk / p.ks;
        nk = (ks + 1) * nk / p.ks - kbase;
      }
    }
  }
  // LM head with a split tail (E_ARGMAX, tail0 < ntiles): column tiles
  // [0, tail0) run whole; each tile of [tail0, ntiles) runs as ksplit k-range
  // pieces after them, which write fp32 partial tiles for argmax_tail_kernel.
  // Piece u = (column tile - tail0) * ksplit + split; the mtiles pieces that
  // share a weight k-range sit 8 workgroups apart, on one XCD.
  const int main_grid = mtiles * ((tail0 + 7) / 8) * 8;
  const bool tail = EPI == E_ARGMAX && bid >= main_grid;
  if (tail) {
    const int t = bid - main_grid, j = t >> 3;
    const int u = (j / mtiles) * 8 + (t & 7);
    if (u >= (ntiles - tail0) * g.ksplit) return;  // padding workgroup
    mt = j % mtiles;
    nt = tail0 + u / g.ksplit;
    ks = u % g.ksplit;
    kbase = ks * nk / g.ksplit;
    nk = (ks + 1) * nk / g.ksplit - kbase;
  } else {
    const int j = bid >> 3;
    mt = j % mtg;
    nt = (j / mtg) * 8 + (bid & 7);
    if (nt >= tail0) return;  // padding workgroup of the XCD-aligned grid
  }
  const int m0 = mt * BM, n0 = nt * BN;
  if (m0 >= rows) return;
  auto out_row = [&](int m) { return g.rmap ? g.rmap[m] : m; };
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, col = l & 15, kg = l >> 4;
  const int wm = w / WN, wn = w % WN;

  // DMA instruction i of this wave fills tile rows r = 8 (w + NW i) + l/8
  // (lane l), LDS slot l%8, i.e. global chunk (l%8) ^ ((r >> 1) & 7); since
  // the group starts 8-aligned, (r >> 1) & 7 = 4 ((w + NW i) & 1) + (l/8) / 2
  ARow<uint16_t, AL> ar[LA];
  const uint16_t* bp[LB];
  const int lr = l >> 3;
  auto lchunk = [&](int i) { return ((l & 7) ^ ((((w + NW * i) & 1) << 2) | (lr >> 1))) * 8; };
  int lca[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    ar[i].init(g, out_row(min(m0 + 8 * (w + NW * i) + lr, rows - 1)));
    lca[i] = lchunk(i);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i)
    bp[i] = weight_row<uint16_t, BMAP>(g, min(n0 + 8 * (w + NW * i) + lr, g.N - 1)) + lchunk(i);
  auto issue = [&](unsigned char* st, int kt) {
    const int k0 = (kbase + kt) * 64;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      if (LA_EVEN || w + NW * i < BM / 8)
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)ar[i].at(k0 + lca[i], g.d),
            (__attribute__((address_space(3))) void*)(st + (w + NW * i) * 1024), 16, 0, 0);
    // the LM head's weights stream once per launch: non-temporal (cache
    // policy nt), so they do not push A and the layer weights out of the caches
    constexpr int BPOL = EPI == E_ARGMAX ? 2 : 0;
#pragma unroll
    for (int i = 0; i < LB; ++i)
      __builtin_amdgcn_global_load_lds(
          (__attribute__((address_space(1))) void*)(bp[i] + k0),
          (__attribute__((address_space(3))) void*)(st + BM * 128 + (w + NW * i) * 1024), 16, 0, BPOL);
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  // substep s reads 16-byte chunk 4s + kg of each fragment row
  const int ar0 = wm * (BM / WM) + col, br0 = wn * (BN / WN) + col;
  const int aoff0 = swz64(ar0, kg), aoff1 = swz64(ar0, 4 + kg);
  const int boff0 = BM * 128 + swz64(br0, kg), boff1 = BM * 128 + swz64(br0, 4 + kg);

  issue(st0, 0);
  if (1 < nk) issue(st1, 1);
  if (S == 3 && 2 < nk) issue(st2, 2);
  uint4 fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];
  // k-tile 0 must land; the later prologue tiles may stay in flight
  if (S == 3 && 2 < nk) wait_vmcnt<2 * (LA + LB)>();
  else if (1 < nk) {
    // this wave's DMAs of k-tile 1 may stay in flight (one fewer A row group
    // for the waves past the last one of an uneven split)
    if (LA_EVEN || w + NW * (LA - 1) < BM / 8) wait_vmcnt<LA + LB>();
    else wait_vmcnt<LA - 1 + LB>();
  } else {
    wait_vmcnt<0>();
  }
  // Plain s_barrier: this wave's DMA of the stage has landed (the wait above).
  // A fenced __syncthreads would also wait for the DMA still in flight.
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < TI; ++i) fa0[i] = *reinterpret_cast<const uint4*>(st0 + aoff0 + i * 2048);
#pragma unroll
  for (int jj = 0; jj < TJ; ++jj) fb0[jj] = *reinterpret_cast<const uint4*>(st0 + boff0 + jj * 2048);

  auto mfmas = [&](const uint4 (&xa)[TI], const uint4 (&xb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = mfma16(xa[i], xb[jj], acc[i][jj]);
  };
  // k-tile kt in stage `cur`; on entry fa0/fb0 hold its first substep.  `cur`
  // and `nxt` are distinct stages; saying so (restrict) lets the compiler keep
  // the DMA into `cur` in flight across the reads of `nxt`.
  auto step = [&](unsigned char* __restrict__ cur, const unsigned char* __restrict__ nxt, int kt) {
#pragma unroll
    for (int i = 0; i < TI; ++i) fa1[i] = *reinterpret_cast<const uint4*>(cur + aoff1 + i * 2048);
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) fb1[jj] = *reinterpret_cast<const uint4*>(cur + boff1 + jj * 2048);
    mfmas(fa0, fb0);
    wait_lgkm0();  // this wave's reads of `cur` are done
    if (kt + 1 < nk) {
      // the DMA of k-tile kt+1 (this wave's part) has landed; with three stages
      // the one of kt+2 may still be in flight
      if (S == 3 && kt + 2 < nk) wait_vmcnt<LA + LB>();
      else wait_vmcnt<0>();
      asm volatile("s_barrier" ::: "memory");  // ... everyone's, and `cur` is free
      if (kt + S < nk) issue(cur, kt + S);
#pragma unroll
      for (int i = 0; i < TI; ++i) fa0[i] = *reinterpret_cast<const uint4*>(nxt + aoff0 + i * 2048);
#pragma unroll
      for (int jj = 0; jj < TJ; ++jj) fb0[jj] = *reinterpret_cast<const uint4*>(nxt + boff0 + jj * 2048);
    }
    mfmas(fa1, fb1);
  };
  if constexpr (S == 2) {
    for (int kt = 0; kt < nk; kt += 2) {
      step(st0, st1, kt);
      if (kt + 1 < nk) step(st1, st0, kt + 1);
    }
  } else {
    for (int kt = 0; kt < nk; kt += 3) {
      step(st0, st1, kt);
      if (kt + 1 < nk) step(st1, st2, kt + 1);
      if (kt + 2 < nk) step(st2, st0, kt + 2);
    }
  }

  // lane (kg, col) holds C[row 4kg + r of MFMA tile i][col of tile jj]
  if (EPI != E_ARGMAX && part) {
    float* P = g.part + (long long)ks * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / WM) + i * 16 + kg * 4 + r;
        if (m >= rows) continue;  // partials by compact row: the reduction maps them
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj) {
          const int n = n0 + wn * (BN / WN) + jj * 16 + col;
          if (n < g.N) P[(long long)m * g.N + n] = acc[i][jj][r];
        }
      }
  } else if constexpr (EPI == E_PART) {
    // (always split: handled above)
  } else if constexpr (EPI == E_ARGMAX) {
    if (tail) {
      // partial tile [BM][BN] of piece ks of tail tile (nt - tail0, mt)
      float* P = g.part + ((long long)((nt - tail0) * mtiles + mt) * g.ksplit + ks) * (BM * BN);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lrow = wm * (BM / WM) + i * 16 + kg * 4 + r;
#pragma unroll
          for (int jj = 0; jj < TJ; ++jj) P[lrow * BN + wn * (BN / WN) + jj * 16 + col] = acc[i][jj][r];
        }
      return;
    }
    __syncthreads();  // every fragment read is done; no DMA is in flight
    uint64_t* s_best = reinterpret_cast<uint64_t*>(st0);  // [WN][BM]
    static_assert(WN * BM * 8 <= STAGE, "argmax scratch fits one stage");
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = wm * (BM / WM) + i * 16 + kg * 4 + r;
        uint64_t best = 0ull;
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj) {
          const int n = n0 + wn * (BN / WN) + jj * 16 + col;
          if (n < g.N) {
            if (g.logits && m0 + lrow < g.M) g.logits[(long long)(m0 + lrow) * g.ldl + n] = acc[i][jj][r];
            const uint64_t k = argmax_key(acc[i][jj][r], n);
            best = k > best ? k : best;
          }
        }
        best = row16_max_key(best);
        if (col == 0) s_best[wn * BM + lrow] = best;
      }
    __syncthreads();
    for (int lr = tid; lr < BM; lr += NT) {
      if (m0 + lr < g.M) {
        uint64_t bk = s_best[lr];
        for (int v = 1; v < WN; ++v) bk = s_best[v * BM + lr] > bk ? s_best[v * BM + lr] : bk;
        g.keys[(long long)(m0 + lr) * g.parts + nt] = bk;
      }
    }
  } else if constexpr (EPI != E_QKV && (BN / WN == 32 || BN / WN == 64)) {
    // Row-vector epilogue.  Each wave stages its fp32 (BM/WM) x (BN/WN) tile
    // in a private LDS region (the stages are free: every fragment read has
    // returned and no DMA is in flight after the barrier), then writes rows as
    // 16-byte pieces of 8 bf16 (and reads the residual the same way).
    // Rows 4kg+r of a C fragment land 4 rows apart; a 64-float row stride
    // gets an XOR of 16 (row/4 % 4) floats, a 32-float one a 4-float pad,
    // so the 4 row groups of a store fall in distinct banks.
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int LD = WTN == 64 ? 64 : WTN + 4;
    constexpr int WBYTES = WTM * LD * 4;
    constexpr int PER = STAGE / WBYTES;  // wave regions per stage object
    static_assert(PER >= 1 && (NW + PER - 1) / PER <= S, "wave regions fit the stages");
    auto cpos = [&](int r, int c) { return r * LD + (WTN == 64 ? (c ^ (((r >> 2) & 3) << 4)) : c); };
    __syncthreads();
    unsigned char* reg = (w / PER == 0) ? st0 : (w / PER == 1 ? st1 : st2);
    float* ct = reinterpret_cast<float*>(reg + (w % PER) * WBYTES);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int jj = 0; jj < TJ; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) ct[cpos(i * 16 + kg * 4 + r, jj * 16 + col)] = acc[i][jj][r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int mw = m0 + wm * WTM, nw0 = n0 + wn * WTN;
    if constexpr (EPI == E_SILU) {
      // logical columns (32q + c, 32q + 16 + c) -> output column nw0/2 + 16q + c
      constexpr int SEG = WTN / 16;  // 8-output pieces per row
      for (int e = l; e < WTM * SEG; e += 64) {
        const int rr = e / SEG, sg = e % SEG, q = sg >> 1, c0 = (sg & 1) * 8;
        const int m = mw + rr;
        if (m >= rows || nw0 + 32 * q >= g.N) continue;
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float gt = ct[cpos(rr, 32 * q + c0 + t)], up = ct[cpos(rr, 32 * q + 16 + c0 + t)];
          v[t] = gt / (1.0f + expf(-gt)) * up;
        }
        uint4 o;
        o.x = f2bf2(v[0], v[1]); o.y = f2bf2(v[2], v[3]); o.z = f2bf2(v[4], v[5]); o.w = f2bf2(v[6], v[7]);
        *reinterpret_cast<uint4*>((uint16_t*)g.out + (long long)out_row(m) * g.ldo + (nw0 >> 1) + 16 * q + c0) = o;
      }
    } else {
      constexpr int SEG = WTN / 8;
      for (int e = l; e < WTM * SEG; e += 64) {
        const int rr = e / SEG, c0 = (e % SEG) * 8;
        const int m = mw + rr, n = nw0 + c0;
        if (m >= rows || n >= g.N) continue;
        const float4 a0 = *reinterpret_cast<const float4*>(ct + cpos(rr, c0));
        const float4 a1 = *reinterpret_cast<const float4*>(ct + cpos(rr, c0 + 4));
        float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const long long o = (long long)out_row(m) * g.ldo + n;
        if constexpr (EPI == E_RESID) {
          const uint4 rv = *reinterpret_cast<const uint4*>((const uint16_t*)g.resid + o);
          const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[2 * t] += __uint_as_float(rw[t] << 16);
            v[2 * t + 1] += __uint_as_float(rw[t] & 0xFFFF0000u);
          }
        }
        uint4 ov;
        ov.x = f2bf2(v[0], v[1]); ov.y = f2bf2(v[2], v[3]); ov.z = f2bf2(v[4], v[5]); ov.w = f2bf2(v[6], v[7]);
        *reinterpret_cast<uint4*>((uint16_t*)g.out + o) = ov;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mc = m0 + wm * (BM / WM) + i * 16 + kg * 4 + r;
        if (mc >= rows) continue;
        const int m = out_row(mc);
        if (EPI == E_STORE || EPI == E_RESID) {
#pragma unroll
          for (int jj = 0; jj < TJ; ++jj) {
            const int n = n0 + wn * (BN / WN) + jj * 16 + col;
            if (n < g.N) epi_one<uint16_t, EPI>(g, m, n, acc[i][jj][r]);
          }
        } else {
          // a wave's BN/2 columns are whole 32-column blocks: tiles (2q, 2q+1) pair up
#pragma unroll
          for (int q = 0; q < TJ / 2; ++q) {
            const int nb = n0 + wn * (BN / WN) + q * 32;
            if (nb < g.N) epi_pair<uint16_t, EPI>(g, m, nb, col, acc[i][2 * q][r], acc[i][2 * q + 1][r]);
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 LM head, 17..128 rows: a deep ring of 32-wide k-steps in MFMA
// fragment order
// ---------------------------------------------------------------------------
// WGPC persistent workgroups per CU, each over an equal, contiguous range of
// 16-column tiles (so no round of tiles runs on a few CUs while the rest
// idle), taken in chunks of at most 16 tiles (256 columns) with all M <= BM
// rows.  Each stage
// holds one 32-wide k-step of both operands as 1 KB fragment blocks: block
// (16-row tile t) has lane l's 16 bytes at 16 l, i.e. rows 16t + l%16 and
// k-chunk l/16, which is the operand layout of v_mfma_f32_16x16x32_bf16, so
// every fragment read is one contiguous 1 KB per wave (no bank conflicts, no
// swizzle).  The weight blocks come from the fragment-order copy (each DMA
// instruction moves one whole 1 KB block); the row blocks gather 16 rows x
// 64 B of the row-major operand.  A stage is (BM + 256) x 64 B, so several
// k-steps per CU are in flight (two workgroups of three stages, or one of
// six): with 17..128 rows a k-step is little MFMA work, and the weight stream
// from HBM needs that depth to hide its latency.  The
// pipeline runs across chunk boundaries (step gs = chunk * ksteps + k-step);
// at a chunk's last k-step the tile's row maxima fold into a running
// (value, index) key per row, written once per workgroup at the end.
// Fragment reads run one k-step ahead of the MFMAs.
template <int BM, int WM, int WN, int S, int WGPC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WM * WN * WGPC / 4, WM * WN * WGPC / 4)))
void lmhead_ring_kernel(GemmArgs g) {
  constexpr int BN = 256, CT = BN / 16, NW = WM * WN, NT = 64 * NW;
  constexpr int TI = BM / WM / 16, TJ = BN / WN / 16;  // MFMA tiles per wave
  static_assert(TI * 16 * WM == BM && TJ * 16 * WN == BN, "whole MFMA tiles per wave");
  static_assert(NT >= BM, "one thread per row keeps the row's running key");
  constexpr int NA = BM / 16, NB = CT, NBLK = NA + NB;  // fragment blocks per stage
  constexpr int Q = (NBLK + NW - 1) / NW;              // DMAs per wave per stage
  constexpr int STAGE = NBLK * 1024;
  static_assert(S >= 3 && S <= 7 && WGPC * (S * STAGE + WN * BM * 8) <= 160 * 1024, "rings fit the LDS");
  static_assert((S - 1) * Q < 64, "ring depth within the vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[S * STAGE];
  __shared__ uint64_t s_best[WN * BM];

  if (active_rows(g.nact, g.rpr, g.M) <= 0) return;
  const int ksteps = g.K / 32, ntw = g.N / 16, G = gridDim.x, gid = blockIdx.x;
  const int t0 = int((long long)gid * ntw / G), nt = int((long long)(gid + 1) * ntw / G) - t0;
  const int nch = (nt + CT - 1) / CT, total = nch * ksteps;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, col = l & 15, kg = l >> 4;
  const int wm = w / WN, wn = w % WN;
  auto chunk_first = [&](int c) { return t0 + c * nt / nch; };

  // DMA q of this wave fills block j = w + NW q of each stage (a wave whose
  // block would lie past the last one repeats its first: the same bytes to
  // the same place, so every wave issues Q DMAs per stage and one vmcnt
  // serves all).  Row block t: lane l loads A[16t + l%16][32 s + 8 (l/16)];
  // weight block u: the fragment-order copy's block (tile u of the chunk, s),
  // past the chunk's last tile that tile again (its columns are not used).
  const uint16_t* asrc[Q];
  int wu_[Q];
  uint32_t dst[Q];
  const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = wu + NW * q < NBLK ? wu + NW * q : wu;
    dst[q] = uint32_t(j * 1024);
    wu_[q] = j - NA;
    asrc[q] = (const uint16_t*)g.A + (long long)min(16 * j + col, g.M - 1) * g.lda + 8 * kg;
  }
  const uint16_t* Wp = (const uint16_t*)g.Wp + 8 * l;
  const uint32_t base = lds_addr(ring);
  // The DMAs run through the steps in order (the prologue's, then one step
  // ahead of each k-step), so the issue position (chunk ic, k-step is) is
  // kept as counters, and each DMA's source at k-step 0 of the chunk (src0)
  // and its advance per k-step (32 elements of a row, or one 512-element
  // weight block) are set once per chunk: no division on the per-step path.
  int ic = 0, is = 0;
  const uint16_t* src0[Q];
  int adv[Q];
  auto set_chunk = [&](int c) {
    const int c0 = chunk_first(c), c1 = chunk_first(c + 1);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const bool isa = wu_[q] < 0;
      src0[q] = isa ? asrc[q] : Wp + (long long)min(c0 + wu_[q], c1 - 1) * ksteps * 512;
      adv[q] = isa ? 32 : 512;
    }
  };
  set_chunk(0);
  auto issue = [&](int slot) {
#pragma unroll
    for (int q = 0; q < Q; ++q) dma16(src0[q] + (long long)is * adv[q], base + slot * STAGE + dst[q]);
    if (++is == ksteps) {
      is = 0;
      if (++ic < nch) set_chunk(ic);
    }
  };
  // at most n later steps of this wave's DMAs still in flight
  auto wait_steps = [&](int n) {
    if (n >= 6) wait_vmcnt<(S > 6 ? 6 : 0) * Q>();
    else if (n == 5) wait_vmcnt<(S > 5 ? 5 : 0) * Q>();
    else if (n == 4) wait_vmcnt<(S > 4 ? 4 : 0) * Q>();
    else if (n == 3) wait_vmcnt<(S > 3 ? 3 : 0) * Q>();
    else if (n == 2) wait_vmcnt<2 * Q>();
    else if (n == 1) wait_vmcnt<Q>();
    else wait_vmcnt<0>();
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int aoff = wm * TI * 1024 + 16 * l, boff = (NA + wn * TJ) * 1024 + 16 * l;
  uint4 fa[2][TI], fb[2][TJ];
  auto read = [&](int buf, const unsigned char* st) {
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[buf][i] = *reinterpret_cast<const uint4*>(st + aoff + i * 1024);
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) fb[buf][jj] = *reinterpret_cast<const uint4*>(st + boff + jj * 1024);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = mfma16(fa[buf][i], fb[buf][jj], acc[i][jj]);
  };
  uint64_t run = 0ull;  // thread tid < BM: the running key of row tid
  // after a chunk's last k-step: lane (kg, col) holds C[row 4kg + r of MFMA
  // tile i][column col of tile jj]; the row maxima over the chunk's columns
  // fold into `run`, and the accumulators restart
  auto fold = [&](int c) {
    const int c0 = chunk_first(c), ncol = (chunk_first(c + 1) - c0) * 16;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = wm * (BM / WM) + i * 16 + kg * 4 + r;
        uint64_t best = 0ull;
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj) {
          const int cc = (wn * TJ + jj) * 16 + col, n = c0 * 16 + cc;
          if (cc < ncol) {
            if (g.logits && lrow < g.M) g.logits[(long long)lrow * g.ldl + n] = acc[i][jj][r];
            const uint64_t k = argmax_key(acc[i][jj][r], n);
            best = k > best ? k : best;
          }
        }
        best = row16_max_key(best);
        if (col == 0) s_best[wn * BM + lrow] = best;
      }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the keys are in LDS (lgkmcnt(0)); a plain barrier, so the DMAs in
    // flight stay in flight
    wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
    if (tid < BM) {
#pragma unroll
      for (int v = 0; v < WN; ++v) run = s_best[v * BM + tid] > run ? s_best[v * BM + tid] : run;
    }
    // s_best is written again only after the next chunk's k-steps, each of
    // which passes a barrier
  };

  // prologue: every slot filled, step 0 read
#pragma unroll
  for (int j = 0; j < S; ++j)
    if (j < total) issue(j);
  wait_steps(total - 1 < S - 1 ? total - 1 : S - 1);
  asm volatile("s_barrier" ::: "memory");
  read(0, ring);
  // step gs: its fragments are in registers (buffer gs & 1)
  int slot = 0, ks = 0, ch = 0;
  auto iter = [&](int gs, int buf) {
    if (gs + 1 < total) {
      const int later = total - 2 - gs;
      wait_steps(later < S - 2 ? later : S - 2);  // step gs+1 has landed (this wave's part)
      // everyone's part has landed, and everyone has read step gs's slot
      // (before this barrier), which the next DMA refills
      asm volatile("s_barrier" ::: "memory");
      if (gs + S < total) issue(slot);  // step gs + S
      slot = slot + 1 == S ? 0 : slot + 1;
      read(buf ^ 1, ring + slot * STAGE);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(buf);
    __builtin_amdgcn_sched_barrier(0);
    if (++ks == ksteps) {
      fold(ch++);
      ks = 0;
    }
  };
  for (int gs = 0; gs < total; gs += 2) {
    iter(gs, 0);
    if (gs + 1 < total) iter(gs + 1, 1);
  }
  if (tid < BM && tid < g.M) g.keys[(long long)tid * g.parts + gid] = run;
}

// ---------------------------------------------------------------------------
// fp32: plain FMA, 16x32 output tile per workgroup
// ---------------------------------------------------------------------------
template <int EPI, int AL, int BMAP>
__global__ __launch_bounds__(512) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float tile[16 * 33];
  const int i = threadIdx.x >> 5, c = threadIdx.x & 31;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 32;
  const int m = m0 + i, n = n0 + c;
  float s = 0.f;
  if (m < g.M && n < g.N) {
    const float* w = weight_row<float, BMAP>(g, n);
    ARow<float, AL> ar;
    ar.init(g, m);
    for (int k = 0; k < g.K; ++k) s = fmaf(*ar.at(k, g.d), w[k], s);
  }
  tile[i * 33 + c] = s;
  __syncthreads();
  if (EPI == E_ARGMAX) {
    epilogue_argmax(g, tile, 33, m0, 16, n0, 32, blockIdx.x);
  } else {
    epilogue<float, EPI>(g, tile, 33, m0, 16, n0, 32);
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <typename F>
static hipError_t set_lds(F* fn, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

// ---------------------------------------------------------------------------
// Fragment-order copy of a row-major weight [N, K] (bf16): 1 KB block (t, s)
// holds, for lane l, W[16t + l%16][32s + 8(l/16) .. +8] at bytes 16 l.  A wave
// that streams tile t then reads one contiguous 1 KB per MFMA k-step.
// ---------------------------------------------------------------------------
template <int BMAP>
__global__ __launch_bounds__(256) void pack_frag16_kernel(GemmArgs g, uint4* __restrict__ out) {
  const int ks = g.K >> 5;
  const long long total = (long long)(g.N >> 4) * ks * 64;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = int(i & 63);
    const long long ts = i >> 6;
    const int s = int(ts % ks);
    const int t = int(ts / ks);
    const uint16_t* row = weight_row<uint16_t, BMAP>(g, t * 16 + (l & 15));
    out[i] = ld16(row + s * 32 + (l >> 4) * 8);
  }
}

hipError_t launch_pack_frag16(int bmap, const GemmArgs& g, void* out, hipStream_t st) {
  const long long total = (long long)(g.N / 16) * (g.K / 32) * 64;
  long long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (bmap == B_QKV)
    hipLaunchKernelGGL(pack_frag16_kernel<B_QKV>, dim3(unsigned(blocks)), dim3(256), 0, st, g, (uint4*)out);
  else if (bmap == B_GATEUP)
    hipLaunchKernelGGL(pack_frag16_kernel<B_GATEUP>, dim3(unsigned(blocks)), dim3(256), 0, st, g, (uint4*)out);
  else
    hipLaunchKernelGGL(pack_frag16_kernel<B_PLAIN>, dim3(unsigned(blocks)), dim3(256), 0, st, g, (uint4*)out);
  return hipGetLastError();
}

// Which kernel serves a bf16 GEMM of this shape (M rows, N logical columns).
//  * LM head (E_ARGMAX): the LDS-resident wide kernel up to 16 rows; tiled
//    64x256, 128x256 or 256x256 above (a 64-row tile streams the weights once
//    at ~4.9 TB/s where the split-K kernel managed ~1.4 TB/s).
//  * Dense, up to 16 rows: split-K over waves (weights from the fragment-order copy).
//  * Dense, 17..64 rows: tiled 64x128 when there are >= 32 column tiles,
//    split-K otherwise (few tiles leave most CUs idle).
//  * Dense, 65..256 rows (more: pe_mm.hip): tiled 128x128 with two stages and two workgroups per CU
//    when those tiles outnumber the CUs; otherwise 64x128 tiles (three stages,
//    two workgroups per CU), which spread a small grid over more CUs (fc, O and
//    down at c=64, cache-cold weights: 50/38/69 us against 59/43/76 us).
#ifndef PE_LM_RING
#define PE_LM_RING 1
#endif
enum Variant { V_WIDE, V_RING, V_SKINNY, V_A64, V_A128, V_A192, V_A224, V_A256, V_D64, V_D128S2 };

static Variant pick(int epi, int M, int N, int K, int num_cus) {
  if (epi == E_ARGMAX) {
    const size_t wide_lds = size_t(M) * (K / 8 + 1) * 16;
    if (M <= 16 && wide_lds <= 140 * 1024) return V_WIDE;
    if (PE_LM_RING && M <= 128 && K % 32 == 0) return V_RING;
    if (M <= 64) return V_A64;
    if (M > 384 && M <= 448) return V_A224;  // two 224-row tiles instead of 256 + 192 valid rows
    if (M > 128 && M <= 192) return V_A192;  // one 192-row tile, not 256 with 64+ idle rows
    return M <= 128 ? V_A128 : V_A256;
  }
  if (M <= 16) return V_SKINNY;
  if (M <= 64) return (N + 127) / 128 >= 32 ? V_D64 : V_SKINNY;
  const long long tiles = (long long)((M + 127) / 128) * ((N + 127) / 128);
  return tiles > num_cus ? V_D128S2 : V_D64;
}
constexpr int kArgmaxBN = 256;  // columns per tile of every tiled LM-head variant

int gemm_argmax_parts(int dtype, int M, int N, int K, int num_cus) {
  if (dtype != 1) return (N + 31) / 32;
  switch (pick(E_ARGMAX, M, N, K, num_cus)) {
    case V_WIDE: return std::min(num_cus, N / 16);
    case V_RING: return std::min((M <= 64 ? 2 : 1) * num_cus, N / 16);  // run_ring's grid
    case V_SKINNY: return (N + 15) / 16;
    default: return (N + kArgmaxBN - 1) / kArgmaxBN;
  }
}

bool gemm_folds_norm(int dtype, int M, int K) {
  return dtype == 1 && M >= 1 && M <= 16 && K >= 32 && K % 32 == 0 && K / 16 <= kSsqMaxParts;
}

template <int EPI, int AL, int BMAP, int MT>
static hipError_t run_skinny(const GemmArgs& g, hipStream_t st) {
  constexpr int NTW = BMAP == B_PLAIN ? 1 : (BMAP == B_GATEUP && MT == 1) ? PE_SKINNY_NTW_GU : 2;
  constexpr int U = NTW + MT <= 2 ? PE_SKINNY_U_NARROW : NTW + MT <= 3 ? 8 : NTW + MT <= 5 ? PE_SKINNY_U_WIDE : 3;
  const int ksteps = g.K / 32;
  int nw = ksteps / 4;
  nw = nw < 1 ? 1 : (nw > 16 ? 16 : nw);
  while (nw > 1 && nw * MT * NTW > 128) --nw;
  size_t lds = size_t(nw) * MT * NTW * 256 * 4 + size_t(MT * 16) * (NTW * 16 + 4) * 4;
  const int grid = (g.N + NTW * 16 - 1) / (NTW * 16);
  if (EPI == E_ARGMAX && g.parts != grid) return hipErrorInvalidValue;
  if (g.rmap) return hipErrorInvalidValue;  // row maps: the tiled and large-batch kernels only
  // folded RMSNorm: the producer writes one partial per 16-column tile
  if (g.ssq_out && (MT != 1 || NTW != 1 || !(EPI == E_STORE || EPI == E_RESID) || g.ssq_n != grid))
    return hipErrorInvalidValue;
  auto launch = [&](auto fn) -> hipError_t {
    hipError_t e = set_lds(fn, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * nw), lds, st, g);
    return hipGetLastError();
  };
  if (g.norm_gain) {
    if constexpr (MT == 1 && AL == A_PLAIN && (EPI == E_QKV || EPI == E_SILU)) {
      if (!g.ssq_in || g.ssq_n < 1 || g.ssq_n > kSsqMaxParts || 16 * g.ssq_n > 256 * nw || 2 * g.K > 1024 * nw ||
          g.K % 32 || g.M > 16)
        return hipErrorInvalidValue;
      // partials from byte 0 (their DMA slots, 1 KB per wave, lie inside the
      // partial-reduction buffer); gains past that buffer and the tile, with
      // room for every wave's 1 KB DMA slot
      lds = (lds + 15) / 16 * 16 + std::max(size_t(g.K) * 2, size_t(1024) * nw);
      // a batch of k-steps fewer than without the norm (its LDS reads and
      // temporaries need the registers): QKV at K = 2880 keeps one batch per wave
      constexpr int UN = NTW >= 4 ? U - 1 : U - 2;
      return launch(gemm_skinny_kernel<EPI, AL, BMAP, MT, NTW, UN, 1>);
    } else {
      return hipErrorInvalidValue;
    }
  }
  return launch(gemm_skinny_kernel<EPI, AL, BMAP, MT, NTW, U, 0>);
}

template <int U>
static hipError_t run_wide(const GemmArgs& g, int num_cus, hipStream_t st) {
  const size_t lds = size_t(g.M) * (g.K / 8 + 1) * 16;
  const int grid = std::min(num_cus, g.N / 16);
  if (g.parts != grid) return hipErrorInvalidValue;
  auto fn = lmhead_wide_kernel<U>;
  hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(512), lds, st, g);
  return hipGetLastError();
}

// widest chunk (<= 16 k-steps) that divides the k-step count
static hipError_t run_wide_any(const GemmArgs& g, int num_cus, hipStream_t st) {
  const int ks = g.K / 32;
  if (ks % 16 == 0) return run_wide<16>(g, num_cus, st);
  if (ks % 15 == 0) return run_wide<15>(g, num_cus, st);
  if (ks % 12 == 0) return run_wide<12>(g, num_cus, st);
  if (ks % 10 == 0) return run_wide<10>(g, num_cus, st);
  if (ks % 9 == 0) return run_wide<9>(g, num_cus, st);
  if (ks % 8 == 0) return run_wide<8>(g, num_cus, st);
  if (ks % 6 == 0) return run_wide<6>(g, num_cus, st);
  if (ks % 5 == 0) return run_wide<5>(g, num_cus, st);
  if (ks % 4 == 0) return run_wide<4>(g, num_cus, st);
  if (ks % 3 == 0) return run_wide<3>(g, num_cus, st);
  if (ks % 2 == 0) return run_wide<2>(g, num_cus, st);
  return run_wide<1>(g, num_cus, st);
}

// Tail split of a tiled LM head.  Its tiles run in rounds of `slots`
// workgroups (CUs x workgroups per CU); when the last round would hold at most
// half a round, the column tiles it needs run instead as `ks` k-range pieces
// each (at least PE_TAIL_MIN_KTILES k-tiles per piece, at most one round of
// pieces, partial tiles within `cap` floats), so the last round is short.
// Returns ks (1: no split) and the first tail column tile.
int argmax_tail_split(int mtiles, int ntiles, int nk, int slots, long long tile_floats, long long cap,
                      int* tail0) {
  *tail0 = ntiles;
  const long long T = (long long)mtiles * ntiles, rem = T % slots;
  if (T < slots || rem == 0 || rem > slots / 2 || tile_floats <= 0) return 1;
  const int ncols = int((rem + mtiles - 1) / mtiles);
  const long long tt = (long long)ncols * mtiles;
  long long ks = slots / tt;
  ks = std::min<long long>(ks, nk / PE_TAIL_MIN_KTILES);
  ks = std::min<long long>(ks, cap / (tt * tile_floats));
  if (ks < 2) return 1;
  *tail0 = ntiles - ncols;
  return int(ks);
}

// Adds the k-split partial tiles of the tail column tiles [tail0, ntiles) in
// split order and writes each row's partial argmax key (and the logits when
// they are asked for).  One wave per (tail tile, row), 4 columns per lane.
template <int BM>
__global__ __launch_bounds__(256) void argmax_tail_kernel(GemmArgs g, int mtiles, int ntiles, int tail0) {
  constexpr int BN = 256;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (wave >= (ntiles - tail0) * mtiles * BM) return;
  const int tt = wave / BM, lrow = wave - tt * BM;
  const int mt = tt % mtiles, nt = tail0 + tt / mtiles, m = mt * BM + lrow;
  if (m >= g.M) return;
  const float* P = g.part + (long long)tt * g.ksplit * (BM * BN) + lrow * BN + 4 * l;
  const long long off[1] = {0};
  float4 sm[1];
  sum_splits<1>(P, BM * BN, g.ksplit, off, sm);  // the pieces in split order
  const float v[4] = {sm[0].x, sm[0].y, sm[0].z, sm[0].w};
  const int n0 = nt * BN + 4 * l;
  uint64_t best = 0ull;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (n0 + t < g.N) {
      if (g.logits) g.logits[(long long)m * g.ldl + n0 + t] = v[t];
      const uint64_t k = argmax_key(v[t], n0 + t);
      best = k > best ? k : best;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t k = shfl_xor_u64(best, o);
    best = k > best ? k : best;
  }
  if (l == 0) g.keys[(long long)m * g.parts + nt] = best;
}

template <int EPI, int AL, int BMAP, int BM, int BN, int WM, int WN, int S>
static hipError_t run_tiled(const GemmArgs& g, hipStream_t st, int slots = 0) {
  if (g.K % 64) return hipErrorInvalidValue;  // whole 64-wide k-tiles (and A_FC halves)
  const int mtiles = (g.M + BM - 1) / BM, ntiles = (g.N + BN - 1) / BN;
  if (EPI == E_ARGMAX && g.parts != ntiles) return hipErrorInvalidValue;
  GemmArgs ga = g;
  int tail0 = ntiles, ks = 1;
  if constexpr (EPI == E_ARGMAX) {
    static_assert(EPI != E_ARGMAX || BN == 256, "the tail reduction takes 256-column tiles");
    if (slots > 0 && g.part)
      ks = argmax_tail_split(mtiles, ntiles, g.K / 64, slots, (long long)BM * BN, g.part_cap, &tail0);
    ga.ksplit = ks;
  }
  const int ntail = (ntiles - tail0) * ks;
  const int grid = mtiles * ((tail0 + 7) / 8) * 8 + (ntail ? mtiles * ((ntail + 7) / 8) * 8 : 0);
  hipLaunchKernelGGL((gemm_tiled_kernel<EPI, AL, BMAP, BM, BN, WM, WN, S>), dim3(grid),
                     dim3(64 * WM * WN), 0, st, ga, mtiles, ntiles, tail0, 0, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !ntail) return e;
  if constexpr (EPI == E_ARGMAX) {
    const int waves = (ntiles - tail0) * mtiles * BM;
    hipLaunchKernelGGL(argmax_tail_kernel<BM>, dim3((waves + 3) / 4), dim3(256), 0, st, ga, mtiles, ntiles,
                       tail0);
    e = hipGetLastError();
  }
  return e;
}

// Split-K sum and epilogue: the ksplit fp32 partials of each output are added
// in a fixed order (deterministic), then the epilogue the unsplit kernel would
// have fused runs on the sum.  Store / residual: 8 consecutive columns per
// thread; SiLU.mul: 8 outputs from 8 gate and 8 up columns; QKV: one RoPE pair.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int BM, int ntiles, int dslots, int dcap) {
  // with a row map: partial row m (compact) is output row rmap[m]; rows past
  // the compact count were not computed
  const int rows = g.rmap ? min(g.M, *g.rcount) : g.M;
  // a split planned on the device (dslots > 0): the same plan as the product's
  const int KS = dslots > 0 ? tile_plan(min(rows, active_rows(g.nact, g.rpr, g.M)), BM, ntiles, g.K / 64, dslots, dcap).ks
                            : g.ksplit;
  if (KS <= 1) return;  // the product ran its epilogue itself
  const long long MN = (long long)g.M * g.N;
  const long long stride = (long long)gridDim.x * blockDim.x;
  auto out_row = [&](int m) { return g.rmap ? g.rmap[m] : m; };
  // 8 consecutive sums from two float4 sums
  auto to8 = [](const float4& a, const float4& b, float (&v)[8]) {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  };
  if constexpr (EPI == E_STORE || EPI == E_RESID) {
    const int per_row = g.N / 8;
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < (long long)rows * per_row; e += stride) {
      const int m = int(e / per_row), n = int(e % per_row) * 8;
      const long long b = (long long)m * g.N + n, off[2] = {b, b + 4};
      float4 sm[2];
      sum_splits<2>(g.part, MN, KS, off, sm);
      float v[8];
      to8(sm[0], sm[1], v);
      const long long o = (long long)out_row(m) * g.ldo + n;
      if constexpr (EPI == E_RESID) {
        const uint4 rv = *reinterpret_cast<const uint4*>((const uint16_t*)g.resid + o);
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] += __uint_as_float(rw[t] << 16);
          v[2 * t + 1] += __uint_as_float(rw[t] & 0xFFFF0000u);
        }
      }
      uint4 ov;
      ov.x = f2bf2(v[0], v[1]); ov.y = f2bf2(v[2], v[3]); ov.z = f2bf2(v[4], v[5]); ov.w = f2bf2(v[6], v[7]);
      *reinterpret_cast<uint4*>((uint16_t*)g.out + o) = ov;
    }
  } else if constexpr (EPI == E_SILU) {
    // logical columns (32q + c, 32q + 16 + c) -> output column 16q + c
    const int per_row = g.N / 16;
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < (long long)rows * per_row; e += stride) {
      const int m = int(e / per_row), pc = int(e % per_row), q = pc >> 1, c0 = (pc & 1) * 8;
      const long long b = (long long)m * g.N + 32 * q + c0, off[4] = {b, b + 4, b + 16, b + 20};
      float4 sm[4];
      sum_splits<4>(g.part, MN, KS, off, sm);
      float gt[8], up[8], v[8];
      to8(sm[0], sm[1], gt);
      to8(sm[2], sm[3], up);
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = gt[t] / (1.0f + expf(-gt[t])) * up[t];
      uint4 o;
      o.x = f2bf2(v[0], v[1]); o.y = f2bf2(v[2], v[3]); o.z = f2bf2(v[4], v[5]); o.w = f2bf2(v[6], v[7]);
      *reinterpret_cast<uint4*>((uint16_t*)g.out + (long long)out_row(m) * g.ldo + 16 * q + c0) = o;
    }
  } else {
    static_assert(EPI == E_QKV, "split-K epilogues: store, residual, SiLU.mul, QKV");
    // 8 RoPE pairs per thread: logical columns nb + c0 .. +7 and their
    // partners 16 further, so q and k leave as 16-byte stores (V is d-major
    // inside a block: one element per position row)
    const int per_row = g.N / 16;
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < (long long)rows * per_row; e += stride) {
      const int mr = int(e / per_row), pr = int(e % per_row), nb = (pr >> 1) * 32, c0 = (pr & 1) * 8;
      const int cm = g.dedup_k ? dedup_row(mr, g.dedup_k) : mr;  // row of the sums (one split then)
      const int m = out_row(mr);  // row of the positions, slots and q rows
      const long long b = (long long)cm * g.N + nb + c0, off[4] = {b, b + 4, b + 16, b + 20};
      float4 sm[4];
      sum_splits<4>(g.part, MN, KS, off, sm);
      float lo[8], hi[8];
      to8(sm[0], sm[1], lo);
      to8(sm[2], sm[3], hi);
      constexpr int hd = 64;  // bf16 storage implies head_dim 64 (checked at context creation)
      if (nb < g.nq + g.nk) {
        const bool isq = nb < g.nq;
        const int j = isq ? nb : nb - g.nq;
        const int head = j / hd, sb = (j % hd) >> 4;
        const int dlo = (sb >> 1) * 16 + c0, dhi = dlo + (hd >> 1);
        const int pos = g.positions[m];
        float olo[8], ohi[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          float cs, sn;
          rope_sincos(g, pos, dlo + t, cs, sn);
          olo[t] = lo[t] * cs - hi[t] * sn;
          ohi[t] = hi[t] * cs + lo[t] * sn;
        }
        const uint4 vlo = {f2bf2(olo[0], olo[1]), f2bf2(olo[2], olo[3]), f2bf2(olo[4], olo[5]), f2bf2(olo[6], olo[7])};
        const uint4 vhi = {f2bf2(ohi[0], ohi[1]), f2bf2(ohi[2], ohi[3]), f2bf2(ohi[4], ohi[5]), f2bf2(ohi[6], ohi[7])};
        uint16_t* dst = nullptr;
        if (isq) {
          dst = (uint16_t*)g.qout + ((long long)m * (g.nq / hd) + head) * hd;
        } else {
          const long long slot = g.slots[m];
          if (slot >= 0 && slot < g.num_slots) dst = (uint16_t*)g.kcache + (slot * g.Hkv + head) * hd;
        }
        if (dst) {
          *reinterpret_cast<uint4*>(dst + dlo) = vlo;
          *reinterpret_cast<uint4*>(dst + dhi) = vhi;
        }
      } else {
        const long long slot = g.slots[m];
        if (slot >= 0 && slot < g.num_slots) {
          const int j = nb - g.nq - g.nk;
          const int head = j / hd, jb = j % hd;
          const int bsl = __builtin_ctz(g.block_size);  // a power of two (checked at context creation)
          const long long blk = slot >> bsl, off = slot & (g.block_size - 1);
          uint16_t* vp = (uint16_t*)g.vcache + (((blk * g.Hkv + head) * hd) << bsl) + off;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            vp[(long long)(jb + c0 + t) << bsl] = f2bf(lo[t]);
            vp[(long long)(jb + 16 + c0 + t) << bsl] = f2bf(hi[t]);
          }
        }
      }
    }
  }
}

// Dense tiled GEMM, split over K when its output tiles are fewer than the CUs,
// into about PE_SPLITK_WG_PER_CU workgroups per CU; each split keeps at least
// PE_SPLITK_MIN_KTILES k-tiles (splitting grids that already cover the CUs
// measured slower: c=64 fc/O/down).
template <int EPI, int AL, int BMAP, int BM, int BN, int WM, int WN, int S>
static hipError_t run_tiled_dense(const GemmArgs& g, int num_cus, hipStream_t st) {
  if (g.K % 64) return hipErrorInvalidValue;
  const int mtiles = (g.M + BM - 1) / BM, ntiles = (g.N + BN - 1) / BN, nk = g.K / 64;
  const long long tiles = (long long)mtiles * ntiles, target = (long long)PE_SPLITK_WG_PER_CU * num_cus;
  const long long work = (long long)g.M * (EPI == E_QKV || EPI == E_SILU ? g.N / 16 : g.N / 8);
  const long long blocks = std::min<long long>((work + 255) / 256, 8LL * num_cus);
  if (g.rmap) {
    // row map: the rows are counted on the device, which plans the split; the
    // grid covers the largest plan of any row count up to M
    const int slots = int(target);
    const long long capl = g.part ? std::min<long long>(g.part_cap / ((long long)g.M * g.N), 64) : 0;
    const int cap = int(capl);
    const bool can_split = g.part && g.N % 32 == 0 && nk / PE_SPLITK_MIN_KTILES >= 2 && cap >= 2;
    const int dslots = can_split ? slots : 0;
    long long grid = 0;
    for (int mt = 1; mt <= mtiles; ++mt) {
      const TilePlan p = tile_plan(mt * BM, BM, ntiles, nk, dslots, cap);
      grid = std::max<long long>(grid, (long long)p.per * p.ks);
    }
    hipLaunchKernelGGL((gemm_tiled_kernel<EPI, AL, BMAP, BM, BN, WM, WN, S>), dim3(unsigned(grid)),
                       dim3(64 * WM * WN), 0, st, g, mtiles, ntiles, ntiles, dslots, cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !can_split) return e;
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(unsigned(blocks)), dim3(256), 0, st, g, BM, ntiles, dslots,
                       cap);
    return hipGetLastError();
  }
  long long ks = 1;
  if (g.part && tiles < num_cus && g.N % 32 == 0) {
    ks = (target + tiles - 1) / tiles;
    ks = std::min<long long>(ks, nk / PE_SPLITK_MIN_KTILES);
    ks = std::min<long long>(ks, g.part_cap / ((long long)g.M * g.N));
  }
  if (ks <= 1) return run_tiled<EPI, AL, BMAP, BM, BN, WM, WN, S>(g, st);
  GemmArgs gp = g;
  gp.ksplit = int(ks);
  const long long per = (long long)mtiles * ((ntiles + 7) / 8) * 8;
  hipLaunchKernelGGL((gemm_tiled_kernel<E_PART, AL, BMAP, BM, BN, WM, WN, S>), dim3(unsigned(per * ks)),
                     dim3(64 * WM * WN), 0, st, gp, mtiles, ntiles, ntiles, 0, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(unsigned(blocks)), dim3(256), 0, st, gp, BM, ntiles, 0, 0);
  return hipGetLastError();
}

// LM head on the deep ring (17..256 rows; needs the fragment-order copy)
template <int BM, int WM, int WN, int S, int WGPC>
static hipError_t run_ring(const GemmArgs& g, int num_cus, hipStream_t st) {
  const int grid = std::min(WGPC * num_cus, g.N / 16);
  if (g.parts != grid || g.M > BM || g.K % 32 || g.N % 16 || !g.Wp) return hipErrorInvalidValue;
  hipLaunchKernelGGL((lmhead_ring_kernel<BM, WM, WN, S, WGPC>), dim3(grid), dim3(64 * WM * WN), 0, st, g);
  return hipGetLastError();
}

template <int EPI, int AL, int BMAP>
static hipError_t run_bf16(const GemmArgs& g, int num_cus, hipStream_t st) {
  if (EPI != E_ARGMAX && (g.M > kMmMinRows || (g.M > kRowMapMinRows && EPI != E_SILU)))
    return launch_mm(AL, BMAP, EPI, g, num_cus, st);
  if (g.nrm_out) return hipErrorInvalidValue;  // the fused following norm: large-batch kernels only
  if (g.dedup_k) return hipErrorInvalidValue;  // compact first-layer rows: large batches only
  const Variant v = pick(EPI, g.M, g.N, g.K, num_cus);
  if constexpr (EPI == E_ARGMAX) {
    // 17..128 rows: the deep ring (K sweep, K = 3, 5, 7: 157 -> 153, 170 ->
    // 158, 174 -> 160 us); 129..256 rows measured slower on it (four 32 KB
    // stages: 198 -> 206, 205 -> 217 us) and stay on the 64-wide ring
    if (v == V_RING) {
      if (!g.Wp || AL != A_PLAIN || BMAP != B_PLAIN) return hipErrorInvalidValue;
      // up to 64 rows: two workgroups per CU, each a three-stage ring of
      // four waves (K sweep, 48 rows: 155 -> 127 us); 65..128 rows: one
      // workgroup of eight waves and six stages (two of four waves and three
      // stages measured 446 us against 158)
      if (g.M <= 64) return run_ring<64, 1, 4, 3, 2>(g, num_cus, st);
      // 65..96 rows on 96-row stages (K sweep K = 5, 80 rows: 165 -> 153 us
      // against the 128-row ring; two workgroups of four waves and three
      // stages measured 236 us)
      if (g.M <= 96) return run_ring<96, 2, 4, 6, 1>(g, num_cus, st);
      return run_ring<128, 2, 4, 6, 1>(g, num_cus, st);
    }
    switch (v) {
      case V_WIDE: return run_wide_any(g, num_cus, st);
      // workgroups per CU: two 64-row tiles (80 KB of LDS each), one otherwise
      case V_A64: return run_tiled<EPI, AL, BMAP, 64, kArgmaxBN, 1, 4, 2>(g, st, 2 * num_cus);
      case V_A128: return run_tiled<EPI, AL, BMAP, 128, kArgmaxBN, 2, 4, 2>(g, st, num_cus);
      case V_A192: return run_tiled<EPI, AL, BMAP, 192, kArgmaxBN, 2, 4, 2>(g, st, num_cus);
      case V_A224: return run_tiled<EPI, AL, BMAP, 224, kArgmaxBN, 2, 4, 2>(g, st, num_cus);
      default: return run_tiled<EPI, AL, BMAP, 256, kArgmaxBN, 4, 2, 2>(g, st, num_cus);
    }
  } else {
    if ((g.norm_gain || g.ssq_out) && v != V_SKINNY) return hipErrorInvalidValue;  // folded norm: small batches only
    switch (v) {
      case V_SKINNY:
        if (g.M <= 16) return run_skinny<EPI, AL, BMAP, 1>(g, st);
        if (g.M <= 32) return run_skinny<EPI, AL, BMAP, 2>(g, st);
        if (g.M <= 48) return run_skinny<EPI, AL, BMAP, 3>(g, st);
        return run_skinny<EPI, AL, BMAP, 4>(g, st);
      case V_D64: return run_tiled_dense<EPI, AL, BMAP, 64, 128, 1, 4, 3>(g, num_cus, st);
      default: return run_tiled_dense<EPI, AL, BMAP, 128, 128, 2, 2, 2>(g, num_cus, st);
    }
  }
}

template <int EPI, int AL, int BMAP>
static hipError_t run_f32(const GemmArgs& g, hipStream_t st) {
  dim3 grid((g.N + 31) / 32, (g.M + 15) / 16);
  if (EPI == E_ARGMAX && g.parts != int(grid.x)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI, AL, BMAP>), grid, dim3(512), 0, st, g);
  return hipGetLastError();
}

template <int EPI, int AL, int BMAP>
static hipError_t run(int dtype, const GemmArgs& g, int num_cus, hipStream_t st) {
  return dtype == 1 ? run_bf16<EPI, AL, BMAP>(g, num_cus, st) : run_f32<EPI, AL, BMAP>(g, st);
}

hipError_t launch_argmax_tokens(int M, int Kd, int parts, const uint64_t* keys, int32_t* tokens,
                                int tstride, const int32_t* seq_lens, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_tokens_kernel, dim3(M), dim3(256), 0, st, M, Kd, parts, keys, tokens,
                     tstride, seq_lens);
  return hipGetLastError();
}

hipError_t launch_argmax_verify(int B, int K, int parts, const uint64_t* keys, int32_t* tokens,
                                const int32_t* seq_lens, const int32_t* target, int32_t* acc,
                                int32_t* bonus, const int32_t* nact, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (K < 1 || K > 64) return hipErrorInvalidValue;
  const int waves = K < 16 ? K : 16;
  hipLaunchKernelGGL(argmax_verify_kernel, dim3(unsigned(B)), dim3(64 * waves), 0, st, K, parts, keys,
                     tokens, seq_lens, target, acc, bonus, nact);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int aload, int bmap, int epi, const GemmArgs& g, int num_cus,
                       hipStream_t st) {
  if (g.M <= 0) return hipSuccess;
  if (aload == A_FC && bmap == B_PLAIN && epi == E_STORE) return run<E_STORE, A_FC, B_PLAIN>(dtype, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_QKV && epi == E_QKV) return run<E_QKV, A_PLAIN, B_QKV>(dtype, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_PLAIN && epi == E_RESID) return run<E_RESID, A_PLAIN, B_PLAIN>(dtype, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_GATEUP && epi == E_SILU) return run<E_SILU, A_PLAIN, B_GATEUP>(dtype, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_PLAIN && epi == E_ARGMAX) return run<E_ARGMAX, A_PLAIN, B_PLAIN>(dtype, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_PLAIN && epi == E_STORE) return run<E_STORE, A_PLAIN, B_PLAIN>(dtype, g, num_cus, st);
  return hipErrorInvalidValue;
}

}  // namespace pe
