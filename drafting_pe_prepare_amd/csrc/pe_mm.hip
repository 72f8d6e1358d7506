// Dense contractions of the drafter at larger batch (more than 256 rows):
// out[m, n] = sum_k A[m, k] W[n, k] with a fused epilogue.  "P-EAGLE: parallel
// speculative decoding in vLLM", Architecture and mechanism, Step 2: fc over
// concat(emb, h) and the N-layer Transformer, over all K positions of every
// request in one pass.  (The LM head runs on the 16x16x32 ring of
// pe_gemm.hip, which measured faster on its shape.)
//
// gfx950 design
//  * v_mfma_f32_32x32x16_bf16.  Measured on this chip, the 32x32x16 form
//    issues at ~2.0-2.1 PFLOP/s, the 16x16x32 form at ~1.3 PFLOP/s (half rate),
//    so the large tiles use 32x32 outputs.  Lane l supplies A[l%32][8(l/32)+j]
//    and B^T[l%32][8(l/32)+j] (both operands K-contiguous) and holds
//    C[8(i/4) + 4(l/32) + i%4][l%32] in accumulator register i.
//  * Both operands stream through a two-stage LDS ring of 64-wide k-tiles,
//    filled by global_load_lds_dwordx4 (one instruction moves 8 whole
//    128-byte rows).  Row r's 16-byte chunk c sits at slot c ^ ((r >> 1) & 7):
//    gfx950's LDS serves 16 lanes of a 16-byte read per clock (256 B over 64
//    banks), and under this swizzle the 16 rows a fragment read touches per
//    clock fall on distinct banks (measured 218 B/clk/CU against 124 with
//    the 128-byte c ^ (r & 7) swizzle).
//  * Column pairs an epilogue needs together (rotate-half RoPE partners, gate
//    and up) sit 32 logical columns apart in one 64-column block, i.e. in the
//    same lane of two neighbouring 32x32 tiles.  For QKV that is the plain
//    [Wq; Wk; Wv] row order (head_dim 64: dims i and i + 32 pair up).
//  * Output tiles fewer than the workgroup slots of the chip are split over k
//    into fp32 partials, summed in a fixed order by mm_reduce_kernel, which
//    also runs the RoPE + KV-write epilogue of the QKV product.
#include <algorithm>

#include "pe_common.h"
#include "pe_internal.h"

#ifndef PE_MM_SPLIT_MIN_KTILES
#define PE_MM_SPLIT_MIN_KTILES 6  // fewest 64-wide k-tiles per split
#endif

namespace pe {


// logical weight row n of the 32-apart pairings (see above)
template <int BMAP>
__device__ __forceinline__ const uint16_t* mm_weight_row(const GemmArgs& g, int n) {
  const long long K = g.K;
  if (BMAP == B_GATEUP) {
    const int t = n >> 6, r = n & 63;
    return (r < 32 ? (const uint16_t*)g.W0 : (const uint16_t*)g.W1) + (long long)(t * 32 + (r & 31)) * K;
  } else if (BMAP == B_QKV) {
    if (n < g.nq) return (const uint16_t*)g.W0 + (long long)n * K;
    if (n < g.nq + g.nk) return (const uint16_t*)g.W1 + (long long)(n - g.nq) * K;
    return (const uint16_t*)g.W2 + (long long)(n - g.nq - g.nk) * K;
  }
  return (const uint16_t*)g.W0 + (long long)n * K;
}


// Slot of compact row m of a MASK-deduplicated first layer (K+2 rows per
// request: copied slots 0..K and one MASK slot).
__device__ __forceinline__ int dedup_slot(int m, int K) { return (m / (K + 2)) * (2 * K) + m % (K + 2); }

// ---------------------------------------------------------------------------
// The tiled kernel.  BM x BN output tile, WM x WN waves of (BM/WM) x (BN/WN).
// KT: k-tile width (64: 128-byte stage rows, 32: 64-byte rows); S: stages in
// the LDS ring, so S-1 k-tiles are in flight while one is consumed.
// With a split (mm_plan), workgroup b takes copy s = b / per of the tile
// grid, summing k-tiles [s nk / ks, (s+1) nk / ks) into fp32 partials.
// ---------------------------------------------------------------------------
// Stage row r (RB bytes) keeps its 16-byte chunk c at slot c ^ swz(r): the
// 16 rows one clock of a fragment read touches then fall on distinct banks of
// the 256-byte bank window (two 128-byte rows or four 64-byte rows per window).
template <int RB>
__device__ __forceinline__ int mm_swz(int r) {
  return RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

// The split of a product over k, chosen from the rows it computes (on the
// device: with a row map the count is known only there).  T output tiles
// (column tiles rounded up to whole groups of 8, see the block mapping) run
// in one round of `slots` workgroups: ks = floor(slots / T) splits, so that
// T * ks <= slots, at least PE_MM_SPLIT_MIN_KTILES k-tiles each and within
// the partial-sum buffer (cap_splits copies of [M][N]).  With ks == 1 the kernel
// runs the fused epilogue itself, unless `force_part` (the QKV product, whose
// RoPE + KV-write epilogue runs on the fp32 sums).
struct MmPlan { int mt, per, ks; };
__host__ __device__ inline MmPlan mm_plan(int rows, int BM, int ntiles, int nkt, int slots, int cap_splits) {
  MmPlan p;
  p.mt = (rows + BM - 1) / BM;
  p.per = p.mt * ((ntiles + 7) / 8) * 8;
  p.ks = 1;
  if (p.per > 0 && p.per < slots) {
    // (two splits for tiles filling more than half the slots, one and a half
    // rounds, measured slower or level: K sweep gate/up 181 -> 202 us,
    // largest graph fc 109 -> 125 us, drafting round after a prompt -13 us)
    int ks = slots / p.per;
    const int kmax = nkt / PE_MM_SPLIT_MIN_KTILES;
    ks = ks < kmax ? ks : kmax;
    ks = ks < cap_splits ? ks : cap_splits;
    p.ks = ks > 1 ? ks : 1;
  }
  return p;
}
// rows the product computes: the active requests' rows, and with a row map
// the mapped (compact) rows
__device__ __forceinline__ int mm_rows(const GemmArgs& g) {
  const int r = active_rows(g.nact, g.rpr, g.M);
  return g.rmap ? min(r, *g.rcount) : r;
}

template <int EPI, int AL, int BMAP, int BM, int BN, int WM, int WN, int KT, int S, int OCC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void mm_kernel(GemmArgs g, int ntiles, int slots, int cap_splits) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN, TI = WTM / 32, TJ = WTN / 32;
  static_assert(TI * 32 * WM == BM && TJ * 32 * WN == BN, "whole 32x32 tiles per wave");
  static_assert(KT == 32 || KT == 64, "k-tiles of 32 or 64");
  constexpr int RB = KT * 2, CPR = RB / 16, RPG = 1024 / RB;  // row bytes, chunks per row, rows per DMA
  constexpr int GA = BM / RPG, GB = BN / RPG;                 // DMA row groups of each operand
  static_assert(GA * RPG == BM && GB * RPG == BN, "whole DMA row groups");
  constexpr int QA = (GA + NW - 1) / NW, QB = (GB + NW - 1) / NW, Q = QA + QB;  // DMAs per wave per k-tile
  static_assert(S >= 2 && S <= 5 && (S - 1) * Q < 64, "ring depth within the vmcnt range");
  constexpr int NS = KT / 16;                                  // MFMA substeps per k-tile
  constexpr int STAGE = (BM + BN) * RB;
  // distinct LDS objects, so the compiler sees that the DMA into one stage
  // and the fragment reads of another do not alias
  __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE], st1[STAGE], st2[S > 2 ? STAGE : 16],
      st3[S > 3 ? STAGE : 16], st4[S > 4 ? STAGE : 16];

  const int Mk = g.M, Nk = g.N;
  const int cnt = mm_rows(g);  // rows computed (compact rows with a map)
  const int nkt = g.K / KT;
  const MmPlan plan = mm_plan(cnt, BM, ntiles, g.K / 64, slots, cap_splits);
  const bool part = EPI == E_QKV || plan.ks > 1;  // fp32 partial sums instead of the fused epilogue
  // one item per workgroup: the tiles fit in one round when split
  // (T * ks <= slots), otherwise the grid covers every tile
  int bid = blockIdx.x, ks = 0, mt, nt;
  if (bid >= plan.per * plan.ks) return;  // the grid covers the largest plan
  ks = bid / plan.per;
  bid -= ks * plan.per;
  // workgroups that share a weight tile run back to back on one XCD
  // (workgroup b runs on XCD b % 8)
  {
    const int j = bid >> 3;
    mt = j % plan.mt;
    nt = (j / plan.mt) * 8 + (bid & 7);
    if (nt >= ntiles) return;
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int ksplit = plan.ks;
  const int kb = ks * nkt / ksplit, nk = (ks + 1) * nkt / ksplit - kb;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w / WN, wn = w % WN;

  // DMA instruction q < QA of this wave fills A-role row group j = w + NW q
  // (stage rows RPG j .. RPG j + RPG-1), instruction QA + q the B-role group
  // GA + w + NW q; lane l takes row RPG j + l/CPR and slot l%CPR, i.e. global
  // chunk (l%CPR) ^ swz(row).  A wave whose group would lie past its operand
  // repeats another of that operand's groups (the same bytes to the same
  // place), so every wave issues Q DMAs per k-tile and one vmcnt serves all;
  // the operand of each instruction is known at compile time.
  const uint16_t* lo[Q];
  const uint16_t* hi[QA];
  uint32_t dst[Q];
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform copy for the LDS addresses
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const bool isa = q < QA;
    const int jj = wu + NW * (isa ? q : q - QA), gn = isa ? GA : GB;
    const int j = (isa ? 0 : GA) + (jj < gn ? jj : wu % gn);
    dst[q] = uint32_t(j * 1024);
    const int r = RPG * j + l / CPR;
    const int c = ((l % CPR) ^ mm_swz<RB>(r)) * 8;
    if (isa) {
      const int m = g.rmap ? g.rmap[min(m0 + r, cnt - 1)] : min(m0 + r, Mk - 1);
      if (AL == A_FC) {
        const int sl = g.dedup_k ? dedup_slot(m, g.dedup_k) : m;
        int id = g.ids[sl];
        id = id < 0 ? 0 : (id >= g.vocab ? g.vocab - 1 : id);
        lo[q] = (const uint16_t*)g.embed + (long long)id * g.d + c;
        hi[q] = (const uint16_t*)g.hid + (long long)sl * g.d - g.d + c;
      } else {
        lo[q] = (const uint16_t*)g.A + (long long)m * g.lda + c;
        hi[q] = lo[q];
      }
    } else {
      const int n = min(n0 + r - BM, Nk - 1);
      lo[q] = mm_weight_row<BMAP>(g, n) + c;
    }
  }
  auto issue = [&](unsigned char* st, int kt) {
    const int k0 = (kb + kt) * KT;
    const uint32_t sb = lds_addr(st);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      if (q < QA) {
        dma16((AL == A_FC && k0 >= g.d) ? hi[q] + k0 : lo[q] + k0, sb + dst[q]);
      } else {
        dma16(lo[q] + k0, sb + dst[q]);
      }
    }
  };
  // wait until at most n k-tiles of this wave's DMAs are in flight
  auto wait_tiles = [&](int n) {
    if (n >= 4) wait_vmcnt<(S > 4 ? 4 : 0) * Q>();
    else if (n == 3) wait_vmcnt<(S > 3 ? 3 : 0) * Q>();
    else if (n == 2) wait_vmcnt<(S > 2 ? 2 : 0) * Q>();
    else if (n == 1) wait_vmcnt<Q>();
    else wait_vmcnt<0>();
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment rows: A-role row wm*WTM + 32 i + l%32, B-role row BM + wn*WTN +
  // 32 j + l%32; substep s (16 of the tile's k) reads chunk 2s + l/32
  const int sw = mm_swz<RB>(l & 31);
  const int abase = (wm * WTM + (l & 31)) * RB, bbase = (BM + wn * WTN + (l & 31)) * RB;
  uint4 fa[2][TI], fb[2][TJ];
  auto load = [&](int buf, const unsigned char* st, int s) {
    const int x = ((2 * s + (l >> 5)) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[buf][i] = *reinterpret_cast<const uint4*>(st + abase + x + i * 32 * RB);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[buf][j] = *reinterpret_cast<const uint4*>(st + bbase + x + j * 32 * RB);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32(fa[buf][i], fb[buf][j], acc[i][j]);
  };
  auto stage = [&](int j) -> unsigned char* {
    return j == 0 ? st0 : j == 1 ? st1 : j == 2 ? st2 : j == 3 ? st3 : st4;
  };

  const int pre = nk < S ? nk : S;
#pragma unroll
  for (int j = 0; j < S; ++j)
    if (j < pre) issue(stage(j), j);
  wait_tiles(pre - 1);                      // this wave's DMAs of k-tile 0 have landed
  asm volatile("s_barrier" ::: "memory");   // ... and everyone's
  load(0, st0, 0);
  // k-tile kt sits in `cur`; on entry fa[0]/fb[0] hold its first substep.
  // `cur` and `nxt` are distinct stages (restrict), so the DMA into `cur` can
  // stay in flight across the reads of `nxt`.
  // The fragment reads of substep s+1 are issued before the MFMAs of substep
  // s, and sched_barrier keeps the compiler from sinking each read down to its
  // first use (it otherwise does, and every MFMA then waits out an LDS round
  // trip).  Each substep starts with an explicit lgkmcnt(0): the reads it
  // waits for were issued one MFMA group earlier, and with the counter known
  // to be clear the compiler puts no wait of its own (a full one, whenever a
  // scalar load might be in flight) between the new reads and the MFMAs.
  auto tile = [&](unsigned char* __restrict__ cur, const unsigned char* __restrict__ nxt, int kt) {
#pragma unroll
    for (int s = 0; s + 1 < NS; ++s) {
      wait_lgkm0();
      load((s + 1) & 1, cur, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();  // this wave's reads of `cur` have returned
    if (kt + 1 < nk) {
      // k-tile kt+1 must land; kt+2 .. kt+S-1 (those issued) may stay in flight
      const int later = nk - 2 - kt;
      wait_tiles(later < S - 2 ? later : S - 2);
      asm volatile("s_barrier" ::: "memory");   // everyone's, and `cur` is free
      if (kt + S < nk) issue(cur, kt + S);
      load(NS & 1, nxt, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma((NS - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt0 = 0; kt0 < nk; kt0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (kt0 + j < nk) tile(stage(j), stage((j + 1) % S), kt0 + j);
  }

  // lane l holds C[32 i + 8 (r/4) + 4 (l/32) + r%4][32 j + l%32] of the wave tile
  const int rbase = wm * WTM + 4 * (l >> 5), cbase = wn * WTN + (l & 31);
  if (part) {
    float* P = g.part + (long long)ks * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + rbase + 32 * i + 8 * (r >> 2) + (r & 3);
        if (m >= cnt) continue;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int n = n0 + cbase + 32 * j;
          if (n < g.N) P[(long long)m * g.N + n] = acc[i][j][r];
        }
      }
    return;
  }
  if constexpr (EPI == E_STORE || EPI == E_RESID) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mc = m0 + rbase + 32 * i + 8 * (r >> 2) + (r & 3);
        if (mc >= cnt) continue;
        const int m = g.rmap ? g.rmap[mc] : mc;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int n = n0 + cbase + 32 * j;
          if (n >= g.N) continue;
          const long long o = (long long)m * g.ldo + n;
          float v = acc[i][j][r];
          if (EPI == E_RESID) v += bf2f(((const uint16_t*)g.resid)[o]);
          ((uint16_t*)g.out)[o] = f2bf(v);
        }
      }
  } else if constexpr (EPI == E_SILU) {
    static_assert(TJ % 2 == 0, "gate/up pairs are neighbouring 32-column tiles");
    // logical block 64 t: columns 64 t + c (gate) and 64 t + 32 + c (up) ->
    // output column 32 t + c
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mc = m0 + rbase + 32 * i + 8 * (r >> 2) + (r & 3);
        if (mc >= cnt) continue;
        const int m = g.rmap ? g.rmap[mc] : mc;
#pragma unroll
        for (int q = 0; q < TJ / 2; ++q) {
          const int n = n0 + cbase + 64 * q;  // gate column
          if (n >= g.N) continue;
          const float gt = acc[i][2 * q][r], up = acc[i][2 * q + 1][r];
          const float v = gt / (1.0f + expf(-gt)) * up;
          ((uint16_t*)g.out)[(long long)m * g.ldo + ((n >> 6) << 5) + (n & 31)] = f2bf(v);
        }
      }
  } else {
    static_assert(EPI == E_QKV, "epilogues: partial sums, store, residual, SiLU.mul");
  }
}

// ---------------------------------------------------------------------------
// Split-K sum and epilogue over fp32 partials [ksplit][M][N] in the 32-apart
// logical column order: partials are added in split order (deterministic),
// then the epilogue runs.  Store / residual: 8 consecutive columns per thread;
// SiLU.mul: 8 outputs from 8 gate and 8 up columns; QKV: 8 RoPE pairs (q and
// k leave as 16-byte stores; V is d-major inside a block, one element per
// position row).  With dedup_k the QKV epilogue covers all `rows` slots of the
// parallel layout, slot s reading the sums of compact row dedup_row(s).
// ---------------------------------------------------------------------------
// The split is the product kernel's (mm_plan over the same arguments); with
// ks == 1 that kernel ran the epilogue itself and this one has nothing to do.
template <int EPI>
__global__ __launch_bounds__(256) void mm_reduce_kernel(GemmArgs g, int rows, int rpr, int BM, int ntiles,
                                                        int slots, int cap_splits) {
  const MmPlan plan = mm_plan(mm_rows(g), BM, ntiles, g.K / 64, slots, cap_splits);
  if (EPI != E_QKV && plan.ks == 1) return;
  rows = active_rows(g.nact, rpr, rows);  // rows of inactive requests are skipped
  if (g.rmap) rows = min(rows, *g.rcount);  // compact rows: sums at m, output row rmap[m]
  const int KS = plan.ks;
  const long long MN = (long long)g.M * g.N;
  const long long stride = (long long)gridDim.x * blockDim.x;
  // 8 consecutive sums from two float4 sums
  auto to8 = [](const float4& a, const float4& b, float (&v)[8]) {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  };
  auto pack8 = [](const float (&v)[8]) {
    return uint4{f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7])};
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
      const long long o = (long long)(g.rmap ? g.rmap[m] : m) * g.ldo + n;
      if constexpr (EPI == E_RESID) {
        const uint4 rv = *reinterpret_cast<const uint4*>((const uint16_t*)g.resid + o);
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] += __uint_as_float(rw[t] << 16);
          v[2 * t + 1] += __uint_as_float(rw[t] & 0xFFFF0000u);
        }
      }
      *reinterpret_cast<uint4*>((uint16_t*)g.out + o) = pack8(v);
    }
  } else if constexpr (EPI == E_SILU) {
    const int per_row = g.N / 16;  // 8 outputs per thread, 32 per 64-column block
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < (long long)rows * per_row; e += stride) {
      const int m = int(e / per_row), pc = int(e % per_row), t = pc >> 2, c0 = (pc & 3) * 8;
      const long long b = (long long)m * g.N + 64 * t + c0, off[4] = {b, b + 4, b + 32, b + 36};
      float4 sm[4];
      sum_splits<4>(g.part, MN, KS, off, sm);
      float gt[8], up[8], v[8];
      to8(sm[0], sm[1], gt);
      to8(sm[2], sm[3], up);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = gt[u] / (1.0f + expf(-gt[u])) * up[u];
      *reinterpret_cast<uint4*>((uint16_t*)g.out + (long long)(g.rmap ? g.rmap[m] : m) * g.ldo + 32 * t + c0) =
          pack8(v);
    }
  } else {
    static_assert(EPI == E_QKV, "split-K epilogues: store, residual, SiLU.mul, QKV");
    constexpr int hd = 64;  // bf16 storage implies head_dim 64 (checked at context creation)
    const int per_row = g.N / 16;  // 8 pairs per thread, 4 per 64-column head
    for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < (long long)rows * per_row; e += stride) {
      const int mr = int(e / per_row), pc = int(e % per_row), nb = (pc >> 2) * 64, c0 = (pc & 3) * 8;
      // sums of compact row cm, written to slot m
      const int cm = g.dedup_k ? dedup_row(mr, g.dedup_k) : mr;
      const int m = g.rmap ? g.rmap[mr] : mr;
      const long long b = (long long)cm * g.N + nb + c0, off[4] = {b, b + 4, b + 32, b + 36};
      float4 sm[4];
      sum_splits<4>(g.part, MN, KS, off, sm);
      float lo[8], hi[8];
      to8(sm[0], sm[1], lo);
      to8(sm[2], sm[3], hi);
      if (nb < g.nq + g.nk) {
        const bool isq = nb < g.nq;
        const int head = (isq ? nb : nb - g.nq) / hd;
        const int pos = g.positions[m];
        float olo[8], ohi[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          // angle pos * theta^(-2i/hd) in turns: the fp64 product minus its
          // nearest integer is the exact fraction of a turn for any position;
          // v_sin_f32 / v_cos_f32 take turns
          const double tt = double(pos) * g.rope_turns[c0 + t];
          const float x = float(tt - rint(tt));
          const float sn = __builtin_amdgcn_sinf(x), cs = __builtin_amdgcn_cosf(x);
          olo[t] = lo[t] * cs - hi[t] * sn;
          ohi[t] = hi[t] * cs + lo[t] * sn;
        }
        uint16_t* dst = nullptr;
        if (isq) {
          dst = (uint16_t*)g.qout + ((long long)m * (g.nq / hd) + head) * hd;
        } else {
          const long long slot = g.slots[m];
          if (slot >= 0 && slot < g.num_slots) dst = (uint16_t*)g.kcache + (slot * g.Hkv + head) * hd;
        }
        if (dst) {
          *reinterpret_cast<uint4*>(dst + c0) = pack8(olo);
          *reinterpret_cast<uint4*>(dst + 32 + c0) = pack8(ohi);
        }
      } else {
        const long long slot = g.slots[m];
        if (slot >= 0 && slot < g.num_slots) {
          const int head = (nb - g.nq - g.nk) / hd;
          const int bsl = __builtin_ctz(g.block_size);  // a power of two (checked at context creation)
          const long long blk = slot >> bsl, off = slot & (g.block_size - 1);
          uint16_t* vp = (uint16_t*)g.vcache + (((blk * g.Hkv + head) * hd) << bsl) + off;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            vp[(long long)(c0 + t) << bsl] = f2bf(lo[t]);
            vp[(long long)(32 + c0 + t) << bsl] = f2bf(hi[t]);
          }
        }
      }
    }
  }
}

// Split-K sum + residual with the following RMSNorm (GemmArgs::nrm_out): one
// 256-thread workgroup per output row, thread t over 8-column chunks t and
// t + 256.  The rounded row x (the split sum plus the residual, or with no
// split the row the product stored) stays in registers, its squares are
// summed over the workgroup in a fixed order, and the normalised row goes out
// beside it.
template <int EPI, int MAXC>
__global__ __launch_bounds__(256) void mm_resid_norm_kernel(GemmArgs g, int rows, int rpr, int BM, int ntiles,
                                                            int slots, int cap_splits) {
  __shared__ float s_ss[4];
  const MmPlan plan = mm_plan(mm_rows(g), BM, ntiles, g.K / 64, slots, cap_splits);
  rows = active_rows(g.nact, rpr, rows);
  if (g.rmap) rows = min(rows, *g.rcount);
  const int KS = plan.ks;
  const long long MN = (long long)g.M * g.N;
  const int tid = threadIdx.x, nch = g.N / 8;
  for (int m = blockIdx.x; m < rows; m += gridDim.x) {
    const long long row = g.rmap ? g.rmap[m] : m;
    uint16_t* xr = (uint16_t*)g.out + row * g.ldo;
    // this thread's chunks tid + 256 j (a chunk past the row re-reads the
    // last one, so every load has a valid address; its results are unused);
    // the gains, the residual and every split's partials are all in flight
    // before the first add
    int cc[MAXC];
    uint4 gv[MAXC];
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      cc[j] = min(tid + 256 * j, nch - 1);
      gv[j] = *reinterpret_cast<const uint4*>((const uint16_t*)g.nrm_gain + 8 * cc[j]);
    }
    float x[MAXC][8];
    float ss = 0.f;
    auto unpack = [](const uint4& u, float (&f)[8]) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f[2 * t] = __uint_as_float(w[t] << 16);
        f[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
      }
    };
    uint4 xp[MAXC];  // the stored row, as bf16
    if (KS > 1) {
      uint4 rv[MAXC];
      long long off[2 * MAXC];
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        if constexpr (EPI == E_RESID)
          rv[j] = *reinterpret_cast<const uint4*>((const uint16_t*)g.resid + row * g.ldo + 8 * cc[j]);
        off[2 * j] = (long long)m * g.N + 8 * cc[j];
        off[2 * j + 1] = off[2 * j] + 4;
      }
      float4 sm[2 * MAXC];
      sum_splits<2 * MAXC>(g.part, MN, KS, off, sm);  // the split's partials in a fixed order
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        if (tid + 256 * j < nch) {
          float v[8] = {sm[2 * j].x,     sm[2 * j].y,     sm[2 * j].z,     sm[2 * j].w,
                        sm[2 * j + 1].x, sm[2 * j + 1].y, sm[2 * j + 1].z, sm[2 * j + 1].w};
          if constexpr (EPI == E_RESID) {
            float r[8];
            unpack(rv[j], r);
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] += r[t];
          }
          xp[j] = uint4{f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7])};
          *reinterpret_cast<uint4*>(xr + 8 * cc[j]) = xp[j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < MAXC; ++j)
        if (tid + 256 * j < nch) xp[j] = *reinterpret_cast<const uint4*>(xr + 8 * cc[j]);  // the product stored it
    }
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if (tid + 256 * j < nch) {
        unpack(xp[j], x[j]);
#pragma unroll
        for (int t = 0; t < 8; ++t) ss += x[j][t] * x[j][t];
      }
    }
    if (g.dedup_k > 0 && g.nrm_xfull) {
      // compact row m of a MASK-deduplicated layer: its slot, or the
      // request's K-1 MASK slots for its last row
      const int K = g.dedup_k, r = m / (K + 2), jj = m - r * (K + 2);
      const int s0 = r * 2 * K + jj, ns = jj == K + 1 ? K - 1 : 1;
      for (int t = 0; t < ns; ++t) {
        uint16_t* xf = (uint16_t*)g.nrm_xfull + (long long)(s0 + t) * g.ldo;
#pragma unroll
        for (int j = 0; j < MAXC; ++j)
          if (tid + 256 * j < nch) *reinterpret_cast<uint4*>(xf + 8 * cc[j]) = xp[j];
      }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_ss[tid >> 6] = ss;
    __syncthreads();
    const float tot = ((s_ss[0] + s_ss[1]) + s_ss[2]) + s_ss[3];
    __syncthreads();  // s_ss is written again for the next row
    const float rs = rsqrtf(tot / float(g.N) + g.norm_eps);
    uint16_t* ur = (uint16_t*)g.nrm_out + (g.nrm_rows ? (long long)g.nrm_rows[m] : row) * g.ldo;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if (tid + 256 * j < nch) {
        const uint32_t gw[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
        uint32_t o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          o[t] = f2bf2(x[j][2 * t] * rs * __uint_as_float(gw[t] << 16),
                       x[j][2 * t + 1] * rs * __uint_as_float(gw[t] & 0xFFFF0000u));
        *reinterpret_cast<uint4*>(ur + 8 * cc[j]) = uint4{o[0], o[1], o[2], o[3]};
      }
    }
  }
}
constexpr int kNormMaxChunks = 2;  // rows of up to 2 x 256 x 8 = 4096 columns

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// Dense tiles.  The default is 128 x 128 (four waves of 64 x 64, two
// workgroups per CU).  256 x 256 tiles (eight waves of 128 x 64, one
// workgroup per CU) move half the operand bytes per flop through the caches;
// measured at c=64 they pay off only for gate/up (896 x 15360 x 2880: 90 us
// against 102), where they still fill the chip: the other products, with
// 2880-5120 output columns, run 20-30% slower on them (fewer, split tiles).
struct TileSmall { static constexpr int BM = 128, BN = 128, WM = 2, WN = 2, WGPC = 2, S = 2, OCC = 2; };
struct TileLarge { static constexpr int BM = 256, BN = 256, WM = 2, WN = 4, WGPC = 1, S = 2, OCC = 2; };
struct TileMid { static constexpr int BM = 192, BN = 256, WM = 2, WN = 4, WGPC = 1, S = 2, OCC = 2; };
struct TileWide { static constexpr int BM = 256, BN = 128, WM = 2, WN = 2, WGPC = 1, S = 2, OCC = 2; };
// 65..256 rows (fc, QKV, O, down; the K-sweep drafter): 64 x 128 tiles, one
// workgroup of four waves per CU with a four-stage ring, so three k-tiles are
// in flight when each workgroup has few rows of work per k-tile.  Measured on
// the K-sweep drafter (K = 7): down 94 -> 86, QKV 84 -> 80, fc 36 -> 30 us
// against the 16x16x32 tiled kernel; gate/up, with enough tiles for two
// workgroups per CU, stays there (133 against 156 us).
struct TileDeep { static constexpr int BM = 64, BN = 128, WM = 2, WN = 2, WGPC = 1, S = 4, OCC = 1; };
constexpr int kDKT = 64;

template <int EPI, int AL, int BMAP, class T>
static hipError_t mm_dense(const GemmArgs& g, int num_cus, hipStream_t st) {
  constexpr int BM = T::BM, BN = T::BN, WM = T::WM, WN = T::WN, kDWgPerCu = T::WGPC;
  const int ntiles = (g.N + BN - 1) / BN, slots = kDWgPerCu * num_cus;
  // the QKV epilogue always runs on fp32 sums (one split at least); other
  // products split over k (mm_plan, on the device) when their tiles leave
  // workgroup slots idle
  const long long cap = g.part ? g.part_cap / ((long long)g.M * g.N) : 0;
  const int cap_splits = int(std::min<long long>(cap, 64));
  if (EPI == E_QKV && cap_splits < 1) return hipErrorInvalidValue;
  const bool can_split = cap_splits >= 2 && g.K / 64 >= 2 * PE_MM_SPLIT_MIN_KTILES;
  // the grid covers the plan of every row count up to M (the device plans
  // from the rows it finds): the most items of any number of row tiles
  int grid = 0;
  for (int mt = 1; mt <= (g.M + BM - 1) / BM; ++mt) {
    const MmPlan p = mm_plan(mt * BM, BM, ntiles, g.K / 64, slots, cap_splits);
    grid = std::max(grid, p.per * p.ks);
  }
  hipLaunchKernelGGL((mm_kernel<EPI, AL, BMAP, BM, BN, WM, WN, kDKT, T::S, T::OCC>), dim3(unsigned(grid)),
                     dim3(64 * WM * WN), 0, st, g, ntiles, slots, cap_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (EPI == E_RESID || EPI == E_STORE) {
    if (g.nrm_out) {  // the split sum (or, unsplit, the stored rows) and the following RMSNorm
      if (g.N % 8 || g.N > 2048 * kNormMaxChunks || g.ldo != g.N || (g.nrm_xfull && g.rmap))
        return hipErrorInvalidValue;
      const long long blocks = std::min<long long>(g.M, 16LL * num_cus);
      hipLaunchKernelGGL((mm_resid_norm_kernel<EPI, kNormMaxChunks>), dim3(unsigned(blocks)), dim3(256), 0, st, g, g.M,
                         g.rpr, BM, ntiles, slots, cap_splits);
      return hipGetLastError();
    }
  }
  if (EPI != E_QKV && !can_split) return e;
  // rows the epilogue covers: every slot of a MASK-deduplicated QKV product
  const bool expand = EPI == E_QKV && g.dedup_k;
  const int rows = expand ? g.M / (g.dedup_k + 2) * (2 * g.dedup_k) : g.M;
  const int epi_rpr = expand ? 2 * g.dedup_k : g.rpr;
  const long long work = (long long)rows * (EPI == E_QKV || EPI == E_SILU ? g.N / 16 : g.N / 8);
  const long long blocks = std::min<long long>((work + 255) / 256, 8LL * num_cus);
  hipLaunchKernelGGL(mm_reduce_kernel<EPI>, dim3(unsigned(blocks)), dim3(256), 0, st, g, rows, epi_rpr, BM, ntiles,
                     slots, cap_splits);
  return hipGetLastError();
}

#ifndef PE_MM_T_FC
#define PE_MM_T_FC 0
#endif
#ifndef PE_MM_T_QKV
#define PE_MM_T_QKV 0
#endif
#ifndef PE_MM_T_RESID
#define PE_MM_T_RESID 0
#endif
#ifndef PE_MM_T_GU
#define PE_MM_T_GU -1
#endif
template <int EPI, int AL, int BMAP>
static hipError_t mm_tiles(int tile, const GemmArgs& g, int num_cus, hipStream_t st) {
  if (g.M <= kMmMinRows) return mm_dense<EPI, AL, BMAP, TileDeep>(g, num_cus, st);
  switch (tile) {
    case 1: return mm_dense<EPI, AL, BMAP, TileLarge>(g, num_cus, st);
    case 2: return mm_dense<EPI, AL, BMAP, TileMid>(g, num_cus, st);
    case 3: return mm_dense<EPI, AL, BMAP, TileWide>(g, num_cus, st);
    default: return mm_dense<EPI, AL, BMAP, TileSmall>(g, num_cus, st);
  }
}

hipError_t launch_mm(int aload, int bmap, int epi, const GemmArgs& g, int num_cus, hipStream_t st) {
  if (g.M <= 0) return hipSuccess;
  if (g.K % 64) return hipErrorInvalidValue;  // whole 64-wide k-tiles (and fc halves)
  if (g.N % 64) return hipErrorInvalidValue;  // whole 64-column pair blocks
  if (aload == A_FC && bmap == B_PLAIN && epi == E_STORE) return mm_tiles<E_STORE, A_FC, B_PLAIN>(PE_MM_T_FC, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_QKV && epi == E_QKV) return mm_tiles<E_QKV, A_PLAIN, B_QKV>(PE_MM_T_QKV, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_PLAIN && epi == E_RESID) return mm_tiles<E_RESID, A_PLAIN, B_PLAIN>(PE_MM_T_RESID, g, num_cus, st);
  if (aload == A_PLAIN && bmap == B_GATEUP && epi == E_SILU) {
    int t = PE_MM_T_GU;
    if (t < 0) {
      // The tile shape with the least work per CU: rounds of workgroups x
      // output area per CU and round (two 128x128 workgroups, or one of
      // 192x256 or 256x256 per CU).  Measured at c=64 (672 rows): 192x256
      // one round 80 us, 256x256 one round 91 us, 128x128 two rounds 105 us,
      // i.e. the same time per unit of area on all three.
      const long long rows = g.plan_rows > 0 ? g.plan_rows : g.M;
      auto cost = [&](int bm, int bn, int wgpc) {
        const long long tiles = ((rows + bm - 1) / bm) * ((g.N + bn - 1) / bn), slots = (long long)wgpc * num_cus;
        return ((tiles + slots - 1) / slots) * (long long)bm * bn * wgpc;
      };
      const long long cs = cost(TileSmall::BM, TileSmall::BN, TileSmall::WGPC), cm = cost(TileMid::BM, TileMid::BN, 1),
                      cl = cost(TileLarge::BM, TileLarge::BN, 1);
      t = cs <= cm && cs <= cl ? 0 : (cm <= cl ? 2 : 1);
    }
    return mm_tiles<E_SILU, A_PLAIN, B_GATEUP>(t, g, num_cus, st);
  }
  if (aload == A_PLAIN && bmap == B_PLAIN && epi == E_STORE) return mm_tiles<E_STORE, A_PLAIN, B_PLAIN>(0, g, num_cus, st);
  return hipErrorInvalidValue;
}

}  // namespace pe
