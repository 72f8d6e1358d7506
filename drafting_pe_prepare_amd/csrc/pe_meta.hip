// Batch preparation, hidden-state gather and greedy verification.
//
// "P-EAGLE: parallel speculative decoding in vLLM", vLLM implementation
// details: one fused pass copies the previous token ids and positions, inserts
// the bonus token, fills the parallel-draft slots with the MASK id and emits
// the rejected-token mask, the masked-token mask and the hidden-state map
// (Fused Triton kernel); rejected tokens map to PADDING_SLOT_ID = -1 so they
// make no KV-cache write (KV cache); a separate copy moves hidden states and
// broadcasts the learned placeholder into MASK slots (Hidden-state management).
//
// gfx950 design: one wavefront per request.  Slot j of the request is lane j
// (2K <= 64), so every per-slot field is written by one coalesced store per
// wave; validation uses wave ballots, not loops.  The gather is a plain 16-byte
// vector copy, grid-strided over all rows.
#include "pe_common.h"
#include "pe_internal.h"

namespace pe {

// Validates request r and, when `write`, stores its slot fields; one wave
// (lane = slot).  Returns the error kinds found (0: valid).
// An inactive request (r >= occupancy): padding slots, nothing validated or
// reported.  One wave (lane = slot).
__device__ __forceinline__ void pad_request(const PrepareArgs& a, int r, int lane) {
  const int K = a.K, S = 2 * K, base = r * S;
  if (lane < S) {
    a.ids[base + lane] = 0;
    a.pos[base + lane] = 0;
    a.hsrc[base + lane] = -1;
    a.rej[base + lane] = 1;
    a.msk[base + lane] = 0;
    a.slots[base + lane] = -1;
  }
  if (lane < K) a.draft_rows[r * K + lane] = base + lane;
  if (lane == 0) a.seq_lens[r] = 0;
}
__device__ __forceinline__ bool inactive(const int32_t* nact, int r) { return nact && r >= nact[0]; }

__device__ __forceinline__ uint32_t prepare_request(const PrepareArgs& a, int r, int lane, bool write) {
  const int K = a.K, S = 2 * K, base = r * S;
  const int32_t* vt = a.vt + (long long)r * (K + 1);
  const int32_t* vp = a.vp + (long long)r * (K + 1);
  // every load the wave needs first, at clamped (valid) addresses, so that
  // they are in flight together rather than one round trip after another
  const int acc = a.acc[r];
  const int p0 = vp[0];
  const int bonus = a.bonus[r];
  const int vt_l = vt[lane < K ? lane + 1 : K];  // d_{lane+1}
  const int vp_l = vp[lane < K ? lane : K];

  uint32_t kinds = 0;
  if (acc < 0 || acc > K) kinds |= 1u;
  // accepted drafts (lanes j < a read d_{j+1}) and the bonus token
  bool bad_tok = false;
  if (!(kinds & 1u)) {
    if (lane < acc) bad_tok = (vt_l < 0 || vt_l >= a.vocab);
    if (lane == acc) bad_tok = (bonus < 0 || bonus >= a.vocab);
  }
  if (__ballot(bad_tok)) kinds |= 2u;
  bool bad_pos = (lane <= K) && (vp_l != p0 + lane);
  if (__ballot(bad_pos)) kinds |= 8u;
  if (p0 < 0 || p0 > 0x7FFFFFFF - 2 * K - 1) kinds |= 4u;  // position range
  int seq_len = 0;
  if (kinds == 0) {
    seq_len = p0 + acc + K;
    const int nb = (seq_len + a.block_size - 1) / a.block_size;
    if (nb > a.max_blocks) {
      kinds |= 4u;
    } else {
      bool bad_blk = false;
      const int32_t* btr = a.bt + (long long)r * a.max_blocks;
      // 8 loads in flight per lane; indices past nb re-read entry nb - 1
      for (int b0 = lane; b0 < nb; b0 += 8 * 64) {
        int id[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) id[i] = btr[min(b0 + 64 * i, nb - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) bad_blk |= (id[i] < 0 || id[i] >= a.num_kv_blocks);
      }
      if (__ballot(bad_blk)) kinds |= 4u;
    }
  }

  if (!write) return kinds;
  if (kinds) {
    if (lane < S) {
      a.ids[base + lane] = 0;
      a.pos[base + lane] = 0;
      a.hsrc[base + lane] = -1;
      a.rej[base + lane] = 1;
      a.msk[base + lane] = 0;
      a.slots[base + lane] = -1;
    }
    if (lane < K) a.draft_rows[r * K + lane] = base + lane;
    if (lane == 0) {
      a.seq_lens[r] = 0;
      atomicOr(&a.err[0], kinds);
      atomicMin(&a.err[1], uint32_t(r));
    }
    return kinds;
  }

  const int32_t* btr = a.bt + (long long)r * a.max_blocks;
  if (lane < S) {
    int tok, p, src;
    uint8_t rej = 0, msk = 0;
    if (lane <= K) {
      p = vp_l;
      src = r * (K + 1) + lane;
      if (lane < acc) tok = vt_l;
      else if (lane == acc) tok = bonus;
      else { tok = 0; rej = 1; }
    } else {
      const int m = lane - K;
      tok = a.mask_id;
      p = p0 + acc + m;
      src = -1;
      msk = 1;
    }
    long long slot = -1;
    if (!rej) slot = (long long)btr[p / a.block_size] * a.block_size + p % a.block_size;
    a.ids[base + lane] = tok;
    a.pos[base + lane] = p;
    a.hsrc[base + lane] = src;
    a.rej[base + lane] = rej;
    a.msk[base + lane] = msk;
    a.slots[base + lane] = slot;
  }
  if (lane < K) a.draft_rows[r * K + lane] = (lane == 0) ? base + acc : base + K + lane;
  if (lane == 0) a.seq_lens[r] = seq_len;
  return 0;
}

__global__ __launch_bounds__(256) void prepare_kernel(PrepareArgs a) {
  const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (r >= a.B) return;
  if (inactive(a.nact, r)) pad_request(a, r, threadIdx.x & 63);
  else (void)prepare_request(a, r, threadIdx.x & 63, true);
}

hipError_t launch_prepare(const PrepareArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  const int per = 4;  // requests (waves) per workgroup
  hipLaunchKernelGGL(prepare_kernel, dim3((a.B + per - 1) / per), dim3(64 * per), 0, st, a);
  return hipGetLastError();
}

// draft_hidden[s] = src >= 0 ? H[src] : h_shared, as 16-byte chunks.
__global__ __launch_bounds__(256) void gather_kernel(int rows, int nsrc, int cpr,
                                                     const int32_t* __restrict__ hsrc,
                                                     const uint4* __restrict__ H,
                                                     const uint4* __restrict__ hs,
                                                     uint4* __restrict__ out) {
  const long long total = (long long)rows * cpr;
  for (long long c = blockIdx.x * (long long)blockDim.x + threadIdx.x; c < total;
       c += (long long)gridDim.x * blockDim.x) {
    const int row = int(c / cpr), k = int(c % cpr);
    const int src = hsrc[row];
    const uint4* p = (src >= 0 && src < nsrc) ? H + (long long)src * cpr : hs;
    out[c] = p[k];
  }
}

hipError_t launch_gather(int rows, int nsrc, int row_bytes, const int32_t* hsrc, const void* H,
                         const void* h_shared, void* out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int cpr = row_bytes / 16;
  const long long total = (long long)rows * cpr;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gather_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, rows, nsrc, cpr,
                     hsrc, (const uint4*)H, (const uint4*)h_shared, (uint4*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Drafting round after a prompt ("P-EAGLE: parallel speculative decoding in
// vLLM", Architecture and mechanism, Step 1 and Step 2): request r's S slots
// are the chunk's prompt positions c0..c0+n-1 (token one position later,
// the target's hidden state of the position; the last is the NTP slot with
// the new token), K-1 MASK slots after them, then rejected padding.  One
// workgroup per request, threads striding over the slots; validation with
// workgroup-wide votes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_prepare_kernel(PrefillArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x, K = a.K, S = a.S, L = S - K + 1;
  const long long base = (long long)r * S;
  const int n = a.lens[r], c0 = a.start[r];
  const int32_t* ct = a.ct + (long long)r * L;
  uint32_t kinds = 0;
  if (n < 1 || n > L) {
    kinds |= 1u;
  } else {
    bool bad = false;
    for (int j = 1 + tid; j < n; j += blockDim.x) bad |= ct[j] < 0 || ct[j] >= a.vocab;
    if (tid == 0) bad |= a.newt[r] < 0 || a.newt[r] >= a.vocab;
    if (__syncthreads_or(bad)) kinds |= 2u;
  }
  if (c0 < 0 || c0 > 0x7FFFFFFF - S) kinds |= 4u;
  if (kinds == 0) {
    const int seq_len = c0 + n + K - 1;
    const int nb = (seq_len + a.block_size - 1) / a.block_size;
    bool bad = nb > a.max_blocks;
    if (!bad) {
      const int32_t* btr = a.bt + (long long)r * a.max_blocks;
      for (int b = tid; b < nb; b += blockDim.x) bad |= btr[b] < 0 || btr[b] >= a.num_kv_blocks;
    }
    if (__syncthreads_or(bad)) kinds |= 4u;
  }
  if (kinds) {
    for (int j = tid; j < S; j += blockDim.x) {
      a.ids[base + j] = 0;
      a.pos[base + j] = 0;
      a.hsrc[base + j] = -1;
      a.rej[base + j] = 1;
      a.msk[base + j] = 0;
      a.slots[base + j] = -1;
    }
    if (tid < K) a.draft_rows[r * K + tid] = int(base) + tid;
    if (tid == 0) {
      a.seq_lens[r] = 0;
      atomicOr(&a.err[0], kinds);
      atomicMin(&a.err[1], uint32_t(r));
    }
    return;
  }
  const int32_t* btr = a.bt + (long long)r * a.max_blocks;
  const int valid = n + K - 1;
  for (int j = tid; j < S; j += blockDim.x) {
    int tok = 0, p = 0, src = -1;
    uint8_t rej = 0, msk = 0;
    long long slot = -1;
    if (j < valid) {
      p = c0 + j;
      if (j < n) {
        src = r * L + j;
        tok = j < n - 1 ? ct[j + 1] : a.newt[r];
      } else {
        tok = a.mask_id;
        msk = 1;
      }
      slot = (long long)btr[p / a.block_size] * a.block_size + p % a.block_size;
    } else {
      rej = 1;
    }
    a.ids[base + j] = tok;
    a.pos[base + j] = p;
    a.hsrc[base + j] = src;
    a.rej[base + j] = rej;
    a.msk[base + j] = msk;
    a.slots[base + j] = slot;
  }
  if (tid < K) a.draft_rows[r * K + tid] = int(base) + n - 1 + tid;
  if (tid == 0) a.seq_lens[r] = c0 + valid;
}

hipError_t launch_prefill_prepare(const PrefillArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_prepare_kernel, dim3(unsigned(a.B)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Preparation and hidden-state copy in one launch, for the step graph: one
// workgroup per (slot j, request r).  Every workgroup loads its slot's source
// row (slot j <= K copies target row r(K+1)+j) while wave 0 validates the
// request; an invalid request gets h_shared in every slot, as its hidden-source
// map of -1 says.  Workgroup j == 0 also writes the request's batch fields.
// One workgroup per request: wave 0 prepares the request's slots while every
// thread loads its first PG_CHUNKS 16-byte chunks of the request's 2K
// draft-hidden rows (source row r(K+1)+j for copied slot j, h_shared for the
// MASK slots); once the request is validated the rows are stored (an invalid request's
// copied slots take h_shared, as its -1 map says), and chunks beyond the first
// batch are copied in a loop.  One workgroup per request rather than per slot:
// a launch of many small workgroups is limited by how fast they are
// dispatched (c=64: 896 slot workgroups took ~20 us).
constexpr int PG_CHUNKS = 8;
__global__ __launch_bounds__(1024) void prepare_gather_kernel(PrepareArgs a, int cpr,
                                                              const uint4* __restrict__ H,
                                                              const uint4* __restrict__ hs,
                                                              uint4* __restrict__ out) {
  __shared__ uint32_t s_kinds;
  const int r = blockIdx.x, K = a.K, S = 2 * K, total = S * cpr, nt = blockDim.x;
  if (inactive(a.nact, r)) {  // its draft-hidden rows are not read
    if (threadIdx.x < 64) pad_request(a, r, threadIdx.x);
    return;
  }
  // chunk c of the request's rows, as its map says (returned by value: a
  // pointer select between the two sources would put v in scratch memory)
  auto source = [&](int c) {
    const int j = c / cpr, k = c - j * cpr;
    const long long row = j <= K ? (long long)(r * (K + 1) + j) * cpr : -1;
    return row >= 0 ? H[row + k] : hs[k];
  };
  uint4 v[PG_CHUNKS];
#pragma unroll
  for (int i = 0; i < PG_CHUNKS; ++i) v[i] = source(min(threadIdx.x + i * nt, total - 1));
  if (threadIdx.x < 64) {
    const uint32_t kinds = prepare_request(a, r, threadIdx.x, true);
    if (threadIdx.x == 0) s_kinds = kinds;
  }
  __syncthreads();
  uint4* dst = out + (long long)r * total;
  const bool valid = s_kinds == 0;
#pragma unroll
  for (int i = 0; i < PG_CHUNKS; ++i) {
    const int c = threadIdx.x + i * nt;
    if (c < total && valid) dst[c] = v[i];
  }
  if (valid) {
    for (int c = threadIdx.x + PG_CHUNKS * nt; c < total; c += nt) dst[c] = source(c);
  } else {
    // an invalid request: every slot takes h_shared
    for (int c = threadIdx.x; c < total; c += nt) dst[c] = hs[c % cpr];
  }
}

hipError_t launch_prepare_gather(const PrepareArgs& a, int row_bytes, const void* H,
                                 const void* h_shared, void* out, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (row_bytes % 16) return hipErrorInvalidValue;
  const int cpr = row_bytes / 16;
  if (2 * a.K > 64) {  // prepare_request takes one lane per slot: two launches
    const hipError_t e = launch_prepare(a, st);
    if (e != hipSuccess) return e;
    return launch_gather(a.B * 2 * a.K, a.B * (a.K + 1), row_bytes, a.hsrc, H, h_shared, out, st);
  }
  const long long total = 2LL * a.K * cpr;
  long long threads = (total + PG_CHUNKS - 1) / PG_CHUNKS;
  threads = std::min<long long>(1024, std::max<long long>(64, (threads + 63) / 64 * 64));
  hipLaunchKernelGGL(prepare_gather_kernel, dim3(unsigned(a.B)), dim3(unsigned(threads)), 0, st, a, cpr,
                     (const uint4*)H, (const uint4*)h_shared, (uint4*)out);
  return hipGetLastError();
}

// a' = first j with t[j] != g[j] (else K); bonus' = g[a'].  One wave per request.
__global__ __launch_bounds__(256) void verify_kernel(int B, int K, const int32_t* __restrict__ t,
                                                     const int32_t* __restrict__ g,
                                                     int32_t* __restrict__ acc,
                                                     int32_t* __restrict__ bonus,
                                                     const int32_t* __restrict__ nact) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (r >= B) return;
  if (inactive(nact, r)) {  // an inactive request: accepted 0, bonus PE_PAD_TOKEN
    if (lane == 0) {
      acc[r] = 0;
      bonus[r] = 0;
    }
    return;
  }
  const bool miss = lane < K && t[(long long)r * K + lane] != g[(long long)r * (K + 1) + lane];
  const unsigned long long m = __ballot(miss);
  const int a = m ? (__ffsll((long long)m) - 1) : K;
  if (lane == 0) {
    acc[r] = a;
    bonus[r] = g[(long long)r * (K + 1) + a];
  }
}

// The non-rejected slots of a batch, in order (the rows the large-batch
// dense products compute; a rejected slot's outputs are never read: it makes
// no KV write, attends to nothing and is no draft row).  One 1024-thread
// workgroup: thread t counts its contiguous run of slots, a block-wide scan
// gives each run's first output index, then the runs are written.
__device__ void compact_rows(int R, const uint8_t* __restrict__ rej, int32_t* __restrict__ rmap,
                             int32_t* __restrict__ count) {
  __shared__ int s_w[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (R + 1023) / 1024, r0 = min(R, t * per), r1 = min(R, r0 + per);
  int n = 0;
  for (int r = r0; r < r1; ++r) n += rej[r] ? 0 : 1;
  int inc = n;  // inclusive scan inside the wave, then across the 16 waves
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int base = 0;
  for (int v = 0; v < w; ++v) base += s_w[v];
  int at = base + inc - n;
  for (int r = r0; r < r1; ++r)
    if (!rej[r]) rmap[at++] = r;
  if (t == 1023) *count = base + inc;
}

// The non-rejected draft rows of a batch, in draft-row order: dmap[0..*count),
// and a query mask for the last layer's attention, qskip[s] = 0 exactly for
// those slots.  Only the draft rows feed the LM head, so after the last
// layer's QKV product (which writes every valid slot's KV) the attention
// rows, O product and MLP of the other slots are never read.  One workgroup.
__device__ void draft_map(int R, int D, const int32_t* __restrict__ draft_rows, const uint8_t* __restrict__ rej,
                          int32_t* __restrict__ dmap, int32_t* __restrict__ count, int32_t* __restrict__ dpos,
                          uint8_t* __restrict__ qskip, uint4* __restrict__ z, int zc) {
  __shared__ int s_w[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int s = t; s < R; s += 1024) qskip[s] = 1;
  __syncthreads();  // the draft rows' clears below land after every set
  const int per = (D + 1023) / 1024, i0 = min(D, t * per), i1 = min(D, i0 + per);
  auto live = [&](int i) {
    const int s = draft_rows[i];
    return s >= 0 && s < R && !rej[s];
  };
  int n = 0;
  for (int i = i0; i < i1; ++i) n += live(i) ? 1 : 0;
  int inc = n;  // inclusive scan inside the wave, then across the 16 waves
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int base = 0;
  for (int v = 0; v < w; ++v) base += s_w[v];
  int at = base + inc - n;
  for (int i = i0; i < i1; ++i)
    if (live(i)) {
      const int s = draft_rows[i];
      dpos[at] = i;
      dmap[at++] = s;
      qskip[s] = 0;
    } else if (z) {
      for (int c = 0; c < zc; ++c) z[(long long)i * zc + c] = uint4{0u, 0u, 0u, 0u};
    }
  if (t == 1023) *count = base + inc;
}

// Both maps in one launch: workgroup 0 the row map, workgroup 1 (when the
// draft map is asked for) the draft map; they read the same mask and write
// disjoint outputs.
__global__ __launch_bounds__(1024) void row_maps_kernel(int R, const uint8_t* __restrict__ rej,
                                                        int32_t* __restrict__ rmap, int32_t* __restrict__ rcount,
                                                        int D, const int32_t* __restrict__ draft_rows,
                                                        int32_t* __restrict__ dmap, int32_t* __restrict__ dcount,
                                                        int32_t* __restrict__ dpos, uint8_t* __restrict__ qskip,
                                                        uint4* __restrict__ z, int zc) {
  if (blockIdx.x == 0) compact_rows(R, rej, rmap, rcount);
  else draft_map(R, D, draft_rows, rej, dmap, dcount, dpos, qskip, z, zc);
}

hipError_t launch_row_maps(int R, const uint8_t* rejected, int32_t* rmap, int32_t* rcount, int D,
                           const int32_t* draft_rows, int32_t* dmap, int32_t* dcount, int32_t* dpos, uint8_t* qskip,
                           void* z, int d, hipStream_t st) {
  if (R <= 0 || (draft_rows && D <= 0) || (z && (d <= 0 || d % 8))) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_maps_kernel, dim3(draft_rows ? 2 : 1), dim3(1024), 0, st, R, rejected, rmap, rcount, D,
                     draft_rows, dmap, dcount, dpos, qskip, (uint4*)z, z ? d / 8 : 0);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int K, const int32_t* t, const int32_t* g, int32_t* acc,
                         int32_t* bonus, const int32_t* nact, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(verify_kernel, dim3((B + 3) / 4), dim3(256), 0, st, B, K, t, g, acc, bonus, nact);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Autoregressive comparison: the batches of EAGLE's sequential drafting passes
// ("P-EAGLE: parallel speculative decoding in vLLM", Solving the
// autoregressive drafting bottleneck: one drafter pass per draft token).
// ---------------------------------------------------------------------------

// First pass: the K+1 copied slots of every request, compacted to stride K+1,
// with their hidden rows; the draft row is the NTP slot.  One 64-thread
// workgroup per (request, copied slot).
__global__ __launch_bounds__(64) void ar_first_kernel(ArArgs a) {
  const int K = a.K, S = 2 * K, S1 = K + 1;
  const int r = blockIdx.x / S1, j = blockIdx.x - r * S1;
  const long long src = (long long)r * S + j, dst = blockIdx.x;
  const int cpr = a.row_bytes / 16;
  const uint4* h = (const uint4*)a.hidden + src * cpr;
  uint4* o = (uint4*)a.p_hidden + dst * cpr;
  for (int i = threadIdx.x; i < cpr; i += 64) o[i] = h[i];
  if (threadIdx.x == 0) {
    a.p_ids[dst] = a.ids[src];
    a.p_pos[dst] = a.pos[src];
    a.p_rej[dst] = a.rej[src];
    a.p_slots[dst] = a.slots[src];
    if (j == 0) {
      int acc = a.draft_rows[(long long)r * K] - r * S;  // the NTP slot is copied slot a
      acc = acc < 0 ? 0 : (acc > K ? K : acc);
      a.p_rows[r] = r * S1 + acc;
      const int L = a.seq_lens[r];  // p0 + a + K; the first pass sees p0 + a + 1
      a.p_seq[r] = L > 0 ? L - (K - 1) : 0;
    }
  }
}

// Pass k (drafts t_{k+1}, k = 1..K-1): one slot per request holding t_k at the
// next position, paired with the drafter's output hidden state of the previous
// pass's draft row.  One 64-thread workgroup per request.
__global__ __launch_bounds__(64) void ar_next_kernel(ArArgs a) {
  const int r = blockIdx.x;
  const int cpr = a.row_bytes / 16;
  const int prev = a.p_rows[r];
  const uint4* h = (const uint4*)a.hidden + (long long)prev * cpr;
  uint4* o = (uint4*)a.p_hidden + (long long)r * cpr;
  for (int i = threadIdx.x; i < cpr; i += 64) o[i] = h[i];
  __syncthreads();  // every lane has read p_rows[r] before it is replaced
  if (threadIdx.x == 0) {
    const int L = a.p_seq[r];
    const int tok = a.tokens[(long long)r * a.K + a.k - 1];
    const int p = L;  // the previous pass saw positions [0, L)
    const int blk = (L > 0 && p / a.block_size < a.max_blocks)
                        ? a.bt[(long long)r * a.max_blocks + p / a.block_size] : -1;
    if (L <= 0 || tok < 0 || blk < 0 || blk >= a.num_kv_blocks) {
      a.p_ids[r] = 0;
      a.p_pos[r] = 0;
      a.p_rej[r] = 1;
      a.p_slots[r] = -1;
      a.p_seq[r] = 0;
    } else {
      a.p_ids[r] = tok;
      a.p_pos[r] = p;
      a.p_rej[r] = 0;
      a.p_slots[r] = (long long)blk * a.block_size + p % a.block_size;
      a.p_seq[r] = L + 1;
    }
    a.p_rows[r] = r;
  }
}

hipError_t launch_ar_first(const ArArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(ar_first_kernel, dim3(a.B * (a.K + 1)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ar_next(const ArArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(ar_next_kernel, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

// ---- DFlash-style round ------------------------------------------------------
// "vLLM Speculators: parallel drafting for speculative decoding", comparison
// of P-EAGLE, DFlash and DSpark (DFlash: verifier hidden states are projected
// into the drafter's KV cache; block diffusion drafts the candidates).  Per
// request, one wave (lane = slot, K+1 <= 64): the block [bonus, MASK x K] at
// positions p0+a+1.., every slot seeing the whole block (horizon p0+a+K+1),
// the MASK slots as draft rows, and the KV slots the injection writes (the
// kept context positions p0..p0+a; -1 for rejected ones).  Validation as the
// P-EAGLE preparation; an invalid request becomes padding.
__global__ __launch_bounds__(256) void dflash_prepare_kernel(DflashArgs a) {
  const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= a.B) return;
  const int K = a.K, S = K + 1, base = r * S;
  const bool off = inactive(a.nact, r);  // an inactive request: padding, nothing validated or reported
  const int32_t* vp = a.vp + (long long)r * S;
  const int acc = off ? 0 : a.acc[r], p0 = off ? 0 : vp[0], bonus = off ? 0 : a.bonus[r];
  const int vp_l = off ? lane : vp[lane < K ? lane : K];
  uint32_t kinds = off ? 0x80000000u : 0u;
  if (acc < 0 || acc > K) kinds |= 1u;
  else if (bonus < 0 || bonus >= a.vocab) kinds |= 2u;
  if (__ballot(lane <= K && vp_l != p0 + lane)) kinds |= 8u;
  if (p0 < 0 || p0 > 0x7FFFFFFF - 2 * K - 2) kinds |= 4u;
  const int32_t* btr = a.bt + (long long)r * a.max_blocks;
  if (kinds == 0) {
    const int nb = (p0 + acc + K + 2 + a.block_size - 1) / a.block_size;
    if (nb > a.max_blocks) {
      kinds |= 4u;
    } else {
      bool bad = false;
      // 8 loads in flight per lane; indices past nb re-read entry nb - 1
      for (int b0 = lane; b0 < nb; b0 += 8 * 64) {
        int id[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) id[i] = btr[min(b0 + 64 * i, nb - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) bad |= id[i] < 0 || id[i] >= a.num_kv_blocks;
      }
      if (__ballot(bad)) kinds |= 4u;
    }
  }
  if (kinds) {
    if (lane < S) {
      a.ids[base + lane] = 0;
      a.pos[base + lane] = 0;
      a.apos[base + lane] = 0;
      a.hsrc[base + lane] = -1;
      a.rej[base + lane] = 1;
      a.msk[base + lane] = 0;
      a.slots[base + lane] = -1;
      a.inj[base + lane] = -1;
    }
    if (lane < K) a.draft_rows[r * K + lane] = base + 1 + lane;
    if (lane == 0) {
      a.seq_lens[r] = 0;
      if (!off) {
        atomicOr(&a.err[0], kinds);
        atomicMin(&a.err[1], uint32_t(r));
      }
    }
    return;
  }
  const int bs = a.block_size;
  if (lane < S) {
    const int p = p0 + acc + 1 + lane, c = p0 + lane;
    a.ids[base + lane] = lane == 0 ? bonus : a.mask_id;
    a.pos[base + lane] = p;
    a.apos[base + lane] = p0 + acc + K + 1;
    a.hsrc[base + lane] = -1;
    a.rej[base + lane] = 0;
    a.msk[base + lane] = lane == 0 ? 0 : 1;
    a.slots[base + lane] = (long long)btr[p / bs] * bs + p % bs;
    a.inj[base + lane] = lane <= acc ? (long long)btr[c / bs] * bs + c % bs : -1LL;
  }
  if (lane < K) a.draft_rows[r * K + lane] = base + 1 + lane;
  if (lane == 0) a.seq_lens[r] = p0 + acc + K + 2;
}

hipError_t launch_dflash_prepare(const DflashArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 63) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dflash_prepare_kernel, dim3((a.B + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pe
