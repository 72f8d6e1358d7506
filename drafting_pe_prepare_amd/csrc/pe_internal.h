// Launchers of the libpe kernels, called by the host runtime (pe_api.cpp).
// Every launcher only enqueues work on `st`; shapes were validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

// ---- metadata -------------------------------------------------------------
struct PrepareArgs {
  int B, K, vocab, mask_id, block_size, max_blocks, num_kv_blocks;
  const int32_t *vt, *vp, *acc, *bonus, *bt;
  int32_t *ids, *pos, *hsrc, *draft_rows, *seq_lens;
  uint8_t *rej, *msk;
  int64_t* slots;
  uint32_t* err;  // [0] kinds (OR), [1] first failing request (min)
  const int32_t* nact = nullptr;  // occupancy: requests >= *nact are inactive padding (NULL: all active)
};
hipError_t launch_prepare(const PrepareArgs& a, hipStream_t st);

hipError_t launch_gather(int rows, int nsrc, int row_bytes, const int32_t* hsrc, const void* H,
                         const void* h_shared, void* out, hipStream_t st);

// nact: occupancy (NULL: all active); an inactive request gets accepted 0, bonus 0
hipError_t launch_verify(int B, int K, const int32_t* t, const int32_t* g, int32_t* acc,
                         int32_t* bonus, const int32_t* nact, hipStream_t st);

// Drafting round after a prompt: one workgroup per request.
struct PrefillArgs {
  int B, K, S, vocab, mask_id, block_size, max_blocks, num_kv_blocks;
  const int32_t *ct, *lens, *start, *newt, *bt;  // chunk_tokens [B, S-K+1]
  int32_t *ids, *pos, *hsrc, *draft_rows, *seq_lens;
  uint8_t *rej, *msk;
  int64_t* slots;
  uint32_t* err;
};
hipError_t launch_prefill_prepare(const PrefillArgs& a, hipStream_t st);

// Verification by rejection sampling over fp32 logits: drafter rows [B*K, V],
// verifier rows [B*(K+1), V]; workspace lse [B*(2K+1)], part_ms
// [B*(2K+1)*kLseParts*2], keys [B*kSampleParts].  V % 4 == 0.
constexpr int kSampleParts = 64;
constexpr int kLseParts = 16;
// Draft tokens drawn from softmax(logits / T) of each of M rows (row stride
// ldl): Gumbel-max over kSampleParts vocabulary slices (keys [M*kSampleParts]),
// -1 for a padded request (seq_lens[row / Kd] == 0).
hipError_t launch_sample_drafts(int M, int Kd, int V, int ldl, float inv_temp, const float* logits,
                                const uint64_t* seed, uint64_t* keys, int32_t* tokens, int tstride,
                                const int32_t* seq_lens, hipStream_t st);
hipError_t launch_verify_sampled(int B, int K, int V, float inv_temp, const int32_t* draft_tokens,
                                 const float* draft_logits, const float* target_logits,
                                 const uint64_t* seed, float* lse, float* part_ms, uint64_t* keys,
                                 int32_t* accepted, int32_t* next_tokens, hipStream_t st);

// Step-graph fusions: preparation + hidden-state copy; argmax + verification.
hipError_t launch_prepare_gather(const PrepareArgs& a, int row_bytes, const void* H,
                                 const void* h_shared, void* out, hipStream_t st);
hipError_t launch_argmax_verify(int B, int K, int parts, const uint64_t* keys, int32_t* tokens,
                                const int32_t* seq_lens, const int32_t* target, int32_t* acc,
                                int32_t* bonus, const int32_t* nact, hipStream_t st);

// DFlash-style round: the block batch (S = K+1 slots per request), each
// slot's attention horizon (apos) and the KV slots of the injected context
// rows [B*(K+1)] (-1: not written).
struct DflashArgs {
  int B, K, vocab, mask_id, block_size, max_blocks, num_kv_blocks;
  const int32_t *vp, *acc, *bonus, *bt;
  int32_t *ids, *pos, *apos, *hsrc, *draft_rows, *seq_lens;
  uint8_t *rej, *msk;
  int64_t *slots, *inj;
  uint32_t* err;
  const int32_t* nact = nullptr;  // occupancy, as PrepareArgs::nact
};
hipError_t launch_dflash_prepare(const DflashArgs& a, hipStream_t st);

// ---- autoregressive comparison --------------------------------------------
// Pass batches of sequential drafting, built on the device from the parallel
// batch (stride 2K) so that a captured graph replays them.
struct ArArgs {
  int B, K, row_bytes, block_size, max_blocks, num_kv_blocks;
  // parallel batch
  const int32_t *ids, *pos, *draft_rows, *seq_lens;
  const uint8_t* rej;
  const int64_t* slots;
  const int32_t* bt;
  const void* hidden;     // first pass: draft hidden [B*2K, d]; later: residual stream of the previous pass
  const int32_t* tokens;  // [B, K] drafted so far; pass k reads column k-1
  int k;
  // pass batch (workspace)
  int32_t *p_ids, *p_pos, *p_rows, *p_seq;
  uint8_t* p_rej;
  int64_t* p_slots;
  void* p_hidden;
};
hipError_t launch_ar_first(const ArArgs& a, hipStream_t st);
hipError_t launch_ar_next(const ArArgs& a, hipStream_t st);

// ---- normalisation --------------------------------------------------------
// out[i] = x[row(i)] * rsqrt(mean(x^2) + eps) * gain; row(i) = rows_idx ? rows_idx[i] : i
// (scatter: out[row(i)] instead of out[i])
hipError_t launch_rmsnorm(int dtype, int rows, int d, const void* x, const void* gain, void* out,
                          const int32_t* rows_idx, int rows_bound, float eps, hipStream_t st, bool scatter = false);
// bf16 RMSNorm of the compact rows of a MASK-deduplicated first layer (K+2
// per request, see GemmArgs::dedup_k) that also writes each raw row x[m] to
// its slots of the full layout: x_full[s] = x[dedup_row(s, K)] for all B*2K s.
// One launch, two maps.  The non-rejected rows of a batch of R slots, in
// order: rmap[0..*rcount).  With draft_rows set, also the non-rejected draft
// rows (draft_rows[0..D) in order): dmap[0..*dcount), their draft indices
// dpos[0..*dcount) (draft_rows[dpos[m]] = dmap[m]), and qskip[s] = 0 for
// exactly those slots (1 elsewhere); with z set too (bf16, [D, d]), the rows
// of z at the other draft indices are zeroed (the fused final norm writes the
// non-rejected ones only).
hipError_t launch_row_maps(int R, const uint8_t* rejected, int32_t* rmap, int32_t* rcount, int D,
                           const int32_t* draft_rows, int32_t* dmap, int32_t* dcount, int32_t* dpos, uint8_t* qskip,
                           void* z, int d, hipStream_t st);
hipError_t launch_rmsnorm_expand(int rows, int d, const void* x, const void* gain, void* out, void* x_full,
                                 int K, float eps, hipStream_t st);

// ---- GEMM  out[m, n] = sum_k A[m, k] W[n, k]  + fused epilogue -------------
enum ALoad { A_PLAIN = 0, A_FC = 1 };
enum BMap { B_PLAIN = 0, B_QKV = 1, B_GATEUP = 2 };
enum Epi { E_STORE = 0, E_RESID = 1, E_SILU = 2, E_QKV = 3, E_ARGMAX = 4, E_PART = 5 };

struct GemmArgs {
  int M, N, K;  // N counts logical columns (2*I for gate/up; q+k+v dims for QKV)
  // A operand
  const void* A;  int lda;                        // A_PLAIN: A[m*lda + k]
  const void* embed; const int32_t* ids;          // A_FC: k < d -> embed[ids[m]*d + k]
  const void* hid; int d; int vocab;              //       k >= d -> hid[m*d + k - d]
  // B operand (weights, row-major [rows, K])
  const void* W0; const void* W1; const void* W2;
  const void* Wp;  // optional fragment-order copy of W0 (see launch_pack_frag16)
  int nq, nk;                                     // B_QKV: rows of Wq, Wk (Wv follows)
  // epilogue
  void* out; int ldo; const void* resid;          // E_STORE / E_RESID / E_SILU
  const int32_t* positions; const int64_t* slots; // E_QKV
  void* qout; void* kcache; void* vcache;
  int Hkv, hd, block_size; long long num_slots;
  const double* rope_turns;  // [hd/2] theta^(-2i/hd) / (2 pi): RoPE angle per position, in turns
  uint64_t* keys; int parts;                      // E_ARGMAX: keys[row * parts + part]
  int32_t* tokens; float* logits; int ldl;         // logits[row * ldl + n]
  const int32_t* seq_lens; int Kd;
  // split-K: fp32 partial sums [ksplit][M][N] (logical columns) for GEMMs with
  // too few output tiles to fill the chip; the epilogue runs after the sum
  float* part; long long part_cap;  // capacity in floats (0: never split)
  int ksplit;
  // MASK-slot deduplication in the parallel-step layout (K = dedup_k > 0):
  // the K-1 MASK slots of a request share one input row, so the first layer's
  // fc and QKV products run on K+2 rows per request (copied slots 0..K and
  // one MASK slot).  fc (A_FC): compact row m reads slot
  // (m / (K+2)) * 2K + m % (K+2).  E_QKV epilogue over fp32 sums: slot m reads
  // compact row dedup_row(m, K).
  int dedup_k;
  // occupancy (large-batch kernels): when set, only the first *nact * rpr
  // rows (rpr rows per request) are computed; later rows are inactive padding
  const int32_t* nact;
  int rpr;
  // row map (large-batch kernels): when set, compact row m < *rcount stands
  // for row rmap[m] of A and of the output, and rows past *rcount are not
  // computed (the forward pass maps the non-rejected slots, whose outputs are
  // the only ones anything reads).  Not combined with dedup_k.
  const int32_t* rmap;
  const int32_t* rcount;
  // rows the tile shape is chosen for (0: M); with a row map the count is
  // known only on the device, and this is its expected size
  int plan_rows;
  // RMSNorm folded into small-batch products (at most 16 rows, every dense
  // product on gemm_skinny).  A producer of x (E_STORE / E_RESID) with
  // ssq_out set also writes, for each 16-column tile p of its output, the sum
  // of squares of every stored (rounded) row: ssq_out[row * ssq_n + p].  A
  // consumer (A_PLAIN) with norm_gain set reads its A rows x through the
  // norm: rs = rsqrt(sum_p ssq_in[row * ssq_n + p] / K + norm_eps), operand
  // bf16((x * rs) * gain), as rmsnorm_kernel would have stored it.
  float* ssq_out;
  const float* ssq_in;
  const void* norm_gain;
  float norm_eps;
  int ssq_n;
  // RMSNorm fused after a large-batch residual product (E_RESID on
  // launch_mm): with nrm_out set, the product's split-K sum also normalises
  // every output row it writes, nrm_out[row] = bf16((x * rs) * nrm_gain) with
  // rs = rsqrt(mean(x^2) + norm_eps) over the stored (rounded) x, as
  // rmsnorm_kernel would have.  With nrm_rows set, compact row m's
  // normalised row goes to nrm_out[nrm_rows[m]] instead.  A store product
  // (E_STORE) takes it too (no residual); with dedup_k and nrm_xfull set, each
  // stored row x also goes to its slots of the full layout,
  // nrm_xfull[s] = x[dedup_row(s, dedup_k)].
  void* nrm_out;
  const void* nrm_gain;
  const int32_t* nrm_rows;
  void* nrm_xfull;
};
// Whether a product of M rows can take its RMSNorm folded in (see GemmArgs):
// bf16, at most 16 rows, K % 32 == 0, K / 16 <= kSsqMaxParts partial sums.
constexpr int kSsqMaxParts = 256;
bool gemm_folds_norm(int dtype, int M, int K);
// rows of an M-row operand with rpr rows per request that belong to active requests
__device__ __forceinline__ int active_rows(const int32_t* nact, int rpr, int M) {
  if (!nact) return M;
  const long long n = (long long)max(nact[0], 0) * rpr;
  return n < M ? int(n) : M;
}
__host__ __device__ inline int dedup_row(int slot, int K) {
  const int j = slot % (2 * K);
  return (slot / (2 * K)) * (K + 2) + (j < K + 1 ? j : K + 1);
}
hipError_t launch_gemm(int dtype, int aload, int bmap, int epi, const GemmArgs& g, int num_cus,
                       hipStream_t st);
// Copies the logical bf16 weight of a GEMM (W0/W1/W2 through the bmap row
// mapping; N % 16 == 0, K % 32 == 0) into fragment order: 1 KB block (16-row
// tile t, k-step s) holds lane l's 16 B at byte 16 l, i.e.
// W[16t + l%16][32s + 8(l/16) .. +8].
hipError_t launch_pack_frag16(int bmap, const GemmArgs& g, void* out, hipStream_t st);
// Number of partial argmax keys per row the E_ARGMAX GEMM of this shape writes.
int gemm_argmax_parts(int dtype, int M, int N, int K, int num_cus);
// After an E_ARGMAX GEMM: max over each row's partial keys -> tokens[row *
// tstride] (-1 for a padded request, seq_lens[row / Kd] == 0).
hipError_t launch_argmax_tokens(int M, int Kd, int parts, const uint64_t* keys, int32_t* tokens,
                                int tstride, const int32_t* seq_lens, hipStream_t st);

// ---- attention ------------------------------------------------------------
constexpr int kAttnMaxB = 1024;  // requests (or slot groups) per attention launch
struct AttnArgs {
  int B, S, Hq, Hkv, hd, block_size, max_blocks;
  long long num_slots;
  float scale;
  const void* q;                  // [B*S, Hq, hd]
  const void* kcache; const void* vcache;
  const int32_t* positions; const uint8_t* rej; const int32_t* seq_lens; const int32_t* bt;
  void* out;                      // [B*S, Hq*hd]
  float* part_o; float* part_ml;  // split-KV partials (bf16 path)
  int32_t* plan_off;              // [B+2] steps before each request, then the workgroups with a range; written by the partial kernel for the merge
  int vpr;                        // consecutive (virtual) requests per block-table row
  int grid;                       // workgroups of the partial kernel (each takes an equal range of steps)
};
// ---- large-batch dense products (more than 256 rows) -------------------------
// Dense products with more rows than PE_MM_MIN_ROWS run on launch_mm; from
// kRowMapMinRows + 1 rows up so do all but gate/up (a four-stage ring of
// 64 x 128 tiles, see pe_mm.hip); smaller ones, and gate/up up to
// PE_MM_MIN_ROWS rows, on the kernels of pe_gemm.hip.  The LM head stays on
// pe_gemm.hip at every size: at 448 rows x 201088 x 2880 its ring (224 x 256
// tiles) measured 524-568 us against 572-692 us for the best 32x32x16 tiles.
#ifndef PE_MM_MIN_ROWS
#define PE_MM_MIN_ROWS 256
#endif
constexpr int kMmMinRows = PE_MM_MIN_ROWS;
// Row maps (GemmArgs::rmap: rejected slots skipped, the last layer's draft
// rows only) from this many rows up: such products run on gemm_tiled (65..256
// rows) or the large-batch kernels, never on gemm_skinny.
constexpr int kRowMapMinRows = 64;
// 32x32x16 MFMA tiles; QKV and gate/up pair their epilogue columns 32 apart
// (see pe_mm.hip).  E_QKV runs on fp32 sums (g.part); with g.dedup_k the
// product covers the K+2 compact rows per request and the epilogue every slot.
hipError_t launch_mm(int aload, int bmap, int epi, const GemmArgs& g, int num_cus, hipStream_t st);

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st);
// Context length of each group of Sv consecutive slots (vpr groups per
// request): 1 + the highest position of a non-rejected slot in the group,
// capped by the request's seq_len (0 when the group has none).
hipError_t launch_attn_group_lens(int Bv, int Sv, int vpr, const int32_t* positions, const uint8_t* rej,
                                  const int32_t* seq_lens, int32_t* out, hipStream_t st);
// Split-KV partials of a launch over B requests with `grid` workgroups
// (sizes the partial buffers).
long long attn_max_items(int B, int Hkv, int grid);

}  // namespace pe
