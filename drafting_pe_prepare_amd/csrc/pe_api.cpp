// Host runtime of libpe: the C ABI declared in include/pe.h.
//
// A context owns the workspace of one drafter (activations sized for
// max_num_seqs requests, split-KV attention partials, argmax keys, the device
// error word) and at most one captured step graph.  Every entry point
// validates its arguments on the host, then only enqueues kernels on the
// context's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pe.h"
#include "pe_internal.h"

// Products of more rows than this write the following RMSNorm in their
// split-K sums on the large-batch kernels (up to 16 rows the small-batch
// products fold it in instead).  From 17 rows, against separate norm
// launches: K sweep K = 1 (32 rows) 504 -> 482 us.
#ifndef PE_POSTNORM_MIN_ROWS
#define PE_POSTNORM_MIN_ROWS 16
#endif


namespace {

thread_local std::string g_err;

pe_status fail(pe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pe_status fail(pe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

pe_status hipfail(hipError_t e, const char* what) {
  return fail(PE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define PE_HIP(call, what)                        \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hipfail(e_, what); \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

struct pe_ctx {
  pe_config cfg;
  pe_weights w;
  std::vector<pe_layer_weights> layers;
  hipStream_t stream = nullptr;
  int device = 0;
  int num_cus = 256;
  size_t esz = 2;
  // workspace
  void* x = nullptr;     // [R, d]   residual stream
  void* u = nullptr;     // [R, d]   normalised rows
  void* q = nullptr;     // [R, Hq*hd] rotated queries
  void* attn = nullptr;  // [R, Hq*hd] attention output
  void* mlp = nullptr;   // [R, I]   SiLU(gate) * up
  void* z = nullptr;     // [D, d]   final-norm draft rows
  uint64_t* keys = nullptr;   // [D, parts] partial argmax keys of the LM head
  uint32_t* err = nullptr;    // [2] kinds, first request
  float* part_o = nullptr;
  float* part_ml = nullptr;
  int32_t* plan_off = nullptr;  // split-KV plan handed from the partial to the merge kernel
  float* sample_lse = nullptr;     // rejection sampling: log-sum-exp per logit row
  float* sample_parts = nullptr;   // rejection sampling: (max, sum exp) per row slice
  uint64_t* sample_keys = nullptr; // rejection sampling: partial draw keys
  int32_t* group_lens = nullptr; // attention context length per slot group (bf16)
  int attn_group = 64;           // slots per attention workgroup: 512 / G rounded down to a power of two
  int groups_max = 0;            // slot groups the attention buffers are sized for
  void* xc = nullptr;  // [B(K+2), d] first-layer fc output on the MASK-deduplicated rows (bf16)
  float* splitk = nullptr;      // split-K GEMM partials (bf16 storage)
  int32_t* rmap = nullptr;      // [R] non-rejected slots of a large-batch pass, then their count
  int32_t* dmap = nullptr;      // [2D+1] non-rejected draft rows of a large-batch pass, their count, their draft indices
  uint8_t* qskip = nullptr;     // [R] last-layer attention: 0 for the non-rejected draft rows
  float* ssq = nullptr;         // [16][d/16] per-tile sums of squares of x (RMSNorm folded into small-batch products)
  long long splitk_cap = 0;     // floats
  double* rope_turns = nullptr;  // RoPE frequencies in turns per position
  void* lm_packed = nullptr;  // fragment-order copy of the LM head (bf16)
  // fragment-order copies of the small-batch GEMM weights (bf16): fc, then per
  // layer qkv (RoPE-paired columns), o, gate/up (paired), down
  void* fc_packed = nullptr;
  std::vector<void*> layer_packed;  // 4 per layer
  // autoregressive comparison: the batch of one sequential pass (B*(K+1) slots)
  int32_t *ar_ids = nullptr, *ar_pos = nullptr, *ar_rows = nullptr, *ar_seq = nullptr;
  uint8_t* ar_rej = nullptr;
  int64_t* ar_slots = nullptr;
  void* ar_hidden = nullptr;
  int attn_grid = 512;
  long long items_max = 0;
  // step graph
  const int32_t* nact = nullptr;  // occupancy of the step being captured (NULL: every request active)
  int64_t graph_captures = 0, graph_replays = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  hipStream_t capture_stream = nullptr;  // private: the default stream cannot be captured
  int graph_B = -1;
  pe_step_args graph_args;
  std::vector<void*> graph_kv;
  // profiling
  bool prof_on = false;
  bool capturing = false;
  std::vector<hipEvent_t> ev_free;
  struct Rec { int phase; hipEvent_t a, b; };
  std::vector<Rec> recs;
  double prof_ms[PE_PH_COUNT] = {};
  int64_t prof_n[PE_PH_COUNT] = {};
};

namespace {

// Brackets one phase's launches with an event pair when profiling is on.
struct Timed {
  pe_ctx* c;
  int phase;
  hipEvent_t a = nullptr, b = nullptr;
  static hipEvent_t take(pe_ctx* c) {
    if (!c->ev_free.empty()) { hipEvent_t e = c->ev_free.back(); c->ev_free.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  Timed(pe_ctx* ctx, int ph) : c(ctx), phase(ph) {
    if (!c->prof_on || c->capturing || c->recs.size() > 200000) return;
    a = take(c);
    b = take(c);
    if (a && b) (void)hipEventRecord(a, c->stream);
  }
  ~Timed() {
    if (a && b) {
      (void)hipEventRecord(b, c->stream);
      c->recs.push_back({phase, a, b});
    } else {
      if (a) c->ev_free.push_back(a);
      if (b) c->ev_free.push_back(b);
    }
  }
};

}  // namespace

namespace {

void free_ctx(pe_ctx* c) {
  if (!c) return;
  if (c->gexec) (void)hipGraphExecDestroy(c->gexec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->capture_stream) (void)hipStreamDestroy(c->capture_stream);
  for (auto& r : c->recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
  for (hipEvent_t e : c->ev_free) (void)hipEventDestroy(e);
  void* bufs[] = {c->x, c->u, c->q, c->attn, c->mlp, c->z, c->keys, c->err,
                  c->part_o, c->part_ml, c->plan_off, c->rope_turns, c->lm_packed, c->splitk, c->group_lens, c->rmap, c->dmap, c->qskip, c->ssq,
                  c->sample_lse, c->sample_keys, c->sample_parts};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
  if (c->fc_packed) (void)hipFree(c->fc_packed);
  void* ar[] = {c->ar_ids, c->ar_pos, c->ar_rows, c->ar_seq, c->ar_rej, c->ar_slots, c->ar_hidden};
  for (void* p : ar)
    if (p) (void)hipFree(p);
  for (void* p : c->layer_packed)
    if (p) (void)hipFree(p);
  if (c->xc) (void)hipFree(c->xc);
  delete c;
}

pe_status check_cfg(const pe_config* c) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->dtype != PE_F32 && c->dtype != PE_BF16) return fail(PE_ERR_INVALID_ARG, "dtype %d", c->dtype);
  if (c->K < 1 || c->K > 32) return fail(PE_ERR_INVALID_ARG, "K=%d outside [1,32]", c->K);
  if (c->max_num_seqs < 1 || c->max_num_seqs > 1024)
    return fail(PE_ERR_INVALID_ARG, "max_num_seqs=%d outside [1,1024]", c->max_num_seqs);
  if (c->max_prefill_slots < 0 || c->max_prefill_slots > (1 << 26))
    return fail(PE_ERR_INVALID_ARG, "max_prefill_slots=%d outside [0,2^26]", c->max_prefill_slots);
  if (c->d < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->mlp < 1 ||
      c->layers < 1 || c->vocab < 1 || c->block_size < 1)
    return fail(PE_ERR_INVALID_ARG, "non-positive dimension");
  if (c->n_q_heads % c->n_kv_heads) return fail(PE_ERR_INVALID_ARG, "n_q_heads %% n_kv_heads != 0");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(PE_ERR_INVALID_ARG, "mask_id outside [0,vocab)");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(PE_ERR_INVALID_ARG, "rms_eps/rope_theta");
  if (c->vocab % 16) return fail(PE_ERR_UNSUPPORTED, "vocab must be a multiple of 16");
  if (c->block_size < 16 || (c->block_size & (c->block_size - 1)))
    return fail(PE_ERR_UNSUPPORTED, "block_size must be a power of two >= 16");
  if (c->head_dim % 32) return fail(PE_ERR_UNSUPPORTED, "head_dim must be a multiple of 32");
  if (c->dtype == PE_BF16) {
    if (c->head_dim != 64) return fail(PE_ERR_UNSUPPORTED, "bf16 kernels need head_dim 64");
    if (c->d % 64) return fail(PE_ERR_UNSUPPORTED, "bf16 kernels need d %% 64 == 0");
    if (c->mlp % 64) return fail(PE_ERR_UNSUPPORTED, "bf16 kernels need mlp %% 64 == 0");
  } else {
    if (c->head_dim > 128) return fail(PE_ERR_UNSUPPORTED, "fp32 kernels need head_dim <= 128");
    if (c->d % 4) return fail(PE_ERR_UNSUPPORTED, "fp32 kernels need d %% 4 == 0");
    if (c->mlp % 16) return fail(PE_ERR_UNSUPPORTED, "fp32 kernels need mlp %% 16 == 0");
  }
  return PE_OK;
}

pe_status check_w(const pe_config* c, const pe_weights* w) {
  if (!w) return fail(PE_ERR_INVALID_ARG, "weights is NULL");
  const void* top[] = {w->embed, w->w_fc, w->final_norm, w->lm_head};
  for (const void* p : top)
    if (!p || !aligned(p, 16)) return fail(PE_ERR_INVALID_ARG, "weight pointer NULL or not 16-byte aligned");
  if (!w->layers) return fail(PE_ERR_INVALID_ARG, "weights.layers is NULL");
  for (int l = 0; l < c->layers; ++l) {
    const pe_layer_weights& L = w->layers[l];
    const void* ps[] = {L.attn_norm, L.wq, L.wk, L.wv, L.wo, L.mlp_norm, L.w_gate, L.w_up, L.w_down};
    for (const void* p : ps)
      if (!p || !aligned(p, 16))
        return fail(PE_ERR_INVALID_ARG, "layer %d weight pointer NULL or not 16-byte aligned", l);
  }
  return PE_OK;
}

template <typename T>
pe_status alloc(T** p, size_t bytes, const char* what) {
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(p), bytes);
  if (e != hipSuccess) return fail(PE_ERR_NOMEM, "hipMalloc %s (%zu bytes): %s", what, bytes, hipGetErrorString(e));
  return PE_OK;
}

pe_status check_B(const pe_ctx* c, int32_t B) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  if (B < 0 || B > c->cfg.max_num_seqs)
    return fail(PE_ERR_INVALID_ARG, "B=%d outside [0, max_num_seqs=%d]", B, c->cfg.max_num_seqs);
  return PE_OK;
}

pe_status check_batch(const pe_batch* b) {
  if (!b) return fail(PE_ERR_INVALID_ARG, "batch is NULL");
  if (!b->input_ids || !b->positions || !b->hidden_src || !b->is_rejected || !b->is_masked ||
      !b->slot_mapping || !b->draft_rows || !b->seq_lens)
    return fail(PE_ERR_INVALID_ARG, "a batch buffer is NULL");
  if (!aligned(b->input_ids, 4) || !aligned(b->positions, 4) || !aligned(b->hidden_src, 4) ||
      !aligned(b->draft_rows, 4) || !aligned(b->seq_lens, 4) || !aligned(b->slot_mapping, 8))
    return fail(PE_ERR_INVALID_ARG, "a batch buffer is misaligned");
  return PE_OK;
}

}  // namespace

extern "C" {

const char* pe_last_error(void) { return g_err.c_str(); }

const char* pe_status_string(pe_status s) {
  switch (s) {
    case PE_OK: return "PE_OK";
    case PE_ERR_INVALID_ARG: return "PE_ERR_INVALID_ARG";
    case PE_ERR_NOMEM: return "PE_ERR_NOMEM";
    case PE_ERR_HIP: return "PE_ERR_HIP";
    case PE_ERR_UNSUPPORTED: return "PE_ERR_UNSUPPORTED";
  }
  return "unknown";
}

pe_status pe_create(const pe_config* cfg, const pe_weights* w, void* stream, pe_ctx** out) {
  g_err.clear();
  if (!out) return fail(PE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  pe_status s = check_cfg(cfg);
  if (s != PE_OK) return s;
  if ((s = check_w(cfg, w)) != PE_OK) return s;

  pe_ctx* c = new pe_ctx();
  c->cfg = *cfg;
  c->w = *w;
  c->layers.assign(w->layers, w->layers + cfg->layers);
  c->w.layers = c->layers.data();
  c->stream = reinterpret_cast<hipStream_t>(stream);
  c->esz = cfg->dtype == PE_BF16 ? 2 : 4;
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e != hipSuccess) {
    free_ctx(c);
    return hipfail(e, "device query");
  }
  c->attn_grid = 2 * c->num_cus;  // attention workgroups: two 512-thread workgroups per CU

  const pe_config& k = c->cfg;
  // rows: a decode round (2K slots per request) or a prefill batch
  const size_t R = std::max(size_t(k.max_num_seqs) * 2 * k.K, size_t(k.max_prefill_slots));
  const size_t D = size_t(k.max_num_seqs) * k.K;
  const size_t qd = size_t(k.n_q_heads) * k.head_dim;
  // bf16 attention: a workgroup holds at most 512 query rows (slots x query
  // heads per KV head); longer requests run as groups of attn_group slots
  const int G = k.n_q_heads / k.n_kv_heads;
  c->attn_group = 1;
  while (c->attn_group * 2 * G <= 512) c->attn_group *= 2;
  const int Sd = 2 * k.K;
  const int dec_groups = Sd * G > 512 ? (Sd + c->attn_group - 1) / c->attn_group : 1;
  c->groups_max = std::max(k.max_num_seqs * dec_groups, k.max_prefill_slots / std::max(c->attn_group, 1));
  c->groups_max = std::min(std::max(c->groups_max, k.max_num_seqs), 1024);
  // query rows of one attention item: S*G when that fits a workgroup, else
  // a group's; a prefill batch may bring any S with S*G <= 512
  size_t QN = Sd * G <= 512 ? size_t(Sd) * G : size_t(c->attn_group) * G;
  if (k.max_prefill_slots > 0) QN = 512;
  c->items_max = pe::attn_max_items(c->groups_max, k.n_kv_heads, c->attn_grid);
  // partial argmax keys: the most any LM-head launch can need (B*K draft rows
  // of a parallel pass, B of a sequential one)
  size_t key_slots = 0;
  for (int m = 1; m <= k.max_num_seqs * k.K; ++m)
    key_slots = std::max(key_slots, size_t(m) * pe::gemm_argmax_parts(k.dtype, m, k.vocab, k.d, c->num_cus));
  const size_t R1 = size_t(k.max_num_seqs) * (k.K + 1);
  struct { void** p; size_t bytes; const char* what; } plan[] = {
      {&c->x, R * k.d * c->esz, "x"},
      {&c->u, R * k.d * c->esz, "u"},
      {&c->q, R * qd * c->esz, "q"},
      {&c->attn, R * qd * c->esz, "attn"},
      {&c->mlp, R * size_t(k.mlp) * c->esz, "mlp"},
      {&c->z, D * k.d * c->esz, "z"},
      {reinterpret_cast<void**>(&c->keys), key_slots * 8, "argmax keys"},
      {reinterpret_cast<void**>(&c->err), 16, "err"},
      {reinterpret_cast<void**>(&c->rope_turns), size_t(k.head_dim / 2) * 8, "rope"},
      {reinterpret_cast<void**>(&c->rmap), (R + 1) * 4, "row map"},
      {reinterpret_cast<void**>(&c->dmap), (2 * D + 1) * 4, "draft row map"},
      {reinterpret_cast<void**>(&c->qskip), R, "last-layer query mask"},
      {reinterpret_cast<void**>(&c->ar_ids), R1 * 4, "ar ids"},
      {reinterpret_cast<void**>(&c->ar_pos), R1 * 4, "ar positions"},
      {reinterpret_cast<void**>(&c->ar_rows), size_t(k.max_num_seqs) * 4, "ar rows"},
      {reinterpret_cast<void**>(&c->ar_seq), size_t(k.max_num_seqs) * 4, "ar seq_lens"},
      {reinterpret_cast<void**>(&c->ar_rej), R1, "ar rejected"},
      {reinterpret_cast<void**>(&c->ar_slots), R1 * 8, "ar slots"},
      {&c->ar_hidden, R1 * k.d * c->esz, "ar hidden"},
      {reinterpret_cast<void**>(&c->sample_lse), size_t(k.max_num_seqs) * (2 * k.K + 1) * 4, "sampling lse"},
      {reinterpret_cast<void**>(&c->sample_keys), D * pe::kSampleParts * 8, "sampling keys"},
      {reinterpret_cast<void**>(&c->sample_parts), size_t(k.max_num_seqs) * (2 * k.K + 1) * pe::kLseParts * 8,
       "sampling row slices"},
  };
  for (auto& p : plan) {
    if ((s = alloc(p.p, p.bytes, p.what)) != PE_OK) { free_ctx(c); return s; }
  }
  if (k.dtype == PE_BF16) {
    if ((s = alloc(&c->part_o, size_t(c->items_max) * QN * k.head_dim * 4, "attn partials")) != PE_OK ||
        (s = alloc(&c->part_ml, size_t(c->items_max) * QN * 2 * 4, "attn stats")) != PE_OK ||
        (s = alloc(&c->plan_off, size_t(pe::kAttnMaxB + 2) * 4, "attn plan")) != PE_OK) {
      free_ctx(c);
      return s;
    }
    if ((s = alloc(&c->group_lens, size_t(c->groups_max) * 4, "attention group lengths")) != PE_OK) {
      free_ctx(c);
      return s;
    }
    // split-K partials: GEMMs whose output tiles are too few to fill the chip
    // sum k-ranges into here first, the k-split tail of a small-batch LM head
    // writes its partial tiles here, and at large batch the QKV product's
    // RoPE + KV-write epilogue runs on its fp32 sums here (64 MB, or those
    // sums over every row when larger)
    c->splitk_cap = std::max<long long>(16LL << 20, (long long)R * (qd + 2 * k.n_kv_heads * k.head_dim));
    if ((s = alloc(&c->splitk, size_t(c->splitk_cap) * 4, "split-K partials")) != PE_OK) {
      free_ctx(c);
      return s;
    }
    if ((s = alloc(&c->ssq, size_t(16) * pe::kSsqMaxParts * 4, "row sums of squares")) != PE_OK) {
      free_ctx(c);
      return s;
    }
  }
  // RoPE frequencies theta^(-2i/hd) in turns per position (divided by 2 pi), in double
  std::vector<double> turns(k.head_dim / 2);
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < k.head_dim / 2; ++i)
    turns[i] = std::pow(double(k.rope_theta), -2.0 * i / double(k.head_dim)) / two_pi;
  const uint32_t err0[4] = {0u, 0xFFFFFFFFu, 0u, 0u};
  e = hipMemcpy(c->rope_turns, turns.data(), turns.size() * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->err, err0, 16, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    free_ctx(c);
    return hipfail(e, "workspace init");
  }
  if (k.dtype == PE_BF16) {
    // The LM head streams V*d*2 bytes per step; a copy in MFMA-fragment order lets
    // every wave load one contiguous 1 KB per k-step (full lines, non-temporal).
    pe::GemmArgs pg;
    std::memset(&pg, 0, sizeof pg);
    pg.hd = k.head_dim;
    auto pack = [&](int bmap, const void* w0, const void* w1, const void* w2, int N, int K, int nq,
                    int nk, void** dst, const char* what) -> pe_status {
      pe_status st2 = alloc(dst, size_t(N) * K * 2, what);
      if (st2 != PE_OK) return st2;
      pg.W0 = w0; pg.W1 = w1; pg.W2 = w2; pg.N = N; pg.K = K; pg.nq = nq; pg.nk = nk;
      hipError_t e2 = pe::launch_pack_frag16(bmap, pg, *dst, c->stream);
      return e2 == hipSuccess ? PE_OK : hipfail(e2, what);
    };
    const int qd = k.n_q_heads * k.head_dim, kvd = k.n_kv_heads * k.head_dim;
    s = pack(pe::B_PLAIN, w->lm_head, nullptr, nullptr, k.vocab, k.d, 0, 0, &c->lm_packed, "pack LM head");
    if (s == PE_OK) s = pack(pe::B_PLAIN, w->w_fc, nullptr, nullptr, k.d, 2 * k.d, 0, 0, &c->fc_packed, "pack fc");
    c->layer_packed.assign(size_t(4) * k.layers, nullptr);
    for (int l = 0; l < k.layers && s == PE_OK; ++l) {
      const pe_layer_weights& L = c->layers[l];
      void** lp = &c->layer_packed[4 * l];
      s = pack(pe::B_QKV, L.wq, L.wk, L.wv, qd + 2 * kvd, k.d, qd, kvd, &lp[0], "pack qkv");
      if (s == PE_OK) s = pack(pe::B_PLAIN, L.wo, nullptr, nullptr, k.d, qd, 0, 0, &lp[1], "pack o");
      if (s == PE_OK) s = pack(pe::B_GATEUP, L.w_gate, L.w_up, nullptr, 2 * k.mlp, k.d, 0, 0, &lp[2], "pack gate/up");
      if (s == PE_OK) s = pack(pe::B_PLAIN, L.w_down, nullptr, nullptr, k.d, k.mlp, 0, 0, &lp[3], "pack down");
    }
    if (s == PE_OK && (e = hipStreamSynchronize(c->stream)) != hipSuccess) s = hipfail(e, "pack sync");
    if (s != PE_OK) {
      free_ctx(c);
      return s;
    }
    // the MASK-deduplicated first-layer fc rows of a parallel step (large batches)
    if (size_t(k.max_num_seqs) * (k.K + 2) > size_t(pe::kRowMapMinRows) && k.K >= 3) {
      if ((s = alloc(&c->xc, size_t(k.max_num_seqs) * (k.K + 2) * k.d * 2, "deduplicated fc rows")) != PE_OK) {
        free_ctx(c);
        return s;
      }
    }
  }
  *out = c;
  return PE_OK;
}

pe_status pe_destroy(pe_ctx* ctx) {
  if (!ctx) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  (void)hipStreamSynchronize(ctx->stream);
  free_ctx(ctx);
  return PE_OK;
}

pe_status pe_set_stream(pe_ctx* ctx, void* stream) {
  if (!ctx) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  ctx->stream = reinterpret_cast<hipStream_t>(stream);
  return PE_OK;
}

}  // extern "C"

// Checks the arguments of a preparation and fills its kernel arguments.
static pe_status prepare_args(pe_ctx* ctx, int32_t B, const int32_t* verify_tokens,
                              const int32_t* verify_positions, const int32_t* num_accepted,
                              const int32_t* bonus_tokens, const int32_t* block_table,
                              int32_t max_blocks, int32_t num_kv_blocks, const pe_batch* out,
                              pe::PrepareArgs& a) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if ((s = check_batch(out)) != PE_OK) return s;
  if (B == 0) return PE_OK;
  if (!verify_tokens || !verify_positions || !num_accepted || !bonus_tokens || !block_table)
    return fail(PE_ERR_INVALID_ARG, "a prepare input is NULL");
  if (max_blocks < 1 || num_kv_blocks < 1) return fail(PE_ERR_INVALID_ARG, "max_blocks/num_kv_blocks < 1");
  a.B = B;
  a.K = ctx->cfg.K;
  a.vocab = ctx->cfg.vocab;
  a.mask_id = ctx->cfg.mask_id;
  a.block_size = ctx->cfg.block_size;
  a.max_blocks = max_blocks;
  a.num_kv_blocks = num_kv_blocks;
  a.vt = verify_tokens;
  a.vp = verify_positions;
  a.acc = num_accepted;
  a.bonus = bonus_tokens;
  a.bt = block_table;
  a.ids = out->input_ids;
  a.pos = out->positions;
  a.hsrc = out->hidden_src;
  a.draft_rows = out->draft_rows;
  a.seq_lens = out->seq_lens;
  a.rej = out->is_rejected;
  a.msk = out->is_masked;
  a.slots = out->slot_mapping;
  a.err = ctx->err;
  a.nact = ctx->nact;
  return PE_OK;
}

static pe_status check_gather(pe_ctx* ctx, int32_t B, const pe_batch* batch, const void* target_hidden,
                              const void* h_shared, void* draft_hidden) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if (!batch || !batch->hidden_src) return fail(PE_ERR_INVALID_ARG, "batch.hidden_src is NULL");
  if (B == 0) return PE_OK;
  if (!target_hidden || !h_shared || !draft_hidden || !aligned(target_hidden, 16) ||
      !aligned(h_shared, 16) || !aligned(draft_hidden, 16))
    return fail(PE_ERR_INVALID_ARG, "hidden buffers NULL or not 16-byte aligned");
  return PE_OK;
}

extern "C" {

pe_status pe_prepare(pe_ctx* ctx, int32_t B, const int32_t* verify_tokens,
                     const int32_t* verify_positions, const int32_t* num_accepted,
                     const int32_t* bonus_tokens, const int32_t* block_table, int32_t max_blocks,
                     int32_t num_kv_blocks, const pe_batch* out) {
  pe::PrepareArgs a;
  pe_status s = prepare_args(ctx, B, verify_tokens, verify_positions, num_accepted, bonus_tokens,
                             block_table, max_blocks, num_kv_blocks, out, a);
  if (s != PE_OK || B == 0) return s;
  Timed tm(ctx, PE_PH_PREPARE);
  PE_HIP(pe::launch_prepare(a, ctx->stream), "prepare launch");
  return PE_OK;
}

pe_status pe_gather_hidden(pe_ctx* ctx, int32_t B, const pe_batch* batch, const void* target_hidden,
                           const void* h_shared, void* draft_hidden) {
  pe_status s = check_gather(ctx, B, batch, target_hidden, h_shared, draft_hidden);
  if (s != PE_OK || B == 0) return s;
  const int K = ctx->cfg.K;
  Timed tm(ctx, PE_PH_GATHER);
  PE_HIP(pe::launch_gather(B * 2 * K, B * (K + 1), int(ctx->cfg.d * ctx->esz), batch->hidden_src,
                           target_hidden, h_shared, draft_hidden, ctx->stream),
         "gather launch");
  return PE_OK;
}

static const void* packed(const pe_ctx* c, int layer, int which) {
  return c->layer_packed.empty() ? nullptr : c->layer_packed[4 * layer + which];
}

// One drafter pass over B requests of S slots each: fc -> decoder layers ->
// final norm on the Kd draft rows per request -> LM head + argmax.
struct Pass {
  int B, S, Kd;
  const int32_t *ids, *pos, *draft_rows, *seq_lens;
  const uint8_t* rej;
  const int64_t* slots;
  const void* hidden;  // [B*S, d]
  int32_t* tokens;     // draft row i -> tokens[i * tstride]
  int tstride;
  float* logits;       // draft row i -> logits[i * ldl ...], or NULL
  int ldl;
  // when set (tstride 1, Kd = K): greedy verification fused into the argmax
  const int32_t* vtarget = nullptr;
  int32_t *vacc = nullptr, *vbonus = nullptr;
  // when set: draft tokens drawn from softmax(logits / T) instead of argmax
  const uint64_t* seed = nullptr;
  float inv_temp = 1.f;
  // the parallel-step layout (S = 2K: copied slots 0..K, MASK slots K+1..2K-1)
  bool parallel_layout = false;
  // input x = emb(token) alone (no hidden state, no fc)
  bool embed_input = false;
  // when set: the position up to which each slot attends (else its own)
  const int32_t* attn_pos = nullptr;
};

static pe_status forward_pass(pe_ctx* ctx, const Pass& P, const int32_t* block_table,
                              int32_t max_blocks, int32_t num_kv_blocks, void* const* k_cache,
                              void* const* v_cache) {
  const pe_config& k = ctx->cfg;
  const int B = P.B, S = P.S, R = B * S, D = B * P.Kd, d = k.d;
  const int qd = k.n_q_heads * k.head_dim, kvd = k.n_kv_heads * k.head_dim;
  const long long num_slots = (long long)num_kv_blocks * k.block_size;
  hipStream_t st = ctx->stream;
  const int dt = k.dtype;

  pe::GemmArgs g0;
  std::memset(&g0, 0, sizeof g0);
  g0.d = d;
  g0.vocab = k.vocab;
  g0.hd = k.head_dim;
  g0.Hkv = k.n_kv_heads;
  g0.block_size = k.block_size;
  g0.num_slots = num_slots;
  g0.part = ctx->splitk;
  g0.part_cap = ctx->splitk_cap;
  g0.nact = ctx->nact;
  g0.rpr = S;

  // The last layer after its QKV product (which writes every valid slot's
  // KV): only the draft rows feed the LM head, so attention keeps only their
  // queries and the O product, MLP norm and MLP run on their rows alone
  // (through a row map of the non-rejected draft rows).
  const bool draft_only = dt == PE_BF16 && R > pe::kRowMapMinRows && P.draft_rows;
  // Above 16 rows the fc, O and down products run on the large-batch kernels,
  // whose split-K sum writes each output row whole: it also writes the
  // following RMSNorm (the MLP norm after O, the next layer's attention norm
  // after down, and after the last layer's down on the draft rows the final
  // norm, into z at each row's draft index), so those norms need no launch of
  // their own.  The draft rows it does not compute (rejected: padded
  // requests) get zero rows in z.  (Above 16 rows no norm is folded into the
  // small-batch products.)
  const bool post_norm = dt == PE_BF16 && R > PE_POSTNORM_MIN_ROWS && d <= 4096;
  const bool final_fused = post_norm && draft_only;
  int32_t* const dpos = ctx->dmap + D + 1;
  // the dense products above 64 rows compute only the non-rejected slots: a
  // rejected slot's outputs are never read (no KV write, no attention, not a
  // draft row); the map comes from the batch's rejected mask
  if (dt == PE_BF16 && R > pe::kRowMapMinRows) {
    Timed tm(ctx, PE_PH_FC);
    PE_HIP(pe::launch_row_maps(R, P.rej, ctx->rmap, ctx->rmap + R, D, draft_only ? P.draft_rows : nullptr, ctx->dmap,
                               ctx->dmap + D, dpos, ctx->qskip, final_fused ? ctx->z : nullptr, d, st),
           "row maps");
    g0.rmap = ctx->rmap;
    g0.rcount = ctx->rmap + R;
  }

  // RMSNorm folded into the small-batch products (at most 16 rows: every dense
  // product runs on gemm_skinny): fc, O and down also write per-tile sums of
  // squares of the x rows they store, and QKV and gate/up read x through the
  // norm, so the attention and MLP norms need no launch of their own
  const bool fold = pe::gemm_folds_norm(dt, R, d) && ctx->ssq && d % 16 == 0;
  auto ssq_out = [&](pe::GemmArgs& g) {
    if (fold) { g.ssq_out = ctx->ssq; g.ssq_n = d / 16; }
  };
  auto norm_after = [&](pe::GemmArgs& g, const void* gain) {
    g.nrm_out = ctx->u; g.nrm_gain = gain; g.norm_eps = k.rms_eps;
  };
  auto norm_in = [&](pe::GemmArgs& g, const void* gain) {
    g.A = ctx->x;
    g.ssq_in = ctx->ssq; g.ssq_n = d / 16;
    g.norm_gain = gain; g.norm_eps = k.rms_eps;
  };

  // a dense GEMM with its fused epilogue
  auto dense = [&](int aload, int bmap, int epi, const pe::GemmArgs& g, const char* what) -> pe_status {
    if (g.nrm_out)  // the following norm in the split-K sum: the large-batch kernels at any row count
      PE_HIP(pe::launch_mm(aload, bmap, epi, g, ctx->num_cus, st), what);
    else
      PE_HIP(pe::launch_gemm(dt, aload, bmap, epi, g, ctx->num_cus, st), what);
    return PE_OK;
  };
  pe_status ds = PE_OK;

  // MASK-slot deduplication of the first layer.  In the parallel-step layout
  // the K-1 MASK slots of a request all carry emb(MASK) and h_shared, so the
  // first layer's fc, norm and (pre-RoPE) QKV rows of those slots are equal:
  // at large batch fc and QKV run on K+2 rows per request (copied slots and
  // one MASK slot), the norm writes the fc rows out to every slot, and the QKV
  // epilogue (RoPE at each slot's own position, KV write) runs for every slot.
  const int Kc = k.K, Rc = B * (Kc + 2);
  const bool dd = P.parallel_layout && dt == PE_BF16 && ctx->xc && Kc >= 3 && Rc > pe::kRowMapMinRows;

  if (P.embed_input) {
    Timed tm(ctx, PE_PH_GATHER);
    PE_HIP(pe::launch_gather(R, k.vocab, int(d * ctx->esz), P.ids, ctx->w.embed, ctx->w.embed, ctx->x, st),
           "embedding rows");
  } else {
    // fc over concat(emb(token), hidden)
    pe::GemmArgs g = g0;
    g.M = R; g.N = d; g.K = 2 * d;
    g.embed = ctx->w.embed; g.ids = P.ids; g.hid = P.hidden;
    g.W0 = ctx->w.w_fc; g.Wp = ctx->fc_packed;
    g.out = ctx->x; g.ldo = d;
    Timed tm(ctx, PE_PH_FC);
    if (dd) {
      g.M = Rc;
      g.rpr = Kc + 2;
      g.dedup_k = Kc;
      g.out = ctx->xc;
      g.rmap = nullptr;
      g.rcount = nullptr;
    }
    ssq_out(g);
    if (post_norm) {  // the first layer's attention norm (and the MASK rows' expansion) in its sum
      norm_after(g, ctx->layers[0].attn_norm);
      if (dd) g.nrm_xfull = ctx->x;
    }
    if ((ds = dense(pe::A_FC, pe::B_PLAIN, pe::E_STORE, g, "fc")) != PE_OK) return ds;
  }
  for (int l = 0; l < k.layers; ++l) {
    const pe_layer_weights& L = ctx->layers[l];
    const bool first_dd = l == 0 && dd;
    const bool last_draft = draft_only && l == k.layers - 1;
    const bool fold_attn = fold && (l > 0 || !P.embed_input);  // the embedding gather writes no sums
    // (with post_norm the fc product, or after layer 0 the down product, wrote it)
    if (!fold_attn && !(post_norm && (l > 0 || !P.embed_input))) {
      Timed tm(ctx, PE_PH_NORM);
      if (first_dd)
        PE_HIP(pe::launch_rmsnorm_expand(Rc, d, ctx->xc, L.attn_norm, ctx->u, ctx->x, Kc, k.rms_eps, st),
               "attn norm");
      else
        PE_HIP(pe::launch_rmsnorm(dt, R, d, ctx->x, L.attn_norm, ctx->u, nullptr, R, k.rms_eps, st), "attn norm");
    }
    {
      pe::GemmArgs g = g0;
      g.M = R; g.N = qd + 2 * kvd; g.K = d;
      g.A = ctx->u; g.lda = d;
      g.W0 = L.wq; g.W1 = L.wk; g.W2 = L.wv; g.nq = qd; g.nk = kvd;
      g.Wp = packed(ctx, l, 0);
      g.positions = P.pos; g.slots = P.slots;
      g.qout = ctx->q; g.kcache = k_cache[l]; g.vcache = v_cache[l];
      g.rope_turns = ctx->rope_turns;
      if (fold_attn) norm_in(g, L.attn_norm);
      Timed tm(ctx, PE_PH_QKV);
      if (first_dd) {
        // compact rows; the epilogue covers every slot
        g.M = Rc;
        g.rpr = Kc + 2;
        g.dedup_k = Kc;
        g.rmap = nullptr;
        g.rcount = nullptr;
      }
      if ((ds = dense(pe::A_PLAIN, pe::B_QKV, pe::E_QKV, g, "qkv")) != PE_OK) return ds;
    }
    {
      pe::AttnArgs a;
      std::memset(&a, 0, sizeof a);
      a.B = B; a.S = S; a.Hq = k.n_q_heads; a.Hkv = k.n_kv_heads; a.hd = k.head_dim;
      a.block_size = k.block_size; a.max_blocks = max_blocks; a.num_slots = num_slots;
      a.scale = 1.0f / std::sqrt(float(k.head_dim));
      a.q = ctx->q; a.kcache = k_cache[l]; a.vcache = v_cache[l];
      a.positions = P.attn_pos ? P.attn_pos : P.pos; a.seq_lens = P.seq_lens;
      a.rej = last_draft ? ctx->qskip : P.rej;  // queries computed: valid slots (last layer: draft rows)
      a.bt = block_table; a.out = ctx->attn;
      a.part_o = ctx->part_o; a.part_ml = ctx->part_ml; a.plan_off = ctx->plan_off;
      a.vpr = 1;
      const int G = k.n_q_heads / k.n_kv_heads;
      // the steps of all (request, KV head) streams are cut into equal ranges,
      // one per workgroup
      a.grid = ctx->attn_grid;
      if (dt == PE_BF16 && S * G > 512) {
        // groups of attn_group consecutive slots attend as requests of their
        // own (same block table row, context up to the group's last position)
        const int Sv = ctx->attn_group;
        if (S % Sv || (long long)B * (S / Sv) > ctx->groups_max)
          return fail(PE_ERR_UNSUPPORTED, "attention: %d slots per request in groups of %d (at most %d groups)",
                      S, Sv, ctx->groups_max);
        a.vpr = S / Sv;
        a.B = B * a.vpr;
        a.S = Sv;
        Timed tg(ctx, PE_PH_ATTN);
        PE_HIP(pe::launch_attn_group_lens(a.B, Sv, a.vpr, a.positions, P.rej, P.seq_lens, ctx->group_lens, st),
               "attention group lengths");
        a.seq_lens = ctx->group_lens;
      }
      if (pe::attn_max_items(a.B, k.n_kv_heads, a.grid) > ctx->items_max)
        return fail(PE_ERR_UNSUPPORTED, "attention: %d requests exceed the partial buffers", a.B);
      Timed tm(ctx, PE_PH_ATTN);
      PE_HIP(pe::launch_attention(dt, a, st), "attention");
    }
    {
      pe::GemmArgs g = g0;
      g.M = R; g.N = d; g.K = qd;
      g.A = ctx->attn; g.lda = qd;
      g.W0 = L.wo; g.Wp = packed(ctx, l, 1);
      g.out = ctx->x; g.resid = ctx->x; g.ldo = d;
      if (last_draft) { g.M = R; g.rmap = ctx->dmap; g.rcount = ctx->dmap + D; g.plan_rows = D; }
      ssq_out(g);
      if (post_norm) norm_after(g, L.mlp_norm);
      Timed tm(ctx, PE_PH_O);
      if ((ds = dense(pe::A_PLAIN, pe::B_PLAIN, pe::E_RESID, g, "o proj")) != PE_OK) return ds;
    }
    if (!fold && !post_norm) {
      Timed tm(ctx, PE_PH_NORM);
      if (last_draft)  // the draft rows, in place
        PE_HIP(pe::launch_rmsnorm(dt, D, d, ctx->x, L.mlp_norm, ctx->u, P.draft_rows, R, k.rms_eps, st, true),
               "mlp norm");
      else
        PE_HIP(pe::launch_rmsnorm(dt, R, d, ctx->x, L.mlp_norm, ctx->u, nullptr, R, k.rms_eps, st), "mlp norm");
    }
    {
      pe::GemmArgs g = g0;
      g.M = R; g.N = 2 * k.mlp; g.K = d;
      g.A = ctx->u; g.lda = d;
      g.W0 = L.w_gate; g.W1 = L.w_up; g.Wp = packed(ctx, l, 2);
      g.out = ctx->mlp; g.ldo = k.mlp;
      if (last_draft) { g.rmap = ctx->dmap; g.rcount = ctx->dmap + D; g.plan_rows = D; }
      if (fold) norm_in(g, L.mlp_norm);
      Timed tm(ctx, PE_PH_GATEUP);
      if ((ds = dense(pe::A_PLAIN, pe::B_GATEUP, pe::E_SILU, g, "gate/up")) != PE_OK) return ds;
    }
    {
      pe::GemmArgs g = g0;
      g.M = R; g.N = d; g.K = k.mlp;
      g.A = ctx->mlp; g.lda = k.mlp;
      g.W0 = L.w_down; g.Wp = packed(ctx, l, 3);
      g.out = ctx->x; g.resid = ctx->x; g.ldo = d;
      if (last_draft) { g.rmap = ctx->dmap; g.rcount = ctx->dmap + D; g.plan_rows = D; }
      ssq_out(g);  // the next layer's attention norm
      if (post_norm && l + 1 < k.layers) norm_after(g, ctx->layers[l + 1].attn_norm);
      if (final_fused && last_draft) {  // the final norm, at the draft indices
        norm_after(g, ctx->w.final_norm);
        g.nrm_out = ctx->z;
        g.nrm_rows = dpos;
      }
      Timed tm(ctx, PE_PH_DOWN);
      if ((ds = dense(pe::A_PLAIN, pe::B_PLAIN, pe::E_RESID, g, "down")) != PE_OK) return ds;
    }
  }
  if (!final_fused) {
    Timed tm(ctx, PE_PH_NORM);
    PE_HIP(pe::launch_rmsnorm(dt, D, d, ctx->x, ctx->w.final_norm, ctx->z, P.draft_rows, R,
                              k.rms_eps, st),
           "final norm");
  }
  {
    pe::GemmArgs g = g0;
    g.M = D; g.N = k.vocab; g.K = d;
    g.A = ctx->z; g.lda = d;
    g.W0 = ctx->w.lm_head;
    g.Wp = ctx->lm_packed;
    g.keys = ctx->keys; g.logits = P.logits; g.ldl = P.ldl;
    g.rpr = P.Kd;
    g.rmap = nullptr;  // draft rows are never rejected
    g.rcount = nullptr;
    g.parts = pe::gemm_argmax_parts(dt, D, k.vocab, d, ctx->num_cus);
    g.seq_lens = P.seq_lens; g.Kd = P.Kd;
    {
      Timed tm(ctx, PE_PH_LMHEAD);
      PE_HIP(pe::launch_gemm(dt, pe::A_PLAIN, pe::B_PLAIN, pe::E_ARGMAX, g, ctx->num_cus, st), "lm head");
    }
    Timed tm(ctx, PE_PH_ARGMAX);
    if (P.seed)
      PE_HIP(pe::launch_sample_drafts(D, P.Kd, k.vocab, P.ldl, P.inv_temp, P.logits, P.seed, ctx->sample_keys,
                                      P.tokens, P.tstride, P.seq_lens, st),
             "draft sampling");
    else if (P.vtarget)
      PE_HIP(pe::launch_argmax_verify(B, P.Kd, g.parts, ctx->keys, P.tokens, P.seq_lens, P.vtarget,
                                      P.vacc, P.vbonus, ctx->nact, st),
             "argmax + verify");
    else
      PE_HIP(pe::launch_argmax_tokens(D, P.Kd, g.parts, ctx->keys, P.tokens, P.tstride, P.seq_lens, st),
             "argmax");
  }
  return PE_OK;
}


static pe_status check_forward(pe_ctx* ctx, int32_t B, const pe_batch* batch, const void* draft_hidden,
                               const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                               void* const* k_cache, void* const* v_cache, int32_t* draft_tokens,
                               float* logits, bool need_hidden = true) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if ((s = check_batch(batch)) != PE_OK) return s;
  if (B == 0) return PE_OK;
  const pe_config& k = ctx->cfg;
  if (need_hidden && (!draft_hidden || !aligned(draft_hidden, 16))) return fail(PE_ERR_INVALID_ARG, "draft_hidden");
  if (!block_table || max_blocks < 1 || num_kv_blocks < 1) return fail(PE_ERR_INVALID_ARG, "block table");
  if (!k_cache || !v_cache) return fail(PE_ERR_INVALID_ARG, "k_cache/v_cache arrays are NULL");
  for (int l = 0; l < k.layers; ++l)
    if (!k_cache[l] || !v_cache[l] || !aligned(k_cache[l], 16) || !aligned(v_cache[l], 16))
      return fail(PE_ERR_INVALID_ARG, "KV cache of layer %d NULL or misaligned", l);
  if (!draft_tokens) return fail(PE_ERR_INVALID_ARG, "draft_tokens is NULL");
  if (logits && !aligned(logits, 4)) return fail(PE_ERR_INVALID_ARG, "logits misaligned");
  return PE_OK;
}

pe_status pe_draft_forward(pe_ctx* ctx, int32_t B, const pe_batch* batch, const void* draft_hidden,
                           const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                           void* const* k_cache, void* const* v_cache, int32_t* draft_tokens,
                           float* logits) {
  pe_status s = check_forward(ctx, B, batch, draft_hidden, block_table, max_blocks, num_kv_blocks,
                              k_cache, v_cache, draft_tokens, logits);
  if (s != PE_OK || B == 0) return s;
  const int K = ctx->cfg.K;
  Pass P;
  P.B = B; P.S = 2 * K; P.Kd = K; P.parallel_layout = true;
  P.ids = batch->input_ids; P.pos = batch->positions; P.draft_rows = batch->draft_rows;
  P.seq_lens = batch->seq_lens; P.rej = batch->is_rejected; P.slots = batch->slot_mapping;
  P.hidden = draft_hidden;
  P.tokens = draft_tokens; P.tstride = 1;
  P.logits = logits; P.ldl = ctx->cfg.vocab;
  return forward_pass(ctx, P, block_table, max_blocks, num_kv_blocks, k_cache, v_cache);
}

pe_status pe_ar_draft(pe_ctx* ctx, int32_t B, const pe_batch* batch, const void* draft_hidden,
                      const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                      void* const* k_cache, void* const* v_cache, int32_t* draft_tokens,
                      float* logits) {
  pe_status s = check_forward(ctx, B, batch, draft_hidden, block_table, max_blocks, num_kv_blocks,
                              k_cache, v_cache, draft_tokens, logits);
  if (s != PE_OK || B == 0) return s;
  const pe_config& k = ctx->cfg;
  const int K = k.K;
  pe::ArArgs a;
  std::memset(&a, 0, sizeof a);
  a.B = B; a.K = K; a.row_bytes = int(k.d * ctx->esz); a.block_size = k.block_size;
  a.max_blocks = max_blocks; a.num_kv_blocks = num_kv_blocks;
  a.ids = batch->input_ids; a.pos = batch->positions; a.draft_rows = batch->draft_rows;
  a.seq_lens = batch->seq_lens; a.rej = batch->is_rejected; a.slots = batch->slot_mapping;
  a.bt = block_table; a.tokens = draft_tokens;
  a.p_ids = ctx->ar_ids; a.p_pos = ctx->ar_pos; a.p_rows = ctx->ar_rows; a.p_seq = ctx->ar_seq;
  a.p_rej = ctx->ar_rej; a.p_slots = ctx->ar_slots; a.p_hidden = ctx->ar_hidden;
  Pass P;
  P.B = B; P.Kd = 1;
  P.ids = ctx->ar_ids; P.pos = ctx->ar_pos; P.draft_rows = ctx->ar_rows; P.seq_lens = ctx->ar_seq;
  P.rej = ctx->ar_rej; P.slots = ctx->ar_slots; P.hidden = ctx->ar_hidden;
  P.tstride = K; P.ldl = K * k.vocab;
  for (int step = 0; step < K; ++step) {
    {
      Timed tm(ctx, PE_PH_AR);
      if (step == 0) {
        a.hidden = draft_hidden;
        PE_HIP(pe::launch_ar_first(a, ctx->stream), "ar first pass batch");
      } else {
        a.hidden = ctx->x;  // residual stream after the last layer of the previous pass
        a.k = step;
        PE_HIP(pe::launch_ar_next(a, ctx->stream), "ar pass batch");
      }
    }
    P.S = step == 0 ? K + 1 : 1;
    P.tokens = draft_tokens + step;
    P.logits = logits ? logits + (size_t)step * k.vocab : nullptr;
    s = forward_pass(ctx, P, block_table, max_blocks, num_kv_blocks, k_cache, v_cache);
    if (s != PE_OK) return s;
  }
  return PE_OK;
}

// ---- drafting round after a prompt ----------------------------------------
static pe_status check_prefill_shape(pe_ctx* ctx, int32_t B, int32_t S) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if (S < ctx->cfg.K) return fail(PE_ERR_INVALID_ARG, "S=%d below K=%d", S, ctx->cfg.K);
  if ((long long)B * S > ctx->cfg.max_prefill_slots)
    return fail(PE_ERR_INVALID_ARG, "B*S=%lld above max_prefill_slots=%d", (long long)B * S,
                ctx->cfg.max_prefill_slots);
  return PE_OK;
}

pe_status pe_prefill_prepare(pe_ctx* ctx, int32_t B, int32_t S, const int32_t* chunk_tokens,
                             const int32_t* chunk_lens, const int32_t* start_pos,
                             const int32_t* new_tokens, const int32_t* block_table,
                             int32_t max_blocks, int32_t num_kv_blocks, const pe_batch* out) {
  pe_status s = check_prefill_shape(ctx, B, S);
  if (s != PE_OK) return s;
  if ((s = check_batch(out)) != PE_OK) return s;
  if (B == 0) return PE_OK;
  if (!chunk_tokens || !chunk_lens || !start_pos || !new_tokens || !block_table)
    return fail(PE_ERR_INVALID_ARG, "a prefill input is NULL");
  if (max_blocks < 1 || num_kv_blocks < 1) return fail(PE_ERR_INVALID_ARG, "max_blocks/num_kv_blocks < 1");
  pe::PrefillArgs a;
  a.B = B; a.K = ctx->cfg.K; a.S = S;
  a.vocab = ctx->cfg.vocab; a.mask_id = ctx->cfg.mask_id; a.block_size = ctx->cfg.block_size;
  a.max_blocks = max_blocks; a.num_kv_blocks = num_kv_blocks;
  a.ct = chunk_tokens; a.lens = chunk_lens; a.start = start_pos; a.newt = new_tokens; a.bt = block_table;
  a.ids = out->input_ids; a.pos = out->positions; a.hsrc = out->hidden_src;
  a.draft_rows = out->draft_rows; a.seq_lens = out->seq_lens;
  a.rej = out->is_rejected; a.msk = out->is_masked; a.slots = out->slot_mapping;
  a.err = ctx->err;
  Timed tm(ctx, PE_PH_PREPARE);
  PE_HIP(pe::launch_prefill_prepare(a, ctx->stream), "prefill prepare launch");
  return PE_OK;
}

pe_status pe_prefill_gather(pe_ctx* ctx, int32_t B, int32_t S, const pe_batch* batch,
                            const void* target_hidden, const void* h_shared, void* draft_hidden) {
  pe_status s = check_prefill_shape(ctx, B, S);
  if (s != PE_OK) return s;
  if ((s = check_gather(ctx, B, batch, target_hidden, h_shared, draft_hidden)) != PE_OK || B == 0) return s;
  const int L = S - ctx->cfg.K + 1;
  Timed tm(ctx, PE_PH_GATHER);
  PE_HIP(pe::launch_gather(B * S, B * L, int(ctx->cfg.d * ctx->esz), batch->hidden_src, target_hidden,
                           h_shared, draft_hidden, ctx->stream),
         "prefill gather launch");
  return PE_OK;
}

pe_status pe_prefill_forward(pe_ctx* ctx, int32_t B, int32_t S, const pe_batch* batch,
                             const void* draft_hidden, const int32_t* block_table, int32_t max_blocks,
                             int32_t num_kv_blocks, void* const* k_cache, void* const* v_cache,
                             int32_t* draft_tokens, float* logits) {
  pe_status s = check_prefill_shape(ctx, B, S);
  if (s != PE_OK) return s;
  s = check_forward(ctx, B, batch, draft_hidden, block_table, max_blocks, num_kv_blocks, k_cache, v_cache,
                    draft_tokens, logits);
  if (s != PE_OK || B == 0) return s;
  const int G = ctx->cfg.n_q_heads / ctx->cfg.n_kv_heads, Sv = ctx->attn_group;
  if (ctx->cfg.dtype == PE_BF16 && S * G > 512 && (S % Sv || (long long)B * (S / Sv) > ctx->groups_max))
    return fail(PE_ERR_UNSUPPORTED, "attention: %d slots per request in groups of %d (at most %d groups)", S,
                Sv, ctx->groups_max);
  Pass P;
  P.B = B; P.S = S; P.Kd = ctx->cfg.K;
  P.ids = batch->input_ids; P.pos = batch->positions; P.draft_rows = batch->draft_rows;
  P.seq_lens = batch->seq_lens; P.rej = batch->is_rejected; P.slots = batch->slot_mapping;
  P.hidden = draft_hidden;
  P.tokens = draft_tokens; P.tstride = 1;
  P.logits = logits; P.ldl = ctx->cfg.vocab;
  return forward_pass(ctx, P, block_table, max_blocks, num_kv_blocks, k_cache, v_cache);
}

// ---- DFlash-style round: KV injection + one bidirectional block --------------
pe_status pe_dflash_prepare(pe_ctx* ctx, int32_t B, const int32_t* verify_positions, const int32_t* num_accepted,
                            const int32_t* bonus_tokens, const int32_t* block_table, int32_t max_blocks,
                            int32_t num_kv_blocks, const pe_batch* out, int32_t* attn_positions,
                            int64_t* inject_slots) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if ((s = check_batch(out)) != PE_OK) return s;
  if (B == 0) return PE_OK;
  if (!verify_positions || !num_accepted || !bonus_tokens || !block_table)
    return fail(PE_ERR_INVALID_ARG, "a prepare input is NULL");
  if (!attn_positions || !inject_slots || !aligned(attn_positions, 4) || !aligned(inject_slots, 8))
    return fail(PE_ERR_INVALID_ARG, "attn_positions/inject_slots NULL or misaligned");
  if (max_blocks < 1 || num_kv_blocks < 1) return fail(PE_ERR_INVALID_ARG, "max_blocks/num_kv_blocks < 1");
  if (ctx->cfg.K > 63) return fail(PE_ERR_UNSUPPORTED, "K=%d: the block needs K+1 <= 64 slots", ctx->cfg.K);
  pe::DflashArgs a;
  a.B = B; a.K = ctx->cfg.K;
  a.vocab = ctx->cfg.vocab; a.mask_id = ctx->cfg.mask_id; a.block_size = ctx->cfg.block_size;
  a.max_blocks = max_blocks; a.num_kv_blocks = num_kv_blocks;
  a.vp = verify_positions; a.acc = num_accepted; a.bonus = bonus_tokens; a.bt = block_table;
  a.ids = out->input_ids; a.pos = out->positions; a.apos = attn_positions; a.hsrc = out->hidden_src;
  a.draft_rows = out->draft_rows; a.seq_lens = out->seq_lens;
  a.rej = out->is_rejected; a.msk = out->is_masked; a.slots = out->slot_mapping; a.inj = inject_slots;
  a.err = ctx->err;
  a.nact = ctx->nact;
  Timed tm(ctx, PE_PH_PREPARE);
  PE_HIP(pe::launch_dflash_prepare(a, ctx->stream), "dflash prepare launch");
  return PE_OK;
}

pe_status pe_dflash_inject(pe_ctx* ctx, int32_t B, const int32_t* verify_positions, const int64_t* inject_slots,
                           const void* target_hidden, const void* const* wk_inject, const void* const* wv_inject,
                           int32_t num_kv_blocks, void* const* k_cache, void* const* v_cache) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if (B == 0) return PE_OK;
  const pe_config& k = ctx->cfg;
  if (!verify_positions || !inject_slots || !aligned(inject_slots, 8))
    return fail(PE_ERR_INVALID_ARG, "verify_positions/inject_slots NULL or misaligned");
  if (!target_hidden || !aligned(target_hidden, 16)) return fail(PE_ERR_INVALID_ARG, "target_hidden");
  if (num_kv_blocks < 1) return fail(PE_ERR_INVALID_ARG, "num_kv_blocks < 1");
  if (!wk_inject || !wv_inject || !k_cache || !v_cache) return fail(PE_ERR_INVALID_ARG, "a per-layer array is NULL");
  for (int l = 0; l < k.layers; ++l)
    if (!wk_inject[l] || !wv_inject[l] || !k_cache[l] || !v_cache[l] || !aligned(wk_inject[l], 16) ||
        !aligned(wv_inject[l], 16) || !aligned(k_cache[l], 16) || !aligned(v_cache[l], 16))
      return fail(PE_ERR_INVALID_ARG, "injection weights or KV cache of layer %d NULL or misaligned", l);
  const int kvd = k.n_kv_heads * k.head_dim;
  for (int l = 0; l < k.layers; ++l) {
    pe::GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.M = B * (k.K + 1); g.N = 2 * kvd; g.K = k.d;
    g.A = target_hidden; g.lda = k.d;
    g.d = k.d; g.vocab = k.vocab;
    g.W1 = wk_inject[l]; g.W2 = wv_inject[l]; g.nq = 0; g.nk = kvd;
    g.positions = verify_positions; g.slots = inject_slots;
    g.kcache = k_cache[l]; g.vcache = v_cache[l];
    g.Hkv = k.n_kv_heads; g.hd = k.head_dim; g.block_size = k.block_size;
    g.num_slots = (long long)num_kv_blocks * k.block_size;
    g.rope_turns = ctx->rope_turns;
    g.part = ctx->splitk; g.part_cap = ctx->splitk_cap;
    Timed tm(ctx, PE_PH_QKV);
    PE_HIP(pe::launch_gemm(k.dtype, pe::A_PLAIN, pe::B_QKV, pe::E_QKV, g, ctx->num_cus, ctx->stream), "kv injection");
  }
  return PE_OK;
}

pe_status pe_dflash_forward(pe_ctx* ctx, int32_t B, const pe_batch* batch, const int32_t* attn_positions,
                            const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                            void* const* k_cache, void* const* v_cache, int32_t* draft_tokens, float* logits) {
  // the block's input is the embedding alone: no hidden states
  pe_status s = check_forward(ctx, B, batch, nullptr, block_table, max_blocks, num_kv_blocks, k_cache, v_cache,
                              draft_tokens, logits, false);
  if (s != PE_OK || B == 0) return s;
  if (!attn_positions || !aligned(attn_positions, 4)) return fail(PE_ERR_INVALID_ARG, "attn_positions");
  Pass P;
  P.B = B; P.S = ctx->cfg.K + 1; P.Kd = ctx->cfg.K;
  P.ids = batch->input_ids; P.pos = batch->positions; P.draft_rows = batch->draft_rows;
  P.seq_lens = batch->seq_lens; P.rej = batch->is_rejected; P.slots = batch->slot_mapping;
  P.hidden = nullptr; P.embed_input = true; P.attn_pos = attn_positions;
  P.tokens = draft_tokens; P.tstride = 1;
  P.logits = logits; P.ldl = ctx->cfg.vocab;
  return forward_pass(ctx, P, block_table, max_blocks, num_kv_blocks, k_cache, v_cache);
}

// ---- stochastic drafting and verification by rejection sampling ------------
static pe_status check_sampling(float temperature, const uint64_t* seed) {
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(PE_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (!seed || !aligned(seed, 8)) return fail(PE_ERR_INVALID_ARG, "seed NULL or not 8-byte aligned");
  return PE_OK;
}

pe_status pe_draft_forward_sampled(pe_ctx* ctx, int32_t B, const pe_batch* batch, const void* draft_hidden,
                                   const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                                   void* const* k_cache, void* const* v_cache, float temperature,
                                   const uint64_t* seed, int32_t* draft_tokens, float* logits) {
  pe_status s = check_forward(ctx, B, batch, draft_hidden, block_table, max_blocks, num_kv_blocks,
                              k_cache, v_cache, draft_tokens, logits);
  if (s != PE_OK) return s;
  if ((s = check_sampling(temperature, seed)) != PE_OK || B == 0) return s;
  if (!logits || !aligned(logits, 16))
    return fail(PE_ERR_INVALID_ARG, "sampled drafting draws from the logits: NULL or not 16-byte aligned");
  const int K = ctx->cfg.K;
  Pass P;
  P.B = B; P.S = 2 * K; P.Kd = K; P.parallel_layout = true;
  P.ids = batch->input_ids; P.pos = batch->positions; P.draft_rows = batch->draft_rows;
  P.seq_lens = batch->seq_lens; P.rej = batch->is_rejected; P.slots = batch->slot_mapping;
  P.hidden = draft_hidden;
  P.tokens = draft_tokens; P.tstride = 1;
  P.logits = logits; P.ldl = ctx->cfg.vocab;
  P.seed = seed; P.inv_temp = 1.f / temperature;
  return forward_pass(ctx, P, block_table, max_blocks, num_kv_blocks, k_cache, v_cache);
}

pe_status pe_verify_sampled(pe_ctx* ctx, int32_t B, const int32_t* draft_tokens, const float* draft_logits,
                            const float* target_logits, float temperature, const uint64_t* seed,
                            int32_t* num_accepted, int32_t* next_tokens) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if ((s = check_sampling(temperature, seed)) != PE_OK || B == 0) return s;
  if (!draft_tokens || !num_accepted || !next_tokens) return fail(PE_ERR_INVALID_ARG, "a verify buffer is NULL");
  if (!draft_logits || !target_logits || !aligned(draft_logits, 16) || !aligned(target_logits, 16))
    return fail(PE_ERR_INVALID_ARG, "logit rows NULL or not 16-byte aligned");
  Timed tm(ctx, PE_PH_VERIFY);
  PE_HIP(pe::launch_verify_sampled(B, ctx->cfg.K, ctx->cfg.vocab, 1.f / temperature, draft_tokens, draft_logits,
                                   target_logits, seed, ctx->sample_lse, ctx->sample_parts, ctx->sample_keys,
                                   num_accepted,
                                   next_tokens, ctx->stream),
         "sampled verify launch");
  return PE_OK;
}

}  // extern "C"

// ---- sampled verification without allocation --------------------------------
// Workspace of pe_verify_sampled_noalloc in a file-scope device array (one copy
// per GPU, held until the process ends): partial argmax keys [B * kSampleParts]
// u64, then per-slice (max, sum exp) [rows * kLseParts * 2] and per-row
// log-sum-exp [rows] fp32, rows = B (2K + 1).
namespace {
constexpr int kNaMaxRows = 8192;  // B (2K + 1)
constexpr int kNaMaxReq = 2048;   // B
constexpr size_t kNaKeyBytes = size_t(kNaMaxReq) * pe::kSampleParts * 8;
constexpr size_t kNaPartBytes = size_t(kNaMaxRows) * pe::kLseParts * 2 * 4;
constexpr size_t kNaLseBytes = size_t(kNaMaxRows) * 4;
constexpr int kNaMaxDevices = 64;
std::mutex g_na_mu;
void* g_na_ptr[kNaMaxDevices] = {};  // device address of `scratch` on each device, once looked up
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNaKeyBytes + kNaPartBytes + kNaLseBytes];

// The device address of this GPU's `scratch`: host code must use it, never the
// array's name (a host-side stand-in).  Looked up once per device, with that
// device current.
static pe_status noalloc_scratch(void** out) {
  int dev = 0;
  PE_HIP(hipGetDevice(&dev), "current device");
  if (dev < 0 || dev >= kNaMaxDevices) return fail(PE_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_na_mu);
  if (!g_na_ptr[dev]) {
    void* p = nullptr;
    PE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address");
    if (!p) return fail(PE_ERR_HIP, "scratch address is NULL");
    g_na_ptr[dev] = p;
  }
  *out = g_na_ptr[dev];
  return PE_OK;
}

extern "C" {

pe_status pe_verify_sampled_noalloc(int32_t B, int32_t K, int32_t vocab, const int32_t* draft_tokens,
                                    const float* draft_logits, const float* target_logits, float temperature,
                                    const uint64_t* seed, int32_t* num_accepted, int32_t* next_tokens,
                                    void* stream) {
  g_err.clear();
  if (B < 0 || K < 1 || K > 32) return fail(PE_ERR_INVALID_ARG, "B=%d K=%d (B >= 0, 1 <= K <= 32)", B, K);
  if (vocab < 4 || vocab % 4) return fail(PE_ERR_INVALID_ARG, "vocab=%d must be a positive multiple of 4", vocab);
  if (B > kNaMaxReq || (long long)B * (2 * K + 1) > kNaMaxRows)
    return fail(PE_ERR_UNSUPPORTED, "B=%d, K=%d: beyond the fixed workspace (B <= %d, B (2K+1) <= %d)", B, K,
                kNaMaxReq, kNaMaxRows);
  pe_status s = check_sampling(temperature, seed);
  if (s != PE_OK || B == 0) return s;
  if (!draft_tokens || !num_accepted || !next_tokens) return fail(PE_ERR_INVALID_ARG, "a verify buffer is NULL");
  if (!draft_logits || !target_logits || !aligned(draft_logits, 16) || !aligned(target_logits, 16))
    return fail(PE_ERR_INVALID_ARG, "logit rows NULL or not 16-byte aligned");
  void* base = nullptr;
  if ((s = noalloc_scratch(&base)) != PE_OK) return s;
  unsigned char* b = static_cast<unsigned char*>(base);
  uint64_t* keys = reinterpret_cast<uint64_t*>(b);
  float* parts = reinterpret_cast<float*>(b + kNaKeyBytes);
  float* lse = reinterpret_cast<float*>(b + kNaKeyBytes + kNaPartBytes);
  PE_HIP(pe::launch_verify_sampled(B, K, vocab, 1.f / temperature, draft_tokens, draft_logits, target_logits, seed,
                                   lse, parts, keys, num_accepted, next_tokens,
                                   reinterpret_cast<hipStream_t>(stream)),
         "sampled verify launch");
  return PE_OK;
}

pe_status pe_verify(pe_ctx* ctx, int32_t B, const int32_t* draft_tokens, const int32_t* target_tokens,
                    int32_t* num_accepted, int32_t* bonus_tokens) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if (B == 0) return PE_OK;
  if (!draft_tokens || !target_tokens || !num_accepted || !bonus_tokens)
    return fail(PE_ERR_INVALID_ARG, "a verify buffer is NULL");
  Timed tm(ctx, PE_PH_VERIFY);
  PE_HIP(pe::launch_verify(B, ctx->cfg.K, draft_tokens, target_tokens, num_accepted, bonus_tokens, ctx->nact,
                           ctx->stream),
         "verify launch");
  return PE_OK;
}

// The parallel step with two launch fusions (preparation + hidden-state copy,
// argmax + verification); every argument is checked as the four entry points
// check it, and the results are the same.
static pe_status run_parallel_step(pe_ctx* ctx, int32_t B, const pe_step_args* a) {
  pe::PrepareArgs pa;
  pe_status s = prepare_args(ctx, B, a->verify_tokens, a->verify_positions, a->num_accepted,
                             a->bonus_tokens, a->block_table, a->max_blocks, a->num_kv_blocks,
                             &a->batch, pa);
  if (s != PE_OK) return s;
  if ((s = check_gather(ctx, B, &a->batch, a->target_hidden, a->h_shared, a->draft_hidden)) != PE_OK)
    return s;
  if ((s = check_forward(ctx, B, &a->batch, a->draft_hidden, a->block_table, a->max_blocks,
                         a->num_kv_blocks, a->k_cache, a->v_cache, a->draft_tokens, a->logits)) != PE_OK)
    return s;
  if (B == 0) return PE_OK;
  if (!a->target_tokens || !a->accepted_out || !a->bonus_out)
    return fail(PE_ERR_INVALID_ARG, "a verify buffer is NULL");
  const int K = ctx->cfg.K;
  {
    Timed tm(ctx, PE_PH_PREPARE);
    PE_HIP(pe::launch_prepare_gather(pa, int(ctx->cfg.d * ctx->esz), a->target_hidden, a->h_shared,
                                     a->draft_hidden, ctx->stream),
           "prepare + gather launch");
  }
  Pass P;
  P.B = B; P.S = 2 * K; P.Kd = K; P.parallel_layout = true;
  P.ids = a->batch.input_ids; P.pos = a->batch.positions; P.draft_rows = a->batch.draft_rows;
  P.seq_lens = a->batch.seq_lens; P.rej = a->batch.is_rejected; P.slots = a->batch.slot_mapping;
  P.hidden = a->draft_hidden;
  P.tokens = a->draft_tokens; P.tstride = 1;
  P.logits = a->logits; P.ldl = ctx->cfg.vocab;
  P.vtarget = a->target_tokens; P.vacc = a->accepted_out; P.vbonus = a->bonus_out;
  return forward_pass(ctx, P, a->block_table, a->max_blocks, a->num_kv_blocks, a->k_cache, a->v_cache);
}

static pe_status run_step(pe_ctx* ctx, int32_t B, const pe_step_args* a) {
  if (a->mode == PE_STEP_PARALLEL) return run_parallel_step(ctx, B, a);
  if (a->mode == PE_STEP_DFLASH) {
    pe_status s = pe_dflash_prepare(ctx, B, a->verify_positions, a->num_accepted, a->bonus_tokens, a->block_table,
                                    a->max_blocks, a->num_kv_blocks, &a->batch, a->attn_positions, a->inject_slots);
    if (s != PE_OK) return s;
    s = pe_dflash_inject(ctx, B, a->verify_positions, a->inject_slots, a->target_hidden, a->wk_inject,
                         a->wv_inject, a->num_kv_blocks, a->k_cache, a->v_cache);
    if (s != PE_OK) return s;
    s = pe_dflash_forward(ctx, B, &a->batch, a->attn_positions, a->block_table, a->max_blocks, a->num_kv_blocks,
                          a->k_cache, a->v_cache, a->draft_tokens, a->logits);
    if (s != PE_OK) return s;
    return pe_verify(ctx, B, a->draft_tokens, a->target_tokens, a->accepted_out, a->bonus_out);
  }
  pe_status s = pe_prepare(ctx, B, a->verify_tokens, a->verify_positions, a->num_accepted,
                           a->bonus_tokens, a->block_table, a->max_blocks, a->num_kv_blocks, &a->batch);
  if (s != PE_OK) return s;
  s = pe_gather_hidden(ctx, B, &a->batch, a->target_hidden, a->h_shared, a->draft_hidden);
  if (s != PE_OK) return s;
  s = pe_ar_draft(ctx, B, &a->batch, a->draft_hidden, a->block_table, a->max_blocks, a->num_kv_blocks,
          a->k_cache, a->v_cache, a->draft_tokens, a->logits);
  if (s != PE_OK) return s;
  return pe_verify(ctx, B, a->draft_tokens, a->target_tokens, a->accepted_out, a->bonus_out);
}

pe_status pe_step_graph(pe_ctx* ctx, int32_t B, const pe_step_args* args) {
  pe_status s = check_B(ctx, B);
  if (s != PE_OK) return s;
  if (!args || !args->k_cache || !args->v_cache) return fail(PE_ERR_INVALID_ARG, "step args");
  if (args->mode != PE_STEP_PARALLEL && args->mode != PE_STEP_AUTOREGRESSIVE && args->mode != PE_STEP_DFLASH)
    return fail(PE_ERR_INVALID_ARG, "step mode %d", args->mode);
  const bool dfl = args->mode == PE_STEP_DFLASH;
  if (dfl && (!args->wk_inject || !args->wv_inject)) return fail(PE_ERR_INVALID_ARG, "injection weight arrays");
  const int nl = ctx->cfg.layers;
  // the captured pointers: KV caches, and the injection weights of a DFlash round
  std::vector<void*> kv(dfl ? 4 * nl : 2 * nl);
  for (int l = 0; l < nl; ++l) {
    kv[l] = args->k_cache[l];
    kv[nl + l] = args->v_cache[l];
    if (dfl) {
      kv[2 * nl + l] = const_cast<void*>(args->wk_inject[l]);
      kv[3 * nl + l] = const_cast<void*>(args->wv_inject[l]);
    }
  }
  const bool same = ctx->gexec && ctx->graph_B == B &&
                    std::memcmp(&ctx->graph_args, args, sizeof *args) == 0 && ctx->graph_kv == kv;
  if (!same) {
    if (ctx->gexec) {
      // the graph being replaced may still run on the context's stream
      PE_HIP(hipStreamSynchronize(ctx->stream), "sync before recapture");
      (void)hipGraphExecDestroy(ctx->gexec);
      ctx->gexec = nullptr;
    }
    if (ctx->graph) { (void)hipGraphDestroy(ctx->graph); ctx->graph = nullptr; }
    if (!ctx->capture_stream)
      PE_HIP(hipStreamCreateWithFlags(&ctx->capture_stream, hipStreamNonBlocking), "capture stream");
    // capture records launches without running them, so the work already
    // queued on the context's stream needs no wait: the graph's launches are
    // enqueued behind it
    PE_HIP(hipStreamBeginCapture(ctx->capture_stream, hipStreamCaptureModeRelaxed), "begin capture");
    hipStream_t user = ctx->stream;
    ctx->stream = ctx->capture_stream;
    ctx->capturing = true;
    ctx->nact = args->num_active;
    s = run_step(ctx, B, args);
    ctx->nact = nullptr;
    ctx->capturing = false;
    ctx->stream = user;
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(ctx->capture_stream, &graph);
    if (s != PE_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return s;
    }
    if (e != hipSuccess) return hipfail(e, "end capture");
    ctx->graph = graph;
    PE_HIP(hipGraphInstantiate(&ctx->gexec, graph, nullptr, nullptr, 0), "graph instantiate");
    ctx->graph_B = B;
    ctx->graph_args = *args;
    ctx->graph_kv = kv;
    ++ctx->graph_captures;
  }
  PE_HIP(hipGraphLaunch(ctx->gexec, ctx->stream), "graph launch");
  ++ctx->graph_replays;
  return PE_OK;
}

pe_status pe_step_graph_stats(pe_ctx* ctx, int64_t* captures, int64_t* replays) {
  if (!ctx || !captures || !replays) return fail(PE_ERR_INVALID_ARG, "NULL argument");
  *captures = ctx->graph_captures;
  *replays = ctx->graph_replays;
  return PE_OK;
}

pe_status pe_choose_depth(const int32_t* Ks, const double* draft_us, int32_t n, double alpha,
                          double verify_fixed_us, double verify_per_token_us, int32_t* best_K,
                          double* tokens_per_us) {
  if (!Ks || !draft_us || !best_K || !tokens_per_us || n < 1) return fail(PE_ERR_INVALID_ARG, "depth selection arguments");
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(PE_ERR_INVALID_ARG, "alpha %g outside [0, 1]", alpha);
  if (!(verify_fixed_us >= 0.0) || !(verify_per_token_us >= 0.0))
    return fail(PE_ERR_INVALID_ARG, "verifier costs must be >= 0");
  int best = -1;
  double best_rate = -1.0;
  for (int i = 0; i < n; ++i) {
    const int K = Ks[i];
    if (K < 1 || K > 32) return fail(PE_ERR_INVALID_ARG, "K=%d outside [1, 32]", K);
    const double cost = draft_us[i] + verify_fixed_us + verify_per_token_us * (K + 1);
    if (!(draft_us[i] > 0.0) || !(cost > 0.0)) return fail(PE_ERR_INVALID_ARG, "draft cost of K=%d not positive", K);
    double e = 0.0, a = 1.0;
    for (int j = 0; j <= K; ++j) { e += a; a *= alpha; }
    const double rate = e / cost;
    if (rate > best_rate || (rate == best_rate && K < best)) { best = K; best_rate = rate; }
  }
  *best_K = best;
  *tokens_per_us = best_rate;
  return PE_OK;
}

pe_status pe_get_device_error(pe_ctx* ctx, uint32_t* kinds, int32_t* first_request) {
  if (!ctx || !kinds || !first_request) return fail(PE_ERR_INVALID_ARG, "NULL argument");
  uint32_t h[4] = {0, 0, 0, 0};
  const uint32_t err0[4] = {0u, 0xFFFFFFFFu, 0u, 0u};
  PE_HIP(hipStreamSynchronize(ctx->stream), "sync");
  PE_HIP(hipMemcpy(h, ctx->err, 16, hipMemcpyDeviceToHost), "read error word");
  PE_HIP(hipMemcpy(ctx->err, err0, 16, hipMemcpyHostToDevice), "clear error word");
  *kinds = h[0];
  *first_request = h[0] ? int32_t(h[1]) : -1;
  return PE_OK;
}

pe_status pe_profile_enable(pe_ctx* ctx, int on) {
  if (!ctx) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  ctx->prof_on = on != 0;
  return PE_OK;
}

pe_status pe_profile_read(pe_ctx* ctx, double* ms, int64_t* launches, int reset) {
  if (!ctx || !ms || !launches) return fail(PE_ERR_INVALID_ARG, "NULL argument");
  PE_HIP(hipStreamSynchronize(ctx->stream), "sync");
  for (auto& r : ctx->recs) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
      ctx->prof_ms[r.phase] += t;
      ctx->prof_n[r.phase] += 1;
    }
    ctx->ev_free.push_back(r.a);
    ctx->ev_free.push_back(r.b);
  }
  ctx->recs.clear();
  for (int i = 0; i < PE_PH_COUNT; ++i) {
    ms[i] = ctx->prof_ms[i];
    launches[i] = ctx->prof_n[i];
    if (reset) { ctx->prof_ms[i] = 0.0; ctx->prof_n[i] = 0; }
  }
  return PE_OK;
}

}  // extern "C"
