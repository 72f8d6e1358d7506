"""Thin ctypes binding of libpe.so (include/pe.h).

Argument marshalling only: every step of the draft path runs in the HIP
kernels of libpe.so.  PyTorch provides device memory and the stream.  The
functions carry the C names (pe_prepare, pe_gather_hidden, pe_draft_forward,
pe_verify, pe_step_graph, pe_get_device_error) and take a Context first.

torch is imported before the library is loaded so that libpe.so binds to the
HIP runtime torch already loaded (one runtime, shareable streams).  If
libpe.so is missing this module raises; there is no fallback.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PE_LIB") or os.path.join(_HERE, "libpe.so")

PE_F32, PE_BF16 = 0, 1
DEVERR_ACCEPTED, DEVERR_TOKEN, DEVERR_BLOCK, DEVERR_LAYOUT = 1, 2, 4, 8

EXPORTS = ("pe_create", "pe_destroy", "pe_set_stream", "pe_prepare", "pe_gather_hidden",
           "pe_draft_forward", "pe_ar_draft", "pe_verify", "pe_prefill_prepare", "pe_prefill_gather",
           "pe_prefill_forward", "pe_draft_forward_sampled", "pe_verify_sampled", "pe_choose_depth",
           "pe_dflash_prepare", "pe_dflash_inject", "pe_dflash_forward", "pe_step_graph",
           "pe_step_graph_stats", "pe_verify_sampled_noalloc", "pe_get_device_error",
           "pe_profile_enable", "pe_profile_read", "pe_last_error", "pe_status_string")
PHASES = ("prepare", "gather", "fc", "norm", "qkv", "attn", "o", "gateup", "down", "lmhead",
          "verify", "argmax", "ar")
STEP_PARALLEL, STEP_AUTOREGRESSIVE, STEP_DFLASH = 0, 1, 2

vp, i32 = ctypes.c_void_p, ctypes.c_int32


class PeConfig(ctypes.Structure):
    _fields_ = [(n, i32) for n in ("K", "max_num_seqs", "d", "n_q_heads", "n_kv_heads", "head_dim",
                                   "mlp", "layers", "vocab", "block_size", "mask_id", "dtype")] + \
               [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_prefill_slots", i32)]


class PeLayerWeights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm",
                                  "w_gate", "w_up", "w_down")]


class PeWeights(ctypes.Structure):
    _fields_ = [("embed", vp), ("w_fc", vp), ("layers", ctypes.POINTER(PeLayerWeights)),
                ("final_norm", vp), ("lm_head", vp)]


BATCH_FIELDS = ("input_ids", "positions", "hidden_src", "is_rejected", "is_masked",
                "slot_mapping", "draft_rows", "seq_lens")


class PeBatch(ctypes.Structure):
    _fields_ = [(n, vp) for n in BATCH_FIELDS]


class PeStepArgs(ctypes.Structure):
    _fields_ = [("verify_tokens", vp), ("verify_positions", vp), ("num_accepted", vp),
                ("bonus_tokens", vp), ("block_table", vp), ("max_blocks", i32),
                ("num_kv_blocks", i32), ("batch", PeBatch), ("target_hidden", vp),
                ("h_shared", vp), ("draft_hidden", vp), ("k_cache", ctypes.POINTER(vp)),
                ("v_cache", ctypes.POINTER(vp)), ("draft_tokens", vp), ("logits", vp),
                ("target_tokens", vp), ("accepted_out", vp), ("bonus_out", vp),
                ("mode", i32), ("wk_inject", ctypes.POINTER(vp)), ("wv_inject", ctypes.POINTER(vp)),
                ("attn_positions", vp), ("inject_slots", vp), ("num_active", vp)]


class PeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "PE_OK", 1: "PE_ERR_INVALID_ARG", 2: "PE_ERR_NOMEM", 3: "PE_ERR_HIP",
           4: "PE_ERR_UNSUPPORTED"}
_lib = None


def load(path: str = LIB_PATH):
    """Load libpe.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with "
                                "`python -m drafting_pe_prepare_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.pe_create.argtypes = [P(PeConfig), P(PeWeights), vp, P(vp)]
    lib.pe_destroy.argtypes = [vp]
    lib.pe_set_stream.argtypes = [vp, vp]
    lib.pe_prepare.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, i32, P(PeBatch)]
    lib.pe_gather_hidden.argtypes = [vp, i32, P(PeBatch), vp, vp, vp]
    lib.pe_draft_forward.argtypes = [vp, i32, P(PeBatch), vp, vp, i32, i32, P(vp), P(vp), vp, vp]
    lib.pe_ar_draft.argtypes = [vp, i32, P(PeBatch), vp, vp, i32, i32, P(vp), P(vp), vp, vp]
    lib.pe_verify.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.pe_prefill_prepare.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, i32, i32, P(PeBatch)]
    lib.pe_prefill_gather.argtypes = [vp, i32, i32, P(PeBatch), vp, vp, vp]
    lib.pe_prefill_forward.argtypes = [vp, i32, i32, P(PeBatch), vp, vp, i32, i32, P(vp), P(vp), vp, vp]
    lib.pe_draft_forward_sampled.argtypes = [vp, i32, P(PeBatch), vp, vp, i32, i32, P(vp), P(vp),
                                             ctypes.c_float, vp, vp, vp]
    lib.pe_verify_sampled.argtypes = [vp, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.pe_dflash_prepare.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, P(PeBatch), vp, vp]
    lib.pe_dflash_inject.argtypes = [vp, i32, vp, vp, vp, P(vp), P(vp), i32, P(vp), P(vp)]
    lib.pe_dflash_forward.argtypes = [vp, i32, P(PeBatch), vp, vp, i32, i32, P(vp), P(vp), vp, vp]
    lib.pe_choose_depth.argtypes = [P(i32), P(ctypes.c_double), i32, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_double, P(i32), P(ctypes.c_double)]
    lib.pe_step_graph.argtypes = [vp, i32, P(PeStepArgs)]
    lib.pe_step_graph_stats.argtypes = [vp, P(ctypes.c_int64), P(ctypes.c_int64)]
    lib.pe_verify_sampled_noalloc.argtypes = [i32, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp]
    lib.pe_get_device_error.argtypes = [vp, P(ctypes.c_uint32), P(i32)]
    lib.pe_profile_enable.argtypes = [vp, ctypes.c_int]
    lib.pe_profile_read.argtypes = [vp, P(ctypes.c_double), P(ctypes.c_int64), ctypes.c_int]
    lib.pe_last_error.argtypes = []
    lib.pe_status_string.argtypes = [ctypes.c_int]
    lib.pe_last_error.restype = ctypes.c_char_p
    lib.pe_status_string.restype = ctypes.c_char_p
    for n in EXPORTS[:-2]:
        getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise PeError(status, _lib.pe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"
    return t.data_ptr()


def _stream_handle(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Batch:
    """Device buffers of a pe_batch for up to `max_B` requests."""

    def __init__(self, max_B: int, K: int, device="cuda", S: int = None):
        S = 2 * K if S is None else S
        self.S = S
        n = max_B * S
        i = dict(dtype=torch.int32, device=device)
        self.input_ids = torch.zeros(n, **i)
        self.positions = torch.zeros(n, **i)
        self.hidden_src = torch.zeros(n, **i)
        self.is_rejected = torch.zeros(n, dtype=torch.uint8, device=device)
        self.is_masked = torch.zeros(n, dtype=torch.uint8, device=device)
        self.slot_mapping = torch.zeros(n, dtype=torch.int64, device=device)
        self.draft_rows = torch.zeros(max_B * K, **i)
        self.seq_lens = torch.zeros(max_B, **i)
        self.c = PeBatch(*[_ptr(getattr(self, f)) for f in BATCH_FIELDS])

    def host(self, B: int, K: int) -> dict:
        S = self.S
        n = {f: B * S for f in BATCH_FIELDS}
        n["draft_rows"], n["seq_lens"] = B * K, B
        return {f: getattr(self, f)[:n[f]].cpu().numpy() for f in BATCH_FIELDS}


class Context:
    """A libpe context: one drafter's weights (borrowed) and workspace."""

    def __init__(self, cfg, weights: dict, max_num_seqs: int, stream=None, max_prefill_slots: int = 0):
        lib = load()
        self.cfg = cfg
        self.weights = weights  # keep the device tensors alive
        dtype = PE_BF16 if cfg.dtype == "bf16" else PE_F32
        self.c_cfg = PeConfig(cfg.K, max_num_seqs, cfg.d, cfg.n_q_heads, cfg.n_kv_heads,
                              cfg.head_dim, cfg.mlp, cfg.layers, cfg.vocab, cfg.block_size,
                              cfg.mask_id, dtype, cfg.rms_eps, cfg.rope_theta, max_prefill_slots)
        L = len(weights["layers"])
        self.c_layers = (PeLayerWeights * L)(*[
            PeLayerWeights(*[_ptr(lw[n]) for n, _ in PeLayerWeights._fields_])
            for lw in weights["layers"]])
        self.c_w = PeWeights(_ptr(weights["embed"]), _ptr(weights["w_fc"]),
                             ctypes.cast(self.c_layers, ctypes.POINTER(PeLayerWeights)),
                             _ptr(weights["final_norm"]), _ptr(weights["lm_head"]))
        h = vp()
        _check(lib.pe_create(ctypes.byref(self.c_cfg), ctypes.byref(self.c_w),
                             _stream_handle(stream), ctypes.byref(h)))
        self.h = h
        self.max_num_seqs = max_num_seqs

    def close(self):
        if self.h:
            _check(_lib.pe_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr_array(ts):
    return (vp * len(ts))(*[_ptr(t) for t in ts])


def pe_set_stream(ctx: Context, stream=None):
    _check(_lib.pe_set_stream(ctx.h, _stream_handle(stream)))


def pe_prepare(ctx: Context, B, verify_tokens, verify_positions, num_accepted, bonus_tokens,
               block_table, num_kv_blocks, batch: Batch):
    max_blocks = block_table.shape[1] if block_table.dim() == 2 else 1
    _check(_lib.pe_prepare(ctx.h, B, _ptr(verify_tokens), _ptr(verify_positions),
                           _ptr(num_accepted), _ptr(bonus_tokens), _ptr(block_table),
                           max_blocks, num_kv_blocks, ctypes.byref(batch.c)))


def pe_gather_hidden(ctx: Context, B, batch: Batch, target_hidden, h_shared, draft_hidden):
    _check(_lib.pe_gather_hidden(ctx.h, B, ctypes.byref(batch.c), _ptr(target_hidden),
                                 _ptr(h_shared), _ptr(draft_hidden)))


def pe_draft_forward(ctx: Context, B, batch: Batch, draft_hidden, block_table, num_kv_blocks,
                     k_caches, v_caches, draft_tokens, logits=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(_lib.pe_draft_forward(ctx.h, B, ctypes.byref(batch.c), _ptr(draft_hidden),
                                 _ptr(block_table), block_table.shape[1], num_kv_blocks,
                                 kc, vc, _ptr(draft_tokens), _ptr(logits)))


def pe_ar_draft(ctx: Context, B, batch: Batch, draft_hidden, block_table, num_kv_blocks,
                k_caches, v_caches, draft_tokens, logits=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(_lib.pe_ar_draft(ctx.h, B, ctypes.byref(batch.c), _ptr(draft_hidden),
                            _ptr(block_table), block_table.shape[1], num_kv_blocks,
                            kc, vc, _ptr(draft_tokens), _ptr(logits)))


def pe_prefill_prepare(ctx: Context, B, S, chunk_tokens, chunk_lens, start_pos, new_tokens,
                       block_table, num_kv_blocks, batch: Batch):
    max_blocks = block_table.shape[1] if block_table.dim() == 2 else 1
    _check(_lib.pe_prefill_prepare(ctx.h, B, S, _ptr(chunk_tokens), _ptr(chunk_lens), _ptr(start_pos),
                                   _ptr(new_tokens), _ptr(block_table), max_blocks, num_kv_blocks,
                                   ctypes.byref(batch.c)))


def pe_prefill_gather(ctx: Context, B, S, batch: Batch, target_hidden, h_shared, draft_hidden):
    _check(_lib.pe_prefill_gather(ctx.h, B, S, ctypes.byref(batch.c), _ptr(target_hidden),
                                  _ptr(h_shared), _ptr(draft_hidden)))


def pe_prefill_forward(ctx: Context, B, S, batch: Batch, draft_hidden, block_table, num_kv_blocks,
                       k_caches, v_caches, draft_tokens, logits=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(_lib.pe_prefill_forward(ctx.h, B, S, ctypes.byref(batch.c), _ptr(draft_hidden),
                                   _ptr(block_table), block_table.shape[1], num_kv_blocks,
                                   kc, vc, _ptr(draft_tokens), _ptr(logits)))


def pe_draft_forward_sampled(ctx: Context, B, batch: Batch, draft_hidden, block_table, num_kv_blocks,
                             k_caches, v_caches, temperature, seed, draft_tokens, logits=None):
    """seed: a device tensor holding one 64-bit key (int64)."""
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(_lib.pe_draft_forward_sampled(ctx.h, B, ctypes.byref(batch.c), _ptr(draft_hidden),
                                         _ptr(block_table), block_table.shape[1], num_kv_blocks,
                                         kc, vc, float(temperature), _ptr(seed), _ptr(draft_tokens),
                                         _ptr(logits)))


def pe_verify_sampled(ctx: Context, B, draft_tokens, draft_logits, target_logits, temperature, seed,
                      num_accepted, next_tokens):
    _check(_lib.pe_verify_sampled(ctx.h, B, _ptr(draft_tokens), _ptr(draft_logits), _ptr(target_logits),
                                  float(temperature), _ptr(seed), _ptr(num_accepted), _ptr(next_tokens)))


def pe_dflash_prepare(ctx: Context, B, verify_positions, num_accepted, bonus_tokens, block_table,
                      num_kv_blocks, batch: Batch, attn_positions, inject_slots):
    """batch: a Batch with S = K+1; attn_positions int32 and inject_slots
    int64 device tensors of B*(K+1) elements."""
    _check(_lib.pe_dflash_prepare(ctx.h, B, _ptr(verify_positions), _ptr(num_accepted), _ptr(bonus_tokens),
                                  _ptr(block_table), block_table.shape[1], num_kv_blocks, ctypes.byref(batch.c),
                                  _ptr(attn_positions), _ptr(inject_slots)))


def pe_dflash_inject(ctx: Context, B, verify_positions, inject_slots, target_hidden, wk_inject, wv_inject,
                     num_kv_blocks, k_caches, v_caches):
    _check(_lib.pe_dflash_inject(ctx.h, B, _ptr(verify_positions), _ptr(inject_slots), _ptr(target_hidden),
                                 _ptr_array(wk_inject), _ptr_array(wv_inject), num_kv_blocks,
                                 _ptr_array(k_caches), _ptr_array(v_caches)))


def pe_dflash_forward(ctx: Context, B, batch: Batch, attn_positions, block_table, num_kv_blocks,
                      k_caches, v_caches, draft_tokens, logits=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(_lib.pe_dflash_forward(ctx.h, B, ctypes.byref(batch.c), _ptr(attn_positions), _ptr(block_table),
                                  block_table.shape[1], num_kv_blocks, kc, vc, _ptr(draft_tokens), _ptr(logits)))


def pe_choose_depth(Ks, draft_us, alpha, verify_fixed_us=0.0, verify_per_token_us=0.0):
    """Host-only: (best K, tokens per microsecond)."""
    n = len(Ks)
    ks = (i32 * n)(*[int(k) for k in Ks])
    ts = (ctypes.c_double * n)(*[float(t) for t in draft_us])
    best, rate = i32(0), ctypes.c_double(0.0)
    _check(load().pe_choose_depth(ks, ts, n, float(alpha), float(verify_fixed_us), float(verify_per_token_us),
                                  ctypes.byref(best), ctypes.byref(rate)))
    return int(best.value), float(rate.value)


def pe_verify(ctx: Context, B, draft_tokens, target_tokens, num_accepted, bonus_tokens):
    _check(_lib.pe_verify(ctx.h, B, _ptr(draft_tokens), _ptr(target_tokens),
                          _ptr(num_accepted), _ptr(bonus_tokens)))


def make_step_args(verify_tokens, verify_positions, num_accepted, bonus_tokens, block_table,
                   num_kv_blocks, batch: Batch, target_hidden, h_shared, draft_hidden,
                   k_caches, v_caches, draft_tokens, target_tokens, accepted_out, bonus_out,
                   logits=None, mode=STEP_PARALLEL, num_active=None) -> PeStepArgs:
    """num_active: None, or a device int32 tensor of one element holding the
    occupancy (requests at or past it are inactive padding)."""
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    a = PeStepArgs(_ptr(verify_tokens), _ptr(verify_positions), _ptr(num_accepted),
                   _ptr(bonus_tokens), _ptr(block_table), block_table.shape[1], num_kv_blocks,
                   batch.c, _ptr(target_hidden), _ptr(h_shared), _ptr(draft_hidden),
                   ctypes.cast(kc, ctypes.POINTER(vp)), ctypes.cast(vc, ctypes.POINTER(vp)),
                   _ptr(draft_tokens), _ptr(logits), _ptr(target_tokens), _ptr(accepted_out),
                   _ptr(bonus_out), mode)
    a.num_active = _ptr(num_active)
    a._keep = (kc, vc)
    return a


def make_dflash_step_args(verify_positions, num_accepted, bonus_tokens, block_table, num_kv_blocks,
                          batch: Batch, target_hidden, k_caches, v_caches, wk_inject, wv_inject,
                          attn_positions, inject_slots, draft_tokens, target_tokens, accepted_out, bonus_out,
                          logits=None, num_active=None) -> PeStepArgs:
    """Step arguments of a DFlash-style round (batch: a Batch with S = K+1)."""
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    wk, wv = _ptr_array(wk_inject), _ptr_array(wv_inject)
    a = PeStepArgs(None, _ptr(verify_positions), _ptr(num_accepted), _ptr(bonus_tokens), _ptr(block_table),
                   block_table.shape[1], num_kv_blocks, batch.c, _ptr(target_hidden), None, None,
                   ctypes.cast(kc, ctypes.POINTER(vp)), ctypes.cast(vc, ctypes.POINTER(vp)),
                   _ptr(draft_tokens), _ptr(logits), _ptr(target_tokens), _ptr(accepted_out),
                   _ptr(bonus_out), STEP_DFLASH, ctypes.cast(wk, ctypes.POINTER(vp)),
                   ctypes.cast(wv, ctypes.POINTER(vp)), _ptr(attn_positions), _ptr(inject_slots),
                   _ptr(num_active))
    a._keep = (kc, vc, wk, wv)
    return a


def pe_step_graph(ctx: Context, B, args: PeStepArgs):
    _check(_lib.pe_step_graph(ctx.h, B, ctypes.byref(args)))


def pe_verify_sampled_noalloc(B, K, vocab, draft_tokens, draft_logits, target_logits, temperature, seed,
                              num_accepted, next_tokens, stream=None):
    """pe_verify_sampled without a context or allocation; stream: a
    torch.cuda.Stream, or None for torch's current stream."""
    _check(_lib.pe_verify_sampled_noalloc(B, K, vocab, _ptr(draft_tokens), _ptr(draft_logits),
                                          _ptr(target_logits), ctypes.c_float(temperature), _ptr(seed),
                                          _ptr(num_accepted), _ptr(next_tokens), _stream_handle(stream)))


def pe_step_graph_stats(ctx: Context):
    """(captures, replays) of pe_step_graph on this context."""
    c, r = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.pe_step_graph_stats(ctx.h, ctypes.byref(c), ctypes.byref(r)))
    return int(c.value), int(r.value)


def pe_get_device_error(ctx: Context):
    k, f = ctypes.c_uint32(), i32()
    _check(_lib.pe_get_device_error(ctx.h, ctypes.byref(k), ctypes.byref(f)))
    return int(k.value), int(f.value)


# ---------------------------------------------------------------------------
# host <-> device marshalling of the synthetic inputs
# ---------------------------------------------------------------------------
def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy storage array -> device tensor with the same bytes (uint16 ->
    bfloat16 bit patterns, int/float as they are)."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy storage array (bfloat16 -> uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def upload_weights(w: dict, device="cuda") -> dict:
    out = {k: to_device(v, device) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: to_device(v, device) for k, v in lw.items()} for lw in w["layers"]]
    return out


def pe_profile_enable(ctx: Context, on: bool = True):
    _check(_lib.pe_profile_enable(ctx.h, 1 if on else 0))


def pe_profile_read(ctx: Context, reset: bool = True) -> dict:
    """{phase: (total ms, launches)} since the last reset; synchronizes."""
    ms = (ctypes.c_double * len(PHASES))()
    n = (ctypes.c_int64 * len(PHASES))()
    _check(_lib.pe_profile_read(ctx.h, ms, n, 1 if reset else 0))
    return {p: (ms[i], n[i]) for i, p in enumerate(PHASES)}
