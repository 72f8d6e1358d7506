"""Seeded synthetic inputs for the P-EAGLE parallel-draft step.

This module only draws numbers.  It holds none of the method's arithmetic, so
the CPU oracle and the HIP path can both be fed from it without sharing any
computation.  Every tensor has its own PCG64 stream keyed by
(seed, crc32(tensor name), chunk index), so any tensor can be regenerated on
its own and the result does not depend on how many threads draw it.

Storage dtypes: "f32" tensors are float32 arrays; "bf16" tensors are uint16
arrays holding bfloat16 bit patterns, rounded to nearest-even from float32.

Distributions (per workload, see configs.py):
  * linear and embedding weights  N(0, weight_std)
  * RMSNorm gains                 1 + 0.1 N(0, 1)
  * h_shared, target hidden       N(0, 1)
  * cached prefix K/V             N(0, 1)
  * token ids                     uniform in [0, V-1)   (V-1 is the MASK id)
  * prefix length p0              fixed, lognormal(ln median, sigma) rounded and
                                  clipped to [128, 16384], or uniform
  * accepted count a              uniform in 0..K, or a fixed value
  * block tables                  a seeded random permutation of a pool of
                                  sum_r ceil((p0_r + 2K) / block_size) blocks
"""
from concurrent.futures import ThreadPoolExecutor
import os
import zlib

import numpy as np

from .configs import Workload

_CHUNK = 1 << 20
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (inputs only)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(arr: np.ndarray) -> np.ndarray:
    """Storage array (float32 or bf16 bits) -> float32 values."""
    if arr.dtype == np.uint16:
        return bf16_to_f32(arr)
    return np.asarray(arr, dtype=np.float32)


def _key(seed: int, name: str):
    return [int(seed), zlib.crc32(name.encode())]


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0,
           dtype: str = "bf16") -> np.ndarray:
    """N(mean, std) tensor of `shape`, stored as `dtype`, drawn chunk by chunk."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    key = _key(seed, name)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(key + [c]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = bf16_bits(v) if dtype == "bf16" else v

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def integers(seed: int, name: str, lo: int, hi: int, shape) -> np.ndarray:
    """Uniform int32 in [lo, hi)."""
    g = np.random.Generator(np.random.PCG64(_key(seed, name)))
    return g.integers(lo, hi, size=shape, dtype=np.int64).astype(np.int32)


def weights(w: Workload, seed: int = None) -> dict:
    """Drafter parameters.  Linear weights are row-major [out, in]."""
    s = w.seed if seed is None else seed
    dt, std, d = w.dtype, w.weight_std, w.d
    qd, kvd = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    out = {
        "embed": normal(s, "embed", (w.vocab, d), std, dtype=dt),
        "h_shared": normal(s, "h_shared", (d,), 1.0, dtype=dt),
        "w_fc": normal(s, "w_fc", (d, 2 * d), std, dtype=dt),
        "final_norm": normal(s, "final_norm", (d,), 0.1, 1.0, dtype=dt),
        "lm_head": normal(s, "lm_head", (w.vocab, d), std, dtype=dt),
        "layers": [],
    }
    for li in range(w.layers):
        p = f"layer{li}."
        out["layers"].append({
            "attn_norm": normal(s, p + "attn_norm", (d,), 0.1, 1.0, dtype=dt),
            "wq": normal(s, p + "wq", (qd, d), std, dtype=dt),
            "wk": normal(s, p + "wk", (kvd, d), std, dtype=dt),
            "wv": normal(s, p + "wv", (kvd, d), std, dtype=dt),
            "wo": normal(s, p + "wo", (d, qd), std, dtype=dt),
            "mlp_norm": normal(s, p + "mlp_norm", (d,), 0.1, 1.0, dtype=dt),
            "w_gate": normal(s, p + "w_gate", (w.mlp, d), std, dtype=dt),
            "w_up": normal(s, p + "w_up", (w.mlp, d), std, dtype=dt),
            "w_down": normal(s, p + "w_down", (d, w.mlp), std, dtype=dt),
        })
    return out


def inject_weights(w: Workload, seed: int = None) -> list:
    """Per layer (Wk_inj, Wv_inj) [Hkv*hd, d]: the projections that write
    verifier hidden states into the drafter's KV cache."""
    s = w.seed if seed is None else seed
    kvd = w.n_kv_heads * w.head_dim
    return [(normal(s, f"layer{li}.wk_inj", (kvd, w.d), w.weight_std, dtype=w.dtype),
             normal(s, f"layer{li}.wv_inj", (kvd, w.d), w.weight_std, dtype=w.dtype))
            for li in range(w.layers)]


def prefix_lengths(w: Workload, seed: int) -> np.ndarray:
    kind, a, b = w.prefix
    g = np.random.Generator(np.random.PCG64(_key(seed, "prefix")))
    if kind == "fixed":
        return np.full(w.batch, int(a), dtype=np.int32)
    if kind == "lognormal":
        v = np.rint(g.lognormal(np.log(a), b, size=w.batch))
        return np.clip(v, 128, 16384).astype(np.int32)
    if kind == "uniform":
        return g.integers(int(a), int(b) + 1, size=w.batch).astype(np.int32)
    raise ValueError(kind)


def step_inputs(w: Workload, seed: int = None, kv: bool = True, extra: int = 0) -> dict:
    """One round's inputs: the previous verify batch, its outcome, the block
    tables, the target hidden states, the cached K/V pool and the target
    tokens the next verify compares against.  Block tables cover p0 + 2K +
    extra positions per request."""
    s = w.seed if seed is None else seed
    B, K, bs = w.batch, w.K, w.block_size
    p0 = prefix_lengths(w, s)
    vt = integers(s, "verify_tokens", 0, w.vocab - 1, (B, K + 1))
    vp = (p0[:, None] + np.arange(K + 1, dtype=np.int32)[None, :]).astype(np.int32)
    if w.accepted == "uniform":
        a = integers(s, "num_accepted", 0, K + 1, (B,))
    else:
        a = np.full(B, int(w.accepted), dtype=np.int32)
    bonus = integers(s, "bonus", 0, w.vocab - 1, (B,))
    tgt = integers(s, "target_tokens", 0, w.vocab - 1, (B, K + 1))

    need = (p0.astype(np.int64) + 2 * K + extra + bs - 1) // bs
    nblocks = int(need.sum())
    max_blocks = int(need.max()) if B else 1
    g = np.random.Generator(np.random.PCG64(_key(s, "block_table")))
    perm = g.permutation(nblocks).astype(np.int32)
    bt = np.zeros((B, max_blocks), dtype=np.int32)
    off = 0
    for r in range(B):
        bt[r, :need[r]] = perm[off:off + need[r]]
        off += int(need[r])

    out = {
        "verify_tokens": vt, "verify_positions": vp, "num_accepted": a,
        "bonus_tokens": bonus, "target_tokens": tgt, "block_table": bt,
        "num_kv_blocks": nblocks, "prefix": p0,
        "target_hidden": normal(s, "target_hidden", (B * (K + 1), w.d), 1.0, dtype=w.dtype),
    }
    if kv:
        out["kv"] = kv_pool(w, nblocks, s)
    return out


def round_ring(w: Workload, inp: dict, n: int, seed: int = None) -> dict:
    """n rounds of the per-round draws, for rotating a step's inputs between
    timed replays: accepted counts, bonus and verify tokens, target tokens.
    Round 0 is `inp` itself (step_inputs' draw); rounds 1..n-1 are drawn like
    it from streams of their own.  Prefix lengths, block tables, hidden
    states and the KV pool stay those of `inp`."""
    s = w.seed if seed is None else seed
    B, K = w.batch, w.K
    keys = ("num_accepted", "bonus_tokens", "verify_tokens", "target_tokens")
    out = {k: [np.asarray(inp[k], dtype=np.int32)] for k in keys}
    for i in range(1, n):
        if w.accepted == "uniform":
            a = integers(s, f"ring{i}.num_accepted", 0, K + 1, (B,))
        else:
            a = np.full(B, int(w.accepted), dtype=np.int32)
        out["num_accepted"].append(a)
        out["bonus_tokens"].append(integers(s, f"ring{i}.bonus", 0, w.vocab - 1, (B,)))
        out["verify_tokens"].append(integers(s, f"ring{i}.verify_tokens", 0, w.vocab - 1, (B, K + 1)))
        out["target_tokens"].append(integers(s, f"ring{i}.target_tokens", 0, w.vocab - 1, (B, K + 1)))
    return {k: np.stack(v) for k, v in out.items()}


def prefill_inputs(w: Workload, S: int, lens, start, seed: int = None, kv: bool = True) -> dict:
    """Inputs of a drafting round that follows a prompt (or a chunk of one):
    per request a chunk of prompt tokens, its length n, the position c0 it
    starts at, the token after it, the target's hidden states of the chunk
    [B*L, d] (L = S-K+1 rows per request) and a block table covering
    c0+n+K-1 positions.  lens: ("fixed", n) or ("uniform", lo, hi) chunk
    lengths; start: ("fixed", c0) or ("uniform", lo, hi) start positions."""
    s = w.seed if seed is None else seed
    B, K, bs = w.batch, w.K, w.block_size
    L = S - K + 1

    def draw(spec, name):
        if spec[0] == "fixed":
            return np.full(B, int(spec[1]), dtype=np.int32)
        return integers(s, name, int(spec[1]), int(spec[2]) + 1, (B,))

    n = draw(lens, "prefill_lens")
    c0 = draw(start, "prefill_start")
    ct = integers(s, "prefill_tokens", 0, w.vocab - 1, (B, L))
    nt = integers(s, "prefill_new", 0, w.vocab - 1, (B,))
    need = (c0.astype(np.int64) + n + K - 1 + bs - 1) // bs
    nblocks = int(need.sum())
    max_blocks = int(need.max()) if B else 1
    g = np.random.Generator(np.random.PCG64(_key(s, "prefill_block_table")))
    perm = g.permutation(nblocks).astype(np.int32)
    bt = np.zeros((B, max_blocks), dtype=np.int32)
    off = 0
    for r in range(B):
        bt[r, :need[r]] = perm[off:off + need[r]]
        off += int(need[r])
    out = {
        "chunk_tokens": ct, "chunk_lens": n, "start_pos": c0, "new_tokens": nt,
        "block_table": bt, "num_kv_blocks": nblocks, "S": S,
        "target_hidden": normal(s, "prefill_hidden", (B * L, w.d), 1.0, dtype=w.dtype),
    }
    if kv:
        out["kv"] = kv_pool(w, nblocks, s)
    return out


def kv_pool(w: Workload, nblocks: int, seed: int) -> list:
    """Per layer: K cache [num_slots, Hkv, hd] and V cache
    [num_blocks, Hkv, hd, block_size] (V is stored d-major inside a block)."""
    bs, hkv, hd = w.block_size, w.n_kv_heads, w.head_dim
    pool = []
    for li in range(w.layers):
        kc = normal(seed, f"kcache{li}", (nblocks * bs, hkv, hd), 1.0, dtype=w.dtype)
        vc = normal(seed, f"vcache{li}", (nblocks, hkv, hd, bs), 1.0, dtype=w.dtype)
        pool.append((kc, vc))
    return pool
