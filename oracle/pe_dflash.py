"""Plain fp64 NumPy oracle of a DFlash-style drafting round: verifier hidden
states injected into the drafter's KV cache, then one block of MASK slots
drafted in a single pass.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: "vLLM Speculators: parallel drafting for speculative decoding",
comparison of P-EAGLE, DFlash and DSpark (DFlash): the verifier's hidden
states are projected and written straight into the drafter's KV cache, so the
drafter attends to the verifier's state without a longer input, and the
candidate tokens come from block diffusion.  The page gives no more than
that; the readings taken here:

  D1 injection   per drafter layer l, each context token c of the previous
                 verify batch that the verifier kept (j <= a) gets
                   k = RoPE(Wk_inj[l] h_c) at its position, v = Wv_inj[l] h_c
                 (h_c: the verifier's hidden state there; dedicated per-layer
                 weights [Hkv*hd, d], no norm) written to its paged KV slot;
                 rejected tokens (j > a) write nothing.
  D2 block       the block is [bonus, MASK x K] at positions p0+a+1 ..
                 p0+a+K+1; its input is the token embedding alone.
  D3 attention   block diffusion: every block slot sees the whole block and
                 the cached context, i.e. positions [0, p0+a+K+1]; the
                 block's own K/V are written to its slots first (the next
                 round's injection overwrites them).
  D4 drafts      one denoising step: the LM head on MASK slot i (i = 1..K)
                 gives the draft for that slot's own position; argmax, lowest
                 index on ties.
  The decoder layers are the drafter's (same weights and rounding points as
  pe_oracle.draft_forward: R2..R7); injected k and v are rounded once (R3).
"""
import numpy as np

from .pe_oracle import (PADDING_SLOT_ID, ERR_ACCEPTED, ERR_TOKEN, ERR_BLOCK, ERR_LAYOUT,
                        widen, _rounder, slot_of, rmsnorm, rope, silu, attend, _KV, _matmul_rows)


def dflash_prepare(verify_positions, num_accepted, bonus_tokens, block_table, num_kv_blocks, K,
                   vocab, mask_id, block_size):
    """Block batch (S = K+1 slots per request) and injection slots.

    Request r: p0 = vp[r, 0], a = num_accepted[r].
      injection row r(K+1)+j (j = 0..K): KV slot of position p0+j if j <= a,
                                         else PADDING_SLOT_ID (D1)
      block slot r(K+1)+i (i = 0..K):    token bonus (i = 0) or mask_id,
                                         position p0+a+1+i, attention horizon
                                         p0+a+K+1 (D3), its paged KV slot
      draft_rows: r(K+1)+1 .. r(K+1)+K (D4); seq_len = p0+a+K+2.
    Validation as prepare(): a outside [0, K], bonus outside [0, V), positions
    not p0..p0+K, p0 < 0 or a missing block for [0, seq_len) turn the request
    into padding (every slot rejected, positions 0, KV slots -1, seq_len 0).
    """
    vp = np.asarray(verify_positions, dtype=np.int64)
    acc = np.asarray(num_accepted, dtype=np.int64)
    bonus = np.asarray(bonus_tokens, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    B = acc.shape[0]
    S = K + 1
    n = B * S
    ids = np.zeros(n, np.int32)
    pos = np.zeros(n, np.int32)
    apos = np.zeros(n, np.int32)
    hsrc = np.full(n, -1, np.int32)
    rej = np.zeros(n, np.uint8)
    msk = np.zeros(n, np.uint8)
    slots = np.full(n, PADDING_SLOT_ID, np.int64)
    inj = np.full(n, PADDING_SLOT_ID, np.int64)
    draft_rows = np.zeros(B * K, np.int32)
    seq_lens = np.zeros(B, np.int32)
    err_kinds, err_first = 0, -1
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0
    for r in range(B):
        base = r * S
        a, p0 = int(acc[r]), int(vp[r, 0])
        kinds = 0
        if not 0 <= a <= K:
            kinds |= ERR_ACCEPTED
        elif not 0 <= int(bonus[r]) < vocab:
            kinds |= ERR_TOKEN
        if any(int(vp[r, j]) != p0 + j for j in range(K + 1)):
            kinds |= ERR_LAYOUT
        if p0 < 0:
            kinds |= ERR_BLOCK
        if kinds == 0:
            seq_len = p0 + a + K + 2
            nb = (seq_len + block_size - 1) // block_size
            if nb > max_blocks or any(not 0 <= int(bt[r, b]) < num_kv_blocks for b in range(nb)):
                kinds |= ERR_BLOCK
        if kinds:
            err_kinds |= kinds
            if err_first < 0:
                err_first = r
            rej[base:base + S] = 1
            draft_rows[r * K:(r + 1) * K] = base + 1 + np.arange(K)
            continue
        for j in range(a + 1):
            inj[base + j] = slot_of(bt[r], p0 + j, block_size)
        for i in range(S):
            s = base + i
            ids[s] = bonus[r] if i == 0 else mask_id
            msk[s] = 0 if i == 0 else 1
            pos[s] = p0 + a + 1 + i
            apos[s] = p0 + a + K + 1
            slots[s] = slot_of(bt[r], int(pos[s]), block_size)
        draft_rows[r * K:(r + 1) * K] = base + 1 + np.arange(K)
        seq_lens[r] = p0 + a + K + 2
    return {
        "input_ids": ids, "positions": pos, "hidden_src": hsrc, "is_rejected": rej,
        "is_masked": msk, "slot_mapping": slots, "draft_rows": draft_rows, "seq_lens": seq_lens,
        "attn_positions": apos, "inject_slots": inj,
        "error_kinds": err_kinds, "error_first": err_first,
    }


def dflash_inject(cfg, verify_positions, inject_slots, target_hidden, inject_weights, kv,
                  precision="bf16"):
    """Reading D1 for every layer.  inject_weights: per layer (Wk_inj, Wv_inj)
    storage arrays [Hkv*hd, d]; kv: per layer (K cache, V cache) storage
    arrays (V d-major inside each block, as the drafter's cache).

    Returns per layer (slot ids, k rows, v rows) as stored, in row order."""
    R = _rounder(precision)
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim
    pos = np.asarray(verify_positions, dtype=np.int64).reshape(-1)
    slots = np.asarray(inject_slots, dtype=np.int64).reshape(-1)
    h = widen(target_hidden)
    keep = np.nonzero(slots >= 0)[0]
    out = []
    for wk, wv in inject_weights:
        k = R(rope((h[keep] @ widen(wk).T).reshape(-1, Hkv, hd), pos[keep], cfg.rope_theta))
        v = R((h[keep] @ widen(wv).T).reshape(-1, Hkv, hd))
        out.append((slots[keep], k, v))
    return out


def apply_writes(kv, writes, block_size, dtype):
    """Copies of the caches with (slot, k, v) writes stored in the storage
    format (bf16 bits or float32); later writes to a slot win."""
    from .pe_oracle import round_bf16
    out = []
    for (kc, vc), (sl, k, v) in zip(kv, writes):
        kc, vc = kc.copy(), vc.copy()
        for i, s in enumerate(sl):
            s = int(s)
            kr, vr = k[i], v[i]
            if dtype == "bf16":
                kr = (round_bf16(kr).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
                vr = (round_bf16(vr).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            kc[s] = kr
            vc[s // block_size, :, :, s % block_size] = vr
        out.append((kc, vc))
    return out


def dflash_forward(params, cfg, batch, kv, block_table, precision="bf16", requests=None,
                   want_logits=True):
    """Readings D2-D4: one drafter pass over the K+1 block slots per request.

    Per layer (pre-norm, as pe_oracle.draft_forward): u = RMSNorm(x); q, k, v
    with RoPE at each slot's position; the block's KV writes land first; each
    slot attends to positions [0, attn_position] of its request (D3); x +=
    Wo o; x += Wd (silu(Wg u) * Wu u).  Then z = RMSNorm(x) on the MASK slots,
    logits = W_lm z, tokens = argmax.

    kv: per layer storage arrays holding the cached context (after the
    injection); not modified.  Returns tokens [len(requests)*K] (-1 for a
    padded request), logits (if want_logits), kv_writes per layer."""
    R = _rounder(precision)
    K, bs = cfg.K, cfg.block_size
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = Hq // Hkv
    S = K + 1
    B = len(batch["seq_lens"])
    reqs = list(range(B)) if requests is None else list(requests)
    rows = np.concatenate([np.arange(r * S, (r + 1) * S) for r in reqs]) if reqs else np.zeros(0, np.int64)
    n = rows.shape[0]
    ids = np.asarray(batch["input_ids"])[rows]
    pos = np.asarray(batch["positions"])[rows]
    apos = np.asarray(batch["attn_positions"])[rows]
    rej = np.asarray(batch["is_rejected"])[rows]
    slots = np.asarray(batch["slot_mapping"])[rows]
    seq_lens = np.asarray(batch["seq_lens"])
    bt = np.asarray(block_table)

    x = widen(np.asarray(params["embed"])[ids])
    writes = []
    for li, lw in enumerate(params["layers"]):
        cache = _KV(kv[li][0], kv[li][1], bs)
        u = R(rmsnorm(x, widen(lw["attn_norm"]), cfg.rms_eps))
        q = R(rope((u @ widen(lw["wq"]).T).reshape(n, Hq, hd), pos, cfg.rope_theta))
        k = R(rope((u @ widen(lw["wk"]).T).reshape(n, Hkv, hd), pos, cfg.rope_theta))
        v = R((u @ widen(lw["wv"]).T).reshape(n, Hkv, hd))
        wl = [i for i in range(n) if slots[i] >= 0]
        for i in wl:
            cache.write(int(slots[i]), k[i], v[i])
        writes.append((slots[wl].astype(np.int64), k[wl], v[wl]))
        o = np.zeros((n, Hq, hd))
        for ri, r in enumerate(reqs):
            L = int(seq_lens[r])
            if L == 0:
                continue
            kr, vr = cache.read(np.array([slot_of(bt[r], p, bs) for p in range(L)], np.int64))
            for j in range(S):
                i = ri * S + j
                if rej[i]:
                    continue
                top = int(apos[i]) + 1
                for hh in range(Hq):
                    o[i, hh] = attend(q[i, hh], kr[:top, hh // group], vr[:top, hh // group])
        o = R(o.reshape(n, Hq * hd))
        x = R(x + o @ widen(lw["wo"]).T)
        u = R(rmsnorm(x, widen(lw["mlp_norm"]), cfg.rms_eps))
        m = R(silu(u @ widen(lw["w_gate"]).T) * (u @ widen(lw["w_up"]).T))
        x = R(x + m @ widen(lw["w_down"]).T)

    dr = np.asarray(batch["draft_rows"]).reshape(B, K)
    local = {int(g): i for i, g in enumerate(rows)}
    drows = np.array([local[int(dr[r, m])] for r in reqs for m in range(K)], np.int64)
    z = R(rmsnorm(x[drows], widen(params["final_norm"]), cfg.rms_eps))
    logits = _matmul_rows(z, np.asarray(params["lm_head"]))
    tokens = np.argmax(logits, axis=1).astype(np.int32)
    for ri, r in enumerate(reqs):
        if seq_lens[r] == 0:
            tokens[ri * K:(ri + 1) * K] = -1
    out = {"tokens": tokens, "kv_writes": writes, "rows": rows, "x_final": x}
    if want_logits:
        out["logits"] = logits
    return out
