"""Plain fp64 NumPy oracle of the P-EAGLE parallel-draft step.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and literal on
purpose: loops over requests and slots, library matmuls for the dense steps,
no blocking, fusion or reordering.

Precision modes
---------------
"f64"  : fp64 arithmetic, nothing rounded.  Used against the fp32 GPU path.
"bf16" : fp64 arithmetic, and every value the GPU path *stores* as bfloat16 is
         rounded to the nearest bfloat16 (ties to even) at the same point:
           R1 fc output                       x = R(W_fc [E; Hd])
           R2 every RMSNorm output            u = R(rmsnorm(x))
           R3 q and k after RoPE, v           q = R(rope(Wq u)), v = R(Wv u)
                                              (one rounding: the projection is
                                              not rounded before RoPE)
           R4 attention output                o = R(softmax(q.K) V)
           R5 residual after the O proj       x = R(x + Wo o)
           R6 SiLU-and-mul, residual after    m = R(silu(Wg u) * (Wu u)),
              the down proj                   x = R(x + Wd m)
           R7 final RMSNorm output            z = R(rmsnorm(x))
         Logits are never rounded.  The pages state no precision at all; this
         list is the numerics contract both sides implement independently.
"""
import numpy as np

PAD_TOKEN = 0            # token id written into rejected slots
PADDING_SLOT_ID = -1     # KV slot id of a slot that must not write the cache

# device error kinds (bitmask), one request turns into padding on any of them
ERR_ACCEPTED = 1         # num_accepted outside [0, K]
ERR_TOKEN = 2            # an accepted draft or the bonus token outside [0, V)
ERR_BLOCK = 4            # p0 < 0, or a block needed for [0, seq_len) missing
ERR_LAYOUT = 8           # verify positions are not p0, p0+1, ..., p0+K


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def widen(a) -> np.ndarray:
    """Storage -> fp64.  uint16 arrays hold bfloat16 bit patterns (the high
    half of an IEEE float32); float arrays are taken as they are."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (8 significant bits,
    ties to even), returned as fp64.  Works on the fp64 bit pattern: keep the
    top 7 of the 52 stored mantissa bits, add half an ulp minus one plus the
    kept lsb, truncate.  A carry out of the mantissa bumps the exponent, which
    is the correct rounding.  bfloat16's exponent range equals float32's; the
    values met here are far from both ends of it."""
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    drop = np.uint64(45)
    lsb = (b >> drop) & np.uint64(1)
    b = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return b.view(np.float64).reshape(np.shape(x))


def _rounder(precision):
    if precision == "bf16":
        return round_bf16
    if precision == "f64":
        return lambda v: v
    raise ValueError(precision)


# ----------------------------------------------------------------------------
# (a) batch preparation
# ----------------------------------------------------------------------------
def slot_of(block_table_row, pos, block_size):
    """Paged KV slot of sequence position `pos`: block id * block_size + offset."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


def prepare(verify_tokens, verify_positions, num_accepted, bonus_tokens,
            block_table, num_kv_blocks, K, vocab, mask_id, block_size):
    """Draft-batch metadata for one round.

    Follows "P-EAGLE: parallel speculative decoding in vLLM", vLLM
    implementation details (Fused Triton kernel; KV cache), and Architecture
    and mechanism, Step 2 (Parallel Drafting).

    Each request r had a verify batch of K+1 tokens vt = [x0, d1..dK] at
    positions p0..p0+K; a drafts were accepted and the target then produced
    the bonus token.  The draft batch gives every request S = 2K slots at base
    r*S (readings: fixed stride; rejected slots stay in place and are masked):

      copied slots j = 0..K  position vp[j], hidden row r(K+1)+j (the target's
                             hidden state at that position, paired with the
                             embedding of the token one position later):
                               j <  a   token d_{j+1}      (accepted draft)
                               j == a   token bonus        (the NTP position)
                               j >  a   rejected: token PAD_TOKEN,
                                        KV slot PADDING_SLOT_ID
      MASK slots  m = 1..K-1 token mask_id, position p0+a+m (contiguous after
                             the NTP slot), hidden row -1 = h_shared

    Every slot that is not rejected maps to its paged KV slot.  draft_rows[r]
    lists the slots whose LM-head outputs are t_1..t_K: the NTP slot, then the
    MASK slots.  seq_len = p0+a+K = the cached prefix plus the valid slots.

    is_masked comes from the slot's role, never from its token: a real token
    may equal mask_id.

    A request whose inputs are out of range (kinds ERR_*) becomes padding:
    every slot rejected with token PAD_TOKEN, position 0, hidden row -1, KV
    slot -1; draft_rows r*S+i; seq_len 0.  The error word is the OR of the
    kinds and the lowest failing request index.
    """
    vt = np.asarray(verify_tokens, dtype=np.int64)
    vp = np.asarray(verify_positions, dtype=np.int64)
    acc = np.asarray(num_accepted, dtype=np.int64)
    bonus = np.asarray(bonus_tokens, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    B = acc.shape[0]
    S = 2 * K
    n = B * S
    ids = np.zeros(n, np.int32)
    pos = np.zeros(n, np.int32)
    hsrc = np.full(n, -1, np.int32)
    rej = np.zeros(n, np.uint8)
    msk = np.zeros(n, np.uint8)
    slots = np.full(n, PADDING_SLOT_ID, np.int64)
    draft_rows = np.zeros(B * K, np.int32)
    seq_lens = np.zeros(B, np.int32)
    err_kinds, err_first = 0, -1
    req_kinds = np.zeros(B, np.int32)
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0

    for r in range(B):
        base = r * S
        a = int(acc[r])
        p0 = int(vp[r, 0])
        kinds = 0
        if not 0 <= a <= K:
            kinds |= ERR_ACCEPTED
        else:
            for t in list(vt[r, 1:a + 1]) + [bonus[r]]:
                if not 0 <= int(t) < vocab:
                    kinds |= ERR_TOKEN
        if any(int(vp[r, j]) != p0 + j for j in range(K + 1)):
            kinds |= ERR_LAYOUT
        if p0 < 0:
            kinds |= ERR_BLOCK
        if kinds == 0:
            seq_len = p0 + a + K
            nb = (seq_len + block_size - 1) // block_size
            if nb > max_blocks:
                kinds |= ERR_BLOCK
            else:
                for b in range(nb):
                    if not 0 <= int(bt[r, b]) < num_kv_blocks:
                        kinds |= ERR_BLOCK
        req_kinds[r] = kinds
        if kinds:
            err_kinds |= kinds
            if err_first < 0:
                err_first = r
            rej[base:base + S] = 1
            for i in range(K):
                draft_rows[r * K + i] = base + i
            continue

        for j in range(K + 1):
            s = base + j
            pos[s] = vp[r, j]
            hsrc[s] = r * (K + 1) + j
            if j < a:
                ids[s] = vt[r, j + 1]
            elif j == a:
                ids[s] = bonus[r]
            else:
                ids[s] = PAD_TOKEN
                rej[s] = 1
            if not rej[s]:
                slots[s] = slot_of(bt[r], int(pos[s]), block_size)
        for m in range(1, K):
            s = base + K + m
            ids[s] = mask_id
            pos[s] = p0 + a + m
            hsrc[s] = -1
            msk[s] = 1
            slots[s] = slot_of(bt[r], int(pos[s]), block_size)
        draft_rows[r * K] = base + a
        for m in range(1, K):
            draft_rows[r * K + m] = base + K + m
        seq_lens[r] = p0 + a + K

    return {
        "input_ids": ids, "positions": pos, "hidden_src": hsrc,
        "is_rejected": rej, "is_masked": msk, "slot_mapping": slots,
        "draft_rows": draft_rows, "seq_lens": seq_lens,
        "error_kinds": err_kinds, "error_first": err_first,
        "request_kinds": req_kinds,
    }


def prepare_prefill(chunk_tokens, chunk_lens, start_pos, new_tokens, block_table,
                    num_kv_blocks, K, S, vocab, mask_id, block_size):
    """Draft-batch metadata for the drafting round that follows a prompt.

    Follows "P-EAGLE: parallel speculative decoding in vLLM", Architecture and
    mechanism: Step 1 (Prefilling: the target returns a hidden state for every
    prompt position and one new token) and Step 2 (Parallel Drafting: a prompt
    position pairs the target's hidden state there with the embedding of the
    token one position later; the NTP position pairs the new token with the
    last hidden state; positions 2..K take the MASK embedding and h_shared).

    Request r covers prompt positions c0..c0+n-1 in this call (c0 =
    start_pos[r], n = chunk_lens[r]); positions below c0 were drafted by
    earlier calls and are in the KV cache.  chunk_tokens[r, j] is the prompt
    token at position c0+j; new_tokens[r] is the token after the chunk (the
    target's new token when the chunk ends the prompt, else the next prompt
    token: an earlier chunk is the same call with its drafts ignored, whose
    MASK-slot KV the next chunk overwrites).  Readings: the batch has a fixed
    stride of S slots per request, L = S-K+1 >= n; hidden rows of the chunk
    are target_hidden[r*L + j]:

      copied slots j = 0..n-1    position c0+j, hidden row r*L+j, token
                                 chunk_tokens[r, j+1] (j < n-1) or
                                 new_tokens[r] (j = n-1: the NTP position)
      MASK slots   j = n..n+K-2  token mask_id, position c0+j, hidden -1
      padding      j >= n+K-1    rejected: token PAD_TOKEN, position 0,
                                 hidden -1, KV slot PADDING_SLOT_ID

    draft_rows[r] = r*S+n-1 .. r*S+n+K-2 (NTP, then MASK slots);
    seq_len = c0+n+K-1.  A request with n outside [1, L] (ERR_ACCEPTED), a
    token it reads outside [0, V) (ERR_TOKEN), c0 < 0 or a block of
    [0, seq_len) missing (ERR_BLOCK) becomes padding as in prepare().
    """
    ct = np.asarray(chunk_tokens, dtype=np.int64)
    nl = np.asarray(chunk_lens, dtype=np.int64)
    c0s = np.asarray(start_pos, dtype=np.int64)
    nt = np.asarray(new_tokens, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    B = nl.shape[0]
    L = S - K + 1
    n_all = B * S
    ids = np.zeros(n_all, np.int32)
    pos = np.zeros(n_all, np.int32)
    hsrc = np.full(n_all, -1, np.int32)
    rej = np.zeros(n_all, np.uint8)
    msk = np.zeros(n_all, np.uint8)
    slots = np.full(n_all, PADDING_SLOT_ID, np.int64)
    draft_rows = np.zeros(B * K, np.int32)
    seq_lens = np.zeros(B, np.int32)
    err_kinds, err_first = 0, -1
    req_kinds = np.zeros(B, np.int32)
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0

    for r in range(B):
        base = r * S
        n = int(nl[r])
        c0 = int(c0s[r])
        kinds = 0
        if not 1 <= n <= L:
            kinds |= ERR_ACCEPTED
        else:
            for t in list(ct[r, 1:n]) + [nt[r]]:
                if not 0 <= int(t) < vocab:
                    kinds |= ERR_TOKEN
        if c0 < 0:
            kinds |= ERR_BLOCK
        if kinds == 0:
            seq_len = c0 + n + K - 1
            nb = (seq_len + block_size - 1) // block_size
            if nb > max_blocks:
                kinds |= ERR_BLOCK
            else:
                for b in range(nb):
                    if not 0 <= int(bt[r, b]) < num_kv_blocks:
                        kinds |= ERR_BLOCK
        req_kinds[r] = kinds
        rej[base:base + S] = 1
        if kinds:
            err_kinds |= kinds
            if err_first < 0:
                err_first = r
            for i in range(K):
                draft_rows[r * K + i] = base + i
            continue

        for j in range(n + K - 1):
            s = base + j
            rej[s] = 0
            pos[s] = c0 + j
            if j < n:
                hsrc[s] = r * L + j
                ids[s] = ct[r, j + 1] if j < n - 1 else nt[r]
            else:
                ids[s] = mask_id
                msk[s] = 1
            slots[s] = slot_of(bt[r], int(pos[s]), block_size)
        for i in range(K):
            draft_rows[r * K + i] = base + n - 1 + i
        seq_lens[r] = c0 + n + K - 1

    return {
        "input_ids": ids, "positions": pos, "hidden_src": hsrc,
        "is_rejected": rej, "is_masked": msk, "slot_mapping": slots,
        "draft_rows": draft_rows, "seq_lens": seq_lens,
        "error_kinds": err_kinds, "error_first": err_first,
        "request_kinds": req_kinds,
    }


# ----------------------------------------------------------------------------
# (b) hidden-state gather
# ----------------------------------------------------------------------------
def gather_hidden(hidden_src, target_hidden, h_shared):
    """Row s of the draft hidden states is target_hidden[hidden_src[s]] when
    hidden_src[s] >= 0 and h_shared otherwise.  A pure copy, bit for bit, in
    whatever storage format the rows have.

    "P-EAGLE: parallel speculative decoding in vLLM", vLLM implementation
    details (Hidden-state management): target hidden states move to their new
    slots and the learned placeholder is broadcast into the MASK slots;
    Architecture and mechanism, Step 2 (MTP positions use the shared hidden
    state h_shared)."""
    src = np.asarray(hidden_src)
    th = np.asarray(target_hidden)
    out = np.empty((src.shape[0], th.shape[1]), dtype=th.dtype)
    for s in range(src.shape[0]):
        out[s] = th[src[s]] if src[s] >= 0 else np.asarray(h_shared)
    return out


# ----------------------------------------------------------------------------
# (c) drafter forward
# ----------------------------------------------------------------------------
def rmsnorm(x, gain, eps):
    """x / sqrt(mean(x^2) + eps) * gain, per row (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope(x, positions, theta):
    """Rotary position embedding, rotate-half pairing: within each head of
    size hd, dimension i < hd/2 pairs with i + hd/2 and the pair turns by the
    angle position * theta^(-2i/hd).  x: [rows, heads, hd]."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def attend(q, keys, values):
    """Scaled dot-product attention of one query head over a context.
    q: [hd]; keys, values: [T, hd].  softmax(keys.q / sqrt(hd)) . values."""
    sc = keys @ q / np.sqrt(q.shape[-1])
    p = np.exp(sc - sc.max())
    p /= p.sum()
    return p @ values


def _matmul_rows(x, w_storage, chunk=32768):
    """x [n, k] fp64 times w [m, k]^T with w converted chunk by chunk."""
    m = w_storage.shape[0]
    out = np.empty((x.shape[0], m), dtype=np.float64)
    for lo in range(0, m, chunk):
        out[:, lo:lo + chunk] = x @ widen(w_storage[lo:lo + chunk]).T
    return out


class _KV:
    """One layer's paged cache: K [num_slots, Hkv, hd] and V stored d-major
    inside each block, [num_blocks, Hkv, hd, block_size].  Reads go to the
    storage arrays; writes of this step go to an overlay (slot -> row)."""

    def __init__(self, kc, vc, block_size):
        self.kc, self.vc, self.bs = kc, vc, block_size
        self.k_new, self.v_new = {}, {}

    def write(self, slot, k, v):
        self.k_new[slot] = k
        self.v_new[slot] = v

    def read(self, slots):
        k = widen(self.kc[slots])
        v = widen(self.vc[slots // self.bs, :, :, slots % self.bs])
        for i, s in enumerate(slots):
            s = int(s)
            if s in self.k_new:
                k[i] = self.k_new[s]
                v[i] = self.v_new[s]
        return k, v


def draft_forward(params, cfg, batch, draft_hidden, kv, block_table,
                  precision="bf16", requests=None, want_logits=True):
    """One drafter forward over every slot of the draft batch.

    "P-EAGLE: parallel speculative decoding in vLLM", Architecture and
    mechanism, Step 2: each position's input combines a token embedding and a
    hidden state; all positions pass through the N-layer Transformer and the
    LM head, which predicts t_1..t_K at once.  vLLM implementation details
    (KV cache): slots mapped to -1 make no cache write.

    Readings (the pages name only "N-layer Transformer + LM head"):
      x = W_fc [emb(token); hidden]      no bias, no norm before fc
      per layer, pre-norm:
        u = RMSNorm(x); q, k, v = Wq u, Wk u, Wv u; RoPE on q and k at the
        slot's position; every KV write of the layer lands before any read;
        each non-rejected slot attends causally to positions [0, position]
        of its request through the block table (GQA, scale 1/sqrt(hd));
        x += Wo o; u = RMSNorm(x); x += Wd (silu(Wg u) * Wu u)
      z = RMSNorm(x) on the draft rows; logits = W_lm z; token = argmax,
      lowest index on ties.

    params: storage arrays as drawn (uint16 = bf16 bits, or float32).
    batch: from prepare() (S = 2K slots per request) or prepare_prefill()
    (any fixed S); the slot count per request is read from its size.
    kv: per layer (K cache, V cache) storage arrays; they are not modified.
    requests: subset of request indices to compute (rows are independent
    apart from attention, which stays inside one request).

    Returns dict: tokens [len(requests)*K] (int32, -1 for padded requests),
    logits [len(requests)*K, V] fp64 (if want_logits), kv_writes: per layer
    (slot ids, k rows, v rows) as stored, rows: the draft rows computed,
    x_final: the residual stream [rows, d] after the last layer.
    """
    R = _rounder(precision)
    K = cfg.K
    bs = cfg.block_size
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = Hq // Hkv
    B = len(batch["seq_lens"])
    S = len(batch["input_ids"]) // B if B else 2 * K  # slots per request (2K per decode round)
    reqs = list(range(B)) if requests is None else list(requests)
    rows = np.concatenate([np.arange(r * S, (r + 1) * S) for r in reqs]) if reqs else np.zeros(0, np.int64)
    n = rows.shape[0]
    ids = np.asarray(batch["input_ids"])[rows]
    pos = np.asarray(batch["positions"])[rows]
    rej = np.asarray(batch["is_rejected"])[rows]
    slots = np.asarray(batch["slot_mapping"])[rows]
    seq_lens = np.asarray(batch["seq_lens"])
    bt = np.asarray(block_table)

    emb = widen(np.asarray(params["embed"])[ids])
    hid = widen(np.asarray(draft_hidden)[rows])
    x = R(np.concatenate([emb, hid], axis=1) @ widen(params["w_fc"]).T)

    writes = []
    for li, lw in enumerate(params["layers"]):
        cache = _KV(kv[li][0], kv[li][1], bs)
        u = R(rmsnorm(x, widen(lw["attn_norm"]), cfg.rms_eps))
        q = (u @ widen(lw["wq"]).T).reshape(n, Hq, hd)
        k = (u @ widen(lw["wk"]).T).reshape(n, Hkv, hd)
        v = R((u @ widen(lw["wv"]).T).reshape(n, Hkv, hd))
        q = R(rope(q, pos, cfg.rope_theta))
        k = R(rope(k, pos, cfg.rope_theta))
        # all writes of the layer first
        w_slots, w_k, w_v = [], [], []
        for i in range(n):
            if slots[i] >= 0:
                cache.write(int(slots[i]), k[i], v[i])
                w_slots.append(int(slots[i]))
                w_k.append(k[i])
                w_v.append(v[i])
        writes.append((np.asarray(w_slots, np.int64),
                       np.asarray(w_k).reshape(-1, Hkv, hd),
                       np.asarray(w_v).reshape(-1, Hkv, hd)))
        # then the reads
        o = np.zeros((n, Hq, hd))
        for ri, r in enumerate(reqs):
            L = int(seq_lens[r])
            if L == 0:
                continue
            ctx_slots = np.array([slot_of(bt[r], p, bs) for p in range(L)], np.int64)
            kr, vr = cache.read(ctx_slots)
            for j in range(S):
                i = ri * S + j
                if rej[i]:
                    continue
                p = int(pos[i])
                for h in range(Hq):
                    g = h // group
                    o[i, h] = attend(q[i, h], kr[:p + 1, g], vr[:p + 1, g])
        o = R(o.reshape(n, Hq * hd))
        x = R(x + o @ widen(lw["wo"]).T)
        u = R(rmsnorm(x, widen(lw["mlp_norm"]), cfg.rms_eps))
        m = R(silu(u @ widen(lw["w_gate"]).T) * (u @ widen(lw["w_up"]).T))
        x = R(x + m @ widen(lw["w_down"]).T)

    # draft rows of the computed requests, in request order
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


# ----------------------------------------------------------------------------
# (d) greedy verification
# ----------------------------------------------------------------------------
def verify(draft_tokens, target_tokens):
    """Accepted length and bonus token per request.

    a' = the first j in 0..K-1 where the draft t_{j+1} differs from the
    target's token g_j, or K when all K drafts match; bonus' = g_{a'}.  The
    verifier accepts the longest matching prefix of the drafts ("AWS and vLLM
    ship P-EAGLE", Integration and numbers: acceptance length counts the drafts
    the verifier accepts per round; "P-EAGLE: parallel speculative decoding in
    vLLM", Benchmarks, Acceptance length).  Greedy: exact token equality."""
    t = np.asarray(draft_tokens)
    g = np.asarray(target_tokens)
    B, K = t.shape
    acc = np.zeros(B, np.int32)
    bon = np.zeros(B, np.int32)
    for r in range(B):
        j = 0
        while j < K and t[r, j] == g[r, j]:
            j += 1
        acc[r] = j
        bon[r] = g[r, j]
    return acc, bon


# ----------------------------------------------------------------------------
# an ordinary autoregressive EAGLE step, written independently of the slot
# layout, for the K=1 and causality pins
# ----------------------------------------------------------------------------
def eagle_step(params, cfg, prefix_k, prefix_v, tokens, hiddens, start_pos,
               precision="bf16", return_hidden=False):
    """One request, token by token: input i pairs emb(tokens[i]) with
    hiddens[i] at position start_pos+i, appended after a contiguous cached
    prefix (prefix_k/prefix_v per layer: [p0, Hkv, hd] fp64, p0 = start_pos).
    Each token runs every layer, appends its K/V and attends to everything
    cached so far.  Returns the logits of every input token [n, V] (and, with
    return_hidden, the residual stream after the last layer [n, d] and the
    per-layer caches grown by the new tokens).

    This is EAGLE drafting as "P-EAGLE: parallel speculative decoding in vLLM"
    describes it before the parallel change (Solving the autoregressive
    drafting bottleneck): one drafter pass per position."""
    R = _rounder(precision)
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = Hq // Hkv
    caches = [[list(np.asarray(prefix_k[li])), list(np.asarray(prefix_v[li]))]
              for li in range(len(params["layers"]))]
    wfc = widen(params["w_fc"])
    out, xs = [], []
    for i, (tok, h) in enumerate(zip(tokens, hiddens)):
        p = start_pos + i
        inp = np.concatenate([widen(np.asarray(params["embed"])[int(tok)]), widen(h)])
        x = R(wfc @ inp)
        for li, lw in enumerate(params["layers"]):
            u = R(rmsnorm(x[None], widen(lw["attn_norm"]), cfg.rms_eps)[0])
            q = R(rope((widen(lw["wq"]) @ u).reshape(1, Hq, hd), [p], cfg.rope_theta)[0])
            k = R(rope((widen(lw["wk"]) @ u).reshape(1, Hkv, hd), [p], cfg.rope_theta)[0])
            v = R((widen(lw["wv"]) @ u).reshape(Hkv, hd))
            kc, vc = caches[li]
            assert len(kc) == p, "cache length must equal the position"
            kc.append(k)
            vc.append(v)
            ka, va = np.asarray(kc), np.asarray(vc)
            o = np.stack([attend(q[hh], ka[:, hh // group], va[:, hh // group])
                          for hh in range(Hq)])
            o = R(o.reshape(-1))
            x = R(x + widen(lw["wo"]) @ o)
            u = R(rmsnorm(x[None], widen(lw["mlp_norm"]), cfg.rms_eps)[0])
            m = R(silu(widen(lw["w_gate"]) @ u) * (widen(lw["w_up"]) @ u))
            x = R(x + widen(lw["w_down"]) @ m)
        xs.append(x)
        z = R(rmsnorm(x[None], widen(params["final_norm"]), cfg.rms_eps))
        out.append(_matmul_rows(z, np.asarray(params["lm_head"]))[0])
    if return_hidden:
        return np.asarray(out), np.asarray(xs), caches
    return np.asarray(out)


def ar_draft(params, cfg, prefix_k, prefix_v, accepted_tokens, bonus, hiddens, start_pos,
             precision="bf16", return_state=False):
    """Autoregressive EAGLE drafting of K tokens for one request: the first
    pass runs over the accepted drafts and the bonus token (paired with the
    target's hidden states); every later pass feeds back the token it just
    drafted together with the drafter's own output hidden state (the residual
    stream after the last layer) of the previous position.  This is the
    sequential baseline of "P-EAGLE: parallel speculative decoding in vLLM",
    Solving the autoregressive drafting bottleneck (K drafts need K passes).
    Returns (tokens [K], logits [K, V]), and with return_state also the
    hidden states fed into passes 2..K [K-1, d] and the per-layer K/V of
    positions 0..start_pos+len(accepted)+K-1 (lists of [Hkv, hd] rows)."""
    toks = list(accepted_tokens) + [bonus]
    lg, xs, caches = eagle_step(params, cfg, prefix_k, prefix_v, toks, hiddens, start_pos,
                                precision, return_hidden=True)
    out_t, out_l = [int(np.argmax(lg[-1]))], [lg[-1]]
    h = xs[-1]
    fed = []
    pos = start_pos + len(toks)
    for _ in range(1, cfg.K):
        fed.append(h)
        ks = [np.asarray(c[0]) for c in caches]
        vs = [np.asarray(c[1]) for c in caches]
        lg, xs, caches = eagle_step(params, cfg, ks, vs, [out_t[-1]], [h], pos, precision,
                                    return_hidden=True)
        out_t.append(int(np.argmax(lg[-1])))
        out_l.append(lg[-1])
        h = xs[-1]
        pos += 1
    if return_state:
        return (np.asarray(out_t, np.int32), np.asarray(out_l),
                np.asarray(fed).reshape(-1, cfg.d), caches)
    return np.asarray(out_t, np.int32), np.asarray(out_l)


# ----------------------------------------------------------------------------
# draft depth selection
# ----------------------------------------------------------------------------
def expected_tokens(K, alpha):
    """Tokens a round emits when each draft is kept with probability alpha
    given that every earlier one was (reading: the pages give no acceptance
    model): sum_{i=0..K} alpha^i -- the kept prefix plus the emitted token."""
    return float(sum(alpha ** i for i in range(K + 1)))


def choose_depth(Ks, draft_us, alpha, verify_fixed_us, verify_per_token_us):
    """The depth with the most tokens per microsecond ("P-EAGLE: parallel
    speculative decoding in vLLM", Speculative depth efficiency: throughput
    peaks at the depth where the extra accepted tokens stop paying for the
    deeper draft; "vLLM Speculators: parallel drafting for speculative
    decoding", Limits of autoregressive drafting: K is tuned to the drafting
    cost).  A round at depth K costs draft_us + verify_fixed_us +
    verify_per_token_us * (K + 1).  Ties go to the smaller K.
    Returns (K, tokens per microsecond)."""
    best, best_rate = None, -1.0
    for K, t in sorted(zip(Ks, draft_us)):
        rate = expected_tokens(K, alpha) / (t + verify_fixed_us + verify_per_token_us * (K + 1))
        if rate > best_rate:
            best, best_rate = K, rate
    return best, best_rate
