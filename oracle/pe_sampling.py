"""Plain NumPy oracle of stochastic drafting and verification by rejection
sampling.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"vLLM Speculators: parallel drafting for speculative decoding", Production
integration (verification uses rejection sampling, so the output keeps the
verifier's distribution): the pages name the method and its guarantee only.  The steps below are the
standard speculative-sampling acceptance rule that carries that guarantee:

  drafts    t_j ~ q_j = softmax(z_j / T)            (the drafter's row j)
  accept    t_j while U_j < min(1, p_j(t_j) / q_j(t_j)),   p_j = softmax(y_j / T)
  on the first rejection at j: emit a sample of norm(max(0, p_j - q_j)), a' = j
  all accepted: emit a sample of p_K (the bonus), a' = K

Random numbers (the contract both sides implement from the published
definition): Philox4x32-10 ("Parallel random numbers: as easy as 1, 2, 3",
Salmon, Moraes, Dror, Shaw, SC 2011) with key (seed mod 2^32, seed >> 32)
and counter (c0, c1, 0, stream); an output word x gives
U = (floor(x / 512) + 1/2) / 2^23 in (0, 1), a lattice that float32 holds
exactly (so both sides draw the same U and 1 - U is never rounded to 0).
Per-token noise takes all four output words of a block: token v of a row
uses word v mod 4 of the block at c0 = v div 4 (the block function is the
costly part).  Streams:
  STREAM_DRAFT    counter (v div 4, i): Gumbel noise of draft row i = r*K + j, token v
  STREAM_ACCEPT   counter (j, r), word 0: the acceptance uniform of request r, draft j
  STREAM_RESIDUAL counter (v div 4, r): Gumbel noise of the token emitted for request r
A sample of a distribution w over the vocabulary is argmax_v(log w(v) + G_v)
with G = -log(-log U) (the Gumbel-max identity); ties go to the lowest index.
"""
import numpy as np

STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESIDUAL = 0, 1, 2

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32(counter, key, rounds=10):
    """Philox4x32 block function (Salmon et al. 2011).  counter: [..., 4],
    key: [..., 2] unsigned 32-bit values (broadcast); returns [..., 4] uint32.
    Each round multiplies words 0 and 2 by the two round multipliers, takes
    the high and low halves of the 64-bit products, XORs the high halves with
    the other two words and the round key, and permutes; the key is bumped by
    the two Weyl constants between rounds."""
    c = [np.asarray(counter, dtype=np.uint64)[..., i] & _MASK for i in range(4)]
    k0 = np.asarray(key, dtype=np.uint64)[..., 0] & _MASK
    k1 = np.asarray(key, dtype=np.uint64)[..., 1] & _MASK
    for rnd in range(rounds):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack([x.astype(np.uint32) for x in c], axis=-1)


def uniform(seed, stream, c0, c1, word=0):
    """U in (0, 1) from output word `word` of counter (c0, c1, 0, stream)
    under key `seed` (64-bit)."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.broadcast_to(np.asarray(c1, dtype=np.uint64), c0.shape)
    word = np.broadcast_to(np.asarray(word, dtype=np.int64), c0.shape)
    ctr = np.stack([c0, c1, np.zeros_like(c0), np.full_like(c0, stream)], axis=-1)
    key = np.array([int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    out = philox4x32(ctr, key)
    x = np.take_along_axis(out, word[..., None], axis=-1)[..., 0].astype(np.float64)
    return (np.floor(x / 512.0) + 0.5) / 2.0 ** 23


def token_uniforms(seed, stream, V, row):
    """U of tokens 0..V-1 of one row: word v mod 4 of block (v div 4, row)."""
    v = np.arange(V)
    return uniform(seed, stream, v // 4, row, v % 4)


def gumbel(u):
    return -np.log(-np.log(u))


def log_softmax(logits, T):
    z = np.asarray(logits, dtype=np.float64) / T
    m = z.max(axis=-1, keepdims=True)
    return z - m - np.log(np.exp(z - m).sum(axis=-1, keepdims=True))


def sample_drafts(draft_logits, T, seed):
    """Draft tokens t_i ~ softmax(z_i / T) for every draft row i (Gumbel-max
    with STREAM_DRAFT noise).  draft_logits [D, V] -> int32 [D]."""
    z = np.asarray(draft_logits, dtype=np.float64)
    D, V = z.shape
    out = np.zeros(D, np.int32)
    for i in range(D):
        g = gumbel(token_uniforms(seed, STREAM_DRAFT, V, i))
        out[i] = int(np.argmax(z[i] / T + g))
    return out


def rejection_verify(draft_tokens, draft_logits, target_logits, T, seed):
    """Verification by rejection sampling.  draft_tokens [B, K], draft_logits
    [B, K, V] (the drafter's rows t_1..t_K came from), target_logits [B, K+1, V]
    (the verifier's rows at the same K+1 positions).  Returns (accepted [B]:
    drafts kept, next_token [B]: the residual sample at the first rejection,
    or the bonus sample from the last target row)."""
    t = np.asarray(draft_tokens)
    B, K = t.shape
    V = np.asarray(target_logits).shape[-1]
    acc = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for r in range(B):
        lq = log_softmax(draft_logits[r], T)      # [K, V]
        lp = log_softmax(target_logits[r], T)     # [K+1, V]
        a = K
        for j in range(K):
            ratio = np.exp(lp[j, t[r, j]] - lq[j, t[r, j]])
            u = uniform(seed, STREAM_ACCEPT, j, r)
            if not u < min(1.0, ratio):
                a = j
                break
        g = gumbel(token_uniforms(seed, STREAM_RESIDUAL, V, r))
        if a < K:
            w = np.maximum(np.exp(lp[a]) - np.exp(lq[a]), 0.0)
            with np.errstate(divide="ignore"):
                score = np.log(w) + g
        else:
            score = lp[K] + g
        acc[r] = a
        nxt[r] = int(np.argmax(score))
    return acc, nxt
