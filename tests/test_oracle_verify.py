"""Pins of the oracle's greedy verification: exhaustive brute force over small
alphabets, and a closed multi-round loop in which target tokens are planted so
that chosen accept counts happen."""
import itertools

import numpy as np
import pytest

import oracle as O
from drafting_pe_prepare_amd import configs, synth


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_verify_exhaustive_alphabet3(K):
    t = np.array(list(itertools.product(range(3), repeat=K)))
    g = np.array(list(itertools.product(range(3), repeat=K + 1)))
    T = np.repeat(t, len(g), axis=0)
    G = np.tile(g, (len(t), 1))
    acc, bon = O.verify(T, G)
    # brute force: the largest j whose prefix of length j matches entirely
    for i in range(len(T)):
        best = max(j for j in range(K + 1) if all(T[i, :j] == G[i, :j]))
        assert acc[i] == best
        assert bon[i] == G[i, best]
        assert 0 <= acc[i] <= K


def test_verify_all_match_gives_K_and_last_target():
    acc, bon = O.verify([[4, 5, 6]], [[4, 5, 6, 9]])
    assert acc[0] == 3 and bon[0] == 9


def test_closed_loop_rounds():
    """Rounds chained as in serving: the next verify batch is [bonus, t_1..t_K]
    at the positions after the accepted prefix; targets are planted so that a
    drawn accept count happens; every round's metadata, KV writes and verify
    result are checked against what the plant fixes."""
    w = configs.TINY.with_(d=64, mlp=128, vocab=256, n_q_heads=2, n_kv_heads=1,
                           dtype="bf16", weight_std=0.125, K=3, batch=2,
                           accepted="uniform", prefix=("fixed", 20, 0))
    prm = synth.weights(w)
    inp = synth.step_inputs(w)
    # block tables with room for several rounds
    bs, B, K = 16, w.batch, w.K
    nb = 8
    bt = np.arange(B * nb, dtype=np.int32).reshape(B, nb)[:, ::-1].copy()
    kv = synth.kv_pool(w, B * nb, 3)
    kv = [(kc.copy(), vc.copy()) for kc, vc in kv]
    vt, vp = inp["verify_tokens"], inp["verify_positions"]
    a, bonus = inp["num_accepted"], inp["bonus_tokens"]
    rng = np.random.default_rng(4)
    for rnd in range(5):
        H = synth.normal(50 + rnd, "H", (B * (K + 1), w.d))
        b = O.prepare(vt, vp, a, bonus, bt, B * nb, K, w.vocab, w.mask_id, bs)
        assert b["error_kinds"] == 0
        hd = O.gather_hidden(b["hidden_src"], H, prm["h_shared"])
        out = O.draft_forward(prm, w, b, hd, kv, bt, "bf16")
        # apply the KV writes, as the device cache would hold them
        slots, kr, vr = out["kv_writes"][0]
        kc, vc = kv[0]
        kc[slots] = synth.bf16_bits(kr.astype(np.float32))
        vc[slots // bs, :, :, slots % bs] = synth.bf16_bits(vr.astype(np.float32))
        t = out["tokens"].reshape(B, K)
        want = rng.integers(0, K + 1, size=B)
        g = rng.integers(0, w.vocab - 1, size=(B, K + 1)).astype(np.int32)
        for r in range(B):
            g[r, :want[r]] = t[r, :want[r]]
            if want[r] < K and g[r, want[r]] == t[r, want[r]]:
                g[r, want[r]] = (t[r, want[r]] + 1) % (w.vocab - 1)
        acc, bon = O.verify(t, g)
        np.testing.assert_array_equal(acc, want)
        np.testing.assert_array_equal(bon, g[np.arange(B), want])
        # next round
        p0 = vp[:, 0] + a + 1
        vt = np.concatenate([bonus[:, None], t], axis=1).astype(np.int32)
        vp = (p0[:, None] + np.arange(K + 1)[None, :]).astype(np.int32)
        a, bonus = acc, bon
        assert np.all(b["seq_lens"] == vp[:, 0] - 1 + K)
