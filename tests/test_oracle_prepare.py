"""Pins of the oracle's batch preparation and hidden-state gather against what
the pages fix: a hand-worked example, counting invariants, the uniqueness of
KV slots (the reason PADDING_SLOT_ID exists) and the error paths."""
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "prepare_k4_a2.txt")


def _golden():
    rows, extra = [], {}
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0].isdigit():
            rows.append([int(v) for v in parts])
        else:
            extra[parts[0]] = [int(v) for v in parts[1:]]
    return np.array(rows), extra


@pytest.mark.parametrize("case,col,bt", [
    ("identity", 6, [0, 1, 2, 3, 4, 5]),
    ("permuted", 7, [7, 3, 9, 2, 5, 8]),
])
def test_prepare_hand_worked_example(case, col, bt):
    g, extra = _golden()
    out = O.prepare([[100, 101, 102, 103, 104]], [[64, 65, 66, 67, 68]], [2], [555],
                    [bt], num_kv_blocks=10, K=4, vocab=1024, mask_id=1023, block_size=16)
    assert out["error_kinds"] == 0
    np.testing.assert_array_equal(out["input_ids"], g[:, 1])
    np.testing.assert_array_equal(out["positions"], g[:, 2])
    np.testing.assert_array_equal(out["hidden_src"], g[:, 3])
    np.testing.assert_array_equal(out["is_rejected"], g[:, 4])
    np.testing.assert_array_equal(out["is_masked"], g[:, 5])
    np.testing.assert_array_equal(out["slot_mapping"], g[:, col])
    np.testing.assert_array_equal(out["draft_rows"], extra["draft_rows"])
    np.testing.assert_array_equal(out["seq_lens"], extra["seq_len"])


def _random_case(rng, B, K, bs=16, vocab=50, mask_id=49):
    p0 = rng.integers(0, 300, size=B)
    a = rng.integers(0, K + 1, size=B)
    vt = rng.integers(0, vocab, size=(B, K + 1))
    vp = p0[:, None] + np.arange(K + 1)[None, :]
    bonus = rng.integers(0, vocab, size=B)
    need = (p0 + 2 * K + bs - 1) // bs
    perm = rng.permutation(int(need.sum()) + 5)
    bt = np.zeros((B, int(need.max())), np.int64)
    off = 0
    for r in range(B):
        bt[r, :need[r]] = perm[off:off + need[r]]
        off += need[r]
    return vt, vp, a, bonus, bt, len(perm)


@pytest.mark.parametrize("K", list(range(1, 16)))
def test_prepare_invariants_every_accept_count(K):
    """For every a in 0..K: K-1 masked, K-a rejected, a+K valid slots; every
    rejected slot maps to -1; valid positions are exactly [p0, p0+a+K), one
    slot each; the non-negative KV slots are pairwise distinct (positions of
    rejected and MASK slots coincide, so without -1 two slots would write one
    cache row); draft rows are the NTP slot then the MASK slots."""
    rng = np.random.default_rng(100 + K)
    bs, vocab, M = 16, 50, 49
    for a_fixed in range(K + 1):
        vt, vp, a, bonus, bt, nkv = _random_case(rng, 6, K, bs, vocab, M)
        a[:] = a_fixed
        vt[:, 1::2] = M            # real tokens equal to the MASK id
        out = O.prepare(vt, vp, a, bonus, bt, nkv, K, vocab, M, bs)
        assert out["error_kinds"] == 0
        S = 2 * K
        for r in range(6):
            sl = slice(r * S, (r + 1) * S)
            rej, msk = out["is_rejected"][sl], out["is_masked"][sl]
            slots, pos = out["slot_mapping"][sl], out["positions"][sl]
            assert msk.sum() == K - 1
            assert rej.sum() == K - a_fixed
            valid = (rej == 0)
            assert valid.sum() == a_fixed + K
            assert np.all(slots[rej == 1] == -1)
            assert np.all(slots[valid] >= 0)
            p0 = vp[r, 0]
            assert sorted(pos[valid].tolist()) == list(range(p0, p0 + a_fixed + K))
            assert out["seq_lens"][r] == p0 + a_fixed + K
            # masked slots are exactly the last K-1 slots, whatever the tokens
            np.testing.assert_array_equal(msk, [0] * (K + 1) + [1] * (K - 1))
            np.testing.assert_array_equal(out["input_ids"][sl][msk == 1], M)
            np.testing.assert_array_equal(out["hidden_src"][sl][msk == 1], -1)
            np.testing.assert_array_equal(out["hidden_src"][sl][:K + 1],
                                          r * (K + 1) + np.arange(K + 1))
            # the slot of a valid position is its paged address
            for s in np.nonzero(valid)[0]:
                p = pos[s]
                assert slots[s] == bt[r, p // bs] * bs + p % bs
            dr = out["draft_rows"][r * K:(r + 1) * K]
            assert dr[0] == r * S + a_fixed
            np.testing.assert_array_equal(dr[1:], r * S + K + np.arange(1, K))
            # token of slot j<a is the accepted draft d_{j+1}, slot a the bonus
            ids = out["input_ids"][sl]
            np.testing.assert_array_equal(ids[:a_fixed], vt[r, 1:a_fixed + 1])
            assert ids[a_fixed] == bonus[r]
        allslots = out["slot_mapping"][out["slot_mapping"] >= 0]
        assert len(np.unique(allslots)) == len(allslots)


def test_prepare_is_masked_from_role_not_token():
    out = O.prepare([[9, 9, 9, 9]], [[10, 11, 12, 13]], [3], [9], [[0, 1]],
                    2, K=3, vocab=10, mask_id=9, block_size=16)
    np.testing.assert_array_equal(out["input_ids"], [9, 9, 9, 9, 9, 9])
    np.testing.assert_array_equal(out["is_masked"], [0, 0, 0, 0, 1, 1])
    np.testing.assert_array_equal(out["is_rejected"], 0)


@pytest.mark.parametrize("mutate,kind", [
    (lambda c: c["a"].__setitem__(1, 5), O.ERR_ACCEPTED),
    (lambda c: c["a"].__setitem__(1, -1), O.ERR_ACCEPTED),
    (lambda c: c["bonus"].__setitem__(1, 50), O.ERR_TOKEN),
    (lambda c: (c["a"].__setitem__(1, 2), c["vt"].__setitem__((1, 2), -3)), O.ERR_TOKEN),
    (lambda c: c["bt"].__setitem__((1, 0), -1), O.ERR_BLOCK),
    (lambda c: c["bt"].__setitem__((1, 0), 10 ** 6), O.ERR_BLOCK),
    (lambda c: c["vp"].__setitem__((1, 3), 0), O.ERR_LAYOUT),
])
def test_prepare_error_requests_become_padding(mutate, kind):
    rng = np.random.default_rng(5)
    K = 4
    vt, vp, a, bonus, bt, nkv = _random_case(rng, 3, K)
    a[:] = 1
    c = {"vt": vt, "vp": vp, "a": a, "bonus": bonus, "bt": bt}
    mutate(c)
    out = O.prepare(vt, vp, a, bonus, bt, nkv, K, 50, 49, 16)
    assert out["error_kinds"] & kind
    assert out["error_first"] == 1
    S = 2 * K
    sl = slice(S, 2 * S)
    assert np.all(out["slot_mapping"][sl] == -1)
    assert np.all(out["is_rejected"][sl] == 1)
    assert out["seq_lens"][1] == 0
    # the other requests are untouched
    assert out["seq_lens"][0] > 0 and out["seq_lens"][2] > 0
    assert out["request_kinds"][0] == 0 and out["request_kinds"][2] == 0


def test_prepare_block_table_too_short():
    out = O.prepare([[1, 2, 3]], [[30, 31, 32]], [2], [4], [[0, 1]], 5, K=2,
                    vocab=10, mask_id=9, block_size=16)
    # seq_len 34 needs 3 blocks, the table has 2
    assert out["error_kinds"] == O.ERR_BLOCK and out["error_first"] == 0


def test_prepare_empty_batch():
    out = O.prepare(np.zeros((0, 5)), np.zeros((0, 5)), np.zeros(0), np.zeros(0),
                    np.zeros((0, 1)), 1, K=4, vocab=10, mask_id=9, block_size=16)
    assert out["input_ids"].shape == (0,) and out["draft_rows"].shape == (0,)
    assert out["error_kinds"] == 0


def test_gather_mask_rows_are_h_shared_and_copies_are_exact():
    rng = np.random.default_rng(1)
    K, B, d = 5, 3, 8
    vt, vp, a, bonus, bt, nkv = _random_case(rng, B, K)
    out = O.prepare(vt, vp, a, bonus, bt, nkv, K, 50, 49, 16)
    H = rng.integers(0, 65535, size=(B * (K + 1), d)).astype(np.uint16)
    hs = rng.integers(0, 65535, size=d).astype(np.uint16)
    Hd = O.gather_hidden(out["hidden_src"], H, hs)
    assert Hd.dtype == np.uint16
    for s, src in enumerate(out["hidden_src"]):
        if out["is_masked"][s]:
            np.testing.assert_array_equal(Hd[s], hs)
        else:
            np.testing.assert_array_equal(Hd[s], H[src])


def test_replay_ring_rounds_are_valid_inputs():
    """Every round of the pre-drawn ring the bench rotates through is a batch
    the preparation accepts with no error (accepted counts in 0..K, token ids
    in range), round 0 is the step's own draw, and the rounds differ."""
    from drafting_pe_prepare_amd import configs, synth
    for w in (configs.C1, configs.C64):
        inp = synth.step_inputs(w, kv=False)
        ring = synth.round_ring(w, inp, 32)
        B, K = w.batch, w.K
        assert ring["num_accepted"].shape == (32, B)
        assert ring["verify_tokens"].shape == (32, B, K + 1)
        np.testing.assert_array_equal(ring["num_accepted"][0], inp["num_accepted"])
        np.testing.assert_array_equal(ring["target_tokens"][0], inp["target_tokens"])
        assert len({tuple(r.tolist()) for r in ring["verify_tokens"].reshape(32, -1)}) == 32
        for i in (0, 1, 31):
            out = O.prepare(ring["verify_tokens"][i], inp["verify_positions"], ring["num_accepted"][i],
                            ring["bonus_tokens"][i], inp["block_table"], inp["num_kv_blocks"], K,
                            w.vocab, w.vocab - 1, w.block_size)
            assert out["error_kinds"] == 0
            assert np.all((ring["num_accepted"][i] >= 0) & (ring["num_accepted"][i] <= K))
