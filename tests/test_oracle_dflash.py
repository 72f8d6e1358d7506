"""Pins of the DFlash-style round's oracle (oracle/pe_dflash.py).

Each pin rests on something other than the oracle's own code: a layout worked
out by hand, RoPE restated as a complex rotation, and the whole round written
as dense, unpaged masked attention over one contiguous sequence per request."""
import numpy as np

import oracle as O
from drafting_pe_prepare_amd import configs, synth

TINY = configs.TINY


def test_prepare_hand_worked():
    K, bs, V, M = 3, 4, 50, 49
    vp = np.array([[5, 6, 7, 8], [20, 21, 22, 23], [0, 1, 2, 3]], np.int32)
    a = np.array([1, 4, 3], np.int32)          # r1: a > K
    bonus = np.array([7, 9, 50], np.int32)     # r2: bonus == V
    bt = np.array([[2, 0, 5, 1, 1, 1, 1], [3, 3, 3, 3, 3, 3, 3], [4, 4, 4, 4, 4, 4, 4]], np.int32)
    out = O.dflash_prepare(vp, a, bonus, bt, 6, K, V, M, bs)
    S = K + 1
    # r0: context positions 5, 6 kept; block at 7..10 (block table 2, 0, 5)
    np.testing.assert_array_equal(out["inject_slots"][:S], [1, 2, -1, -1])
    np.testing.assert_array_equal(out["input_ids"][:S], [7, M, M, M])
    np.testing.assert_array_equal(out["positions"][:S], [7, 8, 9, 10])
    np.testing.assert_array_equal(out["attn_positions"][:S], [10, 10, 10, 10])
    np.testing.assert_array_equal(out["slot_mapping"][:S], [3, 20, 21, 22])
    np.testing.assert_array_equal(out["is_masked"][:S], [0, 1, 1, 1])
    np.testing.assert_array_equal(out["is_rejected"][:S], [0, 0, 0, 0])
    np.testing.assert_array_equal(out["draft_rows"], [1, 2, 3, 5, 6, 7, 9, 10, 11])
    np.testing.assert_array_equal(out["seq_lens"], [11, 0, 0])
    # r1, r2: padding
    for r in (1, 2):
        sl = slice(r * S, (r + 1) * S)
        assert (out["is_rejected"][sl] == 1).all()
        assert (out["slot_mapping"][sl] == -1).all() and (out["inject_slots"][sl] == -1).all()
    assert out["error_kinds"] == O.ERR_ACCEPTED | O.ERR_TOKEN and out["error_first"] == 1


def test_prepare_block_checks():
    K, bs = 2, 4
    vp = np.array([[4, 5, 6], [4, 5, 6], [4, 6, 7]], np.int32)
    a = np.array([2, 2, 0], np.int32)
    bonus = np.array([1, 1, 1], np.int32)
    # r0 needs [0, 4+2+2+2) = 10 positions -> 3 blocks, all present
    # r1: its third block is out of range; r2: positions not consecutive
    bt = np.array([[0, 1, 2], [0, 1, 9], [0, 1, 2]], np.int32)
    out = O.dflash_prepare(vp, a, bonus, bt, 3, K, 10, 9, bs)
    np.testing.assert_array_equal(out["seq_lens"], [10, 0, 0])
    np.testing.assert_array_equal(out["inject_slots"][:3], [4, 5, 6])
    np.testing.assert_array_equal(out["positions"][:3], [7, 8, 9])
    np.testing.assert_array_equal(out["slot_mapping"][:3], [7, 8, 9])
    assert out["error_kinds"] == O.ERR_BLOCK | O.ERR_LAYOUT and out["error_first"] == 1
    # one position short of the last block: bt with 2 columns
    out = O.dflash_prepare(vp[:1], a[:1], bonus[:1], bt[:1, :2], 3, K, 10, 9, bs)
    assert out["error_kinds"] == O.ERR_BLOCK


def test_inject_identity_projection_is_a_complex_rotation():
    w = TINY.with_(d=128, batch=2, K=3)
    hd, half = w.head_dim, w.head_dim // 2
    rng = np.random.default_rng(3)
    h = rng.standard_normal((2 * (w.K + 1), w.d)).astype(np.float32)
    vp = np.array([[9, 10, 11, 12], [0, 1, 2, 3]], np.int32)
    slots = np.array([5, 6, -1, -1, 40, 41, 42, 43], np.int64)
    eye = np.eye(w.d, dtype=np.float32)
    (sl, k, v), = O.dflash_inject(w, vp, slots, h, [(eye, eye)], None, precision="f64")
    keep = [0, 1, 4, 5, 6, 7]
    np.testing.assert_array_equal(sl, slots[keep])
    np.testing.assert_array_equal(v.reshape(len(keep), -1), h[keep].astype(np.float64))
    pos = vp.reshape(-1)[keep]
    hk = h[keep].astype(np.float64).reshape(len(keep), w.n_kv_heads, hd)
    z = hk[..., :half] + 1j * hk[..., half:]
    ang = pos[:, None, None] * w.rope_theta ** (-2.0 * np.arange(half) / hd)[None, None, :]
    z = z * np.exp(1j * ang)
    np.testing.assert_allclose(k, np.concatenate([z.real, z.imag], axis=-1), rtol=1e-12, atol=1e-12)


def _dense_round(prm, w, inj_w, inp):
    """The round for each request as one contiguous sequence: positions below
    p0 come from the cache pool (read through the block table), p0..p0+a from
    the injected projections, and the K+1 block positions from the block's own
    keys and values; every block query sees every position (no mask).
    float32 workloads only (the cache stores float32)."""
    K, Hq, Hkv, hd = w.K, w.n_q_heads, w.n_kv_heads, w.head_dim
    G, bs = Hq // Hkv, w.block_size
    f = O.widen
    logits = []
    for r in range(w.batch):
        p0, a = int(inp["verify_positions"][r, 0]), int(inp["num_accepted"][r])
        H = f(inp["target_hidden"])[r * (K + 1):r * (K + 1) + a + 1]
        ids = np.array([inp["bonus_tokens"][r]] + [w.mask_id] * K)
        bpos = p0 + a + 1 + np.arange(K + 1)
        x = f(prm["embed"])[ids]
        for li, lw in enumerate(prm["layers"]):
            kc, vc = inp["kv"][li]
            sl = np.array([int(inp["block_table"][r, p // bs]) * bs + p % bs for p in range(p0)], np.int64)
            k_pre = f(kc[sl]).reshape(p0, Hkv, hd)
            v_pre = f(vc[sl // bs, :, :, sl % bs]).reshape(p0, Hkv, hd)
            wk, wv = inj_w[li]
            k_inj = O.rope((H @ f(wk).T).reshape(-1, Hkv, hd), p0 + np.arange(a + 1), w.rope_theta)
            v_inj = (H @ f(wv).T).reshape(-1, Hkv, hd)
            # the injected rows are read back from the cache (float32 storage)
            k_inj, v_inj = (t.astype(np.float32).astype(np.float64) for t in (k_inj, v_inj))
            u = O.rmsnorm(x, f(lw["attn_norm"]), w.rms_eps)
            q = O.rope((u @ f(lw["wq"]).T).reshape(-1, Hq, hd), bpos, w.rope_theta)
            kb = O.rope((u @ f(lw["wk"]).T).reshape(-1, Hkv, hd), bpos, w.rope_theta)
            vb = (u @ f(lw["wv"]).T).reshape(-1, Hkv, hd)
            keys = np.concatenate([k_pre, k_inj, kb])          # [L, Hkv, hd]
            vals = np.concatenate([v_pre, v_inj, vb])
            kq = np.repeat(keys, G, axis=1)                    # [L, Hq, hd]
            vq = np.repeat(vals, G, axis=1)
            sc = np.einsum("shd,lhd->hsl", q, kq) / np.sqrt(hd)
            p = np.exp(sc - sc.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
            o = np.einsum("hsl,lhd->shd", p, vq).reshape(K + 1, Hq * hd)
            x = x + o @ f(lw["wo"]).T
            u = O.rmsnorm(x, f(lw["mlp_norm"]), w.rms_eps)
            x = x + O.silu(u @ f(lw["w_gate"]).T) * (u @ f(lw["w_up"]).T) @ f(lw["w_down"]).T
        z = O.rmsnorm(x[1:], f(prm["final_norm"]), w.rms_eps)
        logits.append(z @ f(prm["lm_head"]).T)
    return np.concatenate(logits)


def _oracle_round(prm, w, inj_w, inp, precision):
    prep = O.dflash_prepare(inp["verify_positions"], inp["num_accepted"], inp["bonus_tokens"],
                            inp["block_table"], inp["num_kv_blocks"], w.K, w.vocab, w.mask_id, w.block_size)
    writes = O.dflash_inject(w, inp["verify_positions"], prep["inject_slots"], inp["target_hidden"], inj_w,
                             inp["kv"], precision=precision)
    kv = O.apply_writes(inp["kv"], writes, w.block_size, w.dtype)
    return prep, writes, O.dflash_forward(prm, w, prep, kv, inp["block_table"], precision=precision)


def test_forward_matches_dense_sequence_round():
    w = TINY.with_(batch=3, K=3, layers=2, accepted="uniform", prefix=("uniform", 20, 40))
    prm = synth.weights(w)
    inj_w = synth.inject_weights(w)
    inp = synth.step_inputs(w, extra=2)
    inp["num_accepted"][:] = [0, 3, 1]
    _, _, out = _oracle_round(prm, w, inj_w, inp, "f64")
    want = _dense_round(prm, w, inj_w, inp)
    np.testing.assert_allclose(out["logits"], want, rtol=1e-9, atol=1e-9 * np.abs(want).max())
    np.testing.assert_array_equal(out["tokens"], np.argmax(want, axis=1))


def test_block_writes_and_padding():
    w = TINY.with_(batch=2, K=3, accepted="uniform")
    prm = synth.weights(w)
    inj_w = synth.inject_weights(w)
    inp = synth.step_inputs(w, extra=2)
    inp["num_accepted"][:] = [2, 7]        # request 1 becomes padding
    prep, writes, out = _oracle_round(prm, w, inj_w, inp, "f64")
    assert (out["tokens"][w.K:] == -1).all() and (out["tokens"][:w.K] >= 0).all()
    # injection: positions p0..p0+2 of request 0 only; block: its K+1 slots only
    assert len(writes[0][0]) == 3
    np.testing.assert_array_equal(out["kv_writes"][0][0], prep["slot_mapping"][:w.K + 1])
    assert prep["error_kinds"] == O.ERR_ACCEPTED and prep["error_first"] == 1
