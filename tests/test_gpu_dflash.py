"""GPU parity of the DFlash-style round (pe_dflash_prepare, pe_dflash_inject,
pe_dflash_forward) against the oracle's dflash_prepare, dflash_inject and
dflash_forward on the same seeded inputs: block batch, attention horizons and
injection slots bit for bit; injected and block K/V rows within two bf16 ulps
(1e-5 relative in fp32) at exactly the oracle's slots and nowhere else;
tokens and logits within the one-pass bound (2e-2 x RMS in bf16 per
sqrt(layer), 1e-4 in fp32).  Each side injects with its own arithmetic and
drafts from its own caches."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from drafting_pe_prepare_amd import configs, synth
from drafting_pe_prepare_amd import binding as pb

from pe_gpu import Setup, assert_kv, assert_metadata_equal, assert_tokens_logits, logit_tol, oracle_precision

pytestmark = pytest.mark.gpu

SMALL_BF16 = configs.TINY.with_(dtype="bf16", d=256, mlp=1024, vocab=1024, weight_std=1 / 16)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pb.load()


def run_dflash(st, inj_w, inp):
    w = st.w
    B, K = w.batch, w.K
    t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
         ("verify_positions", "num_accepted", "bonus_tokens", "block_table", "target_hidden")}
    kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
    wk = [pb.to_device(a) for a, _ in inj_w]
    wv = [pb.to_device(b) for _, b in inj_w]
    nkv = int(inp["num_kv_blocks"])
    batch = pb.Batch(B, K, S=K + 1)
    apos = torch.full((B * (K + 1),), -7, dtype=torch.int32, device="cuda")
    inj = torch.full((B * (K + 1),), -7, dtype=torch.int64, device="cuda")
    pb.pe_dflash_prepare(st.ctx, B, t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                         t["block_table"], nkv, batch, apos, inj)
    pb.pe_dflash_inject(st.ctx, B, t["verify_positions"], inj, t["target_hidden"], wk, wv, nkv,
                        [k for k, _ in kv], [v for _, v in kv])
    torch.cuda.synchronize()
    kv_inj = [(pb.to_host(k), pb.to_host(v)) for k, v in kv]
    tok = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros((B * K, w.vocab), dtype=torch.float32, device="cuda")
    pb.pe_dflash_forward(st.ctx, B, batch, apos, t["block_table"], nkv, [k for k, _ in kv], [v for _, v in kv],
                         tok, lg)
    torch.cuda.synchronize()
    return {
        "batch": batch.host(B, K), "attn_positions": apos.cpu().numpy(), "inject_slots": inj.cpu().numpy(),
        "kv_inj": kv_inj, "kv": [(pb.to_host(k), pb.to_host(v)) for k, v in kv],
        "tokens": tok.cpu().numpy(), "logits": lg.cpu().numpy(), "error": pb.pe_get_device_error(st.ctx),
    }


def _check(w, seed, bad=None, requests=None):
    _say(f"dflash case {w.name} B={w.batch} K={w.K} d={w.d} dtype={w.dtype} seed={seed} bad={bad} "
         f"requests={requests}")
    st = Setup(w, seed)
    try:
        inj_w = synth.inject_weights(w, seed)
        inp = synth.step_inputs(w, seed, extra=2)
        if bad is not None:
            inp["num_accepted"][bad] = w.K + 1
        g = run_dflash(st, inj_w, inp)
        prec = oracle_precision(w)
        ob = O.dflash_prepare(inp["verify_positions"], inp["num_accepted"], inp["bonus_tokens"],
                              inp["block_table"], inp["num_kv_blocks"], w.K, w.vocab, w.mask_id, w.block_size)
        assert_metadata_equal(g["batch"], ob)
        np.testing.assert_array_equal(g["attn_positions"], ob["attn_positions"])
        np.testing.assert_array_equal(g["inject_slots"], ob["inject_slots"])
        assert g["error"] == ((0, -1) if bad is None else (O.ERR_ACCEPTED, bad))
        writes = O.dflash_inject(w, inp["verify_positions"], ob["inject_slots"], inp["target_hidden"], inj_w,
                                 inp["kv"], precision=prec)
        assert_kv(w, g["kv_inj"], inp, {"kv_writes": writes})
        kv_o = O.apply_writes(inp["kv"], writes, w.block_size, w.dtype)
        fw = O.dflash_forward(st.prm, w, ob, kv_o, inp["block_table"], precision=prec, requests=requests)
        K = w.K
        reqs = list(range(w.batch)) if requests is None else list(requests)
        good = [i for i, r in enumerate(reqs) if r != bad]
        rows = np.concatenate([np.arange(r * K, (r + 1) * K) for r in reqs])
        orows = np.concatenate([np.arange(i * K, (i + 1) * K) for i in good])
        grows = rows.reshape(-1, K)[good].reshape(-1)
        tight = assert_tokens_logits(g["tokens"], g["logits"], fw["logits"][orows], logit_tol(w), grows)
        if bad is not None:
            assert np.all(g["tokens"][bad * K:(bad + 1) * K] == -1)
        # the block's own K/V: at its slots only (for the requests computed)
        assert_kv(w, g["kv"], {"kv": g["kv_inj"]}, _block_writes(w, fw, ob, requests, g))
        return tight
    finally:
        st.close()


def _block_writes(w, fw, ob, requests, g):
    """Oracle block writes of the computed requests, plus (for requests not
    computed) the GPU's own rows at their block slots, so that the off-slot
    comparison covers the whole cache."""
    if requests is None:
        return fw
    out = []
    S = w.K + 1
    others = [r for r in range(w.batch) if r not in set(requests)]
    oth = np.concatenate([ob["slot_mapping"][r * S:(r + 1) * S] for r in others]) if others else np.zeros(0, np.int64)
    oth = oth[oth >= 0]
    bs = w.block_size
    for li, (sl, k, v) in enumerate(fw["kv_writes"]):
        kc, vc = g["kv"][li]
        gk = O.widen(kc[oth])
        gv = O.widen(vc[oth // bs, :, :, oth % bs])
        out.append((np.concatenate([sl, oth]), np.concatenate([k, gk]), np.concatenate([v, gv])))
    return {"kv_writes": out}


def test_dflash_tiny_f32():
    _check(configs.TINY.with_(batch=3, K=4, accepted="uniform"), seed=71, bad=1)


@pytest.mark.parametrize("K,B,seed", [(3, 4, 72), (1, 2, 73), (7, 3, 74)])
def test_dflash_small_bf16(K, B, seed):
    _check(SMALL_BF16.with_(K=K, batch=B, accepted="uniform"), seed=seed, bad=B - 1 if K == 3 else None)


def test_dflash_c1_shape_bf16():
    _check(configs.C1.with_(batch=2), seed=75)


def test_dflash_c64_shape_bf16_sampled_requests():
    _check(configs.C64, seed=76, requests=[0, 29, 63])


def test_dflash_argument_errors_and_empty_batch():
    """Host-side checks fail before any launch; B = 0 is a no-op; a block
    table that covers p0 + 2K positions but not the block's last two turns
    requests with a = K into padding (device error word, kind 4)."""
    w = SMALL_BF16.with_(K=3, batch=2, accepted="3", prefix=("fixed", 58, 0))  # p0 + 2K = 64: 4 blocks
    _say(f"dflash errors {w.name} K={w.K} B={w.batch}")
    st = Setup(w, 77)
    try:
        inp = synth.step_inputs(w, 77)                     # no room for the block's last two positions
        inj_w = synth.inject_weights(w, 77)
        B, K = w.batch, w.K
        t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
             ("verify_positions", "num_accepted", "bonus_tokens", "block_table", "target_hidden")}
        kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
        ks, vs = [k for k, _ in kv], [v for _, v in kv]
        nkv = int(inp["num_kv_blocks"])
        batch = pb.Batch(B, K, S=K + 1)
        apos = torch.zeros(B * (K + 1), dtype=torch.int32, device="cuda")
        inj = torch.zeros(B * (K + 1), dtype=torch.int64, device="cuda")
        tok = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
        with pytest.raises(pb.PeError):
            pb.pe_dflash_prepare(st.ctx, B, t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                                 t["block_table"], nkv, batch, None, inj)
        wk = [pb.to_device(a) for a, _ in inj_w]
        wv = [pb.to_device(b) for _, b in inj_w]
        with pytest.raises(pb.PeError):
            pb.pe_dflash_inject(st.ctx, B, t["verify_positions"], None, t["target_hidden"], wk, wv, nkv, ks, vs)
        with pytest.raises(pb.PeError):
            pb.pe_dflash_forward(st.ctx, B, batch, None, t["block_table"], nkv, ks, vs, tok)
        with pytest.raises(pb.PeError):
            pb.pe_dflash_forward(st.ctx, B + 1, batch, apos, t["block_table"], nkv, ks, vs, tok)  # > max_num_seqs
        pb.pe_dflash_prepare(st.ctx, 0, t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                             t["block_table"], nkv, batch, apos, inj)
        pb.pe_dflash_prepare(st.ctx, B, t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                             t["block_table"], nkv, batch, apos, inj)
        pb.pe_dflash_inject(st.ctx, B, t["verify_positions"], inj, t["target_hidden"], wk, wv, nkv, ks, vs)
        pb.pe_dflash_forward(st.ctx, B, batch, apos, t["block_table"], nkv, ks, vs, tok)
        torch.cuda.synchronize()
        ob = O.dflash_prepare(inp["verify_positions"], inp["num_accepted"], inp["bonus_tokens"],
                              inp["block_table"], nkv, K, w.vocab, w.mask_id, w.block_size)
        need = inp["prefix"] + 2 * K + 2
        short = [r for r in range(B) if (need[r] + w.block_size - 1) // w.block_size > inp["block_table"].shape[1]]
        assert pb.pe_get_device_error(st.ctx) == ((O.ERR_BLOCK, short[0]) if short else (0, -1))
        assert_metadata_equal(batch.host(B, K), ob)
        for r in short:
            assert np.all(tok.cpu().numpy()[r * K:(r + 1) * K] == -1)
        # the pool is untouched by padded requests (their slots are all -1)
        if len(short) == B:
            for (kc, vc), (kc0, vc0) in zip(kv, inp["kv"]):
                np.testing.assert_array_equal(pb.to_host(kc), kc0)
                np.testing.assert_array_equal(pb.to_host(vc), vc0)
    finally:
        st.close()


@pytest.mark.parametrize("case", ["bf16_padded", "bf16_large"])
def test_dflash_step_graph_replays_equal_eager(case):
    """pe_step_graph in DFlash mode (prepare -> inject -> forward -> verify):
    four replays, with eager work and the caches reset between them, each
    equal to the four eager entry points bit for bit (block batch, horizons,
    injection slots, tokens, logits, verification, KV cache, error word), and
    the last replay against the oracle.  The large case (B=40: 320 block rows)
    runs the block's dense GEMMs on the large-batch 32x32-MFMA tiles."""
    B = 40 if case == "bf16_large" else 5
    w = SMALL_BF16.with_(K=7, batch=B, accepted="uniform", prefix=("uniform", 40, 400))
    _say(f"dflash graph case {case} B={B} K={w.K}")
    st = Setup(w, 79)
    try:
        inp = synth.step_inputs(w, 79, extra=2)
        inj_w = synth.inject_weights(w, 79)
        if case == "bf16_padded":
            inp["num_accepted"][2] = w.K + 1
        K = w.K
        t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
             ("verify_positions", "num_accepted", "bonus_tokens", "block_table", "target_tokens", "target_hidden")}
        kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
        kv0 = [(k.clone(), v.clone()) for k, v in kv]
        ks, vs = [k for k, _ in kv], [v for _, v in kv]
        wk = [pb.to_device(a) for a, _ in inj_w]
        wv = [pb.to_device(b) for _, b in inj_w]
        nkv = int(inp["num_kv_blocks"])
        batch = pb.Batch(B, K, S=K + 1)
        apos = torch.zeros(B * (K + 1), dtype=torch.int32, device="cuda")
        inj = torch.zeros(B * (K + 1), dtype=torch.int64, device="cuda")
        tok = torch.zeros(B * K, dtype=torch.int32, device="cuda")
        lg = torch.zeros((B * K, w.vocab), dtype=torch.float32, device="cuda")
        acc = torch.zeros(B, dtype=torch.int32, device="cuda")
        bon = torch.zeros(B, dtype=torch.int32, device="cuda")
        # eager
        pb.pe_dflash_prepare(st.ctx, B, t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                             t["block_table"], nkv, batch, apos, inj)
        pb.pe_dflash_inject(st.ctx, B, t["verify_positions"], inj, t["target_hidden"], wk, wv, nkv, ks, vs)
        pb.pe_dflash_forward(st.ctx, B, batch, apos, t["block_table"], nkv, ks, vs, tok, lg)
        pb.pe_verify(st.ctx, B, tok, t["target_tokens"], acc, bon)
        torch.cuda.synchronize()
        eager = {"batch": batch.host(B, K), "apos": apos.cpu().numpy(), "inj": inj.cpu().numpy(),
                 "tokens": tok.cpu().numpy(), "logits": lg.cpu().numpy(), "acc": acc.cpu().numpy(),
                 "bon": bon.cpu().numpy(), "kv": [(pb.to_host(k), pb.to_host(v)) for k, v in kv],
                 "error": pb.pe_get_device_error(st.ctx)}
        args = pb.make_dflash_step_args(t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                                        t["block_table"], nkv, batch, t["target_hidden"], ks, vs, wk, wv,
                                        apos, inj, tok, t["target_tokens"], acc, bon, logits=lg)
        for rep in range(4):
            for (k, v), (k0, v0) in zip(kv, kv0):
                k.copy_(k0)
                v.copy_(v0)
            tok.fill_(-5)
            lg.fill_(0.0)
            apos.fill_(-3)
            inj.fill_(-3)
            pb.pe_step_graph(st.ctx, B, args)
            torch.cuda.synchronize()
            _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays
            got = batch.host(B, K)
            for f in pb.BATCH_FIELDS:
                np.testing.assert_array_equal(got[f], eager["batch"][f], err_msg=f"{f} replay {rep}")
            np.testing.assert_array_equal(apos.cpu().numpy(), eager["apos"])
            np.testing.assert_array_equal(inj.cpu().numpy(), eager["inj"])
            np.testing.assert_array_equal(tok.cpu().numpy(), eager["tokens"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(lg.cpu().numpy(), eager["logits"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(acc.cpu().numpy(), eager["acc"])
            np.testing.assert_array_equal(bon.cpu().numpy(), eager["bon"])
            for (k, v), (ke, ve) in zip(kv, eager["kv"]):
                np.testing.assert_array_equal(pb.to_host(k), ke)
                np.testing.assert_array_equal(pb.to_host(v), ve)
            assert pb.pe_get_device_error(st.ctx) == eager["error"]
        if case == "bf16_padded":
            assert eager["error"] == (O.ERR_ACCEPTED, 2)
            assert np.all(eager["tokens"][2 * K:3 * K] == -1)
        # the graph's outputs against the oracle: block batch, horizons and
        # injection slots bit for bit, tokens and logits of the round drafted
        # on the oracle's injected cache, and the greedy verification (the
        # cache itself equals the eager one above, which _check compares)
        prec = oracle_precision(w)
        ob = O.dflash_prepare(inp["verify_positions"], inp["num_accepted"], inp["bonus_tokens"],
                              inp["block_table"], inp["num_kv_blocks"], w.K, w.vocab, w.mask_id, w.block_size)
        assert_metadata_equal(batch.host(B, K), ob)
        np.testing.assert_array_equal(apos.cpu().numpy(), ob["attn_positions"])
        np.testing.assert_array_equal(inj.cpu().numpy(), ob["inject_slots"])
        writes = O.dflash_inject(w, inp["verify_positions"], ob["inject_slots"], inp["target_hidden"], inj_w,
                                 inp["kv"], precision=prec)
        kv_o = O.apply_writes(inp["kv"], writes, w.block_size, w.dtype)
        reqs = [0, 1, 3] if case == "bf16_padded" else [0, 17, 39]
        fw = O.dflash_forward(st.prm, w, ob, kv_o, inp["block_table"], precision=prec, requests=reqs)
        rows = np.concatenate([np.arange(r * K, (r + 1) * K) for r in reqs])
        assert_tokens_logits(tok.cpu().numpy()[rows], lg.cpu().numpy()[rows], fw["logits"], logit_tol(w))
        o_acc, o_bon = O.verify(tok.cpu().numpy().reshape(B, K), inp["target_tokens"])
        np.testing.assert_array_equal(acc.cpu().numpy(), o_acc)
        np.testing.assert_array_equal(bon.cpu().numpy(), o_bon)
    finally:
        st.close()
