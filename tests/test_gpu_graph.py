"""The captured step graph against the CPU oracle.

"P-EAGLE: parallel speculative decoding in vLLM", vLLM implementation
details, KV cache and CUDA Graphs: one graph is captured for the K x
max_num_seqs draft rows of the largest batch and serves every step.  Here the
graph is captured once at B = max_num_seqs with an occupancy read on the
device; replays at several occupancies must give, for every active request,
exactly what the oracle gives for that request, leave the inactive requests as
padding (no KV write, draft tokens -1, accepted 0, bonus 0, nothing in the
device error word), and never recapture.  The graph's fused kernels
(preparation + hidden-state copy, argmax + verification) are compared with the
oracle here directly, not only with the eager entry points."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from drafting_pe_prepare_amd import binding as pb
from drafting_pe_prepare_amd import configs, synth

from pe_gpu import GraphRun, Setup, assert_kv, assert_tokens_logits, logit_tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pb.load()


SMALL_BF16 = configs.TINY.with_(dtype="bf16", d=256, mlp=1024, vocab=1024, prefix=("fixed", 64, 0),
                                weight_std=1 / 16)
PAD = {"input_ids": 0, "positions": 0, "hidden_src": -1, "is_rejected": 1, "is_masked": 0,
       "slot_mapping": -1}


def check_against_oracle(w, prm, inp, g, n, requests=None):
    """Outputs of one replay at occupancy n against the oracle.  requests:
    the active requests whose forward the oracle computes (default: all n)."""
    B, K, S = w.batch, w.K, 2 * w.K
    acc_in = inp["num_accepted"]
    ob = O.prepare(inp["verify_tokens"], inp["verify_positions"], acc_in, inp["bonus_tokens"],
                   inp["block_table"], inp["num_kv_blocks"], K, w.vocab, w.mask_id, w.block_size)
    act = np.arange(n * S)
    for f in pb.BATCH_FIELDS:
        if f == "draft_rows":
            np.testing.assert_array_equal(g["batch"][f][:n * K], ob[f][:n * K], err_msg=f)
            np.testing.assert_array_equal(g["batch"][f][n * K:], np.arange(n * S, B * S).reshape(-1, S)[:, :K].ravel()
                                          if n < B else [], err_msg=f)
        elif f == "seq_lens":
            np.testing.assert_array_equal(g["batch"][f][:n], ob[f][:n], err_msg=f)
            assert np.all(g["batch"][f][n:] == 0)
        else:
            np.testing.assert_array_equal(g["batch"][f][act], ob[f][act], err_msg=f)
            assert np.all(g["batch"][f][n * S:] == PAD[f]), f
    hd = O.gather_hidden(ob["hidden_src"], inp["target_hidden"], prm["h_shared"])
    np.testing.assert_array_equal(g["draft_hidden"][act], hd[act])
    reqs = list(range(n)) if requests is None else list(requests)
    # the oracle's view of the batch: inactive requests are not part of it
    err_reqs = [r for r in range(n) if ob["seq_lens"][r] == 0]
    want_err = (0, -1)
    if err_reqs:
        kinds = 0
        for r in err_reqs:
            a = int(acc_in[r])
            kinds |= O.ERR_ACCEPTED if (a < 0 or a > K) else 0
        want_err = (kinds, err_reqs[0])
    assert g["error"] == want_err, (g["error"], want_err)
    assert np.all(g["tokens"][n * K:] == -1)
    for r in err_reqs:
        assert np.all(g["tokens"][r * K:(r + 1) * K] == -1)
    assert np.all(g["accepted"][n:] == 0) and np.all(g["bonus"][n:] == 0)
    if reqs:
        fw = O.draft_forward(prm, w, ob, hd, inp["kv"], inp["block_table"],
                             "bf16" if w.dtype == "bf16" else "f64", requests=reqs)
        rows = np.concatenate([np.arange(r * K, (r + 1) * K) for r in reqs])
        valid = [i for i, r in enumerate(reqs) if ob["seq_lens"][r] > 0]
        vrows = np.concatenate([np.arange(i * K, (i + 1) * K) for i in valid]) if valid else np.zeros(0, int)
        if len(vrows):
            assert_tokens_logits(g["tokens"][rows], g["logits"][rows] if g["logits"] is not None else None,
                                 fw["logits"][vrows], logit_tol(w), rows=vrows)
        if requests is None:
            assert_kv(w, g["kv"], inp, fw)
    if n:
        acc, bon = O.verify(g["tokens"][:n * K].reshape(n, K), inp["target_tokens"][:n])
        np.testing.assert_array_equal(g["accepted"][:n], acc)
        np.testing.assert_array_equal(g["bonus"][:n], bon)


@pytest.mark.parametrize("case", ["bf16_large", "bf16_mid", "f32_small"])
def test_one_capture_serves_every_occupancy(case):
    """Captured once at B = max_num_seqs, replayed at occupancies B, 1, 7, 0
    and B again.  bf16_large: 32 requests x 14 slots (448 forward rows: the
    large-batch GEMMs with MASK-deduplicated first layer, 224 draft rows);
    request 15 carries an invalid accepted count, reported only while it is
    active.  bf16_mid: 12 requests x 14 slots, two layers (168 forward rows,
    84 draft rows: the 65..256-row products on row maps with the split
    planned on the device, MASK deduplication, the draft-rows-only last
    layer).  f32_small: 3 requests of the 64-token fp32 drafter."""
    if case == "bf16_large":
        w = SMALL_BF16.with_(K=7, batch=32, accepted="uniform", prefix=("uniform", 40, 400))
        plan = [32, 1, 7, 0, 32]
        bad = 15
    elif case == "bf16_mid":
        w = SMALL_BF16.with_(K=7, batch=12, layers=2, accepted="uniform", prefix=("uniform", 40, 400))
        plan = [12, 1, 5, 0, 12]
        bad = 4
    else:
        w = configs.TINY.with_(K=4, batch=3, accepted="uniform", prefix=("uniform", 40, 200))
        plan = [3, 1, 0, 2]
        bad = None
    _say(f"case {case}: B={w.batch} K={w.K} dtype={w.dtype}")
    st = Setup(w, seed=31)
    try:
        inp = synth.step_inputs(w, seed=31)
        if bad is not None:
            inp["num_accepted"][bad] = w.K + 2
        gr = GraphRun(st, inp, occupancy=True)
        for n in plan:
            _say(f"  occupancy {n}")
            g = gr.run(n)
            check_against_oracle(w, st.prm, inp, g, n)
        caps, reps = pb.pe_step_graph_stats(st.ctx)
        assert caps == 1 and reps == len(plan), (caps, reps)
    finally:
        st.close()


@pytest.mark.slow
def test_c64_graph_against_oracle():
    """The c=64 20B-class step through the captured graph (the one bench.py
    times), at full occupancy and at 17 of 64: every active request's
    metadata, hidden rows, tokens and verification, and the sampled requests'
    logits and tokens against the oracle; one capture for both."""
    w = configs.C64
    st = Setup(w)
    try:
        inp = synth.step_inputs(w)
        gr = GraphRun(st, inp, occupancy=True)
        for n, reqs in ((64, [0, 16, 63]), (17, [0, 16])):
            _say(f"  c64 graph, occupancy {n}, oracle requests {reqs}")
            g = gr.run(n)
            check_against_oracle(w, st.prm, inp, g, n, requests=reqs)
        assert pb.pe_step_graph_stats(st.ctx)[0] == 1
    finally:
        st.close()


def test_sequential_graph_with_occupancy():
    """The sequential-drafting graph (PE_STEP_AUTOREGRESSIVE) captured at 6
    requests and replayed at occupancy 2: the inactive requests are padding
    (tokens -1, no KV write) and each active request's K passes match the
    oracle's sequential drafting pass by pass."""
    from pe_gpu import assert_ar_request, written_slots_ar
    w = SMALL_BF16.with_(K=4, batch=6, accepted="uniform", prefix=("uniform", 40, 300))
    st = Setup(w, seed=33)
    try:
        inp = synth.step_inputs(w, seed=33)
        gr = GraphRun(st, inp, mode=pb.STEP_AUTOREGRESSIVE, occupancy=True)
        g = gr.run(2)
        K = w.K
        assert g["error"] == (0, -1)
        assert np.all(g["tokens"][2 * K:] == -1)
        assert np.all(g["accepted"][2:] == 0) and np.all(g["bonus"][2:] == 0)
        for r in (0, 1):
            assert_ar_request(w, g, inp, st.prm, r, logit_tol(w))
        written = written_slots_ar(w, inp, [0, 1])
        for (kc_g, vc_g), (kc0, vc0) in zip(g["kv"], inp["kv"]):
            mask = np.ones(kc0.shape[0], bool)
            mask[written] = False
            np.testing.assert_array_equal(kc_g[mask], kc0[mask])
            vg = vc_g.transpose(0, 3, 1, 2).reshape(-1, w.n_kv_heads, w.head_dim)
            v0 = vc0.transpose(0, 3, 1, 2).reshape(-1, w.n_kv_heads, w.head_dim)
            np.testing.assert_array_equal(vg[mask], v0[mask])
        assert pb.pe_step_graph_stats(st.ctx)[0] == 1
    finally:
        st.close()
