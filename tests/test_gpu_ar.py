"""GPU parity of the sequential (autoregressive) drafting passes, pe_ar_draft:
the same kernels run as one pass over the K+1 copied slots and K-1 passes of
one slot per request, against the oracle's ar_draft on the same seeded
inputs.  Pass k's logits within k x the one-pass bound (2e-2 x RMS in bf16,
1e-4 in fp32; later passes take the drafter's own rounded state as input);
tokens equal wherever the oracle's top-2 gap clears the bound (a tight pass
may pick another near-maximal token, after which the passes are not
compared); KV unchanged off the written positions."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from drafting_pe_prepare_amd import configs, synth
from drafting_pe_prepare_amd import binding as pb

from pe_gpu import Setup, assert_ar_request, logit_tol, run_step, written_slots_ar

pytestmark = pytest.mark.gpu

SMALL_BF16 = configs.TINY.with_(dtype="bf16", d=256, mlp=1024, vocab=1024, prefix=("fixed", 64, 0),
                                weight_std=1 / 16)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pb.load()


def _kv_unchanged_off(w, gpu_kv, inp, slots):
    keep = np.ones(inp["kv"][0][0].shape[0], bool)
    keep[slots] = False
    for li, ((kg, vg), (k0, v0)) in enumerate(zip(gpu_kv, inp["kv"])):
        np.testing.assert_array_equal(kg[keep], k0[keep], err_msg=f"K layer {li}")
        vg2 = vg.transpose(0, 3, 1, 2).reshape(-1, w.n_kv_heads, w.head_dim)
        v02 = v0.transpose(0, 3, 1, 2).reshape(-1, w.n_kv_heads, w.head_dim)
        np.testing.assert_array_equal(vg2[keep], v02[keep], err_msg=f"V layer {li}")


def _check(w, seed, bad=()):
    _say(f"ar case {w.name} B={w.batch} K={w.K} d={w.d} dtype={w.dtype} seed={seed} bad={bad}")
    st = Setup(w, seed)
    try:
        inp = synth.step_inputs(w, seed)
        for r in bad:
            inp["num_accepted"][r] = w.K + 3
        g = run_step(st, inp, ar=True)
        good = [r for r in range(w.batch) if r not in bad]
        for r in bad:
            assert np.all(g["tokens"][r * w.K:(r + 1) * w.K] == -1)
        assert g["error"][0] == (1 if bad else 0)
        compared = sum(assert_ar_request(w, g, inp, st.prm, r, logit_tol(w)) for r in good)
        _kv_unchanged_off(w, g["kv"], inp, written_slots_ar(w, inp, good))
        return compared
    finally:
        st.close()


def test_ar_tiny_f32():
    assert _check(configs.TINY, None) == configs.TINY.K


@pytest.mark.parametrize("K,B,seed", [(4, 3, 21), (1, 2, 22), (7, 2, 23), (15, 1, 24)])
def test_ar_small_bf16(K, B, seed):
    w = SMALL_BF16.with_(K=K, batch=B, accepted="uniform", prefix=("uniform", 20, 300))
    assert _check(w, seed) >= B


def test_ar_small_bf16_tiled_first_pass():
    """20 requests x 5 copied slots: the first pass runs the tiled GEMMs,
    the later passes the small-batch ones."""
    w = SMALL_BF16.with_(K=4, batch=20, accepted="uniform", prefix=("uniform", 20, 200))
    assert _check(w, 25) >= 20


def test_ar_padded_request():
    w = SMALL_BF16.with_(K=4, batch=3, accepted="uniform")
    _check(w, 26, bad=(1,))


def test_ar_step_graph_replays_match_eager():
    """The step graph in sequential mode equals eager pe_ar_draft on every
    replay, with eager work and synchronization between replays, and the
    last replay matches the oracle's sequential drafting pass by pass."""
    w = SMALL_BF16.with_(K=5, batch=4, accepted="uniform", prefix=("uniform", 40, 400))
    st = Setup(w, seed=27)
    try:
        inp = synth.step_inputs(w, seed=27)
        eager = run_step(st, inp, ar=True)
        B, K = w.batch, w.K
        t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
             ("verify_tokens", "verify_positions", "num_accepted", "bonus_tokens", "block_table",
              "target_tokens", "target_hidden")}
        kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
        kv0 = [(k.clone(), v.clone()) for k, v in kv]
        batch = pb.Batch(B, K)
        dh = torch.zeros((B * 2 * K, w.d), dtype=torch.bfloat16, device="cuda")
        tok = torch.zeros(B * K, dtype=torch.int32, device="cuda")
        lg = torch.zeros((B * K, w.vocab), dtype=torch.float32, device="cuda")
        acc = torch.zeros(B, dtype=torch.int32, device="cuda")
        bon = torch.zeros(B, dtype=torch.int32, device="cuda")
        args = pb.make_step_args(t["verify_tokens"], t["verify_positions"], t["num_accepted"],
                                 t["bonus_tokens"], t["block_table"], inp["num_kv_blocks"], batch,
                                 t["target_hidden"], st.dev["h_shared"], dh,
                                 [k for k, _ in kv], [v for _, v in kv], tok, t["target_tokens"],
                                 acc, bon, logits=lg, mode=pb.STEP_AUTOREGRESSIVE)
        for rep in range(3):
            for (k, v), (k0, v0) in zip(kv, kv0):
                k.copy_(k0)
                v.copy_(v0)
            tok.fill_(-5)
            lg.fill_(0.0)
            pb.pe_step_graph(st.ctx, B, args)
            torch.cuda.synchronize()
            _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays
            np.testing.assert_array_equal(tok.cpu().numpy(), eager["tokens"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(lg.cpu().numpy(), eager["logits"], err_msg=f"replay {rep}")
            np.testing.assert_array_equal(acc.cpu().numpy(), eager["accepted"])
            np.testing.assert_array_equal(bon.cpu().numpy(), eager["bonus"])
            for (k, v), (ke, ve) in zip(kv, eager["kv"]):
                np.testing.assert_array_equal(pb.to_host(k), ke)
                np.testing.assert_array_equal(pb.to_host(v), ve)
        # the graph's passes against the oracle's sequential drafting
        g = {"tokens": tok.cpu().numpy(), "logits": lg.cpu().numpy(),
             "kv": [(pb.to_host(k), pb.to_host(v)) for k, v in kv]}
        for r in range(B):
            assert_ar_request(w, g, inp, st.prm, r, logit_tol(w))
        acc_o, bon_o = O.verify(g["tokens"].reshape(B, K), inp["target_tokens"])
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
        np.testing.assert_array_equal(bon.cpu().numpy(), bon_o)
    finally:
        st.close()


@pytest.mark.slow
def test_ar_full_c1():
    """The c=1 20B-class workload at full size, drafted sequentially."""
    assert _check(configs.C1, None) >= 1
