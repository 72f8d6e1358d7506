"""GPU parity of the drafting round after a prompt (pe_prefill_prepare,
pe_prefill_gather, pe_prefill_forward) against the oracle's prepare_prefill,
gather_hidden and draft_forward on the same seeded inputs: batch fields and
drafter inputs bit for bit, tokens and logits within the one-pass bound
(2e-2 x RMS in bf16 per sqrt(layer), 1e-4 in fp32), KV written at exactly the
oracle's slots.  Covers requests longer than one attention workgroup (slot
groups), padding requests, and a prompt drafted in two chunks."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from drafting_pe_prepare_amd import configs, synth
from drafting_pe_prepare_amd import binding as pb

from pe_gpu import Setup, assert_kv, assert_metadata_equal, assert_tokens_logits, logit_tol, oracle_precision

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


def run_prefill(st, inp, kv=None, want_logits=True):
    """prefill prepare -> gather -> forward on the GPU; returns host copies
    (the KV caches given as device tensors are updated in place)."""
    w = st.w
    B, K, S = w.batch, w.K, inp["S"]
    t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
         ("chunk_tokens", "chunk_lens", "start_pos", "new_tokens", "block_table", "target_hidden")}
    if kv is None:
        kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
    batch = pb.Batch(B, K, S=S)
    nkv = int(inp["num_kv_blocks"])
    pb.pe_prefill_prepare(st.ctx, B, S, t["chunk_tokens"], t["chunk_lens"], t["start_pos"],
                          t["new_tokens"], t["block_table"], nkv, batch)
    sdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dh = torch.zeros((B * S, w.d), dtype=sdt, device="cuda")
    pb.pe_prefill_gather(st.ctx, B, S, batch, t["target_hidden"], st.dev["h_shared"], dh)
    tok = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros((B * K, w.vocab), dtype=torch.float32, device="cuda") if want_logits else None
    pb.pe_prefill_forward(st.ctx, B, S, batch, dh, t["block_table"], nkv,
                          [k for k, _ in kv], [v for _, v in kv], tok, lg)
    torch.cuda.synchronize()
    return {
        "batch": batch.host(B, K),
        "draft_hidden": pb.to_host(dh),
        "tokens": tok.cpu().numpy(),
        "logits": lg.cpu().numpy() if want_logits else None,
        "kv": [(pb.to_host(k), pb.to_host(v)) for k, v in kv],
        "kv_dev": kv,
        "error": pb.pe_get_device_error(st.ctx),
    }


def oracle_prefill(w, prm, inp, kv=None, precision=None):
    b = O.prepare_prefill(inp["chunk_tokens"], inp["chunk_lens"], inp["start_pos"], inp["new_tokens"],
                          inp["block_table"], inp["num_kv_blocks"], w.K, inp["S"], w.vocab, w.mask_id,
                          w.block_size)
    hd = O.gather_hidden(b["hidden_src"], inp["target_hidden"], prm["h_shared"])
    fw = O.draft_forward(prm, w, b, hd, inp["kv"] if kv is None else kv, inp["block_table"],
                         precision or oracle_precision(w))
    return b, hd, fw


def _check(w, S, lens, start, seed, bad=None):
    _say(f"prefill case {w.name} B={w.batch} K={w.K} S={S} d={w.d} G={w.n_q_heads // w.n_kv_heads} "
         f"dtype={w.dtype} lens={lens} start={start} seed={seed} bad={bad}")
    st = Setup(w, seed, max_prefill_slots=w.batch * S)
    try:
        inp = synth.prefill_inputs(w, S, lens, start, seed)
        if bad is not None:
            inp["chunk_lens"][bad] = S  # > L: the request becomes padding
        g = run_prefill(st, inp)
        ob, ohd, fw = oracle_prefill(w, st.prm, inp)
        assert_metadata_equal(g["batch"], ob)
        np.testing.assert_array_equal(g["draft_hidden"], ohd)
        assert g["error"] == ((0, -1) if bad is None else (O.ERR_ACCEPTED, bad))
        K = w.K
        good = [r for r in range(w.batch) if r != bad]
        rows = np.concatenate([np.arange(r * K, (r + 1) * K) for r in good])
        tight = assert_tokens_logits(g["tokens"], g["logits"], fw["logits"][rows], logit_tol(w), rows)
        if bad is not None:
            assert np.all(g["tokens"][bad * K:(bad + 1) * K] == -1)
            assert np.all(fw["tokens"][bad * K:(bad + 1) * K] == -1)
        assert_kv(w, g["kv"], inp, fw)
        return tight
    finally:
        st.close()


def test_prefill_tiny_f32():
    _check(configs.TINY.with_(K=4, batch=2), 24, ("uniform", 1, 21), ("uniform", 0, 50), seed=61)


@pytest.mark.parametrize("K,B,S,seed", [(4, 3, 40, 62), (1, 2, 64, 63), (7, 2, 16, 64)])
def test_prefill_small_bf16_one_group(K, B, S, seed):
    """S x (query heads per KV head) <= 512: a request is one attention item set."""
    _check(SMALL_BF16.with_(K=K, batch=B), S, ("uniform", 1, S - K + 1), ("uniform", 0, 90), seed)


@pytest.mark.parametrize("S,lens,start,seed", [
    (256, ("uniform", 100, 250), ("uniform", 0, 200), 65),
    (192, ("fixed", 186), ("fixed", 0), 66),
])
def test_prefill_small_bf16_slot_groups(S, lens, start, seed):
    """8 query heads per KV head: 64-slot groups attend as requests of their
    own over the same block table row (S/64 groups per request)."""
    w = SMALL_BF16.with_(K=7, batch=2, n_q_heads=8, n_kv_heads=1)
    _check(w, S, lens, start, seed)


def test_prefill_large_batch_gemms_d1024():
    """448 slots of d = 1024: large-batch 32x32-MFMA GEMMs with the fused epilogues, 7 slot
    groups."""
    w = SMALL_BF16.with_(K=7, batch=1, d=1024, mlp=2048, n_q_heads=16, n_kv_heads=2,
                         weight_std=1 / 32)
    _check(w, 448, ("fixed", 442), ("fixed", 37), seed=67)


def test_prefill_large_batch_gemms():
    """640 slots of d = 256: large-batch 32x32-MFMA GEMMs with the fused epilogues, 10 slot
    groups."""
    w = SMALL_BF16.with_(K=7, batch=1, n_q_heads=8, n_kv_heads=1)
    _check(w, 640, ("fixed", 600), ("fixed", 21), seed=72)


def test_prefill_padded_request():
    _check(SMALL_BF16.with_(K=3, batch=3), 48, ("uniform", 10, 46), ("uniform", 0, 60), seed=68, bad=1)


def test_prefill_two_chunks_on_the_gpu():
    """The first chunk's call writes KV that the second chunk reads on the
    GPU; the final drafts equal the oracle's one-chunk drafts, and the KV of
    the whole prompt equals the oracle's."""
    w = SMALL_BF16.with_(K=5, batch=1, n_q_heads=8, n_kv_heads=1)
    S, n, n1 = 192, 180, 77
    st = Setup(w, 69, max_prefill_slots=S)
    try:
        inp = synth.prefill_inputs(w, S, ("fixed", n), ("fixed", 0), 69)
        first = dict(inp)
        first["chunk_lens"] = np.array([n1], np.int32)
        first["new_tokens"] = np.array([inp["chunk_tokens"][0, n1]], np.int32)
        g1 = run_prefill(st, first, want_logits=False)
        second = dict(inp)
        ct = np.zeros_like(inp["chunk_tokens"])
        ct[0, :n - n1] = inp["chunk_tokens"][0, n1:n]
        second["chunk_tokens"] = ct
        second["chunk_lens"] = np.array([n - n1], np.int32)
        second["start_pos"] = np.array([n1], np.int32)
        th = np.zeros_like(inp["target_hidden"])
        th[:n - n1] = inp["target_hidden"][n1:n]
        second["target_hidden"] = th
        g2 = run_prefill(st, second, kv=g1["kv_dev"])
        assert g1["error"] == (0, -1) and g2["error"] == (0, -1)
        ob, ohd, fw = oracle_prefill(w, st.prm, inp)
        assert_tokens_logits(g2["tokens"], g2["logits"], fw["logits"], logit_tol(w))
        assert_kv(w, g2["kv"], inp, fw)
    finally:
        st.close()


def test_prefill_rejects_oversized_batches():
    w = SMALL_BF16.with_(K=3, batch=2, n_q_heads=8, n_kv_heads=1)
    st = Setup(w, 70, max_prefill_slots=2 * 100)
    try:
        batch = pb.Batch(2, w.K, S=100)
        z = torch.zeros(1024, dtype=torch.int32, device="cuda")
        with pytest.raises(RuntimeError):  # S below K
            pb.pe_prefill_prepare(st.ctx, 2, 2, z, z, z, z, z.view(2, -1), 4, batch)
        with pytest.raises(RuntimeError):  # B*S above max_prefill_slots
            pb.pe_prefill_prepare(st.ctx, 2, 101, z, z, z, z, z.view(2, -1), 4, batch)
        # S = 100 slots with 8 query heads per KV head: not a multiple of the 64-slot group
        dh = torch.zeros((200, w.d), dtype=torch.bfloat16, device="cuda")
        tok = torch.zeros(6, dtype=torch.int32, device="cuda")
        kv = [(torch.zeros((64, 1, 64), dtype=torch.bfloat16, device="cuda"),
               torch.zeros((4, 1, 64, 16), dtype=torch.bfloat16, device="cuda"))]
        with pytest.raises(RuntimeError):
            pb.pe_prefill_forward(st.ctx, 2, 100, batch, dh, z.view(2, -1), 4,
                                  [k for k, _ in kv], [v for _, v in kv], tok)
    finally:
        st.close()


@pytest.mark.slow
def test_prefill_full_c1():
    """The c=1 20B-class drafter after a 2048-position prompt (S = 2112: 33
    slot groups), every output checked."""
    _check(configs.C1.with_(batch=1), 2112, ("fixed", 2048), ("fixed", 0), seed=71)
