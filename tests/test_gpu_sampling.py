"""GPU parity of stochastic drafting and verification by rejection sampling
(pe_draft_forward_sampled, pe_verify_sampled) against the oracle
(oracle/pe_sampling.py) on the same seeded inputs and the same Philox keys.

Where floating point decides an integer (accept or reject; the winning draw)
both sides decide on identical fp32 logits; a decision is compared exactly
when its margin clears the fp32-vs-fp64 rounding (|U - min(1, p/q)| > 1e-4,
top-2 gap of the draw > 1e-3), otherwise the GPU's choice must be a valid
near-maximal one.  The drafted tokens come from the drafter's logits, which
differ from the oracle's within the one-pass bound: compared where the
Gumbel-perturbed top-2 gap clears twice that bound."""
import sys

import numpy as np
import pytest
import torch
from scipy import stats

import oracle as O
from drafting_pe_prepare_amd import configs, synth
from drafting_pe_prepare_amd import binding as pb

from pe_gpu import Setup, logit_tol, oracle_step, run_step

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


def _seed_dev(seed):
    return torch.tensor([seed], dtype=torch.int64, device="cuda")


def _verify_gpu(ctx, tokens, zq, zp, T, seed):
    B = tokens.shape[0]
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    pb.pe_verify_sampled(ctx, B, pb.to_device(np.ascontiguousarray(tokens.astype(np.int32))),
                         pb.to_device(np.ascontiguousarray(zq)), pb.to_device(np.ascontiguousarray(zp)),
                         T, _seed_dev(seed), acc, nxt)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy()


def _logits(B, K, V, seed, agree):
    rng = np.random.default_rng(seed)
    zq = rng.normal(0, 2.0, (B, K, V)).astype(np.float32)
    zp = rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32)
    zp[:, :K] = (agree * zq + (1 - agree) * zp[:, :K]).astype(np.float32)
    return zq, zp


def _margins(tokens, zq, zp, T, seed, a):
    """Smallest |U_j - min(1, p/q)| over the acceptance tests request r ran."""
    B, K = tokens.shape
    out = np.full(B, np.inf)
    for r in range(B):
        lq = O.log_softmax(zq[r], T)
        lp = O.log_softmax(zp[r], T)
        for j in range(min(a[r] + 1, K)):
            t = tokens[r, j]
            ratio = min(1.0, float(np.exp(lp[j, t] - lq[j, t])))
            out[r] = min(out[r], abs(O.uniform(seed, O.STREAM_ACCEPT, j, r) - ratio))
    return out


def _emit_scores(zq, zp, T, seed, r, a):
    V = zp.shape[-1]
    lp = O.log_softmax(zp[r], T)
    g = O.gumbel(O.token_uniforms(seed, O.STREAM_RESIDUAL, V, r))
    if a < zq.shape[1]:
        lq = O.log_softmax(zq[r], T)
        w = np.maximum(np.exp(lp[a]) - np.exp(lq[a]), 0.0)
        with np.errstate(divide="ignore"):
            return np.log(w) + g
    return lp[-1] + g


@pytest.mark.parametrize("T,agree", [(1.0, 0.9), (0.7, 0.97), (1.6, 0.6)])
def test_verify_sampled_matches_oracle(T, agree):
    w = SMALL_BF16.with_(K=4, batch=48)
    st = Setup(w, 90)
    try:
        B, K, V = 48, 4, w.vocab
        compared = skipped = 0
        for seed in (11, 12, 13):
            zq, zp = _logits(B, K, V, seed, agree)
            tokens = O.sample_drafts(zq.reshape(B * K, V), T, seed).reshape(B, K)
            acc_o, nxt_o = O.rejection_verify(tokens, zq, zp, T, seed)
            acc_g, nxt_g = _verify_gpu(st.ctx, tokens, zq.reshape(B * K, V), zp.reshape(B * (K + 1), V), T, seed)
            marg = _margins(tokens, zq, zp, T, seed, acc_o)
            for r in range(B):
                if marg[r] < 1e-4:
                    skipped += 1
                    continue
                assert acc_g[r] == acc_o[r], (seed, r, acc_g[r], acc_o[r])
                sc = _emit_scores(zq, zp, T, seed, r, acc_o[r])
                srt = np.sort(sc[np.isfinite(sc)])
                if len(srt) > 1 and srt[-1] - srt[-2] > 1e-3:
                    assert nxt_g[r] == nxt_o[r], (seed, r)
                else:
                    assert sc[nxt_g[r]] >= srt[-1] - 1e-3
                compared += 1
        _say(f"  T={T} agree={agree}: {compared} requests compared, {skipped} near-tie")
        assert compared >= 130
        assert 0 < np.mean([a for a in acc_o]) < K or agree < 0.7
    finally:
        st.close()


def test_verify_sampled_keeps_the_verifier_distribution():
    """1024 independent requests over the same logits (the counters differ
    by request): the first emitted token follows softmax(target row 0 / T)."""
    B, K, V, T = 1024, 2, 16, 1.0
    w = SMALL_BF16.with_(K=K, batch=B, vocab=V)
    st = Setup(w, 91)
    try:
        rng = np.random.default_rng(5)
        zq1 = rng.normal(0, 1.0, (K, V)).astype(np.float32)
        zp1 = rng.normal(0, 1.0, (K + 1, V)).astype(np.float32)
        zq = np.broadcast_to(zq1, (B, K, V)).copy()
        zp = np.broadcast_to(zp1, (B, K + 1, V)).copy()
        first = []
        for seed in (21, 22):
            tokens = O.sample_drafts(zq.reshape(B * K, V), T, seed).reshape(B, K)
            acc, nxt = _verify_gpu(st.ctx, tokens, zq.reshape(B * K, V), zp.reshape(B * (K + 1), V), T, seed)
            first.extend(np.where(acc >= 1, tokens[:, 0], nxt))
        p0 = np.exp(O.log_softmax(zp1[0], T))
        counts = np.bincount(first, minlength=V).astype(float)
        assert stats.chisquare(counts, p0 * counts.sum()).pvalue > 1e-4
    finally:
        st.close()


def test_verify_sampled_padded_request_and_errors():
    w = SMALL_BF16.with_(K=3, batch=4)
    st = Setup(w, 92)
    try:
        B, K, V = 4, 3, 1024
        zq, zp = _logits(B, K, V, 7, 0.9)
        tokens = O.sample_drafts(zq.reshape(B * K, V), 1.0, 7).reshape(B, K)
        tokens[2] = -1
        acc, nxt = _verify_gpu(st.ctx, tokens, zq.reshape(B * K, V), zp.reshape(B * (K + 1), V), 1.0, 7)
        assert acc[2] == 0 and 0 <= nxt[2] < V
        z = torch.zeros(64, dtype=torch.int32, device="cuda")
        f = torch.zeros(4096, dtype=torch.float32, device="cuda")
        with pytest.raises(RuntimeError):  # temperature must be > 0
            pb.pe_verify_sampled(st.ctx, B, z, f, f, 0.0, _seed_dev(1), z, z)
        with pytest.raises(RuntimeError):  # seed pointer required
            pb.pe_verify_sampled(st.ctx, B, z, f, f, 1.0, None, z, z)
    finally:
        st.close()


@pytest.mark.parametrize("T", [0.8, 1.5])
def test_draft_forward_sampled_matches_oracle(T):
    """Drafts drawn on the GPU from its own logits equal the oracle's draws
    from the oracle's logits wherever the perturbed top-2 gap clears twice the
    logit bound; the logits are those of the greedy pass, bit for bit."""
    w = SMALL_BF16.with_(K=4, batch=6, accepted="uniform", prefix=("uniform", 30, 300))
    st = Setup(w, 93)
    try:
        inp = synth.step_inputs(w, seed=93)
        greedy = run_step(st, inp)
        seed = 4242
        B, K = w.batch, w.K
        t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
             ("verify_tokens", "verify_positions", "num_accepted", "bonus_tokens", "block_table",
              "target_hidden")}
        kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
        batch = pb.Batch(B, K)
        nkv = int(inp["num_kv_blocks"])
        pb.pe_prepare(st.ctx, B, t["verify_tokens"], t["verify_positions"], t["num_accepted"],
                      t["bonus_tokens"], t["block_table"], nkv, batch)
        dh = torch.zeros((B * 2 * K, w.d), dtype=torch.bfloat16, device="cuda")
        pb.pe_gather_hidden(st.ctx, B, batch, t["target_hidden"], st.dev["h_shared"], dh)
        tok = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
        lg = torch.zeros((B * K, w.vocab), dtype=torch.float32, device="cuda")
        pb.pe_draft_forward_sampled(st.ctx, B, batch, dh, t["block_table"], nkv, [k for k, _ in kv],
                                    [v for _, v in kv], T, _seed_dev(seed), tok, lg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lg.cpu().numpy(), greedy["logits"])
        _, _, fw = oracle_step(w, st.prm, inp)
        ol = fw["logits"]
        want = O.sample_drafts(ol, T, seed)
        got = tok.cpu().numpy()
        tol = logit_tol(w) * float(np.sqrt(np.mean(ol ** 2))) / T
        V = w.vocab
        compared = 0
        for i in range(B * K):
            sc = ol[i] / T + O.gumbel(O.token_uniforms(seed, O.STREAM_DRAFT, V, i))
            srt = np.sort(sc)
            if srt[-1] - srt[-2] > 2 * tol:
                assert got[i] == want[i], (i, got[i], want[i])
                compared += 1
            else:
                assert sc[got[i]] >= srt[-1] - 2 * tol
        assert compared >= B * K // 2
    finally:
        st.close()


def test_verify_sampled_full_vocabulary():
    """The 20B-class vocabulary (201088 tokens: each row's log-sum-exp and
    draws run over all of its slices, the trip count bench.py times) against
    the oracle on the same fp32 logits and Philox keys."""
    V, B, K, T = 201088, 6, 7, 1.0
    w = SMALL_BF16.with_(K=K, batch=B, vocab=V)
    st = Setup(w, 94)
    try:
        compared = skipped = 0
        for seed in (31, 32):
            zq, zp = _logits(B, K, V, seed, 0.95)
            tokens = O.sample_drafts(zq.reshape(B * K, V), T, seed).reshape(B, K)
            acc_o, nxt_o = O.rejection_verify(tokens, zq, zp, T, seed)
            acc_g, nxt_g = _verify_gpu(st.ctx, tokens, zq.reshape(B * K, V), zp.reshape(B * (K + 1), V), T, seed)
            marg = _margins(tokens, zq, zp, T, seed, acc_o)
            for r in range(B):
                if marg[r] < 1e-4:
                    skipped += 1
                    continue
                assert acc_g[r] == acc_o[r], (seed, r, acc_g[r], acc_o[r])
                sc = _emit_scores(zq, zp, T, seed, r, acc_o[r])
                srt = np.sort(sc[np.isfinite(sc)])
                if len(srt) > 1 and srt[-1] - srt[-2] > 1e-3:
                    assert nxt_g[r] == nxt_o[r], (seed, r)
                else:
                    assert sc[nxt_g[r]] >= srt[-1] - 1e-3
                compared += 1
        _say(f"  V={V}: {compared} requests compared, {skipped} near-tie")
        assert compared >= 10
    finally:
        st.close()


def test_draft_forward_sampled_full_vocabulary():
    """Sampled drafting over a 201088-token vocabulary (the LM head's
    argmax-free path and every draw slice at full size) against the oracle's
    draws from its own logits."""
    T = 1.0
    w = SMALL_BF16.with_(K=7, batch=2, vocab=201088, accepted="uniform", prefix=("uniform", 30, 300),
                         weight_std=1 / 16)
    st = Setup(w, 95)
    try:
        inp = synth.step_inputs(w, seed=95)
        seed = 777
        B, K = w.batch, w.K
        t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
             ("verify_tokens", "verify_positions", "num_accepted", "bonus_tokens", "block_table",
              "target_hidden")}
        kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
        batch = pb.Batch(B, K)
        nkv = int(inp["num_kv_blocks"])
        pb.pe_prepare(st.ctx, B, t["verify_tokens"], t["verify_positions"], t["num_accepted"],
                      t["bonus_tokens"], t["block_table"], nkv, batch)
        dh = torch.zeros((B * 2 * K, w.d), dtype=torch.bfloat16, device="cuda")
        pb.pe_gather_hidden(st.ctx, B, batch, t["target_hidden"], st.dev["h_shared"], dh)
        tok = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
        lg = torch.zeros((B * K, w.vocab), dtype=torch.float32, device="cuda")
        pb.pe_draft_forward_sampled(st.ctx, B, batch, dh, t["block_table"], nkv, [k for k, _ in kv],
                                    [v for _, v in kv], T, _seed_dev(seed), tok, lg)
        torch.cuda.synchronize()
        _, _, fw = oracle_step(w, st.prm, inp)
        ol = fw["logits"]
        rms = float(np.sqrt(np.mean(ol ** 2)))
        assert np.max(np.abs(lg.cpu().numpy() - ol)) <= logit_tol(w) * rms
        want = O.sample_drafts(ol, T, seed)
        got = tok.cpu().numpy()
        tol = logit_tol(w) * rms / T
        V = w.vocab
        compared = 0
        for i in range(B * K):
            sc = ol[i] / T + O.gumbel(O.token_uniforms(seed, O.STREAM_DRAFT, V, i))
            srt = np.sort(sc)
            if srt[-1] - srt[-2] > 2 * tol:
                assert got[i] == want[i], (i, got[i], want[i])
                compared += 1
            else:
                assert sc[got[i]] >= srt[-1] - 2 * tol
        _say(f"  V={V}: {compared} of {B * K} draws compared exactly")
        assert compared >= B * K // 2
    finally:
        st.close()
