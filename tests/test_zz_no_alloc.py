"""pe_verify_sampled_noalloc (the allocation-free variant of
pe_verify_sampled, workspace in the library's fixed device array) against
pe_verify_sampled on the same logits and Philox keys: accepted counts and
emitted tokens bit for bit, on two calls in a row, the second with a smaller
batch (the workspace keeps the first call's contents); and oversized batches
rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle as O
from drafting_pe_prepare_amd import binding as pb
from drafting_pe_prepare_amd import configs

from pe_gpu import Setup

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pb.load()


def _logits(B, K, V, seed):
    rng = np.random.default_rng(seed)
    zq = rng.normal(0, 2.0, (B, K, V)).astype(np.float32)
    zp = rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32)
    zp[:, :K] = (0.9 * zq + 0.1 * zp[:, :K]).astype(np.float32)
    return zq, zp


def test_noalloc_verify_sampled_equals_the_context_entry_point():
    K, V, T = 5, 4096, 0.9
    w = configs.TINY.with_(dtype="bf16", d=256, mlp=1024, vocab=V, K=K, batch=96)
    st = Setup(w, 96)
    try:
        seed = torch.tensor([1234], dtype=torch.int64, device="cuda")
        for B, s in ((96, 41), (13, 42)):  # the second call is smaller
            zq, zp = _logits(B, K, V, s)
            tokens = O.sample_drafts(zq.reshape(B * K, V), T, 1234).reshape(B, K).astype(np.int32)
            tok = pb.to_device(np.ascontiguousarray(tokens))
            q = pb.to_device(np.ascontiguousarray(zq.reshape(B * K, V)))
            p = pb.to_device(np.ascontiguousarray(zp.reshape(B * (K + 1), V)))
            out = []
            for noalloc in (False, True):
                acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
                nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
                if noalloc:
                    pb.pe_verify_sampled_noalloc(B, K, V, tok, q, p, T, seed, acc, nxt)
                else:
                    pb.pe_verify_sampled(st.ctx, B, tok, q, p, T, seed, acc, nxt)
                torch.cuda.synchronize()
                out.append((acc.cpu().numpy(), nxt.cpu().numpy()))
            np.testing.assert_array_equal(out[1][0], out[0][0], err_msg=f"accepted, B={B}")
            np.testing.assert_array_equal(out[1][1], out[0][1], err_msg=f"next tokens, B={B}")
            assert np.all((out[1][0] >= 0) & (out[1][0] <= K))
    finally:
        st.close()


def test_noalloc_rejects_sizes_beyond_its_workspace():
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    seed = torch.tensor([1], dtype=torch.int64, device="cuda")
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        pb.pe_verify_sampled_noalloc(2049, 1, 16, z, f, f, 1.0, seed, z, z)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        pb.pe_verify_sampled_noalloc(300, 15, 16, z, f, f, 1.0, seed, z, z)  # 300 x 31 rows > 8192
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        pb.pe_verify_sampled_noalloc(4, 3, 18, z, f, f, 1.0, seed, z, z)  # vocab not a multiple of 4
    pb.pe_verify_sampled_noalloc(0, 3, 16, z, f, f, 1.0, seed, z, z)  # empty batch: nothing to do
