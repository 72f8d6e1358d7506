"""CPU oracle for the P-EAGLE parallel-draft step.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or run anything in this package.  The
HIP library never calls it, and it shares no code with the HIP path: it is a
plain, slow, fp64 NumPy restatement of what the step computes, used to check
the GPU results.

What it follows (page titles as published):
  * "P-EAGLE: parallel speculative decoding in vLLM" -- Architecture and
    mechanism (Step 2, Parallel Drafting: input construction for prompt, NTP
    and MTP positions; one N-layer Transformer + LM head pass predicting
    t_1..t_K), vLLM implementation details (Fused Triton kernel: the batch
    metadata; Hidden-state management: the hidden-state copy; KV cache:
    PADDING_SLOT_ID = -1 for rejected tokens); Architecture and mechanism,
    Step 1 (Prefilling) for the drafting round that follows a prompt.
  * "vLLM Speculators: parallel drafting for speculative decoding" --
    Production integration (verification by rejection sampling keeps the
    verifier's output distribution): pe_sampling.py.
  * "AWS and vLLM ship P-EAGLE" -- How it works (learned mask embedding and
    shared hidden vector for positions that do not exist yet); Integration and
    numbers (acceptance length = drafts the verifier accepts per round).

Where the pages leave a step open, the reading taken is stated at the function
that takes it.  Parity status of every function is pinned by tests under
tests/ (test_oracle_*.py); acceptance length on trained weights is parity
unpinned (no trained weights exist here).
"""
from .pe_sampling import (  # noqa: F401
    STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESIDUAL, philox4x32, uniform, token_uniforms, gumbel, log_softmax,
    sample_drafts, rejection_verify,
)
from .pe_oracle import (  # noqa: F401
    PAD_TOKEN, PADDING_SLOT_ID, ERR_ACCEPTED, ERR_TOKEN, ERR_BLOCK, ERR_LAYOUT,
    round_bf16, widen, prepare, prepare_prefill, gather_hidden, rmsnorm, rope, silu,
    attend, draft_forward, verify, eagle_step, ar_draft, slot_of, expected_tokens, choose_depth,
)
from .pe_dflash import dflash_prepare, dflash_inject, dflash_forward, apply_writes  # noqa: F401,E402
