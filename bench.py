#!/usr/bin/env python
"""Throughput of the P-EAGLE parallel-draft step on one MI355X.

A step is one pass of the whole hot path over one batch: pe_prepare ->
pe_gather_hidden -> pe_draft_forward -> pe_verify, replayed as one hipGraph
(pe_step_graph).  Inputs are seeded synthetic tensors already resident in
HBM when the timed region starts.

Default workload: the c=1 20B-class drafter (B=1, K=7, d=2880, 64q/8kv x 64,
MLP 7680, 1 layer, V=201088, bf16, prefix 2048).  The same run also measures
the c=64 workload (B=64, lognormal prefixes) and reports it under "c64".

Output: one JSON line.  `roofline` is for the dominant kernel (the LM head):
algorithmic bytes (or flops) per launch divided by its average duration, taken
from HIP events around each launch on the library's stream during an eager
timed pass of the same steps.  `cpu_baseline` times the CPU oracle on the
host on a bounded sample of the c=1 step.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
RING = 256                  # pre-drawn rounds the replay distribution rotates through
METRIC = "draft tokens/s and us per parallel-draft step, K=7, c=1 and c=64 (1 GPU)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="c1_20b")
    p.add_argument("--no-c64", action="store_true", help="skip the c=64 measurement")
    p.add_argument("--no-ksweep", action="store_true",
                   help="skip the K sweep of the 4-layer d=2048 drafter")
    p.add_argument("--no-ar", action="store_true",
                   help="skip the sequential (autoregressive) comparison")
    p.add_argument("--no-maxbatch", action="store_true",
                   help="skip the B=256 largest-graph workload")
    p.add_argument("--no-sampling", action="store_true",
                   help="skip the stochastic drafting / rejection-sampling verification timing")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the drafting round after a 2048-position prompt")
    p.add_argument("--no-dflash", action="store_true",
                   help="skip the DFlash-style round (KV injection + one bidirectional block)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run three plain 1 GiB device-to-device copies (the reference "
                        "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    return p.parse_args()


def copy_calibration():
    import torch
    x = torch.empty(2 ** 29, dtype=torch.bfloat16, device="cuda")
    x.fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 2 ** 30, "copies": 3}), flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of one step (measurement section)
# ---------------------------------------------------------------------------
def weight_bytes(w):
    e = 2 if w.dtype == "bf16" else 4
    d, qd, kvd = w.d, w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    layer = (qd * d + 2 * kvd * d + d * qd + 3 * w.mlp * d + 2 * d) * e
    return {"fc": 2 * d * d * e, "layers": w.layers * layer, "lm_head": w.vocab * d * e,
            "final_norm": d * e}


def step_work(w, inp):
    """Algorithmic HBM bytes and flops of one step on these inputs."""
    e = 2 if w.dtype == "bf16" else 4
    B, K, d = w.batch, w.K, w.d
    a = inp["num_accepted"].astype(int)
    p0 = inp["verify_positions"][:, 0].astype(int)
    seq = p0 + a + K
    kvrow = w.n_kv_heads * w.head_dim * e * 2          # K and V of one position
    wb = weight_bytes(w)
    bytes_ = sum(wb.values())
    bytes_ += B * 2 * K * d * e                          # embedding rows
    bytes_ += B * (K + 1) * d * e + d * e                # target hidden + h_shared
    bytes_ += 2 * B * 2 * K * d * e                      # draft hidden write + read
    bytes_ += w.layers * int(seq.sum()) * kvrow          # KV read
    bytes_ += w.layers * int((a + K).sum()) * kvrow      # KV write (valid slots)
    valid = int((a + K).sum())
    # Work whose results reach an output (draft tokens, KV writes): fc, the
    # norms and the QKV product of every valid slot in every layer; attention,
    # O and the MLP of every valid slot below the last layer, and of the draft
    # rows alone in the last one (the other slots' results there are never read)
    fl = attention_mlp_flops(w, [list(range(p0[r], p0[r] + a[r] + 1)) + [p0[r] + a[r] + m for m in range(1, K)]
                                 for r in range(B)],
                             [list(range(p0[r] + a[r], p0[r] + a[r] + K)) for r in range(B)])
    return {"bytes": bytes_, "flops": fl + 2 * B * K * w.vocab * d, "weight_bytes": sum(wb.values())}


def attention_mlp_flops(w, valid_pos, draft_pos, ctx_len=None):
    """Drafter flops below the LM head: valid_pos[r] / draft_pos[r] are the
    positions of request r's valid slots and draft rows; a slot at position q
    attends to q+1 positions (ctx_len[r] each when given: a bidirectional
    block).  fc + QKV on every valid slot of every layer; attention, O and MLP
    on the valid slots below the last layer and on the draft rows in it."""
    d, qd, kvd = w.d, w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    pre, post = qd * d + 2 * kvd * d, d * qd + 3 * w.mlp * d
    nvalid = sum(len(p) for p in valid_pos)
    ndraft = sum(len(p) for p in draft_pos)
    att = lambda sets: sum((ctx_len[r] * len(ps)) if ctx_len is not None else sum(q + 1 for q in ps)
                           for r, ps in enumerate(sets))
    flops = 2 * nvalid * (2 * d * d + w.layers * pre)
    flops += 2 * nvalid * (w.layers - 1) * post + 2 * ndraft * post
    flops += 4 * w.head_dim * w.n_q_heads * ((w.layers - 1) * att(valid_pos) + att(draft_pos))
    return flops


def ar_work(w, inp):
    """Algorithmic HBM bytes of the sequential comparison: every pass
    streams the whole drafter; pass 1 reads the context [0, p0+a] and writes
    the accepted slots' KV, pass k > 1 reads [0, p0+a+k-1] and writes one
    position."""
    e = 2 if w.dtype == "bf16" else 4
    B, K, d = w.batch, w.K, w.d
    a = inp["num_accepted"].astype(int)
    p0 = inp["verify_positions"][:, 0].astype(int)
    kvrow = w.n_kv_heads * w.head_dim * e * 2
    passes_bytes = K * sum(weight_bytes(w).values())
    ctx_read = int((K * (p0 + a) + K * (K + 1) // 2).sum())
    writes = int((a + K).sum())
    act = B * (K + 1) * d * e * 3 + (K - 1) * B * d * e * 3  # emb, hidden in, hidden copy
    return passes_bytes + w.layers * (ctx_read + writes) * kvrow + act


def measured_traffic(workload):
    """HBM bytes per LM-head launch from the committed rocprofv3 counter runs
    (profiles/traffic.json: FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy
    calibration), or None when the GEMM source changed since they were taken."""
    import hashlib
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        src = open(os.path.join(ROOT, "drafting_pe_prepare_amd", "csrc", "pe_gemm.hip"), "rb").read()
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest() != t.get("pe_gemm_sha256") or workload not in t:
        return None
    e = t[workload]
    return e["fetch_bytes"] + e["write_bytes"]


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------
def measure(w, steps, warmup, prm=None, dev=None, label="", with_ar=True):
    import numpy as np
    import torch
    from drafting_pe_prepare_amd import binding as pb
    from drafting_pe_prepare_amd import synth

    t_setup = time.time()
    if prm is None:
        prm = synth.weights(w)
    if dev is None:
        dev = pb.upload_weights(prm)
    inp = synth.step_inputs(w)
    B, K = w.batch, w.K
    ctx = pb.Context(w, dev, max_num_seqs=B)
    t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
         ("verify_tokens", "verify_positions", "num_accepted", "bonus_tokens", "block_table",
          "target_tokens", "target_hidden")}
    kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
    batch = pb.Batch(B, K)
    sdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dh = torch.zeros((B * 2 * K, w.d), dtype=sdt, device="cuda")
    tok = torch.zeros(B * K, dtype=torch.int32, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    ks, vs = [k for k, _ in kv], [v for _, v in kv]
    args = pb.make_step_args(t["verify_tokens"], t["verify_positions"], t["num_accepted"],
                             t["bonus_tokens"], t["block_table"], inp["num_kv_blocks"], batch,
                             t["target_hidden"], dev["h_shared"], dh, ks, vs, tok,
                             t["target_tokens"], acc, bon)
    torch.cuda.synchronize()
    print(f"[bench] {label} setup {time.time() - t_setup:.1f}s", file=sys.stderr, flush=True)

    for _ in range(warmup):
        pb.pe_step_graph(ctx, B, args)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        pb.pe_step_graph(ctx, B, args)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    ms_step = wall * 1e3 / steps
    err = pb.pe_get_device_error(ctx)
    assert err == (0, -1), f"device error word {err}"
    print(f"[bench] {label} graph: {ms_step * 1e3:.1f} us/step (events {ev_ms * 1e3 / steps:.1f})",
          file=sys.stderr, flush=True)

    # per-replay distribution (HIP events around each replay, after the timed
    # region), then the same with the caches flushed before every replay.
    # Reading 512 MiB on the stream ahead of the step (a max over the buffer)
    # evicts L2 and the 256 MB Infinity Cache, so the step starts with every
    # weight in HBM: the state after a target forward pass, which reads its
    # weights and writes little.  An in-place add over the same buffer also
    # leaves the caches full of dirty lines, whose write-back the step then
    # pays as well: reported beside it as the write-flushed case.
    # Each replay of the distribution takes the next of RING pre-drawn rounds
    # (accepted counts, bonus, verify and target tokens), copied into the
    # graph's input buffers ahead of its events, outside the timed replay.
    ring = {k: pb.to_device(np.ascontiguousarray(v)) for k, v in synth.round_ring(w, inp, RING).items()}
    saved = {k: t[k].clone() for k in ring}
    def replay_us(n, flush=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            for k, v in ring.items():
                t[k].copy_(v[i % RING].view_as(t[k]))
            if flush is not None:
                flush()
            a.record(stream)
            pb.pe_step_graph(ctx, B, args)
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    dist = replay_us(min(RING, max(50, steps)))
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    flush_words = flush_buf.view(torch.int32)
    ncold = min(50, max(20, steps // 4))
    cold = replay_us(ncold, lambda: torch.amax(flush_words))
    cold_w = replay_us(ncold, lambda: flush_buf.add_(1))
    del flush_buf, flush_words
    for k in ring:  # the eager and sequential passes below take round 0 again
        t[k].copy_(saved[k])
    err = pb.pe_get_device_error(ctx)
    assert err == (0, -1), f"device error word {err}"
    print(f"[bench] {label} replays: median {np.median(dist):.1f} us, cache-flushed median "
          f"{np.median(cold):.1f} us (write-flushed {np.median(cold_w):.1f} us)", file=sys.stderr, flush=True)

    # the sequential comparison: the same kernels as K drafting passes, one graph
    ar = None
    if with_ar:
        ar_args = pb.make_step_args(t["verify_tokens"], t["verify_positions"], t["num_accepted"],
                                    t["bonus_tokens"], t["block_table"], inp["num_kv_blocks"], batch,
                                    t["target_hidden"], dev["h_shared"], dh, ks, vs, tok,
                                    t["target_tokens"], acc, bon, mode=pb.STEP_AUTOREGRESSIVE)
        ar_steps = max(10, steps // 4)
        for _ in range(max(3, warmup // 4)):
            pb.pe_step_graph(ctx, B, ar_args)
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for _ in range(ar_steps):
            pb.pe_step_graph(ctx, B, ar_args)
        torch.cuda.synchronize()
        ar_ms = (time.perf_counter() - ta) * 1e3 / ar_steps
        err = pb.pe_get_device_error(ctx)
        assert err == (0, -1), f"device error word {err}"
        print(f"[bench] {label} sequential: {ar_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        ar_bytes = ar_work(w, inp)
        ar = {"value": B * K / (ar_ms * 1e-3), "us_per_step": ar_ms * 1e3, "steps": ar_steps,
              "passes": K, "algorithmic_bytes": ar_bytes,
              "hbm_GBs": ar_bytes / (ar_ms * 1e-3) / 1e9,
              "hbm_frac": ar_bytes / (ar_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
              "parallel_speedup": ar_ms / ms_step,
              "mode": "pe_ar_draft: copied slots, then K-1 one-slot passes fed with the drafter's "
                      "residual stream; same kernels, one graph per step"}

    # eager pass with per-phase HIP events on the library's stream
    pb.pe_profile_enable(ctx, True)
    pb.pe_profile_read(ctx, reset=True)
    torch.cuda.synchronize()
    te = time.perf_counter()
    for _ in range(steps):
        pb.pe_prepare(ctx, B, t["verify_tokens"], t["verify_positions"], t["num_accepted"],
                      t["bonus_tokens"], t["block_table"], inp["num_kv_blocks"], batch)
        pb.pe_gather_hidden(ctx, B, batch, t["target_hidden"], dev["h_shared"], dh)
        pb.pe_draft_forward(ctx, B, batch, dh, t["block_table"], inp["num_kv_blocks"], ks, vs, tok)
        pb.pe_verify(ctx, B, tok, t["target_tokens"], acc, bon)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te) * 1e3 / steps
    prof = pb.pe_profile_read(ctx, reset=True)
    pb.pe_profile_enable(ctx, False)
    phases_us = {p: (ms / n * 1e3 if n else 0.0) for p, (ms, n) in prof.items()}
    per_step_us = {p: ms / steps * 1e3 for p, (ms, n) in prof.items()}

    work = step_work(w, inp)
    D = B * K
    lm_us = phases_us["lmhead"]
    lm_bytes = w.vocab * w.d * 2 + D * w.d * 2 + D * 4
    lm_flops = 2 * D * w.vocab * w.d
    if w.batch <= 4:
        roof = {"kernel": "lm_head+argmax", "bound": "hbm",
                "achieved": lm_bytes / (lm_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"kernel": "lm_head+argmax", "bound": "mfma",
                "achieved": lm_flops / (lm_us * 1e-6) / 1e12, "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name)
    roof["avg_launch_us"] = lm_us
    roof["algorithmic_per_launch"] = lm_bytes if roof["bound"] == "hbm" else lm_flops
    step_s = ms_step * 1e-3
    out = {
        "value": B * K / step_s,
        "ms_per_step": ms_step,
        "us_per_step": ms_step * 1e3,
        "event_us_per_step": ev_ms * 1e3 / steps,
        "replay_us": {"replays": int(dist.size), "median": float(np.median(dist)),
                      "p10": float(np.percentile(dist, 10)), "p90": float(np.percentile(dist, 90)),
                      "timing": "HIP events around each graph replay, after the timed steps; replay i takes "
                                f"round i mod {RING} of a pre-drawn ring (accepted counts, bonus, verify and "
                                "target tokens), copied in outside its events"},
        "cache_flushed": {"replays": int(cold.size), "median_us": float(np.median(cold)),
                          "p10_us": float(np.percentile(cold, 10)), "p90_us": float(np.percentile(cold, 90)),
                          "value": B * K / (float(np.median(cold)) * 1e-6),
                          "flush": "max over a 512 MiB buffer on the stream before each replay (not timed): "
                                   "L2 and Infinity Cache hold other, clean data",
                          "write_flushed": {"median_us": float(np.median(cold_w)),
                                            "p10_us": float(np.percentile(cold_w, 10)),
                                            "p90_us": float(np.percentile(cold_w, 90)),
                                            "flush": "512 MiB in-place add before each replay: the caches "
                                                     "also hold dirty lines the step must write back"}},
        "eager_us_per_step": eager_ms * 1e3,
        "roofline": roof,
        "step": {"algorithmic_bytes": work["bytes"], "algorithmic_flops": work["flops"],
                 "hbm_GBs": work["bytes"] / step_s / 1e9,
                 "hbm_frac": work["bytes"] / step_s / 1e9 / HBM_PEAK_GBS,
                 "mfma_TFs": work["flops"] / step_s / 1e12,
                 "mfma_frac": work["flops"] / step_s / 1e12 / MFMA_BF16_PEAK_TFS},
        "autoregressive": ar,
        "phases_us_per_launch": {p: round(v, 2) for p, v in phases_us.items()},
        "phases_us_per_step": {p: round(v, 2) for p, v in per_step_us.items()},
        "config": {"workload": w.name, "batch": B, "K": K, "d": w.d, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "mlp": w.mlp,
                   "layers": w.layers, "vocab": w.vocab, "prefix": list(w.prefix),
                   "mean_seq_len": float((inp["verify_positions"][:, 0] + inp["num_accepted"] + K).mean()),
                   "seed": w.seed, "graph": True},
    }
    ctx.close()
    del kv, t
    torch.cuda.empty_cache()
    return out, prm, dev


def ksweep(steps, warmup):
    """Step cost against draft depth on the deeper drafter (B=16, d=2048,
    32q/4kv x 64, MLP 6144, 4 layers, V=151936, prefix 4096), parallel and
    sequential, same weights at every K."""
    import torch
    from drafting_pe_prepare_amd import binding as pb
    from drafting_pe_prepare_amd import configs, synth
    base = configs.KSWEEP
    prm = synth.weights(base)
    dev = pb.upload_weights(prm)
    rows = []
    for K in base.Ks:
        r, _, _ = measure(base.with_(K=K), steps, warmup, prm=prm, dev=dev, label=f"ksweep K={K}")
        ar = r["autoregressive"]
        rows.append({"K": K, "us_per_step": r["us_per_step"], "draft_tokens_per_s": r["value"],
                     "hbm_frac": r["step"]["hbm_frac"], "mfma_frac": r["step"]["mfma_frac"],
                     "sequential_us_per_step": ar["us_per_step"],
                     "sequential_draft_tokens_per_s": ar["value"],
                     "parallel_speedup": ar["parallel_speedup"],
                     "lm_head_us": r["phases_us_per_step"]["lmhead"],
                     "phases_us_per_step": r["phases_us_per_step"]})
    del dev
    torch.cuda.empty_cache()
    # depth selection from the measured step costs (pe_choose_depth): per-draft
    # acceptance alpha, verifier cost 0 (drafting-bound) or a nominal 2 ms pass
    Ks = [r["K"] for r in rows]
    choice = []
    for fixed in (0.0, 2000.0):
        for alpha in (0.6, 0.7, 0.8, 0.9):
            kp, rp = pb.pe_choose_depth(Ks, [r["us_per_step"] for r in rows], alpha, fixed, 0.0)
            ka, ra = pb.pe_choose_depth(Ks, [r["sequential_us_per_step"] for r in rows], alpha, fixed, 0.0)
            choice.append({"alpha": alpha, "verify_fixed_us": fixed, "parallel_K": kp,
                           "parallel_tokens_per_s": rp * 1e6 * base.batch,
                           "sequential_K": ka, "sequential_tokens_per_s": ra * 1e6 * base.batch})
    return {"workload": base.name, "batch": base.batch, "d": base.d, "layers": base.layers,
            "vocab": base.vocab, "prefix": list(base.prefix), "seed": base.seed, "rows": rows,
            "depth_choice": choice}


def prefill(w, prm, dev, prompt, steps, warmup):
    """The drafting round after a prompt of `prompt` positions (one request,
    the c=1 drafter): prompt positions + NTP + K-1 MASK slots in one pass,
    S padded to a multiple of the 64-slot attention group; eager calls
    (prepare, gather, forward), timed with events on the library's stream."""
    import numpy as np
    import torch
    from drafting_pe_prepare_amd import binding as pb
    from drafting_pe_prepare_amd import synth
    B, K = 1, w.K
    S = (prompt + K - 1 + 63) // 64 * 64
    w1 = w.with_(batch=B)
    inp = synth.prefill_inputs(w1, S, ("fixed", prompt), ("fixed", 0))
    ctx = pb.Context(w1, dev, max_num_seqs=B, max_prefill_slots=B * S)
    t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
         ("chunk_tokens", "chunk_lens", "start_pos", "new_tokens", "block_table", "target_hidden")}
    kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
    ks, vs = [k for k, _ in kv], [v for _, v in kv]
    batch = pb.Batch(B, K, S=S)
    dh = torch.zeros((B * S, w.d), dtype=torch.bfloat16, device="cuda")
    tok = torch.zeros(B * K, dtype=torch.int32, device="cuda")
    nkv = int(inp["num_kv_blocks"])

    def round_():
        pb.pe_prefill_prepare(ctx, B, S, t["chunk_tokens"], t["chunk_lens"], t["start_pos"],
                              t["new_tokens"], t["block_table"], nkv, batch)
        pb.pe_prefill_gather(ctx, B, S, batch, t["target_hidden"], dev["h_shared"], dh)
        pb.pe_prefill_forward(ctx, B, S, batch, dh, t["block_table"], nkv, ks, vs, tok)

    for _ in range(warmup):
        round_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        round_()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    err = pb.pe_get_device_error(ctx)
    assert err == (0, -1), f"device error word {err}"
    pb.pe_profile_enable(ctx, True)
    pb.pe_profile_read(ctx, reset=True)
    for _ in range(max(3, steps // 4)):
        round_()
    prof = pb.pe_profile_read(ctx, reset=True)
    pb.pe_profile_enable(ctx, False)
    n_prof = max(3, steps // 4)
    phases = {p: round(ms / n_prof * 1e3, 2) for p, (ms, n) in prof.items() if n}
    print(f"[bench] prefill {prompt}: {us:.1f} us/round", file=sys.stderr, flush=True)
    valid = prompt + K - 1  # prompt positions 0..prompt-1 (the last is the NTP slot), then K-1 MASK slots
    flops = attention_mlp_flops(w, [list(range(valid))], [list(range(prompt - 1, valid))]) \
        + 2 * B * K * w.vocab * w.d
    ctx.close()
    return {"workload": f"{w.name} drafting round after a {prompt}-position prompt (B=1, K={K}, S={S})",
            "us_per_round": us, "prompt_positions_per_s": prompt / (us * 1e-6),
            "draft_tokens_per_s": B * K / (us * 1e-6), "algorithmic_flops": flops,
            "mfma_TFs": flops / (us * 1e-6) / 1e12,
            "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS,
            "phases_us_per_round": phases, "timing": "eager calls, HIP events, inputs resident"}


def dflash(w, prm, dev, steps, warmup):
    """A DFlash-style round on workload w (same drafter weights, plus seeded
    per-layer injection projections): pe_dflash_prepare, pe_dflash_inject
    (verifier hidden states of the kept context positions into every layer's
    KV cache), pe_dflash_forward (K+1 block slots [bonus, MASK x K], the K
    MASK slots drafting); eager calls, HIP events on the library's stream,
    inputs resident; then the same round as one replayed graph (the timed
    figure)."""
    import numpy as np
    import torch
    from drafting_pe_prepare_amd import binding as pb
    from drafting_pe_prepare_amd import synth
    B, K, d = w.batch, w.K, w.d
    inp = synth.step_inputs(w, extra=2)
    inj_w = synth.inject_weights(w)
    ctx = pb.Context(w, dev, max_num_seqs=B)
    t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
         ("verify_positions", "num_accepted", "bonus_tokens", "block_table", "target_hidden")}
    kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
    ks, vs = [k for k, _ in kv], [v for _, v in kv]
    wk = [pb.to_device(a) for a, _ in inj_w]
    wv = [pb.to_device(b) for _, b in inj_w]
    batch = pb.Batch(B, K, S=K + 1)
    apos = torch.zeros(B * (K + 1), dtype=torch.int32, device="cuda")
    inj = torch.zeros(B * (K + 1), dtype=torch.int64, device="cuda")
    tok = torch.zeros(B * K, dtype=torch.int32, device="cuda")
    nkv = int(inp["num_kv_blocks"])

    def round_():
        pb.pe_dflash_prepare(ctx, B, t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                             t["block_table"], nkv, batch, apos, inj)
        pb.pe_dflash_inject(ctx, B, t["verify_positions"], inj, t["target_hidden"], wk, wv, nkv, ks, vs)
        pb.pe_dflash_forward(ctx, B, batch, apos, t["block_table"], nkv, ks, vs, tok)

    for _ in range(warmup):
        round_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        round_()
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_us = ev0.elapsed_time(ev1) * 1e3 / steps
    # the same round captured once and replayed (pe_step_graph, DFlash mode;
    # greedy verification against seeded target tokens included)
    tt = pb.to_device(np.ascontiguousarray(inp["target_tokens"]))
    acc_o = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon_o = torch.zeros(B, dtype=torch.int32, device="cuda")
    args = pb.make_dflash_step_args(t["verify_positions"], t["num_accepted"], t["bonus_tokens"], t["block_table"],
                                    nkv, batch, t["target_hidden"], ks, vs, wk, wv, apos, inj, tok, tt, acc_o, bon_o)
    for _ in range(warmup):
        pb.pe_step_graph(ctx, B, args)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        pb.pe_step_graph(ctx, B, args)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    err = pb.pe_get_device_error(ctx)
    assert err == (0, -1), f"device error word {err}"
    n_prof = max(3, steps // 4)
    pb.pe_profile_enable(ctx, True)
    pb.pe_profile_read(ctx, reset=True)
    for _ in range(n_prof):
        round_()
    prof = pb.pe_profile_read(ctx, reset=True)
    pb.pe_profile_enable(ctx, False)
    phases = {p: round(ms / n_prof * 1e3, 2) for p, (ms, n) in prof.items() if n}
    print(f"[bench] dflash {w.name}: graph {us:.1f} us/round (eager {eager_us:.1f})", file=sys.stderr, flush=True)
    qd, kvd = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    acc = inp["num_accepted"].astype(np.int64)
    p0 = inp["prefix"].astype(np.int64)
    ctx_len = p0 + acc + K + 2                       # attended positions per request
    layer_w = qd * d + 2 * kvd * d + d * qd + 3 * w.mlp * d
    rows_inj = int((acc + 1).sum())
    # block rows (no fc: embedding input): QKV on all K+1 block slots, and
    # attention, O and MLP on the K draft rows alone in the last layer
    blk = [list(range(K + 1))] * B
    flops = (w.layers * 2 * rows_inj * 2 * kvd * d
             + attention_mlp_flops(w, blk, [list(range(1, K + 1))] * B, ctx_len=[int(c) for c in ctx_len])
             - 2 * B * (K + 1) * 2 * d * d  # no fc in the block pass
             + 2 * B * K * w.vocab * d)
    nbytes = 2 * (w.layers * (2 * kvd * d + layer_w) + w.vocab * d) \
        + 2 * w.layers * 2 * kvd * int(ctx_len.sum())
    ctx.close()
    return {"workload": f"{w.name} DFlash-style round (B={B}, K={K}: {K + 1} block slots, {K} drafts per request)",
            "us_per_round": us, "eager_us_per_round": eager_us, "draft_tokens_per_s": B * K / (us * 1e-6),
            "algorithmic_bytes": nbytes, "hbm_GBs": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_flops": flops, "mfma_TFs": flops / (us * 1e-6) / 1e12,
            "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS,
            "phases_us_per_round": phases,
            "timing": "graph replays (prepare, injection, block pass, greedy verify), HIP events, inputs resident; "
                      "phases from an eager pass"}


def sampling(w, prm, dev, steps, T=1.0):
    """Stochastic drafting and rejection-sampling verification on workload w:
    the parallel forward with logits written, greedy and with Gumbel draws,
    and pe_verify_sampled over those logits and seeded verifier logits (eager
    calls, HIP events on the library's stream, inputs resident)."""
    import numpy as np
    import torch
    from drafting_pe_prepare_amd import binding as pb
    from drafting_pe_prepare_amd import synth
    B, K, V = w.batch, w.K, w.vocab
    inp = synth.step_inputs(w)
    ctx = pb.Context(w, dev, max_num_seqs=B)
    t = {k: pb.to_device(np.ascontiguousarray(inp[k])) for k in
         ("verify_tokens", "verify_positions", "num_accepted", "bonus_tokens", "block_table", "target_hidden")}
    kv = [(pb.to_device(kc), pb.to_device(vc)) for kc, vc in inp["kv"]]
    ks, vs = [k for k, _ in kv], [v for _, v in kv]
    batch = pb.Batch(B, K)
    nkv = int(inp["num_kv_blocks"])
    dh = torch.zeros((B * 2 * K, w.d), dtype=torch.bfloat16, device="cuda")
    tok = torch.zeros(B * K, dtype=torch.int32, device="cuda")
    lg = torch.zeros((B * K, V), dtype=torch.float32, device="cuda")
    tl = synth.normal(w.seed, "verifier_logits", (B * (K + 1), V), 2.0, dtype="f32")
    tl = pb.to_device(np.ascontiguousarray(tl))
    seed = torch.tensor([12345], dtype=torch.int64, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    pb.pe_prepare(ctx, B, t["verify_tokens"], t["verify_positions"], t["num_accepted"], t["bonus_tokens"],
                  t["block_table"], nkv, batch)
    pb.pe_gather_hidden(ctx, B, batch, t["target_hidden"], dev["h_shared"], dh)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    greedy = timed(lambda: pb.pe_draft_forward(ctx, B, batch, dh, t["block_table"], nkv, ks, vs, tok, lg))
    sampled = timed(lambda: pb.pe_draft_forward_sampled(ctx, B, batch, dh, t["block_table"], nkv, ks, vs,
                                                        T, seed, tok, lg))
    verify = timed(lambda: pb.pe_verify_sampled(ctx, B, tok, lg, tl, T, seed, acc, nxt))
    err = pb.pe_get_device_error(ctx)
    assert err == (0, -1), f"device error word {err}"
    ctx.close()
    vbytes = B * (2 * K + 2) * V * 4  # log-sum-exp over every row, then at least one emitting row
    print(f"[bench] sampling {w.name}: forward {greedy:.1f} -> {sampled:.1f} us, verify {verify:.1f} us",
          file=sys.stderr, flush=True)
    return {"workload": w.name, "temperature": T,
            "forward_with_logits_greedy_us": greedy, "forward_with_logits_sampled_us": sampled,
            "verify_sampled_us": verify,
            "verify_bytes_min": vbytes, "verify_GBs": vbytes / (verify * 1e-6) / 1e9,
            "timing": "eager calls, HIP events, inputs resident; verifier logits seeded N(0, 2)"}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------
def cpu_baseline(w, prm, seconds):
    import numpy as np
    import oracle as O
    from drafting_pe_prepare_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    inp = synth.step_inputs(w)
    n, t0 = 0, time.perf_counter()
    while True:
        b = O.prepare(inp["verify_tokens"], inp["verify_positions"], inp["num_accepted"],
                      inp["bonus_tokens"], inp["block_table"], inp["num_kv_blocks"], w.K,
                      w.vocab, w.mask_id, w.block_size)
        hd = O.gather_hidden(b["hidden_src"], inp["target_hidden"], prm["h_shared"])
        fw = O.draft_forward(prm, w, b, hd, inp["kv"], inp["block_table"], "bf16", want_logits=False)
        O.verify(fw["tokens"].reshape(w.batch, w.K), inp["target_tokens"])
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or el / n * (n + 1) > 3 * seconds:
            break
    return {"value": w.batch * w.K * n / el, "unit": "draft tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} full {w.name} step(s) (B={w.batch}, K={w.K}; prepare+gather+forward"
                      f"+verify, fp64 with bf16 storage rounding) in {el:.1f}s"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request across GPUs with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from drafting_pe_prepare_amd import binding as pb
    from drafting_pe_prepare_amd import configs
    pb.load()
    assert torch.cuda.is_available(), "no GPU"
    w = configs.BY_NAME[args.workload]
    main_res, prm, dev = measure(w, args.steps, args.warmup, label=w.name, with_ar=not args.no_ar)
    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "us_per_step": main_res["us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hidden/KV; no trained weights)",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
        "step": main_res["step"],
        "phases_us_per_step": main_res["phases_us_per_step"],
        "event_us_per_step": main_res["event_us_per_step"],
        "eager_us_per_step": main_res["eager_us_per_step"],
        "replay_us": main_res["replay_us"],
        "cache_flushed": main_res["cache_flushed"],
        "autoregressive": main_res["autoregressive"],
    }
    if not args.no_c64 and w.name == "c1_20b":
        c64, _, _ = measure(configs.C64, max(20, args.steps // 4), max(5, args.warmup // 4),
                            prm=prm, dev=dev, label="c64_20b", with_ar=not args.no_ar)
        line["c64"] = {k: c64[k] for k in ("value", "us_per_step", "roofline", "step", "replay_us",
                                            "cache_flushed", "autoregressive", "phases_us_per_step", "config")}
        line["c64"]["config"]["weights"] = "same drafter weights as the c=1 workload"
    if not args.no_maxbatch and w.name == "c1_20b":
        mb, _, _ = measure(configs.MAXB, max(10, args.steps // 10), 3, prm=prm, dev=dev,
                           label="maxbatch_20b", with_ar=False)
        line["maxbatch"] = {k: mb[k] for k in ("value", "us_per_step", "step", "phases_us_per_step", "replay_us",
                                               "cache_flushed", "config")}
        line["maxbatch"]["config"]["weights"] = "same drafter weights as the c=1 workload"
    if not args.no_ksweep and w.name == "c1_20b":
        line["ksweep"] = ksweep(max(20, args.steps // 5), max(3, args.warmup // 4))
    if not args.no_sampling and w.name == "c1_20b":
        line["sampling"] = {"c1": sampling(w, prm, dev, max(10, args.steps // 10)),
                            "c64": sampling(configs.C64, prm, dev, max(5, args.steps // 20))}
    if not args.no_prefill and w.name == "c1_20b":
        line["prefill"] = prefill(w, prm, dev, 2048, max(10, args.steps // 10), 3)
    if not args.no_dflash and w.name == "c1_20b":
        line["dflash"] = {"c1": dflash(w, prm, dev, max(20, args.steps // 5), 3),
                          "c64": dflash(configs.C64, prm, dev, max(10, args.steps // 10), 3)}
    if not args.no_cpu_baseline:
        del dev
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline(w, prm, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line, default=lambda o: o.item() if hasattr(o, "item") else str(o)), flush=True)


if __name__ == "__main__":
    main()
