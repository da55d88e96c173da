#!/usr/bin/env python3
"""Benchmark of the DSpine draft round on one MI355X.

One step is one speculative round of the hot path for B requests: the
library materializes the context features that the previous round committed
(W = 16 positions per request: feature fusion, K/V projection, ring store),
then runs one masked-block draft forward (embedding gather, 5 layers of
attention + SwiGLU + bridge, final norm).  Inputs are seeded synthetic
tensors of the workload's geometry, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is draft forwards per second (each forward
covers B blocks).  ``roofline`` reports the dominant kernel (the gate/up
projection, about half of all bytes a step reads) against MI355X's HBM
bandwidth, timed with HIP events on the library's stream inside the timed
region.  ``cpu_baseline`` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes(wts, names):
    return sum(int(wts[n].nbytes) for n in names if n in wts)


def step_algorithmic_bytes(g, wts, B, W, frontiers, commit):
    """Bytes one step must move at least: every weight the forward and the
    materializer read once, visible context K/V, features, ring writes."""
    L = g.n_layers
    per_layer = ["g_in", "wq", "wk", "wv", "gq", "gk", "wo", "g_post", "w_gate", "w_up", "w_down"]
    if g.bridge:
        per_layer += ["R", "W_l"]
    if getattr(g, "conv", False):
        per_layer += ["attn_conv_w", "attn_conv_base", "mlp_conv_w", "mlp_conv_base"]
    fwd = sum(weight_bytes(wts, [f"l{l}.{n}" for n in per_layer]) for l in range(L))
    fwd += weight_bytes(wts, ["g_final"])
    elt = 2 if g.dtype == "bf16" else 4
    if g.bridge:
        fwd += L * weight_bytes(wts, ["bridge_G", "bridge_Gp", "bridge_A", "bridge_b"])
        fwd += L * B * g.code_dim * elt                    # anchor codebook rows
    fwd += B * 2 * g.hidden * elt                          # anchor + mask embedding rows
    ctx = 0
    for l in range(L):
        S = g.windows[l]
        for F in frontiers:
            n = F if S == 0 else min(F, S - 1)             # row 0 sees the most keys
            ctx += n * g.kv_dim * 2 * elt
    mat = weight_bytes(wts, ["w_feat", "g_ctx"]) + sum(
        weight_bytes(wts, [f"l{l}.wk", f"l{l}.wv", f"l{l}.gk"]) for l in range(L))
    mat += B * commit * g.n_feat_layers * g.hidden * elt   # committed features
    mat += B * commit * L * g.kv_dim * 2 * elt             # ring writes
    out = B * W * g.hidden * 4
    return fwd + ctx + mat + out, fwd, ctx, mat


def cpu_baseline(g, wts, seed, F, commit, W, anchor):
    """The oracle, as it stands, on one request: the context is set up untimed
    (its live window), then one step (materialize `commit` positions + one
    B=1 forward) is timed once."""
    import numpy as np
    import synth
    from oracle import dspine_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()
                       if d.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    keep = min(F, max(s for s in g.windows)) if all(s > 0 for s in g.windows) else F
    ctx = O.materialize(g, wts, O.empty_context(g, F - keep),
                        synth.make_features(g, seed, 0, keep, start=F - keep))
    feats = synth.make_features(g, seed, 0, commit, start=F)
    t0 = time.perf_counter()
    ctx = O.materialize(g, wts, ctx, feats)
    O.draft_forward(g, wts, [ctx], [anchor], W)
    dt = time.perf_counter() - t0
    return dt, threads


MFMA_PEAK_TFLOPS = 2500.0          # MI355X dense bf16/fp16 matrix-core peak


def prefill_measure(model, g, seed, n_req=8, chunk=32768, reps=5):
    """One materialize call over n_req fresh rings, each given a chunk of
    `chunk` feature rows: only a chunk's final S rows are stored (and read),
    the frontier advances by the whole chunk.  Returns the prefill record."""
    import torch
    import synth
    import block_drafter_amd as bd
    S = max(g.windows)
    keep = min(chunk, S) if all(w > 0 for w in g.windows) else chunk
    width = g.n_feat_layers * g.hidden
    chunks = []
    for b in range(n_req):
        t = torch.empty((chunk, width), dtype=torch.bfloat16, device="cuda")
        t[chunk - keep:] = bd.to_device(synth.make_features(g, seed, b, keep, start=chunk - keep))
        chunks.append(t)
    ctxs = [model.new_context() for _ in range(n_req)]
    ws = model.workspace(n_req, 16, n_req * keep)
    torch.cuda.synchronize()

    def call():
        for c in ctxs:
            c.frontier = 0
        model.materialize(ctxs, chunks, workspace=ws)

    call()                                    # warm-up (twice: the first pass over
    call()                                    # fresh chunk memory also warms translations)
    torch.cuda.synchronize()
    bd.profile_enable(["ctx_gemm", "ctx_store"])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    bd.profile_enable([])
    ms = e0.elapsed_time(e1) / reps
    gemm_ms, gemm_n = bd.profile_read("ctx_gemm")
    store_ms, _ = bd.profile_read("ctx_store")
    kvd = g.n_kv_heads * g.head_dim
    flop = n_req * keep * 2.0 * g.hidden * (width + g.n_layers * 2 * kvd)   # a1 + a2 per call
    gemm_avg = gemm_ms / reps
    tflops = flop / (gemm_avg * 1e-3) / 1e12
    del chunks
    torch.cuda.empty_cache()
    return {
        "workload": f"{n_req} requests x one {chunk}-token chunk into fresh {S}-slot rings "
                    f"({keep} stored rows each), one materialize call",
        "ms_per_call": round(ms, 4),
        "chunk_tok_per_s": round(n_req * chunk / (ms * 1e-3), 1),
        "stored_tok_per_s": round(n_req * keep / (ms * 1e-3), 1),
        "gemm_ms_per_call": round(gemm_avg, 4),
        "store_ms_per_call": round(store_ms / reps, 4),
        "roofline": {
            "kernel": "gemm_tile (feature fusion W_feat + K/V projection of every layer)",
            "bound": "mfma",
            "achieved": round(tflops, 1),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
            "flop_per_call": flop,
            "launches_per_call": gemm_n // reps,
        },
    }


def prefill_noskip_measure(g, wts, seed, n_req=8, chunk=32768, reps=2):
    """The materializer without the window skip: the same weights under a
    geometry whose layers are all full attention, so every one of the
    n_req x chunk positions is fused, projected and stored.  Features are
    seeded N(0,1) bf16 drawn on the device (only the timing is used)."""
    import torch
    import synth
    import block_drafter_amd as bd
    gfull = synth.with_geometry(g, windows=(0,) * g.n_layers)
    model = bd.Model.from_numpy(gfull, wts)
    width = g.n_feat_layers * g.hidden
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    chunks = [torch.randn((chunk, width), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(n_req)]
    ctxs = [model.new_context(full_capacity=chunk) for _ in range(n_req)]
    ws = model.workspace(n_req, 16, 16384)

    def call():
        for c in ctxs:
            c.frontier = 0
        model.materialize(ctxs, chunks, workspace=ws)

    call()
    torch.cuda.synchronize()
    bd.profile_enable(["ctx_gemm"])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    bd.profile_enable([])
    ms = e0.elapsed_time(e1) / reps
    gemm_ms, _ = bd.profile_read("ctx_gemm")
    kvd = g.n_kv_heads * g.head_dim
    flop = n_req * chunk * 2.0 * g.hidden * (width + g.n_layers * 2 * kvd)
    tflops = flop / (gemm_ms / reps * 1e-3) / 1e12
    model.close()
    del chunks, ctxs, ws, model
    torch.cuda.empty_cache()
    return {
        "workload": f"{n_req} requests x one {chunk}-token chunk, every position stored (all layers full "
                    f"attention), materialized in blocks of 16384 rows",
        "ms_per_call": round(ms, 3),
        "chunk_tok_per_s": round(n_req * chunk / (ms * 1e-3), 1),
        "gemm_ms_per_call": round(gemm_ms / reps, 3),
        "flop_per_call": flop,
        "achieved_tflops": round(tflops, 1),
        "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
    }


def propose_measure(model, g, ctxs, anchors, W, ws, steps, fwd_ms, K=16):
    """One dspine_draft_propose call per step (the forward, then head scores,
    top-16, the refinement table and the greedy walk), timed over `steps`
    calls; the LM head's score GEMM is timed by its own event pairs.  Its
    roofline is HBM: the bf16 head is read once per call."""
    import torch
    import block_drafter_amd as bd
    B = len(ctxs)
    pws = model.propose_workspace(B, W, K)
    o = model.propose(ctxs, anchors, W, K, workspace=ws, propose_workspace=pws)
    for _ in range(3):
        model.propose(ctxs, anchors, W, K, workspace=ws, propose_workspace=pws, outputs=o)
    torch.cuda.synchronize()
    bd.profile_enable(["head", "tail"])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        model.propose(ctxs, anchors, W, K, workspace=ws, propose_workspace=pws, outputs=o)
    e1.record()
    torch.cuda.synchronize()
    bd.profile_enable([])
    ms = e0.elapsed_time(e1) / steps
    head_ms, head_n = bd.profile_read("head")
    tail_ms, _ = bd.profile_read("tail")
    elt = 2 if g.dtype == "bf16" else 4
    M = B * W
    head_bytes = g.vocab * g.hidden * elt + M * g.hidden * 4 + M * g.vocab * 4
    head_avg = head_ms / max(1, head_n)
    achieved = head_bytes / (head_avg * 1e-3) / 1e9
    return {
        "workload": f"one draft forward + proposal tail, B={B}, W={W}, top-{K}, greedy walk, "
                    f"{g.vocab}-row bf16 LM head",
        "ms_per_call": round(ms, 4),
        "proposals_per_s": round(1000.0 / ms, 3),
        "tail_ms": round(ms - fwd_ms, 4),
        "head_ms": round(head_avg, 4),
        "refine_walk_ms": round(tail_ms / steps, 4),
        "roofline": {
            "kernel": "gemm_stream (LM head scores of every row)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "bytes_per_launch": head_bytes,
            "avg_launch_us": round(head_avg * 1000, 2),
            "launches": head_n,
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dspine27b_b1",
                    choices=["dspine27b_b1", "dspine27b_b8", "dspine27b_causal_b8", "dflash35b_b8",
                             "dflash2_27b_b8", "tiny_fp32"])
    ap.add_argument("--commit", type=int, default=16,
                    help="positions materialized per request per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the context-prefill measurement (27B workloads)")
    ap.add_argument("--no-propose", action="store_true",
                    help="skip the proposal-tail measurement (workloads with a bridge)")
    ap.add_argument("--breakdown", action="store_true",
                    help="after the timed region, time every kernel class for a few steps")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times and exit (calibrates "
                         "hardware byte counters against a known traffic)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        n = args.copy_probe // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the draft round is "
              "data-parallel over requests with no exchange, so N GPUs would run N independent "
              "copies.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import block_drafter_amd as bd

    bd.lib()                                  # fails loudly without the built library
    wl = synth.WORKLOADS[args.workload]
    g, B, W = wl.geom, wl.B, wl.W
    frontiers = list(wl.frontiers)
    total_steps = args.warmup + args.steps
    log(f"workload {wl.name}: B={B} W={W} frontiers={frontiers}")

    t = time.time()
    wts = synth.make_weights(g, wl.seed)
    log(f"weights generated in {time.time() - t:.1f}s")
    # the shared LM head of the proposal tail (packed with the projections)
    with_propose = bool(g.bridge) and not args.no_propose
    head = synth.make_lm_head(g, wl.seed) if with_propose else None
    t = time.time()
    model = bd.Model.from_numpy(g, wts, lm_head=head)
    del head
    torch.cuda.synchronize()
    log(f"weights uploaded in {time.time() - t:.1f}s")
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, B)]

    # contexts: the live window of every local layer holds the last S positions
    # before F (a chunk longer than the ring stores only its final window), so
    # the setup materializes exactly those positions from frontier F - S.
    full = any(s == 0 for s in g.windows)
    smax = max(g.windows)
    extra_steps = min(5, total_steps) if args.breakdown else 0   # the breakdown pass below
    ctxs, pending = [], []
    for b, F in enumerate(frontiers):
        cap = (F + args.commit * (total_steps + extra_steps) + 16) if full else 0
        c = model.new_context(full_capacity=cap)
        keep = F if full else min(F, smax)
        c.frontier = F - keep
        feats = bd.to_device(synth.make_features(g, wl.seed, b, keep, start=F - keep))
        model.materialize([c], [feats], workspace=model.workspace(B, W, max(keep, 256)))
        del feats
        pending.append(bd.to_device(synth.make_features(g, wl.seed, b, args.commit * total_steps, start=F)))
        ctxs.append(c)
    torch.cuda.synchronize()
    ws = model.workspace(B, W, max(256, args.commit * B))
    out = torch.empty((B, W, g.hidden), dtype=torch.float32, device="cuda")
    log("contexts ready")

    def step(i):
        fs = [p[i * args.commit:(i + 1) * args.commit] for p in pending]
        model.materialize(ctxs, fs, workspace=ws)
        model.forward(ctxs, anchors, W, out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    step_bytes, fwd_bytes, ctx_bytes, mat_bytes = step_algorithmic_bytes(
        g, wts, B, W, [c.frontier for c in ctxs], args.commit)

    # the gate/up launches are timed live, on a sample: every 6th launch (a
    # stride prime to the 5 layers, so the sample rotates through them); each
    # timed launch idles the GPU for a few microseconds around its events
    bd.profile_stride(6)
    bd.profile_enable(["gemm_gate_up"])
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    t0 = time.perf_counter()
    for i in range(args.warmup, total_steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    bd.profile_enable([])
    bd.profile_stride(1)
    gpu_ms = ev0.elapsed_time(ev1)
    gu_ms, gu_n = bd.profile_read("gemm_gate_up")
    ms_per_step = gpu_ms / args.steps
    value = 1000.0 / ms_per_step

    # dominant kernel: the gate/up projection of one layer
    elt = 2 if g.dtype == "bf16" else 4
    M = B * W
    gu_bytes = 2 * g.ffn * g.hidden * elt + M * g.hidden * elt + M * g.ffn * elt
    gu_avg_ms = gu_ms / max(1, gu_n)
    achieved = gu_bytes / (gu_avg_ms * 1e-3) / 1e9

    # the draft forward alone (same inputs, after the timed steps)
    fwd_ev0 = torch.cuda.Event(enable_timing=True)
    fwd_ev1 = torch.cuda.Event(enable_timing=True)
    fwd_ev0.record()
    for _ in range(args.steps):
        model.forward(ctxs, anchors, W, out=out, workspace=ws)
    fwd_ev1.record()
    torch.cuda.synchronize()
    fwd_ms = fwd_ev0.elapsed_time(fwd_ev1) / args.steps

    propose = None
    if with_propose:
        propose = propose_measure(model, g, ctxs, anchors, W, ws, args.steps, fwd_ms)
        propose["roofline"]["traffic"] = None
        if wl.name == "dspine27b_b1":
            from block_drafter_amd import profsum
            rec = profsum.read_traffic(os.path.join(ROOT, "profiles", "traffic_gemm_stream_lm_head_dspine27b_b1.md"))
            if rec is not None and rec[1] == profsum.source_hash():
                propose["roofline"]["traffic"] = rec[0]

    # HBM traffic of the same kernel from the PMC runs summarised under
    # profiles/ (null unless they were taken on this workload with the
    # current kernel sources)
    traffic = None
    if wl.name == "dspine27b_b1":
        from block_drafter_amd import profsum
        rec = profsum.read_traffic(os.path.join(ROOT, "profiles", "traffic_gemm_stream_gate_up_dspine27b_b1.md"))
        if rec is not None and rec[1] == profsum.source_hash():
            traffic = rec[0]

    breakdown = None
    if args.breakdown:
        bd.profile_enable(bd.PROF_KINDS)
        for i in range(min(5, total_steps)):
            step(i % total_steps)
        torch.cuda.synchronize()
        bd.profile_enable([])
        breakdown = {}
        for k in bd.PROF_KINDS:
            ms, n = bd.profile_read(k)
            breakdown[k] = {"ms_per_step": round(ms / min(5, total_steps), 4), "launches_per_step": n // min(5, total_steps)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one request's step ...")
        dt, threads = cpu_baseline(g, wts, wl.seed, frontiers[0], args.commit, W, anchors[0])
        cpu = {"value": round(1.0 / (dt * B), 6), "unit": "forwards/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"one step of request 0 (materialize {args.commit} positions + one "
                         f"B=1 forward, float64 numpy), timed once; forwards/s = 1 / ({B} x "
                         f"{dt:.2f} s)"}

    res = {
        "metric": "draft-block forwards/s at 27B geometry (B=1,8); ctx-prefill tok/s; % roofline",
        "value": round(value, 3),
        "unit": "forwards/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": g.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": B, "W": W, "context": frontiers, "layers": g.n_layers,
            "hidden": g.hidden, "windows": list(g.windows), "bridge": bool(g.bridge),
            "step": f"materialize {args.commit} committed positions per request + one draft forward",
            "blocks_per_s": round(value * B, 3),
            "step_algorithmic_bytes": step_bytes,
            "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
            "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "bytes_forward_weights": fwd_bytes, "bytes_context_kv": ctx_bytes,
            "bytes_materialize": mat_bytes, "wall_s": round(wall, 3),
            "forward_only_ms": round(fwd_ms, 4),
            "forward_only_per_s": round(1000.0 / fwd_ms, 3),
            "forward_only_GBps": round((fwd_bytes + ctx_bytes + B * W * g.hidden * 4) / (fwd_ms * 1e-3) / 1e9, 1),
            "operands": "bf16 weights widened to fp16 in registers x fp16 activations, fp32 accumulate",
        },
        "roofline": {
            "kernel": "gemm_stream (gate/up projection + SwiGLU)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM, PMC FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_avg_ms * 1000, 2),
            "launches": gu_n,
        },
        "cpu_baseline": cpu,
    }
    if breakdown is not None:
        res["breakdown"] = breakdown
    if propose is not None:
        res["propose"] = propose
    if not args.no_prefill and g.dtype == "bf16" and g.hidden == 5120:
        del ctxs, pending, ws
        torch.cuda.empty_cache()
        log("context prefill: 8 requests x one 32768-token chunk ...")
        pw = synth.WORKLOADS["prefill27b"]
        res["prefill"] = prefill_measure(model, g, pw.seed, n_req=pw.B, chunk=pw.prefill_chunk)
        log("context prefill without the window skip ...")
        res["prefill"]["no_skip"] = prefill_noskip_measure(g, wts, pw.seed, n_req=pw.B, chunk=pw.prefill_chunk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
