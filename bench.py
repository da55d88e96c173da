#!/usr/bin/env python3
"""Benchmark of the DSpine draft round on one MI355X.

One step is one speculative round of the hot path for B requests: the
library materializes the context features that the previous round committed
(W = 16 positions per request: feature fusion, K/V projection, ring store),
then runs one masked-block draft forward (embedding gather, 5 layers of
attention + SwiGLU + bridge, final norm).  Inputs are seeded synthetic
tensors of the workload's geometry, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is draft forwards per second (each forward
covers B blocks) of the headline workload (27B geometry, B=1).  ``roofline``
reports the dominant kernel (the gate/up projection, about half of all bytes
a step reads) against MI355X's HBM bandwidth, timed with HIP events on the
library's stream inside the timed region.  ``cpu_baseline`` times the CPU
oracle on a bounded sample.  With the default workload the same line also
carries ``b8`` (the 27B geometry at B=8, the other half of the metric) and
``dflash35b_b8`` (the 35B-style plain DFlash drafter at B=8), each with the
same step, forward-only and gate/up roofline fields, ``propose`` (forward
plus proposal tail) and ``prefill`` (context materialization of 8 x 32768
positions).
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


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if info:
            return max(d.get("num_threads", 1) for d in info), info[0].get("internal_api", "blas")
    except Exception:
        pass
    return os.cpu_count() or 1, "unknown"


def cpu_baseline(g, wts, seed, frontiers, commit, W, anchors, repeats=3, warmup=1):
    """The oracle, as it stands, on the workload's step: every request's
    context is set up untimed (its live window), then one step (materialize
    `commit` positions of every request + one forward over all of them) is
    run `warmup` times untimed and `repeats` times timed; the median is
    returned with the individual times."""
    import numpy as np
    import synth
    from oracle import dspine_oracle as O
    threads, api = _blas_threads()
    ctxs0 = []
    for b, F in enumerate(frontiers):
        keep = min(F, max(s for s in g.windows)) if all(s > 0 for s in g.windows) else F
        ctxs0.append(O.materialize(g, wts, O.empty_context(g, F - keep),
                                   synth.make_features(g, seed, b, keep, start=F - keep)))
    feats = [synth.make_features(g, seed, b, commit, start=F) for b, F in enumerate(frontiers)]

    def step():
        ctxs = [O.materialize(g, wts, c, f) for c, f in zip(ctxs0, feats)]
        O.draft_forward(g, wts, ctxs, list(anchors), W)

    for _ in range(warmup):
        step()
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), times, threads, api


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
    call_tflops = flop / (ms * 1e-3) / 1e12
    return {
        "workload": f"{n_req} requests x one {chunk}-token chunk into fresh {S}-slot rings "
                    f"({keep} stored rows each), one materialize call",
        "ms_per_call": round(ms, 4),
        "computed_tok_per_s": round(n_req * keep / (ms * 1e-3), 1),
        "computed_tok_note": f"positions fused, projected and stored per second: the final {keep} of "
                             f"each chunk, the only ones any layer's window keeps",
        "chunk_advance_tok_per_s": round(n_req * chunk / (ms * 1e-3), 1),
        "gemm_ms_per_call": round(gemm_avg, 4),
        "store_ms_per_call": round(store_ms / reps, 4),
        "roofline": {
            "kernel": "whole materialize call (feature fusion W_feat + K/V projection tile GEMMs, "
                      "context norm, head norm + RoPE + ring store)",
            "bound": "mfma",
            "achieved": round(call_tflops, 1),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(call_tflops / MFMA_PEAK_TFLOPS, 4),
            "flop_per_call": flop,
        },
        "gemm_only": {
            "kernel": "gemm_tile (W_feat + K/V projection of every layer), HIP events around its launches",
            "achieved": round(tflops, 1),
            "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
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


def propose_measure(model, g, ctxs, anchors, W, ws, steps, fwd_ms, K=16, retrieve=0):
    """One dspine_draft_propose call per step (the forward, then head scores,
    top-16, the refinement table and the greedy walk), timed over `steps`
    calls; the LM head's score GEMM is timed by its own event pairs.  Its
    roofline is HBM: the head is read once per call (bf16, or with
    ``retrieve`` its FP8 copy and row scales, then the retrieval of
    ``retrieve`` candidates per row and their BF16 rescoring)."""
    import torch
    import block_drafter_amd as bd
    B = len(ctxs)
    pws = model.propose_workspace(B, W, K)
    o = model.propose(ctxs, anchors, W, K, workspace=ws, propose_workspace=pws, retrieve=retrieve)
    for _ in range(3):
        model.propose(ctxs, anchors, W, K, workspace=ws, propose_workspace=pws, outputs=o, retrieve=retrieve)
    torch.cuda.synchronize()
    bd.profile_enable(["head", "tail"])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        model.propose(ctxs, anchors, W, K, workspace=ws, propose_workspace=pws, outputs=o, retrieve=retrieve)
    e1.record()
    torch.cuda.synchronize()
    bd.profile_enable([])
    ms = e0.elapsed_time(e1) / steps
    head_ms, head_n = bd.profile_read("head")
    tail_ms, _ = bd.profile_read("tail")
    elt = 2 if g.dtype == "bf16" else 4
    M = B * W
    if retrieve:
        head_bytes = g.vocab * g.hidden + 4 * g.vocab + M * g.hidden * 4 + M * g.vocab * 4
    else:
        head_bytes = g.vocab * g.hidden * elt + M * g.hidden * 4 + M * g.vocab * 4
    head_avg = head_ms / max(1, head_n)
    achieved = head_bytes / (head_avg * 1e-3) / 1e9
    how = (f"FP8 row-scaled retrieval of {retrieve} candidates per row, BF16 rescoring" if retrieve
           else "direct bf16 LM head")
    return {
        "workload": f"one draft forward + proposal tail, B={B}, W={W}, top-{K}, greedy walk, "
                    f"{g.vocab}-row LM head: {how}",
        "ms_per_call": round(ms, 4),
        "proposals_per_s": round(1000.0 / ms, 3),
        "tail_ms": round(ms - fwd_ms, 4),
        "head_ms": round(head_avg, 4),
        "refine_walk_ms": round(tail_ms / steps, 4),
        "roofline": {
            "kernel": ("gemm_stream (FP8 LM head scores of every row)" if retrieve
                       else "gemm_stream (LM head scores of every row)"),
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


def measure_workload(name, args, with_propose, gate_up_traffic_md=None):
    """Times one forward workload: `args.warmup` untimed steps, then
    `args.steps` timed steps (materialize the committed positions of every
    request + one draft forward), the gate/up GEMM timed live on a sample of
    its launches, then the forward alone and (with a bridge) the proposal
    call.  Returns (record, state) where state keeps what later legs reuse."""
    import torch
    import synth
    import block_drafter_amd as bd
    wl = synth.WORKLOADS[name]
    g, B, W = wl.geom, wl.B, wl.W
    frontiers = list(wl.frontiers)
    total_steps = args.warmup + args.steps
    log(f"workload {wl.name}: B={B} W={W} frontiers={frontiers}")

    t = time.time()
    wts = synth.make_weights(g, wl.seed)
    log(f"weights generated in {time.time() - t:.1f}s")
    with_propose = with_propose and bool(g.bridge)
    head = synth.make_lm_head(g, wl.seed) if with_propose else None
    t = time.time()
    model = bd.Model.from_numpy(g, wts, lm_head=head)
    del head
    torch.cuda.synchronize()
    log(f"weights uploaded in {time.time() - t:.1f}s")
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, B)]

    # contexts: the live window of every local layer holds the last S positions
    # before F (a chunk longer than the ring stores only its final window), so
    # the setup materializes exactly those positions from frontier F - S.  A
    # full-attention layer needs every position: those contexts are
    # materialized in full.
    full = any(s == 0 for s in g.windows)
    smax = max(g.windows)
    extra_steps = min(5, total_steps) if args.breakdown else 0   # the breakdown pass below
    ctxs, pending = [], []
    setup_ws = None
    for b, F in enumerate(frontiers):
        cap = (F + args.commit * (total_steps + extra_steps) + 16) if full else 0
        c = model.new_context(full_capacity=cap)
        keep = F if full else min(F, smax)
        c.frontier = F - keep
        for s0 in range(0, keep, 16384):
            n = min(16384, keep - s0)
            feats = bd.to_device(synth.make_features(g, wl.seed, b, n, start=F - keep + s0))
            setup_ws = model.workspace(B, W, max(n, 256))
            model.materialize([c], [feats], workspace=setup_ws)
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
    fwd_total_bytes = fwd_bytes + ctx_bytes + B * W * g.hidden * 4
    fwd_gbps = fwd_total_bytes / (fwd_ms * 1e-3) / 1e9

    propose = None
    if with_propose:
        propose = propose_measure(model, g, ctxs, anchors, W, ws, args.steps, fwd_ms)
        if g.dtype == "bf16":
            propose["fp8_retrieval"] = propose_measure(model, g, ctxs, anchors, W, ws, args.steps, fwd_ms,
                                                       retrieve=128)
            propose["fp8_retrieval"]["roofline"]["traffic"] = None
        propose["roofline"]["traffic"] = None
        if wl.name == "dspine27b_b1":
            from block_drafter_amd import profsum
            for rec_key, md in ((None, "traffic_gemm_stream_lm_head_dspine27b_b1.md"),
                                ("fp8_retrieval", "traffic_gemm_stream_fp8_head_dspine27b_b1.md")):
                rec = profsum.read_traffic(os.path.join(ROOT, "profiles", md))
                if rec is not None and rec[1] == profsum.source_hash() and (rec_key is None or rec_key in propose):
                    (propose if rec_key is None else propose[rec_key])["roofline"]["traffic"] = rec[0]

    # HBM traffic of the same kernel from the PMC runs summarised under
    # profiles/ (null unless they were taken on this workload with the
    # current kernel sources)
    traffic = None
    if gate_up_traffic_md is not None:
        from block_drafter_amd import profsum
        rec = profsum.read_traffic(os.path.join(ROOT, "profiles", gate_up_traffic_md))
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
            breakdown[k] = {"ms_per_step": round(ms / min(5, total_steps), 4),
                            "launches_per_step": n // min(5, total_steps)}

    rec = {
        "workload": wl.name, "B": B, "W": W, "context": frontiers, "layers": g.n_layers,
        "hidden": g.hidden, "windows": list(g.windows), "bridge": bool(g.bridge),
        "block_causal": bool(g.block_causal),
        "step": f"materialize {args.commit} committed positions per request + one draft forward",
        "steps_per_s": round(value, 3),
        "ms_per_step": round(ms_per_step, 4),
        "blocks_per_s": round(value * B, 3),
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_forward_weights": fwd_bytes, "bytes_context_kv": ctx_bytes,
        "bytes_materialize": mat_bytes, "wall_s": round(wall, 3),
        "forward_only_ms": round(fwd_ms, 4),
        "forward_only_per_s": round(1000.0 / fwd_ms, 3),
        "forward_only_bytes": fwd_total_bytes,
        "forward_only_GBps": round(fwd_gbps, 1),
        "forward_only_hbm_frac": round(fwd_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {
            "kernel": f"gemm_stream (gate/up projection + SwiGLU, M={M})",
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
    }
    if breakdown is not None:
        rec["breakdown"] = breakdown
    if propose is not None:
        rec["propose"] = propose
    state = {"wl": wl, "g": g, "wts": wts, "model": model, "anchors": anchors, "frontiers": frontiers}
    del ctxs, pending, ws, out, setup_ws
    return rec, state


def release(state):
    import torch
    state["model"].close()
    state.clear()
    torch.cuda.empty_cache()


def oracle_record(g, wts, wl, args, anchors, note, repeats=3, warmup=1):
    log(f"timing the CPU oracle on the {wl.name} step ...")
    med, times, threads, api = cpu_baseline(g, wts, wl.seed, list(wl.frontiers), args.commit, wl.W, anchors,
                                            repeats=repeats, warmup=warmup)
    how = (f"{warmup} warm-up run(s) then {repeats} timed, median {med:.2f} s "
           f"({', '.join(f'{t:.2f}' for t in times)})" if repeats > 1 else
           f"timed once ({med:.2f} s), in the same process after the headline oracle's warm-up")
    return {"value": round(1.0 / med, 6), "unit": "forwards/s", "cores": int(threads), "kind": "oracle",
            "blas": api,
            "sample": f"{note}: one step of the {wl.name} workload (materialize {args.commit} positions "
                      f"of each of its {wl.B} requests + one B={wl.B} forward, float64 numpy), {how}; "
                      f"forwards/s = 1 / that time"}


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
    ap.add_argument("--no-extra", action="store_true",
                    help="with the default workload: skip the 27B B=8 and 35B B=8 records")
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

    import torch
    import synth
    import block_drafter_amd as bd

    bd.lib()                                  # fails loudly without the built library
    headline = args.workload
    traffic_md = "traffic_gemm_stream_gate_up_dspine27b_b1.md" if headline == "dspine27b_b1" else None
    rec, st = measure_workload(headline, args, not args.no_propose, traffic_md)
    g, wl = st["g"], st["wl"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_record(g, st["wts"], wl, args, st["anchors"], "headline workload")

    res = {
        "metric": "draft-block forwards/s at 27B geometry (B=1,8); ctx-prefill tok/s; % roofline",
        "value": rec["steps_per_s"],
        "unit": "forwards/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": g.dtype,
        "data": "synthetic",
        "config": {k: v for k, v in rec.items() if k not in ("roofline", "propose", "breakdown")},
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
    }
    res["config"]["operands"] = ("bf16 weights widened to fp16 in registers x fp16 activations, "
                                 "fp32 accumulate")
    if "breakdown" in rec:
        res["breakdown"] = rec["breakdown"]
    if "propose" in rec:
        res["propose"] = rec["propose"]
    if not args.no_prefill and g.dtype == "bf16" and g.hidden == 5120:
        log("context prefill: 8 requests x one 32768-token chunk ...")
        pw = synth.WORKLOADS["prefill27b"]
        res["prefill"] = prefill_measure(st["model"], g, pw.seed, n_req=pw.B, chunk=pw.prefill_chunk)
        log("context prefill without the window skip ...")
        res["prefill"]["no_skip"] = prefill_noskip_measure(g, st["wts"], pw.seed, n_req=pw.B,
                                                           chunk=pw.prefill_chunk)
    release(st)

    # the other half of the metric (27B at B=8) and the 35B plain-DFlash
    # workload, each as its own record of the same fields
    if headline == "dspine27b_b1" and not args.no_extra:
        for name, key in (("dspine27b_b8", "b8"), ("dflash35b_b8", "dflash35b_b8")):
            r, st = measure_workload(name, args, not args.no_propose and name == "dspine27b_b8")
            if name == "dspine27b_b8" and not args.no_cpu_baseline:
                r["cpu_baseline"] = oracle_record(st["g"], st["wts"], st["wl"], args, st["anchors"],
                                                  "B=8 record", repeats=1, warmup=0)
            res[key] = r
            release(st)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
