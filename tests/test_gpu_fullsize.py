"""GPU parity at the full workload shapes, in the launch configurations the
bench times.

The oracle cannot recompute everything at these sizes in seconds, so each
test compares:

* the whole draft-forward output, with the oracle attending over the
  GPU's own rings (copied back and widened).  This isolates the forward from
  the materialiser;
* the stored K/V of sampled requests at sampled positions (window edges,
  both ends of the context, random positions), each recomputed by the
  oracle on its own;
* at B=1, the whole rings and the forward end to end, with the oracle
  materialising its own rings.

Tolerances are those of the small tests: max |gpu - oracle| / rms(oracle)
<= 2e-2 for hidden states and stored K/V (one bf16 ulp of storage
rounding allowed on stored values)."""
import gc

import numpy as np
import pytest

import synth
from oracle import dspine_oracle as O
from tests.gpu_cases import TOL_BF16, rel_err, storage_err, to_np64

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_drafter_amd as bd
    bd.lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def say(msg):
    print(f"[fullsize] {msg}", flush=True)


def gpu_ring_context(g, ctx, F: int) -> O.RequestContext:
    """The GPU's rings as an oracle context (positions of the live window,
    widened exactly)."""
    layers = []
    for l in range(g.n_layers):
        S = g.windows[l]
        lo = O.live_lo(S, F)
        pos = np.arange(lo, F)
        slots = pos % S if S > 0 else pos
        K = to_np64(ctx.k[l])[:, slots, :]          # [nkv, n, D]
        V = to_np64(ctx.v[l])[:, slots, :]
        n = len(pos)
        layers.append(O.LayerContext(lo, K.transpose(1, 0, 2).reshape(n, g.kv_dim),
                                     V.transpose(1, 0, 2).reshape(n, g.kv_dim)))
    return O.RequestContext(F, layers)


def check_rings_whole(g, ctx, octx, cap_full=0, label=""):
    for l in range(g.n_layers):
        S = g.windows[l]
        cap = S if S > 0 else cap_full
        Ko, Vo = O.ring_image(g, octx, l, cap)
        for name, gpu_t, orc in (("K", ctx.k[l], Ko), ("V", ctx.v[l], Vo)):
            gv = to_np64(gpu_t)
            live = ~np.isnan(orc)
            assert np.all(np.isfinite(gv[live])), f"{label} layer {l} {name}: non-finite live slot"
            err = storage_err(gv[live], orc[live], True)
            assert err <= TOL_BF16, f"{label} layer {l} {name}: {err:.3e}"


def check_forward(g, wts, gpu_out, octxs, anchors, W, label):
    ref = O.draft_forward(g, wts, octxs, anchors, W)
    for i in range(len(octxs)):
        err = rel_err(gpu_out[i], ref[i])
        say(f"{label} request {i}: rel err {err:.3e}")
        assert err <= TOL_BF16, f"{label} request {i}: rel err {err:.3e}"


def check_ring_positions(g, wts, seed, b, ctx, F, pos, label):
    """Stored K/V at the given positions against the oracle recomputing
    exactly those positions (feature row -> context feature -> K/V)."""
    rows = np.stack([synth.make_features(g, seed, b, 1, start=int(p))[0] for p in pos])
    c = O.context_features(g, wts, rows)
    for l in range(g.n_layers):
        k, v = O.context_kv(g, wts, l, c, pos)
        Sl = g.windows[l]
        live = pos >= O.live_lo(Sl, F)
        slots = (pos % Sl) if Sl > 0 else pos
        Kg = to_np64(ctx.k[l])[:, slots[live], :].transpose(1, 0, 2).reshape(-1, g.kv_dim)
        Vg = to_np64(ctx.v[l])[:, slots[live], :].transpose(1, 0, 2).reshape(-1, g.kv_dim)
        for name, gv, ov in (("K", Kg, k[live]), ("V", Vg, v[live])):
            assert np.all(np.isfinite(gv)), f"{label} layer {l} {name}: non-finite stored value"
            err = storage_err(gv, ov, True)
            assert err <= TOL_BF16, f"{label} layer {l} {name}: {err:.3e}"


def sample_positions(F, S, seed, n=24):
    """Window edges, both ends of the context and random positions in it."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, F - S - 1, F - S, F - S + 1, F - 2, F - 1]
    return np.unique(np.clip(np.concatenate([edges, rng.integers(0, F, size=n)]), 0, F - 1))


def setup_windows(model, g, wl, extra_steps=0, commit=16):
    """The bench's setup: each request's live window is materialised from
    F - keep (a chunk longer than the ring keeps only its tail anyway)."""
    import torch
    import block_drafter_amd as bd
    full = any(s == 0 for s in g.windows)
    smax = max(g.windows)
    ctxs = []
    for b, F in enumerate(wl.frontiers):
        cap = (F + commit * extra_steps + 64) if full else 0
        c = model.new_context(full_capacity=cap, fill=float("nan"))
        keep = F if full else min(F, smax)
        c.frontier = F - keep
        feats = bd.to_device(synth.make_features(g, wl.seed, b, keep, start=F - keep))
        model.materialize([c], [feats], workspace=model.workspace(wl.B, wl.W, min(keep, 4096)))
        del feats
        ctxs.append(c)
    torch.cuda.synchronize()
    return ctxs


def test_dspine27b_b1_full_size():
    """27B geometry, B=1, W=16, F=4096: one 4096-token chunk into fresh rings
    (only the last 2048 positions are stored), the forward, then one bench
    step (16 committed positions) and the forward again."""
    import torch
    import block_drafter_amd as bd
    wl = synth.WORKLOADS["dspine27b_b1"]
    g = wl.geom
    say("dspine27b_b1: weights")
    wts = synth.make_weights(g, wl.seed)
    model = bd.Model.from_numpy(g, wts)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, 1)]
    F = wl.frontiers[0]
    feats = synth.make_features(g, wl.seed, 0, F + 16)
    ctx = model.new_context(fill=float("nan"))
    say("dspine27b_b1: materialize 4096 (tile GEMM path) + forward")
    model.materialize([ctx], [bd.to_device(feats[:F])], workspace=model.workspace(1, 16, 4096))
    gpu = to_np64(model.forward([ctx], anchors, wl.W))
    octx = O.materialize(g, wts, O.empty_context(g), feats[:F])
    check_rings_whole(g, ctx, octx, label="F=4096")
    check_forward(g, wts, gpu, [octx], anchors, wl.W, "F=4096")
    say("dspine27b_b1: commit 16 (streamed GEMM path) + forward")
    model.materialize([ctx], [bd.to_device(feats[F:])], workspace=model.workspace(1, 16, 256))
    gpu2 = to_np64(model.forward([ctx], anchors, wl.W))
    octx2 = O.materialize(g, wts, octx, feats[F:])
    check_rings_whole(g, ctx, octx2, label="F=4112")
    check_forward(g, wts, gpu2, [octx2], anchors, wl.W, "F=4112")
    model.close()


def test_dspine27b_b8_full_size():
    """27B geometry, B=8, W=16, per-request contexts U{1024..16384}."""
    import block_drafter_amd as bd
    wl = synth.WORKLOADS["dspine27b_b8"]
    g = wl.geom
    say(f"dspine27b_b8: frontiers {wl.frontiers}")
    wts = synth.make_weights(g, wl.seed)
    model = bd.Model.from_numpy(g, wts)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, wl.B)]
    ctxs = setup_windows(model, g, wl)
    say("dspine27b_b8: forward")
    gpu = to_np64(model.forward(ctxs, anchors, wl.W))
    # the whole batch against the oracle reading the GPU's rings
    check_forward(g, wts, gpu, [gpu_ring_context(g, c, F) for c, F in zip(ctxs, wl.frontiers)],
                  anchors, wl.W, "gpu rings")
    # stored K/V of the shortest and the longest context at sampled positions
    # (positions before a request's window were never materialised)
    for b in (int(np.argmin(wl.frontiers)), int(np.argmax(wl.frontiers))):
        F = wl.frontiers[b]
        S = max(g.windows)
        pos = sample_positions(F, S, 3003 + b)
        pos = pos[pos >= F - min(F, S)]
        check_ring_positions(g, wts, wl.seed, b, ctxs[b], F, pos, f"request {b}")
    model.close()


def test_dflash35b_b8_full_size():
    """35B-style plain DFlash (no bridge), B=8, W=16, F=32768 each: 5 local
    layers (S=4096) and one full layer holding all 32768 positions."""
    import block_drafter_amd as bd
    wl = synth.WORKLOADS["dflash35b_b8"]
    g = wl.geom
    say("dflash35b_b8: weights")
    wts = synth.make_weights(g, wl.seed)
    model = bd.Model.from_numpy(g, wts)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, wl.B)]
    say("dflash35b_b8: materialize 8 x 32768")
    ctxs = setup_windows(model, g, wl)
    say("dflash35b_b8: forward")
    gpu = to_np64(model.forward(ctxs, anchors, wl.W))
    check_forward(g, wts, gpu, [gpu_ring_context(g, c, F) for c, F in zip(ctxs, wl.frontiers)],
                  anchors, wl.W, "gpu rings")
    # sampled positions of two requests, each recomputed on its own
    for b in (0, 5):
        F = wl.frontiers[b]
        check_ring_positions(g, wts, wl.seed, b, ctxs[b], F, sample_positions(F, max(g.windows), 4004 + b),
                             f"request {b}")
    model.close()


def test_prefill27b_full_size():
    """27B prefill: every request materialises one 32768-token chunk into a
    fresh ring in a single call; only its last 2048 rows may be read (the
    rest of the chunk is NaN here, so reading any of it would poison the
    rings), and the frontier advances by 32768.  Then one B=8 forward."""
    import torch
    import block_drafter_amd as bd
    wl = synth.WORKLOADS["prefill27b"]
    g = wl.geom
    n = wl.prefill_chunk
    S = max(g.windows)
    say("prefill27b: weights")
    wts = synth.make_weights(g, wl.seed)
    model = bd.Model.from_numpy(g, wts)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, wl.B)]
    chunks = []
    for b in range(wl.B):
        t = torch.full((n, g.n_feat_layers * g.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        t[n - S:] = bd.to_device(synth.make_features(g, wl.seed, b, S, start=n - S))
        chunks.append(t)
    ctxs = [model.new_context(fill=float("nan")) for _ in range(wl.B)]
    say("prefill27b: one materialize call, 8 x 32768 tokens")
    model.materialize(ctxs, chunks, workspace=model.workspace(wl.B, wl.W, wl.B * S))
    torch.cuda.synchronize()
    assert all(c.frontier == n for c in ctxs)
    del chunks
    say("prefill27b: forward")
    gpu = to_np64(model.forward(ctxs, anchors, wl.W))
    check_forward(g, wts, gpu, [gpu_ring_context(g, c, n) for c in ctxs], anchors, wl.W, "gpu rings")
    for b in (0, 7):
        pos = sample_positions(n, S, 5005 + b)
        pos = pos[pos >= n - S]
        check_ring_positions(g, wts, wl.seed, b, ctxs[b], n, pos, f"request {b}")
        # every slot of every layer holds a stored (finite) value
        for l in range(g.n_layers):
            assert bool(torch.isfinite(ctxs[b].k[l]).all()) and bool(torch.isfinite(ctxs[b].v[l]).all())
    model.close()


def test_dspine27b_causal_b8_full_size():
    """The 27B checkpoint's own attention: block-causal, 8192-position windows,
    B=8 with contexts U{1024..16384} (windows both partly filled and
    truncated).  Besides parity, causality fixes a property the GPU must
    keep at any size: rows 0..W'-1 of a W-block equal a W'-block run with the
    same anchors and frontiers (the bridge only sends messages forward and
    block key j is visible to row i only when j <= i)."""
    import block_drafter_amd as bd
    wl = synth.WORKLOADS["dspine27b_causal_b8"]
    g = wl.geom
    assert g.block_causal and set(g.windows) == {8192}
    say(f"dspine27b_causal_b8: frontiers {wl.frontiers}")
    wts = synth.make_weights(g, wl.seed)
    model = bd.Model.from_numpy(g, wts)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, wl.B)]
    ctxs = setup_windows(model, g, wl)
    say("dspine27b_causal_b8: forward W=16")
    gpu = to_np64(model.forward(ctxs, anchors, wl.W))
    check_forward(g, wts, gpu, [gpu_ring_context(g, c, F) for c, F in zip(ctxs, wl.frontiers)],
                  anchors, wl.W, "gpu rings")
    for Wp in (5, 8):
        say(f"dspine27b_causal_b8: forward W={Wp}, prefix of the W=16 block")
        short = to_np64(model.forward(ctxs, anchors, Wp))
        for i in range(wl.B):
            err = rel_err(short[i], gpu[i, :Wp])
            assert err <= TOL_BF16, f"W={Wp} prefix, request {i}: rel err {err:.3e}"
    b = int(np.argmax(wl.frontiers))
    F = wl.frontiers[b]
    pos = sample_positions(F, 8192, 6006)
    pos = pos[pos >= F - min(F, 8192)]
    check_ring_positions(g, wts, wl.seed, b, ctxs[b], F, pos, f"request {b}")
    model.close()


def test_dflash2_27b_b8_full_size():
    """DFlash2 27B geometry: dynamic grouped convolution (group width 16)
    around attention and MLP, five local layers, B=8, contexts U{1024..16384}."""
    import block_drafter_amd as bd
    wl = synth.WORKLOADS["dflash2_27b_b8"]
    g = wl.geom
    say(f"dflash2_27b_b8: frontiers {wl.frontiers}")
    wts = synth.make_weights(g, wl.seed)
    model = bd.Model.from_numpy(g, wts)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, wl.B)]
    ctxs = setup_windows(model, g, wl)
    say("dflash2_27b_b8: forward")
    gpu = to_np64(model.forward(ctxs, anchors, wl.W))
    check_forward(g, wts, gpu, [gpu_ring_context(g, c, F) for c, F in zip(ctxs, wl.frontiers)],
                  anchors, wl.W, "gpu rings")
    model.close()
