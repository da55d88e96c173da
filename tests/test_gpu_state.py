"""GPU tests of the draft context as state, and of stream capture.

- Checkpoint / restore [NIF, ring storage]: a request's draft context is its
  per-layer K/V rings plus the frontier (the pages' device fork, turn
  checkpoints and restore carry exactly that).  A copy restored into the
  same or into fresh rings gives a bit-identical forward.
- Graph replay [PHY, 融合 kernel: the injection runs inside the drafter's
  existing graph]: the calls only enqueue kernels on the given stream, so a
  forward and a propose call captured into a HIP graph replay bit-identical
  to the eager calls, with eager work and synchronisations between replays.
- Window edges [NIF, draft attention; ring storage]: position F - S stays
  in the ring of a local layer but no block row may see it, while row 0
  sees F - S + 1.  Large finite sentinels written into those ring slots must
  leave the forward bit-identical (F - S) and must change it (F - S + 1).
- A float32 geometry with a local window of several 32-key tiles, compared
  with the oracle at 1e-4."""
import numpy as np
import pytest

import synth
from oracle import dspine_oracle as O
from tests.gpu_cases import Case, Run, rel_err, tol_for, to_np64

pytestmark = pytest.mark.gpu

# a bridge, a local and a full layer; vocab a multiple of 16 (proposal head)
G_S = synth.Geometry(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                     n_feat_layers=3, code_dim=64, msg_dim=32, vocab=512, windows=(24, 0))
# windows of 2048 keys (16 key splits of 128) on both layers
G_W = synth.Geometry(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                     n_feat_layers=2, code_dim=64, msg_dim=32, vocab=512, windows=(2048, 2048))
# float32 with a 100-key local window (four 32-key tiles, the last ragged)
G_F32 = synth.Geometry(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                       n_feat_layers=2, code_dim=64, msg_dim=32, vocab=512, windows=(100, 0), dtype="f32")


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_drafter_amd as bd
    bd.lib()


def say(msg):
    print(f"[state] {msg}", flush=True)


def _snapshot(ctx):
    return ([k.clone() for k in ctx.k], [v.clone() for v in ctx.v], ctx.frontier)


def _restore(ctx, snap):
    ks, vs, F = snap
    for dst, src in zip(ctx.k, ks):
        dst.copy_(src)
    for dst, src in zip(ctx.v, vs):
        dst.copy_(src)
    ctx.frontier = F


def test_checkpoint_restore_bit_identical():
    import torch
    import block_drafter_amd as bd
    say("checkpoint/restore: 2 requests, F = 50, 120, advance by 40")
    case = Case(G_S, 95, 2, 16, [50, 120], full_capacity=400)
    run = Run(case)
    out0 = run.gpu_forward()
    snaps = [_snapshot(c) for c in run.ctxs]
    # advance every context by 40 more committed positions
    more = [bd.to_device(synth.make_features(G_S, 95, b, 40, start=F)) for b, F in enumerate(case.frontiers)]
    run.model.materialize(run.ctxs, more)
    out1 = run.gpu_forward()
    assert not np.array_equal(out0, out1)
    # restore in place
    for c, s in zip(run.ctxs, snaps):
        _restore(c, s)
    torch.cuda.synchronize()
    assert np.array_equal(run.gpu_forward(), out0)
    # fork: the checkpoint restored into fresh rings serves the same forward
    forks = [run.model.new_context(full_capacity=400, fill=float("nan")) for _ in range(2)]
    for c, s in zip(forks, snaps):
        _restore(c, s)
    out_fork = to_np64(run.model.forward(forks, run.anchors, 16))
    assert np.array_equal(out_fork, out0)
    # re-committing the same positions after the restore reproduces the advance exactly
    run.model.materialize(forks, more)
    out_re = to_np64(run.model.forward(forks, run.anchors, 16))
    assert np.array_equal(out_re, out1)
    # and the oracle agrees with the advanced state
    orc = [O.materialize(G_S, run.wts, run.oracle_ctx(b), synth.make_features(G_S, 95, b, 40, start=F))
           for b, F in enumerate(case.frontiers)]
    ref = O.draft_forward(G_S, run.wts, orc, run.anchors, 16)
    for b in range(2):
        assert rel_err(out1[b], ref[b]) <= tol_for(G_S)


def _outputs_equal(a, b):
    return all(np.array_equal(a[k], b[k]) for k in a)


def test_graph_replay_forward_and_propose():
    import torch
    import block_drafter_amd as bd
    say("graph replay: forward and propose, B=3, W=16, 4 replays each")
    wts = synth.make_weights(G_S, 96)
    head = synth.make_lm_head(G_S, 96)
    model = bd.Model.from_numpy(G_S, wts, lm_head=head)
    case = Case(G_S, 96, 3, 16, [45, 90, 12])
    run = Run(case, model=model, wts=wts)
    B, W, K = 3, 16, 16
    ws = model.workspace(B, W, 256)
    pws = model.propose_workspace(B, W, K)
    u = torch.from_numpy(synth.make_uniforms(96, B, W - 1)).cuda()

    out_eager = model.forward(run.ctxs, run.anchors, W, workspace=ws).clone()
    prop_eager = {k: v.clone() for k, v in model.propose(run.ctxs, run.anchors, W, K, walk="sampled",
                                                          temperature=0.7, uniforms=u, workspace=ws,
                                                          propose_workspace=pws).items()}
    torch.cuda.synchronize()

    out_g = torch.empty_like(out_eager)
    prop_g = {k: torch.empty_like(v) for k, v in prop_eager.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream's neighbour
        model.forward(run.ctxs, run.anchors, W, out=out_g, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_fwd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_fwd):
        model.forward(run.ctxs, run.anchors, W, out=out_g, workspace=ws)
    g_prop = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_prop):
        model.propose(run.ctxs, run.anchors, W, K, walk="sampled", temperature=0.7, uniforms=u,
                      workspace=ws, propose_workspace=pws, outputs=prop_g)
    torch.cuda.synchronize()

    scratch = torch.empty_like(out_eager)
    want = {k: v.cpu().numpy() for k, v in prop_eager.items()}
    for rep in range(4):
        out_g.fill_(float("nan"))
        for v in prop_g.values():
            v.zero_()
        g_fwd.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_eager), f"forward replay {rep}"
        # eager work on the same workspace between replays
        model.forward(run.ctxs, run.anchors, W, out=scratch, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(scratch, out_eager)
        g_prop.replay()
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in prop_g.items()}
        assert _outputs_equal(got, want), f"propose replay {rep}"


def _slot_fill(ctx, layer, slot, value):
    ctx.k[layer][:, slot, :] = value
    ctx.v[layer][:, slot, :] = value


def test_window_edges_with_sentinels():
    """Local windows of 2048 keys cut into 16 key splits: a wrapped ring
    (F = 5000) and a ring exactly full (F = 2048)."""
    import torch
    say("window edges: S = 2048, F = 5000 (wrapped) and 2048 (full ring)")
    S = 2048
    run = Run(Case(G_W, 97, 2, 16, [5000, 2048]))
    clean = run.gpu_forward()
    snaps = [_snapshot(c) for c in run.ctxs]
    # position F - S lives in the ring but is outside every row's window
    for b, F in enumerate(run.case.frontiers):
        for l in range(G_W.n_layers):
            _slot_fill(run.ctxs[b], l, (F - S) % S, 1.0e4)
    torch.cuda.synchronize()
    assert np.array_equal(run.gpu_forward(), clean)
    for c, s in zip(run.ctxs, snaps):
        _restore(c, s)
    # position F - S + 1 is row 0's first visible key
    for b, F in enumerate(run.case.frontiers):
        _slot_fill(run.ctxs[b], 0, (F - S + 1) % S, 1.0e4)
    torch.cuda.synchronize()
    hit = run.gpu_forward()
    for b in range(2):
        assert not np.array_equal(hit[b, 0], clean[b, 0]), f"request {b}: row 0 ignored its first key"
    # and the clean state matches the oracle
    for c, s in zip(run.ctxs, snaps):
        _restore(c, s)
    orc = run.oracle_forward()
    for b in range(2):
        assert rel_err(clean[b], orc[b]) <= tol_for(G_W)


def test_float32_multi_tile_local_window():
    say("float32, local window 100: frontiers 0, 50, 99, 100, 101, 333")
    fr = [0, 50, 99, 100, 101, 333]
    run = Run(Case(G_F32, 98, len(fr), 16, fr))
    gpu = run.gpu_forward()
    orc = run.oracle_forward()
    for b in range(len(fr)):
        err = rel_err(gpu[b], orc[b])
        assert err <= 1e-4, f"request {b} (F = {fr[b]}): {err:.3e}"
    for b in range(len(fr)):
        for (l, name, err, sentinel_ok) in run.ring_errors(b):
            assert err <= 1e-4 and sentinel_ok, (b, l, name, err)
