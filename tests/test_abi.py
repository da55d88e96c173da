"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before any GPU work.  Weight and
ring pointers here are fake (aligned, never dereferenced): only host-side
validation runs."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
import block_drafter_amd as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspine.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bd.LIB_PATH):
        from block_drafter_amd import build
        build.build()
    return bd.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspine_[a-z_]+)\s*\(", src)))


def test_header_functions_are_exported(L):
    names = header_functions()
    assert "dspine_draft_forward" in names and "dspine_ctx_materialize" in names and "dspine_bridge" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(bd.EXPORTS), "binding and header disagree"
    assert L.dspine_version().decode().startswith("dspine")


FAKE = 0x10000


def fake_weights(g):
    ws = bd.Weights_c()
    addr = [FAKE]

    def nxt():
        addr[0] += 0x1000
        return addr[0]

    for n in bd._GLOBAL_FIELDS:
        setattr(ws, n, nxt())
    for l in range(g.n_layers):
        for n in bd._LAYER_FIELDS:
            setattr(ws.layer[l], n, nxt())
    return ws


def make_model(L, g):
    gs = bd.geometry_struct(g)
    h = ctypes.c_void_p()
    rc = L.dspine_model_create(ctypes.byref(gs), ctypes.byref(fake_weights(g)), ctypes.byref(h))
    assert rc == 0, L.dspine_last_error()
    return h


def fake_ctx(g, frontier, full_cap=0):
    c = bd.Ctx_c()
    for l in range(g.n_layers):
        c.k_ring[l] = FAKE + 0x100 * (2 * l + 1)
        c.v_ring[l] = FAKE + 0x100 * (2 * l + 2)
        c.capacity[l] = g.windows[l] if g.windows[l] > 0 else full_cap
    c.frontier = frontier
    return c


def test_model_create_rejections(L):
    g = synth.G_27B
    h = ctypes.c_void_p()
    assert L.dspine_model_create(None, None, ctypes.byref(h)) == bd.E_ARG
    for bad in (dict(head_dim=96), dict(hidden=5000), dict(n_q_heads=24), dict(code_dim=1000),
                dict(code_dim=0), dict(n_layers=0), dict(ffn=100), dict(vocab=0)):
        gb = synth.with_geometry(g, **bad)
        if "n_layers" in bad:
            gs = bd.geometry_struct(g)
            gs.n_layers = 0
        else:
            gs = bd.geometry_struct(gb)
        rc = L.dspine_model_create(ctypes.byref(gs), ctypes.byref(fake_weights(g)), ctypes.byref(h))
        assert rc == bd.E_UNSUPPORTED, (bad, L.dspine_last_error())
    ws = fake_weights(g)
    ws.layer[3].w_down = None
    gs = bd.geometry_struct(g)
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == bd.E_ARG
    assert b"w_down" in L.dspine_last_error()
    ws = fake_weights(g)
    ws.codebook = FAKE + 8           # misaligned
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == bd.E_ARG


def test_sizes_match_page_figures(L):
    """Ring payload at the 27B geometry: 5 layers x (K + V) x 8 x 128 x 2048
    x 2 bytes = 40 MiB, the ring image the DFlash maintainer notes give."""
    g = synth.G_27B
    h = make_model(L, g)
    total = sum(2 * L.dspine_ring_bytes(h, l, 2048) for l in range(5))
    assert total == 40 * 2 ** 20
    assert L.dspine_ring_bytes(h, 0, 1024) == 0          # a local ring must hold exactly S slots
    assert L.dspine_workspace_bytes(h, 8, 16, 2048) > L.dspine_workspace_bytes(h, 1, 16, 0) > 0
    assert L.dspine_workspace_bytes(h, 9, 16, 0) == 0
    L.dspine_model_destroy(h)


def call_forward(L, h, B, W, ctxs, anchors, ws_bytes=1 << 40, out=FAKE, ws=FAKE):
    arr = (bd.Ctx_c * max(1, len(ctxs)))(*ctxs)
    aid = (ctypes.c_int32 * max(1, len(anchors)))(*anchors)
    return L.dspine_draft_forward(h, B, W, arr, aid, out, ws, ws_bytes, None)


def test_forward_rejections_before_any_launch(L):
    g = synth.G_27B
    h = make_model(L, g)
    c = fake_ctx(g, 4096)
    assert call_forward(L, h, 0, 16, [c], [1]) == bd.E_UNSUPPORTED
    assert call_forward(L, h, 9, 16, [c] * 9, [1] * 9) == bd.E_UNSUPPORTED
    assert call_forward(L, h, 1, 1, [c], [1]) == bd.E_UNSUPPORTED
    assert call_forward(L, h, 1, 17, [c], [1]) == bd.E_UNSUPPORTED
    assert call_forward(L, h, 1, 16, [c], [g.vocab]) == bd.E_ARG
    assert call_forward(L, h, 1, 16, [c], [-1]) == bd.E_ARG
    assert call_forward(L, h, 1, 16, [c], [5], ws_bytes=1024) == bd.E_WORKSPACE
    assert call_forward(L, h, 1, 16, [c], [5], out=FAKE + 4) == bd.E_ARG
    assert call_forward(L, h, 1, 16, [c], [5], ws=0) == bd.E_ARG
    bad = fake_ctx(g, -1)
    assert call_forward(L, h, 1, 16, [bad], [5]) == bd.E_STATE
    bad = fake_ctx(g, 10)
    bad.capacity[2] = 4096
    assert call_forward(L, h, 1, 16, [bad], [5]) == bd.E_STATE
    assert b"capacity" in L.dspine_last_error()
    bad = fake_ctx(g, 10)
    bad.v_ring[4] = None
    assert call_forward(L, h, 1, 16, [bad], [5]) == bd.E_ARG
    L.dspine_model_destroy(h)


def test_forward_noalloc_rejections_before_any_launch(L):
    """The allocation-free forward checks its arguments like the forward and
    refuses calls whose workspace plan exceeds its static scratch, before it
    touches the GPU."""
    g = synth.G_27B
    h = make_model(L, g)
    c = fake_ctx(g, 4096)

    def call(B, W, ctxs, anchors, out=FAKE):
        arr = (bd.Ctx_c * len(ctxs))(*ctxs)
        aid = (ctypes.c_int32 * len(anchors))(*anchors)
        return L.dspine_draft_forward_noalloc(h, B, W, arr, aid, out, None)

    assert call(0, 16, [c], [1]) == bd.E_UNSUPPORTED
    assert call(1, 17, [c], [1]) == bd.E_UNSUPPORTED
    assert call(1, 16, [c], [g.vocab]) == bd.E_ARG
    assert call(1, 16, [c], [5], out=FAKE + 4) == bd.E_ARG
    assert call(1, 16, [fake_ctx(g, -1)], [5]) == bd.E_STATE
    # B * W = 128 rows at 27B needs about 144 MB of workspace: more than the scratch
    assert call(8, 16, [c] * 8, [5] * 8) == bd.E_WORKSPACE
    assert b"scratch" in L.dspine_last_error()
    # 32 rows fit; the unpacked model is refused next
    assert L.dspine_workspace_bytes(h, 2, 16, 0) <= 40 << 20 < L.dspine_workspace_bytes(h, 4, 16, 0)
    assert call(2, 16, [c] * 2, [5] * 2) == bd.E_STATE
    assert b"pack" in L.dspine_last_error()
    L.dspine_model_destroy(h)


def test_full_layer_capacity_checks(L):
    g = synth.G_35B_DFLASH
    h = make_model(L, g)
    c = fake_ctx(g, 32768, full_cap=32000)
    assert call_forward(L, h, 1, 16, [c], [5]) == bd.E_STATE
    # materialize: the full layer must hold the new frontier
    c = fake_ctx(g, 100, full_cap=200)
    arr = (bd.Ctx_c * 1)(c)
    feats = (ctypes.c_void_p * 1)(FAKE)
    n = (ctypes.c_int64 * 1)(101)
    assert L.dspine_ctx_materialize(h, 1, arr, feats, n, FAKE, 1 << 40, None) == bd.E_STATE
    assert arr[0].frontier == 100                      # unchanged on error
    n[0] = -3
    assert L.dspine_ctx_materialize(h, 1, arr, feats, n, FAKE, 1 << 40, None) == bd.E_ARG
    L.dspine_model_destroy(h)


def test_materialize_rejections(L):
    g = synth.G_27B
    h = make_model(L, g)
    c = fake_ctx(g, 0)
    arr = (bd.Ctx_c * 1)(c)
    feats = (ctypes.c_void_p * 1)(None)
    n = (ctypes.c_int64 * 1)(16)
    assert L.dspine_ctx_materialize(h, 1, arr, feats, n, FAKE, 1 << 40, None) == bd.E_ARG
    feats[0] = FAKE
    assert L.dspine_ctx_materialize(h, 0, arr, feats, n, FAKE, 1 << 40, None) == bd.E_UNSUPPORTED
    assert L.dspine_ctx_materialize(h, 1, arr, feats, n, FAKE, 4096, None) == bd.E_WORKSPACE
    # zero tokens is a no-op that needs no workspace and launches nothing
    n[0] = 0
    assert L.dspine_ctx_materialize(h, 1, arr, feats, n, None, 0, None) == 0
    assert arr[0].frontier == 0
    L.dspine_model_destroy(h)


def test_unpacked_model_refuses_valid_calls(L):
    """Projection weights must be packed (fragment order) before any call
    that launches work; argument errors are still reported first."""
    g = synth.G_27B
    h = make_model(L, g)
    assert L.dspine_packed_bytes(h) == 256 + sum(               # 256: the weight range check's maxima
        int(np.prod(synth.weight_shape(g, n))) * 2
        for n in synth.weight_names(g) if n.split(".")[-1] in bd._PROJECTIONS)
    c = fake_ctx(g, 4096)
    assert call_forward(L, h, 1, 16, [c], [5]) == bd.E_STATE
    assert b"pack" in L.dspine_last_error()
    assert call_forward(L, h, 1, 17, [c], [5]) == bd.E_UNSUPPORTED
    aid = (ctypes.c_int32 * 1)(3)
    assert L.dspine_bridge(h, 0, 1, 16, FAKE, aid, None, FAKE, 1 << 40, None) == bd.E_STATE
    assert L.dspine_pack_weights(h, FAKE + 16, 1 << 40, None) == bd.E_ARG     # misaligned dst
    assert L.dspine_pack_weights(h, FAKE, 1024, None) == bd.E_WORKSPACE
    L.dspine_model_destroy(h)


def test_bridge_rejections(L):
    g = synth.G_35B_DFLASH                     # no bridge in this geometry
    h = make_model(L, g)
    aid = (ctypes.c_int32 * 1)(3)
    assert L.dspine_bridge(h, 0, 1, 16, FAKE, aid, None, FAKE, 1 << 40, None) == bd.E_UNSUPPORTED
    L.dspine_model_destroy(h)
    g = synth.G_27B
    h = make_model(L, g)
    assert L.dspine_bridge(h, 5, 1, 16, FAKE, aid, None, FAKE, 1 << 40, None) == bd.E_ARG
    assert L.dspine_bridge(h, 0, 1, 16, None, aid, None, FAKE, 1 << 40, None) == bd.E_ARG
    assert L.dspine_bridge(h, 0, 1, 16, FAKE, aid, FAKE + 4, FAKE, 1 << 40, None) == bd.E_ARG
    L.dspine_model_destroy(h)


def test_profile_stride_rejects_zero(L):
    assert L.dspine_profile_stride(0) != 0
    assert L.dspine_profile_stride(1) == 0


def call_propose(L, h, B, W, ctxs, anchors, prop, pws=FAKE, pws_bytes=1 << 40, out=FAKE):
    arr = (bd.Ctx_c * len(ctxs))(*ctxs)
    aid = (ctypes.c_int32 * len(anchors))(*anchors)
    return L.dspine_draft_propose(h, B, W, arr, aid, out, ctypes.byref(prop) if prop is not None else None,
                                  FAKE, 1 << 40, pws, pws_bytes, None)


def good_proposal(K=16, walk=bd.WALK_GREEDY):
    p = bd.Proposal_c()
    p.topk = K
    p.walk = walk
    p.temperature = 1.0
    p.uniforms = FAKE if walk == bd.WALK_SAMPLED else None
    for n in ("cand", "cand_scores", "table", "choice", "tokens", "q"):
        setattr(p, n, FAKE + 0x4000)
    return p


def test_propose_rejections_before_any_launch(L):
    g = synth.G_27B
    h = make_model(L, g)                           # no lm_head
    c = fake_ctx(g, 4096)
    assert L.dspine_propose_workspace_bytes(h, 1, 16, 16) == 0
    assert call_propose(L, h, 1, 16, [c], [5], good_proposal()) == bd.E_UNSUPPORTED
    assert b"lm_head" in L.dspine_last_error()
    L.dspine_model_destroy(h)

    ws = fake_weights(g)
    ws.lm_head = FAKE + 0x100000
    gs = bd.geometry_struct(g)
    h = ctypes.c_void_p()
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == 0
    head_bytes = g.vocab * g.hidden * 2
    fp8_bytes = g.vocab * g.hidden + 4 * g.vocab          # the FP8 copy and its row scales
    assert L.dspine_packed_bytes(h) == head_bytes + fp8_bytes + 256 + sum(
        int(np.prod(synth.weight_shape(g, n))) * 2
        for n in synth.weight_names(g) if n.split(".")[-1] in bd._PROJECTIONS)
    need = L.dspine_propose_workspace_bytes(h, 8, 16, 16)
    assert need >= 8 * 16 * g.vocab * 4                    # every row's head scores
    assert L.dspine_propose_workspace_bytes(h, 8, 16, 17) == 0
    assert L.dspine_propose_workspace_bytes(h, 8, 16, 0) == 0
    assert call_propose(L, h, 1, 16, [c], [5], None) == bd.E_ARG
    assert call_propose(L, h, 1, 16, [c], [5], good_proposal(K=0)) == bd.E_ARG
    assert call_propose(L, h, 1, 16, [c], [5], good_proposal(K=17)) == bd.E_ARG
    p = good_proposal()
    p.walk = 2
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG
    p = good_proposal(walk=bd.WALK_SAMPLED)
    p.temperature = 0.0
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG
    p = good_proposal(walk=bd.WALK_SAMPLED)
    p.uniforms = None
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG
    p = good_proposal(walk=bd.WALK_SAMPLED)
    p.q = None
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG
    assert b"q" in L.dspine_last_error()
    p = good_proposal()
    p.table = None
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG
    # FP8 retrieval: R in K..128
    for R in (8, 129, -1):
        p = good_proposal()
        p.retrieve = R
        assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG, R
    p = good_proposal()
    p.retrieve = 128
    p.retrieved = FAKE + 4
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_ARG
    assert call_propose(L, h, 1, 16, [c], [5], good_proposal(), pws_bytes=1024) == bd.E_WORKSPACE
    assert call_propose(L, h, 1, 16, [c], [g.vocab], good_proposal()) == bd.E_ARG
    assert call_propose(L, h, 1, 17, [c], [5], good_proposal()) == bd.E_UNSUPPORTED
    # valid arguments: the model is not packed yet
    assert call_propose(L, h, 1, 16, [c], [5], good_proposal()) == bd.E_STATE
    p = good_proposal()
    p.retrieve = 128
    assert call_propose(L, h, 1, 16, [c], [5], p) == bd.E_STATE
    L.dspine_model_destroy(h)

    g = synth.G_TINY                               # float32: no FP8 copy of the head
    ws = fake_weights(g)
    ws.lm_head = FAKE + 0x100000
    gs = bd.geometry_struct(g)
    h = ctypes.c_void_p()
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == 0
    assert L.dspine_packed_bytes(h) == g.vocab * g.hidden * 4 + sum(
        int(np.prod(synth.weight_shape(g, n))) * 4
        for n in synth.weight_names(g) if n.split(".")[-1] in bd._PROJECTIONS)
    p = good_proposal()
    p.retrieve = 128
    cf = fake_ctx(g, 100, full_cap=200)
    assert call_propose(L, h, 1, 16, [cf], [5], p) == bd.E_UNSUPPORTED
    assert b"BF16" in L.dspine_last_error()
    L.dspine_model_destroy(h)

    g = synth.G_35B_DFLASH                         # no bridge to refine
    ws = fake_weights(g)
    ws.lm_head = FAKE + 0x100000
    gs = bd.geometry_struct(g)
    h = ctypes.c_void_p()
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == 0
    assert call_propose(L, h, 1, 16, [fake_ctx(g, 100, full_cap=200)], [5], good_proposal()) == bd.E_UNSUPPORTED
    L.dspine_model_destroy(h)


def test_conv_geometry_checks(L):
    """DFlash2's convolution: the group width must be a multiple of 4 that
    splits hidden into a multiple of 16 groups, and each layer needs its
    four convolution tensors."""
    g = synth.G_27B_DFLASH2
    ws = fake_weights(g)
    gs = bd.geometry_struct(g)
    h = ctypes.c_void_p()
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == 0
    two = sum(int(np.prod(synth.weight_shape(g, n))) * 2 for n in synth.weight_names(g)
              if n.split(".")[-1] in bd._PROJECTIONS)
    assert L.dspine_packed_bytes(h) == two + 256               # W_delta of both branches packed too
    assert L.dspine_workspace_bytes(h, 8, 16, 0) > 0
    L.dspine_model_destroy(h)
    for bad in (6, 7, 640, -16):                               # not a multiple of 4; 8 groups; negative
        gs = bd.geometry_struct(synth.with_geometry(g, conv_group=bad))
        assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == bd.E_UNSUPPORTED, bad
    ws.layer[3].mlp_conv_base = None
    gs = bd.geometry_struct(g)
    assert L.dspine_model_create(ctypes.byref(gs), ctypes.byref(ws), ctypes.byref(h)) == bd.E_ARG
    assert b"mlp_conv_base" in L.dspine_last_error()
