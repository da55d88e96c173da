"""GPU parity: the HIP library against the CPU oracle on identical seeded
inputs (small and medium shapes; the full-size shapes are in
test_gpu_fullsize.py).  Masks and indices compare bit-exactly; hidden
states and stored K/V compare with max |gpu - oracle| / rms(oracle) <= 2e-2
(bf16) or 1e-4 (float32), as the tolerance statement of the method fixes."""
import math

import numpy as np
import pytest

import synth
from oracle import dspine_oracle as O
from tests.gpu_cases import Case, Run, bf16_ulp, rel_err, storage_err, tol_for, to_np64

pytestmark = pytest.mark.gpu

# geometries that meet the kernels' limits, each exercising other paths
G_A = synth.Geometry(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                     n_feat_layers=3, code_dim=64, msg_dim=32, vocab=512, windows=(24, 0))
G_B = synth.Geometry(hidden=512, n_layers=3, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                     n_feat_layers=2, code_dim=128, msg_dim=64, vocab=1000, windows=(40, 0, 33))
G_C = synth.Geometry(hidden=384, n_layers=2, n_q_heads=16, n_kv_heads=2, head_dim=64, ffn=768,
                     n_feat_layers=2, code_dim=0, msg_dim=0, vocab=300, windows=(17, 64))
G_D = synth.Geometry(hidden=256, n_layers=2, n_q_heads=2, n_kv_heads=2, head_dim=128, ffn=256,
                     n_feat_layers=1, code_dim=96, msg_dim=64, vocab=128, windows=(20, 5),
                     block_causal=True)


# DFlash2's dynamic grouped convolution (group width 16), with and without a bridge
G_E = synth.Geometry(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                     n_feat_layers=2, code_dim=0, msg_dim=0, vocab=512, windows=(24, 0), conv_group=16)
G_F = synth.Geometry(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024,
                     n_feat_layers=2, code_dim=64, msg_dim=32, vocab=512, windows=(40, 33), conv_group=16,
                     block_causal=True)
G_E32 = synth.with_geometry(G_E, dtype="f32")


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_drafter_amd as bd
    bd.lib()


def check_run(run: Run, requests=None, W=None):
    g = run.case.g
    gpu = run.gpu_forward(W)
    req = list(range(run.case.B)) if requests is None else requests
    orc = run.oracle_forward(req, W)
    for i, b in enumerate(req):
        err = rel_err(gpu[b], orc[i])
        assert err <= tol_for(g), f"request {b}: rel err {err:.3e}"
    for b in req:
        for (l, name, err, sentinel_ok) in run.ring_errors(b):
            assert err <= tol_for(g), f"request {b} layer {l} {name}: {err:.3e}"
            assert sentinel_ok, f"request {b} layer {l} {name}: non-live slot written"
    return gpu, orc


def test_tiny_fp32_config():
    """The tiny float32 drafter: B=1, W=16, 128 context positions, full attention."""
    wl = synth.WORKLOADS["tiny_fp32"]
    run = Run(Case(wl.geom, wl.seed, wl.B, wl.W, wl.frontiers))
    check_run(run)


@pytest.mark.parametrize("g", [G_A, G_B, G_C, G_D], ids=["A", "B", "C", "D"])
def test_small_geometries_ragged_batch(g):
    # ragged frontiers: empty context, shorter than the window, wrapped ring
    fr = [0, 7, 23, 61, 130][: 5]
    run = Run(Case(g, 77, len(fr), 16, fr))
    check_run(run)


def test_many_key_splits():
    """Long contexts on a full-attention layer: the keys are cut into ten
    splits (two merge batches), the last one ragged, and a second request
    with a third of the keys (splits past its end are empty)."""
    run = Run(Case(G_B, 81, 2, 16, [1200, 333]))
    check_run(run)


@pytest.mark.parametrize("W", [2, 5, 16])
def test_block_widths(W):
    run = Run(Case(G_B, 78, 3, W, [45, 90, 12]))
    check_run(run, W=W)


def test_chunked_and_truncated_materialization():
    """Sub-chunks, and chunks longer than the ring (only the final window is
    stored, the frontier advances by the whole chunk)."""
    chunks = [[100], [3, 30, 1, 66], [40, 41, 19]]
    run = Run(Case(G_B, 79, 3, 16, [100, 100, 100], chunks=chunks, shared_features=True))
    gpu, _ = check_run(run)
    # the three ways of reaching frontier 100 agree with each other on the GPU
    # too.  The first call (143 rows) runs the tile GEMMs (bf16 x bf16); the
    # later calls run the streamed GEMM, whose prologue (fused at <= 32 rows,
    # the pre-scale kernel above) passes the normalised context features
    # through bf16 as well, so both paths project the same operand values up
    # to the fp32 summation order of the feature projection: about one
    # context-feature element per call lands on the other side of a bf16
    # rounding boundary, which moves every K/V element of that row by about
    # 2^-8 |c_i w_i|.  So almost every stored element is identical, and each
    # difference is within one bf16 step at the layer's rms (one ulp of the
    # element itself can be smaller than that for elements near zero)
    for l in range(G_B.n_layers):
        for ring in ("k", "v"):
            a = to_np64(getattr(run.ctxs[0], ring)[l])
            for b in (1, 2):
                c = to_np64(getattr(run.ctxs[b], ring)[l])
                assert np.array_equal(np.isnan(a), np.isnan(c))
                m = ~np.isnan(a)
                d = np.abs(a[m] - c[m])
                step = np.maximum(bf16_ulp(a[m]), 2.0 ** -8 * np.sqrt(np.mean(a[m] ** 2)))
                same = float(np.mean(d == 0))
                print(f"layer {l} {ring} request {b}: identical {same:.5f}, beyond one ulp "
                      f"{int(np.sum(d > bf16_ulp(a[m])))}, max / step {float(np.max(d / step)):.3f}")
                assert same > 0.99, (l, ring, b, same)
                assert np.all(d <= step), (l, ring, b, float(np.max(d / step)))


def test_debug_visible_bit_exact():
    g = synth.with_geometry(G_A, windows=(24, 0))
    run = Run(Case(g, 80, 5, 16, [0, 7, 23, 24, 130]))
    for l in range(2):
        lo_hi, slot, nblk = run.model.debug_visible(l, run.ctxs, 16)
        lo_hi = lo_hi.cpu().numpy()
        slot = slot.cpu().numpy()
        nblk = nblk.cpu().numpy()
        S = g.windows[l]
        for b, F in enumerate(run.case.frontiers):
            for i in range(16):
                lo, hi = O.visible_context_interval(S, F, i)
                assert (lo_hi[b, i, 0], lo_hi[b, i, 1]) == (lo, hi)
                want_slot = -1 if lo >= hi else (lo % S if S else lo)
                assert slot[b, i] == want_slot
                nb = sum(O.key_visible(S, g.block_causal, F + i, F + j, True, i, j) for j in range(16))
                assert nblk[b, i] == nb
    # the closed form: a row with full left context sees S-1-i context keys
    lo_hi0, _, _ = run.model.debug_visible(0, run.ctxs, 16)
    lo_hi0 = lo_hi0.cpu().numpy()
    for i in range(16):
        assert lo_hi0[4, i, 1] - lo_hi0[4, i, 0] == 24 - 1 - i


def test_debug_visible_causal_and_narrow_window():
    g = synth.with_geometry(G_D, windows=(5, 0))
    run = Run(Case(g, 81, 2, 8, [3, 50]))
    lo_hi, slot, nblk = run.model.debug_visible(0, run.ctxs, 8)
    nblk = nblk.cpu().numpy()
    for i in range(8):
        # block-causal and |i-j| < 5: j in (i-5, i]
        assert nblk[1, i] == min(i + 1, 5)


def test_request_isolation_bit_exact():
    """Changing another request (anchor, context) leaves a request's output
    bit-identical: rows of different requests never mix."""
    run = Run(Case(G_B, 82, 3, 16, [50, 70, 20]))
    a = run.gpu_forward()
    run.anchors[1] = (run.anchors[1] + 17) % G_B.vocab
    run.ctxs[2].frontier = 15            # a shorter (still materialized) context
    b = run.gpu_forward()
    assert np.array_equal(a[0], b[0])
    assert not np.array_equal(a[1], b[1])
    c = run.gpu_forward()
    assert np.array_equal(b, c)          # and runs are reproducible


def test_stored_v_passes_through_bf16():
    run = Run(Case(G_A, 83, 1, 16, [60]))
    import torch
    for l in range(2):
        v = run.ctxs[0].v[l]
        bits = v.view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF
        live = ~np.isnan(to_np64(v))
        exp = (bits >> 10) & 0x1F
        normal = live & (exp > 0) & (exp < 31)
        assert np.all((bits[normal] & 0x7) == 0)
        k = run.ctxs[0].k[l].view(torch.int16).cpu().numpy()
        assert k.dtype == np.int16   # K is stored as bfloat16 patterns


@pytest.mark.parametrize("with_override", [False, True])
def test_bridge_call(with_override):
    import torch
    g = G_B
    run = Run(Case(g, 84, 2, 16, [10, 10]))
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 16, g.hidden)) * 2.0
    xt = torch.tensor(x, dtype=torch.float32, device="cuda")
    pred = None
    if with_override:
        ids = rng.integers(0, g.vocab, size=(2, 16))
        cb = synth.to_float(run.wts["codebook"])
        pred = math.sqrt(g.code_dim) * cb[ids]
        pred_t = torch.tensor(pred, dtype=torch.float32, device="cuda")
    run.model.bridge(1, xt, run.anchors, None if pred is None else pred_t)
    torch.cuda.synchronize()
    got = to_np64(xt)
    x32 = x.astype(np.float32).astype(np.float64)
    for b in range(2):
        want = O.bridge(g, run.wts, 1, x32[b], run.anchors[b],
                        None if pred is None else pred[b].astype(np.float32).astype(np.float64))
        assert np.array_equal(got[b, 0], x32[b, 0])          # no write at the anchor
        assert rel_err(got[b], want) <= tol_for(g)


def test_bridge_identity_gives_plain_dflash_on_gpu():
    """With the gate closed (b = -1e4) the GPU forward equals the same
    weights run with the bridge removed, exactly."""
    import block_drafter_amd as bd
    g = G_A
    wts = synth.make_weights(g, 85, {"bridge_b": synth.normal(1, 1, (g.msg_dim,), 0.0, -1e4, g.dtype)})
    case = Case(g, 85, 2, 16, [30, 5])
    a = Run(case, wts=wts).gpu_forward()
    g_off = synth.with_geometry(g, code_dim=0, msg_dim=0)
    m_off = bd.Model.from_numpy(g_off, {k: v for k, v in wts.items()})
    b = Run(Case(g_off, 85, 2, 16, [30, 5]), model=m_off, wts=wts).gpu_forward()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("g", [G_E, G_F, G_E32], ids=["E", "F", "E-fp32"])
@pytest.mark.parametrize("B,W", [(1, 16), (3, 7), (8, 16), (5, 2)])
def test_dflash2_convolution(g, B, W):
    """DFlash2's convolution around attention and MLP: ragged frontiers, a
    block row 0 per request (no tap before it), both operand paths (B*W up
    to 32 rows fused, more pre-scaled), with and without the bridge."""
    rng = np.random.default_rng(90 + B)
    fr = [int(v) for v in rng.integers(5, 70, size=B)]
    run = Run(Case(g, 91 + B, B, W, fr))
    check_run(run)


def test_counters_return_to_zero():
    """The workspace's counters (8192 stream-K tile arrivals, then the fused
    bridge's 69, 32 words apart: its hand-off counters, timeout flag,
    fourth-phase counter and per-block arrival counters) are zero again after
    every call,
    as the header promises; the fused bridge with its folded norm (16 rows
    and fewer), the fused bridge without it (32 rows) and the multi-launch
    bridge all run here."""
    import torch
    run = Run(Case(G_B, 86, 2, 16, [50, 70]))
    ws = run.model.workspace(8, 16, 256)
    for B, W in ((2, 16), (1, 16), (2, 7), (8, 16)):
        ctxs = (run.ctxs * 4)[:B]
        anchors = (run.anchors * 4)[:B]
        run.model.forward(ctxs, anchors, W, workspace=ws)
        torch.cuda.synchronize()
        words = ws[: 4 * (8192 + 69 * 32)].view(torch.int32).cpu().numpy()
        assert not np.any(words), f"B={B} W={W}: nonzero counter words at {np.nonzero(words)[0][:8]}"


def test_ffn_hidden_beyond_fp16_range():
    """The SwiGLU hidden is the one GEMM operand that no norm bounds: with
    gate and up weights scaled by 1000 (N(0, 1000^2 / H)) the hidden rows
    reach about 1e6, far past fp16's 65504.  A BF16 model keeps the hidden
    in bf16 and multiplies it by the bf16 down weights, so the forward still
    matches the oracle (fp64, no rounding of the hidden)."""
    import block_drafter_amd as bd
    g = G_B
    base = synth.make_weights(g, 87)
    big = {}
    for l in range(g.n_layers):
        for n in ("w_gate", "w_up"):
            w = synth.to_float(base[f"l{l}.{n}"]) * 1000.0
            big[f"l{l}.{n}"] = synth.f32_to_bf16_bits(w.astype(np.float32))
    wts = synth.make_weights(g, 87, big)
    run = Run(Case(g, 87, 2, 16, [40, 9]), wts=wts)
    gpu = run.gpu_forward()
    assert np.all(np.isfinite(gpu))
    orc = run.oracle_forward()
    for b in range(2):
        err = rel_err(gpu[b], orc[b])
        print(f"request {b}: rel err {err:.3e}")
        assert err <= tol_for(g), f"request {b}: {err:.3e}"


def test_pack_rejects_weights_beyond_fp16_range():
    """Weights that the GEMMs widen to fp16 operands must lie within fp16's
    range: packing refuses a larger one (E_UNSUPPORTED, naming the matrix).
    The down projection multiplies bf16 x bf16 and takes any bf16 value."""
    import block_drafter_amd as bd
    g = G_A
    wq = synth.to_float(synth.make_weights(g, 88)["l1.wq"])
    wq[3, 5] = 1.0e5
    wts = synth.make_weights(g, 88, {"l1.wq": synth.f32_to_bf16_bits(wq.astype(np.float32))})
    with pytest.raises(bd.DSpineError) as e:
        bd.Model.from_numpy(g, wts)
    assert e.value.code == bd.E_UNSUPPORTED and "wq" in str(e.value)
    wd = synth.to_float(synth.make_weights(g, 88)["l0.w_down"])
    wd[1, 2] = 1.0e5
    wts = synth.make_weights(g, 88, {"l0.w_down": synth.f32_to_bf16_bits(wd.astype(np.float32))})
    model = bd.Model.from_numpy(g, wts)
    model.close()
