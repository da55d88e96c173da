"""GPU parity of the proposal tail (dspine_draft_propose) against the oracle.

Floating-point values (head scores, the transition table) compare with
max |gpu - oracle| / rms(oracle) <= 2e-2 (bf16) or 1e-4 (float32).  Where a
float decides an integer (the top-K ranking, the walk's argmax or draw),
both sides take the decision on the same numbers: the oracle's ranking and
walk run on the GPU's own scores and table and must agree bit for bit.  The
table is evaluated by the oracle on the GPU's candidates, so a near-tie at
the K-th rank cannot make the two tables index different tokens.  The
candidates themselves are also checked in the oracle's exact arithmetic:
each rank's oracle score is within tolerance of the oracle's own top-K."""
import numpy as np
import pytest

import synth
from oracle import dspine_oracle as O
from tests.gpu_cases import Case, Run, TOL_BF16, rel_err, tol_for, to_np64

pytestmark = pytest.mark.gpu

# small geometries whose vocabularies are multiples of 16 (the head's packed blocks)
G_A = synth.Geometry(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                     n_feat_layers=3, code_dim=64, msg_dim=32, vocab=512, windows=(24, 0))
# code and message widths of 256: the refinement GEMMs take the MFMA tile path
G_T = synth.Geometry(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024,
                     n_feat_layers=2, code_dim=256, msg_dim=256, vocab=2048, windows=(32, 0),
                     block_causal=True)


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_drafter_amd as bd
    bd.lib()


def say(msg):
    print(f"[propose] {msg}", flush=True)


def gpu_propose(model, ctxs, anchors, W, K, walk, temperature, uniforms, retrieve=0):
    import torch
    u = torch.from_numpy(uniforms).cuda() if uniforms is not None else None
    res = model.propose(ctxs, anchors, W, K, walk=walk, temperature=temperature, uniforms=u,
                        keep_scores=True, retrieve=retrieve)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in res.items()}
    out["out"] = out["out"].astype(np.float64)
    return out


def check_proposal(g, wts, head, gp, octxs, anchors, W, K, walk, temperature, uniforms, label,
                   requests=None):
    """gp: the GPU's results for all B requests; the oracle runs on
    `requests` (default all) with the contexts octxs (one per listed request)."""
    tol = tol_for(g)
    B = gp["cand"].shape[0]
    req = list(range(B)) if requests is None else list(requests)
    V = g.vocab
    scores = gp["scores"].reshape(B, W, V).astype(np.float64)
    # integer decisions on the GPU's own numbers: bit-exact
    for b in range(B):
        for t in range(W - 1):
            ref = O.top_k(scores[b, t + 1], K)
            assert np.array_equal(gp["cand"][b, t], ref), f"{label} request {b} row {t + 1}: top-{K}"
            assert np.array_equal(gp["cand_scores"][b, t].astype(np.float64), scores[b, t + 1, ref])
        T = gp["table"][b].astype(np.float64)
        if walk == "greedy":
            ch = O.greedy_walk(T)
        else:
            ch, q = O.sampled_walk(T, temperature, uniforms[b])
            assert np.max(np.abs(gp["q"][b] - q)) <= 1e-12, f"{label} request {b}: q"
        assert np.array_equal(gp["choice"][b], ch), f"{label} request {b}: walk"
        assert np.array_equal(gp["tokens"][b], gp["cand"][b, np.arange(W - 1), ch])
    # float values against the oracle, on the GPU's candidates
    orc = O.propose(g, wts, head, octxs, [anchors[b] for b in req], W, K, walk, temperature,
                    None if uniforms is None else uniforms[req], cand_override=gp["cand"][req])
    for i, b in enumerate(req):
        e_out = rel_err(gp["out"][b], orc["out"][i])
        e_sc = rel_err(scores[b, 1:], orc["scores"][i])
        e_tab = rel_err(gp["table"][b].astype(np.float64), orc["table"][i])
        say(f"{label} request {b}: out {e_out:.2e} scores {e_sc:.2e} table {e_tab:.2e}")
        assert e_out <= tol and e_sc <= tol and e_tab <= tol, label
        # the GPU's candidates are (near-)best in the oracle's arithmetic too:
        # with every score within e of the oracle's, the oracle score of the
        # GPU's k-th pick is within 2e of the oracle's k-th best
        e = np.max(np.abs(scores[b, 1:] - orc["scores"][i]))
        for t in range(W - 1):
            best = np.sort(orc["scores"][i][t])[::-1][:K]
            got = orc["scores"][i][t][gp["cand"][b, t]]
            assert np.max(np.abs(got - best)) <= 2 * e + 1e-12, f"{label} request {b} row {t + 1}: ranks"
    return orc


def check_walk_on_gpu_table(gp, W, walk, temperature, uniforms, label):
    B = gp["cand"].shape[0]
    for b in range(B):
        T = gp["table"][b].astype(np.float64)
        if walk == "greedy":
            ch = O.greedy_walk(T)
        else:
            ch, q = O.sampled_walk(T, temperature, uniforms[b])
            assert np.max(np.abs(gp["q"][b] - q)) <= 1e-12, f"{label} request {b}: q"
        assert np.array_equal(gp["choice"][b], ch), f"{label} request {b}: walk"
        assert np.array_equal(gp["tokens"][b], gp["cand"][b, np.arange(W - 1), ch])


def check_retrieval(g, wts, head, fp8, gp, octxs, anchors, W, K, R, walk, temperature, uniforms, label,
                    requests=None):
    """FP8 retrieval on the GPU against the oracle.  Decisions are checked
    on the GPU's own numbers, bit for bit: the R retrieved are the oracle's
    top-R of the GPU's FP8 scores, and the K kept are the oracle's order of
    the GPU's rescored values.  The FP8 scores themselves equal the oracle's
    FP8 head applied to the GPU's fp16 operand rows up to fp32 summation
    (2e-5 of rms: a single code differing from the oracle's would move a
    score by about 1e-3 of rms), and the rescoring equals E . h on the
    GPU's fp32 rows to 1e-5.  The table, the walk and the forward follow
    check_proposal's rules."""
    codes, scales = fp8
    B = gp["cand"].shape[0]
    req = list(range(B)) if requests is None else list(requests)
    V = g.vocab
    approx = gp["scores"].reshape(B, W, V).astype(np.float64)
    h = gp["out"]
    h16 = h.astype(np.float16).astype(np.float64)
    for b in range(B):
        ref = O.head_scores_fp8(codes, scales, h16[b, 1:])
        e = rel_err(approx[b, 1:], ref)
        assert e <= 2e-5, f"{label} request {b}: FP8 scores {e:.2e}"
        for t in range(W - 1):
            ids = gp["retrieved"][b, t]
            assert np.array_equal(ids, O.top_k(approx[b, t + 1], R)), f"{label} request {b} row {t + 1}: retrieval"
            resc = gp["rescored"][b, t].astype(np.float64)
            ex = O.head_scores(head, h[b, t + 1], ids)[0]
            assert np.max(np.abs(resc - ex)) <= 1e-5 * np.sqrt(np.mean(ex * ex)), f"{label}: rescoring"
            keep = np.lexsort((ids, -resc))[:K]
            assert np.array_equal(gp["cand"][b, t], ids[keep]), f"{label} request {b} row {t + 1}: kept"
            assert np.array_equal(gp["cand_scores"][b, t].astype(np.float64), resc[keep])
    check_walk_on_gpu_table(gp, W, walk, temperature, uniforms, label)
    orc = O.propose(g, wts, head, octxs, [anchors[b] for b in req], W, K, walk, temperature,
                    None if uniforms is None else uniforms[req], cand_override=gp["cand"][req],
                    retrieve=R, fp8_head=fp8)
    tol = tol_for(g)
    for i, b in enumerate(req):
        e_out = rel_err(gp["out"][b], orc["out"][i])
        e_sc = rel_err(approx[b, 1:], orc["scores"][i])
        e_tab = rel_err(gp["table"][b].astype(np.float64), orc["table"][i])
        e_cs = rel_err(gp["cand_scores"][b].astype(np.float64), orc["cand_scores"][i])
        say(f"{label} request {b}: out {e_out:.2e} fp8 scores {e_sc:.2e} kept scores {e_cs:.2e} table {e_tab:.2e}")
        assert e_out <= tol and e_sc <= tol and e_tab <= tol and e_cs <= tol, label
        # near-best in the oracle's arithmetic: the oracle's own retrieval on
        # its own rows keeps K tokens whose BF16 scores match the GPU's
        # picks rank by rank, within twice the largest score difference.
        # (Only with R well above K: with R close to K the retrieval boundary
        # itself decides, where the two sides' FP8 scores legitimately
        # differ by the forward's tolerance.)
        if R < 4 * K:
            continue
        for t in range(W - 1):
            ids_o, ex_o, keep_o, kept_o = O.retrieve_and_rescore(orc["scores"][i][t], head, orc["out"][i][t + 1], R, K)
            union = np.union1d(ids_o, gp["retrieved"][b, t])
            d = np.max(np.abs(O.head_scores(head, orc["out"][i][t + 1], union)[0] -
                              O.head_scores(head, h[b, t + 1], union)[0]))
            got = O.head_scores(head, orc["out"][i][t + 1], gp["cand"][b, t])[0]
            assert np.max(np.abs(np.sort(got)[::-1] - kept_o)) <= 2 * d + 1e-12, f"{label} request {b} row {t + 1}"
    return orc


@pytest.mark.parametrize("which,walk,R", [("A", "sampled", 128), ("T", "greedy", 128), ("T-R16", "sampled", 16),
                                          ("A-B8", "greedy", 128)])
def test_propose_fp8_retrieval_small(which, walk, R):
    """FP8 row-scaled retrieval: one slice (vocab 512) and several slices
    with the refinement's tile path (vocab 2048), R = K, and 128 rows (the
    FP8 GEMM's large-block path)."""
    import block_drafter_amd as bd
    if which == "A":
        case, K = Case(G_A, 171, 3, 9, (40, 7, 25)), 5
    elif which == "A-B8":
        case, K = Case(G_A, 176, 8, 16, (5, 60, 33, 18, 70, 2, 44, 29)), 16
    elif which == "T-R16":
        case, K = Case(G_T, 173, 2, 16, (21, 50)), 16
    else:
        case, K = Case(G_T, 172, 3, 16, (50, 33, 9)), 16
    g = case.g
    wts = synth.make_weights(g, case.seed)
    head = synth.make_lm_head(g, case.seed)
    model = bd.Model.from_numpy(g, wts, lm_head=head)
    run = Run(case, model=model, wts=wts)
    uni = synth.make_uniforms(case.seed, case.B, case.W - 1) if walk == "sampled" else None
    say(f"fp8 {which} {walk}: B={case.B} W={case.W} K={K} R={R}")
    gp = gpu_propose(model, run.ctxs, run.anchors, case.W, K, walk, 0.7, uni, retrieve=R)
    check_retrieval(g, wts, head, O.quantize_head_fp8(head), gp, [run.oracle_ctx(b) for b in range(case.B)],
                    run.anchors, case.W, K, R, walk, 0.7, uni, which)
    # the forward inside the call is the forward, and the direct path is unchanged
    assert np.array_equal(run.gpu_forward(), gp["out"])
    model.close()


@pytest.mark.parametrize("which,walk", [("tiny_fp32", "greedy"), ("A", "sampled"), ("T", "greedy"),
                                        ("T", "sampled"), ("A-W2-K1", "sampled"), ("T-W2", "greedy"),
                                        ("A-B8", "sampled")])
def test_propose_small(which, walk):
    """Edge cases too: W = 2 (one proposal row, conditioned only on the
    anchor), K = 1 (the walk has one choice), and the largest batch."""
    import block_drafter_amd as bd
    if which == "tiny_fp32":
        wl = synth.WORKLOADS["tiny_fp32"]
        case = Case(wl.geom, wl.seed, 1, wl.W, wl.frontiers)
        K = 16
    elif which == "A":
        case = Case(G_A, 71, 3, 9, (40, 7, 25))
        K = 5
    elif which == "A-W2-K1":
        case = Case(G_A, 74, 2, 2, (30, 3))
        K = 1
    elif which == "T-W2":
        case = Case(G_T, 75, 4, 2, (12, 40, 1, 25))
        K = 16
    elif which == "A-B8":
        case = Case(G_A, 76, 8, 16, (5, 60, 33, 18, 70, 2, 44, 29))
        K = 16
    else:
        case = Case(G_T, 72, 3, 16, (50, 33, 9))
        K = 16
    g = case.g
    wts = synth.make_weights(g, case.seed)
    head = synth.make_lm_head(g, case.seed)
    model = bd.Model.from_numpy(g, wts, lm_head=head)
    run = Run(case, model=model, wts=wts)
    uni = synth.make_uniforms(case.seed, case.B, case.W - 1) if walk == "sampled" else None
    say(f"{which} {walk}: B={case.B} W={case.W} K={K}")
    gp = gpu_propose(model, run.ctxs, run.anchors, case.W, K, walk, 0.7, uni)
    check_proposal(g, wts, head, gp, [run.oracle_ctx(b) for b in range(case.B)], run.anchors, case.W, K,
                   walk, 0.7, uni, which)
    # the forward inside the call is the forward
    fwd = run.gpu_forward()
    assert np.array_equal(fwd, gp["out"])
    model.close()


def test_propose_rows_are_per_request():
    """Changing another request's anchor and frontier leaves a request's
    proposal bit-identical (the longest context, which sets the attention
    splits, is unchanged)."""
    import block_drafter_amd as bd
    case = Case(G_T, 73, 2, 12, (45, 30))
    g = case.g
    wts = synth.make_weights(g, case.seed)
    head = synth.make_lm_head(g, case.seed)
    model = bd.Model.from_numpy(g, wts, lm_head=head)
    run = Run(case, model=model, wts=wts)
    a = gpu_propose(model, run.ctxs, run.anchors, case.W, 16, "greedy", 1.0, None)
    run.anchors[1] = (run.anchors[1] + 17) % g.vocab
    run.ctxs[1].frontier = 20
    b = gpu_propose(model, run.ctxs, run.anchors, case.W, 16, "greedy", 1.0, None)
    for k in ("cand", "table", "tokens", "out"):
        assert np.array_equal(a[k][0], b[k][0]), k
    assert not np.array_equal(a["out"][1], b["out"][1])
    c = gpu_propose(model, run.ctxs, run.anchors, case.W, 16, "greedy", 1.0, None)
    for k in ("cand", "table", "tokens", "out"):
        assert np.array_equal(b[k], c[k]), k          # and runs are reproducible
    model.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,walk,requests", [("dspine27b_b1", "greedy", None),
                                                ("dspine27b_b8", "sampled", (0, 5))])
def test_propose_full_size(name, walk, requests):
    """The 27B geometry with a 248320-row head, K = 16: B=1 (greedy walk) and
    B=8 (sampled walk, oracle on two requests over the GPU's rings)."""
    import torch
    import block_drafter_amd as bd
    from tests.test_gpu_fullsize import gpu_ring_context, setup_windows
    wl = synth.WORKLOADS[name]
    g = wl.geom
    say(f"{name}: weights and head")
    wts = synth.make_weights(g, wl.seed)
    head = synth.make_lm_head(g, wl.seed)
    model = bd.Model.from_numpy(g, wts, lm_head=head)
    anchors = [int(a) for a in synth.make_anchor_ids(g, wl.seed, wl.B)]
    ctxs = setup_windows(model, g, wl)
    uni = synth.make_uniforms(wl.seed, wl.B, wl.W - 1) if walk == "sampled" else None
    say(f"{name}: propose ({walk})")
    gp = gpu_propose(model, ctxs, anchors, wl.W, 16, walk, 1.0, uni)
    req = list(range(wl.B)) if requests is None else list(requests)
    say(f"{name}: oracle on requests {req}")
    octxs = [gpu_ring_context(g, ctxs[b], wl.frontiers[b]) for b in req]
    check_proposal(g, wts, head, gp, octxs, anchors, wl.W, 16, walk, 1.0, uni, name, requests=req)
    # the same call with FP8 row-scaled retrieval of 128 candidates per row
    say(f"{name}: propose with FP8 retrieval ({walk})")
    gp8 = gpu_propose(model, ctxs, anchors, wl.W, 16, walk, 1.0, uni, retrieve=128)
    assert np.array_equal(gp8["out"], gp["out"])
    say(f"{name}: oracle FP8 head")
    fp8 = O.quantize_head_fp8(head)
    check_retrieval(g, wts, head, fp8, gp8, octxs, anchors, wl.W, 16, 128, walk, 1.0, uni, name + " fp8",
                    requests=req)
    model.close()
    del model
    torch.cuda.empty_cache()
