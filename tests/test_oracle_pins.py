"""Pins of the CPU oracle against what the sources and mathematics fix.

Each test ties one part of the oracle to something other than the oracle's
own code: closed forms, hand-worked examples, special cases that reduce to a
simpler computation, invariants, brute force, and the figures the pages print
(tests/golden/page_figures.json).  A plausible slip in the oracle (a dropped
term, a wrong sign or index, a transposed operand) fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import dspine_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# a small geometry whose widths all differ, so a transposed operand fails on shape
G_NS = synth.Geometry(hidden=96, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=160,
                      n_feat_layers=3, code_dim=48, msg_dim=24, vocab=64, windows=(12, 0),
                      dtype="f32")


def small_model(g, seed=7, overrides=None):
    return synth.make_weights(g, seed, overrides)


def build_context(g, wts, F, seed=11, request=0, chunks=None):
    ctx = O.empty_context(g)
    feats = synth.make_features(g, seed, request, F)
    if chunks is None:
        chunks = [F]
    s = 0
    for n in chunks:
        ctx = O.materialize(g, wts, ctx, feats[s:s + n])
        s += n
    return ctx


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b)))


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def test_round_bf16_ties_and_values():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1)
    assert O.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert O.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert O.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    assert O.round_bf16(np.array([-3.0]))[0] == -3.0
    # largest finite bf16 and overflow
    assert O.round_bf16(np.array([3.3895313892515355e38]))[0] == 3.3895313892515355e38
    assert np.isinf(O.round_bf16(np.array([3.4e38]))[0])


def test_round_bf16_agrees_with_float32_bit_rounding():
    # the input generator rounds float32 with an integer trick on 32-bit
    # patterns; the oracle rounds float64 patterns.  Two routes, one answer.
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    via_gen = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), via_gen)


def test_round_fp16_of_bf16_is_exact_in_normal_range():
    rng = np.random.default_rng(1)
    x = O.round_bf16(rng.standard_normal(100_000) * 3)
    x = x[np.abs(x) > 2.0 ** -14]
    assert np.array_equal(O.round_fp16(x), x)
    assert O.round_fp16(np.array([1 + 2.0 ** -11]))[0] == 1.0     # tie to even
    assert O.round_fp16(np.array([2.0 ** -24 * 0.75]))[0] == 2.0 ** -24   # subnormal step


# ---------------------------------------------------------------------------
# plain RMSNorm
# ---------------------------------------------------------------------------
def test_rmsnorm_constant_vector_closed_form():
    for kappa in (0.5, 3.0, -2.0):
        x = np.full((1, 8), kappa)
        w = np.linspace(0.5, 2.0, 8)
        got = O.plain_rmsnorm(x, w, 1e-6)
        want = w * kappa / math.sqrt(kappa * kappa + 1e-6)
        assert np.allclose(got[0], want, rtol=1e-15, atol=0)


def test_rmsnorm_unit_rms_output_and_scale_invariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    y = O.plain_rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    y2 = O.plain_rmsnorm(7.5 * x, np.ones(64), 0.0)
    assert np.allclose(y, y2, rtol=1e-13)
    # eps sits inside the square root: a zero row stays zero
    assert np.all(O.plain_rmsnorm(np.zeros((1, 4)), np.ones(4), 1e-6) == 0)


def test_head_rmsnorm_normalises_each_head_separately():
    x = np.concatenate([np.full(4, 2.0), np.full(4, -8.0)])[None]
    got = O.head_rmsnorm(x, np.ones(4), 0.0, 4)
    assert np.allclose(got, np.concatenate([np.ones(4), -np.ones(4)])[None])


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_rope_unit_vectors_hand_values():
    D = 4
    # pair j=0 rotates by p*theta^0 = p radians: e_0 at p=1 -> (cos 1, ., sin 1, .)
    e0 = np.array([[1.0, 0, 0, 0]])
    y = O.rope_1d(e0, np.array([1]), 1e4, D)[0]
    assert np.allclose(y, [0.5403023058681398, 0, 0.8414709848078965, 0], atol=1e-15)
    # pair j=1 has inverse frequency theta^(-2/4) = 1/100 at theta=1e4: p=100 -> 1 rad
    e1 = np.array([[0, 1.0, 0, 0]])
    y = O.rope_1d(e1, np.array([100]), 1e4, D)[0]
    assert np.allclose(y, [0, 0.5403023058681398, 0, 0.8414709848078965], atol=1e-14)
    # the second half rotates the other way round: e_2 -> (-sin, ., cos, .)
    e2 = np.array([[0, 0, 1.0, 0]])
    y = O.rope_1d(e2, np.array([1]), 1e4, D)[0]
    assert np.allclose(y, [-0.8414709848078965, 0, 0.5403023058681398, 0], atol=1e-15)


def test_rope_identity_norm_composition_relative():
    rng = np.random.default_rng(3)
    D = 16
    x = rng.standard_normal((1, 3 * D))
    assert np.array_equal(O.rope_1d(x, np.array([0]), 1e7, D), x)
    p1, p2 = 37, 1234
    y = O.rope_1d(x, np.array([p1]), 1e7, D)
    # rotation per pair preserves every pair's length
    xh = x.reshape(3, D)
    yh = y.reshape(3, D)
    assert np.allclose(xh[:, :8] ** 2 + xh[:, 8:] ** 2, yh[:, :8] ** 2 + yh[:, 8:] ** 2, rtol=1e-13)
    # rotations compose
    assert np.allclose(O.rope_1d(y, np.array([p2]), 1e7, D), O.rope_1d(x, np.array([p1 + p2]), 1e7, D),
                       atol=1e-11)
    # scores depend only on the position difference
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((1, D))
    s1 = (O.rope_1d(q, np.array([500]), 1e7, D) @ O.rope_1d(k, np.array([480]), 1e7, D).T)[0, 0]
    s2 = (O.rope_1d(q, np.array([9020]), 1e7, D) @ O.rope_1d(k, np.array([9000]), 1e7, D).T)[0, 0]
    assert abs(s1 - s2) < 1e-10


# ---------------------------------------------------------------------------
# visibility (a3)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S,F,W", [(8, 20, 5), (12, 12, 4), (16, 40, 16), (2048, 4096, 16)])
def test_window_counts_with_full_left_context(S, F, W):
    for i in range(W):
        n = sum(O.key_visible(S, False, F + i, p, False) for p in range(max(0, F - 3 * S), F))
        assert n == S - 1 - i if i < S else n == 0
        lo, hi = O.visible_context_interval(S, F, i)
        assert hi - lo == max(0, S - 1 - i)
        assert lo == F + i - S + 1 if i < S else lo == F
        nb = sum(O.key_visible(S, False, F + i, F + j, True, i, j) for j in range(W))
        assert nb == W if W <= S else nb <= W


def test_window_endpoints():
    S = 10
    assert O.key_visible(S, False, 100, 100 - (S - 1), False)
    assert not O.key_visible(S, False, 100, 100 - S, False)
    assert O.key_visible(S, False, 100, 100 + S - 1, True)
    assert not O.key_visible(S, False, 100, 100 + S, True)
    assert O.key_visible(0, False, 10 ** 6, 0, False)          # full layer
    # block-causal: later block rows hidden, earlier visible
    assert not O.key_visible(S, True, 100, 101, True, 0, 1)
    assert O.key_visible(S, True, 101, 100, True, 1, 0)


def test_partial_window_intervals():
    # fewer than S positions exist: the symmetric window is clipped at 0
    assert O.visible_context_interval(2048, 1500, 0) == (0, 1500)
    assert O.visible_context_interval(2048, 2040, 15) == (8, 2040)
    assert O.visible_context_interval(0, 77, 3) == (0, 77)
    assert O.visible_context_interval(8, 0, 0) == (0, 0)


# ---------------------------------------------------------------------------
# attention (a6)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("windows,F", [((12, 0), 30), ((12, 0), 7), ((5, 40), 9)])
def test_attention_bruteforce_matches_vectorised(causal, windows, F):
    g = synth.with_geometry(G_NS, windows=windows, block_causal=causal)
    wts = small_model(g)
    ctx = build_context(g, wts, F)
    rng = np.random.default_rng(4)
    W = 6
    q = rng.standard_normal((W, g.q_dim))
    k = rng.standard_normal((W, g.kv_dim))
    v = rng.standard_normal((W, g.kv_dim))
    for layer in range(g.n_layers):
        a = O.block_attention(g, layer, ctx, q, k, v)
        b = O.block_attention_bruteforce(g, layer, ctx, q, k, v)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_attention_single_key_returns_its_value():
    # W=1 with no context: the only key is the row itself, softmax weight 1
    g = synth.with_geometry(G_NS, windows=(0, 0))
    ctx = O.empty_context(g, 0)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, g.q_dim))
    k = rng.standard_normal((1, g.kv_dim))
    v = rng.standard_normal((1, g.kv_dim))
    out = O.block_attention(g, 0, ctx, q, k, v)
    grp = g.n_q_heads // g.n_kv_heads
    for h in range(g.n_q_heads):
        kvh = h // grp
        assert np.allclose(out[0, h * 16:(h + 1) * 16], v[0, kvh * 16:(kvh + 1) * 16], rtol=1e-15)


def test_attention_mha_equals_gqa_with_repeated_heads():
    g = synth.with_geometry(G_NS, windows=(12, 0))
    g_mha = synth.with_geometry(g, n_kv_heads=g.n_q_heads)
    wts = small_model(g)
    ctx = build_context(g, wts, 25)
    grp = g.n_q_heads // g.n_kv_heads
    D = g.head_dim

    def rep(a):   # repeat every KV head grp times along the head axis
        n = a.shape[0]
        return np.repeat(a.reshape(n, g.n_kv_heads, D), grp, axis=1).reshape(n, -1)

    ctx_mha = O.RequestContext(ctx.frontier, [O.LayerContext(lc.lo, rep(lc.k), rep(lc.v))
                                              for lc in ctx.layers])
    rng = np.random.default_rng(6)
    W = 5
    q = rng.standard_normal((W, g.q_dim))
    k = rng.standard_normal((W, g.kv_dim))
    v = rng.standard_normal((W, g.kv_dim))
    for layer in range(2):
        a = O.block_attention(g, layer, ctx, q, k, v)
        b = O.block_attention(g_mha, layer, ctx_mha, q, rep(k), rep(v))
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_attention_reads_through_ring_slots_like_flat_positions():
    # truncation equivalence (iii): attention that fetches every context key
    # from its ring slot p mod S equals attention over keys by position.
    g = synth.with_geometry(G_NS, windows=(12, 9))
    wts = small_model(g)
    ctx = build_context(g, wts, 53, chunks=[20, 1, 32])
    rng = np.random.default_rng(8)
    W = 7
    q = rng.standard_normal((W, g.q_dim))
    k = rng.standard_normal((W, g.kv_dim))
    v = rng.standard_normal((W, g.kv_dim))
    D = g.head_dim
    grp = g.n_q_heads // g.n_kv_heads
    for layer in range(2):
        S = g.windows[layer]
        K, V = O.ring_image(g, ctx, layer, S)
        F = ctx.frontier
        want = O.block_attention(g, layer, ctx, q, k, v)
        got = np.zeros_like(want)
        for h in range(g.n_q_heads):
            kvh = h // grp
            for i in range(W):
                lo, hi = O.visible_context_interval(S, F, i)
                keys = [K[kvh, p % S] for p in range(lo, hi)] + [k[j, kvh * D:(kvh + 1) * D] for j in range(W)]
                vals = [V[kvh, p % S] for p in range(lo, hi)] + [v[j, kvh * D:(kvh + 1) * D] for j in range(W)]
                s = np.array([q[i, h * D:(h + 1) * D] @ kk for kk in keys]) / math.sqrt(D)
                e = np.exp(s - s.max())
                got[i, h * D:(h + 1) * D] = (e[:, None] * np.array(vals)).sum(0) / e.sum()
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# context materialization (a1-a3)
# ---------------------------------------------------------------------------
def test_context_hand_worked():
    """Lf=2, H=2: s = [1,2,3,4]; W_feat picks s0 and s3 -> u = [1,4], rms(u) =
    sqrt(8.5); gain [2, 0.5] -> c = [2,2]/sqrt(8.5).  W_k = I and the head
    norm of c is [1,1]; position 0 is unrotated, position 1 turns pair (0,1) by
    one radian -> [cos1 - sin1, cos1 + sin1].  v = [[0,2],[1,0]] c."""
    g = synth.Geometry(hidden=2, n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn=1,
                       n_feat_layers=2, code_dim=0, msg_dim=0, vocab=4, windows=(0,), eps=0.0,
                       rope_theta=1e4, dtype="f32")
    f32 = lambda a: np.array(a, dtype=np.float32)
    wts = synth.make_weights(g, 1, {
        "w_feat": f32([[1, 0, 0, 0], [0, 0, 0, 1]]), "g_ctx": f32([2, 0.5]),
        "l0.wk": f32([[1, 0], [0, 1]]), "l0.gk": f32([1, 1]), "l0.wv": f32([[0, 2], [1, 0]]),
    })
    feats = f32([[1, 2, 3, 4], [1, 2, 3, 4]])
    ctx = O.materialize(g, wts, O.empty_context(g), feats)
    assert np.allclose(ctx.layers[0].k[0], [1.0, 1.0], rtol=1e-7)
    assert np.allclose(ctx.layers[0].v[0], [1.3719886811400706, 0.6859943405700353], rtol=1e-7)
    assert np.allclose(ctx.layers[0].k[1], [-0.30116867893975674, 1.3817732906760363], rtol=1e-6)


def test_chunk_truncation_and_subchunks():
    g = synth.with_geometry(G_NS, windows=(12, 9), dtype="bf16")
    wts = small_model(g)
    n = 40
    feats = synth.make_features(g, 11, 0, n)
    one = O.materialize(g, wts, O.empty_context(g), feats)
    # (ii) the same chunk in sub-chunks
    parts = O.empty_context(g)
    for a, b in [(0, 3), (3, 17), (17, 18), (18, 40)]:
        parts = O.materialize(g, wts, parts, feats[a:b])
    # (i) only the last max(S) positions, from a context whose frontier is n - 12
    tail = O.materialize(g, wts, O.empty_context(g, n - 12), feats[n - 12:])
    for layer in range(2):
        S = g.windows[layer]
        r1 = O.ring_image(g, one, layer, S)
        for other in (parts, tail):
            r2 = O.ring_image(g, other, layer, S)
            for a, b in zip(r1, r2):
                assert np.array_equal(np.isnan(a), np.isnan(b))
                m = ~np.isnan(a)
                assert np.max(np.abs(a[m] - b[m])) <= 1e-2 * np.sqrt(np.mean(a[m] ** 2))
                assert np.mean(a[m] == b[m]) > 0.999   # identical up to rare rounding flips
    assert one.frontier == parts.frontier == tail.frontier == n
    assert one.layers[0].lo == n - 12 and one.layers[1].lo == n - 9


def test_stored_formats_are_bf16_and_fp16_of_bf16():
    g = synth.with_geometry(G_NS, dtype="bf16")
    wts = small_model(g)
    ctx = build_context(g, wts, 30)
    for lc in ctx.layers:
        assert np.array_equal(O.round_bf16(lc.k), lc.k)
        assert np.array_equal(O.round_bf16(lc.v), lc.v)
        assert np.array_equal(O.round_fp16(lc.v), lc.v)


def test_full_layer_keeps_everything_local_layer_keeps_window():
    g = synth.with_geometry(G_NS, windows=(12, 0))
    wts = small_model(g)
    ctx = build_context(g, wts, 50, chunks=[30, 20])
    assert ctx.layers[0].lo == 38 and ctx.layers[0].k.shape[0] == 12
    assert ctx.layers[1].lo == 0 and ctx.layers[1].k.shape[0] == 50


# ---------------------------------------------------------------------------
# the bridge (a9-a11)
# ---------------------------------------------------------------------------
def bridge_geom():
    return synth.Geometry(hidden=2, n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn=1,
                          n_feat_layers=1, code_dim=2, msg_dim=1, vocab=4, windows=(0,), eps=0.0,
                          dtype="f32")


def bridge_weights(g):
    f32 = lambda a: np.array(a, dtype=np.float32)
    s2 = math.sqrt(2.0)
    return synth.make_weights(g, 1, {
        "l0.R": f32([[1, 0], [0, 1]]),
        "bridge_G": f32([[0, 1]]), "bridge_Gp": f32([[1, 0]]), "bridge_A": f32([[2, 0]]),
        "bridge_b": f32([-9 * s2 / 5]),
        "l0.W_l": f32([[1], [-1]]),
        "codebook": f32([[0, 1], [1, 0], [0.6, 0.8], [0.8, 0.6]]),
    })


def test_bridge_hand_worked():
    """Receiver x1=[3,4]: rho=5/sqrt2, z=[3,4]/rho, c1=sqrt2*[3,4]/5.  Anchor
    id 1: c0 = sqrt2*[1,0].  Gate argument: G c1 + Gp c0 + b = 4sqrt2/5 + sqrt2
    - 9sqrt2/5 = 0 -> gate 1/2.  Message: 1/2 * A c0 = sqrt2.  Write: rho * W_l
    * sqrt2 = (5/sqrt2)*[sqrt2, -sqrt2] = [5, -5] -> x1' = [8, -1]."""
    g = bridge_geom()
    wts = bridge_weights(g)
    x = np.array([[1.0, 1.0], [3.0, 4.0]])
    out = O.bridge(g, wts, 0, x, anchor_id=1)
    assert np.array_equal(out[0], x[0])
    assert np.allclose(out[1], [8.0, -1.0], rtol=0, atol=1e-6)   # b and weights carry fp32 rounding
    # codes: norms sqrt(r) and the anchor code from the codebook row
    rho, c = O.bridge_codes(g, wts, 0, x, 1)
    assert np.allclose(rho, [1.0, 5 / math.sqrt(2)], rtol=1e-15)
    assert np.allclose(c[0], [math.sqrt(2), 0.0], rtol=1e-15)
    assert np.allclose(c[1], [3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5], rtol=1e-15)


def test_bridge_predecessor_override():
    """With the predecessor code of receiver 1 replaced by sqrt2*C[3] =
    sqrt2*[0.8,0.6]: gate arg = 4sqrt2/5 + 0.8sqrt2 - 9sqrt2/5 = -0.2sqrt2,
    message = sigmoid(-0.2sqrt2) * 1.6sqrt2, write = rho W_l m."""
    g = bridge_geom()
    wts = bridge_weights(g)
    x = np.array([[1.0, 1.0], [3.0, 4.0]])
    s2 = math.sqrt(2.0)
    pred = np.zeros((2, 2))
    pred[1] = s2 * np.array([0.8, 0.6], dtype=np.float32).astype(np.float64)
    out = O.bridge(g, wts, 0, x, anchor_id=1, pred_codes=pred)
    m = 1.6 * s2 / (1.0 + math.exp(0.2 * s2))
    w = (5 / s2) * m
    assert np.allclose(out[1], [3 + w, 4 - w], atol=1e-6)


def test_bridge_zero_row_gives_zero_code_and_no_write():
    g = bridge_geom()
    wts = bridge_weights(g)
    x = np.array([[1.0, 1.0], [0.0, 0.0], [2.0, 5.0]])
    g2 = synth.with_geometry(g, eps=1e-6)
    rho, c = O.bridge_codes(g2, wts, 0, x, 1)
    assert rho[1] == 0 and np.all(c[1] == 0)
    out = O.bridge(g2, wts, 0, x, 1)
    assert np.array_equal(out[1], x[1])        # rho = 0: no write


def test_bridge_code_norm_is_sqrt_r():
    g = G_NS
    wts = small_model(synth.with_geometry(g, dtype="f32"))
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, g.hidden)) * 3
    rho, c = O.bridge_codes(g, wts, 1, x, 5)
    norms = np.linalg.norm(c, axis=-1)
    assert np.allclose(norms[1:], math.sqrt(g.code_dim), rtol=1e-5)
    # anchor code: sqrt(r) times a unit row (unit up to the fp32 rounding of the row)
    assert abs(norms[0] - math.sqrt(g.code_dim)) < 1e-5


def test_bridge_adjacency_and_anchor():
    g = G_NS
    wts = small_model(g)
    rng = np.random.default_rng(10)
    W = 8
    x = rng.standard_normal((W, g.hidden))
    base = O.bridge(g, wts, 0, x, 3)
    assert np.array_equal(base[0], x[0])
    for j in range(W):
        xp = x.copy()
        xp[j] += rng.standard_normal(g.hidden)
        out = O.bridge(g, wts, 0, xp, 3)
        # the anchor's code comes from the codebook, so a change to row 0
        # reaches no other row; any other row j reaches j and j+1 only
        changed = {0} if j == 0 else {j, j + 1}
        for t in range(W):
            same = np.array_equal(out[t], base[t])
            assert same == (t not in changed), (j, t)


# ---------------------------------------------------------------------------
# one decoder layer, hand-worked (a4-a8, a12)
# ---------------------------------------------------------------------------
def test_decoder_layer_hand_worked():
    """H=2, one head of width 2, FFN width 1, one block row and no context.
    With a single key the attention output is v.  x=[1,1] -> n = g_in*x =
    [1,2]; v = n; W_o v = [0,6]; y = [1,7] (rms 5); g_post = [0.5, 1] -> m =
    [0.1, 1.4]; gate = 100*0.1 = 10, up = 5*0.1 = 0.5; SiLU(10)*0.5 =
    5/(1+e^-10); x' = [1 + 5/(1+e^-10), 7].  Final norm divides by
    sqrt(mean(x'^2))."""
    g = synth.Geometry(hidden=2, n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn=1,
                       n_feat_layers=1, code_dim=0, msg_dim=0, vocab=4, windows=(0,), eps=0.0,
                       rope_theta=1e4, dtype="f32")
    f32 = lambda a: np.array(a, dtype=np.float32)
    wts = synth.make_weights(g, 1, {
        "embed": f32([[0, 0], [1, 1], [0, 0], [5, 5]]),
        "l0.g_in": f32([1, 2]), "l0.wq": f32([[1, 0], [0, 1]]), "l0.wk": f32([[1, 0], [0, 1]]),
        "l0.wv": f32([[1, 0], [0, 1]]), "l0.gq": f32([1, 1]), "l0.gk": f32([1, 1]),
        "l0.wo": f32([[0, 0], [0, 3]]), "l0.g_post": f32([0.5, 1]),
        "l0.w_gate": f32([[100, 0]]), "l0.w_up": f32([[5, 0]]), "l0.w_down": f32([[1], [0]]),
        "g_final": f32([1, 1]),
    })
    ctx = O.empty_context(g, 0)
    out, states = O.draft_forward(g, wts, [ctx], [1], W=1, return_layers=True)
    x1 = np.array([1 + 4.9997730106564875, 7.0])
    assert np.allclose(states[0][0], x1, rtol=1e-12)
    r = math.sqrt((x1[0] ** 2 + 49.0) / 2)
    assert np.allclose(out[0, 0], x1 / r, rtol=1e-12)


def test_layer_with_zero_output_maps_is_identity():
    g = synth.with_geometry(G_NS, code_dim=0, msg_dim=0)
    z = lambda name: np.zeros(synth.weight_shape(g, name), np.float32)
    wts = small_model(g, overrides={f"l{l}.{n}": z(f"l{l}.{n}") for l in range(2) for n in ("wo", "w_down")})
    ctx = build_context(g, wts, 20)
    out, states = O.draft_forward(g, wts, [ctx], [3], W=5, return_layers=True)
    x0 = O.block_input(g, wts, 3, 5)
    assert np.array_equal(states[-1], x0)


# ---------------------------------------------------------------------------
# whole-forward invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("which", ["W_l", "A", "gate_closed", "init"])
def test_bridge_identity_reduces_to_plain_dflash(which):
    """[PHY, 门控与写回]: with W_l = 0 (or no message, or a closed gate) every
    write is zero and the forward is exactly the bridge-free DFlash forward."""
    g = G_NS
    ov = {}
    if which in ("W_l", "init"):
        for l in range(g.n_layers):
            ov[f"l{l}.W_l"] = np.zeros(synth.weight_shape(g, f"l{l}.W_l"), np.float32)
    if which == "A":
        ov["bridge_A"] = np.zeros(synth.weight_shape(g, "bridge_A"), np.float32)
    if which == "gate_closed":
        ov["bridge_b"] = np.full(g.msg_dim, -1e4, np.float32)
    if which == "init":
        ov["bridge_Gp"] = np.zeros(synth.weight_shape(g, "bridge_Gp"), np.float32)
        ov["bridge_b"] = np.zeros(g.msg_dim, np.float32)
    wts = small_model(g, overrides=ov)
    g_off = synth.with_geometry(g, code_dim=0, msg_dim=0)
    ctxs = [build_context(g, wts, 30, request=0), build_context(g, wts, 9, request=1)]
    a = O.draft_forward(g, wts, ctxs, [3, 17], W=6)
    b = O.draft_forward(g_off, wts, ctxs, [3, 17], W=6)
    assert np.array_equal(a, b)
    # and the bridge does change things when it is active
    c = O.draft_forward(g, small_model(g), ctxs, [3, 17], W=6)
    assert not np.allclose(c, b)


def test_no_cross_request_leakage():
    g = G_NS
    wts = small_model(g)
    c0 = build_context(g, wts, 30, request=0)
    c1 = build_context(g, wts, 19, request=1)
    c1b = build_context(g, wts, 25, seed=99, request=1)
    a = O.draft_forward(g, wts, [c0, c1], [3, 17], W=6)
    b = O.draft_forward(g, wts, [c0, c1b], [3, 40], W=6)
    assert rel_err(b[0], a[0]) < 1e-12
    assert rel_err(b[1], a[1]) > 1e-3


def test_rope_shift_invariance_of_forward():
    """Re-materialising the same features Delta positions later (with Delta
    unseen filler positions in front) leaves every output unchanged: only
    position differences enter the scores.  Windows are full in both runs."""
    g = synth.with_geometry(G_NS, windows=(12, 20))
    wts = small_model(g)
    F, delta, W = 40, 1000, 6
    feats = synth.make_features(g, 11, 0, F)
    a_ctx = O.materialize(g, wts, O.empty_context(g), feats)
    b_ctx = O.materialize(g, wts, O.empty_context(g, delta), feats)
    a = O.draft_forward(g, wts, [a_ctx], [3], W)
    b = O.draft_forward(g, wts, [b_ctx], [3], W)
    assert rel_err(b, a) < 1e-5


def test_window_wider_than_context_equals_full_attention():
    g = synth.with_geometry(G_NS, windows=(64, 64))
    g_full = synth.with_geometry(G_NS, windows=(0, 0))
    wts = small_model(g)
    ctx = build_context(g, wts, 40)                       # F + W <= 64
    a = O.draft_forward(g, wts, [ctx], [3], 8)
    b = O.draft_forward(g_full, wts, [ctx], [3], 8)
    assert np.array_equal(a, b)


def test_bidirectional_block_is_not_prefix_stable_but_causal_is():
    """[NIF, draft attention]: with a non-causal block a shorter block need
    not match the prefix of a longer one; with block-causal attention and no
    bridge reach beyond t-1 the first rows of a W-block equal a W'-block."""
    for causal in (False, True):
        g = synth.with_geometry(G_NS, block_causal=causal)
        wts = small_model(g)
        ctx = build_context(g, wts, 30)
        a = O.draft_forward(g, wts, [ctx], [3], 8)
        b = O.draft_forward(g, wts, [ctx], [3], 5)
        if causal:
            assert rel_err(b[0], a[0, :5]) < 1e-12
        else:
            assert rel_err(b[0], a[0, :5]) > 1e-4


# ---------------------------------------------------------------------------
# figures the pages print
# ---------------------------------------------------------------------------
def test_page_figures():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    g27 = synth.G_27B
    per_pos = O.ring_bytes_per_position(g27)
    assert per_pos == fig["draft_kv_bytes_per_position"]["value"]
    assert per_pos * 8192 / 2 ** 20 == fig["draft_kv_window_8192_mib"]["value"]
    assert per_pos * 131072 / 2 ** 30 == fig["draft_kv_131072_gib"]["value"]
    assert per_pos * 2048 / 2 ** 20 == fig["ring_image_mib"]["value"]
    assert g27.vocab * g27.code_dim * 2 / 2 ** 20 == fig["codebook_mib"]["value"]
    assert g27.vocab * (512 + 1024) * 2 / 2 ** 20 == fig["greedy_tail_tables_mib"]["value"]
    n = O.bridge_parameter_count(4096, 5, 1024, 512)
    assert n == 33_030_656 and round(n / 1e6) == fig["bridge_parameters_millions_approx"]["value"]
    geo = fig["drafter_27b_geometry"]
    assert (g27.hidden, g27.n_layers, g27.ffn) == (geo["hidden"], geo["n_layers"], geo["ffn"])
    assert g27.q_dim == geo["q_width"] and g27.n_feat_layers * g27.hidden == geo["feature_concat_width"]
    assert (g27.code_dim, g27.msg_dim, g27.rope_theta) == (geo["code_dim"], geo["msg_dim"], geo["rope_theta"])
    for name, shape in (("l0.R", (1024, 5120)), ("l0.W_l", (5120, 512)), ("codebook", (248320, 1024)),
                        ("w_feat", (5120, 25600)), ("l0.wq", (4096, 5120))):
        assert synth.weight_shape(g27, name) == shape


# ---------------------------------------------------------------------------
# proposal tail: candidates, last-write refinement, transition table, walk
# [FLZ, "The last write is refined using discrete candidates"];
# [PHY, 前驱条件解码与 transition cache]
# ---------------------------------------------------------------------------
def propose_setup(overrides=None, B=1, W=5):
    g = G_NS
    wts = small_model(g, overrides=overrides)
    head = synth.make_lm_head(g, 7)
    ctxs = [build_context(g, wts, 10 + 3 * b, request=b) for b in range(B)]
    anchors = [5 + 17 * b for b in range(B)]
    return g, wts, head, ctxs, anchors, W


def test_top_k_against_sorted_bruteforce():
    rng = np.random.default_rng(3)
    scores = rng.integers(0, 5, size=50).astype(np.float64)      # many ties
    ranked = [i for _, i in sorted((-s, i) for i, s in enumerate(scores))]
    for K in (1, 7, 50):
        assert list(O.top_k(scores, K)) == ranked[:K]


def test_head_scores_are_row_dot_products():
    g, wts, head, ctxs, anchors, W = propose_setup()
    h = np.random.default_rng(4).standard_normal((2, g.hidden))
    s = O.head_scores(head, h)
    assert s.shape == (2, g.vocab)
    E = synth.to_float(head)
    for n in range(2):
        for v in (0, 13, g.vocab - 1):
            assert abs(s[n, v] - math.fsum(E[v, k] * h[n, k] for k in range(g.hidden))) < 1e-12
    assert np.max(np.abs(O.head_scores(head, h, [13, 2])[:, 0] - s[:, 13])) < 1e-14


# ---------------------------------------------------------------------------
# FP8 row-scaled retrieval
# ---------------------------------------------------------------------------
def e4m3_values():
    """Every finite non-negative OCP E4M3 value, from the format's definition:
    bits eeee.mmm, bias 7; exponent field 0 is subnormal (m/8 * 2^-6); field
    15 with mantissa 7 is NaN (no infinities)."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            out.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(sorted(set(out)))


def test_fp8_e4m3_hand_values():
    r = O.round_fp8_e4m3
    assert r(448.0) == 448.0 and r(-448.0) == -448.0
    assert r(440.0) == 448.0 and r(415.0) == 416.0           # steps of 32 in [256, 512)
    assert r(1.0625) == 1.0                                   # tie: even mantissa 0
    assert r(1.1875) == 1.25                                  # tie: 1.125 (m=1) vs 1.25 (m=2)
    assert r(0.3) == 0.3125                                   # 9.6 steps of 2^-5
    assert r(2.0 ** -10) == 0.0                               # tie between 0 and 2^-9
    assert r(3 * 2.0 ** -10) == 2.0 ** -8                     # tie between 2^-9 and 2^-8
    assert r(2.0 ** -9) == 2.0 ** -9 and r(2.0 ** -6) == 2.0 ** -6
    assert r(-0.0) == 0.0 and r(7.4) == 7.5


def test_fp8_e4m3_fixed_points_and_midpoints():
    vals = e4m3_values()
    assert len(vals) == 127 and vals[-1] == 448.0 and vals[1] == 2.0 ** -9
    assert np.array_equal(O.round_fp8_e4m3(vals), vals)
    assert np.array_equal(O.round_fp8_e4m3(-vals), -vals)
    mids = (vals[:-1] + vals[1:]) / 2
    got = O.round_fp8_e4m3(mids)
    # ties go to the neighbour whose mantissa is even (its step count is even)
    lo, hi = vals[:-1], vals[1:]
    mant_lo = np.array([round((v / 2.0 ** max(math.frexp(v)[1] - 1, -6)) * 8) % 2 if v > 0 else 0 for v in lo])
    want = np.where(mant_lo == 0, lo, hi)
    assert np.array_equal(got, want)
    # just off the midpoints the nearest value wins
    assert np.array_equal(O.round_fp8_e4m3(mids * (1 - 1e-9)), lo)
    assert np.array_equal(O.round_fp8_e4m3(mids * (1 + 1e-9)), hi)


def test_fp8_e4m3_matches_torch_cast():
    """torch's float8_e4m3fn cast (ties to even) on float32 inputs of every
    magnitude the head codes take, subnormals included."""
    import torch
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 8.7, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    x = np.concatenate([x, (e4m3_values()[:-1] + e4m3_values()[1:]).astype(np.float32) / 2])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.round_fp8_e4m3(x.astype(np.float64)), want)


def test_fp8_head_scales_and_codes():
    rng = np.random.default_rng(13)
    E = rng.standard_normal((40, 64)) * np.exp2(rng.uniform(-20, 10, (40, 1)))
    E[3] = 0.0
    E[5, :] = 0.25
    E[5, 7] = 448.0 * 2.0 ** -3              # max exactly 448 x a power of two
    head = synth.f32_to_bf16_bits(E.astype(np.float32))
    Ew = synth.to_float(head)
    codes, sc = O.quantize_head_fp8(head)
    mant, _ = np.frexp(sc)
    assert np.all(mant == 0.5)                                   # powers of two
    nz = np.arange(40) != 3
    top = np.max(np.abs(Ew), axis=1)[nz] / sc[nz]
    assert np.all(top <= 448) and np.all(top > 224)              # the smallest such power of two
    m = np.max(np.abs(codes), axis=1)
    assert np.all(m[nz] <= 448) and np.all(m[nz] >= 224)
    assert sc[3] == 1.0 and np.all(codes[3] == 0)
    assert sc[5] == 2.0 ** -3 and codes[5, 7] == 448.0 and codes[5, 0] == 2.0
    assert np.array_equal(O.round_fp8_e4m3(codes), codes)       # codes are E4M3 values
    # one rounding of E / s: within half a step of the E4M3 grid
    x = Ew / sc[:, None]
    assert np.all(np.abs(codes - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10) + 1e-300)


def test_fp8_scores_exact_for_representable_head():
    """A head whose rows are E4M3 values times a power of two (max at 448 x
    2^k) is held exactly by the FP8 copy: its approximate scores equal the
    BF16 scores, and the retrieval keeps the direct path's top-K."""
    rng = np.random.default_rng(14)
    vals = e4m3_values()
    V, H = 300, 32
    k = np.exp2(rng.integers(-12, -4, (V, 1)))
    E = rng.choice(np.concatenate([vals, -vals]), size=(V, H)) * k
    E[:, 0] = 448.0 * k[:, 0]
    head = synth.f32_to_bf16_bits(E.astype(np.float32))
    assert np.array_equal(synth.to_float(head), E)
    codes, sc = O.quantize_head_fp8(head)
    h = rng.standard_normal((3, H))
    approx = O.head_scores_fp8(codes, sc, h)
    exact = O.head_scores(head, h)
    assert np.max(np.abs(approx - exact)) <= 1e-12 * np.max(np.abs(exact))
    for n in range(3):
        ids, ex, keep, kept = O.retrieve_and_rescore(approx[n], head, h[n], 20, 5)
        assert list(keep) == list(O.top_k(exact[n], 5))


def test_retrieval_covering_the_vocabulary_is_the_direct_path():
    """R >= V: every token is rescored with the BF16 head, so the K kept are
    the direct path's top-K, best first, ties by the smaller id."""
    g, wts, head, ctxs, anchors, W = propose_setup()
    rng = np.random.default_rng(15)
    h = rng.standard_normal((4, g.hidden))
    codes, sc = O.quantize_head_fp8(head)
    approx = O.head_scores_fp8(codes, sc, h)
    exact = O.head_scores(head, h)
    for n in range(4):
        ids, ex, keep, kept = O.retrieve_and_rescore(approx[n], head, h[n], g.vocab, 6)
        assert sorted(ids) == list(range(g.vocab))
        assert list(keep) == list(O.top_k(exact[n], 6))
        assert np.max(np.abs(kept - exact[n, keep])) <= 1e-12 * np.max(np.abs(kept))
        # the approximation is close but not exact (the FP8 codes round)
        assert 0 < np.max(np.abs(approx[n] - exact[n])) < 0.1 * np.sqrt(np.mean(exact[n] ** 2))


def test_retrieval_keeps_the_fp8_best_and_can_miss_the_bf16_best():
    """The kept tokens are the R best FP8 scores re-sorted by their BF16
    scores, so a token whose FP8 score falls outside the R best is lost even
    when its BF16 score is the best [FLZ: rescoring does not prove that the
    retrieval held the global BF16 top-16].  Hand case, H = 1, h = 1: token 0
    has E = 1 (exact in FP8), token 1 has E = 1 + 2^-7 whose FP8 code rounds
    to 1 (scale 2^-8: 258 -> 256), token 2 has E = 0.5; with R = 1 the FP8
    tie goes to token 0 and token 1, the BF16 best, is missed."""
    head = synth.f32_to_bf16_bits(np.array([[1.0], [1.0 + 2.0 ** -7], [0.5]], dtype=np.float32))
    codes, sc = O.quantize_head_fp8(head)
    assert list(sc) == [2.0 ** -8, 2.0 ** -8, 2.0 ** -9] and list(codes[:, 0]) == [256.0, 256.0, 256.0]
    h = np.array([1.0])
    approx = O.head_scores_fp8(codes, sc, h[None])[0]
    assert list(approx) == [1.0, 1.0, 0.5]
    ids, ex, keep, kept = O.retrieve_and_rescore(approx, head, h, 1, 1)
    assert list(ids) == [0] and list(keep) == [0]
    ids, ex, keep, kept = O.retrieve_and_rescore(approx, head, h, 2, 2)
    assert list(ids) == [0, 1] and list(keep) == [1, 0] and list(kept) == [1.0 + 2.0 ** -7, 1.0]
    # ties in the BF16 rescoring keep the smaller token first
    head2 = synth.f32_to_bf16_bits(np.array([[0.75], [0.75], [0.25]], dtype=np.float32))
    c2, s2 = O.quantize_head_fp8(head2)
    a2 = O.head_scores_fp8(c2, s2, h[None])[0]
    ids, ex, keep, kept = O.retrieve_and_rescore(a2, head2, h, 3, 2)
    assert list(keep) == [0, 1]


def test_propose_with_retrieval_uses_rescored_candidates():
    """The proposal with FP8 retrieval: candidates are the rescored best K of
    the R retrieved, their scores are BF16 head scores, and with R = V the
    whole proposal equals the direct path's."""
    g, wts, head, ctxs, anchors, W = propose_setup()
    direct = O.propose(g, wts, head, ctxs, anchors, W, K=4)
    full = O.propose(g, wts, head, ctxs, anchors, W, K=4, retrieve=g.vocab)
    for k in ("cand", "cand_scores", "table", "choice", "tokens"):
        assert np.array_equal(direct[k], full[k]) or np.max(np.abs(direct[k] - full[k])) < 1e-12, k
    part = O.propose(g, wts, head, ctxs, anchors, W, K=4, retrieve=8)
    assert part["retrieved"].shape == (len(ctxs), W - 1, 8)
    for b in range(len(ctxs)):
        for t in range(W - 1):
            ids = part["retrieved"][b, t]
            assert list(ids) == list(O.top_k(part["scores"][b, t], 8))
            assert set(part["cand"][b, t]) <= set(ids)
            assert np.all(np.diff(part["cand_scores"][b, t]) <= 0)


def test_anchor_conditioned_table_reproduces_forward_scores():
    """Row 1's predecessor is the anchor, whose code the forward's own last
    write already used: every row of T_1 equals the forward's head scores on
    row 1's candidates (the refinement path and the forward path agree)."""
    g, wts, head, ctxs, anchors, W = propose_setup()
    res = O.propose(g, wts, head, ctxs, anchors, W, K=4)
    T, cand, sc = res["table"][0], res["cand"][0], res["scores"][0]
    assert T.shape == (W - 1, 4, 4) and cand.shape == (W - 1, 4)
    for i in range(4):
        assert rel_err(T[0, i], sc[0, cand[0]]) < 1e-12
    # candidates are the forward's top-4 of each row
    for t in range(W - 1):
        assert list(cand[t]) == list(O.top_k(sc[t], 4))
        assert np.all(np.diff(sc[t, cand[t]]) <= 0)


def test_predicted_code_predecessor_reproduces_forward_row():
    """If a predecessor candidate's codebook row equals the predicted code
    of row t-1 (divided by sqrt(r)), refining with that candidate redoes the
    forward's own last write, so its row of T_t equals the forward's scores."""
    g, wts, head, ctxs, anchors, W = propose_setup()
    res = O.propose(g, wts, head, ctxs, anchors, W, K=4)
    cand = res["cand"][0]
    _, u = O.draft_forward(g, wts, ctxs, anchors, W, return_last_prewrite=True)
    rho, c = O.bridge_codes(g, wts, g.n_layers - 1, u[0], anchors[0])
    for t in (2, 3):
        i0 = next(i for i in range(4) if cand[t - 2][i] != anchors[0])
        book = wts["codebook"].copy()
        book[cand[t - 2][i0]] = (c[t - 1] / math.sqrt(g.code_dim)).astype(book.dtype)
        res2 = O.propose(g, dict(wts, codebook=book), head, ctxs, anchors, W, K=4, cand_override=res["cand"])
        assert rel_err(res2["table"][0][t - 1, i0], res["scores"][0][t - 1, cand[t - 1]]) < 1e-5


@pytest.mark.parametrize("which", ["W_last_zero", "gate_closed"])
def test_table_without_last_write_is_the_forward_scores(which):
    """With the last layer's write off, refinement changes nothing: every
    T_t[i, :] equals the forward's scores on row t's candidates."""
    g = G_NS
    L = g.n_layers - 1
    ov = {f"l{L}.W_l": np.zeros((g.hidden, g.msg_dim), np.float32)} if which == "W_last_zero" else \
        {"bridge_b": np.full(g.msg_dim, -1e4, np.float32)}
    g, wts, head, ctxs, anchors, W = propose_setup(ov)
    res = O.propose(g, wts, head, ctxs, anchors, W, K=4)
    T, cand, sc = res["table"][0], res["cand"][0], res["scores"][0]
    for t in range(W - 1):
        for i in range(4):
            assert rel_err(T[t, i], sc[t, cand[t]]) < 1e-12


def test_table_rows_depend_on_the_predecessor():
    g, wts, head, ctxs, anchors, W = propose_setup()
    T = O.propose(g, wts, head, ctxs, anchors, W, K=4)["table"][0]
    for t in range(1, W - 1):
        assert np.max(np.abs(T[t, 0] - T[t, 1])) > 1e-6


def test_greedy_walk_hand_example():
    T = np.array([[[1, 3, 2], [9, 9, 9], [9, 9, 9]],        # row 1: anchor row 0 -> 1
                  [[0, 0, 0], [5, 4, 6], [0, 9, 0]],        # row 2: given 1 -> 2
                  [[1, 0, 0], [0, 2, 0], [0, 0, -1]]],      # row 3: given 2 -> 0 (tie, smaller index)
                 dtype=np.float64)
    assert list(O.greedy_walk(T)) == [1, 2, 0]


def test_sampled_walk_definition():
    from scipy.special import softmax
    T = np.array([[[0.0, 0.0], [0.0, 0.0]],       # row 1 (anchor row 0): p = (1/2, 1/2)
                  [[1.0, 2.0], [7.0, -7.0]]])     # row 2, given choice 0 or 1
    # inverse CDF: u = 0.5 equals p_0 exactly, so the first j with cdf > u is 1
    ch, q = O.sampled_walk(T, 1.0, np.array([0.5, 0.0]))
    assert list(ch) == [1, 0] and q[0] == 0.5
    assert abs(q[1] - softmax(np.array([7.0, -7.0]))[0]) < 1e-15
    # temperature divides the scores
    ch, q = O.sampled_walk(T, 2.0, np.array([0.49, 0.999]))
    assert list(ch) == [0, 1]
    assert abs(q[1] - softmax(np.array([1.0, 2.0]) / 2.0)[1]) < 1e-15


def test_sampled_walk_frequencies_and_cold_limit():
    rng = np.random.default_rng(5)
    row = np.array([0.3, -1.0, 1.2, 0.0])
    T = np.tile(row, (1, 4, 1))
    p = np.exp(row - row.max())
    p /= p.sum()
    n = 20000
    counts = np.zeros(4)
    for u in rng.random(n):
        counts[O.sampled_walk(T, 1.0, np.array([u]))[0][0]] += 1
    assert np.all(np.abs(counts / n - p) <= 4 * np.sqrt(p * (1 - p) / n))
    # a cold temperature follows the greedy chain
    g, wts, head, ctxs, anchors, W = propose_setup()
    Tm = O.propose(g, wts, head, ctxs, anchors, W, K=4)["table"][0]
    cold, _ = O.sampled_walk(Tm, 1e-6, rng.random(W - 1) * 0.98 + 0.01)
    assert list(cold) == list(O.greedy_walk(Tm))


def test_proposals_are_per_request():
    g, wts, head, ctxs, anchors, W = propose_setup(B=2)
    both = O.propose(g, wts, head, ctxs, anchors, W, K=4)
    for b in range(2):
        one = O.propose(g, wts, head, [ctxs[b]], [anchors[b]], W, K=4)
        assert np.array_equal(one["cand"][0], both["cand"][b])
        assert rel_err(one["table"][0], both["table"][b]) < 1e-12
        assert np.array_equal(one["tokens"][0], both["tokens"][b])


# ---------------------------------------------------------------------------
# DFlash2 dynamic grouped convolution [NIF, DFlash2 layer equations]
# ---------------------------------------------------------------------------
G_CONV = synth.Geometry(hidden=96, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=160,
                        n_feat_layers=2, code_dim=0, msg_dim=0, vocab=64, windows=(12, 0),
                        dtype="f32", conv_group=16)


def test_conv_hand_worked():
    """H = 32 (two groups of 16), W = 2; rows of ones and twos.  delta rows
    are ordered (side, tap, group): row 0 = (0,0,0) reads 0.5 x channel 0,
    row 3 = (0,1,1) reads 0.1 x channel 16.  Base: side 0 taps (1, 0.25),
    side 1 taps (2, 0).  Worked by hand:
      side 0, row 0: group 0 (1 + 0.5*1) * 1 = 1.5; group 1: 1 * 1 = 1
      side 0, row 1: group 0 (1 + 0.5*2) * 2 + 0.25 * 1 = 4.25;
                     group 1 1 * 2 + (0.25 + 0.1*2) * 1 = 2.45
      side 1: 2 x the input everywhere."""
    g = synth.Geometry(hidden=32, n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=64, ffn=64,
                       n_feat_layers=1, code_dim=0, msg_dim=0, vocab=16, windows=(0,), dtype="f32",
                       conv_group=16)
    Wd = np.zeros((8, 32), np.float32)
    Wd[0, 0] = 0.5
    Wd[3, 16] = 0.1
    base = np.zeros((4, 32), np.float32)
    base[0], base[1], base[2], base[3] = 1.0, 0.25, 2.0, 0.0
    wts = {"l0.attn_conv_w": Wd, "l0.attn_conv_base": base}
    X = np.stack([np.ones(32), 2 * np.ones(32)])
    d = O.conv_delta(g, wts, 0, "attn", X)
    out0 = O.conv_apply(g, wts, 0, "attn", 0, X, d)
    assert np.allclose(out0[0, :16], 1.5) and np.allclose(out0[0, 16:], 1.0)
    assert np.allclose(out0[1, :16], 4.25) and np.allclose(out0[1, 16:], 2.45)
    out1 = O.conv_apply(g, wts, 0, "attn", 1, X, d)
    assert np.allclose(out1, 2 * X)


def test_conv_rows_look_back_one():
    g = G_CONV
    wts = small_model(g)
    X = np.random.default_rng(8).standard_normal((6, g.hidden))
    d = O.conv_delta(g, wts, 0, "mlp", X)
    a = O.conv_apply(g, wts, 0, "mlp", 0, X, d)
    X2 = X.copy()
    X2[2] += 1.0
    b = O.conv_apply(g, wts, 0, "mlp", 0, X2, O.conv_delta(g, wts, 0, "mlp", X2))
    changed = np.any(a != b, axis=1)
    assert list(changed) == [False, False, True, True, False, False]


def test_conv_identity_reduces_to_dflash():
    """Zero delta projections, current-row taps 1 and previous-row taps 0 on
    both sides: the DFlash2 forward is the DFlash forward."""
    g = G_CONV
    plain = dataclasses_replace(g, conv_group=0)
    wts = small_model(g)
    ov = dict(wts)
    for l in range(g.n_layers):
        for br in ("attn", "mlp"):
            ov[f"l{l}.{br}_conv_w"] = np.zeros_like(wts[f"l{l}.{br}_conv_w"])
            ov[f"l{l}.{br}_conv_base"] = np.array([[1.0], [0.0], [1.0], [0.0]], np.float32) * \
                np.ones((1, g.hidden), np.float32)
    ctx = build_context(g, ov, 20)
    a = O.draft_forward(g, ov, [ctx], [3], 7)
    b = O.draft_forward(plain, ov, [ctx], [3], 7)
    assert np.array_equal(a, b)
    assert rel_err(O.draft_forward(g, wts, [ctx], [3], 7), b) > 1e-3   # the live conv changes it


@pytest.mark.parametrize("branch", ["attn", "mlp"])
def test_conv_finish_is_linear_in_the_branch_output(branch):
    """The finish side applies the delta of the branch's normalised input to
    the branch output, so scaling the branch output map by 2 scales the
    branch's contribution x_next - x by exactly 2 (the other branch off)."""
    g = G_CONV
    wts = small_model(g)
    ctx = build_context(g, wts, 15)
    x = np.random.default_rng(9).standard_normal((7, g.hidden))
    off, scale = ("l0.w_down", "l0.wo") if branch == "attn" else ("l0.wo", "l0.w_down")
    w1 = dict(wts)
    w1[off] = np.zeros_like(wts[off])
    w2 = dict(w1)
    w2[scale] = (2 * wts[scale]).astype(wts[scale].dtype)
    d1 = O.decoder_layer(g, w1, 0, [ctx], x, 7) - x
    d2 = O.decoder_layer(g, w2, 0, [ctx], x, 7) - x
    assert np.max(np.abs(d2 - 2 * d1)) < 1e-12 * np.max(np.abs(d1))
    assert np.max(np.abs(d1)) > 1e-3


def test_conv_has_no_history_across_requests():
    g = G_CONV
    wts = small_model(g)
    ctxs = [build_context(g, wts, 15, request=b) for b in range(2)]
    both = O.draft_forward(g, wts, ctxs, [3, 9], 6)
    for b in range(2):
        one = O.draft_forward(g, wts, [ctxs[b]], [[3, 9][b]], 6)
        assert rel_err(one[0], both[b]) < 1e-12


def dataclasses_replace(g, **kw):
    return synth.with_geometry(g, **kw)


def test_conv_prepare_and_finish_sides():
    """Prepare side = identity, finish side = 2 x identity (zero deltas): the
    DFlash2 forward equals the plain forward with W_o and W_down doubled."""
    g = G_CONV
    plain = dataclasses_replace(g, conv_group=0)
    wts = small_model(g)
    ov = dict(wts)
    doubled = dict(wts)
    for l in range(g.n_layers):
        for br in ("attn", "mlp"):
            ov[f"l{l}.{br}_conv_w"] = np.zeros_like(wts[f"l{l}.{br}_conv_w"])
            ov[f"l{l}.{br}_conv_base"] = np.array([[1.0], [0.0], [2.0], [0.0]], np.float32) * \
                np.ones((1, g.hidden), np.float32)
        for n in ("wo", "w_down"):
            doubled[f"l{l}.{n}"] = 2 * wts[f"l{l}.{n}"]
    ctx = build_context(g, ov, 20)
    a = O.draft_forward(g, ov, [ctx], [3], 7)
    b = O.draft_forward(plain, doubled, [ctx], [3], 7)
    assert rel_err(a, b) < 1e-12


@pytest.mark.parametrize("branch", ["attn", "mlp"])
def test_conv_branch_ignores_the_residual_scale(branch):
    """Each branch's delta comes from its normalised input, so a branch's
    contribution x_next - x (the other branch off) does not change when the
    residual is scaled (up to the norm's epsilon)."""
    g = G_CONV
    wts = small_model(g)
    ctx = build_context(g, wts, 15)
    off = "l0.w_down" if branch == "attn" else "l0.wo"
    w1 = dict(wts)
    w1[off] = np.zeros_like(wts[off])
    x = np.random.default_rng(10).standard_normal((7, g.hidden))
    d1 = O.decoder_layer(g, w1, 0, [ctx], x, 7) - x
    d2 = O.decoder_layer(g, w1, 0, [ctx], 3.0 * x, 7) - 3.0 * x
    assert rel_err(d2, d1) < 1e-5
