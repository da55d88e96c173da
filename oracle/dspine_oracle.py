"""CPU oracle for the DSpine draft-block hot path.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this module.  The product path (the HIP library and its
binding) never calls it, and it imports nothing from the product package.

Everything is float64 numpy, written step by step from the sources below,
with no fusion, blocking or reordering beyond what the definitions state.
The only roundings are the ones the sources fix for stored context K/V.

Sources (cited by tag):
  [FLZ] "DSpine for Qwen3.8-27B: Causal Features Through Depth" (flozi.net guide)
  [PHY] "DSpine 完全拆解：相邻因果注入如何让并行草稿沿网络深度建立 token 依赖"
        (pinghaoyang.com.cn article)
  [DSP] "DSpark, every bolt and rivet" (lab-artifacts tutorial)
  [NIF] NInfer maintainer notes, "DFlash" (docs/maintainer/dflash.md)

Tensor conventions: uint16 arrays hold bfloat16 bit patterns; matrices are
``[out, in]`` (y = W x).  A model is the dict made by ``synth.make_weights``
plus its ``synth.Geometry``.

Pins (tests/test_oracle_pins.py): every function below is tied to something
other than this code: closed forms (RMSNorm, window counts), hand-worked
examples (context, bridge, decoder layer, the DFlash2 convolution, the
walks, the FP8 rounding and a retrieval that misses the BF16 best), brute
force (attention, top-K), a library routine (torch's float8_e4m3fn cast for
the FP8 rounding), special cases that reduce to a simpler computation
(bridge or convolution switched off gives plain DFlash; the
anchor-conditioned or predicted-code refinement gives the forward's own
scores; an FP8-representable head scores exactly; retrieving the whole
vocabulary is the direct path), invariants (RoPE shift, request
independence, one-row look-back) and the figures the pages print.  Parity unpinned: the absolute output values
at the 27B and 35B geometries, for which the pages print no worked example;
there the GPU is compared with this oracle on identical inputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) or floats -> float64 (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even (done in exact integer
    arithmetic on the float64 bit pattern).  Returns float64 values."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    # bf16 keeps 7 fraction bits; float64 has 52: drop 45 bits with RNE.
    drop = np.uint64(45)
    half = np.uint64(1) << (drop - np.uint64(1))
    lsb = (bits >> drop) & np.uint64(1)
    rounded = (bits + half - np.uint64(1) + lsb) >> drop << drop
    out = rounded.view(np.float64).copy()
    # exponent range: bf16 shares float32's range; values beyond it overflow.
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.sign(out[big]) * np.inf
    small = np.abs(x) < 2.0 ** -126   # bf16 subnormals: a fixed step of 2^-133
    if np.any(small):
        step = 2.0 ** -133
        out[small] = np.round(x[small] / step) * step   # numpy rounds halves to even
    return out


def round_fp16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest IEEE half value (ties to even); float64 out."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# elementary operations
# ---------------------------------------------------------------------------
def plain_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """[NIF, context conditioning]: w * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return widen(w) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def head_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float, head_dim: int) -> np.ndarray:
    """[NIF, layer equations]: plain RMSNorm over each head of width D, one
    weight vector [D] shared by all heads of the projection."""
    shp = x.shape
    xh = x.reshape(shp[:-1] + (shp[-1] // head_dim, head_dim))
    return plain_rmsnorm(xh, w, eps).reshape(shp)


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """inverse frequency of rotation pair j: theta^(-2j/D), j < D/2."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / head_dim)


def rope_1d(x: np.ndarray, positions: np.ndarray, theta: float, head_dim: int) -> np.ndarray:
    """[NIF, context K/V and layer equations]: one-dimensional RoPE over the
    full head in split-half form: pair (j, j + D/2) is rotated by the angle
    position * theta^(-2j/D).

    x: [T, n_heads*D]; positions: [T] absolute integer positions."""
    T = x.shape[0]
    half = head_dim // 2
    xh = x.reshape(T, -1, head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(head_dim, theta)[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = xh[..., :half]
    x2 = xh[..., half:]
    out = np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)
    return out.reshape(x.shape)


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = W x for rows of x; W is [out, in]."""
    return np.asarray(x, dtype=np.float64) @ widen(w).T


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax; entries equal to -inf get zero weight."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# context: a1-a3
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class LayerContext:
    """Context K/V of one draft layer for one request, by absolute position.

    ``k[p - lo]`` / ``v[p - lo]`` hold position p for p in [lo, frontier):
    exactly the live interval [NIF, ring storage]."""
    lo: int
    k: np.ndarray          # [n, nkv*D] float64 (already rounded to storage type)
    v: np.ndarray


@dataclasses.dataclass
class RequestContext:
    frontier: int
    layers: List[LayerContext]


def empty_context(g, frontier: int = 0) -> RequestContext:
    """A context whose frontier is ``frontier`` with nothing stored (positions
    below the frontier that are never materialized are simply absent)."""
    return RequestContext(frontier, [LayerContext(frontier, np.zeros((0, g.kv_dim)),
                                                  np.zeros((0, g.kv_dim)))
                                     for _ in range(g.n_layers)])


def live_lo(window: int, frontier: int) -> int:
    """[NIF, ring storage]: live interval is [max(0, F - S), F) for a local
    layer of window S; a full layer (S = 0) keeps every position."""
    if window == 0:
        return 0
    return max(0, frontier - window)


def context_features(g, wts: Dict[str, np.ndarray], feats: np.ndarray) -> np.ndarray:
    """a1 [NIF, context conditioning]; [DSP §5.1]: s_t is the concatenation
    of the recorded target residuals; c_t = plain_rmsnorm(W_feature s_t,
    context_norm), no bias."""
    u = linear(widen(feats), wts["w_feat"])
    return plain_rmsnorm(u, wts["g_ctx"], g.eps)


def context_kv(g, wts, layer: int, c: np.ndarray, positions: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """a2 [NIF, context K/V]: k = rope_1d(head_rmsnorm(W_k c, key_norm), t),
    v = W_v c, using the layer's own K/V weights.  Storage [NIF, fused
    context materializer]: K is stored as BF16 (no rounding before the head
    norm) and V as FP16_RNE(BF16(v)).  A float32 model stores both unrounded
    beyond float32 (reading: the BF16/FP16 contract belongs to the BF16
    drafter)."""
    p = f"l{layer}."
    k = rope_1d(head_rmsnorm(linear(c, wts[p + "wk"]), wts[p + "gk"], g.eps, g.head_dim),
                positions, g.rope_theta, g.head_dim)
    v = linear(c, wts[p + "wv"])
    if g.dtype == "bf16":
        k = round_bf16(k)
        v = round_fp16(round_bf16(v))
    else:
        k = k.astype(np.float32).astype(np.float64)
        v = v.astype(np.float32).astype(np.float64)
    return k, v


def materialize(g, wts, ctx: RequestContext, feats: np.ndarray) -> RequestContext:
    """a1-a3 for one request and one chunk of n new positions [F, F+n).

    [NIF, context prefill]: only the feature and K/V projections run.  A
    chunk longer than a local ring stores only its final live window while
    the frontier still advances by the whole chunk.  Returns a new context."""
    n = feats.shape[0]
    F0 = ctx.frontier
    F1 = F0 + n
    new_layers = []
    # positions that some layer keeps
    need_lo = F1
    for l in range(g.n_layers):
        need_lo = min(need_lo, max(F0, live_lo(g.windows[l], F1)))
    c = None
    if need_lo < F1:
        c_rows = context_features(g, wts, feats[need_lo - F0:])
    for l in range(g.n_layers):
        lo_new = live_lo(g.windows[l], F1)
        old = ctx.layers[l]
        keep_from = max(F0, lo_new)
        if keep_from < F1:
            pos = np.arange(keep_from, F1)
            k_new, v_new = context_kv(g, wts, l, c_rows[keep_from - need_lo:], pos)
        else:
            k_new = np.zeros((0, g.kv_dim))
            v_new = np.zeros((0, g.kv_dim))
        # surviving old positions: [max(old.lo, lo_new), F0)
        s = max(old.lo, lo_new)
        k_old = old.k[max(0, s - old.lo):]
        v_old = old.v[max(0, s - old.lo):]
        lo = s if k_old.shape[0] > 0 else keep_from
        new_layers.append(LayerContext(lo, np.concatenate([k_old, k_new]),
                                       np.concatenate([v_old, v_new])))
    return RequestContext(F1, new_layers)


def ring_image(g, ctx: RequestContext, layer: int, capacity: int) -> Tuple[np.ndarray, np.ndarray]:
    """Ring storage view [NIF, ring storage]: position p sits in slot p mod S
    of a local layer (slot p of a full layer).  Layout [nkv, capacity, D];
    slots holding no live position are NaN."""
    lc = ctx.layers[layer]
    S = g.windows[layer]
    K = np.full((g.n_kv_heads, capacity, g.head_dim), np.nan)
    V = np.full((g.n_kv_heads, capacity, g.head_dim), np.nan)
    for i in range(lc.k.shape[0]):
        p = lc.lo + i
        slot = p % S if S > 0 else p
        K[:, slot, :] = lc.k[i].reshape(g.n_kv_heads, g.head_dim)
        V[:, slot, :] = lc.v[i].reshape(g.n_kv_heads, g.head_dim)
    return K, V


# ---------------------------------------------------------------------------
# a3: visibility
# ---------------------------------------------------------------------------
def key_visible(window: int, block_causal: bool, p_query: int, p_key: int,
                key_is_block: bool, q_index: int = 0, k_index: int = 0) -> bool:
    """[NIF, draft attention]: a local layer allows |p_key - p_query| < S
    (distance S-1 in, S out); a full layer allows every populated key.
    [PHY, 块因果注意力] / [FLZ]: the block-causal variant additionally hides
    block keys after the query row."""
    if window > 0 and abs(p_key - p_query) >= window:
        return False
    if key_is_block and block_causal and k_index > q_index:
        return False
    return True


def visible_context_interval(window: int, frontier: int, row: int) -> Tuple[int, int]:
    """Closed form of the context positions row i (at F+i) sees: the
    predicate clipped to the populated positions [0, F)."""
    if window == 0:
        return 0, frontier
    lo = max(0, frontier + row - window + 1)
    return min(lo, frontier), frontier


# ---------------------------------------------------------------------------
# a6: attention
# ---------------------------------------------------------------------------
def block_attention(g, layer: int, ctx: RequestContext, q: np.ndarray, k: np.ndarray,
                    v: np.ndarray) -> np.ndarray:
    """[NIF, layer equations]: attention(q, concat(K_ctx, k), concat(V_ctx, v),
    scale 1/sqrt(D), layer mask), vectorised.  q: [W, nq*D]; k, v: [W, nkv*D]
    for block positions F..F+W-1.  Q head h reads KV head h // (nq/nkv)
    (reading: contiguous grouping)."""
    W = q.shape[0]
    F = ctx.frontier
    S = g.windows[layer]
    lc = ctx.layers[layer]
    D = g.head_dim
    grp = g.n_q_heads // g.n_kv_heads
    ctx_pos = np.arange(lc.lo, lc.lo + lc.k.shape[0])
    blk_pos = F + np.arange(W)
    key_pos = np.concatenate([ctx_pos, blk_pos])
    K = np.concatenate([lc.k, k]).reshape(-1, g.n_kv_heads, D)
    V = np.concatenate([lc.v, v]).reshape(-1, g.n_kv_heads, D)
    n_ctx = ctx_pos.shape[0]
    # mask [W, n_keys]
    qpos = blk_pos[:, None]
    allowed = np.ones((W, key_pos.shape[0]), dtype=bool)
    if S > 0:
        allowed &= np.abs(key_pos[None, :] - qpos) < S
    if g.block_causal:
        jj = np.arange(W)[None, :]
        ii = np.arange(W)[:, None]
        allowed[:, n_ctx:] &= jj <= ii
    out = np.zeros((W, g.n_q_heads, D))
    qh = q.reshape(W, g.n_q_heads, D)
    for h in range(g.n_q_heads):
        kvh = h // grp
        s = qh[:, h, :] @ K[:, kvh, :].T / math.sqrt(D)
        s = np.where(allowed, s, -np.inf)
        out[:, h, :] = softmax_rows(s) @ V[:, kvh, :]
    return out.reshape(W, -1)


def block_attention_bruteforce(g, layer: int, ctx: RequestContext, q: np.ndarray,
                               k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Second attention for tiny inputs: explicit loops over (head, query,
    key), the predicate evaluated per pair through ``key_visible``, keys read
    from their logical positions, softmax accumulated in float64."""
    W = q.shape[0]
    F = ctx.frontier
    S = g.windows[layer]
    lc = ctx.layers[layer]
    D = g.head_dim
    grp = g.n_q_heads // g.n_kv_heads
    out = np.zeros((W, g.n_q_heads * D))
    for h in range(g.n_q_heads):
        kvh = h // grp
        for i in range(W):
            qi = q[i, h * D:(h + 1) * D]
            keys = []
            for p in range(0, F):
                if p < lc.lo or p >= lc.lo + lc.k.shape[0]:
                    continue
                if key_visible(S, g.block_causal, F + i, p, False):
                    r = p - lc.lo
                    keys.append((lc.k[r, kvh * D:(kvh + 1) * D], lc.v[r, kvh * D:(kvh + 1) * D]))
            for j in range(W):
                if key_visible(S, g.block_causal, F + i, F + j, True, i, j):
                    keys.append((k[j, kvh * D:(kvh + 1) * D], v[j, kvh * D:(kvh + 1) * D]))
            scores = [float(np.dot(qi, kk)) / math.sqrt(D) for kk, _ in keys]
            mx = max(scores)
            wsum = 0.0
            acc = np.zeros(D)
            for sc, (_, vv) in zip(scores, keys):
                e = math.exp(sc - mx)
                wsum += e
                acc += e * vv
            out[i, h * D:(h + 1) * D] = acc / wsum
    return out


# ---------------------------------------------------------------------------
# a9-a11: the bridge
# ---------------------------------------------------------------------------
def bridge_codes(g, wts, layer: int, x: np.ndarray, anchor_id: int) -> Tuple[np.ndarray, np.ndarray]:
    """a9 [FLZ, "The bridge", equations for r, z, c]; [PHY, 统一转移空间]:
    rho_t = sqrt(mean_i x_{t,i}^2) (no floor), z_t = R_l x_t / (rho_t + eps),
    c_t = sqrt(r) z_t / (||z_t||_2 + eps).  The anchor row takes sqrt(r) times
    its token's codebook row instead.  Returns (rho [W], c [W, r])."""
    r = g.code_dim
    rho = np.sqrt(np.mean(x * x, axis=-1))
    z = linear(x / (rho[:, None] + g.eps), wts[f"l{layer}.R"])
    c = math.sqrt(r) * z / (np.linalg.norm(z, axis=-1, keepdims=True) + g.eps)
    c[0] = math.sqrt(r) * widen(wts["codebook"][anchor_id])
    return rho, c


def bridge_write(g, wts, layer: int, x: np.ndarray, rho: np.ndarray, c: np.ndarray,
                 pred_codes: Optional[np.ndarray] = None) -> np.ndarray:
    """a10-a11 [FLZ, "The bridge", equations for m and x']; [PHY, 门控与写回]:
    g_t = sigmoid(G c_t + G_p c_{t-1} + b), m_t = g_t * (A c_{t-1}),
    x'_t = x_t + rho_t W_l m_t for t >= 1.  The anchor row (t = 0) gets no
    message [FLZ]; [PHY]: the anchor only sends.  All codes come from the
    pre-write states, so every row is written from the same inputs.

    ``pred_codes`` [W, r], when given, replaces c_{t-1} for receiver t (row 0
    unused): the hook used to redo the last write with a known predecessor."""
    W = x.shape[0]
    out = x.copy()
    for t in range(1, W):
        cp = c[t - 1] if pred_codes is None else pred_codes[t]
        out[t] = bridge_write_row(g, wts, layer, x[t], rho[t], c[t], cp)
    return out


def bridge_write_row(g, wts, layer: int, x_t: np.ndarray, rho_t: float, c_t: np.ndarray,
                     cp: np.ndarray) -> np.ndarray:
    """One receiver row of the write: gate from the receiver's own code c_t
    and the predecessor code cp, message A cp, written back scaled by the
    receiver's RMS rho_t [FLZ, "The bridge", equations for m and x']."""
    gate = sigmoid(linear(c_t[None], wts["bridge_G"])[0]
                   + linear(cp[None], wts["bridge_Gp"])[0] + widen(wts["bridge_b"]))
    m = gate * linear(cp[None], wts["bridge_A"])[0]
    return x_t + rho_t * linear(m[None], wts[f"l{layer}.W_l"])[0]


def bridge(g, wts, layer: int, x: np.ndarray, anchor_id: int,
           pred_codes: Optional[np.ndarray] = None) -> np.ndarray:
    """One bridge on one request block x [W, H] (read, then write)."""
    rho, c = bridge_codes(g, wts, layer, x, anchor_id)
    return bridge_write(g, wts, layer, x, rho, c, pred_codes)


# ---------------------------------------------------------------------------
# a4-a12: the draft forward
# ---------------------------------------------------------------------------
def block_input(g, wts, anchor_id: int, W: int) -> np.ndarray:
    """a4 [NIF, draft input]: target embeddings of the anchor followed by W-1
    MASK tokens at positions F..F+W-1."""
    emb = wts["embed"]
    rows = [anchor_id] + [g.mask_token_id] * (W - 1)
    return widen(emb[rows])


# ---------------------------------------------------------------------------
# DFlash2 dynamic grouped convolution [NIF, DFlash2 layer equations]
# ---------------------------------------------------------------------------
def conv_delta(g, wts, layer: int, branch: str, X: np.ndarray) -> np.ndarray:
    """delta = W_delta X reshaped to [W, 2 sides, 2 taps, H/16 groups] for one
    request block X [W, H] (the branch's normalised input)."""
    d = linear(X, wts[f"l{layer}.{branch}_conv_w"])
    return d.reshape(X.shape[0], 2, 2, g.conv_groups)


def conv_apply(g, wts, layer: int, branch: str, side: int, X: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """Conv_side(X)[i, g, j] = (base[side,0,g,j] + delta[i,side,0,g]) X[i,g,j]
    + [i >= 1] (base[side,1,g,j] + delta[i,side,1,g]) X[i-1,g,j]: per-channel
    base coefficients, increments shared by the channels of a group, no tap
    before row 0 and no history across requests [NIF, DFlash2 layer
    equations].  X [W, H] is one request's block."""
    W, G, gw = X.shape[0], g.conv_groups, g.conv_group
    base = widen(wts[f"l{layer}.{branch}_conv_base"]).reshape(2, 2, G, gw)
    Xg = X.reshape(W, G, gw)
    out = (base[side, 0][None] + delta[:, side, 0, :, None]) * Xg
    out[1:] += (base[side, 1][None] + delta[1:, side, 1, :, None]) * Xg[:-1]
    return out.reshape(W, g.hidden)


def conv_blocks(g, wts, layer: int, branch: str, side: int, X: np.ndarray, deltas, W: int) -> np.ndarray:
    """conv_apply on each request's rows of stacked X [B*W, H]."""
    return np.concatenate([conv_apply(g, wts, layer, branch, side, X[b * W:(b + 1) * W], deltas[b])
                           for b in range(len(deltas))])


def decoder_layer(g, wts, layer: int, ctxs: Sequence[RequestContext], x: np.ndarray, W: int,
                  attn_fn=block_attention) -> np.ndarray:
    """a5-a8 [NIF, layer equations]: n = plain_rmsnorm(x, input_norm); q and k
    are head-RMSNormed and rotated; attention over context plus block; y = x +
    W_o a; m = plain_rmsnorm(y, post_attention_norm); x_next = y +
    W_down(SiLU(W_gate m) * W_up m).  With conv_group > 0 (DFlash2) each
    branch's normalised input goes through the prepare side of its
    convolution and the branch output through the finish side, with the
    delta projected from that normalised input.  x is [B*W, H]: rows of all requests are
    stacked for the row-wise linear maps; attention runs per request."""
    p = f"l{layer}."
    B = len(ctxs)
    n = plain_rmsnorm(x, wts[p + "g_in"], g.eps)
    if g.conv:      # DFlash2: prepare the attention branch's input
        d_a = [conv_delta(g, wts, layer, "attn", n[b * W:(b + 1) * W]) for b in range(B)]
        n = conv_blocks(g, wts, layer, "attn", 0, n, d_a, W)
    pos = np.concatenate([np.arange(c.frontier, c.frontier + W) for c in ctxs])
    q = rope_1d(head_rmsnorm(linear(n, wts[p + "wq"]), wts[p + "gq"], g.eps, g.head_dim),
                pos, g.rope_theta, g.head_dim)
    k = rope_1d(head_rmsnorm(linear(n, wts[p + "wk"]), wts[p + "gk"], g.eps, g.head_dim),
                pos, g.rope_theta, g.head_dim)
    v = linear(n, wts[p + "wv"])
    a = np.zeros((B * W, g.q_dim))
    for b in range(B):
        sl = slice(b * W, (b + 1) * W)
        a[sl] = attn_fn(g, layer, ctxs[b], q[sl], k[sl], v[sl])
    o = linear(a, wts[p + "wo"])
    if g.conv:      # finish: the output side, with the prepare's delta
        o = conv_blocks(g, wts, layer, "attn", 1, o, d_a, W)
    y = x + o
    m = plain_rmsnorm(y, wts[p + "g_post"], g.eps)
    if g.conv:
        d_m = [conv_delta(g, wts, layer, "mlp", m[b * W:(b + 1) * W]) for b in range(B)]
        m = conv_blocks(g, wts, layer, "mlp", 0, m, d_m, W)
    z = linear(silu(linear(m, wts[p + "w_gate"])) * linear(m, wts[p + "w_up"]), wts[p + "w_down"])
    if g.conv:
        z = conv_blocks(g, wts, layer, "mlp", 1, z, d_m, W)
    return y + z


def draft_forward(g, wts, ctxs: Sequence[RequestContext], anchor_ids: Sequence[int], W: int,
                  attn_fn=block_attention, return_layers: bool = False,
                  return_last_prewrite: bool = False):
    """a4-a12: one masked-block forward over B requests.

    After every decoder layer (the last one included) the bridge writes
    predecessor messages [FLZ, "The bridge"]; [PHY, 融合 kernel]; then the
    next stage normalises: the next layer's input norm, or the final plain
    RMSNorm [NIF, after the layers].  With code_dim == 0 there is no bridge
    and this is the plain DFlash forward.  Returns [B, W, H]; with
    ``return_last_prewrite`` also the last layer's states before its bridge
    write, u_L [B, W, H] (what the last-write refinement starts from)."""
    B = len(ctxs)
    x = np.concatenate([block_input(g, wts, int(anchor_ids[b]), W) for b in range(B)])
    states = []
    prewrite = None
    for l in range(g.n_layers):
        x = decoder_layer(g, wts, l, ctxs, x, W, attn_fn)
        if l == g.n_layers - 1:
            prewrite = x.copy().reshape(B, W, g.hidden)
        if g.bridge:
            for b in range(B):
                sl = slice(b * W, (b + 1) * W)
                x[sl] = bridge(g, wts, l, x[sl], int(anchor_ids[b]))
        states.append(x.copy())
    out = plain_rmsnorm(x, wts["g_final"], g.eps).reshape(B, W, g.hidden)
    if return_layers:
        return out, states
    if return_last_prewrite:
        return out, prewrite
    return out


# ---------------------------------------------------------------------------
# proposal tail: candidate retrieval, last-write refinement, transition
# table, conditional walk
# ---------------------------------------------------------------------------
HEAD_SLICE = 8192     # vocabulary rows widened at a time (bounds memory only)


def head_scores(lm_head: np.ndarray, h: np.ndarray, ids: Optional[np.ndarray] = None) -> np.ndarray:
    """Scores of the shared LM head, E_v . h, for every vocabulary row (or
    only the rows ``ids``) [PHY, 前驱条件解码与 transition cache: the head's
    score for token v is the dot product of its output-embedding row with the
    final-normed state].  h is [n, H]; returns [n, V] (or [n, len(ids)]).
    Each score is one independent dot product, so slicing the rows of the
    head changes nothing but memory use."""
    h = np.atleast_2d(h)
    if ids is not None:
        return h @ widen(lm_head[np.asarray(ids)]).T
    V = lm_head.shape[0]
    out = np.empty((h.shape[0], V))
    for v0 in range(0, V, HEAD_SLICE):
        v1 = min(V, v0 + HEAD_SLICE)
        out[:, v0:v1] = h @ widen(lm_head[v0:v1]).T
    return out


def top_k(scores: np.ndarray, K: int) -> np.ndarray:
    """The K best tokens of one score row, best first [FLZ, "The last write is
    refined using discrete candidates": the direct path multiplies by the
    head and retains the top 16].  Equal scores rank the smaller token id
    first (a reading: the pages fix no tie order)."""
    order = np.lexsort((np.arange(scores.shape[0]), -scores))
    return order[:K].astype(np.int64)


# ---------------------------------------------------------------------------
# FP8 row-scaled candidate retrieval [FLZ, "The last write is refined using
# discrete candidates": the optimized path scores the whole vocabulary
# approximately with a row-scaled FP8 head, keeps 128 candidates, rescores
# them with the original BF16 head and keeps the best 16]
# ---------------------------------------------------------------------------
FP8_E4M3_MAX = 448.0      # largest finite OCP E4M3 value, 1.75 x 2^8
RETRIEVE = 128            # candidates the FP8 scores keep per row


def round_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest OCP FP8 E4M3 value, ties to even, as float64.  E4M3 keeps 3
    fraction bits with exponent bias 7: normal binades 2^-6 .. 2^8 (step
    2^(e-3) in binade 2^e) and subnormals in steps of 2^-9 below 2^-6.
    Inputs must be finite with |x| <= 448 (the row scale below keeps the
    head's values there), so nothing saturates."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    mant, ex = np.frexp(a)                  # a = mant * 2^ex, mant in [0.5, 1)
    e = np.maximum(ex - 1, -6)              # binade exponent, floored at the subnormal range
    step = np.ldexp(1.0, e - 3)
    return np.copysign(np.round(a / step) * step, x)   # numpy rounds halves to even


def quantize_head_fp8(lm_head: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The row-scaled FP8 copy of the head.  Reading (the pages fix only
    "row-scaled FP8"): row v's scale s_v is the smallest power of two with
    max_k |E_v[k]| / s_v <= 448 (1 for an all-zero row), and its codes are
    E_v / s_v rounded to E4M3, ties to even.  Dividing by a power of two is
    exact, so each code is one rounding of the BF16 value.  Returns the codes
    [V, H] (float32, which holds every E4M3 value exactly) and the scales [V]
    (float64).  Rows are processed in slices (bounds memory only)."""
    V = lm_head.shape[0]
    codes = np.empty(lm_head.shape, dtype=np.float32)
    s = np.ones(V)
    for v0 in range(0, V, HEAD_SLICE):
        v1 = min(V, v0 + HEAD_SLICE)
        E = widen(lm_head[v0:v1])
        m = np.max(np.abs(E), axis=1)
        nz = m > 0
        mant, ex = np.frexp(m[nz] / FP8_E4M3_MAX)    # m / 448 = mant * 2^ex
        sv = np.ones_like(m)
        sv[nz] = np.where(mant == 0.5, np.ldexp(1.0, ex - 1), np.ldexp(1.0, ex))
        s[v0:v1] = sv
        codes[v0:v1] = round_fp8_e4m3(E / sv[:, None])
    return codes, s


def head_scores_fp8(codes: np.ndarray, scales: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Approximate head scores s_v * (q_v . h) of every vocabulary row for the
    rows of h [n, H]; returns [n, V]."""
    h = np.atleast_2d(h)
    V = codes.shape[0]
    out = np.empty((h.shape[0], V))
    for v0 in range(0, V, HEAD_SLICE):
        v1 = min(V, v0 + HEAD_SLICE)
        out[:, v0:v1] = (h @ codes[v0:v1].astype(np.float64).T) * scales[None, v0:v1]
    return out


def retrieve_and_rescore(approx: np.ndarray, lm_head: np.ndarray, h: np.ndarray, R: int,
                         K: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """One proposal row: the R best approximate scores (ties: smaller token
    first), their exact BF16 head scores E_v . h, and the K best of those
    (same order rule).  Returns (retrieved ids [R], their exact scores [R],
    the K kept ids, their exact scores)."""
    ids = top_k(approx, R)
    exact = head_scores(lm_head, h, ids)[0]
    keep = np.lexsort((ids, -exact))[:K]
    return ids, exact, ids[keep], exact[keep]


def transition_table(g, wts, lm_head: np.ndarray, u: np.ndarray, anchor_id: int,
                     cand: np.ndarray) -> np.ndarray:
    """T_t[i, j] for one request [PHY, 前驱条件解码与 transition cache, the
    equation for T_t and the last-write refinement steps]; [FLZ, "The last
    write is refined using discrete candidates"].

    u [W, H] is the last layer's pre-write state; cand [W-1, K] holds the
    candidates of rows 1..W-1.  For receiver row t the last layer's bridge
    write is redone from u with the predecessor code replaced by the known
    token's code sqrt(r) C[s]: s is the i-th candidate of row t-1, or the
    anchor for row 1 (the first proposal is conditioned on the real anchor,
    so all K rows of T_1 use it).  The refined state is final-normed and
    scored by the head on row t's own candidates only.  Returns
    [W-1, K, K], entry [t-1, i, j]."""
    L = g.n_layers - 1
    W, K = u.shape[0], cand.shape[1]
    rho, c = bridge_codes(g, wts, L, u, anchor_id)
    sr = math.sqrt(g.code_dim)
    T = np.zeros((W - 1, K, K))
    for t in range(1, W):
        preds = [anchor_id] * K if t == 1 else [int(v) for v in cand[t - 2]]
        for i, s in enumerate(preds):
            x = bridge_write_row(g, wts, L, u[t], rho[t], c[t], sr * widen(wts["codebook"][s]))
            h = plain_rmsnorm(x, wts["g_final"], g.eps)
            T[t - 1, i] = head_scores(lm_head, h, cand[t - 1])[0]
    return T


def greedy_walk(T: np.ndarray) -> np.ndarray:
    """Left-to-right choice [PHY, transition cache, selection stage]: row 1's
    choice maximises T_1 on the anchor's row, each later row maximises the
    row of T_t picked by the previous choice.  Equal scores pick the smaller
    candidate index (the better initial rank).  Returns candidate indices
    [W-1]."""
    n = T.shape[0]
    choice = np.zeros(n, dtype=np.int64)
    i = 0
    for t in range(n):
        choice[t] = int(np.argmax(T[t, i]))     # first maximum
        i = int(choice[t])
    return choice


def sampled_walk(T: np.ndarray, temperature: float, uniforms: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Sampled chain [FLZ, "The last write is refined using discrete
    candidates": conditional probabilities are built, the chain is drawn and
    the probabilities are kept for verification; the factors are computed in
    float64].  At row t the probabilities are softmax(T_t[i*, :] / temperature)
    over the K candidates, i* the previous choice (0 at row 1, the anchor).
    The draw takes the given uniform u in [0, 1) and picks the first j whose
    cumulative probability exceeds u (inverse CDF; the last j if rounding
    leaves u above the total).  The normaliser and the cumulative sum are
    taken left to right over the candidates.  Returns (choices [W-1], q
    [W-1]), q the probability of each chosen candidate."""
    n, K = T.shape[0], T.shape[2]
    choice = np.zeros(n, dtype=np.int64)
    q = np.zeros(n)
    i = 0
    for t in range(n):
        s = np.asarray(T[t, i], dtype=np.float64) / float(temperature)
        e = np.exp(s - np.max(s))
        total = 0.0
        for v in e:                 # left to right (the pages fix no order)
            total += v
        p = e / total
        cdf = 0.0
        j = K - 1
        for jj in range(K):
            cdf += p[jj]
            if float(uniforms[t]) < cdf:
                j = jj
                break
        choice[t] = j
        q[t] = p[j]
        i = j
    return choice, q


def propose(g, wts, lm_head: np.ndarray, ctxs: Sequence[RequestContext], anchor_ids: Sequence[int],
            W: int, K: int, walk: str = "greedy", temperature: float = 1.0,
            uniforms: Optional[np.ndarray] = None, cand_override: Optional[np.ndarray] = None,
            retrieve: int = 0, fp8_head: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> dict:
    """The proposal tail after the draft forward, per request: head scores of
    rows 1..W-1 and their top-K candidates, the transition tables, and the
    walk.  With ``retrieve`` = R > 0 the candidates come from the FP8
    retrieval instead: the R best FP8 scores, rescored with the BF16 head,
    the best K kept (``fp8_head`` = quantize_head_fp8(lm_head), computed
    here when not given); ``scores`` then holds the FP8 scores and
    ``retrieved`` / ``rescored`` [B,W-1,R] the R ids and their BF16 scores.
    ``cand_override`` [B, W-1, K] replaces the candidate ids (to evaluate the
    tables on another implementation's candidates).  Returns a dict of
    float64/int64 arrays: out [B,W,H], scores [B,W-1,V], cand [B,W-1,K],
    cand_scores [B,W-1,K] (BF16 head scores), table [B,W-1,K,K], choice
    [B,W-1], tokens [B,W-1], q [B,W-1] (sampled walk only)."""
    assert g.bridge, "the refinement redoes the last bridge write"
    out, u = draft_forward(g, wts, ctxs, anchor_ids, W, return_last_prewrite=True)
    B = len(ctxs)
    res = {"out": out, "scores": [], "cand": [], "cand_scores": [], "table": [], "choice": [],
           "tokens": [], "q": []}
    if retrieve:
        res["retrieved"], res["rescored"] = [], []
        if fp8_head is None:
            fp8_head = quantize_head_fp8(lm_head)
    for b in range(B):
        if retrieve:
            sc = head_scores_fp8(fp8_head[0], fp8_head[1], out[b, 1:])
            rows = [retrieve_and_rescore(sc[t], lm_head, out[b, 1 + t], retrieve, K) for t in range(W - 1)]
            res["retrieved"].append(np.stack([r[0] for r in rows]))
            res["rescored"].append(np.stack([r[1] for r in rows]))
            cand = np.stack([r[2] for r in rows])
        else:
            sc = head_scores(lm_head, out[b, 1:])
            cand = np.stack([top_k(sc[t], K) for t in range(W - 1)])
        if cand_override is not None:
            cand = np.asarray(cand_override[b], dtype=np.int64)
        T = transition_table(g, wts, lm_head, u[b], int(anchor_ids[b]), cand)
        if walk == "greedy":
            ch, q = greedy_walk(T), np.zeros(W - 1)
        else:
            ch, q = sampled_walk(T, temperature, uniforms[b])
        res["scores"].append(sc)
        res["cand"].append(cand)
        res["cand_scores"].append(np.stack([head_scores(lm_head, out[b, 1 + t], cand[t])[0]
                                            for t in range(W - 1)]) if retrieve
                                  else np.take_along_axis(sc, cand, axis=1))
        res["table"].append(T)
        res["choice"].append(ch)
        res["tokens"].append(cand[np.arange(W - 1), ch])
        res["q"].append(q)
    return {k: (v if k == "out" else np.stack(v)) for k, v in res.items()}


# ---------------------------------------------------------------------------
# size arithmetic
# ---------------------------------------------------------------------------
def ring_bytes_per_position(g) -> int:
    """Bytes of stored context K/V per retained position over all layers:
    2-byte K and 2-byte V per KV head coordinate [FLZ, cache section];
    [NIF, ring storage]."""
    elt = 2 if g.dtype == "bf16" else 4
    return g.n_layers * 2 * elt * g.n_kv_heads * g.head_dim


def bridge_parameter_count(hidden: int, n_layers: int, code_dim: int, msg_dim: int) -> int:
    """Per layer R_l [r, H] and W_l [H, a]; shared G, G_p, A [a, r] and b [a]
    [FLZ, "The bridge"]; [PHY, 门控与写回]."""
    return n_layers * (code_dim * hidden + hidden * msg_dim) + 3 * msg_dim * code_dim + msg_dim
