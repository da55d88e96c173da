"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage type once, and describes the five workload shapes.
Both sides (the CPU oracle and the HIP library) consume exactly the bits made
here.

Conventions
-----------
* A ``numpy.uint16`` array carries bfloat16 bit patterns; a ``numpy.float32``
  array carries fp32 values.  ``to_float`` widens either to float64 exactly.
* Matrices use the ``[out, in]`` row-major layout of a linear layer.
* Every tensor is drawn from its own generator,
  ``numpy.random.default_rng([seed, tensor_index, chunk_index])``, in chunks of
  ``CHUNK`` elements, so the result does not depend on thread count.
* Linear weights are N(0, 1/fan_in); norm gains are 1 + 0.1 N(0,1); the bridge
  bias is 0.1 N(0,1); embeddings and target features are N(0,1); codebook rows
  are N(0,1) and then L2-normalised in float64 before the one rounding.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

CHUNK = 1 << 20


# ---------------------------------------------------------------------------
# storage rounding used only to produce the input bits
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(a: np.ndarray) -> np.ndarray:
    """Widen a stored tensor (bf16 bits or fp32) to float64, exactly."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Geometry:
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    n_feat_layers: int
    code_dim: int          # r; 0 disables the bridge (plain DFlash)
    msg_dim: int           # a
    vocab: int
    windows: tuple         # per layer S_l; 0 = full attention
    eps: float = 1e-6
    rope_theta: float = 1e7
    dtype: str = "bf16"    # "bf16" or "f32"
    block_causal: bool = False
    conv_group: int = 0    # DFlash2 dynamic grouped convolution group width; 0 = none

    @property
    def conv(self) -> bool:
        return self.conv_group > 0

    @property
    def conv_groups(self) -> int:
        return self.hidden // self.conv_group if self.conv_group else 0

    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def bridge(self) -> bool:
        return self.code_dim > 0

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    geom: Geometry
    seed: int
    B: int
    W: int
    frontiers: tuple            # per request context length before the forward
    prefill_chunk: Optional[int] = None   # config with one big chunk per request
    note: str = ""


G_TINY = Geometry(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  ffn=768, n_feat_layers=2, code_dim=64, msg_dim=32, vocab=1024,
                  windows=(0, 0), dtype="f32")

G_27B = Geometry(hidden=5120, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                 ffn=17408, n_feat_layers=5, code_dim=1024, msg_dim=512, vocab=248320,
                 windows=(2048,) * 5)

# The 27B checkpoint's own attention: block-causal, 8192-position windows.
G_27B_CAUSAL = Geometry(hidden=5120, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        ffn=17408, n_feat_layers=5, code_dim=1024, msg_dim=512, vocab=248320,
                        windows=(8192,) * 5, block_causal=True)

# DFlash2 27B: five local layers, dynamic grouped convolution of group width 16, no bridge
G_27B_DFLASH2 = Geometry(hidden=5120, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         ffn=17408, n_feat_layers=5, code_dim=0, msg_dim=0, vocab=248320,
                         windows=(2048,) * 5, conv_group=16)

G_35B_DFLASH = Geometry(hidden=2048, n_layers=6, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        ffn=6144, n_feat_layers=8, code_dim=0, msg_dim=0, vocab=248320,
                        windows=(4096,) * 5 + (0,))


def _uniform_frontiers(seed: int, B: int, lo: int, hi: int) -> tuple:
    rng = np.random.default_rng([seed, 999])
    return tuple(int(v) for v in rng.integers(lo, hi + 1, size=B))


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", G_TINY, 1001, B=1, W=16, frontiers=(128,),
                          note="tiny fp32 drafter, full attention, 128 context positions"),
    "dspine27b_b1": Workload("dspine27b_b1", G_27B, 1002, B=1, W=16, frontiers=(4096,),
                             note="27B geometry, one block, 4096 context tokens"),
    "dspine27b_b8": Workload("dspine27b_b8", G_27B, 1003, B=8, W=16,
                             frontiers=_uniform_frontiers(1003, 8, 1024, 16384),
                             note="27B geometry, 8 blocks, context lengths U{1024..16384}"),
    "dspine27b_causal_b8": Workload("dspine27b_causal_b8", G_27B_CAUSAL, 1006, B=8, W=16,
                                    frontiers=_uniform_frontiers(1006, 8, 1024, 16384),
                                    note="27B geometry with block-causal attention and 8192-position "
                                         "windows, 8 blocks, context lengths U{1024..16384}"),
    "dflash2_27b_b8": Workload("dflash2_27b_b8", G_27B_DFLASH2, 1007, B=8, W=16,
                               frontiers=_uniform_frontiers(1007, 8, 1024, 16384),
                               note="DFlash2 27B geometry: dynamic grouped convolution (two taps, "
                                    "group width 16) around attention and MLP, no bridge"),
    "dflash35b_b8": Workload("dflash35b_b8", G_35B_DFLASH, 1004, B=8, W=16,
                             frontiers=(32768,) * 8,
                             note="35B-A3B-style plain DFlash, bridge off, 5 local + 1 full layer"),
    "prefill27b": Workload("prefill27b", G_27B, 1005, B=8, W=16, frontiers=(32768,) * 8,
                           prefill_chunk=32768,
                           note="27B prefill: one 32768-token chunk per request into a fresh "
                                "2048 ring, then a B=8 forward"),
}


# ---------------------------------------------------------------------------
# generation
# ---------------------------------------------------------------------------
_POOL: Optional[_cf.ThreadPoolExecutor] = None


def _pool() -> _cf.ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = int(os.environ.get("SYNTH_THREADS", min(16, os.cpu_count() or 1)))
        _POOL = _cf.ThreadPoolExecutor(max_workers=max(1, n))
    return _POOL


def normal(seed: int, index: int, shape, scale: float = 1.0, shift: float = 0.0,
           out_dtype: str = "bf16", rows: Optional[tuple] = None) -> np.ndarray:
    """N(shift, scale^2) values of ``shape``; rounded once to ``out_dtype``.

    ``rows=(r0, r1)`` returns only rows r0..r1-1 of the leading axis, with
    exactly the values the whole tensor has there."""
    n = int(np.prod(shape)) if len(shape) else 1
    row_elems = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    r0, r1 = rows if rows is not None else (0, shape[0] if len(shape) else 1)
    e0, e1 = r0 * row_elems, r1 * row_elems
    m = e1 - e0
    out = np.empty(m, dtype=np.uint16 if out_dtype == "bf16" else np.float32)
    c_first, c_last = e0 // CHUNK, (e1 - 1) // CHUNK if m > 0 else -1

    def work(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.default_rng([seed, index, c])
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        if shift != 0.0:
            v += np.float32(shift)
        a, b = max(lo, e0), min(hi, e1)
        v = v[a - lo:b - lo]
        out[a - e0:b - e0] = f32_to_bf16_bits(v) if out_dtype == "bf16" else v

    chunks = range(c_first, c_last + 1)
    if len(chunks) <= 1:
        for c in chunks:
            work(c)
    else:
        list(_pool().map(work, chunks))
    return out.reshape(((r1 - r0),) + tuple(shape[1:]) if len(shape) else ())


def unit_rows(seed: int, index: int, rows: int, cols: int, out_dtype: str) -> np.ndarray:
    """Rows drawn N(0,1) and L2-normalised in float64 before the one rounding."""
    out = np.empty((rows, cols), dtype=np.uint16 if out_dtype == "bf16" else np.float32)
    rpc = max(1, CHUNK // cols)
    nchunks = (rows + rpc - 1) // rpc

    def work(c):
        lo = c * rpc
        hi = min(rows, lo + rpc)
        g = np.random.default_rng([seed, index, c])
        v = g.standard_normal((hi - lo, cols), dtype=np.float32).astype(np.float64)
        v /= np.sqrt((v * v).sum(axis=1, keepdims=True))
        v = v.astype(np.float32)
        out[lo:hi] = f32_to_bf16_bits(v) if out_dtype == "bf16" else v

    list(_pool().map(work, range(nchunks)))
    return out


def weight_names(g: Geometry) -> List[str]:
    """Draw order of the model tensors (index in this list = tensor_index)."""
    names = ["w_feat", "g_ctx"]
    for l in range(g.n_layers):
        names += [f"l{l}.g_in", f"l{l}.wq", f"l{l}.wk", f"l{l}.wv", f"l{l}.gq", f"l{l}.gk",
                  f"l{l}.wo", f"l{l}.g_post", f"l{l}.w_gate", f"l{l}.w_up", f"l{l}.w_down"]
        if g.bridge:
            names += [f"l{l}.R", f"l{l}.W_l"]
    if g.bridge:
        names += ["bridge_G", "bridge_Gp", "bridge_A", "bridge_b", "codebook"]
    names += ["g_final", "embed"]
    if g.conv:      # appended last: the other tensors keep their draw indices
        for l in range(g.n_layers):
            names += [f"l{l}.attn_conv_w", f"l{l}.attn_conv_base", f"l{l}.mlp_conv_w", f"l{l}.mlp_conv_base"]
    return names


def weight_shape(g: Geometry, name: str) -> tuple:
    H, F = g.hidden, g.ffn
    base = name.split(".")[-1]
    table = {
        "w_feat": (H, g.n_feat_layers * H), "g_ctx": (H,), "g_final": (H,),
        "g_in": (H,), "g_post": (H,), "wq": (g.q_dim, H), "wk": (g.kv_dim, H),
        "wv": (g.kv_dim, H), "gq": (g.head_dim,), "gk": (g.head_dim,), "wo": (H, g.q_dim),
        "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
        "R": (g.code_dim, H), "W_l": (H, g.msg_dim),
        "bridge_G": (g.msg_dim, g.code_dim), "bridge_Gp": (g.msg_dim, g.code_dim),
        "bridge_A": (g.msg_dim, g.code_dim), "bridge_b": (g.msg_dim,),
        "codebook": (g.vocab, g.code_dim), "embed": (g.vocab, H),
        "attn_conv_w": (4 * g.conv_groups, H), "mlp_conv_w": (4 * g.conv_groups, H),
        "attn_conv_base": (4, H), "mlp_conv_base": (4, H),
    }
    return table[base]


def make_weights(g: Geometry, seed: int, overrides: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """All model tensors for geometry ``g``; ``overrides`` replaces named tensors."""
    overrides = overrides or {}
    out: Dict[str, np.ndarray] = {}
    for idx, name in enumerate(weight_names(g)):
        if name in overrides:
            out[name] = overrides[name]
            continue
        shape = weight_shape(g, name)
        base = name.split(".")[-1]
        if base.startswith("g_") or base in ("gq", "gk"):
            out[name] = normal(seed, idx, shape, 0.1, 1.0, g.dtype)
        elif base == "bridge_b":
            out[name] = normal(seed, idx, shape, 0.1, 0.0, g.dtype)
        elif base == "codebook":
            out[name] = unit_rows(seed, idx, shape[0], shape[1], g.dtype)
        elif base == "embed":
            out[name] = normal(seed, idx, shape, 1.0, 0.0, g.dtype)
        elif base.endswith("_conv_base"):
            # rows (side, tap): the current-row taps near 1, the previous-row taps near 0
            b = normal(seed, idx, shape, 0.1, 0.0, "f32")
            b[0] += 1.0
            b[2] += 1.0
            out[name] = f32_to_bf16_bits(b) if g.dtype == "bf16" else b
        elif base.endswith("_conv_w"):
            out[name] = normal(seed, idx, shape, 0.1 / math.sqrt(shape[1]), 0.0, g.dtype)
        else:
            out[name] = normal(seed, idx, shape, 1.0 / math.sqrt(shape[1]), 0.0, g.dtype)
    return out


FEATURE_INDEX_BASE = 10_000
ANCHOR_INDEX = 20_000


# Every request has one feature sequence of FEATURE_ROWS positions; the
# features of positions [p0, p1) are rows p0..p1-1 of it, whatever chunking
# a test or the bench materializes them in.
FEATURE_ROWS = 1 << 20


def make_features(g: Geometry, seed: int, request: int, n_tok: int, start: int = 0) -> np.ndarray:
    """Target residual features ~ N(0,1) of positions [start, start + n_tok)
    of one request: ``[n_tok, Lf*H]``."""
    return normal(seed, FEATURE_INDEX_BASE + request, (FEATURE_ROWS, g.n_feat_layers * g.hidden),
                  1.0, 0.0, g.dtype, rows=(start, start + n_tok))


def make_anchor_ids(g: Geometry, seed: int, B: int, stream: int = 0) -> np.ndarray:
    rng = np.random.default_rng([seed, ANCHOR_INDEX + stream])
    return rng.integers(0, g.vocab, size=B, dtype=np.int64).astype(np.int32)


def with_geometry(g: Geometry, **kw) -> Geometry:
    return dataclasses.replace(g, **kw)


LM_HEAD_INDEX = 30_000
UNIFORM_INDEX = 40_000


def make_lm_head(g: Geometry, seed: int) -> np.ndarray:
    """The shared LM head [vocab, H] ~ N(0, 1/H) (the target's output
    embedding, used by the proposal tail); drawn only when asked for."""
    return normal(seed, LM_HEAD_INDEX, (g.vocab, g.hidden), 1.0 / math.sqrt(g.hidden), 0.0, g.dtype)


def make_uniforms(seed: int, B: int, n: int, stream: int = 0) -> np.ndarray:
    """Uniform draws in [0, 1) for the sampled walk, float64 [B, n]."""
    rng = np.random.default_rng([seed, UNIFORM_INDEX + stream])
    return rng.random((B, n))
