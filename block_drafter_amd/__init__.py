"""Python binding of the DSpine draft-block library (``libdspine.so``).

Argument marshalling only: PyTorch allocates device memory and supplies the
HIP stream; every step of the hot path runs in the library's HIP kernels.
There is no fallback: if the library is missing, import-time loading fails
with an error that says how to build it.

Geometry objects are duck-typed: any object with the attributes ``hidden,
n_layers, n_q_heads, n_kv_heads, head_dim, ffn, n_feat_layers, code_dim,
msg_dim, vocab, mask_token_id, block_causal, windows, eps, rope_theta,
dtype`` ("bf16" or "f32").  Weight dictionaries use the tensor names
``w_feat, g_ctx, g_final, embed, codebook, bridge_{G,Gp,A,b}`` and per layer
``l{i}.{g_in,wq,wk,wv,gq,gk,wo,g_post,w_gate,w_up,w_down,R,W_l}``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspine.so")

MAX_LAYERS = 16
MAX_BATCH = 8
OK, E_ARG, E_UNSUPPORTED, E_WORKSPACE, E_STATE, E_HIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1


class DSpineError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dspine error {code}: {msg}")
        self.code = code


class Geometry_c(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_feat_layers", ctypes.c_int32), ("code_dim", ctypes.c_int32),
                ("msg_dim", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("mask_token_id", ctypes.c_int32), ("block_causal", ctypes.c_int32),
                ("window", ctypes.c_int32 * MAX_LAYERS), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("conv_group", ctypes.c_int32)]


_LAYER_FIELDS = ["g_in", "wq", "wk", "wv", "gq", "gk", "wo", "g_post", "w_gate", "w_up",
                 "w_down", "R", "W_l", "attn_conv_w", "attn_conv_base", "mlp_conv_w", "mlp_conv_base"]


class LayerWeights_c(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


_GLOBAL_FIELDS = ["embed", "w_feat", "g_ctx", "g_final", "codebook", "bridge_G", "bridge_Gp",
                  "bridge_A", "bridge_b"]
# matrices the library streams from its packed copy
_PROJECTIONS = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "R", "W_l", "w_feat",
                "bridge_G", "bridge_Gp", "bridge_A", "lm_head", "attn_conv_w", "mlp_conv_w"}


# packed, but also read row-major by the library (kept after packing)
_READ_ROW_MAJOR = {"lm_head"}


class Weights_c(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _GLOBAL_FIELDS] + [
        ("layer", LayerWeights_c * MAX_LAYERS), ("lm_head", ctypes.c_void_p)]


MAX_TOPK = 16
WALK_GREEDY, WALK_SAMPLED = 0, 1


MAX_RETRIEVE = 128


class Proposal_c(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_int32), ("walk", ctypes.c_int32), ("retrieve", ctypes.c_int32),
                ("temperature", ctypes.c_double),
                ("uniforms", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("retrieved", ctypes.c_void_p),
                ("rescored", ctypes.c_void_p), ("cand", ctypes.c_void_p),
                ("cand_scores", ctypes.c_void_p), ("table", ctypes.c_void_p),
                ("choice", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("q", ctypes.c_void_p)]


class Ctx_c(ctypes.Structure):
    _fields_ = [("k_ring", ctypes.c_void_p * MAX_LAYERS), ("v_ring", ctypes.c_void_p * MAX_LAYERS),
                ("capacity", ctypes.c_int64 * MAX_LAYERS), ("frontier", ctypes.c_int64)]


EXPORTS = {
    "dspine_model_create": (ctypes.c_int, [ctypes.POINTER(Geometry_c), ctypes.POINTER(Weights_c),
                                           ctypes.POINTER(ctypes.c_void_p)]),
    "dspine_model_destroy": (None, [ctypes.c_void_p]),
    "dspine_packed_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "dspine_pack_weights": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "dspine_ring_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64]),
    "dspine_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int64]),
    "dspine_ctx_materialize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(Ctx_c),
                                              ctypes.POINTER(ctypes.c_void_p),
                                              ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]),
    "dspine_draft_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(Ctx_c), ctypes.POINTER(ctypes.c_int32),
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "dspine_draft_forward_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                    ctypes.POINTER(Ctx_c), ctypes.POINTER(ctypes.c_int32),
                                                    ctypes.c_void_p, ctypes.c_void_p]),
    "dspine_bridge": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]),
    "dspine_propose_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                         ctypes.c_int]),
    "dspine_draft_propose": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(Ctx_c), ctypes.POINTER(ctypes.c_int32),
                                            ctypes.c_void_p, ctypes.POINTER(Proposal_c),
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "dspine_debug_visible": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.POINTER(Ctx_c), ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dspine_profile_enable": (ctypes.c_int, [ctypes.c_uint32]),
    "dspine_profile_stride": (ctypes.c_int, [ctypes.c_uint32]),
    "dspine_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int64)]),
    "dspine_last_error": (ctypes.c_char_p, []),
    "dspine_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library (built in-tree by ``python -m block_drafter_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m block_drafter_amd.build` "
                              "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise DSpineError(rc, lib().dspine_last_error().decode())


def geometry_struct(g) -> Geometry_c:
    gs = Geometry_c()
    for f in ("hidden", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "n_feat_layers",
              "code_dim", "msg_dim", "vocab", "mask_token_id"):
        setattr(gs, f, int(getattr(g, f)))
    gs.block_causal = int(bool(g.block_causal))
    for l, s in enumerate(g.windows):
        gs.window[l] = int(s)
    gs.eps = float(g.eps)
    gs.rope_theta = float(g.rope_theta)
    gs.dtype = BF16 if g.dtype == "bf16" else F32
    gs.conv_group = int(getattr(g, "conv_group", 0))
    return gs


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray, device="cuda"):
    """Upload one stored tensor (bf16 bits as uint16, or float32) unchanged."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


class Model:
    """A model handle over device weights (borrowed by the library)."""

    def __init__(self, geom, weights: Dict[str, "torch.Tensor"], drop_row_major: bool = True):
        self.geom = geom
        self.weights = weights               # keeps the tensors alive
        self._gs = geometry_struct(geom)
        ws = Weights_c()
        for n in _GLOBAL_FIELDS:
            t = weights.get(n)
            setattr(ws, n, t.data_ptr() if t is not None else None)
        for l in range(geom.n_layers):
            for n in _LAYER_FIELDS:
                t = weights.get(f"l{l}.{n}")
                setattr(ws.layer[l], n, t.data_ptr() if t is not None else None)
        head = weights.get("lm_head")
        ws.lm_head = head.data_ptr() if head is not None else None
        self._ws = ws
        h = ctypes.c_void_p()
        _check(lib().dspine_model_create(ctypes.byref(self._gs), ctypes.byref(ws), ctypes.byref(h)))
        self.handle = h
        self._workspace = None
        # projections in fragment order (the library's streaming layout); the
        # row-major matrices are dropped once the packing kernels have run
        torch = _torch()
        nbytes = lib().dspine_packed_bytes(self.handle)
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        _check(lib().dspine_pack_weights(self.handle, self.packed.data_ptr(), nbytes,
                                         torch.cuda.current_stream().cuda_stream))
        if drop_row_major:
            torch.cuda.current_stream().synchronize()
            for name in list(self.weights):
                if name.split(".")[-1] in _PROJECTIONS and name not in _READ_ROW_MAJOR:
                    del self.weights[name]

    @classmethod
    def from_numpy(cls, geom, wts: Dict[str, np.ndarray], device="cuda", lm_head: Optional[np.ndarray] = None):
        t = {k: to_device(v, device) for k, v in wts.items()}
        if lm_head is not None:
            t["lm_head"] = to_device(lm_head, device)
        return cls(geom, t)

    def close(self):
        if self.handle:
            lib().dspine_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- sizes -------------------------------------------------------------
    def ring_bytes(self, layer: int, capacity: int) -> int:
        n = lib().dspine_ring_bytes(self.handle, layer, capacity)
        if n == 0:
            _check(E_ARG)
        return n

    def workspace_bytes(self, max_batch: int, max_width: int, max_rows: int) -> int:
        n = lib().dspine_workspace_bytes(self.handle, max_batch, max_width, max_rows)
        if n == 0:
            _check(E_ARG)
        return n

    def workspace(self, max_batch=MAX_BATCH, max_width=16, max_rows=2048):
        """A zero-filled device workspace (reused while large enough)."""
        torch = _torch()
        need = self.workspace_bytes(max_batch, max_width, max_rows)
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.zeros(need, dtype=torch.uint8, device="cuda")
        return self._workspace

    # -- contexts ------------------------------------------------------------
    def new_context(self, full_capacity: int = 0, fill: Optional[float] = None) -> "Context":
        return Context(self, full_capacity, fill)

    # -- calls ---------------------------------------------------------------
    def materialize(self, ctxs: Sequence["Context"], feats: Sequence, workspace=None, stream=None):
        torch = _torch()
        n = len(ctxs)
        arr = (Ctx_c * n)(*[c.struct for c in ctxs])
        ptrs = (ctypes.c_void_p * n)(*[f.data_ptr() if f is not None and f.numel() else None
                                       for f in feats])
        ntok = (ctypes.c_int64 * n)(*[0 if f is None else int(f.shape[0]) for f in feats])
        ws = workspace if workspace is not None else self.workspace(
            max_rows=max(1, min(16384, sum(int(x) for x in ntok))))
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib().dspine_ctx_materialize(self.handle, n, arr, ptrs, ntok, ws.data_ptr(),
                                            ws.numel(), st))
        for c, s in zip(ctxs, arr):
            c.struct.frontier = s.frontier

    def forward(self, ctxs: Sequence["Context"], anchor_ids: Sequence[int], W: int,
                out=None, workspace=None, stream=None):
        torch = _torch()
        B = len(ctxs)
        arr = (Ctx_c * B)(*[c.struct for c in ctxs])
        aid = (ctypes.c_int32 * B)(*[int(a) for a in anchor_ids])
        if out is None:
            out = torch.empty((B, W, self.geom.hidden), dtype=torch.float32, device="cuda")
        ws = workspace if workspace is not None else self.workspace()
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib().dspine_draft_forward(self.handle, B, W, arr, aid, out.data_ptr(),
                                          ws.data_ptr(), ws.numel(), st))
        return out

    def forward_noalloc(self, ctxs: Sequence["Context"], anchor_ids: Sequence[int], W: int, out=None, stream=None):
        """dspine_draft_forward_noalloc: the forward on the library's static scratch (no workspace)."""
        torch = _torch()
        B = len(ctxs)
        arr = (Ctx_c * B)(*[c.struct for c in ctxs])
        aid = (ctypes.c_int32 * B)(*[int(a) for a in anchor_ids])
        if out is None:
            out = torch.empty((B, W, self.geom.hidden), dtype=torch.float32, device="cuda")
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib().dspine_draft_forward_noalloc(self.handle, B, W, arr, aid, out.data_ptr(), st))
        return out

    def propose_workspace(self, max_batch=MAX_BATCH, max_width=16, topk=MAX_TOPK):
        """Device workspace of the proposal tail (reused while large enough)."""
        torch = _torch()
        need = lib().dspine_propose_workspace_bytes(self.handle, max_batch, max_width, topk)
        if need == 0:
            _check(E_ARG)
        if getattr(self, "_pworkspace", None) is None or self._pworkspace.numel() < need:
            self._pworkspace = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self._pworkspace

    def propose(self, ctxs: Sequence["Context"], anchor_ids: Sequence[int], W: int, topk: int = MAX_TOPK,
                walk: str = "greedy", temperature: float = 1.0, uniforms=None, keep_scores: bool = False,
                out=None, workspace=None, propose_workspace=None, stream=None, outputs=None,
                retrieve: int = 0):
        """One draft forward plus the proposal tail.  Returns a dict of device
        tensors: out [B,W,H], cand/cand_scores [B,W-1,K], table [B,W-1,K,K],
        choice/tokens [B,W-1], q [B,W-1] (float64), scores [B*W,vocab] when
        keep_scores.  ``uniforms``: device float64 [B, W-1] for the sampled
        walk.  ``retrieve`` = R > 0: FP8 retrieval of R candidates per row,
        rescored with the BF16 head (``scores`` then holds the FP8 scores,
        and with keep_scores ``retrieved`` / ``rescored`` [B,W-1,R] are
        returned too).  ``outputs`` reuses a dict returned by an earlier call."""
        torch = _torch()
        B, K = len(ctxs), int(topk)
        arr = (Ctx_c * B)(*[c.struct for c in ctxs])
        aid = (ctypes.c_int32 * B)(*[int(a) for a in anchor_ids])
        dev = "cuda"
        o = outputs if outputs is not None else {
            "out": out if out is not None else torch.empty((B, W, self.geom.hidden), dtype=torch.float32, device=dev),
            "cand": torch.empty((B, W - 1, K), dtype=torch.int32, device=dev),
            "cand_scores": torch.empty((B, W - 1, K), dtype=torch.float32, device=dev),
            "table": torch.empty((B, W - 1, K, K), dtype=torch.float32, device=dev),
            "choice": torch.empty((B, W - 1), dtype=torch.int32, device=dev),
            "tokens": torch.empty((B, W - 1), dtype=torch.int32, device=dev),
            "q": torch.empty((B, W - 1), dtype=torch.float64, device=dev),
        }
        if keep_scores and "scores" not in o:
            o["scores"] = torch.empty((B * W, self.geom.vocab), dtype=torch.float32, device=dev)
        if keep_scores and retrieve and "retrieved" not in o:
            o["retrieved"] = torch.empty((B, W - 1, retrieve), dtype=torch.int32, device=dev)
            o["rescored"] = torch.empty((B, W - 1, retrieve), dtype=torch.float32, device=dev)
        pr = Proposal_c()
        pr.topk = K
        pr.walk = WALK_GREEDY if walk == "greedy" else WALK_SAMPLED
        pr.retrieve = int(retrieve)
        pr.retrieved = o["retrieved"].data_ptr() if retrieve and "retrieved" in o else None
        pr.rescored = o["rescored"].data_ptr() if retrieve and "rescored" in o else None
        pr.temperature = float(temperature)
        pr.uniforms = uniforms.data_ptr() if uniforms is not None else None
        pr.scores = o["scores"].data_ptr() if "scores" in o else None
        for n in ("cand", "cand_scores", "table", "choice", "tokens", "q"):
            setattr(pr, n, o[n].data_ptr())
        ws = workspace if workspace is not None else self.workspace()
        pws = propose_workspace if propose_workspace is not None else self.propose_workspace(B, W, K)
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib().dspine_draft_propose(self.handle, B, W, arr, aid, o["out"].data_ptr(), ctypes.byref(pr),
                                          ws.data_ptr(), ws.numel(), pws.data_ptr(), pws.numel(), st))
        return o

    def bridge(self, layer: int, x, anchor_ids: Sequence[int], pred_codes=None,
               workspace=None, stream=None):
        """In place on x: float32 [B, W, H] on the device."""
        torch = _torch()
        B, W = int(x.shape[0]), int(x.shape[1])
        aid = (ctypes.c_int32 * B)(*[int(a) for a in anchor_ids])
        ws = workspace if workspace is not None else self.workspace()
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib().dspine_bridge(self.handle, layer, B, W, x.data_ptr(), aid,
                                   None if pred_codes is None else pred_codes.data_ptr(),
                                   ws.data_ptr(), ws.numel(), st))
        return x

    def debug_visible(self, layer: int, ctxs: Sequence["Context"], W: int):
        torch = _torch()
        B = len(ctxs)
        arr = (Ctx_c * B)(*[c.struct for c in ctxs])
        lo_hi = torch.empty((B, W, 2), dtype=torch.int64, device="cuda")
        slot = torch.empty((B, W), dtype=torch.int32, device="cuda")
        nblk = torch.empty((B, W), dtype=torch.int32, device="cuda")
        _check(lib().dspine_debug_visible(self.handle, layer, B, W, arr, lo_hi.data_ptr(),
                                          slot.data_ptr(), nblk.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream))
        return lo_hi, slot, nblk


PROF_KINDS = ["gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down", "bridge", "norm",
              "ctx_gemm", "ctx_store", "head", "tail", "conv"]


def profile_enable(kinds: Sequence[str]):
    mask = 0
    for k in kinds:
        mask |= 1 << PROF_KINDS.index(k)
    _check(lib().dspine_profile_enable(mask))


def profile_stride(stride: int):
    """Record only every `stride`-th launch scope of each enabled class."""
    _check(lib().dspine_profile_stride(stride))


def profile_read(kind: str):
    """(total milliseconds, launches) recorded for one kernel class; clears it."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().dspine_profile_read(PROF_KINDS.index(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class Context:
    """Per-request draft context: one K and one V ring per layer (device
    tensors owned here) plus the host-side frontier."""

    def __init__(self, model: Model, full_capacity: int = 0, fill: Optional[float] = None):
        torch = _torch()
        g = model.geom
        self.model = model
        self.struct = Ctx_c()
        self.k, self.v = [], []
        kdt = torch.bfloat16 if g.dtype == "bf16" else torch.float32
        vdt = torch.float16 if g.dtype == "bf16" else torch.float32
        for l in range(g.n_layers):
            S = int(g.windows[l])
            cap = S if S > 0 else int(full_capacity)
            shape = (g.n_kv_heads, cap, g.head_dim)
            if fill is None:
                k = torch.empty(shape, dtype=kdt, device="cuda")
                v = torch.empty(shape, dtype=vdt, device="cuda")
            else:
                k = torch.full(shape, fill, dtype=kdt, device="cuda")
                v = torch.full(shape, fill, dtype=vdt, device="cuda")
            self.k.append(k)
            self.v.append(v)
            self.struct.k_ring[l] = k.data_ptr()
            self.struct.v_ring[l] = v.data_ptr()
            self.struct.capacity[l] = cap
        self.struct.frontier = 0

    @property
    def frontier(self) -> int:
        return int(self.struct.frontier)

    @frontier.setter
    def frontier(self, v: int):
        self.struct.frontier = int(v)
