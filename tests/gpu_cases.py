"""Shared machinery of the GPU parity tests: build one seeded case, run it
through the HIP library and through the CPU oracle, and compare.

Nothing here computes the method: the GPU side only calls the binding, the
expected side only calls ``oracle``.  Both consume the bits made by ``synth``."""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

import synth
from oracle import dspine_oracle as O

TOL_BF16 = 2e-2     # max |gpu - oracle| / rms(oracle), bf16 weights and operands
TOL_F32 = 1e-4      # same, float32 model


def tol_for(g) -> float:
    return TOL_BF16 if g.dtype == "bf16" else TOL_F32


def rel_err(gpu: np.ndarray, orc: np.ndarray) -> float:
    return float(np.max(np.abs(gpu - orc)) / np.sqrt(np.mean(orc * orc)))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (7 stored fraction bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def storage_err(gpu: np.ndarray, orc: np.ndarray, bf16: bool) -> float:
    """Stored K/V: both sides round to the storage format, so a tiny upstream
    difference may land on the neighbouring bf16 value.  Allow that one ulp,
    then measure what is left relative to rms, like the hidden states."""
    d = np.abs(gpu - orc)
    if bf16:
        d = np.maximum(0.0, d - bf16_ulp(orc))
    return float(np.max(d) / np.sqrt(np.mean(orc * orc)))


def to_np64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class Case:
    g: synth.Geometry
    seed: int
    B: int
    W: int
    frontiers: Sequence[int]
    chunks: Optional[Sequence[Sequence[int]]] = None   # per request: sizes summing to F
    anchors: Optional[Sequence[int]] = None
    full_capacity: int = 0
    shared_features: bool = False      # every request reads request 0's features


class Run:
    """One case on both sides.  Oracle work is done lazily per request."""

    def __init__(self, case: Case, model=None, wts=None, sentinel=True):
        import torch
        import block_drafter_amd as bd
        self.case = case
        g = case.g
        self.wts = wts if wts is not None else synth.make_weights(g, case.seed)
        self.model = model if model is not None else bd.Model.from_numpy(g, self.wts)
        self.anchors = (list(case.anchors) if case.anchors is not None
                        else [int(a) for a in synth.make_anchor_ids(g, case.seed, case.B)])
        cap = case.full_capacity or (max(case.frontiers) + 64)
        self.feats = [synth.make_features(g, case.seed, 0 if case.shared_features else b, F)
                      for b, F in enumerate(case.frontiers)]
        self.ctxs = [self.model.new_context(full_capacity=cap, fill=float("nan") if sentinel else None)
                     for _ in range(case.B)]
        self.cap = cap
        self.chunks = case.chunks or [[F] for F in case.frontiers]
        # materialize on the GPU: step k of every request in one call
        dev = [bd.to_device(f) for f in self.feats]
        steps = max(len(c) for c in self.chunks)
        offs = [0] * case.B
        for k in range(steps):
            sel, fs = [], []
            for b in range(case.B):
                if k < len(self.chunks[b]):
                    n = self.chunks[b][k]
                    sel.append(self.ctxs[b])
                    fs.append(dev[b][offs[b]:offs[b] + n])
                    offs[b] += n
            if sel:
                self.model.materialize(sel, fs)
        torch.cuda.synchronize()
        self._orc_ctx = {}

    def oracle_ctx(self, b: int) -> O.RequestContext:
        if b not in self._orc_ctx:
            ctx = O.empty_context(self.case.g)
            s = 0
            for n in self.chunks[b]:
                ctx = O.materialize(self.case.g, self.wts, ctx, self.feats[b][s:s + n])
                s += n
            self._orc_ctx[b] = ctx
        return self._orc_ctx[b]

    def gpu_forward(self, W=None):
        import torch
        out = self.model.forward(self.ctxs, self.anchors, W or self.case.W)
        torch.cuda.synchronize()
        return to_np64(out)

    def oracle_forward(self, requests: Optional[List[int]] = None, W=None):
        req = list(range(self.case.B)) if requests is None else requests
        return O.draft_forward(self.case.g, self.wts, [self.oracle_ctx(b) for b in req],
                               [self.anchors[b] for b in req], W or self.case.W)

    def ring_errors(self, b: int):
        """(max rel error over live slots, sentinel intact elsewhere) per layer and K/V."""
        g = self.case.g
        ctx = self.oracle_ctx(b)
        res = []
        for l in range(g.n_layers):
            S = g.windows[l]
            cap = S if S > 0 else self.cap
            Ko, Vo = O.ring_image(g, ctx, l, cap)
            for name, gpu, orc in (("K", self.ctxs[b].k[l], Ko), ("V", self.ctxs[b].v[l], Vo)):
                gv = to_np64(gpu)
                live = ~np.isnan(orc)
                err = storage_err(gv[live], orc[live], g.dtype == "bf16") if live.any() else 0.0
                res.append((l, name, err, bool(np.all(np.isnan(gv[~live])))))
        return res
