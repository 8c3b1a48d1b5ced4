"""Shared helpers of the GPU parity tests: seeded inputs, row sampling and
comparison against the fp64 oracle at the tolerances the library is held to.

Tolerances (fp64 oracle as reference):
  fp32 inputs: O and LSE max-abs <= 1e-5; gradients relative Frobenius <= 1e-5
  bf16 inputs: O max-abs <= 1e-2 (fp32 O output), LSE max-abs <= 2e-3,
               gradients relative Frobenius <= 1e-2.
A bf16 O output is additionally allowed half a bf16 ulp of the reference value:
the rounding of the output type itself, which the fp32-output run excludes.
"""
from __future__ import annotations

import math

import numpy as np

import ttt_synth as syn
from oracle import ttt_oracle as O

TOL = {"fp32": dict(o=1e-5, lse=1e-5, grad=1e-5), "bf16": dict(o=1e-2, lse=2e-3, grad=1e-2)}


def torch_dtype(w):
    import torch
    return torch.float32 if w.dtype == "fp32" else torch.bfloat16


def upload(x: np.ndarray, w, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch_dtype(w))


class Inputs:
    """Host (float32, bf16-valued for bf16 workloads) and device copies of one workload's tensors."""

    def __init__(self, w: syn.Workload, dev, passes=None, with_grad=True, lengths=None):
        import torch
        self.w = w
        K = w.K if passes is None else passes
        self.q = {p: syn.draw(w, syn.KIND_Q, p) for p in range(1, K + 1)}
        self.k = [syn.draw(w, syn.KIND_K, t) for t in range(1, K + 1)]
        self.v = [syn.draw(w, syn.KIND_V, t) for t in range(1, K + 1)]
        self.do = {p: syn.draw(w, syn.KIND_DO, p) for p in range(1, K + 1)} if with_grad else {}
        self.gq = {p: upload(x, w, dev) for p, x in self.q.items()}
        self.gk = [upload(x, w, dev) for x in self.k]
        self.gv = [upload(x, w, dev) for x in self.v]
        self.gdo = {p: upload(x, w, dev) for p, x in self.do.items()}
        self.lengths = list(lengths) if lengths is not None else w.lengths()
        self.cu_host = syn.cu_seqlens_of(self.lengths)
        self.cu = torch.from_numpy(self.cu_host).to(dev) if w.layout == "thd" else None
        self.layout = w.layout

    def kw(self):
        return dict(cu_seqlens=self.cu, rope_base=self.w.rope_base)

    def slices(self):
        return O.sequences(self.layout, self.q[1].shape, self.cu_host)


def lse_at(lse: np.ndarray, layout, sl, h, rows):
    rows = np.asarray(rows)
    return lse[sl.b, h, rows] if layout == "bshd" else lse[h, sl.start + rows]


def row_at(x: np.ndarray, layout, sl, h, rows):
    rows = np.asarray(rows)
    return x[sl.b, rows, h] if layout == "bshd" else x[sl.start + rows, h]


def sample_rows(inp: Inputs, n: int, seed: int, passes):
    """n query rows uniform over (sequence-row, head, pass) plus forced edge rows:
    i in {0, 1, last} of every sequence and every pass, tile borders 127/128.
    Returns {(p, seq, h): sorted rows}."""
    w = inp.w
    rng = np.random.default_rng(1000 + seed)
    lens = np.asarray(inp.lengths)
    cum = np.concatenate([[0], np.cumsum(lens)])
    out = {}

    def add(p, s, h, i):
        out.setdefault((p, s, h), set()).add(int(i))

    passes = list(passes)
    seen = 0
    while seen < n:  # n distinct random rows
        t = int(rng.integers(0, cum[-1]))
        h = int(rng.integers(0, w.Hq))
        p = passes[int(rng.integers(0, len(passes)))]
        s = int(np.searchsorted(cum, t, side="right") - 1)
        key = (p, s, h)
        before = len(out.get(key, ()))
        add(p, s, h, t - cum[s])
        seen += len(out[key]) - before
    for p in passes:
        for s, L in enumerate(lens):
            h = int(rng.integers(0, w.Hq))
            for i in {0, 1, L - 1, min(127, L - 1), min(128, L - 1)}:
                if 0 <= i < L:
                    add(p, s, h, i)
    return {k_: np.array(sorted(v)) for k_, v in out.items()}


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 1e-30)
    return 2.0 ** (np.floor(np.log2(ax)) - 8)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rel_fro(a, b):
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / (nb if nb > 0 else 1.0))


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()
