"""Seeded synthetic inputs for the multi-pass TTT draft attention.

This module is shared by the GPU tests / benchmark and by the fp64 CPU oracle.
It holds no attention arithmetic: it only draws N(0, 1) tensors from seeded
PCG64 streams, rounds them to bfloat16 (round-to-nearest-even) when the
workload is bf16, and builds the packed-sequence lengths of the varlen
workload.

Workloads (the five shapes this library is tested and measured on):

  tiny_fp32   B=1, S=64,    Hq=2,  Hkv=1, D=32,  K=3, fp32, RoPE base 1e4, fwd+bwd
  fwd_s2k     B=1, S=2048,  Hq=32, Hkv=8, D=128, K=3, bf16, RoPE base 1e6, fwd only
  b4_s4k      B=4, S=4096,  Hq=32, Hkv=8, D=128, K=7, bf16, RoPE base 1e6, fwd+bwd
  thd_32k     16 packed sequences, lengths in [256, 4096], T=32768,
              Hq=32, Hkv=8, D=128, K=3, bf16, RoPE base 1e6, fwd+bwd
  s32k        B=1, S=32768, Hq=32, Hkv=8, D=128, K=7, bf16, RoPE base 1e6, fwd+bwd

Every tensor has its own stream, keyed by (workload seed, tensor kind, pass),
so any one tensor can be regenerated without drawing the others.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "thd_lengths", "cu_seqlens_of", "BlockWorkload", "BLOCK_WORKLOADS",
           "block_anchors",
           "draw", "draw_device", "round_bf16", "bf16_bits", "KIND_Q", "KIND_K", "KIND_V", "KIND_DO"]

KIND_Q, KIND_K, KIND_V, KIND_DO = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # seed of every stream of this workload
    layout: str                # "bshd" or "thd"
    B: int
    S: int                     # per-sequence length (bshd) / total tokens T (thd)
    Hq: int
    Hkv: int
    D: int
    K: int                     # number of TTT passes in one unroll
    dtype: str                 # "fp32" or "bf16"
    rope_base: float
    backward: bool
    num_seqs: int = 0          # thd only
    min_len: int = 0           # thd only
    max_len: int = 0           # thd only

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def lengths(self) -> list[int]:
        """Sequence lengths: B copies of S (bshd) or the packed lengths (thd)."""
        if self.layout == "bshd":
            return [self.S] * self.B
        return thd_lengths(self.num_seqs, self.S, self.min_len, self.max_len, self.index)

    @property
    def tokens(self) -> int:
        return self.B * self.S if self.layout == "bshd" else self.S

    def q_shape(self):
        return (self.B, self.S, self.Hq, self.D) if self.layout == "bshd" else (self.S, self.Hq, self.D)

    def kv_shape(self):
        return (self.B, self.S, self.Hkv, self.D) if self.layout == "bshd" else (self.S, self.Hkv, self.D)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 0, "bshd", 1, 64, 2, 1, 32, 3, "fp32", 1e4, True),
    "fwd_s2k": Workload("fwd_s2k", 1, "bshd", 1, 2048, 32, 8, 128, 3, "bf16", 1e6, False),
    "b4_s4k": Workload("b4_s4k", 2, "bshd", 4, 4096, 32, 8, 128, 7, "bf16", 1e6, True),
    "thd_32k": Workload("thd_32k", 3, "thd", 1, 32768, 32, 8, 128, 3, "bf16", 1e6, True,
                        num_seqs=16, min_len=256, max_len=4096),
    "s32k": Workload("s32k", 4, "bshd", 1, 32768, 32, 8, 128, 7, "bf16", 1e6, True),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def thd_lengths(num_seqs: int, total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Packed lengths: num_seqs i.i.d. integers U{lo..hi}, rescaled to sum to `total`.

    The draws are rescaled proportionally and rounded by largest remainder, then
    clamped to [lo, hi]; any residue the clamp leaves is handed out one token at
    a time, in sequence order, to sequences that still have room.
    """
    assert num_seqs * lo <= total <= num_seqs * hi
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    raw = rng.integers(lo, hi + 1, num_seqs).astype(np.float64)
    x = raw * total / raw.sum()
    f = np.floor(x).astype(np.int64)
    rem = total - int(f.sum())
    order = np.argsort(-(x - f), kind="stable")
    f[order[:rem]] += 1
    f = np.clip(f, lo, hi)
    res = total - int(f.sum())
    step = 1 if res > 0 else -1
    s = 0
    while res != 0:
        if lo <= f[s] + step <= hi:
            f[s] += step
            res -= step
        s = (s + 1) % num_seqs
    return [int(v) for v in f]


def cu_seqlens_of(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (((u >> 16) & 1) + 0x7FFF)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def draw_device(w: Workload, kind: int, pass_index: int, device, shape: Optional[tuple] = None):
    """N(0,1) torch tensor drawn on `device` from a seeded torch generator, in the
    workload's dtype (bf16: fp32 draws rounded to nearest even).  A different
    stream from `draw`; used where the host copy is not needed (benchmarks)."""
    import torch
    if shape is None:
        shape = w.q_shape() if kind in (KIND_Q, KIND_DO) else w.kv_shape()
    gen = torch.Generator(device=device)
    gen.manual_seed((w.index * 1000003 + kind * 1009 + pass_index) & 0x7FFFFFFF)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if w.dtype == "bf16" else x


def draw(w: Workload, kind: int, pass_index: int, shape: Optional[tuple] = None) -> np.ndarray:
    """N(0,1) float32 tensor for (workload, kind, pass), rounded to bf16 for bf16 workloads.

    kind: KIND_Q / KIND_K / KIND_V / KIND_DO; pass_index is 1-based.
    The default shape is the workload's Q shape (Q, dO) or KV shape (K, V).
    """
    if shape is None:
        shape = w.q_shape() if kind in (KIND_Q, KIND_DO) else w.kv_shape()
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.index, kind, pass_index])))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if w.dtype == "bf16":
        x = round_bf16(x)
    return x


# ----------------------------------------------------------------------------- block drafting
@dataclasses.dataclass(frozen=True)
class BlockWorkload:
    """Block-draft attention shape: nblk blocks of bs draft slots per batch row,
    each anchored in a context of ctx_len tokens."""
    name: str
    index: int
    B: int
    ctx_len: int
    bs: int
    nblk: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    rope_base: float

    @property
    def rows(self) -> int:
        return self.nblk * self.bs

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q_shape(self):
        return (self.B, self.rows, self.Hq, self.D)

    def blk_shape(self):
        return (self.B, self.rows, self.Hkv, self.D)

    def ctx_shape(self):
        return (self.B, self.ctx_len, self.Hkv, self.D)

    def as_workload(self) -> Workload:
        """The Workload whose streams this block workload draws from (its seed and dtype)."""
        return Workload(self.name, self.index, "bshd", self.B, self.rows, self.Hq, self.Hkv, self.D, 1,
                        self.dtype, self.rope_base, False)


BLOCK_WORKLOADS = {
    # 256 blocks of 16 slots per batch row over a 4096-token context
    "blk_b4_c4k": BlockWorkload("blk_b4_c4k", 5, 4, 4096, 16, 256, 32, 8, 128, "bf16", 1e6),
}


def block_anchors(B: int, nblk: int, ctx_len: int, seed: int) -> np.ndarray:
    """int32 [B, nblk] anchor positions, i.i.d. uniform in [0, ctx_len], ascending per batch row."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    a = rng.integers(0, ctx_len + 1, size=(B, nblk))
    return np.sort(a, axis=1).astype(np.int32)
