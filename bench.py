"""Benchmark of libtttattn on one MI355X: the full multi-pass TTT attention unroll.

One step = the whole hot path over one batch of synthetic inputs: the forward of
passes p = 1..K, then the backward of passes p = K..1 (every kernel of the
library's bf16 path runs each step).  Inputs are resident in HBM before the
timed region.  Prints ONE JSON line (see the keys below).

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload b4_s4k]

Throughput counts causal useful FLOPs only: per pass, forward
4*D*Hq*(trunk visible pairs + branch pairs) and backward 2.5x that.  Per-kernel
durations come from HIP events recorded around each launch (through the
library's launch trace hook) over the timed region; each kernel's roofline
uses its own algorithmic work per launch.  The fp64 CPU oracle is timed on a
bounded sample of the same workload on the host (rank 0) as a baseline only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16 = 2.5e15     # MI355X dense bf16/fp16 MFMA, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, bytes/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="b4_s4k")
    ap.add_argument("--head-dim", type=int, default=0, metavar="D",
                    help="run the unroll at head_dim D (32 or 64: bf16 on zero-padded heads) instead of the "
                         "workload's 128; FLOPs count the D-dim work")
    ap.add_argument("--bwd-stored-ds", action="store_true",
                    help="backward with stored dS: dK/dV writes dS, dQ = dS K~ (bwd_mode STORED_DS)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-times", action="store_true", help="skip the per-kernel event timing")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="sliding-window trunk of W keys for the unroll (0: the full causal trunk)")
    ap.add_argument("--ring", type=int, default=0, metavar="CP",
                    help="instead of the unroll, time the ring-step forward of the last pass over a zig-zag ring "
                         "of CP ranks emulated on this GPU, per chunk shape (prints its own JSON line)")
    ap.add_argument("--block", action="store_true",
                    help="instead of the unroll, time the block-draft forward on the blk_b4_c4k shape "
                         "(prints its own JSON line)")
    ap.add_argument("--block-thd", action="store_true",
                    help="instead of the unroll, time packed (THD) block drafting: the thd_32k sequences as "
                         "contexts, 64 blocks of 16 slots per sequence (prints its own JSON line)")
    ap.add_argument("--soft-ce", action="store_true",
                    help="instead of the attention unroll, time the per-pass soft cross-entropy (forward + "
                         "backward for passes 1..7) on B=4, S=4096, V=32000 bf16 logits (prints its own JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy a 256 MiB buffer 3 times (a plain copy kernel of known size "
                         "that scales the HBM byte counters of a profiler run)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- work accounting
WINDOW = 0  # sliding-window trunk of the measured unroll (0: full causal trunk)


def trunk_pairs(w) -> int:
    """Visible (query, key) pairs of the trunk per head per pass: sum over sequences of L(L+1)/2,
    or of sum_i min(i + 1, W) with a sliding window of W keys."""
    if WINDOW <= 0:
        return sum(L * (L + 1) // 2 for L in w.lengths())
    W = WINDOW
    return sum((min(L, W) * (min(L, W) + 1)) // 2 + max(0, L - W) * W for L in w.lengths())


def useful_flops(w, p: int) -> tuple[float, float]:
    """(forward, backward) causal useful FLOPs of pass p."""
    fwd = 4.0 * w.D * w.Hq * (trunk_pairs(w) + (p - 1) * w.tokens)
    return fwd, 2.5 * fwd


def kernel_work(w, name: str, p: int):
    """(amount, unit) of algorithmic work of one launch of kernel `name` at pass p."""
    tp = trunk_pairs(w)
    T = w.tokens
    row_q, row_kv = w.Hq * w.D * 2, w.Hkv * w.D * 2     # bf16 bytes per token
    if name == "trunk_fwd":            # S = QK^T and O = PV over the visible trunk pairs
        return 4.0 * w.D * w.Hq * tp, "flop"
    if name == "trunk_dkdv":           # S, dP, dV, dK
        return 8.0 * w.D * w.Hq * tp, "flop"
    if name == "trunk_dq":             # S, dP, dQ
        return 6.0 * w.D * w.Hq * tp, "flop"
    if name == "trunk_dq_ds":          # dQ from the stored dS blocks: read them and K~^T, write dQ
        n = (w.S + 31) // 32           # (plus, past pass 1, the branch epilogue's Q, dO and pass keys)
        ds_bytes = w.B * w.Hq * n * (n + 1) // 2 * 2048
        branch = T * 2 * row_q + (p - 1) * T * row_kv * 4 if p > 1 else 0
        return float(ds_bytes + T * row_q + T * row_kv + branch), "byte"
    if name == "branch_bwd":           # read Q, dO, LSE, Delta, (p-1) K, V; write (p-1) dK, dV
        return float(T * (2 * row_q + w.Hq * 8) + (p - 1) * T * row_kv * 4), "byte"
    if name == "prep_kv":              # read K, V (bf16); write rotated fp16 K~ rows and V^T
        return float(T * row_kv * 4), "byte"
    if name == "prep_kq":              # read K, Q; write K~ rows, K~^T and Q~ rows (fp16)
        return float(T * row_kv * 3 + T * row_q * 2), "byte"
    if name == "bwd_delta":
        return float(T * row_q * 2 + T * w.Hq * 4), "byte"
    return 0.0, "byte"


# ----------------------------------------------------------------------------- traffic from committed counters
def source_digest() -> str:
    """Digest of the HIP sources' code: comments and whitespace do not count, so a
    comment-only edit keeps the committed counter figures valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_ttt_attn_amd", "csrc")
    strip = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"', re.S)
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, fn)) as f:
                text = f.read()
            code = strip.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
            h.update(fn.encode() + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/<kernel>_<workload>_traffic.md, or None
    when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source digest:\s*`?([0-9a-f]+)", text)
    m_b = re.search(r"HBM bytes per launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def committed_kernel_time(kernel: str, workload: str):
    """Average launch duration (us) of `kernel` in the rocprofv3 kernel-trace summary
    profiles/kernels_<workload>.md, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"Source digest:\s*`?([0-9a-f]+)", text)
    m_t = re.search(r"^\|\s*" + re.escape(kernel) + r"\s*\|\s*\d+\s*\|\s*([0-9.]+)\s*\|", text, re.M)
    if not m_src or not m_t or m_src.group(1) != source_digest():
        return None
    return float(m_t.group(1))


# ----------------------------------------------------------------------------- CPU oracle baseline
def cpu_baseline(w, seconds: float):
    import numpy as np
    from threadpoolctl import threadpool_info

    import ttt_synth as syn
    from oracle import ttt_oracle as O

    p = w.K
    L = w.S if w.layout == "bshd" else w.lengths()[0]
    shp_q = (1, L, w.Hq, w.D)
    shp_kv = (1, L, w.Hkv, w.D)
    q = syn.draw(w, syn.KIND_Q, p, shp_q)
    ks = [syn.draw(w, syn.KIND_K, t, shp_kv) for t in range(1, p + 1)]
    vs = [syn.draw(w, syn.KIND_V, t, shp_kv) for t in range(1, p + 1)]
    do = syn.draw(w, syn.KIND_DO, p, shp_q)
    sl = O.Slice(0, 0, L)
    rng = np.random.default_rng(5)
    order = rng.permutation(L)
    r = w.Hq // w.Hkv
    done = 0
    flops = 0.0
    t0 = time.perf_counter()
    while done < L and time.perf_counter() - t0 < seconds:
        rows = np.sort(order[done: done + 64])
        O.fwd_group_rows(q, ks, vs, p, sl, 0, {h: rows for h in range(r)}, layout="bshd", Hq=w.Hq, Hkv=w.Hkv,
                         scale=w.scale, base=w.rope_base)
        O.bwd_rows(q, ks, vs, do, p, sl, 0, rows, layout="bshd", Hq=w.Hq, Hkv=w.Hkv, scale=w.scale,
                   base=w.rope_base)
        flops += 3.5 * 4.0 * w.D * r * float(np.sum(rows + p))
        done += len(rows)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} query rows x {r} heads of one KV group at pass {p} of {w.name} (sequence length {L}), "
                      f"forward + backward, {dt:.1f} s"}


# ----------------------------------------------------------------------------- main
def ring_main(args, w, dev):
    """Ring-step forward of pass K over a zig-zag ring of cp ranks (chunks of S/(2 cp) rows),
    emulated on one GPU: per chunk shape (diagonal step with the branch, full off-diagonal
    step, merge) and the whole ring against one whole-sequence call."""
    import torch

    import attention_ttt_attn_amd as tk
    import ttt_synth as syn

    cp, K = args.ring, w.K
    if w.layout == "thd":
        ring_thd_main(args, w, dev)
        return
    if w.layout != "bshd" or w.S % (2 * cp):
        print(f"--ring needs a BSHD workload whose length divides into {2 * cp} chunks", file=sys.stderr)
        sys.exit(2)
    c = w.S // (2 * cp)
    q = syn.draw_device(w, syn.KIND_Q, K, dev)
    ks = [syn.draw_device(w, syn.KIND_K, t, dev) for t in range(1, K + 1)]
    vs = [syn.draw_device(w, syn.KIND_V, t, dev) for t in range(1, K + 1)]
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    o_a = torch.empty((w.B, c, w.Hq, w.D), dtype=torch.float32, device=dev)
    l_a = torch.empty((w.B, w.Hq, c), dtype=torch.float32, device=dev)
    o_b, l_b = torch.empty_like(o_a), torch.empty_like(l_a)
    kw = dict(rope_base=w.rope_base, workspace=ws)

    def step(qc, kc, out, lse):
        qa, ka = qc * c, kc * c
        sk = [ks[0][:, ka:ka + c]] + [k[:, qa:qa + c] for k in ks[1:K]]
        sv = [vs[0][:, ka:ka + c]] + [v[:, qa:qa + c] for v in vs[1:K]]
        tk.fwd_chunk(q[:, qa:qa + c], sk, sv, K, q_offset=qa, kv_offset=ka, with_branch=qc == kc, out=out,
                     lse=lse, **kw)

    def ring():
        for r in range(cp):
            for qc in (r, 2 * cp - 1 - r):
                step(qc, 0, o_a, l_a)
                for kc in range(1, qc + 1):
                    step(qc, kc, o_b, l_b)
                    tk.merge(o_a, l_a, o_b, l_b, out=o_a, lse=l_a)

    o_s = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.float32, device=dev)
    l_s = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    single = lambda: tk.fwd(q, ks, vs, K, o_fp32=True, out=o_s, lse=l_s, **kw)
    # backward steps: the rows' whole-sequence O / LSE, dO
    o_b16, l_full = tk.fwd(q, ks, vs, K, rope_base=w.rope_base)
    do = syn.draw_device(w, syn.KIND_DO, K, dev)

    def bstep(qc, kc):
        qa, ka = qc * c, kc * c
        sk = [ks[0][:, ka:ka + c]] + [k[:, qa:qa + c] for k in ks[1:K]]
        sv = [vs[0][:, ka:ka + c]] + [v[:, qa:qa + c] for v in vs[1:K]]
        tk.bwd_chunk(q[:, qa:qa + c], sk, sv, o_b16[:, qa:qa + c], l_full[:, :, qa:qa + c], do[:, qa:qa + c], K,
                     q_offset=qa, kv_offset=ka, with_branch=qc == kc, rope_base=w.rope_base, workspace=ws)
    shapes = {
        "diag_step": lambda: step(cp, cp, o_a, l_a),
        "full_step": lambda: step(2 * cp - 1, 0, o_a, l_a),
        "merge": lambda: tk.merge(o_a, l_a, o_b, l_b, out=o_a, lse=l_a),
        "ring_total": ring,
        "single_call": single,
        "bwd_diag_step": lambda: bstep(cp, cp),
        "bwd_full_step": lambda: bstep(2 * cp - 1, 0),
    }
    n = max(args.steps, 1)
    res = {}
    for name, fn in shapes.items():
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"avg_us": round(e0.elapsed_time(e1) * 1e3 / n, 2)}
    per_head = 4.0 * w.D * w.Hq * w.B
    flops = {"diag_step": per_head * (c * (c + 1) // 2 + (K - 1) * c), "full_step": per_head * c * c,
             "ring_total": useful_flops(w, K)[0], "single_call": useful_flops(w, K)[0],
             "bwd_diag_step": 2.5 * per_head * (c * (c + 1) // 2 + (K - 1) * c), "bwd_full_step": 2.5 * per_head * c * c}
    for name, f in flops.items():
        res[name]["tflops"] = round(f / (res[name]["avg_us"] * 1e-6) / 1e12, 1)
    res["merge"]["gbps"] = round(w.B * c * w.Hq * (w.D * 4 * 3 + 12) / (res["merge"]["avg_us"] * 1e-6) / 1e9, 1)
    steps_per_ring = sum(qc + 1 for r in range(cp) for qc in (r, 2 * cp - 1 - r))
    out = {"metric": "ring-step forward time per chunk shape", "value": res["ring_total"]["avg_us"], "unit": "us",
           "higher_is_better": False, "n_gpus": 1, "steps": n, "warmup": args.warmup, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": w.name, "pass": K, "cp": cp, "chunk_rows": c, "ring_steps": steps_per_ring,
                      "merges": steps_per_ring - 2 * cp, "o": "fp32 partials, fp32 merge"},
           "shapes": res, "source_digest": source_digest()}
    print(json.dumps(out), flush=True)


def ring_thd_main(args, w, dev):
    """Packed (THD) ring steps of pass K: every sequence of the packed workload is cut into 2 cp
    chunks ([c L / 2cp, (c+1) L / 2cp)), and step (qc, kc) packs chunk qc's rows and chunk kc's
    keys of every sequence in one call.  The chunks' rows are gathered before the timed region
    (a ring rank holds its chunks contiguous)."""
    import numpy as np
    import torch

    import attention_ttt_attn_amd as tk
    import ttt_synth as syn

    cp, K = args.ring, w.K
    nc = 2 * cp
    lens = w.lengths()
    cu = syn.cu_seqlens_of(lens)
    q = syn.draw_device(w, syn.KIND_Q, K, dev)
    ks = [syn.draw_device(w, syn.KIND_K, t, dev) for t in range(1, K + 1)]
    vs = [syn.draw_device(w, syn.KIND_V, t, dev) for t in range(1, K + 1)]
    do = syn.draw_device(w, syn.KIND_DO, K, dev)
    gcu = torch.from_numpy(cu).to(dev)
    o_full, l_full = tk.fwd(q, ks, vs, K, cu_seqlens=gcu, rope_base=w.rope_base)
    span = lambda c: [(c * L // nc, (c + 1) * L // nc - c * L // nc) for L in lens]
    chunks = []
    for c in range(nc):
        sp = span(c)
        rows = torch.as_tensor(np.concatenate([np.arange(cu[s] + a, cu[s] + a + n) for s, (a, n) in enumerate(sp)]),
                               device=dev)
        i32 = lambda x: torch.as_tensor(np.asarray(x, np.int32), device=dev)
        chunks.append(dict(
            n=len(rows), cu=i32(np.concatenate([[0], np.cumsum([n for _, n in sp])])), off=i32([a for a, _ in sp]),
            q=q.index_select(0, rows), k=[t.index_select(0, rows) for t in ks], v=[t.index_select(0, rows) for t in vs],
            o=o_full.index_select(0, rows), lse=l_full.index_select(1, rows).contiguous(), do=do.index_select(0, rows),
            pairs=[(a, n) for a, n in sp]))
    ws = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    maxpos = max(lens) + K

    def args_of(qc, kc):
        a, b = chunks[qc], chunks[kc]
        sk = [b["k"][0]] + a["k"][1:K]
        sv = [b["v"][0]] + a["v"][1:K]
        geo = dict(cu_seqlens=a["cu"], kv_cu_seqlens=b["cu"], q_offsets=a["off"], kv_offsets=b["off"],
                   max_position=maxpos, with_branch=qc == kc, rope_base=w.rope_base, workspace=ws)
        return a, sk, sv, geo

    bufs = {}

    def step(qc, kc, slot):
        a, sk, sv, geo = args_of(qc, kc)
        key = (qc, slot)
        if key not in bufs:
            bufs[key] = (torch.empty((a["n"], w.Hq, w.D), dtype=torch.float32, device=dev),
                         torch.empty((w.Hq, a["n"]), dtype=torch.float32, device=dev))
        o_, l_ = bufs[key]
        tk.fwd_chunk(a["q"], sk, sv, K, out=o_, lse=l_, **geo)
        return o_, l_

    def ring():
        for r in range(cp):
            for qc in (r, nc - 1 - r):
                oa, la = step(qc, 0, 0)
                for kc in range(1, qc + 1):
                    ob, lb = step(qc, kc, 1)
                    tk.merge(oa, la, ob, lb, out=oa, lse=la, cu_seqlens=chunks[qc]["cu"])

    def bstep(qc, kc):
        a, sk, sv, geo = args_of(qc, kc)
        tk.bwd_chunk(a["q"], sk, sv, a["o"], a["lse"], a["do"], K, **geo)

    o_s = torch.empty(q.shape, dtype=torch.float32, device=dev)
    l_s = torch.empty(l_full.shape, dtype=torch.float32, device=dev)
    m_a = step(cp, cp, 0)
    m_b = step(cp, 0, 1)
    shapes = {
        "diag_step": lambda: step(cp, cp, 0),
        "full_step": lambda: step(nc - 1, 0, 0),
        "merge": lambda: tk.merge(m_a[0], m_a[1], m_b[0], m_b[1], out=m_a[0], lse=m_a[1], cu_seqlens=chunks[cp]["cu"]),
        "ring_total": ring,
        "single_call": lambda: tk.fwd(q, ks, vs, K, cu_seqlens=gcu, o_fp32=True, out=o_s, lse=l_s,
                                      rope_base=w.rope_base, workspace=ws),
        "bwd_diag_step": lambda: bstep(cp, cp),
        "bwd_full_step": lambda: bstep(nc - 1, 0),
    }
    n = max(args.steps, 1)
    res = {}
    for name, fn in shapes.items():
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"avg_us": round(e0.elapsed_time(e1) * 1e3 / n, 2)}
    per_head = 4.0 * w.D * w.Hq
    diag = sum(nq * (nq + 1) // 2 + (K - 1) * nq for _, nq in chunks[cp]["pairs"])
    full = sum(nq * nk for (_, nq), (_, nk) in zip(chunks[nc - 1]["pairs"], chunks[0]["pairs"]))
    flops = {"diag_step": per_head * diag, "full_step": per_head * full, "ring_total": useful_flops(w, K)[0],
             "single_call": useful_flops(w, K)[0], "bwd_diag_step": 2.5 * per_head * diag,
             "bwd_full_step": 2.5 * per_head * full}
    for name, f in flops.items():
        res[name]["tflops"] = round(f / (res[name]["avg_us"] * 1e-6) / 1e12, 1)
    res["merge"]["gbps"] = round(chunks[cp]["n"] * w.Hq * (w.D * 4 * 3 + 12) / (res["merge"]["avg_us"] * 1e-6) / 1e9, 1)
    steps_per_ring = sum(qc + 1 for r in range(cp) for qc in (r, nc - 1 - r))
    out = {"metric": "packed (THD) ring-step forward time per chunk shape", "value": res["ring_total"]["avg_us"],
           "unit": "us", "higher_is_better": False, "n_gpus": 1, "steps": n, "warmup": args.warmup, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": w.name, "pass": K, "cp": cp, "sequences": len(lens),
                      "chunk_rows_total": [c["n"] for c in chunks], "ring_steps": steps_per_ring,
                      "merges": steps_per_ring - nc, "o": "fp32 partials, fp32 merge"},
           "shapes": res, "source_digest": source_digest()}
    print(json.dumps(out), flush=True)


def block_thd_main(args, dev):
    """Packed (THD) block drafting, forward + backward: the 16 thd_32k sequences (T = 32768) as
    contexts, 64 blocks of 16 slots per sequence (16384 block rows), anchors uniform in each
    sequence's context.  Useful FLOPs as in the BSHD block bench."""
    import numpy as np
    import torch

    import attention_ttt_attn_amd as tk
    import ttt_synth as syn

    w = syn.workload("thd_32k")
    bs, nb, Hq, Hkv, D = 16, 64, w.Hq, w.Hkv, w.D
    ctx = w.lengths()
    ns = len(ctx)
    T, Tc = ns * nb * bs, sum(ctx)
    rng = np.random.default_rng(w.index)
    anchors = np.concatenate([np.sort(rng.integers(0, c + 1, nb)) for c in ctx]).astype(np.int32)
    q = syn.draw_device(w, syn.KIND_Q, 1, dev, (T, Hq, D))
    kb = syn.draw_device(w, syn.KIND_K, 2, dev, (T, Hkv, D))
    vb = syn.draw_device(w, syn.KIND_V, 2, dev, (T, Hkv, D))
    kc = syn.draw_device(w, syn.KIND_K, 1, dev, (Tc, Hkv, D))
    vc = syn.draw_device(w, syn.KIND_V, 1, dev, (Tc, Hkv, D))
    do = syn.draw_device(w, syn.KIND_DO, 1, dev, (T, Hq, D))
    cu = torch.as_tensor(np.arange(ns + 1, dtype=np.int32) * nb * bs, device=dev)
    ccu = torch.from_numpy(syn.cu_seqlens_of(ctx)).to(dev)
    ga = torch.from_numpy(anchors).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    grads = [torch.empty_like(t) for t in (q, kc, vc, kb, vb)]
    geo = dict(cu_seqlens=cu, ctx_cu_seqlens=ccu, rope_base=w.rope_base, workspace=ws)
    pairs = int((anchors.astype(np.int64) + bs).sum()) * bs     # per head (anchors lie inside their contexts)
    flops_f = 4.0 * D * Hq * pairs

    def run():
        tk.block_fwd(q, kc, vc, kb, vb, ga, bs, out=o, lse=lse, **geo)
        tk.block_bwd(q, kc, vc, kb, vb, ga, bs, o, lse, do, dq=grads[0], dk_ctx=grads[1], dv_ctx=grads[2],
                     dk_blk=grads[3], dv_blk=grads[4], **geo)
    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    events = []
    cur = torch.cuda.current_stream()

    def hook(name, phase, stream):
        s_ = cur if not stream or stream == cur.cuda_stream else torch.cuda.ExternalStream(stream)
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(s_)
        if phase == 0:
            events.append([name, ev, None])
        else:
            events[-1][2] = ev

    n = max(args.steps, 1)
    tk.set_trace_hook(hook)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    tk.set_trace_hook(None)
    call_ms = e0.elapsed_time(e1) / n
    ks = {}
    for name, a, b in events:
        k = ks.setdefault(name, [0, 0.0])
        k[0] += 1
        k[1] += a.elapsed_time(b)
    kern = {k: {"avg_us": round(v[1] * 1e3 / v[0], 2), "launches_per_call": v[0] // n} for k, v in ks.items()}
    fwd_us = kern["block_fwd"]["avg_us"]
    achieved = flops_f / (fwd_us * 1e-6)
    kern["block_fwd"]["tflops"] = round(achieved / 1e12, 1)
    ctx_pairs = int(anchors.astype(np.int64).sum()) * bs
    for name, f in (("block_dkdv_ctx", 8.0 * D * Hq * ctx_pairs), ("block_dq", 6.0 * D * Hq * pairs)):
        if name in kern:
            kern[name]["tflops"] = round(f / (kern[name]["avg_us"] * 1e-6) / 1e12, 1)
    value = 3.5 * flops_f / (call_ms * 1e-3) / 1e12
    out = {"metric": "packed (THD) block-draft attention fwd+bwd TFLOP/s (useful FLOPs)", "value": round(value, 2),
           "unit": "TFLOP/s", "frac_of_peak": round(value * 1e12 / PEAK_MFMA_BF16, 4),
           "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(call_ms, 4), "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "blk_thd_32k", "sequences": ns, "ctx_rows": Tc, "block_size": bs,
                      "blocks_per_sequence": nb, "block_rows": T, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                      "step": "forward then backward", "useful_tflop_per_step": round(3.5 * flops_f / 1e12, 4)},
           "roofline": {"kernel": "block_fwd", "bound": "mfma", "achieved": round(achieved / 1e12, 2),
                        "peak": 2500.0, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16, 4),
                        "traffic": None, "work_per_launch": flops_f, "avg_launch_us": fwd_us},
           "kernels": kern, "source_digest": source_digest()}
    print(json.dumps(out), flush=True)


def block_main(args, dev):
    """Block-draft forward + backward: 256 blocks of 16 slots per batch row over a 4096-token
    context (B=4, Hq=32, Hkv=8, D=128).  Useful FLOPs: forward 4*D per (slot, head, visible
    key), the visible keys of a slot being its block's context prefix plus the bs block
    keys; backward 2.5x that."""
    import numpy as np
    import torch

    import attention_ttt_attn_amd as tk
    import ttt_synth as syn

    bw = syn.BLOCK_WORKLOADS["blk_b4_c4k"]
    w = bw.as_workload()
    q = syn.draw_device(w, syn.KIND_Q, 1, dev, bw.q_shape())
    kc = syn.draw_device(w, syn.KIND_K, 1, dev, bw.ctx_shape())
    vc = syn.draw_device(w, syn.KIND_V, 1, dev, bw.ctx_shape())
    kb = syn.draw_device(w, syn.KIND_K, 2, dev, bw.blk_shape())
    vb = syn.draw_device(w, syn.KIND_V, 2, dev, bw.blk_shape())
    anchors = syn.block_anchors(bw.B, bw.nblk, bw.ctx_len, bw.index)
    ga = torch.from_numpy(anchors).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((bw.B, bw.Hq, bw.rows), dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    pairs = int((np.clip(anchors, 0, bw.ctx_len).astype(np.int64) + bw.bs).sum()) * bw.bs   # per head
    flops_f = 4.0 * bw.D * bw.Hq * pairs
    flops = 3.5 * flops_f
    do = syn.draw_device(w, syn.KIND_DO, 1, dev, bw.q_shape())
    grads = [torch.empty_like(t) for t in (q, kc, vc, kb, vb)]

    def run():
        tk.block_fwd(q, kc, vc, kb, vb, ga, bw.bs, rope_base=bw.rope_base, out=o, lse=lse, workspace=ws)
        tk.block_bwd(q, kc, vc, kb, vb, ga, bw.bs, o, lse, do, rope_base=bw.rope_base, dq=grads[0], dk_ctx=grads[1],
                     dv_ctx=grads[2], dk_blk=grads[3], dv_blk=grads[4], workspace=ws)
    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    events = []
    cur = torch.cuda.current_stream()

    def hook(name, phase, stream):
        s = cur if not stream or stream == cur.cuda_stream else torch.cuda.ExternalStream(stream)
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(s)
        if phase == 0:
            events.append([name, ev, None])
        else:
            events[-1][2] = ev

    n = max(args.steps, 1)
    tk.set_trace_hook(hook)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    tk.set_trace_hook(None)
    call_ms = e0.elapsed_time(e1) / n
    ks = {}
    for name, a, b in events:
        k = ks.setdefault(name, [0, 0.0])
        k[0] += 1
        k[1] += a.elapsed_time(b)
    kern = {k: {"avg_us": round(v[1] * 1e3 / v[0], 2), "launches_per_call": v[0] // n} for k, v in ks.items()}
    fwd_us = kern["block_fwd"]["avg_us"]
    achieved = flops_f / (fwd_us * 1e-6)
    kern["block_fwd"]["tflops"] = round(achieved / 1e12, 1)
    # dK/dV of the context keys: S, dP, dV, dK over the context pairs; dQ: S, dP, dQ over all pairs
    ctx_pairs = int(np.clip(anchors, 0, bw.ctx_len).astype(np.int64).sum()) * bw.bs
    for name, f in (("block_dkdv_ctx", 8.0 * bw.D * bw.Hq * ctx_pairs), ("block_dq", 6.0 * bw.D * bw.Hq * pairs)):
        if name in kern:
            kern[name]["tflops"] = round(f / (kern[name]["avg_us"] * 1e-6) / 1e12, 1)
    row_kv = bw.Hkv * bw.D * 2
    kern["prep_ctx"]["gbps"] = round(bw.B * bw.ctx_len * row_kv * 4 / (kern["prep_ctx"]["avg_us"] * 1e-6) / 1e9, 1)
    kern["prep_blk"]["gbps"] = round(bw.B * bw.rows * row_kv * 4 / (kern["prep_blk"]["avg_us"] * 1e-6) / 1e9, 1)
    value = flops / (call_ms * 1e-3) / 1e12
    out = {"metric": "block-draft attention fwd+bwd TFLOP/s (useful FLOPs)", "value": round(value, 2),
           "unit": "TFLOP/s", "frac_of_peak": round(value * 1e12 / PEAK_MFMA_BF16, 4),
           "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(call_ms, 4), "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": bw.name, "batch": bw.B, "ctx_len": bw.ctx_len, "block_size": bw.bs,
                      "blocks": bw.nblk, "q_heads": bw.Hq, "kv_heads": bw.Hkv, "head_dim": bw.D,
                      "step": "forward then backward", "useful_tflop_per_step": round(flops / 1e12, 4)},
           "roofline": {"kernel": "block_fwd", "bound": "mfma", "achieved": round(achieved / 1e12, 2),
                        "peak": 2500.0, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16, 4),
                        "traffic": None, "work_per_launch": flops_f, "avg_launch_us": fwd_us},
           "kernels": kern, "source_digest": source_digest()}
    print(json.dumps(out), flush=True)


def soft_ce_main(args, dev):
    """Per-pass soft cross-entropy over a K=7 unroll: pass p scores its student logits against the
    teacher rows p ahead.  HBM-bound: forward reads student + teacher once, backward reads them
    again and writes the gradient (algorithmic bytes, counted rows only for the reads)."""
    import torch

    import attention_ttt_attn_amd as tk

    B, S, V, K = 4, 4096, 32000, 7
    gen = torch.Generator(device=dev)
    gen.manual_seed(60)
    teacher = (torch.randn((B, S, V), generator=gen, device=dev) * 2).to(torch.bfloat16)
    students = [(torch.randn((B, S, V), generator=gen, device=dev) * 2).to(torch.bfloat16) for _ in range(K)]
    grads = [torch.empty_like(x) for x in students]
    dloss = torch.ones(1, device=dev)

    def step():
        for p in range(1, K + 1):
            stats, row_lse, _ = tk.soft_ce_fwd(students[p - 1], teacher, p)
            tk.soft_ce_bwd(students[p - 1], teacher, p, row_lse, stats, dloss, dstudent=grads[p - 1])

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    events = []
    cur = torch.cuda.current_stream()

    def hook(name, phase, stream):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(cur)
        if phase == 0:
            events.append([name, ev, None])
        else:
            events[-1][2] = ev

    n = max(args.steps, 1)
    tk.set_trace_hook(hook)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    tk.set_trace_hook(None)
    ms = e0.elapsed_time(e1) / n
    rows = sum(B * (S - p) for p in range(1, K + 1))
    fwd_bytes = rows * V * 2 * 2
    bwd_bytes = rows * V * 2 * 2 + B * S * V * 2 * K
    ks = {}
    for name, a, b in events:
        k = ks.setdefault(name, [0, 0.0])
        k[0] += 1
        k[1] += a.elapsed_time(b)
    kern = {k: {"avg_us": round(v[1] * 1e3 / v[0], 2)} for k, v in ks.items()}
    kern["soft_ce_fwd"]["gbps"] = round(fwd_bytes / K / (kern["soft_ce_fwd"]["avg_us"] * 1e-6) / 1e9, 1)
    kern["soft_ce_bwd"]["gbps"] = round(bwd_bytes / K / (kern["soft_ce_bwd"]["avg_us"] * 1e-6) / 1e9, 1)
    value = (fwd_bytes + bwd_bytes) / (ms * 1e-3) / 1e9
    bw_dom = kern["soft_ce_bwd"]["gbps"]
    out = {"metric": "per-pass soft cross-entropy fwd+bwd GB/s (algorithmic bytes)", "value": round(value, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "ce_b4_s4k_v32k", "batch": B, "seq_len": S, "vocab": V, "passes": K,
                      "teacher_offset": "p", "step": "fwd+bwd for p = 1..7"},
           "roofline": {"kernel": "soft_ce_bwd", "bound": "hbm", "achieved": bw_dom, "peak": 8000.0,
                        "unit": "GB/s", "frac": round(bw_dom / 8000.0, 4), "traffic": None,
                        "work_per_launch": bwd_bytes / K, "avg_launch_us": kern["soft_ce_bwd"]["avg_us"]},
           "kernels": kern, "source_digest": source_digest()}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} (WORLD_SIZE {world}) is not supported; "
              "the per-pass attention shards over (batch x KV-head group) with no exchange, so N GPUs "
              "would each run this benchmark on their own share.", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_ttt_attn_amd as tk
    import ttt_synth as syn

    tk.library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.block:
        block_main(args, dev)
        return
    if args.block_thd:
        block_thd_main(args, dev)
        return
    if args.soft_ce:
        soft_ce_main(args, dev)
        return
    global WINDOW
    WINDOW = max(0, args.window)
    w = syn.workload(args.workload)
    if args.head_dim:
        import dataclasses
        w = dataclasses.replace(w, D=args.head_dim, name=f"{w.name}_d{args.head_dim}")
    if args.ring:
        ring_main(args, w, dev)
        return
    K = w.K
    cu = torch.from_numpy(syn.cu_seqlens_of(w.lengths())).to(dev) if w.layout == "thd" else None

    q = {p: syn.draw_device(w, syn.KIND_Q, p, dev) for p in range(1, K + 1)}
    ks = [syn.draw_device(w, syn.KIND_K, t, dev) for t in range(1, K + 1)]
    vs = [syn.draw_device(w, syn.KIND_V, t, dev) for t in range(1, K + 1)]
    do = {p: syn.draw_device(w, syn.KIND_DO, p, dev) for p in range(1, K + 1)}
    o = {p: torch.empty_like(q[p]) for p in q}
    lse_shape = (w.Hq, w.S) if w.layout == "thd" else (w.B, w.Hq, w.S)
    lse = {p: torch.empty(lse_shape, dtype=torch.float32, device=dev) for p in q}
    dq = {p: torch.empty_like(q[p]) for p in q}
    dk = {p: [torch.empty_like(ks[0]) for _ in range(p)] for p in q}
    dv = {p: [torch.empty_like(vs[0]) for _ in range(p)] for p in q}
    d_f = tk.make_desc(q[K], ks, K, cu_seqlens=cu, rope_base=w.rope_base)
    ws_bytes = max(tk.workspace_bytes(d_f, False), tk.workspace_bytes(d_f, True))
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    kw = dict(cu_seqlens=cu, rope_base=w.rope_base, workspace=ws, window=WINDOW)
    kwb = dict(kw, stored_ds=args.bwd_stored_ds)

    def step():
        for p in range(1, K + 1):
            tk.fwd(q[p], ks, vs, p, out=o[p], lse=lse[p], **kw)
        for p in range(K, 0, -1):
            tk.bwd(q[p], ks, vs, o[p], lse[p], do[p], p, dq=dq[p], dks=dk[p], dvs=dv[p], **kwb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, per-kernel HIP events recorded on the launch stream
    events = []
    cur_pass = [0]

    cur = torch.cuda.current_stream()

    def hook(name, phase, stream):
        # record on the stream the library launches this kernel on (it may be
        # the library's side stream rather than the caller's)
        s = cur if not stream or stream == cur.cuda_stream else torch.cuda.ExternalStream(stream)
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(s)
        if phase == 0:
            events.append([name, cur_pass[0], ev, None])
        else:
            events[-1][3] = ev

    if not args.no_kernel_times:
        tk.set_trace_hook(hook)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        for p in range(1, K + 1):
            cur_pass[0] = p
            tk.fwd(q[p], ks, vs, p, out=o[p], lse=lse[p], **kw)
        for p in range(K, 0, -1):
            cur_pass[0] = p
            tk.bwd(q[p], ks, vs, o[p], lse[p], do[p], p, dq=dq[p], dks=dk[p], dvs=dv[p], **kwb)
    end.record()
    torch.cuda.synchronize()
    tk.set_trace_hook(None)
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps

    flops_step = sum(sum(useful_flops(w, p)) for p in range(1, K + 1))
    fwd_flops_step = sum(useful_flops(w, p)[0] for p in range(1, K + 1))
    value = flops_step / (ms_step * 1e-3) / 1e12

    # per-kernel statistics
    kstats = {}
    for name, p, e0, e1 in events:
        dt = e0.elapsed_time(e1)
        work, unit = kernel_work(w, name, p)
        s = kstats.setdefault(name, {"launches": 0, "ms": 0.0, "work": 0.0, "unit": unit})
        s["launches"] += 1
        s["ms"] += dt
        s["work"] += work
    by_pass = {}
    for name, p, e0, e1 in events:
        if name == "trunk_fwd":
            by_pass.setdefault(p, []).append(e0.elapsed_time(e1))
    kernels = {}
    for name, s in sorted(kstats.items(), key=lambda kv: -kv[1]["ms"]):
        avg_ms = s["ms"] / s["launches"]
        rate = s["work"] / (s["ms"] * 1e-3) if s["ms"] > 0 else 0.0
        ent = {"avg_us": round(avg_ms * 1e3, 2), "ms_per_step": round(s["ms"] / args.steps, 4),
               "launches_per_step": s["launches"] // args.steps}
        if s["unit"] == "flop":
            ent["tflops"] = round(rate / 1e12, 1)
            ent["frac_of_peak"] = round(rate / PEAK_MFMA_BF16, 4)
        elif s["work"] > 0:
            ent["gbps"] = round(rate / 1e9, 1)
            ent["frac_of_peak"] = round(rate / PEAK_HBM, 4)
        kernels[name] = ent
    if by_pass:
        kernels["trunk_fwd"]["avg_us_by_pass"] = {str(p): round(1e3 * sum(v) / len(v), 2)
                                                  for p, v in sorted(by_pass.items())}

    # the committed profiles cover the default configuration of each workload:
    # their kernel times and traffic are attached only to a run of that configuration
    profiled_cfg = args.window == 0 and not args.bwd_stored_ds and args.head_dim in (0, 128)
    roofline = None
    if kstats:
        dom = max(kstats, key=lambda n: kstats[n]["ms"])
        s = kstats[dom]
        per_launch = s["work"] / s["launches"]
        avg_s = s["ms"] / s["launches"] * 1e-3
        achieved = per_launch / avg_s
        mfma = s["unit"] == "flop"
        roofline = {"kernel": dom, "bound": "mfma" if mfma else "hbm",
                    "achieved": round(achieved / (1e12 if mfma else 1e9), 2),
                    "peak": 2500.0 if mfma else 8000.0, "unit": "TFLOP/s" if mfma else "GB/s",
                    "frac": round(achieved / (PEAK_MFMA_BF16 if mfma else PEAK_HBM), 4),
                    "traffic": committed_traffic(dom, w.name) if profiled_cfg else None,
                    "work_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 2),
                    "profile_avg_launch_us": committed_kernel_time(dom, w.name) if profiled_cfg else None}
    # the trunk forward alone against the 45% of bf16 peak bar
    gate = None
    if "trunk_fwd" in kstats:
        s = kstats["trunk_fwd"]
        rate = s["work"] / (s["ms"] * 1e-3)
        gate = {"kernel": "trunk_fwd", "achieved": round(rate / 1e12, 2), "unit": "TFLOP/s",
                "frac": round(rate / PEAK_MFMA_BF16, 4), "bar": 0.45,
                "avg_launch_us": round(s["ms"] / s["launches"] * 1e3, 2),
                "profile_avg_launch_us": committed_kernel_time("trunk_fwd", w.name) if profiled_cfg else None}

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # sanity: the outputs are finite
    assert all(torch.isfinite(o[p]).all().item() and torch.isfinite(dq[p]).all().item() for p in q)

    out = {
        "metric": "TTT attn fwd+bwd TFLOP/s (causal useful FLOPs) and % of MI355X bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "frac_of_peak": round(value * 1e12 / PEAK_MFMA_BF16, 4),
        "config": {"workload": w.name, "layout": w.layout, "batch": w.B, "seq_len": w.S, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "passes": K, "rope_base": w.rope_base,
                   "step": f"fwd p=1..{K} then bwd p={K}..1", "useful_tflop_per_step": round(flops_step / 1e12, 4),
                   "fwd_useful_tflop_per_step": round(fwd_flops_step / 1e12, 4),
                   "mfma_operands": "fp16 Q~K~^T and dS, bf16 P.V, dO.V, P^T.dO; fp32 accumulate",
                   "parallelism": "single GPU", "window": WINDOW,
                   "bwd": "stored dS" if args.bwd_stored_ds else "recompute"},
        "roofline": roofline,
        "gate": gate,
        "kernels": kernels,
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
