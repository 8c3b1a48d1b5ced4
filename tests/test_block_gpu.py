"""GPU parity of ttt_attn_block_fwd (block-draft attention) against the fp64 oracle.

Blocks of bs slots anchored in a context: every slot sees the context keys
before its block's anchor and all keys of its own block.  Small cases compare
every element (ragged row counts, every block size, the three workgroup
shapes the head ratio selects, anchors at 0 and at the context end, repeated,
unsorted and out-of-range anchors, an empty context); the full-size case
compares >= 4096 sampled rows.
"""
import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import TOL, bf16_half_ulp, max_abs, rel_fro, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def tk():
    import attention_ttt_attn_amd as m
    m.library()
    return m


class BlockInputs:
    def __init__(self, bw: syn.BlockWorkload, dev, anchors=None):
        w = bw.as_workload()
        self.bw = bw
        self.q = syn.draw(w, syn.KIND_Q, 1, bw.q_shape())
        self.kc = syn.draw(w, syn.KIND_K, 1, bw.ctx_shape())
        self.vc = syn.draw(w, syn.KIND_V, 1, bw.ctx_shape())
        self.kb = syn.draw(w, syn.KIND_K, 2, bw.blk_shape())
        self.vb = syn.draw(w, syn.KIND_V, 2, bw.blk_shape())
        self.anchors = (syn.block_anchors(bw.B, bw.nblk, bw.ctx_len, bw.index) if anchors is None
                        else np.asarray(anchors, dtype=np.int32))
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
        self.gq, self.gkc, self.gvc, self.gkb, self.gvb = map(up, (self.q, self.kc, self.vc, self.kb, self.vb))
        self.ga = torch.from_numpy(self.anchors).to(dev)

    def run(self, tk, o_fp32):
        o, lse = tk.block_fwd(self.gq, self.gkc, self.gvc, self.gkb, self.gvb, self.ga, self.bw.bs,
                              rope_base=self.bw.rope_base, o_fp32=o_fp32)
        torch.cuda.synchronize()
        return to_np(o), to_np(lse)


def check_full(tk, inp, label):
    bw = inp.bw
    o_ref, l_ref = O.block_fwd(inp.q, inp.kc, inp.vc, inp.kb, inp.vb, inp.anchors, bw.bs, base=bw.rope_base)
    for o_fp32 in (True, False):
        og, lg = inp.run(tk, o_fp32)
        eo = np.abs(og - o_ref)
        if not o_fp32:
            eo = eo - bf16_half_ulp(o_ref)
        el = max_abs(lg, l_ref)
        print(f"{label} o_fp32={o_fp32}: O max-abs {eo.max():.3e} LSE max-abs {el:.3e}")
        assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
        assert eo.max() <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


def edge_anchors(B, nblk, ctx_len, seed):
    a = syn.block_anchors(B, nblk, ctx_len, seed)
    a[:, 0] = 0                          # no context
    a[:, -1] = ctx_len                   # the whole context
    if nblk > 3:
        a[:, 2] = a[:, 1]                # a repeated anchor
    return np.sort(a, axis=1)


@pytest.mark.parametrize("bs,nblk,Hq,Hkv", [(1, 77, 8, 2), (4, 37, 8, 2), (16, 9, 8, 2), (32, 5, 8, 2),
                                            (8, 19, 4, 2), (2, 70, 2, 2)])
def test_block_small(dev, tk, bs, nblk, Hq, Hkv):
    # row counts 77..160: ragged last work item; head ratios 4, 2, 1 select 32-, 64- and 128-row work items
    bw = syn.BlockWorkload(f"blk_small_{bs}", 31, 2, 300, bs, nblk, Hq, Hkv, 128, "bf16", 1e6)
    inp = BlockInputs(bw, dev, edge_anchors(2, nblk, 300, 31 + bs))
    check_full(tk, inp, f"bs={bs} nblk={nblk} Hq={Hq} Hkv={Hkv}")


def test_block_unsorted_and_clamped_anchors(dev, tk):
    bw = syn.BlockWorkload("blk_unsorted", 32, 1, 200, 8, 12, 8, 2, 128, "bf16", 1e4)
    anchors = np.array([[150, 3, 200, -5, 77, 77, 0, 260, 1, 199, 64, 128]], dtype=np.int32)
    check_full(tk, BlockInputs(bw, dev, anchors), "unsorted/clamped")


def test_block_empty_context(dev, tk):
    bw = syn.BlockWorkload("blk_noctx", 33, 2, 0, 16, 6, 8, 2, 128, "bf16", 1e6)
    check_full(tk, BlockInputs(bw, dev, np.zeros((2, 6), dtype=np.int32)), "empty context")


def test_block_fullsize(dev, tk):
    """256 blocks of 16 slots over a 4096-token context, B=4, Hq=32, Hkv=8: >= 4096
    sampled rows (plus the first and last slot of the first, middle and last block)."""
    bw = syn.BLOCK_WORKLOADS["blk_b4_c4k"]
    inp = BlockInputs(bw, dev)
    og, lg = inp.run(tk, True)
    rng = np.random.default_rng(34)
    N = bw.rows
    eo = el = 0.0
    n = 0
    forced = [0, bw.bs - 1, N // 2, N // 2 + bw.bs - 1, N - bw.bs, N - 1]
    for b in range(bw.B):
        for h in range(bw.Hq):
            rows = np.unique(np.concatenate([rng.integers(0, N, 32), forced]))
            o_ref, l_ref = O.block_fwd_rows(inp.q, inp.kc, inp.vc, inp.kb, inp.vb, inp.anchors, bw.bs, b, h, rows,
                                            base=bw.rope_base)
            eo = max(eo, max_abs(og[b, rows, h], o_ref))
            el = max(el, max_abs(lg[b, h, rows], l_ref))
            n += len(rows)
    print(f"blk_b4_c4k: {n} sampled rows, O max-abs {eo:.3e} LSE max-abs {el:.3e}")
    assert n >= 4096
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


# ----------------------------------------------------------------------------- backward
def run_bwd(tk, inp, dout_np, o_fp32=False):
    bw = inp.bw
    gdo = torch.from_numpy(np.ascontiguousarray(dout_np)).to(inp.gq.device).to(torch.bfloat16)
    o, lse = tk.block_fwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, bw.bs, rope_base=bw.rope_base,
                          o_fp32=o_fp32)
    grads = tk.block_bwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, bw.bs, o, lse, gdo,
                         rope_base=bw.rope_base)
    torch.cuda.synchronize()
    return [to_np(t) for t in grads]


def draw_dout(bw):
    return syn.draw(bw.as_workload(), syn.KIND_DO, 1, bw.q_shape())


BWD_NAMES = ("dq", "dk_ctx", "dv_ctx", "dk_blk", "dv_blk")


def check_bwd_full(tk, inp, label):
    bw = inp.bw
    do = draw_dout(bw)
    got = run_bwd(tk, inp, do)
    ref = O.block_bwd(inp.q, inp.kc, inp.vc, inp.kb, inp.vb, inp.anchors, bw.bs, do, base=bw.rope_base)
    for name, gg, rr in zip(BWD_NAMES, got, ref):
        if rr.size == 0:
            continue
        e = rel_fro(gg, rr)
        print(f"{label} {name}: rel Frobenius {e:.3e}")
        assert np.all(np.isfinite(gg)) and e <= TOL["bf16"]["grad"], name


@pytest.mark.parametrize("bs,nblk,Hq,Hkv", [(1, 77, 8, 2), (4, 37, 8, 2), (16, 9, 8, 2), (32, 5, 8, 2),
                                            (8, 19, 4, 2), (2, 70, 2, 2)])
def test_block_bwd_small(dev, tk, bs, nblk, Hq, Hkv):
    bw = syn.BlockWorkload(f"blkb_small_{bs}", 35, 2, 300, bs, nblk, Hq, Hkv, 128, "bf16", 1e6)
    inp = BlockInputs(bw, dev, edge_anchors(2, nblk, 300, 35 + bs))
    check_bwd_full(tk, inp, f"bwd bs={bs} nblk={nblk} Hq={Hq} Hkv={Hkv}")


def test_block_bwd_unsorted_and_empty_context(dev, tk):
    bw = syn.BlockWorkload("blkb_unsorted", 36, 1, 200, 8, 12, 8, 2, 128, "bf16", 1e4)
    anchors = np.array([[150, 3, 200, -5, 77, 77, 0, 260, 1, 199, 64, 128]], dtype=np.int32)
    check_bwd_full(tk, BlockInputs(bw, dev, anchors), "bwd unsorted/clamped")
    bw0 = syn.BlockWorkload("blkb_noctx", 37, 2, 0, 16, 6, 8, 2, 128, "bf16", 1e6)
    check_bwd_full(tk, BlockInputs(bw0, dev, np.zeros((2, 6), dtype=np.int32)), "bwd empty context")


def test_block_bwd_fullsize(dev, tk):
    """blk_b4_c4k backward, checked where the oracle's values are exact from a subset of
    rows: dQ of sampled rows; dK/dV of whole blocks (all their slots, all heads of the
    group); context dK/dV of the keys past the anchor of the 8th-last block (seen only
    by the last 8 blocks' rows)."""
    bw = syn.BLOCK_WORKLOADS["blk_b4_c4k"]
    inp = BlockInputs(bw, dev)
    do = draw_dout(bw)
    dq, dkc, dvc, dkb, dvb = run_bwd(tk, inp, do)
    rng = np.random.default_rng(38)
    r = bw.Hq // bw.Hkv
    N = bw.rows
    acc = {k: ([], []) for k in BWD_NAMES}
    nrows = 0
    for b in range(bw.B):
        for g in range(bw.Hkv):
            blocks = np.unique(np.concatenate([rng.integers(0, bw.nblk, 2), [bw.nblk - 1]]))
            tail0 = bw.nblk - 8
            rows = np.unique(np.concatenate([np.arange(n * bw.bs, (n + 1) * bw.bs) for n in blocks] +
                                            [np.arange(tail0 * bw.bs, N)]))
            j0 = int(np.clip(inp.anchors[b, tail0 - 1], 0, bw.ctx_len))   # keys >= j0: last 8 blocks only
            sk = np.zeros((bw.ctx_len, bw.D)), np.zeros((bw.ctx_len, bw.D))
            sb = np.zeros((N, bw.D)), np.zeros((N, bw.D))
            for h in range(g * r, (g + 1) * r):
                q_, kc_, vc_, kb_, vb_ = O.block_bwd_rows(inp.q, inp.kc, inp.vc, inp.kb, inp.vb, inp.anchors, bw.bs,
                                                          do, b, h, rows, base=bw.rope_base)
                acc["dq"][0].append(dq[b, rows, h])
                acc["dq"][1].append(q_)
                sk[0][:] += kc_
                sk[1][:] += vc_
                sb[0][:] += kb_
                sb[1][:] += vb_
                nrows += len(rows)
            brow = np.concatenate([np.arange(n * bw.bs, (n + 1) * bw.bs) for n in blocks])
            acc["dk_blk"][0].append(dkb[b, brow, g]); acc["dk_blk"][1].append(sb[0][brow])
            acc["dv_blk"][0].append(dvb[b, brow, g]); acc["dv_blk"][1].append(sb[1][brow])
            acc["dk_ctx"][0].append(dkc[b, j0:, g]); acc["dk_ctx"][1].append(sk[0][j0:])
            acc["dv_ctx"][0].append(dvc[b, j0:, g]); acc["dv_ctx"][1].append(sk[1][j0:])
    assert nrows >= 4096
    for name in BWD_NAMES:
        e = rel_fro(np.concatenate(acc[name][0]), np.concatenate(acc[name][1]))
        print(f"blk_b4_c4k bwd {name}: rel Frobenius {e:.3e} over sampled rows/keys")
        assert e <= TOL["bf16"]["grad"], name
