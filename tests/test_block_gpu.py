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
from ttt_cases import TOL, bf16_half_ulp, max_abs, to_np

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
