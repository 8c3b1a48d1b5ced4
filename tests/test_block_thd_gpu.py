"""Packed (THD) block drafting on the GPU (through the C ABI) against the fp64 oracle.

Each sequence holds whole blocks of bs slots and has its own context; a block's
anchor clamps to its own sequence's context, and sequences never see each
other.  The cases mix sequences with long, short and empty contexts, a
context without block rows, out-of-range and repeated anchors, and the three
workgroup shapes the head ratio selects; every element of O, LSE and the five
gradients is compared with the oracle's packed block drafting.
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


class ThdBlock:
    """Packed block rows / contexts: seqs = [(blocks, context rows)]."""

    def __init__(self, dev, seqs, bs, Hq, Hkv, seed, base=1e6, D=128):
        rng = np.random.default_rng(seed)
        self.bs, self.base = bs, base
        self.cu = np.concatenate([[0], np.cumsum([n * bs for n, _ in seqs])]).astype(np.int32)
        self.ccu = np.concatenate([[0], np.cumsum([c for _, c in seqs])]).astype(np.int32)
        T, Tc = int(self.cu[-1]), int(self.ccu[-1])
        draw = lambda shape: syn.round_bf16(rng.standard_normal(shape).astype(np.float32))
        self.q, self.kb, self.vb = draw((T, Hq, D)), draw((T, Hkv, D)), draw((T, Hkv, D))
        self.kc, self.vc = draw((Tc, Hkv, D)), draw((Tc, Hkv, D))
        self.do = draw((T, Hq, D))
        anchors = []
        for n, c in seqs:
            a = rng.integers(0, c + 1, n)
            if n >= 4:
                a[0], a[1], a[2], a[3] = 0, c, c + 7, -3     # no context, all of it, past it, negative
            if n >= 6:
                a[5] = a[4]                                  # a repeated anchor
            anchors.append(a)
        self.anchors = np.concatenate(anchors + [np.zeros(0, np.int64)]).astype(np.int32)
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
        self.gq, self.gkb, self.gvb, self.gkc, self.gvc, self.gdo = map(up, (self.q, self.kb, self.vb, self.kc,
                                                                             self.vc, self.do))
        self.ga = torch.from_numpy(self.anchors).to(dev)
        self.gcu = torch.from_numpy(self.cu).to(dev)
        self.gccu = torch.from_numpy(self.ccu).to(dev)

    def geo(self):
        return dict(cu_seqlens=self.gcu, ctx_cu_seqlens=self.gccu, rope_base=self.base, check_cu_seqlens=True)

    def oracle_geo(self):
        return dict(cu_seqlens=self.cu, ctx_cu_seqlens=self.ccu, base=self.base)


SEQS = [(3, 300), (1, 0), (7, 65), (0, 100), (12, 1000), (2, 5), (5, 129)]


@pytest.mark.parametrize("bs,Hq,Hkv", [(16, 8, 2), (8, 4, 2), (4, 2, 2), (32, 8, 2)])
def test_thd_block_fwd_bwd(dev, tk, bs, Hq, Hkv):
    inp = ThdBlock(dev, SEQS, bs, Hq, Hkv, 70 + bs)
    o_ref, l_ref = O.block_fwd_thd(inp.q, inp.kc, inp.vc, inp.kb, inp.vb, inp.anchors, bs, **inp.oracle_geo())
    for o_fp32 in (True, False):
        o, lse = tk.block_fwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, bs, o_fp32=o_fp32, **inp.geo())
        torch.cuda.synchronize()
        og, lg = to_np(o), to_np(lse)
        eo = np.abs(og - o_ref)
        if not o_fp32:
            eo = eo - bf16_half_ulp(o_ref)
        el = max_abs(lg, l_ref)
        print(f"thd block bs={bs} {Hq}/{Hkv} o_fp32={o_fp32}: O {eo.max():.3e} LSE {el:.3e}")
        assert np.all(np.isfinite(og)) and eo.max() <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
    grads = tk.block_bwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, bs, o, lse, inp.gdo, **inp.geo())
    torch.cuda.synchronize()
    ref = O.block_bwd_thd(inp.q, inp.kc, inp.vc, inp.kb, inp.vb, inp.anchors, bs, inp.do, **inp.oracle_geo())
    names = ["dq", "dk_ctx", "dv_ctx", "dk_blk", "dv_blk"]
    errs = {n: rel_fro(to_np(g), r) for n, g, r in zip(names, grads, ref)}
    print(f"thd block bs={bs} bwd: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL["bf16"]["grad"], errs
    # the context of the sequence without block rows gets exact zeros
    a, e = int(inp.ccu[3]), int(inp.ccu[4])
    assert not to_np(grads[1])[a:e].any() and not to_np(grads[2])[a:e].any()


def test_thd_block_equals_bshd(dev, tk):
    """Equal sequences packed as THD give the BSHD call's results."""
    bs, nblk, ctx, B = 16, 9, 200, 3
    inp = ThdBlock(dev, [(nblk, ctx)] * B, bs, 8, 2, 75)
    as_b = lambda t: t.reshape(B, t.shape[0] // B, *t.shape[1:])
    o_t, l_t = tk.block_fwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, bs, o_fp32=True, **inp.geo())
    o_b, l_b = tk.block_fwd(as_b(inp.gq), as_b(inp.gkc), as_b(inp.gvc), as_b(inp.gkb), as_b(inp.gvb),
                            inp.ga.reshape(B, nblk), bs, o_fp32=True, rope_base=inp.base)
    g_t = tk.block_bwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, bs, o_t.to(torch.bfloat16), l_t, inp.gdo,
                       **inp.geo())
    g_b = tk.block_bwd(as_b(inp.gq), as_b(inp.gkc), as_b(inp.gvc), as_b(inp.gkb), as_b(inp.gvb),
                       inp.ga.reshape(B, nblk), bs, as_b(o_t.to(torch.bfloat16)), l_b, as_b(inp.gdo),
                       rope_base=inp.base)
    torch.cuda.synchronize()
    assert torch.equal(as_b(o_t), o_b) and torch.equal(l_t, l_b.permute(1, 0, 2).reshape(l_t.shape))
    for x, y in zip(g_t, g_b):
        assert torch.equal(as_b(x), y)
    print("THD block drafting over equal sequences == BSHD, bitwise (forward and backward)")


def test_thd_block_rejects_partial_blocks(dev, tk):
    inp = ThdBlock(dev, [(2, 50), (3, 20)], 16, 8, 2, 76)
    bad = inp.gcu.clone()
    bad[1] += 8                                   # sequence 0 no longer holds whole blocks
    with pytest.raises(tk.TTTAttnError, match="whole blocks"):
        tk.block_fwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, 16, cu_seqlens=bad,
                     ctx_cu_seqlens=inp.gccu, rope_base=inp.base, check_cu_seqlens=True)


def test_thd_block_fullsize(dev, tk):
    """The packed block-draft bench shape (the 16 thd_32k sequences as contexts, 64 blocks of 16 slots
    each, 16384 block rows, 32/8 heads): O and LSE against the oracle on >= 4096 sampled rows, and the
    context dK/dV of one whole sequence and KV head (every block row that sees it) plus dQ on the
    sampled rows' heads against the oracle."""
    w = syn.workload("thd_32k")
    ctx = w.lengths()
    inp = ThdBlock(dev, [(64, c) for c in ctx], 16, w.Hq, w.Hkv, 77)
    o, lse = tk.block_fwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, 16, o_fp32=True, **inp.geo())
    grads = tk.block_bwd(inp.gq, inp.gkc, inp.gvc, inp.gkb, inp.gvb, inp.ga, 16, o.to(torch.bfloat16), lse, inp.gdo,
                         **inp.geo())
    torch.cuda.synchronize()
    og, lg = to_np(o), to_np(lse)
    rng = np.random.default_rng(78)
    eo = el = 0.0
    n = 0
    bs = 16
    for s in range(len(ctx)):
        a, e, ca, ce = int(inp.cu[s]), int(inp.cu[s + 1]), int(inp.ccu[s]), int(inp.ccu[s + 1])
        sub = lambda x: x[None]
        for h in rng.choice(w.Hq, 4, replace=False):
            rows = np.unique(np.concatenate([rng.integers(0, e - a, 72), [0, bs - 1, e - a - 1]]))
            o_ref, l_ref = O.block_fwd_rows(sub(inp.q[a:e]), sub(inp.kc[ca:ce]), sub(inp.vc[ca:ce]), sub(inp.kb[a:e]),
                                            sub(inp.vb[a:e]), inp.anchors[None, a // bs:e // bs], bs, 0, int(h), rows,
                                            base=inp.base)
            eo = max(eo, max_abs(og[a + rows, h], o_ref))
            el = max(el, max_abs(lg[h, a + rows], l_ref))
            n += len(rows)
    print(f"blk_thd_32k: {n} sampled rows, O max-abs {eo:.3e} LSE max-abs {el:.3e}")
    assert n >= 4096 and eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
    # one whole (sequence, KV head): context dK/dV from every row of its 64 blocks (4 heads), and dQ
    s, g = int(np.argmax(ctx)), 3
    a, e, ca, ce = int(inp.cu[s]), int(inp.cu[s + 1]), int(inp.ccu[s]), int(inp.ccu[s + 1])
    r = w.Hq // w.Hkv
    dkc = np.zeros((ce - ca, w.D))
    dvc = np.zeros((ce - ca, w.D))
    dqs, dqr = [], []
    for hh in range(g * r, (g + 1) * r):
        dq_, dkc_, dvc_, _, _ = O.block_bwd_rows(inp.q[None, a:e], inp.kc[None, ca:ce], inp.vc[None, ca:ce],
                                                 inp.kb[None, a:e], inp.vb[None, a:e],
                                                 inp.anchors[None, a // bs:e // bs], bs, inp.do[None, a:e], 0, hh,
                                                 np.arange(e - a), base=inp.base)
        dkc += dkc_
        dvc += dvc_
        dqs.append(to_np(grads[0])[a:e, hh])
        dqr.append(dq_)
    e_k = rel_fro(to_np(grads[1])[ca:ce, g], dkc)
    e_v = rel_fro(to_np(grads[2])[ca:ce, g], dvc)
    e_q = rel_fro(np.stack(dqs), np.stack(dqr))
    print(f"blk_thd_32k bwd vs oracle, sequence {s} (context {ce - ca}) KV head {g}: dK_ctx {e_k:.2e} "
          f"dV_ctx {e_v:.2e} dQ {e_q:.2e}")
    assert max(e_k, e_v, e_q) <= TOL["bf16"]["grad"]
