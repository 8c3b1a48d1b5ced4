"""GPU parity of ttt_attn_fwd against the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import TOL, Inputs, bf16_half_ulp, lse_at, max_abs, rel_fro, row_at, sample_rows, to_np

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


def full_check(tk, inp, p, o_fp32, label):
    w = inp.w
    kw = inp.kw()
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=o_fp32, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout=w.layout, cu_seqlens=inp.cu_host, base=w.rope_base)
    og, lg = to_np(o), to_np(lse)
    tol = TOL[w.dtype]
    eo = np.abs(og - o_ref)
    if not o_fp32 and w.dtype == "bf16":
        eo = eo - bf16_half_ulp(o_ref)
    el = max_abs(lg, l_ref)
    print(f"{label} p={p} o_fp32={o_fp32}: O max-abs {eo.max():.3e} LSE max-abs {el:.3e}")
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    assert eo.max() <= tol["o"], f"O error {eo.max()}"
    assert el <= tol["lse"], f"LSE error {el}"


def test_tiny_fp32_forward_all_passes(dev, tk):
    w = syn.workload("tiny_fp32")
    inp = Inputs(w, dev, with_grad=False)
    for p in range(1, w.K + 1):
        full_check(tk, inp, p, True, "tiny_fp32")


@pytest.mark.parametrize("p", [1, 2, 5])
def test_bf16_bshd_small(dev, tk, p):
    # two batches of 300 rows: 3 query tiles with a ragged tail, GQA 4:1
    w = syn.Workload("bshd_small", 11, "bshd", 2, 300, 8, 2, 128, 5, "bf16", 1e6, False)
    inp = Inputs(w, dev, with_grad=False)
    full_check(tk, inp, p, True, "bshd_small")
    full_check(tk, inp, p, False, "bshd_small")


@pytest.mark.parametrize("p", [1, 3])
def test_bf16_thd_small(dev, tk, p):
    lens = [1, 63, 64, 65, 200, 129, 3, 130]
    w = syn.Workload("thd_small", 12, "thd", 1, sum(lens), 4, 1, 128, 3, "bf16", 1e4, False)
    inp = Inputs(w, dev, with_grad=False, lengths=lens)
    full_check(tk, inp, p, True, "thd_small")
    full_check(tk, inp, p, False, "thd_small")


def test_bf16_no_rope_and_custom_scale(dev, tk):
    w = syn.Workload("norope", 13, "bshd", 1, 130, 2, 2, 128, 3, "bf16", 0.0, False)
    inp = Inputs(w, dev, with_grad=False)
    o, lse = tk.fwd(inp.gq[3], inp.gk, inp.gv, 3, softmax_scale=0.05, o_fp32=True)
    o_ref, l_ref = O.fwd(inp.q[3], inp.k, inp.v, 3, layout="bshd", scale=0.05, base=0.0)
    assert max_abs(to_np(o), o_ref) <= 1e-2 and max_abs(to_np(lse), l_ref) <= 2e-3


def sampled_fwd_check(tk, inp, n_rows, seed, o_fp32=True):
    w = inp.w
    passes = range(1, w.K + 1)
    rows = sample_rows(inp, n_rows, seed, passes)
    outs = {}
    for p in passes:
        o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=o_fp32, **inp.kw())
        torch.cuda.synchronize()
        outs[p] = (to_np(o), to_np(lse))
    slices = inp.slices()
    eo = el = 0.0
    n = 0
    for (p, s, h), rr in rows.items():
        sl = slices[s]
        o_ref, l_ref = O.fwd_rows(inp.q[p], inp.k, inp.v, p, sl, h, rr, layout=w.layout, Hq=w.Hq, Hkv=w.Hkv,
                                  scale=w.scale, base=w.rope_base)
        og = row_at(outs[p][0], w.layout, sl, h, rr)
        lg = lse_at(outs[p][1], w.layout, sl, h, rr)
        e = np.abs(og - o_ref)
        if not o_fp32:
            e = e - bf16_half_ulp(o_ref)
        eo = max(eo, float(e.max()))
        el = max(el, max_abs(lg, l_ref))
        n += len(rr)
    print(f"{w.name}: {n} sampled rows, O max-abs {eo:.3e}, LSE max-abs {el:.3e}")
    assert n >= n_rows
    assert eo <= TOL[w.dtype]["o"] and el <= TOL[w.dtype]["lse"]


def test_fwd_s2k_sampled(dev, tk):
    inp = Inputs(syn.workload("fwd_s2k"), dev, with_grad=False)
    sampled_fwd_check(tk, inp, 4096, 0)


@pytest.mark.parametrize("qscale", [8.0, 24.0])
def test_bf16_wide_score_range(dev, tk, qscale):
    """Scores spanning about +-50 (q x 8) and +-150 (q x 24): the running max moves by more
    than its lazy threshold (8 in log2 units) many times per row, and the branch keys can
    dominate or vanish.  RoPE is off, so the fp16 score operands are the bf16 inputs
    exactly and the comparison isolates the online softmax; forward and backward."""
    w = syn.Workload(f"wide_{int(qscale)}", 16, "bshd", 2, 300, 8, 2, 128, 3, "bf16", 0.0, True)
    inp = Inputs(w, dev)
    for p in (1, 3):
        inp.q[p] = syn.round_bf16(inp.q[p] * np.float32(qscale))
        inp.gq[p] = torch.from_numpy(inp.q[p]).to(dev).to(torch.bfloat16)
        o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=0.0)
        eo, el = max_abs(to_np(o), o_ref), max_abs(to_np(lse), l_ref)
        # the backward takes the fp32 O: with one dominant key dP - Delta cancels, and a bf16 O
        # would put its 2^-9 rounding into Delta = <dO, O> (the oracle's Delta uses its exact O)
        dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p)
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="bshd", base=0.0)
        eg = max([rel_fro(to_np(dq), dq_r)] + [rel_fro(to_np(dks[t]), dk_r[t]) for t in range(p)] +
                 [rel_fro(to_np(dvs[t]), dv_r[t]) for t in range(p)])
        lse_range = float(l_ref.max() - l_ref.min())
        print(f"q x {qscale} p={p}: LSE spans {lse_range:.1f}; O max-abs {eo:.2e} LSE max-abs {el:.2e} "
              f"grads {eg:.2e}")
        assert lse_range > 40.0
        assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"] and eg <= TOL["bf16"]["grad"]
