"""GPU parity of ttt_attn_bwd against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import TOL, Inputs, rel_fro, to_np

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


def full_bwd_check(tk, inp, p, label):
    w = inp.w
    kw = inp.kw()
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **kw)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout=w.layout, cu_seqlens=inp.cu_host,
                                   base=w.rope_base)
    errs = {"dq": rel_fro(to_np(dq), dq_ref)}
    for t in range(p):
        errs[f"dk{t + 1}"] = rel_fro(to_np(dks[t]), dk_ref[t])
        errs[f"dv{t + 1}"] = rel_fro(to_np(dvs[t]), dv_ref[t])
    worst = max(errs.values())
    print(f"{label} p={p}: grad rel-Frobenius worst {worst:.3e} " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert np.isfinite(worst) and worst <= TOL[w.dtype]["grad"], errs


def test_tiny_fp32_backward_all_passes(dev, tk):
    w = syn.workload("tiny_fp32")
    inp = Inputs(w, dev)
    for p in range(1, w.K + 1):
        full_bwd_check(tk, inp, p, "tiny_fp32")


def test_fp32_thd_backward(dev, tk):
    lens = [5, 70, 1, 33]
    w = syn.Workload("thd_f32", 21, "thd", 1, sum(lens), 4, 2, 64, 3, "fp32", 1e4, True)
    inp = Inputs(w, dev, lengths=lens)
    for p in (1, 3):
        full_bwd_check(tk, inp, p, "thd_f32")


@pytest.mark.parametrize("p", [1, 2, 4])
def test_bf16_bshd_small_backward(dev, tk, p):
    # 2 x 300 rows: 3 query tiles / 3 key tiles with a ragged tail, GQA 4:1
    w = syn.Workload("bshd_small_bwd", 14, "bshd", 2, 300, 8, 2, 128, 4, "bf16", 1e6, True)
    full_bwd_check(tk, Inputs(w, dev), p, "bshd_small")


@pytest.mark.parametrize("hq,hkv,layout", [(8, 1, "bshd"), (6, 2, "bshd"), (16, 2, "thd"), (2, 1, "bshd")])
def test_bf16_gqa_ratios_backward(dev, tk, hq, hkv, layout):
    """GQA 8:1 and 3:1 (a KV group's query heads span several dQ work items, so the branch
    gradients come from their own kernel), 8:1 THD, and 2:1 (the dQ epilogue produces them)."""
    lens = [130, 1, 64, 97]
    S = sum(lens) if layout == "thd" else 160
    w = syn.Workload(f"gqa_{hq}_{hkv}", 27, layout, 1 if layout == "thd" else 2, S, hq, hkv, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev, lengths=lens if layout == "thd" else None)
    full_bwd_check(tk, inp, 3, f"gqa {hq}:{hkv} {layout}")


@pytest.mark.parametrize("p", [1, 3])
def test_bf16_thd_small_backward(dev, tk, p):
    lens = [1, 63, 64, 65, 200, 129, 3, 130]
    w = syn.Workload("thd_small_bwd", 15, "thd", 1, sum(lens), 4, 1, 128, 3, "bf16", 1e4, True)
    full_bwd_check(tk, Inputs(w, dev, lengths=lens), p, "thd_small")


@pytest.mark.parametrize("hq,hkv,layout", [(8, 1, "bshd"), (8, 2, "bshd"), (16, 2, "thd")])
def test_bf16_backward_aux_stream(dev, tk, hq, hkv, layout):
    """The backward's optional second stream (desc.aux_stream): none, the binding's own and one of
    the caller's give bitwise the same gradients (GQA 8:1: the branch kernel on it; 4:1: Delta), and
    the call stays ordered on its stream (the inputs are rewritten right after the call)."""
    lens = [130, 1, 64, 97]
    S = sum(lens) if layout == "thd" else 160
    w = syn.Workload(f"aux_{hq}_{hkv}", 28, layout, 1 if layout == "thd" else 2, S, hq, hkv, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev, lengths=lens if layout == "thd" else None)
    kw = inp.kw()
    p = 3
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
    mine = torch.cuda.Stream()
    res = []
    for aux in (None, "auto", mine):
        dout = inp.gdo[p].clone()
        g = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, dout, p, aux_stream=aux, **kw)
        dout.fill_(float("nan"))  # ordered after the call's kernels on the current stream
        torch.cuda.synchronize()
        res.append([g[0]] + list(g[1]) + list(g[2]))
    for other in res[1:]:
        for x, y in zip(res[0], other):
            assert torch.equal(x, y)
    assert all(torch.isfinite(x.float()).all() for x in res[0])
    print(f"aux stream {hq}:{hkv} {layout}: none, binding-owned and caller-owned aux streams bitwise equal")


def test_bf16_bwd_chunk_aux_stream(dev, tk):
    """A ring step's backward terms (GQA 8:1: the branch kernel runs on the aux stream) are bitwise
    the same with and without the second stream."""
    w = syn.Workload("aux_chunk", 29, "bshd", 1, 192, 8, 1, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    p, qa, n, ka, m = 3, 64, 96, 32, 100
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **inp.kw())
    sk = [inp.gk[0][:, ka:ka + m]] + [k[:, qa:qa + n] for k in inp.gk[1:p]]
    sv = [inp.gv[0][:, ka:ka + m]] + [v[:, qa:qa + n] for v in inp.gv[1:p]]
    res = []
    for aux in (None, "auto"):
        g = tk.bwd_chunk(inp.gq[p][:, qa:qa + n], sk, sv, o[:, qa:qa + n], lse[:, :, qa:qa + n],
                         inp.gdo[p][:, qa:qa + n], p, q_offset=qa, kv_offset=ka, with_branch=True,
                         rope_base=w.rope_base, aux_stream=aux)
        torch.cuda.synchronize()
        res.append([g[0]] + list(g[1]) + list(g[2]))
    assert len(res[0]) == 1 + 2 * p
    for x, y in zip(*res):
        assert torch.equal(x, y)
    assert all(torch.isfinite(x).all() for x in res[0]) and any(x.abs().max() > 0 for x in res[0][1 + p:])
    print("bwd_chunk GQA 8:1 with branch: no aux stream and the binding's aux stream bitwise equal")
