"""bf16 head_dim 32 and 64 on the GPU (through the C ABI) against the fp64 oracle.

These head sizes run the D = 128 kernels on zero-padded copies of the heads: each
D-dim head is spread over 128 entries so that the rotate-half pairs and angles
are the D-dim ones, and every padded entry stays zero.  Checked here: forward O
(bf16 and fp32 output) and LSE, and every gradient, for BSHD and THD (ragged
lengths), GQA 4:1, passes 1 and 3, a sliding window, an explicit softmax scale and
the stored-dS backward; and that the padding changes nothing outside the caller's
tensors.
"""
import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import TOL, Inputs, bf16_half_ulp, max_abs, rel_fro, to_np

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


THD_LENS = [1, 63, 64, 65, 200, 129, 3]


def check(tk, inp, p, label, window=0, scale=0.0, stored_ds=False):
    w = inp.w
    kw = inp.kw()
    for o_fp32 in (True, False):
        o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=o_fp32, window=window, softmax_scale=scale, **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout=w.layout, cu_seqlens=inp.cu_host,
                             scale=scale if scale > 0 else None, base=w.rope_base, window=window)
        eo = np.abs(to_np(o) - o_ref)
        if not o_fp32:
            eo = eo - bf16_half_ulp(o_ref)
        el = max_abs(to_np(lse), l_ref)
        print(f"{label} p={p} o_fp32={o_fp32}: O {eo.max():.3e} LSE {el:.3e}")
        assert eo.max() <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, window=window, softmax_scale=scale,
                          stored_ds=stored_ds, **kw)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout=w.layout, cu_seqlens=inp.cu_host,
                             scale=scale if scale > 0 else None, base=w.rope_base, window=window)
    errs = {"dq": rel_fro(to_np(dq), dq_r)}
    for t in range(p):
        errs[f"dk{t + 1}"] = rel_fro(to_np(dks[t]), dk_r[t])
        errs[f"dv{t + 1}"] = rel_fro(to_np(dvs[t]), dv_r[t])
    print(f"{label} p={p} bwd: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL["bf16"]["grad"], errs


@pytest.mark.parametrize("D", [32, 64])
def test_bshd_head_dim(dev, tk, D):
    w = syn.Workload(f"hd{D}_bshd", 61, "bshd", 2, 300, 8, 2, D, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    for p in (1, 3):
        check(tk, inp, p, f"bshd D={D}")
    check(tk, inp, 3, f"bshd D={D} stored dS", stored_ds=True)


@pytest.mark.parametrize("D", [32, 64])
def test_thd_head_dim(dev, tk, D):
    w = syn.Workload(f"hd{D}_thd", 62, "thd", 1, sum(THD_LENS), 8, 2, D, 3, "bf16", 1e4, True)
    check(tk, Inputs(w, dev, lengths=THD_LENS), 3, f"thd D={D}")


def test_head_dim_window_and_scale(dev, tk):
    w = syn.Workload("hd64_win", 63, "bshd", 1, 257, 4, 2, 64, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    check(tk, inp, 3, "D=64 window 50", window=50)
    check(tk, inp, 2, "D=64 scale 0.18", scale=0.18)


@pytest.mark.parametrize("o_fp32", [False, True])
def test_head_dim_strided_outputs_untouched(dev, tk, o_fp32):
    """O written into a slice of a wider buffer: [.., 2D] (16-byte aligned rows, the vector
    unpadding) and [.., D+1] from entry 1 (unaligned, the per-entry unpadding).  The result equals
    the contiguous call's bitwise and the rest of the buffer is left as it was."""
    D, p = 64, 2
    w = syn.Workload("hd64_strided", 64, "bshd", 2, 100, 8, 2, D, p, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    dt = torch.float32 if o_fp32 else torch.bfloat16
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=o_fp32, **inp.kw())
    for width, lo in ((2 * D, 0), (D + 1, 1)):
        big = torch.full((2, 100, 8, width), 7.0, dtype=dt, device=dev)
        out = big[..., lo:lo + D]
        tk.fwd(inp.gq[p], inp.gk, inp.gv, p, out=out, o_fp32=o_fp32, **inp.kw())
        torch.cuda.synchronize()
        assert torch.equal(out, o)
        rest = torch.ones_like(big, dtype=torch.bool)
        rest[..., lo:lo + D] = False
        assert torch.all(big[rest] == 7.0).item()
