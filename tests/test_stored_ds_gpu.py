"""Backward with stored dS (bwd_mode STORED_DS: bf16 BSHD passes without a window).

The dK/dV kernel writes every causal 32x32 block of the fp16 dS (one power-of-two
scale per KV group) into the workspace, and dQ~ = dS K~ is formed from those blocks
instead of recomputing S and dP.  Checked against the fp64 oracle for the shape
classes the blocks and the dQ work items meet -- S = 1, S a multiple of 32 and not,
GQA 4:1 (four heads per work item), 2:1 (two row blocks per work item), 1:1 and 3:1
(four row blocks of one head), 8:1 (two work items per group; branch gradients from
their own kernel) -- and for the recomputing backward (the default) on the same
inputs; plus bitwise determinism of the stored-dS backward.
"""
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


# (B, S, Hq, Hkv, passes checked)
CASES = [
    (2, 300, 8, 2, (1, 3)),   # 4:1, S not a multiple of 32
    (1, 1, 4, 4, (2,)),       # one token, 1:1
    (2, 96, 4, 2, (1, 2)),    # 2:1, S a multiple of 32
    (1, 161, 6, 2, (3,)),     # 3:1
    (1, 257, 16, 2, (3,)),    # 8:1
    (1, 600, 8, 2, (7,)),     # 4:1, seven passes
]


def grads_vs_oracle(tk, inp, p, stored):
    w = inp.w
    kw = inp.kw()
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, stored_ds=stored, **kw)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout=w.layout, base=w.rope_base)
    errs = {"dq": rel_fro(to_np(dq), dq_r)}
    for t in range(p):
        errs[f"dk{t + 1}"] = rel_fro(to_np(dks[t]), dk_r[t])
        errs[f"dv{t + 1}"] = rel_fro(to_np(dvs[t]), dv_r[t])
    return (dq, dks, dvs), errs


@pytest.mark.parametrize("B,S,Hq,Hkv,passes", CASES)
def test_stored_ds_backward_matches_oracle(dev, tk, B, S, Hq, Hkv, passes):
    w = syn.Workload(f"sds_{B}x{S}_{Hq}_{Hkv}", 90 + S % 17, "bshd", B, S, Hq, Hkv, 128, max(passes), "bf16", 1e6,
                     True)
    inp = Inputs(w, dev)
    for p in passes:
        for stored in (True, False):
            (dq, _, _), errs = grads_vs_oracle(tk, inp, p, stored)
            tag = "stored dS" if stored else "recompute"
            print(f"B{B} S{S} {Hq}/{Hkv} p={p} {tag}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
            assert torch.isfinite(dq.float()).all().item()
            assert max(errs.values()) <= TOL["bf16"]["grad"], errs


def test_stored_ds_backward_is_deterministic(dev, tk):
    w = syn.Workload("sds_det", 97, "bshd", 2, 333, 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    p = 3
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **inp.kw())
    a = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, stored_ds=True, **inp.kw())
    b = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, stored_ds=True, **inp.kw())
    torch.cuda.synchronize()
    for x, y in [(a[0], b[0])] + list(zip(a[1], b[1])) + list(zip(a[2], b[2])):
        assert torch.equal(x, y)
    print("stored-dS backward: two runs bitwise equal")
