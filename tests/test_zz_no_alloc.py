"""ttt_attn_fwd_noalloc (static per-GPU scratch instead of a workspace argument)
against ttt_attn_fwd on the same inputs: the two run the same kernels, so O and
LSE must be bitwise equal.  Two calls in a row, the second smaller (the scratch
keeps the first call's contents), in BSHD and THD; a call whose workspace need
exceeds the scratch is refused before any launch."""
import numpy as np
import pytest

import ttt_synth as syn
from ttt_cases import Inputs

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


def both(tk, inp, p, o_fp32):
    kw = inp.kw()
    q = inp.gq[p]
    o_ref, l_ref = tk.fwd(q, inp.gk, inp.gv, p, o_fp32=o_fp32, **kw)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32 if o_fp32 else q.dtype, device=q.device)
    lse = torch.full(l_ref.shape, float("nan"), dtype=torch.float32, device=q.device)
    tk.fwd_noalloc(q, inp.gk, inp.gv, p, out, lse, **kw)
    torch.cuda.synchronize()
    return (o_ref, l_ref), (out, lse)


def test_noalloc_forward_matches_workspace_forward(dev, tk):
    big = syn.Workload("noalloc_big", 51, "bshd", 2, 600, 8, 2, 128, 3, "bf16", 1e6, True)
    small = syn.Workload("noalloc_small", 52, "bshd", 1, 100, 4, 1, 128, 2, "bf16", 1e4, True)
    lens = [1, 130, 64, 77]
    thd = syn.Workload("noalloc_thd", 53, "thd", 1, sum(lens), 8, 2, 128, 3, "bf16", 1e6, True)
    cases = [(Inputs(big, dev, with_grad=False), 3, False), (Inputs(small, dev, with_grad=False), 2, True),
             (Inputs(thd, dev, with_grad=False, lengths=lens), 3, False)]
    for inp, p, o_fp32 in cases:
        (o_ref, l_ref), (o, l) = both(tk, inp, p, o_fp32)
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), inp.w.name
        print(f"{inp.w.name}: allocation-free forward equals ttt_attn_fwd bitwise")


def test_noalloc_refuses_problems_past_the_scratch(dev, tk):
    w = syn.Workload("noalloc_huge", 54, "bshd", 4, 4096, 32, 8, 128, 2, "bf16", 1e6, True)
    q = torch.zeros(w.q_shape(), dtype=torch.bfloat16, device=dev)
    ks = [torch.zeros(w.kv_shape(), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    with pytest.raises(tk.TTTAttnError) as e:
        tk.fwd_noalloc(q, ks, ks, 2, out, lse, rope_base=w.rope_base)
    assert e.value.status == 5  # TTT_ERR_WORKSPACE
    # the refusal launched nothing and left the library usable
    inp = Inputs(syn.Workload("noalloc_after", 55, "bshd", 1, 70, 4, 2, 128, 2, "bf16", 1e6, True), dev,
                 with_grad=False)
    (o_ref, l_ref), (o, l) = both(tk, inp, 2, True)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
