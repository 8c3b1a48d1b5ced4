"""Edge cases of the HIP path through the C ABI (GPU)."""
import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import TOL, Inputs, max_abs, rel_fro, to_np

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


def test_repeated_calls_are_bitwise_identical(dev, tk):
    """Stateless and re-entrant: interleaved repeated calls (the activation-recompute
    pattern) give bitwise-equal outputs; the backward uses no atomics."""
    w = syn.Workload("rep", 31, "bshd", 2, 200, 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    kw = inp.kw()
    o1, l1 = tk.fwd(inp.gq[3], inp.gk, inp.gv, 3, **kw)
    g1 = tk.bwd(inp.gq[3], inp.gk, inp.gv, o1, l1, inp.gdo[3], 3, **kw)
    tk.fwd(inp.gq[2], inp.gk, inp.gv, 2, **kw)                 # an unrelated call in between
    o2, l2 = tk.fwd(inp.gq[3], inp.gk, inp.gv, 3, **kw)
    g2 = tk.bwd(inp.gq[3], inp.gk, inp.gv, o2, l2, inp.gdo[3], 3, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1[0], g2[0])
    for a, b in zip(g1[1] + g1[2], g2[1] + g2[2]):
        assert torch.equal(a, b)


def test_zero_tokens_is_a_no_op(dev, tk):
    q = torch.zeros((1, 0, 4, 128), dtype=torch.bfloat16, device=dev)
    k = [torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device=dev)] * 2
    o, lse = tk.fwd(q, k, k, 2, rope_base=1e4)
    dq, dks, dvs = tk.bwd(q, k, k, o, lse, q, 2, rope_base=1e4)
    assert o.numel() == 0 and dq.numel() == 0


def test_thd_with_empty_and_single_token_sequences(dev, tk):
    lens = [0, 1, 5, 0, 70, 1]
    w = syn.Workload("thd_edge", 32, "thd", 1, sum(lens), 4, 2, 128, 3, "bf16", 1e4, True)
    inp = Inputs(w, dev, lengths=lens)
    kw = inp.kw()
    for p in (1, 3):
        o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, check_cu_seqlens=True, **kw)
        dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="thd", cu_seqlens=inp.cu_host, base=w.rope_base)
        g_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="thd", cu_seqlens=inp.cu_host, base=w.rope_base)
        assert max_abs(to_np(o), o_ref) <= 1e-2 and max_abs(to_np(lse), l_ref) <= 2e-3
        assert rel_fro(to_np(dq), g_ref[0]) <= 1e-2
        for t in range(p):
            assert rel_fro(to_np(dks[t]), g_ref[1][t]) <= 1e-2
            assert rel_fro(to_np(dvs[t]), g_ref[2][t]) <= 1e-2


def test_thd_more_sequences_than_one_scheduler_pass(dev, tk):
    # 1500 sequences of 0..8 tokens, two longer ones placed past the first
    # 1024: the varlen scheduler lays out slots in passes of 1024 sequences
    # (the second pass adds the first one's offset), and past 1024 sequences
    # it lists tiles sequence by sequence in index order, in the same passes.
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 9, 1500).tolist()
    lens[700], lens[1200] = 300, 129
    w = syn.Workload("thd_many", 33, "thd", 1, sum(lens), 4, 2, 128, 2, "bf16", 1e4, True)
    inp = Inputs(w, dev, lengths=lens)
    kw = inp.kw()
    for p in (1, 2):
        o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, check_cu_seqlens=True, **kw)
        dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="thd", cu_seqlens=inp.cu_host, base=w.rope_base)
        g_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="thd", cu_seqlens=inp.cu_host, base=w.rope_base)
        assert max_abs(to_np(o), o_ref) <= 1e-2 and max_abs(to_np(lse), l_ref) <= 2e-3
        assert rel_fro(to_np(dq), g_ref[0]) <= 1e-2
        for t in range(p):
            assert rel_fro(to_np(dks[t]), g_ref[1][t]) <= 1e-2
            assert rel_fro(to_np(dvs[t]), g_ref[2][t]) <= 1e-2


def test_invalid_cu_seqlens_rejected_when_checked(dev, tk):
    q = torch.zeros((10, 4, 128), dtype=torch.bfloat16, device=dev)
    k = [torch.zeros((10, 2, 128), dtype=torch.bfloat16, device=dev)]
    for bad in ([0, 6, 4, 10], [1, 5, 10], [0, 5, 9]):
        cu = torch.tensor(bad, dtype=torch.int32, device=dev)
        with pytest.raises(tk.TTTAttnError) as e:
            tk.fwd(q, k, k, 1, cu_seqlens=cu, check_cu_seqlens=True)
        assert e.value.status == 2


def test_sixteen_passes(dev, tk):
    w = syn.Workload("p16", 33, "bshd", 1, 90, 4, 1, 128, 16, "bf16", 1e4, True)
    inp = Inputs(w, dev)
    p = 16
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **inp.kw())
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **inp.kw())
    torch.cuda.synchronize()
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=w.rope_base)
    g_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="bshd", base=w.rope_base)
    assert max_abs(to_np(o), o_ref) <= 1e-2 and max_abs(to_np(lse), l_ref) <= 2e-3
    errs = [rel_fro(to_np(dq), g_ref[0])] + [rel_fro(to_np(dks[t]), g_ref[1][t]) for t in range(p)] + \
           [rel_fro(to_np(dvs[t]), g_ref[2][t]) for t in range(p)]
    assert max(errs) <= 1e-2, errs


def test_strided_views_and_side_stream(dev, tk):
    """q/k/v as strided views into larger buffers, launched on a non-default stream."""
    w = syn.Workload("strided", 34, "bshd", 2, 130, 4, 2, 128, 2, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    p = 2
    big_q = torch.zeros((2, 130, 6, 128), dtype=torch.bfloat16, device=dev)
    big_q[:, :, 1:5] = inp.gq[p]
    qv = big_q[:, :, 1:5]
    big_k = [torch.zeros((2, 130, 3, 128), dtype=torch.bfloat16, device=dev) for _ in range(p)]
    big_v = [torch.zeros((2, 130, 3, 128), dtype=torch.bfloat16, device=dev) for _ in range(p)]
    for t in range(p):
        big_k[t][:, :, 1:3] = inp.gk[t]
        big_v[t][:, :, 1:3] = inp.gv[t]
    kv_ = [x[:, :, 1:3] for x in big_k]
    vv_ = [x[:, :, 1:3] for x in big_v]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        o, lse = tk.fwd(qv, kv_, vv_, p, o_fp32=True, rope_base=w.rope_base, stream=st)
        dq, dks, dvs = tk.bwd(qv, kv_, vv_, o, lse, inp.gdo[p], p, rope_base=w.rope_base, stream=st)
    st.synchronize()
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=w.rope_base)
    g_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="bshd", base=w.rope_base)
    assert max_abs(to_np(o), o_ref) <= 1e-2 and max_abs(to_np(lse), l_ref) <= 2e-3
    assert rel_fro(to_np(dq), g_ref[0]) <= 1e-2
    assert max(rel_fro(to_np(dks[t]), g_ref[1][t]) for t in range(p)) <= 1e-2


def test_fp32_head_dims(dev, tk):
    for D in (32, 64, 128):
        w = syn.Workload(f"f32d{D}", 35, "bshd", 1, 40, 2, 1, D, 2, "fp32", 1e4, True)
        inp = Inputs(w, dev)
        o, lse = tk.fwd(inp.gq[2], inp.gk, inp.gv, 2, rope_base=w.rope_base)
        dq, dks, dvs = tk.bwd(inp.gq[2], inp.gk, inp.gv, o, lse, inp.gdo[2], 2, rope_base=w.rope_base)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd(inp.q[2], inp.k, inp.v, 2, layout="bshd", base=w.rope_base)
        g_ref = O.bwd(inp.q[2], inp.k, inp.v, inp.do[2], 2, layout="bshd", base=w.rope_base)
        assert max_abs(to_np(o), o_ref) <= 1e-5 and max_abs(to_np(lse), l_ref) <= 1e-5
        assert rel_fro(to_np(dq), g_ref[0]) <= 1e-5
        assert max(rel_fro(to_np(dks[t]), g_ref[1][t]) for t in range(2)) <= 1e-5


def test_stream_argument_not_current(dev, tk):
    """Launch on a stream that is not torch's current one, without making it current: the
    binding allocates outputs and workspace on that stream, so blocks the current stream
    allocates meanwhile cannot be handed the workspace while the kernels still use it."""
    w = syn.Workload("side_stream", 36, "bshd", 2, 400, 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    p = 3
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, rope_base=w.rope_base, stream=st)
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, rope_base=w.rope_base, stream=st)
    junk = [torch.full((1 << 22,), float("nan"), device=dev) for _ in range(16)]  # current-stream churn
    st.synchronize()
    del junk
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=w.rope_base)
    g_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="bshd", base=w.rope_base)
    assert max_abs(to_np(o), o_ref) <= 1e-2 and max_abs(to_np(lse), l_ref) <= 2e-3
    assert rel_fro(to_np(dq), g_ref[0]) <= 1e-2
    assert max(rel_fro(to_np(dks[t]), g_ref[1][t]) for t in range(p)) <= 1e-2
    assert max(rel_fro(to_np(dvs[t]), g_ref[2][t]) for t in range(p)) <= 1e-2
