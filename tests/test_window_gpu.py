"""GPU parity of the sliding-window trunk (descriptor window W: row i sees pass-1 keys i-W < j <= i).

Forward and backward against the fp64 oracle on BSHD and THD inputs (windows from 1 to beyond the sequence,
tile borders, GQA), a window of at least L equal bit for bit to no window, windowed ring steps joined over a
zig-zag ring equal to one windowed call, and sampled rows / exact key windows at B=4, S=4096, K=7.
"""
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


def check(tk, inp, p, window, label, bwd=True):
    w = inp.w
    kw = dict(inp.kw(), window=window)
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout=w.layout, cu_seqlens=inp.cu_host, base=w.rope_base,
                         window=window)
    eo, el = max_abs(to_np(o), o_ref), max_abs(to_np(lse), l_ref)
    msg = f"{label} p={p} W={window}: O {eo:.2e} LSE {el:.2e}"
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], msg
    if bwd:
        ob, lb = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
        dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, ob, lb, inp.gdo[p], p, **kw)
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout=w.layout, cu_seqlens=inp.cu_host,
                                 base=w.rope_base, window=window)
        errs = [rel_fro(to_np(dq), dq_r)] + [rel_fro(to_np(dks[t]), dk_r[t]) for t in range(p)] + \
               [rel_fro(to_np(dvs[t]), dv_r[t]) for t in range(p)]
        msg += f" grads worst {max(errs):.2e}"
        assert max(errs) <= TOL["bf16"]["grad"], msg
    print(msg)


@pytest.mark.parametrize("window", [1, 37, 64, 200])
def test_window_bshd(dev, tk, window):
    w = syn.Workload("win_bshd", 61, "bshd", 2, 300, 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    for p in (1, 3):
        check(tk, inp, p, window, "bshd")


def test_window_thd_and_head_ratios(dev, tk):
    lens = [1, 63, 64, 65, 200, 129, 3, 130]
    w = syn.Workload("win_thd", 62, "thd", 1, sum(lens), 4, 1, 128, 3, "bf16", 1e4, True)
    check(tk, Inputs(w, dev, lengths=lens), 3, 50, "thd")
    w2 = syn.Workload("win_r2", 63, "bshd", 1, 257, 4, 2, 128, 2, "bf16", 1e6, True)
    check(tk, Inputs(w2, dev), 2, 96, "r=2")
    w1 = syn.Workload("win_r1", 64, "bshd", 1, 257, 2, 2, 128, 2, "bf16", 1e6, True)
    check(tk, Inputs(w1, dev), 2, 33, "r=1")


def test_window_at_least_length_is_full(dev, tk):
    w = syn.Workload("win_full", 65, "bshd", 1, 200, 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    a = tk.fwd(inp.gq[3], inp.gk, inp.gv, 3, rope_base=w.rope_base)
    b = tk.fwd(inp.gq[3], inp.gk, inp.gv, 3, rope_base=w.rope_base, window=200)
    c = tk.fwd(inp.gq[3], inp.gk, inp.gv, 3, rope_base=w.rope_base, window=10 ** 6)
    ga = tk.bwd(inp.gq[3], inp.gk, inp.gv, a[0], a[1], inp.gdo[3], 3, rope_base=w.rope_base)
    gb = tk.bwd(inp.gq[3], inp.gk, inp.gv, a[0], a[1], inp.gdo[3], 3, rope_base=w.rope_base, window=1000)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[0], c[0])
    assert torch.equal(ga[0], gb[0]) and all(torch.equal(x, y) for x, y in zip(ga[1] + ga[2], gb[1] + gb[2]))


def test_window_ring(dev, tk):
    """Windowed ring steps over a zig-zag ring of 2 ranks equal one windowed call."""
    w = syn.Workload("win_ring", 66, "bshd", 2, 512, 8, 2, 128, 3, "bf16", 1e6, False)
    inp = Inputs(w, dev, with_grad=False)
    p, cp, W = 3, 2, 100
    S = w.S
    c = S // (2 * cp)
    so, sl = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, rope_base=w.rope_base, window=W)
    ro = torch.empty_like(so)
    rl = torch.empty_like(sl)
    for qc in range(2 * cp):
        qa = qc * c
        acc_o = torch.zeros((w.B, c, w.Hq, w.D), dtype=torch.float32, device=dev)
        acc_l = torch.full((w.B, w.Hq, c), -float("inf"), dtype=torch.float32, device=dev)
        for kc in range(qc + 1):
            ka = kc * c
            sk = [inp.gk[0][:, ka:ka + c]] + [k[:, qa:qa + c] for k in inp.gk[1:p]]
            sv = [inp.gv[0][:, ka:ka + c]] + [v[:, qa:qa + c] for v in inp.gv[1:p]]
            o, l = tk.fwd_chunk(inp.gq[p][:, qa:qa + c], sk, sv, p, q_offset=qa, kv_offset=ka, with_branch=kc == qc,
                                rope_base=w.rope_base, window=W)
            tk.merge(acc_o, acc_l, o, l, out=acc_o, lse=acc_l)
        ro[:, qa:qa + c] = acc_o
        rl[:, :, qa:qa + c] = acc_l
    torch.cuda.synchronize()
    d_o, d_l = (ro - so).abs().max().item(), (rl - sl).abs().max().item()
    print(f"windowed ring vs single call: O {d_o:.2e} LSE {d_l:.2e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"]


def test_window_fullsize(dev, tk):
    """B=4, S=4096, K=7 workload with W=512 at pass 7: >= 4096 sampled forward rows and dQ rows, and the trunk
    dK/dV of key rows [1024, 1088) of every (batch, KV head), exact from rows [1024, 1088 + W)."""
    w = syn.workload("b4_s4k")
    inp = Inputs(w, dev, passes=w.K)
    p, W = w.K, 512
    kw = dict(rope_base=w.rope_base, window=W)
    o32, l32 = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **kw)
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **kw)
    torch.cuda.synchronize()
    og, lg, dqg, dkg, dvg = to_np(o32), to_np(l32), to_np(dq), to_np(dks[0]), to_np(dvs[0])
    rng = np.random.default_rng(67)
    r = w.Hq // w.Hkv
    eo = el = 0.0
    n = 0
    gq, rq, gk, rk, gv, rv = [], [], [], [], [], []
    k0, k1 = 1024, 1088
    rows_k = np.arange(k0, k1 + W)
    for b in range(w.B):
        sl = O.Slice(b, 0, w.S)
        for g in range(w.Hkv):
            rows = np.unique(np.concatenate([rng.integers(0, w.S, 128), [0, 511, 512, 513, 4095]]))
            heads = {g * r + hh: rows for hh in range(r)}
            ref = O.fwd_group_rows(inp.q[p], inp.k, inp.v, p, sl, g, heads, layout="bshd", Hq=w.Hq, Hkv=w.Hkv,
                                   scale=w.scale, base=w.rope_base, window=W)
            for h, (o_r, l_r) in ref.items():
                eo = max(eo, max_abs(og[b, rows, h], o_r))
                el = max(el, max_abs(lg[b, h, rows], l_r))
                n += len(rows)
            dq_r, dk_r, dv_r = O.bwd_rows(inp.q[p], inp.k, inp.v, inp.do[p], p, sl, g, rows_k, layout="bshd",
                                          Hq=w.Hq, Hkv=w.Hkv, scale=w.scale, base=w.rope_base, window=W)
            for hh in range(r):
                gq.append(dqg[b, rows_k, g * r + hh]); rq.append(dq_r[hh])
            gk.append(dkg[b, k0:k1, g]); rk.append(dk_r[k0:k1])
            gv.append(dvg[b, k0:k1, g]); rv.append(dv_r[k0:k1])
    eq = rel_fro(np.concatenate(gq), np.concatenate(rq))
    ek = rel_fro(np.concatenate(gk), np.concatenate(rk))
    ev = rel_fro(np.concatenate(gv), np.concatenate(rv))
    print(f"W=512 full size: {n} rows O {eo:.2e} LSE {el:.2e}; dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
    assert n >= 4096
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
    assert max(eq, ek, ev) <= TOL["bf16"]["grad"]
