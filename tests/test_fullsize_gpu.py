"""Parity at the full workload sizes, in the launch configuration bench.py uses.

The oracle cannot evaluate every row of these workloads in seconds, so each
check compares sampled outputs it computes one by one:
  * forward: >= 4096 query rows drawn uniformly over (sequence row, head, pass)
    plus forced edge rows (first/second/last row of every sequence, tile
    borders), O max-abs and LSE max-abs;
  * dQ: >= 4096 sampled rows, relative Frobenius over the stacked rows (the
    oracle evaluates those rows exactly); the same evaluation also gives the
    exact gradients of the branch keys at those rows (a branch key is seen by
    its own row only);
  * trunk dK/dV: the last W rows of a (sequence, KV head) slice, whose trunk
    keys are seen only by rows inside the window, so the oracle's gradient
    there is exact.
"""
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


def gather_rows(t, layout, sl, h, rows):
    """Rows of head h of sequence sl, from a device tensor, as a float64 host array."""
    idx = torch.as_tensor(np.asarray(rows), device=t.device)
    x = t[sl.b].index_select(0, idx)[:, h] if layout == "bshd" else t.index_select(0, idx + sl.start)[:, h]
    return x.double().cpu().numpy()


def gather_lse(t, layout, sl, h, rows):
    idx = torch.as_tensor(np.asarray(rows), device=t.device)
    x = t[sl.b, h].index_select(0, idx) if layout == "bshd" else t[h].index_select(0, idx + sl.start)
    return x.double().cpu().numpy()


def run_fullsize(tk, name, dev, n_rows=4096, window=256, check_bwd=True):
    w = syn.workload(name)
    inp = Inputs(w, dev, with_grad=check_bwd)
    kw = inp.kw()
    slices = inp.slices()
    passes = list(range(1, w.K + 1))
    rows = sample_rows(inp, n_rows, 7, passes)
    r = w.Hq // w.Hkv
    eo = el = 0.0
    n_f = 0
    dq_g, dq_r, bk_g, bk_r, bv_g, bv_r = [], [], [], [], [], []
    tk_g, tk_r, tv_g, tv_r = [], [], [], []
    rng = np.random.default_rng(11)
    tail_passes = {1, w.K, (1 + w.K) // 2}
    for p in passes:
        o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **kw)
        torch.cuda.synchronize()
        by_group = {}
        for (pp, s, h), rr in rows.items():
            if pp == p:
                by_group.setdefault((s, h // r), {})[h] = rr
        for (s, g), heads in by_group.items():
            sl = slices[s]
            ref = O.fwd_group_rows(inp.q[p], inp.k, inp.v, p, sl, g, heads, layout=w.layout, Hq=w.Hq,
                                   Hkv=w.Hkv, scale=w.scale, base=w.rope_base)
            for h, rr in heads.items():
                o_ref, l_ref = ref[h]
                eo = max(eo, max_abs(gather_rows(o, w.layout, sl, h, rr), o_ref))
                el = max(el, max_abs(gather_lse(lse, w.layout, sl, h, rr), l_ref))
                n_f += len(rr)
        if not check_bwd:
            continue
        ob, lb = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
        dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, ob, lb, inp.gdo[p], p, **kw)
        torch.cuda.synchronize()
        # dQ rows and branch dK/dV at the same rows (all heads of the group)
        for (s, g), heads in by_group.items():
            sl = slices[s]
            rr = np.array(sorted(set(np.concatenate(list(heads.values())).tolist())))
            dq_ref, dk_ref, dv_ref = O.bwd_rows(inp.q[p], inp.k, inp.v, inp.do[p], p, sl, g, rr, layout=w.layout,
                                                Hq=w.Hq, Hkv=w.Hkv, scale=w.scale, base=w.rope_base)
            for hh in range(r):
                h = g * r + hh
                if h in heads:
                    sel = np.searchsorted(rr, heads[h])
                    dq_g.append(gather_rows(dq, w.layout, sl, h, heads[h]))
                    dq_r.append(dq_ref[hh][sel])
            for q in range(2, p + 1):
                bk_g.append(gather_rows(dks[q - 1], w.layout, sl, g, rr))
                bk_r.append(dk_ref[(q - 1) * sl.L + rr])
                bv_g.append(gather_rows(dvs[q - 1], w.layout, sl, g, rr))
                bv_r.append(dv_ref[(q - 1) * sl.L + rr])
        # trunk dK/dV: the last `window` rows of one random (sequence, KV head)
        if p in tail_passes:
            s = int(rng.integers(len(slices)))
            g = int(rng.integers(w.Hkv))
            sl = slices[s]
            rr = np.arange(max(0, sl.L - window), sl.L)
            _, dk_ref, dv_ref = O.bwd_rows(inp.q[p], inp.k, inp.v, inp.do[p], p, sl, g, rr, layout=w.layout,
                                           Hq=w.Hq, Hkv=w.Hkv, scale=w.scale, base=w.rope_base)
            tk_g.append(gather_rows(dks[0], w.layout, sl, g, rr))
            tk_r.append(dk_ref[rr])
            tv_g.append(gather_rows(dvs[0], w.layout, sl, g, rr))
            tv_r.append(dv_ref[rr])
        del dq, dks, dvs, ob, lb
    tol = TOL[w.dtype]
    print(f"{name}: forward {n_f} sampled rows: O max-abs {eo:.3e}, LSE max-abs {el:.3e}")
    assert n_f >= n_rows
    assert eo <= tol["o"] and el <= tol["lse"]
    if check_bwd:
        errs = {"dq": rel_fro(np.concatenate(dq_g), np.concatenate(dq_r)),
                "dk_branch": rel_fro(np.concatenate(bk_g), np.concatenate(bk_r)),
                "dv_branch": rel_fro(np.concatenate(bv_g), np.concatenate(bv_r)),
                "dk_trunk_tail": rel_fro(np.concatenate(tk_g), np.concatenate(tk_r)),
                "dv_trunk_tail": rel_fro(np.concatenate(tv_g), np.concatenate(tv_r))}
        n_dq = sum(len(x) for x in dq_g)
        print(f"{name}: backward {n_dq} sampled dQ rows: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        assert n_dq >= n_rows
        assert max(errs.values()) <= tol["grad"], errs


def test_b4_s4k_fullsize(dev, tk):
    run_fullsize(tk, "b4_s4k", dev)


def test_thd_32k_fullsize(dev, tk):
    run_fullsize(tk, "thd_32k", dev)


def test_s32k_fullsize(dev, tk):
    run_fullsize(tk, "s32k", dev, window=192)
