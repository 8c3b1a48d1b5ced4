"""Seeded random problem shapes, forward and backward, every element against the fp64 oracle.

Each case draws a layout (BSHD, or THD with 1-5 packed sequences, empty ones included), a
GQA ratio (1, 2, 3, 4 or 8 query heads per KV head), a head size (bf16: 128 mostly, 64 or 32
on the padded path; fp32: 32, 64 or 128), sequence lengths up to 300 with ragged tails, a pass
index 1..4, a RoPE base and, for bf16, sometimes a sliding window.  The fixed cases the other
files test were chosen by hand; these are not, so a combination nobody thought of gets
exercised.  Tolerances are the library's (`ttt_cases.TOL`)."""
import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import TOL, Inputs, max_abs, rel_fro, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 24


def draw_case(n: int):
    rng = np.random.default_rng([2024, n])
    fp32 = n % 7 == 3
    layout = "thd" if rng.random() < 0.5 else "bshd"
    hkv = int(rng.choice([1, 2]))
    r = int(rng.choice([1, 2, 3, 4, 8]))
    if fp32:
        D = int(rng.choice([32, 64, 128]))
    else:
        D = int(rng.choice([128, 128, 128, 64, 32]))
    K = 4
    p = int(rng.integers(1, K + 1))
    base = float(rng.choice([1e4, 1e6]))
    if layout == "bshd":
        B, S = int(rng.integers(1, 4)), int(rng.integers(1, 301))
        lengths = None
        L = S
    else:
        ns = int(rng.integers(1, 6))
        lengths = [int(x) for x in rng.integers(0, 251, ns)]
        if n % 3 == 0:
            lengths.insert(len(lengths) // 2, 0)  # an empty sequence between others
        if sum(lengths) == 0:
            lengths[0] = 7
        B, S = 1, sum(lengths)
        L = max(lengths)
    window = 0
    if not fp32 and rng.random() < 0.4:
        window = int(rng.integers(1, max(2, L) + 1))
    w = syn.Workload(f"rand{n}", 200 + n, layout, B, S, hkv * r, hkv, D, K, "fp32" if fp32 else "bf16", base, True)
    return w, lengths, p, window


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


@pytest.mark.parametrize("n", range(N_CASES))
def test_random_shape(dev, tk, n):
    w, lengths, p, window = draw_case(n)
    inp = Inputs(w, dev, passes=p, lengths=lengths)
    kw = dict(inp.kw(), window=window)
    label = (f"case {n}: {w.layout} B{w.B} S{w.S} {w.Hq}/{w.Hkv} D{w.D} {w.dtype} p={p} window={window} "
             f"base={w.rope_base:g}" + (f" lengths={lengths}" if lengths else ""))
    print(label, flush=True)
    o32, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **kw)
    o, lse2 = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **kw)
    dq, dks, dvs = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse2, inp.gdo[p], p, **kw)
    torch.cuda.synchronize()
    geo = dict(layout=w.layout, cu_seqlens=inp.cu_host, base=w.rope_base, window=window)
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, **geo)
    dq_ref, dk_ref, dv_ref = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, **geo)
    tol = TOL[w.dtype]
    eo, el = max_abs(to_np(o32), o_ref), max_abs(to_np(lse), l_ref)
    errs = {"dq": rel_fro(to_np(dq), dq_ref)}
    for t in range(p):
        errs[f"dk{t + 1}"] = rel_fro(to_np(dks[t]), dk_ref[t])
        errs[f"dv{t + 1}"] = rel_fro(to_np(dvs[t]), dv_ref[t])
    worst = max(errs.values())
    print(f"  O max-abs {eo:.2e} LSE max-abs {el:.2e} grad rel-Frobenius worst {worst:.2e}")
    assert np.isfinite(eo) and eo <= tol["o"] and el <= tol["lse"]
    assert np.isfinite(worst) and worst <= tol["grad"], errs
