"""Seeded random ring steps and block-drafting problems against the fp64 oracle.

Ring steps (BSHD): a query chunk at a random offset against a pass-1 key chunk at another
(before, across or after the rows, possibly empty), with or without the branch, a random GQA
ratio, pass and sometimes a sliding window; the step's partial O / LSE and its backward terms
(fed the oracle's whole-sequence O and LSE) are compared element by element.  Block drafting
(BSHD): random context length (zero included), block size, block count, head ratio and anchors
(unsorted, repeated, out of range), forward and all five gradients.  Hand-picked cases of both
live in test_ring_gpu.py and test_block_gpu.py."""
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


def zero_bound(*ts):
    """A bound for gradients whose exact value is 0 by cancellation (e.g. a row that sees one key:
    P = 1, so dS = dP - Delta, two fp32 sums of the same products in different orders): 1e-5 of
    sigma * max ||dO_i|| * max ||v_j|| * max ||k_j||, the size of one dS * k term."""
    s = 1.0
    for x in ts:
        s *= max(1.0, float(np.sqrt((np.asarray(x, np.float64) ** 2).sum(-1)).max(initial=0.0)))
    return 1e-5 * s / np.sqrt(ts[0].shape[-1])


def check_grads(pairs, bound, exact_zero=False):
    """Relative Frobenius per gradient; an all-zero reference needs |g| <= bound (exactly 0 when no
    key is visible at all)."""
    msg = []
    for name, g, rr in pairs:
        g = to_np(g)
        assert g.shape == rr.shape, (name, g.shape, rr.shape)
        if rr.size == 0:
            continue
        if not np.any(rr):
            gm = float(np.abs(g).max())
            assert (gm == 0.0) if exact_zero else (gm <= bound), (name, gm, bound)
            msg.append(f"{name}~0 ({gm:.0e})")
            continue
        e = rel_fro(g, rr)
        msg.append(f"{name}={e:.1e}")
        assert np.all(np.isfinite(g)) and e <= TOL["bf16"]["grad"], (name, e)
    return " ".join(msg)


def ring_case(n: int):
    rng = np.random.default_rng([2025, n])
    hkv = int(rng.choice([1, 2]))
    r = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(40, 321))
    K = 3
    p = int(rng.integers(1, K + 1))
    qa = int(rng.integers(0, S))
    nq = int(rng.integers(1, S - qa + 1))
    ka = int(rng.integers(0, S))
    m = int(rng.integers(0, S - ka + 1))
    br = bool(rng.random() < 0.6)
    window = int(rng.integers(1, S + 1)) if rng.random() < 0.3 else 0
    w = syn.Workload(f"rstep{n}", 300 + n, "bshd", int(rng.integers(1, 3)), S, hkv * r, hkv, 128, K, "bf16",
                     float(rng.choice([1e4, 1e6])), True)
    return w, p, qa, nq, ka, m, br, window


@pytest.mark.parametrize("n", range(12))
def test_random_ring_step(dev, tk, n):
    w, p, qa, nq, ka, m, br, window = ring_case(n)
    print(f"ring step {n}: B{w.B} S{w.S} {w.Hq}/{w.Hkv} p={p} q@{qa}+{nq} kv@{ka}+{m} branch={br} "
          f"window={window} base={w.rope_base:g}", flush=True)
    inp = Inputs(w, dev, passes=p)
    base = w.rope_base
    sk = [inp.gk[0][:, ka:ka + m]] + [k[:, qa:qa + nq] for k in inp.gk[1:p]]
    sv = [inp.gv[0][:, ka:ka + m]] + [v[:, qa:qa + nq] for v in inp.gv[1:p]]
    rbk = [k[:, qa:qa + nq] for k in inp.k[1:p]] if br else None
    rbv = [v[:, qa:qa + nq] for v in inp.v[1:p]] if br else None
    # forward: the step's partial O and LSE
    o, l = tk.fwd_chunk(inp.gq[p][:, qa:qa + nq], sk, sv, p, q_offset=qa, kv_offset=ka, with_branch=br,
                        rope_base=base, window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = O.fwd_chunk(inp.q[p][:, qa:qa + nq], inp.k[0][:, ka:ka + m], inp.v[0][:, ka:ka + m], rbk, rbv,
                               p, q_offset=qa, kv_offset=ka, base=base, window=window)
    og, lg = to_np(o), to_np(l)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lg), empty)
    eo = max_abs(og, o_ref)
    el = max_abs(lg[~empty], l_ref[~empty]) if (~empty).any() else 0.0
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], (eo, el)
    assert np.all(og[np.transpose(empty, (0, 2, 1))] == 0)
    # backward terms, fed the oracle's whole-sequence O (bf16) and LSE
    o_full, l_full = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=base, window=window)
    o16 = syn.round_bf16(o_full.astype(np.float32))
    go = torch.from_numpy(o16).to(dev).to(torch.bfloat16)
    gl = torch.from_numpy(np.ascontiguousarray(l_full, dtype=np.float32)).to(dev)
    dq, dks, dvs = tk.bwd_chunk(inp.gq[p][:, qa:qa + nq], sk, sv, go[:, qa:qa + nq], gl[:, :, qa:qa + nq],
                                inp.gdo[p][:, qa:qa + nq], p, q_offset=qa, kv_offset=ka, with_branch=br,
                                rope_base=base, window=window)
    torch.cuda.synchronize()
    rq, rk0, rv0, rkb, rvb = O.bwd_chunk(inp.q[p][:, qa:qa + nq], inp.k[0][:, ka:ka + m], inp.v[0][:, ka:ka + m],
                                         rbk, rbv, p, inp.do[p][:, qa:qa + nq], o16[:, qa:qa + nq],
                                         l_full[:, :, qa:qa + nq], q_offset=qa, kv_offset=ka, base=base,
                                         window=window)
    pairs = [("dq", dq, rq), ("dk1", dks[0], rk0), ("dv1", dvs[0], rv0)]
    pairs += [(f"dk{t + 2}", dks[1 + t], rkb[t]) for t in range(len(rkb))]
    pairs += [(f"dv{t + 2}", dvs[1 + t], rvb[t]) for t in range(len(rvb))]
    assert len(dks) == 1 + len(rkb) and len(dvs) == 1 + len(rvb)
    bound = zero_bound(inp.do[p], inp.v[0], inp.k[0])
    msg = check_grads(pairs, bound, exact_zero=bool(empty.all()))  # no visible key at all: exactly 0
    print(f"  O {eo:.2e} LSE {el:.2e} empty rows {int(empty.sum())}; " + msg)


def block_case(n: int):
    rng = np.random.default_rng([2026, n])
    hkv = int(rng.choice([1, 2]))
    r = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32]))
    nblk = int(rng.integers(1, max(2, 160 // bs) + 1))
    ctx = 0 if rng.random() < 0.2 else int(rng.integers(1, 400))
    B = int(rng.integers(1, 3))
    bw = syn.BlockWorkload(f"rblk{n}", 400 + n, B, ctx, bs, nblk, hkv * r, hkv, 128, "bf16",
                           float(rng.choice([1e4, 1e6])))
    anchors = rng.integers(-3, ctx + 4, (B, nblk)).astype(np.int32)
    if nblk > 2:
        anchors[:, 1] = anchors[:, 0]  # a repeated anchor
    return bw, anchors


@pytest.mark.parametrize("n", range(10))
def test_random_block(dev, tk, n):
    bw, anchors = block_case(n)
    print(f"block {n}: B{bw.B} ctx{bw.ctx_len} bs{bw.bs} nblk{bw.nblk} {bw.Hq}/{bw.Hkv} base={bw.rope_base:g}",
          flush=True)
    w = bw.as_workload()
    q = syn.draw(w, syn.KIND_Q, 1, bw.q_shape())
    kc, vc = syn.draw(w, syn.KIND_K, 1, bw.ctx_shape()), syn.draw(w, syn.KIND_V, 1, bw.ctx_shape())
    kb, vb = syn.draw(w, syn.KIND_K, 2, bw.blk_shape()), syn.draw(w, syn.KIND_V, 2, bw.blk_shape())
    do = syn.draw(w, syn.KIND_DO, 1, bw.q_shape())
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
    gq, gkc, gvc, gkb, gvb, gdo = map(up, (q, kc, vc, kb, vb, do))
    ga = torch.from_numpy(anchors).to(dev)
    o32, lse = tk.block_fwd(gq, gkc, gvc, gkb, gvb, ga, bw.bs, rope_base=bw.rope_base, o_fp32=True)
    o, lse2 = tk.block_fwd(gq, gkc, gvc, gkb, gvb, ga, bw.bs, rope_base=bw.rope_base)
    grads = tk.block_bwd(gq, gkc, gvc, gkb, gvb, ga, bw.bs, o, lse2, gdo, rope_base=bw.rope_base)
    torch.cuda.synchronize()
    o_ref, l_ref = O.block_fwd(q, kc, vc, kb, vb, anchors, bw.bs, base=bw.rope_base)
    eo, el = max_abs(to_np(o32), o_ref), max_abs(to_np(lse), l_ref)
    assert np.isfinite(eo) and eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], (eo, el)
    ref = O.block_bwd(q, kc, vc, kb, vb, anchors, bw.bs, do, base=bw.rope_base)
    keys = np.concatenate([kc.reshape(-1, kc.shape[-1]), kb.reshape(-1, kb.shape[-1])])
    vals = np.concatenate([vc.reshape(-1, vc.shape[-1]), vb.reshape(-1, vb.shape[-1])])
    bound = zero_bound(do.reshape(-1, do.shape[-1]), vals, keys)
    msg = check_grads(zip(("dq", "dk_ctx", "dv_ctx", "dk_blk", "dv_blk"), grads, ref), bound)
    print(f"  O {eo:.2e} LSE {el:.2e}; " + msg)
