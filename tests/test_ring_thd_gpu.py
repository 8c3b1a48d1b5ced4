"""Packed (THD) ring steps on the GPU (through the C ABI) against the fp64 oracle.

In a THD ring step every sequence of the packed batch takes its own step: its
query rows at its own position offset against its own block of pass-1 keys
(packed by kv_cu_seqlens) at its own key offset.  Single steps are checked
against the oracle's packed step, with sequences whose key block is longer or
shorter than their query rows, empty on either side, or entirely after the
rows; a zig-zag ring over packed sequences of ragged lengths, joined with the
merge kernel, must equal one whole-sequence THD call and the oracle, and its
summed backward terms the whole-sequence THD gradients.
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


LENS = [1, 63, 64, 65, 200, 129, 3, 0, 130, 77]


def i32(x, dev):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=dev)


def gather_rows(cu, spans):
    """Packed token indices of spans [(start, n)] (sequence-relative) of every sequence."""
    return np.concatenate([np.arange(cu[s] + a, cu[s] + a + n) for s, (a, n) in enumerate(spans)] +
                          [np.zeros(0, np.int64)]).astype(np.int64)


def cu_of(spans):
    return np.concatenate([[0], np.cumsum([n for _, n in spans])]).astype(np.int64)


def step_cases(lens, seed):
    """Per sequence: (query span, key span) with a mix of geometries."""
    rng = np.random.default_rng(seed)
    qs, ks = [], []
    for s, L in enumerate(lens):
        kind = s % 5
        if L == 0:
            qs.append((0, 0)); ks.append((0, 0))
            continue
        a = int(rng.integers(0, L))
        n = int(rng.integers(1, L - a + 1))
        if kind == 0:        # the whole causal prefix of the rows: more keys than rows
            qs.append((a, n)); ks.append((0, a + n))
        elif kind == 1:      # a key block that starts inside the rows
            ka = int(rng.integers(0, a + n)); qs.append((a, n)); ks.append((ka, int(rng.integers(0, L - ka + 1))))
        elif kind == 2:      # rows without keys
            qs.append((a, n)); ks.append((min(a, L - 1), 0))
        elif kind == 3:      # keys without rows
            qs.append((a, 0)); ks.append((0, L))
        else:                # keys all after the rows (every row sees none of them)
            n = max(1, min(n, L - 1 - a)) if a < L - 1 else 1
            qs.append((a, n)); ks.append((min(a + n, L - 1), L - min(a + n, L - 1)))
    return qs, ks


def thd_step(tk, inp, p, qs, ks, with_branch, dev, bwd=None):
    """Runs one packed step; returns the host arrays the oracle takes and the GPU results."""
    cu = inp.cu_host
    qr, kr = gather_rows(cu, qs), gather_rows(cu, ks)
    ccu, kcu = cu_of(qs), cu_of(ks)
    qo, ko = [a for a, _ in qs], [a for a, _ in ks]
    geo = dict(cu_seqlens=i32(ccu, dev), kv_cu_seqlens=i32(kcu, dev), q_offsets=i32(qo, dev),
               kv_offsets=i32(ko, dev), max_position=max(inp.lengths) + p, check_cu_seqlens=True)
    iq, ik = torch.as_tensor(qr, device=dev), torch.as_tensor(kr, device=dev)
    gq = inp.gq[p].index_select(0, iq)
    sk = [inp.gk[0].index_select(0, ik)] + [k.index_select(0, iq) for k in inp.gk[1:p]]
    sv = [inp.gv[0].index_select(0, ik)] + [v.index_select(0, iq) for v in inp.gv[1:p]]
    host = dict(q=inp.q[p][qr], k0=inp.k[0][kr], v0=inp.v[0][kr],
                bk=[k[qr] for k in inp.k[1:p]] if with_branch else None,
                bv=[v[qr] for v in inp.v[1:p]] if with_branch else None,
                geo=dict(cu_seqlens=ccu, kv_cu_seqlens=kcu, q_offsets=qo, kv_offsets=ko), qr=qr, kr=kr)
    if bwd is None:
        o, l = tk.fwd_chunk(gq, sk, sv, p, with_branch=with_branch, rope_base=inp.w.rope_base, **geo)
        return host, (o, l)
    go, gl, gdo = bwd
    res = tk.bwd_chunk(gq, sk, sv, go.index_select(0, iq), gl.index_select(1, iq), gdo.index_select(0, iq), p,
                       with_branch=with_branch, rope_base=inp.w.rope_base, **geo)
    return host, res


def test_thd_steps_match_oracle_step(dev, tk):
    """Single packed steps (ten sequences, five geometries), with and without the branch."""
    w = syn.Workload("thd_step", 31, "thd", 1, sum(LENS), 8, 2, 128, 3, "bf16", 1e6, False)
    inp = Inputs(w, dev, with_grad=False, lengths=LENS)
    p = 3
    for seed, br in ((0, True), (1, False), (2, True)):
        qs, ks = step_cases(LENS, 40 + seed)
        host, (o, l) = thd_step(tk, inp, p, qs, ks, br, dev)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd_chunk_thd(host["q"], host["k0"], host["v0"], host["bk"], host["bv"], p,
                                       base=w.rope_base, **host["geo"])
        og, lg = to_np(o), to_np(l)
        empty = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(lg), empty), seed
        assert np.all(og[empty.T] == 0)
        eo, el = max_abs(og, o_ref), max_abs(lg[~empty], l_ref[~empty])
        print(f"thd step seed {seed} branch={br}: {len(host['qr'])} rows, {len(host['kr'])} keys, "
              f"O {eo:.3e} LSE {el:.3e}, rows without keys {int(empty.any(0).sum())}")
        assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


def test_thd_bwd_steps_match_oracle_step(dev, tk):
    """Backward terms of packed steps, fed the oracle's whole-sequence O (bf16) and LSE; keys of a
    sequence without rows, and keys no row sees, get exact zeros."""
    w = syn.Workload("thd_bstep", 32, "thd", 1, sum(LENS), 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev, lengths=LENS)
    p = 3
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="thd", cu_seqlens=inp.cu_host, base=w.rope_base)
    o16 = syn.round_bf16(o_ref.astype(np.float32))
    go = torch.from_numpy(o16).to(dev).to(torch.bfloat16)
    gl = torch.from_numpy(np.ascontiguousarray(l_ref, dtype=np.float32)).to(dev)
    for seed, br in ((0, True), (1, False)):
        qs, ks = step_cases(LENS, 50 + seed)
        host, (dq, dks, dvs) = thd_step(tk, inp, p, qs, ks, br, dev, bwd=(go, gl, inp.gdo[p]))
        torch.cuda.synchronize()
        qr = host["qr"]
        rq, rk0, rv0, rkb, rvb = O.bwd_chunk_thd(host["q"], host["k0"], host["v0"], host["bk"], host["bv"], p,
                                                 inp.do[p][qr], o16[qr], l_ref[:, qr], base=w.rope_base,
                                                 **host["geo"])
        pairs = [("dq", dq, rq), ("dk1", dks[0], rk0), ("dv1", dvs[0], rv0)]
        pairs += [(f"dk{t + 2}", dks[1 + t], rkb[t]) for t in range(len(rkb))]
        pairs += [(f"dv{t + 2}", dvs[1 + t], rvb[t]) for t in range(len(rvb))]
        errs = []
        for name, g, r in pairs:
            g = to_np(g)
            assert g.shape == r.shape, (name, g.shape, r.shape)
            zero = ~np.any(r.reshape(r.shape[0], -1), axis=1)      # rows / keys with no term at all
            assert not np.any(g[zero]), (seed, name)
            e = rel_fro(g, r)
            errs.append(f"{name}={e:.1e}")
            assert e <= TOL["bf16"]["grad"], (seed, name, e)
        print(f"thd bwd step seed {seed} branch={br}: " + " ".join(errs))


def zigzag_thd(tk, inp, p, cp, dev, o=None, lse=None):
    """Zig-zag ring over packed sequences: sequence s is cut into 2 cp chunks ([c L // 2cp,
    (c+1) L // 2cp)), and step (qc, kc) packs chunk qc's rows and chunk kc's keys of every
    sequence.  Forward (o is None): the rows' results joined with the merge kernel into fp32.
    Backward: every step's terms summed into whole-sequence fp32 gradients."""
    lens = inp.lengths
    nc = 2 * cp
    spans = lambda c: [(c * L // nc, (c + 1) * L // nc - c * L // nc) for L in lens]
    T, Hq, D = inp.q[p].shape
    if o is None:
        out_o = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
        out_l = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    else:
        gq = torch.zeros((T, Hq, D), dtype=torch.float32, device=dev)
        gk = [torch.zeros(inp.gk[0].shape, dtype=torch.float32, device=dev) for _ in range(p)]
        gv = [torch.zeros(inp.gv[0].shape, dtype=torch.float32, device=dev) for _ in range(p)]
    for qc in range(nc):
        qs = spans(qc)
        qr = torch.as_tensor(gather_rows(inp.cu_host, qs), device=dev)
        ccu = i32(cu_of(qs), dev)
        if o is None:
            acc_o = torch.zeros((len(qr), Hq, D), dtype=torch.float32, device=dev)
            acc_l = torch.full((Hq, len(qr)), -float("inf"), dtype=torch.float32, device=dev)
        for kc in range(nc):
            ks = spans(kc)
            if o is None:
                _, (so, sl) = thd_step(tk, inp, p, qs, ks, kc == qc, dev)
                tk.merge(acc_o, acc_l, so, sl, out=acc_o, lse=acc_l, cu_seqlens=ccu)
            else:
                host, (dq, dks, dvs) = thd_step(tk, inp, p, qs, ks, kc == qc, dev, bwd=(o, lse, inp.gdo[p]))
                kr = torch.as_tensor(host["kr"], device=dev)
                gq.index_add_(0, qr, dq)
                gk[0].index_add_(0, kr, dks[0])
                gv[0].index_add_(0, kr, dvs[0])
                for t in range(1, len(dks)):
                    gk[t].index_add_(0, qr, dks[t])
                    gv[t].index_add_(0, qr, dvs[t])
        if o is None:
            out_o.index_copy_(0, qr, acc_o)
            out_l.index_copy_(1, qr, acc_l)
    torch.cuda.synchronize()
    return (out_o, out_l) if o is None else (gq, gk, gv)


@pytest.mark.parametrize("p,cp", [(1, 2), (3, 2), (4, 3)])
def test_thd_zigzag_ring(dev, tk, p, cp):
    w = syn.Workload("thd_ring", 33, "thd", 1, sum(LENS), 8, 2, 128, 4, "bf16", 1e6, True)
    inp = Inputs(w, dev, lengths=LENS)
    ro, rl = zigzag_thd(tk, inp, p, cp, dev)
    so, sl = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **inp.kw())
    torch.cuda.synchronize()
    d_o, d_l = (ro - so).abs().max().item(), (rl - sl).abs().max().item()
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="thd", cu_seqlens=inp.cu_host, base=w.rope_base)
    eo, el = max_abs(to_np(ro), o_ref), max_abs(to_np(rl), l_ref)
    print(f"thd ring p={p} cp={cp}: vs single THD call O {d_o:.3e} LSE {d_l:.3e}; vs oracle O {eo:.3e} LSE {el:.3e}")
    assert max(d_o, eo) <= TOL["bf16"]["o"] and max(d_l, el) <= TOL["bf16"]["lse"]
    if p == 1:
        return
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **inp.kw())
    gq, gk, gv = zigzag_thd(tk, inp, p, cp, dev, o=o, lse=lse)
    sq, sk, sv = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **inp.kw())
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="thd", cu_seqlens=inp.cu_host,
                             base=w.rope_base)
    errs = {"dq": (rel_fro(to_np(gq), to_np(sq)), rel_fro(to_np(gq), dq_r))}
    for t in range(p):
        errs[f"dk{t + 1}"] = (rel_fro(to_np(gk[t]), to_np(sk[t])), rel_fro(to_np(gk[t]), dk_r[t]))
        errs[f"dv{t + 1}"] = (rel_fro(to_np(gv[t]), to_np(sv[t])), rel_fro(to_np(gv[t]), dv_r[t]))
    print(f"thd ring bwd p={p} cp={cp}: " + " ".join(f"{k}={a:.1e}/{b:.1e}" for k, (a, b) in errs.items()))
    for k, (a, b) in errs.items():
        assert a <= TOL["bf16"]["grad"] and b <= TOL["bf16"]["grad"], (k, a, b)


def test_thd_step_rejects_bad_kv_cu(dev, tk):
    """check_cu_seqlens also validates kv_cu_seqlens: it must end at the packed key rows."""
    w = syn.Workload("thd_bad", 34, "thd", 1, sum(LENS), 8, 2, 128, 2, "bf16", 1e6, False)
    inp = Inputs(w, dev, with_grad=False, lengths=LENS)
    qs = [(0, L) for L in LENS]
    kcu = cu_of(qs)
    kcu[-1] -= 1
    with pytest.raises(tk.TTTAttnError, match="kv_cu_seqlens"):
        tk.fwd_chunk(inp.gq[2], [inp.gk[0]], [inp.gv[0]], 2, with_branch=False, cu_seqlens=inp.cu,
                     kv_cu_seqlens=i32(kcu, dev), q_offsets=i32(np.zeros(len(LENS)), dev),
                     kv_offsets=i32(np.zeros(len(LENS)), dev), max_position=300, check_cu_seqlens=True)


def test_thd_ring_fullsize_thd_32k(dev, tk):
    """thd_32k (16 packed sequences of 256..4096 tokens, T = 32768, 32/8 heads) over a zig-zag ring of
    2 ranks (every sequence in 4 chunks) at pass 3: the ring's merged O and LSE against one
    whole-sequence THD call on every element and against the oracle on >= 4096 sampled rows (plus
    every sequence's first, second and last row); the backward terms summed over the ring against
    the whole-sequence backward on every element."""
    from ttt_cases import sample_rows
    w = syn.workload("thd_32k")
    inp = Inputs(w, dev, passes=w.K)
    p, cp = w.K, 2
    ro, rl = zigzag_thd(tk, inp, p, cp, dev)
    so, sl = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, **inp.kw())
    torch.cuda.synchronize()
    d_o, d_l = (ro - so).abs().max().item(), (rl - sl).abs().max().item()
    print(f"thd_32k ring cp={cp} p={p}: vs single THD call O {d_o:.3e} LSE {d_l:.3e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"]
    slices = inp.slices()
    eo = el = 0.0
    n = 0
    ro_np, rl_np = to_np(ro), to_np(rl)
    for (pp, s, h), rows in sample_rows(inp, 4096, 31, [p]).items():
        sl_ = slices[s]
        o_ref, l_ref = O.fwd_rows(inp.q[p], inp.k, inp.v, p, sl_, h, rows, layout="thd", Hq=w.Hq, Hkv=w.Hkv,
                                  scale=w.scale, base=w.rope_base)
        eo = max(eo, max_abs(ro_np[sl_.start + rows, h], o_ref))
        el = max(el, max_abs(rl_np[h, sl_.start + rows], l_ref))
        n += len(rows)
    print(f"thd_32k ring vs oracle on {n} sampled rows: O {eo:.3e} LSE {el:.3e}")
    assert n >= 4096 and eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, **inp.kw())
    gq, gk, gv = zigzag_thd(tk, inp, p, cp, dev, o=o, lse=lse)
    sq, sk, sv = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, **inp.kw())
    torch.cuda.synchronize()
    errs = [rel_fro(to_np(gq), to_np(sq))] + [rel_fro(to_np(gk[t]), to_np(sk[t])) for t in range(p)] + \
           [rel_fro(to_np(gv[t]), to_np(sv[t])) for t in range(p)]
    print(f"thd_32k ring bwd vs single THD call: worst rel Frobenius {max(errs):.2e}")
    assert max(errs) <= TOL["bf16"]["grad"]
