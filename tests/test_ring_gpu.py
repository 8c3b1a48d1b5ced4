"""Ring steps and the joint-LSE merge on the GPU (through the C ABI).

A zig-zag context-parallel ring is emulated on one GPU: the sequence is split
into 2*cp chunks, rank r owns query chunks r and 2*cp-1-r, and each query chunk
meets every pass-1 key chunk once (the branch keys are folded in once, on the
diagonal step); the partial results are joined with ttt_attn_merge into fp32
accumulators.  The joined result must match a single whole-sequence
ttt_attn_fwd call and the fp64 oracle; single steps are checked against the
oracle's ring step, and the merge kernel against the oracle's merge.
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


def zigzag_ring(tk, q, ks, vs, p, cp, rope_base, with_empty_steps=False):
    """(O fp32 [B,S,Hq,D], LSE [B,Hq,S]) of pass p joined over a zig-zag ring of cp ranks."""
    B, S, Hq, D = q.shape
    c = S // (2 * cp)
    assert c * 2 * cp == S
    out_o = torch.empty((B, S, Hq, D), dtype=torch.float32, device=q.device)
    out_l = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    for r in range(cp):
        for qc in (r, 2 * cp - 1 - r):
            qa = qc * c
            acc_o = torch.zeros((B, c, Hq, D), dtype=torch.float32, device=q.device)
            acc_l = torch.full((B, Hq, c), -float("inf"), dtype=torch.float32, device=q.device)
            for kc in range(2 * cp if with_empty_steps else qc + 1):
                ka = kc * c
                diag = kc == qc
                sk = [ks[0][:, ka:ka + c]] + [k[:, qa:qa + c] for k in ks[1:p]]
                sv = [vs[0][:, ka:ka + c]] + [v[:, qa:qa + c] for v in vs[1:p]]
                o, l = tk.fwd_chunk(q[:, qa:qa + c], sk, sv, p, q_offset=qa, kv_offset=ka, with_branch=diag,
                                    rope_base=rope_base)
                if kc > qc:
                    torch.cuda.synchronize()
                    assert torch.all(o == 0).item() and torch.all(l == -float("inf")).item()
                tk.merge(acc_o, acc_l, o, l, out=acc_o, lse=acc_l)
            out_o[:, qa:qa + c] = acc_o
            out_l[:, :, qa:qa + c] = acc_l
    torch.cuda.synchronize()
    return out_o, out_l


def check_ring(tk, inp, p, cp, label, oracle=True):
    w = inp.w
    ro, rl = zigzag_ring(tk, inp.gq[p], inp.gk, inp.gv, p, cp, w.rope_base, with_empty_steps=True)
    so, sl = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, rope_base=w.rope_base)
    torch.cuda.synchronize()
    d_o = (ro - so).abs().max().item()
    d_l = (rl - sl).abs().max().item()
    print(f"{label} p={p} cp={cp}: ring vs single call O {d_o:.3e} LSE {d_l:.3e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"]
    if oracle:
        o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=w.rope_base)
        eo, el = max_abs(to_np(ro), o_ref), max_abs(to_np(rl), l_ref)
        print(f"{label} p={p} cp={cp}: ring vs oracle O {eo:.3e} LSE {el:.3e}")
        assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("p,cp", [(1, 2), (3, 2), (3, 3)])
def test_ring_ragged_chunks(dev, tk, p, cp):
    # S = 600: chunks of 150 (cp=2) or 100 (cp=3) rows, neither a multiple of a tile; GQA 4:1
    w = syn.Workload("ring_small", 21, "bshd", 2, 600, 8, 2, 128, 3, "bf16", 1e6, False)
    inp = Inputs(w, dev, with_grad=False)
    check_ring(tk, inp, p, cp, "ring_small")


def test_ring_steps_match_oracle_step(dev, tk):
    """Single ring steps: diagonal with branch, full off-diagonal, a partial key block,
    a step whose keys all follow the rows (empty), and a zero-length key block."""
    w = syn.Workload("ring_step", 22, "bshd", 1, 384, 4, 2, 128, 4, "bf16", 1e6, False)
    inp = Inputs(w, dev, with_grad=False)
    p = 4
    cases = [  # (q_offset, n, kv_offset, m, with_branch)
        (128, 128, 128, 128, True),
        (256, 128, 0, 128, False),
        (200, 70, 150, 90, True),
        (0, 96, 100, 64, False),
        (0, 96, 100, 64, True),
        (40, 33, 40, 0, True),
    ]
    for qa, n, ka, m, br in cases:
        sk = [inp.gk[0][:, ka:ka + m]] + [k[:, qa:qa + n] for k in inp.gk[1:p]]
        sv = [inp.gv[0][:, ka:ka + m]] + [v[:, qa:qa + n] for v in inp.gv[1:p]]
        o, l = tk.fwd_chunk(inp.gq[p][:, qa:qa + n], sk, sv, p, q_offset=qa, kv_offset=ka, with_branch=br,
                            rope_base=w.rope_base)
        torch.cuda.synchronize()
        o_ref, l_ref = O.fwd_chunk(inp.q[p][:, qa:qa + n], inp.k[0][:, ka:ka + m], inp.v[0][:, ka:ka + m],
                                   [k[:, qa:qa + n] for k in inp.k[1:p]] if br else None,
                                   [v[:, qa:qa + n] for v in inp.v[1:p]] if br else None,
                                   p, q_offset=qa, kv_offset=ka, base=w.rope_base)
        og, lg = to_np(o), to_np(l)
        empty = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(lg), empty), (qa, n, ka, m, br)
        eo = max_abs(og, o_ref)
        el = max_abs(lg[~empty], l_ref[~empty])
        print(f"step q@{qa}+{n} kv@{ka}+{m} branch={br}: O {eo:.3e} LSE {el:.3e} empty rows {int(empty.sum())}")
        assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]
        assert np.all(og[np.transpose(empty, (0, 2, 1))] == 0)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_merge_kernel_matches_oracle(dev, tk, dtype):
    g = torch.Generator().manual_seed(23)
    B, n, H, D = 2, 77, 4, 128
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    oa = torch.randn((B, n, H, D), generator=g).to(tdt)
    ob = torch.randn((B, n, H, D), generator=g).to(tdt)
    la = torch.randn((B, H, n), generator=g) * 3
    lb = torch.randn((B, H, n), generator=g) * 3
    la[0, 1, :5] = -float("inf")          # one side empty
    lb[1, 2, 10:15] = -float("inf")
    la[1, 3, 20:24] = -float("inf")       # both sides empty
    lb[1, 3, 20:24] = -float("inf")
    oa[1, 20:24, 3] = 0
    ob[1, 20:24, 3] = 0
    ga, gb, gla, glb = oa.to(dev), ob.to(dev), la.to(dev), lb.to(dev)
    o, l = tk.merge(ga, gla, gb, glb)
    torch.cuda.synchronize()
    o_ref, l_ref = O.merge(oa.double().numpy(), la.double().numpy(), ob.double().numpy(), lb.double().numpy())
    og, lg = to_np(o), to_np(l)
    assert np.array_equal(np.isneginf(lg), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    el = max_abs(lg[fin], l_ref[fin])
    err = np.abs(og - o_ref)
    if dtype == "bf16":
        err = err - bf16_half_ulp(o_ref)
    print(f"merge {dtype}: O {err.max():.3e} LSE {el:.3e}")
    assert el <= 1e-5 and err.max() <= 1e-5
    # in place into o_a gives the same result
    o2, l2 = tk.merge(ga, gla, gb, glb, out=ga, lse=gla)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(l2, l)


def test_ring_fullsize_b4_s4k(dev, tk):
    """The B=4, S=4096, Hq=32, Hkv=8, K=7 workload over a 4-rank zig-zag ring (chunks of
    512 rows) at the last pass: ring vs single call on every element, and vs the oracle
    on sampled rows."""
    w = syn.workload("b4_s4k")
    inp = Inputs(w, dev, passes=w.K, with_grad=False)
    p, cp = w.K, 4
    ro, rl = zigzag_ring(tk, inp.gq[p], inp.gk, inp.gv, p, cp, w.rope_base)
    so, sl = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, o_fp32=True, rope_base=w.rope_base)
    torch.cuda.synchronize()
    d_o = (ro - so).abs().max().item()
    d_l = (rl - sl).abs().max().item()
    print(f"b4_s4k p={p} cp={cp}: ring vs single call O {d_o:.3e} LSE {d_l:.3e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"]
    rng = np.random.default_rng(24)
    eo = el = 0.0
    nrow = 0
    r = w.Hq // w.Hkv
    for b in range(w.B):
        sl_ = O.Slice(b, 0, w.S)
        for g in range(w.Hkv):
            # chunk borders of the ring (511/512, ...) plus random rows, 2 heads of the group
            rows = np.unique(np.concatenate([rng.integers(0, w.S, 72), [0, 511, 512, 1023, 1024, 3583, 3584, 4095]]))
            heads = {g * r + int(h): rows for h in rng.choice(r, 2, replace=False)}
            ref = O.fwd_group_rows(inp.q[p], inp.k, inp.v, p, sl_, g, heads, layout="bshd", Hq=w.Hq, Hkv=w.Hkv,
                                   scale=w.scale, base=w.rope_base)
            for h, (o_ref, l_ref) in ref.items():
                idx = torch.as_tensor(rows, device=dev)
                og = ro[b].index_select(0, idx)[:, h].double().cpu().numpy()
                lg = rl[b, h].index_select(0, idx).double().cpu().numpy()
                eo, el = max(eo, max_abs(og, o_ref)), max(el, max_abs(lg, l_ref))
                nrow += len(rows)
    print(f"b4_s4k ring vs oracle on {nrow} sampled rows: O {eo:.3e} LSE {el:.3e}")
    assert nrow >= 4096
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


# ----------------------------------------------------------------------------- ring backward
def zigzag_ring_bwd(tk, q, ks, vs, o, lse, dout, p, cp, rope_base, window=0):
    """Whole-sequence gradients of pass p summed from the backward terms of every step of a zig-zag
    ring of cp ranks (fp32 sums of fp32 terms); o/lse are the rows' whole-sequence outputs."""
    B, S, Hq, D = q.shape
    c = S // (2 * cp)
    gq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    gk = [torch.zeros(ks[0].shape, dtype=torch.float32, device=q.device) for _ in range(p)]
    gv = [torch.zeros(vs[0].shape, dtype=torch.float32, device=q.device) for _ in range(p)]
    for r in range(cp):
        for qc in (r, 2 * cp - 1 - r):
            qa = qc * c
            for kc in range(2 * cp):
                ka = kc * c
                diag = kc == qc
                sk = [ks[0][:, ka:ka + c]] + [k[:, qa:qa + c] for k in ks[1:p]]
                sv = [vs[0][:, ka:ka + c]] + [v[:, qa:qa + c] for v in vs[1:p]]
                dq, dks, dvs = tk.bwd_chunk(q[:, qa:qa + c], sk, sv, o[:, qa:qa + c], lse[:, :, qa:qa + c],
                                            dout[:, qa:qa + c], p, q_offset=qa, kv_offset=ka, with_branch=diag,
                                            rope_base=rope_base, window=window)
                gq[:, qa:qa + c] += dq
                gk[0][:, ka:ka + c] += dks[0]
                gv[0][:, ka:ka + c] += dvs[0]
                for t in range(1, len(dks)):
                    gk[t][:, qa:qa + c] += dks[t]
                    gv[t][:, qa:qa + c] += dvs[t]
    torch.cuda.synchronize()
    return gq, gk, gv


def test_ring_bwd_steps_match_oracle_step(dev, tk):
    """Single ring-step backward terms against the oracle's step terms, both fed the oracle's own
    whole-sequence O (rounded to bf16) and LSE: diagonal with branch, full off-diagonal, a partial
    key block, keys all after the rows (every term exactly 0), a zero-length key block (branch
    terms only) and a one-row chunk."""
    w = syn.Workload("ringb_step", 26, "bshd", 1, 192, 4, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    p = 3
    o_ref, l_ref = O.fwd(inp.q[p], inp.k, inp.v, p, layout="bshd", base=w.rope_base)
    o16 = syn.round_bf16(o_ref.astype(np.float32))
    go = torch.from_numpy(o16).to(dev).to(torch.bfloat16)
    gl = torch.from_numpy(np.ascontiguousarray(l_ref, dtype=np.float32)).to(dev)
    cases = [  # (q_offset, n, kv_offset, m, with_branch)
        (64, 64, 64, 64, True),
        (128, 64, 0, 64, False),
        (100, 35, 75, 45, True),
        (0, 48, 50, 32, False),
        (20, 17, 20, 0, True),
        (150, 1, 100, 51, True),
    ]
    for qa, n, ka, m, br in cases:
        sk = [inp.gk[0][:, ka:ka + m]] + [k[:, qa:qa + n] for k in inp.gk[1:p]]
        sv = [inp.gv[0][:, ka:ka + m]] + [v[:, qa:qa + n] for v in inp.gv[1:p]]
        dq, dks, dvs = tk.bwd_chunk(inp.gq[p][:, qa:qa + n], sk, sv, go[:, qa:qa + n], gl[:, :, qa:qa + n],
                                    inp.gdo[p][:, qa:qa + n], p, q_offset=qa, kv_offset=ka, with_branch=br,
                                    rope_base=w.rope_base)
        torch.cuda.synchronize()
        rq, rk0, rv0, rkb, rvb = O.bwd_chunk(
            inp.q[p][:, qa:qa + n], inp.k[0][:, ka:ka + m], inp.v[0][:, ka:ka + m],
            [k[:, qa:qa + n] for k in inp.k[1:p]] if br else None, [v[:, qa:qa + n] for v in inp.v[1:p]] if br else None,
            p, inp.do[p][:, qa:qa + n], o16[:, qa:qa + n], l_ref[:, :, qa:qa + n], q_offset=qa, kv_offset=ka,
            base=w.rope_base)
        pairs = [("dq", dq, rq), ("dk1", dks[0], rk0), ("dv1", dvs[0], rv0)]
        pairs += [(f"dk{t + 2}", dks[1 + t], rkb[t]) for t in range(len(rkb))]
        pairs += [(f"dv{t + 2}", dvs[1 + t], rvb[t]) for t in range(len(rvb))]
        assert len(dks) == 1 + len(rkb) and len(dvs) == 1 + len(rvb)
        errs = []
        for name, g, r in pairs:
            g = to_np(g)
            assert g.shape == r.shape, (name, g.shape, r.shape)
            if r.size == 0:
                continue
            if not np.any(r):
                assert not np.any(g), (qa, n, ka, m, br, name)  # a step without visible keys adds exactly 0
                errs.append(f"{name}=0")
                continue
            e = rel_fro(g, r)
            errs.append(f"{name}={e:.1e}")
            assert e <= TOL["bf16"]["grad"], (qa, n, ka, m, br, name, e)
        print(f"bwd step q@{qa}+{n} kv@{ka}+{m} branch={br}: " + " ".join(errs))


@pytest.mark.parametrize("cp,window", [(2, 0), (3, 0), (2, 100)])
def test_ring_bwd_ragged(dev, tk, cp, window):
    w = syn.Workload("ringb_small", 25, "bshd", 2, 600, 8, 2, 128, 3, "bf16", 1e6, True)
    inp = Inputs(w, dev)
    p = 3
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, rope_base=w.rope_base, window=window)
    gq, gk, gv = zigzag_ring_bwd(tk, inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, cp, w.rope_base, window)
    sq, sk, sv = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, rope_base=w.rope_base, window=window)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = O.bwd(inp.q[p], inp.k, inp.v, inp.do[p], p, layout="bshd", base=w.rope_base, window=window)
    errs = {"dq": (rel_fro(to_np(gq), to_np(sq)), rel_fro(to_np(gq), dq_r))}
    for t in range(p):
        errs[f"dk{t + 1}"] = (rel_fro(to_np(gk[t]), to_np(sk[t])), rel_fro(to_np(gk[t]), dk_r[t]))
        errs[f"dv{t + 1}"] = (rel_fro(to_np(gv[t]), to_np(sv[t])), rel_fro(to_np(gv[t]), dv_r[t]))
    print(f"ring bwd cp={cp} W={window}: " + " ".join(f"{k}={a:.1e}/{b:.1e}" for k, (a, b) in errs.items()))
    for k, (a, b) in errs.items():
        assert a <= TOL["bf16"]["grad"] and b <= TOL["bf16"]["grad"], (k, a, b)


def test_ring_bwd_fullsize_b4_s4k(dev, tk):
    """B=4, S=4096, K=7 at pass 7 over a 4-rank zig-zag ring: every gradient element summed from the
    ring's backward terms vs one whole-sequence backward (itself checked against the oracle)."""
    w = syn.workload("b4_s4k")
    inp = Inputs(w, dev, passes=w.K)
    p, cp = w.K, 4
    o, lse = tk.fwd(inp.gq[p], inp.gk, inp.gv, p, rope_base=w.rope_base)
    gq, gk, gv = zigzag_ring_bwd(tk, inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, cp, w.rope_base)
    sq, sk, sv = tk.bwd(inp.gq[p], inp.gk, inp.gv, o, lse, inp.gdo[p], p, rope_base=w.rope_base)
    torch.cuda.synchronize()
    errs = [rel_fro(to_np(gq), to_np(sq))] + [rel_fro(to_np(gk[t]), to_np(sk[t])) for t in range(p)] + \
           [rel_fro(to_np(gv[t]), to_np(sv[t])) for t in range(p)]
    print(f"b4_s4k ring bwd vs single call: worst rel Frobenius {max(errs):.2e}")
    assert max(errs) <= TOL["bf16"]["grad"]
    # and against the oracle: the ring-summed trunk dK/dV of one whole (batch, KV head)
    # slice (4096 keys, every row that sees them), and 512 sampled dQ rows of its heads
    b, g = 1, 3
    sl = O.Slice(b, 0, w.S)
    keys = np.arange(w.S)
    dk_ref, dv_ref = O.bwd_trunk_keys(inp.q[p], inp.k, inp.v, inp.do[p], p, sl, g, keys, layout="bshd", Hq=w.Hq,
                                      Hkv=w.Hkv, scale=w.scale, base=w.rope_base)
    rows = np.sort(np.random.default_rng(27).choice(w.S, 512, replace=False))
    dq_ref, _, _ = O.bwd_rows(inp.q[p], inp.k, inp.v, inp.do[p], p, sl, g, rows, layout="bshd", Hq=w.Hq, Hkv=w.Hkv,
                              scale=w.scale, base=w.rope_base, need_kv=False)
    r = w.Hq // w.Hkv
    e_k = rel_fro(to_np(gk[0][b, :, g]), dk_ref)
    e_v = rel_fro(to_np(gv[0][b, :, g]), dv_ref)
    gq_b = to_np(gq[b])
    e_q = rel_fro(np.stack([gq_b[rows, g * r + hh] for hh in range(r)]), dq_ref)
    print(f"b4_s4k ring bwd vs oracle: trunk dK {e_k:.2e} dV {e_v:.2e} over {w.S} keys, dQ {e_q:.2e} over {len(rows)} rows x {r} heads")
    assert max(e_k, e_v, e_q) <= TOL["bf16"]["grad"]
