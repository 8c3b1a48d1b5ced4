"""Pins of the fp64 oracle against things other than itself.

Each check derives the expected value independently: torch's fp64
scaled_dot_product_attention (a library routine) on keys rotated through the
complex-number form of rotate-half, closed forms, RoPE group identities, fp64
autograd of an independently written brute force, central finite
differences, and layout equivalences.  The last test plants mistakes in the
oracle (on the CPU) and checks that the pins catch each of them.
"""
import contextlib
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ttt_oracle as O

F64 = torch.float64


# ----------------------------------------------------------------------------- independent helpers
def rope_complex(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """Rotate-half RoPE written as complex multiplication: (x1 + i x2) * e^{i pos theta_k}."""
    if base == 0:
        return x.clone()
    D = x.shape[-1]
    theta = torch.tensor([math.pow(base, -2.0 * k / D) for k in range(D // 2)], dtype=F64)
    ang = pos.to(F64)[..., None] * theta
    z = torch.complex(x[..., : D // 2], x[..., D // 2:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def dense_reference(q, ks, vs, p, scale, base, requires_grad=False):
    """One sequence, BSHD with B=1 squeezed: q [S,Hq,D], ks/vs list of [S,Hkv,D] (torch fp64).

    Builds the concatenated keys [K1; K2; ...; Kp] rotated at their positions and
    the explicit boolean mask from tril/eye blocks, then calls torch's SDPA."""
    S, Hq, D = q.shape
    Hkv = ks[0].shape[1]
    r = Hq // Hkv
    i = torch.arange(S)
    qr = rope_complex(q, (i + p - 1)[:, None].expand(S, Hq), base)
    krs = [rope_complex(ks[0], i[:, None].expand(S, Hkv), base)]
    for t in range(1, p):
        krs.append(rope_complex(ks[t], (i + t)[:, None].expand(S, Hkv), base))
    kc = torch.cat(krs, 0)                     # [pS, Hkv, D]
    vc = torch.cat(list(vs[:p]), 0)
    mask = torch.cat([torch.tril(torch.ones(S, S, dtype=torch.bool))] +
                     [torch.eye(S, dtype=torch.bool)] * (p - 1), dim=1)   # [S, pS]
    qh = qr.permute(1, 0, 2)                                        # [Hq, S, D]
    kh = kc.permute(1, 0, 2).repeat_interleave(r, 0)
    vh = vc.permute(1, 0, 2).repeat_interleave(r, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    s = (qh @ kh.transpose(-1, -2)) * scale
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)  # [Hq, S]
    return o.permute(1, 0, 2), lse


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def make(S=13, Hq=4, Hkv=2, D=8, p=3, seed=0, B=None):
    shp_q = (S, Hq, D) if B is None else (B, S, Hq, D)
    shp_k = (S, Hkv, D) if B is None else (B, S, Hkv, D)
    q = rand(shp_q, seed)
    ks = [rand(shp_k, seed + 10 + t) for t in range(p)]
    vs = [rand(shp_k, seed + 20 + t) for t in range(p)]
    do = rand(shp_q, seed + 30)
    return q, ks, vs, do


# ----------------------------------------------------------------------------- pin checks (also run on planted mistakes)
def check_rope_complex_form():
    x = rand((5, 16), 1)
    pos = np.array([0, 1, 7, 100, 4097])
    for base in (1e4, 1e6):
        a = O.rotate_half(x, pos, base)
        b = rope_complex(torch.tensor(x), torch.tensor(pos), base).numpy()
        assert np.max(np.abs(a - b)) < 1e-12


def check_rope_single_pair():
    D, base = 16, 1e4
    for k in (0, 3, 7):
        e = np.zeros(D); e[k] = 1.0
        for m, n in ((5, 2), (40, 3), (9, 9)):
            s = O.rotate_half(e, m, base) @ O.rotate_half(e, n, base)
            assert abs(s - math.cos((m - n) * math.pow(base, -2.0 * k / D))) < 1e-12


def check_rope_group():
    x, y = rand((6, 32), 2), rand((6, 32), 3)
    base = 1e6
    m, n = np.array([0, 3, 50, 9, 1000, 31]), np.array([1, 1, 2, 40, 999, 0])
    assert np.max(np.abs(O.rotate_half(x, 0, base) - x)) == 0
    assert np.max(np.abs(O.unrotate_half(O.rotate_half(x, m, base), m, base) - x)) < 1e-12
    assert np.max(np.abs(O.rotate_half(O.rotate_half(x, m, base), n, base) - O.rotate_half(x, m + n, base))) < 1e-12
    for c in (1, 17, 32768):
        a = (O.rotate_half(x, m + c, base) * O.rotate_half(y, n + c, base)).sum(-1)
        b = (O.rotate_half(x, m, base) * O.rotate_half(y, n, base)).sum(-1)
        assert np.max(np.abs(a - b)) < 1e-12


def check_zero_query_closed_form(layout="bshd"):
    """Q = 0: every visible score is 0, so LSE_i = ln(i + p) and O_i is the mean of
    the visible value rows: V1[0..i] and Vq[i] for q = 2..p."""
    Hq, Hkv, D = 4, 2, 8
    lens = [7, 1, 12, 5]
    for p in (1, 2, 4):
        if layout == "bshd":
            B, S = 2, 9
            q = np.zeros((B, S, Hq, D))
            ks = [rand((B, S, Hkv, D), 40 + t) for t in range(p)]
            vs = [rand((B, S, Hkv, D), 50 + t) for t in range(p)]
            o, lse = O.fwd(q, ks, vs, p, layout="bshd", base=1e4)
            for b in range(B):
                for i in range(S):
                    for h in range(Hq):
                        g = h // (Hq // Hkv)
                        vis = [vs[0][b, j, g] for j in range(i + 1)] + [vs[t][b, i, g] for t in range(1, p)]
                        assert abs(lse[b, h, i] - math.log(i + p)) < 1e-12
                        assert np.max(np.abs(o[b, i, h] - np.mean(vis, axis=0))) < 1e-12
        else:
            cu = np.concatenate([[0], np.cumsum(lens)])
            T = int(cu[-1])
            q = np.zeros((T, Hq, D))
            ks = [rand((T, Hkv, D), 60 + t) for t in range(p)]
            vs = [rand((T, Hkv, D), 70 + t) for t in range(p)]
            o, lse = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=cu, base=1e6)
            for s in range(len(lens)):
                for i in range(lens[s]):
                    t0 = cu[s] + i
                    for h in range(Hq):
                        g = h // (Hq // Hkv)
                        vis = [vs[0][cu[s] + j, g] for j in range(i + 1)] + [vs[t][t0, g] for t in range(1, p)]
                        assert abs(lse[h, t0] - math.log(i + p)) < 1e-12
                        assert np.max(np.abs(o[t0, h] - np.mean(vis, axis=0))) < 1e-12


def check_sdpa_brute_force():
    """Any p, RoPE on or off: oracle == torch SDPA over concatenated keys with an explicit mask."""
    for p, base, (Hq, Hkv) in ((1, 1e4, (2, 1)), (2, 1e6, (4, 2)), (3, 1e4, (4, 4)), (5, 1e6, (6, 2)), (4, 0.0, (2, 2))):
        q, ks, vs, _ = make(S=11, Hq=Hq, Hkv=Hkv, D=8, p=p, seed=p)
        scale = 0.3
        o, lse = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=[0, 11], scale=scale, base=base)
        ro, rl = dense_reference(torch.tensor(q), [torch.tensor(k) for k in ks], [torch.tensor(v) for v in vs],
                                 p, scale, base)
        assert np.max(np.abs(o - ro.numpy())) < 1e-12
        assert np.max(np.abs(lse - rl.numpy())) < 1e-12


def check_p1_is_causal_sdpa():
    q, ks, vs, _ = make(S=17, Hq=4, Hkv=2, D=16, p=1, seed=5)
    base = 1e6
    o, lse = O.fwd(q, ks, vs, 1, layout="thd", cu_seqlens=[0, 17], base=base)
    i = torch.arange(17)
    qr = rope_complex(torch.tensor(q), i[:, None].expand(17, 4), base).permute(1, 0, 2)
    kr = rope_complex(torch.tensor(ks[0]), i[:, None].expand(17, 2), base).permute(1, 0, 2).repeat_interleave(2, 0)
    vh = torch.tensor(vs[0]).permute(1, 0, 2).repeat_interleave(2, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vh, is_causal=True)
    assert np.max(np.abs(o - ref.permute(1, 0, 2).numpy())) < 1e-12


def check_merge_invariant():
    """Trunk-only causal softmax and branch-only softmax, merged by logaddexp, equal the oracle."""
    S, Hq, Hkv, D, p, base = 10, 2, 1, 8, 4, 1e4
    q, ks, vs, _ = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=7)
    scale = 1 / math.sqrt(D)
    o, lse = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=[0, S], scale=scale, base=base)
    i = torch.arange(S)
    qt = torch.tensor(q)
    for h in range(Hq):
        qr = rope_complex(qt[:, h], i + p - 1, base)                       # [S, D]
        kt = rope_complex(torch.tensor(ks[0][:, 0]), i, base)
        st = (qr @ kt.T * scale).masked_fill(~torch.tril(torch.ones(S, S, dtype=torch.bool)), -math.inf)
        lt = torch.logsumexp(st, -1)
        ot = torch.softmax(st, -1) @ torch.tensor(vs[0][:, 0])
        sb = torch.stack([(qr * rope_complex(torch.tensor(ks[t][:, 0]), i + t, base)).sum(-1) * scale
                          for t in range(1, p)], -1)                        # [S, p-1]
        lb = torch.logsumexp(sb, -1)
        ob = (torch.softmax(sb, -1)[..., None] * torch.stack([torch.tensor(vs[t][:, 0]) for t in range(1, p)], 1)).sum(1)
        l = torch.logaddexp(lt, lb)
        om = torch.exp(lt - l)[:, None] * ot + torch.exp(lb - l)[:, None] * ob
        assert np.max(np.abs(lse[h] - l.numpy())) < 1e-12
        assert np.max(np.abs(o[:, h] - om.numpy())) < 1e-12


def check_branch_relative_position():
    """Branch score of pass q at pass p depends on p - q only: shifting every row's
    position leaves it unchanged (rows i and i' with equal data give equal scores)."""
    D, base, p = 16, 1e6, 5
    S = 6
    q1 = rand((1, 1, D), 80)
    k1 = [rand((1, 1, D), 81 + t) for t in range(p)]
    q = np.repeat(q1, S, axis=0); ks = [np.repeat(k, S, axis=0) for k in k1]; vs = [np.ones((S, 1, D)) * t for t in range(p)]
    ks[0] = np.zeros((S, 1, D))  # zero trunk keys: every trunk score is 0
    lse_rows = []
    o, lse = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=[0, S], base=base)
    # remove the trunk's (i+1) zero-score terms: exp(lse) - (i + 1) = sum of branch exps
    for i in range(S):
        lse_rows.append(math.log(math.exp(lse[0, i]) - (i + 1)))
    assert max(lse_rows) - min(lse_rows) < 1e-12


def check_grad_autograd():
    for p, (Hq, Hkv), base in ((1, (2, 1), 1e4), (3, (4, 2), 1e6), (4, (2, 2), 0.0)):
        S, D = 9, 8
        q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=11 + p)
        scale = 0.4
        dq, dk, dv = O.bwd(q, ks, vs, do, p, layout="thd", cu_seqlens=[0, S], scale=scale, base=base)
        qt = torch.tensor(q, requires_grad=True)
        kt = [torch.tensor(k, requires_grad=True) for k in ks]
        vt = [torch.tensor(v, requires_grad=True) for v in vs]
        ro, _ = dense_reference(qt, kt, vt, p, scale, base)
        (ro * torch.tensor(do)).sum().backward()
        assert np.max(np.abs(dq - qt.grad.numpy())) < 1e-10
        for t in range(p):
            assert np.max(np.abs(dk[t] - kt[t].grad.numpy())) < 1e-10
            assert np.max(np.abs(dv[t] - vt[t].grad.numpy())) < 1e-10


def check_grad_finite_difference():
    S, Hq, Hkv, D, p, base = 6, 2, 1, 4, 3, 1e4
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=21)
    kw = dict(layout="thd", cu_seqlens=[0, S], scale=0.5, base=base)
    dq, dk, dv = O.bwd(q, ks, vs, do, p, **kw)

    def loss(q_, ks_, vs_):
        o, _ = O.fwd(q_, ks_, vs_, p, **kw)
        return float((o * do).sum())

    h = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(6):
        idx = tuple(int(rng.integers(n)) for n in q.shape)
        qp, qm = q.copy(), q.copy(); qp[idx] += h; qm[idx] -= h
        fd = (loss(qp, ks, vs) - loss(qm, ks, vs)) / (2 * h)
        assert abs(fd - dq[idx]) <= 1e-7 * max(1.0, abs(fd))
        t = int(rng.integers(p))
        idx = tuple(int(rng.integers(n)) for n in ks[0].shape)
        for arr, grad in ((ks, dk), (vs, dv)):
            ap = [a.copy() for a in arr]; am = [a.copy() for a in arr]
            ap[t][idx] += h; am[t][idx] -= h
            if arr is ks:
                fd = (loss(q, ap, vs) - loss(q, am, vs)) / (2 * h)
            else:
                fd = (loss(q, ks, ap) - loss(q, ks, am)) / (2 * h)
            assert abs(fd - grad[t][idx]) <= 1e-7 * max(1.0, abs(fd))


def check_thd_equals_bshd():
    B, S, Hq, Hkv, D, p, base = 3, 7, 4, 2, 8, 3, 1e6
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=31, B=B)
    o1, l1 = O.fwd(q, ks, vs, p, layout="bshd", base=base)
    cu = [0, 7, 14, 21]
    flat = lambda x: x.reshape(B * S, *x.shape[2:])
    o2, l2 = O.fwd(flat(q), [flat(k) for k in ks], [flat(v) for v in vs], p, layout="thd", cu_seqlens=cu, base=base)
    assert np.max(np.abs(flat(o1) - o2)) == 0
    assert np.max(np.abs(l1.transpose(1, 0, 2).reshape(Hq, B * S) - l2)) == 0
    g1 = O.bwd(q, ks, vs, do, p, layout="bshd", base=base)
    g2 = O.bwd(flat(q), [flat(k) for k in ks], [flat(v) for v in vs], flat(do), p, layout="thd", cu_seqlens=cu, base=base)
    assert np.max(np.abs(flat(g1[0]) - g2[0])) == 0
    for t in range(p):
        assert np.max(np.abs(flat(g1[1][t]) - g2[1][t])) == 0
        assert np.max(np.abs(flat(g1[2][t]) - g2[2][t])) == 0


def check_thd_isolation():
    lens = [5, 8, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, D, p = int(cu[-1]), 2, 1, 8, 3
    q, ks, vs, do = make(S=T, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=41)
    o1, l1 = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=cu, base=1e4)
    q2, ks2, vs2 = q.copy(), [k.copy() for k in ks], [v.copy() for v in vs]
    sl = slice(cu[1], cu[2])
    q2[sl] += 1.0; ks2[0][sl] -= 2.0; ks2[2][sl] *= 3.0; vs2[0][sl] += 5.0; vs2[1][sl] -= 1.0
    o2, l2 = O.fwd(q2, ks2, vs2, p, layout="thd", cu_seqlens=cu, base=1e4)
    keep = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    assert np.array_equal(o1[keep], o2[keep]) and np.array_equal(l1[:, keep], l2[:, keep])
    assert not np.allclose(o1[sl], o2[sl])


def check_gqa_is_repeated_kv():
    S, Hq, Hkv, D, p = 8, 6, 2, 8, 3
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=51)
    kw = dict(layout="thd", cu_seqlens=[0, S], base=1e6)
    o1, l1 = O.fwd(q, ks, vs, p, **kw)
    rep = lambda x: np.repeat(x, Hq // Hkv, axis=1)
    o2, l2 = O.fwd(q, [rep(k) for k in ks], [rep(v) for v in vs], p, **kw)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14
    g1 = O.bwd(q, ks, vs, do, p, **kw)
    g2 = O.bwd(q, [rep(k) for k in ks], [rep(v) for v in vs], do, p, **kw)
    assert np.max(np.abs(g1[0] - g2[0])) < 1e-13
    for t in range(p):
        sumg = lambda x: x.reshape(S, Hkv, Hq // Hkv, D).sum(2)
        assert np.max(np.abs(g1[1][t] - sumg(g2[1][t]))) < 1e-13
        assert np.max(np.abs(g1[2][t] - sumg(g2[2][t]))) < 1e-13


def check_sampled_rows_match_full():
    """bwd_rows over a row subset gives exact key gradients for keys all of whose rows are included."""
    S, Hq, Hkv, D, p, base = 12, 4, 2, 8, 3, 1e6
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=61)
    kw = dict(layout="thd", Hq=Hq, Hkv=Hkv, scale=1 / math.sqrt(D), base=base)
    dQ, dK, dV = O.bwd(q, ks, vs, do, p, layout="thd", cu_seqlens=[0, S], base=base)
    sl = O.Slice(0, 0, S)
    rows = np.arange(8, S)
    dq, dk, dv = O.bwd_rows(q, ks, vs, do, p, sl, 1, rows, **kw)
    assert np.max(np.abs(dq[0] - dQ[8:, 2])) < 1e-13
    assert np.max(np.abs(dk[8:S] - dK[0][8:, 1])) < 1e-13           # trunk keys j >= 8
    assert np.max(np.abs(dv[S + 8: 2 * S] - dV[1][8:, 1])) < 1e-13  # branch keys of pass 2 at rows >= 8
    o, l = O.fwd_rows(q, ks, vs, p, sl, 3, [0, 5, 11], layout="thd", Hq=Hq, Hkv=Hkv, scale=1 / math.sqrt(D), base=base)
    of, lf = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=[0, S], base=base)
    assert np.max(np.abs(o - of[[0, 5, 11], 3])) < 1e-14 and np.max(np.abs(l - lf[3, [0, 5, 11]])) < 1e-14


def _dense_bshd(q, ks, vs, p, scale, base):
    """dense_reference for a B=1 BSHD batch, returned as (O [S, Hq, D], LSE [Hq, S]) numpy."""
    o, l = dense_reference(torch.tensor(q[0]), [torch.tensor(k[0]) for k in ks], [torch.tensor(v[0]) for v in vs],
                           p, scale, base)
    return o.numpy(), l.numpy()


def check_chunk_rows_match_dense():
    """A ring step whose key block is the whole causal prefix (with the branch) gives
    exactly the dense masked-softmax rows; row and key offsets shift positions only."""
    S, Hq, Hkv, D, p, base, scale = 12, 4, 2, 8, 3, 1e4, 0.4
    q, ks, vs, _ = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=71, B=1)
    ro, rl = _dense_bshd(q, ks, vs, p, scale, base)
    a, n = 5, 4                                  # rows 5..8 against keys 0..8
    o, l = O.fwd_chunk(q[:, a:a + n], ks[0][:, :a + n], vs[0][:, :a + n], [k[:, a:a + n] for k in ks[1:]],
                       [v[:, a:a + n] for v in vs[1:]], p, q_offset=a, kv_offset=0, scale=scale, base=base)
    assert np.max(np.abs(o[0] - ro[a:a + n])) < 1e-12
    assert np.max(np.abs(l[0] - rl[:, a:a + n])) < 1e-12


def check_chunk_ring_partition():
    """Zig-zag ring: split the sequence into 2c chunks, rank r owning query chunks r and
    2c-1-r; merging every rank's steps over all key chunks (branch folded in once, on
    the diagonal step) gives the dense result."""
    S, Hq, Hkv, D, p, base, scale, cp = 16, 2, 1, 8, 4, 1e6, 0.35, 2
    q, ks, vs, _ = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=73, B=1)
    ro, rl = _dense_bshd(q, ks, vs, p, scale, base)
    c = S // (2 * cp)
    for r in range(cp):
        for qc in (r, 2 * cp - 1 - r):
            qa = qc * c
            acc_o = np.zeros((1, c, Hq, D)); acc_l = np.full((1, Hq, c), -np.inf)
            for kc in range(2 * cp):
                ka = kc * c
                br = kc == qc
                o, l = O.fwd_chunk(q[:, qa:qa + c], ks[0][:, ka:ka + c], vs[0][:, ka:ka + c],
                                   [k[:, qa:qa + c] for k in ks[1:]] if br else None,
                                   [v[:, qa:qa + c] for v in vs[1:]] if br else None,
                                   p, q_offset=qa, kv_offset=ka, scale=scale, base=base)
                if kc > qc:
                    assert np.all(l == -np.inf) and np.all(o == 0)
                acc_o, acc_l = O.merge(acc_o, acc_l, o, l)
            assert np.max(np.abs(acc_o[0] - ro[qa:qa + c])) < 1e-12
            assert np.max(np.abs(acc_l[0] - rl[:, qa:qa + c])) < 1e-12


def check_merge_closed_form():
    """Two single-key partial results: merged O is the two-way softmax average of the
    values and LSE is log(e^s1 + e^s2); -inf partners leave the other side unchanged."""
    rng = np.random.default_rng(75)
    s1, s2 = rng.standard_normal((1, 3, 5)), rng.standard_normal((1, 3, 5))
    v1, v2 = rng.standard_normal((1, 5, 3, 4)), rng.standard_normal((1, 5, 3, 4))
    o, l = O.merge(v1, s1, v2, s2)
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    w1r = np.transpose(w1, (0, 2, 1))[..., None]
    assert np.max(np.abs(o - (w1r * v1 + (1 - w1r) * v2))) < 1e-14
    assert np.max(np.abs(l - np.log(np.exp(s1) + np.exp(s2)))) < 1e-14
    ninf = np.full_like(s1, -np.inf)
    o2, l2 = O.merge(v1, s1, np.zeros_like(v2), ninf)
    assert np.array_equal(l2, s1) and np.max(np.abs(o2 - v1)) < 1e-15
    o3, l3 = O.merge(np.zeros_like(v1), ninf, np.zeros_like(v2), ninf)
    assert np.all(l3 == -np.inf) and np.all(o3 == 0)


def _block_case(B=1, ctx_len=11, bs=4, nblk=3, Hq=4, Hkv=2, D=8, seed=81):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, nblk * bs, Hq, D))
    kb = rng.standard_normal((B, nblk * bs, Hkv, D))
    vb = rng.standard_normal((B, nblk * bs, Hkv, D))
    kc = rng.standard_normal((B, ctx_len, Hkv, D))
    vc = rng.standard_normal((B, ctx_len, Hkv, D))
    return q, kc, vc, kb, vb


def check_block_sdpa_mask():
    """Block drafting == torch SDPA over [context keys ; block keys] rotated at their
    positions with an explicit mask (context j < anchor, whole own block), incl.
    anchors 0 (no context) and ctx_len (whole context)."""
    ctx_len, bs, nblk, Hq, Hkv, D, base, scale = 11, 4, 4, 4, 2, 8, 1e4, 0.3
    q, kc, vc, kb, vb = _block_case(ctx_len=ctx_len, bs=bs, nblk=nblk, Hq=Hq, Hkv=Hkv, D=D)
    anchors = np.array([[0, 3, 7, ctx_len]])
    o, lse = O.block_fwd(q, kc, vc, kb, vb, anchors, bs, scale=scale, base=base)
    N = nblk * bs
    rows = torch.arange(N)
    slot_pos = torch.tensor([int(anchors[0, r // bs]) + r % bs for r in range(N)])
    qr = rope_complex(torch.tensor(q[0]), slot_pos[:, None].expand(N, Hq), base)
    kcr = rope_complex(torch.tensor(kc[0]), torch.arange(ctx_len)[:, None].expand(ctx_len, Hkv), base)
    kbr = rope_complex(torch.tensor(kb[0]), slot_pos[:, None].expand(N, Hkv), base)
    keys = torch.cat([kcr, kbr], 0)
    vals = torch.cat([torch.tensor(vc[0]), torch.tensor(vb[0])], 0)
    anc = torch.tensor([int(anchors[0, r // bs]) for r in range(N)])
    mask = torch.cat([torch.arange(ctx_len)[None, :] < anc[:, None],
                      (rows[None, :] // bs) == (rows[:, None] // bs)], dim=1)          # [N, ctx_len + N]
    r = Hq // Hkv
    qh = qr.permute(1, 0, 2)
    kh = keys.permute(1, 0, 2).repeat_interleave(r, 0)
    vh = vals.permute(1, 0, 2).repeat_interleave(r, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    sc = (qh @ kh.transpose(-1, -2)) * scale
    rl = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)
    assert np.max(np.abs(o[0] - ref.permute(1, 0, 2).numpy())) < 1e-12
    assert np.max(np.abs(lse[0] - rl.numpy())) < 1e-12


def check_block_zero_query_closed_form():
    """Zero queries: every score is 0, so LSE = ln(visible context keys + bs) and O is
    the mean of the visible values (pins the cut at the anchor exactly)."""
    ctx_len, bs, nblk = 9, 2, 5
    q, kc, vc, kb, vb = _block_case(ctx_len=ctx_len, bs=bs, nblk=nblk, Hq=2, Hkv=1, D=8, seed=83)
    q[:] = 0
    anchors = np.array([[0, 1, 4, 8, 9]])
    o, lse = O.block_fwd(q, kc, vc, kb, vb, anchors, bs, base=1e6)
    for r in range(nblk * bs):
        a = int(anchors[0, r // bs])
        blk = r // bs
        vis = np.concatenate([vc[0, :a, 0], vb[0, blk * bs:(blk + 1) * bs, 0]], axis=0)
        for h in range(2):
            assert abs(lse[0, h, r] - math.log(a + bs)) < 1e-12
            assert np.max(np.abs(o[0, r, h] - vis.mean(axis=0))) < 1e-12


def check_block_size1_is_causal():
    """One slot per block anchored at its own row, with the block key/value equal to the
    context key/value of that row: causal attention of row i over rows 0..i."""
    S, Hq, Hkv, D, base = 10, 4, 2, 8, 1e6
    q, ks, vs, _ = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=1, seed=85, B=1)
    anchors = np.arange(S)[None, :]
    o, lse = O.block_fwd(q, ks[0], vs[0], ks[0], vs[0], anchors, 1, base=base)
    ro, rl = _dense_bshd(q, ks, vs, 1, 1 / math.sqrt(D), base)
    assert np.max(np.abs(o[0] - ro)) < 1e-12 and np.max(np.abs(lse[0] - rl)) < 1e-12


def check_block_grad_autograd():
    """Block-draft gradients == fp64 torch autograd through SDPA over [context ; block]
    keys with the explicit block mask (GQA, anchors 0 .. ctx_len)."""
    ctx_len, bs, nblk, Hq, Hkv, D, base = 9, 4, 4, 4, 2, 8, 1e4
    q, kc, vc, kb, vb = _block_case(ctx_len=ctx_len, bs=bs, nblk=nblk, Hq=Hq, Hkv=Hkv, D=D, seed=87)
    dout = np.random.default_rng(88).standard_normal(q.shape)
    anchors = np.array([[0, 2, 6, ctx_len]])
    scale = 1 / math.sqrt(D)
    got = O.block_bwd(q, kc, vc, kb, vb, anchors, bs, dout, base=base)
    N, r = nblk * bs, Hq // Hkv
    T = [torch.tensor(x[0], requires_grad=True) for x in (q, kc, vc, kb, vb)]
    tq, tkc, tvc, tkb, tvb = T
    slot_pos = torch.tensor([int(anchors[0, i // bs]) + i % bs for i in range(N)])
    qr = rope_complex(tq, slot_pos[:, None].expand(N, Hq), base)
    keys = torch.cat([rope_complex(tkc, torch.arange(ctx_len)[:, None].expand(ctx_len, Hkv), base),
                      rope_complex(tkb, slot_pos[:, None].expand(N, Hkv), base)], 0)
    vals = torch.cat([tvc, tvb], 0)
    anc = torch.tensor([int(anchors[0, i // bs]) for i in range(N)])
    rows = torch.arange(N)
    mask = torch.cat([torch.arange(ctx_len)[None, :] < anc[:, None], (rows[None, :] // bs) == (rows[:, None] // bs)], 1)
    out = torch.nn.functional.scaled_dot_product_attention(
        qr.permute(1, 0, 2), keys.permute(1, 0, 2).repeat_interleave(r, 0),
        vals.permute(1, 0, 2).repeat_interleave(r, 0), attn_mask=mask, scale=scale).permute(1, 0, 2)
    (out * torch.tensor(dout[0])).sum().backward()
    for mine, t in zip(got, T):
        assert np.max(np.abs(mine[0] - t.grad.numpy())) < 1e-10


def _block_torch_ref(q, kc, vc, kb, vb, anchors, bs, scale, base):
    """One sequence, torch fp64 with autograd: SDPA over [context ; block] keys rotated at
    their positions with the explicit block mask; anchors clamped to [0, ctx_len]."""
    N, Hq, _ = q.shape
    ctx_len, Hkv = kc.shape[0], kc.shape[1]
    T = [torch.tensor(x, requires_grad=True) for x in (q, kc, vc, kb, vb)]
    tq, tkc, tvc, tkb, tvb = T
    anc = torch.tensor([min(max(int(anchors[i // bs]), 0), ctx_len) for i in range(N)])
    slot_pos = anc + torch.arange(N) % bs
    keys = torch.cat([rope_complex(tkc, torch.arange(ctx_len)[:, None].expand(ctx_len, Hkv), base),
                      rope_complex(tkb, slot_pos[:, None].expand(N, Hkv), base)], 0)
    vals = torch.cat([tvc, tvb], 0)
    rows = torch.arange(N)
    mask = torch.cat([torch.arange(ctx_len)[None, :] < anc[:, None], (rows[None, :] // bs) == (rows[:, None] // bs)], 1)
    r = Hq // Hkv
    qh = rope_complex(tq, slot_pos[:, None].expand(N, Hq), base).permute(1, 0, 2)
    kh = keys.permute(1, 0, 2).repeat_interleave(r, 0)
    vh = vals.permute(1, 0, 2).repeat_interleave(r, 0)
    out = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale).permute(1, 0, 2)
    lse = torch.logsumexp(((qh @ kh.transpose(-1, -2)) * scale).masked_fill(~mask, -math.inf), dim=-1)
    return out, lse, T


def check_block_thd_sdpa_and_grad():
    """Packed (THD) block drafting: three sequences with their own block counts, contexts
    (one empty) and anchors (some past the context, one negative) == per-sequence torch SDPA
    with the explicit block mask, forward and fp64 autograd gradients."""
    bs, Hq, Hkv, D, base = 4, 4, 2, 8, 1e4
    scale = 1 / math.sqrt(D)
    nblks, ctxs = [2, 3, 1], [7, 0, 12]
    cu = np.concatenate([[0], np.cumsum(nblks)]) * bs
    cc = np.concatenate([[0], np.cumsum(ctxs)])
    rng = np.random.default_rng(89)
    T, Tc = int(cu[-1]), int(cc[-1])
    q = rng.standard_normal((T, Hq, D))
    kb, vb = rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    kc, vc = rng.standard_normal((Tc, Hkv, D)), rng.standard_normal((Tc, Hkv, D))
    dout = rng.standard_normal((T, Hq, D))
    anchors = np.array([3, 9, 0, 2, -1, 12])               # 9 > 7 and 2 > 0 clamp; -1 -> 0
    geo = dict(cu_seqlens=cu, ctx_cu_seqlens=cc, base=base)
    o, lse = O.block_fwd_thd(q, kc, vc, kb, vb, anchors, bs, **geo)
    dq, dkc, dvc, dkb, dvb = O.block_bwd_thd(q, kc, vc, kb, vb, anchors, bs, dout, **geo)
    for s in range(3):
        a, e, ca, ce = int(cu[s]), int(cu[s + 1]), int(cc[s]), int(cc[s + 1])
        ro, rl, Ts = _block_torch_ref(q[a:e], kc[ca:ce], vc[ca:ce], kb[a:e], vb[a:e], anchors[a // bs:e // bs], bs,
                                      scale, base)
        assert np.max(np.abs(o[a:e] - ro.detach().numpy())) < 1e-12
        assert np.max(np.abs(lse[:, a:e] - rl.detach().numpy())) < 1e-12
        (ro * torch.tensor(dout[a:e])).sum().backward()
        for mine, t in zip((dq[a:e], dkc[ca:ce], dvc[ca:ce], dkb[a:e], dvb[a:e]), Ts):
            assert mine.shape == t.shape and (mine.size == 0 or np.max(np.abs(mine - t.grad.numpy())) < 1e-10)


def check_soft_ce_library():
    """Row cross-entropies == torch cross_entropy with probability targets; the gradient
    == fp64 autograd of the mean over counted rows; offset and mask select the rows."""
    rng = np.random.default_rng(91)
    B, S, V, off = 2, 9, 13, 3
    st = rng.standard_normal((B, S, V)) * 2
    te = rng.standard_normal((B, S, V)) * 2
    mask = np.ones((B, S), dtype=np.uint8)
    mask[1, 2] = 0
    loss, grad, row_ce = O.soft_ce(st, te, off, mask)
    rows = [(b, i) for b in range(B) for i in range(S) if i + off < S and mask[b, i]]
    x = torch.tensor(st, requires_grad=True)
    xs = torch.stack([x[b, i] for b, i in rows])
    tg = torch.softmax(torch.stack([torch.tensor(te[b, i + off]) for b, i in rows]), -1)
    ce = torch.nn.functional.cross_entropy(xs, tg, reduction="none")
    ref = ce.mean()
    ref.backward()
    assert abs(loss - ref.item()) < 1e-12
    assert np.max(np.abs(grad - x.grad.numpy())) < 1e-12
    assert np.max(np.abs(np.array([row_ce[b, i] for b, i in rows]) - ce.detach().numpy())) < 1e-12
    assert np.all(row_ce[:, S - off:] == 0) and row_ce[1, 2] == 0


def check_soft_ce_closed_forms():
    """A one-hot teacher gives the hard cross-entropy lse(s) - s[label]; a constant
    student row gives ln V; student == teacher gives the teacher's entropy."""
    rng = np.random.default_rng(92)
    B, S, V, off = 1, 5, 11, 1
    st = rng.standard_normal((B, S, V))
    te = np.full((B, S, V), -1e4)
    labels = rng.integers(0, V, S)
    te[0, np.arange(S), labels] = 0.0
    _, _, row_ce = O.soft_ce(st, te, off)
    for i in range(S - off):
        x = st[0, i]
        lse = math.log(np.exp(x).sum())
        assert abs(row_ce[0, i] - (lse - x[labels[i + off]])) < 1e-9
    const = np.zeros((B, S, V))
    _, _, rc = O.soft_ce(const, rng.standard_normal((B, S, V)), off)
    assert np.max(np.abs(rc[0, :S - off] - math.log(V))) < 1e-12
    y = rng.standard_normal((B, S, V))
    _, _, rc2 = O.soft_ce(np.roll(y, -off, axis=1), y, off)  # student row i equals teacher row i + offset
    p = np.exp(y) / np.exp(y).sum(-1, keepdims=True)
    ent = -(p * np.log(p)).sum(-1)
    assert np.max(np.abs(rc2[0, :S - off] - ent[0, off:])) < 1e-12


def check_soft_ce_grouped_library():
    """Per-row teacher rows (a table into a teacher of another length, with rows outside it
    uncounted) and per-group normalisation with weights == torch cross_entropy with
    probability targets and fp64 autograd of sum_g w_g mean_g over rows chosen here."""
    rng = np.random.default_rng(93)
    B, S, St, V, G = 2, 9, 11, 13, 3
    st = rng.standard_normal((B, S, V)) * 2
    te = rng.standard_normal((B, St, V)) * 2
    table = rng.integers(-1, St + 2, (B, S))
    groups = rng.integers(-1, G + 1, (B, S))
    mask = np.ones((B, S), dtype=np.uint8)
    mask[0, 4] = 0
    w = np.array([0.5, 1.0, 2.0])
    loss, grad, row_ce, means, counts = O.soft_ce_grouped(st, te, 0, mask, teacher_rows=table, groups=groups,
                                                          num_groups=G, weights=w)
    x = torch.tensor(st, requires_grad=True)
    total = torch.zeros((), dtype=F64)
    for g in range(G):
        rows = [(b, i) for b in range(B) for i in range(S)
                if groups[b, i] == g and 0 <= table[b, i] < St and mask[b, i]]
        assert counts[g] == len(rows)
        if not rows:
            continue
        xs = torch.stack([x[b, i] for b, i in rows])
        tg = torch.softmax(torch.stack([torch.tensor(te[b, table[b, i]]) for b, i in rows]), -1)
        ce = torch.nn.functional.cross_entropy(xs, tg, reduction="none")
        assert abs(means[g] - ce.mean().item()) < 1e-12
        assert np.max(np.abs(np.array([row_ce[b, i] for b, i in rows]) - ce.detach().numpy())) < 1e-12
        total = total + w[g] * ce.mean()
    total.backward()
    assert abs(loss - total.item()) < 1e-12
    assert np.max(np.abs(grad - x.grad.numpy())) < 1e-12


def _band_mask(S, p, window):
    """[S, p*S] visibility with a trunk band j in (i - window, i], built from tril/triu and eye blocks."""
    ones = torch.ones(S, S, dtype=torch.bool)
    trunk = torch.tril(ones) & torch.triu(ones, diagonal=-(window - 1))
    return torch.cat([trunk] + [torch.eye(S, dtype=torch.bool)] * (p - 1), dim=1)


def _window_dense(q, ks, vs, p, scale, base, window, grad=False):
    """torch SDPA over the concatenated rotated keys of one THD sequence with the band mask."""
    S, Hq, D = q.shape
    Hkv = ks[0].shape[1]
    r = Hq // Hkv
    i = torch.arange(S)
    T = [torch.tensor(x, requires_grad=grad) for x in [q] + list(ks[:p]) + list(vs[:p])]
    tq, tk_, tv = T[0], T[1:1 + p], T[1 + p:]
    qr = rope_complex(tq, (i + p - 1)[:, None].expand(S, Hq), base)
    kc = torch.cat([rope_complex(tk_[t], (i + t)[:, None].expand(S, Hkv), base) for t in range(p)], 0)
    vc = torch.cat(list(tv), 0)
    mask = _band_mask(S, p, window)
    qh, kh, vh = qr.permute(1, 0, 2), kc.permute(1, 0, 2).repeat_interleave(r, 0), vc.permute(1, 0, 2).repeat_interleave(r, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale).permute(1, 0, 2)
    lse = torch.logsumexp(((qh @ kh.transpose(-1, -2)) * scale).masked_fill(~mask, -math.inf), -1)
    return o, lse, T


def check_window_sdpa_and_grad():
    """Sliding-window trunk == SDPA with a band mask (window 1, 3, L-1), forward and fp64 autograd."""
    S, Hq, Hkv, D, p, base = 12, 4, 2, 8, 3, 1e4
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=95)
    scale = 1 / math.sqrt(D)
    for window in (1, 3, S - 1):
        o, lse = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=[0, S], scale=scale, base=base, window=window)
        ro, rl, T = _window_dense(q, ks, vs, p, scale, base, window, grad=True)
        assert np.max(np.abs(o - ro.detach().numpy())) < 1e-12
        assert np.max(np.abs(lse - rl.detach().numpy())) < 1e-12
        (ro * torch.tensor(do)).sum().backward()
        dq, dk, dv = O.bwd(q, ks, vs, do, p, layout="thd", cu_seqlens=[0, S], scale=scale, base=base, window=window)
        assert np.max(np.abs(dq - T[0].grad.numpy())) < 1e-10
        for t in range(p):
            assert np.max(np.abs(dk[t] - T[1 + t].grad.numpy())) < 1e-10
            assert np.max(np.abs(dv[t] - T[1 + p + t].grad.numpy())) < 1e-10


def check_window_closed_forms():
    """Zero queries: LSE_i = ln(min(i+1, W) + p - 1); a window of L or more is the full trunk."""
    S, p, W = 10, 3, 4
    q, ks, vs, _ = make(S=S, Hq=2, Hkv=1, D=8, p=p, seed=96)
    q[:] = 0
    _, lse = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=[0, S], base=1e6, window=W)
    for i in range(S):
        assert abs(lse[0, i] - math.log(min(i + 1, W) + p - 1)) < 1e-12
    q2, ks2, vs2, _ = make(S=S, Hq=2, Hkv=1, D=8, p=p, seed=97)
    a = O.fwd(q2, ks2, vs2, p, layout="thd", cu_seqlens=[0, S], base=1e6, window=S)
    b = O.fwd(q2, ks2, vs2, p, layout="thd", cu_seqlens=[0, S], base=1e6)
    assert np.max(np.abs(a[0] - b[0])) == 0 and np.max(np.abs(a[1] - b[1])) == 0


def check_window_ring_partition():
    """Windowed ring steps over a zig-zag partition, merged, equal the windowed dense rows."""
    S, Hq, Hkv, D, p, base, scale, cp, W = 16, 2, 1, 8, 3, 1e6, 0.35, 2, 5
    q, ks, vs, _ = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=98, B=1)
    ro, rl, _ = _window_dense(q[0], [k[0] for k in ks], [v[0] for v in vs], p, scale, base, W)
    ro, rl = ro.numpy(), rl.numpy()
    c = S // (2 * cp)
    for qc in range(2 * cp):
        qa = qc * c
        acc_o = np.zeros((1, c, Hq, D)); acc_l = np.full((1, Hq, c), -np.inf)
        for kc in range(2 * cp):
            ka = kc * c
            br = kc == qc
            o, l = O.fwd_chunk(q[:, qa:qa + c], ks[0][:, ka:ka + c], vs[0][:, ka:ka + c],
                               [k[:, qa:qa + c] for k in ks[1:]] if br else None,
                               [v[:, qa:qa + c] for v in vs[1:]] if br else None,
                               p, q_offset=qa, kv_offset=ka, scale=scale, base=base, window=W)
            acc_o, acc_l = O.merge(acc_o, acc_l, o, l)
        assert np.max(np.abs(acc_o[0] - ro[qa:qa + c])) < 1e-12
        assert np.max(np.abs(acc_l[0] - rl[:, qa:qa + c])) < 1e-12


def check_chunk_bwd_partition():
    """Ring-step backward terms summed over a zig-zag partition (branch on the diagonal step,
    whole-sequence O and LSE) equal the whole-sequence backward, with and without a window."""
    S, Hq, Hkv, D, p, base, cp = 16, 4, 2, 8, 3, 1e4, 2
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=99, B=1)
    for window in (0, 6):
        o, lse = O.fwd(q, ks, vs, p, base=base, window=window)
        dQ, dK, dV = O.bwd(q, ks, vs, do, p, base=base, window=window)
        c = S // (2 * cp)
        gq = np.zeros_like(dQ)
        gk = [np.zeros_like(dK[0]) for _ in range(p)]
        gv = [np.zeros_like(dV[0]) for _ in range(p)]
        for qc in range(2 * cp):
            qa = qc * c
            for kc in range(2 * cp):
                ka = kc * c
                br = kc == qc
                dq_, dk0, dv0, dkb, dvb = O.bwd_chunk(
                    q[:, qa:qa + c], ks[0][:, ka:ka + c], vs[0][:, ka:ka + c],
                    [k[:, qa:qa + c] for k in ks[1:]] if br else None, [v[:, qa:qa + c] for v in vs[1:]] if br else None,
                    p, do[:, qa:qa + c], o[:, qa:qa + c], lse[:, :, qa:qa + c], q_offset=qa, kv_offset=ka, base=base,
                    window=window)
                gq[:, qa:qa + c] += dq_
                gk[0][:, ka:ka + c] += dk0
                gv[0][:, ka:ka + c] += dv0
                for t in range(len(dkb)):
                    gk[t + 1][:, qa:qa + c] += dkb[t]
                    gv[t + 1][:, qa:qa + c] += dvb[t]
        assert np.max(np.abs(gq - dQ)) < 1e-12
        for t in range(p):
            assert np.max(np.abs(gk[t] - dK[t])) < 1e-12 and np.max(np.abs(gv[t] - dV[t])) < 1e-12


def check_trunk_keys_grad_autograd():
    """dK/dV of a range of trunk keys, from every row that sees them with full-row
    statistics (the form the full-size GPU tests use) == fp64 autograd through SDPA over
    the concatenated keys, for a whole trunk, an inner key range and a windowed range."""
    S, Hq, Hkv, D, p, base = 14, 4, 2, 8, 3, 1e4
    q, ks, vs, do = make(S=S, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=97)
    scale = 1 / math.sqrt(D)
    sl = O.Slice(0, 0, S)
    for window, keys in ((0, np.arange(S)), (0, np.arange(3, 9)), (4, np.arange(2, 11))):
        ro, _, T = _window_dense(q, ks, vs, p, scale, base, window if window else S, grad=True)
        (ro * torch.tensor(do)).sum().backward()
        for g in range(Hkv):
            dk, dv = O.bwd_trunk_keys(q, ks, vs, do, p, sl, g, keys, layout="thd", Hq=Hq, Hkv=Hkv, scale=scale,
                                      base=base, window=window)
            assert np.max(np.abs(dk - T[1].grad.numpy()[keys, g])) < 1e-10
            assert np.max(np.abs(dv - T[1 + p].grad.numpy()[keys, g])) < 1e-10


def check_thd_chunk_ring_partition():
    """Packed (THD) ring steps: sequences of different lengths (one empty) each split into 4
    zig-zag chunks; step (qc, kc) packs chunk qc's rows and chunk kc's keys of every sequence
    at their own offsets.  Merging each row's steps gives the whole-sequence THD forward, and
    summing the steps' backward terms its gradients."""
    lens, Hq, Hkv, D, p, base = [8, 12, 0, 4], 4, 2, 8, 3, 1e4
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, ks, vs, do = make(S=T, Hq=Hq, Hkv=Hkv, D=D, p=p, seed=101)
    ro, rl = O.fwd(q, ks, vs, p, layout="thd", cu_seqlens=cu, base=base)
    dQ, dK, dV = O.bwd(q, ks, vs, do, p, layout="thd", cu_seqlens=cu, base=base)
    nc = 4
    rows = lambda c: np.concatenate([np.arange(cu[s] + c * (n // nc), cu[s] + (c + 1) * (n // nc))
                                     for s, n in enumerate(lens)]).astype(np.int64)
    ccu = lambda: np.concatenate([[0], np.cumsum([n // nc for n in lens])])
    offs = lambda c: np.array([c * (n // nc) for n in lens])
    acc = {}
    gq, gk, gv = np.zeros_like(dQ), [np.zeros_like(dK[0]) for _ in range(p)], [np.zeros_like(dV[0]) for _ in range(p)]
    for qc in range(nc):
        qr = rows(qc)
        acc_o, acc_l = np.zeros((1, len(qr), Hq, D)), np.full((1, Hq, len(qr)), -np.inf)
        for kc in range(nc):
            kr = rows(kc)
            br = kc == qc
            args = (q[qr], ks[0][kr], vs[0][kr], [k[qr] for k in ks[1:]] if br else None,
                    [v[qr] for v in vs[1:]] if br else None, p)
            geo = dict(cu_seqlens=ccu(), kv_cu_seqlens=ccu(), q_offsets=offs(qc), kv_offsets=offs(kc), base=base)
            o, l = O.fwd_chunk_thd(*args, **geo)
            acc_o, acc_l = O.merge(acc_o, acc_l, o[None], l[None])
            dq_, dk0, dv0, dkb, dvb = O.bwd_chunk_thd(*args, do[qr], ro[qr], rl[:, qr], **geo)
            gq[qr] += dq_
            gk[0][kr] += dk0
            gv[0][kr] += dv0
            for t in range(len(dkb)):
                gk[t + 1][qr] += dkb[t]
                gv[t + 1][qr] += dvb[t]
        assert np.max(np.abs(acc_o[0] - ro[qr])) < 1e-12
        assert np.max(np.abs(acc_l[0] - rl[:, qr])) < 1e-12
    assert np.max(np.abs(gq - dQ)) < 1e-12
    for t in range(p):
        assert np.max(np.abs(gk[t] - dK[t])) < 1e-12 and np.max(np.abs(gv[t] - dV[t])) < 1e-12
    # one step whose keys are each sequence's whole causal prefix (more key rows than
    # query rows): the dense rows exactly
    qc = 2
    qr = rows(qc)
    kr = np.concatenate([np.arange(cu[s], cu[s] + (qc + 1) * (n // nc)) for s, n in enumerate(lens)]).astype(np.int64)
    kcu = np.concatenate([[0], np.cumsum([(qc + 1) * (n // nc) for n in lens])])
    o, l = O.fwd_chunk_thd(q[qr], ks[0][kr], vs[0][kr], [k[qr] for k in ks[1:]], [v[qr] for v in vs[1:]], p,
                           cu_seqlens=ccu(), kv_cu_seqlens=kcu, q_offsets=offs(qc), kv_offsets=np.zeros(len(lens)),
                           base=base)
    assert np.max(np.abs(o - ro[qr])) < 1e-12 and np.max(np.abs(l - rl[:, qr])) < 1e-12


PINS = [check_rope_complex_form, check_rope_single_pair, check_rope_group, check_zero_query_closed_form,
        lambda: check_zero_query_closed_form("thd"), check_sdpa_brute_force, check_p1_is_causal_sdpa,
        check_merge_invariant, check_branch_relative_position, check_grad_autograd,
        check_grad_finite_difference, check_thd_equals_bshd, check_thd_isolation, check_gqa_is_repeated_kv,
        check_sampled_rows_match_full, check_chunk_rows_match_dense, check_chunk_ring_partition,
        check_merge_closed_form, check_block_sdpa_mask, check_block_zero_query_closed_form,
        check_block_size1_is_causal, check_block_grad_autograd, check_soft_ce_library, check_soft_ce_closed_forms,
        check_window_sdpa_and_grad, check_window_closed_forms, check_window_ring_partition, check_chunk_bwd_partition,
        check_trunk_keys_grad_autograd, check_soft_ce_grouped_library, check_thd_chunk_ring_partition,
        check_block_thd_sdpa_and_grad]


@pytest.mark.parametrize("pin", PINS, ids=[f"pin{i}" for i in range(len(PINS))])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------- planted mistakes
@contextlib.contextmanager
def planted(name, fn):
    old = getattr(O, name)
    setattr(O, name, fn)
    try:
        yield
    finally:
        setattr(O, name, old)


def _orig(name):
    return getattr(O, name)


def _mask_no_branch(i, p, L, window=0):
    m = np.zeros(p * L, dtype=bool); m[O.trunk_window_start(i, window): i + 1] = True; return m


def _mask_strict_causal(i, p, L, window=0):
    m = _orig_mask(i, p, L, window); m[i] = i == 0; return m


def _mask_branch_next_row(i, p, L, window=0):
    m = np.zeros(p * L, dtype=bool); m[O.trunk_window_start(i, window): i + 1] = True
    for q in range(2, p + 1):
        m[(q - 1) * L + min(i + 1, L - 1)] = True
    return m


_orig_mask = O.ttt_mask_row
_orig_rot = O.rotate_half
_orig_qpos = O.query_position
_orig_kpos = O.key_position
_orig_inv = O.inv_freq
_orig_blk = O._row_block_fwd
_orig_merge = O.merge


def _rot_sign(x, pos, base):
    return _orig_rot(x, -np.asarray(pos, dtype=np.float64), base)


def _rot_pairing(x, pos, base):
    # adjacent-pair (interleaved) rotation instead of rotate-half
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * _orig_inv(D, base)
    c, s = np.cos(ang), np.sin(ang)
    y = x.copy()
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return y


def _blk_transposed_v(gk, q_rot, rows, p, L, scale, window=0):
    P, lse, O_, cols = _orig_blk(gk, q_rot, rows, p, L, scale, window)
    return P, lse, P @ gk.vals[cols][:, ::-1], cols


def _trunk_keys_late_rows(q, ks, vs, dout, p, sl, g, keys, *, layout, Hq, Hkv, scale, base, window=0):
    """bwd_trunk_keys with its row range starting one row late (i > min(keys))."""
    keys = np.asarray(keys, dtype=np.int64)
    r = Hq // Hkv
    gk = O._GroupKeys(sl, g, ks, vs, p, layout, base)
    lo = int(keys.min()) + 1
    hi = sl.L if window <= 0 else min(sl.L, int(keys.max()) + window)
    dk = np.zeros((len(keys), gk.keys.shape[-1]))
    dv = np.zeros_like(dk)
    for hh in range(r):
        qs, dos = sl.take(q, layout, g * r + hh), sl.take(dout, layout, g * r + hh)
        for blk in O._blocks(np.arange(lo, hi), O._block_rows(sl.L, p)):
            qr = O.rotate_half(qs[blk], O.query_position(blk, p), base)
            P, _, O_, cols = O._row_block_fwd(gk, qr, blk, p, sl.L, scale, window)
            delta = (dos[blk] * O_).sum(axis=1)
            Pk = P[:, np.searchsorted(cols, keys)] * (keys[None, :] <= blk[:, None])
            dS = Pk * (dos[blk] @ gk.vals[keys].T - delta[:, None])
            dk += scale * (dS.T @ qr)
            dv += Pk.T @ dos[blk]
    return O.unrotate_half(dk, gk.pos[keys], base), dv


_orig_counted = O.soft_ce_rows_counted


def _ce_counted_ignores_groups(B, S, off, mask=None, *, teacher_rows=None, teacher_len=None, groups=None, num_groups=1):
    return _orig_counted(B, S, off, mask, teacher_rows=teacher_rows, teacher_len=teacher_len)


MISTAKES = [
    ("ttt_mask_row", _mask_no_branch),
    ("ttt_mask_row", _mask_strict_causal),
    ("ttt_mask_row", _mask_branch_next_row),
    ("rotate_half", _rot_sign),
    ("rotate_half", _rot_pairing),
    ("query_position", lambda i, p: np.asarray(i) + p),
    ("query_position", lambda i, p: np.asarray(i)),
    ("key_position", lambda q, j: np.asarray(j)),
    ("key_position", lambda q, j: np.asarray(j) + q),
    ("inv_freq", lambda D, base: np.power(np.float64(base), -1.0 * np.arange(D // 2) / D)),
    ("_row_block_fwd", _blk_transposed_v),
    ("ring_visible", lambda qp, kp, w=0: np.asarray(kp)[None, :] < np.asarray(qp)[:, None]),
    ("ring_visible", lambda qp, kp, w=0: np.asarray(kp)[None, :] <= np.asarray(qp)[:, None] + 1),
    ("merge", lambda oa, la, ob, lb: _orig_merge(ob, la, oa, lb)),
    ("block_visible_ctx", lambda a, L: int(min(max(a + 1, 0), L))),
    ("block_slot_position", lambda a, t: int(a) + np.asarray(t) + 1),
    ("block_slot_position", lambda a, t: np.asarray(t)),
    ("soft_ce_rows_counted", lambda B, S, off, mask=None, **kw: np.arange(S)[None, :].repeat(B, 0) + off <= S),
    ("trunk_window_start", lambda i, w: 0 if w <= 0 else max(0, i - w + 2)),
    ("trunk_window_start", lambda i, w: 0 if w <= 0 else max(0, i - w)),
    ("ring_visible", lambda qp, kp, w=0: np.asarray(kp)[None, :] <= np.asarray(qp)[:, None]),
    ("soft_ce_rows_counted", lambda B, S, off, mask=None, **kw: np.ones((B, S), dtype=bool) & (np.arange(S)[None, :] + off < S)),
    ("merge", lambda oa, la, ob, lb: (_orig_merge(oa, la, ob, lb)[0], np.maximum(la, lb))),
    ("bwd_trunk_keys", _trunk_keys_late_rows),
    ("soft_ce_teacher_rows", lambda B, S, off, tr=None: np.arange(S)[None, :].repeat(B, 0) + off),
    ("soft_ce_rows_counted", _ce_counted_ignores_groups),
    ("_thd_segments", lambda cu, kc: [(int(cu[s]), int(cu[s + 1]), int(cu[s]), int(cu[s + 1]))
                                      for s in range(len(cu) - 1)]),
    ("_block_thd_segments", lambda cu, cc, bs: [(int(cu[s]), int(cu[s + 1]), 0, int(cc[s + 1]) - int(cc[s]))
                                                for s in range(len(cu) - 1)]),
]


@pytest.mark.parametrize("name,fn", MISTAKES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(MISTAKES)])
def test_planted_mistake_is_caught(name, fn):
    caught = 0
    with planted(name, fn):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught += 1
    assert caught >= 1, f"no pin catches a planted mistake in {name}"
