"""GPU parity of the per-pass soft cross-entropy (ttt_soft_ce_fwd / _bwd) against the fp64 oracle.

Student row i of pass p is scored against the teacher distribution at row i + p; rows without a teacher row or
with mask 0 are not counted; the loss is the mean over counted rows.  bf16 logits, fp32 loss/LSE, bf16 gradient
(compared by relative Frobenius norm, which bf16 rounding bounds by about 2e-3).
"""
import math

import numpy as np
import pytest

import ttt_synth as syn
from oracle import ttt_oracle as O
from ttt_cases import rel_fro, to_np

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


def logits(seed, shape, scale=2.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * scale
    return syn.round_bf16(x)


def run(tk, dev, st, te, off, mask=None, dloss=1.0):
    gs = torch.from_numpy(st).to(dev).to(torch.bfloat16)
    gt = torch.from_numpy(te).to(dev).to(torch.bfloat16)
    gm = torch.from_numpy(mask).to(dev) if mask is not None else None
    stats, row_lse, row_ce = tk.soft_ce_fwd(gs, gt, off, mask=gm)
    gd = torch.tensor([dloss], dtype=torch.float32, device=dev)
    g = tk.soft_ce_bwd(gs, gt, off, row_lse, stats, gd, mask=gm)
    torch.cuda.synchronize()
    return to_np(stats), to_np(row_lse), to_np(row_ce), to_np(g)


@pytest.mark.parametrize("off,masked", [(1, False), (3, True), (7, False)])
def test_soft_ce_small(dev, tk, off, masked):
    B, S, V = 2, 37, 1000
    st, te = logits(41, (B, S, V)), logits(42, (B, S, V))
    mask = None
    if masked:
        mask = (np.random.default_rng(43).random((B, S)) > 0.3).astype(np.uint8)
    stats, row_lse, row_ce, g = run(tk, dev, st, te, off, mask, dloss=0.75)
    loss, grad, rce = O.soft_ce(st, te, off, mask)
    counted = O.soft_ce_rows_counted(B, S, off, mask)
    print(f"off={off} masked={masked}: loss {stats[0]:.7f} ref {loss:.7f}, count {stats[1]:.0f}")
    assert int(stats[1]) == int(counted.sum())
    assert abs(stats[0] - loss) <= 1e-5 * max(1.0, abs(loss))
    assert np.max(np.abs(row_ce - rce)) <= 2e-5
    lse_ref = np.log(np.exp(st.astype(np.float64)).sum(-1))
    assert np.max(np.abs(row_lse[..., 0][counted] - lse_ref[counted])) <= 2e-5
    assert np.all(g[~counted] == 0)
    e = rel_fro(g, 0.75 * grad)
    print(f"  grad rel Frobenius {e:.3e}")
    assert e <= 4e-3


def test_soft_ce_edges(dev, tk):
    # no counted row: loss 0, count 0, zero gradient
    st, te = logits(44, (1, 5, 64)), logits(45, (1, 5, 64))
    stats, _, row_ce, g = run(tk, dev, st, te, 5)
    assert stats[0] == 0 and stats[1] == 0 and np.all(row_ce == 0) and np.all(g == 0)
    # the smallest vocab, one row
    st, te = logits(46, (1, 2, 8)), logits(47, (1, 2, 8))
    stats, _, _, g = run(tk, dev, st, te, 1)
    loss, grad, _ = O.soft_ce(st, te, 1)
    assert stats[1] == 1 and abs(stats[0] - loss) <= 1e-5 and rel_fro(g, grad) <= 4e-3
    # a full-size vocabulary (152064) and peaked logits
    st, te = logits(48, (1, 3, 152064), 6.0), logits(49, (1, 3, 152064), 6.0)
    stats, _, row_ce, g = run(tk, dev, st, te, 1)
    loss, grad, rce = O.soft_ce(st, te, 1)
    print(f"V=152064: loss {stats[0]:.6f} ref {loss:.6f}; grad rel Frobenius {rel_fro(g, grad):.3e}")
    assert abs(stats[0] - loss) <= 1e-5 * max(1.0, abs(loss)) and rel_fro(g, grad) <= 4e-3


def test_soft_ce_fullsize(dev, tk):
    """B=4, S=4096, V=32000 at pass 7: the loss equals the oracle's loss over every counted
    row (fp64 row cross-entropies summed in 512-row chunks, then divided by the count), and
    >= 512 sampled rows (row CE, LSE, gradient) match the oracle."""
    B, S, V, off = 4, 4096, 32000, 7
    gen = torch.Generator(device=dev)
    gen.manual_seed(50)
    gs = (torch.randn((B, S, V), generator=gen, device=dev) * 2).to(torch.bfloat16)
    gt = (torch.randn((B, S, V), generator=gen, device=dev) * 2).to(torch.bfloat16)
    stats, row_lse, row_ce = tk.soft_ce_fwd(gs, gt, off)
    g = tk.soft_ce_bwd(gs, gt, off, row_lse, stats, torch.ones(1, device=dev))
    torch.cuda.synchronize()
    st_, rl, rc = to_np(stats), to_np(row_lse), to_np(row_ce)
    n = B * (S - off)
    assert int(st_[1]) == n
    total = 0.0
    for b in range(B):
        for i0 in range(0, S - off, 512):
            i1 = min(i0 + 512, S - off)
            _, _, rce = O.soft_ce(to_np(gs[b:b + 1, i0:i1]), to_np(gt[b:b + 1, i0 + off:i1 + off]), 0)
            total += float(rce.sum())
    loss_ref = total / n
    print(f"full size: loss {st_[0]:.7f}, oracle over all {n} counted rows {loss_ref:.7f}")
    assert abs(st_[0] - loss_ref) <= 1e-5 * max(1.0, abs(loss_ref))
    rng = np.random.default_rng(51)
    rows = [(int(b), int(i)) for b, i in zip(rng.integers(0, B, 512), rng.integers(0, S - off, 512))]
    rows += [(0, 0), (B - 1, S - off - 1)]
    ece = el = 0.0
    gg, gr = [], []
    for b, i in rows:
        s_row = to_np(gs[b, i])[None, None]
        t_row = to_np(gt[b, i + off])[None, None]
        _, grad1, rce1 = O.soft_ce(s_row, t_row, 0)
        ece = max(ece, abs(rc[b, i] - rce1[0, 0]))
        lse = math.log(np.exp(s_row.astype(np.float64)).sum())
        el = max(el, abs(rl[b, i, 0] - lse))
        gg.append(to_np(g[b, i]))
        gr.append(grad1[0, 0] / n)
    e = rel_fro(np.stack(gg), np.stack(gr))
    print(f"full size: {len(rows)} rows, row CE max-abs {ece:.2e}, LSE max-abs {el:.2e}, grad rel Frobenius {e:.2e}")
    assert ece <= 5e-5 and el <= 5e-5 and e <= 4e-3


@pytest.mark.parametrize("bs,nblk", [(8, 9), (16, 4)])
def test_soft_ce_block_slots(dev, tk, bs, nblk):
    """Block-draft slots: slot t of the block anchored at a is scored against teacher row
    a + t + 1 of a longer target sequence (rows past its end uncounted), normalised per
    slot index (bs groups), with decaying per-slot weights as the upstream gradient."""
    B, St, V = 2, 300, 1000
    S = nblk * bs
    rng = np.random.default_rng(60 + bs)
    anchors = np.sort(rng.integers(0, St, (B, nblk)), axis=1)
    anchors[:, -1] = St - bs // 2                         # the last block runs past the target's end
    t_idx = np.arange(S) % bs
    table = (np.repeat(anchors, bs, axis=1) + t_idx[None, :] + 1).astype(np.int32)
    groups = np.broadcast_to(t_idx, (B, S)).astype(np.int32).copy()
    mask = (rng.random((B, S)) > 0.1).astype(np.uint8)
    st, te = logits(61, (B, S, V)), logits(62, (B, St, V))
    w = (0.8 ** np.arange(bs)).astype(np.float32)
    up = lambda x: torch.from_numpy(x).to(dev)
    gs, gt = up(st).to(torch.bfloat16), up(te).to(torch.bfloat16)
    gtab, ggrp, gm = up(table), up(groups), up(mask)
    stats, row_lse, row_ce = tk.soft_ce_fwd(gs, gt, 0, mask=gm, teacher_rows=gtab, groups=ggrp, num_groups=bs)
    g = tk.soft_ce_bwd(gs, gt, 0, row_lse, stats, up(w), mask=gm, teacher_rows=gtab, groups=ggrp, num_groups=bs)
    torch.cuda.synchronize()
    stats, row_ce, g = to_np(stats), to_np(row_ce), to_np(g)
    loss1, _, rce, means, counts = O.soft_ce_grouped(st, te, 0, mask, teacher_rows=table, groups=groups,
                                                     num_groups=bs)
    _, grad_w, _, _, _ = O.soft_ce_grouped(st, te, 0, mask, teacher_rows=table, groups=groups, num_groups=bs,
                                           weights=w)
    counted = O.soft_ce_rows_counted(B, S, 0, mask, teacher_rows=table, teacher_len=St, groups=groups,
                                     num_groups=bs)
    print(f"bs={bs}: loss {stats[0]:.6f} ref {loss1:.6f}, counted {stats[1]:.0f}/{B * S}, per-slot counts "
          f"{stats[3::2].astype(int).tolist()}")
    assert int(stats[1]) == int(counted.sum()) < B * S
    assert np.array_equal(stats[3::2].astype(int), counts)
    assert np.max(np.abs(stats[2::2] - means)) <= 2e-5 * max(1.0, np.abs(means).max())
    assert abs(stats[0] - loss1) <= 1e-5 * max(1.0, abs(loss1))
    assert np.max(np.abs(row_ce - rce)) <= 2e-5
    assert np.all(g[~counted] == 0)
    e = rel_fro(g, grad_w)
    print(f"  grad (slot weights 0.8^t) rel Frobenius {e:.3e}")
    assert e <= 4e-3
