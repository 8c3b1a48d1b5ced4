"""fp64 CPU oracle of the multi-pass EAGLE-3 TTT draft attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The GPU library
never uses it, and this module uses nothing from the GPU library.

What is computed (one call = one TTT pass p, 1-based):

* Pass p's query at row i attends to two key sets (NeMo-RL issue "DFlash/DSpark
  and EAGLE-3 TTT draft co-training for speculative decoding (Megatron
  backend)", section "What I'm working on", item 1; NeMo-RL PR #3725,
  self-review comment: multi-pass staircase visibility):
    - the trunk: pass-1 keys/values at rows j <= i of the same sequence (causal);
    - the branch: the keys/values that passes q = 2..p produced at the same row i.
  Both sets are expressed here as ONE explicit boolean mask row over the
  concatenated keys [K(1)_0..L-1 ; K(2)_0..L-1 ; ... ; K(p)_0..L-1] of the
  sequence, and a single softmax is taken over the allowed entries.  That is
  the exact value the two-part trunk+branch method with its joint
  log-sum-exp merge reaches (issue above, item 1: exact joint-LSE merge).

* Rotary embedding, rotate-half pairing (PR #3725 self-review: rotate-half
  oracle), applied to queries and keys, never to values, with
  theta_k = base^(-2k/D) in fp64 and the pair (k, k + D/2).
  Positions (issue above, item 1: inference-aligned per-pass RoPE offsets;
  reading: a pass-p draft token sits p-1 positions after its row):
    query of pass p at row i      -> position i + p - 1
    trunk key (pass 1) at row j   -> position j
    branch key of pass q at row i -> position i + q - 1
  base == 0 disables the rotation.

* Layouts: padded BSHD ([B, S, H, D], every row of every batch is valid) and
  packed THD ([T, H, D] with cu_seqlens; rows of one sequence never see another
  sequence, positions restart at 0 per sequence) (issue above, item 4: THD
  varlen layout).  GQA: query head h uses key/value head h // (Hq / Hkv).

* LSE is the natural-log sum of exp of the scaled scores.  Per-row LSE layout:
  [B, Hq, S] (BSHD) or [Hq, T] (THD).

* Backward (standard softmax-attention chain rule, with the merged LSE):
    Delta_i = <dO_i, O_i>
    dS_a    = P_a * (<dO_i, v_a> - Delta_i)
    dq_i    = scale * R(pos_q)^T sum_a dS_a R(pos_a) k_a
    dk_a    = scale * R(pos_a)^T sum_{rows i, heads h of the group} dS_a R(pos_q) q_i
    dv_a    = sum_{rows i, heads h of the group} P_a dO_i
  Gradients are returned per tensor (dK(q), dV(q) for q = 1..p); nothing is
  accumulated across calls.

* Block drafting (issue above, item 2: anchor + mask-token blocks, attention
  bidirectional inside a block, trunk cut at the anchor).  Reading: block n of
  bs slots has anchor position a_n; slot t is the token at position a_n + t
  (slot 0 is the anchor itself, slots 1.. the mask tokens); every slot of the
  block sees the context keys at positions j < a_n and all bs keys of its own
  block, rotated at their positions.  `block_fwd` returns O and LSE per slot;
  `block_bwd` the gradients of q, the context K/V and the block K/V by the
  same chain rule as the TTT backward below.  Packed (THD) block drafting,
  `block_fwd_thd` / `block_bwd_thd`: every sequence holds whole blocks and has
  its own context (issue above, item 4: the block-draft attention on the THD
  layout); sequences never see each other and anchors clamp to the
  sequence's own context.

* Distillation loss (issue above, item 3: chunked soft cross-entropy, normalised
  per pass over the whole batch; PR #3725 self-review: teacher_offset =
  pass_index + 1).  Reading: pass p's student logits at row i are scored
  against the teacher distribution softmax(teacher logits at row i + offset) of
  the same sequence, offset = p for 1-based p; rows with no such teacher row or
  with mask 0 are not counted; loss = (sum of counted rows' cross-entropies) /
  (number of counted rows).  The gradient is (softmax(student) - teacher
  distribution) / count on counted rows and 0 elsewhere.  Chunking the tokens
  only bounds memory and does not change the value.  The same issue item names
  per-slot normalisation for block drafting: `soft_ce_grouped` takes a table of
  teacher rows per student row (a block slot at position a + t is scored
  against teacher row a + t + 1, the rule above: query position + 1) and a
  normalisation group per row (the slot index); each group's loss is the mean
  over its own counted rows, and the loss is their (optionally weighted) sum.

* Sliding-window trunk (issue above, item 4: sliding-window layers).  Reading:
  with window W > 0, row i's trunk is the pass-1 keys j with i - W < j <= i
  (the last W positions up to its own); the branch is unchanged; W = 0 is the
  full causal trunk.

* Ring steps (issue above, item 4: context parallelism, where pass-1 K/V
  travel around a zig-zag ring and partial results are joined by the joint-LSE
  merge): `fwd_chunk` is the attention of a block of query rows at sequence
  positions q_offset.. against a block of pass-1 keys at positions kv_offset..
  (visible iff key position <= query row position), optionally with the
  branch keys of those rows; `merge` joins two partial results over disjoint
  key sets: LSE = ln(e^LSE_a + e^LSE_b), O = e^(LSE_a - LSE) O_a +
  e^(LSE_b - LSE) O_b.  A row that sees no key has O = 0 and LSE = -inf.
  Packed (THD) ring steps, `fwd_chunk_thd` / `bwd_chunk_thd`: every sequence s
  of the batch takes its own ring step (its query rows at positions
  q_offsets[s].., its pass-1 key rows kv_cu[s]..kv_cu[s+1] at positions
  kv_offsets[s]..), and sequences never see each other (the THD rule above).

Everything is fp64; inputs are upcast from whatever float type they hold.
No blocking, fusion or reordering beyond evaluating rows in independent
groups.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = ["inv_freq", "rotate_half", "unrotate_half", "query_position", "key_position",
           "ttt_mask_row", "trunk_window_start", "sequences", "fwd", "bwd", "fwd_rows", "fwd_group_rows", "bwd_rows",
           "bwd_trunk_keys", "Slice",
           "fwd_chunk", "bwd_chunk", "fwd_chunk_thd", "bwd_chunk_thd", "merge", "ring_visible", "block_visible_ctx", "block_fwd_rows", "block_fwd",
           "block_bwd_rows", "block_bwd", "block_fwd_thd", "block_bwd_thd", "soft_ce_rows_counted", "soft_ce_teacher_rows", "soft_ce", "soft_ce_grouped"]


# ----------------------------------------------------------------------------- RoPE
def inv_freq(D: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/D), k = 0..D/2-1, in fp64."""
    k = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * k / D)


def rotate_half(x: np.ndarray, pos, base: float) -> np.ndarray:
    """R(pos) x with rotate-half pairing: for k < D/2,
    y_k = x_k cos(pos*theta_k) - x_{k+D/2} sin(pos*theta_k),
    y_{k+D/2} = x_{k+D/2} cos(pos*theta_k) + x_k sin(pos*theta_k).
    x: [..., D]; pos broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def unrotate_half(g: np.ndarray, pos, base: float) -> np.ndarray:
    """R(pos)^T g, the transpose (= inverse) rotation."""
    return rotate_half(g, -np.asarray(pos, dtype=np.float64), base)


def query_position(i, p: int):
    return np.asarray(i) + (p - 1)


def key_position(q: int, j):
    """Position of the key that pass q produced at row j (q = 1 is the trunk)."""
    return np.asarray(j) + (q - 1)


# ----------------------------------------------------------------------------- mask
def trunk_window_start(i: int, window: int) -> int:
    """First pass-1 key row i sees: 0 without a window, else i - window + 1 (clamped at 0)."""
    return 0 if window <= 0 else max(0, i - window + 1)


def ttt_mask_row(i: int, p: int, L: int, window: int = 0) -> np.ndarray:
    """Explicit visibility of row i at pass p over the concatenated keys of a
    length-L sequence, [K(1)_0..L-1 ; K(2)_0..L-1 ; ... ; K(p)_0..L-1].
    window > 0 limits the trunk to the last `window` keys j <= i."""
    m = np.zeros(p * L, dtype=bool)
    m[trunk_window_start(i, window): i + 1] = True   # trunk: pass-1 keys j <= i (inside the window)
    for q in range(2, p + 1):              # branch: passes 2..p at the same row
        m[(q - 1) * L + i] = True
    return m


# ----------------------------------------------------------------------------- layouts
class Slice:
    """One sequence of the batch: batch index b (BSHD) and token range [start, start+L)."""

    def __init__(self, b: int, start: int, L: int):
        self.b, self.start, self.L = b, start, L

    def take(self, x: np.ndarray, layout: str, head: int) -> np.ndarray:
        """[L, D] fp64 copy of head `head` of this sequence from a BSHD or THD tensor."""
        if layout == "bshd":
            return np.asarray(x[self.b, :, head], dtype=np.float64)
        return np.asarray(x[self.start: self.start + self.L, head], dtype=np.float64)


def sequences(layout: str, shape: Sequence[int], cu_seqlens=None) -> list:
    if layout == "bshd":
        B, S = shape[0], shape[1]
        return [Slice(b, 0, S) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [Slice(0, int(cu[s]), int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)]


def _lse_index(layout: str, sl: Slice, h: int, i):
    if layout == "bshd":
        return (sl.b, h, i)
    return (h, sl.start + np.asarray(i))


def _row_index(layout: str, sl: Slice, i):
    if layout == "bshd":
        return (sl.b, i)
    return (sl.start + np.asarray(i),)


# ----------------------------------------------------------------------------- core
class _GroupKeys:
    """Rotated concatenated keys and values of one (sequence, KV head) slice."""

    def __init__(self, sl: Slice, g: int, ks, vs, p: int, layout: str, base: float):
        L = sl.L
        rows = np.arange(L)
        kt, vt = [], []
        for q in range(1, p + 1):
            kt.append(rotate_half(sl.take(ks[q - 1], layout, g), key_position(q, rows), base))
            vt.append(sl.take(vs[q - 1], layout, g))
        self.keys = np.concatenate(kt, axis=0)     # [p*L, D] rotated
        self.vals = np.concatenate(vt, axis=0)     # [p*L, D]
        self.pos = np.concatenate([key_position(q, rows) for q in range(1, p + 1)])


def _candidate_columns(rows: np.ndarray, p: int, L: int) -> np.ndarray:
    """Concatenated-key columns that any row of the block can see: the trunk prefix
    up to the block's last row and every pass's key at the block's rows."""
    cols = [np.arange(int(rows.max()) + 1)]
    for q in range(2, p + 1):
        cols.append((q - 1) * L + rows)
    return np.unique(np.concatenate(cols))


def _row_block_fwd(gk: _GroupKeys, q_rot: np.ndarray, rows: np.ndarray, p: int, L: int, scale: float,
                   window: int = 0):
    """Scores, probabilities, LSE and O for a block of query rows (one head).

    The explicit mask rows are evaluated on the block's candidate columns; the
    assertion checks that no allowed key lies outside them, so the softmax over
    the candidates equals the softmax over all p*L concatenated keys."""
    cols = _candidate_columns(rows, p, L)
    full = np.stack([ttt_mask_row(int(i), p, L, window) for i in rows])  # [n, p*L]
    mask = full[:, cols]
    assert np.array_equal(mask.sum(axis=1), full.sum(axis=1))
    s = scale * (q_rot @ gk.keys[cols].T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    P = np.exp(s - lse[:, None])
    O = P @ gk.vals[cols]
    return P, lse, O, cols


def _blocks(rows: np.ndarray, n: int):
    for a in range(0, len(rows), n):
        yield rows[a: a + n]


def _block_rows(L: int, p: int) -> int:
    # keep a block's [n, p*L] mask near 16 MB
    return max(1, min(256, (16 << 20) // max(1, p * L)))


def fwd_group_rows(q, ks, vs, p: int, sl: Slice, g: int, rows_by_head, *, layout: str, Hq: int, Hkv: int,
                   scale: float, base: float, window: int = 0):
    """{h: (O [n, D], LSE [n])} for the requested rows of the query heads h of KV
    group g in sequence `sl`, at pass p (the group's rotated keys are built once)."""
    gk = _GroupKeys(sl, g, ks, vs, p, layout, base)
    out = {}
    for h, rows in rows_by_head.items():
        assert h // (Hq // Hkv) == g
        rows = np.asarray(rows, dtype=np.int64)
        qs = sl.take(q, layout, h)
        O = np.empty((len(rows), qs.shape[-1]))
        lse = np.empty(len(rows))
        a = 0
        for blk in _blocks(rows, _block_rows(sl.L, p)):
            qr = rotate_half(qs[blk], query_position(blk, p), base)
            _, l_, o_, _ = _row_block_fwd(gk, qr, blk, p, sl.L, scale, window)
            O[a: a + len(blk)] = o_
            lse[a: a + len(blk)] = l_
            a += len(blk)
        out[h] = (O, lse)
    return out


def fwd_rows(q, ks, vs, p: int, sl: Slice, h: int, rows, *, layout: str, Hq: int, Hkv: int,
             scale: float, base: float, window: int = 0):
    """O [n, D] and LSE [n] for rows `rows` of sequence `sl`, query head h, at pass p."""
    g = h // (Hq // Hkv)
    return fwd_group_rows(q, ks, vs, p, sl, g, {h: rows}, layout=layout, Hq=Hq, Hkv=Hkv, scale=scale,
                          base=base, window=window)[h]


def fwd(q, ks, vs, p: int, *, layout: str = "bshd", cu_seqlens=None, scale: Optional[float] = None,
        base: float = 0.0, window: int = 0):
    """Full forward of pass p.  q: [B,S,Hq,D] or [T,Hq,D]; ks, vs: p tensors of
    [B,S,Hkv,D] or [T,Hkv,D] (index 0 = trunk).  Returns (O fp64 like q, LSE fp64)."""
    assert len(ks) >= p and len(vs) >= p and p >= 1
    Hq, D = q.shape[-2], q.shape[-1]
    Hkv = ks[0].shape[-2]
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    O = np.zeros(q.shape, dtype=np.float64)
    if layout == "bshd":
        lse = np.zeros((q.shape[0], Hq, q.shape[1]))
    else:
        lse = np.zeros((Hq, q.shape[0]))
    r = Hq // Hkv
    for sl in sequences(layout, q.shape, cu_seqlens):
        rows = np.arange(sl.L)
        for g in range(Hkv):
            res = fwd_group_rows(q, ks, vs, p, sl, g, {h: rows for h in range(g * r, (g + 1) * r)},
                                 layout=layout, Hq=Hq, Hkv=Hkv, scale=scale, base=base, window=window)
            for h, (o_, l_) in res.items():
                O[_row_index(layout, sl, rows) + (h,)] = o_
                lse[_lse_index(layout, sl, h, rows)] = l_
    return O, lse


def bwd_rows(q, ks, vs, dout, p: int, sl: Slice, g: int, rows, *, layout: str, Hq: int,
             Hkv: int, scale: float, base: float, need_kv: bool = True, window: int = 0):
    """Backward contributions of query rows `rows` (all r heads of KV group g).

    Returns (dq [r, n, D] for those rows, dk [p*L, D], dv [p*L, D]) where dk, dv
    hold only the contributions of the given rows, over the concatenated keys.
    A key's gradient is complete when `rows` holds every row that sees it
    (trunk key j: all rows i >= j; branch key (q, i): row i)."""
    rows = np.asarray(rows, dtype=np.int64)
    r = Hq // Hkv
    gk = _GroupKeys(sl, g, ks, vs, p, layout, base)
    D = gk.keys.shape[-1]
    dq = np.zeros((r, len(rows), D))
    dk_rot = np.zeros_like(gk.keys)
    dv = np.zeros_like(gk.vals)
    touched = np.zeros(len(gk.keys), dtype=bool)
    for hh in range(r):
        h = g * r + hh
        qs = sl.take(q, layout, h)
        dos = sl.take(dout, layout, h)
        a = 0
        for blk in _blocks(rows, _block_rows(sl.L, p)):
            qr = rotate_half(qs[blk], query_position(blk, p), base)
            P, lse, O, cols = _row_block_fwd(gk, qr, blk, p, sl.L, scale, window)
            keys, vals = gk.keys[cols], gk.vals[cols]
            do = dos[blk]
            delta = (do * O).sum(axis=1)
            dP = do @ vals.T
            dS = P * (dP - delta[:, None])
            dq_rot = scale * (dS @ keys)
            dq[hh, a: a + len(blk)] = unrotate_half(dq_rot, query_position(blk, p), base)
            if need_kv:
                dk_rot[cols] += scale * (dS.T @ qr)
                dv[cols] += P.T @ do
                touched[cols] = True
            a += len(blk)
    dk = np.zeros_like(dk_rot)             # keys no row reached keep a zero gradient
    idx = np.flatnonzero(touched)
    dk[idx] = unrotate_half(dk_rot[idx], gk.pos[idx], base)
    return dq, dk, dv


def bwd_trunk_keys(q, ks, vs, dout, p: int, sl: Slice, g: int, keys, *, layout: str, Hq: int, Hkv: int,
                   scale: float, base: float, window: int = 0):
    """Exact dK, dV ([n, D] each) of the pass-1 (trunk) keys `keys` of KV group g in
    sequence `sl`: the same chain rule as `bwd_rows`, summed over every row that sees
    one of those keys (rows i >= min(keys), and i < max(keys) + window with a
    window), each row's probabilities, O and Delta taken over its full visible key
    set.  Only the products that reach the requested keys are formed, so a slice of
    a long sequence costs about one forward over its rows."""
    keys = np.asarray(keys, dtype=np.int64)
    r = Hq // Hkv
    gk = _GroupKeys(sl, g, ks, vs, p, layout, base)
    D = gk.keys.shape[-1]
    lo = int(keys.min())
    hi = sl.L if window <= 0 else min(sl.L, int(keys.max()) + window)
    rows = np.arange(lo, hi)
    dk_rot = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for hh in range(r):
        h = g * r + hh
        qs = sl.take(q, layout, h)
        dos = sl.take(dout, layout, h)
        for blk in _blocks(rows, _block_rows(sl.L, p)):
            qr = rotate_half(qs[blk], query_position(blk, p), base)
            P, lse, O, cols = _row_block_fwd(gk, qr, blk, p, sl.L, scale, window)
            do = dos[blk]
            delta = (do * O).sum(axis=1)
            at = np.searchsorted(cols, keys)                 # the requested keys among the block's columns
            ok = (at < len(cols)) & (cols[np.minimum(at, len(cols) - 1)] == keys)
            Pk = np.zeros((len(blk), len(keys)))
            Pk[:, ok] = P[:, at[ok]]
            dS = Pk * (do @ gk.vals[keys].T - delta[:, None])
            dk_rot += scale * (dS.T @ qr)
            dv += Pk.T @ do
    dk = unrotate_half(dk_rot, gk.pos[keys], base)
    return dk, dv


def bwd(q, ks, vs, dout, p: int, *, layout: str = "bshd", cu_seqlens=None,
        scale: Optional[float] = None, base: float = 0.0, window: int = 0):
    """Full backward of pass p.  Returns (dQ like q, [dK(1..p)], [dV(1..p)]) in fp64."""
    Hq, D = q.shape[-2], q.shape[-1]
    Hkv = ks[0].shape[-2]
    r = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    dQ = np.zeros(q.shape)
    dK = [np.zeros(ks[0].shape) for _ in range(p)]
    dV = [np.zeros(vs[0].shape) for _ in range(p)]
    for sl in sequences(layout, q.shape, cu_seqlens):
        rows = np.arange(sl.L)
        for g in range(Hkv):
            dq, dk, dv = bwd_rows(q, ks, vs, dout, p, sl, g, rows, layout=layout, Hq=Hq,
                                  Hkv=Hkv, scale=scale, base=base, window=window)
            for hh in range(r):
                dQ[_row_index(layout, sl, rows) + (g * r + hh,)] = dq[hh]
            for qq in range(p):
                dK[qq][_row_index(layout, sl, rows) + (g,)] = dk[qq * sl.L:(qq + 1) * sl.L]
                dV[qq][_row_index(layout, sl, rows) + (g,)] = dv[qq * sl.L:(qq + 1) * sl.L]
    return dQ, dK, dV


# ----------------------------------------------------------------------------- ring steps
def ring_visible(q_pos, k_pos, window: int = 0) -> np.ndarray:
    """[n, m] causal visibility of pass-1 keys at sequence positions k_pos to the
    query rows at sequence positions q_pos (a row sees its own position); with a
    window, only the last `window` positions up to the row's own."""
    k = np.asarray(k_pos)[None, :]
    q = np.asarray(q_pos)[:, None]
    vis = k <= q
    if window > 0:
        vis = vis & (k > q - window)
    return vis


def fwd_chunk(q, k0, v0, branch_ks, branch_vs, p: int, *, q_offset: int, kv_offset: int,
              scale: Optional[float] = None, base: float = 0.0, window: int = 0):
    """One ring step of pass p, BSHD.  q: [B, n, Hq, D] rows at sequence positions
    q_offset + i; k0, v0: [B, m, Hkv, D] pass-1 keys at positions kv_offset + j;
    branch_ks, branch_vs: None, or the p-1 tensors [B, n, Hkv, D] of passes 2..p
    at the same rows.  Query row i is rotated to position q_offset + i + p - 1,
    trunk key j to kv_offset + j, the pass-q branch key of row i to
    q_offset + i + q - 1.  Returns (O [B, n, Hq, D], LSE [B, Hq, n]) in fp64,
    normalised over the keys this step sees."""
    B, n, Hq, D = q.shape
    m, Hkv = k0.shape[1], k0.shape[2]
    r = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(n)
    qpos = q_offset + rows
    O = np.zeros((B, n, Hq, D))
    lse = np.full((B, Hq, n), -np.inf)
    for b in range(B):
        for g in range(Hkv):
            kr = rotate_half(np.asarray(k0[b, :, g], np.float64), kv_offset + np.arange(m), base)   # [m, D]
            vv = np.asarray(v0[b, :, g], np.float64)
            vis = ring_visible(qpos, kv_offset + np.arange(m), window)                             # [n, m]
            bk, bv = [], []
            if branch_ks is not None:
                for t in range(2, p + 1):
                    bk.append(rotate_half(np.asarray(branch_ks[t - 2][b, :, g], np.float64),
                                          key_position(t, qpos), base))                          # [n, D]
                    bv.append(np.asarray(branch_vs[t - 2][b, :, g], np.float64))
            for h in range(g * r, (g + 1) * r):
                qr = rotate_half(np.asarray(q[b, :, h], np.float64), query_position(qpos, p), base)
                for i in range(n):
                    s = [scale * (kr[vis[i]] @ qr[i])]
                    vals = [vv[vis[i]]]
                    for t in range(len(bk)):
                        s.append(np.array([scale * (bk[t][i] @ qr[i])]))
                        vals.append(bv[t][i][None, :])
                    s = np.concatenate(s)
                    if s.size == 0:
                        continue                    # no visible key: O = 0, LSE = -inf
                    mx = s.max()
                    w = np.exp(s - mx)
                    lse[b, h, i] = mx + math.log(w.sum())
                    O[b, i, h] = (w / w.sum()) @ np.concatenate(vals, axis=0)
    return O, lse


def bwd_chunk(q, k0, v0, branch_ks, branch_vs, p: int, dout, o, lse, *, q_offset: int, kv_offset: int,
              scale: Optional[float] = None, base: float = 0.0, window: int = 0):
    """Backward contributions of one ring step (same inputs and positions as fwd_chunk).

    o and lse are the rows' final outputs over every key of the sequence (the
    merged ring result), so that P = exp(s - lse) and Delta = <dout, o> are the
    whole-sequence values; the step contributes the chain-rule terms of its own
    keys.  Returns (dq [B, n, Hq, D], dk0 [B, m, Hkv, D], dv0, [dk of passes 2..p],
    [dv of passes 2..p]) in fp64 (the branch lists are empty without branch
    keys); summing every step's terms gives the whole-sequence gradients."""
    B, n, Hq, D = q.shape
    m, Hkv = k0.shape[1], k0.shape[2]
    r = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(n)
    qpos = q_offset + rows
    kpos = kv_offset + np.arange(m)
    nb = p - 1 if branch_ks is not None else 0
    dq = np.zeros((B, n, Hq, D))
    dk0, dv0 = np.zeros((B, m, Hkv, D)), np.zeros((B, m, Hkv, D))
    dkb = [np.zeros((B, n, Hkv, D)) for _ in range(nb)]
    dvb = [np.zeros((B, n, Hkv, D)) for _ in range(nb)]
    for b in range(B):
        for g in range(Hkv):
            kr = rotate_half(np.asarray(k0[b, :, g], np.float64), kpos, base)
            vv = np.asarray(v0[b, :, g], np.float64)
            vis = ring_visible(qpos, kpos, window)
            bk = [rotate_half(np.asarray(branch_ks[t][b, :, g], np.float64), key_position(t + 2, qpos), base)
                  for t in range(nb)]
            bv = [np.asarray(branch_vs[t][b, :, g], np.float64) for t in range(nb)]
            dk_rot = np.zeros((m, D))
            dkb_rot = [np.zeros((n, D)) for _ in range(nb)]
            for h in range(g * r, (g + 1) * r):
                qr = rotate_half(np.asarray(q[b, :, h], np.float64), query_position(qpos, p), base)
                for i in range(n):
                    do = np.asarray(dout[b, i, h], np.float64)
                    delta = do @ np.asarray(o[b, i, h], np.float64)
                    L_i = float(lse[b, h, i])
                    dq_rot = np.zeros(D)
                    js = np.flatnonzero(vis[i])
                    if js.size:
                        P = np.exp(scale * (kr[js] @ qr[i]) - L_i)
                        dS = P * (vv[js] @ do - delta)
                        dq_rot += scale * (dS @ kr[js])
                        dk_rot[js] += scale * dS[:, None] * qr[i][None, :]
                        dv0[b, js, g] += P[:, None] * do[None, :]
                    for t in range(nb):
                        Pb = math.exp(scale * (bk[t][i] @ qr[i]) - L_i)
                        dSb = Pb * (bv[t][i] @ do - delta)
                        dq_rot += scale * dSb * bk[t][i]
                        dkb_rot[t][i] += scale * dSb * qr[i]
                        dvb[t][b, i, g] += Pb * do
                    dq[b, i, h] = unrotate_half(dq_rot, query_position(q_offset + i, p), base)
            dk0[b, :, g] = unrotate_half(dk_rot, kpos, base)
            for t in range(nb):
                dkb[t][b, :, g] = unrotate_half(dkb_rot[t], key_position(t + 2, qpos), base)
    return dq, dk0, dv0, dkb, dvb


def _thd_segments(cu_seqlens, kv_cu_seqlens):
    cu = [int(x) for x in cu_seqlens]
    kc = [int(x) for x in kv_cu_seqlens]
    if len(cu) != len(kc):
        raise ValueError("cu_seqlens and kv_cu_seqlens must list the same sequences")
    return [(cu[s], cu[s + 1], kc[s], kc[s + 1]) for s in range(len(cu) - 1)]


def fwd_chunk_thd(q, k0, v0, branch_ks, branch_vs, p: int, *, cu_seqlens, kv_cu_seqlens, q_offsets, kv_offsets,
                  scale: Optional[float] = None, base: float = 0.0, window: int = 0):
    """A packed (THD) ring step: q [T, Hq, D] holds the query rows of every sequence
    (cu_seqlens), k0 / v0 [Tk, Hkv, D] their pass-1 key rows (kv_cu_seqlens), branch_ks /
    branch_vs None or p-1 tensors [T, Hkv, D] at the query rows.  Sequence s is the ring
    step fwd_chunk of its own rows at q_offsets[s] against its own keys at kv_offsets[s].
    Returns (O [T, Hq, D], LSE [Hq, T])."""
    T, Hq, D = q.shape
    O = np.zeros((T, Hq, D))
    lse = np.full((Hq, T), -np.inf)
    for s, (a, e, ka, ke) in enumerate(_thd_segments(cu_seqlens, kv_cu_seqlens)):
        if e == a:
            continue
        bk = None if branch_ks is None else [np.asarray(t)[None, a:e] for t in branch_ks]
        bv = None if branch_vs is None else [np.asarray(t)[None, a:e] for t in branch_vs]
        o, l = fwd_chunk(np.asarray(q)[None, a:e], np.asarray(k0)[None, ka:ke], np.asarray(v0)[None, ka:ke], bk, bv,
                         p, q_offset=int(q_offsets[s]), kv_offset=int(kv_offsets[s]), scale=scale, base=base,
                         window=window)
        O[a:e] = o[0]
        lse[:, a:e] = l[0]
    return O, lse


def bwd_chunk_thd(q, k0, v0, branch_ks, branch_vs, p: int, dout, o, lse, *, cu_seqlens, kv_cu_seqlens, q_offsets,
                  kv_offsets, scale: Optional[float] = None, base: float = 0.0, window: int = 0):
    """Backward terms of a packed (THD) ring step (inputs as fwd_chunk_thd; o, lse the rows'
    whole-sequence outputs, LSE [Hq, T]): each sequence's bwd_chunk.  Returns (dq [T, Hq, D],
    dk0 [Tk, Hkv, D], dv0, [branch dk], [branch dv]); keys of a sequence without query rows
    get zeros."""
    T, Hq, D = q.shape
    Tk, Hkv = np.asarray(k0).shape[0], np.asarray(k0).shape[1]
    nb = p - 1 if branch_ks is not None else 0
    dq = np.zeros((T, Hq, D))
    dk0, dv0 = np.zeros((Tk, Hkv, D)), np.zeros((Tk, Hkv, D))
    dkb = [np.zeros((T, Hkv, D)) for _ in range(nb)]
    dvb = [np.zeros((T, Hkv, D)) for _ in range(nb)]
    for s, (a, e, ka, ke) in enumerate(_thd_segments(cu_seqlens, kv_cu_seqlens)):
        if e == a:
            continue
        bk = None if branch_ks is None else [np.asarray(t)[None, a:e] for t in branch_ks]
        bv = None if branch_vs is None else [np.asarray(t)[None, a:e] for t in branch_vs]
        r = bwd_chunk(np.asarray(q)[None, a:e], np.asarray(k0)[None, ka:ke], np.asarray(v0)[None, ka:ke], bk, bv, p,
                      np.asarray(dout)[None, a:e], np.asarray(o)[None, a:e], np.asarray(lse)[None, :, a:e],
                      q_offset=int(q_offsets[s]), kv_offset=int(kv_offsets[s]), scale=scale, base=base,
                      window=window)
        dq[a:e] = r[0][0]
        dk0[ka:ke] = r[1][0]
        dv0[ka:ke] = r[2][0]
        for t in range(nb):
            dkb[t][a:e] = r[3][t][0]
            dvb[t][a:e] = r[4][t][0]
    return dq, dk0, dv0, dkb, dvb


def merge(o_a, lse_a, o_b, lse_b):
    """Joint-LSE merge of two partial results over disjoint key sets of the same rows.
    o_*: [B, n, H, D]; lse_*: [B, H, n].  Rows with both LSEs -inf get O = 0, LSE = -inf."""
    la = np.asarray(lse_a, np.float64)
    lb = np.asarray(lse_b, np.float64)
    mx = np.maximum(la, lb)
    empty = mx == -np.inf
    mx_safe = np.where(empty, 0.0, mx)
    ea, eb = np.exp(la - mx_safe), np.exp(lb - mx_safe)
    tot = ea + eb
    L = np.where(empty, -np.inf, mx_safe + np.log(np.where(empty, 1.0, tot)))
    wa = np.where(empty, 0.0, ea / np.where(empty, 1.0, tot))
    wb = np.where(empty, 0.0, eb / np.where(empty, 1.0, tot))
    to_rows = lambda w: np.transpose(w, (0, 2, 1))[..., None]          # [B, H, n] -> [B, n, H, 1]
    return to_rows(wa) * np.asarray(o_a, np.float64) + to_rows(wb) * np.asarray(o_b, np.float64), L


# ----------------------------------------------------------------------------- block drafting
def block_visible_ctx(anchor: int, ctx_len: int) -> int:
    """Number of context keys (positions 0..n-1) a block anchored at `anchor` sees."""
    return int(min(max(anchor, 0), ctx_len))


def block_slot_position(anchor: int, t):
    """Sequence position of slot t of a block anchored at `anchor`."""
    return int(anchor) + np.asarray(t)


def block_fwd_rows(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs: int, b: int, h: int, rows, *,
                   scale: Optional[float] = None, base: float = 0.0):
    """O [n, D] and LSE [n] of block-draft rows `rows` (row = block * bs + slot) of
    batch b, query head h.  q, k_blk, v_blk: [B, nblk*bs, H, D]; k_ctx, v_ctx:
    [B, ctx_len, Hkv, D]; anchors: [B, nblk]."""
    Hq, D = q.shape[-2], q.shape[-1]
    Hkv, ctx_len = k_ctx.shape[-2], k_ctx.shape[1]
    g = h // (Hq // Hkv)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((len(rows), D))
    lse = np.full(len(rows), -np.inf)
    kc_all = rotate_half(np.asarray(k_ctx[b, :, g], np.float64), np.arange(ctx_len), base)  # key j at position j
    for n_i, row in enumerate(rows):
        blk, t = int(row) // bs, int(row) % bs
        a = int(min(max(int(anchors[b, blk]), 0), ctx_len))      # anchors are clamped to [0, ctx_len]
        nc = block_visible_ctx(a, ctx_len)
        qr = rotate_half(np.asarray(q[b, row, h], np.float64), block_slot_position(a, t), base)
        kc = kc_all[:nc]
        kb = rotate_half(np.asarray(k_blk[b, blk * bs:(blk + 1) * bs, g], np.float64),
                         block_slot_position(a, np.arange(bs)), base)
        keys = np.concatenate([kc, kb], axis=0)
        vals = np.concatenate([np.asarray(v_ctx[b, :nc, g], np.float64),
                               np.asarray(v_blk[b, blk * bs:(blk + 1) * bs, g], np.float64)], axis=0)
        s = scale * (keys @ qr)
        mx = s.max()
        w = np.exp(s - mx)
        lse[n_i] = mx + math.log(w.sum())
        O[n_i] = (w / w.sum()) @ vals
    return O, lse


def block_fwd(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs: int, *, scale: Optional[float] = None,
              base: float = 0.0):
    """Block-draft forward over every row: (O [B, nblk*bs, Hq, D], LSE [B, Hq, nblk*bs]) in fp64."""
    B, N, Hq, D = q.shape
    O = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            o_, l_ = block_fwd_rows(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs, b, h, np.arange(N), scale=scale,
                                    base=base)
            O[b, :, h] = o_
            lse[b, h] = l_
    return O, lse


def block_bwd_rows(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs: int, dout, b: int, h: int, rows, *,
                   scale: Optional[float] = None, base: float = 0.0):
    """Backward contributions of block-draft rows `rows` of batch b, query head h.

    Returns (dq [n, D], dk_ctx [ctx_len, D], dv_ctx [ctx_len, D], dk_blk [N, D],
    dv_blk [N, D]) where the key gradients hold only these rows' contributions
    (a key's gradient is complete once every row that sees it is included)."""
    Hq, D = q.shape[-2], q.shape[-1]
    Hkv, ctx_len = k_ctx.shape[-2], k_ctx.shape[1]
    N = q.shape[1]
    g = h // (Hq // Hkv)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((len(rows), D))
    dkc_rot, dvc = np.zeros((ctx_len, D)), np.zeros((ctx_len, D))
    dkb, dvb = np.zeros((N, D)), np.zeros((N, D))
    kc_all = rotate_half(np.asarray(k_ctx[b, :, g], np.float64), np.arange(ctx_len), base)
    for n_i, row in enumerate(rows):
        blk, t = int(row) // bs, int(row) % bs
        a = int(min(max(int(anchors[b, blk]), 0), ctx_len))
        nc = block_visible_ctx(a, ctx_len)
        pq = block_slot_position(a, t)
        qr = rotate_half(np.asarray(q[b, row, h], np.float64), pq, base)
        pb = block_slot_position(a, np.arange(bs))
        kbr = rotate_half(np.asarray(k_blk[b, blk * bs:(blk + 1) * bs, g], np.float64), pb, base)
        keys = np.concatenate([kc_all[:nc], kbr], axis=0)
        vals = np.concatenate([np.asarray(v_ctx[b, :nc, g], np.float64),
                               np.asarray(v_blk[b, blk * bs:(blk + 1) * bs, g], np.float64)], axis=0)
        s_ = scale * (keys @ qr)
        mx = s_.max()
        P = np.exp(s_ - mx)
        P /= P.sum()
        o = P @ vals
        do = np.asarray(dout[b, row, h], np.float64)
        dS = P * (vals @ do - do @ o)
        dq[n_i] = unrotate_half(scale * (dS @ keys), pq, base)
        dk_rot = scale * dS[:, None] * qr[None, :]
        dv = P[:, None] * do[None, :]
        dkc_rot[:nc] += dk_rot[:nc]
        dvc[:nc] += dv[:nc]
        dkb[blk * bs:(blk + 1) * bs] += unrotate_half(dk_rot[nc:], pb, base)
        dvb[blk * bs:(blk + 1) * bs] += dv[nc:]
    dkc = unrotate_half(dkc_rot, np.arange(ctx_len), base)
    return dq, dkc, dvc, dkb, dvb


def block_bwd(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs: int, dout, *, scale: Optional[float] = None,
              base: float = 0.0):
    """Block-draft backward over every row: (dQ, dK_ctx, dV_ctx, dK_blk, dV_blk) in fp64,
    shaped like q, k_ctx, v_ctx, k_blk, v_blk (GQA: key gradients summed over the group)."""
    B, N, Hq, D = q.shape
    dQ = np.zeros(q.shape)
    dKc, dVc = np.zeros(k_ctx.shape), np.zeros(v_ctx.shape)
    dKb, dVb = np.zeros(k_blk.shape), np.zeros(v_blk.shape)
    r = Hq // k_ctx.shape[-2]
    for b in range(B):
        for h in range(Hq):
            dq, dkc, dvc, dkb, dvb = block_bwd_rows(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs, dout, b, h,
                                                    np.arange(N), scale=scale, base=base)
            dQ[b, :, h] = dq
            dKc[b, :, h // r] += dkc
            dVc[b, :, h // r] += dvc
            dKb[b, :, h // r] += dkb
            dVb[b, :, h // r] += dvb
    return dQ, dKc, dVc, dKb, dVb


def _block_thd_segments(cu_seqlens, ctx_cu_seqlens, bs: int):
    cu = [int(x) for x in cu_seqlens]
    cc = [int(x) for x in ctx_cu_seqlens]
    if len(cu) != len(cc):
        raise ValueError("cu_seqlens and ctx_cu_seqlens must list the same sequences")
    if any(x % bs for x in cu):
        raise ValueError("every sequence holds whole blocks")
    return [(cu[s], cu[s + 1], cc[s], cc[s + 1]) for s in range(len(cu) - 1)]


def block_fwd_thd(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs: int, *, cu_seqlens, ctx_cu_seqlens,
                  scale: Optional[float] = None, base: float = 0.0):
    """Packed (THD) block drafting: q, k_blk, v_blk [T, H, D] hold every sequence's block
    rows (cu_seqlens, whole blocks each), k_ctx, v_ctx [Tc, Hkv, D] their contexts
    (ctx_cu_seqlens), anchors [T / bs] one per block in packed order.  Sequence s is
    block_fwd of its own rows, context and anchors (clamped to its own context length).
    Returns (O [T, Hq, D], LSE [Hq, T])."""
    T, Hq, D = q.shape
    O = np.zeros((T, Hq, D))
    lse = np.full((Hq, T), -np.inf)
    anchors = np.asarray(anchors)
    for a, e, ca, ce in _block_thd_segments(cu_seqlens, ctx_cu_seqlens, bs):
        if e == a:
            continue
        o, l = block_fwd(np.asarray(q)[None, a:e], np.asarray(k_ctx)[None, ca:ce], np.asarray(v_ctx)[None, ca:ce],
                         np.asarray(k_blk)[None, a:e], np.asarray(v_blk)[None, a:e], anchors[None, a // bs:e // bs],
                         bs, scale=scale, base=base)
        O[a:e] = o[0]
        lse[:, a:e] = l[0]
    return O, lse


def block_bwd_thd(q, k_ctx, v_ctx, k_blk, v_blk, anchors, bs: int, dout, *, cu_seqlens, ctx_cu_seqlens,
                  scale: Optional[float] = None, base: float = 0.0):
    """Backward of block_fwd_thd: each sequence's block_bwd.  Returns (dQ [T, Hq, D],
    dK_ctx, dV_ctx [Tc, Hkv, D], dK_blk, dV_blk [T, Hkv, D]); context rows of a sequence
    without block rows get zeros."""
    dQ = np.zeros(np.shape(q))
    dKc, dVc = np.zeros(np.shape(k_ctx)), np.zeros(np.shape(v_ctx))
    dKb, dVb = np.zeros(np.shape(k_blk)), np.zeros(np.shape(v_blk))
    anchors = np.asarray(anchors)
    for a, e, ca, ce in _block_thd_segments(cu_seqlens, ctx_cu_seqlens, bs):
        if e == a:
            continue
        r = block_bwd(np.asarray(q)[None, a:e], np.asarray(k_ctx)[None, ca:ce], np.asarray(v_ctx)[None, ca:ce],
                      np.asarray(k_blk)[None, a:e], np.asarray(v_blk)[None, a:e], anchors[None, a // bs:e // bs], bs,
                      np.asarray(dout)[None, a:e], scale=scale, base=base)
        dQ[a:e], dKc[ca:ce], dVc[ca:ce], dKb[a:e], dVb[a:e] = (x[0] for x in r)
    return dQ, dKc, dVc, dKb, dVb


# ----------------------------------------------------------------------------- distillation loss
def soft_ce_teacher_rows(B: int, S: int, offset: int, teacher_rows=None) -> np.ndarray:
    """int [B, S]: the teacher row each student row is scored against: the given table, or
    row i + offset of the same sequence."""
    if teacher_rows is not None:
        return np.asarray(teacher_rows, dtype=np.int64).reshape(B, S)
    return np.arange(S)[None, :].repeat(B, axis=0) + offset


def soft_ce_rows_counted(B: int, S: int, offset: int, mask=None, *, teacher_rows=None, teacher_len=None,
                         groups=None, num_groups: int = 1) -> np.ndarray:
    """bool [B, S]: row i is counted iff its teacher row exists (0 <= row < teacher_len,
    default S), mask[b, i] != 0 and its group is one of 0..num_groups-1."""
    tr = soft_ce_teacher_rows(B, S, offset, teacher_rows)
    ok = (tr >= 0) & (tr < (S if teacher_len is None else teacher_len))
    if mask is not None:
        ok = ok & (np.asarray(mask) != 0)
    if groups is not None:
        g = np.asarray(groups).reshape(B, S)
        ok = ok & (g >= 0) & (g < num_groups)
    return ok


def soft_ce_grouped(student, teacher, offset: int, mask=None, *, teacher_rows=None, groups=None,
                    num_groups: int = 1, weights=None):
    """Soft cross-entropy with per-row teacher rows and per-group normalisation.

    student [B, S, V], teacher [B, St, V] logits.  Row (b, i) is scored against
    softmax(teacher[b, teacher row]) (teacher row i + offset unless a table is given);
    counted rows per soft_ce_rows_counted.  Group g's loss is the mean of its counted
    rows' cross-entropies (0 when it has none); loss = sum_g w_g mean_g (w_g = 1 unless
    weights are given).  Returns (loss, grad [B, S, V] of that loss, row_ce [B, S],
    means [G], counts [G]) in fp64."""
    s = np.asarray(student, np.float64)
    t = np.asarray(teacher, np.float64)
    B, S, V = s.shape
    G = num_groups
    w = np.ones(G) if weights is None else np.asarray(weights, np.float64)
    tr = soft_ce_teacher_rows(B, S, offset, teacher_rows)
    counted = soft_ce_rows_counted(B, S, offset, mask, teacher_rows=teacher_rows, teacher_len=t.shape[1],
                                   groups=groups, num_groups=G)
    grp = np.zeros((B, S), dtype=np.int64) if groups is None else np.asarray(groups, np.int64).reshape(B, S)
    counts = np.array([int((counted & (grp == g)).sum()) for g in range(G)])
    row_ce = np.zeros((B, S))
    grad = np.zeros((B, S, V))
    for b in range(B):
        for i in range(S):
            if not counted[b, i]:
                continue
            x = s[b, i]
            y = t[b, tr[b, i]]
            lx = x.max() + math.log(np.exp(x - x.max()).sum())          # log-sum-exp of the student row
            py = np.exp(y - y.max())
            py /= py.sum()                                               # teacher distribution
            row_ce[b, i] = -(py * (x - lx)).sum()
            g = grp[b, i]
            grad[b, i] = w[g] * (np.exp(x - lx) - py) / counts[g]
    means = np.array([row_ce[counted & (grp == g)].sum() / counts[g] if counts[g] else 0.0 for g in range(G)])
    loss = float((w * means).sum())
    return loss, grad, row_ce, means, counts


def soft_ce(student, teacher, offset: int, mask=None):
    """Per-pass soft cross-entropy.  student, teacher: [B, S, V] logits.  Returns
    (loss, grad [B, S, V], row_ce [B, S]) in fp64 (row_ce is 0 on rows not counted)."""
    loss, grad, row_ce, _, _ = soft_ce_grouped(student, teacher, offset, mask)
    return loss, grad, row_ce
