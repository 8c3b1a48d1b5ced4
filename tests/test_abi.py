"""Boundary tests of the C ABI that need no GPU.

Every invalid argument is rejected on the host before anything is launched,
so these run on a machine without a GPU: pointers below are aligned integer
stand-ins that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import attention_ttt_attn_amd as tk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, never dereferenced


def header_functions():
    text = open(os.path.join(ROOT, "include", "tttattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = tk.library()
    names = header_functions()
    assert {"ttt_attn_fwd", "ttt_attn_bwd", "ttt_attn_workspace_bytes", "ttt_attn_status_string",
            "ttt_attn_last_error", "ttt_attn_abi_version", "ttt_attn_set_trace_hook"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ttt_attn_abi_version() == 4


def test_status_strings():
    lib = tk.library()
    for code in range(8):
        assert lib.ttt_attn_status_string(code).decode()
    assert lib.ttt_attn_status_string(99).decode() == "unknown status"


def good_desc(layout=tk.LAYOUT_BSHD, dtype=tk.DTYPE_BF16, D=128, p=3):
    d = tk.Desc()
    d.struct_size = ctypes.sizeof(tk.Desc)
    d.layout, d.dtype, d.o_dtype = layout, dtype, dtype
    d.batch, d.seqlen = 2, 100
    d.num_seqs = 3
    d.cu_seqlens = FAKE if layout == tk.LAYOUT_THD else None
    d.num_q_heads, d.num_kv_heads, d.head_dim = 8, 2, D
    d.pass_index = p
    d.softmax_scale = 0.0
    d.rope_base = 1e6
    return d


def ptrs(n, base=FAKE):
    arr = (ctypes.c_void_p * 16)()
    for i in range(min(n, 16)):
        arr[i] = base + 256 * i
    return arr


def call_fwd(d, q=FAKE, k=None, v=None, o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40):
    lib = tk.library()
    n = max(d.pass_index, 1) if d is not None else 1
    k = ptrs(n) if k is None else k
    v = ptrs(n) if v is None else v
    return lib.ttt_attn_fwd(ctypes.byref(d) if d is not None else None, q, k, v, o, lse, ws, ws_bytes, None)


def call_bwd(d, **kw):
    lib = tk.library()
    n = max(d.pass_index, 1)
    a = dict(q=FAKE, k=ptrs(n), v=ptrs(n), o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=ptrs(n), dv=ptrs(n),
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.ttt_attn_bwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                            a["dv"], a["ws"], a["ws_bytes"], None)


def err():
    return tk.library().ttt_attn_last_error().decode()


def test_null_descriptor_and_abi_mismatch():
    assert call_fwd(None) == 1 and "NULL" in err()
    d = good_desc()
    d.struct_size = 8
    assert call_fwd(d) == 7 and "struct_size" in err()


@pytest.mark.parametrize("field,value,code", [
    ("layout", 5, 2), ("dtype", 9, 3), ("num_kv_heads", 3, 2), ("num_q_heads", 0, 2), ("head_dim", 96, 3),
    ("head_dim", 31, 2), ("pass_index", 0, 2), ("pass_index", 17, 2), ("batch", 0, 2), ("seqlen", -1, 2),
    ("rope_base", -5.0, 2), ("rope_base", 0.5, 2), ("softmax_scale", float("nan"), 2),
])
def test_bad_descriptor_fields(field, value, code):
    d = good_desc()
    setattr(d, field, value)
    assert call_fwd(d) == code, err()
    assert err()


def test_bf16_head_dim_and_o_dtype_rules():
    lib = tk.library()
    # bf16 head_dim 32 / 64 run on zero-padded heads: a workspace for the padded copies
    # plus the D = 128 call's own; refused before any launch when it is too small
    w128 = lib.ttt_attn_workspace_bytes(ctypes.byref(good_desc(D=128)), 0)
    for D in (32, 64):
        d = good_desc(D=D)
        w = lib.ttt_attn_workspace_bytes(ctypes.byref(d), 0)
        assert w > w128
        assert lib.ttt_attn_workspace_bytes(ctypes.byref(d), 1) > w
        assert call_fwd(d, ws_bytes=w - 1) == 5 and "workspace" in err()
        assert call_fwd(d, q=None) == 1
    for D in (48, 96):
        assert call_fwd(good_desc(D=D)) == 3 and "head_dim" in err()
    # the padded route serves the whole-sequence calls only
    assert call_chunk(good_desc(D=64), good_chunk()) == 3 and "head_dim" in err()
    assert call_block(block_desc(), good_block()) != 3
    d64 = block_desc()
    d64.head_dim = 64
    assert call_block(d64, good_block()) == 3 and "head_dim" in err()
    d = good_desc(dtype=tk.DTYPE_FP32)
    d.o_dtype = tk.DTYPE_BF16
    assert call_fwd(d) == 3 and "o_dtype" in err()


def test_thd_needs_cu_seqlens_and_sequences():
    d = good_desc(layout=tk.LAYOUT_THD)
    d.cu_seqlens = None
    assert call_fwd(d) == 1 and "cu_seqlens" in err()
    d = good_desc(layout=tk.LAYOUT_THD)
    d.num_seqs = 0
    assert call_fwd(d) == 2


def test_null_and_misaligned_pointers():
    d = good_desc()
    assert call_fwd(d, q=None) == 1 and "q is NULL" in err()
    assert call_fwd(d, q=FAKE + 2) == 4 and "aligned" in err()
    assert call_fwd(d, o=None) == 1
    assert call_fwd(d, lse=None) == 1
    assert call_fwd(d, lse=FAKE + 2) == 4
    k = ptrs(3)
    k[2] = None
    assert call_fwd(d, k=k) == 1 and "k[2]" in err()
    v = ptrs(3)
    v[1] = FAKE + 8
    assert call_fwd(d, v=v) == 4 and "v[1]" in err()
    dk = ptrs(3)
    dk[0] = None
    assert call_bwd(d, dk=dk) == 1 and "dk[0]" in err()
    assert call_bwd(d, dout=None) == 1 and "dout" in err()


def test_strides_alignment():
    d = good_desc()
    d.q_stride[:] = (100 * 8 * 128, 8 * 128, 130)   # 130 elements = 260 bytes: not a multiple of 16 bytes
    assert call_fwd(d) == 4 and "stride" in err()
    d = good_desc()
    d.kv_stride[:] = (-1, 256, 128)
    assert call_fwd(d) == 2


def test_workspace_checks():
    lib = tk.library()
    d = good_desc()
    need_f = lib.ttt_attn_workspace_bytes(ctypes.byref(d), 0)
    need_b = lib.ttt_attn_workspace_bytes(ctypes.byref(d), 1)
    assert need_f > 0 and need_b > need_f
    assert call_fwd(d, ws=None) == 5 and "NULL" in err()
    assert call_fwd(d, ws_bytes=need_f - 1) == 5 and "smaller" in err()
    assert call_fwd(d, ws=FAKE + 16) == 5 and "256-byte" in err()
    assert call_bwd(d, ws_bytes=need_b - 1) == 5
    bad = good_desc()
    bad.pass_index = 0
    assert lib.ttt_attn_workspace_bytes(ctypes.byref(bad), 0) == 0 and err()


def test_workspace_grows_with_problem():
    lib = tk.library()
    d1, d2 = good_desc(), good_desc()
    d2.seqlen = 1000
    d3 = good_desc()
    d3.pass_index = 7
    w = lambda d, b: lib.ttt_attn_workspace_bytes(ctypes.byref(d), b)
    assert w(d2, 0) > w(d1, 0) and w(d2, 1) > w(d1, 1)
    assert w(d3, 0) >= w(d1, 0)       # the RoPE table grows by p - 1 positions
    t = good_desc(layout=tk.LAYOUT_THD)
    assert w(t, 0) > 0


def test_error_text_is_thread_local():
    import threading
    d = good_desc()
    assert call_fwd(d, q=None) == 1
    seen = {}

    def other():
        seen["text"] = err()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["text"] == "" and "q is NULL" in err()


# ----------------------------------------------------------------------------- ring steps and merge
def good_chunk(q_offset=256, kv_offset=0, kv_len=300, with_branch=1):
    c = tk.Chunk()
    c.struct_size = ctypes.sizeof(tk.Chunk)
    c.with_branch = with_branch
    c.q_offset, c.kv_offset, c.kv_len = q_offset, kv_offset, kv_len
    return c


def call_chunk(d, c, q=FAKE, k=None, v=None, o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40):
    lib = tk.library()
    k = ptrs(d.pass_index) if k is None else k
    v = ptrs(d.pass_index) if v is None else v
    return lib.ttt_attn_fwd_chunk(ctypes.byref(d), ctypes.byref(c) if c is not None else None, q, k, v, o, lse, ws,
                                  ws_bytes, None)


def test_chunk_struct_matches_header():
    assert ctypes.sizeof(tk.Chunk) == 88
    text = open(os.path.join(ROOT, "include", "tttattn.h")).read()
    assert "ttt_attn_chunk" in text and "kv0_stride[3]" in text
    for f in ("q_offsets", "kv_offsets", "kv_cu_seqlens", "max_position"):
        assert f in text


def thd_chunk(kv_len=300, max_position=5000):
    c = good_chunk(q_offset=0, kv_offset=0, kv_len=kv_len)
    c.q_offsets, c.kv_offsets, c.kv_cu_seqlens = FAKE, FAKE + 256, FAKE + 512
    c.max_position = max_position
    return c


def test_thd_chunk_validation():
    lib = tk.library()
    d = good_desc(layout=tk.LAYOUT_THD)
    w = lambda c: lib.ttt_attn_chunk_workspace_bytes(ctypes.byref(d), ctypes.byref(c))
    assert w(thd_chunk()) > 0
    for f in ("q_offsets", "kv_offsets", "kv_cu_seqlens"):
        c = thd_chunk()
        setattr(c, f, None)
        assert call_chunk(d, c) == 1 and "kv_cu_seqlens" in err()
    c = thd_chunk()
    c.q_offset = 5
    assert call_chunk(d, c) == 2 and "per-sequence" in err()
    for mp in (0, (1 << 30) + 1):
        assert call_chunk(d, thd_chunk(max_position=mp)) == 2 and "max_position" in err()
    assert call_chunk(d, thd_chunk(kv_len=1 << 30)) == 2 and "key" in err()
    # BSHD ring steps refuse the THD fields
    c = good_chunk()
    c.kv_cu_seqlens = FAKE
    assert call_chunk(good_desc(), c) == 2 and "THD fields" in err()
    # the workspace holds both row sets and the RoPE table of max_position rows
    assert w(thd_chunk(kv_len=4096)) > w(thd_chunk(kv_len=64))
    assert w(thd_chunk(max_position=100000)) > w(thd_chunk(max_position=5000))


def test_chunk_validation():
    lib = tk.library()
    d = good_desc()
    assert call_chunk(d, None) == 1 and "chunk" in err()
    c = good_chunk()
    c.struct_size = 8
    assert call_chunk(d, c) == 7 and "struct_size" in err()
    assert call_chunk(good_desc(layout=tk.LAYOUT_THD), good_chunk(q_offset=0)) == 1 and "THD" in err()
    assert call_chunk(good_desc(dtype=tk.DTYPE_FP32), good_chunk()) == 3 and "bf16" in err()
    for q_off, kv_off, kv_len in ((-1, 0, 10), (0, -64, 10), (0, 0, -1)):
        assert call_chunk(d, good_chunk(q_off, kv_off, kv_len)) == 2 and ">= 0" in err()
    assert call_chunk(d, good_chunk(q_offset=(1 << 30) - 50)) == 2 and "2^30" in err()
    assert call_chunk(d, good_chunk(kv_offset=1 << 30, kv_len=1)) == 2 and "2^30" in err()
    c = good_chunk()
    c.kv0_stride[:] = (300 * 2 * 128, 2 * 128, 100)     # head stride of 100 elements: not 16-byte aligned
    assert call_chunk(d, c) == 4 and "kv0" in err()
    assert lib.ttt_attn_chunk_workspace_bytes(ctypes.byref(d), None) == 0 and "chunk" in err()


def test_chunk_pointer_checks_follow_branch_flag():
    d = good_desc()                                    # p = 3
    k = ptrs(3)
    k[2] = None
    assert call_chunk(d, good_chunk(with_branch=1), k=k) == 1 and "k[2]" in err()
    k0 = ptrs(3)
    k0[0] = None
    assert call_chunk(d, good_chunk(with_branch=0), k=k0) == 1 and "k[0]" in err()
    # without the branch only pass 1 is read: a NULL k[2] passes the pointer checks and
    # the call stops at the (too small) workspace instead
    assert call_chunk(d, good_chunk(with_branch=0), k=k, ws_bytes=16) == 5
    assert call_chunk(d, good_chunk(), q=None) == 1 and "q is NULL" in err()
    assert call_chunk(d, good_chunk(), lse=FAKE + 2) == 4


def test_chunk_workspace_tracks_key_block():
    lib = tk.library()
    d = good_desc()
    w = lambda c: lib.ttt_attn_chunk_workspace_bytes(ctypes.byref(d), ctypes.byref(c))
    small, big = w(good_chunk(kv_len=64)), w(good_chunk(kv_len=4096))
    assert 0 < small < big
    assert call_chunk(d, good_chunk(kv_len=4096), ws_bytes=big - 1) == 5 and "smaller" in err()
    # the RoPE table covers the furthest position of either block
    assert w(good_chunk(q_offset=0, kv_offset=100000, kv_len=64)) > w(good_chunk(q_offset=0, kv_offset=0, kv_len=64))


def test_merge_validation():
    lib = tk.library()
    d = good_desc()
    d.o_dtype = tk.DTYPE_FP32
    call = lambda oa=FAKE, la=FAKE, ob=FAKE, lb=FAKE, o=FAKE, l=FAKE, desc=d: lib.ttt_attn_merge(
        ctypes.byref(desc), oa, la, ob, lb, o, l, None)
    assert call(oa=None) == 1 and "o_a" in err()
    assert call(ob=FAKE + 4) == 4 and "o_b" in err()
    assert call(o=None) == 1
    assert call(lb=None) == 1 and "lse_b" in err()
    assert call(l=FAKE + 2) == 4 and "lse" in err()
    bad = good_desc()
    bad.num_q_heads = 0
    assert call(desc=bad) == 2


# ----------------------------------------------------------------------------- block drafting
def good_block(bs=16, ctx_len=300, anchors=FAKE):
    bk = tk.Block()
    bk.struct_size = ctypes.sizeof(tk.Block)
    bk.block_size, bk.ctx_len, bk.anchors = bs, ctx_len, anchors
    return bk


def block_desc(rows=128):
    d = good_desc(p=1)
    d.seqlen = rows
    return d


def call_block(d, bk, q=FAKE, kc=FAKE, vc=FAKE, kb=FAKE, vb=FAKE, o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return tk.library().ttt_attn_block_fwd(ctypes.byref(d), ctypes.byref(bk) if bk is not None else None, q, kc, vc,
                                           kb, vb, o, lse, ws, ws_bytes, None)


def test_block_struct_matches_header():
    assert ctypes.sizeof(tk.Block) == 56
    text = open(os.path.join(ROOT, "include", "tttattn.h")).read()
    assert "ttt_attn_block" in text and "ctx_cu_seqlens" in text


def test_thd_block_validation():
    lib = tk.library()
    d = good_desc(layout=tk.LAYOUT_THD, p=1)         # 100 rows: not whole blocks of 16
    d.seqlen = 128
    bk = good_block()
    assert call_block(d, bk) == 1 and "ctx_cu_seqlens" in err()
    bk.ctx_cu_seqlens = FAKE
    w = lambda dd, b: lib.ttt_attn_block_workspace_bytes(ctypes.byref(dd), ctypes.byref(b), 0)
    assert w(d, bk) > 0
    assert call_block(d, bk, ws_bytes=16) == 5      # the arguments pass; the workspace is too small
    d2 = good_desc(layout=tk.LAYOUT_THD, p=1)
    assert call_block(d2, bk) == 2 and "blocks" in err()
    # BSHD refuses a context cu_seqlens
    b2 = good_block()
    b2.ctx_cu_seqlens = FAKE
    assert call_block(block_desc(), b2) == 2 and "ctx_cu_seqlens" in err()
    # the workspace holds both row sets per sequence
    big = good_block(ctx_len=8192)
    big.ctx_cu_seqlens = FAKE
    assert w(d, big) > w(d, bk)
    assert lib.ttt_attn_block_workspace_bytes(ctypes.byref(d), ctypes.byref(bk), 1) > w(d, bk)


def test_block_validation():
    lib = tk.library()
    d = block_desc()
    assert call_block(d, None) == 1 and "block" in err()
    bk = good_block()
    bk.struct_size = 4
    assert call_block(d, bk) == 7
    for bs in (0, 3, 64):
        assert call_block(d, good_block(bs=bs)) == 3 and "block_size" in err()
    assert call_block(block_desc(rows=100), good_block(bs=16)) == 2 and "blocks" in err()
    assert call_block(d, good_block(ctx_len=-1)) == 2 and "ctx_len" in err()
    dd = block_desc()
    dd.pass_index = 2
    assert call_block(dd, good_block()) == 2 and "pass_index" in err()
    assert call_block(good_desc(layout=tk.LAYOUT_THD, p=1), good_block()) == 1 and "ctx_cu_seqlens" in err()
    assert call_block(good_desc(dtype=tk.DTYPE_FP32, p=1), good_block()) == 3
    assert call_block(d, good_block(anchors=None)) == 1 and "anchors" in err()
    assert call_block(d, good_block(anchors=FAKE + 2)) == 4
    assert call_block(d, good_block(), kb=None) == 1 and "k_blk" in err()
    assert call_block(d, good_block(), kc=FAKE + 8) == 4 and "k_ctx" in err()
    assert call_block(d, good_block(), lse=None) == 1
    bk = good_block()
    bk.ctx_stride[:] = (300 * 256, 256, 100)
    assert call_block(d, bk) == 4 and "ctx stride" in err()
    need = lib.ttt_attn_block_workspace_bytes(ctypes.byref(d), ctypes.byref(good_block()), 0)
    assert need > 0 and call_block(d, good_block(), ws_bytes=need - 1) == 5
    need_b = lib.ttt_attn_block_workspace_bytes(ctypes.byref(d), ctypes.byref(good_block()), 1)
    assert need_b > need


def test_block_empty_context_pointers_may_be_null():
    # ctx_len = 0: the context is never read, so NULL k_ctx / v_ctx pass the pointer checks
    # (the call then stops at the workspace check, before any launch)
    assert call_block(block_desc(), good_block(ctx_len=0), kc=None, vc=None, ws_bytes=16) == 5
    assert call_block(block_desc(), good_block(ctx_len=5), kc=None, ws_bytes=16) == 1


def test_block_workspace_grows():
    lib = tk.library()
    w = lambda d, bk: lib.ttt_attn_block_workspace_bytes(ctypes.byref(d), ctypes.byref(bk), 0)
    assert w(block_desc(128), good_block(ctx_len=4096)) > w(block_desc(128), good_block(ctx_len=64))
    assert w(block_desc(4096), good_block()) > w(block_desc(128), good_block())


def call_block_bwd(d, bk, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kb=FAKE, vb=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dkc=FAKE, dvc=FAKE,
             dkb=FAKE, dvb=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return tk.library().ttt_attn_block_bwd(ctypes.byref(d), ctypes.byref(bk), a["q"], a["kc"], a["vc"], a["kb"],
                                           a["vb"], a["o"], a["lse"], a["dout"], a["dq"], a["dkc"], a["dvc"],
                                           a["dkb"], a["dvb"], a["ws"], a["ws_bytes"], None)


def test_block_bwd_validation():
    d = block_desc()
    assert call_block_bwd(d, good_block(bs=3)) == 3
    for name in ("q", "kb", "vb", "o", "dout", "dq", "dkb", "dvb"):
        assert call_block_bwd(d, good_block(), **{name: None}) == 1, name
    for name in ("kc", "vc", "dkc", "dvc"):
        assert call_block_bwd(d, good_block(), **{name: None}) == 1, name
        # an empty context is never touched: NULL passes, and the call stops at the workspace check
        assert call_block_bwd(d, good_block(ctx_len=0), ws_bytes=16, **{name: None}) == 5, name
    assert call_block_bwd(d, good_block(), lse=FAKE + 2) == 4
    assert call_block_bwd(d, good_block(anchors=None)) == 1
    assert call_block_bwd(d, good_block(), ws_bytes=100) == 5


# ----------------------------------------------------------------------------- soft cross-entropy
def ce_desc(B=2, S=100, V=4096, off=1):
    d = tk.SoftCeDesc()
    d.struct_size = ctypes.sizeof(tk.SoftCeDesc)
    d.batch, d.seqlen, d.vocab, d.teacher_offset = B, S, V, off
    return d


def test_soft_ce_struct_and_validation():
    lib = tk.library()
    assert ctypes.sizeof(tk.SoftCeDesc) == 88
    fwd = lambda d, s=FAKE, t=FAKE, st=FAKE, ll=FAKE, rc=FAKE, ws=FAKE, n=1 << 40: lib.ttt_soft_ce_fwd(
        ctypes.byref(d) if d is not None else None, s, t, st, ll, rc, ws, n, None)
    bwd = lambda d, s=FAKE, t=FAKE, ll=FAKE, st=FAKE, dl=FAKE, g=FAKE: lib.ttt_soft_ce_bwd(
        ctypes.byref(d), s, t, ll, st, dl, g, None)
    assert fwd(None) == 1
    d = ce_desc()
    d.struct_size = 4
    assert fwd(d) == 7
    assert fwd(ce_desc(V=100)) == 2 and "vocab" in err()
    assert fwd(ce_desc(V=0)) == 2
    assert fwd(ce_desc(off=-1)) == 2 and "teacher_offset" in err()
    assert fwd(ce_desc(B=0)) == 2
    d = ce_desc()
    d.student_stride[:] = (100 * 4100, 4100)
    assert fwd(d) == 4 and "student" in err()
    d = ce_desc()
    d.teacher_stride[:] = (100 * 4096, 4000)
    assert fwd(d) == 2 and "teacher" in err()
    assert fwd(ce_desc(), s=None) == 1 and "student" in err()
    assert fwd(ce_desc(), t=FAKE + 8) == 4 and "teacher" in err()
    assert fwd(ce_desc(), st=None) == 1
    assert fwd(ce_desc(), ll=FAKE + 2) == 4
    assert fwd(ce_desc(), rc=None, ws=None) == 5 and "workspace" in err()
    assert fwd(ce_desc(), rc=None, n=16) == 5
    assert lib.ttt_soft_ce_workspace_bytes(ctypes.byref(ce_desc())) >= 2 * 100 * 4
    assert bwd(ce_desc(), g=None) == 1 and "dstudent" in err()
    assert bwd(ce_desc(), dl=None) == 1 and "dloss" in err()
    assert bwd(ce_desc(), ll=FAKE + 2) == 4
    # per-row teacher rows and normalisation groups
    d = ce_desc()
    d.num_groups = 65
    assert fwd(d) == 2 and "num_groups" in err()
    d = ce_desc()
    d.num_groups = -1
    assert fwd(d) == 2
    d = ce_desc()
    d.teacher_seqlen = -3
    assert fwd(d) == 2 and "teacher_seqlen" in err()
    d = ce_desc()
    d.groups = FAKE + 2
    assert fwd(d) == 4 and "groups" in err()
    d = ce_desc()
    d.teacher_rows = FAKE + 1
    assert bwd(d) == 4


def test_window_validation():
    d = good_desc()
    d.window = -1
    assert call_fwd(d) == 2 and "window" in err()
    d = good_desc(dtype=tk.DTYPE_FP32)
    d.window = 8
    assert call_fwd(d) == 3 and "window" in err()
    d = block_desc()
    d.window = 4
    assert call_block(d, good_block()) == 3 and "window" in err()
    assert ctypes.sizeof(tk.Desc) == 152


def test_chunk_bwd_validation():
    lib = tk.library()
    d = good_desc()
    call = lambda c, **kw: lib.ttt_attn_bwd_chunk(
        ctypes.byref(d), ctypes.byref(c) if c is not None else None, kw.get("q", FAKE), kw.get("k", ptrs(3)),
        kw.get("v", ptrs(3)), kw.get("o", FAKE), kw.get("lse", FAKE), kw.get("dout", FAKE), kw.get("dq", FAKE),
        kw.get("dk", ptrs(3)), kw.get("dv", ptrs(3)), FAKE, kw.get("ws_bytes", 1 << 40), None)
    assert call(None) == 1 and "chunk" in err()
    assert call(good_chunk(), dq=None) == 1 and "dq" in err()
    dk = ptrs(3)
    dk[2] = None
    assert call(good_chunk(with_branch=1), dk=dk) == 1 and "dk[2]" in err()
    # without the branch only pass 1 is touched: the call stops at the workspace check
    assert call(good_chunk(with_branch=0), dk=dk, ws_bytes=16) == 5
    assert lib.ttt_attn_chunk_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(good_chunk())) > \
        lib.ttt_attn_chunk_workspace_bytes(ctypes.byref(d), ctypes.byref(good_chunk()))
    dt = good_desc(layout=tk.LAYOUT_THD)
    assert lib.ttt_attn_bwd_chunk(ctypes.byref(dt), ctypes.byref(good_chunk(q_offset=0)), FAKE, ptrs(3), ptrs(3),
                                  FAKE, FAKE, FAKE, FAKE, ptrs(3), ptrs(3), FAKE, 1 << 40, None) == 1
    assert "kv_cu_seqlens" in err()
    # a THD ring step stops at the (too small) workspace once its arguments pass
    assert lib.ttt_attn_bwd_chunk(ctypes.byref(dt), ctypes.byref(thd_chunk()), FAKE, ptrs(3), ptrs(3), FAKE, FAKE,
                                  FAKE, FAKE, ptrs(3), ptrs(3), FAKE, 16, None) == 5


def test_token_stride_limit():
    lib = tk.library()
    d = good_desc()
    d.o_stride[0], d.o_stride[1], d.o_stride[2] = (1 << 26) * 64, 1 << 26, 128
    assert lib.ttt_attn_workspace_bytes(ctypes.byref(d), 0) == 0 and "token stride" in err()
    d = good_desc()
    d.kv_stride[0], d.kv_stride[1], d.kv_stride[2] = (1 << 25) * 64, 1 << 25, 128
    assert lib.ttt_attn_workspace_bytes(ctypes.byref(d), 0) > 0


def test_noalloc_forward_refusals():
    """The allocation-free forward refuses, before touching the GPU, a problem whose workspace
    exceeds its static scratch, and THD's host-side cu_seqlens check (a synchronisation)."""
    lib = tk.library()
    d = good_desc()
    d.batch, d.seqlen, d.num_q_heads, d.num_kv_heads = 4, 4096, 32, 8
    assert tk.workspace_bytes(d, False) > (64 << 20)
    rc = lib.ttt_attn_fwd_noalloc(ctypes.byref(d), FAKE, ptrs(3), ptrs(3), FAKE, FAKE, None)
    assert rc == 5 and "static" in lib.ttt_attn_last_error().decode()
    d2 = good_desc(layout=tk.LAYOUT_THD)
    d2.check_cu_seqlens = 1
    assert lib.ttt_attn_fwd_noalloc(ctypes.byref(d2), FAKE, ptrs(3), ptrs(3), FAKE, FAKE, None) == 3
    bad = good_desc(p=0)
    assert lib.ttt_attn_fwd_noalloc(ctypes.byref(bad), FAKE, ptrs(3), ptrs(3), FAKE, FAKE, None) == 2


def test_slab_offset_limit():
    """Problems whose workspace slabs would overflow the kernels' 32-bit offsets are refused;
    the largest accepted ones still plan a workspace."""
    lib = tk.library()
    d = good_desc()
    d.batch, d.num_q_heads, d.num_kv_heads = 1, 8, 8
    d.seqlen = 8_000_000                         # 2 * 127 * slots just below 2^31
    assert tk.workspace_bytes(d, True) > 0
    d.seqlen = 8_500_000                         # 2 * 127 * slots past 2^31
    assert lib.ttt_attn_workspace_bytes(ctypes.byref(d), 1) == 0
    assert "32-bit" in lib.ttt_attn_last_error().decode()
    rc = lib.ttt_attn_fwd(ctypes.byref(d), FAKE, ptrs(3), ptrs(3), FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == 2
    d.batch, d.num_q_heads, d.seqlen = 2, 64, 4_500_000   # 4 B Hq slots past 2^31
    assert lib.ttt_attn_workspace_bytes(ctypes.byref(d), 1) == 0


def test_bwd_mode_stored_ds_workspace():
    """bwd_mode: STORED_DS keeps the trunk dS of bf16 BSHD passes without a window (B * Hq
    causal 32x32 blocks of 2 KB each, n (n + 1) / 2 with n = ceil(S / 32)) when they fit the
    cap; RECOMPUTE (the default), THD, a window and fp32 need none of it; any other value is
    refused."""
    lib = tk.library()
    w = lambda d, b: lib.ttt_attn_workspace_bytes(ctypes.byref(d), b)
    rec = good_desc()
    sto = good_desc()
    sto.bwd_mode = tk.BWD_STORED_DS
    assert rec.bwd_mode == tk.BWD_RECOMPUTE == 0
    n = (rec.seqlen + 31) // 32
    blocks = rec.batch * rec.num_q_heads * n * (n + 1) // 2
    assert w(sto, 1) - w(rec, 1) >= blocks * 2048
    assert w(sto, 1) - w(rec, 1) < blocks * 2048 + 4096   # plus the V bounds
    assert w(sto, 0) == w(rec, 0)                           # forward: unchanged
    for mk in (lambda: good_desc(layout=tk.LAYOUT_THD), lambda: good_desc(dtype=tk.DTYPE_FP32)):
        r, a = mk(), mk()
        a.bwd_mode = tk.BWD_STORED_DS
        assert w(a, 1) == w(r, 1)
    r, a = good_desc(), good_desc()
    a.window = r.window = 16
    a.bwd_mode = tk.BWD_STORED_DS
    assert w(a, 1) == w(r, 1)
    # past the cap (one 65536-token sequence, 32 heads: 64 GiB of blocks) it recomputes
    big, big_r = good_desc(), good_desc()
    for d in (big, big_r):
        d.batch, d.seqlen, d.num_q_heads, d.num_kv_heads = 1, 65536, 32, 8
    big.bwd_mode = tk.BWD_STORED_DS
    n = 65536 // 32
    assert 32 * n * (n + 1) // 2 * 2048 > tk.STORED_DS_MAX_BYTES
    assert w(big, 1) == w(big_r, 1) > 0
    d = good_desc()
    d.bwd_mode = 2
    assert w(d, 1) == 0 and "bwd_mode" in err()
    assert call_bwd(d) == 2 and "bwd_mode" in err()
