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
    assert lib.ttt_attn_abi_version() == 1


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
    d = good_desc(D=64)
    assert call_fwd(d) == 3 and "head_dim" in err()
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
