"""Python binding of libtttattn (multi-pass EAGLE-3 TTT draft attention, MI355X).

Thin ctypes marshalling over the C ABI in include/tttattn.h: torch is used only
to own device memory and to name the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path, and
importing the functions fails loudly when the built library is missing.

    o, lse = fwd(q, ks, vs, p, rope_base=1e6)
    dq, dks, dvs = bwd(q, ks, vs, o, lse, dout, p, rope_base=1e6)

`ks`/`vs` are the pass 1..p key/value tensors (index 0 = pass 1 = trunk).  BSHD
tensors are [B, S, H, D]; pass `cu_seqlens` (int32 on the device) for THD
tensors [T, H, D].
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Sequence

__all__ = ["fwd", "bwd", "workspace_bytes", "set_trace_hook", "TTTAttnError", "library", "library_path", "Desc",
           "LAYOUT_BSHD", "LAYOUT_THD", "DTYPE_BF16", "DTYPE_FP32", "STATUS", "fwd_noalloc"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libtttattn.so")

LAYOUT_BSHD, LAYOUT_THD = 0, 1
DTYPE_BF16, DTYPE_FP32 = 0, 1
STATUS = {0: "TTT_OK", 1: "TTT_ERR_NULL_ARG", 2: "TTT_ERR_BAD_SHAPE", 3: "TTT_ERR_UNSUPPORTED",
          4: "TTT_ERR_MISALIGNED", 5: "TTT_ERR_WORKSPACE", 6: "TTT_ERR_HIP", 7: "TTT_ERR_ABI"}
MAX_PASSES = 16
BWD_RECOMPUTE, BWD_STORED_DS = 0, 1
STORED_DS_MAX_BYTES = 40 << 30


class Desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("layout", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("check_cu_seqlens", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("pass_index", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("q_stride", ctypes.c_int64 * 3),
        ("kv_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("window", ctypes.c_int32),
        ("bwd_mode", ctypes.c_int32),
        ("aux_stream", ctypes.c_void_p),
    ]


class Chunk(ctypes.Structure):
    """One ring step: query rows at q_offset.., pass-1 keys at kv_offset.. (ttt_attn_chunk); THD:
    per-sequence offsets and packed key rows."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("with_branch", ctypes.c_int32),
        ("q_offset", ctypes.c_int64),
        ("kv_offset", ctypes.c_int64),
        ("kv_len", ctypes.c_int64),
        ("kv0_stride", ctypes.c_int64 * 3),
        ("q_offsets", ctypes.c_void_p),
        ("kv_offsets", ctypes.c_void_p),
        ("kv_cu_seqlens", ctypes.c_void_p),
        ("max_position", ctypes.c_int64),
    ]


class Block(ctypes.Structure):
    """Block-draft shape (ttt_attn_block)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("block_size", ctypes.c_int32),
        ("ctx_len", ctypes.c_int64),
        ("anchors", ctypes.c_void_p),
        ("ctx_stride", ctypes.c_int64 * 3),
        ("ctx_cu_seqlens", ctypes.c_void_p),
    ]


class SoftCeDesc(ctypes.Structure):
    """Per-pass soft cross-entropy shape (ttt_soft_ce_desc)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("teacher_offset", ctypes.c_int32),
        ("teacher_seqlen", ctypes.c_int32),
        ("student_stride", ctypes.c_int64 * 2),
        ("teacher_stride", ctypes.c_int64 * 2),
        ("mask", ctypes.c_void_p),
        ("teacher_rows", ctypes.c_void_p),
        ("groups", ctypes.c_void_p),
        ("num_groups", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


# void (*)(void* user, const char* kernel, int phase, void* stream)
TRACE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int, ctypes.c_void_p)
_trace_ref = None


def set_trace_hook(fn) -> None:
    """Install fn(kernel_name: str, phase: int, stream_handle: int) around every
    kernel launch of later calls on this thread (phase 0 before, 1 after);
    None removes it."""
    global _trace_ref
    if fn is None:
        _trace_ref = None
        library().ttt_attn_set_trace_hook(TRACE_FN(), None)
        return
    _trace_ref = TRACE_FN(lambda user, name, phase, stream: fn(name.decode(), phase, stream))
    library().ttt_attn_set_trace_hook(_trace_ref, None)


class TTTAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libtttattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"libtttattn.so not found at {library_path}; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(library_path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.ttt_attn_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int]
        lib.ttt_attn_workspace_bytes.restype = sz
        lib.ttt_attn_fwd.argtypes = [ctypes.POINTER(Desc), vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp,
                                     sz, vp]
        lib.ttt_attn_fwd.restype = ctypes.c_int
        lib.ttt_attn_fwd_noalloc.argtypes = [ctypes.POINTER(Desc), vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                             vp, vp]
        lib.ttt_attn_fwd_noalloc.restype = ctypes.c_int
        lib.ttt_attn_bwd.argtypes = [ctypes.POINTER(Desc), vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp,
                                     ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp]
        lib.ttt_attn_bwd.restype = ctypes.c_int
        lib.ttt_attn_chunk_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Chunk)]
        lib.ttt_attn_chunk_workspace_bytes.restype = sz
        lib.ttt_attn_fwd_chunk.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Chunk), vp, ctypes.POINTER(vp),
                                           ctypes.POINTER(vp), vp, vp, vp, sz, vp]
        lib.ttt_attn_fwd_chunk.restype = ctypes.c_int
        lib.ttt_attn_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Chunk)]
        lib.ttt_attn_chunk_bwd_workspace_bytes.restype = sz
        lib.ttt_attn_bwd_chunk.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Chunk), vp, ctypes.POINTER(vp),
                                           ctypes.POINTER(vp), vp, vp, vp, vp, ctypes.POINTER(vp),
                                           ctypes.POINTER(vp), vp, sz, vp]
        lib.ttt_attn_bwd_chunk.restype = ctypes.c_int
        lib.ttt_attn_merge.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp]
        lib.ttt_attn_merge.restype = ctypes.c_int
        lib.ttt_attn_block_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Block), ctypes.c_int]
        lib.ttt_attn_block_workspace_bytes.restype = sz
        lib.ttt_attn_block_fwd.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Block), vp, vp, vp, vp, vp, vp, vp,
                                           vp, sz, vp]
        lib.ttt_attn_block_fwd.restype = ctypes.c_int
        lib.ttt_attn_block_bwd.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Block)] + [vp] * 14 + [sz, vp]
        lib.ttt_attn_block_bwd.restype = ctypes.c_int
        lib.ttt_soft_ce_workspace_bytes.argtypes = [ctypes.POINTER(SoftCeDesc)]
        lib.ttt_soft_ce_workspace_bytes.restype = sz
        lib.ttt_soft_ce_fwd.argtypes = [ctypes.POINTER(SoftCeDesc), vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ttt_soft_ce_fwd.restype = ctypes.c_int
        lib.ttt_soft_ce_bwd.argtypes = [ctypes.POINTER(SoftCeDesc), vp, vp, vp, vp, vp, vp, vp]
        lib.ttt_soft_ce_bwd.restype = ctypes.c_int
        lib.ttt_attn_status_string.argtypes = [ctypes.c_int]
        lib.ttt_attn_status_string.restype = ctypes.c_char_p
        lib.ttt_attn_last_error.argtypes = []
        lib.ttt_attn_last_error.restype = ctypes.c_char_p
        lib.ttt_attn_abi_version.argtypes = []
        lib.ttt_attn_abi_version.restype = ctypes.c_int
        lib.ttt_attn_set_trace_hook.argtypes = [TRACE_FN, ctypes.c_void_p]
        lib.ttt_attn_set_trace_hook.restype = None
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise TTTAttnError(status, library().ttt_attn_last_error().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _strides3(t, thd: bool):
    s = t.stride()
    if s[-1] != 1:
        raise ValueError("the head_dim axis must be contiguous")
    return (0, s[0], s[1]) if thd else (s[0], s[1], s[2])


def make_desc(q, ks, p: int, *, cu_seqlens=None, softmax_scale: float = 0.0, rope_base: float = 0.0,
              o_dtype: Optional[int] = None, o_like=None, check_cu_seqlens: bool = False, window: int = 0) -> Desc:
    thd = cu_seqlens is not None
    d = Desc()
    d.struct_size = ctypes.sizeof(Desc)
    d.layout = LAYOUT_THD if thd else LAYOUT_BSHD
    d.dtype = _dtype_code(q)
    d.o_dtype = d.dtype if o_dtype is None else o_dtype
    if thd:
        d.batch, d.seqlen = 1, q.shape[0]
        d.num_seqs = cu_seqlens.numel() - 1
        d.cu_seqlens = cu_seqlens.data_ptr()
    else:
        d.batch, d.seqlen = q.shape[0], q.shape[1]
    d.check_cu_seqlens = int(bool(check_cu_seqlens))
    d.num_q_heads, d.head_dim = q.shape[-2], q.shape[-1]
    d.num_kv_heads = ks[0].shape[-2]
    d.pass_index = p
    d.softmax_scale = softmax_scale
    d.rope_base = rope_base
    d.q_stride[:] = _strides3(q, thd)
    d.kv_stride[:] = _strides3(ks[0], thd)
    d.o_stride[:] = _strides3(o_like if o_like is not None else q, thd)
    d.window = int(window)
    return d


def workspace_bytes(desc: Desc, for_bwd: bool) -> int:
    return int(library().ttt_attn_workspace_bytes(ctypes.byref(desc), int(bool(for_bwd))))


def _ptrs(ts):
    arr = (ctypes.c_void_p * MAX_PASSES)()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr()
    return arr


def _on_stream(fn):
    """Runs a call with its `stream` argument current, so that the outputs and the workspace it
    allocates belong to the stream its kernels run on: the caching allocator then hands the
    workspace to other work only after that stream's kernels."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with _torch().cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapped


_AUX_STREAMS = {}


def _aux_stream(aux, device) -> int:
    """Handle of a backward call's second stream: "auto" = one per device, created on first use at
    the default priority and kept by this module; None = none (the whole call on its stream); or a
    torch.cuda.Stream of the caller's."""
    if aux is None:
        return 0
    if isinstance(aux, str):
        if aux != "auto":
            raise ValueError(f"aux_stream: 'auto', None or a torch.cuda.Stream, not {aux!r}")
        torch = _torch()
        key = torch.device(device).index
        if key not in _AUX_STREAMS:
            _AUX_STREAMS[key] = torch.cuda.Stream(device=device)
        aux = _AUX_STREAMS[key]
    return int(aux.cuda_stream)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, ws):
    torch = _torch()
    if nbytes == 0:
        return None
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    return ws


def _ws_ptr(ws):
    if ws is None:
        return None, 0
    addr = ws.data_ptr()
    aligned = (addr + 255) & ~255
    return ctypes.c_void_p(aligned), ws.numel() - (aligned - addr)


@_on_stream
def fwd(q, ks: Sequence, vs: Sequence, p: int, *, cu_seqlens=None, softmax_scale: float = 0.0,
        rope_base: float = 0.0, o_fp32: bool = False, out=None, lse=None, workspace=None, stream=None,
        check_cu_seqlens: bool = False, window: int = 0):
    """Forward of TTT pass p.  Returns (o, lse); lse is fp32 [B,Hq,S] or [Hq,T]."""
    torch = _torch()
    thd = cu_seqlens is not None
    o_dtype = DTYPE_FP32 if (o_fp32 or q.dtype == torch.float32) else _dtype_code(q)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if o_dtype == DTYPE_FP32 else q.dtype, device=q.device)
    if lse is None:
        shape = (q.shape[-2], q.shape[0]) if thd else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    d = make_desc(q, ks, p, cu_seqlens=cu_seqlens, softmax_scale=softmax_scale, rope_base=rope_base,
                  o_dtype=o_dtype, o_like=out, check_cu_seqlens=check_cu_seqlens, window=window)
    if any(t.stride() != ks[0].stride() for t in list(ks[:p]) + list(vs[:p])):
        raise ValueError("every k and v must share one set of strides")
    nbytes = workspace_bytes(d, False)
    ws = _workspace(nbytes, q.device, workspace)
    wp, wn = _ws_ptr(ws)
    _check(library().ttt_attn_fwd(ctypes.byref(d), q.data_ptr(), _ptrs(ks[:p]), _ptrs(vs[:p]), out.data_ptr(),
                                  lse.data_ptr(), wp, wn, _stream(stream)))
    return out, lse


@_on_stream
def fwd_noalloc(q, ks: Sequence, vs: Sequence, p: int, out, lse, *, cu_seqlens=None, softmax_scale: float = 0.0,
                rope_base: float = 0.0, stream=None, window: int = 0):
    """Forward of TTT pass p through ttt_attn_fwd_noalloc: the library's static per-GPU scratch
    replaces the workspace, and the caller passes the outputs (nothing is allocated here)."""
    torch = _torch()
    o_dtype = DTYPE_FP32 if out.dtype == torch.float32 else _dtype_code(out)
    d = make_desc(q, ks, p, cu_seqlens=cu_seqlens, softmax_scale=softmax_scale, rope_base=rope_base,
                  o_dtype=o_dtype, o_like=out, window=window)
    if any(t.stride() != ks[0].stride() for t in list(ks[:p]) + list(vs[:p])):
        raise ValueError("every k and v must share one set of strides")
    _check(library().ttt_attn_fwd_noalloc(ctypes.byref(d), q.data_ptr(), _ptrs(ks[:p]), _ptrs(vs[:p]),
                                          out.data_ptr(), lse.data_ptr(), _stream(stream)))
    return out, lse


@_on_stream
def bwd(q, ks: Sequence, vs: Sequence, o, lse, dout, p: int, *, cu_seqlens=None, softmax_scale: float = 0.0,
        rope_base: float = 0.0, dq=None, dks=None, dvs=None, workspace=None, stream=None,
        check_cu_seqlens: bool = False, window: int = 0, stored_ds: bool = False, aux_stream="auto"):
    """Backward of TTT pass p.  Returns (dq, [dk_1..dk_p], [dv_1..dv_p]).  stored_ds: the dK/dV kernel
    stores dS and dQ is formed from it (BWD_STORED_DS; bf16 BSHD without a window, else ignored).
    aux_stream: the second stream the HBM-bound kernels may run on ("auto", None or a stream)."""
    torch = _torch()
    o_dtype = _dtype_code(o)
    d = make_desc(q, ks, p, cu_seqlens=cu_seqlens, softmax_scale=softmax_scale, rope_base=rope_base,
                  o_dtype=o_dtype, o_like=o, check_cu_seqlens=check_cu_seqlens, window=window)
    d.bwd_mode = BWD_STORED_DS if stored_ds else BWD_RECOMPUTE
    d.aux_stream = _aux_stream(aux_stream, q.device)
    if dout.stride() != o.stride():
        raise ValueError("dout must have the strides of o")
    like = lambda t: torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)
    if dq is None:
        dq = like(q)
    if dks is None:
        dks = [like(ks[0]) for _ in range(p)]
    if dvs is None:
        dvs = [like(vs[0]) for _ in range(p)]
    # gradients are written with the strides of their primal
    if dq.stride() != q.stride() or any(t.stride() != ks[0].stride() for t in list(dks[:p]) + list(dvs[:p])):
        raise ValueError("dq must have the strides of q, dk/dv those of k")
    if any(t.stride() != ks[0].stride() for t in list(ks[:p]) + list(vs[:p])):
        raise ValueError("every k and v must share one set of strides")
    nbytes = workspace_bytes(d, True)
    ws = _workspace(nbytes, q.device, workspace)
    wp, wn = _ws_ptr(ws)
    _check(library().ttt_attn_bwd(ctypes.byref(d), q.data_ptr(), _ptrs(ks[:p]), _ptrs(vs[:p]), o.data_ptr(),
                                  lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), _ptrs(dks[:p]), _ptrs(dvs[:p]),
                                  wp, wn, _stream(stream)))
    return dq, dks, dvs


def make_chunk(q_offset: int, kv_offset: int, k0, *, with_branch: bool, thd=None) -> Chunk:
    """thd: None (BSHD), or (q_offsets, kv_offsets, kv_cu_seqlens, max_position) with device int32
    tensors for the per-sequence offsets and the packed key rows."""
    c = Chunk()
    c.struct_size = ctypes.sizeof(Chunk)
    c.with_branch = int(bool(with_branch))
    c.q_offset, c.kv_offset = int(q_offset), int(kv_offset)
    if thd is None:
        c.kv_len = k0.shape[1]
        c.kv0_stride[:] = _strides3(k0, False)
    else:
        qo, ko, kcu, max_position = thd
        for name, t in (("q_offsets", qo), ("kv_offsets", ko), ("kv_cu_seqlens", kcu)):
            if t.dtype != _torch().int32 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 tensor")
        c.kv_len = k0.shape[0]
        c.kv0_stride[:] = _strides3(k0, True)
        c.q_offsets, c.kv_offsets, c.kv_cu_seqlens = qo.data_ptr(), ko.data_ptr(), kcu.data_ptr()
        c.max_position = int(max_position)
    return c


def _thd_chunk(cu_seqlens, kv_cu_seqlens, q_offsets, kv_offsets, max_position):
    if cu_seqlens is None:
        if any(x is not None for x in (kv_cu_seqlens, q_offsets, kv_offsets)):
            raise ValueError("kv_cu_seqlens, q_offsets and kv_offsets belong to THD (cu_seqlens) ring steps")
        return None
    if any(x is None for x in (kv_cu_seqlens, q_offsets, kv_offsets)):
        raise ValueError("a THD ring step needs kv_cu_seqlens, q_offsets and kv_offsets")
    n = cu_seqlens.numel() - 1
    if q_offsets.numel() != n or kv_offsets.numel() != n or kv_cu_seqlens.numel() != n + 1:
        raise ValueError("q_offsets / kv_offsets need one entry per sequence, kv_cu_seqlens one more")
    return (q_offsets, kv_offsets, kv_cu_seqlens, max_position)


@_on_stream
def fwd_chunk(q, ks: Sequence, vs: Sequence, p: int, *, q_offset: int = 0, kv_offset: int = 0, with_branch: bool,
              softmax_scale: float = 0.0, rope_base: float = 0.0, o_fp32: bool = True, out=None, lse=None,
              workspace=None, stream=None, window: int = 0, cu_seqlens=None, kv_cu_seqlens=None, q_offsets=None,
              kv_offsets=None, max_position: int = 0, check_cu_seqlens: bool = False):
    """One ring step (bf16): the rows of q (positions q_offset..) against the pass-1 keys ks[0], vs[0]
    (positions kv_offset..), plus the branch keys ks[1:p], vs[1:p] of those rows when with_branch.
    THD (cu_seqlens): q [T, Hq, D] packs every sequence's query rows, ks[0] / vs[0] [Tk, Hkv, D] their
    pass-1 keys (kv_cu_seqlens); sequence s takes its step at q_offsets[s] / kv_offsets[s], and every
    position stays below max_position.  Returns (o, lse) normalised over the keys this step sees
    (rows that see none: o = 0, lse = -inf); lse is [B, Hq, S] or [Hq, T]."""
    torch = _torch()
    thd = _thd_chunk(cu_seqlens, kv_cu_seqlens, q_offsets, kv_offsets, max_position)
    o_dtype = DTYPE_FP32 if o_fp32 else _dtype_code(q)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if o_dtype == DTYPE_FP32 else q.dtype, device=q.device)
    if lse is None:
        shape = (q.shape[1], q.shape[0]) if thd else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    branch_ks = list(ks[1:p]) if with_branch else []
    d = make_desc(q, (branch_ks or [ks[0]]), p, softmax_scale=softmax_scale, rope_base=rope_base, o_dtype=o_dtype,
                  o_like=out, window=window, cu_seqlens=cu_seqlens, check_cu_seqlens=check_cu_seqlens)
    if branch_ks and any(t.stride() != branch_ks[0].stride() for t in branch_ks + list(vs[1:p])):
        raise ValueError("every branch k and v must share one set of strides")
    if vs[0].stride() != ks[0].stride():
        raise ValueError("k[0] and v[0] must share one set of strides")
    c = make_chunk(q_offset, kv_offset, ks[0], with_branch=with_branch, thd=thd)
    nbytes = int(library().ttt_attn_chunk_workspace_bytes(ctypes.byref(d), ctypes.byref(c)))
    if nbytes == 0:
        raise TTTAttnError(2, library().ttt_attn_last_error().decode())
    ws = _workspace(nbytes, q.device, workspace)
    wp, wn = _ws_ptr(ws)
    n = p if with_branch else 1
    _check(library().ttt_attn_fwd_chunk(ctypes.byref(d), ctypes.byref(c), q.data_ptr(), _ptrs(ks[:n]),
                                        _ptrs(vs[:n]), out.data_ptr(), lse.data_ptr(), wp, wn, _stream(stream)))
    return out, lse


@_on_stream
def bwd_chunk(q, ks: Sequence, vs: Sequence, o, lse, dout, p: int, *, q_offset: int = 0, kv_offset: int = 0,
              with_branch: bool, softmax_scale: float = 0.0, rope_base: float = 0.0, window: int = 0,
              workspace=None, stream=None, cu_seqlens=None, kv_cu_seqlens=None, q_offsets=None, kv_offsets=None,
              max_position: int = 0, check_cu_seqlens: bool = False, aux_stream="auto"):
    """Backward terms of one ring step (bf16 inputs; BSHD, or THD as in fwd_chunk): o, lse, dout are
    the query rows' whole-sequence values.  Returns fp32 (dq, [dk0, branch dk...], [dv0, branch
    dv...]); the branch lists hold passes 2..p only with with_branch.  Summing the steps' terms
    gives the whole-sequence gradients.  aux_stream: as for bwd."""
    torch = _torch()
    thd = _thd_chunk(cu_seqlens, kv_cu_seqlens, q_offsets, kv_offsets, max_position)
    n_br = p - 1 if with_branch else 0
    branch_ks = list(ks[1:p]) if with_branch else []
    d = make_desc(q, (branch_ks or [ks[0]]), p, softmax_scale=softmax_scale, rope_base=rope_base,
                  o_dtype=_dtype_code(o), o_like=o, window=window, cu_seqlens=cu_seqlens,
                  check_cu_seqlens=check_cu_seqlens)
    d.aux_stream = _aux_stream(aux_stream, q.device)
    if dout.stride() != o.stride():
        raise ValueError("dout must have the strides of o")
    lse = lse.contiguous()  # the C ABI reads the step rows' LSE as a dense [B, Hq, rows] / [Hq, T] array
    c = make_chunk(q_offset, kv_offset, ks[0], with_branch=with_branch, thd=thd)

    def like32(t):  # fp32 output with t's element strides (dense layouts keep their strides)
        return torch.empty_strided(t.shape, t.stride(), dtype=torch.float32, device=t.device)
    dq = like32(q)
    dks = [like32(ks[0])] + [like32(t) for t in branch_ks]
    dvs = [like32(vs[0])] + [like32(t) for t in list(vs[1:p])[:n_br]]
    nbytes = int(library().ttt_attn_chunk_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(c)))
    if nbytes == 0:
        raise TTTAttnError(2, library().ttt_attn_last_error().decode())
    ws = _workspace(nbytes, q.device, workspace)
    wp, wn = _ws_ptr(ws)
    nptr = 1 + n_br
    kp, vp_ = _ptrs(list(ks[:nptr])), _ptrs(list(vs[:nptr]))
    if ks[0].numel() == 0:
        kp[0] = vp_[0] = None
    gk, gv = _ptrs(dks), _ptrs(dvs)
    if ks[0].numel() == 0:
        gk[0] = gv[0] = None
    _check(library().ttt_attn_bwd_chunk(ctypes.byref(d), ctypes.byref(c), q.data_ptr(), kp, vp_, o.data_ptr(),
                                        lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), gk, gv, wp, wn,
                                        _stream(stream)))
    return dq, dks, dvs


@_on_stream
def merge(o_a, lse_a, o_b, lse_b, *, out=None, lse=None, cu_seqlens=None, stream=None):
    """Joint-LSE merge of two partial results over disjoint key sets of the same rows.
    out/lse may be o_a/lse_a (in-place accumulation).  Returns (o, lse)."""
    torch = _torch()
    if o_a.shape != o_b.shape or o_a.dtype != o_b.dtype or o_a.stride() != o_b.stride():
        raise ValueError("o_a and o_b must match in shape, dtype and strides")
    if out is None:
        out = torch.empty_strided(o_a.shape, o_a.stride(), dtype=o_a.dtype, device=o_a.device)
    if lse is None:
        lse = torch.empty_like(lse_a)
    if out.stride() != o_a.stride():
        raise ValueError("out must have the strides of o_a")
    thd = cu_seqlens is not None
    d = Desc()
    d.struct_size = ctypes.sizeof(Desc)
    d.layout = LAYOUT_THD if thd else LAYOUT_BSHD
    d.dtype = DTYPE_BF16 if o_a.dtype != torch.float32 else DTYPE_FP32
    d.o_dtype = _dtype_code(o_a)
    if thd:
        d.batch, d.seqlen = 1, o_a.shape[0]
        d.num_seqs = cu_seqlens.numel() - 1
        d.cu_seqlens = cu_seqlens.data_ptr()
    else:
        d.batch, d.seqlen = o_a.shape[0], o_a.shape[1]
    d.num_q_heads = d.num_kv_heads = o_a.shape[-2]
    d.head_dim = o_a.shape[-1]
    d.pass_index = 1
    d.q_stride[:] = _strides3(o_a, thd) if o_a.dtype != torch.float32 or d.dtype == DTYPE_FP32 else (0, 0, 0)
    d.kv_stride[:] = (0, 0, 0)
    d.o_stride[:] = _strides3(o_a, thd)
    _check(library().ttt_attn_merge(ctypes.byref(d), o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                    lse_b.data_ptr(), out.data_ptr(), lse.data_ptr(), _stream(stream)))
    return out, lse


def make_block(block_size: int, k_ctx, anchors, ctx_cu_seqlens=None) -> Block:
    """ctx_cu_seqlens: None (BSHD), or the device int32 cu_seqlens of the packed contexts (THD)."""
    thd = ctx_cu_seqlens is not None
    bk = Block()
    bk.struct_size = ctypes.sizeof(Block)
    bk.block_size = int(block_size)
    bk.ctx_len = k_ctx.shape[0] if thd else k_ctx.shape[1]
    bk.anchors = anchors.data_ptr() if anchors is not None else None
    bk.ctx_stride[:] = _strides3(k_ctx, thd) if k_ctx.numel() else (0, 0, 0)
    if thd:
        if ctx_cu_seqlens.dtype != _torch().int32 or not ctx_cu_seqlens.is_contiguous():
            raise ValueError("ctx_cu_seqlens must be a contiguous int32 tensor")
        bk.ctx_cu_seqlens = ctx_cu_seqlens.data_ptr()
    return bk


def _block_thd(cu_seqlens, ctx_cu_seqlens):
    if (cu_seqlens is None) != (ctx_cu_seqlens is None):
        raise ValueError("THD block drafting takes both cu_seqlens and ctx_cu_seqlens")
    if cu_seqlens is not None and ctx_cu_seqlens.numel() != cu_seqlens.numel():
        raise ValueError("cu_seqlens and ctx_cu_seqlens must list the same sequences")
    return cu_seqlens is not None


@_on_stream
def block_fwd(q, k_ctx, v_ctx, k_blk, v_blk, anchors, block_size: int, *, softmax_scale: float = 0.0,
              rope_base: float = 0.0, o_fp32: bool = False, out=None, lse=None, workspace=None, stream=None,
              cu_seqlens=None, ctx_cu_seqlens=None, check_cu_seqlens: bool = False):
    """Block-draft forward (bf16).  BSHD: q [B, N, Hq, D] with N = nblk * block_size;
    k_ctx, v_ctx [B, ctx_len, Hkv, D]; k_blk, v_blk [B, N, Hkv, D]; anchors int32
    [B, nblk] on the device; returns (o, lse [B, Hq, N]).  THD (cu_seqlens of the block
    rows, whole blocks per sequence, and ctx_cu_seqlens of the contexts): q [T, Hq, D],
    k_ctx, v_ctx [Tc, Hkv, D], anchors [T / block_size]; returns (o, lse [Hq, T])."""
    torch = _torch()
    thd = _block_thd(cu_seqlens, ctx_cu_seqlens)
    o_dtype = DTYPE_FP32 if o_fp32 else _dtype_code(q)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if o_dtype == DTYPE_FP32 else q.dtype, device=q.device)
    if lse is None:
        shape = (q.shape[1], q.shape[0]) if thd else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    if anchors.dtype != torch.int32:
        raise TypeError("anchors must be int32")
    if k_blk.stride() != v_blk.stride() or k_ctx.stride() != v_ctx.stride():
        raise ValueError("k and v of the context (and of the blocks) must share strides")
    d = make_desc(q, [k_blk], 1, softmax_scale=softmax_scale, rope_base=rope_base, o_dtype=o_dtype, o_like=out,
                  cu_seqlens=cu_seqlens, check_cu_seqlens=check_cu_seqlens)
    bk = make_block(block_size, k_ctx, anchors, ctx_cu_seqlens)
    nbytes = int(library().ttt_attn_block_workspace_bytes(ctypes.byref(d), ctypes.byref(bk), 0))
    if nbytes == 0:
        raise TTTAttnError(2, library().ttt_attn_last_error().decode())
    ws = _workspace(nbytes, q.device, workspace)
    wp, wn = _ws_ptr(ws)
    ptr = lambda t: t.data_ptr() if t.numel() else None
    _check(library().ttt_attn_block_fwd(ctypes.byref(d), ctypes.byref(bk), q.data_ptr(), ptr(k_ctx), ptr(v_ctx),
                                        k_blk.data_ptr(), v_blk.data_ptr(), out.data_ptr(), lse.data_ptr(), wp, wn,
                                        _stream(stream)))
    return out, lse


@_on_stream
def block_bwd(q, k_ctx, v_ctx, k_blk, v_blk, anchors, block_size: int, o, lse, dout, *, softmax_scale: float = 0.0,
              rope_base: float = 0.0, dq=None, dk_ctx=None, dv_ctx=None, dk_blk=None, dv_blk=None, workspace=None,
              stream=None, cu_seqlens=None, ctx_cu_seqlens=None, check_cu_seqlens: bool = False):
    """Block-draft backward (BSHD, or THD as in block_fwd).  Returns (dq, dk_ctx, dv_ctx, dk_blk, dv_blk)."""
    torch = _torch()
    _block_thd(cu_seqlens, ctx_cu_seqlens)
    like = lambda t: torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)
    dq = like(q) if dq is None else dq
    dk_ctx = like(k_ctx) if dk_ctx is None else dk_ctx
    dv_ctx = like(v_ctx) if dv_ctx is None else dv_ctx
    dk_blk = like(k_blk) if dk_blk is None else dk_blk
    dv_blk = like(v_blk) if dv_blk is None else dv_blk
    if dout.stride() != o.stride():
        raise ValueError("dout must have the strides of o")
    if dq.stride() != q.stride() or dk_blk.stride() != k_blk.stride() or dv_blk.stride() != k_blk.stride():
        raise ValueError("gradients take the strides of their primal")
    if k_ctx.numel() and (dk_ctx.stride() != k_ctx.stride() or dv_ctx.stride() != k_ctx.stride()):
        raise ValueError("gradients take the strides of their primal")
    if k_blk.stride() != v_blk.stride() or k_ctx.stride() != v_ctx.stride():
        raise ValueError("k and v of the context (and of the blocks) must share strides")
    d = make_desc(q, [k_blk], 1, softmax_scale=softmax_scale, rope_base=rope_base, o_dtype=_dtype_code(o), o_like=o,
                  cu_seqlens=cu_seqlens, check_cu_seqlens=check_cu_seqlens)
    bk = make_block(block_size, k_ctx, anchors, ctx_cu_seqlens)
    nbytes = int(library().ttt_attn_block_workspace_bytes(ctypes.byref(d), ctypes.byref(bk), 1))
    if nbytes == 0:
        raise TTTAttnError(2, library().ttt_attn_last_error().decode())
    ws = _workspace(nbytes, q.device, workspace)
    wp, wn = _ws_ptr(ws)
    ptr = lambda t: t.data_ptr() if t.numel() else None
    _check(library().ttt_attn_block_bwd(ctypes.byref(d), ctypes.byref(bk), q.data_ptr(), ptr(k_ctx), ptr(v_ctx),
                                        k_blk.data_ptr(), v_blk.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        dout.data_ptr(), dq.data_ptr(), ptr(dk_ctx), ptr(dv_ctx), dk_blk.data_ptr(),
                                        dv_blk.data_ptr(), wp, wn, _stream(stream)))
    return dq, dk_ctx, dv_ctx, dk_blk, dv_blk


def make_soft_ce_desc(student, teacher, teacher_offset: int, mask=None, teacher_rows=None, groups=None,
                      num_groups: int = 1) -> SoftCeDesc:
    d = SoftCeDesc()
    d.struct_size = ctypes.sizeof(SoftCeDesc)
    d.batch, d.seqlen, d.vocab = student.shape
    if teacher.shape[0] != student.shape[0] or teacher.shape[2] != student.shape[2]:
        raise ValueError("student [B, S, V] and teacher [B, St, V] logits must share B and V")
    if teacher.shape[1] != student.shape[1] and teacher_rows is None:
        raise ValueError("a teacher of another length needs teacher_rows")
    if student.stride(-1) != 1 or teacher.stride(-1) != 1:
        raise ValueError("the vocab axis must be contiguous")
    d.teacher_offset = int(teacher_offset)
    d.teacher_seqlen = teacher.shape[1]
    d.student_stride[:] = student.stride()[:2]
    d.teacher_stride[:] = teacher.stride()[:2]
    d.mask = mask.data_ptr() if mask is not None else None
    d.teacher_rows = teacher_rows.data_ptr() if teacher_rows is not None else None
    d.groups = groups.data_ptr() if groups is not None else None
    d.num_groups = int(num_groups)
    return d


@_on_stream
def soft_ce_fwd(student, teacher, teacher_offset: int, *, mask=None, row_ce=None, teacher_rows=None, groups=None,
                num_groups: int = 1, stream=None):
    """Per-pass soft cross-entropy.  student bf16 [B, S, V], teacher bf16 [B, St, V]; mask uint8
    [B, S]; teacher_rows / groups int32 [B, S] (per-row teacher row, normalisation group).
    Returns (stats [2 + 2G] = (loss, counted rows, then (mean, count) per group),
    row_lse [B, S, 2], row_ce [B, S])."""
    torch = _torch()
    d = make_soft_ce_desc(student, teacher, teacher_offset, mask, teacher_rows, groups, num_groups)
    B, S, _ = student.shape
    stats = torch.empty(2 + 2 * max(1, int(num_groups)), dtype=torch.float32, device=student.device)
    row_lse = torch.empty((B, S, 2), dtype=torch.float32, device=student.device)
    if row_ce is None:
        row_ce = torch.empty((B, S), dtype=torch.float32, device=student.device)
    _check(library().ttt_soft_ce_fwd(ctypes.byref(d), student.data_ptr(), teacher.data_ptr(), stats.data_ptr(),
                                     row_lse.data_ptr(), row_ce.data_ptr(), None, 0, _stream(stream)))
    return stats, row_lse, row_ce


@_on_stream
def soft_ce_bwd(student, teacher, teacher_offset: int, row_lse, stats, dloss, *, mask=None, teacher_rows=None,
                groups=None, num_groups: int = 1, dstudent=None, stream=None):
    """Gradient with respect to the student logits (bf16, student strides); dloss: fp32 device
    [G], the upstream gradient of each group's mean."""
    torch = _torch()
    d = make_soft_ce_desc(student, teacher, teacher_offset, mask, teacher_rows, groups, num_groups)
    if dloss.numel() < max(1, int(num_groups)):
        raise ValueError("dloss needs one value per group")
    if dstudent is None:
        dstudent = torch.empty_strided(student.shape, student.stride(), dtype=student.dtype, device=student.device)
    if dstudent.stride() != student.stride():
        raise ValueError("dstudent must have the strides of student")
    _check(library().ttt_soft_ce_bwd(ctypes.byref(d), student.data_ptr(), teacher.data_ptr(), row_lse.data_ptr(),
                                     stats.data_ptr(), dloss.data_ptr(), dstudent.data_ptr(), _stream(stream)))
    return dstudent
