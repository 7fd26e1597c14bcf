"""Python binding of libattn_sink.so: sink attention forward / backward on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and the current stream. The functions raise if the library was
not built (``python -m attention_learnable_sinks_attn_amd.build``); there is no fallback.

The operation (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section
"GPT-OSS中的带注意力槽的注意力机制"): softmax over each row's visible scores plus one learnable
per-head logit S_h, which takes probability mass but adds nothing to the output.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = ["fwd", "bwd", "bwd_noalloc", "decode_fwd", "decode_fwd_ordered", "bwd_workspace_bytes", "decode_workspace_bytes", "bwd_kernel_names",
           "decode_kernel_names", "check_cu_seqlens", "library_path", "load_library", "AttnSinkError",
           "ERROR_CODES", "HEAD_DIMS"]

HEAD_DIMS = (64, 128)  # head_dim values the kernels are built for
_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libattn_sink.so")
_lib = None

ERROR_CODES = {
    0: "ATTN_SINK_OK", -1: "ATTN_SINK_ERR_NULL_PTR", -2: "ATTN_SINK_ERR_BAD_SHAPE",
    -3: "ATTN_SINK_ERR_UNSUPPORTED", -4: "ATTN_SINK_ERR_BAD_WINDOW", -5: "ATTN_SINK_ERR_WORKSPACE",
    -6: "ATTN_SINK_ERR_HIP", -7: "ATTN_SINK_ERR_ALIGN", -8: "ATTN_SINK_ERR_BAD_SEQLENS", -9: "ATTN_SINK_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_SINK_NOALLOC_SCRATCH_BYTES


class AttnSinkError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERROR_CODES.get(code, code)} ({_strerror(code)})")
        self.code = code


class Shape(ctypes.Structure):
    """Mirror of ``attn_sink_shape`` in include/attn_sink.h."""
    _fields_ = [("total_tokens", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("num_heads_q", ctypes.c_int32), ("num_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("out_dtype", ctypes.c_int32)]


class DecodeShape(ctypes.Structure):
    """Mirror of ``attn_sink_decode_shape`` in include/attn_sink.h."""
    _fields_ = [("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("max_q", ctypes.c_int32), ("max_k", ctypes.c_int32), ("num_heads_q", ctypes.c_int32),
                ("num_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libattn_sink.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m attention_learnable_sinks_attn_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    shp = ctypes.POINTER(Shape)
    lib.attn_sink_fwd.argtypes = [vp, vp, vp, vp, i32, i32, vp, shp, vp, vp, vp]
    lib.attn_sink_fwd.restype = i32
    lib.attn_sink_bwd_workspace_bytes.argtypes = [shp]
    lib.attn_sink_bwd_workspace_bytes.restype = sz
    bwd_args = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, shp, vp, sz, vp, vp, vp, vp, vp]
    lib.attn_sink_bwd.argtypes = bwd_args
    lib.attn_sink_bwd.restype = i32
    lib.attn_sink_bwd_timed.argtypes = bwd_args + [ctypes.POINTER(ctypes.c_void_p), i32]
    lib.attn_sink_bwd_timed.restype = i32
    lib.attn_sink_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, shp, vp, vp, vp, vp, vp]
    lib.attn_sink_bwd_noalloc.restype = i32
    lib.attn_sink_bwd_num_kernels.argtypes = []
    lib.attn_sink_bwd_num_kernels.restype = i32
    lib.attn_sink_bwd_kernel_name.argtypes = [i32]
    lib.attn_sink_bwd_kernel_name.restype = ctypes.c_char_p
    dshp = ctypes.POINTER(DecodeShape)
    lib.attn_sink_decode_workspace_bytes.argtypes = [dshp]
    lib.attn_sink_decode_workspace_bytes.restype = sz
    lib.attn_sink_decode_fwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, dshp, vp, sz, vp, vp, vp]
    lib.attn_sink_decode_fwd.restype = i32
    lib.attn_sink_decode_fwd_timed.argtypes = [vp, vp, vp, vp, i32, vp, vp, dshp, vp, sz, vp, vp, vp,
                                               ctypes.POINTER(ctypes.c_void_p), i32]
    lib.attn_sink_decode_fwd_timed.restype = i32
    lib.attn_sink_decode_fwd_ordered.argtypes = [vp, vp, vp, vp, i32, vp, vp, dshp, vp, vp, vp]
    lib.attn_sink_decode_fwd_ordered.restype = i32
    lib.attn_sink_decode_num_kernels.restype = i32
    lib.attn_sink_decode_kernel_name.argtypes = [i32]
    lib.attn_sink_decode_kernel_name.restype = ctypes.c_char_p
    lib.attn_sink_check_cu_seqlens.argtypes = [vp, i32, i32, i32]
    lib.attn_sink_check_cu_seqlens.restype = i32
    lib.attn_sink_strerror.argtypes = [i32]
    lib.attn_sink_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load_library().attn_sink_strerror(int(code)).decode()
    except Exception:  # pragma: no cover - message only
        return "?"


_OUT_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


def make_shape(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
               softmax_scale: Optional[float], out_dtype: torch.dtype = torch.float32) -> Shape:
    if out_dtype not in _OUT_DTYPES:
        raise TypeError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    return Shape(int(q.shape[0]), int(cu_seqlens.numel()) - 1, int(max_seqlen), int(q.shape[1]), int(k.shape[1]),
                 int(q.shape[2]), float(softmax_scale) if softmax_scale else 0.0, _OUT_DTYPES[out_dtype])


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else (t.data_ptr() or None)


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _shape_of(t: torch.Tensor, name: str, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor, cu_seqlens: torch.Tensor,
               total_k: Optional[int] = None):
    """Shapes the kernels assume (they trust every size): q [Tq, Hq, d], k / v [Tk, Hkv, d] with the
    same d, Hq a multiple of Hkv, sinks [Hq], cu_seqlens 1-D with at least two entries."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError(f"q and k must be 3-D [tokens, heads, head_dim], got {tuple(q.shape)} and {tuple(k.shape)}")
    T, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if k.shape[2] != d:
        raise ValueError(f"k has head_dim {k.shape[2]}, q has {d}")
    if total_k is None and Tk != T:
        raise ValueError(f"k has {Tk} tokens, q has {T}")
    _shape_of(v, "v", k.shape)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"query heads ({Hq}) must be a multiple of KV heads ({Hkv})")
    _shape_of(sinks, "sinks", (Hq,))
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError(f"cu_seqlens must be 1-D with at least 2 entries, got {tuple(cu_seqlens.shape)}")


def check_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int, max_seqlen: int, what: str = "cu_seqlens"):
    """Debug validation of packed-sequence offsets (copies them to the host, so it synchronises):
    cu[0] = 0, non-decreasing, cu[-1] = total_tokens, every length <= max_seqlen. The kernels trust
    these values; an understated max_seqlen would leave rows unwritten. Raises AttnSinkError."""
    host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    rc = load_library().attn_sink_check_cu_seqlens(host.data_ptr(), int(host.numel()) - 1, int(total_tokens),
                                                   int(max_seqlen))
    if rc != 0:
        raise AttnSinkError(rc, what)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor, cu_seqlens: torch.Tensor,
        max_seqlen: int, causal: bool = True, window: int = 0, softmax_scale: Optional[float] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        out_dtype: torch.dtype = torch.float32, validate_seqlens: bool = False):
    """Forward. q [T,Hq,D], k/v [T,Hkv,D] bf16 (D = 64 or 128); sinks [Hq] fp32; cu_seqlens [B+1] int32 (device).
    Returns (out [T,Hq,D] in ``out_dtype`` (fp32, or bf16 for inference; the backward needs fp32),
    lse [Hq,T] fp32). ``validate_seqlens`` checks cu_seqlens against T and max_seqlen on the host
    first (a synchronising copy; see check_cu_seqlens)."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    _check(sinks, "sinks", torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _check_qkv(q, k, v, sinks, cu_seqlens)
    T, Hq, d = q.shape
    if out is None:
        out = torch.empty((T, Hq, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    _check(out, "out", out_dtype, dev)
    _check(lse, "lse", torch.float32, dev)
    _shape_of(out, "out", (T, Hq, d))
    _shape_of(lse, "lse", (Hq, T))
    if validate_seqlens:
        check_cu_seqlens(cu_seqlens, T, max_seqlen)
    shape = make_shape(q, k, cu_seqlens, max_seqlen, softmax_scale, out_dtype)
    rc = lib.attn_sink_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), int(bool(causal)), int(window), _ptr(cu_seqlens),
                           ctypes.byref(shape), _ptr(out), _ptr(lse), _stream(dev))
    if rc != 0:
        raise AttnSinkError(rc, "attn_sink_fwd")
    return out, lse


def bwd_workspace_bytes(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int) -> int:
    return int(load_library().attn_sink_bwd_workspace_bytes(ctypes.byref(make_shape(q, k, cu_seqlens, max_seqlen, None))))


def bwd_kernel_names() -> Sequence[str]:
    lib = load_library()
    return [lib.attn_sink_bwd_kernel_name(i).decode() for i in range(lib.attn_sink_bwd_num_kernels())]


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = True, window: int = 0,
        softmax_scale: Optional[float] = None, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
        dv: Optional[torch.Tensor] = None, dsinks: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, events: Optional[Sequence[int]] = None,
        validate_seqlens: bool = False):
    """Backward. Returns (dq [T,Hq,D], dk [T,Hkv,D], dv [T,Hkv,D], dsinks [Hq]), all fp32.
    ``events``: optional raw hipEvent_t handles (num kernels + 1) recorded around each kernel; an
    entry may be None (nothing recorded there). ``validate_seqlens``: as in fwd."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(t, n, torch.bfloat16, dev)
    for t, n in ((sinks, "sinks"), (out, "out"), (lse, "lse")):
        _check(t, n, torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _check_qkv(q, k, v, sinks, cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    _shape_of(out, "out", (T, Hq, d))
    _shape_of(dout, "dout", (T, Hq, d))
    _shape_of(lse, "lse", (Hq, T))
    dq = torch.empty((T, Hq, d), dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty((T, Hkv, d), dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty((T, Hkv, d), dtype=torch.float32, device=dev) if dv is None else dv
    dsinks = torch.empty((Hq,), dtype=torch.float32, device=dev) if dsinks is None else dsinks
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dsinks, "dsinks")):
        _check(t, n, torch.float32, dev)
    _shape_of(dq, "dq", (T, Hq, d))
    _shape_of(dk, "dk", (T, Hkv, d))
    _shape_of(dv, "dv", (T, Hkv, d))
    _shape_of(dsinks, "dsinks", (Hq,))
    if validate_seqlens:
        check_cu_seqlens(cu_seqlens, T, max_seqlen)
    shape = make_shape(q, k, cu_seqlens, max_seqlen, softmax_scale)
    need = int(lib.attn_sink_bwd_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", workspace.dtype, dev)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), _ptr(lse), _ptr(dout), int(bool(causal)), int(window),
            _ptr(cu_seqlens), ctypes.byref(shape), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), _stream(dev)]
    if events is None:
        rc = lib.attn_sink_bwd(*args)
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        rc = lib.attn_sink_bwd_timed(*args, arr, len(events))
    if rc != 0:
        raise AttnSinkError(rc, "attn_sink_bwd")
    return dq, dk, dv, dsinks



def bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor, out: torch.Tensor,
                lse: torch.Tensor, dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = True,
                window: int = 0, softmax_scale: Optional[float] = None, *, dq: torch.Tensor, dk: torch.Tensor,
                dv: torch.Tensor, dsinks: torch.Tensor):
    """Backward through attn_sink_bwd_noalloc: same results as ``bwd``, but the library takes its
    workspace from a static per-GPU scratch array (no allocation by the library; the caller passes
    every output). Calls that overlap on one GPU race on that array. Returns (dq, dk, dv, dsinks)."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(t, n, torch.bfloat16, dev)
    for t, n in ((sinks, "sinks"), (out, "out"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv"),
                 (dsinks, "dsinks")):
        _check(t, n, torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _check_qkv(q, k, v, sinks, cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    for t, n, shp in ((out, "out", (T, Hq, d)), (dout, "dout", (T, Hq, d)), (lse, "lse", (Hq, T)),
                      (dq, "dq", (T, Hq, d)), (dk, "dk", (T, Hkv, d)), (dv, "dv", (T, Hkv, d)),
                      (dsinks, "dsinks", (Hq,))):
        _shape_of(t, n, shp)
    shape = make_shape(q, k, cu_seqlens, max_seqlen, softmax_scale)
    rc = lib.attn_sink_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), _ptr(lse), _ptr(dout),
                                   int(bool(causal)), int(window), _ptr(cu_seqlens), ctypes.byref(shape), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(dsinks), _stream(dev))
    if rc != 0:
        raise AttnSinkError(rc, "attn_sink_bwd_noalloc")
    return dq, dk, dv, dsinks


def make_decode_shape(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor, max_q: int, max_k: int,
                      softmax_scale: Optional[float], out_dtype: torch.dtype) -> DecodeShape:
    if out_dtype not in _OUT_DTYPES:
        raise TypeError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    return DecodeShape(int(q.shape[0]), int(k.shape[0]), int(cu_seqlens_q.numel()) - 1, int(max_q), int(max_k),
                       int(q.shape[1]), int(k.shape[1]), int(q.shape[2]),
                       float(softmax_scale) if softmax_scale else 0.0, _OUT_DTYPES[out_dtype])


def decode_kernel_names():
    lib = load_library()
    return [lib.attn_sink_decode_kernel_name(i).decode() for i in range(lib.attn_sink_decode_num_kernels())]


def decode_workspace_bytes(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor, max_q: int,
                           max_k: int) -> int:
    shape = make_decode_shape(q, k, cu_seqlens_q, max_q, max_k, None, torch.float32)
    return int(load_library().attn_sink_decode_workspace_bytes(ctypes.byref(shape)))


def decode_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, max_q: int, max_k: int, window: int = 0,
               softmax_scale: Optional[float] = None, out_dtype: torch.dtype = torch.float32,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, events: Optional[Sequence[int]] = None,
               validate_seqlens: bool = False):
    """Decode forward: q [Tq,Hq,D] (each sequence's last Nq_b tokens), k/v [Tk,Hkv,D] caches, bf16;
    sinks [Hq] fp32; cu_seqlens_q / cu_seqlens_k [B+1] int32 (device). Returns (out [Tq,Hq,64] in
    ``out_dtype``, lse [Hq,Tq] fp32). ``events``: optional raw hipEvent_t handles (num kernels + 1)
    recorded around each kernel; an entry may be None (nothing recorded there).
    ``validate_seqlens``: check both offset arrays on the host first (see check_cu_seqlens)."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    _check(sinks, "sinks", torch.float32, dev)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    _check_qkv(q, k, v, sinks, cu_seqlens_q, total_k=int(k.shape[0]))
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError(f"cu_seqlens_k {tuple(cu_seqlens_k.shape)} and cu_seqlens_q {tuple(cu_seqlens_q.shape)} differ")
    Tq, Hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, Hq, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    _check(out, "out", out_dtype, dev)
    _check(lse, "lse", torch.float32, dev)
    _shape_of(out, "out", (Tq, Hq, d))
    _shape_of(lse, "lse", (Hq, Tq))
    if validate_seqlens:
        check_cu_seqlens(cu_seqlens_q, Tq, max_q, "cu_seqlens_q")
        check_cu_seqlens(cu_seqlens_k, int(k.shape[0]), max_k, "cu_seqlens_k")
    shape = make_decode_shape(q, k, cu_seqlens_q, max_q, max_k, softmax_scale, out_dtype)
    need = int(lib.attn_sink_decode_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", workspace.dtype, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), int(window), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            ctypes.byref(shape), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
            _stream(dev))
    if events is None:
        rc = lib.attn_sink_decode_fwd(*args)
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        rc = lib.attn_sink_decode_fwd_timed(*args, arr, len(events))
    if rc != 0:
        raise AttnSinkError(rc, "attn_sink_decode_fwd")
    return out, lse


def decode_fwd_ordered(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor,
                       cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_q: int, max_k: int,
                       window: int = 0, softmax_scale: Optional[float] = None, out_dtype: torch.dtype = torch.float32,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       validate_seqlens: bool = False):
    """Decode forward through attn_sink_decode_fwd_ordered: the same arguments and outputs as
    ``decode_fwd`` (no workspace), with results equal bit for bit to ``fwd``'s rows for the same
    tokens (causal, same window, scale and out_dtype); slower on long caches."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    _check(sinks, "sinks", torch.float32, dev)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    _check_qkv(q, k, v, sinks, cu_seqlens_q, total_k=int(k.shape[0]))
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError(f"cu_seqlens_k {tuple(cu_seqlens_k.shape)} and cu_seqlens_q {tuple(cu_seqlens_q.shape)} differ")
    Tq, Hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, Hq, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    _check(out, "out", out_dtype, dev)
    _check(lse, "lse", torch.float32, dev)
    _shape_of(out, "out", (Tq, Hq, d))
    _shape_of(lse, "lse", (Hq, Tq))
    if validate_seqlens:
        check_cu_seqlens(cu_seqlens_q, Tq, max_q, "cu_seqlens_q")
        check_cu_seqlens(cu_seqlens_k, int(k.shape[0]), max_k, "cu_seqlens_k")
    shape = make_decode_shape(q, k, cu_seqlens_q, max_q, max_k, softmax_scale, out_dtype)
    rc = lib.attn_sink_decode_fwd_ordered(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), int(window), _ptr(cu_seqlens_q),
                                          _ptr(cu_seqlens_k), ctypes.byref(shape), _ptr(out), _ptr(lse), _stream(dev))
    if rc != 0:
        raise AttnSinkError(rc, "attn_sink_decode_fwd_ordered")
    return out, lse
