"""ctypes binding of liblinattn.so (include/linattn.h), taking torch tensors.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  If the library has not been built
this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_DTYPE_F32 = 0
LA_DTYPE_BF16 = 1
LA_OK = 0

# every symbol declared in include/linattn.h
EXPORTS = ("la_abi_version", "la_status_string", "la_noncausal_workspace_bytes",
           "la_forward_noncausal", "la_causal_workspace_bytes", "la_forward_causal",
           "la_causal_plan", "la_state_sums_workspace_bytes", "la_state_sums",
           "la_causal_segments", "la_decode_step", "la_forward_causal_state",
           "la_noncausal_varlen_workspace_bytes", "la_forward_noncausal_varlen",
           "la_causal_varlen_workspace_bytes", "la_forward_causal_varlen", "la_decode_step_masked",
           "la_favor_noncausal_workspace_bytes", "la_favor_forward_noncausal", "la_favor_decode_step",
           "la_favor_causal_workspace_bytes", "la_favor_forward_causal", "la_forward_noncausal_noalloc",
           # include/la_ceiling.h
           "la_ceiling_copy", "la_ceiling_read_sink_words", "la_ceiling_read", "la_ceiling_causal_pattern")

LA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/linattn.h

_lib = None
_lock = threading.Lock()


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, la_status_string(status), status))


def load():
    """Load liblinattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liblinattn.so is not built (run `python -m efficient_attention_amd.build` "
                               "or __graft_entry__.build()); there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        lib.la_abi_version.argtypes = []
        lib.la_abi_version.restype = I
        lib.la_status_string.argtypes = [I]
        lib.la_status_string.restype = ctypes.c_char_p
        lib.la_noncausal_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
        lib.la_noncausal_workspace_bytes.restype = SZ
        lib.la_forward_noncausal.argtypes = [P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]
        lib.la_forward_noncausal.restype = I
        lib.la_forward_noncausal_noalloc.argtypes = [P, P, P, P, I64, I64, I64, I64, I, P]
        lib.la_forward_noncausal_noalloc.restype = I
        lib.la_causal_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
        lib.la_causal_workspace_bytes.restype = SZ
        lib.la_forward_causal.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, P, SZ, P]
        lib.la_forward_causal.restype = I
        lib.la_forward_causal_state.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, P, SZ, P]
        lib.la_forward_causal_state.restype = I
        lib.la_causal_plan.argtypes = [I64, I64, I64, I64, I64, I, ctypes.POINTER(I64)]
        lib.la_causal_plan.restype = I
        lib.la_state_sums_workspace_bytes.argtypes = [I64, I64, I64, I64, I, I64, I64]
        lib.la_state_sums_workspace_bytes.restype = SZ
        lib.la_state_sums.argtypes = [P, P, P, I64, I64, I64, I64, I, I64, I64, P, SZ, P]
        lib.la_state_sums.restype = I
        lib.la_causal_segments.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I, I64, P]
        lib.la_causal_segments.restype = I
        lib.la_decode_step.argtypes = [P, P, P, P, P, P, I64, I64, I64, I, P]
        lib.la_decode_step.restype = I
        lib.la_decode_step_masked.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I, P]
        lib.la_decode_step_masked.restype = I
        lib.la_noncausal_varlen_workspace_bytes.argtypes = [P, I64, I64, I64, I]
        lib.la_noncausal_varlen_workspace_bytes.restype = SZ
        lib.la_forward_noncausal_varlen.argtypes = [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]
        lib.la_forward_noncausal_varlen.restype = I
        lib.la_causal_varlen_workspace_bytes.argtypes = [P, I64, I64, I64, I64, I]
        lib.la_causal_varlen_workspace_bytes.restype = SZ
        lib.la_forward_causal_varlen.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]
        lib.la_forward_causal_varlen.restype = I
        F = ctypes.c_float
        lib.la_favor_noncausal_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
        lib.la_favor_noncausal_workspace_bytes.restype = SZ
        lib.la_favor_forward_noncausal.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, F, I, P, SZ, P]
        lib.la_favor_forward_noncausal.restype = I
        lib.la_favor_decode_step.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, F, I, P]
        lib.la_favor_decode_step.restype = I
        lib.la_favor_causal_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I64, I]
        lib.la_favor_causal_workspace_bytes.restype = SZ
        lib.la_favor_forward_causal.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, F, I,
                                                P, SZ, P]
        lib.la_favor_forward_causal.restype = I
        lib.la_ceiling_copy.argtypes = [P, P, SZ, P]
        lib.la_ceiling_copy.restype = I
        lib.la_ceiling_read_sink_words.argtypes = []
        lib.la_ceiling_read_sink_words.restype = SZ
        lib.la_ceiling_read.argtypes = [P, SZ, P, P]
        lib.la_ceiling_read.restype = I
        lib.la_ceiling_causal_pattern.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P]
        lib.la_ceiling_causal_pattern.restype = I
        _lib = lib
    return _lib


def la_abi_version() -> int:
    return load().la_abi_version()


def la_status_string(status: int) -> str:
    return load().la_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return LA_DTYPE_BF16
    raise TypeError("linear attention supports float32 and bfloat16 tensors, got %s" % t.dtype)


def la_noncausal_workspace_bytes(B: int, H: int, n: int, d: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_noncausal_workspace_bytes(B, H, n, d, code))


def la_causal_workspace_bytes(B: int, H: int, n: int, d: int, chunk: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_causal_workspace_bytes(B, H, n, d, chunk, code))


# One reusable workspace per (device, stream) for calls that are not given one: calls queued on
# one stream never use it concurrently, and each call initialises the part it uses.  It grows to
# the largest size asked for; release_workspaces() drops them (torch's caching allocator keeps the
# memory for reuse until torch.cuda.empty_cache()).
_ws_cache: dict = {}


def workspace(nbytes: int, device: torch.device, stream_handle: int) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    key = (device.index, stream_handle)
    with _lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            _ws_cache[key] = buf
    return buf


def release_workspaces(device=None) -> int:
    """Drop the cached workspaces (of one device, or all); returns how many bytes they held.
    Call it when no queued call can still use them (e.g. after a synchronisation), or pass the
    workspaces explicitly (ws=) to keep their lifetime in the caller's hands."""
    idx = None if device is None else torch.device(device).index
    freed = 0
    with _lock:
        for key in [k for k in _ws_cache if idx is None or k[0] == idx]:
            freed += _ws_cache.pop(key).numel()
    return freed


def _on_stream(fn):
    """Run an entry point with `stream` (a torch stream or a raw hipStream_t handle) as the
    current stream, so that the tensors it allocates (out, workspace, states) come from that
    stream's pool and are not handed to other work while its kernels still use them."""
    names = list(inspect.signature(fn).parameters)
    pos = names.index("stream")
    assert pos == len(names) - 1, "stream must be the last parameter"

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        if len(args) > pos:  # given positionally
            kwargs["stream"] = args[pos]
            args = args[:pos]
        stream = kwargs.pop("stream", None)
        if stream is None:
            return fn(*args, **kwargs)
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(s):
            return fn(*args, stream=s, **kwargs)
    return wrapper


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_qkv(q, k, v, ndim):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dim() != ndim:
            raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ: %s %s %s" % (q.shape, k.shape, v.shape))
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v dtypes differ")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")


def _out_like(q, out):
    if out is None:
        return torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor with the shape, dtype and device of q")
    return out


@_on_stream
def la_forward_noncausal(q, k, v, out=None, ws=None, stream=None):
    """Non-causal forward over [B, H, n, d] tensors; returns out."""
    _check_qkv(q, k, v, 4)
    out = _out_like(q, out)
    B, H, n, d = q.shape
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_noncausal_workspace_bytes(B, H, n, d, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    st = load().la_forward_noncausal(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     B, H, n, d, code, ws.data_ptr() if ws is not None else None,
                                     ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_forward_noncausal")
    return out


@_on_stream
def la_forward_noncausal_noalloc(q, k, v, out=None, stream=None):
    """la_forward_noncausal with the library's own per-GPU scratch instead of a workspace (the C
    entry point allocates nothing; pass `out` to allocate nothing here either); returns out."""
    _check_qkv(q, k, v, 4)
    out = _out_like(q, out)
    B, H, n, d = q.shape
    st = load().la_forward_noncausal_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                             B, H, n, d, _dtype_code(q), _stream_handle(q.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_forward_noncausal_noalloc")
    return out


@_on_stream
def la_forward_causal(q, k, v, chunk: int = 128, out=None, ws=None, stream=None):
    """Causal (j <= i) forward over [B, H, n, d] tensors; returns out."""
    _check_qkv(q, k, v, 4)
    out = _out_like(q, out)
    B, H, n, d = q.shape
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_causal_workspace_bytes(B, H, n, d, chunk, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    st = load().la_forward_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  B, H, n, d, chunk, code,
                                  ws.data_ptr() if ws is not None else None,
                                  ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_forward_causal")
    return out


@_on_stream
def la_forward_causal_state(q, k, v, chunk: int = 128, S0=None, z0=None, out=None, Sn=None, zn=None,
                            final_state: bool = True, ws=None, stream=None):
    """Causal forward continuing from the state (S0 [B, H, d, d], z0 [B, H, d], fp32; None for
    the zero state).  Returns (out, Sn, zn) with the state after the last token (allocated
    unless given), or (out, None, None) when final_state is False."""
    _check_qkv(q, k, v, 4)
    B, H, n, d = q.shape
    if (S0 is None) != (z0 is None):
        raise ValueError("give both S0 and z0, or neither")
    if final_state:
        if Sn is None:
            Sn = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
        if zn is None:
            zn = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    else:
        Sn = zn = None
    for name, t, shape in (("S0", S0, (B, H, d, d)), ("z0", z0, (B, H, d)),
                           ("Sn", Sn, (B, H, d, d)), ("zn", zn, (B, H, d))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape
                              or not t.is_contiguous() or t.device != q.device):
            raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s" % (name, shape, q.device))
    out = _out_like(q, out)
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_causal_workspace_bytes(B, H, n, d, chunk, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = load().la_forward_causal_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        ptr(S0), ptr(z0), ptr(Sn), ptr(zn), B, H, n, d, chunk, code,
                                        ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_forward_causal_state")
    return out, Sn, zn


@_on_stream
def la_decode_step(q, k, v, S, z, out=None, stream=None):
    """One decode step over [B, H, d] tensors; S [B, H, d, d] and z [B, H, d] (fp32) are
    updated in place; returns out."""
    _check_qkv(q, k, v, 3)
    B, H, d = q.shape
    for name, t, shape in (("S", S, (B, H, d, d)), ("z", z, (B, H, d))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s" % (name, shape, q.device))
    out = _out_like(q, out)
    sh = _stream_handle(q.device, stream)
    st = load().la_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), S.data_ptr(), z.data_ptr(),
                               out.data_ptr(), B, H, d, _dtype_code(q), sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_decode_step")
    return out


def la_causal_plan(B: int, H: int, n: int, d: int, chunk: int, dtype) -> int:
    """Segment length la_forward_causal uses for this shape."""
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    out = ctypes.c_int64(0)
    st = load().la_causal_plan(B, H, n, d, chunk, code, ctypes.byref(out))
    if st != LA_OK:
        raise LinAttnError(st, "la_causal_plan")
    return int(out.value)


def la_state_sums_workspace_bytes(B: int, H: int, n: int, d: int, dtype, seg_len: int, nseg: int) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_state_sums_workspace_bytes(B, H, n, d, code, seg_len, nseg))


@_on_stream
def la_state_sums(k, v, seg_len: int, nseg: int, sums=None, ws=None, stream=None):
    """Per-segment [S | z] sums of [B, H, n, d] keys/values: returns fp32 [B, H, nseg, d*d + d]."""
    _check_qkv(k, k, v, 4)
    B, H, n, d = k.shape
    code = _dtype_code(k)
    if sums is None:
        sums = torch.empty((B, H, nseg, d * d + d), dtype=torch.float32, device=k.device)
    elif sums.dtype != torch.float32 or tuple(sums.shape) != (B, H, nseg, d * d + d) or not sums.is_contiguous():
        raise ValueError("sums must be a contiguous float32 tensor of shape %s" % ((B, H, nseg, d * d + d),))
    sh = _stream_handle(k.device, stream)
    need = la_state_sums_workspace_bytes(B, H, n, d, code, seg_len, nseg)
    if ws is None:
        ws = workspace(need, k.device, sh)
    st = load().la_state_sums(k.data_ptr(), v.data_ptr(), sums.data_ptr(), B, H, n, d, code, seg_len, nseg,
                              ws.data_ptr() if ws is not None else None,
                              ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_state_sums")
    return sums


def _check_segment_sums(sums, B, H, n, d, seg_len, device):
    """The sums la_causal_segments reads: [B, H, ceil(n / seg_len) - 1, d*d + d] fp32 on `device`
    (the leading segments' [S | z]), or None when each head is one segment."""
    if seg_len <= 0:
        raise ValueError("seg_len must be positive")
    lead = -(-n // seg_len) - 1 if n > 0 else 0
    if lead <= 0:
        if sums is not None:
            raise ValueError("one segment per head takes no sums (sums must be None)")
        return
    shape = (B, H, lead, d * d + d)
    if sums is None or sums.dtype != torch.float32 or tuple(sums.shape) != shape \
            or not sums.is_contiguous() or sums.device != device:
        raise ValueError("sums must be a contiguous float32 tensor of shape %s on %s (the "
                         "ceil(n / seg_len) - 1 leading segments' sums)" % (shape, device))


@_on_stream
def la_causal_segments(q, k, v, sums, seg_len: int, chunk: int = 128, out=None, stream=None):
    """Chunked causal pass where segment s starts from the sum of sums[:, :, :s]."""
    _check_qkv(q, k, v, 4)
    out = _out_like(q, out)
    B, H, n, d = q.shape
    _check_segment_sums(sums, B, H, n, d, seg_len, q.device)
    sh = _stream_handle(q.device, stream)
    st = load().la_causal_segments(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   sums.data_ptr() if sums is not None else None,
                                   B, H, n, d, chunk, _dtype_code(q), seg_len, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_causal_segments")
    return out


# ----------------------------------------------------------------------------- variable lengths
def _offsets(cu_seqlens):
    """Host int64 array of sequence offsets (list, numpy array or CPU tensor)."""
    if isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be a 1-D array of nseq + 1 offsets")
    return cu


def _check_varlen(q, k, v, cu, heads):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have the same shape and dtype")
    d = q.shape[-1]
    if q.numel() != int(heads) * int(cu[-1]) * d:
        raise ValueError("q holds %d elements, the offsets call for H * cu[-1] * d = %d"
                         % (q.numel(), int(heads) * int(cu[-1]) * d))
    return d


def la_noncausal_varlen_workspace_bytes(cu_seqlens, heads: int, d: int, dtype) -> int:
    cu = _offsets(cu_seqlens)
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_noncausal_varlen_workspace_bytes(cu.ctypes.data, cu.size - 1, heads, d, code))


def la_causal_varlen_workspace_bytes(cu_seqlens, heads: int, d: int, chunk: int, dtype) -> int:
    cu = _offsets(cu_seqlens)
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_causal_varlen_workspace_bytes(cu.ctypes.data, cu.size - 1, heads, d, chunk, code))


@_on_stream
def la_forward_noncausal_varlen(q, k, v, cu_seqlens, heads: int, out=None, ws=None, stream=None):
    """Non-causal forward over a variable-length batch: sequence s is the [heads, n_s, d] block
    at token offset cu_seqlens[s] (q, k, v hold heads * cu_seqlens[-1] rows of d); returns out."""
    cu = _offsets(cu_seqlens)
    d = _check_varlen(q, k, v, cu, heads)
    out = _out_like(q, out)
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_noncausal_varlen_workspace_bytes(cu, heads, d, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    st = load().la_forward_noncausal_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            cu.ctypes.data, cu.size - 1, heads, d, code,
                                            ws.data_ptr() if ws is not None else None,
                                            ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_forward_noncausal_varlen")
    return out


@_on_stream
def la_forward_causal_varlen(q, k, v, cu_seqlens, heads: int, chunk: int = 128, out=None, ws=None, stream=None):
    """Causal forward over a variable-length batch (layout as la_forward_noncausal_varlen)."""
    cu = _offsets(cu_seqlens)
    d = _check_varlen(q, k, v, cu, heads)
    out = _out_like(q, out)
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_causal_varlen_workspace_bytes(cu, heads, d, chunk, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    st = load().la_forward_causal_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         cu.ctypes.data, cu.size - 1, heads, d, chunk, code,
                                         ws.data_ptr() if ws is not None else None,
                                         ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_forward_causal_varlen")
    return out


@_on_stream
def la_decode_step_masked(q, k, v, S, z, active, out=None, stream=None):
    """la_decode_step for the sequences whose flag in `active` (uint8/bool GPU tensor [B]) is set;
    the others keep their state and out."""
    _check_qkv(q, k, v, 3)
    B, H, d = q.shape
    for name, t, shape in (("S", S, (B, H, d, d)), ("z", z, (B, H, d))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s" % (name, shape, q.device))
    if active.dtype not in (torch.uint8, torch.bool) or tuple(active.shape) != (B,) or active.device != q.device \
            or not active.is_contiguous():
        raise ValueError("active must be a contiguous uint8/bool tensor of shape (%d,) on %s" % (B, q.device))
    out = _out_like(q, out)
    sh = _stream_handle(q.device, stream)
    st = load().la_decode_step_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), S.data_ptr(), z.data_ptr(),
                                      out.data_ptr(), active.data_ptr(), B, H, d, _dtype_code(q), sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_decode_step_masked")
    return out


# ---------------------------------------------------------------- FAVOR+ feature map
def _check_proj(w, q):
    if not isinstance(w, torch.Tensor) or w.dim() != 2 or w.shape[1] != q.shape[-1]:
        raise ValueError("w must be a [m, d] tensor with d = %d" % q.shape[-1])
    if w.dtype != q.dtype or w.device != q.device or not w.is_contiguous():
        raise ValueError("w must be contiguous, with the dtype and device of q")
    return int(w.shape[0])


def la_favor_noncausal_workspace_bytes(B: int, H: int, n: int, d: int, m: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_favor_noncausal_workspace_bytes(B, H, n, d, m, code))


@_on_stream
def la_favor_forward_noncausal(q, k, v, w, scale: float, out=None, ws=None, stream=None):
    """Non-causal attention with FAVOR+ features phi(x) = exp(W x' - |x'|^2/2)/sqrt(m), x' =
    scale x, over [B, H, n, d] tensors and the projection w [m, d]; returns out."""
    _check_qkv(q, k, v, 4)
    m = _check_proj(w, q)
    out = _out_like(q, out)
    B, H, n, d = q.shape
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_favor_noncausal_workspace_bytes(B, H, n, d, m, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    st = load().la_favor_forward_noncausal(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), out.data_ptr(), B, H, n, d, m,
        float(scale), code, ws.data_ptr() if ws is not None else None,
        ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_favor_forward_noncausal")
    return out


@_on_stream
def la_favor_decode_step(q, k, v, w, S, z, c, scale: float, out=None, stream=None):
    """One FAVOR+ decode step over [B, H, d] tensors; the state (S [B, H, m, d], z [B, H, m],
    c [B, H], fp32; true state exp(c) (S, z)) is updated in place; returns out."""
    _check_qkv(q, k, v, 3)
    m = _check_proj(w, q)
    B, H, d = q.shape
    for name, t, shape in (("S", S, (B, H, m, d)), ("z", z, (B, H, m)), ("c", c, (B, H))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s" % (name, shape, q.device))
    out = _out_like(q, out)
    sh = _stream_handle(q.device, stream)
    st = load().la_favor_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(),
                                     S.data_ptr(), z.data_ptr(), c.data_ptr(), out.data_ptr(),
                                     B, H, d, m, float(scale), _dtype_code(q), sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_favor_decode_step")
    return out


def la_favor_causal_workspace_bytes(B: int, H: int, n: int, d: int, m: int, chunk: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().la_favor_causal_workspace_bytes(B, H, n, d, m, chunk, code))


@_on_stream
def la_favor_forward_causal(q, k, v, w, scale: float, chunk: int = 64, out=None, final_state: bool = False,
                            Sn=None, zn=None, cn=None, ws=None, stream=None):
    """Causal attention with FAVOR+ features over [B, H, n, d] tensors.  Returns out, or with
    final_state (out, Sn, zn, cn): the state after the last token as exp(cn) (Sn, zn)."""
    _check_qkv(q, k, v, 4)
    m = _check_proj(w, q)
    B, H, n, d = q.shape
    if final_state:
        if Sn is None:
            Sn = torch.empty((B, H, m, d), dtype=torch.float32, device=q.device)
        if zn is None:
            zn = torch.empty((B, H, m), dtype=torch.float32, device=q.device)
        if cn is None:
            cn = torch.empty((B, H), dtype=torch.float32, device=q.device)
        for name, t, shape in (("Sn", Sn, (B, H, m, d)), ("zn", zn, (B, H, m)), ("cn", cn, (B, H))):
            if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() \
                    or t.device != q.device:
                raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s" % (name, shape, q.device))
    else:
        Sn = zn = cn = None
    out = _out_like(q, out)
    code = _dtype_code(q)
    sh = _stream_handle(q.device, stream)
    need = la_favor_causal_workspace_bytes(B, H, n, d, m, chunk, code)
    if ws is None:
        ws = workspace(need, q.device, sh)
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = load().la_favor_forward_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), out.data_ptr(),
                                        ptr(Sn), ptr(zn), ptr(cn), B, H, n, d, m, chunk, float(scale), code,
                                        ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, sh)
    if st != LA_OK:
        raise LinAttnError(st, "la_favor_forward_causal")
    if final_state:
        return out, Sn, zn, cn
    return out


# ---------------------------------------------------------------- memory-system ceilings (include/la_ceiling.h)
def _check_bytes_tensor(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError("%s must be a contiguous GPU tensor" % name)
    return t.numel() * t.element_size()


@_on_stream
def la_ceiling_copy(src, dst, stream=None):
    """dst = src (same number of bytes, a multiple of 16) by the plain-copy measurement kernel."""
    nb = _check_bytes_tensor(src, "src")
    if _check_bytes_tensor(dst, "dst") != nb:
        raise ValueError("src and dst must hold the same number of bytes")
    st = load().la_ceiling_copy(src.data_ptr(), dst.data_ptr(), nb, _stream_handle(src.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_ceiling_copy")
    return dst


@_on_stream
def la_ceiling_read(src, sink=None, stream=None):
    """Reads every byte of src once; returns the per-workgroup XOR words (uint32 as int32)."""
    nb = _check_bytes_tensor(src, "src")
    words = int(load().la_ceiling_read_sink_words())
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=src.device)
    elif sink.dtype != torch.int32 or sink.numel() < words or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 tensor of at least %d words" % words)
    st = load().la_ceiling_read(src.data_ptr(), nb, sink.data_ptr(), _stream_handle(src.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_ceiling_read")
    return sink


@_on_stream
def la_ceiling_causal_pattern(q, k, v, seg_len: int, out=None, stream=None):
    """out = q + k + v ([B, H, n, 128] bf16) with the chunked causal kernel's memory pattern."""
    _check_qkv(q, k, v, 4)
    out = _out_like(q, out)
    B, H, n, d = q.shape
    if q.dtype != torch.bfloat16:
        raise ValueError("the causal pattern measurement takes bf16 tensors")
    st = load().la_ceiling_causal_pattern(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, n, d,
                                          seg_len, _stream_handle(q.device, stream))
    if st != LA_OK:
        raise LinAttnError(st, "la_ceiling_causal_pattern")
    return out
