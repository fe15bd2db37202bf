"""Python binding of libmxfa.so -- argument marshalling only.

The functions carry the names of the C entry points declared in
``include/mxfa.h``. They check tensor shapes (which the C ABI cannot see),
allocate outputs with torch when none are given, and call the library on
torch's current stream for the tensors' device. Every step of the attention
runs in the HIP kernels of libmxfa.so; there is no other implementation here.
If the library is not built, every call raises ``MxfaError``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "MxfaError",
    "library_path",
    "load_library",
    "mxfa_fwd",
    "mxfa_fwd_varlen",
    "mxfa_fwd_varlen_workspace_bytes",
    "mxfa_fwd_varlen_noalloc",
    "mxfa_decode_splitkv",
    "mxfa_decode_splitkv_paged",
    "mxfa_decode_splitkv_fp8",
    "mxfa_decode_splitkv_gqa",
    "mxfa_decode_splitkv_gqa_workspace_bytes",
    "mxfa_decode_splitkv_gqa_num_splits",
    "mxfa_decode_splitkv_workspace_bytes",
    "mxfa_decode_splitkv_num_splits",
    "mxfa_version",
    "mxfa_clock_probe",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_lib = None

MXFA_OK, MXFA_ERR_INVALID_ARG, MXFA_ERR_UNSUPPORTED, MXFA_ERR_WORKSPACE, MXFA_ERR_HIP = range(5)
MXFA_F32, MXFA_BF16 = 0, 1
_STATUS = {1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}

_c_int, _c_float, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

# C signatures of include/mxfa.h.
_SIGNATURES = {
    "mxfa_fwd": (_c_int, [_vp] * 5 + [_c_int] * 10 + [_c_float, _c_float, _vp]),
    "mxfa_fwd_varlen": (_c_int, [_vp] * 7 + [_c_int] * 12 + [_c_float, _c_float, _vp, _sz, _vp]),
    "mxfa_fwd_varlen_workspace_bytes": (_sz, [_c_int] * 4),
    "mxfa_fwd_varlen_noalloc": (_c_int, [_vp] * 7 + [_c_int] * 12 + [_c_float, _c_float, _vp]),
    "mxfa_decode_splitkv": (_c_int, [_vp] * 6 + [_c_int] * 12 + [_c_float, _c_float, _c_int, _vp, _sz, _vp]),
    "mxfa_decode_splitkv_paged": (_c_int, [_vp] * 7 + [_c_int] * 14 + [_c_float, _c_float, _c_int, _vp, _sz, _vp]),
    "mxfa_decode_splitkv_fp8": (_c_int, [_vp] * 6 + [_c_int] * 12 + [_c_float] * 3 + [_c_int, _vp, _sz, _vp]),
    "mxfa_decode_splitkv_gqa": (_c_int, [_vp] * 7 + [_c_int] * 11 + [_c_float, _c_float, _c_int, _vp, _sz, _vp]),
    "mxfa_decode_splitkv_gqa_workspace_bytes": (_sz, [_c_int] * 7),
    "mxfa_decode_splitkv_gqa_num_splits": (_c_int, [_c_int] * 6),
    "mxfa_decode_splitkv_workspace_bytes": (_sz, [_c_int] * 7),
    "mxfa_decode_splitkv_num_splits": (_c_int, [_c_int] * 6),
    "mxfa_last_error": (ctypes.c_char_p, []),
    "mxfa_version": (ctypes.c_char_p, []),
    "mxfa_clock_probe": (_c_int, [_vp, _c_int, _vp]),
}


class MxfaError(RuntimeError):
    """A non-OK mxfa_status, or the library is missing."""

    def __init__(self, message: str, status: int = -1):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libmxfa.so")


def load_library(path: str | None = None):
    """Load libmxfa.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or library_path()
        if not os.path.exists(p):
            raise MxfaError(f"{p} is not built; run __graft_entry__.build() or "
                            "python -m tiled_attention_amd.build")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(status: int) -> None:
    if status != MXFA_OK:
        msg = load_library().mxfa_last_error().decode(errors="replace")
        raise MxfaError(f"mxfa: {_STATUS.get(status, status)}: {msg}", status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MXFA_BF16
    if t.dtype == torch.float32:
        return MXFA_F32
    raise MxfaError(f"unsupported dtype {t.dtype}", MXFA_ERR_UNSUPPORTED)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise MxfaError(msg, MXFA_ERR_INVALID_ARG)


def _tensors_ok(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        _need(t.is_cuda, "tensors must live on a GPU")
        _need(t.is_contiguous(), "tensors must be contiguous")
        dev = dev or t.device
        _need(t.device == dev, "tensors must share one device")
    return dev


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _scale(scale, head_dim):
    return float(scale) if scale is not None else float(head_dim) ** -0.5


def mxfa_version() -> str:
    return load_library().mxfa_version().decode()


def mxfa_clock_probe(out, interval_us=50):
    """Enqueue the shader-clock probe on the current stream of ``out``'s device.

    ``out`` is an int64 GPU tensor with at least 2 elements; [0] receives the
    shader-clock cycles, [1] the 100 MHz real-time ticks of the interval, so
    ``out[0] / out[1] * 100`` is the clock in MHz once the stream has run it.
    """
    lib = load_library()
    _need(out.dtype == torch.int64 and out.numel() >= 2, "out must be an int64 tensor of >= 2 elements")
    dev = _tensors_ok(out)
    with torch.cuda.device(dev):
        st = lib.mxfa_clock_probe(_ptr(out), int(interval_us), _stream(dev))
    _check(st)


def mxfa_fwd(q, k, v, *, causal=False, window=(-1, -1), softcap=0.0, scale=None, out=None, lse=None,
             return_lse=True):
    """Dense forward: q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d] -> (o [B,Sq,Hq,d], lse [B,Hq,Sq] fp32)."""
    lib = load_library()
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be [B, S, H, d]")
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    _need(k.shape == (b, sk, hkv, d) and v.shape == (b, sk, hkv, d), "k/v shapes do not match q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse is None or (lse.shape == (b, hq, sq) and lse.dtype == torch.float32), "lse must be [B,Hq,Sq] fp32")
    dev = _tensors_ok(q, k, v, out, lse)
    with torch.cuda.device(dev):
        st = lib.mxfa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, sq, sk, hq, hkv, d,
                          _dtype_code(q), int(bool(causal)), int(window[0]), int(window[1]),
                          float(softcap), _scale(scale, d), _stream(dev))
    _check(st)
    return out, lse


def mxfa_fwd_varlen_workspace_bytes(batch, max_seqlen_q, heads_q, head_dim) -> int:
    return int(load_library().mxfa_fwd_varlen_workspace_bytes(batch, max_seqlen_q, heads_q, head_dim))


def mxfa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                    window=(-1, -1), softcap=0.0, scale=None, workspace=None, out=None, lse=None,
                    return_lse=True):
    """Packed forward: q [Tq,Hq,d], k/v [Tk,Hkv,d], int32 cu_seqlens [B+1] on the GPU.

    Returns (o [Tq,Hq,d], lse [Hq,Tq] fp32). ``workspace`` is a uint8 GPU
    tensor of at least mxfa_fwd_varlen_workspace_bytes() bytes for the work
    list (allocated here when None).
    """
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [T, H, d]")
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    _need(k.shape == (tk, hkv, d) and v.shape == (tk, hkv, d), "k/v shapes do not match q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape, "cu_seqlens shapes differ")
    batch = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse is None or (lse.shape == (hq, tq) and lse.dtype == torch.float32), "lse must be [Hq,Tq] fp32")
    dev = _tensors_ok(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, workspace)
    with torch.cuda.device(dev):
        if workspace is None:
            nbytes = mxfa_fwd_varlen_workspace_bytes(batch, int(max_seqlen_q), hq, d)
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        st = lib.mxfa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k), tq, tk, hq,
                                 hkv, d, _dtype_code(q), int(bool(causal)), int(window[0]), int(window[1]),
                                 float(softcap), _scale(scale, d), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return out, lse


def mxfa_fwd_varlen_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                            window=(-1, -1), softcap=0.0, scale=None, out=None, lse=None, return_lse=True):
    """mxfa_fwd_varlen without a workspace: the library keeps the work list in its own static device
    array (for callers that cannot allocate). Pass ``out`` (and ``lse``) to keep the call free of
    allocations; otherwise they are allocated here. Same result as mxfa_fwd_varlen, bit for bit.
    """
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [T, H, d]")
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    _need(k.shape == (tk, hkv, d) and v.shape == (tk, hkv, d), "k/v shapes do not match q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape, "cu_seqlens shapes differ")
    batch = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse is None or (lse.shape == (hq, tq) and lse.dtype == torch.float32), "lse must be [Hq,Tq] fp32")
    dev = _tensors_ok(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k)
    with torch.cuda.device(dev):
        st = lib.mxfa_fwd_varlen_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                         _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k), tq, tk,
                                         hq, hkv, d, _dtype_code(q), int(bool(causal)), int(window[0]),
                                         int(window[1]), float(softcap), _scale(scale, d), _stream(dev))
    _check(st)
    return out, lse


def mxfa_decode_splitkv_num_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits=0) -> int:
    s = load_library().mxfa_decode_splitkv_num_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv,
                                                      num_splits)
    if s <= 0:
        raise MxfaError("mxfa: " + load_library().mxfa_last_error().decode(errors="replace"))
    return s


def mxfa_decode_splitkv_workspace_bytes(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, head_dim_v,
                                        num_splits=0) -> int:
    return int(load_library().mxfa_decode_splitkv_workspace_bytes(batch, max_seqlen_q, max_seqlen_k, heads_q,
                                                                  heads_kv, head_dim_v, num_splits))


def mxfa_decode_splitkv(q, kv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, head_dim_v=512,
                        causal=False, window=(-1, -1), softcap=0.0, scale=None, num_splits=0, workspace=None,
                        out=None, lse=None, return_lse=True):
    """Latent-KV split decode: q [Tq,Hq,576], kv [Tk,Hkv,576] bf16; V = kv[..., :head_dim_v].

    Returns (o [Tq,Hq,head_dim_v] bf16, lse [Hq,Tq] fp32). ``workspace`` is a
    uint8 GPU tensor of at least mxfa_decode_splitkv_workspace_bytes() bytes
    (allocated here when None).
    """
    lib = load_library()
    _need(q.dim() == 3 and kv.dim() == 3, "q and kv must be [T, H, d]")
    tq, hq, dqk = q.shape
    tk, hkv = kv.shape[0], kv.shape[1]
    _need(kv.shape[2] == dqk, "q and kv head dims differ")
    _need(kv.dtype == q.dtype, "q and kv must share a dtype")
    _need(q.dtype == torch.bfloat16, "decode supports bf16")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape, "cu_seqlens shapes differ")
    batch = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty((tq, hq, head_dim_v), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need(out.shape == (tq, hq, head_dim_v) and out.dtype == q.dtype, "out must be [Tq,Hq,head_dim_v]")
    _need(lse is None or (lse.shape == (hq, tq) and lse.dtype == torch.float32), "lse must be [Hq,Tq] fp32")
    dev = _tensors_ok(q, kv, out, lse, cu_seqlens_q, cu_seqlens_k, workspace)
    with torch.cuda.device(dev):
        if workspace is None:
            nbytes = mxfa_decode_splitkv_workspace_bytes(batch, int(max_seqlen_q), int(max_seqlen_k), hq, hkv,
                                                         head_dim_v, num_splits)
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        st = lib.mxfa_decode_splitkv(_ptr(q), _ptr(kv), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                     _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k), tq, tk,
                                     hq, hkv, dqk, int(head_dim_v), int(bool(causal)), int(window[0]),
                                     int(window[1]), float(softcap), _scale(scale, dqk), int(num_splits),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(dev))
    _check(st)
    return out, lse


def mxfa_decode_splitkv_paged(q, kv_cache, cu_seqlens_q, cache_seqlens, block_table, max_seqlen_q, max_seqlen_k, *,
                              head_dim_v=512, causal=False, window=(-1, -1), softcap=0.0, scale=None,
                              num_splits=0, workspace=None, out=None, lse=None, return_lse=True):
    """Latent-KV split decode over a paged cache.

    q [Tq,Hq,576] bf16; kv_cache [num_pages, page_size, Hkv, 576] bf16;
    cache_seqlens int32 [B]; block_table int32 [B, max_pages]: sequence b's key
    j is row j % page_size of page block_table[b, j // page_size]. V is
    kv[..., :head_dim_v]. Returns (o [Tq,Hq,head_dim_v] bf16, lse [Hq,Tq] fp32).
    """
    lib = load_library()
    _need(q.dim() == 3 and kv_cache.dim() == 4, "q must be [T, H, d] and kv_cache [pages, page_size, H, d]")
    tq, hq, dqk = q.shape
    num_pages, page_size, hkv = kv_cache.shape[0], kv_cache.shape[1], kv_cache.shape[2]
    _need(kv_cache.shape[3] == dqk, "q and kv_cache head dims differ")
    _need(kv_cache.dtype == q.dtype, "q and kv_cache must share a dtype")
    _need(q.dtype == torch.bfloat16, "decode supports bf16")
    _need(cu_seqlens_q.dtype == torch.int32 and cache_seqlens.dtype == torch.int32 and
          block_table.dtype == torch.int32, "cu_seqlens_q, cache_seqlens and block_table must be int32")
    _need(cu_seqlens_q.dim() == 1 and cache_seqlens.dim() == 1 and block_table.dim() == 2,
          "cu_seqlens_q [B+1], cache_seqlens [B], block_table [B, max_pages]")
    batch = cu_seqlens_q.shape[0] - 1
    _need(cache_seqlens.shape[0] == batch and block_table.shape[0] == batch, "batch sizes differ")
    if out is None:
        out = torch.empty((tq, hq, head_dim_v), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need(out.shape == (tq, hq, head_dim_v) and out.dtype == q.dtype, "out must be [Tq,Hq,head_dim_v]")
    _need(lse is None or (lse.shape == (hq, tq) and lse.dtype == torch.float32), "lse must be [Hq,Tq] fp32")
    dev = _tensors_ok(q, kv_cache, out, lse, cu_seqlens_q, cache_seqlens, block_table, workspace)
    max_pages = block_table.shape[1]
    if block_table.numel() == 0:  # the C call wants a non-null table even when it holds no pages
        block_table = torch.zeros(1, dtype=torch.int32, device=q.device)
    with torch.cuda.device(dev):
        if workspace is None:
            nbytes = mxfa_decode_splitkv_workspace_bytes(batch, int(max_seqlen_q), int(max_seqlen_k), hq, hkv,
                                                         head_dim_v, num_splits)
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        st = lib.mxfa_decode_splitkv_paged(_ptr(q), _ptr(kv_cache), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                           _ptr(cache_seqlens), _ptr(block_table), batch, int(max_seqlen_q),
                                           int(max_seqlen_k), tq, num_pages, page_size, max_pages,
                                           hq, hkv, dqk, int(head_dim_v), int(bool(causal)), int(window[0]),
                                           int(window[1]), float(softcap), _scale(scale, dqk), int(num_splits),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(dev))
    _check(st)
    return out, lse


def mxfa_decode_splitkv_gqa_num_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits=0) -> int:
    s = load_library().mxfa_decode_splitkv_gqa_num_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv,
                                                          num_splits)
    if s <= 0:
        raise MxfaError("mxfa: " + load_library().mxfa_last_error().decode(errors="replace"))
    return s


def mxfa_decode_splitkv_gqa_workspace_bytes(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, head_dim,
                                            num_splits=0) -> int:
    return int(load_library().mxfa_decode_splitkv_gqa_workspace_bytes(batch, max_seqlen_q, max_seqlen_k, heads_q,
                                                                      heads_kv, head_dim, num_splits))


def mxfa_decode_splitkv_gqa(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                            window=(-1, -1), softcap=0.0, scale=None, num_splits=0, workspace=None, out=None,
                            lse=None, return_lse=True):
    """Standard-head split decode: q [Tq,Hq,d], k/v [Tk,Hkv,d] bf16 (d = 64 or 128), int32 cu_seqlens.

    Returns (o [Tq,Hq,d] bf16, lse [Hq,Tq] fp32). ``workspace`` is a uint8 GPU
    tensor of at least mxfa_decode_splitkv_gqa_workspace_bytes() bytes
    (allocated here when None and needed).
    """
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [T, H, d]")
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    _need(k.shape == (tk, hkv, d) and v.shape == (tk, hkv, d), "k/v shapes do not match q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _need(q.dtype == torch.bfloat16, "decode supports bf16")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape, "cu_seqlens shapes differ")
    batch = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse is None or (lse.shape == (hq, tq) and lse.dtype == torch.float32), "lse must be [Hq,Tq] fp32")
    dev = _tensors_ok(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, workspace)
    with torch.cuda.device(dev):
        if workspace is None:
            nbytes = mxfa_decode_splitkv_gqa_workspace_bytes(batch, int(max_seqlen_q), int(max_seqlen_k), hq, hkv,
                                                             d, num_splits)
            if nbytes > 0:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = lib.mxfa_decode_splitkv_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                         _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k), tq, tk,
                                         hq, hkv, d, int(bool(causal)), int(window[0]), int(window[1]),
                                         float(softcap), _scale(scale, d), int(num_splits), _ptr(workspace),
                                         ws_bytes, _stream(dev))
    _check(st)
    return out, lse


def mxfa_decode_splitkv_fp8(q, kv8, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, kv_scale, *,
                            head_dim_v=512, causal=False, window=(-1, -1), softcap=0.0, scale=None, num_splits=0,
                            workspace=None, out=None, lse=None, return_lse=True):
    """Latent-KV split decode over an fp8 cache: q [Tq,Hq,576] bf16; kv8 [Tk,Hkv,576] OCP e4m3 codes
    (uint8 or torch.float8_e4m3fn); key rows are kv_scale * kv8, values their first head_dim_v channels.

    Returns (o [Tq,Hq,head_dim_v] bf16, lse [Hq,Tq] fp32); workspace as for mxfa_decode_splitkv.
    """
    lib = load_library()
    _need(q.dim() == 3 and kv8.dim() == 3, "q and kv8 must be [T, H, d]")
    _need(kv8.dtype in (torch.uint8, torch.float8_e4m3fn), "kv8 must hold e4m3 codes (uint8 or float8_e4m3fn)")
    tq, hq, dqk = q.shape
    tk, hkv = kv8.shape[0], kv8.shape[1]
    _need(kv8.shape[2] == dqk, "q and kv8 head dims differ")
    _need(q.dtype == torch.bfloat16, "q must be bf16")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape, "cu_seqlens shapes differ")
    batch = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty((tq, hq, head_dim_v), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need(out.shape == (tq, hq, head_dim_v) and out.dtype == q.dtype, "out must be [Tq,Hq,head_dim_v]")
    _need(lse is None or (lse.shape == (hq, tq) and lse.dtype == torch.float32), "lse must be [Hq,Tq] fp32")
    dev = _tensors_ok(q, kv8, out, lse, cu_seqlens_q, cu_seqlens_k, workspace)
    with torch.cuda.device(dev):
        if workspace is None:
            nbytes = mxfa_decode_splitkv_workspace_bytes(batch, int(max_seqlen_q), int(max_seqlen_k), hq, hkv,
                                                         head_dim_v, num_splits)
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        st = lib.mxfa_decode_splitkv_fp8(_ptr(q), _ptr(kv8), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                         _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k), tq, tk,
                                         hq, hkv, dqk, int(head_dim_v), int(bool(causal)), int(window[0]),
                                         int(window[1]), float(softcap), _scale(scale, dqk), float(kv_scale),
                                         int(num_splits), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return out, lse
