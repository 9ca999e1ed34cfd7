"""Thin Python binding of libfa.so (exact attention forward on MI355X).

Argument marshalling only: the functions below check dtypes, shapes,
contiguity and device, allocate outputs with torch, and pass raw device
pointers and torch's current HIP stream to the C ABI (include/fa.h).  Every
step of the computation runs in the library's HIP kernels; there is no CPU
or PyTorch fallback.  If libfa.so is missing, every call raises.

The names match the C entry points (fa_fwd, fa_fwd_ex, fa_decode_splitk,
fa_decode_splitk_mq, fa_bwd, their workspace-size and fa_check_* companions,
fa_status_str, fa_abi_version).
"""

import ctypes
import math
import os
import pathlib

# torch must own the process's HIP runtime before libfa.so is loaded, so that
# the library binds to the very same runtime (both carry the soname
# libamdhip64.so.7) and pointers and streams mean the same thing on both sides.
import torch

__all__ = [
    "FA_F32", "FA_BF16", "FaError", "lib", "lib_path",
    "FA_ALIGN_BOTTOM_RIGHT", "FA_ALIGN_TOP_LEFT",
    "fa_fwd", "fa_fwd_ex", "fa_decode_splitk", "fa_decode_splitk_workspace_bytes",
    "fa_check_fwd", "fa_check_fwd_ex", "fa_check_decode", "fa_bwd_ex", "fa_check_bwd_ex", "keep_256_for", "fa_bwd", "fa_bwd_workspace_bytes", "fa_check_bwd",
    "fa_decode_splitk_mq", "fa_decode_splitk_mq_workspace_bytes", "fa_check_decode_mq",
    "fa_decode_splitk_static", "FA_STATIC_SCRATCH_BYTES",
    "fa_status_str", "fa_abi_version",
]

FA_F32 = 0
FA_BF16 = 1
FA_ALIGN_BOTTOM_RIGHT = 0
FA_ALIGN_TOP_LEFT = 1
FA_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024  # include/fa.h
_ALIGN = {"bottom_right": FA_ALIGN_BOTTOM_RIGHT, "top_left": FA_ALIGN_TOP_LEFT}
_STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
           4: "FA_ERR_WORKSPACE", 5: "FA_ERR_HIP"}

_LIB_PATH = pathlib.Path(__file__).resolve().with_name("libfa.so")
_lib = None

_vp, _fp, _ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_i, _f, _sz, _u64 = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64

_SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _fp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_check_fwd": (_i, [_vp, _vp, _vp, _fp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i]),
    "fa_fwd_ex": (_i, [_vp, _vp, _vp, _fp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _i, _i,
                       _u64, _i, _vp]),
    "fa_check_fwd_ex": (_i, [_vp, _vp, _vp, _fp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _i,
                             _i, _u64, _i]),
    "fa_bwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _fp, _ip, _vp, _vp, _vp,
                       _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _i, _i, _u64, _vp, _sz, _vp]),
    "fa_check_bwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _fp, _ip, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _i, _i, _u64, _vp, _sz]),
    "fa_decode_splitk_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "fa_decode_splitk": (_i, [_vp, _vp, _vp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_check_decode": (_i, [_vp, _vp, _vp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz]),
    "fa_decode_splitk_static": (_i, [_vp, _vp, _vp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_decode_splitk_mq_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "fa_decode_splitk_mq": (_i, [_vp, _vp, _vp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz,
                                 _vp]),
    "fa_check_decode_mq": (_i, [_vp, _vp, _vp, _ip, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz]),
    "fa_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _fp, _ip, _vp, _vp, _vp,
                    _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "fa_check_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _fp, _ip, _vp, _vp, _vp,
                          _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz]),
    "fa_status_str": (ctypes.c_char_p, [_i]),
    "fa_abi_version": (_i, []),
}


class FaError(RuntimeError):
    """A nonzero fa_status from the library, or a binding-level misuse."""

    def __init__(self, status, msg=None):
        self.status = status
        super().__init__(msg or f"{_STATUS.get(status, status)}: {fa_status_str(status)}")


def lib_path():
    return _LIB_PATH


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def lib():
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m online_softmax_05_amd.build`")
        handle = ctypes.CDLL(str(_LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        runtimes = _hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are mapped in this process: {sorted(runtimes)}")
        _lib = handle
    return _lib


def fa_status_str(status):
    return lib().fa_status_str(int(status)).decode()


def fa_abi_version():
    return lib().fa_abi_version()


def fa_decode_splitk_workspace_bytes(B, H, Nk_max, dv, chunk=512):
    return lib().fa_decode_splitk_workspace_bytes(B, H, Nk_max, dv, chunk)


def fa_check_fwd(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, block_n):
    """Host-only validation; pointers are plain integers (or None)."""
    return lib().fa_check_fwd(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale,
                              int(causal), block_n)


def fa_check_fwd_ex(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, align,
                    window_left, window_right, keep_256, seed, block_n):
    """Host-only validation of fa_fwd_ex; pointers are plain integers (or None)."""
    return lib().fa_check_fwd_ex(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale,
                                 int(causal), int(align), int(window_left), int(window_right), int(keep_256),
                                 int(seed) & 0xFFFFFFFFFFFFFFFF, block_n)


def keep_256_for(dropout_p):
    """The byte threshold T of a dropout probability p: round((1 - p) * 256),
    at least 1 (keep probability T/256; T = 256 is no dropout)."""
    p = float(dropout_p)
    if not 0.0 <= p < 1.0:
        raise FaError(3, f"dropout probability must lie in [0, 1), got {p}")
    return max(1, min(256, int(round((1.0 - p) * 256.0))))


def fa_check_decode(q, k, v, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, dtype, scale, workspace,
                    workspace_bytes):
    return lib().fa_check_decode(q, k, v, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, dtype, scale,
                                 workspace, workspace_bytes)


# --------------------------------------------------------------------------
# torch-facing calls
# --------------------------------------------------------------------------

def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise FaError(3, f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, dims=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise FaError(1, f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise FaError(3, f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise FaError(3, f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise FaError(2, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise FaError(3, f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise FaError(2, f"{name} must have {dims} dims, got {tuple(t.shape)}")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _fwd_prepare(q, k, v, bias, k_len, scale, out, lse, want_lse):
    _need(q, "q", dims=4)
    dev = q.device
    _need(k, "k", dtype=q.dtype, dims=4, device=dev)
    _need(v, "v", dtype=q.dtype, dims=4, device=dev)
    B, H, Nq, dk = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, H, Nk, dk) or tuple(v.shape) != (B, H, Nk, dv):
        raise FaError(2, f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if bias is not None:
        _need(bias, "bias", dtype=torch.float32, dims=4, device=dev)
        if tuple(bias.shape) != (B, H, Nq, Nk):
            raise FaError(2, f"bias must be {(B, H, Nq, Nk)}, got {tuple(bias.shape)}")
    if k_len is not None:
        _need(k_len, "k_len", dtype=torch.int32, dims=1, device=dev)
        if k_len.shape[0] != B:
            raise FaError(2, f"k_len must have {B} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=q.dtype, device=dev)
    else:
        _need(out, "out", dtype=q.dtype, dims=4, device=dev)
        if tuple(out.shape) != (B, H, Nq, dv):
            raise FaError(2, "out has the wrong shape")
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need(lse, "lse", dtype=torch.float32, dims=3, device=dev)
        if tuple(lse.shape) != (B, H, Nq):
            raise FaError(2, "lse has the wrong shape")
    return (B, H, Nq, Nk, dk, dv), float(scale), out, lse


def fa_fwd(q, k, v, *, bias=None, k_len=None, scale=None, causal=False, block_n=0, out=None, lse=None,
           want_lse=True):
    """Attention forward: q [B,H,Nq,dk], k [B,H,Nk,dk], v [B,H,Nk,dv] (bf16 or fp32),
    bias fp32 [B,H,Nq,Nk] or None, k_len int32 [B] or None.  Returns (o, lse)."""
    dims, scale, out, lse = _fwd_prepare(q, k, v, bias, k_len, scale, out, lse, want_lse)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(k_len), _ptr(out), _ptr(lse),
                      *dims, _dtype_code(q), scale, int(bool(causal)), int(block_n), _stream(q.device))
    if st != 0:
        raise FaError(st)
    return out, lse


def _masks(align, window_left, window_right, keep_256, dropout_p):
    if align not in _ALIGN:
        raise FaError(3, f"align must be one of {sorted(_ALIGN)}, got {align!r}")
    wl = -1 if window_left is None else int(window_left)
    wr = -1 if window_right is None else int(window_right)
    if wl < 0 and window_left is not None or wr < 0 and window_right is not None:
        raise FaError(3, "window widths must be None or >= 0")
    keep = keep_256_for(dropout_p) if keep_256 is None else int(keep_256)
    return _ALIGN[align], wl, wr, keep


def fa_fwd_ex(q, k, v, *, bias=None, k_len=None, scale=None, causal=False, align="bottom_right",
              window_left=None, window_right=None, dropout_p=0.0, keep_256=None, seed=0, block_n=0, out=None,
              lse=None, want_lse=True):
    """fa_fwd with the mask variants and dropout: ``align`` "bottom_right"
    (row i at key position i + Nk - Nq) or "top_left" (at position i);
    ``window_left`` / ``window_right`` None (open) or a width w >= 0 around
    that position; dropout of P with probability ``dropout_p`` (passed as the
    byte threshold keep_256_for(p), or ``keep_256`` directly) and the 64-bit
    ``seed`` of the counter-based mask."""
    al, wl, wr, keep = _masks(align, window_left, window_right, keep_256, dropout_p)
    dims, scale, out, lse = _fwd_prepare(q, k, v, bias, k_len, scale, out, lse, want_lse)
    st = lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(k_len), _ptr(out), _ptr(lse),
                         *dims, _dtype_code(q), scale, int(bool(causal)), al, wl, wr, keep,
                         int(seed) & 0xFFFFFFFFFFFFFFFF, int(block_n), _stream(q.device))
    if st != 0:
        raise FaError(st)
    return out, lse


def fa_decode_splitk(q, k_cache, v_cache, k_len, *, scale=None, chunk=512, out=None, lse=None,
                     workspace=None, want_lse=True):
    """Single-token decode: q [B,H,dk], caches [B,H,Nk_max,d], k_len int32 [B]
    (required).  The fp32 workspace is allocated with torch unless given.
    Returns (o [B,H,dv], lse [B,H])."""
    _need(q, "q", dims=3)
    dev = q.device
    _need(k_cache, "k_cache", dtype=q.dtype, dims=4, device=dev)
    _need(v_cache, "v_cache", dtype=q.dtype, dims=4, device=dev)
    _need(k_len, "k_len", dtype=torch.int32, dims=1, device=dev)
    B, H, dk = q.shape
    Nk, dv = k_cache.shape[2], v_cache.shape[3]
    if tuple(k_cache.shape) != (B, H, Nk, dk) or tuple(v_cache.shape) != (B, H, Nk, dv):
        raise FaError(2, "cache shapes do not match q")
    if k_len.shape[0] != B:
        raise FaError(2, f"k_len must have {B} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    need = fa_decode_splitk_workspace_bytes(B, H, Nk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    else:
        _need(workspace, "workspace", dtype=torch.float32, dims=1, device=dev)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = lib().fa_decode_splitk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_len), _ptr(out), _ptr(lse),
                                B, H, Nk, dk, dv, int(chunk), _dtype_code(q), float(scale),
                                _ptr(workspace), workspace.numel() * 4, _stream(dev))
    if st != 0:
        raise FaError(st)
    return out, lse


def fa_decode_splitk_static(q, k_cache, v_cache, k_len, *, out, lse=None, scale=None, chunk=512):
    """fa_decode_splitk without a workspace, for callers that cannot allocate:
    the partial states live in the library's static device scratch
    (FA_STATIC_SCRATCH_BYTES per GPU).  The caller passes the outputs
    (o [B,H,dv] in q's dtype; lse fp32 [B,H] or None); nothing is allocated
    here.  Calls that overlap in time on one GPU race on the scratch.
    Returns (out, lse)."""
    _need(q, "q", dims=3)
    dev = q.device
    _need(k_cache, "k_cache", dtype=q.dtype, dims=4, device=dev)
    _need(v_cache, "v_cache", dtype=q.dtype, dims=4, device=dev)
    _need(k_len, "k_len", dtype=torch.int32, dims=1, device=dev)
    B, H, dk = q.shape
    Nk, dv = k_cache.shape[2], v_cache.shape[3]
    if tuple(k_cache.shape) != (B, H, Nk, dk) or tuple(v_cache.shape) != (B, H, Nk, dv):
        raise FaError(2, "cache shapes do not match q")
    if k_len.shape[0] != B:
        raise FaError(2, f"k_len must have {B} entries")
    _need(out, "out", dtype=q.dtype, dims=3, device=dev)
    if tuple(out.shape) != (B, H, dv):
        raise FaError(2, f"out must have shape {(B, H, dv)}")
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, dims=2, device=dev)
        if tuple(lse.shape) != (B, H):
            raise FaError(2, f"lse must have shape {(B, H)}")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    st = lib().fa_decode_splitk_static(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_len), _ptr(out), _ptr(lse),
                                       B, H, Nk, dk, dv, int(chunk), _dtype_code(q), float(scale), _stream(dev))
    if st != 0:
        raise FaError(st)
    return out, lse


def fa_bwd_workspace_bytes(B, H, Nq):
    return lib().fa_bwd_workspace_bytes(B, H, Nq)


def fa_check_bwd_ex(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale,
                    causal, align, window_left, window_right, keep_256, seed, workspace, workspace_bytes):
    """Host-only validation of fa_bwd_ex (integer addresses; nothing is dereferenced)."""
    return lib().fa_check_bwd_ex(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype,
                                 float(scale), causal, align, window_left, window_right, keep_256,
                                 int(seed) & 0xFFFFFFFFFFFFFFFF, workspace, workspace_bytes)


def fa_check_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale,
                 causal, workspace, workspace_bytes):
    """Host-only validation (integer addresses; nothing is dereferenced)."""
    return lib().fa_check_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype,
                              float(scale), causal, workspace, workspace_bytes)


def _bwd_prepare(q, k, v, o, dout, lse, bias, k_len, scale, dq, dk, dv, workspace):
    _need(q, "q", dims=4)
    dev = q.device
    _need(k, "k", dtype=q.dtype, dims=4, device=dev)
    _need(v, "v", dtype=q.dtype, dims=4, device=dev)
    _need(o, "o", dtype=q.dtype, dims=4, device=dev)
    _need(dout, "dout", dtype=q.dtype, dims=4, device=dev)
    _need(lse, "lse", dtype=torch.float32, dims=3, device=dev)
    B, H, Nq, d_k = q.shape
    Nk, d_v = k.shape[2], v.shape[3]
    if (tuple(k.shape) != (B, H, Nk, d_k) or tuple(v.shape) != (B, H, Nk, d_v)
            or tuple(o.shape) != (B, H, Nq, d_v) or tuple(dout.shape) != (B, H, Nq, d_v)
            or tuple(lse.shape) != (B, H, Nq)):
        raise FaError(2, "q/k/v/o/dout/lse shapes do not match")
    if bias is not None:
        _need(bias, "bias", dtype=torch.float32, dims=4, device=dev)
        if tuple(bias.shape) != (B, H, Nq, Nk):
            raise FaError(2, "bias must be [B,H,Nq,Nk]")
    if k_len is not None:
        _need(k_len, "k_len", dtype=torch.int32, dims=1, device=dev)
        if k_len.shape[0] != B:
            raise FaError(2, f"k_len must have {B} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    need = fa_bwd_workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    else:
        _need(workspace, "workspace", dtype=torch.float32, dims=1, device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ptrs = [_ptr(x) for x in (q, k, v, o, dout, lse, bias, k_len, dq, dk, dv)]
    return ptrs, (B, H, Nq, Nk, d_k, d_v), float(scale), (dq, dk, dv), workspace


def fa_bwd(q, k, v, o, dout, lse, *, bias=None, k_len=None, scale=None, causal=False, dq=None, dk=None,
           dv=None, workspace=None):
    """Gradients of fa_fwd by recomputation from its output ``o`` and ``lse``:
    q [B,H,Nq,dk], k [B,H,Nk,dk], v [B,H,Nk,dv], o and dout [B,H,Nq,dv],
    lse fp32 [B,H,Nq]; bias, k_len, scale and causal as given to fa_fwd.
    Returns (dq, dk, dv) in the input dtype."""
    ptrs, dims, scale, grads, workspace = _bwd_prepare(q, k, v, o, dout, lse, bias, k_len, scale, dq, dk, dv,
                                                       workspace)
    st = lib().fa_bwd(*ptrs, *dims, _dtype_code(q), scale, int(bool(causal)), _ptr(workspace),
                      workspace.numel() * 4, _stream(q.device))
    if st != 0:
        raise FaError(st)
    return grads


def fa_bwd_ex(q, k, v, o, dout, lse, *, bias=None, k_len=None, scale=None, causal=False, align="bottom_right",
              window_left=None, window_right=None, dropout_p=0.0, keep_256=None, seed=0, dq=None, dk=None, dv=None,
              workspace=None):
    """Gradients of fa_fwd_ex: the same masks, alignment, dropout
    probability (or keep_256) and seed as the forward call that produced
    ``o`` and ``lse``.  Returns (dq, dk, dv) in the input dtype."""
    al, wl, wr, keep = _masks(align, window_left, window_right, keep_256, dropout_p)
    ptrs, dims, scale, grads, workspace = _bwd_prepare(q, k, v, o, dout, lse, bias, k_len, scale, dq, dk, dv,
                                                       workspace)
    st = lib().fa_bwd_ex(*ptrs, *dims, _dtype_code(q), scale, int(bool(causal)), al, wl, wr, keep,
                         int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(workspace), workspace.numel() * 4, _stream(q.device))
    if st != 0:
        raise FaError(st)
    return grads


def fa_decode_splitk_mq_workspace_bytes(B, H, Nq, Nk_max, dv, chunk=512):
    return lib().fa_decode_splitk_mq_workspace_bytes(B, H, Nq, Nk_max, dv, chunk)


def fa_check_decode_mq(q, k, v, k_len, o, lse, B, H, Nq, Nk_max, dk, dv, chunk, dtype, scale, causal, workspace,
                       workspace_bytes):
    """Host-only validation (integer addresses; nothing is dereferenced)."""
    return lib().fa_check_decode_mq(q, k, v, k_len, o, lse, B, H, Nq, Nk_max, dk, dv, chunk, dtype, float(scale),
                                    causal, workspace, workspace_bytes)


def fa_decode_splitk_mq(q, k_cache, v_cache, k_len, *, causal=True, scale=None, chunk=512, out=None, lse=None,
                        workspace=None, want_lse=True):
    """Split-KV attention of Nq <= 16 query rows per sequence (the sequence's
    last Nq positions): q [B,H,Nq,dk], caches [B,H,Nk_max,d], k_len int32 [B].
    Returns (o [B,H,Nq,dv], lse [B,H,Nq])."""
    _need(q, "q", dims=4)
    dev = q.device
    _need(k_cache, "k_cache", dtype=q.dtype, dims=4, device=dev)
    _need(v_cache, "v_cache", dtype=q.dtype, dims=4, device=dev)
    _need(k_len, "k_len", dtype=torch.int32, dims=1, device=dev)
    B, H, Nq, dk = q.shape
    Nk, dv = k_cache.shape[2], v_cache.shape[3]
    if tuple(k_cache.shape) != (B, H, Nk, dk) or tuple(v_cache.shape) != (B, H, Nk, dv):
        raise FaError(2, "cache shapes do not match q")
    if k_len.shape[0] != B:
        raise FaError(2, f"k_len must have {B} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    need = fa_decode_splitk_mq_workspace_bytes(B, H, Nq, Nk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    else:
        _need(workspace, "workspace", dtype=torch.float32, dims=1, device=dev)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    st = lib().fa_decode_splitk_mq(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_len), _ptr(out), _ptr(lse),
                                   B, H, Nq, Nk, dk, dv, int(chunk), _dtype_code(q), float(scale),
                                   int(bool(causal)), _ptr(workspace), workspace.numel() * 4, _stream(dev))
    if st != 0:
        raise FaError(st)
    return out, lse
