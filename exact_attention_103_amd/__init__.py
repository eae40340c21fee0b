"""Exact fused attention forward and split-KV decode for MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libfa.so`` (declared in
``include/fa.h``).  The functions named like the C entry points take raw
device pointers and sizes; ``fwd`` and ``decode`` accept torch tensors,
allocate outputs (and the decode workspace) with torch and pass torch's
current HIP stream.  Every step of the computation runs in the HIP kernels:
if the library is missing this module raises instead of computing anything.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FAError", "lib", "fa_fwd", "fa_decode_splitkv", "fa_decode_workspace_size",
    "fa_decode_num_splits", "fa_decode_max_splits", "fa_strerror",
    "fa_last_hip_error", "fa_fwd_kernel_name", "fa_decode_kernel_name",
    "fa_bwd", "fa_bwd_workspace_size", "fa_bwd_kernel_name",
    "fa_decode_serve", "fa_decode_serve_workspace_size", "fa_decode_serve_num_splits",
    "fa_decode_serve_kernel_name", "fa_fwd_fp8", "fa_fwd_fp8_kernel_name",
    "fa_fwd_fp8_devscale", "fa_fp8_quantize", "fa_fp8_quantize_workspace_size",
    "fa_fp8_quantize_kernel_name", "fa_build_is_serial", "fa_decode_splitkv_noalloc",
    "DECODE_NOALLOC_SCRATCH_BYTES", "decode_noalloc",
    "fwd", "fwd_fp8", "fp8_quantize", "decode", "decode_serve", "bwd", "EXPORTED_SYMBOLS",
    "LIB_PATH", "SERIAL_LIB_PATH", "load_library",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
# Race-check build of the same sources (staged copies never overlap compute);
# only tests load it.
SERIAL_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_serial.so")

FA_OK = 0

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_cs = ctypes.c_char_p

# name -> (restype, argtypes); mirrors include/fa.h
_SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "fa_decode_splitkv": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                               _vp, _sz, _vp]),
    "fa_decode_workspace_size": (_sz, [_i, _i, _i, _i]),
    "fa_decode_num_splits": (_i, [_i, _i, _i, _i, _i]),
    "fa_decode_max_splits": (_i, [_i]),
    "fa_strerror": (_cs, [_i]),
    "fa_last_hip_error": (_cs, []),
    "fa_fwd_kernel_name": (_cs, [_i, _i, _i, _i]),
    "fa_decode_kernel_name": (_cs, [_i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                    _i, _vp, _sz, _vp]),
    "fa_bwd_workspace_size": (_sz, [_i, _i, _i]),
    "fa_bwd_kernel_name": (_cs, [_i, _i, _i]),
    "fa_decode_serve": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                             _vp, _sz, _vp]),
    "fa_decode_serve_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "fa_decode_serve_num_splits": (_i, [_i, _i, _i, _i, _i, _i]),
    "fa_decode_serve_kernel_name": (_cs, [_i, _i, _i, _i]),
    "fa_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _f, _f, _i,
                        _vp]),
    "fa_fwd_fp8_kernel_name": (_cs, [_i, _i]),
    "fa_fwd_fp8_devscale": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                 _vp, _i, _vp]),
    "fa_fp8_quantize_workspace_size": (_sz, [_i, _i]),
    "fa_fp8_quantize": (_i, [_vp, _vp, _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "fa_fp8_quantize_kernel_name": (_cs, [_i, _i]),
    "fa_build_is_serial": (_i, []),
    "fa_decode_splitkv_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                       _vp]),
}

# FA_DECODE_NOALLOC_SCRATCH_BYTES of include/fa.h: the fixed scratch of
# fa_decode_splitkv_noalloc.
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


class FAError(RuntimeError):
    """A negative status returned by libfa.so."""

    def __init__(self, status: int, where: str):
        text = lib().fa_strerror(status).decode()
        if status == -7:
            text += " (" + lib().fa_last_hip_error().decode() + ")"
        super().__init__(f"{where}: {text} [status {status}]")
        self.status = status


def load_library(path=LIB_PATH):
    """Open a build of the C ABI (libfa.so, or the race-check build
    libfa_serial.so) with every declared signature set.  Raises if the file
    has not been built."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_attention_103_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """The loaded libfa.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


# --- Entry points with the C names: raw pointers (ints) and sizes. ---------

def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream=None):
    return lib().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
                        stream)


def fa_decode_splitkv(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale,
                      num_splits, workspace, workspace_bytes, stream=None):
    return lib().fa_decode_splitkv(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d,
                                   scale, num_splits, workspace, workspace_bytes,
                                   stream)


def fa_decode_splitkv_noalloc(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale,
                              num_splits, stream=None):
    return lib().fa_decode_splitkv_noalloc(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d,
                                           scale, num_splits, stream)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal,
           workspace, workspace_bytes, stream=None):
    return lib().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                        int(causal), workspace, workspace_bytes, stream)


def fa_decode_serve(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                    num_splits, workspace, workspace_bytes, stream=None):
    return lib().fa_decode_serve(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                                 scale, int(causal), num_splits, workspace, workspace_bytes,
                                 stream)


def fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale, v_descale,
               causal, stream=None):
    return lib().fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale,
                            v_descale, int(causal), stream)


def fa_fwd_fp8_kernel_name(d, causal):
    r = lib().fa_fwd_fp8_kernel_name(d, int(causal))
    return r.decode() if r else None


def fa_fwd_fp8_devscale(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale,
                        v_descale, causal, stream=None):
    return lib().fa_fwd_fp8_devscale(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale,
                                     k_descale, v_descale, int(causal), stream)


def fa_fp8_quantize_workspace_size(rows, d):
    return lib().fa_fp8_quantize_workspace_size(rows, d)


def fa_fp8_quantize(x, codes, descale, signs, rows, d, workspace, workspace_bytes, stream=None):
    return lib().fa_fp8_quantize(x, codes, descale, signs, rows, d, workspace, workspace_bytes,
                                 stream)


def fa_fp8_quantize_kernel_name(d, stage):
    r = lib().fa_fp8_quantize_kernel_name(d, stage)
    return r.decode() if r else None


def fa_decode_serve_workspace_size(B, Hq, Nq, d, num_splits):
    return lib().fa_decode_serve_workspace_size(B, Hq, Nq, d, num_splits)


def fa_decode_serve_num_splits(B, Hq, Hkv, Nq, Nk, d):
    return lib().fa_decode_serve_num_splits(B, Hq, Hkv, Nq, Nk, d)


def fa_decode_serve_kernel_name(d, hq_per_kv, Nq, stage):
    r = lib().fa_decode_serve_kernel_name(d, hq_per_kv, Nq, stage)
    return r.decode() if r else None


def fa_bwd_workspace_size(B, Hq, Nq):
    return lib().fa_bwd_workspace_size(B, Hq, Nq)


def fa_bwd_kernel_name(d, causal, stage):
    r = lib().fa_bwd_kernel_name(d, int(causal), stage)
    return r.decode() if r else None


def fa_build_is_serial():
    return lib().fa_build_is_serial()


def fa_decode_workspace_size(B, Hq, d, num_splits):
    return lib().fa_decode_workspace_size(B, Hq, d, num_splits)


def fa_decode_num_splits(B, Hq, Hkv, Nk, d):
    return lib().fa_decode_num_splits(B, Hq, Hkv, Nk, d)


def fa_decode_max_splits(Nk):
    return lib().fa_decode_max_splits(Nk)


def fa_strerror(status):
    return lib().fa_strerror(status).decode()


def fa_last_hip_error():
    return lib().fa_last_hip_error().decode()


def fa_fwd_kernel_name(d, causal, Nq, Nk):
    r = lib().fa_fwd_kernel_name(d, int(causal), Nq, Nk)
    return r.decode() if r else None


def fa_decode_kernel_name(d, hq_per_kv, stage):
    r = lib().fa_decode_kernel_name(d, hq_per_kv, stage)
    return r.decode() if r else None


# --- torch-facing helpers (marshalling only). ------------------------------

def _check_bf16(name, t, ndim):
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(name, t, dtype, shape, like):
    """A caller-supplied output must match exactly what the kernel writes:
    the C ABI sees only a pointer, so an undersized tensor would be
    overwritten past its end."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(t, need, like):
    """(pointer, size in bytes) of a workspace tensor, allocated when None."""
    import torch
    if t is None:
        t = torch.empty(max(need, 16), dtype=torch.uint8, device=like.device)
    if not t.is_cuda or t.device != like.device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {like.device}")
    return t, t.numel() * t.element_size()


def _stream_ptr():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """O, LSE = attention(q, k, v); q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] bf16."""
    import torch
    _check_bf16("q", q, 4)
    _check_bf16("k", k, 4)
    _check_bf16("v", v, 4)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B][Hkv][Nk][d] with q's B and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_out("out", out, torch.bfloat16, (B, Hq, Nq, d), q)
    _check_out("lse", lse, torch.float32, (B, Hq, Nq), q)
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd")
    return out, lse


def decode(q, k_cache, v_cache, scale=None, num_splits=0, out=None, lse=None,
           workspace=None):
    """Split-KV decode: q [B][Hq][d], caches [B][Hkv][Nk][d] bf16 -> O, LSE."""
    import torch
    _check_bf16("q", q, 3)
    _check_bf16("k_cache", k_cache, 4)
    _check_bf16("v_cache", v_cache, 4)
    B, Hq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Nk, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [B][Hkv][Nk][d] with q's B and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = num_splits
    if S == 0:
        S = fa_decode_num_splits(B, Hq, Hkv, Nk, d)
        if S < 0:
            raise FAError(S, "fa_decode_num_splits")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out("out", out, torch.bfloat16, (B, Hq, d), q)
    _check_out("lse", lse, torch.float32, (B, Hq), q)
    workspace, ws_bytes = _workspace(workspace, fa_decode_workspace_size(B, Hq, d, S), q)
    rc = fa_decode_splitkv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nk, d,
                           float(scale), S, workspace.data_ptr(), ws_bytes,
                           _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_decode_splitkv")
    return out, lse


def decode_noalloc(q, k_cache, v_cache, out, lse, scale=None, num_splits=0):
    """Split-KV decode through the allocation-free entry point: the caller
    passes the outputs (out bf16 [B][Hq][d], lse fp32 [B][Hq]) and nothing is
    allocated; the split partials live in the library's fixed scratch."""
    import torch
    _check_bf16("q", q, 3)
    _check_bf16("k_cache", k_cache, 4)
    _check_bf16("v_cache", v_cache, 4)
    B, Hq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Nk, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [B][Hkv][Nk][d] with q's B and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_out("out", out, torch.bfloat16, (B, Hq, d), q)
    _check_out("lse", lse, torch.float32, (B, Hq), q)
    rc = fa_decode_splitkv_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nk, d,
                                   float(scale), num_splits, _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_decode_splitkv_noalloc")
    return out, lse


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, workspace=None):
    """dQ, dK, dV of attention; q/o/dout [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] bf16,
    lse [B][Hq][Nq] fp32 (the forward's outputs o and lse)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_bf16(name, t, 4)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B][Hkv][Nk][d] with q's B and d")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B][Hq][Nq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    workspace, ws_bytes = _workspace(workspace, fa_bwd_workspace_size(B, Hq, Nq), q)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq,
                Nk, d, float(scale), int(bool(causal)), workspace.data_ptr(), ws_bytes,
                _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_bwd")
    return dq, dk, dv


def decode_serve(q, k_cache, v_cache, seqlens=None, causal=False, scale=None, num_splits=0,
                 out=None, lse=None, workspace=None):
    """Serving-shaped decode: q [B][Hq][Nq][d] (Nq <= 16), caches
    [B][Hkv][Nk][d] bf16 (Nk = capacity), seqlens int32 [B] device tensor or
    None -> O [B][Hq][Nq][d], LSE [B][Hq][Nq]."""
    import torch
    _check_bf16("q", q, 4)
    _check_bf16("k_cache", k_cache, 4)
    _check_bf16("v_cache", v_cache, 4)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Nk, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [B][Hkv][Nk][d] with q's B and d")
    sl = 0
    if seqlens is not None:
        if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,) or not seqlens.is_cuda:
            raise ValueError("seqlens must be an int32 [B] device tensor")
        sl = seqlens.contiguous().data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = num_splits
    if S == 0:
        S = fa_decode_serve_num_splits(B, Hq, Hkv, Nq, Nk, d)
        if S < 0:
            raise FAError(S, "fa_decode_serve_num_splits")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_out("out", out, torch.bfloat16, (B, Hq, Nq, d), q)
    _check_out("lse", lse, torch.float32, (B, Hq, Nq), q)
    workspace, ws_bytes = _workspace(workspace, fa_decode_serve_workspace_size(B, Hq, Nq, d, S), q)
    rc = fa_decode_serve(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), sl or None,
                         out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                         int(bool(causal)), S, workspace.data_ptr(), ws_bytes,
                         _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_decode_serve")
    return out, lse


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False, scale=None, out=None,
            lse=None):
    """O, LSE of attention on fp8 e4m3 inputs (uint8 tensors [B][H][N][d],
    real value = byte value * descale) -> O bf16, LSE fp32."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.uint8 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 (fp8 e4m3 bytes) device tensor "
                             "[B][H][N][d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B][Hkv][Nk][d] with q's B and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_out("out", out, torch.bfloat16, (B, Hq, Nq, d), q)
    _check_out("lse", lse, torch.float32, (B, Hq, Nq), q)
    descales = (q_descale, k_descale, v_descale)
    if all(isinstance(x, torch.Tensor) for x in descales):
        for name, t in zip(("q_descale", "k_descale", "v_descale"), descales):
            if t.dtype != torch.float32 or t.numel() != 1 or not t.is_cuda:
                raise ValueError(f"{name} must be a one-element float32 device tensor")
        rc = fa_fwd_fp8_devscale(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                 *(t.data_ptr() for t in descales), int(bool(causal)),
                                 _stream_ptr())
        if rc != FA_OK:
            raise FAError(rc, "fa_fwd_fp8_devscale")
        return out, lse
    rc = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                    Hq, Hkv, Nq, Nk, d, float(scale), float(q_descale), float(k_descale),
                    float(v_descale), int(bool(causal)), _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_fp8")
    return out, lse


def fp8_quantize(x, signs=None, codes=None, descale=None, workspace=None):
    """Incoherent processing and per-tensor e4m3 quantisation of a bf16
    device tensor [..., d] (d = 32, 64, 128 or 256): rotated by diag(signs) H_d /
    sqrt(d) when `signs` (int8 device tensor [d], negative = -1) is given.
    Returns (codes uint8 tensor of x's shape, descale float32 device tensor
    [1]) with codes * descale approximating the rotated x."""
    import torch
    _check_bf16("x", x, x.dim())
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if signs is not None and (signs.dtype != torch.int8 or tuple(signs.shape) != (d,)
                              or not signs.is_cuda):
        raise ValueError("signs must be an int8 device tensor of shape [d]")
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check_out("codes", codes, torch.uint8, tuple(x.shape), x)
    _check_out("descale", descale, torch.float32, (1,), x)
    workspace, ws_bytes = _workspace(workspace, fa_fp8_quantize_workspace_size(rows, d), x)
    rc = fa_fp8_quantize(x.data_ptr(), codes.data_ptr(), descale.data_ptr(),
                         signs.data_ptr() if signs is not None else None, rows, d,
                         workspace.data_ptr(), ws_bytes, _stream_ptr())
    if rc != FA_OK:
        raise FAError(rc, "fa_fp8_quantize")
    return codes, descale
