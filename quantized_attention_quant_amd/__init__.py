"""Python binding of libsage — argument marshalling only.

Each function here has the name of a C entry point declared in
``include/sage.h`` and does nothing but check shapes/dtypes on the host,
allocate outputs and the workspace through PyTorch (device memory is the only
thing PyTorch provides), and pass raw pointers plus the current HIP stream to
the library.  Every step of the computation runs in the library's HIP
kernels.  There is no fallback: if ``libsage.so`` is missing or fails to load,
every call raises ``SageError``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

__all__ = [
    "SageError", "LIB_PATH", "lib", "PV_MODES",
    "sage_status_string", "sage_quant_qk_workspace_size", "sage_quant_qk", "sage_quant_v_fp8",
    "sage_attn_workspace_size", "sage_attn_fwd", "sage_attn_fwd_noalloc", "sage_attn_varlen_workspace_size",
    "sage_attn_varlen_fwd", "sage_test_workspace_layout", "sage_test_qk_tiles",
    "sage_test_attn_from_workspace", "sage_test_attn_varlen_from_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage.so")
PV_MODES = {"fp16": 0, "fp8": 1, "mxfp4": 2}
LAYOUT_HND = 0
OPT_SMOOTH_Q = 1        # sage_option_t bits
OPT_Q_PER_TOKEN = 2


def _options(smooth_q: bool, q_per_token: bool) -> int:
    return (OPT_SMOOTH_Q if smooth_q else 0) | (OPT_Q_PER_TOKEN if q_per_token else 0)

# exported symbol -> (restype, argtypes)
_c = ctypes
_P = _c.c_void_p
SIGNATURES = {
    "sage_status_string": (_c.c_char_p, [_c.c_int]),
    "sage_quant_qk_workspace_size": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int]),
    "sage_quant_qk": (_c.c_int, [_P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _P, _c.c_int64,
                                 _c.c_float, _P, _P, _P, _P, _P, _P, _c.c_int, _P, _c.c_size_t, _P]),
    "sage_quant_v_fp8": (_c.c_int, [_P, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _P, _c.c_int64,
                                    _P, _P, _P]),
    "sage_attn_workspace_size": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                               _c.c_int]),
    "sage_attn_fwd": (_c.c_int, [_P, _P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                 _c.c_int, _c.c_int, _c.c_int, _c.c_float, _P, _c.c_size_t, _P]),
    "sage_attn_fwd_noalloc": (_c.c_int, [_P, _P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                         _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float, _P]),
    "sage_attn_varlen_workspace_size": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int64, _c.c_int, _c.c_int,
                                                      _c.c_int, _c.c_int, _c.c_int]),
    "sage_attn_varlen_fwd": (_c.c_int, [_P, _P, _P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int64, _c.c_int,
                                        _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float, _P,
                                        _c.c_size_t, _P]),
    "sage_test_workspace_layout": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int64,
                                              _c.c_int, _c.c_int, _c.c_int, _c.POINTER(_c.c_size_t)]),
    "sage_test_qk_tiles": (_c.c_int, [_P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _P, _c.c_int, _P, _P]),
    "sage_test_attn_from_workspace": (_c.c_int, [_P, _P, _P, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                                 _c.c_int, _c.c_int, _c.c_int, _P, _c.c_size_t, _P]),
    "sage_test_attn_varlen_from_workspace": (_c.c_int, [_P, _P, _P, _P, _c.c_int, _c.c_int, _c.c_int64, _c.c_int,
                                                        _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _P,
                                                        _c.c_size_t, _P]),
}


class SageError(RuntimeError):
    """A libsage call failed (or the library is not available)."""


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libsage.so from this package directory (raises SageError if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SageError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        try:
            handle = ctypes.CDLL(LIB_PATH)
        except OSError as e:
            raise SageError(f"cannot load {LIB_PATH}: {e}") from e
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def sage_status_string(status: int) -> str:
    return lib().sage_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise SageError(f"{what} failed: {sage_status_string(status)} (status {status})")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _alloc_ws(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise SageError(f"workspace smaller than {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _varlen_dims(q: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int):
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    H, T, d = q.shape
    return int(cu_seqlens.numel()) - 1, int(max_seqlen), T, H, d


# ----------------------------------------------------------------------------
def sage_quant_qk_workspace_size(B: int, H: int, d: int) -> int:
    return int(lib().sage_quant_qk_workspace_size(B, H, d))


def sage_quant_qk(q: torch.Tensor, k: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                  max_seqlen: Optional[int] = None, sm_scale: float = 0.0,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  smooth_q: bool = False, q_per_token: bool = False) -> Dict[str, torch.Tensor]:
    """Dense q,k [B,H,N,d] or varlen packed [H,T,d] (+cu_seqlens, max_seqlen).

    Returns dict(q_int8, k_int8, q_scale, k_scale, k_mean[, q_mean with
    smooth_q]) as device tensors in the layouts documented for the C entry
    point (q_scale per token with q_per_token)."""
    L = lib()
    if cu_seqlens is None:
        _need(q, "q", torch.float16, 4)
        _need(k, "k", torch.float16, 4)
        B, H, N, d = q.shape
        T = 0
    else:
        _need(q, "q", torch.float16, 3)
        _need(k, "k", torch.float16, 3)
        B, N, T, H, d = _varlen_dims(q, cu_seqlens, max_seqlen)
    if k.shape != q.shape:
        raise ValueError("q and k shapes differ")
    dev = q.device
    out = dict(
        q_int8=torch.empty(q.shape, dtype=torch.int8, device=dev),
        k_int8=torch.empty(q.shape, dtype=torch.int8, device=dev),
        q_scale=torch.empty(tuple(q.shape[:-1]) if q_per_token else (B, H, -(-N // 128)), dtype=torch.float32,
                            device=dev),
        k_scale=torch.empty((B, H, -(-N // 64)), dtype=torch.float32, device=dev),
        k_mean=torch.empty((B, H, d), dtype=torch.float32, device=dev),
    )
    if smooth_q:
        out["q_mean"] = torch.empty((B, H, -(-N // 128), d), dtype=torch.float32, device=dev)
    ws = _alloc_ws(sage_quant_qk_workspace_size(B, H, d), dev, workspace)
    st = L.sage_quant_qk(q.data_ptr(), k.data_ptr(), B, H, N, d, LAYOUT_HND, _ptr(cu_seqlens), T, float(sm_scale),
                         out["q_int8"].data_ptr(), out["k_int8"].data_ptr(), out["q_scale"].data_ptr(),
                         out["k_scale"].data_ptr(), out["k_mean"].data_ptr(), _ptr(out.get("q_mean")),
                         _options(smooth_q, q_per_token), ws.data_ptr(), ws.numel() * ws.element_size(),
                         _stream(stream))
    _check(st, "sage_quant_qk")
    return out


def sage_quant_v_fp8(v: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                     max_seqlen: Optional[int] = None, stream=None):
    """Returns (v_fp8 uint8 codes, same layout as v; v_scale fp32 [B,H,d])."""
    L = lib()
    if cu_seqlens is None:
        _need(v, "v", torch.float16, 4)
        B, H, N, d = v.shape
        T = 0
    else:
        _need(v, "v", torch.float16, 3)
        B, N, T, H, d = _varlen_dims(v, cu_seqlens, max_seqlen)
    codes = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    scale = torch.empty((B, H, d), dtype=torch.float32, device=v.device)
    st = L.sage_quant_v_fp8(v.data_ptr(), B, H, N, d, LAYOUT_HND, _ptr(cu_seqlens), T, codes.data_ptr(),
                            scale.data_ptr(), _stream(stream))
    _check(st, "sage_quant_v_fp8")
    return codes, scale


def sage_attn_workspace_size(B: int, H: int, N: int, d: int, pv_mode: str = "fp16",
                             H_kv: Optional[int] = None, smooth_q: bool = False, q_per_token: bool = False) -> int:
    return int(lib().sage_attn_workspace_size(B, H, H if H_kv is None else H_kv, N, d, PV_MODES[pv_mode],
                                              _options(smooth_q, q_per_token)))


def _lse_out(return_lse: bool, lse: Optional[torch.Tensor], shape, device) -> Optional[torch.Tensor]:
    if lse is not None:
        _need(lse, "lse", torch.float32, len(shape))
        if tuple(lse.shape) != tuple(shape):
            raise ValueError(f"lse must have shape {tuple(shape)}")
        return lse
    return torch.empty(shape, dtype=torch.float32, device=device) if return_lse else None


def sage_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool = False,
                  pv_mode: str = "fp16", sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None, return_lse: bool = False,
                  lse: Optional[torch.Tensor] = None, smooth_q: bool = False, q_per_token: bool = False):
    """Dense forward: q fp16 [B,H,N,d], k and v fp16 [B,H_kv,N,d] (H_kv divides H).
    smooth_q selects Q smoothing, q_per_token per-token Q scales.  Returns o
    fp16 [B,H,N,d], or (o, lse fp32 [B,H,N]) when return_lse or lse is given."""
    L = lib()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.float16, 4)
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must be [B,H_kv,N,d] with q's B, N and d")
    H_kv = k.shape[1]
    if pv_mode not in PV_MODES:
        raise ValueError(f"pv_mode must be one of {list(PV_MODES)}")
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", torch.float16, 4)
    lse_t = _lse_out(return_lse, lse, (B, H, N), q.device)
    opts = _options(smooth_q, q_per_token)
    ws = _alloc_ws(sage_attn_workspace_size(B, H, N, d, pv_mode, H_kv, smooth_q, q_per_token), q.device, workspace)
    st = L.sage_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse_t), B, H, H_kv, N, d,
                         LAYOUT_HND, int(bool(is_causal)), PV_MODES[pv_mode], opts, float(sm_scale),
                         ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sage_attn_fwd")
    return o if lse_t is None else (o, lse_t)


NOALLOC_SCRATCH_BYTES = 256 << 20   # SAGE_NOALLOC_SCRATCH_BYTES of include/sage.h


def sage_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool = False,
                          pv_mode: str = "fp16", sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                          stream=None, return_lse: bool = False, lse: Optional[torch.Tensor] = None,
                          smooth_q: bool = False, q_per_token: bool = False):
    """sage_attn_fwd without a workspace: the library's per-GPU scratch array
    holds the pre-pass results (calls that overlap on one GPU race).  Returns
    o fp16 [B,H,N,d], or (o, lse)."""
    L = lib()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.float16, 4)
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must be [B,H_kv,N,d] with q's B, N and d")
    H_kv = k.shape[1]
    if pv_mode not in PV_MODES:
        raise ValueError(f"pv_mode must be one of {list(PV_MODES)}")
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", torch.float16, 4)
    lse_t = _lse_out(return_lse, lse, (B, H, N), q.device)
    st = L.sage_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse_t), B, H, H_kv, N,
                                 d, LAYOUT_HND, int(bool(is_causal)), PV_MODES[pv_mode],
                                 _options(smooth_q, q_per_token), float(sm_scale), _stream(stream))
    _check(st, "sage_attn_fwd_noalloc")
    return o if lse_t is None else (o, lse_t)


def sage_attn_varlen_workspace_size(nseq: int, max_seqlen: int, total_tokens: int, H: int, d: int,
                                    pv_mode: str = "fp16", H_kv: Optional[int] = None,
                                    smooth_q: bool = False, q_per_token: bool = False) -> int:
    return int(lib().sage_attn_varlen_workspace_size(nseq, max_seqlen, total_tokens, H, H if H_kv is None else H_kv,
                                                     d, PV_MODES[pv_mode], _options(smooth_q, q_per_token)))


def sage_attn_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                         max_seqlen: int, is_causal: bool = False, pv_mode: str = "fp16", sm_scale: float = 0.0,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None, return_lse: bool = False, lse: Optional[torch.Tensor] = None,
                         smooth_q: bool = False, q_per_token: bool = False):
    """Packed forward: q fp16 [H,T,d], k and v fp16 [H_kv,T,d], int32 cu_seqlens [nseq+1]
    (device).  Returns o fp16 [H,T,d], or (o, lse fp32 [H,T])."""
    L = lib()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.float16, 3)
    nseq, N, T, H, d = _varlen_dims(q, cu_seqlens, max_seqlen)
    if k.shape != v.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("k and v must be [H_kv,T,d] with q's T and d")
    H_kv = k.shape[0]
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", torch.float16, 3)
    lse_t = _lse_out(return_lse, lse, (H, T), q.device)
    ws = _alloc_ws(sage_attn_varlen_workspace_size(nseq, N, T, H, d, pv_mode, H_kv, smooth_q, q_per_token), q.device,
                   workspace)
    st = L.sage_attn_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse_t),
                                cu_seqlens.data_ptr(), nseq, N, T, H, H_kv, d, int(bool(is_causal)),
                                PV_MODES[pv_mode], _options(smooth_q, q_per_token), float(sm_scale), ws.data_ptr(),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sage_attn_varlen_fwd")
    return o if lse_t is None else (o, lse_t)


def sage_test_workspace_layout(varlen: bool, B: int, H: int, N: int, total_tokens: int, d: int,
                               pv_mode: str = "fp16", H_kv: Optional[int] = None,
                               smooth_q: bool = False, q_per_token: bool = False) -> Sequence[int]:
    """Byte offsets [0..10] of the workspace regions and [11] its total size."""
    arr = (ctypes.c_size_t * 12)()
    st = lib().sage_test_workspace_layout(int(bool(varlen)), B, H, H if H_kv is None else H_kv, N, total_tokens, d,
                                          PV_MODES[pv_mode], _options(smooth_q, q_per_token), arr)
    _check(st, "sage_test_workspace_layout")
    return list(arr)


def sage_test_qk_tiles(q_int8: torch.Tensor, k_int8: torch.Tensor, tile_list: torch.Tensor,
                       stream=None) -> torch.Tensor:
    """int32 [n,128,64] Q̂K̂ᵀ tiles for rows of tile_list (int32 [n,4]: b,h,q_block,k_block)."""
    _need(q_int8, "q_int8", torch.int8, 4)
    _need(k_int8, "k_int8", torch.int8, 4)
    _need(tile_list, "tile_list", torch.int32, 2)
    B, H, N, d = q_int8.shape
    n = tile_list.shape[0]
    out = torch.empty((n, 128, 64), dtype=torch.int32, device=q_int8.device)
    st = lib().sage_test_qk_tiles(q_int8.data_ptr(), k_int8.data_ptr(), B, H, N, d, tile_list.data_ptr(), n,
                                  out.data_ptr(), _stream(stream))
    _check(st, "sage_test_qk_tiles")
    return out


def sage_test_attn_from_workspace(out: torch.Tensor, workspace: torch.Tensor, v: Optional[torch.Tensor] = None,
                                  is_causal: bool = False, pv_mode: str = "fp16", stream=None,
                                  H_kv: Optional[int] = None, smooth_q: bool = False,
                                  q_per_token: bool = False, q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run only the fused attention kernel on a workspace filled by sage_attn_fwd
    (same shapes and options; v: that call's fp16 V, read directly in fp16 PV
    mode; q: that call's fp16 Q, which the kernel quantises itself without
    options in fp16/fp8 PV mode); out fp16 [B,H,N,d] is written and returned."""
    _need(out, "out", torch.float16, 4)
    if v is not None:
        _need(v, "v", torch.float16, 4)
    if q is not None:
        _need(q, "q", torch.float16, 4)
    B, H, N, d = out.shape
    st = lib().sage_test_attn_from_workspace(out.data_ptr(), 0 if q is None else q.data_ptr(),
                                             0 if v is None else v.data_ptr(), B, H,
                                             H if H_kv is None else H_kv, N, d,
                                             int(bool(is_causal)), PV_MODES[pv_mode], _options(smooth_q, q_per_token),
                                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                             _stream(stream))
    _check(st, "sage_test_attn_from_workspace")
    return out


def sage_test_attn_varlen_from_workspace(out: torch.Tensor, workspace: torch.Tensor, cu_seqlens: torch.Tensor,
                                         max_seqlen: int, v: Optional[torch.Tensor] = None,
                                         is_causal: bool = False, pv_mode: str = "fp16", stream=None,
                                         H_kv: Optional[int] = None, smooth_q: bool = False,
                                         q_per_token: bool = False, q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run only the fused attention kernel on a workspace filled by
    sage_attn_varlen_fwd (same cu_seqlens, shapes and options; v, q as for
    sage_test_attn_from_workspace, packed [H_kv,T,d] / [H,T,d]); out fp16
    [H,T,d] is written and returned."""
    _need(out, "out", torch.float16, 3)
    if v is not None:
        _need(v, "v", torch.float16, 3)
    if q is not None:
        _need(q, "q", torch.float16, 3)
    nseq, N, T, H, d = _varlen_dims(out, cu_seqlens, max_seqlen)
    st = lib().sage_test_attn_varlen_from_workspace(out.data_ptr(), 0 if q is None else q.data_ptr(),
                                                    0 if v is None else v.data_ptr(), cu_seqlens.data_ptr(), nseq,
                                                    N, T, H, H if H_kv is None else H_kv, d, int(bool(is_causal)),
                                                    PV_MODES[pv_mode], _options(smooth_q, q_per_token),
                                                    workspace.data_ptr(),
                                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "sage_test_attn_varlen_from_workspace")
    return out
