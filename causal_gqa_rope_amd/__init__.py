"""Python binding of libcgr: fused causal GQA + RoPE attention forward on gfx950.

Argument marshalling only. Every step of the computation runs in the HIP
kernels of ``libcgr.so``; torch supplies device memory and the current
stream. The functions carry the names of the C entry points declared in
``include/cgr.h`` (``cgr_rope_tables``, ``cgr_gqa_rope_attn_fwd``,
``cgr_gqa_rope_attn_fwd_varlen``, ``cgr_gqa_rope_attn_bwd``,
``cgr_gqa_rope_attn_bwd_varlen``, ``cgr_rope_rotate``,
``cgr_gqa_rope_attn_decode``, ...); the short names (``rope_tables``,
``gqa_rope_attn_fwd``, ``gqa_rope_attn_fwd_varlen``, ``gqa_rope_attn_bwd``,
``gqa_rope_attn_bwd_varlen``, ``rope_rotate``, ``gqa_rope_attn_decode``) are
the same functions.

The library leaves the HIP runtime's symbols unresolved; before loading it,
the binding makes the runtime torch already loaded globally visible, so the
kernels run on torch's runtime instance. There is no fallback: without the
built library (``python -m causal_gqa_rope_amd.build``) every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "CgrError",
    "library",
    "library_path",
    "cgr_rope_tables",
    "cgr_gqa_rope_attn_fwd",
    "cgr_attn_fwd_workspace_size",
    "cgr_attn_fwd_rotate_keys",
    "cgr_gqa_rope_attn_fwd_rotated",
    "cgr_gqa_rope_attn_fwd_varlen",
    "cgr_gqa_rope_attn_fwd_varlen_noalloc",
    "cgr_attn_fwd_varlen_workspace_size",
    "cgr_attn_fwd_varlen_rotated_workspace_size",
    "cgr_varlen_device_status",
    "cgr_attn_bwd_workspace_size",
    "cgr_gqa_rope_attn_bwd",
    "cgr_attn_bwd_varlen_workspace_size",
    "cgr_gqa_rope_attn_bwd_varlen",
    "cgr_rope_rotate",
    "cgr_attn_decode_workspace_size",
    "cgr_gqa_rope_attn_decode",
    "cgr_rmsnorm_qkv_rope_workspace_size",
    "cgr_rmsnorm_qkv_rope",
    "cgr_version",
    "rope_tables",
    "gqa_rope_attn_fwd",
    "gqa_rope_attn_fwd_varlen",
    "gqa_rope_attn_bwd",
    "gqa_rope_attn_bwd_varlen",
    "rope_rotate",
    "gqa_rope_attn_decode",
    "rmsnorm_qkv_rope",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libcgr.so")

# Status codes (cgr_status).
CGR_OK, CGR_ERR_INVALID_ARG, CGR_ERR_UNSUPPORTED, CGR_ERR_ALIGNMENT, CGR_ERR_WORKSPACE, CGR_ERR_HIP = range(6)
_STATUS_NAMES = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "ALIGNMENT", 4: "WORKSPACE", 5: "HIP"}
CGR_F32, CGR_BF16 = 0, 1
CGR_ROPE_INTERLEAVED, CGR_ROPE_HALF = 0, 1
CGR_MASK_NONE, CGR_MASK_CAUSAL = 0, 1
CGR_QK_F16, CGR_QK_BF16 = 0, 1

EXPORTED_SYMBOLS = (
    "cgr_rope_tables",
    "cgr_gqa_rope_attn_fwd",
    "cgr_attn_fwd_workspace_size",
    "cgr_attn_fwd_rotate_keys",
    "cgr_gqa_rope_attn_fwd_rotated",
    "cgr_attn_fwd_varlen_workspace_size",
    "cgr_attn_fwd_varlen_rotated_workspace_size",
    "cgr_gqa_rope_attn_fwd_varlen",
    "cgr_gqa_rope_attn_fwd_varlen_noalloc",
    "cgr_varlen_device_status",
    "cgr_attn_bwd_workspace_size",
    "cgr_gqa_rope_attn_bwd",
    "cgr_attn_bwd_varlen_workspace_size",
    "cgr_gqa_rope_attn_bwd_varlen",
    "cgr_rope_rotate",
    "cgr_attn_decode_workspace_size",
    "cgr_gqa_rope_attn_decode",
    "cgr_rmsnorm_qkv_rope_workspace_size",
    "cgr_rmsnorm_qkv_rope",
    "cgr_attn_fwd_fp8_workspace_size",
    "cgr_gqa_rope_attn_fwd_fp8",
    "cgr_last_error",
    "cgr_version",
)


class CgrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cgr status {status} ({_STATUS_NAMES.get(status, '?')}): {message}")
        self.status = status


_LIB = None


def _make_hip_runtime_global() -> None:
    """Promote the HIP runtime torch loaded to RTLD_GLOBAL (no second runtime is loaded)."""
    import torch.cuda  # noqa: F401  (loads torch's HIP libraries)
    with open("/proc/self/maps") as f:
        paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    if not paths:
        raise CgrError(CGR_ERR_HIP, "no HIP runtime (libamdhip64) is loaded in this process")
    mode = ctypes.RTLD_GLOBAL | getattr(os, "RTLD_NOLOAD", 4)
    for p in paths:
        ctypes.CDLL(p, mode=mode)


def library() -> ctypes.CDLL:
    """Load libcgr.so (once) and declare its C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(library_path):
        raise CgrError(CGR_ERR_HIP, f"{library_path} is not built: run python -m causal_gqa_rope_amd.build")
    _make_hip_runtime_global()
    lib = ctypes.CDLL(library_path)
    vp, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.cgr_rope_tables.argtypes = [i32, i32, f64, vp, vp, vp]
    lib.cgr_rope_tables.restype = i32
    lib.cgr_attn_fwd_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.cgr_attn_fwd_workspace_size.restype = ctypes.c_size_t
    lib.cgr_gqa_rope_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp,
                                          i32, i32, i32, i32, f32, i32, vp, vp, ctypes.c_size_t, vp]
    lib.cgr_gqa_rope_attn_fwd.restype = i32
    lib.cgr_attn_fwd_rotate_keys.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, i32, i32, i32, vp, vp,
                                             ctypes.c_size_t, vp]
    lib.cgr_attn_fwd_rotate_keys.restype = i32
    lib.cgr_gqa_rope_attn_fwd_rotated.argtypes = lib.cgr_gqa_rope_attn_fwd.argtypes
    lib.cgr_gqa_rope_attn_fwd_rotated.restype = i32
    lib.cgr_attn_fwd_fp8_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.cgr_attn_fwd_fp8_workspace_size.restype = ctypes.c_size_t
    lib.cgr_gqa_rope_attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, f32, vp, vp,
                                              i32, i32, i32, f32, vp, vp, ctypes.c_size_t, vp]
    lib.cgr_gqa_rope_attn_fwd_fp8.restype = i32
    lib.cgr_attn_fwd_varlen_workspace_size.argtypes = [i32, i32]
    lib.cgr_attn_fwd_varlen_workspace_size.restype = ctypes.c_size_t
    lib.cgr_attn_fwd_varlen_rotated_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.cgr_attn_fwd_varlen_rotated_workspace_size.restype = ctypes.c_size_t
    lib.cgr_gqa_rope_attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                 i32, i32, vp, vp, i32, i32, i32, i32, f32, i32, vp,
                                                 ctypes.c_size_t, vp]
    lib.cgr_gqa_rope_attn_fwd_varlen.restype = i32
    lib.cgr_gqa_rope_attn_fwd_varlen_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                         vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.cgr_gqa_rope_attn_fwd_varlen_noalloc.restype = i32
    lib.cgr_attn_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.cgr_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.cgr_gqa_rope_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          i32, vp, vp, i32, i32, i32, i32, f32, i32, vp, ctypes.c_size_t,
                                          vp]
    lib.cgr_gqa_rope_attn_bwd.restype = i32
    lib.cgr_attn_bwd_varlen_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.cgr_attn_bwd_varlen_workspace_size.restype = ctypes.c_size_t
    lib.cgr_gqa_rope_attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                 i32, i32, i32, vp, vp, i32, i32, i32, i32, f32, i32, vp,
                                                 ctypes.c_size_t, vp]
    lib.cgr_gqa_rope_attn_bwd_varlen.restype = i32
    lib.cgr_rope_rotate.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, vp]
    lib.cgr_rope_rotate.restype = i32
    lib.cgr_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.cgr_attn_decode_workspace_size.restype = ctypes.c_size_t
    i64 = ctypes.c_int64
    lib.cgr_gqa_rope_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i64, i32, i32,
                                             i32, i32, i32, vp, vp, i32, i32, i32, f32, vp, ctypes.c_size_t,
                                             vp]
    lib.cgr_gqa_rope_attn_decode.restype = i32
    lib.cgr_rmsnorm_qkv_rope_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.cgr_rmsnorm_qkv_rope_workspace_size.restype = ctypes.c_size_t
    lib.cgr_rmsnorm_qkv_rope.argtypes = [vp, vp, f32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp,
                                         vp, i32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.cgr_rmsnorm_qkv_rope.restype = i32
    lib.cgr_varlen_device_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.cgr_varlen_device_status.restype = i32
    lib.cgr_last_error.argtypes = []
    lib.cgr_last_error.restype = ctypes.c_char_p
    lib.cgr_version.argtypes = []
    lib.cgr_version.restype = i32
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != CGR_OK:
        msg = library().cgr_last_error()
        raise CgrError(status, msg.decode() if msg else "")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_DTYPES = {torch.float32: CGR_F32, torch.bfloat16: CGR_BF16}
_STYLES = {"interleaved": CGR_ROPE_INTERLEAVED, "half": CGR_ROPE_HALF}
_QK = {"f16": CGR_QK_F16, "bf16": CGR_QK_BF16}


def _dev_tensor(name: str, t: torch.Tensor, dtype=None) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise CgrError(CGR_ERR_INVALID_ARG, f"{name} must be a CUDA/HIP tensor")
    if not t.is_contiguous():
        raise CgrError(CGR_ERR_INVALID_ARG, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise CgrError(CGR_ERR_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")


def cgr_version() -> int:
    return int(library().cgr_version())


def cgr_rope_tables(max_pos: int, head_dim: int, base: float,
                    device=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """cos, sin float32 [max_pos, head_dim/2] of p * base^(-2i/head_dim) (see include/cgr.h)."""
    lib = library()
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    half = max(head_dim // 2, 1)
    cos = torch.empty((max(max_pos, 1), half), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    with torch.cuda.device(device):
        _check(lib.cgr_rope_tables(int(max_pos), int(head_dim), float(base), _ptr(cos), _ptr(sin),
                                   _stream(device)))
    return cos, sin


def _dense_fwd_args(q, k, v, rope_cos, rope_sin, causal, rope_style, window, softmax_scale, qk_operand, out, lse,
                    return_lse, seqlens):
    """Checks and the C argument list (without workspace and stream) of a dense forward call."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, k, v must be 4-D [B, T, heads, head_dim]")
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise CgrError(CGR_ERR_INVALID_ARG, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise CgrError(CGR_ERR_UNSUPPORTED, "q, k, v must all be float32 or all bfloat16")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, q.dtype)
    if out.shape != q.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev_tensor("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, H, T):
            raise CgrError(CGR_ERR_INVALID_ARG, "lse must be [B, H, T]")
    if seqlens is not None:
        _dev_tensor("seqlens", seqlens, torch.int32)
        if tuple(seqlens.shape) != (B,):
            raise CgrError(CGR_ERR_INVALID_ARG, "seqlens must be [B]")
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T, H, k.shape[2], D, _DTYPES[q.dtype],
            _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], _STYLES[rope_style],
            CGR_MASK_CAUSAL if causal else CGR_MASK_NONE, int(window),
            0.0 if softmax_scale is None else float(softmax_scale), _QK[qk_operand], _ptr(seqlens)]
    return args, out, lse


def cgr_gqa_rope_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rope_cos: torch.Tensor,
                          rope_sin: torch.Tensor, *, causal: bool = True, rope_style: str = "interleaved",
                          window: int = 0, softmax_scale: Optional[float] = None, qk_operand: str = "f16",
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_lse: bool = True, workspace=None, seqlens: Optional[torch.Tensor] = None):
    """Dense forward: q [B,T,H,d], k/v [B,T,KV,d] -> (o [B,T,H,d], lse [B,H,T] float32 or None).

    workspace: None allocates one (bf16 I/O: the keys are then rotated once up
    front), a uint8 device tensor of cgr_attn_fwd_workspace_size bytes is used
    as given, and False passes none (the keys are rotated on every tile).
    seqlens: optional int32 device tensor [B] of valid tokens per entry (right
    padding): keys past them are hidden, rows past them are left unwritten.
    """
    lib = library()
    args, out, lse = _dense_fwd_args(q, k, v, rope_cos, rope_sin, causal, rope_style, window, softmax_scale,
                                     qk_operand, out, lse, return_lse, seqlens)
    B, T, _, D = q.shape
    if workspace is None and q.dtype == torch.bfloat16:
        workspace = torch.empty(int(lib.cgr_attn_fwd_workspace_size(B, T, k.shape[2], D)), dtype=torch.uint8,
                                device=q.device)
    if workspace is False or workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        _dev_tensor("workspace", workspace)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_fwd(*args, ws_ptr, ws_bytes, _stream(q.device)))
    return out, lse


def cgr_attn_fwd_rotate_keys(k: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                             workspace: torch.Tensor, *, rope_style: str = "interleaved", qk_operand: str = "f16",
                             seqlens: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The first half of a dense bf16 forward: k [B,T,KV,d] rotated once into `workspace`
    (uint8, cgr_attn_fwd_workspace_size bytes). Returns the workspace."""
    lib = library()
    _dev_tensor("k", k, torch.bfloat16)
    _dev_tensor("workspace", workspace)
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if k.dim() != 4:
        raise CgrError(CGR_ERR_INVALID_ARG, "k must be 4-D [B, T, n_kv_head, head_dim]")
    B, T, KV, D = k.shape
    if seqlens is not None:
        _dev_tensor("seqlens", seqlens, torch.int32)
    with torch.cuda.device(k.device):
        _check(lib.cgr_attn_fwd_rotate_keys(
            _ptr(k), B, T, KV, D, CGR_BF16, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], _STYLES[rope_style],
            _QK[qk_operand], _ptr(seqlens), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(k.device)))
    return workspace


def cgr_gqa_rope_attn_fwd_rotated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rope_cos: torch.Tensor,
                                  rope_sin: torch.Tensor, workspace: torch.Tensor, *, causal: bool = True,
                                  rope_style: str = "interleaved", window: int = 0,
                                  softmax_scale: Optional[float] = None, qk_operand: str = "f16",
                                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                  return_lse: bool = True, seqlens: Optional[torch.Tensor] = None):
    """The second half of a dense bf16 forward: attention over the keys that
    cgr_attn_fwd_rotate_keys left in `workspace` (same k, tables, style, operand, seqlens)."""
    lib = library()
    args, out, lse = _dense_fwd_args(q, k, v, rope_cos, rope_sin, causal, rope_style, window, softmax_scale,
                                     qk_operand, out, lse, return_lse, seqlens)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_fwd_rotated(*args, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _stream(q.device)))
    return out, lse


def cgr_attn_fwd_fp8_workspace_size(B: int, T: int, n_kv_head: int, head_dim: int) -> int:
    return int(library().cgr_attn_fwd_fp8_workspace_size(int(B), int(T), int(n_kv_head), int(head_dim)))


def cgr_gqa_rope_attn_fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_descale: float, k_descale: float,
                              v_descale: float, rope_cos: torch.Tensor, rope_sin: torch.Tensor, *,
                              causal: bool = True, rope_style: str = "interleaved",
                              softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, return_lse: bool = True, workspace=None,
                              seqlens: Optional[torch.Tensor] = None):
    """fp8 forward: q [B,T,H,128], k/v [B,T,KV,128] as torch.float8_e4m3fn (the real inputs are the
    codes times the descales) -> (o [B,T,H,128] bfloat16, lse [B,H,T] float32 or None).
    seqlens: optional int32 [B] device tensor of valid tokens per entry (right padding)."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, torch.float8_e4m3fn)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, k, v must be 4-D [B, T, heads, head_dim]")
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise CgrError(CGR_ERR_INVALID_ARG, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _dev_tensor("out", out, torch.bfloat16)
    if out.shape != q.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev_tensor("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, H, T):
            raise CgrError(CGR_ERR_INVALID_ARG, "lse must be [B, H, T]")
    if seqlens is not None:
        _dev_tensor("seqlens", seqlens, torch.int32)
        if seqlens.numel() != B:
            raise CgrError(CGR_ERR_INVALID_ARG, "seqlens must hold B entries")
    if workspace is None:
        workspace = torch.empty(max(16, int(lib.cgr_attn_fwd_fp8_workspace_size(B, T, k.shape[2], D))),
                                dtype=torch.uint8, device=q.device)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_fwd_fp8(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T, H, k.shape[2], D, float(q_descale),
            float(k_descale), float(v_descale), _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
            _STYLES[rope_style], CGR_MASK_CAUSAL if causal else CGR_MASK_NONE,
            0.0 if softmax_scale is None else float(softmax_scale), _ptr(seqlens), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out, lse


def cgr_attn_fwd_workspace_size(B: int, T: int, n_kv_head: int, head_dim: int) -> int:
    return int(library().cgr_attn_fwd_workspace_size(int(B), int(T), int(n_kv_head), int(head_dim)))


def cgr_attn_fwd_varlen_workspace_size(num_seqs: int, total_tokens: int) -> int:
    return int(library().cgr_attn_fwd_varlen_workspace_size(int(num_seqs), int(total_tokens)))


def cgr_attn_fwd_varlen_rotated_workspace_size(num_seqs: int, total_tokens: int, n_kv_head: int,
                                               head_dim: int) -> int:
    return int(library().cgr_attn_fwd_varlen_rotated_workspace_size(int(num_seqs), int(total_tokens),
                                                                     int(n_kv_head), int(head_dim)))


def cgr_gqa_rope_attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                 cu_seqlens: torch.Tensor, max_seqlen: int, rope_cos: torch.Tensor,
                                 rope_sin: torch.Tensor, *, causal: bool = True,
                                 rope_style: str = "interleaved", window: int = 0,
                                 softmax_scale: Optional[float] = None,
                                 qk_operand: str = "f16", out: Optional[torch.Tensor] = None,
                                 lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                                 workspace: Optional[torch.Tensor] = None, rotate_keys_once: bool = True):
    """Packed forward: q [total,H,d], k/v [total,KV,d], cu_seqlens int32 [n+1] (device).

    Without a workspace one is allocated: for bf16 with room for the once-rotated
    keys unless rotate_keys_once is False (then K is rotated per tile).
    Returns (o [total,H,d], lse [H,total] float32 or None).
    """
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, k, v must be 3-D [total, heads, head_dim]")
    total, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != total or k.shape[2] != D:
        raise CgrError(CGR_ERR_INVALID_ARG, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise CgrError(CGR_ERR_UNSUPPORTED, "q, k, v must all be float32 or all bfloat16")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    nseq = cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, q.dtype)
    if lse is None and return_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev_tensor("lse", lse, torch.float32)
    need = lib.cgr_attn_fwd_varlen_workspace_size(max(nseq, 1), total)
    if rotate_keys_once and q.dtype == torch.bfloat16:
        need = max(need, lib.cgr_attn_fwd_varlen_rotated_workspace_size(max(nseq, 1), total, k.shape[1], D))
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=q.device)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_fwd_varlen(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), nseq, total,
            int(max_seqlen), H, k.shape[1], D, _DTYPES[q.dtype], _ptr(rope_cos), _ptr(rope_sin),
            rope_cos.shape[0], _STYLES[rope_style], CGR_MASK_CAUSAL if causal else CGR_MASK_NONE,
            int(window), 0.0 if softmax_scale is None else float(softmax_scale), _QK[qk_operand],
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out, lse


def cgr_gqa_rope_attn_fwd_varlen_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                         cu_seqlens: torch.Tensor, max_seqlen: int, rope_cos: torch.Tensor,
                                         rope_sin: torch.Tensor, *, out: torch.Tensor, lse: Optional[torch.Tensor],
                                         causal: bool = True, rope_style: str = "interleaved", window: int = 0,
                                         softmax_scale: Optional[float] = None, qk_operand: str = "f16",
                                         device_status: Optional[torch.Tensor] = None):
    """The packed forward that allocates nothing (its schedule lives in the
    library's own device array): the caller passes out [total,H,d], lse [H,total]
    float32 (or None) and optionally device_status (int32 device tensor [1])."""
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, k, v must be 3-D [total, heads, head_dim]")
    total, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != total or k.shape[2] != D:
        raise CgrError(CGR_ERR_INVALID_ARG, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise CgrError(CGR_ERR_UNSUPPORTED, "q, k, v must all be float32 or all bfloat16")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    _dev_tensor("out", out, q.dtype)
    if lse is not None:
        _dev_tensor("lse", lse, torch.float32)
    if device_status is not None:
        _dev_tensor("device_status", device_status, torch.int32)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_fwd_varlen_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), cu_seqlens.numel() - 1, total,
            int(max_seqlen), H, k.shape[1], D, _DTYPES[q.dtype], _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
            _STYLES[rope_style], CGR_MASK_CAUSAL if causal else CGR_MASK_NONE, int(window),
            0.0 if softmax_scale is None else float(softmax_scale), _QK[qk_operand], _ptr(device_status),
            _stream(q.device)))
    return out, lse


def cgr_varlen_device_status(workspace: torch.Tensor) -> int:
    """Device error word of the last varlen call on `workspace` (0 = well formed). Synchronises."""
    lib = library()
    st = ctypes.c_int32(-1)
    with torch.cuda.device(workspace.device):
        _check(lib.cgr_varlen_device_status(_ptr(workspace), _stream(workspace.device), ctypes.byref(st)))
    return int(st.value)


def cgr_attn_bwd_workspace_size(B: int, T: int, n_head: int, n_kv_head: int, head_dim: int) -> int:
    return int(library().cgr_attn_bwd_workspace_size(int(B), int(T), int(n_head), int(n_kv_head),
                                                      int(head_dim)))


def cgr_gqa_rope_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                          lse: torch.Tensor, dout: torch.Tensor, rope_cos: torch.Tensor,
                          rope_sin: torch.Tensor, *, causal: bool = True, rope_style: str = "interleaved",
                          window: int = 0, softmax_scale: Optional[float] = None, qk_operand: str = "f16",
                          dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                          dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Dense backward: the forward's q, k, v, o [B,T,.,d], lse [B,H,T] and dL/dO -> (dq, dk, dv).

    Every argument that the forward also takes must be the same as in that
    forward call (bf16 tensors only).
    """
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev_tensor(n, t, torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, k, v must be 4-D [B, T, heads, head_dim]")
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise CgrError(CGR_ERR_INVALID_ARG, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if o.shape != q.shape or dout.shape != q.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "o and dout must have q's shape")
    _dev_tensor("lse", lse, torch.float32)
    if tuple(lse.shape) != (B, H, T):
        raise CgrError(CGR_ERR_INVALID_ARG, "lse must be [B, H, T]")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _dev_tensor(n, t, torch.bfloat16)
        if t.shape != ref.shape:
            raise CgrError(CGR_ERR_INVALID_ARG, f"{n} must have shape {tuple(ref.shape)}")
    need = lib.cgr_attn_bwd_workspace_size(B, T, H, k.shape[2], D)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=q.device)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            B, T, H, k.shape[2], D, CGR_BF16, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
            _STYLES[rope_style], CGR_MASK_CAUSAL if causal else CGR_MASK_NONE, int(window),
            0.0 if softmax_scale is None else float(softmax_scale), _QK[qk_operand],
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


def cgr_attn_bwd_varlen_workspace_size(num_seqs: int, total_tokens: int, n_head: int, n_kv_head: int,
                                       head_dim: int) -> int:
    return int(library().cgr_attn_bwd_varlen_workspace_size(int(num_seqs), int(total_tokens), int(n_head),
                                                             int(n_kv_head), int(head_dim)))


def cgr_gqa_rope_attn_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                                 lse: torch.Tensor, dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                                 rope_cos: torch.Tensor, rope_sin: torch.Tensor, *, causal: bool = True,
                                 rope_style: str = "interleaved", window: int = 0,
                                 softmax_scale: Optional[float] = None, qk_operand: str = "f16",
                                 dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                                 dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Packed backward: the packed forward's q, k, v, o [total,.,d], lse [H,total],
    cu_seqlens and dL/dO -> (dq, dk, dv).

    Every argument that the forward also takes must be the same as in that
    forward call (bf16 tensors only).
    """
    lib = library()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev_tensor(n, t, torch.bfloat16)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, k, v must be 3-D [total, heads, head_dim]")
    total, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != total or k.shape[2] != D:
        raise CgrError(CGR_ERR_INVALID_ARG, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if o.shape != q.shape or dout.shape != q.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "o and dout must have q's shape")
    _dev_tensor("lse", lse, torch.float32)
    if tuple(lse.shape) != (H, total):
        raise CgrError(CGR_ERR_INVALID_ARG, "lse must be [H, total]")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    nseq = cu_seqlens.numel() - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _dev_tensor(n, t, torch.bfloat16)
        if t.shape != ref.shape:
            raise CgrError(CGR_ERR_INVALID_ARG, f"{n} must have shape {tuple(ref.shape)}")
    need = lib.cgr_attn_bwd_varlen_workspace_size(max(nseq, 1), total, H, k.shape[1], D)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=q.device)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_bwd_varlen(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(cu_seqlens), nseq, total, int(max_seqlen), H, k.shape[1], D, CGR_BF16, _ptr(rope_cos),
            _ptr(rope_sin), rope_cos.shape[0], _STYLES[rope_style], CGR_MASK_CAUSAL if causal else CGR_MASK_NONE,
            int(window), 0.0 if softmax_scale is None else float(softmax_scale), _QK[qk_operand],
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


def cgr_rope_rotate(x: torch.Tensor, positions: torch.Tensor, rope_cos: torch.Tensor,
                    rope_sin: torch.Tensor, *, rope_style: str = "interleaved",
                    out: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None):
    """out[t, h] = R(positions[t]) x[t, h] for x [N, n_heads, d] (bf16 or f32); out may be x."""
    lib = library()
    _dev_tensor("x", x)
    if x.dim() != 3:
        raise CgrError(CGR_ERR_INVALID_ARG, "x must be [n_tokens, n_heads, head_dim]")
    if x.dtype not in _DTYPES:
        raise CgrError(CGR_ERR_UNSUPPORTED, "x must be float32 or bfloat16")
    _dev_tensor("positions", positions, torch.int32)
    if positions.numel() != x.shape[0]:
        raise CgrError(CGR_ERR_INVALID_ARG, "positions must have one entry per token")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != x.shape[2] // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    out = torch.empty_like(x) if out is None else out
    _dev_tensor("out", out, x.dtype)
    if out.shape != x.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "out must have x's shape")
    if status is not None:
        _dev_tensor("status", status, torch.int32)
    with torch.cuda.device(x.device):
        _check(lib.cgr_rope_rotate(_ptr(x), _ptr(out), _ptr(positions), x.shape[0], x.shape[1], x.shape[2],
                                   _DTYPES[x.dtype], _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
                                   _STYLES[rope_style], _ptr(status), _stream(x.device)))
    return out


def cgr_attn_decode_workspace_size(B: int, Tq: int, max_seqlen: int, n_head: int, n_kv_head: int,
                                   head_dim: int) -> int:
    return int(library().cgr_attn_decode_workspace_size(int(B), int(Tq), int(max_seqlen), int(n_head),
                                                        int(n_kv_head), int(head_dim)))


def cgr_gqa_rope_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             cache_seqlens: torch.Tensor, max_seqlen: int, rope_cos: torch.Tensor,
                             rope_sin: torch.Tensor, *, rope_style: str = "interleaved", window: int = 0,
                             softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                             workspace: Optional[torch.Tensor] = None):
    """Decode: q [B,Tq,H,d] against caches k/v indexed [B,S,KV,d] (keys rotated) with
    lengths cache_seqlens int32 [B] (device). The caches may be strided views (a
    head-major [B,KV,S,d] buffer viewed as [B,S,KV,d] with .transpose(1, 2)), with
    head_dim contiguous and the same strides for k and v.
    Returns (o [B,Tq,H,d], lse [B,H,Tq] float32 or None)."""
    lib = library()
    _dev_tensor("q", q, torch.bfloat16)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.bfloat16:
            raise CgrError(CGR_ERR_INVALID_ARG, f"{n} must be a bfloat16 CUDA/HIP tensor")
        if t.dim() != 4 or t.stride(3) != 1:
            raise CgrError(CGR_ERR_INVALID_ARG, f"{n} must be 4-D [B,S,KV,d] with head_dim contiguous")
    if k_cache.stride() != v_cache.stride() or v_cache.shape != k_cache.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "k_cache and v_cache must share shape and strides")
    _dev_tensor("cache_seqlens", cache_seqlens, torch.int32)
    if q.dim() != 4:
        raise CgrError(CGR_ERR_INVALID_ARG, "q must be [B,Tq,H,d]")
    B, Tq, H, D = q.shape
    S, KV = k_cache.shape[1], k_cache.shape[2]
    sb, st, sh = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    if k_cache.shape[0] != B or k_cache.shape[3] != D or cache_seqlens.numel() != B:
        raise CgrError(CGR_ERR_INVALID_ARG, "q, caches and cache_seqlens disagree on B or head_dim")
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    out = torch.empty_like(q) if out is None else out
    _dev_tensor("out", out, torch.bfloat16)
    if out.shape != q.shape:
        raise CgrError(CGR_ERR_INVALID_ARG, "out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev_tensor("lse", lse, torch.float32)
    need = lib.cgr_attn_decode_workspace_size(B, Tq, int(max_seqlen), H, KV, D)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=q.device)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(q.device):
        _check(lib.cgr_gqa_rope_attn_decode(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(out), _ptr(lse), B, Tq, S,
            sb, st, sh, int(max_seqlen), H, KV, D, CGR_BF16, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
            _STYLES[rope_style], int(window), 0.0 if softmax_scale is None else float(softmax_scale),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out, lse


def cgr_rmsnorm_qkv_rope_workspace_size(n_tokens: int, n_embd: int, n_head: int, n_kv_head: int,
                                        head_dim: int) -> int:
    return int(library().cgr_rmsnorm_qkv_rope_workspace_size(int(n_tokens), int(n_embd), int(n_head),
                                                             int(n_kv_head), int(head_dim)))


def cgr_rmsnorm_qkv_rope(x: torch.Tensor, norm_weight: torch.Tensor, eps: float, w_qkv: torch.Tensor,
                         positions: torch.Tensor, n_head: int, n_kv_head: int, rope_cos: torch.Tensor,
                         rope_sin: torch.Tensor, *, rope_style: str = "interleaved", rotate_q: bool = True,
                         rotate_k: bool = True, q: Optional[torch.Tensor] = None,
                         k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """x [N, C] (bf16), norm_weight [C], w_qkv [(H + 2 KV) d, C], positions int32 [N] (device)
    -> q [N, H, d], k [N, KV, d], v [N, KV, d]: RMSNorm, projections, RoPE on q and/or k."""
    lib = library()
    for n, tns in (("x", x), ("norm_weight", norm_weight), ("w_qkv", w_qkv)):
        _dev_tensor(n, tns, torch.bfloat16)
    _dev_tensor("positions", positions, torch.int32)
    if x.dim() != 2 or norm_weight.dim() != 1 or w_qkv.dim() != 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "x must be [N, C], norm_weight [C], w_qkv [O, C]")
    N, C = x.shape
    O = w_qkv.shape[0]
    if norm_weight.shape[0] != C or w_qkv.shape[1] != C or positions.numel() != N:
        raise CgrError(CGR_ERR_INVALID_ARG, "x, norm_weight, w_qkv and positions disagree on sizes")
    heads = int(n_head) + 2 * int(n_kv_head)
    if O % heads:
        raise CgrError(CGR_ERR_INVALID_ARG, "w_qkv rows must be (n_head + 2 n_kv_head) * head_dim")
    D = O // heads
    _dev_tensor("rope_cos", rope_cos, torch.float32)
    _dev_tensor("rope_sin", rope_sin, torch.float32)
    if rope_cos.shape != rope_sin.shape or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2:
        raise CgrError(CGR_ERR_INVALID_ARG, "rope tables must be [max_pos, head_dim/2]")
    q = torch.empty((N, n_head, D), dtype=torch.bfloat16, device=x.device) if q is None else q
    k = torch.empty((N, n_kv_head, D), dtype=torch.bfloat16, device=x.device) if k is None else k
    v = torch.empty((N, n_kv_head, D), dtype=torch.bfloat16, device=x.device) if v is None else v
    for n, tns, shp in (("q", q, (N, n_head, D)), ("k", k, (N, n_kv_head, D)), ("v", v, (N, n_kv_head, D))):
        _dev_tensor(n, tns, torch.bfloat16)
        if tuple(tns.shape) != shp:
            raise CgrError(CGR_ERR_INVALID_ARG, f"{n} must have shape {shp}")
    need = lib.cgr_rmsnorm_qkv_rope_workspace_size(N, C, int(n_head), int(n_kv_head), D)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=x.device)
    _dev_tensor("workspace", workspace)
    with torch.cuda.device(x.device):
        _check(lib.cgr_rmsnorm_qkv_rope(
            _ptr(x), _ptr(norm_weight), float(eps), _ptr(w_qkv), _ptr(positions), _ptr(q), _ptr(k), _ptr(v),
            N, C, int(n_head), int(n_kv_head), D, CGR_BF16, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
            _STYLES[rope_style], int(bool(rotate_q)) | (int(bool(rotate_k)) << 1), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(x.device)))
    return q, k, v


rope_tables = cgr_rope_tables
gqa_rope_attn_fwd = cgr_gqa_rope_attn_fwd
attn_fwd_rotate_keys = cgr_attn_fwd_rotate_keys
gqa_rope_attn_fwd_rotated = cgr_gqa_rope_attn_fwd_rotated
gqa_rope_attn_fwd_fp8 = cgr_gqa_rope_attn_fwd_fp8
gqa_rope_attn_fwd_varlen = cgr_gqa_rope_attn_fwd_varlen
gqa_rope_attn_fwd_varlen_noalloc = cgr_gqa_rope_attn_fwd_varlen_noalloc
gqa_rope_attn_bwd = cgr_gqa_rope_attn_bwd
gqa_rope_attn_bwd_varlen = cgr_gqa_rope_attn_bwd_varlen
rope_rotate = cgr_rope_rotate
gqa_rope_attn_decode = cgr_gqa_rope_attn_decode
rmsnorm_qkv_rope = cgr_rmsnorm_qkv_rope
