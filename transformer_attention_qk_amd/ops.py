"""PyTorch-facing binding of libattn: tensors in, tensors out.

PyTorch provides device memory and the current HIP stream; every computation runs in the HIP
kernels behind the C ABI (include/attn.h). These wrappers only check tensor properties, allocate
outputs and pass raw pointers.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.ATTN_BF16, torch.float32: _lib.ATTN_F32}


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, name: str, shape=None, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def sssl_windows(T: int, n_layer: int, pattern: str = "SSSL") -> list[int]:
    """Per-layer windows of a layer pattern (host-only C call)."""
    lib = _lib.load()
    buf = (ctypes.c_int * max(n_layer, 1))()
    _lib.check("attn_sssl_windows", lib.attn_sssl_windows(T, n_layer, pattern.encode(), buf))
    return list(buf[:n_layer])


def rope_table(T: int, d: int, base: float = 10000.0, device=None) -> tuple[torch.Tensor, torch.Tensor]:
    """fp32 [T, d/2] cos and sin tables of the rotary embedding, computed on the GPU."""
    lib = _lib.load()
    device = device or torch.device("cuda", torch.cuda.current_device())
    cos = torch.empty((T, d // 2), dtype=torch.float32, device=device)
    sin = torch.empty((T, d // 2), dtype=torch.float32, device=device)
    _lib.check("attn_rope_table", lib.attn_rope_table(_ptr(cos), _ptr(sin), T, d, float(base),
                                                      _stream_handle()))
    return cos, sin


def qknorm_rope(q: torch.Tensor | None, k: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                eps: float = 1e-6, q_out: torch.Tensor | None = None,
                k_out: torch.Tensor | None = None):
    """QK-RMSNorm + RoPE of q, k [B, H, T, d]; outputs may be q, k themselves (in place).
    With q None only k is processed (the returned q_out is None)."""
    lib = _lib.load()
    _require(k, "k")
    if k.dim() != 4 or k.dtype not in _DTYPES:
        raise ValueError("k must be [B, H, T, d] bf16 or fp32")
    B, H, T, d = k.shape
    if q is not None:
        _require(q, "q", k.shape, k.dtype)
    _require(cos, "cos", (cos.shape[0], d // 2), torch.float32)
    _require(sin, "sin", cos.shape, torch.float32)
    if cos.shape[0] < T:
        raise ValueError("rope tables are shorter than the sequence")
    if q is not None:
        q_out = torch.empty_like(q) if q_out is None else q_out
        _require(q_out, "q_out", k.shape, k.dtype)
    else:
        q_out = None
    k_out = torch.empty_like(k) if k_out is None else k_out
    _require(k_out, "k_out", k.shape, k.dtype)
    rc = lib.attn_qknorm_rope(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(cos), _ptr(sin),
                              B, H, T, d, float(eps), _DTYPES[k.dtype], _stream_handle())
    _lib.check("attn_qknorm_rope", rc)
    return q_out, k_out


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int = -1,
             causal: bool = True, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, want_lse: bool = True):
    """softmax(q k^T / sqrt(d) + mask) v and its logsumexp for [B, H, T, d] tensors.

    Returns (out, lse); lse is fp32 [B, H, T] (None when want_lse is False and none was given).
    """
    lib = _lib.load()
    _require(q, "q")
    if q.dim() != 4 or q.dtype not in _DTYPES:
        raise ValueError("q must be [B, H, T, d] bf16 or fp32")
    B, H, T, d = q.shape
    _require(k, "k", q.shape, q.dtype)
    _require(v, "v", q.shape, q.dtype)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", (B, H, T), torch.float32)
    rc = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, T, d, int(window),
                      int(bool(causal)), _DTYPES[q.dtype], _stream_handle())
    _lib.check("attn_fwd", rc)
    return out, lse


def attn_fwd_qnorm(q: torch.Tensor, kn: torch.Tensor, v: torch.Tensor, cos: torch.Tensor,
                   sin: torch.Tensor, window: int = -1, causal: bool = True, eps: float = 1e-6,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   want_lse: bool = True):
    """Attention of raw bf16 q (normalised and rotated inside the kernel) against already
    normalised and rotated keys kn. Returns (out, lse)."""
    lib = _lib.load()
    _require(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    _require(kn, "kn", q.shape, q.dtype)
    _require(v, "v", q.shape, q.dtype)
    _require(cos, "cos", (cos.shape[0], d // 2), torch.float32)
    _require(sin, "sin", cos.shape, torch.float32)
    if cos.shape[0] < T:
        raise ValueError("rope tables are shorter than the sequence")
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", (B, H, T), torch.float32)
    rc = lib.attn_fwd_qnorm(_ptr(q), _ptr(kn), _ptr(v), _ptr(out), _ptr(lse), _ptr(cos),
                            _ptr(sin), B, H, T, d, float(eps), int(window), int(bool(causal)),
                            _lib.ATTN_BF16, _stream_handle())
    _lib.check("attn_fwd_qnorm", rc)
    return out, lse


def attn_fwd_qknorm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cos: torch.Tensor,
                    sin: torch.Tensor, window: int = -1, causal: bool = True, eps: float = 1e-6,
                    k_work: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, want_lse: bool = True):
    """QK-norm + RoPE of raw bf16 q, k and attention in one library call.

    Returns (out, lse, k_work); k_work holds RoPE(RMSNorm(k)) (it may be ``k`` itself).
    """
    lib = _lib.load()
    _require(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    _require(k, "k", q.shape, q.dtype)
    _require(v, "v", q.shape, q.dtype)
    _require(cos, "cos", (cos.shape[0], d // 2), torch.float32)
    _require(sin, "sin", cos.shape, torch.float32)
    if cos.shape[0] < T:
        raise ValueError("rope tables are shorter than the sequence")
    k_work = torch.empty_like(k) if k_work is None else k_work
    _require(k_work, "k_work", q.shape, q.dtype)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", (B, H, T), torch.float32)
    rc = lib.attn_fwd_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(k_work), _ptr(out), _ptr(lse),
                             _ptr(cos), _ptr(sin), B, H, T, d, float(eps), int(window),
                             int(bool(causal)), _lib.ATTN_BF16, _stream_handle())
    _lib.check("attn_fwd_qknorm", rc)
    return out, lse, k_work


def attention_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cos: torch.Tensor,
                    sin: torch.Tensor, window: int = -1, eps: float = 1e-6,
                    qn: torch.Tensor | None = None, kn: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """One attention layer: QK-norm + RoPE of raw q, k, then causal attention with ``window``
    (two calls: attn_qknorm_rope writes the normalised q and k, attn_fwd reads them)."""
    qn, kn = qknorm_rope(q, k, cos, sin, eps, qn, kn)
    return attn_fwd(qn, kn, v, window=window, causal=True, out=out, lse=lse)
