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
_LAYOUTS = {"bhtd": _lib.ATTN_LAYOUT_BHTD, "bthd": _lib.ATTN_LAYOUT_BTHD}


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


def _geometry(q: torch.Tensor | None, k: torch.Tensor, layout: str):
    """(B, H, H_kv, T, d) of q and k stored as [B, H, T, d] ("bhtd") or [B, T, H, d] ("bthd");
    k (and v) may have fewer heads than q (grouped-query attention)."""
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}, got {layout!r}")
    if k.dim() != 4 or (q is not None and q.dim() != 4):
        raise ValueError("q and k must be 4-d tensors")
    if layout == "bhtd":
        B, H_kv, T, d = k.shape
        H = q.shape[1] if q is not None else H_kv
    else:
        B, T, H_kv, d = k.shape
        H = q.shape[2] if q is not None else H_kv
    if q is not None:
        want = (B, H, T, d) if layout == "bhtd" else (B, T, H, d)
        if tuple(q.shape) != want:
            raise ValueError(f"q has shape {tuple(q.shape)}, k {tuple(k.shape)}: they differ in "
                             "more than the head count")
        if H % H_kv != 0:
            raise ValueError(f"k's head count {H_kv} must divide q's {H}")
    return B, H, H_kv, T, d


def _rope_tables(cos: torch.Tensor, sin: torch.Tensor, T: int, d: int) -> None:
    _require(cos, "cos", (cos.shape[0], d // 2), torch.float32)
    _require(sin, "sin", cos.shape, torch.float32)
    if cos.shape[0] < T:
        raise ValueError("rope tables are shorter than the sequence")


def _lse(lse: torch.Tensor | None, want: bool, B: int, H: int, T: int, device):
    if lse is None and want:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=device)
    if lse is not None:
        _require(lse, "lse", (B, H, T), torch.float32)
    return lse


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
                k_out: torch.Tensor | None = None, layout: str = "bhtd"):
    """QK-RMSNorm + RoPE of q [B, H, T, d] and k [B, H_kv, T, d] (or [B, T, H, d] and
    [B, T, H_kv, d] with layout "bthd"); outputs may be q, k themselves (in place).
    With q None only k is processed (the returned q_out is None)."""
    lib = _lib.load()
    _require(k, "k")
    if k.dtype not in _DTYPES:
        raise ValueError("k must be bf16 or fp32")
    if q is not None:
        _require(q, "q", dtype=k.dtype)
    B, H, H_kv, T, d = _geometry(q, k, layout)
    _rope_tables(cos, sin, T, d)
    if q is not None:
        q_out = torch.empty_like(q) if q_out is None else q_out
        _require(q_out, "q_out", q.shape, q.dtype)
    else:
        q_out = None
    k_out = torch.empty_like(k) if k_out is None else k_out
    _require(k_out, "k_out", k.shape, k.dtype)
    rc = lib.attn_qknorm_rope_ex(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(cos), _ptr(sin),
                                 B, H, H_kv, T, d, _LAYOUTS[layout], float(eps), _DTYPES[k.dtype],
                                 _stream_handle())
    _lib.check("attn_qknorm_rope_ex", rc)
    return q_out, k_out


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int = -1,
             causal: bool = True, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, want_lse: bool = True, layout: str = "bhtd"):
    """softmax(q k^T / sqrt(d) + mask) v and its logsumexp. q is [B, H, T, d], k and v
    [B, H_kv, T, d] with H_kv dividing H (or [B, T, heads, d] with layout "bthd").

    Returns (out, lse); out has q's shape, lse is fp32 [B, H, T] (None when want_lse is False
    and none was given).
    """
    lib = _lib.load()
    _require(q, "q")
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bf16 or fp32")
    _require(k, "k", dtype=q.dtype)
    B, H, H_kv, T, d = _geometry(q, k, layout)
    _require(v, "v", k.shape, q.dtype)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    lse = _lse(lse, want_lse, B, H, T, q.device)
    rc = lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, H_kv, T, d,
                         _LAYOUTS[layout], int(window), int(bool(causal)), _DTYPES[q.dtype],
                         _stream_handle())
    _lib.check("attn_fwd_ex", rc)
    return out, lse


def attn_fwd_qnorm(q: torch.Tensor, kn: torch.Tensor, v: torch.Tensor, cos: torch.Tensor,
                   sin: torch.Tensor, window: int = -1, causal: bool = True, eps: float = 1e-6,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   want_lse: bool = True, layout: str = "bhtd"):
    """Attention of raw bf16 q (normalised and rotated inside the kernel) against already
    normalised and rotated keys kn. Shapes as in attn_fwd. Returns (out, lse)."""
    lib = _lib.load()
    _require(q, "q", dtype=torch.bfloat16)
    _require(kn, "kn", dtype=q.dtype)
    B, H, H_kv, T, d = _geometry(q, kn, layout)
    _require(v, "v", kn.shape, q.dtype)
    _rope_tables(cos, sin, T, d)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    lse = _lse(lse, want_lse, B, H, T, q.device)
    rc = lib.attn_fwd_qnorm_ex(_ptr(q), _ptr(kn), _ptr(v), _ptr(out), _ptr(lse), _ptr(cos),
                               _ptr(sin), B, H, H_kv, T, d, _LAYOUTS[layout], float(eps),
                               int(window), int(bool(causal)), _lib.ATTN_BF16, _stream_handle())
    _lib.check("attn_fwd_qnorm_ex", rc)
    return out, lse


def attn_fwd_qknorm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cos: torch.Tensor,
                    sin: torch.Tensor, window: int = -1, causal: bool = True, eps: float = 1e-6,
                    k_work: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, want_lse: bool = True,
                    layout: str = "bhtd", write_k: bool = True):
    """QK-norm + RoPE of raw bf16 q, k and attention in one library call. Shapes as in attn_fwd.

    Returns (out, lse, k_work); k_work holds RoPE(RMSNorm(k)) (it may be ``k`` itself). With
    write_k False (d 32 or 64) the keys are normalised inside the attention kernel, nothing is
    written for them and k_work is returned as None.
    """
    lib = _lib.load()
    _require(q, "q", dtype=torch.bfloat16)
    _require(k, "k", dtype=q.dtype)
    B, H, H_kv, T, d = _geometry(q, k, layout)
    _require(v, "v", k.shape, q.dtype)
    _rope_tables(cos, sin, T, d)
    if write_k:
        k_work = torch.empty_like(k) if k_work is None else k_work
        _require(k_work, "k_work", k.shape, q.dtype)
    elif k_work is not None:
        raise ValueError("k_work is not written when write_k is False")
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    lse = _lse(lse, want_lse, B, H, T, q.device)
    rc = lib.attn_fwd_qknorm_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(k_work), _ptr(out), _ptr(lse),
                                _ptr(cos), _ptr(sin), B, H, H_kv, T, d, _LAYOUTS[layout],
                                float(eps), int(window), int(bool(causal)), _lib.ATTN_BF16,
                                _stream_handle())
    _lib.check("attn_fwd_qknorm_ex", rc)
    return out, lse, k_work


def attention_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cos: torch.Tensor,
                    sin: torch.Tensor, window: int = -1, eps: float = 1e-6,
                    qn: torch.Tensor | None = None, kn: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                    layout: str = "bhtd"):
    """One attention layer: QK-norm + RoPE of raw q, k, then causal attention with ``window``
    (two calls: attn_qknorm_rope_ex writes the normalised q and k, attn_fwd_ex reads them)."""
    qn, kn = qknorm_rope(q, k, cos, sin, eps, qn, kn, layout=layout)
    return attn_fwd(qn, kn, v, window=window, causal=True, out=out, lse=lse, layout=layout)


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
             lse: torch.Tensor, dout: torch.Tensor, window: int = -1, causal: bool = True,
             dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
             dv: torch.Tensor | None = None, delta: torch.Tensor | None = None,
             layout: str = "bhtd"):
    """Gradients (dq, dk, dv) of sum(dout * out) for (out, lse) = attn_fwd(q, k, v, window,
    causal, layout=layout). ``delta`` (fp32 [B, H, T], rowsum(dout * out)) is a by-product."""
    lib = _lib.load()
    _require(q, "q")
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bf16 or fp32")
    _require(k, "k", dtype=q.dtype)
    B, H, H_kv, T, d = _geometry(q, k, layout)
    _require(v, "v", k.shape, q.dtype)
    _require(out, "out", q.shape, q.dtype)
    _require(dout, "dout", q.shape, q.dtype)
    _require(lse, "lse", (B, H, T), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if delta is None else delta
    _require(dq, "dq", q.shape, q.dtype)
    _require(dk, "dk", k.shape, q.dtype)
    _require(dv, "dv", k.shape, q.dtype)
    _require(delta, "delta", (B, H, T), torch.float32)
    rc = lib.attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(delta),
                         _ptr(dq), _ptr(dk), _ptr(dv), B, H, H_kv, T, d, _LAYOUTS[layout],
                         int(window), int(bool(causal)), _DTYPES[q.dtype], _stream_handle())
    _lib.check("attn_bwd_ex", rc)
    return dq, dk, dv


def qknorm_rope_bwd(q: torch.Tensor | None, k: torch.Tensor, dq_in: torch.Tensor | None,
                    dk_in: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, eps: float = 1e-6,
                    dq_out: torch.Tensor | None = None, dk_out: torch.Tensor | None = None,
                    layout: str = "bhtd"):
    """Gradients of the raw q, k of qknorm_rope given the gradients of its outputs; outputs may
    be dq_in, dk_in themselves (in place). With q None only k is processed."""
    lib = _lib.load()
    _require(k, "k")
    if k.dtype not in _DTYPES:
        raise ValueError("k must be bf16 or fp32")
    if (q is None) != (dq_in is None):
        raise ValueError("q and dq_in are given together")
    if q is not None:
        _require(q, "q", dtype=k.dtype)
    B, H, H_kv, T, d = _geometry(q, k, layout)
    _rope_tables(cos, sin, T, d)
    _require(dk_in, "dk_in", k.shape, k.dtype)
    dk_out = torch.empty_like(k) if dk_out is None else dk_out
    _require(dk_out, "dk_out", k.shape, k.dtype)
    if q is not None:
        _require(dq_in, "dq_in", q.shape, q.dtype)
        dq_out = torch.empty_like(q) if dq_out is None else dq_out
        _require(dq_out, "dq_out", q.shape, q.dtype)
    else:
        dq_out = None
    rc = lib.attn_qknorm_rope_bwd_ex(_ptr(q), _ptr(k), _ptr(dq_in), _ptr(dk_in), _ptr(dq_out),
                                     _ptr(dk_out), _ptr(cos), _ptr(sin), B, H, H_kv, T, d,
                                     _LAYOUTS[layout], float(eps), _DTYPES[k.dtype],
                                     _stream_handle())
    _lib.check("attn_qknorm_rope_bwd_ex", rc)
    return dq_out, dk_out


def attention_layer_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                             cos: torch.Tensor, sin: torch.Tensor, window: int = -1,
                             eps: float = 1e-6, layout: str = "bhtd"):
    """Gradients (dq, dk, dv) with respect to the raw q, k, v of one attention layer
    (attention_layer or attn_fwd_qknorm, whose out and lse are passed in): the normalised,
    rotated q and k are recomputed (attn_qknorm_rope_ex), attn_bwd_ex runs on them, and
    attn_qknorm_rope_bwd_ex turns their gradients into those of the raw rows, in place."""
    qn, kn = qknorm_rope(q, k, cos, sin, eps, layout=layout)
    dqn, dkn, dv = attn_bwd(qn, kn, v, out, lse, dout, window=window, causal=True, layout=layout)
    dq, dk = qknorm_rope_bwd(q, k, dqn, dkn, cos, sin, eps, dq_out=dqn, dk_out=dkn, layout=layout)
    return dq, dk, dv


def _gate_shape(v: torch.Tensor, layout: str) -> tuple[int, int, int, int, tuple]:
    """(B, H_kv, T, d, logits shape) of v stored in `layout`."""
    if v.dim() != 4:
        raise ValueError("v must be 4-D")
    if layout == "bhtd":
        B, H_kv, T, d = v.shape
        return B, H_kv, T, d, (B, H_kv, T)
    B, T, H_kv, d = v.shape
    return B, H_kv, T, d, (B, T, H_kv)


def value_gate(v: torch.Tensor, ve: torch.Tensor, gate_logits: torch.Tensor,
               out: torch.Tensor | None = None, layout: str = "bhtd") -> torch.Tensor:
    """v + 2 sigmoid(gate_logits) ve per row (attn_value_gate_ex); out may be v (in place)."""
    lib = _lib.load()
    _require(v, "v")
    if v.dtype not in _DTYPES:
        raise ValueError("v must be bf16 or fp32")
    B, H_kv, T, d, zs = _gate_shape(v, layout)
    _require(ve, "ve", v.shape, v.dtype)
    _require(gate_logits, "gate_logits", zs, v.dtype)
    out = torch.empty_like(v) if out is None else out
    _require(out, "out", v.shape, v.dtype)
    rc = lib.attn_value_gate_ex(_ptr(v), _ptr(ve), _ptr(gate_logits), _ptr(out), B, H_kv, T, d,
                                _LAYOUTS[layout], _DTYPES[v.dtype], _stream_handle())
    _lib.check("attn_value_gate_ex", rc)
    return out


def value_gate_bwd(ve: torch.Tensor, gate_logits: torch.Tensor, dv: torch.Tensor,
                   dve: torch.Tensor | None = None, dgate_logits: torch.Tensor | None = None,
                   layout: str = "bhtd"):
    """(dve, dgate_logits) of the gate given dv, the gradient of the gated rows
    (attn_value_gate_bwd_ex); the gradient of v is dv itself. dve may be dv (in place)."""
    lib = _lib.load()
    _require(dv, "dv")
    if dv.dtype not in _DTYPES:
        raise ValueError("dv must be bf16 or fp32")
    B, H_kv, T, d, zs = _gate_shape(dv, layout)
    _require(ve, "ve", dv.shape, dv.dtype)
    _require(gate_logits, "gate_logits", zs, dv.dtype)
    dve = torch.empty_like(dv) if dve is None else dve
    _require(dve, "dve", dv.shape, dv.dtype)
    dgate_logits = torch.empty_like(gate_logits) if dgate_logits is None else dgate_logits
    _require(dgate_logits, "dgate_logits", zs, dv.dtype)
    rc = lib.attn_value_gate_bwd_ex(_ptr(ve), _ptr(gate_logits), _ptr(dv), _ptr(dve),
                                    _ptr(dgate_logits), B, H_kv, T, d, _LAYOUTS[layout],
                                    _DTYPES[dv.dtype], _stream_handle())
    _lib.check("attn_value_gate_bwd_ex", rc)
    return dve, dgate_logits


def attn_fwd_qknorm_ve(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ve: torch.Tensor,
                       gate_logits: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                       window: int = -1, causal: bool = True, eps: float = 1e-6,
                       k_work: torch.Tensor | None = None, v_work: torch.Tensor | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       want_lse: bool = True, layout: str = "bhtd"):
    """A layer with a value embedding in one library call (attn_fwd_qknorm_ve_ex): QK-norm +
    RoPE of raw bf16 q, k, the gate on v, then attention. Returns (out, lse, k_work, v_work)."""
    lib = _lib.load()
    _require(q, "q", dtype=torch.bfloat16)
    _require(k, "k", dtype=q.dtype)
    B, H, H_kv, T, d = _geometry(q, k, layout)
    _require(v, "v", k.shape, q.dtype)
    _require(ve, "ve", k.shape, q.dtype)
    _require(gate_logits, "gate_logits", _gate_shape(v, layout)[4], q.dtype)
    _rope_tables(cos, sin, T, d)
    k_work = torch.empty_like(k) if k_work is None else k_work
    _require(k_work, "k_work", k.shape, q.dtype)
    v_work = torch.empty_like(v) if v_work is None else v_work
    _require(v_work, "v_work", v.shape, q.dtype)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    lse = _lse(lse, want_lse, B, H, T, q.device)
    rc = lib.attn_fwd_qknorm_ve_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(gate_logits),
                                   _ptr(k_work), _ptr(v_work), _ptr(out), _ptr(lse), _ptr(cos),
                                   _ptr(sin), B, H, H_kv, T, d, _LAYOUTS[layout], float(eps),
                                   int(window), int(bool(causal)), _lib.ATTN_BF16,
                                   _stream_handle())
    _lib.check("attn_fwd_qknorm_ve_ex", rc)
    return out, lse, k_work, v_work


def attention_layer_ve_backward(q: torch.Tensor, k: torch.Tensor, v_work: torch.Tensor,
                                ve: torch.Tensor, gate_logits: torch.Tensor, out: torch.Tensor,
                                lse: torch.Tensor, dout: torch.Tensor, cos: torch.Tensor,
                                sin: torch.Tensor, window: int = -1, eps: float = 1e-6,
                                layout: str = "bhtd"):
    """Gradients (dq, dk, dv, dve, dgate_logits) of a layer with a value embedding, from the
    gated v_work, out and lse of attn_fwd_qknorm_ve: the layer backward on v_work, then the
    gate's backward (the gradient of v is that of v_work)."""
    dq, dk, dv = attention_layer_backward(q, k, v_work, out, lse, dout, cos, sin, window, eps,
                                          layout)
    dve, dz = value_gate_bwd(ve, gate_logits, dv, layout=layout)
    return dq, dk, dv, dve, dz


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           lengths: torch.Tensor | None = None, window: int = -1,
           out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
           want_lse: bool = True, workspace: torch.Tensor | None = None, layout: str = "bhtd"):
    """One generation step: q [B, H, d] (the newest token's normalised, rotated query) against
    k_cache, v_cache [B, H_kv, S, d] (or [B, S, H_kv, d] with layout "bthd") holding lengths[b]
    tokens each (int32 [B] on the GPU; None: all S). Returns (out [B, H, d], lse [B, H]).
    The split-over-keys workspace is allocated here unless given (the library allocates none)."""
    lib = _lib.load()
    _require(q, "q")
    if q.dim() != 3 or q.dtype not in _DTYPES:
        raise ValueError("q must be [B, H, d] bf16 or fp32")
    _require(k_cache, "k_cache", dtype=q.dtype)
    _require(v_cache, "v_cache", k_cache.shape, q.dtype)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be 4-d")
    B, H, d = q.shape
    if layout == "bhtd":
        _, H_kv, S, _ = k_cache.shape
    elif layout == "bthd":
        _, S, H_kv, _ = k_cache.shape
    else:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}, got {layout!r}")
    if k_cache.shape[0] != B or k_cache.shape[3] != d or H % H_kv:
        raise ValueError("k_cache must hold the batch, head dim and a kv head count dividing H")
    if lengths is not None:
        _require(lengths, "lengths", (B,), torch.int32)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", (B, H), torch.float32)
    need = lib.attn_decode_workspace_bytes(B, H, S, d, int(window))
    if need < 0:
        raise ValueError("invalid decode shape")
    if workspace is None:
        workspace = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=q.device)
    _require(workspace, "workspace")
    rc = lib.attn_decode_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths), _ptr(out),
                            _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            B, H, H_kv, S, d, _LAYOUTS[layout], int(window), _DTYPES[q.dtype],
                            _stream_handle())
    _lib.check("attn_decode_ex", rc)
    return out, lse


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   lengths: torch.Tensor | None = None, window: int = -1,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   layout: str = "bhtd"):
    """``decode`` through the allocation-free entry point (attn_decode_noalloc_ex): the split
    partials use the library's fixed device scratch instead of a workspace. With ``out`` and
    ``lse`` given, nothing is allocated here either."""
    lib = _lib.load()
    _require(q, "q")
    if q.dim() != 3 or q.dtype not in _DTYPES:
        raise ValueError("q must be [B, H, d] bf16 or fp32")
    _require(k_cache, "k_cache", dtype=q.dtype)
    _require(v_cache, "v_cache", k_cache.shape, q.dtype)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be 4-d")
    B, H, d = q.shape
    if layout == "bhtd":
        _, H_kv, S, _ = k_cache.shape
    elif layout == "bthd":
        _, S, H_kv, _ = k_cache.shape
    else:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}, got {layout!r}")
    if k_cache.shape[0] != B or k_cache.shape[3] != d or H % H_kv:
        raise ValueError("k_cache must hold the batch, head dim and a kv head count dividing H")
    if lengths is not None:
        _require(lengths, "lengths", (B,), torch.int32)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.shape, q.dtype)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _require(lse, "lse", (B, H), torch.float32)
    rc = lib.attn_decode_noalloc_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths),
                                    _ptr(out), _ptr(lse), B, H, H_kv, S, d, _LAYOUTS[layout],
                                    int(window), _DTYPES[q.dtype], _stream_handle())
    _lib.check("attn_decode_noalloc_ex", rc)
    return out, lse
