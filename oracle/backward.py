"""fp64 CPU oracle of the backward pass: gradients of QK-RMSNorm, RoPE and causal / sliding-window
softmax attention, written out from the chain rule applied to their plain definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): shares no code with the GPU path.

Source: [HABR] "Подробный технический разбор реализации Autoresearch, ИИ-исследователя Андрея
Карпаты" (habr.com, article 1010198), train.py listing: the training loop calls
``loss.backward()`` on the model whose attention block is ``CausalSelfAttention.forward``, and
``GPT.estimate_flops`` counts the attention's backward as twice its forward. The pages print no
backward formulas; the gradients below are the exact derivatives of the forward definitions in
``oracle/attention.py`` (reading R14), pinned against finite differences of that forward and
against autograd of library routines.

For one head with scale c = 1/sqrt(d), P = softmax(c Q K^T + mask) and O = P V, given dO:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij   (= dO_i . O_i)
    dS = P * (dP - D)        (row-wise D)
    dQ = c dS K
    dK = c dS^T Q

With grouped-query heads (R13) the kv-head gradients sum over the query heads of the group.
The prologue y = R_t (x / sqrt(mean(x^2) + eps)) (rotation R_t of position t) has
dx = r (g - xh * mean(g * xh)) with r = 1/sqrt(mean(x^2) + eps), xh = r x and g = R_t^T dy
(the rotation is orthogonal, so its backward is the rotation by the opposite angles).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import (EPS_DEFAULT, ROPE_BASE_DEFAULT, _key_range, kv_head, qknorm_rope,
                        rope_cos_sin, visible)


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                       window: int = -1, causal: bool = True, block: int = 256):
    """Gradients (dq, dk, dv) of sum(dout * O) for O = attention(q, k, v, window, causal), fp64.

    q, dout: [B, H, T, d]; k, v: [B, H_kv, T, d] (H_kv divides H, R13). Rows are processed in
    blocks over the key range they can see; entries outside it have zero weight and contribute
    nothing to any gradient.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, T, d) or v.shape[:3] != k.shape[:3] or dout.shape[:3] != q.shape[:3]:
        raise ValueError("q, dout must be [B, H, T, d] and k, v [B, H_kv, T, d]")
    if not causal and window >= 0:
        raise ValueError("a window needs causal=True")
    c = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        rows = np.arange(r0, r1)
        lo, hi = _key_range(r0, r1, T, window, causal)
        keys = np.arange(lo, hi)
        vis = visible(rows[:, None], keys[None, :], window, causal)
        for b in range(B):
            for h in range(H):
                g = kv_head(h, H, H_kv)
                Kb, Vb = k[b, g, lo:hi], v[b, g, lo:hi]
                s = np.where(vis, c * (q[b, h, r0:r1] @ Kb.T), -np.inf)
                m = np.max(s, axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / np.sum(e, axis=1, keepdims=True)
                do = dout[b, h, r0:r1]
                dp = do @ Vb.T
                D = np.sum(p * dp, axis=1, keepdims=True)
                ds = p * (dp - D)
                dv[b, g, lo:hi] += p.T @ do
                dq[b, h, r0:r1] += c * (ds @ Kb)
                dk[b, g, lo:hi] += c * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv


def rope_apply_backward(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Backward of the half-split rotation ([HABR] ``apply_rotary_emb``): y1 = x1 cos + x2 sin,
    y2 = -x1 sin + x2 cos, so dx1 = dy1 cos - dy2 sin and dx2 = dy1 sin + dy2 cos."""
    dy = np.asarray(dy, dtype=np.float64)
    h = dy.shape[-1] // 2
    g1, g2 = dy[..., :h], dy[..., h:]
    return np.concatenate([g1 * cos - g2 * sin, g1 * sin + g2 * cos], axis=-1)


def rms_norm_backward(x: np.ndarray, g: np.ndarray, eps: float = EPS_DEFAULT) -> np.ndarray:
    """Backward of the weightless RMSNorm ([HABR] ``norm``) over the last axis: for
    xh = r x with r = (mean(x^2) + eps)^(-1/2), dx = r (g - xh mean(g xh))."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = r * x
    return r * (g - xh * np.mean(g * xh, axis=-1, keepdims=True))


def qknorm_rope_backward(x: np.ndarray, dy: np.ndarray, eps: float = EPS_DEFAULT,
                         base: float = ROPE_BASE_DEFAULT) -> np.ndarray:
    """Gradient with respect to raw rows x [..., T, d] of y = RoPE(RMSNorm(x)), given dy."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape[-2], x.shape[-1]
    cos, sin = rope_cos_sin(T, d, base)
    return rms_norm_backward(x, rope_apply_backward(dy, cos, sin), eps)


def attention_layer_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                             window: int = -1, causal: bool = True, eps: float = EPS_DEFAULT,
                             base: float = ROPE_BASE_DEFAULT):
    """Gradients (dq, dk, dv) with respect to the raw q, k and v of one attention layer
    (``attention_layer``: QK-norm + RoPE, then attention)."""
    qn, kn = qknorm_rope(q, k, eps, base)
    dqn, dkn, dv = attention_backward(qn, kn, v, dout, window, causal)
    return (qknorm_rope_backward(q, dqn, eps, base), qknorm_rope_backward(k, dkn, eps, base), dv)
