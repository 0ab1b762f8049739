"""fp64 CPU oracle of the value-embedding gate that precedes the attention call in layers with a
value embedding, and of its gradients.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): shares no code with the GPU path.

Source: [HABR] "Подробный технический разбор реализации Autoresearch, ИИ-исследователя Андрея
Карпаты" (habr.com, article 1010198), train.py listing, ``CausalSelfAttention.forward``, the
value-residual step. For a layer that has a value embedding, ve is viewed per kv head like v. The
gate is twice the logistic sigmoid of the ``ve_gate`` linear layer applied to the first channels
of x, one value per (batch, token, kv head), so it lies in (0, 2) and 1 leaves the sum v + ve.
v becomes v + gate * ve, the gate broadcast over the head dimension, before the rotation, the
norm and the attention call.

Reading R16: the ``ve_gate`` linear layer is one of the projections, outside the attention
block's kernels. The functions here take its output z (the gate logits) as an input. Tensors use
the oracle's [B, H_kv, T, d] order, and z is [B, H_kv, T].
"""

from __future__ import annotations

import numpy as np

from .attention import EPS_DEFAULT, ROPE_BASE_DEFAULT, attention_layer
from .backward import attention_layer_backward


def gate_of(z: np.ndarray) -> np.ndarray:
    """2 * sigmoid(z), in fp64, without overflow for large |z| (sigmoid(z) = 1 / (1 + e^-z) for
    z >= 0 and e^z / (1 + e^z) for z < 0)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return 2.0 * np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def value_gate(v: np.ndarray, ve: np.ndarray, z: np.ndarray) -> np.ndarray:
    """v + gate_of(z) * ve with one gate per row (the gate broadcast over the last axis).

    v, ve: [..., T, d]; z: [..., T]."""
    v = np.asarray(v, dtype=np.float64)
    ve = np.asarray(ve, dtype=np.float64)
    if ve.shape != v.shape or np.shape(z) != v.shape[:-1]:
        raise ValueError("ve must have v's shape and z v's shape without the last axis")
    return v + gate_of(z)[..., None] * ve


def value_gate_backward(ve: np.ndarray, z: np.ndarray, dv_gated: np.ndarray):
    """Gradients (dv, dve, dz) of sum(dv_gated * value_gate(v, ve, z)).

    With g = 2 sigmoid(z): dv = dv_gated, dve = g dv_gated, and since
    d g / d z = 2 sigmoid(z) (1 - sigmoid(z)) = g (1 - g / 2), dz = g (1 - g / 2) sum_j ve_j dv_j.
    """
    ve = np.asarray(ve, dtype=np.float64)
    dv_gated = np.asarray(dv_gated, dtype=np.float64)
    g = gate_of(z)
    return dv_gated.copy(), g[..., None] * dv_gated, g * (1.0 - g / 2.0) * np.sum(ve * dv_gated,
                                                                                 axis=-1)


def attention_layer_ve(q, k, v, ve, z, window: int = -1, causal: bool = True,
                       eps: float = EPS_DEFAULT, base: float = ROPE_BASE_DEFAULT, rows=None):
    """One layer with a value embedding: the gate on v, then ``attention_layer`` (QK-norm + RoPE
    of q and k, then attention). k, v, ve: [B, H_kv, T, d]; z: [B, H_kv, T]."""
    return attention_layer(q, k, value_gate(v, ve, z), window, causal, eps, base, rows=rows)


def attention_layer_ve_backward(q, k, v, ve, z, dout, window: int = -1, causal: bool = True,
                                eps: float = EPS_DEFAULT, base: float = ROPE_BASE_DEFAULT):
    """Gradients (dq, dk, dv, dve, dz) of sum(dout * attention_layer_ve(...)[0])."""
    vg = value_gate(v, ve, z)
    dq, dk, dvg = attention_layer_backward(q, k, vg, dout, window, causal, eps, base)
    dv, dve, dz = value_gate_backward(ve, z, dvg)
    return dq, dk, dv, dve, dz
