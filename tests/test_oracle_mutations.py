"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show that at least one pin
catches each: a pin that cannot fail pins nothing."""

import math
import types

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def _mutant(**overrides):
    ns = types.SimpleNamespace()
    for n in ("attention", "attention_layer", "qknorm_rope", "rms_norm", "rope_apply",
              "rope_cos_sin", "sssl_windows", "visible"):
        setattr(ns, n, getattr(oracle, n))
    for n, f in overrides.items():
        setattr(ns, n, f)
    return ns


def _attention_with(scale_fn=None, vis_fn=None, lse_fn=None):
    """A copy of the oracle's attention with one step swapped out."""
    def att(q, k, v, window=-1, causal=True, rows=None, block=256):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        B, H, T, d = q.shape
        ridx = np.arange(T)
        keys = np.arange(T)
        vis = (vis_fn or oracle.visible)(ridx[:, None], keys[None, :], window, causal)
        out = np.zeros((B, H, T, v.shape[-1]))
        lse = np.zeros((B, H, T))
        for b in range(B):
            for h in range(H):
                s = (q[b, h] @ k[b, h].T) * (scale_fn(d) if scale_fn else 1 / math.sqrt(d))
                s = np.where(vis, s, -np.inf)
                m = s.max(1, keepdims=True)
                l = (lse_fn or (lambda s, m: m + np.log(np.exp(s - m).sum(1, keepdims=True))))(s, m)
                out[b, h] = np.exp(s - l) @ v[b, h]
                lse[b, h] = l[:, 0]
        return out, lse
    return att


def _layer_with(att):
    def layer(q, k, v, window=-1, causal=True, eps=1e-6, base=10000.0, rows=None):
        qn, kn = oracle.qknorm_rope(q, k, eps, base)
        return att(qn, kn, v, window, causal)
    return layer


def _fails(o, checks):
    for c in checks:
        try:
            c(o)
        except AssertionError:
            return True
    return False


def test_unmutated_copy_passes():
    att = _attention_with()
    o = _mutant(attention=att, attention_layer=_layer_with(att))
    assert not _fails(o, [pins.check_worked_example, pins.check_brute_force,
                          pins.check_zero_query_closed_form, pins.check_window_zero])


@pytest.mark.parametrize("name,overrides", [
    ("no 1/sqrt(d) scale", dict(scale_fn=lambda d: 1.0)),
    ("scale 1/d", dict(scale_fn=lambda d: 1.0 / d)),
    ("exclusive window i-j<W", dict(vis_fn=lambda i, j, w, c: (j <= i) & (((i - j) < w) if w >= 0 else True))),
    ("mask above diagonal kept", dict(vis_fn=lambda i, j, w, c: np.ones(np.broadcast(i, j).shape, bool))),
    ("lse without max shift back", dict(lse_fn=lambda s, m: np.log(np.exp(s - m).sum(1, keepdims=True)))),
])
def test_attention_mutations_are_caught(name, overrides):
    att = _attention_with(**overrides)
    o = _mutant(attention=att, attention_layer=_layer_with(att))
    assert _fails(o, [pins.check_worked_example, pins.check_brute_force,
                      pins.check_zero_query_closed_form, pins.check_window_zero]), name


def _rope_flipped_sign(x, cos, sin):
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], -1)


def _rope_interleaved(x, cos, sin):
    y = np.array(x, dtype=np.float64, copy=True)
    a, b = x[..., 0::2], x[..., 1::2]
    y[..., 0::2] = a * cos + b * sin
    y[..., 1::2] = -a * sin + b * cos
    return y


def _cos_sin_wrong_base_exponent(T, d, base=10000.0):
    j = np.arange(d // 2)
    th = np.outer(np.arange(T), base ** (-j / d))
    return np.cos(th), np.sin(th)


@pytest.mark.parametrize("name,overrides", [
    ("rope sign transposed", dict(rope_apply=_rope_flipped_sign)),
    ("rope interleaved pairs", dict(rope_apply=_rope_interleaved)),
    ("rope exponent -j/d", dict(rope_cos_sin=_cos_sin_wrong_base_exponent)),
    ("rms norm over sum not mean", dict(rms_norm=lambda x, eps=1e-6: np.asarray(x) / np.sqrt((np.asarray(x) ** 2).sum(-1, keepdims=True) + eps))),
    ("rms norm without eps", dict(rms_norm=lambda x, eps=1e-6: np.asarray(x) / np.sqrt((np.asarray(x) ** 2).mean(-1, keepdims=True)))),
    ("last layer not forced long", dict(sssl_windows=lambda T, n, p="SSSL": [T if p[l % len(p)] == "L" else T // 2 for l in range(n)])),
])
def test_prologue_mutations_are_caught(name, overrides):
    o = _mutant(**overrides)
    checks = [pins.check_rope_special_values, pins.check_rope_invariants, pins.check_rms_norm,
              pins.check_worked_example_qknorm, pins.check_sssl_windows]
    assert _fails(o, checks), name


def _gqa_interleaved(q, k, v, window=-1, causal=True, rows=None, block=256):
    """Query head h attends with kv head h % H_kv instead of h // (H / H_kv)."""
    H, H_kv = q.shape[1], k.shape[1]
    idx = [h % H_kv for h in range(H)]
    return oracle.attention(q, np.asarray(k)[:, idx], np.asarray(v)[:, idx], window, causal,
                            rows=rows, block=block)


def test_gqa_mapping_mutation_is_caught():
    assert _fails(_mutant(attention=_gqa_interleaved), [pins.check_gqa_head_mapping])
