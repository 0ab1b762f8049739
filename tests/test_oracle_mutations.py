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


# ---------------------------------------------------------------------------------------------
# Backward pass: planted mistakes in copies of the gradient formulas.
# ---------------------------------------------------------------------------------------------

def _backward_with(keep_delta=True, p_factor=True, dk_scale=None, dq_scale=None, dv_transposed=False):
    def bwd(q, k, v, do, window=-1, causal=True, block=256):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        B, H, T, d = q.shape
        H_kv = k.shape[1]
        c = 1 / math.sqrt(d)
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        vis = oracle.visible(i, j, window, causal)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                g = h // (H // H_kv)
                s = np.where(vis, c * q[b, h] @ k[b, g].T, -np.inf)
                p = np.exp(s - s.max(1, keepdims=True))
                p /= p.sum(1, keepdims=True)
                dp = do[b, h] @ v[b, g].T
                D = (p * dp).sum(1, keepdims=True) if keep_delta else 0.0
                ds = (p if p_factor else 1.0) * (dp - D) * vis
                dv[b, g] += (p @ do[b, h]) if dv_transposed else (p.T @ do[b, h])
                dq[b, h] += (dq_scale(d) if dq_scale else c) * ds @ k[b, g]
                dk[b, g] += (dk_scale(d) if dk_scale else c) * ds.T @ q[b, h]
        return dq, dk, dv
    return bwd


def _layer_bwd_with(att_bwd, pro_bwd=None):
    def layer(q, k, v, do, window=-1, causal=True, eps=1e-6, base=10000.0):
        qn, kn = oracle.qknorm_rope(q, k, eps, base)
        dqn, dkn, dv = att_bwd(qn, kn, v, do, window, causal)
        pb = pro_bwd or oracle.qknorm_rope_backward
        return pb(q, dqn, eps, base), pb(k, dkn, eps, base), dv
    return layer


BWD_CHECKS = [pins.check_backward_finite_differences, pins.check_layer_backward_finite_differences,
              pins.check_backward_torch_autograd, pins.check_backward_invariants]


def test_unmutated_backward_copy_passes():
    bwd = _backward_with()
    o = _mutant(attention_backward=bwd, attention_layer_backward=_layer_bwd_with(bwd),
                rms_norm_backward=oracle.rms_norm_backward,
                rope_apply_backward=oracle.rope_apply_backward)
    assert not _fails(o, BWD_CHECKS)


@pytest.mark.parametrize("name,kw", [
    ("no D subtracted", dict(keep_delta=False)),
    ("dS without the P factor", dict(p_factor=False)),
    ("dK without the 1/sqrt(d) scale", dict(dk_scale=lambda d: 1.0)),
    ("dQ scaled by 1/d", dict(dq_scale=lambda d: 1.0 / d)),
    ("dV from P instead of P^T", dict(dv_transposed=True)),
])
def test_backward_mutations_are_caught(name, kw):
    bwd = _backward_with(**kw)
    o = _mutant(attention_backward=bwd, attention_layer_backward=_layer_bwd_with(bwd),
                rms_norm_backward=oracle.rms_norm_backward,
                rope_apply_backward=oracle.rope_apply_backward)
    assert _fails(o, BWD_CHECKS), name


def _pro_bwd_rotation_sign(x, dy, eps=1e-6, base=10000.0):
    """Prologue backward that rotates dy forward instead of back."""
    T, d = np.asarray(x).shape[-2:]
    cos, sin = oracle.rope_cos_sin(T, d, base)
    return oracle.rms_norm_backward(x, oracle.rope_apply(dy, cos, sin), eps)


def _pro_bwd_no_projection(x, dy, eps=1e-6, base=10000.0):
    """Prologue backward that drops the norm's projection term (treats r as a constant)."""
    x = np.asarray(x, np.float64)
    T, d = x.shape[-2:]
    cos, sin = oracle.rope_cos_sin(T, d, base)
    r = 1 / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)
    return r * oracle.rope_apply_backward(dy, cos, sin)


@pytest.mark.parametrize("name,fn", [("rotation forward in backward", _pro_bwd_rotation_sign),
                                     ("norm backward without projection", _pro_bwd_no_projection)])
def test_prologue_backward_mutations_are_caught(name, fn):
    o = _mutant(attention_backward=oracle.attention_backward,
                attention_layer_backward=_layer_bwd_with(oracle.attention_backward, fn),
                rms_norm_backward=oracle.rms_norm_backward,
                rope_apply_backward=oracle.rope_apply_backward)
    assert _fails(o, BWD_CHECKS), name


def _decode_with(lo_fn=None, hi_off=0, kv_map=None):
    def dec(q, k, v, lengths=None, window=-1):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        B, H, d = q.shape
        H_kv, S = k.shape[1], k.shape[2]
        lengths = [S] * B if lengths is None else list(lengths)
        out, lse = np.zeros((B, H, v.shape[-1])), np.zeros((B, H))
        for b in range(B):
            n = lengths[b]
            lo = lo_fn(n, window) if lo_fn else (0 if window < 0 else max(0, n - 1 - window))
            hi = max(lo + 1, n + hi_off)
            for h in range(H):
                g = kv_map(h, H, H_kv) if kv_map else h // (H // H_kv)
                s = k[b, g, lo:hi] @ q[b, h] / math.sqrt(d)
                l = s.max() + np.log(np.exp(s - s.max()).sum())
                out[b, h], lse[b, h] = np.exp(s - l) @ v[b, g, lo:hi], l
        return out, lse
    return dec


def test_unmutated_decode_copy_passes():
    assert not _fails(_mutant(decode_attention=_decode_with()), [pins.check_decode])


@pytest.mark.parametrize("name,kw", [
    ("window one key short", dict(lo_fn=lambda n, w: 0 if w < 0 else min(n - 1, max(0, n - w)))),
    ("newest key left out", dict(hi_off=-1)),
    ("kv heads interleaved", dict(kv_map=lambda h, H, H_kv: h % H_kv)),
])
def test_decode_mutations_are_caught(name, kw):
    assert _fails(_mutant(decode_attention=_decode_with(**kw)), [pins.check_decode]), name


# Value-embedding gate (R16): each plausible slip in the gate or its gradients fails a pin.
def _gate_mutant(gate_of=None, value_gate=None, value_gate_backward=None):
    o = types.SimpleNamespace()
    for n in ("attention", "attention_layer", "attention_layer_backward", "gate_of", "value_gate",
              "value_gate_backward", "attention_layer_ve", "attention_layer_ve_backward"):
        setattr(o, n, getattr(oracle, n))
    if gate_of is not None:
        o.gate_of = gate_of
    if value_gate is not None:
        o.value_gate = value_gate
    if value_gate_backward is not None:
        o.value_gate_backward = value_gate_backward
    vg = o.value_gate
    o.attention_layer_ve = lambda q, k, v, ve, z, window=-1, causal=True, eps=1e-6, base=1e4, rows=None: \
        oracle.attention_layer(q, k, vg(v, ve, z), window, causal, eps, base, rows=rows)

    def layer_bwd(q, k, v, ve, z, dout, window=-1, causal=True, eps=1e-6, base=1e4):
        dq, dk, dvg = oracle.attention_layer_backward(q, k, vg(v, ve, z), dout, window, causal,
                                                      eps, base)
        return (dq, dk) + tuple(o.value_gate_backward(ve, z, dvg))
    o.attention_layer_ve_backward = layer_bwd
    return o


def _sig(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


GATE_MUTANTS = {
    "gate without the factor 2": dict(gate_of=lambda z: _sig(z)),
    "gate of -z": dict(gate_of=lambda z: 2 * _sig(-np.asarray(z, np.float64))),
    "one gate per head, not per token": dict(
        value_gate=lambda v, ve, z: v + oracle.gate_of(z).mean(axis=-1, keepdims=True)[..., None] * ve),
    "v and ve swapped": dict(value_gate=lambda v, ve, z: ve + oracle.gate_of(z)[..., None] * v),
    "dz without the sigmoid's (1 - g/2)": dict(value_gate_backward=lambda ve, z, dy: (
        dy, oracle.gate_of(z)[..., None] * dy, oracle.gate_of(z) * np.sum(ve * dy, -1))),
    "dve without the gate": dict(value_gate_backward=lambda ve, z, dy: (
        dy, dy, oracle.value_gate_backward(ve, z, dy)[2])),
}


def test_unmutated_gate_copy_passes():
    o = _gate_mutant()
    for c in pins.VALUE_GATE_CHECKS:
        c(o)


@pytest.mark.parametrize("name", list(GATE_MUTANTS))
def test_gate_mutations_are_caught(name):
    assert _fails(_gate_mutant(**GATE_MUTANTS[name]), pins.VALUE_GATE_CHECKS), name


# Row blocks and sampled rows: the key range of a block that starts past the window, and the
# order of sampled rows.
def _key_range_drops_boundary(r0, r1, T, window, causal):
    """Key range one short at the window's inclusive boundary key r0 - W of a later block."""
    if not causal:
        return 0, T
    return (0 if window < 0 else max(0, r0 - window + 1)), min(T, r1)


def _key_range_one_past(r0, r1, T, window, causal):
    """Key range that ends one key early (the block's last row loses its own key)."""
    if not causal:
        return 0, T
    return (0 if window < 0 else max(0, r0 - window)), min(T, r1 - 1)


@pytest.mark.parametrize("name,fn", [("window boundary key dropped", _key_range_drops_boundary),
                                     ("block's last key dropped", _key_range_one_past)])
def test_key_range_mutations_are_caught(name, fn, monkeypatch):
    import sys
    monkeypatch.setattr(sys.modules["oracle.attention"], "_key_range", fn)
    monkeypatch.setattr(sys.modules["oracle.backward"], "_key_range", fn)
    assert _fails(oracle, [pins.check_blocked_rows]), name
    assert _fails(oracle, [pins.check_backward_blocked]), name


def _attention_sorted_rows(q, k, v, window=-1, causal=True, rows=None, block=256):
    """Sampled rows returned in sorted order instead of the order asked for."""
    if rows is not None:
        rows = np.sort(np.asarray(rows))
    return oracle.attention(q, k, v, window, causal, rows=rows, block=block)


def test_sampled_row_order_mutation_is_caught():
    assert _fails(_mutant(attention=_attention_sorted_rows), [pins.check_blocked_rows])


def test_key_range_unmutated_passes():
    assert not _fails(oracle, [pins.check_blocked_rows, pins.check_backward_blocked])
