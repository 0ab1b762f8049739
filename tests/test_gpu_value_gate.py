"""GPU parity of the value-embedding gate (attn_value_gate_ex, attn_fwd_qknorm_ve_ex,
attn_value_gate_bwd_ex) against the fp64 oracle, through the C ABI.

Tolerances. The gate is fp32 arithmetic with one rounding of each output: for bf16 outputs
|gpu - oracle| <= 2^-8 |oracle| (half an ulp is 2^-9 relative; the rest covers fp32's exp and the
FMA), plus 1e-6 (|v| + 2 |ve|) for fp32's own rounding; fp32 outputs 1e-5 of that scale. The layer
keeps the fused layer's bound, 2e-2 on out and lse, which was derived for values of N(0, 1) draws
(|v| up to about 4): every error term of the bf16 path (weights, output and q, k roundings) is
proportional to the size of the values, so out's bound is scaled by max(1, max |v'| / 4) for the
gated values v' (up to |v| + 2 |ve|). Gradients keep the layer backward's bound (2e-2 of
max(1, max |oracle|)). Every case prints its name before touching the GPU.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_qk_amd import _lib, inputs, ops

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    torch.cuda.synchronize()


def to_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    """[B, H, T, d] (or [B, H, T]) stored in `layout` on the GPU."""
    x = x.to("cuda")
    return (x.transpose(1, 2) if layout == "bthd" else x).contiguous()


def from_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    return (x.transpose(1, 2) if layout == "bthd" else x).contiguous().cpu()


def gate_inputs(B, H_kv, T, d, dtype, seed, scale=3.0):
    v = inputs.make_random((B, H_kv, T, d), dtype, seed)
    ve = inputs.make_random((B, H_kv, T, d), dtype, seed + 1)
    z = (inputs.make_random((B, H_kv, T), torch.float32, seed + 2) * scale).to(dtype)
    # exact extremes in the first rows: 0 (gate 1), far negative (gate 0), far positive (gate 2)
    n = min(3, z.numel())
    z.view(-1)[:n] = torch.tensor([0.0, -60.0, 60.0][:n], dtype=dtype)
    return v, ve, z


def assert_gate_close(got, ref, v, ve, dt):
    scale = np.abs(f64(v)) + 2 * np.abs(f64(ve))
    err = np.abs(f64(got) - ref)
    bound = (2.0 ** -8 * np.abs(ref) + 1e-6 * scale) if dt == "bf16" else 1e-5 * scale + 1e-7
    say(f"   max err {err.max():.3e}")
    assert np.all(err <= bound), float(err.max())


CASES = [(dt, d, B, H_kv, T, lay) for dt in ("bf16", "f32") for d in (16, 32, 64, 128)
         for (B, H_kv, T, lay) in ((1, 1, 1, "bhtd"), (2, 3, 67, "bthd"), (1, 2, 130, "bhtd"))]


@pytest.mark.parametrize("dt,d,B,H_kv,T,layout", CASES,
                         ids=[f"{c[0]}-d{c[1]}-B{c[2]}k{c[3]}T{c[4]}-{c[5]}" for c in CASES])
def test_value_gate_parity(dt, d, B, H_kv, T, layout):
    say(f"value gate {dt} d={d} B={B} H_kv={H_kv} T={T} {layout}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    v, ve, z = gate_inputs(B, H_kv, T, d, dtype, 500 + d + T)
    vd, ved, zd = (to_layout(x, layout) for x in (v, ve, z))
    out = ops.value_gate(vd, ved, zd, layout=layout)
    inplace = vd.clone()
    ops.value_gate(inplace, ved, zd, out=inplace, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(inplace, out)
    ref = oracle.value_gate(f64(v), f64(ve), f64(z))
    assert_gate_close(from_layout(out, layout), ref, v, ve, dt)
    # the exact gates of the first rows: v + ve, v, v + 2 ve (up to the output's rounding)
    got = f64(from_layout(out, layout))
    for i, g in enumerate((1.0, 0.0, 2.0)[:min(3, z.numel())]):
        idx = np.unravel_index(i, z.shape)
        want = f64(v)[idx] + g * f64(ve)[idx]
        assert np.allclose(got[idx], want, rtol=2.0 ** -8 if dt == "bf16" else 1e-6, atol=1e-6)


@pytest.mark.parametrize("dt,d,B,H_kv,T,layout", CASES,
                         ids=[f"{c[0]}-d{c[1]}-B{c[2]}k{c[3]}T{c[4]}-{c[5]}" for c in CASES])
def test_value_gate_bwd_parity(dt, d, B, H_kv, T, layout):
    say(f"value gate bwd {dt} d={d} B={B} H_kv={H_kv} T={T} {layout}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    _, ve, z = gate_inputs(B, H_kv, T, d, dtype, 600 + d + T)
    dv = inputs.make_random((B, H_kv, T, d), dtype, 610 + d)
    ved, zd, dvd = (to_layout(x, layout) for x in (ve, z, dv))
    dve, dz = ops.value_gate_bwd(ved, zd, dvd, layout=layout)
    dve2 = dvd.clone()
    _, dz2 = ops.value_gate_bwd(ved, zd, dve2, dve=dve2, layout=layout)  # in place
    torch.cuda.synchronize()
    assert torch.equal(dve2, dve) and torch.equal(dz2, dz)
    _, rve, rz = oracle.value_gate_backward(f64(ve), f64(z), f64(dv))
    e_ve = np.abs(f64(from_layout(dve, layout)) - rve)
    e_z = np.abs(f64(from_layout(dz, layout)) - rz)
    dot_scale = np.sum(np.abs(f64(ve) * f64(dv)), axis=-1)
    say(f"   max err dve {e_ve.max():.3e} dz {e_z.max():.3e}")
    if dt == "bf16":
        assert np.all(e_ve <= 2.0 ** -8 * np.abs(rve) + 1e-6 * np.abs(f64(dv)))
        assert np.all(e_z <= 2.0 ** -8 * np.abs(rz) + 1e-5 * dot_scale)
    else:
        assert np.all(e_ve <= 1e-6 * np.abs(f64(dv)) + 1e-7)
        assert np.all(e_z <= 1e-5 * dot_scale + 1e-7)


LAYER_CASES = [(32, 1, 4, 4, 100, -1, "bhtd"), (64, 2, 4, 2, 190, 50, "bthd"),
               (128, 1, 4, 1, 257, 90, "bhtd"), (64, 1, 2, 2, 1, -1, "bthd")]


@pytest.mark.parametrize("d,B,H,H_kv,T,window,layout", LAYER_CASES,
                         ids=[f"d{c[0]}-B{c[1]}H{c[2]}k{c[3]}T{c[4]}-W{c[5]}-{c[6]}"
                              for c in LAYER_CASES])
def test_layer_with_value_embedding(d, B, H, H_kv, T, window, layout):
    """attn_fwd_qknorm_ve_ex against the oracle's layer; its v_work equals attn_value_gate_ex's
    output and its out, lse and k_work equal attn_fwd_qknorm_ex on v_work, bit for bit."""
    say(f"layer with value embedding d={d} B={B} H={H} H_kv={H_kv} T={T} W={window} {layout}")
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 701)
    k = inputs.make_random((B, H_kv, T, d), torch.bfloat16, 702)
    v, ve, z = gate_inputs(B, H_kv, T, d, torch.bfloat16, 703)
    qd, kd, vd, ved, zd = (to_layout(x, layout) for x in (q, k, v, ve, z))
    cos, sin = ops.rope_table(T, d)
    out, lse, kw, vw = ops.attn_fwd_qknorm_ve(qd, kd, vd, ved, zd, cos, sin, window=window,
                                              layout=layout)
    vg = ops.value_gate(vd, ved, zd, layout=layout)
    o2, l2, kw2 = ops.attn_fwd_qknorm(qd, kd, vg, cos, sin, window=window, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(vw, vg) and torch.equal(kw, kw2)
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    # in place: v_work = v, k_work = k
    vi, ki = vd.clone(), kd.clone()
    o3, l3, _, _ = ops.attn_fwd_qknorm_ve(qd, ki, vi, ved, zd, cos, sin, window=window,
                                          k_work=ki, v_work=vi, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(vi, vg) and torch.equal(ki, kw) and torch.equal(o3, out)
    ro, rl = oracle.attention_layer_ve(f64(q), f64(k), f64(v), f64(ve), f64(z), window=window)
    eo = float(np.max(np.abs(f64(from_layout(out, layout)) - ro)))
    el = float(np.max(np.abs(f64(lse) - rl)))
    vmax = float(np.max(np.abs(oracle.value_gate(f64(v), f64(ve), f64(z)))))
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e} max|v'|={vmax:.2f}")
    assert eo <= BF16_TOL * max(1.0, vmax / 4) and el <= BF16_TOL


@pytest.mark.parametrize("d,B,H,H_kv,T,window,layout", LAYER_CASES[:3],
                         ids=[f"d{c[0]}-B{c[1]}H{c[2]}k{c[3]}T{c[4]}-W{c[5]}-{c[6]}"
                              for c in LAYER_CASES[:3]])
def test_layer_with_value_embedding_backward(d, B, H, H_kv, T, window, layout):
    say(f"layer with value embedding backward d={d} B={B} H={H} H_kv={H_kv} T={T} W={window} "
        f"{layout}")
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 711)
    k = inputs.make_random((B, H_kv, T, d), torch.bfloat16, 712)
    v, ve, z = gate_inputs(B, H_kv, T, d, torch.bfloat16, 713, scale=1.0)
    do = inputs.make_random((B, H, T, d), torch.bfloat16, 714)
    qd, kd, vd, ved, zd, dod = (to_layout(x, layout) for x in (q, k, v, ve, z, do))
    cos, sin = ops.rope_table(T, d)
    out, lse, _, vw = ops.attn_fwd_qknorm_ve(qd, kd, vd, ved, zd, cos, sin, window=window,
                                             layout=layout)
    grads = ops.attention_layer_ve_backward(qd, kd, vw, ved, zd, out, lse, dod, cos, sin,
                                            window=window, layout=layout)
    torch.cuda.synchronize()
    ref = oracle.attention_layer_ve_backward(f64(q), f64(k), f64(v), f64(ve), f64(z), f64(do),
                                             window=window)
    for name, g, r in zip(("dq", "dk", "dv", "dve", "dz"), grads, ref):
        err = float(np.max(np.abs(f64(from_layout(g, layout)) - r)))
        scale = max(1.0, float(np.max(np.abs(r))))
        say(f"   {name}: max|err|={err:.3e} max|ref|={np.max(np.abs(r)):.3e}")
        assert err <= BF16_TOL * scale, name


def test_layer_with_value_embedding_full_size():
    """The headline shape (B=16, H=12, T=1024, d=64, window 512): every gated row against the
    oracle, and sampled rows of sampled heads of the attention."""
    B, H, T, d, window = 16, 12, 1024, 64, 512
    say(f"layer with value embedding full size B={B} H={H} T={T} d={d} W={window}")
    q, k, v = inputs.make_qkv(2, 1)
    _, ve, z = gate_inputs(B, H, T, d, torch.bfloat16, 721, scale=1.0)
    cos, sin = ops.rope_table(T, d)
    out, lse, _, vw = ops.attn_fwd_qknorm_ve(q.cuda(), k.cuda(), v.cuda(), ve.cuda(), z.cuda(),
                                             cos, sin, window=window)
    torch.cuda.synchronize()
    ref_v = oracle.value_gate(f64(v), f64(ve), f64(z))
    assert_gate_close(vw.cpu(), ref_v, v, ve, "bf16")
    rng = np.random.default_rng(7)
    rows = np.array(sorted({0, 1, window, window + 1, T - 1} |
                           set(int(x) for x in rng.choice(T, 30, replace=False))))
    for b, h in ((0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = oracle.attention_layer_ve(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(ve[sl]),
                                           f64(z[sl]), window=window, rows=rows)
        eo = float(np.max(np.abs(f64(out[b, h, rows]) - ro[0, 0])))
        el = float(np.max(np.abs(f64(lse[b, h, rows]) - rl[0, 0])))
        vmax = float(np.max(np.abs(ref_v[b, h])))
        say(f"   head ({b},{h}) max|dO|={eo:.3e} max|dLSE|={el:.3e} max|v'|={vmax:.2f}")
        assert eo <= BF16_TOL * max(1.0, vmax / 4) and el <= BF16_TOL
