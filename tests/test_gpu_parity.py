"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on identical inputs.

Tolerances (max-abs against the oracle): bf16 paths 2e-2 on outputs; fp32 paths 1e-5. The bf16
budget comes from rounding q, k (after the prologue) to bf16, rounding the softmax weights to
bf16 before the P v product and rounding the output to bf16; the tests also print the measured
error. Every case prints its name before touching the GPU.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_qk_amd import _lib, inputs, ops

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5
# LSE on the bf16 path: the row sums add the bf16-rounded weights (the values the P V product
# uses), each within a relative 2^-9 of the exact weight, so ln of the sum moves by at most 2^-9;
# 2^-8 leaves room for the fp32 arithmetic around it.
BF16_LSE_TOL = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    torch.cuda.synchronize()


def run_layer(q, k, v, window, eps=1e-6, causal=True):
    """Prologue + attention on the GPU for CPU tensors q, k, v; returns CPU tensors."""
    T, d = q.shape[2], q.shape[3]
    cos, sin = ops.rope_table(T, d)
    qd, kd, vd = dev(q), dev(k), dev(v)
    qn, kn = ops.qknorm_rope(qd, kd, cos, sin, eps)
    out, lse = ops.attn_fwd(qn, kn, vd, window=window, causal=causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# ---------------------------------------------------------------------------------------------
# RoPE table and prologue
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,d", [(1, 16), (3, 32), (64, 16), (1024, 64), (8192, 128)])
def test_rope_table(T, d):
    say(f"rope_table T={T} d={d}")
    cos, sin = ops.rope_table(T, d)
    torch.cuda.synchronize()
    rc, rs = oracle.rope_cos_sin(T, d)
    assert np.max(np.abs(f64(cos) - rc)) <= 1e-7
    assert np.max(np.abs(f64(sin) - rs)) <= 1e-7


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 7), (1, 2, 130)], ids=str)
def test_qknorm_rope_parity(dtype, d, shape):
    B, H, T = shape
    say(f"qknorm_rope {dtype} d={d} B={B} H={H} T={T}")
    q = inputs.make_random((B, H, T, d), dtype, 100 + d) * 3
    k = inputs.make_random((B, H, T, d), dtype, 200 + d, "uniform")
    cos, sin = ops.rope_table(T, d)
    qn, kn = ops.qknorm_rope(dev(q), dev(k), cos, sin, 1e-6)
    torch.cuda.synchronize()
    rq, rk = oracle.qknorm_rope(f64(q), f64(k), 1e-6)
    for g, r in ((qn, rq), (kn, rk)):
        err = np.abs(f64(g) - r)
        if dtype == torch.bfloat16:
            bound = 2.0 ** -8 * np.abs(r) + 2.0 ** -20
        else:
            bound = 2e-6 * np.abs(r) + 1e-6
        assert np.all(err <= bound), f"max err {err.max()}"
    # in place gives the same bits
    qd, kd = dev(q), dev(k)
    ops.qknorm_rope(qd, kd, cos, sin, 1e-6, q_out=qd, k_out=kd)
    torch.cuda.synchronize()
    assert torch.equal(qd, qn) and torch.equal(kd, kn)


# ---------------------------------------------------------------------------------------------
# Attention on raw inputs (no prologue)
# ---------------------------------------------------------------------------------------------

RAW_CASES = []
for _d in (32, 64, 128):
    for _T in (1, 3, 63, 65, 130, 300):
        for _w, _c in ((-1, 1), (0, 1), (1, 1), (17, 1), (100, 1), (_T - 1, 1), (_T + 5, 1), (-1, 0)):
            if _w >= _T + 5 and _T > 3:
                continue
            RAW_CASES.append(("bf16", _d, _T, _w, _c))
for _d in (16, 32, 64, 128):
    for _T in (1, 5, 64, 97):
        for _w, _c in ((-1, 1), (0, 1), (9, 1), (-1, 0)):
            RAW_CASES.append(("f32", _d, _T, _w, _c))


@pytest.mark.parametrize("dt,d,T,window,causal", RAW_CASES,
                         ids=[f"{c[0]}-d{c[1]}-T{c[2]}-W{c[3]}-c{c[4]}" for c in RAW_CASES])
def test_attn_fwd_raw_parity(dt, d, T, window, causal):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H = 1, 2
    say(f"attn_fwd raw {dt} d={d} T={T} W={window} causal={causal}")
    seed = 1000 * d + T
    q = inputs.make_random((B, H, T, d), dtype, seed)
    k = inputs.make_random((B, H, T, d), dtype, seed + 1)
    v = inputs.make_random((B, H, T, d), dtype, seed + 2)
    out, lse = ops.attn_fwd(dev(q), dev(k), dev(v), window=window, causal=bool(causal))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), window=window, causal=bool(causal))
    eo = np.max(np.abs(f64(out) - ro))
    el = np.max(np.abs(f64(lse) - rl))
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    assert eo <= tol
    assert el <= (BF16_LSE_TOL if dt == "bf16" else F32_TOL)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_attn_fwd_peaky_scores(d):
    """Keys close to scaled copies of the queries: large, sharply peaked scores exercise the
    running-maximum rescaling."""
    say(f"attn_fwd peaky d={d}")
    B, H, T = 1, 2, 257
    q = inputs.make_random((B, H, T, d), torch.float32, 7)
    noise = inputs.make_random((B, H, T, d), torch.float32, 8)
    k = (4.0 * q + 0.1 * noise).to(torch.bfloat16)
    q = q.to(torch.bfloat16)
    v = inputs.make_random((B, H, T, d), torch.bfloat16, 9)
    for window in (-1, 31):
        out, lse = ops.attn_fwd(dev(q), dev(k), dev(v), window=window)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(f64(q), f64(k), f64(v), window=window)
        eo = np.max(np.abs(f64(out) - ro))
        say(f"   W={window} max|dO|={eo:.3e} max|dLSE|={np.max(np.abs(f64(lse) - rl)):.3e}")
        assert eo <= BF16_TOL
        assert np.max(np.abs(f64(lse) - rl)) <= BF16_LSE_TOL * max(1.0, np.max(np.abs(rl)))


# ---------------------------------------------------------------------------------------------
# Whole layer (prologue + attention) per workload
# ---------------------------------------------------------------------------------------------

def reduced_shape(w):
    # several query tiles and a ragged tail, small enough for the oracle in seconds
    return (1, 2, min(w.T, 520), w.d)


@pytest.mark.parametrize("index", range(len(inputs.WORKLOADS)),
                         ids=[w.name for w in inputs.WORKLOADS])
def test_layer_parity_reduced(index):
    w = inputs.WORKLOADS[index]
    shape = reduced_shape(w)
    T = shape[2]
    wins = oracle.sssl_windows(T, w.n_layer, w.pattern)
    assert ops.sssl_windows(T, w.n_layer, w.pattern) == wins
    for layer, window in enumerate(wins):
        say(f"layer parity reduced {w.name} shape={shape} layer={layer} W={window}")
        q, k, v = inputs.make_qkv(index, layer, shape)
        out, lse = run_layer(q, k, v, window)
        ro, rl = oracle.attention_layer(f64(q), f64(k), f64(v), window=window)
        eo = np.max(np.abs(f64(out) - ro))
        el = np.max(np.abs(f64(lse) - rl))
        say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        tol = BF16_TOL if w.dtype == "bf16" else F32_TOL
        assert eo <= tol
        assert el <= (2e-2 if w.dtype == "bf16" else F32_TOL)


SAMPLE_HEADS = 3
SAMPLE_ROWS = 48


def sample_rows(T, window, rng):
    fixed = {0, 1, 2, T - 1, T - 2, T // 2, T // 2 + 1}
    if window >= 0:
        fixed |= {min(T - 1, window - 1), min(T - 1, window), min(T - 1, window + 1)}
    extra = rng.choice(T, size=SAMPLE_ROWS - len(fixed), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)))


@pytest.mark.parametrize("index", range(len(inputs.WORKLOADS)),
                         ids=[w.name for w in inputs.WORKLOADS])
def test_layer_parity_full_size_sampled(index):
    """Every layer of the workload at its real shape, launched as the bench launches it; the
    oracle checks sampled rows of sampled heads, and the outputs, which start as NaN, must all be
    written (the kernel's item order reaches every (head, query block))."""
    w = inputs.WORKLOADS[index]
    wins = ops.sssl_windows(w.T, w.n_layer, w.pattern)
    rng = np.random.default_rng(index)
    cos, sin = ops.rope_table(w.T, w.d)
    for layer, window in enumerate(wins):
        say(f"layer parity full {w.name} B={w.B} H={w.H} T={w.T} d={w.d} layer={layer} W={window}")
        q, k, v = inputs.make_qkv(index, layer)
        qd, kd, vd = dev(q), dev(k), dev(v)
        qn, kn = ops.qknorm_rope(qd, kd, cos, sin, 1e-6)
        out0 = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device="cuda")
        lse0 = torch.full((w.B, w.H, w.T), float("nan"), dtype=torch.float32, device="cuda")
        out, lse = ops.attn_fwd(qn, kn, vd, window=window, out=out0, lse=lse0)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
        heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H)))
                                               for _ in range(SAMPLE_HEADS - 2)]
        rows = sample_rows(w.T, window, rng)
        worst_o = worst_l = 0.0
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            ro, rl = oracle.attention_layer(f64(q[sl]), f64(k[sl]), f64(v[sl]), window=window,
                                            rows=rows)
            go = f64(out[b, h, rows])
            gl = f64(lse[b, h, rows])
            worst_o = max(worst_o, float(np.max(np.abs(go - ro[0, 0]))))
            worst_l = max(worst_l, float(np.max(np.abs(gl - rl[0, 0]))))
        say(f"   max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
        tol = BF16_TOL if w.dtype == "bf16" else F32_TOL
        assert worst_o <= tol
        assert worst_l <= (2e-2 if w.dtype == "bf16" else F32_TOL)
        del qd, kd, vd, qn, kn, out, lse


# ---------------------------------------------------------------------------------------------
# Closed forms and invariants on the GPU
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt,d,qscale", [("f32", 16, 2.0), ("bf16", 64, 4.0)])
def test_worked_example_on_gpu(dt, d, qscale):
    """The query and three keys of "Lendo uma Projeção", zero-padded to d, with the query scaled
    so that q.k / sqrt(d) equals the page's q.k / 2 exactly; V = e_j. Row 0 must give the
    closed-form weights (sqrt(e), sqrt(e), 1) / (2 sqrt(e) + 1) and LSE ln(2 sqrt(e) + 1)."""
    say(f"worked example {dt} d={d}")
    from tests.oracle_pins import worked_example_inputs
    g = worked_example_inputs()
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    T = 3
    q = torch.zeros((1, 1, T, d), dtype=torch.float32)
    k = torch.zeros((1, 1, T, d), dtype=torch.float32)
    v = torch.zeros((1, 1, T, d), dtype=torch.float32)
    q[0, 0, 0, :4] = torch.tensor(g["q"], dtype=torch.float32) * qscale
    k[0, 0, :, :4] = torch.tensor(g["keys"], dtype=torch.float32)
    for j in range(3):
        v[0, 0, j, j] = 1.0
    assert math.sqrt(d) / qscale == g["sqrt_d_k"]
    out, lse = ops.attn_fwd(dev(q.to(dtype)), dev(k.to(dtype)), dev(v.to(dtype)), window=-1,
                            causal=False)
    torch.cuda.synchronize()
    se = math.exp(0.5)
    w = np.array([se, se, 1.0]) / (2 * se + 1)
    o = f64(out)[0, 0]
    tol = 4e-3 if dt == "bf16" else 1e-6
    assert np.max(np.abs(o[0, :3] - w)) <= tol
    assert np.all(o[0, 3:] == 0)
    # bf16: the row sum adds the bf16-rounded weights (e^-0.5 rounds to 0.60546875)
    ltol = BF16_LSE_TOL if dt == "bf16" else 1e-5
    assert abs(float(lse[0, 0, 0]) - math.log(2 * se + 1)) <= ltol
    assert np.max(np.abs(o[1:, :3] - 1 / 3)) <= tol
    assert np.max(np.abs(f64(lse)[0, 0, 1:] - math.log(3))) <= 1e-5


@pytest.mark.parametrize("dt,d", [("f32", 16), ("bf16", 32), ("bf16", 64), ("bf16", 128)])
def test_zero_query_closed_form(dt, d):
    """Raw q = 0 through the layer: the prologue maps it to 0, all scores are 0, O_i is the mean
    of the visible v_j and LSE_i = ln(min(i, W) + 1) (inclusive window)."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, T = 1, 2, 300
    q = torch.zeros((B, H, T, d), dtype=dtype)
    k = inputs.make_random((B, H, T, d), dtype, 11)
    v = inputs.make_random((B, H, T, d), dtype, 12)
    vv = f64(v)
    for window in (-1, 0, 1, 63, 64, 100, 299):
        say(f"zero query {dt} d={d} W={window}")
        out, lse = run_layer(q, k, v, window)
        n = np.arange(T) + 1 if window < 0 else np.minimum(np.arange(T), window) + 1
        np.testing.assert_allclose(f64(lse)[0, 0], np.log(n), rtol=0, atol=2e-6)
        cs = np.cumsum(vv, axis=2)
        lo = np.arange(T) + 1 - n
        ref = (cs[:, :, np.arange(T)] - np.where(lo[None, None, :, None] > 0,
                                                 cs[:, :, np.maximum(lo - 1, 0)], 0.0)) / n[:, None]
        tol = 8e-3 if dt == "bf16" else 2e-6
        assert np.max(np.abs(f64(out) - ref)) <= tol


@pytest.mark.parametrize("d", [32, 64, 128])
def test_masked_keys_have_no_influence_bitwise(d):
    """Rewriting k, v at keys a row cannot see (future keys, keys beyond the window) to +-1e4
    leaves that row's output and LSE bitwise unchanged."""
    B, H, T = 1, 1, 400
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 21)
    k = inputs.make_random((B, H, T, d), torch.bfloat16, 22)
    v = inputs.make_random((B, H, T, d), torch.bfloat16, 23)
    for window in (-1, 70):
        out, lse = ops.attn_fwd(dev(q), dev(k), dev(v), window=window)
        # rows at the edges of the waves' 32-row blocks, the 64-key tiles and the 128-row items
        for i in (0, 5, 31, 32, 57, 63, 64, 95, 96, 100, 127, 128, 200, 255, 256, 383, 384, 399):
            say(f"mask perturbation d={d} W={window} row={i}")
            k2, v2 = k.clone(), v.clone()
            j = torch.arange(T)
            hidden = (j > i) | ((i - j > window) if window >= 0 else torch.zeros(T, dtype=torch.bool))
            sign = torch.where(j % 2 == 0, 1.0, -1.0)[:, None]
            k2[0, 0][hidden] = (1e4 * sign[hidden]).to(torch.bfloat16).expand(-1, d)
            v2[0, 0][hidden] = (-1e4 * sign[hidden]).to(torch.bfloat16).expand(-1, d)
            out2, lse2 = ops.attn_fwd(dev(q), dev(k2), dev(v2), window=window)
            torch.cuda.synchronize()
            assert torch.equal(out2[0, 0, i], out[0, 0, i])
            assert torch.equal(lse2[0, 0, i], lse[0, 0, i])


@pytest.mark.parametrize("dt,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 16)])
def test_window_T_is_full_causal_bitwise(dt, d):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, T = 2, 2, 333
    say(f"window=T bitwise {dt} d={d}")
    q, k, v = (dev(inputs.make_random((B, H, T, d), dtype, s)) for s in (31, 32, 33))
    ref_o, ref_l = ops.attn_fwd(q, k, v, window=-1)
    for window in (T - 1, T, T + 100, 1 << 30):
        o, l = ops.attn_fwd(q, k, v, window=window)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), window


@pytest.mark.parametrize("index", [2, 4], ids=["andrea120m_sssl", "long_sssl"])
def test_deterministic_bitwise(index):
    """Two runs of the same layer give identical bits (no atomics, no order-dependent sums)."""
    w = inputs.WORKLOADS[index]
    shape = (2, 2, min(w.T, 2048), w.d)
    q, k, v = (dev(x) for x in inputs.make_qkv(index, 0, shape))
    for window in (shape[2] // 2, -1):
        say(f"determinism {w.name} W={window}")
        a = ops.attn_fwd(q, k, v, window=window)
        b = ops.attn_fwd(q, k, v, window=window)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dt,d", [("bf16", 64), ("f32", 16)])
def test_outputs_stay_inside_their_buffers(dt, d):
    """Canary regions around out and lse are untouched."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, T = 1, 3, 197
    say(f"canaries {dt} d={d}")
    q, k, v = (dev(inputs.make_random((B, H, T, d), dtype, s)) for s in (41, 42, 43))
    n = B * H * T * d
    pad = 64
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=dtype, device="cuda")
    lbuf = torch.full((B * H * T + 2 * pad,), -3.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n].view(B, H, T, d)
    lse = lbuf[pad:pad + B * H * T].view(B, H, T)
    ops.attn_fwd(q, k, v, window=50, out=out, lse=lse)
    cos, sin = ops.rope_table(T, d)
    qb = torch.full((n + 2 * pad,), 5.0, dtype=dtype, device="cuda")
    qo = qb[pad:pad + n].view(B, H, T, d)
    ops.qknorm_rope(q, k, cos, sin, q_out=qo)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 7.0) and torch.all(obuf[pad + n:] == 7.0)
    assert torch.all(lbuf[:pad] == -3.0) and torch.all(lbuf[pad + B * H * T:] == -3.0)
    assert torch.all(qb[:pad] == 5.0) and torch.all(qb[pad + n:] == 5.0)


def test_validation_with_real_buffers():
    """Invalid calls return their status code and leave the output untouched."""
    lib = _lib.load()
    q, k, v = (dev(inputs.make_random((1, 2, 64, 64), torch.bfloat16, s)) for s in (1, 2, 3))
    out = torch.full_like(q, 3.0)
    s = torch.cuda.current_stream().cuda_stream
    cases = [
        (dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
        (dict(causal=0, window=3), _lib.ATTN_ERR_WINDOW),
        (dict(T=0), _lib.ATTN_ERR_SHAPE),
        (dict(dtype=5), _lib.ATTN_ERR_DTYPE),
        (dict(out=q.data_ptr()), _lib.ATTN_ERR_ALIAS),
    ]
    for kw, code in cases:
        a = dict(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), out=out.data_ptr(), lse=None, B=1,
                 H=2, T=64, d=64, window=-1, causal=1, dtype=0)
        a.update(kw)
        say(f"validation {kw}")
        rc = lib.attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["T"],
                          a["d"], a["window"], a["causal"], a["dtype"], s)
        assert rc == code
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    with pytest.raises(_lib.AttnError):
        ops.attn_fwd(q, k, v, window=3, causal=False)
