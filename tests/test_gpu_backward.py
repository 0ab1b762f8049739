"""GPU parity of the backward pass (attn_bwd_ex, attn_qknorm_rope_bwd_ex and the layer backward
built from them) against the fp64 oracle's gradients, through the C ABI.

Tolerances. The forward's bound (max-abs 2e-2 for bf16, 1e-5 for fp32 on outputs of magnitude
about 1) is applied to gradients relative to their size: max |gpu - oracle| <= tol *
max(1, max |oracle|). Every rounding on the bf16 path is relative (bf16 inputs, P and dS rounded
to bf16 with relative error <= 2^-9, fp32 accumulation, one final rounding of each gradient), so
the error scales with the gradient's magnitude. Every case prints its name before touching the GPU.
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
F32_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def to_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    x = x.to("cuda")
    return (x.transpose(1, 2) if layout == "bthd" else x).contiguous()


def from_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    return (x.transpose(1, 2) if layout == "bthd" else x).contiguous().cpu()


def check_grads(gpu, ref, tol, label=""):
    for name, g, r in zip(("dq", "dk", "dv"), gpu, ref):
        err = float(np.max(np.abs(f64(g) - r)))
        scale = max(1.0, float(np.max(np.abs(r))))
        say(f"   {label}{name}: max|err|={err:.3e} max|ref|={np.max(np.abs(r)):.3e}")
        assert err <= tol * scale, (name, err, scale)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    torch.cuda.synchronize()


# (dtype, d, B, H, H_kv, T, window, causal, layout): ragged tails, one-token sequences, windows
# 0, 1, mid and T - 1, non-causal, grouped heads, both layouts.
CASES = []
for _d in (32, 64, 128):
    CASES += [("bf16", _d, 1, 2, 2, 1, -1, 1, "bhtd"), ("bf16", _d, 1, 2, 2, 63, 1, 1, "bhtd"),
              ("bf16", _d, 2, 2, 1, 130, 0, 1, "bthd"), ("bf16", _d, 1, 4, 2, 257, 100, 1, "bhtd"),
              ("bf16", _d, 1, 2, 2, 200, -1, 0, "bhtd"), ("bf16", _d, 2, 4, 1, 300, -1, 1, "bthd"),
              ("bf16", _d, 1, 2, 2, 160, 159, 1, "bhtd")]
for _d in (16, 64, 128):
    CASES += [("f32", _d, 1, 2, 2, 37, -1, 1, "bhtd"), ("f32", _d, 2, 4, 2, 70, 9, 1, "bthd"),
              ("f32", _d, 1, 2, 1, 50, -1, 0, "bhtd")]


@pytest.mark.parametrize("dt,d,B,H,H_kv,T,window,causal,layout", CASES,
                         ids=[f"{c[0]}-d{c[1]}-B{c[2]}H{c[3]}k{c[4]}T{c[5]}-W{c[6]}-c{c[7]}-{c[8]}"
                              for c in CASES])
def test_attn_bwd_parity(dt, d, B, H, H_kv, T, window, causal, layout):
    say(f"attn_bwd {dt} d={d} B={B} H={H} H_kv={H_kv} T={T} W={window} causal={causal} {layout}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q = inputs.make_random((B, H, T, d), dtype, 401)
    k = inputs.make_random((B, H_kv, T, d), dtype, 402)
    v = inputs.make_random((B, H_kv, T, d), dtype, 403)
    do = inputs.make_random((B, H, T, d), dtype, 404)
    qd, kd, vd, dod = (to_layout(x, layout) for x in (q, k, v, do))
    out, lse = ops.attn_fwd(qd, kd, vd, window=window, causal=bool(causal), layout=layout)
    dq, dk, dv = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=window, causal=bool(causal),
                              layout=layout)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), window=window,
                                    causal=bool(causal))
    check_grads([from_layout(x, layout) for x in (dq, dk, dv)], ref,
                BF16_TOL if dt == "bf16" else F32_TOL)


@pytest.mark.parametrize("dt,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 16),
                                  ("f32", 64)])
@pytest.mark.parametrize("layout,H_kv", [("bhtd", 4), ("bthd", 2), ("bthd", 1)])
def test_qknorm_rope_bwd_parity(dt, d, layout, H_kv):
    B, H, T = 2, 4, 67
    say(f"qknorm_rope_bwd {dt} d={d} {layout} H_kv={H_kv}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q = inputs.make_random((B, H, T, d), dtype, 411) * 3
    k = inputs.make_random((B, H_kv, T, d), dtype, 412, "uniform")
    gq = inputs.make_random((B, H, T, d), dtype, 413)
    gk = inputs.make_random((B, H_kv, T, d), dtype, 414)
    cos, sin = ops.rope_table(T, d)
    qd, kd, gqd, gkd = (to_layout(x, layout) for x in (q, k, gq, gk))
    dq, dk = ops.qknorm_rope_bwd(qd, kd, gqd, gkd, cos, sin, layout=layout)
    _, dk_only = ops.qknorm_rope_bwd(None, kd, None, gkd, cos, sin, layout=layout)
    # in place
    gq2, gk2 = gqd.clone(), gkd.clone()
    ops.qknorm_rope_bwd(qd, kd, gq2, gk2, cos, sin, dq_out=gq2, dk_out=gk2, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(dk_only, dk) and torch.equal(gq2, dq) and torch.equal(gk2, dk)
    for g, x, gy in ((dq, q, gq), (dk, k, gk)):
        ref = oracle.qknorm_rope_backward(f64(x), f64(gy))
        err = np.abs(f64(from_layout(g, layout)) - ref)
        rowmax = np.max(np.abs(ref), axis=-1, keepdims=True)
        # fp32 arithmetic, one rounding of the result: relative to the row's largest entry
        bound = (2.0 ** -7 * rowmax + 2.0 ** -20) if dt == "bf16" else (1e-5 * rowmax + 1e-7)
        say(f"   max err {err.max():.3e}")
        assert np.all(err <= bound), f"max err {err.max()}"


@pytest.mark.parametrize("d,window,layout,H_kv", [(32, -1, "bhtd", 4), (64, 50, "bthd", 2),
                                                  (128, 90, "bhtd", 1), (64, -1, "bthd", 4)])
def test_layer_backward_parity(d, window, layout, H_kv):
    """Gradients of the raw q, k, v of one layer (fused forward, then the layer backward)."""
    B, H, T = 2, 4, 190
    say(f"layer backward d={d} W={window} {layout} H_kv={H_kv}")
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 421)
    k = inputs.make_random((B, H_kv, T, d), torch.bfloat16, 422)
    v = inputs.make_random((B, H_kv, T, d), torch.bfloat16, 423)
    do = inputs.make_random((B, H, T, d), torch.bfloat16, 424)
    cos, sin = ops.rope_table(T, d)
    qd, kd, vd, dod = (to_layout(x, layout) for x in (q, k, v, do))
    out, lse, _ = ops.attn_fwd_qknorm(qd, kd, vd, cos, sin, window=window, layout=layout)
    dq, dk, dv = ops.attention_layer_backward(qd, kd, vd, out, lse, dod, cos, sin, window=window,
                                              layout=layout)
    torch.cuda.synchronize()
    ref = oracle.attention_layer_backward(f64(q), f64(k), f64(v), f64(do), window=window)
    check_grads([from_layout(x, layout) for x in (dq, dk, dv)], ref, BF16_TOL)


def test_bwd_layout_and_determinism_bitwise():
    """[B][T][H][d] gives the [B][H][T][d] gradients transposed, bit for bit; repeated calls
    give the same bits; a window of T - 1 equals full causal bit for bit."""
    B, H, H_kv, T, d = 2, 4, 2, 333, 64
    say("bwd layout / determinism / window T-1")
    q, do = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (431, 434))
    k, v = (inputs.make_random((B, H_kv, T, d), torch.bfloat16, s) for s in (432, 433))
    res = {}
    for layout in ("bhtd", "bthd"):
        qd, kd, vd, dod = (to_layout(x, layout) for x in (q, k, v, do))
        out, lse = ops.attn_fwd(qd, kd, vd, window=40, layout=layout)
        g1 = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=40, layout=layout)
        g2 = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=40, layout=layout)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(g1, g2))
        res[layout] = [from_layout(x, layout) for x in g1]
    assert all(torch.equal(a, b) for a, b in zip(res["bhtd"], res["bthd"]))
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    out, lse = ops.attn_fwd(qd, kd, vd, window=-1)
    ga = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=-1)
    gb = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=T - 1)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ga, gb))


def test_bwd_window_zero_closed_form():
    """Window 0: every query sees only its own key, so dq = dk = 0 exactly and dv = dout
    (P = 1 exactly: lse = s_ii)."""
    B, H, T, d = 1, 2, 100, 64
    say("bwd window 0")
    q, k, v, do = (inputs.make_random((B, H, T, d), torch.bfloat16, s).cuda()
                   for s in (441, 442, 443, 444))
    out, lse = ops.attn_fwd(q, k, v, window=0)
    dq, dk, dv = ops.attn_bwd(q, k, v, out, lse, do, window=0)
    torch.cuda.synchronize()
    assert float(dq.float().abs().max()) <= 2e-2 and float(dk.float().abs().max()) <= 2e-2
    assert float((dv.float() - do.float()).abs().max()) <= 2e-2 * float(do.float().abs().max())


def test_bwd_outputs_stay_inside_their_buffers():
    B, H, H_kv, T, d = 1, 4, 2, 150, 64
    say("bwd canaries")
    q, do = (inputs.make_random((B, T, H, d), torch.bfloat16, s).cuda() for s in (451, 454))
    k, v = (inputs.make_random((B, T, H_kv, d), torch.bfloat16, s).cuda() for s in (452, 453))
    out, lse = ops.attn_fwd(q, k, v, window=30, layout="bthd")
    pad = 4096
    bufs = {}
    views = {}
    for name, like in (("dq", q), ("dk", k), ("dv", v)):
        big = torch.full((like.numel() + 2 * pad,), 3.0, dtype=like.dtype, device="cuda")
        bufs[name] = big
        views[name] = big[pad:pad + like.numel()].view(like.shape)
    dbig = torch.full((B * H * T + 2 * pad,), 3.0, dtype=torch.float32, device="cuda")
    delta = dbig[pad:pad + B * H * T].view(B, H, T)
    ops.attn_bwd(q, k, v, out, lse, do, window=30, dq=views["dq"], dk=views["dk"],
                 dv=views["dv"], delta=delta, layout="bthd")
    torch.cuda.synchronize()
    for big in list(bufs.values()) + [dbig]:
        assert bool((big[:pad] == 3.0).all()) and bool((big[-pad:] == 3.0).all())


@pytest.mark.parametrize("dt,d,layout", [("bf16", 64, "bthd"), ("bf16", 128, "bhtd"),
                                          ("bf16", 32, "bhtd"), ("f32", 16, "bthd")])
def test_bwd_delta_by_product(dt, d, layout):
    """delta (written by the dQ kernel in bf16, by its own kernel in fp32) is rowsum(dout * out)
    of the exact values handed over, within fp32 summation rounding; ragged T = 150."""
    B, H, H_kv, T = 2, 4, 2, 150
    say(f"bwd delta {dt} d={d} {layout}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    shp = lambda h: (B, T, h, d) if layout == "bthd" else (B, h, T, d)
    q, do = (inputs.make_random(shp(H), dtype, s).cuda() for s in (471, 474))
    k, v = (inputs.make_random(shp(H_kv), dtype, s).cuda() for s in (472, 473))
    out, lse = ops.attn_fwd(q, k, v, window=40, layout=layout)
    delta = torch.full((B, H, T), 7.0, dtype=torch.float32, device="cuda")
    ops.attn_bwd(q, k, v, out, lse, do, window=40, delta=delta, layout=layout)
    torch.cuda.synchronize()
    ref = np.sum(f64(out) * f64(do), axis=-1)  # [B, T, H] or [B, H, T]
    if layout == "bthd":
        ref = ref.transpose(0, 2, 1)
    err = np.abs(f64(delta) - ref) / np.maximum(1.0, np.abs(ref))
    say(f"   max rel err {float(err.max()):.2e}")
    assert float(err.max()) <= 1e-5


def test_bwd_full_size_sampled():
    """The headline shape's first two layers (windows 512 and, as the last layer, 1024) at full
    size (B=16, H=12, T=1024, d=64); the oracle checks sampled heads in full."""
    w = inputs.workload("andrea120m_sssl")
    rng = np.random.default_rng(5)
    for layer, window in ((0, 512), (3, 1024)):
        say(f"bwd full size {w.name} layer={layer} W={window}")
        q, k, v = inputs.make_qkv(inputs.HEADLINE, layer)
        do = inputs.make_random(q.shape, torch.bfloat16, 460 + layer)
        qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
        out, lse = ops.attn_fwd(qd, kd, vd, window=window)
        dq, dk, dv = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=window)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))):
            sl = (slice(b, b + 1), slice(h, h + 1))
            ref = oracle.attention_backward(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]),
                                            window=window)
            check_grads([x[sl].cpu() for x in (dq, dk, dv)], ref, BF16_TOL, f"({b},{h}) ")
        del dq, dk, dv, out, lse


def test_bwd_validation_with_real_buffers():
    lib = _lib.load()
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    k, v, out, do, dq, dk, dv = (torch.zeros_like(q) for _ in range(7))
    lse = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    delta = torch.zeros_like(lse)
    P = [x.data_ptr() for x in (q, k, v, out, do)]
    args = lambda **kw: dict(dict(zip(("q", "k", "v", "out", "do"), P), lse=lse.data_ptr(),
                                  delta=delta.data_ptr(), dq=dq.data_ptr(), dk=dk.data_ptr(),
                                  dv=dv.data_ptr()), **kw)

    def call(a, **kw):
        d = dict(B=1, H=2, T=64, d=64, window=-1, causal=1, dtype=_lib.ATTN_BF16)
        d.update(kw)
        return lib.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["delta"],
                            a["dq"], a["dk"], a["dv"], d["B"], d["H"], d["T"], d["d"],
                            d["window"], d["causal"], d["dtype"], None)

    assert call(args(lse=None)) == _lib.ATTN_ERR_NULL
    assert call(args(dq=q.data_ptr())) == _lib.ATTN_ERR_ALIAS
    assert call(args(dk=dv.data_ptr())) == _lib.ATTN_ERR_ALIAS
    assert call(args(delta=lse.data_ptr())) == _lib.ATTN_ERR_ALIAS
    assert call(args(), d=16) == _lib.ATTN_ERR_HEAD_DIM
    assert call(args(), causal=0, window=3) == _lib.ATTN_ERR_WINDOW
    assert call(args()) == _lib.ATTN_OK
    torch.cuda.synchronize()


def test_grouped_order_with_a_partial_group_sampled():
    """520 heads at T=1024, d=128: the tiles of all heads (0.5 MB each) exceed the cache budget, so
    the d=128 forward and both backward kernels take the head-grouped order, with a last group of
    8 heads. Sampled heads from the first group, the partial last group and a random one are
    checked against the oracle (forward outputs and all three gradients)."""
    B, H, T, d, window = 65, 8, 1024, 128, 300
    say(f"grouped order B={B} H={H} T={T} d={d} W={window}")
    q, k, v, do = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (471, 472, 473, 474))
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    out, lse = ops.attn_fwd(qd, kd, vd, window=window)
    dq, dk, dv = ops.attn_bwd(qd, kd, vd, out, lse, dod, window=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    heads = [(0, 0), (B - 1, H - 1), (B - 1, 0), (int(rng.integers(B)), int(rng.integers(H)))]
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = oracle.attention(f64(q[sl]), f64(k[sl]), f64(v[sl]), window=window)
        eo = float(np.max(np.abs(f64(out[sl]) - ro)))
        say(f"   head ({b},{h}) forward max|dO|={eo:.3e}")
        assert eo <= BF16_TOL
        ref = oracle.attention_backward(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]),
                                        window=window)
        check_grads([x[sl].cpu() for x in (dq, dk, dv)], ref, BF16_TOL, f"({b},{h}) ")
