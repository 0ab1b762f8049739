"""GPU parity of attn_fwd_qknorm (QK-norm + RoPE of raw q, k and attention in one call) against
the fp64 oracle's attention layer, through the C ABI.

Tolerances match the two-call path: max-abs 2e-2 on outputs and LSE. The bf16 budget: k is
normalised and rounded to bf16 once, q's normalised row is scaled by log2(e)/sqrt(d) and
rounded to bf16 once, the softmax weights are rounded to bf16 before the P v product and the
output is rounded to bf16. Every case prints its name before touching the GPU.
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
LSE_TOL = 2e-2


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


def fused(q, k, v, window, causal=True, eps=1e-6):
    T, d = q.shape[2], q.shape[3]
    cos, sin = ops.rope_table(T, d)
    out, lse, kw = ops.attn_fwd_qknorm(dev(q), dev(k), dev(v), cos, sin, window=window,
                                       causal=causal, eps=eps)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kw.cpu()


def check(out, lse, q, k, v, window, causal=True, eps=1e-6, rows=None):
    ro, rl = oracle.attention_layer(f64(q), f64(k), f64(v), window=window, causal=causal,
                                    eps=eps, rows=rows)
    go, gl = f64(out), f64(lse)
    if rows is not None:
        go, gl = go[:, :, rows], gl[:, :, rows]
    eo = float(np.max(np.abs(go - ro)))
    el = float(np.max(np.abs(gl - rl)))
    # the unavoidable part: the exact result rounded to bf16, against itself
    floor = float(np.max(np.abs(f64(torch.from_numpy(ro).to(torch.bfloat16)) - ro)))
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e} (bf16 rounding floor of O {floor:.3e})")
    assert eo <= BF16_TOL
    assert el <= LSE_TOL
    return eo, el, floor


# (d, B, H, T, window, causal): ragged tails, one-token sequences, windows of 0, 1, mid and
# >= T - 1, non-causal, and more items than the GPU holds workgroups at once.
CASES = []
for d in (32, 64, 128):
    CASES += [(d, 1, 1, 1, -1, 1), (d, 1, 2, 63, 1, 1), (d, 2, 1, 130, 0, 1),
              (d, 1, 3, 257, 100, 1), (d, 1, 2, 300, -1, 0), (d, 2, 2, 384, -1, 1),
              (d, 1, 1, 200, 199, 1)]
CASES += [(64, 40, 16, 256, 128, 1), (32, 64, 12, 200, -1, 1)]


@pytest.mark.parametrize("d,B,H,T,window,causal", CASES,
                         ids=[f"d{c[0]}-B{c[1]}H{c[2]}T{c[3]}-W{c[4]}-c{c[5]}" for c in CASES])
def test_fused_parity(d, B, H, T, window, causal):
    say(f"fused parity d={d} B={B} H={H} T={T} W={window} causal={causal}")
    q, k, v = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (101, 102, 103))
    out, lse, _ = fused(q, k, v, window, bool(causal))
    rows = None
    if B * H * T > 20000:  # large cases: the oracle checks sampled rows
        rows = np.unique(np.r_[0, 1, T // 2, T - 1, np.arange(0, T, 37)])
        sl = (slice(0, 1), slice(0, 1))
        check(out[sl], lse[sl], q[sl], k[sl], v[sl], window, bool(causal), rows=rows)
        sl = (slice(B - 1, B), slice(H - 1, H))
        check(out[sl], lse[sl], q[sl], k[sl], v[sl], window, bool(causal), rows=rows)
    else:
        check(out, lse, q, k, v, window, bool(causal))


@pytest.mark.parametrize("index", [i for i, w in enumerate(inputs.WORKLOADS) if w.dtype == "bf16"],
                         ids=[w.name for w in inputs.WORKLOADS if w.dtype == "bf16"])
def test_fused_layer_parity_reduced(index):
    w = inputs.WORKLOADS[index]
    shape = (1, 2, min(w.T, 520), w.d)
    T = shape[2]
    for layer, window in enumerate(oracle.sssl_windows(T, w.n_layer, w.pattern)):
        say(f"fused layer parity reduced {w.name} shape={shape} layer={layer} W={window}")
        q, k, v = inputs.make_qkv(index, layer, shape)
        out, lse, _ = fused(q, k, v, window)
        check(out, lse, q, k, v, window)


@pytest.mark.parametrize("index", [i for i, w in enumerate(inputs.WORKLOADS) if w.dtype == "bf16"],
                         ids=[w.name for w in inputs.WORKLOADS if w.dtype == "bf16"])
def test_fused_layer_parity_full_size_sampled(index):
    """Every layer at the workload's real shape, launched as the bench launches it; the oracle
    checks sampled rows of sampled heads. The outputs start as NaN and must all be written: every
    (head, query block) item is reached by the kernel's item order, whichever order the launch
    takes (at these shapes the head-grouped one for d <= 64 where the heads divide into rounds)."""
    w = inputs.WORKLOADS[index]
    rng = np.random.default_rng(100 + index)
    cos, sin = ops.rope_table(w.T, w.d)
    for layer, window in enumerate(ops.sssl_windows(w.T, w.n_layer, w.pattern)):
        say(f"fused layer parity full {w.name} B={w.B} H={w.H} T={w.T} d={w.d} layer={layer} "
            f"W={window}")
        q, k, v = inputs.make_qkv(index, layer)
        out0 = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        lse0 = torch.full((w.B, w.H, w.T), float("nan"), dtype=torch.float32, device="cuda")
        out, lse, _ = ops.attn_fwd_qknorm(dev(q), dev(k), dev(v), cos, sin, window=window,
                                          out=out0, lse=lse0)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
        heads = [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]
        fixed = {0, 1, w.T - 1, w.T // 2, min(w.T - 1, window), min(w.T - 1, window + 1)}
        rows = np.array(sorted(fixed | set(int(x) for x in rng.choice(w.T, 40, replace=False))))
        worst = [0.0, 0.0, 0.0]
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            res = check(out[sl].cpu(), lse[sl].cpu(), q[sl], k[sl], v[sl], window, rows=rows)
            worst = [max(a, r) for a, r in zip(worst, res)]
        say(f"   {w.name} layer {layer}: worst max|dO|={worst[0]:.3e} max|dLSE|={worst[1]:.3e} "
            f"floor {worst[2]:.3e}")
        del out, lse



@pytest.mark.parametrize("d,window", [(64, 512), (64, -1), (32, 512), (32, -1)])
@pytest.mark.parametrize("write_k", [True, False])
def test_head_grouped_order_ragged(d, window, write_k):
    """192 heads with a ragged length (T = 1000, eight query blocks, the last one partial): the
    launch takes the head-grouped item order (whole rounds of heads, per-round block
    permutations) at d = 64 with either mask and at d = 32 causal, and the snake order at d = 32
    with W = 512 (two rounds cannot balance that mask's blocks within 8 %). Every output must be
    written (they start as NaN) and sampled rows of sampled heads match the oracle, with the keys
    normalised by the k pass or inside the kernel."""
    B, H, T = 16, 12, 1000
    say(f"head-grouped order ragged d={d} W={window} write_k={write_k}")
    q, k, v = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (301, 302, 303))
    cos, sin = ops.rope_table(T, d)
    out0 = torch.full((B, H, T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse0 = torch.full((B, H, T), float("nan"), dtype=torch.float32, device="cuda")
    out, lse, _ = ops.attn_fwd_qknorm(dev(q), dev(k), dev(v), cos, sin, window=window,
                                      out=out0, lse=lse0, write_k=write_k)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(7)
    rows = np.array(sorted({0, 1, 127, 128, 895, 896, 999} |
                           set(int(x) for x in rng.choice(T, 24, replace=False))))
    for b, h in ((0, 0), (B - 1, H - 1), (5, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        check(out[sl].cpu(), lse[sl].cpu(), q[sl], k[sl], v[sl], window, rows=rows)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fused_matches_two_call_path_and_k_work(d):
    """k_work equals attn_qknorm_rope's k output bitwise; out and lse stay within the bf16
    budget of the two-call path (they differ only in how q is rounded and in the softmax's
    offset)."""
    B, H, T = 2, 3, 333
    say(f"fused vs two-call d={d}")
    q, k, v = (dev(inputs.make_random((B, H, T, d), torch.bfloat16, s)) for s in (111, 112, 113))
    cos, sin = ops.rope_table(T, d)
    for window in (-1, 40):
        out, lse, kw = ops.attn_fwd_qknorm(q, k, v, cos, sin, window=window)
        qn, kn = ops.qknorm_rope(q, k, cos, sin)
        o2, l2 = ops.attn_fwd(qn, kn, v, window=window)
        torch.cuda.synchronize()
        assert torch.equal(kw, kn)
        assert float((out.float() - o2.float()).abs().max()) <= BF16_TOL
        assert float((lse - l2).abs().max()) <= LSE_TOL


@pytest.mark.parametrize("d", [32, 64, 128])
def test_k_only_prologue_and_qnorm_entry(d):
    """attn_qknorm_rope with q = NULL writes the same k as the two-tensor call, and
    attn_fwd_qnorm on those keys gives attn_fwd_qknorm's outputs bitwise (it is that call's
    second kernel)."""
    B, H, T = 2, 2, 300
    say(f"k-only prologue + attn_fwd_qnorm d={d}")
    q, k, v = (dev(inputs.make_random((B, H, T, d), torch.bfloat16, s)) for s in (171, 172, 173))
    cos, sin = ops.rope_table(T, d)
    _, kn_both = ops.qknorm_rope(q, k, cos, sin)
    qo, kn_only = ops.qknorm_rope(None, k, cos, sin)
    assert qo is None
    out, lse = ops.attn_fwd_qnorm(q, kn_only, v, cos, sin, window=77)
    out2, lse2, kw = ops.attn_fwd_qknorm(q, k, v, cos, sin, window=77)
    torch.cuda.synchronize()
    assert torch.equal(kn_only, kn_both) and torch.equal(kw, kn_only)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_fused_in_place_k_work():
    """k_work == k normalises k in place and gives the same outputs."""
    B, H, T, d = 1, 2, 190, 64
    say("fused in place")
    q, k, v = (dev(inputs.make_random((B, H, T, d), torch.bfloat16, s)) for s in (121, 122, 123))
    cos, sin = ops.rope_table(T, d)
    out, lse, kw = ops.attn_fwd_qknorm(q, k, v, cos, sin, window=50)
    k2 = k.clone()
    out2, lse2, kw2 = ops.attn_fwd_qknorm(q, k2, v, cos, sin, window=50, k_work=k2)
    torch.cuda.synchronize()
    assert kw2.data_ptr() == k2.data_ptr()
    assert torch.equal(k2, kw) and torch.equal(out2, out) and torch.equal(lse2, lse)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fused_is_scale_invariant(d):
    """QK-norm removes the rows' scale: raw q, k multiplied by 1e-3 or by 1e3 (per row, with
    eps scaled along so that eps / mean(x^2) is unchanged) give the same outputs within bf16
    rounding, and every output stays within the oracle's tolerance; the bounded softmax has no
    overflow at either end."""
    B, H, T = 1, 2, 150
    q, k, v = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (131, 132, 133))
    for scale in (1e-3, 1.0, 1e3):
        say(f"fused scale invariance d={d} scale={scale}")
        qs = (q.float() * scale).to(torch.bfloat16)
        ks = (k.float() * scale).to(torch.bfloat16)
        eps = 1e-6 * scale * scale
        out, lse, _ = fused(qs, ks, v, 60, eps=eps)
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
        check(out, lse, qs, ks, v, 60, eps=eps)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fused_extreme_scores(d):
    """All q and k rows equal to the same vector: every visible score before rotation is the
    bound sqrt(d) (the rotation then moves each pair's score by the angle between positions)."""
    B, H, T = 1, 1, 260
    base = inputs.make_random((1, 1, 1, d), torch.bfloat16, 141)
    q = base.expand(B, H, T, d).contiguous()
    k = q.clone()
    v = inputs.make_random((B, H, T, d), torch.bfloat16, 142)
    for window in (-1, 7):
        say(f"fused extreme scores d={d} W={window}")
        out, lse, _ = fused(q, k, v, window)
        check(out, lse, q, k, v, window)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fused_masked_keys_have_no_influence_bitwise(d):
    """Rewriting k, v at keys a row cannot see leaves that row's output and LSE bitwise
    unchanged."""
    B, H, T = 1, 1, 400
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 151)
    k = inputs.make_random((B, H, T, d), torch.bfloat16, 152)
    v = inputs.make_random((B, H, T, d), torch.bfloat16, 153)
    cos, sin = ops.rope_table(T, d)
    for window in (-1, 70):
        out, lse, _ = ops.attn_fwd_qknorm(dev(q), dev(k), dev(v), cos, sin, window=window)
        for i in (0, 5, 127, 128, 200, 399):
            say(f"fused mask perturbation d={d} W={window} row={i}")
            k2, v2 = k.clone(), v.clone()
            j = torch.arange(T)
            hidden = (j > i) | ((i - j > window) if window >= 0 else torch.zeros(T, dtype=torch.bool))
            sign = torch.where(j % 2 == 0, 1.0, -1.0)[:, None]
            k2[0, 0][hidden] = (1e4 * sign[hidden]).to(torch.bfloat16).expand(-1, d)
            v2[0, 0][hidden] = (-1e4 * sign[hidden]).to(torch.bfloat16).expand(-1, d)
            out2, lse2, _ = ops.attn_fwd_qknorm(dev(q), dev(k2), dev(v2), cos, sin, window=window)
            torch.cuda.synchronize()
            assert torch.equal(out2[0, 0, i], out[0, 0, i])
            assert torch.equal(lse2[0, 0, i], lse[0, 0, i])


def test_fused_deterministic_bitwise():
    w = inputs.WORKLOADS[inputs.HEADLINE]
    q, k, v = (dev(x) for x in inputs.make_qkv(inputs.HEADLINE, 0))
    cos, sin = ops.rope_table(w.T, w.d)
    for window in (w.T // 2, -1):
        say(f"fused determinism {w.name} W={window}")
        a = ops.attn_fwd_qknorm(q, k, v, cos, sin, window=window)
        b = ops.attn_fwd_qknorm(q, k, v, cos, sin, window=window)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_fused_outputs_stay_inside_their_buffers():
    B, H, T, d = 1, 3, 197, 64
    say("fused canaries")
    q, k, v = (dev(inputs.make_random((B, H, T, d), torch.bfloat16, s)) for s in (161, 162, 163))
    cos, sin = ops.rope_table(T, d)
    n, pad = B * H * T * d, 64
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    kbuf = torch.full((n + 2 * pad,), 5.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * T + 2 * pad,), -3.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n].view(B, H, T, d)
    kw = kbuf[pad:pad + n].view(B, H, T, d)
    lse = lbuf[pad:pad + B * H * T].view(B, H, T)
    ops.attn_fwd_qknorm(q, k, v, cos, sin, window=50, k_work=kw, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 7.0) and torch.all(obuf[pad + n:] == 7.0)
    assert torch.all(kbuf[:pad] == 5.0) and torch.all(kbuf[pad + n:] == 5.0)
    assert torch.all(lbuf[:pad] == -3.0) and torch.all(lbuf[pad + B * H * T:] == -3.0)


def test_fused_validation_with_real_buffers():
    lib = _lib.load()
    B, H, T, d = 1, 2, 64, 64
    q, k, v = (dev(inputs.make_random((B, H, T, d), torch.bfloat16, s)) for s in (1, 2, 3))
    kw = torch.full_like(q, 2.0)
    out = torch.full_like(q, 3.0)
    cos, sin = ops.rope_table(T, d)
    s = torch.cuda.current_stream().cuda_stream
    cases = [
        (dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
        (dict(dtype=_lib.ATTN_F32), _lib.ATTN_ERR_DTYPE),
        (dict(causal=0, window=3), _lib.ATTN_ERR_WINDOW),
        (dict(kw=q.data_ptr()), _lib.ATTN_ERR_ALIAS),
        (dict(out=kw.data_ptr()), _lib.ATTN_ERR_ALIAS),
        (dict(eps=-1.0), _lib.ATTN_ERR_ARG),
        (dict(cos=None), _lib.ATTN_ERR_NULL),
    ]
    for kwargs, code in cases:
        a = dict(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), kw=kw.data_ptr(),
                 out=out.data_ptr(), lse=None, cos=cos.data_ptr(), sin=sin.data_ptr(), B=B, H=H,
                 T=T, d=d, eps=1e-6, window=-1, causal=1, dtype=_lib.ATTN_BF16)
        a.update(kwargs)
        say(f"fused validation {kwargs}")
        rc = lib.attn_fwd_qknorm(a["q"], a["k"], a["v"], a["kw"], a["out"], a["lse"], a["cos"],
                                 a["sin"], a["B"], a["H"], a["T"], a["d"], a["eps"], a["window"],
                                 a["causal"], a["dtype"], s)
        assert rc == code
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(kw == 2.0)
    with pytest.raises(ValueError):
        ops.attn_fwd_qknorm(q.float(), k.float(), v.float(), cos, sin)


@pytest.mark.parametrize("window", [4096, -1])
def test_fused_long_single_head_sampled(window):
    """A long sequence at the limits of one head: T = 131072 (d = 64, bf16, one batch entry and
    two heads), window 4096 and full causal; the oracle checks sampled rows (the first, the
    window's edge, block edges, the last)."""
    B, H, T, d = 1, 2, 131072, 64
    say(f"fused long single head T={T} d={d} W={window}")
    q, k, v = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (141, 142, 143))
    out, lse, _ = fused(q, k, v, window)
    rng = np.random.default_rng(3)
    fixed = {0, 1, 127, 128, 4095, 4096, 4097, T // 2, T - 129, T - 1}
    rows = np.array(sorted(fixed | set(int(x) for x in rng.choice(T, 20, replace=False))))
    for h in range(H):
        sl = (slice(0, 1), slice(h, h + 1))
        check(out[sl], lse[sl], q[sl], k[sl], v[sl], window, rows=rows)


# The layer in one launch (k_work NULL, write_k=False): keys normalised and rotated inside the
# attention kernel, d 32 and 64. Same oracle and tolerances; the rotation angles of the keys are
# formed in fp32 in the kernel instead of read from the fp64-built table.
KIN_CASES = []
for d in (32, 64):
    KIN_CASES += [(d, 1, 1, 1, -1, 1), (d, 1, 2, 63, 1, 1), (d, 2, 1, 130, 0, 1),
                  (d, 1, 3, 257, 100, 1), (d, 1, 2, 300, -1, 0), (d, 2, 2, 384, -1, 1),
                  (d, 1, 1, 200, 199, 1), (d, 1, 2, 700, 333, 1)]
KIN_CASES += [(64, 40, 16, 256, 128, 1), (32, 64, 12, 200, -1, 1)]


@pytest.mark.parametrize("d,B,H,T,window,causal", KIN_CASES,
                         ids=[f"d{c[0]}-B{c[1]}H{c[2]}T{c[3]}-W{c[4]}-c{c[5]}" for c in KIN_CASES])
def test_k_in_kernel_parity(d, B, H, T, window, causal):
    say(f"k in kernel parity d={d} B={B} H={H} T={T} W={window} causal={causal}")
    q, k, v = (inputs.make_random((B, H, T, d), torch.bfloat16, s) for s in (151, 152, 153))
    cos, sin = ops.rope_table(T, d)
    out, lse, kw = ops.attn_fwd_qknorm(dev(q), dev(k), dev(v), cos, sin, window=window,
                                       causal=bool(causal), write_k=False)
    torch.cuda.synchronize()
    assert kw is None
    out, lse = out.cpu(), lse.cpu()
    if B * H * T > 20000:
        rows = np.unique(np.r_[0, 1, T // 2, T - 1, np.arange(0, T, 37)])
        for sl in ((slice(0, 1), slice(0, 1)), (slice(B - 1, B), slice(H - 1, H))):
            check(out[sl], lse[sl], q[sl], k[sl], v[sl], window, bool(causal), rows=rows)
    else:
        check(out, lse, q, k, v, window, bool(causal))


@pytest.mark.parametrize("index", [i for i, w in enumerate(inputs.WORKLOADS)
                                   if w.dtype == "bf16" and w.d <= 64],
                         ids=[w.name for w in inputs.WORKLOADS if w.dtype == "bf16" and w.d <= 64])
def test_k_in_kernel_full_size_sampled(index):
    """Every layer at the workload's real shape with the keys normalised in the kernel; sampled
    rows of sampled heads against the oracle, and every output within the bf16 budget of the
    two-launch layer."""
    w = inputs.WORKLOADS[index]
    rng = np.random.default_rng(200 + index)
    cos, sin = ops.rope_table(w.T, w.d)
    for layer, window in enumerate(ops.sssl_windows(w.T, w.n_layer, w.pattern)):
        say(f"k in kernel full {w.name} B={w.B} H={w.H} T={w.T} d={w.d} layer={layer} "
            f"W={window}")
        q, k, v = inputs.make_qkv(index, layer)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out, lse, _ = ops.attn_fwd_qknorm(qd, kd, vd, cos, sin, window=window, write_k=False)
        o2, l2, _ = ops.attn_fwd_qknorm(qd, kd, vd, cos, sin, window=window)
        torch.cuda.synchronize()
        assert float((out.float() - o2.float()).abs().max()) <= BF16_TOL
        assert float((lse - l2).abs().max()) <= LSE_TOL
        del qd, kd, vd, o2, l2
        heads = [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]
        fixed = {0, 1, w.T - 1, w.T // 2, min(w.T - 1, window), min(w.T - 1, window + 1)}
        rows = np.array(sorted(fixed | set(int(x) for x in rng.choice(w.T, 40, replace=False))))
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            check(out[sl].cpu(), lse[sl].cpu(), q[sl], k[sl], v[sl], window, rows=rows)
        del out, lse


def test_k_in_kernel_gqa_and_bthd():
    """Grouped-query heads and the [B][T][H][d] order with the keys normalised in the kernel."""
    B, H, H_kv, T, d = 2, 6, 2, 290, 64
    say("k in kernel GQA bthd")
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 161)
    k, v = (inputs.make_random((B, H_kv, T, d), torch.bfloat16, s) for s in (162, 163))
    cos, sin = ops.rope_table(T, d)
    for layout in ("bhtd", "bthd"):
        conv = (lambda x: dev(x.transpose(1, 2))) if layout == "bthd" else dev
        out, lse, _ = ops.attn_fwd_qknorm(conv(q), conv(k), conv(v), cos, sin, window=90,
                                          layout=layout, write_k=False)
        o2, l2, _ = ops.attn_fwd_qknorm(conv(q), conv(k), conv(v), cos, sin, window=90,
                                        layout=layout)
        torch.cuda.synchronize()
        assert float((out.float() - o2.float()).abs().max()) <= BF16_TOL
        assert float((lse - l2).abs().max()) <= LSE_TOL
        if layout == "bthd":
            out = out.transpose(1, 2)
        kx = k.repeat_interleave(H // H_kv, dim=1)
        vx = v.repeat_interleave(H // H_kv, dim=1)
        check(out.cpu(), lse.cpu(), q, kx, vx, 90)


def test_k_in_kernel_needs_d_at_most_64():
    B, H, T, d = 1, 1, 64, 128
    q, k, v = (dev(inputs.make_random((B, H, T, d), torch.bfloat16, s)) for s in (1, 2, 3))
    cos, sin = ops.rope_table(T, d)
    with pytest.raises(RuntimeError):
        ops.attn_fwd_qknorm(q, k, v, cos, sin, write_k=False)
