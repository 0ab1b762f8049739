"""GPU parity of the _ex entry points: grouped-query heads (k and v with H_kv < H heads) and the
[B][T][H][d] storage order of the model's projections, against the fp64 oracle, through the C ABI.

Inputs are drawn in [B, H, T, d] order and, for the [B][T][H][d] cases, transposed into that
order before the call; outputs are transposed back before the comparison. Besides the oracle,
every case checks that the kernels' arithmetic does not depend on the addressing: the grouped
[B][T][H][d] result equals, bit for bit, the [B][H][T][d] multi-head result on k and v with each
kv head repeated for its group. Every case prints its name before touching the GPU.
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
BF16_LSE_TOL = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def to_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    """[B, H, T, d] CPU tensor -> contiguous GPU tensor in ``layout``."""
    x = x.to("cuda")
    return (x.transpose(1, 2) if layout == "bthd" else x).contiguous()


def from_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    """GPU tensor in ``layout`` -> [B, H, T, d] CPU tensor."""
    return (x.transpose(1, 2) if layout == "bthd" else x).contiguous().cpu()


def repeat_kv(x: torch.Tensor, group: int) -> torch.Tensor:
    """[B, H_kv, T, d] -> [B, H_kv * group, T, d]: kv head g serves query heads g*group ..
    g*group + group - 1 (the oracle's kv_head mapping)."""
    return x.repeat_interleave(group, dim=1).contiguous()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    torch.cuda.synchronize()


LAYOUT_GROUPS = [(lay, g) for lay in ("bhtd", "bthd") for g in (1, 2, 4)]

# (dtype, d, B, H, T, window, causal): ragged tails, windows, non-causal; H = 4 so that the
# groups 1, 2, 4 give H_kv = 4, 2, 1.
FWD_SHAPES = [("bf16", 32, 2, 4, 130, -1, 1), ("bf16", 64, 1, 4, 333, 100, 1),
              ("bf16", 128, 2, 4, 257, 64, 1), ("bf16", 64, 2, 4, 200, -1, 0),
              ("f32", 16, 1, 4, 97, 9, 1), ("f32", 64, 2, 4, 70, -1, 1)]
FWD_CASES = [s + lg for s in FWD_SHAPES for lg in LAYOUT_GROUPS]


@pytest.mark.parametrize("dt,d,B,H,T,window,causal,layout,group", FWD_CASES,
                         ids=[f"{c[0]}-d{c[1]}-B{c[2]}H{c[3]}T{c[4]}-W{c[5]}-c{c[6]}-{c[7]}-g{c[8]}"
                              for c in FWD_CASES])
def test_attn_fwd_ex_parity(dt, d, B, H, T, window, causal, layout, group):
    say(f"attn_fwd_ex {dt} d={d} B={B} H={H} T={T} W={window} causal={causal} {layout} "
        f"group={group}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    H_kv = H // group
    q = inputs.make_random((B, H, T, d), dtype, 301)
    k = inputs.make_random((B, H_kv, T, d), dtype, 302)
    v = inputs.make_random((B, H_kv, T, d), dtype, 303)
    out, lse = ops.attn_fwd(to_layout(q, layout), to_layout(k, layout), to_layout(v, layout),
                            window=window, causal=bool(causal), layout=layout)
    # the same call as multi-head [B][H][T][d] attention on repeated k, v
    o_ref, l_ref = ops.attn_fwd(q.cuda(), repeat_kv(k, group).cuda(), repeat_kv(v, group).cuda(),
                                window=window, causal=bool(causal))
    torch.cuda.synchronize()
    out = from_layout(out, layout)
    assert torch.equal(out, o_ref.cpu()) and torch.equal(lse.cpu(), l_ref.cpu())
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), window=window, causal=bool(causal))
    eo = float(np.max(np.abs(f64(out) - ro)))
    el = float(np.max(np.abs(f64(lse) - rl)))
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= (BF16_TOL if dt == "bf16" else F32_TOL)
    assert el <= (BF16_LSE_TOL if dt == "bf16" else F32_TOL)


PRO_CASES = [(dt, d) + lg for dt in ("bf16", "f32") for d in (16, 64, 128) for lg in LAYOUT_GROUPS]


@pytest.mark.parametrize("dt,d,layout,group", PRO_CASES,
                         ids=[f"{c[0]}-d{c[1]}-{c[2]}-g{c[3]}" for c in PRO_CASES])
def test_qknorm_rope_ex_parity(dt, d, layout, group):
    B, H, T = 2, 4, 67
    say(f"qknorm_rope_ex {dt} d={d} B={B} H={H} T={T} {layout} group={group}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    H_kv = H // group
    q = inputs.make_random((B, H, T, d), dtype, 311) * 3
    k = inputs.make_random((B, H_kv, T, d), dtype, 312, "uniform")
    cos, sin = ops.rope_table(T, d)
    qn, kn = ops.qknorm_rope(to_layout(q, layout), to_layout(k, layout), cos, sin, layout=layout)
    qr, kr = ops.qknorm_rope(q.cuda(), k.cuda(), cos, sin)  # [B][H][T][d], k with H_kv heads
    _, k_only = ops.qknorm_rope(None, to_layout(k, layout), cos, sin, layout=layout)
    torch.cuda.synchronize()
    qn, kn, k_only = from_layout(qn, layout), from_layout(kn, layout), from_layout(k_only, layout)
    assert torch.equal(qn, qr.cpu()) and torch.equal(kn, kr.cpu()) and torch.equal(k_only, kn)
    rq, rk = oracle.qknorm_rope(f64(q), f64(k))
    for g, r in ((qn, rq), (kn, rk)):
        err = np.abs(f64(g) - r)
        bound = (2.0 ** -8 * np.abs(r) + 2.0 ** -20) if dt == "bf16" else (2e-6 * np.abs(r) + 1e-6)
        assert np.all(err <= bound), f"max err {err.max()}"


FUSED_SHAPES = [(32, 2, 4, 130, -1, 1), (64, 1, 4, 333, 100, 1), (128, 2, 4, 257, 64, 1),
                (64, 1, 4, 150, -1, 0)]
FUSED_CASES = [s + lg for s in FUSED_SHAPES for lg in LAYOUT_GROUPS]


@pytest.mark.parametrize("d,B,H,T,window,causal,layout,group", FUSED_CASES,
                         ids=[f"d{c[0]}-B{c[1]}H{c[2]}T{c[3]}-W{c[4]}-c{c[5]}-{c[6]}-g{c[7]}"
                              for c in FUSED_CASES])
def test_attn_fwd_qknorm_ex_parity(d, B, H, T, window, causal, layout, group):
    say(f"attn_fwd_qknorm_ex d={d} B={B} H={H} T={T} W={window} causal={causal} {layout} "
        f"group={group}")
    H_kv = H // group
    q = inputs.make_random((B, H, T, d), torch.bfloat16, 321)
    k = inputs.make_random((B, H_kv, T, d), torch.bfloat16, 322)
    v = inputs.make_random((B, H_kv, T, d), torch.bfloat16, 323)
    cos, sin = ops.rope_table(T, d)
    qd, kd, vd = to_layout(q, layout), to_layout(k, layout), to_layout(v, layout)
    out, lse, kw = ops.attn_fwd_qknorm(qd, kd, vd, cos, sin, window=window, causal=bool(causal),
                                       layout=layout)
    # its second kernel alone on the returned keys
    out2, lse2 = ops.attn_fwd_qnorm(qd, kw, vd, cos, sin, window=window, causal=bool(causal),
                                    layout=layout)
    # multi-head [B][H][T][d] on repeated k, v
    o_ref, l_ref, _ = ops.attn_fwd_qknorm(q.cuda(), repeat_kv(k, group).cuda(),
                                          repeat_kv(v, group).cuda(), cos, sin, window=window,
                                          causal=bool(causal))
    _, k_only = ops.qknorm_rope(None, kd, cos, sin, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2) and torch.equal(kw, k_only)
    out = from_layout(out, layout)
    assert torch.equal(out, o_ref.cpu()) and torch.equal(lse.cpu(), l_ref.cpu())
    ro, rl = oracle.attention_layer(f64(q), f64(k), f64(v), window=window, causal=bool(causal))
    eo = float(np.max(np.abs(f64(out) - ro)))
    el = float(np.max(np.abs(f64(lse) - rl)))
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= BF16_TOL and el <= BF16_TOL


def test_gqa_outputs_stay_inside_their_buffers():
    """Canaries around q-sized outputs and the smaller k_work of a grouped [B][T][H][d] call."""
    B, H, H_kv, T, d = 2, 8, 2, 190, 64
    say("gqa canaries")
    q = inputs.make_random((B, T, H, d), torch.bfloat16, 331).cuda()
    k = inputs.make_random((B, T, H_kv, d), torch.bfloat16, 332).cuda()
    v = inputs.make_random((B, T, H_kv, d), torch.bfloat16, 333).cuda()
    cos, sin = ops.rope_table(T, d)
    pad = 4096
    big_o = torch.full((q.numel() + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    big_k = torch.full((k.numel() + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big_o[pad:pad + q.numel()].view(q.shape)
    kw = big_k[pad:pad + k.numel()].view(k.shape)
    ops.attn_fwd_qknorm(q, k, v, cos, sin, window=33, out=out, k_work=kw, want_lse=False,
                        layout="bthd")
    torch.cuda.synchronize()
    for big in (big_o, big_k):
        assert bool((big[:pad] == 7.0).all()) and bool((big[-pad:] == 7.0).all())
    assert torch.isfinite(out.float()).all()


def test_ex_validation_with_real_buffers():
    q = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 64, 3, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ops.attn_fwd(q, k, k, layout="bthd")  # 3 kv heads do not divide 4
    lib = _lib.load()
    out = torch.empty_like(q)
    rc = lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(), None,
                         1, 4, 3, 64, 64, 1, -1, 1, _lib.ATTN_BF16, None)
    assert rc == _lib.ATTN_ERR_SHAPE
    rc = lib.attn_fwd_ex(q.data_ptr(), q.data_ptr(), q.data_ptr(), out.data_ptr(), None,
                         1, 4, 4, 64, 64, 5, -1, 1, _lib.ATTN_BF16, None)
    assert rc == _lib.ATTN_ERR_ARG


def test_model_default_shape_sampled():
    """The listing's default model (DEPTH 8, HEAD_DIM 128, d_model 512 so 4 heads, 2048 tokens,
    128 sequences, SSSL windows 1024 / 2048) in its own [B][T][H][d] order, one short and one
    long layer at full size; the oracle checks sampled rows of sampled heads."""
    w = inputs.MODEL_DEFAULT
    rng = np.random.default_rng(7)
    cos, sin = ops.rope_table(w.T, w.d)
    windows = ops.sssl_windows(w.T, w.n_layer, w.pattern)
    for layer in (0, w.n_layer - 1):
        window = windows[layer]
        say(f"model default shape B={w.B} T={w.T} H={w.H} d={w.d} bthd layer={layer} W={window}")
        q, k, v = inputs.make_qkv(inputs.MODEL_DEFAULT_INDEX, layer)  # [B, H, T, d], CPU
        out, lse, _ = ops.attn_fwd_qknorm(to_layout(q, "bthd"), to_layout(k, "bthd"),
                                          to_layout(v, "bthd"), cos, sin, window=window,
                                          layout="bthd")
        torch.cuda.synchronize()
        heads = [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]
        rows = np.array(sorted({0, 1, w.T // 2, w.T - 1, min(w.T - 1, window),
                                min(w.T - 1, window + 1)}
                               | set(int(x) for x in rng.choice(w.T, 30, replace=False))))
        for b, h in heads:
            ro, rl = oracle.attention_layer(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                                            f64(v[b:b + 1, h:h + 1]), window=window, rows=rows)
            go = f64(out[b, rows, h].cpu())
            gl = f64(lse[b, h, rows].cpu())
            eo = float(np.max(np.abs(go - ro[0, 0])))
            el = float(np.max(np.abs(gl - rl[0, 0])))
            say(f"   head ({b},{h}) max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= BF16_TOL and el <= BF16_TOL
        del out, lse
