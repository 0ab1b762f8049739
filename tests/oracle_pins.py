"""Pin checks for the fp64 oracle, written so that a test can run them against a deliberately
broken copy of the oracle too (``test_oracle_mutations.py``).

Each check takes an object ``o`` exposing the oracle's functions (``oracle`` itself, or a
namespace with one function replaced) and raises AssertionError when the pin fails. None of them
re-types the oracle's formulas: they compare against closed forms, values the pages print, brute
force with ``math.fsum``, or an independent library routine.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------------------------
# Worked example: "Lendo uma Projeção" on "Projeção em um Subespaço de Consulta".
# ---------------------------------------------------------------------------------------------

def worked_example_inputs():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    return g


def check_worked_example(o):
    """Raw attention of the printed query against the three printed keys, V = identity.

    Closed form: q.k = (1, 1, 0); divided by sqrt(d_k) = 2 that is (1/2, 1/2, 0); the softmax
    weights are (sqrt(e), sqrt(e), 1) / (2 sqrt(e) + 1) and the logsumexp is ln(2 sqrt(e) + 1).
    Rows 1 and 2 of the embedding use a zero query: weights 1/3 each, logsumexp ln 3.
    """
    g = worked_example_inputs()
    assert g["sqrt_d_k"] == 2 and g["d_k"] == 4
    T, d = 3, 4
    q = np.zeros((1, 1, T, d))
    q[0, 0, 0] = g["q"]
    k = np.array(g["keys"], dtype=np.float64)[None, None]
    v = np.eye(3)[None, None]
    out, lse = o.attention(q, k, v, window=-1, causal=False)
    se = math.exp(0.5)
    w = np.array([se, se, 1.0]) / (2 * se + 1)
    assert abs(sum(w) - 1) < 1e-15
    np.testing.assert_allclose(out[0, 0, 0], w, rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(2 * se + 1)) < 1e-15
    np.testing.assert_allclose(out[0, 0, 1:], np.full((2, 3), 1 / 3), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 1:], [math.log(3)] * 2, rtol=0, atol=1e-15)
    # Printed numbers of the closed form, to 12 digits.
    assert abs(out[0, 0, 0, 0] - 0.383651731190) < 1e-12
    assert abs(out[0, 0, 0, 2] - 0.232696537618) < 1e-12
    assert abs(lse[0, 0, 0] - 1.458020087947) < 1e-12


def check_worked_example_qknorm(o):
    """The same example through QK-norm (no positions, so no rotation).

    Closed form with eps: q_hat = q / sqrt(1/2 + eps), k1_hat = e1 / sqrt(1/4 + eps),
    k2_hat = e3 / sqrt(1/4 + eps), k3_hat = (e2 + e4) / sqrt(1/2 + eps); the scores are
    q_hat.k_hat / 2.
    """
    g = worked_example_inputs()
    eps = 1e-6
    q = np.array(g["q"], dtype=np.float64)
    keys = np.array(g["keys"], dtype=np.float64)
    qn = o.rms_norm(q, eps)
    kn = o.rms_norm(keys, eps)
    np.testing.assert_allclose(qn, q / math.sqrt(0.5 + eps), rtol=1e-15, atol=0)
    np.testing.assert_allclose(kn[0], keys[0] / math.sqrt(0.25 + eps), rtol=1e-15, atol=0)
    np.testing.assert_allclose(kn[2], keys[2] / math.sqrt(0.5 + eps), rtol=1e-15, atol=0)
    s12 = 1.0 / (math.sqrt(0.5 + eps) * math.sqrt(0.25 + eps)) / 2
    z = 2 * math.exp(s12) + 1
    T = 3
    qq = np.zeros((1, 1, T, 4))
    qq[0, 0, 0] = qn
    out, lse = o.attention(qq, kn[None, None], np.eye(3)[None, None], window=-1, causal=False)
    np.testing.assert_allclose(out[0, 0, 0], [math.exp(s12) / z, math.exp(s12) / z, 1 / z], atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(z)) < 1e-14
    assert abs(out[0, 0, 0, 0] - 0.445808) < 1e-6 and abs(out[0, 0, 0, 2] - 0.108384) < 1e-6


# ---------------------------------------------------------------------------------------------
# Brute force with math.fsum on tiny inputs.
# ---------------------------------------------------------------------------------------------

def brute_attention(q, k, v, window, causal):
    """Pure-Python attention of one head: q, k [T][d], v [T][dv] as nested lists."""
    T, d = len(q), len(q[0])
    dv = len(v[0])
    out, lse = [], []
    for i in range(T):
        keys = [j for j in range(T)
                if (not causal) or (j <= i and (window < 0 or i - j <= window))]
        s = {j: math.fsum(q[i][a] * k[j][a] for a in range(d)) / math.sqrt(d) for j in keys}
        m = max(s.values())
        l = m + math.log(math.fsum(math.exp(s[j] - m) for j in keys))
        out.append([math.fsum(math.exp(s[j] - l) * v[j][c] for j in keys) for c in range(dv)])
        lse.append(l)
    return out, lse


def check_brute_force(o, Ts=(1, 2, 5, 9), ds=(2, 4, 8), seed=0):
    rng = _rng(seed)
    for T in Ts:
        for d in ds:
            q = rng.standard_normal((1, 2, T, d)) * 1.5
            k = rng.standard_normal((1, 2, T, d)) * 1.5
            v = rng.standard_normal((1, 2, T, d + 1))
            cases = [(-1, False)] + [(w, True) for w in [-1] + list(range(0, T + 2))]
            for window, causal in cases:
                out, lse = o.attention(q, k, v, window=window, causal=causal)
                for h in range(2):
                    bo, bl = brute_attention(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(),
                                             window, causal)
                    np.testing.assert_allclose(out[0, h], np.array(bo), rtol=0, atol=1e-12,
                                               err_msg=f"T={T} d={d} W={window} causal={causal}")
                    np.testing.assert_allclose(lse[0, h], np.array(bl), rtol=0, atol=1e-12)


def check_sdpa_special_case(o, seed=1):
    """With no prologue, the oracle equals PyTorch's CPU scaled_dot_product_attention in fp64
    with an explicit boolean mask built from the window reading."""
    import torch
    rng = _rng(seed)
    B, H, T, d = 2, 3, 37, 16
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    for window, causal in [(-1, True), (0, True), (5, True), (18, True), (T, True), (-1, False)]:
        if causal:
            mask = (j <= i) & ((i - j <= window) if window >= 0 else True)
        else:
            mask = np.ones((T, T), dtype=bool)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=torch.from_numpy(np.ascontiguousarray(mask)))
        out, _ = o.attention(q, k, v, window=window, causal=causal)
        np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12,
                                   err_msg=f"W={window} causal={causal}")


def _sdpa_reference(q, k, v, window, causal):
    """PyTorch CPU scaled_dot_product_attention in fp64 with an explicit boolean mask built from
    the window reading (key j visible to query i iff j <= i and i - j <= W); kv heads are
    repeated for their query group. Returns (out, lse) as numpy arrays; the logsumexp is
    torch.logsumexp of the masked scaled scores."""
    import torch
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    T, d = q.shape[-2], q.shape[-1]
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = torch.ones(T, T, dtype=torch.bool)
    if causal:
        mask = j <= i
        if window >= 0:
            mask = mask & (i - j <= window)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return out.numpy(), lse.numpy()


def check_blocked_rows(o, seed=18):
    """The oracle's row blocks and its sampled-row path against whole-matrix references.

    At T = 600 the default block of 256 rows gives three blocks, so the key range of a block
    that starts past the window (lo = r0 - W > 0) is exercised at every window around the block
    size, including the inclusive boundary key r0 - W (the window reading of the (W, 0) call in
    the train.py listing's ``CausalSelfAttention.forward``; "A Máscara Causal"). The reference
    is torch's fp64 ``scaled_dot_product_attention`` with an explicit mask over all T keys.
    Then ``rows=`` with unsorted, repeated and non-contiguous query indices that straddle block
    boundaries (tiny blocks of 7 rows, grouped kv heads) must equal the matching rows of the
    full result, and the same through ``attention_layer``."""
    rng = _rng(seed)
    B, H, H_kv, T, d = 1, 2, 1, 600, 8
    q = rng.standard_normal((B, H, T, d)) * 1.5
    k = rng.standard_normal((B, H_kv, T, d)) * 1.5
    v = rng.standard_normal((B, H_kv, T, d + 3))
    for window in (-1, 0, 1, 255, 256, 257, 343, 511, 599):
        ref_o, ref_l = _sdpa_reference(q, k, v, window, True)
        out, lse = o.attention(q, k, v, window=window, causal=True)
        np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12, err_msg=f"W={window}")
        np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12, err_msg=f"W={window}")
    # Sampled rows: block boundaries of 256 and of 7, unsorted, with a repeat.
    rows = np.array([599, 0, 256, 255, 7, 6, 511, 512, 300, 13, 14, 257, 0, 598])
    Ts = 40
    qs, ks, vs = q[:, :, :Ts], k[:, :, :Ts], v[:, :, :Ts]
    rows_s = np.array([39, 0, 7, 6, 13, 14, 21, 3, 35, 20, 7])
    for window, causal in ((-1, True), (0, True), (3, True), (6, True), (7, True), (38, True),
                           (-1, False)):
        full_o, full_l = o.attention(qs, ks, vs, window=window, causal=causal)
        for blk in (1, 7, 256):
            out, lse = o.attention(qs, ks, vs, window=window, causal=causal, rows=rows_s, block=blk)
            np.testing.assert_allclose(out, full_o[:, :, rows_s], rtol=0, atol=1e-13,
                                       err_msg=f"W={window} causal={causal} block={blk}")
            np.testing.assert_allclose(lse, full_l[:, :, rows_s], rtol=0, atol=1e-13)
        ref_o, ref_l = _sdpa_reference(qs, ks, vs, window, causal)
        np.testing.assert_allclose(full_o, ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(full_l, ref_l, rtol=0, atol=1e-12)
    for window in (-1, 256, 300):
        ref_o, ref_l = _sdpa_reference(q, k, v, window, True)
        out, lse = o.attention(q, k, v, window=window, causal=True, rows=rows)
        np.testing.assert_allclose(out, ref_o[:, :, rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_l[:, :, rows], rtol=0, atol=1e-12)
        lo, ll = o.attention_layer(q, k, v, window=window, rows=rows)
        fo, fl = o.attention_layer(q, k, v, window=window)
        np.testing.assert_allclose(lo, fo[:, :, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ll, fl[:, :, rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# Invariants of the definition.
# ---------------------------------------------------------------------------------------------

def check_weights_sum_to_one(o, seed=2):
    """sum_j exp(s_ij - LSE_i) over the visible keys is 1, with s recomputed by einsum."""
    rng = _rng(seed)
    B, H, T, d = 1, 2, 50, 8
    q = rng.standard_normal((B, H, T, d)) * 2
    k = rng.standard_normal((B, H, T, d)) * 2
    v = rng.standard_normal((B, H, T, d))
    for window in (-1, 0, 7, 25):
        _, lse = o.attention(q, k, v, window=window, causal=True)
        s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        vis = (j <= i) & (((i - j) <= window) if window >= 0 else True)
        tot = np.where(vis, np.exp(s - lse[..., None]), 0.0).sum(-1)
        np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)


def check_masked_entries_have_no_weight(o, seed=3):
    """Rewriting k and v at keys a row cannot see leaves that row bitwise unchanged."""
    rng = _rng(seed)
    T, d = 40, 8
    q = rng.standard_normal((1, 1, T, d))
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    for window in (-1, 3, 10):
        out, lse = o.attention(q, k, v, window=window, causal=True)
        for i in (0, 5, 17, 39):
            k2, v2 = k.copy(), v.copy()
            for j in range(T):
                if j > i or (window >= 0 and i - j > window):
                    k2[0, 0, j] = 1e4 * (-1) ** j
                    v2[0, 0, j] = -1e4 * (-1) ** j
            out2, lse2 = o.attention(q, k2, v2, window=window, causal=True)
            assert np.array_equal(out2[0, 0, i], out[0, 0, i]), (window, i)
            assert lse2[0, 0, i] == lse[0, 0, i], (window, i)


def check_window_T_is_causal(o, seed=4):
    """window >= T - 1 (in particular window = T) is the full causal mask."""
    rng = _rng(seed)
    T, d = 33, 4
    q, k, v = (rng.standard_normal((1, 2, T, d)) for _ in range(3))
    ref = o.attention(q, k, v, window=-1, causal=True)
    for window in (T - 1, T, 5 * T):
        out = o.attention(q, k, v, window=window, causal=True)
        np.testing.assert_allclose(out[0], ref[0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(out[1], ref[1], rtol=0, atol=1e-15)
    # window T - 2 is not: the last row loses key 0.
    out = o.attention(q, k, v, window=T - 2, causal=True)
    assert not np.allclose(out[0][0, 0, T - 1], ref[0][0, 0, T - 1])


def check_window_zero(o, seed=5):
    """window = 0: each row sees only itself, so O_i = v_i and LSE_i = q_i.k_i / sqrt(d)."""
    rng = _rng(seed)
    T, d = 20, 8
    q, k, v = (rng.standard_normal((1, 1, T, d)) for _ in range(3))
    out, lse = o.attention(q, k, v, window=0, causal=True)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)
    s = np.array([math.fsum(q[0, 0, i] * k[0, 0, i]) / math.sqrt(d) for i in range(T)])
    np.testing.assert_allclose(lse[0, 0], s, rtol=0, atol=1e-14)


def check_zero_query_closed_form(o, seed=6):
    """Raw q = 0 through the whole layer: QK-norm maps 0 to 0 (eps > 0), every score is 0, so
    O_i is the mean of the visible v_j and LSE_i = ln |A(i)| = ln(min(i, W) + 1) (inclusive window
    reading). The exclusive reading (i - j < W) would give ln(min(i + 1, W))."""
    rng = _rng(seed)
    T, d = 24, 8
    q = np.zeros((1, 1, T, d))
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    for window in (-1, 0, 1, 5, 23):
        out, lse = o.attention_layer(q, k, v, window=window, causal=True)
        for i in range(T):
            n = (i + 1) if window < 0 else (min(i, window) + 1)
            lo = i + 1 - n
            np.testing.assert_allclose(out[0, 0, i], v[0, 0, lo:i + 1].mean(0), rtol=0, atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-14, (window, i)


# ---------------------------------------------------------------------------------------------
# RMSNorm and RoPE.
# ---------------------------------------------------------------------------------------------

def check_rms_norm(o, seed=7):
    """Mean square of the output is m / (m + eps), where m is the input's mean square; scaling x
    by c and eps by c^2 leaves the output unchanged; equals torch's CPU rms_norm in fp64."""
    import torch
    rng = _rng(seed)
    x = rng.standard_normal((5, 7, 64)) * rng.uniform(0.01, 10, size=(5, 7, 1))
    eps = 1e-6
    y = o.rms_norm(x, eps)
    m = (x ** 2).mean(-1)
    np.testing.assert_allclose((y ** 2).mean(-1), m / (m + eps), rtol=1e-14)
    np.testing.assert_allclose(o.rms_norm(3.0 * x, 9 * eps), y, rtol=1e-14)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), eps=eps).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)
    # a zero row stays zero
    assert np.all(o.rms_norm(np.zeros((2, 8)), eps) == 0)


def check_rope_special_values(o):
    """Position 0 is the identity. Rotating the unit vector e_0 at position 1 turns the plane
    (0, d/2) by exactly 1 rad (frequency base**0 = 1): it becomes cos(1) e_0 - sin(1) e_{d/2}.
    Channel pair d/4 has frequency base**(-1/2) = 1/100, so at position 100 it also turns by 1 rad.
    """
    d, T = 16, 101
    h = d // 2
    cos, sin = o.rope_cos_sin(T, d, 10000.0)
    x = np.zeros((T, d))
    x[:, 0] = 1.0
    x[:, h // 2] = 2.0
    y = o.rope_apply(x, cos, sin)
    np.testing.assert_allclose(y[0], x[0], rtol=0, atol=0)
    e = np.zeros(d)
    e[0] = 0.5403023058681398   # cos(1)
    e[h] = -0.8414709848078965  # -sin(1)
    e[h // 2] = 2.0 * math.cos(0.01)
    e[h + h // 2] = -2.0 * math.sin(0.01)
    np.testing.assert_allclose(y[1], e, rtol=0, atol=1e-15)
    # position 100, pair d/4: angle 100 * 10000**(-1/2) = 1 rad
    assert abs(y[100, h // 2] - 2.0 * 0.5403023058681398) < 1e-13
    assert abs(y[100, h + h // 2] + 2.0 * 0.8414709848078965) < 1e-13


def check_rope_invariants(o, seed=8):
    """The rotation keeps every row's norm, only mixes channel j with j + d/2, and the dot
    product of a rotated query and key depends only on their distance."""
    rng = _rng(seed)
    T, d = 40, 32
    cos, sin = o.rope_cos_sin(T, d, 10000.0)
    x = rng.standard_normal((3, T, d))
    y = o.rope_apply(x, cos, sin)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    # pairing: a unit vector on channel j stays inside the plane (j, j + d/2)
    for j in (0, 3, d // 2 - 1):
        e = np.zeros((T, d))
        e[:, j] = 1.0
        ye = o.rope_apply(e, cos, sin)
        others = np.delete(ye, [j, j + d // 2], axis=-1)
        assert np.all(others == 0)
    # relative position: same q vector at every position and same k vector at every position
    qv = rng.standard_normal(d)
    kv = rng.standard_normal(d)
    qr = o.rope_apply(np.tile(qv, (T, 1)), cos, sin)
    kr = o.rope_apply(np.tile(kv, (T, 1)), cos, sin)
    dots = qr @ kr.T
    for delta in (0, 1, 7, 20):
        diag = np.array([dots[i, i - delta] for i in range(delta, T)])
        np.testing.assert_allclose(diag, diag[0], rtol=0, atol=1e-12)


def check_norm_rope_commute(o, seed=9):
    """QK-norm and RoPE commute (the rotation keeps the sum of squares): both orders agree."""
    rng = _rng(seed)
    T, d = 30, 64
    x = rng.standard_normal((2, 3, T, d)) * 3
    cos, sin = o.rope_cos_sin(T, d, 10000.0)
    a = o.rope_apply(o.rms_norm(x, 1e-6), cos, sin)
    b = o.rms_norm(o.rope_apply(x, cos, sin), 1e-6)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    qn, kn = o.qknorm_rope(x, 2 * x, 1e-6, 10000.0)
    np.testing.assert_allclose(qn, a, rtol=0, atol=1e-15)


def check_sssl_windows(o):
    """The SSSL schedule: pattern letter per layer, S = T // 2, L = T, last layer forced to L."""
    assert o.sssl_windows(1024, 4) == [512, 512, 512, 1024]
    assert o.sssl_windows(8192, 4) == [4096, 4096, 4096, 8192]
    assert o.sssl_windows(2048, 8) == [1024, 1024, 1024, 2048, 1024, 1024, 1024, 2048]
    assert o.sssl_windows(1024, 6) == [512, 512, 512, 1024, 512, 1024]
    assert o.sssl_windows(1024, 2, "S") == [512, 1024]
    assert o.sssl_windows(1024, 1) == [1024]
    assert o.sssl_windows(1025, 3, "ss") == [512, 512, 1025]


def check_gqa_head_mapping(o, seed=10):
    """R13: with every value row of kv head g equal to the constant g + 1, each output row is a
    convex combination of equal rows, so out[b, h] is exactly kv_head(h) + 1 = h // (H / H_kv) + 1
    whatever q and k are; with H_kv = H the call is plain multi-head attention."""
    rng = _rng(seed)
    B, H, T, d = 2, 6, 7, 4
    q = rng.standard_normal((B, H, T, d))
    for H_kv in (1, 2, 3, 6):
        k = rng.standard_normal((B, H_kv, T, d))
        v = np.broadcast_to((np.arange(H_kv) + 1.0)[None, :, None, None], (B, H_kv, T, 3)).copy()
        for window in (-1, 2):
            out, lse = o.attention(q, k, v, window=window)
            for h in range(H):
                assert np.allclose(out[:, h], h // (H // H_kv) + 1.0, rtol=0, atol=1e-13), (H_kv, h)
    # Plain multi-head case: each head equals a one-head call on that head.
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    out, lse = o.attention(q, k, v, window=3)
    for h in (0, 4):
        o1, l1 = o.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], window=3)
        assert np.array_equal(out[:, h:h + 1], o1) and np.array_equal(lse[:, h:h + 1], l1)


# ---------------------------------------------------------------------------------------------
# Backward pass (R14): the gradients are pinned to the forward oracle through finite
# differences, to autograd of torch's own attention and norm routines, and to invariants.
# ---------------------------------------------------------------------------------------------

def _fd_grad(f, x, h=1e-6):
    """Central differences of the scalar f at x (fp64), one element at a time."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def check_backward_finite_differences(o, seed=11):
    """attention_backward against central differences of attention's loss sum(dout * O), for
    multi-head and grouped heads, windows and the non-causal mask."""
    rng = _rng(seed)
    for (B, H, H_kv, T, d, window, causal) in [(1, 2, 2, 5, 4, -1, True), (1, 2, 1, 6, 4, 2, True),
                                               (2, 4, 2, 4, 2, 0, True), (1, 1, 1, 4, 3, -1, False)]:
        q = rng.standard_normal((B, H, T, d))
        k = rng.standard_normal((B, H_kv, T, d))
        v = rng.standard_normal((B, H_kv, T, d))
        do = rng.standard_normal((B, H, T, d))
        loss = lambda: float(np.sum(o.attention(q, k, v, window=window, causal=causal)[0] * do))
        dq, dk, dv = o.attention_backward(q, k, v, do, window=window, causal=causal)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            assert np.allclose(g, _fd_grad(loss, x), rtol=0, atol=2e-8), (B, H, H_kv, T, window)


def check_layer_backward_finite_differences(o, seed=12):
    """attention_layer_backward (prologue included) against central differences of
    attention_layer's loss, on raw rows of several scales."""
    rng = _rng(seed)
    for (H, H_kv, T, d, window, scale) in [(2, 2, 5, 4, -1, 1.0), (2, 1, 6, 4, 2, 3.0),
                                           (1, 1, 3, 8, -1, 0.1)]:
        q = scale * rng.standard_normal((1, H, T, d))
        k = scale * rng.standard_normal((1, H_kv, T, d))
        v = rng.standard_normal((1, H_kv, T, d))
        do = rng.standard_normal((1, H, T, d))
        loss = lambda: float(np.sum(o.attention_layer(q, k, v, window=window)[0] * do))
        dq, dk, dv = o.attention_layer_backward(q, k, v, do, window=window)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            assert np.allclose(g, _fd_grad(loss, x), rtol=0, atol=2e-7 / scale), (H, H_kv, T)


def check_backward_torch_autograd(o, seed=13):
    """Library special case: torch's scaled_dot_product_attention with an explicit boolean mask
    and torch's rms_norm, differentiated by autograd in float64 on the CPU; the rotation is
    applied as multiplication of the pairs (x_j + i x_{j+d/2}) by exp(-i theta)."""
    import torch
    import torch.nn.functional as F

    rng = _rng(seed)
    B, H, H_kv, T, d = 2, 4, 2, 37, 8
    for window, causal in ((-1, True), (5, True), (-1, False)):
        arrs = [rng.standard_normal(s) for s in ((B, H, T, d), (B, H_kv, T, d), (B, H_kv, T, d),
                                                (B, H, T, d))]
        q, k, v, do = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in arrs)
        i = torch.arange(T)[:, None]
        j = torch.arange(T)[None, :]
        mask = torch.ones(T, T, dtype=torch.bool)
        if causal:
            mask = j <= i
            if window >= 0:
                mask = mask & (i - j <= window)
        g = H // H_kv
        theta = torch.outer(torch.arange(T, dtype=torch.float64),
                            10000.0 ** (-torch.arange(0, d, 2, dtype=torch.float64) / d))

        def rot(x):
            z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * torch.polar(
                torch.ones_like(theta), -theta)
            return torch.cat([z.real, z.imag], dim=-1)

        for layer in (False, True):
            qq, kk = (rot(F.rms_norm(q, (d,), eps=1e-6)), rot(F.rms_norm(k, (d,), eps=1e-6))) \
                if layer else (q, k)
            out = F.scaled_dot_product_attention(qq, kk.repeat_interleave(g, dim=1),
                                                 v.repeat_interleave(g, dim=1), attn_mask=mask)
            gq, gk, gv = torch.autograd.grad((out * do.detach()).sum(), (q, k, v))
            args = [a.detach().numpy() for a in (q, k, v, do)]
            fn = o.attention_layer_backward if layer else o.attention_backward
            dq, dk, dv = fn(*args, window=window, causal=causal)
            for mine, ref in ((dq, gq), (dk, gk), (dv, gv)):
                assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-11), (window, causal, layer)


def check_backward_blocked(o, seed=19):
    """The backward's row blocks (three blocks of 256 rows at T = 600, windows around the block
    size and the inclusive boundary key r0 - W) against fp64 autograd of torch's
    ``scaled_dot_product_attention`` with an explicit mask over all T keys, grouped kv heads."""
    import torch
    import torch.nn.functional as F

    rng = _rng(seed)
    B, H, H_kv, T, d = 1, 2, 1, 600, 8
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    for window in (-1, 0, 255, 256, 257, 511):
        arrs = [rng.standard_normal(s) for s in ((B, H, T, d), (B, H_kv, T, d), (B, H_kv, T, d),
                                                (B, H, T, d))]
        q, k, v, do = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in arrs)
        mask = j <= i
        if window >= 0:
            mask = mask & (i - j <= window)
        out = F.scaled_dot_product_attention(q, k.repeat_interleave(H // H_kv, dim=1),
                                             v.repeat_interleave(H // H_kv, dim=1), attn_mask=mask)
        gq, gk, gv = torch.autograd.grad((out * do.detach()).sum(), (q, k, v))
        dq, dk, dv = o.attention_backward(*arrs, window=window, causal=True)
        for mine, ref in ((dq, gq), (dk, gk), (dv, gv)):
            assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-11), window


def check_backward_invariants(o, seed=14):
    """Exact properties of the gradients: every row of dS sums to zero, so the keys' gradients
    of a head sum to zero; with window 0 each query sees only its own key, so dq = dk = 0 and
    dv = dout; the norm's gradient is orthogonal to the row when eps = 0 (the norm is then scale
    invariant); the rotation's backward keeps each pair's length."""
    rng = _rng(seed)
    B, H, H_kv, T, d = 2, 4, 2, 19, 8
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H_kv, T, d))
    v = rng.standard_normal((B, H_kv, T, d))
    do = rng.standard_normal((B, H, T, d))
    for window in (-1, 4):
        dq, dk, dv = o.attention_backward(q, k, v, do, window=window)
        assert np.allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    k2 = rng.standard_normal((B, H, T, d))
    v2 = rng.standard_normal((B, H, T, d))
    dq, dk, dv = o.attention_backward(q, k2, v2, do, window=0)
    assert np.allclose(dq, 0.0, atol=1e-14) and np.allclose(dk, 0.0, atol=1e-14)
    assert np.allclose(dv, do, rtol=0, atol=1e-14)
    x = 3.0 * rng.standard_normal((5, 16))
    g = rng.standard_normal((5, 16))
    dx = o.rms_norm_backward(x, g, eps=0.0)
    assert np.allclose(np.sum(dx * x, axis=-1), 0.0, atol=1e-12)
    # a gradient along the output row itself maps to zero (eps = 0): d|xh|^2 is 0
    xh = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    assert np.allclose(o.rms_norm_backward(x, xh, eps=0.0), 0.0, atol=1e-12)
    cos, sin = o.rope_cos_sin(7, 16)
    gy = rng.standard_normal((7, 16))
    gx = o.rope_apply_backward(gy, cos, sin)
    n_in = gy[:, :8] ** 2 + gy[:, 8:] ** 2
    n_out = gx[:, :8] ** 2 + gx[:, 8:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13, atol=0)
    # and it undoes the forward rotation
    assert np.allclose(o.rope_apply_backward(o.rope_apply(gy, cos, sin), cos, sin), gy, atol=1e-13)


def check_decode(o, seed=15):
    """decode_attention against brute force with math.fsum, torch's scaled_dot_product_attention
    on the one query row, the zero-query closed form (uniform weights over the visible keys),
    and the last row of the (independently pinned) causal attention over the whole prefix."""
    import torch
    import torch.nn.functional as F

    rng = _rng(seed)
    B, H, H_kv, S, d = 3, 4, 2, 9, 4
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, H_kv, S, d))
    v = rng.standard_normal((B, H_kv, S, d))
    lengths = [1, 5, 9]
    for window in (-1, 0, 2, 20):
        out, lse = o.decode_attention(q, k, v, lengths, window)
        for b, n in enumerate(lengths):
            lo = 0 if window < 0 else max(0, n - 1 - window)
            for h in range(H):
                g = h // (H // H_kv)
                s = [math.fsum(q[b, h, c] * k[b, g, j, c] for c in range(d)) / math.sqrt(d)
                     for j in range(lo, n)]
                m = max(s)
                ll = m + math.log(math.fsum(math.exp(x - m) for x in s))
                assert abs(lse[b, h] - ll) < 1e-12
                for c in range(d):
                    ref = math.fsum(math.exp(s[i] - ll) * v[b, g, lo + i, c] for i in range(len(s)))
                    assert abs(out[b, h, c] - ref) < 1e-12
                ts = F.scaled_dot_product_attention(
                    torch.tensor(q[b, h][None, None, None]), torch.tensor(k[b, g, lo:n][None, None]),
                    torch.tensor(v[b, g, lo:n][None, None]))
                assert np.allclose(ts.numpy()[0, 0, 0], out[b, h], rtol=0, atol=1e-12)
    out, lse = o.decode_attention(np.zeros_like(q), k, v, lengths, 3)
    for b, n in enumerate(lengths):
        lo = max(0, n - 4)
        for h in range(H):
            g = h // (H // H_kv)
            assert np.allclose(out[b, h], v[b, g, lo:n].mean(axis=0), atol=1e-13)
            assert abs(lse[b, h] - math.log(n - lo)) < 1e-13
    # the newest token's row of the causal attention over the prefix
    for n, window in ((9, -1), (7, 3)):
        qs = rng.standard_normal((1, H, n, d))
        ro, rl = o.attention(qs, k[:1, :, :n], v[:1, :, :n], window=window)
        out, lse = o.decode_attention(qs[:, :, n - 1], k[:1], v[:1], [n], window)
        assert np.allclose(out, ro[:, :, n - 1], atol=1e-13) and np.allclose(lse, rl[:, :, n - 1], atol=1e-13)


# ---------------------------------------------------------------------------------------------
# Value-embedding gate (R16): closed forms of the sigmoid, brute force per row, torch's sigmoid,
# the layer's special cases; its gradients against finite differences and autograd.
# ---------------------------------------------------------------------------------------------

def check_value_gate(o, seed=16):
    """gate = 2 sigmoid(z): exactly 1 at z = 0 (the neutral value), 0 and 2 in the limits,
    gate(z) + gate(-z) = 2; v + gate * ve row by row (pure-Python loop); 2 * torch.sigmoid in
    float64; a layer whose gates are all 0 equals the layer without the embedding, and one whose
    gates are all 1 equals the layer on v + ve."""
    import torch

    rng = _rng(seed)
    assert o.gate_of(np.array(0.0)) == 1.0
    assert o.gate_of(np.array(-800.0)) == 0.0 and o.gate_of(np.array(800.0)) == 2.0
    z = rng.standard_normal(50) * 6
    assert np.allclose(o.gate_of(z) + o.gate_of(-z), 2.0, rtol=0, atol=1e-15)
    assert np.allclose(o.gate_of(z), 2 * torch.sigmoid(torch.tensor(z, dtype=torch.float64)).numpy(),
                       rtol=1e-15, atol=1e-16)
    assert np.all((o.gate_of(z) > 0) & (o.gate_of(z) < 2))
    B, H_kv, T, d = 2, 3, 5, 4
    v = rng.standard_normal((B, H_kv, T, d))
    ve = rng.standard_normal((B, H_kv, T, d))
    z = rng.standard_normal((B, H_kv, T)) * 3
    out = o.value_gate(v, ve, z)
    for b in range(B):
        for h in range(H_kv):
            for t in range(T):
                gt = 2.0 / (1.0 + math.exp(-z[b, h, t]))
                for c in range(d):
                    assert abs(out[b, h, t, c] - (v[b, h, t, c] + gt * ve[b, h, t, c])) < 1e-14
    H = 6
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H_kv, T, d))
    for window in (-1, 2):
        ro, rl = o.attention_layer(q, k, v, window=window)
        go, gl = o.attention_layer_ve(q, k, v, ve, np.full(z.shape, -800.0), window=window)
        assert np.array_equal(ro, go) and np.array_equal(rl, gl)
        ro, rl = o.attention_layer(q, k, v + ve, window=window)
        go, gl = o.attention_layer_ve(q, k, v, ve, np.zeros(z.shape), window=window)
        assert np.array_equal(ro, go) and np.array_equal(rl, gl)


def check_value_gate_backward(o, seed=17):
    """value_gate_backward and attention_layer_ve_backward against central differences of the
    forward oracle, and against autograd of v + 2 * torch.sigmoid(z) * ve in float64."""
    import torch

    rng = _rng(seed)
    B, H_kv, T, d = 1, 2, 4, 3
    v = rng.standard_normal((B, H_kv, T, d))
    ve = rng.standard_normal((B, H_kv, T, d))
    z = rng.standard_normal((B, H_kv, T)) * 2
    dy = rng.standard_normal((B, H_kv, T, d))
    loss = lambda: float(np.sum(o.value_gate(v, ve, z) * dy))
    dv, dve, dz = o.value_gate_backward(ve, z, dy)
    for x, g in ((v, dv), (ve, dve), (z, dz)):
        assert np.allclose(g, _fd_grad(loss, x), rtol=0, atol=1e-8)
    tv, tve, tz = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (v, ve, z))
    y = tv + 2 * torch.sigmoid(tz)[..., None] * tve
    gv, gve, gz = torch.autograd.grad((y * torch.tensor(dy)).sum(), (tv, tve, tz))
    for mine, ref in ((dv, gv), (dve, gve), (dz, gz)):
        assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-14)
    H = 4
    q = rng.standard_normal((B, H, T, d + 1))
    k = rng.standard_normal((B, H_kv, T, d + 1))
    v = rng.standard_normal((B, H_kv, T, d + 1))
    ve = rng.standard_normal((B, H_kv, T, d + 1))
    do = rng.standard_normal((B, H, T, d + 1))
    for window in (-1, 1):
        loss = lambda: float(np.sum(o.attention_layer_ve(q, k, v, ve, z, window=window)[0] * do))
        grads = o.attention_layer_ve_backward(q, k, v, ve, z, do, window=window)
        for x, g in zip((q, k, v, ve, z), grads):
            assert np.allclose(g, _fd_grad(loss, x), rtol=0, atol=3e-7), window


VALUE_GATE_CHECKS = [check_value_gate, check_value_gate_backward]


BACKWARD_CHECKS = [
    check_backward_finite_differences,
    check_layer_backward_finite_differences,
    check_backward_torch_autograd,
    check_backward_blocked,
    check_backward_invariants,
]


ALL_CHECKS = [
    check_worked_example,
    check_worked_example_qknorm,
    check_brute_force,
    check_sdpa_special_case,
    check_blocked_rows,
    check_weights_sum_to_one,
    check_masked_entries_have_no_weight,
    check_window_T_is_causal,
    check_window_zero,
    check_zero_query_closed_form,
    check_rms_norm,
    check_rope_special_values,
    check_rope_invariants,
    check_norm_rope_commute,
    check_sssl_windows,
    check_gqa_head_mapping,
    check_decode,
] + BACKWARD_CHECKS + VALUE_GATE_CHECKS
