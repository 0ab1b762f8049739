"""fp64 CPU oracle: QK-RMSNorm, RoPE and causal / sliding-window softmax attention, written out
from their plain definitions.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``; never by the HIP library or its Python binding. It shares no code, tables or
constants with the GPU path. Everything is float64 numpy. No blocking, fusion or reordering is done
beyond what the definitions state. The one exception is that rows are processed in blocks and each
block only scores the key range that can be visible to it; the skipped entries are exact zeros of
the softmax.

Sources (page title, then the part of the page used):

[HABR]  "Подробный технический разбор реализации Autoresearch, ИИ-исследователя Андрея Карпаты"
        (habr.com, article 1010198), its train.py listing: ``norm``, ``apply_rotary_emb``,
        ``GPT._precompute_rotary_embeddings``, ``GPT._compute_window_sizes``,
        ``CausalSelfAttention.forward``, ``GPT.estimate_flops``.
[GEOM]  "Projeção em um Subespaço de Consulta" (unhomeschool.com, geometry_of_andrea), sections
        "O que a Atenção Calcula", "A Máscara Causal", "Escalonamento por sqrt(d_k)" and
        "Lendo uma Projeção".
[CNOYU] The web3.cnoyu.net commentary on autoresearch's train.py: the passage on QK-norm and on
        the SSSL window pattern.

Readings taken where the pages are silent or disagree:

R1  RMSNorm has no weight and eps = 1e-6 ([HABR] ``norm`` passes no eps or weight).
R2  Norm then RoPE. [HABR] ``CausalSelfAttention.forward`` rotates first and normalises second.
    The two orders give the same result, because the half-split rotation preserves the sum of
    squares of a row and the norm has no weight. A test checks this.
R3  RoPE angles are exact (fp64): theta[t, j] = t * base**(-2j/d), base 10000. [HABR] rounds
    its table to bf16; that is a storage choice of that code and is not copied.
R4  ``window = W >= 0`` makes key j visible to query i iff 0 <= i - j <= W. This is the inclusive
    (W, 0) range of the FlashAttention call in [HABR] ``CausalSelfAttention.forward``. ``W < 0``
    means unlimited, as in [HABR] ``GPT.estimate_flops``.
R5  ``causal = False`` means every key is visible (no window is allowed then).
R6  LSE is the natural-log logsumexp of the scaled scores over the visible keys.
R13 Grouped-query attention ([HABR] ``GPTConfig.n_kv_head`` and ``CausalSelfAttention``: k and v
    carry n_kv_head heads, n_kv_head divides n_head). The pages do not say which query heads share
    a kv head; consecutive groups do: query head h uses kv head h // (n_head // n_kv_head).

Parity pins: the tests under ``tests/test_oracle_*.py`` check every function here against
closed forms, the worked example of [GEOM], brute force and library special cases.
"""

from __future__ import annotations

import math

import numpy as np

EPS_DEFAULT = 1e-6  # R1
ROPE_BASE_DEFAULT = 10000.0  # [HABR] GPT._precompute_rotary_embeddings default base


def sssl_windows(T: int, n_layer: int, pattern: str = "SSSL") -> list[int]:
    """Per-layer window sizes of the SSSL schedule.

    [HABR] ``GPT._compute_window_sizes``: layer l takes ``pattern[l % len(pattern)]``; "L" is the
    full sequence length and "S" is half of it (integer division); the last layer is always "L".
    [CNOYU] describes the same pattern: three half-length windows, then one full layer.
    """
    pattern = pattern.upper()
    if not pattern or any(c not in "SL" for c in pattern):
        raise ValueError(f"window pattern must be a non-empty string over 'S','L', got {pattern!r}")
    if n_layer < 1:
        raise ValueError("n_layer must be >= 1")
    long_w, short_w = T, T // 2
    wins = [long_w if pattern[l % len(pattern)] == "L" else short_w for l in range(n_layer)]
    wins[-1] = long_w
    return wins


def rms_norm(x: np.ndarray, eps: float = EPS_DEFAULT) -> np.ndarray:
    """Weightless RMSNorm over the last axis: x / sqrt(mean(x^2) + eps).

    [HABR] ``norm`` (``F.rms_norm(x, (x.size(-1),))``); R1.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def rope_cos_sin(T: int, d: int, base: float = ROPE_BASE_DEFAULT) -> tuple[np.ndarray, np.ndarray]:
    """cos and sin of theta[t, j] = t * base**(-2j/d), for t < T and j < d/2, as fp64 [T, d/2].

    [HABR] ``GPT._precompute_rotary_embeddings``: the channel frequencies are 1/base**(2j/d) over
    even channel indices 2j, the positions are 0..T-1, and the angles are their outer product. R3.
    """
    if d % 2:
        raise ValueError("head dim must be even for RoPE")
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = 1.0 / (base ** (2.0 * j / d))
    t = np.arange(T, dtype=np.float64)
    theta = np.outer(t, inv_freq)
    return np.cos(theta), np.sin(theta)


def rope_apply(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Half-split rotary embedding of x [..., T, d] at positions 0..T-1.

    [HABR] ``apply_rotary_emb``: with x1 = x[..., :d/2] and x2 = x[..., d/2:],
    y1 = x1*cos + x2*sin and y2 = -x1*sin + x2*cos, concatenated as [y1, y2].
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    y1 = x1 * cos + x2 * sin
    y2 = x1 * (-sin) + x2 * cos
    return np.concatenate([y1, y2], axis=-1)


def qknorm_rope(q: np.ndarray, k: np.ndarray, eps: float = EPS_DEFAULT,
                base: float = ROPE_BASE_DEFAULT) -> tuple[np.ndarray, np.ndarray]:
    """QK-norm then RoPE on q, k [B, H, T, d] (R2).

    [HABR] ``CausalSelfAttention.forward``: q and k are rotated with ``apply_rotary_emb`` and
    normalised with ``norm`` right before the attention call; [CNOYU] describes the same norm
    on the queries and keys just before the dot product.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    T, d = q.shape[-2], q.shape[-1]
    cos, sin = rope_cos_sin(T, d, base)
    return rope_apply(rms_norm(q, eps), cos, sin), rope_apply(rms_norm(k, eps), cos, sin)


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head that query head h of H attends with when k and v have H_kv heads (R13)."""
    if H_kv < 1 or H % H_kv:
        raise ValueError("the kv head count must divide the query head count")
    return h // (H // H_kv)


def visible(i: np.ndarray, j: np.ndarray, window: int = -1, causal: bool = True) -> np.ndarray:
    """Boolean visibility of key j to query i (broadcasting).

    [GEOM] "A Máscara Causal": entries above the diagonal of QK^T are -inf, so token t sees
    tokens 0..t. Window: R4. Non-causal: R5.
    """
    i = np.asarray(i)
    j = np.asarray(j)
    if not causal:
        if window >= 0:
            raise ValueError("a window needs causal=True")
        return np.ones(np.broadcast(i, j).shape, dtype=bool)
    vis = j <= i
    if window >= 0:
        vis &= (i - j) <= window
    return vis


def _key_range(r0: int, r1: int, T: int, window: int, causal: bool) -> tuple[int, int]:
    """Smallest key interval [lo, hi) that holds every key visible to rows r0..r1-1."""
    if not causal:
        return 0, T
    hi = min(T, r1)
    lo = 0 if window < 0 else max(0, r0 - window)
    return lo, hi


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int = -1, causal: bool = True,
              rows: np.ndarray | None = None, block: int = 256) -> tuple[np.ndarray, np.ndarray]:
    """softmax(q k^T / sqrt(d) + mask) v and its logsumexp, in fp64.

    q: [B, H, T, d]; k, v: [B, H_kv, T, d] with H_kv dividing H (R13; H_kv = H is plain
    multi-head attention). Returns (O, LSE) with O [B, H, R, d] and LSE [B, H, R], where R = T,
    or R = len(rows) when ``rows`` (query indices, applied to every head) is given.

    [GEOM] "O que a Atenção Calcula" (softmax(Q K^T / sqrt(d_k)) V: the weights of a row sum to 1
    and mix the rows of V), "Escalonamento por sqrt(d_k)" (the 1/sqrt(d_k) scale) and
    "A Máscara Causal" (masked entries get weight 0). [HABR] ``CausalSelfAttention.forward``
    passes no scale to the attention call, so the default 1/sqrt(d) applies. Mask: R4, R5.
    LSE: R6. The softmax is the plain two-pass form: the row maximum m, then
    LSE = m + ln(sum exp(s - m)), then weights exp(s - LSE).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if (q.ndim != 4 or k.ndim != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]
            or v.shape[:3] != k.shape[:3]):
        raise ValueError("q must be [B, H, T, d] and k, v [B, H_kv, T, d] (q, k the same d)")
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    dv = v.shape[-1]
    if not causal and window >= 0:
        raise ValueError("a window needs causal=True")
    row_idx = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    if row_idx.size and (row_idx.min() < 0 or row_idx.max() >= T):
        raise ValueError("row index out of range")
    R = row_idx.size
    out = np.zeros((B, H, R, dv), dtype=np.float64)
    lse = np.zeros((B, H, R), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for s0 in range(0, R, block):
        ridx = row_idx[s0:s0 + block]
        lo, hi = _key_range(int(ridx.min()), int(ridx.max()) + 1, T, window, causal)
        keys = np.arange(lo, hi)
        vis = visible(ridx[:, None], keys[None, :], window, causal)  # [r, n]
        for b in range(B):
            for h in range(H):
                g = kv_head(h, H, H_kv)
                s = (q[b, h, ridx] @ k[b, g, lo:hi].T) * scale  # [r, n]
                s = np.where(vis, s, -np.inf)
                m = np.max(s, axis=1, keepdims=True)
                row_lse = m + np.log(np.sum(np.exp(s - m), axis=1, keepdims=True))
                p = np.exp(s - row_lse)
                out[b, h, s0:s0 + ridx.size] = p @ v[b, g, lo:hi]
                lse[b, h, s0:s0 + ridx.size] = row_lse[:, 0]
    return out, lse


def attention_layer(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int = -1,
                    causal: bool = True, eps: float = EPS_DEFAULT, base: float = ROPE_BASE_DEFAULT,
                    rows: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """One layer of the attention block: QK-norm + RoPE on raw q, k, then attention.

    [HABR] ``CausalSelfAttention.forward`` from the rotary step to the attention call.
    """
    qn, kn = qknorm_rope(q, k, eps, base)
    return attention(qn, kn, v, window, causal, rows=rows)


def decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     lengths=None, window: int = -1) -> tuple[np.ndarray, np.ndarray]:
    """One generation step: the newest token's query against the cached keys and values, fp64.

    q: [B, H, d] (the query of the token at position n_b - 1); k_cache, v_cache: [B, H_kv, S, d]
    with H_kv dividing H (R13); lengths: n_b per batch (1 <= n_b <= S; None means S). Returns
    (O [B, H, d], LSE [B, H]).

    [GEOM] "A Máscara Causal": training and inference are the same forward pass, so the newest
    token attends exactly as the last row of the causal attention does: to the tokens 0..n-1,
    cut to n - 1 - j <= window when window >= 0 (R4). [CNOYU]/[HABR] generation appends one
    token at a time ("O Que um Modelo de Linguagem Prevê": autoregressive generation).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_cache, dtype=np.float64)
    v = np.asarray(v_cache, dtype=np.float64)
    B, H, d = q.shape
    H_kv, S = k.shape[1], k.shape[2]
    if k.shape != (B, H_kv, S, d) or v.shape[:3] != (B, H_kv, S):
        raise ValueError("k_cache, v_cache must be [B, H_kv, S, d] with q [B, H, d]")
    lengths = [S] * B if lengths is None else [int(n) for n in lengths]
    if any(n < 1 or n > S for n in lengths):
        raise ValueError("lengths must lie in [1, S]")
    out = np.zeros((B, H, v.shape[-1]))
    lse = np.zeros((B, H))
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        n = lengths[b]
        lo = 0 if window < 0 else max(0, n - 1 - window)
        for h in range(H):
            g = kv_head(h, H, H_kv)
            s = (k[b, g, lo:n] @ q[b, h]) * scale
            m = np.max(s)
            row_lse = m + np.log(np.sum(np.exp(s - m)))
            out[b, h] = np.exp(s - row_lse) @ v[b, g, lo:n]
            lse[b, h] = row_lse
    return out, lse
