"""GPU parity of attn_decode_ex (one new query per head against a KV cache) with the fp64
oracle's decode_attention, through the C ABI; plus its agreement with the last row of the
prefill kernel. Tolerances: bf16 max-abs 2e-2 (outputs) and 2e-2 (LSE), fp32 1e-5; the decode
path keeps its weights in fp32, so its errors are the inputs' and the output's rounding only.
Every case prints its name before touching the GPU."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_qk_amd import _lib, inputs, ops

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    torch.cuda.synchronize()


# (dtype, d, B, H, H_kv, S, lengths, window, layout)
CASES = []
for _d in (32, 64, 128):
    CASES += [("bf16", _d, 2, 4, 4, 1, [1, 1], -1, "bhtd"),
              ("bf16", _d, 3, 4, 2, 300, [1, 129, 300], -1, "bhtd"),
              ("bf16", _d, 2, 8, 1, 1000, [1000, 517], 200, "bthd"),
              ("bf16", _d, 2, 4, 2, 260, None, 0, "bthd"),
              ("bf16", _d, 1, 16, 16, 128, [128], 127, "bhtd")]
for _d in (16, 64, 128):
    CASES += [("f32", _d, 2, 4, 2, 150, [150, 3], -1, "bhtd"), ("f32", _d, 2, 2, 2, 90, None, 5, "bthd")]
CASES += [("bf16", 64, 2, 24, 2, 700, [700, 1], -1, "bhtd")]  # 12 query heads per kv head
# Long caches over few heads: the splits are capped, so each wave takes several batches of rows
# (with GQA: re-read for every query head of the group).
CASES += [("bf16", 128, 2, 8, 2, 40000, [40000, 12345], -1, "bhtd"),
          ("bf16", 64, 1, 8, 8, 100000, [99999], 70000, "bthd"),
          ("f32", 128, 1, 4, 2, 70000, None, -1, "bhtd")]
# Many (batch, kv head) pairs and short caches: one split per pair, written without the merge
# (at d = 64 up to 1024 keys; the next size takes the split path).
CASES += [("bf16", 64, 16, 8, 8, 1024, [1024, 1, 513, 1000] * 4, -1, "bhtd"),
          ("bf16", 64, 16, 8, 8, 1025, None, -1, "bhtd"),
          ("bf16", 64, 16, 8, 8, 1100, [1100, 7] * 8, 300, "bthd"),
          ("bf16", 128, 32, 8, 4, 512, None, 100, "bthd"),
          ("bf16", 32, 8, 16, 16, 2048, [2048, 2, 1500, 999] * 2, -1, "bhtd"),
          ("f32", 16, 4, 32, 32, 700, [700, 1, 350, 699], 64, "bhtd")]


@pytest.mark.parametrize("dt,d,B,H,H_kv,S,lengths,window,layout", CASES,
                         ids=[f"{c[0]}-d{c[1]}-B{c[2]}H{c[3]}k{c[4]}S{c[5]}-W{c[7]}-{c[8]}-{i}"
                              for i, c in enumerate(CASES)])
def test_decode_parity(dt, d, B, H, H_kv, S, lengths, window, layout):
    say(f"decode {dt} d={d} B={B} H={H} H_kv={H_kv} S={S} lengths={lengths} W={window} {layout}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q = inputs.make_random((B, H, d), dtype, 501)
    k = inputs.make_random((B, H_kv, S, d), dtype, 502)
    v = inputs.make_random((B, H_kv, S, d), dtype, 503)
    tl = lambda x: (x.transpose(1, 2) if layout == "bthd" else x).contiguous().cuda()
    lens = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda")
    out, lse = ops.decode(q.cuda(), tl(k), tl(v), lens, window=window, layout=layout)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attention(f64(q), f64(k), f64(v), lengths, window)
    eo = float(np.max(np.abs(f64(out) - ro)))
    el = float(np.max(np.abs(f64(lse) - rl)))
    say(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    tol = 2e-2 if dt == "bf16" else 1e-5
    assert eo <= tol and el <= tol


def test_decode_matches_prefill_last_row():
    """A decode step over a prefix equals the last row of the prefill kernel on that prefix
    (within bf16 rounding: prefill rounds its weights to bf16, decode keeps them fp32)."""
    B, H, T, d = 2, 4, 333, 64
    say("decode vs prefill last row")
    q, k, v = (inputs.make_random((B, H, T, d), torch.bfloat16, s).cuda() for s in (511, 512, 513))
    for window in (-1, 100):
        out, lse = ops.attn_fwd(q, k, v, window=window)
        dout, dlse = ops.decode(q[:, :, -1].contiguous(), k, v, None, window=window)
        torch.cuda.synchronize()
        assert float((dout.float() - out[:, :, -1].float()).abs().max()) <= 2e-2
        assert float((dlse - lse[:, :, -1]).abs().max()) <= 2e-2


def test_decode_lengths_only_read_valid_slots():
    """Slots past lengths[b] are never read: filling them with huge values changes nothing
    (bitwise); the workspace may be reused by consecutive calls on one stream."""
    B, H, S, d = 2, 4, 400, 64
    say("decode ignores slots past the length")
    q = inputs.make_random((B, H, d), torch.bfloat16, 521).cuda()
    k, v = (inputs.make_random((B, H, S, d), torch.bfloat16, s).cuda() for s in (522, 523))
    lens = torch.tensor([250, 7], dtype=torch.int32, device="cuda")
    ws = torch.empty((ops._lib.load().attn_decode_workspace_bytes(B, H, S, d, -1) // 4,),
                     dtype=torch.float32, device="cuda")
    o1, l1 = ops.decode(q, k, v, lens, workspace=ws)
    o1, l1 = o1.clone(), l1.clone()
    k2, v2 = k.clone(), v.clone()
    k2[0, :, 250:] = 1e4
    v2[0, :, 250:] = -1e4
    k2[1, :, 7:] = 1e4
    o2, l2 = ops.decode(q, k2, v2, lens, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_validation_with_real_buffers():
    lib = _lib.load()
    q = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 10, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty((1024,), dtype=torch.float32, device="cuda")
    rc = lib.attn_decode(q.data_ptr(), k.data_ptr(), k.data_ptr(), None, out.data_ptr(), None,
                         ws.data_ptr(), 16, 1, 2, 10, 64, -1, _lib.ATTN_BF16, None)
    assert rc == _lib.ATTN_ERR_ARG  # workspace too small
    rc = lib.attn_decode(q.data_ptr(), k.data_ptr(), k.data_ptr(), None, q.data_ptr(), None,
                         ws.data_ptr(), 4096, 1, 2, 10, 64, -1, _lib.ATTN_BF16, None)
    assert rc == _lib.ATTN_ERR_ALIAS
    rc = lib.attn_decode(q.data_ptr(), k.data_ptr(), k.data_ptr(), None, out.data_ptr(), None,
                         ws.data_ptr(), 4096, 1, 2, 10, 64, -1, _lib.ATTN_BF16, None)
    assert rc == _lib.ATTN_OK
    torch.cuda.synchronize()


def test_decode_long_cache():
    """One step against a long cache: S = 131072 (d = 64, bf16, two kv heads shared by four query
    heads), lengths at the cache's end, in its middle and of one token, full and windowed."""
    B, H, H_kv, S, d = 3, 4, 2, 131072, 64
    lengths = [S, S // 2 + 7, 1]
    for window in (-1, 4096):
        print(f"decode long cache S={S} window={window}", flush=True)
        q = inputs.make_random((B, H, d), torch.bfloat16, 151)
        k = inputs.make_random((B, H_kv, S, d), torch.bfloat16, 152)
        v = inputs.make_random((B, H_kv, S, d), torch.bfloat16, 153)
        ln = torch.tensor(lengths, dtype=torch.int32).cuda()
        out, lse = ops.decode(q.cuda(), k.cuda(), v.cuda(), ln, window=window)
        torch.cuda.synchronize()
        f64 = lambda t: t.detach().cpu().to(torch.float64).numpy()
        ro, rl = oracle.decode_attention(f64(q), f64(k), f64(v), lengths, window)
        eo = float(np.max(np.abs(f64(out) - ro)))
        el = float(np.max(np.abs(f64(lse) - rl)))
        print(f"   max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        assert eo <= 2e-2 and el <= 2e-2
