"""GPU check of attn_decode_noalloc_ex, the allocation-free decode entry point (its split
partials live in the library's fixed device scratch): through the C ABI, its outputs must equal
attn_decode_ex's (same kernels, caller workspace) bit for bit on consecutive calls whose sizes
shrink, so that nothing a larger call left in the scratch leaks into a smaller one; both are
also checked against the fp64 oracle's decode_attention (max-abs 2e-2 in bf16, 1e-5 in fp32).
Every call prints its case before touching the GPU."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_qk_amd import _lib, inputs

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


def _case(dt, d, B, H, H_kv, S, lengths, window, layout, seed):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q = inputs.make_random((B, H, d), dtype, seed)
    k = inputs.make_random((B, H_kv, S, d), dtype, seed + 1)
    v = inputs.make_random((B, H_kv, S, d), dtype, seed + 2)
    tl = lambda x: (x.transpose(1, 2) if layout == "bthd" else x).contiguous().cuda()
    lens = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda")
    return dict(dt=dt, d=d, B=B, H=H, H_kv=H_kv, S=S, lengths=lengths, window=window,
                layout=layout, q=q, k=k, v=v, qg=q.cuda(), kg=tl(k), vg=tl(v), lens=lens,
                dtype=dtype)


def _run(c, noalloc):
    lib = _lib.load()
    B, H, d = c["B"], c["H"], c["d"]
    out = torch.full((B, H, d), float("nan"), dtype=c["dtype"], device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    lay = _lib.ATTN_LAYOUT_BTHD if c["layout"] == "bthd" else _lib.ATTN_LAYOUT_BHTD
    dt = _lib.ATTN_BF16 if c["dt"] == "bf16" else _lib.ATTN_F32
    stream = torch.cuda.current_stream().cuda_stream
    lens = c["lens"].data_ptr() if c["lens"] is not None else None
    torch.cuda.synchronize()
    if noalloc:
        before = torch.cuda.memory_allocated()
        rc = lib.attn_decode_noalloc_ex(c["qg"].data_ptr(), c["kg"].data_ptr(), c["vg"].data_ptr(),
                                        lens, out.data_ptr(), lse.data_ptr(), B, H, c["H_kv"],
                                        c["S"], d, lay, c["window"], dt, stream)
        assert torch.cuda.memory_allocated() == before
    else:
        need = lib.attn_decode_workspace_bytes(B, H, c["S"], d, c["window"])
        ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device="cuda")
        rc = lib.attn_decode_ex(c["qg"].data_ptr(), c["kg"].data_ptr(), c["vg"].data_ptr(), lens,
                                out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel() * 4, B,
                                H, c["H_kv"], c["S"], d, lay, c["window"], dt, stream)
    assert rc == _lib.ATTN_OK, lib.attn_strerror(rc).decode()
    torch.cuda.synchronize()
    return out, lse


# Consecutive calls, each smaller than the one before (all but the last two take the split path
# with the merge, i.e. use the scratch; the last is one split per head).
SEQUENCES = [
    [("bf16", 128, 2, 8, 2, 5000, [5000, 3001], -1, "bhtd"),
     ("bf16", 64, 1, 4, 4, 700, [700], 100, "bthd")],
    [("bf16", 64, 1, 8, 8, 100000, [99999], 70000, "bthd"),
     ("bf16", 64, 1, 8, 8, 3000, [2999], -1, "bthd"),
     ("f32", 32, 2, 4, 2, 900, [900, 17], -1, "bhtd")],
    [("f32", 128, 1, 4, 2, 20000, None, -1, "bhtd"),
     ("bf16", 32, 2, 2, 1, 600, [600, 300], 50, "bhtd"),
     ("bf16", 64, 16, 8, 8, 1024, None, -1, "bhtd")],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=[f"seq{i}" for i in range(len(SEQUENCES))])
def test_noalloc_decode_matches_workspace_decode(seq):
    lib = _lib.load()
    for i, spec in enumerate(seq):
        dt, d, B, H, H_kv, S, lengths, window, layout = spec
        say(f"noalloc decode call {i}: {dt} d={d} B={B} H={H} H_kv={H_kv} S={S} "
            f"lengths={lengths} W={window} {layout}")
        assert lib.attn_decode_workspace_bytes(B, H, S, d, window) <= _lib.ATTN_DECODE_SCRATCH_BYTES
        c = _case(*spec, seed=700 + 10 * i)
        o_ref, l_ref = _run(c, noalloc=False)
        o_na, l_na = _run(c, noalloc=True)
        assert torch.equal(o_na.view(torch.int16 if dt == "bf16" else torch.int32),
                           o_ref.view(torch.int16 if dt == "bf16" else torch.int32)), spec
        assert torch.equal(l_na.view(torch.int32), l_ref.view(torch.int32)), spec
        ro, rl = oracle.decode_attention(f64(c["q"]), f64(c["k"]), f64(c["v"]), lengths, window)
        tol = 2e-2 if dt == "bf16" else 1e-5
        eo = float(np.max(np.abs(f64(o_na) - ro)))
        el = float(np.max(np.abs(f64(l_na) - rl)))
        say(f"  bitwise equal to attn_decode_ex; max|dO|={eo:.2e} max|dLSE|={el:.2e} (tol {tol})")
        assert eo <= tol and el <= max(tol, 1e-5), spec


def test_noalloc_decode_rejects_past_the_scratch():
    lib = _lib.load()
    B, H, S, d = 1, _lib.ATTN_DECODE_SCRATCH_BYTES // (130 * 4) + 1, 128, 128
    say(f"noalloc decode past the scratch: B={B} H={H} S={S} d={d} (no launch)")
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 1, S, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    rc = lib.attn_decode_noalloc_ex(q.data_ptr(), k.data_ptr(), k.data_ptr(), None,
                                    out.data_ptr(), None, B, H, 1, S, d, _lib.ATTN_LAYOUT_BHTD,
                                    -1, _lib.ATTN_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.ATTN_ERR_SCRATCH
