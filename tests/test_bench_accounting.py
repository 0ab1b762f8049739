"""The bench's work accounting on the CPU: the closed-form pair count equals the number of
entries the oracle's mask keeps, and the headline stack comes to 83.89 GFLOP."""

import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("T", [1, 2, 3, 17, 64, 130])
def test_visible_pairs_match_the_oracle_mask(T):
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    for window in [-1, 0, 1, 2, T // 2, T - 2, T - 1, T, 3 * T]:
        if window < -1:
            continue
        n = int(oracle.visible(i, j, window, True).sum())
        assert bench.visible_pairs(T, window) == n, (T, window)
    assert bench.visible_pairs(T, -1, causal=False) == int(oracle.visible(i, j, -1, False).sum())


def test_headline_stack_flops():
    wins = oracle.sssl_windows(1024, 4)
    total = sum(bench.attn_flops(16, 12, 1024, 64, W) for W in wins)
    assert total == 83_890_274_304  # 3 x 393,984 + 524,800 pairs per head, x 4d x 192 heads
    assert bench.attn_compulsory_bytes(16, 12, 1024, 64) == 16 * 12 * 1024 * (8 * 64 + 4)


def test_bench_refuses_more_than_one_gpu(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err


def test_prologue_bytes():
    # each tensor read once and written once, bf16
    assert bench.prologue_bytes(16, 12, 1024, 64, tensors=1) == 16 * 12 * 1024 * 64 * 2 * 2
    assert bench.prologue_bytes(16, 12, 1024, 64) == 2 * bench.prologue_bytes(16, 12, 1024, 64, tensors=1)


def test_cpu_baseline_pool_counts_every_head():
    """The CPU baseline's process pool runs every (batch, head) of every layer through the oracle
    and counts the same unmasked FLOPs as the GPU numerator (a small synthetic workload)."""
    import collections

    import torch

    W = collections.namedtuple("W", "name B H T d")
    w = W("tiny", 2, 3, 40, 8)
    g = torch.Generator().manual_seed(0)
    layers = [tuple(torch.randn(2, 3, 40, 8, generator=g) for _ in range(3)) for _ in range(2)]
    wins = [20, 40]
    r = bench.cpu_baseline(w, layers, wins, 2)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    flops = sum(bench.attn_flops(2, 3, 40, 8, W_) for W_ in wins)
    assert abs(r["value"] * 1e12 * r["seconds"] - flops) <= 1e-6 * flops
