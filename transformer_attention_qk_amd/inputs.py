"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws random numbers and describes shapes. It holds none of the method's
arithmetic (no norm, rotation, mask or softmax) so that the oracle and the HIP path share nothing
but their inputs.

Shapes follow the ANDREA family table ("Uma Família de Três" on "O Que um Modelo de Linguagem
Prevê", unhomeschool.com): d_model / heads give the head dims 32 (12M) and 64 (120M, 480M), all
at context 1024. The pages measure attention on no public benchmark, so seeded N(0, 1) tensors
stand in for the q, k, v activations of a trained model. After QK-norm their rows have unit RMS,
as in the model the pages describe.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: str  # "bf16" or "f32": the dtype q, k, v, out are stored and multiplied in
    pattern: str  # layer window pattern over "S"/"L"
    n_layer: int
    v_dist: str = "normal"  # "normal": N(0, 1); "uniform": U(-1, 1)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS: tuple[Workload, ...] = (
    # Tiny fp32 attention, one full causal layer (window = T).
    Workload("tiny_f32", B=1, H=2, T=64, d=16, dtype="f32", pattern="L", n_layer=1),
    # ANDREA-12M shape: d_model 384 / 12 heads, one full causal layer.
    Workload("andrea12m", B=8, H=12, T=1024, d=32, dtype="bf16", pattern="L", n_layer=1),
    # ANDREA-120M shape: d_model 768 / 12 heads, SSSL stack of 4 layers.
    Workload("andrea120m_sssl", B=16, H=12, T=1024, d=64, dtype="bf16", pattern="SSSL", n_layer=4),
    # ANDREA-480M shape: d_model 1536 / 24 heads, SSSL stack of 4 layers.
    Workload("andrea480m_sssl", B=16, H=24, T=1024, d=64, dtype="bf16", pattern="SSSL", n_layer=4),
    # Long context: head dim 128, T = 8192, SSSL stack, v ~ U(-1, 1).
    Workload("long_sssl", B=2, H=16, T=8192, d=128, dtype="bf16", pattern="SSSL", n_layer=4,
             v_dist="uniform"),
)

HEADLINE = 2  # index of the ANDREA-120M SSSL stack

# The default model of the autoresearch train.py listing ("Подробный технический разбор
# реализации Autoresearch", habr.com: DEPTH 8, ASPECT_RATIO 64 so d_model 512, HEAD_DIM 128 so 4
# heads, n_kv_head = n_head, MAX_SEQ_LEN 2048, DEVICE_BATCH_SIZE 128, WINDOW_PATTERN "SSSL").
# Its attention runs on q, k, v in the projections' [B][T][H][d] order; make_qkv draws them in
# [B, H, T, d] order like every workload, and callers transpose.
MODEL_DEFAULT = Workload("autoresearch_default", B=128, H=4, T=2048, d=128, dtype="bf16",
                         pattern="SSSL", n_layer=8)
MODEL_DEFAULT_INDEX = len(WORKLOADS)  # make_qkv index (and seed index) of MODEL_DEFAULT
_ALL = WORKLOADS + (MODEL_DEFAULT,)


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return _ALL[name_or_index]
    for w in _ALL:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def seed_for(index: int, layer: int) -> int:
    """Seed of layer ``layer`` of workload ``index`` (42 + 1000 * index + 10 * layer)."""
    return 42 + 1000 * index + 10 * layer


def make_qkv(index: int, layer: int = 0, shape: tuple[int, int, int, int] | None = None):
    """Raw q, k, v on the CPU for one layer of a workload, in the workload's dtype.

    Drawn in fp32 in the order q, k, v from a CPU generator, then rounded to bf16 (round to
    nearest even) for bf16 workloads. ``shape`` overrides (B, H, T, d) for reduced test sizes.
    """
    w = _ALL[index]
    B, H, T, d = shape if shape is not None else (w.B, w.H, w.T, w.d)
    g = torch.Generator(device="cpu").manual_seed(seed_for(index, layer))
    q = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    if w.v_dist == "uniform":
        v = torch.rand((B, H, T, d), generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        v = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def make_random(shape, dtype: torch.dtype, seed: int, dist: str = "normal") -> torch.Tensor:
    """One seeded CPU tensor (fp32 draw, then cast)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    if dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
    return x.to(dtype)
