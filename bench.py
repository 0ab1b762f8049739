#!/usr/bin/env python3
"""Throughput of the attention block (QK-RMSNorm + RoPE + causal / sliding-window attention
forward) on one MI355X.

One step is one pass of the whole path over one batch of synthetic input: for each layer of the
ANDREA-120M SSSL stack (B=16, H=12, T=1024, d=64, bf16; windows 512, 512, 512, 1024),
QK-RMSNorm + RoPE of that layer's raw q and k and the attention forward with that layer's
window, through the library's one-call layer entry point (attn_fwd_qknorm: a k-only
norm + rotation kernel, then the attention kernel that normalises and rotates q as it loads
it). Inputs are resident in HBM before timing starts; every layer has its own buffers. The
two-call path (attn_qknorm_rope on q and k, then attn_fwd) is timed too and reported beside it,
and so is the layer in one launch ("k_in_kernel": attn_fwd_qknorm_ex with k_work NULL, the keys
normalised and rotated inside the attention kernel; d <= 64).

The value is counted the way the metric names it: TFLOP/s of unmasked attention work
(4 d FLOPs per visible (query, key) pair) over the whole step's time, prologue included.
It prints ONE JSON line on stdout.

The JSON line also carries "backward": the same layers' gradients (attn_bwd_ex on the normalised
q, k, then attn_qknorm_rope_bwd_ex), timed with events around each launch; context only.

The "value_gate" object times the same layers with a value embedding (attn_fwd_qknorm_ve_ex:
the k-only prologue launch also gates v) against the plain layer call, and the gate alone.

The line's "cache_states" object times the attention launch alone in two more cache states:
hot (one layer's launch repeated back to back) and cold (a 512 MiB write before each launch).
The "item_order" object times the attention launches in the default item order and in the snake
order (ATTN_ITEM_ORDER=snake), alternating step by step, in-model and cold, and checks that the
outputs are bitwise the same.

--workload autoresearch_default times the train.py listing's default model instead (B=128, H=4,
T=2048, d=128, eight layers "SSSL" with windows 1024 / 2048) on q, k, v in the projections'
[B][T][H][d] order, and prints its own JSON line (metric named after that shape). The other
bf16 configurations (andrea12m, andrea480m_sssl, long_sssl) run the same way in [B][H][T][d].

Extra modes (used to collect rocprofv3 counters; they print no JSON):
  --only attn|kprologue|attn_unfused|prologue|decode|bwd
                         run only that kernel (decode: its two kernels, or one where a
                         single key split per head suffices; bwd: attn_bwd_ex's kernels, after
                         the two-call forward it reads), --steps times per layer
  --copy-calibration     run a plain 256 MiB device copy (known bytes) for counter scaling
  --dma-calibration      run the attention kernel where it reads every byte once (non-causal,
                         T = 128: one query block per head, each K/V tile read by one item), so
                         the counters of its direct-to-LDS loads can be checked against known bytes
  --issue-rates          run the issue-rate probe (libattn_diag.so, diag/issue_rates.hip): cycles
                         per loop of independent MFMAs, exponentials, FMAs, packs, dot products
                         and adds, alone and interleaved in one wave, with one and two waves per
                         SIMD; prints a table
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
METRIC = "bf16 causal/SWA attention fwd TFLOP/s + % MFMA peak, T=1024 H=12 d=64"
HEADLINE = "andrea120m_sssl"
# The attention kernel's source: its own file and the headers it includes, hashed in this order.
ATTN_SOURCES = [os.path.join(ROOT, "transformer_attention_qk_amd", "csrc", f)
                for f in ("attn_fwd_bf16.hip", "common.hpp", "launch.hpp", "fastdiv.hpp",
                          "tile_ops.hpp")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_fwd_bf16_andrea120m_sssl_traffic.md")


def visible_pairs(T: int, window: int, causal: bool = True) -> int:
    """Number of (query, key) pairs the mask keeps in one head (closed form)."""
    if not causal:
        return T * T
    if window < 0 or window >= T - 1:
        return T * (T + 1) // 2
    W = window
    return W * (W + 1) // 2 + (T - W) * (W + 1)


def attn_flops(B: int, H: int, T: int, d: int, window: int) -> int:
    """Unmasked attention FLOPs of one layer: 2 d for q.k plus 2 d for p v per visible pair."""
    return 4 * d * visible_pairs(T, window) * B * H


def attn_compulsory_bytes(B: int, H: int, T: int, d: int, elem: int = 2) -> int:
    """HBM bytes one attention launch must move: q, k, v read, out written, fp32 lse written."""
    return B * H * T * (4 * d * elem + 4)


def prologue_bytes(B: int, H: int, T: int, d: int, elem: int = 2, tensors: int = 2) -> int:
    """HBM bytes of one prologue launch: each of `tensors` (q and k, or k alone) read and
    written once (the RoPE table is cached)."""
    return B * H * T * 2 * tensors * d * elem


def source_sha(paths: list[str]) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counter(key: str = "traffic_bytes_per_launch") -> float | None:
    """A figure of the committed rocprofv3 counter summary of the attention kernel (HBM bytes per
    launch, or the MFMA busy fraction), if the summary was taken on the current kernel source;
    else None."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(re.escape(key) + r":\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != source_sha(ATTN_SOURCES):
        return None
    return float(val.group(1))


def measured_traffic() -> float | None:
    return measured_counter("traffic_bytes_per_launch")


# What the pages report about the hardware they ran on (context only; none of them gives an
# attention throughput figure).
PAGES_CONTEXT = {
    "attention_throughput_on_pages": None,
    "autoresearch_hardware": "H100 (the train.py listing's experiments; its MFU uses a 989.5 "
                             "TFLOP/s bf16 peak and reports 39.8 % for the whole model's training)",
    "andrea_hardware": "RTX 4090, or an RTX 3060 (the ANDREA family's training)",
    "note": "another machine's whole-model figures, not an attention-kernel target; vs_baseline "
            "stays null",
}


# Inputs of the CPU-baseline workers, set in the parent before the pool forks (so the workers
# inherit them instead of receiving pickled copies): per layer (q, k, v) fp64 [B, H, T, d], the
# windows and the head count per batch.
_CPU_WORK = None


def _cpu_head(bh: int) -> tuple[int, float]:
    """One (batch, head) of every layer through the fp64 oracle, single-threaded BLAS; returns
    (unmasked FLOPs, CPU seconds)."""
    from threadpoolctl import threadpool_limits

    import oracle

    layers, windows, H, T, d = _CPU_WORK
    b, h = divmod(bh, H)
    t0 = time.process_time()
    with threadpool_limits(1):
        for (q, k, v), W in zip(layers, windows):
            oracle.attention_layer(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                   window=W)
    return sum(attn_flops(1, 1, T, d, W) for W in windows), time.process_time() - t0


def cpu_baseline(w, layer_inputs, windows: list[int], workers: int) -> dict:
    """The fp64 oracle on the same workload: a process pool over the (batch, head) pairs, one
    BLAS thread per worker, every head of every layer. Returns TFLOP/s on the same
    unmasked-FLOP numerator as the GPU over the pool's wall time. Must run before the process
    touches the GPU (the pool forks). layer_inputs: each layer's CPU q, k, v [B, H, T, d]."""
    import multiprocessing

    global _CPU_WORK
    _CPU_WORK = ([tuple(x.to(dtype=__import__("torch").float64).numpy() for x in li)
                  for li in layer_inputs], windows, w.H, w.T, w.d)
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        parts = pool.map(_cpu_head, range(w.B * w.H), chunksize=1)
    elapsed = time.perf_counter() - t0
    _CPU_WORK = None
    flops = sum(f for f, _ in parts)
    cpu_s = sum(c for _, c in parts)
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"all {w.B * w.H} heads of all {len(windows)} layers of {w.name} (fp64 QK-norm "
                   f"+ RoPE + attention), a pool of {workers} processes with one BLAS thread "
                   f"each over (batch, head) pairs: {elapsed:.2f} s wall, {cpu_s:.1f} s of CPU; "
                   f"host affinity {len(os.sched_getaffinity(0))} cores"),
        "seconds": elapsed,
        "cpu_seconds": cpu_s,
    }


def issue_rates() -> int:
    """Print the issue-rate probe's table (cycles per loop iteration, max over the waves)."""
    import ctypes
    from transformer_attention_qk_amd import build as _build
    if not os.path.exists(_build.DIAG_PATH):
        print(f"{_build.DIAG_PATH} is missing: build it with __graft_entry__.build()", file=sys.stderr)
        return 1
    lib = ctypes.CDLL(_build.DIAG_PATH)
    lib.attn_diag_issue_name.restype = ctypes.c_char_p
    lib.attn_diag_issue_name.argtypes = [ctypes.c_int]
    lib.attn_diag_issue_rates.restype = ctypes.c_int
    lib.attn_diag_issue_rates.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    names = []
    while lib.attn_diag_issue_name(len(names)) is not None:
        names.append(lib.attn_diag_issue_name(len(names)).decode())
    cyc = (ctypes.c_double * (2 * len(names)))()
    rc = lib.attn_diag_issue_rates(cyc, 2 * len(names))
    if rc != 0:
        print(f"attn_diag_issue_rates failed with HIP error {rc}", file=sys.stderr)
        return 1
    print("| loop body (independent instructions) | 1 wave per SIMD | 2 waves per SIMD |")
    print("|---|---|---|")
    for m, name in enumerate(names):
        print(f"| {name} | {cyc[2 * m]:.1f} | {cyc[2 * m + 1]:.1f} |")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; 20 for autoresearch_default)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 20; 3)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward, decode and value-gate timings")
    ap.add_argument("--no-cache-states", action="store_true",
                    help="skip the hot / cold cache-state runs and the two-call path (so a kernel "
                         "trace of the run holds the in-model launches only)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="CPU-baseline processes (default: the host's cores, at most 16)")
    ap.add_argument("--only", default=None,
                    choices=["attn", "kprologue", "attn_unfused", "prologue", "decode", "bwd"])
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--dma-calibration", action="store_true")
    ap.add_argument("--issue-rates", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the attention path runs on a single MI355X and has no "
              "multi-GPU mode (its (batch, head) work items are independent, so a batch shards "
              "across GPUs without communication). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from transformer_attention_qk_amd import _lib, inputs, ops

    # The CPU baseline runs first, before anything touches the GPU, because its process pool
    # forks. Its inputs are the same seeded tensors the GPU step uses.
    cpu_result = None
    if not (args.no_cpu_baseline or args.only or args.copy_calibration or args.dma_calibration
            or args.issue_rates):
        names0 = [x.name for x in inputs.WORKLOADS] + [inputs.MODEL_DEFAULT.name]
        if args.workload in names0:
            import oracle
            i0 = names0.index(args.workload)
            w0 = inputs.workload(i0)
            if w0.dtype == "bf16":
                win0 = oracle.sssl_windows(w0.T, w0.n_layer, w0.pattern)
                workers = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
                cpu_result = cpu_baseline(w0, [inputs.make_qkv(i0, l) for l in range(len(win0))],
                                          win0, workers)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    _lib.load()
    torch.cuda.set_device(0)

    if args.issue_rates:
        return issue_rates()

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps or 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy calibration: {max(1, args.steps or 1)} copies of {n} bytes read + {n} bytes written",
              file=sys.stderr)
        return 0

    if args.dma_calibration:
        # 4096 heads of 128 rows, d = 64, non-causal: each head is one item whose two K/V tiles
        # and Q block the attention kernel loads once, directly into LDS.
        Bc, Hc, Tc, dc = 64, 64, 128, 64
        xs = [inputs.make_random((Bc, Hc, Tc, dc), torch.bfloat16, 90 + i).cuda() for i in range(3)]
        kn_c = torch.empty_like(xs[1])
        oc, lc = torch.empty_like(xs[0]), torch.empty((Bc, Hc, Tc), dtype=torch.float32, device="cuda")
        cos_c, sin_c = ops.rope_table(Tc, dc)
        ops.qknorm_rope(None, xs[1], cos_c, sin_c, k_out=kn_c)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps or 1)):
            ops.attn_fwd_qnorm(xs[0], kn_c, xs[2], cos_c, sin_c, causal=False, out=oc, lse=lc)
        torch.cuda.synchronize()
        rd = 3 * xs[0].numel() * 2 + 2 * cos_c.numel() * 4
        wr = oc.numel() * 2 + lc.numel() * 4
        print(f"dma calibration: {max(1, args.steps or 1)} launches of attn_fwd_bf16_stream<64, "
              f"non-causal>, each reading {rd} bytes and writing {wr} bytes", file=sys.stderr)
        return 0

    names = [w.name for w in inputs.WORKLOADS] + [inputs.MODEL_DEFAULT.name]
    if args.workload not in names:
        print(f"unknown workload {args.workload!r}; one of {names}", file=sys.stderr)
        return 2
    index = names.index(args.workload)
    w = inputs.workload(index)
    if w.dtype != "bf16":
        print("the bench times bf16 workloads", file=sys.stderr)
        return 2
    model_default = index == inputs.MODEL_DEFAULT_INDEX
    if args.steps is None:
        args.steps = 20 if model_default else 200
    if args.warmup is None:
        args.warmup = 3 if model_default else 20
    layout = "bthd" if model_default else "bhtd"  # the listing's projections give [B][T][H][d]
    windows = ops.sssl_windows(w.T, w.n_layer, w.pattern)
    L = len(windows)

    # Inputs resident in HBM, one set of buffers per layer (drawn in [B, H, T, d] order, stored
    # in the layout the workload runs in).
    q, k, v, qn, kn, out, lse = ([] for _ in range(7))
    for l in range(L):
        ql, kl, vl = inputs.make_qkv(index, l)
        for dst, x in ((q, ql), (k, kl), (v, vl)):
            x = x.cuda()
            dst.append((x.transpose(1, 2) if layout == "bthd" else x).contiguous())
            del x
        del ql, kl, vl
        qn.append(torch.empty_like(q[-1]))
        kn.append(torch.empty_like(k[-1]))
        out.append(torch.empty_like(q[-1]))
        lse.append(torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda"))
    cos, sin = ops.rope_table(w.T, w.d)
    eps = 1e-6
    torch.cuda.synchronize()

    # The timed calls go straight to the C ABI with pointers taken once, so that the host cost
    # of a call (a few microseconds) stays below the GPU time of the kernels it launches and the
    # per-launch events measure the GPU. The tensor-level binding (ops) is checked against the
    # same calls once, before timing.
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    P = [tuple(t.data_ptr() for t in (q[l], k[l], v[l], qn[l], kn[l], out[l], lse[l]))
         for l in range(L)]
    pcos, psin = cos.data_ptr(), sin.data_ptr()
    B, H, T, d = w.B, w.H, w.T, w.d
    bf16 = _lib.ATTN_BF16
    lay = _lib.ATTN_LAYOUT_BTHD if layout == "bthd" else _lib.ATTN_LAYOUT_BHTD

    # The layer as one call, and its two kernels as separate calls (the same launches).
    def layer(l):
        pq, pk, pv, _, pkn, po, pl = P[l]
        return lib.attn_fwd_qknorm_ex(pq, pk, pv, pkn, po, pl, pcos, psin, B, H, H, T, d, lay,
                                      eps, windows[l], 1, bf16, stream)

    def kprologue(l):
        _, pk, _, _, pkn, _, _ = P[l]
        return lib.attn_qknorm_rope_ex(None, pk, None, pkn, pcos, psin, B, H, H, T, d, lay, eps,
                                       bf16, stream)

    def attention(l):
        pq, _, pv, _, pkn, po, pl = P[l]
        return lib.attn_fwd_qnorm_ex(pq, pkn, pv, po, pl, pcos, psin, B, H, H, T, d, lay, eps,
                                     windows[l], 1, bf16, stream)

    # The two-call path.
    def prologue(l):
        pq, pk, _, pqn, pkn, _, _ = P[l]
        return lib.attn_qknorm_rope_ex(pq, pk, pqn, pkn, pcos, psin, B, H, H, T, d, lay, eps,
                                       bf16, stream)

    def attention_unfused(l):
        _, _, pv, pqn, pkn, po, pl = P[l]
        return lib.attn_fwd_ex(pqn, pkn, pv, po, pl, B, H, H, T, d, lay, windows[l], 1, bf16,
                               stream)

    def make_decode():
        """Decode inputs: each layer's newest normalised query (from qn, so the two-call prologue
        must have run) against its normalised keys and values as a full cache of T tokens."""
        qdec = [qn[l][:, :, -1].contiguous() if layout == "bhtd" else qn[l][:, -1].contiguous()
                for l in range(L)]
        dout_dec = [torch.empty_like(x) for x in qdec]
        dlse_dec = [torch.empty((B, H), dtype=torch.float32, device="cuda") for _ in range(L)]
        wsb = [lib.attn_decode_workspace_bytes(B, H, T, d, windows[l]) for l in range(L)]
        ws_dec = [torch.empty((n // 4 + 4,), dtype=torch.float32, device="cuda") for n in wsb]
        PD = [tuple(t.data_ptr() for t in (qdec[l], dout_dec[l], dlse_dec[l], ws_dec[l]))
              for l in range(L)]

        def decode_step(l):
            _, _, pv, _, pkn, _, _ = P[l]
            pqd, pod, pld, pws = PD[l]
            return lib.attn_decode_ex(pqd, pkn, pv, None, pod, pld, pws, wsb[l], B, H, H, T, d,
                                      lay, windows[l], bf16, stream)
        decode_step.buffers = (qdec, dout_dec, dlse_dec, ws_dec)  # alive while it is
        return decode_step, wsb

    def make_backward():
        """Backward inputs: dout per layer and gradient buffers; runs the two-call forward (q, k
        normalised into qn, kn, then out and lse) whose saved tensors the backward reads."""
        dout, dq, dk, dv, delta = ([] for _ in range(5))
        for l in range(L):
            dout.append(inputs.make_random(tuple(q[l].shape), torch.bfloat16, 900 + l).cuda())
            dq.append(torch.empty_like(q[l]))
            dk.append(torch.empty_like(k[l]))
            dv.append(torch.empty_like(v[l]))
            delta.append(torch.empty_like(lse[l]))
        for l in range(L):
            _lib.check("prologue", prologue(l))
            _lib.check("attn_unfused", attention_unfused(l))
        torch.cuda.synchronize()
        PB = [tuple(t.data_ptr() for t in (dout[l], dq[l], dk[l], dv[l], delta[l]))
              for l in range(L)]

        def attention_bwd(l):
            _, _, pv, pqn, pkn, po, pl = P[l]
            pdo, pdq, pdk, pdv, pdl = PB[l]
            return lib.attn_bwd_ex(pqn, pkn, pv, po, pdo, pl, pdl, pdq, pdk, pdv, B, H, H, T, d,
                                   lay, windows[l], 1, bf16, stream)

        def prologue_bwd(l):
            pq, pk, _, _, _, _, _ = P[l]
            _, pdq, pdk, _, _ = PB[l]
            return lib.attn_qknorm_rope_bwd_ex(pq, pk, pdq, pdk, pdq, pdk, pcos, psin, B, H, H, T,
                                               d, lay, eps, bf16, stream)
        attention_bwd.buffers = (dout, dq, dk, dv, delta)  # alive while it is
        return attention_bwd, prologue_bwd

    if args.only:
        # inputs of the chosen kernel only, so a counter run sees no other kernel of its kind
        setup = {"attn": kprologue, "attn_unfused": prologue, "decode": prologue}.get(args.only)
        if setup is not None:
            for l in range(L):
                setup(l)
        torch.cuda.synchronize()
        fn = {"attn": attention, "kprologue": kprologue, "attn_unfused": attention_unfused,
              "prologue": prologue,
              "decode": make_decode()[0] if args.only == "decode" else None,
              "bwd": make_backward()[0] if args.only == "bwd" else None}[args.only]
        for _ in range(args.steps):
            for l in range(L):
                _lib.check(args.only, fn(l))
        torch.cuda.synchronize()
        print(f"ran {args.only} x {args.steps * L}", file=sys.stderr)
        return 0

    for l in range(L):
        for fn in (layer, kprologue, attention, prologue, attention_unfused):
            _lib.check(fn.__name__, fn(l))
    # The binding gives the same bits as the direct call.
    layer(0)
    ref_out = out[0].clone()
    ops.attn_fwd_qknorm(q[0], k[0], v[0], cos, sin, window=windows[0], eps=eps, k_work=kn[0],
                        out=out[0], lse=lse[0], layout=layout)
    torch.cuda.synchronize()
    if not torch.equal(ref_out, out[0]):
        print("bench: binding and direct call disagree", file=sys.stderr)
        return 1

    def step():
        for l in range(L):
            layer(l)

    def step_unfused():
        for l in range(L):
            prologue(l)
            attention_unfused(l)

    def time_steps(fn) -> float:
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def time_launches(first, second) -> tuple[list[float], list[float]]:
        """Per-layer average ms of two back-to-back launches, HIP events around each (the
        kernels run on torch's current stream, where the events are recorded)."""
        ev = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(L)]
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s_ in range(args.steps):
            for l in range(L):
                a_, b_, c_ = ev[s_][l]
                a_.record()
                first(l)
                b_.record()
                second(l)
                c_.record()
        torch.cuda.synchronize()
        t1, t2 = [0.0] * L, [0.0] * L
        for s_ in range(args.steps):
            for l in range(L):
                a_, b_, c_ = ev[s_][l]
                t1[l] += a_.elapsed_time(b_) / args.steps
                t2[l] += b_.elapsed_time(c_) / args.steps
        return t1, t2

    def time_alone(l, before=None) -> float:
        """Average ms of the attention launch of layer l repeated back to back, events around
        each launch; before() runs ahead of each launch, outside the events."""
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a_, b_ in ev:
            if before is not None:
                before()
            a_.record()
            attention(l)
            b_.record()
        torch.cuda.synchronize()
        return sum(a_.elapsed_time(b_) for a_, b_ in ev) / args.steps

    # Timed region 1: whole steps, nothing between the kernels (the value).
    ms_per_step = time_steps(step)
    # Timed region 2: the same launches with events around each kernel (the roofline).
    kpro_ms, attn_ms = time_launches(kprologue, attention)
    # Cache states of the attention launch: "hot" repeats one layer's launch back to back (its
    # inputs stay in the caches); "cold" writes a 512 MiB buffer (twice the Infinity Cache)
    # before each launch. The in-model order above (k just written by the prologue) is the
    # headline state.
    hot_ms = cold_ms = None
    order_cmp = None
    if not args.no_cache_states:
        hot_ms = [time_alone(l) for l in range(L)]
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold_ms = [time_alone(l, lambda: flush.fill_(1)) for l in range(L)]
        # The default item order against the snake order (ATTN_ITEM_ORDER=snake, read by the
        # library at each call): outputs must match bitwise; then the two alternate step by step
        # in one loop (each launch right after its layer's k pass, as in the model; and after a
        # 512 MiB write, cold), so both see the same clocks and caches.
        ref = [o.clone() for o in out] + [x.clone() for x in lse]

        def attention_order(l, snake):
            if snake:
                os.environ["ATTN_ITEM_ORDER"] = "snake"
            try:
                return attention(l)
            finally:
                if snake:
                    del os.environ["ATTN_ITEM_ORDER"]

        for l in range(L):
            _lib.check("attention (snake order)", attention_order(l, True))
        torch.cuda.synchronize()
        same = all(torch.equal(a_, b_) for a_, b_ in zip(ref, list(out) + list(lse)))

        def time_orders(before) -> list[list[float]]:
            evo = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
                    for _ in range(L)] for _ in range(2 * args.steps)]
            torch.cuda.synchronize()
            for s_ in range(2 * args.steps):
                for l in range(L):
                    before(l)
                    a_, b_ = evo[s_][l]
                    a_.record()
                    attention_order(l, s_ % 2 == 1)
                    b_.record()
            torch.cuda.synchronize()
            ms = [[0.0] * L, [0.0] * L]
            for s_ in range(2 * args.steps):
                for l in range(L):
                    a_, b_ = evo[s_][l]
                    ms[s_ % 2][l] += a_.elapsed_time(b_) / args.steps
            return ms

        order_model = time_orders(kprologue)
        order_cold = time_orders(lambda l: flush.fill_(1))
        order_cmp = (same, order_model, order_cold)
        del flush, ref
    # A plain device copy of the k-only prologue's bytes (one k tensor read, one written), the
    # rate an HBM-bound read-and-write pass reaches on this part, beside the prologue's.
    copy_src = k[0].clone()
    copy_dst = torch.empty_like(copy_src)
    copy_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for _ in range(3):
        copy_dst.copy_(copy_src)
    torch.cuda.synchronize()
    for a_, b_ in copy_ev:
        a_.record()
        copy_dst.copy_(copy_src)
        b_.record()
    torch.cuda.synchronize()
    copy_ms = sum(a_.elapsed_time(b_) for a_, b_ in copy_ev) / args.steps
    del copy_src, copy_dst
    def nothing_step(l):
        return 0

    # The two-call path, and the layer in one launch with the keys normalised in the attention
    # kernel (attn_fwd_qknorm_ex with k_work NULL, d <= 64), for comparison.
    kin_ms = None
    if not args.no_cache_states:
        ms_per_step_unfused = time_steps(step_unfused)
        pro_ms, attn_unf_ms = time_launches(prologue, attention_unfused)
        if d <= 64:
            def layer_kin(l):
                pq, pk, pv, _, _, po, pl = P[l]
                return lib.attn_fwd_qknorm_ex(pq, pk, pv, None, po, pl, pcos, psin, B, H, H, T, d,
                                              lay, eps, windows[l], 1, bf16, stream)

            for l in range(L):
                _lib.check("layer_kin", layer_kin(l))

            def step_kin():
                for l in range(L):
                    layer_kin(l)

            ms_per_step_kin = time_steps(step_kin)
            kin_ms, _ = time_launches(layer_kin, nothing_step)

    # Decode (context): one generation step against each layer's keys and values as the cache.
    dec_ms = None
    if not args.no_backward:
        decode_step, _ = make_decode()

        def nothing(l):
            return 0

        for l in range(L):
            _lib.check("decode", decode_step(l))
        dec_ms, _ = time_launches(decode_step, nothing)
        dec_bytes = [B * H * (min(T, W + 1 if W >= 0 else T) * 4 * d + 4 * d) for W in windows]

    # The backward pass (context, not the value): per layer, the gradient of sum(dout * out)
    # through attn_bwd_ex on the normalised q, k the two-call path wrote (kernels: dQ, which also
    # forms delta, then dK/dV), then the prologue's backward attn_qknorm_rope_bwd_ex in place.
    bwd_ms = None
    if not args.no_backward:
        attention_bwd, prologue_bwd = make_backward()
        for l in range(L):
            _lib.check("attn_bwd", attention_bwd(l))
            _lib.check("prologue_bwd", prologue_bwd(l))
        bwd_ms, pro_bwd_ms = time_launches(attention_bwd, prologue_bwd)

    # The value-embedding gate (context): each layer as a layer with a value embedding
    # (attn_fwd_qknorm_ve_ex: the k-only prologue launch also writes the gated v, then the
    # attention), against the same layer without one, and the gate alone (attn_value_gate_ex).
    vg_ms = None
    if not args.no_backward:
        zshape = (B, T, H) if layout == "bthd" else (B, H, T)
        ve_l = [inputs.make_random(tuple(v[l].shape), torch.bfloat16, 950 + l).cuda()
                for l in range(L)]
        z_l = [inputs.make_random(zshape, torch.bfloat16, 960 + l).cuda() for l in range(L)]
        vw_l = [torch.empty_like(v[l]) for l in range(L)]
        PV = [tuple(t.data_ptr() for t in (ve_l[l], z_l[l], vw_l[l])) for l in range(L)]

        def layer_ve(l):
            pq, pk, pv, _, pkn, po, pl = P[l]
            pve, pz, pvw = PV[l]
            return lib.attn_fwd_qknorm_ve_ex(pq, pk, pv, pve, pz, pkn, pvw, po, pl, pcos, psin,
                                             B, H, H, T, d, lay, eps, windows[l], 1, bf16, stream)

        def gate_alone(l):
            _, _, pv, _, _, _, _ = P[l]
            pve, pz, pvw = PV[l]
            return lib.attn_value_gate_ex(pv, pve, pz, pvw, B, H, T, d, lay, bf16, stream)

        for l in range(L):
            _lib.check("layer_ve", layer_ve(l))
            _lib.check("gate_alone", gate_alone(l))
        lve_ms, lplain_ms = time_launches(layer_ve, layer)
        vg_ms, _ = time_launches(gate_alone, nothing_step)
        gate_bytes = B * H * T * (3 * d * 2 + 2)  # v, ve read, v_work written, logits read

    flops_layer = [attn_flops(w.B, w.H, w.T, w.d, W) for W in windows]
    step_flops = sum(flops_layer)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    attn_total_ms = sum(attn_ms)
    achieved = step_flops / (attn_total_ms * 1e-3) / 1e12
    attn_bytes = attn_compulsory_bytes(w.B, w.H, w.T, w.d)
    kpro_bytes = prologue_bytes(w.B, w.H, w.T, w.d, tensors=1)
    pro_bytes = prologue_bytes(w.B, w.H, w.T, w.d, tensors=2)
    # the committed counter summary covers the headline workload only
    traffic = measured_traffic() if w.name == HEADLINE else None
    mfma_busy = measured_counter("mfma_busy") if w.name == HEADLINE else None
    kernel = (f"attn_fwd_bf16_stream<{w.d}, mode, qkn=true>" if w.d <= 64
              else f"attn_fwd_bf16_tile<{w.d}, mode, qkn=true>")

    result = {
        "metric": METRIC if w.name == HEADLINE else (
            "bf16 causal/SWA attention fwd TFLOP/s + % MFMA peak, train.py default model "
            "B=128 H=4 T=2048 d=128 [B,T,H,D]" if model_default else
            f"bf16 causal/SWA attention fwd TFLOP/s + % MFMA peak, {w.name} "
            f"B={w.B} H={w.H} T={w.T} d={w.d}"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "layers": L,
            "windows": windows, "layout": layout,
            "step": "per layer: attn_fwd_qknorm (k-only qknorm_rope kernel + attention kernel "
                    "with in-kernel q norm and rotation)",
            "flops_per_step": step_flops,
        },
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "context": PAGES_CONTEXT,
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else int(traffic),
            "mfma_busy": mfma_busy,
            "avg_launch_us": round(1e3 * attn_total_ms / L, 3),
            "launch_us": [round(1e3 * t, 3) for t in attn_ms],
            "flops_per_launch": flops_layer,
            "compulsory_bytes_per_launch": attn_bytes,
            "compulsory_hbm_gbs": round(attn_bytes * L / (attn_total_ms * 1e-3) / 1e9, 1),
        },
        "k_prologue": {
            "avg_launch_us": round(1e3 * sum(kpro_ms) / L, 3),
            "bytes_per_launch": kpro_bytes,
            "achieved_gbs": round(kpro_bytes * L / (sum(kpro_ms) * 1e-3) / 1e9, 1),
            "peak_gbs": PEAK_HBM_GBS,
            "copy_same_bytes_us": round(1e3 * copy_ms, 3),
            "copy_gbs": round(kpro_bytes / (copy_ms * 1e-3) / 1e9, 1),
        },
    }
    if hot_ms is not None:
        result["cache_states"] = {
            "note": "attention launch alone: hot = one layer's launch repeated back to back; "
                    "cold = a 512 MiB write before each launch; headline = roofline.launch_us "
                    "(in-model order, k just written by the prologue)",
            "hot_launch_us": [round(1e3 * t, 3) for t in hot_ms],
            "hot_tflops": round(step_flops / (sum(hot_ms) * 1e-3) / 1e12, 3),
            "cold_launch_us": [round(1e3 * t, 3) for t in cold_ms],
            "cold_tflops": round(step_flops / (sum(cold_ms) * 1e-3) / 1e12, 3),
        }
        result["two_call_path"] = {
            "ms_per_step": round(ms_per_step_unfused, 5),
            "value": round(step_flops / (ms_per_step_unfused * 1e-3) / 1e12, 3),
            "attn_avg_launch_us": round(1e3 * sum(attn_unf_ms) / L, 3),
            "attn_tflops": round(step_flops / (sum(attn_unf_ms) * 1e-3) / 1e12, 3),
            "prologue_avg_launch_us": round(1e3 * sum(pro_ms) / L, 3),
            "prologue_bytes_per_launch": pro_bytes,
            "prologue_gbs": round(pro_bytes * L / (sum(pro_ms) * 1e-3) / 1e9, 1),
        }
    if order_cmp is not None:
        same, (m_def, m_snk), (c_def, c_snk) = order_cmp
        tf = lambda ms: round(step_flops / (sum(ms) * 1e-3) / 1e12, 3)  # noqa: E731
        result["item_order"] = {
            "note": "the attention launches in the library's item order (head-grouped where the "
                    "heads divide into whole rounds) and in the snake order "
                    "(ATTN_ITEM_ORDER=snake), alternating step by step: in-model (after the "
                    "layer's k pass) and cold (after a 512 MiB write)",
            "outputs_equal": bool(same),
            "default_tflops": tf(m_def),
            "snake_tflops": tf(m_snk),
            "default_launch_us": [round(1e3 * t, 3) for t in m_def],
            "snake_launch_us": [round(1e3 * t, 3) for t in m_snk],
            "default_cold_tflops": tf(c_def),
            "snake_cold_tflops": tf(c_snk),
        }
    if kin_ms is not None:
        result["k_in_kernel"] = {
            "note": "the layer in one launch: attn_fwd_qknorm_ex with k_work NULL normalises and "
                    "rotates each key tile inside the attention kernel (no k pass, no normalised "
                    "k written); the step value uses the two-launch layer (the default, which "
                    "also returns the normalised k)",
            "ms_per_step": round(ms_per_step_kin, 5),
            "value": round(step_flops / (ms_per_step_kin * 1e-3) / 1e12, 3),
            "avg_launch_us": round(1e3 * sum(kin_ms) / L, 3),
            "launch_us": [round(1e3 * t, 3) for t in kin_ms],
        }
    if dec_ms is not None:
        result["decode"] = {
            "note": "one generation step per layer: the newest token of each (batch, head) "
                    "against the layer's normalised keys and values as a full cache of T tokens "
                    "(attn_decode_ex); HBM-bound, bytes = cache rows read + q + out",
            "avg_launch_us": round(1e3 * sum(dec_ms) / L, 3),
            "launch_us": [round(1e3 * t, 3) for t in dec_ms],
            "bytes_per_launch": dec_bytes,
            "achieved_gbs": round(sum(dec_bytes) / (sum(dec_ms) * 1e-3) / 1e9, 1),
            "peak_gbs": PEAK_HBM_GBS,
        }
    if bwd_ms is not None:
        result["backward"] = {
            "note": "gradients of the step's layers (context, not the value); TFLOP/s counts 8 d "
                    "per visible pair, twice the forward, as GPT.estimate_flops does",
            "attn_bwd_avg_launch_us": round(1e3 * sum(bwd_ms) / L, 3),
            "attn_bwd_launch_us": [round(1e3 * t, 3) for t in bwd_ms],
            "attn_bwd_tflops": round(2 * step_flops / (sum(bwd_ms) * 1e-3) / 1e12, 3),
            "prologue_bwd_avg_launch_us": round(1e3 * sum(pro_bwd_ms) / L, 3),
            "prologue_bwd_gbs": round(3 * pro_bytes / 2 * L / (sum(pro_bwd_ms) * 1e-3) / 1e9, 1),
        }
    if vg_ms is not None:
        added = (sum(lve_ms) - sum(lplain_ms)) / L
        result["value_gate"] = {
            "note": "layers with a value embedding (context): attn_fwd_qknorm_ve_ex, whose k-only "
                    "prologue launch also gates v, against attn_fwd_qknorm_ex; and the gate alone "
                    "(attn_value_gate_ex); gate bytes = v, ve read + v_work written + logits",
            "layer_ve_avg_us": round(1e3 * sum(lve_ms) / L, 3),
            "layer_avg_us": round(1e3 * sum(lplain_ms) / L, 3),
            "gate_added_us": round(1e3 * added, 3),
            "gate_bytes_per_layer": gate_bytes,
            "gate_added_gbs": round(gate_bytes / (added * 1e-3) / 1e9, 1) if added > 0 else None,
            "gate_alone_avg_us": round(1e3 * sum(vg_ms) / L, 3),
            "gate_alone_gbs": round(gate_bytes * L / (sum(vg_ms) * 1e-3) / 1e9, 1),
        }
    if cpu_result is not None:
        result["cpu_baseline"] = cpu_result
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
