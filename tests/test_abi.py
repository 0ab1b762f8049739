"""The C ABI on the CPU: libattn.so loads, exports every entry point include/attn.h declares,
and rejects invalid arguments before making any HIP call. No kernel runs here."""

import ctypes
import os
import re

import pytest

import oracle
from transformer_attention_qk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:\w+\s+)*\w+\s*\*?\s*(attn_\w+)\s*\(", src,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_qnorm", "attn_fwd_qknorm", "attn_qknorm_rope",
            "attn_rope_table", "attn_strerror", "attn_sssl_windows", "attn_version",
            "attn_fwd_ex", "attn_bwd", "attn_bwd_ex", "attn_qknorm_rope_bwd", "attn_decode",
            "attn_decode_ex", "attn_decode_workspace_bytes", "attn_value_gate_ex",
            "attn_fwd_qknorm_ve_ex", "attn_value_gate_bwd_ex",
            "attn_decode_noalloc_ex"} <= set(names)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"


def test_strerror_is_total(lib):
    for code in range(-3, 15):
        s = lib.attn_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.attn_strerror(0) == b"ok"
    assert lib.attn_version() >= 100


def _windows(lib, T, n, pattern):
    buf = (ctypes.c_int * max(n, 1))()
    rc = lib.attn_sssl_windows(T, n, None if pattern is None else pattern.encode(), buf)
    return rc, list(buf[:n])


@pytest.mark.parametrize("T", [1, 2, 3, 64, 1000, 1024, 1025, 8192])
@pytest.mark.parametrize("n_layer", [1, 2, 3, 4, 5, 8, 12])
@pytest.mark.parametrize("pattern", ["SSSL", "L", "S", "sl", "SLS", "LLLS"])
def test_sssl_windows_match_oracle(lib, T, n_layer, pattern):
    rc, w = _windows(lib, T, n_layer, pattern)
    assert rc == _lib.ATTN_OK
    assert w == oracle.sssl_windows(T, n_layer, pattern)


def test_sssl_windows_errors(lib):
    buf = (ctypes.c_int * 4)()
    assert lib.attn_sssl_windows(1024, 4, None, buf) == _lib.ATTN_ERR_NULL
    assert lib.attn_sssl_windows(1024, 4, b"SSSL", None) == _lib.ATTN_ERR_NULL
    assert lib.attn_sssl_windows(1024, 4, b"", buf) == _lib.ATTN_ERR_ARG
    assert lib.attn_sssl_windows(1024, 4, b"SSXL", buf) == _lib.ATTN_ERR_ARG
    assert lib.attn_sssl_windows(1024, 0, b"SSSL", buf) == _lib.ATTN_ERR_ARG
    assert lib.attn_sssl_windows(0, 4, b"SSSL", buf) == _lib.ATTN_ERR_SHAPE


# ---------------------------------------------------------------------------------------------
# Validation. The pointers below are fake (never dereferenced): each case breaks exactly one
# rule, and the library must reject it before any HIP call. Where a GPU is present these cases
# are skipped (a validation bug would then launch a kernel on fake pointers); the GPU tier
# repeats them with real buffers.
# ---------------------------------------------------------------------------------------------

no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="fake-pointer validation cases only run where no GPU is present")

P = 1 << 20  # 16-byte aligned fake addresses, far apart
A, Bp, Cp, Dp, Ep, Fp, Gp, Hp = (P * i for i in range(1, 9))


def fwd_args(**kw):
    a = dict(q=A, k=Bp, v=Cp, out=Dp, lse=Ep, B=1, H=2, T=64, d=64, window=-1, causal=1,
             dtype=_lib.ATTN_BF16, stream=None)
    a.update(kw)
    return a


FWD_CASES = [
    ("null q", dict(q=None), _lib.ATTN_ERR_NULL),
    ("null out", dict(out=None), _lib.ATTN_ERR_NULL),
    ("B=0", dict(B=0), _lib.ATTN_ERR_SHAPE),
    ("H=-1", dict(H=-1), _lib.ATTN_ERR_SHAPE),
    ("T=0", dict(T=0), _lib.ATTN_ERR_SHAPE),
    ("bf16 d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("bf16 d=48", dict(d=48), _lib.ATTN_ERR_HEAD_DIM),
    ("f32 d=8", dict(d=8, dtype=_lib.ATTN_F32), _lib.ATTN_ERR_HEAD_DIM),
    ("f32 d=256", dict(d=256, dtype=_lib.ATTN_F32), _lib.ATTN_ERR_HEAD_DIM),
    ("dtype 7", dict(dtype=7), _lib.ATTN_ERR_DTYPE),
    ("causal 2", dict(causal=2), _lib.ATTN_ERR_WINDOW),
    ("window -2", dict(window=-2), _lib.ATTN_ERR_WINDOW),
    ("noncausal window", dict(causal=0, window=5), _lib.ATTN_ERR_WINDOW),
    ("misaligned q", dict(q=A + 8), _lib.ATTN_ERR_ALIGN),
    ("misaligned out", dict(out=Dp + 2), _lib.ATTN_ERR_ALIGN),
    ("misaligned lse", dict(lse=Ep + 2), _lib.ATTN_ERR_ALIGN),
    ("out overlaps v", dict(out=Cp + 64), _lib.ATTN_ERR_ALIAS),
    ("out is q", dict(out=A), _lib.ATTN_ERR_ALIAS),
    ("lse inside k", dict(lse=Bp + 256), _lib.ATTN_ERR_ALIAS),
    ("grid too large", dict(B=1 << 15, H=1 << 15, T=1 << 10, d=32), _lib.ATTN_ERR_SHAPE),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_attn_fwd_rejects_before_any_hip_call(lib, name, kw, code):
    a = fwd_args(**kw)
    rc = lib.attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["T"], a["d"],
                      a["window"], a["causal"], a["dtype"], a["stream"])
    assert rc == code, (name, rc, lib.attn_strerror(rc))


def qkn_args(**kw):
    a = dict(q=A, k=Bp, qo=Cp, ko=Dp, cos=Ep, sin=Fp, B=1, H=2, T=64, d=64, eps=1e-6,
             dtype=_lib.ATTN_BF16, stream=None)
    a.update(kw)
    return a


QKN_CASES = [
    ("null k", dict(k=None), _lib.ATTN_ERR_NULL),
    ("null sin", dict(sin=None), _lib.ATTN_ERR_NULL),
    ("T=0", dict(T=0), _lib.ATTN_ERR_SHAPE),
    ("d=24", dict(d=24), _lib.ATTN_ERR_HEAD_DIM),
    ("d=256", dict(d=256), _lib.ATTN_ERR_HEAD_DIM),
    ("dtype -1", dict(dtype=-1), _lib.ATTN_ERR_DTYPE),
    ("eps < 0", dict(eps=-1.0), _lib.ATTN_ERR_ARG),
    ("eps nan", dict(eps=float("nan")), _lib.ATTN_ERR_ARG),
    ("misaligned cos", dict(cos=Ep + 4), _lib.ATTN_ERR_ALIGN),
    ("q_out overlaps q", dict(qo=A + 16), _lib.ATTN_ERR_ALIAS),
    ("q_out is k", dict(qo=Bp), _lib.ATTN_ERR_ALIAS),
    ("k_out is q_out", dict(ko=Cp), _lib.ATTN_ERR_ALIAS),
    ("q null, q_out given", dict(q=None), _lib.ATTN_ERR_NULL),
    ("q given, q_out null", dict(qo=None), _lib.ATTN_ERR_NULL),
    ("k only, misaligned k_out", dict(q=None, qo=None, ko=Dp + 8), _lib.ATTN_ERR_ALIGN),
    ("k only, k_out overlaps k", dict(q=None, qo=None, ko=Bp + 32), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", QKN_CASES, ids=[c[0] for c in QKN_CASES])
def test_qknorm_rope_rejects_before_any_hip_call(lib, name, kw, code):
    a = qkn_args(**kw)
    rc = lib.attn_qknorm_rope(a["q"], a["k"], a["qo"], a["ko"], a["cos"], a["sin"], a["B"], a["H"],
                              a["T"], a["d"], a["eps"], a["dtype"], a["stream"])
    assert rc == code, (name, rc, lib.attn_strerror(rc))


ROPE_CASES = [
    ("null cos", dict(cos=None), _lib.ATTN_ERR_NULL),
    ("T=0", dict(T=0), _lib.ATTN_ERR_SHAPE),
    ("odd d", dict(d=63), _lib.ATTN_ERR_HEAD_DIM),
    ("d=0", dict(d=0), _lib.ATTN_ERR_HEAD_DIM),
    ("base 1", dict(base=1.0), _lib.ATTN_ERR_ARG),
    ("base inf", dict(base=float("inf")), _lib.ATTN_ERR_ARG),
    ("misaligned sin", dict(sin=Bp + 4), _lib.ATTN_ERR_ALIGN),
    ("sin overlaps cos", dict(sin=A + 16), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope_table_rejects_before_any_hip_call(lib, name, kw, code):
    a = dict(cos=A, sin=Bp, T=64, d=64, base=10000.0, stream=None)
    a.update(kw)
    rc = lib.attn_rope_table(a["cos"], a["sin"], a["T"], a["d"], a["base"], a["stream"])
    assert rc == code, (name, rc, lib.attn_strerror(rc))


def fused_args(**kw):
    a = dict(q=A, k=Bp, v=Cp, kw=Dp, out=Ep, lse=Fp, cos=Gp, sin=Hp, B=1, H=2, T=64, d=64,
             eps=1e-6, window=-1, causal=1, dtype=_lib.ATTN_BF16, stream=None)
    a.update(kw)
    return a


FUSED_CASES = [
    ("null q", dict(q=None), _lib.ATTN_ERR_NULL),
    # k_work NULL: the keys are normalised in the attention kernel (d <= 64 only)
    ("null k_work at d=128", dict(kw=None, d=128), _lib.ATTN_ERR_NULL),
    ("null k_work at d=64 reaches the eps rule", dict(kw=None, eps=-1.0), _lib.ATTN_ERR_ARG),
    ("null k_work at d=32 reaches the alias rule", dict(kw=None, d=32, out=Bp),
     _lib.ATTN_ERR_ALIAS),
    ("null cos", dict(cos=None), _lib.ATTN_ERR_NULL),
    ("f32", dict(dtype=_lib.ATTN_F32), _lib.ATTN_ERR_DTYPE),
    ("dtype 3", dict(dtype=3), _lib.ATTN_ERR_DTYPE),
    ("d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("d=96", dict(d=96), _lib.ATTN_ERR_HEAD_DIM),
    ("B=0", dict(B=0), _lib.ATTN_ERR_SHAPE),
    ("T=-5", dict(T=-5), _lib.ATTN_ERR_SHAPE),
    ("causal 3", dict(causal=3), _lib.ATTN_ERR_WINDOW),
    ("noncausal window", dict(causal=0, window=0), _lib.ATTN_ERR_WINDOW),
    ("eps < 0", dict(eps=-1e-3), _lib.ATTN_ERR_ARG),
    ("eps inf", dict(eps=float("inf")), _lib.ATTN_ERR_ARG),
    ("misaligned v", dict(v=Cp + 8), _lib.ATTN_ERR_ALIGN),
    ("misaligned k_work", dict(kw=Dp + 2), _lib.ATTN_ERR_ALIGN),
    ("misaligned sin", dict(sin=Hp + 4), _lib.ATTN_ERR_ALIGN),
    ("misaligned lse", dict(lse=Fp + 1), _lib.ATTN_ERR_ALIGN),
    ("k_work inside k", dict(kw=Bp + 128), _lib.ATTN_ERR_ALIAS),
    ("k_work is q", dict(kw=A), _lib.ATTN_ERR_ALIAS),
    ("k_work is v", dict(kw=Cp), _lib.ATTN_ERR_ALIAS),
    ("out is k_work", dict(out=Dp), _lib.ATTN_ERR_ALIAS),
    ("out is k", dict(out=Bp), _lib.ATTN_ERR_ALIAS),
    ("lse inside k_work", dict(lse=Dp + 64), _lib.ATTN_ERR_ALIAS),
    ("lse inside out", dict(lse=Ep + 64), _lib.ATTN_ERR_ALIAS),
    ("grid too large", dict(B=1 << 15, H=1 << 15, T=1 << 10, d=32), _lib.ATTN_ERR_SHAPE),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_attn_fwd_qknorm_rejects_before_any_hip_call(lib, name, kw, code):
    a = fused_args(**kw)
    rc = lib.attn_fwd_qknorm(a["q"], a["k"], a["v"], a["kw"], a["out"], a["lse"], a["cos"],
                             a["sin"], a["B"], a["H"], a["T"], a["d"], a["eps"], a["window"],
                             a["causal"], a["dtype"], a["stream"])
    assert rc == code, (name, rc, lib.attn_strerror(rc))


QNORM_CASES = [
    ("null k", dict(k=None), _lib.ATTN_ERR_NULL),
    ("null sin", dict(sin=None), _lib.ATTN_ERR_NULL),
    ("f32", dict(dtype=_lib.ATTN_F32), _lib.ATTN_ERR_DTYPE),
    ("d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("H=0", dict(H=0), _lib.ATTN_ERR_SHAPE),
    ("window -3", dict(window=-3), _lib.ATTN_ERR_WINDOW),
    ("eps nan", dict(eps=float("nan")), _lib.ATTN_ERR_ARG),
    ("misaligned q", dict(q=A + 4), _lib.ATTN_ERR_ALIGN),
    ("misaligned cos", dict(cos=Gp + 8), _lib.ATTN_ERR_ALIGN),
    ("out is q", dict(out=A), _lib.ATTN_ERR_ALIAS),
    ("out inside v", dict(out=Cp + 4096), _lib.ATTN_ERR_ALIAS),
    ("lse inside q", dict(lse=A + 16), _lib.ATTN_ERR_ALIAS),
    ("slab too large", dict(B=1, H=1, T=1 << 23, d=128, **{n: (i + 1) << 40 for i, n in enumerate(
        ("q", "k", "v", "out", "lse", "cos", "sin"))}), _lib.ATTN_ERR_SHAPE),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", QNORM_CASES, ids=[c[0] for c in QNORM_CASES])
def test_attn_fwd_qnorm_rejects_before_any_hip_call(lib, name, kw, code):
    a = fused_args(**kw)
    rc = lib.attn_fwd_qnorm(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cos"], a["sin"],
                            a["B"], a["H"], a["T"], a["d"], a["eps"], a["window"], a["causal"],
                            a["dtype"], a["stream"])
    assert rc == code, (name, rc, lib.attn_strerror(rc))


# ---------------------------------------------------------------------------------------------
# The _ex entry points (grouped-query heads, [B][T][H][d] storage). Every case of the lists above
# must give the same status through the _ex variant with H_kv = H and the [B][H][T][d] layout,
# and the new arguments have rules of their own.
# ---------------------------------------------------------------------------------------------

def _fwd_ex(lib, a):
    return lib.attn_fwd_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"],
                           a.get("H_kv", a["H"]), a["T"], a["d"], a.get("layout", 0), a["window"],
                           a["causal"], a["dtype"], a["stream"])


def _qkn_ex(lib, a):
    return lib.attn_qknorm_rope_ex(a["q"], a["k"], a["qo"], a["ko"], a["cos"], a["sin"], a["B"],
                                   a["H"], a.get("H_kv", a["H"]), a["T"], a["d"],
                                   a.get("layout", 0), a["eps"], a["dtype"], a["stream"])


def _qnorm_ex(lib, a):
    return lib.attn_fwd_qnorm_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cos"], a["sin"],
                                 a["B"], a["H"], a.get("H_kv", a["H"]), a["T"], a["d"],
                                 a.get("layout", 0), a["eps"], a["window"], a["causal"],
                                 a["dtype"], a["stream"])


def _fused_ex(lib, a):
    return lib.attn_fwd_qknorm_ex(a["q"], a["k"], a["v"], a["kw"], a["out"], a["lse"], a["cos"],
                                  a["sin"], a["B"], a["H"], a.get("H_kv", a["H"]), a["T"],
                                  a["d"], a.get("layout", 0), a["eps"], a["window"], a["causal"],
                                  a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("name,kw,code", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_attn_fwd_ex_matches_attn_fwd_on_every_case(lib, name, kw, code):
    assert _fwd_ex(lib, fwd_args(**kw)) == code


@no_gpu
@pytest.mark.parametrize("name,kw,code", QKN_CASES, ids=[c[0] for c in QKN_CASES])
def test_qknorm_rope_ex_matches_qknorm_rope_on_every_case(lib, name, kw, code):
    assert _qkn_ex(lib, qkn_args(**kw)) == code


@no_gpu
@pytest.mark.parametrize("name,kw,code", QNORM_CASES, ids=[c[0] for c in QNORM_CASES])
def test_attn_fwd_qnorm_ex_matches_attn_fwd_qnorm_on_every_case(lib, name, kw, code):
    assert _qnorm_ex(lib, fused_args(**kw)) == code


@no_gpu
@pytest.mark.parametrize("name,kw,code", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_attn_fwd_qknorm_ex_matches_attn_fwd_qknorm_on_every_case(lib, name, kw, code):
    assert _fused_ex(lib, fused_args(**kw)) == code


# Far-apart fake pointers for the cases whose tensors are GiBs long.
_FAR = {n: (i + 1) << 40 for i, n in enumerate(("q", "k", "v", "out", "lse", "cos", "sin"))}
_FAR_KV = 1 << 29  # k's bytes for B=1, H_kv=2, T=2^20, d=128 bf16

EX_RULES = [
    ("H_kv=0", dict(H=4, H_kv=0), _lib.ATTN_ERR_SHAPE),
    ("H_kv=-2", dict(H=4, H_kv=-2), _lib.ATTN_ERR_SHAPE),
    ("H_kv does not divide H", dict(H=4, H_kv=3), _lib.ATTN_ERR_SHAPE),
    ("H_kv > H", dict(H=2, H_kv=4), _lib.ATTN_ERR_SHAPE),
    ("layout 2", dict(layout=2), _lib.ATTN_ERR_ARG),
    ("layout -1", dict(layout=-1), _lib.ATTN_ERR_ARG),
    # k has B*H_kv*T*d elements: an out ending inside k's last row aliases it
    ("out inside the end of a GQA k", dict(H=4, H_kv=2, out=Bp + 2 * 64 * 64 * 2 - 16),
     _lib.ATTN_ERR_ALIAS),
    # [B][T][H][d] rows are H*d*2 bytes apart: (T + 128) of them must stay below 2^31 bytes
    ("bthd slab too large", dict(B=1, H=8, H_kv=2, T=1 << 20, d=128, layout=1, **_FAR),
     _lib.ATTN_ERR_SHAPE),
    # with the same sizes, an out placed right after k (whose extent uses H_kv, not H) passes
    # the overlap checks and stops at the slab rule
    ("out right after a GQA k", dict(B=1, H=8, H_kv=2, T=1 << 20, d=128, layout=1,
                                     **dict(_FAR, out=_FAR["k"] + _FAR_KV)), _lib.ATTN_ERR_SHAPE),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", EX_RULES, ids=[c[0] for c in EX_RULES])
def test_attn_fwd_ex_geometry_rules(lib, name, kw, code):
    assert _fwd_ex(lib, fwd_args(**kw)) == code, name


@no_gpu
@pytest.mark.parametrize("name,kw,code", EX_RULES, ids=[c[0] for c in EX_RULES])
def test_attn_fwd_qnorm_ex_geometry_rules(lib, name, kw, code):
    assert _qnorm_ex(lib, fused_args(**kw)) == code, name


@no_gpu
@pytest.mark.parametrize("name,kw,code", EX_RULES[:6], ids=[c[0] for c in EX_RULES[:6]])
def test_qknorm_rope_ex_geometry_rules(lib, name, kw, code):
    assert _qkn_ex(lib, qkn_args(**kw)) == code, name


@no_gpu
@pytest.mark.parametrize("name,kw,code", EX_RULES[:6], ids=[c[0] for c in EX_RULES[:6]])
def test_attn_fwd_qknorm_ex_geometry_rules(lib, name, kw, code):
    assert _fused_ex(lib, fused_args(**kw)) == code, name


@no_gpu
def test_qknorm_rope_ex_k_extent_uses_kv_heads(lib):
    # q has 4 heads, k 1: k's 8 KiB end where k_out starts, so this is no overlap; q_out inside
    # k's extent is one.
    a = qkn_args(H=4, H_kv=1, qo=Bp + 64 * 64 * 2 - 16)
    assert _qkn_ex(lib, a) == _lib.ATTN_ERR_ALIAS
    a = qkn_args(H=4, H_kv=1, ko=Bp + 64 * 64 * 2, eps=-1.0)
    assert _qkn_ex(lib, a) == _lib.ATTN_ERR_ARG  # reached the eps rule: no alias found first


def test_binding_geometry():
    """Host-side shape logic of the Python binding (no tensor reaches the library)."""
    import torch
    from transformer_attention_qk_amd.ops import _geometry
    q = torch.empty(2, 8, 128, 64)
    k = torch.empty(2, 2, 128, 64)
    assert _geometry(q, k, "bhtd") == (2, 8, 2, 128, 64)
    assert _geometry(q.transpose(1, 2), k.transpose(1, 2), "bthd") == (2, 8, 2, 128, 64)
    assert _geometry(None, k, "bhtd") == (2, 2, 2, 128, 64)
    with pytest.raises(ValueError):
        _geometry(q, torch.empty(2, 3, 128, 64), "bhtd")  # 3 does not divide 8
    with pytest.raises(ValueError):
        _geometry(q, torch.empty(2, 2, 64, 64), "bhtd")  # T differs
    with pytest.raises(ValueError):
        _geometry(q, k, "tbhd")
    with pytest.raises(ValueError):
        _geometry(q, k, "bthd")  # read as [B, T, H, d], the shapes disagree


@no_gpu
def test_row_width_limit(lib):
    # H * d must stay below 2^24 elements (the prologue's per-block row offsets are 32-bit)
    a = qkn_args(H=1 << 18, H_kv=1 << 18, T=1, d=64, **{n: (i + 1) << 40 for i, n in enumerate(
        ("q", "k", "qo", "ko", "cos", "sin"))}, eps=-1.0)
    assert _qkn_ex(lib, a) == _lib.ATTN_ERR_SHAPE
    a["H"] = a["H_kv"] = (1 << 18) - 1  # just below: reaches the eps rule
    assert _qkn_ex(lib, a) == _lib.ATTN_ERR_ARG


# ---------------------------------------------------------------------------------------------
# Backward entry points.
# ---------------------------------------------------------------------------------------------

_BW = {n: (i + 1) * P for i, n in enumerate(("q", "k", "v", "out", "do", "lse", "delta", "dq",
                                              "dk", "dv"))}


def _bwd(lib, **kw):
    a = dict(_BW, B=1, H=2, H_kv=2, T=64, d=64, layout=0, window=-1, causal=1,
             dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_bwd_ex(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["delta"],
                           a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["H_kv"], a["T"], a["d"],
                           a["layout"], a["window"], a["causal"], a["dtype"], None)


BWD_CASES = [
    ("null lse", dict(lse=None), _lib.ATTN_ERR_NULL),
    ("null delta", dict(delta=None), _lib.ATTN_ERR_NULL),
    ("null dv", dict(dv=None), _lib.ATTN_ERR_NULL),
    ("dtype 2", dict(dtype=2), _lib.ATTN_ERR_DTYPE),
    ("bf16 d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("f32 d=48", dict(d=48, dtype=_lib.ATTN_F32), _lib.ATTN_ERR_HEAD_DIM),
    ("H_kv=3", dict(H=4, H_kv=3), _lib.ATTN_ERR_SHAPE),
    ("layout 7", dict(layout=7), _lib.ATTN_ERR_ARG),
    ("noncausal window", dict(causal=0, window=1), _lib.ATTN_ERR_WINDOW),
    ("misaligned dk", dict(dk=_BW["dk"] + 8), _lib.ATTN_ERR_ALIGN),
    ("misaligned delta", dict(delta=_BW["delta"] + 2), _lib.ATTN_ERR_ALIGN),
    ("dq is q", dict(dq=_BW["q"]), _lib.ATTN_ERR_ALIAS),
    ("dv inside dout", dict(dv=_BW["do"] + 64), _lib.ATTN_ERR_ALIAS),
    ("dk is dv", dict(dk=_BW["dv"]), _lib.ATTN_ERR_ALIAS),
    ("delta inside lse", dict(delta=_BW["lse"] + 4), _lib.ATTN_ERR_ALIAS),
    ("delta inside dq", dict(delta=_BW["dq"] + 256), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_attn_bwd_rejects_before_any_hip_call(lib, name, kw, code):
    assert _bwd(lib, **kw) == code, name


@no_gpu
def test_attn_bwd_matches_attn_bwd_ex(lib):
    for name, kw, code in BWD_CASES:
        if "H_kv" in kw or "layout" in kw:
            continue
        a = dict(_BW, B=1, H=2, T=64, d=64, window=-1, causal=1, dtype=_lib.ATTN_BF16)
        a.update(kw)
        rc = lib.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["delta"], a["dq"],
                          a["dk"], a["dv"], a["B"], a["H"], a["T"], a["d"], a["window"],
                          a["causal"], a["dtype"], None)
        assert rc == code, name


_PB = {n: (i + 1) * P for i, n in enumerate(("q", "k", "gq", "gk", "oq", "ok", "cos", "sin"))}


def _pbwd(lib, **kw):
    a = dict(_PB, B=1, H=2, H_kv=2, T=64, d=64, layout=0, eps=1e-6, dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_qknorm_rope_bwd_ex(a["q"], a["k"], a["gq"], a["gk"], a["oq"], a["ok"],
                                       a["cos"], a["sin"], a["B"], a["H"], a["H_kv"], a["T"],
                                       a["d"], a["layout"], a["eps"], a["dtype"], None)


PBWD_CASES = [
    ("null k", dict(k=None), _lib.ATTN_ERR_NULL),
    ("q without dq_in", dict(gq=None), _lib.ATTN_ERR_NULL),
    ("q without dq_out", dict(oq=None), _lib.ATTN_ERR_NULL),
    ("dq_in without q", dict(q=None, oq=None), _lib.ATTN_ERR_NULL),
    ("d=24", dict(d=24), _lib.ATTN_ERR_HEAD_DIM),
    ("eps < 0", dict(eps=-1.0), _lib.ATTN_ERR_ARG),
    ("misaligned dk_out", dict(ok=_PB["ok"] + 4), _lib.ATTN_ERR_ALIGN),
    ("dk_out inside dk_in", dict(ok=_PB["gk"] + 16), _lib.ATTN_ERR_ALIAS),
    ("dk_out is k", dict(ok=_PB["k"]), _lib.ATTN_ERR_ALIAS),
    ("dq_out is dk_in", dict(oq=_PB["gk"]), _lib.ATTN_ERR_ALIAS),
    ("dq_out is q", dict(oq=_PB["q"]), _lib.ATTN_ERR_ALIAS),
    ("k only, dk_out inside k", dict(q=None, gq=None, oq=None, ok=_PB["k"] + 32),
     _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", PBWD_CASES, ids=[c[0] for c in PBWD_CASES])
def test_qknorm_rope_bwd_rejects_before_any_hip_call(lib, name, kw, code):
    assert _pbwd(lib, **kw) == code, name


# ---------------------------------------------------------------------------------------------
# Value-embedding gate.
# ---------------------------------------------------------------------------------------------

_VG = {n: (i + 1) * P for i, n in enumerate(("v", "ve", "z", "vo"))}


def _vg(lib, **kw):
    a = dict(_VG, B=1, H_kv=2, T=64, d=64, layout=0, dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_value_gate_ex(a["v"], a["ve"], a["z"], a["vo"], a["B"], a["H_kv"], a["T"],
                                  a["d"], a["layout"], a["dtype"], None)


VG_CASES = [
    ("null v", dict(v=None), _lib.ATTN_ERR_NULL),
    ("null ve", dict(ve=None), _lib.ATTN_ERR_NULL),
    ("null logits", dict(z=None), _lib.ATTN_ERR_NULL),
    ("null v_out", dict(vo=None), _lib.ATTN_ERR_NULL),
    ("dtype 7", dict(dtype=7), _lib.ATTN_ERR_DTYPE),
    ("d=24", dict(d=24), _lib.ATTN_ERR_HEAD_DIM),
    ("B=0", dict(B=0), _lib.ATTN_ERR_SHAPE),
    ("layout 2", dict(layout=2), _lib.ATTN_ERR_ARG),
    ("misaligned v", dict(v=_VG["v"] + 4), _lib.ATTN_ERR_ALIGN),
    ("misaligned bf16 logits", dict(z=_VG["z"] + 1), _lib.ATTN_ERR_ALIGN),
    ("misaligned f32 logits", dict(z=_VG["z"] + 2, dtype=_lib.ATTN_F32), _lib.ATTN_ERR_ALIGN),
    ("v_out inside v", dict(vo=_VG["v"] + 16), _lib.ATTN_ERR_ALIAS),
    ("v_out is ve", dict(vo=_VG["ve"]), _lib.ATTN_ERR_ALIAS),
    ("v_out over the logits", dict(vo=_VG["z"] - 64), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", VG_CASES, ids=[c[0] for c in VG_CASES])
def test_value_gate_rejects_before_any_hip_call(lib, name, kw, code):
    assert _vg(lib, **kw) == code, name


_VF = {n: (i + 1) * P for i, n in enumerate(("q", "k", "v", "ve", "z", "kw", "vw", "out", "lse",
                                             "cos", "sin"))}


def _vfused(lib, **kw):
    a = dict(_VF, B=1, H=4, H_kv=2, T=64, d=64, layout=0, eps=1e-6, window=-1, causal=1,
             dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_fwd_qknorm_ve_ex(a["q"], a["k"], a["v"], a["ve"], a["z"], a["kw"], a["vw"],
                                     a["out"], a["lse"], a["cos"], a["sin"], a["B"], a["H"],
                                     a["H_kv"], a["T"], a["d"], a["layout"], a["eps"],
                                     a["window"], a["causal"], a["dtype"], None)


VF_CASES = [
    ("null ve", dict(ve=None), _lib.ATTN_ERR_NULL),
    ("null logits", dict(z=None), _lib.ATTN_ERR_NULL),
    ("null v_work", dict(vw=None), _lib.ATTN_ERR_NULL),
    ("null k", dict(k=None), _lib.ATTN_ERR_NULL),
    ("f32", dict(dtype=_lib.ATTN_F32), _lib.ATTN_ERR_DTYPE),
    ("d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("window -2", dict(window=-2), _lib.ATTN_ERR_WINDOW),
    ("H_kv does not divide H", dict(H_kv=3), _lib.ATTN_ERR_SHAPE),
    ("misaligned ve", dict(ve=_VF["ve"] + 8), _lib.ATTN_ERR_ALIGN),
    ("v_work inside v", dict(vw=_VF["v"] + 16), _lib.ATTN_ERR_ALIAS),
    ("v_work is k_work", dict(vw=_VF["kw"]), _lib.ATTN_ERR_ALIAS),
    ("v_work is ve", dict(vw=_VF["ve"]), _lib.ATTN_ERR_ALIAS),
    ("k_work is v", dict(kw=_VF["v"]), _lib.ATTN_ERR_ALIAS),
    ("k_work over the logits", dict(kw=_VF["z"]), _lib.ATTN_ERR_ALIAS),
    ("out is ve", dict(out=_VF["ve"]), _lib.ATTN_ERR_ALIAS),
    ("out is v", dict(out=_VF["v"]), _lib.ATTN_ERR_ALIAS),
    ("lse over the logits", dict(lse=_VF["z"]), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", VF_CASES, ids=[c[0] for c in VF_CASES])
def test_attn_fwd_qknorm_ve_rejects_before_any_hip_call(lib, name, kw, code):
    assert _vfused(lib, **kw) == code, name


_VB = {n: (i + 1) * P for i, n in enumerate(("ve", "z", "dv", "dve", "dz"))}


def _vgb(lib, **kw):
    a = dict(_VB, B=2, H_kv=2, T=64, d=32, layout=1, dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_value_gate_bwd_ex(a["ve"], a["z"], a["dv"], a["dve"], a["dz"], a["B"],
                                      a["H_kv"], a["T"], a["d"], a["layout"], a["dtype"], None)


VGB_CASES = [
    ("null dv", dict(dv=None), _lib.ATTN_ERR_NULL),
    ("null dve", dict(dve=None), _lib.ATTN_ERR_NULL),
    ("null dlogits", dict(dz=None), _lib.ATTN_ERR_NULL),
    ("dtype 2", dict(dtype=2), _lib.ATTN_ERR_DTYPE),
    ("d=48", dict(d=48), _lib.ATTN_ERR_HEAD_DIM),
    ("misaligned dlogits", dict(dz=_VB["dz"] + 1), _lib.ATTN_ERR_ALIGN),
    ("dve inside dv", dict(dve=_VB["dv"] + 16), _lib.ATTN_ERR_ALIAS),
    ("dve is ve", dict(dve=_VB["ve"]), _lib.ATTN_ERR_ALIAS),
    ("dlogits are the logits", dict(dz=_VB["z"]), _lib.ATTN_ERR_ALIAS),
    ("dlogits inside dve", dict(dz=_VB["dve"] + 64), _lib.ATTN_ERR_ALIAS),
    ("dlogits inside dv", dict(dz=_VB["dv"] + 64), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", VGB_CASES, ids=[c[0] for c in VGB_CASES])
def test_value_gate_bwd_rejects_before_any_hip_call(lib, name, kw, code):
    assert _vgb(lib, **kw) == code, name


# ---------------------------------------------------------------------------------------------
# Decode.
# ---------------------------------------------------------------------------------------------

def test_decode_workspace_bytes(lib):
    # B * H * splits * (d + 2) * 4 with keys = min(S, window + 1) and
    # splits = min(ceil(keys / (4 * 4096 / d)), ceil(2048 / (B * H))): 256 keys per split at
    # d = 64, 128 at d = 128, 1024 at d = 16, and about 2048 workgroups at most
    assert lib.attn_decode_workspace_bytes(2, 3, 1000, 64, -1) == 2 * 3 * 4 * 66 * 4
    assert lib.attn_decode_workspace_bytes(2, 3, 1000, 64, 255) == 2 * 3 * 1 * 66 * 4
    assert lib.attn_decode_workspace_bytes(2, 3, 1000, 64, 256) == 2 * 3 * 2 * 66 * 4
    assert lib.attn_decode_workspace_bytes(2, 3, 1000, 128, -1) == 2 * 3 * 8 * 130 * 4
    assert lib.attn_decode_workspace_bytes(2, 3, 1025, 16, -1) == 2 * 3 * 2 * 18 * 4
    assert lib.attn_decode_workspace_bytes(1, 1, 1 << 20, 64, -1) == 2048 * 66 * 4
    assert lib.attn_decode_workspace_bytes(1, 16, 131072, 128, -1) == 16 * 128 * 130 * 4
    assert lib.attn_decode_workspace_bytes(64, 64, 4096, 128, -1) == 64 * 64 * 1 * 130 * 4
    assert lib.attn_decode_workspace_bytes(0, 3, 1000, 64, -1) == -1
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 64, -2) == -1


_DC = {n: (i + 1) * P for i, n in enumerate(("q", "k", "v", "len", "out", "lse", "ws"))}


def _dec(lib, **kw):
    a = dict(_DC, wsb=1 << 20, B=2, H=4, H_kv=2, S=300, d=64, layout=0, window=-1,
             dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_decode_ex(a["q"], a["k"], a["v"], a["len"], a["out"], a["lse"], a["ws"],
                              a["wsb"], a["B"], a["H"], a["H_kv"], a["S"], a["d"], a["layout"],
                              a["window"], a["dtype"], None)


DEC_CASES = [
    ("null q", dict(q=None), _lib.ATTN_ERR_NULL),
    ("null workspace", dict(ws=None), _lib.ATTN_ERR_NULL),
    ("dtype 5", dict(dtype=5), _lib.ATTN_ERR_DTYPE),
    ("bf16 d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("S=0", dict(S=0), _lib.ATTN_ERR_SHAPE),
    ("H_kv=3", dict(H_kv=3), _lib.ATTN_ERR_SHAPE),
    ("layout 3", dict(layout=3), _lib.ATTN_ERR_ARG),
    ("window -2", dict(window=-2), _lib.ATTN_ERR_WINDOW),
    ("misaligned out", dict(out=_DC["out"] + 8), _lib.ATTN_ERR_ALIGN),
    ("misaligned lengths", dict(len=_DC["len"] + 2), _lib.ATTN_ERR_ALIGN),
    ("workspace too small", dict(wsb=2 * 4 * 2 * 66 * 4 - 4), _lib.ATTN_ERR_ARG),
    ("out is q", dict(out=_DC["q"]), _lib.ATTN_ERR_ALIAS),
    ("workspace inside k", dict(ws=_DC["k"] + 4096), _lib.ATTN_ERR_ALIAS),
    ("lse inside workspace", dict(lse=_DC["ws"] + 16), _lib.ATTN_ERR_ALIAS),
    ("out over lengths", dict(out=_DC["len"] - 16), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_rejects_before_any_hip_call(lib, name, kw, code):
    assert _dec(lib, **kw) == code, name


def _dec_noalloc(lib, **kw):
    a = dict(_DC, B=2, H=4, H_kv=2, S=300, d=64, layout=0, window=-1, dtype=_lib.ATTN_BF16)
    a.update(kw)
    return lib.attn_decode_noalloc_ex(a["q"], a["k"], a["v"], a["len"], a["out"], a["lse"],
                                      a["B"], a["H"], a["H_kv"], a["S"], a["d"], a["layout"],
                                      a["window"], a["dtype"], None)


# The largest (B, H) whose workspace fits the fixed scratch at d = 128 with one split per head
# (S = 128 keys): B * H * 130 * 4 bytes <= 8 MiB.
_SCRATCH_HEADS = _lib.ATTN_DECODE_SCRATCH_BYTES // (130 * 4)

DEC_NOALLOC_CASES = [
    ("null q", dict(q=None), _lib.ATTN_ERR_NULL),
    ("null out", dict(out=None), _lib.ATTN_ERR_NULL),
    ("dtype 5", dict(dtype=5), _lib.ATTN_ERR_DTYPE),
    ("bf16 d=16", dict(d=16), _lib.ATTN_ERR_HEAD_DIM),
    ("S=0", dict(S=0), _lib.ATTN_ERR_SHAPE),
    ("H_kv=3", dict(H_kv=3), _lib.ATTN_ERR_SHAPE),
    ("layout 3", dict(layout=3), _lib.ATTN_ERR_ARG),
    ("window -2", dict(window=-2), _lib.ATTN_ERR_WINDOW),
    ("misaligned out", dict(out=_DC["out"] + 8), _lib.ATTN_ERR_ALIGN),
    ("out is q", dict(out=_DC["q"]), _lib.ATTN_ERR_ALIAS),
    ("lse over k", dict(lse=_DC["k"] + 64), _lib.ATTN_ERR_ALIAS),
    ("workspace past the scratch", dict(B=1, H=_SCRATCH_HEADS + 1, H_kv=1, S=128, d=128,
                                        **{n: (i + 1) << 32 for i, n in enumerate(_DC)}),
     _lib.ATTN_ERR_SCRATCH),
    ("workspace at the scratch limit, out over q",
     dict({n: (i + 1) << 32 for i, n in enumerate(_DC)}, B=1, H=_SCRATCH_HEADS, H_kv=1, S=128,
          d=128, out=1 << 32), _lib.ATTN_ERR_ALIAS),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code", DEC_NOALLOC_CASES, ids=[c[0] for c in DEC_NOALLOC_CASES])
def test_decode_noalloc_rejects_before_any_hip_call(lib, name, kw, code):
    assert _dec_noalloc(lib, **kw) == code, name


def test_decode_noalloc_scratch_limit_matches_workspace_sizes(lib):
    # the shape one head past the limit needs more than the scratch; the limit itself fits
    assert lib.attn_decode_workspace_bytes(1, _SCRATCH_HEADS, 128, 128, -1) <= \
        _lib.ATTN_DECODE_SCRATCH_BYTES
    assert lib.attn_decode_workspace_bytes(1, _SCRATCH_HEADS + 1, 128, 128, -1) > \
        _lib.ATTN_DECODE_SCRATCH_BYTES
    assert "scratch" in lib.attn_strerror(_lib.ATTN_ERR_SCRATCH).decode()



def test_issue_rate_probe_loads_and_names_its_modes():
    # The issue-rate probe behind bench.py --issue-rates is a library of its own; here it only
    # loads and names its loops (no kernel runs).
    from transformer_attention_qk_amd import build as _build
    path = _build.DIAG_PATH if os.path.exists(_build.DIAG_PATH) else _build.build_diag_library()
    d = ctypes.CDLL(path)
    d.attn_diag_issue_name.restype = ctypes.c_char_p
    d.attn_diag_issue_name.argtypes = [ctypes.c_int]
    d.attn_diag_issue_rates.restype = ctypes.c_int
    d.attn_diag_issue_rates.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    names = []
    while d.attn_diag_issue_name(len(names)) is not None:
        names.append(d.attn_diag_issue_name(len(names)).decode())
    assert len(names) == 9
    assert names[0].startswith("16 mfma") and "v_dot2c_f32_bf16" in names[7]
    assert d.attn_diag_issue_name(-1) is None
    # too small an output array is refused before any HIP call
    buf = (ctypes.c_double * 4)()
    assert d.attn_diag_issue_rates(buf, 4) != 0
