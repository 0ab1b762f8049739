"""Build-level checks of the gfx950 code (CPU only: hipcc cross-compiles).

The bf16 attention kernel issues its direct global -> LDS loads from inline assembly, which sets
M0 (the hardware register that carries the LDS base of such loads). The compiler is told M0 is
clobbered but treats it as reserved, so this test checks that no compiler-generated instruction
in any attention instantiation reads M0: every mention of M0 must be a write by that assembly.
It also checks that no kernel of any source file spills registers to scratch memory.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_attention_qk_amd", "csrc")
KERNEL_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") and f != "api.hip")
_ISA = {}


def _isa_of(name, tmp_path_factory):
    if name not in _ISA:
        hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
        if not os.path.exists(hipcc):
            pytest.skip("hipcc not available")
        from transformer_attention_qk_amd.build import HIPCC_FLAGS
        flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
        out = tmp_path_factory.mktemp("isa") / (name + ".s")
        cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
               "-o", str(out), os.path.join(CSRC, name)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        _ISA[name] = out.read_text()
    return _ISA[name]


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    return _isa_of("attn_fwd_bf16.hip", tmp_path_factory)


def test_m0_only_written_by_the_dma_assembly(isa):
    lines = [l.split(";")[0].strip() for l in isa.splitlines()]
    uses = [l for l in lines if re.search(r"\bm0\b", l)]
    assert uses, "expected the direct-to-LDS loads to set M0"
    assert all(l.startswith("s_mov_b32 m0,") for l in uses), [l for l in uses if not l.startswith("s_mov_b32 m0,")][:5]


@pytest.mark.parametrize("name", KERNEL_SOURCES)
def test_no_scratch_spills(name, tmp_path_factory):
    isa = _isa_of(name, tmp_path_factory)
    names = re.findall(r"^\s+\.name:\s+(\S+)", isa, re.M)
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", isa)
    assert sizes and len(sizes) == len(names), (len(sizes), len(names))
    spilled = [(n, int(z)) for n, z in zip(names, sizes) if int(z) != 0]
    assert not spilled, spilled
