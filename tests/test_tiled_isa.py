"""Assembly-level guards for the LDS-tiled GEMM (CPU: hipcc cross-compiles
gfx950 here).

The tiled kernels load operands straight into LDS with gfx950's
`buffer_load_dwordx4 ... lds` / `global_load_lds_dwordx4`, issued from
inline asm that writes M0 (the LDS destination) without declaring it
clobbered (the compiler reserves M0).  That is sound only while nothing
else in these kernels keeps a value in M0, so: every M0 write must be one
of those asm blocks' `s_mov_b32 m0, <scalar register>`, directly followed
by an LDS-DMA load, and M0 must appear nowhere else.  The kernels must also
keep every value in registers (no scratch memory: a scratch access in the
K loop would be a vector-memory access the explicit load-count waits do not
expect).
"""
import os
import re
import subprocess
import tempfile

import pytest

from expert_router_gemm_amd import build as b

SRC = os.path.join(b.CSRC, "gemm_tiled.hip")


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm_tiled.s")
        cmd = [b.hipcc(), *b.HIPFLAGS, "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(f"hipcc -S failed:\n{r.stderr[-2000:]}")
        with open(out) as f:
            return f.read()


def _code_lines(text):
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if s:
            yield s


def test_m0_written_only_for_lds_dma(asm):
    lines = list(_code_lines(asm))
    writes = 0
    for i, s in enumerate(lines):
        if not re.search(r"\bm0\b", s):
            continue
        # (the asm operand is any scalar register, vcc's halves included)
        assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", s), f"unexpected use of m0: {s!r}"
        nxt = lines[i + 1] if i + 1 < len(lines) else ""
        assert re.match(r"(buffer_load_dwordx4 .* lds|global_load_lds_dwordx4 )", nxt), (
            f"m0 write not followed by an LDS-DMA load: {s!r} then {nxt!r}")
        writes += 1
    assert writes > 0, "no LDS-DMA loads found"


def test_tiled_kernels_use_no_scratch(asm):
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes, "no kernel metadata found"
    assert all(int(v) == 0 for v in sizes), f"private segment sizes {sizes}"
    assert "scratch_" not in asm, "scratch memory instructions in the tiled kernels"
