"""The GEMM's hand-placed LDS waits are sound in the code the compiler
actually emits: no instruction touches the destination of an inline-asm LDS
read before an lgkmcnt wait retires it (checked on the gfx950 assembly of
every GEMM instantiation, plus planted violations the check must catch)."""

import os
import re
import subprocess

import pytest

from lds_wait_check import check_function, gemm_functions
from mixture_experts_expert_mm_amd import _build


def _asm(tmp_path_factory, src):
    out = tmp_path_factory.mktemp("asm") / (src + ".s")
    cmd = [_build.HIPCC, *[f for f in _build.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return out.read_text()


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "mm_gemm.hip")


@pytest.fixture(scope="module")
def mega_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "mm_mega.hip")


@pytest.mark.parametrize("which,min_kernels", [("gemm", 12), ("mega", 6)])
def test_every_gemm_kernel_waits_before_use(which, min_kernels, request):
    text = request.getfixturevalue(which + "_asm")
    names = gemm_functions(text)
    assert len(names) >= min_kernels
    for n in names:
        report, nreads = check_function(text, n)
        assert nreads > 0, n
        assert report == [], (n, report[:5])


def _plant(text, name, make):
    """Insert make(first_dest_reg) after the 20th inline-asm LDS read of `name`."""
    i = text.index(name + ":")
    j = i
    for _ in range(20):
        j = text.index("ds_read_b128 v[", j + 1)
    reg = int(re.match(r"ds_read_b128 v\[(\d+):", text[j:]).group(1)) + 1
    e = text.index(";;#ASMEND", j) + len(";;#ASMEND")
    return text[:e] + "\n\t" + make(reg) + text[e:]


@pytest.mark.parametrize("make", [lambda r: f"v_mov_b32_e32 v255, v{r}",        # read of an in-flight register
                                  lambda r: f"v_mov_b32_e32 v{r}, 0"])           # write of an in-flight register
def test_check_catches_planted_violation(gemm_asm, make):
    name = gemm_functions(gemm_asm)[0]
    report, _ = check_function(_plant(gemm_asm, name, make), name)
    assert len(report) == 1
