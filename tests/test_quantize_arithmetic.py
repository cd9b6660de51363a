"""The kernels' division of a block's amax by 127 (a product with the f32 reciprocal and one
fused correction, three instructions) equals the IEEE f32 quotient that the quantize is defined
with, for every finite non-negative input: checked exhaustively on the CPU in C. A planted error
(no correction step) is caught, so the check can fail."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    out = tmp_path_factory.mktemp("div127")
    exe = str(out / "div127_check")
    src = os.path.join(HERE, "div127_check.c")
    # -ffp-contract=off: every product and sum is rounded as written (fmaf is the only fused op)
    base = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"]
    res = subprocess.run(base[:1] + ["-fopenmp"] + base[1:], capture_output=True, text=True)
    if res.returncode != 0:  # no OpenMP: one thread
        res = subprocess.run(base, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    # the same check with the correction step removed (q = a * c alone): must report mismatches
    planted = str(out / "div127_planted")
    text = open(src).read().replace("fmaf(fmaf(-q, 127.0f, a), c, q)", "q")
    psrc = str(out / "planted.c")
    open(psrc, "w").write(text)
    pbase = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", psrc, "-o", planted, "-lm"]
    res = subprocess.run(pbase[:1] + ["-fopenmp"] + pbase[1:], capture_output=True, text=True)
    if res.returncode != 0:
        res = subprocess.run(pbase, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe, planted


def test_div127_is_the_ieee_quotient_for_every_input(checker):
    exe, _ = checker
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600).stdout.split()
    assert out[0] == "0", f"{out[0]} inputs differ, the first 0x{out[1]}"


def test_the_check_catches_a_missing_correction(checker):
    _, planted = checker
    out = subprocess.run([planted], capture_output=True, text=True, timeout=600).stdout.split()
    assert int(out[0]) > 0
