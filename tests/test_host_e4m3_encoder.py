"""Host check of the FP4 encoder's arithmetic for E4M3 scales.

The library encodes a group with an E4M3 scale s = 2^E * sig by dividing each
value by sig (correctly rounded: a product with RN(1/sig) and one residual
step) and letting the hardware convert round at 2^E, and it takes the scale
byte in closed form.  tests/host/e4m3_encoder_check.c models that arithmetic
in C and compares it with the encoding rule (jokeuncle.pages.dev, "两张架构图里
藏着 890 字节", section 三: E2M1 values with an E4M3 scale per 16; the rounding
reading: smallest scale with 6 s >= max, nearest value, ties to even) at every
scale code over the fp32 neighbourhoods of every midpoint, grid value and scale
boundary, and on seeded random values.  The GPU codec tests check the kernels
themselves against the oracle bit for bit."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(__file__), "host", "e4m3_encoder_check.c")


def _run(tmp_path, *defines):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path / "e4m3_encoder_check")
    subprocess.run([cc, "-O2", "-ffp-contract=off", *defines, SRC, "-o", exe, "-lm"], check=True)
    return subprocess.run([exe, "4096", "1000000", "11"], capture_output=True, text=True, timeout=120)


def test_e4m3_encoder_arithmetic_matches_rule(tmp_path):
    r = _run(tmp_path)
    assert r.returncode == 0, r.stdout
    counts = r.stdout.split()
    assert counts[-1] == "0" and int(counts[1]) > 1_000_000 and int(counts[3]) > 20_000_000


def test_e4m3_encoder_check_catches_a_missing_residual_step(tmp_path):
    r = _run(tmp_path, "-DWITHOUT_RESIDUAL_STEP")
    assert r.returncode == 1 and int(r.stdout.split()[-1]) > 0
