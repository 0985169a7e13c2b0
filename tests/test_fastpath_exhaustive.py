"""The store kernels' division-free tile arithmetic over its whole domain (CPU).

``tests/c/fastpath_exhaustive.c`` walks every bf16 amax whose tile takes the
kernels' fast path (biased exponent 72..254) and every bf16 x with |x| <= amax,
both signs (980,458,368 pairs): the division-free scale must equal
``amax / 448``, the corrected reciprocal must equal ``1 / scale`` (also from an
estimate up to 3 ulp off), and the corrected quotient must give the same e4m3
code as the IEEE division ``x / scale`` (the encoder is the oracle's).  The
quotient may differ from the division in its last bit for some pairs; the count
is reported.  A second run over one binade takes the plain reciprocal multiply
instead and must report code differences, which shows the comparison is live.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c", "fastpath_exhaustive.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "kvpub_oracle.c")


def _counts(out):
    return {k: int(v) for k, v in re.findall(r"(\w+) (\d+)", out)}


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("fastpath") / "fastpath_exhaustive")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    SRC, ORACLE_SRC, "-lm", "-o", exe], check=True)
    return exe


def _run(exe, *args):
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(16, os.cpu_count() or 1)))
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=600, env=env)


def test_fast_path_codes_equal_division_everywhere(program):
    r = _run(program)
    c = _counts(r.stdout)
    assert c.get("pairs") == 980458368, r.stdout
    assert c["code_differs"] == 0 and c["scale_bad"] == 0, r.stdout
    assert c["recip_bad"] == 0 and c["estimate_bad"] == 0, r.stdout
    assert r.returncode == 0, r.stdout + r.stderr


def test_plain_reciprocal_multiply_is_reported(program):
    r = _run(program, "product", "127")
    c = _counts(r.stdout)
    assert c["code_differs"] > 0 and r.returncode == 1, r.stdout
