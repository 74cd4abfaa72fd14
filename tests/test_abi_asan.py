"""The host-side validation layer under AddressSanitizer (CPU only).

tests/asan/build.py compiles the library's sources with AddressSanitizer on
their host code and links them with a driver that calls every entry point
declared in include/rmm.h with arguments the validation rejects, queries the
workspace sizes over a spread of shapes, and answers k_from_rho queries.  The
driver runs here, without a GPU; an ASan report or a wrong status fails the
test.  The k answers are compared with the oracle's exact ceiling.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
from test_abi import _adversarial_ratios

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def driver():
    if not os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("g++") is None:
        pytest.skip("hipcc and g++ are needed to build the ASan driver")
    import sys
    sys.path.insert(0, os.path.join(HERE, "asan"))
    try:
        import build as asan_build
    finally:
        sys.path.pop(0)
    return asan_build.build()


def _run(driver, stdin_text):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:exitcode=86"
    r = subprocess.run([driver, "k"], input=stdin_text, capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    return r.stdout


def test_validation_layer_under_asan(driver):
    rng = np.random.default_rng(31)
    ratios = _adversarial_ratios(rng, 20000)
    ds = [int(x) for x in rng.integers(1, 2 ** 31 - 1, size=len(ratios))]
    lines = [f"{struct.unpack('<Q', struct.pack('<d', r))[0]:016x} {d}" for r, d in zip(ratios, ds)]
    out = _run(driver, "\n".join(lines) + "\n").split()
    assert len(out) == len(ratios)
    bad = [(repr(r), d, int(k)) for r, d, k in zip(ratios, ds, out) if int(k) != oracle.retained_count(r, d)]
    assert not bad, bad[:10]
