"""Host check of the quantiser's shortcut for x / s (the fp8 quantisation of
the gate-up input, *Ling-2.6-1T on TPU*, §5: tokens quantised per token with
scale amax / 448).  The kernels take y = x * (1/s) for the e4m3 code unless y
lies within 4 binary32 ulps of an e4m3 rounding midpoint, below 2^-6, or 1/s
overflows; then they divide.  y is within 2.5 ulps of the exact quotient, so
away from a midpoint both round to the same code.

`native/e4m3_shortcut.c` (plain C, IEEE binary32 on the host) compares the
two codes for every bf16 x against 2000 scales; the midpoint-only window must
show differences, so that the comparison is known to be able to fail."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("e4m3") / "e4m3_shortcut")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "native", "e4m3_shortcut.c"),
                    "-lm"], check=True)
    return exe


def run(exe, n, window):
    out = subprocess.run([exe, str(n), str(window)], check=True, capture_output=True, text=True).stdout
    pairs, bad = (int(v) for v in out.split())
    return pairs, bad


def test_shortcut_gives_the_quotients_codes(checker):
    pairs, bad = run(checker, 2000, 4)
    assert pairs > 100_000_000 and bad == 0


def test_midpoint_only_window_is_caught(checker):
    pairs, bad = run(checker, 400, 0)
    assert bad > 0
