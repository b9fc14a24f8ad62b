"""The C client of the library (io_aware_attention_amd/example/fa355_example.c),
built by the package build, run as its own process: HIP runtime calls and the C ABI
only, no Python or torch in the path.  It checks a closed form (K = 0: O is the mean
of the visible V rows, lse = ln(i + 1)) and that an unsupported head dimension is
refused, and prints "fa355 example: ok" when everything holds."""
import os
import subprocess

import pytest

from io_aware_attention_amd import build

pytestmark = pytest.mark.gpu


def test_c_client_runs_and_checks_its_closed_form():
    assert os.path.exists(build.EXAMPLE_BIN), "run the package build first"
    r = subprocess.run([build.EXAMPLE_BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "fa355 example: ok" in r.stdout
    assert "d = 96: " in r.stdout and "unsupported" in r.stdout.lower()
