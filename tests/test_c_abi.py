"""The library used from plain C (tests/c_abi/abi_demo.c, C11 with gcc): the header
compiles as C, the host-side contract holds (status strings, workspace sizes,
argument checks), and on the GPU the GQA and MLA entry points, the partition pass
and splitk_reduce() match the fp64 C oracle -- with no Python between the caller and
the library."""
import os
import subprocess

import pytest

from c_abi import build as cbuild


def _run(mode, timeout):
    if not os.path.exists(cbuild.BIN):
        cbuild.build()
    res = subprocess.run([cbuild.BIN, mode], capture_output=True, text=True, timeout=timeout)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "PASSED" in res.stdout


def test_c_abi_host():
    cbuild.build()
    _run("host", 60)


@pytest.mark.gpu
def test_c_abi_gpu():
    _run("gpu", 150)
