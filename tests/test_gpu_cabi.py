"""The C ABI without Python: `tests/cabi/c_abi_check.cpp`, plain host code
built against libkvpage.so by build(), runs one decode step on hipMalloc'd
buffers and checks closed-form results (q = 0: mean of V, lse = ln ctx,
page mass = token share, zero summaries and page maxima) and an invalid
call's status."""

import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "cabi", "kvpage_c_abi_check")


def test_c_abi_check_program():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "build() did not build the C ABI check program"
    say("c abi check", BIN)
    res = subprocess.run([BIN], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "c abi check ok" in res.stdout
