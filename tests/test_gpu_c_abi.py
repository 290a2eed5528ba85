"""The C ABI from a plain-C program (tests/c_abi_example.c): HIP runtime
buffers and a stream of its own, no Python in the path, results checked
against the C oracle inside the program.  __graft_entry__.build() builds it."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_example.bin")


def test_c_program_uses_the_abi(gpu):
    assert os.path.exists(EXE), "tests/c_abi_example.bin is not built; run __graft_entry__.build()"
    print("[case] c_abi_example", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_abi_example: ok" in r.stdout
