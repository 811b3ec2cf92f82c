"""The block driven from a plain C program through the C ABI alone (GPU):
tests/c/abi_demo.c, built by ``__graft_entry__.build()``. It runs a seeded
300-token bf16 block under two chunk settings and checks bit-identity,
finite output and the documented argument errors."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_demo")


def test_c_program_through_the_abi():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build()")
    print("running tests/c/abi_demo", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "abi_demo: ok" in r.stdout
