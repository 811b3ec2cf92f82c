"""The public headers compile as plain C99 and a C program links against the
library (CPU: compile and link only, nothing runs)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import __graft_entry__ as G  # noqa: E402


def test_c_consumer_compiles_and_links(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(ROOT, "memory_bounded_chunked_amd", "libdit_block.so")):
        pytest.skip("library not built")
    r = subprocess.run(G.c_demo_command(str(tmp_path / "abi_demo")), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
