"""The step library driven from plain C++ through its C ABI alone (no Python, no torch):
tests/c_abi_check, built by __graft_entry__.build(), checks step 1 against its closed
form, the skip, half = RNE(master), and flat / chunked / misaligned agreement."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_program_through_the_abi():
    assert os.path.exists(EXE), "tests/c_abi_check is missing: run __graft_entry__.build()"
    print("case c_abi_check", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c_abi_check ok" in r.stdout, r.stdout + r.stderr
