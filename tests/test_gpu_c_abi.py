"""GPU: the library driven from plain C through its ABI only (no Python in
the tested path, as the Red Lite pages test their native code): closed-form
checks of gdn_step and gdn_gate_transform, gdn_seq == repeated gdn_step
bitwise, gdn_step_ex's cached policy == gdn_step bitwise, and argument
errors.  The program is tests/c/gdn_c_check.c, built by __graft_entry__.build()."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_program_through_the_abi():
    exe = os.path.join(HERE, "c", "gdn_c_check")
    assert os.path.exists(exe), "tests/c/gdn_c_check not built (run __graft_entry__.build())"
    print("\n  plain-C ABI check", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0 and "C ABI check ok" in r.stdout
