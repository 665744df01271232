"""liblinbwd.so from a plain C program (tests/native/c_abi_consumer.c, built by the build
step): lin_bwd on integer-valued inputs, exact, on the MFMA kernels and through padded
copies; adamw_step with lr = 0; an error code and message.  No Python in the calls."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "c_abi_consumer")


def test_c_program_on_the_c_abi():
    assert os.path.exists(BIN), "%s is not built (run the build step)" % BIN
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_abi_consumer: ok" in r.stdout
