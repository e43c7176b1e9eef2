"""The C ABI from plain C: tests/c_consumer/lpq_c_consumer (built by the build
step with gcc, linked against liblpq.so, the HIP runtime and the C oracle)
calls every format's entry points on device buffers it allocates itself and
compares every output with the oracle, bit for bit.  It runs as a child
process: no Python binding and no torch are on its path."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_consumer", "lpq_c_consumer")

pytestmark = pytest.mark.gpu


def test_c_consumer_matches_oracle():
    if not os.path.exists(BIN):
        pytest.skip("the C consumer is not built (run the build step)")
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "OK: every C entry point matches the oracle" in res.stdout
