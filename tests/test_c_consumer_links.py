"""Without a GPU, the plain C consumer of the library still starts: its
libraries resolve (the library, the C oracle, the HIP runtime) and it stops
at its first device allocation with exit status 2."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_consumer", "lpq_c_consumer")


def test_c_consumer_links():
    if not os.path.exists(BIN):
        pytest.skip("the C consumer is not built (run the build step)")
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present: the GPU test runs the program instead")
    except ImportError:
        pass
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2, (res.returncode, res.stdout, res.stderr)
    assert "hipMalloc" in res.stderr
