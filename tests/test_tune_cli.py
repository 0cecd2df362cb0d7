"""CPU checks of the tuner's command line: a malformed --shape is refused
before anything touches a device."""

import subprocess
import sys

import pytest


@pytest.mark.parametrize("shape", ["1,2,3", "1,2,64,64,64,f16,sideways", "1,2,64,64,64"])
def test_tune_rejects_malformed_shape(shape):
    r = subprocess.run([sys.executable, "-m", "attention_forward_02_amd.tune", "--shape", shape],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "--shape takes B,H,Nq,Nk,d,dtype[,causal]" in r.stderr
