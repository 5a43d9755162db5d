"""The boundary from plain C: tests/c_consumer.c allocates with the HIP
runtime, calls fr_decode_attn on a one-hot case whose output must equal
chosen V rows bit for bit (ragged key count), and checks that invalid calls
return their status.  It runs as a child process."""
import subprocess

import pytest

from c_consumer_build import build_consumer
from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_plain_c_consumer_runs_bit_exact(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build_consumer(tmp_path / "c_consumer")
    say("c consumer: fr_decode_attn from a C program")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=90)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "bit-exact" in r.stdout
