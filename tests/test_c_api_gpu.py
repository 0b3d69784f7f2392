"""The C ABI used from a C++ host program with no Python or torch in the process
(sequence_attention_amd/c_api_demo, built next to the library by the build step).

The program allocates its buffers with the HIP runtime, calls xs_attn_fwd on a
B = 2, S = 384, H = 3, D = 64, P = 4 share whose keys of each (batch, head)
carry one value row, checks every output element against that row exactly, and
checks the status codes of five invalid calls; it exits 0 only if all hold.
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "sequence_attention_amd", "c_api_demo")


def test_c_program_through_the_c_abi(gpu):
    assert os.path.exists(DEMO), "c_api_demo is missing: run python -m sequence_attention_amd.build"
    print("[case] c_api_demo", flush=True)
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c_api_demo: ok" in r.stdout
