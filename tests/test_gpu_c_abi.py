"""The C ABI from plain C: tests/c_abi/plora_c_abi_test (built by
__graft_entry__.build()) allocates device memory with the HIP runtime, calls
plora_forward, plora_backward_dx and plora_backward_dAdB on the null stream
and checks every output against the fp64 oracle (no Python or PyTorch in that
process)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "plora_c_abi_test")


def test_c_program_against_oracle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert os.path.exists(BIN), "tests/c_abi/plora_c_abi_test is not built (run __graft_entry__.build())"
    print("case c_abi program", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "PASS" in r.stdout
