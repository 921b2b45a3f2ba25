"""GPU test of plora_backward_dAdB_noalloc (the weight-gradient entry point
without a workspace argument, for callers that cannot allocate): through the
C ABI, its dA/dB equal those of plora_backward_dAdB with a caller workspace
bit for bit (the same kernels), on two calls in a row, the second with a
smaller problem (the scratch keeps the first call's contents), in overwrite
and in accumulate mode."""
import numpy as np
import pytest

import workloads
from parity_utils import log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def _case(P, wl):
    import torch
    inp = workloads.make_inputs(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in inp.items()}
    out = run_gpu(P, wl, dev)  # forward, backward_dx and dA/dB with a caller workspace
    d = P.Desc.from_workload(wl)
    return dev, out, d


def _bits(t):
    import torch
    return t.view(torch.int32)


def test_noalloc_matches_workspace_entry_point(P):
    import torch
    # first call: weight-gradient partials (adapters over several 1024-token
    # chunks) and transposes fill a large part of the scratch
    big = workloads.custom(512, 768, [2500, 0, 700, 3100, 1, 64], [16, 8, 64, 32, 1, 33],
                           [32.0, 16.0, 8.0, 16.0, 4.0, 66.0], "bf16", seed=61, name="noalloc_big")
    # second call: smaller, other ranks and widths (reads nothing the first left behind)
    small = workloads.custom(384, 640, [300, 1200, 5], [64, 16, 8], [16.0, 32.0, 8.0], "bf16", seed=62,
                             name="noalloc_small")
    for wl in (big, small):
        log("case %s T=%d workspace %d bytes" % (wl.name, wl.T, P.plora_workspace_bytes(P.Desc.from_workload(wl))))
        dev, out, d = _case(P, wl)
        dA = torch.full_like(out["dA"], float("nan"))
        dB = torch.full_like(out["dB"], float("nan"))
        P.plora_backward_dAdB_noalloc(d, dev["X"], dev["dY"], out["H"], out["G"], dA, dB)
        torch.cuda.synchronize()
        assert torch.equal(_bits(dA), _bits(out["dA"])), wl.name
        assert torch.equal(_bits(dB), _bits(out["dB"])), wl.name
        # accumulate mode: the same batch again doubles every element (x + x is exact)
        P.plora_backward_dAdB_noalloc(d, dev["X"], dev["dY"], out["H"], out["G"], dA, dB, accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(dA), _bits(2 * out["dA"])), wl.name
        assert torch.equal(_bits(dB), _bits(2 * out["dB"])), wl.name


def test_noalloc_fp32_and_no_tokens(P):
    """fp32 problems and problems without tokens need no scratch at all."""
    import torch
    wl = workloads.custom(136, 72, [5, 0, 33, 70], [3, 7, 16, 64], [6.0, 7.0, 32.0, 16.0], "f32", seed=63,
                          name="noalloc_f32")
    dev, out, d = _case(P, wl)
    dA = torch.full_like(out["dA"], float("nan"))
    dB = torch.full_like(out["dB"], float("nan"))
    P.plora_backward_dAdB_noalloc(d, dev["X"], dev["dY"], out["H"], out["G"], dA, dB)
    torch.cuda.synchronize()
    assert torch.equal(_bits(dA), _bits(out["dA"])) and torch.equal(_bits(dB), _bits(out["dB"]))
    z = P.Desc([0, 0, 0], [4, 64], [1.0, 8.0], 256, 320, "bf16")
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    dA = torch.full((68, 256), float("nan"), device="cuda")
    dB = torch.full((68, 320), float("nan"), device="cuda")
    h = torch.empty((0,), device="cuda")
    P.plora_backward_dAdB_noalloc(z, e(0, 256), e(0, 320), h, h, dA, dB)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA).item() == 0 and torch.count_nonzero(dB).item() == 0
