"""GPU parity on randomized packings: adapter counts, token counts (empty,
single-token, ragged, several tiles), ranks 1..128, alphas and layer widths
drawn from a seeded generator, each case compared in full against the fp64
oracle.  The widths are drawn both on and off the multiples of 128 and 64, so
the pipelined kernels and the general ones both run."""
import numpy as np
import pytest

import oracle
import workloads
from parity_utils import check_full, host, log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 13))
    kind = rng.choice(["empty", "tiny", "ragged", "tiles"], size=n, p=[0.15, 0.2, 0.4, 0.25])
    counts = [0 if k == "empty" else int(rng.integers(1, 5)) if k == "tiny" else int(rng.integers(5, 300))
              if k == "ragged" else int(rng.integers(300, 700)) for k in kind]
    ranks = [int(rng.choice([1, 2, 4, 7, 8, 16, 24, 32, 33, 48, 64, 96, 128])) for _ in range(n)]
    alphas = [float(rng.choice([1.0, 4.0, 8.0, 16.0, 32.0, 12.0])) * (1.0 if rng.random() < 0.7 else 1.5)
              for _ in range(n)]
    pick = lambda: int(rng.choice([128, 256, 384, 512, 640])) if rng.random() < 0.6 else 8 * int(rng.integers(4, 90))
    d_in, d_out = pick(), pick()
    dtype = "bf16" if rng.random() < 0.8 else "f32"
    return workloads.custom(d_in, d_out, counts, ranks, alphas, dtype, seed=50 + seed, name="random%d" % seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_packing_full(P, seed):
    wl = random_case(seed)
    log("case %s T=%d d_in=%d d_out=%d N=%d ranks=%s counts=%s dtype=%s" % (
        wl.name, wl.T, wl.d_in, wl.d_out, wl.n_adapters, list(wl.ranks), list(np.diff(wl.offsets)), wl.dtype))
    inp = workloads.make_inputs(wl)
    gpu = {k: host(v) for k, v in run_gpu(P, wl, {k: to_dev(v, wl.dtype) for k, v in inp.items()}).items()}
    ref = oracle.run_workload(wl, inp)
    check_full(wl, gpu, ref)
