"""GPU parity of the production (pipelined) kernels where the result is exact.

Rank-r indexing probe: the inputs of ``tests/exact_probe.py`` make every
product a small integer times a power of two, so every fp32 sum is exact in
any order.  The GPU must then return the oracle's H, G, dA, dB bit for bit,
and Y, dX equal to the one round-to-nearest-even of the oracle's exact value
to bf16 (the operator's single rounding of each output element).  A token
row served by the wrong adapter, a rank column read at the wrong offset or a
tile written to the wrong rows changes the exact value.  The shapes keep
d_in and d_out multiples of 128, so the pipelined GEMMs (both tile widths),
the pipelined shrink (both tile sizes, K slices and their sum) and, for
ranks <= 64, the weight-gradient kernels that stream transposed H/G (with
partials over several token chunks and their fixed-order reduction) all run.

Non-dyadic scales: s_i = alpha_i / r_i that are not powers of two (2/3, 5/3,
7/48) on the same kernels, at the bf16 tolerance for Y, dX and at 1e-4 for the
fp32 outputs H, G, dA, dB (fp32 accumulation of exact bf16 products; H and G
enter the expand and the weight gradients as a bf16 hi/lo pair, about 2^-16
relative).
"""
import numpy as np
import pytest

import oracle
import workloads
from exact_probe import ADAPTER_SETS, probe_inputs
from parity_utils import TOL, TOL_F32_OUT, check_block, h_blocks, host, log, run_gpu, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(512, 768), (4096, 1024)]


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


_cache = {}


def probe_case(shape, set_name):
    """Workload, inputs and oracle outputs (cached per shape and adapter set)."""
    key = (shape, set_name)
    if key not in _cache:
        d_in, d_out = shape
        cfg = ADAPTER_SETS[set_name]
        alphas = [s * r for s, r in zip(cfg["scales"], cfg["ranks"])]
        wl = workloads.custom(d_in, d_out, cfg["counts"], cfg["ranks"], alphas, "bf16",
                              name="probe_%s_%dx%d" % (set_name, d_in, d_out))
        inp = probe_inputs(cfg["counts"], cfg["ranks"], d_in, d_out, seed=17)[0]
        ref = oracle.run_workload(wl, inp)
        _cache[key] = (wl, inp, ref)
    return _cache[key]


def rne_bf16(a):
    """The exact fp64 value rounded once to bf16 (fp64 -> fp32 is exact here:
    small integers times powers of two)."""
    f = np.asarray(a, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), a), "probe value not exact in fp32"
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(f)).reshape(f.shape).astype(np.float64)


@pytest.mark.parametrize("shrink_rows", ["128", "32"])
@pytest.mark.parametrize("tile_p", ["256", "128"])
@pytest.mark.parametrize("set_name", sorted(ADAPTER_SETS))
@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_rank_r_probe_exact(P, shape, set_name, tile_p, shrink_rows, monkeypatch):
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    monkeypatch.setenv("PLORA_SHRINK_TILE_ROWS", shrink_rows)
    wl, inp, ref = probe_case(shape, set_name)
    log("case %s tile_p=%s shrink_rows=%s T=%d" % (wl.name, tile_p, shrink_rows, wl.T))
    gpu = run_gpu(P, wl, {k: to_dev(v, "bf16") for k, v in inp.items()})
    got = {k: host(v) for k, v in gpu.items()}
    for k in ("H", "G", "dA", "dB"):
        bad = np.flatnonzero(got[k].ravel() != ref[k].ravel())
        assert bad.size == 0, "%s: %d elements differ, first at %d: %r vs %r" % (
            k, bad.size, bad[0], got[k].ravel()[bad[0]], ref[k].ravel()[bad[0]])
    for k in ("Y", "dX"):
        want = rne_bf16(ref[k])
        bad = np.argwhere(got[k] != want)
        assert bad.size == 0, "%s: %d elements differ, first at %s: %r vs %r" % (
            k, len(bad), tuple(bad[0]), got[k][tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("tile_p", ["256", "128"])
def test_non_dyadic_scales_pipelined(P, tile_p, monkeypatch):
    """Scales that are not powers of two on the pipelined kernels: s = 16/24,
    20/12, 7/48, 3/33 (and one power of two), random normal inputs."""
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    wl = workloads.custom(512, 768, [600, 90, 0, 1300, 257], [24, 12, 48, 33, 16], [16.0, 20.0, 7.0, 3.0, 32.0],
                          "bf16", seed=41, name="non_dyadic")
    log("case %s tile_p=%s" % (wl.name, tile_p))
    inp = workloads.make_inputs(wl)
    gpu = {k: host(v) for k, v in run_gpu(P, wl, {k: to_dev(v, "bf16") for k, v in inp.items()}).items()}
    ref = oracle.run_workload(wl, inp)
    for i, rows, rr, hs, r, n in h_blocks(wl):
        for k in ("Y", "dX"):
            check_block(gpu[k][rows], ref[k][rows], TOL["bf16"], "%s[segment %d]" % (k, i))
        for k in ("H", "G"):
            check_block(gpu[k][hs], ref[k][hs], TOL_F32_OUT, "%s[adapter %d]" % (k, i))
        for k in ("dA", "dB"):
            check_block(gpu[k][rr], ref[k][rr], TOL_F32_OUT, "%s[adapter %d]" % (k, i))
