"""GPU parity of the shared-input calls: the LoRA shrinks and dA gradients of
up to three projections that read the same input X (q/k/v, gate/up), in one
pass over X, against the single-projection entry points (bitwise) and the
fp64 oracle (H and dA at the fp32-output tolerance)."""
import numpy as np
import pytest

import oracle
import workloads
from parity_utils import check_full, host, log, poison, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def projections(d_in, d_outs, counts, ranks, alphas, dtype, seed):
    """One workload per projection: the same segments, ranks and alphas, the
    same X (projection 0's), their own W, A, B and dY."""
    wls = [workloads.custom(d_in, do, counts, ranks, alphas, dtype, seed=seed + 13 * p, name="proj%d" % p)
           for p, do in enumerate(d_outs)]
    inps = [workloads.make_inputs(w) for w in wls]
    for inp in inps[1:]:
        inp["X"] = inps[0]["X"]
    return wls, inps


def separate(P, wl, dev, d):
    """The single-projection path: forward, backward_dx, backward_dAdB."""
    import torch
    tdt = dev["X"].dtype
    he = P.plora_h_elems(d)
    o = {"Y": poison((wl.T, wl.d_out), tdt), "H": poison((he,), torch.float32),
         "dX": poison((wl.T, wl.d_in), tdt), "G": poison((he,), torch.float32),
         "dA": poison((wl.R, wl.d_in), torch.float32), "dB": poison((wl.R, wl.d_out), torch.float32)}
    P.plora_forward(d, dev["X"], dev["W"], dev["A"], dev["B"], o["Y"], o["H"])
    P.plora_backward_dx(d, dev["dY"], dev["W"], dev["A"], dev["B"], o["dX"], o["G"])
    nb = P.plora_workspace_bytes(d)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    P.plora_backward_dAdB(d, dev["X"], dev["dY"], o["H"], o["G"], o["dA"], o["dB"], ws)
    return o


CASES = [
    # pipelined shapes, ranks <= 64: the shared kernels; adapters of 0, 1, <= 128
    # and > 1024 tokens (K-sliced shrink in the single path, weight-gradient partials)
    ("qkv", 512, [768, 256, 256], [100, 0, 513, 1, 163, 40, 2100], [16, 8, 64, 32, 1, 48, 24],
     [32.0, 16.0, 8.0, 16.0, 4.0, 96.0, 48.0], "bf16"),
    ("gate_up", 1024, [1536, 1536], [300, 77, 1200], [8, 64, 16], [16.0, 128.0, 32.0], "bf16"),
    # ranks up to 128: one pass per projection behind the same entry points
    ("rank128", 512, [384, 256], [70, 300, 5], [128, 8, 33], [256.0, 16.0, 33.0], "bf16"),
    # d_in not a multiple of 64: the general kernels
    ("unaligned", 136, [264, 264, 128], [40, 9, 130], [16, 4, 64], [32.0, 4.0, 64.0], "bf16"),
    ("f32", 256, [192, 64], [33, 0, 90], [8, 16, 4], [16.0, 16.0, 8.0], "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shared_equals_separate_bitwise(P, case):
    import torch
    name, d_in, d_outs, counts, ranks, alphas, dtype = case
    log("case %s np=%d" % (name, len(d_outs)))
    wls, inps = projections(d_in, d_outs, counts, ranks, alphas, dtype, seed=71)
    devs = [{k: to_dev(v, dtype) for k, v in inp.items()} for inp in inps]
    for dv in devs[1:]:
        dv["X"] = devs[0]["X"]
    descs = [P.Desc.from_workload(w) for w in wls]
    sep = [separate(P, w, dv, d) for w, dv, d in zip(wls, devs, descs)]
    n = len(d_outs)
    he = P.plora_h_elems(descs[0])
    X = devs[0]["X"]
    # forward: one shrink pass, then each projection's GEMM with its H given
    H = [poison((he,), torch.float32) for _ in range(n)]
    P.plora_shrink_shared(descs[0], X, [dv["A"] for dv in devs], H)
    Y = [poison((w.T, w.d_out), X.dtype) for w in wls]
    for p in range(n):
        P.plora_forward_expand(descs[p], X, devs[p]["W"], devs[p]["B"], Y[p], H[p])
    # backward: dB alone per projection, one dA pass for all
    dB = [poison((w.R, w.d_out), torch.float32) for w in wls]
    for p in range(n):
        nb = P.plora_workspace_bytes(descs[p])
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        P.plora_backward_dAdB(descs[p], None, devs[p]["dY"], sep[p]["H"], None, None, dB[p], ws)
    dA = [poison((w.R, w.d_in), torch.float32) for w in wls]
    nb = P.plora_workspace_bytes_dA_shared(descs[0], n)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    P.plora_backward_dA_shared(descs[0], X, [s["G"] for s in sep], dA, ws)
    torch.cuda.synchronize()
    for p in range(n):
        assert torch.equal(bits(H[p]), bits(sep[p]["H"])), ("H", p)
        assert torch.equal(bits(Y[p]), bits(sep[p]["Y"])), ("Y", p)
        assert torch.equal(bits(dB[p]), bits(sep[p]["dB"])), ("dB", p)
        assert torch.equal(bits(dA[p]), bits(sep[p]["dA"])), ("dA", p)
    # accumulate: old + new, with old = new, is exactly twice (adapters
    # without tokens stay 0)
    P.plora_backward_dA_shared(descs[0], X, [s["G"] for s in sep], dA, ws, accumulate=True)
    torch.cuda.synchronize()
    for p in range(n):
        assert torch.equal(bits(dA[p]), bits(2.0 * sep[p]["dA"])), ("dA accumulate", p)
    # and against the oracle, per projection (X shared)
    for p in range(n):
        ref = oracle.run_workload(wls[p], inps[p])
        check_full(wls[p], {"H": host(H[p]), "dA": host(dA[p]) / 2.0, "Y": host(Y[p]), "dB": host(dB[p])}, ref,
                   names=("H", "dA", "Y", "dB"))


def test_shared_block_shapes_sampled(P):
    """The decoder block's q/k/v panels at full width (d_in 4096; d_out 4096,
    1024, 1024; 32 adapters of ranks 8..64, 256 tokens each): shared equals
    separate bitwise."""
    import torch
    counts = [256] * 32
    ranks = [8, 16, 32, 64] * 8
    alphas = [2.0 * r for r in ranks]
    wls, inps = projections(4096, [4096, 1024, 1024], counts, ranks, alphas, "bf16", seed=5)
    log("case block qkv T=%d" % wls[0].T)
    devs = [{k: to_dev(v, "bf16") for k, v in inp.items()} for inp in inps]
    for dv in devs[1:]:
        dv["X"] = devs[0]["X"]
    descs = [P.Desc.from_workload(w) for w in wls]
    sep = [separate(P, w, dv, d) for w, dv, d in zip(wls, devs, descs)]
    he = P.plora_h_elems(descs[0])
    H = [poison((he,), torch.float32) for _ in range(3)]
    P.plora_shrink_shared(descs[0], devs[0]["X"], [dv["A"] for dv in devs], H)
    dA = [poison((w.R, w.d_in), torch.float32) for w in wls]
    nb = P.plora_workspace_bytes_dA_shared(descs[0], 3)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    P.plora_backward_dA_shared(descs[0], devs[0]["X"], [s["G"] for s in sep], dA, ws)
    torch.cuda.synchronize()
    for p in range(3):
        assert torch.equal(bits(H[p]), bits(sep[p]["H"])), ("H", p)
        assert torch.equal(bits(dA[p]), bits(sep[p]["dA"])), ("dA", p)


def random_shared_case(seed):
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 10))
    counts = [0 if rng.random() < 0.15 else int(rng.integers(1, 5)) if rng.random() < 0.3 else int(rng.integers(5, 600))
              for _ in range(n)]
    ranks = [int(rng.choice([1, 4, 8, 16, 24, 32, 33, 48, 64, 96, 128] if rng.random() < 0.3 else [4, 8, 16, 32, 64]))
             for _ in range(n)]
    alphas = [float(rng.choice([1.0, 8.0, 16.0, 32.0])) for _ in range(n)]
    d_in = int(rng.choice([256, 512, 768])) if rng.random() < 0.7 else 8 * int(rng.integers(4, 80))
    npan = int(rng.integers(2, 4))
    d_outs = [int(rng.choice([128, 256, 384, 520])) for _ in range(npan)]
    return d_in, d_outs, counts, ranks, alphas


@pytest.mark.parametrize("seed", range(8))
def test_shared_random_bitwise(P, seed):
    """Randomized packings (empty and tiny segments, ranks 1..128, widths on
    and off the tile multiples, 2 or 3 projections): the shared shrink and dA
    equal the single-projection calls bit for bit."""
    import torch
    d_in, d_outs, counts, ranks, alphas = random_shared_case(seed)
    log("case shared_random%d d_in=%d d_outs=%s counts=%s ranks=%s" % (seed, d_in, d_outs, counts, ranks))
    wls, inps = projections(d_in, d_outs, counts, ranks, alphas, "bf16", seed=90 + seed)
    devs = [{k: to_dev(v, "bf16") for k, v in inp.items()} for inp in inps]
    for dv in devs[1:]:
        dv["X"] = devs[0]["X"]
    descs = [P.Desc.from_workload(w) for w in wls]
    sep = [separate(P, w, dv, d) for w, dv, d in zip(wls, devs, descs)]
    n = len(d_outs)
    he = P.plora_h_elems(descs[0])
    H = [poison((max(he, 1),), torch.float32)[:he] for _ in range(n)]
    P.plora_shrink_shared(descs[0], devs[0]["X"], [dv["A"] for dv in devs], H)
    dA = [poison((w.R, w.d_in), torch.float32) for w in wls]
    nb = P.plora_workspace_bytes_dA_shared(descs[0], n)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    P.plora_backward_dA_shared(descs[0], devs[0]["X"], [s["G"] for s in sep], dA, ws)
    torch.cuda.synchronize()
    for p in range(n):
        assert torch.equal(bits(H[p]), bits(sep[p]["H"])), ("H", p)
        assert torch.equal(bits(dA[p]), bits(sep[p]["dA"])), ("dA", p)
