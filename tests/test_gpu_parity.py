"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small problems (several tiles, ragged tails, empty segments, ranks 1..128) are
compared in full.  The full-size workloads (the benchmark's launch
configuration) are compared on sampled token rows for Y/dX/H/G (rows are
independent, so the oracle computes just those rows) and in full for every
adapter's dA/dB (and H/G), adapter by adapter.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity_utils import TOL, check_block, check_full, h_blocks, host, log, run_gpu, to_dev, tol_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def device_inputs(wl, inp):
    return {k: to_dev(v, wl.dtype) for k, v in inp.items()}


def gpu_host(gpu):
    return {k: host(v) for k, v in gpu.items()}


def full_case(P, wl):
    log("case %s T=%d d_in=%d d_out=%d N=%d dtype=%s" % (wl.name, wl.T, wl.d_in, wl.d_out, wl.n_adapters, wl.dtype))
    inp = workloads.make_inputs(wl)
    gpu = gpu_host(run_gpu(P, wl, device_inputs(wl, inp)))
    ref = oracle.run_workload(wl, inp)
    check_full(wl, gpu, ref)
    return inp, gpu, ref


# ---------------------------------------------------------------------------
# small problems, compared in full
# ---------------------------------------------------------------------------

def test_tiny_f32_full(P):
    full_case(P, workloads.config("tiny"))


def test_bf16_ragged_full(P):
    # K tail (320 % 64), feature tail (264 % 256), 1-token and empty segments, ranks 1..128
    wl = workloads.custom(320, 264, [1, 0, 37, 300, 2, 129, 64], [1, 8, 16, 33, 64, 100, 128],
                          [1.0, 16.0, 32.0, 33.0, 128.0, 50.0, 256.0], "bf16", seed=21, name="ragged_bf16")
    full_case(P, wl)


# The pipelined bf16 GEMM has 256- and 128-feature tiles, chosen per shape
# (PLORA_GEMM_TILE_P forces one): the shapes below run under both.
TILE_WIDTHS = pytest.mark.parametrize("tile_p", ["256", "128"])


@TILE_WIDTHS
def test_bf16_multitile_full(P, tile_p, monkeypatch):
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    wl = workloads.custom(512, 768, [700, 5, 0, 395], [16, 8, 32, 64], [32.0, 16.0, 8.0, 16.0], "bf16",
                          seed=22, name="multitile_bf16")
    full_case(P, wl)


@TILE_WIDTHS
def test_bf16_pipelined_tails_full(P, tile_p, monkeypatch):
    # pipelined GEMMs (K % 128 == 0 both ways) with a feature tail in both
    # orientations (640 % 256 and % 128, 384 % 256) and a token tail (777 % 256)
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    wl = workloads.custom(384, 640, [100, 0, 513, 1, 163], [16, 8, 64, 32, 1], [32.0, 16.0, 8.0, 16.0, 4.0],
                          "bf16", seed=29, name="pipe_tails_bf16")
    full_case(P, wl)


def test_shrink_tile_rows_bitwise_equal(P, monkeypatch):
    """32- and 128-token shrink tiles, with and without K slices for every
    adapter, give each token row the same K order (four K quarters, each
    accumulated in order, added in order): equal bits in H, G and everything
    after them."""
    import torch
    wl = workloads.custom(512, 768, [100, 0, 513, 1, 163, 40], [16, 8, 64, 32, 1, 128],
                          [32.0, 16.0, 8.0, 16.0, 4.0, 256.0], "bf16", seed=32, name="shrink_tiles")
    log("case %s" % wl.name)
    inp = workloads.make_inputs(wl)
    dev = device_inputs(wl, inp)
    out = {}
    for rows in ("128", "32"):
        for split in ("0", "1"):
            monkeypatch.setenv("PLORA_SHRINK_TILE_ROWS", rows)
            monkeypatch.setenv("PLORA_SHRINK_SPLIT", split)
            out[rows + split] = run_gpu(P, wl, dev)
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    for v in ("1280", "320", "321"):
        for k in ("H", "G", "Y", "dX", "dA", "dB"):
            assert torch.equal(bits(out["1281"][k]), bits(out[v][k])), (v, k)


# (384, 704): pipelined forward with a feature tail at either width (704 % 256,
# 704 % 128); (712, 640): the same for the backward GEMM (d_in = 712).  817
# tokens: 4 token tiles (one group of 4); 1417: 6 (a group of 4 and one of 2).
@pytest.mark.parametrize("first", [100, 700])
@pytest.mark.parametrize("d_in,d_out", [(384, 704), (712, 640)])
def test_tile_widths_bitwise_equal(P, d_in, d_out, first, monkeypatch):
    """Both tile widths and both L2 group sizes of the tile map give every
    output element the same MFMA sequence: equal bits."""
    import torch
    wl = workloads.custom(d_in, d_out, [first, 0, 513, 1, 163, 40], [16, 8, 64, 32, 1, 128],
                          [32.0, 16.0, 8.0, 16.0, 4.0, 256.0], "bf16", seed=31, name="tile_widths")
    log("case %s" % wl.name)
    inp = workloads.make_inputs(wl)
    dev = device_inputs(wl, inp)
    out = {}
    for tile_p in ("256", "128"):
        for gq in ("2", "4"):
            monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
            monkeypatch.setenv("PLORA_GEMM_GROUP_Q", gq)
            out[tile_p + gq] = run_gpu(P, wl, dev)
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    for v in ("2564", "1282", "1284"):
        for k in ("Y", "dX"):
            assert torch.equal(bits(out["2562"][k]), bits(out[v][k])), (v, k)


@TILE_WIDTHS
def test_max_adapters_and_rank(P, tile_p, monkeypatch):
    # 64 adapters (the ABI maximum), ranks up to 128 (the maximum), empty and 1-token segments
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    n = 64
    counts = [(i * 37) % 97 if i % 9 else 0 for i in range(n)]
    counts[5] = 1
    ranks = [128 if i % 16 == 0 else (i % 8) * 8 + 1 for i in range(n)]
    alphas = [float(2 * r) for r in ranks]
    wl = workloads.custom(256, 512, counts, ranks, alphas, "bf16", seed=30, name="max_adapters")
    full_case(P, wl)


def test_f32_ragged_full(P):
    wl = workloads.custom(136, 72, [5, 0, 33, 70], [3, 7, 16, 64], [6.0, 7.0, 32.0, 16.0], "f32", seed=23,
                          name="ragged_f32")
    full_case(P, wl)


def test_single_token_segments_bf16(P):
    wl = workloads.custom(64, 64, [1] * 40, [(i % 5) * 16 + 1 for i in range(40)], [2.0] * 40, "bf16", seed=24,
                          name="one_token_bf16")
    full_case(P, wl)


def test_no_adapters(P):
    for dtype in ("bf16", "f32"):
        wl = workloads.custom(256, 520, [], [], [], dtype, seed=25, name="frozen_only_" + dtype)
        wl.offsets = np.array([0], np.int64)
        T = 300
        log("case %s T=%d" % (wl.name, T))
        inp = {"W": workloads.draw(25, 1, (520, 256), 1 / 16, dtype), "X": workloads.draw(25, 4, (T, 256), 1.0, dtype),
               "dY": workloads.draw(25, 5, (T, 520), 1.0, dtype)}
        d = P.Desc([0], [], [], 256, 520, dtype, n_tokens=T)
        dev = device_inputs(wl, inp)
        import torch
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        Y = torch.full((T, 520), float("nan"), dtype=tdt, device="cuda")
        dX = torch.full((T, 256), float("nan"), dtype=tdt, device="cuda")
        P.plora_forward(d, dev["X"], dev["W"], None, None, Y, None)
        P.plora_backward_dx(d, dev["dY"], dev["W"], None, None, dX, None)
        torch.cuda.synchronize()
        ref = oracle.packed_lora([0], [], [], 256, 520, X=inp["X"], dY=inp["dY"], W=inp["W"], want=("Y", "dX"), T=T)
        check_block(host(Y), ref["Y"], TOL[dtype], "Y")
        check_block(host(dX), ref["dX"], TOL[dtype], "dX")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_tokens_dAdB(P, dtype):
    """T = 0 with adapters: every segment is empty, so dA_i = dB_i = 0 (the sums
    over S_i are empty); overwrite writes the zeros, accumulate leaves the
    gradients as they were.  Forward and dX touch nothing."""
    import torch
    log("case zero_tokens_dAdB dtype=%s" % dtype)
    ranks, d_in, d_out = [4, 64, 16], 256, 320
    d = P.Desc([0, 0, 0, 0], ranks, [1.0, 8.0, 2.0], d_in, d_out, dtype)
    R = sum(ranks)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    X = torch.empty((0, d_in), dtype=tdt, device="cuda")
    dY = torch.empty((0, d_out), dtype=tdt, device="cuda")
    H = torch.empty((0,), dtype=torch.float32, device="cuda")
    G = torch.empty((0,), dtype=torch.float32, device="cuda")
    Y = torch.empty((0, d_out), dtype=tdt, device="cuda")
    W = torch.zeros((d_out, d_in), dtype=tdt, device="cuda")
    A = torch.zeros((R, d_in), dtype=tdt, device="cuda")
    B = torch.zeros((R, d_out), dtype=tdt, device="cuda")
    P.plora_forward(d, X, W, A, B, Y, H)
    assert P.plora_h_elems(d) == 0
    ws_bytes = P.plora_workspace_bytes(d)
    for ws in (None, torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device="cuda")):
        dA = torch.full((R, d_in), float("nan"), dtype=torch.float32, device="cuda")
        dB = torch.full((R, d_out), float("nan"), dtype=torch.float32, device="cuda")
        P.plora_backward_dAdB(d, X, dY, H, G, dA, dB, ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dA).item() == 0 and torch.count_nonzero(dB).item() == 0
        kA = torch.arange(R * d_in, dtype=torch.float32, device="cuda").reshape(R, d_in)
        kB = torch.arange(R * d_out, dtype=torch.float32, device="cuda").reshape(R, d_out)
        dA.copy_(kA)
        dB.copy_(kB)
        P.plora_backward_dAdB(d, X, dY, H, G, dA, dB, ws, accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(dA, kA) and torch.equal(dB, kB)


# ---------------------------------------------------------------------------
# exact cases
# ---------------------------------------------------------------------------

def rank1_inputs(counts, d_in, d_out, seed):
    rng = np.random.default_rng(seed)
    N = len(counts)
    T = int(sum(counts))
    ks = rng.choice(d_in, size=N, replace=False)
    svals = np.array([2.0 ** (i % 3) for i in range(N)], np.float32)
    c = np.arange(1, N + 1, dtype=np.float32)
    A = np.zeros((N, d_in), np.float32)
    A[np.arange(N), ks] = 1.0
    B = np.repeat(c[:, None], d_out, axis=1).astype(np.float32)
    X = rng.integers(0, 2, size=(T, d_in)).astype(np.float32)
    dY = np.zeros((T, d_out), np.float32)
    dY[np.arange(T), rng.integers(0, d_out, size=T)] = 1.0
    W = np.zeros((d_out, d_in), np.float32)
    return dict(W=W, A=A, B=B, X=X, dY=dY), svals


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rank1_indexing_exact(P, dtype):
    """Rank-1 adapters A_i = e_{k_i}, B_i = (i+1) 1^T, power-of-2 scales, 0/1 inputs:
    every output is a small integer times a power of 2, exact in bf16 and fp32, so
    the GPU must match the oracle bit for bit; a row assigned to the wrong adapter
    would show the wrong (i+1)."""
    counts = [37, 0, 1, 300, 256, 0, 255, 2, 64, 33]
    inp, svals = rank1_inputs(counts, 136, 264, 5)
    wl = workloads.custom(136, 264, counts, [1] * len(counts), svals, dtype, name="rank1_" + dtype)
    log("case %s" % wl.name)
    gpu = gpu_host(run_gpu(P, wl, device_inputs(wl, inp)))
    ref = oracle.run_workload(wl, inp)
    for k in ("Y", "H", "dX", "G", "dA", "dB"):
        assert np.array_equal(gpu[k], ref[k]), k


# (d_in, d_out): general kernels (K not a multiple of 128) and pipelined kernels
SHAPES = [(320, 264), (512, 768)]


@pytest.mark.parametrize("d_in,d_out", SHAPES)
def test_b_zero_matches_frozen_path_bitwise(P, d_in, d_out):
    """B = 0 (LoRA's initial state): Y and dX equal the N = 0 results bit for bit,
    G and dA are exactly zero."""
    import torch
    wl = workloads.custom(d_in, d_out, [100, 0, 300, 7], [8, 16, 64, 128], [16.0, 32.0, 8.0, 256.0], "bf16",
                          seed=26, name="bzero")
    log("case %s" % wl.name)
    inp = workloads.make_inputs(wl)
    inp["B"] = np.zeros_like(inp["B"])
    dev = device_inputs(wl, inp)
    gpu = run_gpu(P, wl, dev)
    d0 = P.Desc([0], [], [], wl.d_in, wl.d_out, "bf16", n_tokens=wl.T)
    Y0 = torch.empty_like(gpu["Y"])
    dX0 = torch.empty_like(gpu["dX"])
    P.plora_forward(d0, dev["X"], dev["W"], None, None, Y0, None)
    P.plora_backward_dx(d0, dev["dY"], dev["W"], None, None, dX0, None)
    torch.cuda.synchronize()
    assert torch.equal(gpu["Y"].view(torch.int16), Y0.view(torch.int16))
    assert torch.equal(gpu["dX"].view(torch.int16), dX0.view(torch.int16))
    assert torch.count_nonzero(gpu["G"]).item() == 0
    assert torch.count_nonzero(gpu["dA"]).item() == 0
    assert torch.count_nonzero(gpu["dB"]).item() > 0


def test_reproducible_bitwise(P):
    import torch
    wl = workloads.custom(512, 768, [3000, 0, 1100, 5], [16, 8, 64, 32], [32.0, 16.0, 8.0, 16.0], "bf16",
                          seed=27, name="repro")
    log("case %s" % wl.name)
    dev = device_inputs(wl, workloads.make_inputs(wl))
    a = run_gpu(P, wl, dev)
    b = run_gpu(P, wl, dev)
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k].view(torch.int32),
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k].view(torch.int32)), k


@pytest.mark.parametrize("d_in,d_out", [(320, 1032), (512, 768)])
@TILE_WIDTHS
def test_packed_equals_separate_bitwise(P, d_in, d_out, tile_p, monkeypatch):
    """The packed call gives each adapter exactly what a call with that adapter alone gives."""
    import torch
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    wl = workloads.custom(d_in, d_out, [129, 0, 2200, 31, 600], [16, 8, 64, 1, 33], [32.0, 16.0, 8.0, 2.0, 66.0],
                          "bf16", seed=28, name="packed_vs_separate")
    log("case %s" % wl.name)
    inp = workloads.make_inputs(wl)
    dev = device_inputs(wl, inp)
    packed = run_gpu(P, wl, dev)
    for i, rows, rr, hs, r, n in h_blocks(wl):
        if n == 0:
            continue
        one = workloads.custom(wl.d_in, wl.d_out, [n], [r], [wl.alphas[i]], "bf16", name="one")
        dev1 = {"W": dev["W"], "A": dev["A"][rr].contiguous(), "B": dev["B"][rr].contiguous(),
                "X": dev["X"][rows].contiguous(), "dY": dev["dY"][rows].contiguous()}
        sep = run_gpu(P, one, dev1)
        bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
        assert torch.equal(bits(packed["Y"][rows]), bits(sep["Y"])), i
        assert torch.equal(bits(packed["dX"][rows]), bits(sep["dX"])), i
        assert torch.equal(bits(packed["H"][hs]), bits(sep["H"])), i
        assert torch.equal(bits(packed["G"][hs]), bits(sep["G"])), i
        assert torch.equal(bits(packed["dA"][rr]), bits(sep["dA"])), i
        assert torch.equal(bits(packed["dB"][rr]), bits(sep["dB"])), i


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows + every adapter's dA/dB in full
# ---------------------------------------------------------------------------

def sampled_case(P, wl, per_segment=4):
    import torch
    log("case %s T=%d d_in=%d d_out=%d N=%d" % (wl.name, wl.T, wl.d_in, wl.d_out, wl.n_adapters))
    inp = workloads.make_inputs(wl)
    gpu = run_gpu(P, wl, device_inputs(wl, inp))
    tol = TOL[wl.dtype]
    rows = workloads.sample_rows(wl, per_segment=per_segment)
    ref = oracle.rows_subproblem(wl, inp, rows, want=("Y", "dX", "H", "G"))
    rows_t = torch.from_numpy(rows).to("cuda")
    Yg, dXg = host(gpu["Y"][rows_t]), host(gpu["dX"][rows_t])
    seg = np.searchsorted(wl.offsets, rows, side="right") - 1
    hoff = np.concatenate([[0], np.cumsum(np.diff(wl.offsets) * wl.ranks)])
    Hg, Gg = host(gpu["H"]), host(gpu["G"])
    for i in np.unique(seg):
        m = seg == i
        check_block(Yg[m], ref["Y"][m], tol, "Y rows of segment %d" % i)
        check_block(dXg[m], ref["dX"][m], tol, "dX rows of segment %d" % i)
    # every adapter: H, G, dA, dB in full (the oracle on that adapter's slice)
    dA, dB = host(gpu["dA"]), host(gpu["dB"])
    for i, rws, rr, hs, r, n in h_blocks(wl):
        one = oracle.packed_lora([0, n], [r], [float(wl.alphas[i])], wl.d_in, wl.d_out, X=inp["X"][rws],
                                 dY=inp["dY"][rws], A=inp["A"][rr], B=inp["B"][rr], want=("H", "G", "dA", "dB"))
        for k, g in (("H", Hg[hs]), ("G", Gg[hs]), ("dA", dA[rr]), ("dB", dB[rr])):
            check_block(g, one[k], tol_of(wl.dtype, k), "%s[adapter %d]" % (k, i))
    del gpu
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_qwen_q_proj(P):
    sampled_case(P, workloads.config("qwen_q"))


@pytest.mark.slow
def test_llama_up_32_adapters(P):
    """The benchmark's workload: 4096 -> 14336, 32 adapters x 2048 tokens."""
    sampled_case(P, workloads.config("llama_up"), per_segment=2)


@pytest.mark.slow
def test_longtail(P):
    sampled_case(P, workloads.config("longtail"))


@pytest.mark.slow
def test_llama_sq_2_adapters(P):
    sampled_case(P, workloads.config("llama_sq", n_adapters=2))


@pytest.mark.slow
@pytest.mark.parametrize("proj", ["k", "down"])
def test_block_projection(P, proj):
    sampled_case(P, workloads.config("block_" + proj, n_adapters=8), per_segment=2)


@pytest.mark.parametrize("name", ["decode_sq", "decode_up"])
def test_decode_shapes_full(P, name):
    """Serving shapes: 64 adapters with 1 to 16 tokens each (many adapters
    per token tile), compared in full (forward only is what serving runs; the
    backward is covered too)."""
    full_case(P, workloads.config(name))


@pytest.mark.slow
def test_mixed_tile_widths_bitwise_equal(P, monkeypatch):
    """qwen_q-sized GEMMs (64 x 14 = 896 tiles of 256 x 256, 3.5 waves on 256
    compute units) run as 256-wide tiles over part of the features and
    128-wide tiles over the rest, in two launches: the result equals a single
    width bit for bit (each output element sees the same MFMA sequence)."""
    import torch
    wl = workloads.config("qwen_q")
    log("case %s T=%d (mixed tile widths)" % (wl.name, wl.T))
    dev = device_inputs(wl, workloads.make_inputs(wl))
    out = {}
    for mode in ("", "256", "128"):
        if mode:
            monkeypatch.setenv("PLORA_GEMM_TILE_P", mode)
        else:
            monkeypatch.delenv("PLORA_GEMM_TILE_P", raising=False)
        out[mode] = run_gpu(P, wl, dev, want=("fwd", "dx"))
    for mode in ("256", "128"):
        for k in ("Y", "dX"):
            assert torch.equal(out[""][k].view(torch.int16), out[mode][k].view(torch.int16)), (mode, k)


@pytest.mark.parametrize("d_in,d_out", [(512, 768), (4096, 1024)])
def test_wgrad_widths_bitwise_equal(P, d_in, d_out, monkeypatch):
    """128- and 256-feature weight-gradient workgroups give every dA/dB element
    the same token sum (the feature tiling does not touch it): equal bits,
    with multi-chunk adapters (partials and their reduction), a feature tail
    and ranks up to 64 (and up to 32)."""
    import torch
    for ranks in ([16, 8, 64, 32, 1, 33], [16, 8, 32, 32, 1, 24]):
        wl = workloads.custom(d_in, d_out, [1500, 0, 513, 1, 2300, 40], ranks, [32.0, 16.0, 8.0, 16.0, 4.0, 66.0],
                              "bf16", seed=33, name="wgrad_widths")
        log("case %s %dx%d ranks %s" % (wl.name, d_in, d_out, ranks))
        dev = device_inputs(wl, workloads.make_inputs(wl))
        out = {}
        for cols in ("256", "128"):
            monkeypatch.setenv("PLORA_WGRAD_COLS", cols)
            out[cols] = run_gpu(P, wl, dev)
        for k in ("dA", "dB"):
            assert torch.equal(out["256"][k].view(torch.int32), out["128"][k].view(torch.int32)), k
