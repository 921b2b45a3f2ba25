"""GPU parity of the decoder-block kernels through the C ABI against the fp64
oracle (oracle/block.py), on the same bf16 inputs.

Tolerances: each kernel rounds its outputs to bf16 once (relative 2^-9), and
attention additionally rounds the softmax weights to bf16 before the product
with V, so outputs are compared blockwise at 1e-2 (rmsnorm, rope, swiglu,
add) and 2e-2 (attention), with the same two-part criterion as the operator
(Frobenius and elementwise)."""
import numpy as np
import pytest

import workloads
from oracle import block as OB
from parity_utils import check_block, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def bf(shape, seed, tid, std=1.0):
    """Seeded bf16-representable fp32 values."""
    return workloads.draw(seed, tid, shape, std, "bf16")


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)


def dev32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def rnd(a):
    """Round to bf16 (what a kernel stores)."""
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(a, np.float32))).reshape(np.shape(a))


@pytest.mark.parametrize("D", [4096, 328, 6000, 10000])
def test_rmsnorm_fwd(P, D):
    import torch
    T = 77
    x, r, w = bf((T, D), 61, 1), bf((T, D), 61, 2, 0.5), bf((1, D), 61, 3)[0]
    h = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    xs = torch.full_like(h, float("nan"))
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    P.plora_rmsnorm_fwd(dev(x), dev(w), h, rstd, res=dev(r), xs_out=xs, eps=1e-5)
    torch.cuda.synchronize()
    xs_ref = x.astype(np.float64) + r  # exact in fp64; the kernel stores it rounded to bf16
    np.testing.assert_array_equal(host(xs), rnd(xs_ref))
    h_ref, rstd_ref = OB.rmsnorm_fwd(rnd(xs_ref), w, 1e-5)
    check_block(host(h), h_ref, 1e-2, "h")
    np.testing.assert_allclose(host(rstd), rstd_ref, rtol=1e-5)
    # without the residual
    P.plora_rmsnorm_fwd(dev(x), dev(w), h, rstd, eps=1e-5)
    torch.cuda.synchronize()
    check_block(host(h), OB.rmsnorm_fwd(x, w, 1e-5)[0], 1e-2, "h (no residual)")


@pytest.mark.parametrize("D", [4096, 328, 10000])
def test_rmsnorm_bwd(P, D):
    import torch
    T = 65
    x, w = bf((T, D), 62, 1), bf((1, D), 62, 2)[0]
    dys = [bf((T, D), 62, 3 + k, 0.1) for k in range(3)]
    dres = bf((T, D), 62, 7, 0.1)
    _, rstd = OB.rmsnorm_fwd(x, w, 1e-5)
    rstd32 = rstd.astype(np.float32)
    dx = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    P.plora_rmsnorm_bwd([dev(d) for d in dys], dev(x), dev(w), dev32(rstd32), dx, dres=dev(dres))
    torch.cuda.synchronize()
    ref = dres + OB.rmsnorm_bwd(dys[0].astype(np.float64) + dys[1] + dys[2], x, w, rstd32.astype(np.float64))
    check_block(host(dx), ref, 1e-2, "dx")
    P.plora_rmsnorm_bwd([dev(dys[0])], dev(x), dev(w), dev32(rstd32), dx)
    torch.cuda.synchronize()
    check_block(host(dx), OB.rmsnorm_bwd(dys[0], x, w, rstd32.astype(np.float64)), 1e-2, "dx (one gradient)")


@pytest.mark.parametrize("inverse", [False, True])
def test_rope(P, inverse):
    import torch
    offs = [0, 1, 300, 300, 1100]
    T, heads = offs[-1], 8
    x = bf((T, heads * 128), 63, 1)
    xd = dev(x)
    P.plora_rope(xd, offs, heads, base=500000.0, inverse=inverse)
    torch.cuda.synchronize()
    pos = OB.positions_of(offs)
    ref = OB.rope_bwd(x, pos) if inverse else OB.rope_fwd(x, pos)
    check_block(host(xd), ref, 1e-2, "rope")


def test_swiglu_and_add(P):
    import torch
    n = (37, 1000)
    g, u, da = bf(n, 64, 1, 3.0), bf(n, 64, 2), bf(n, 64, 3)
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    P.plora_swiglu_fwd(dev(g), dev(u), a)
    dg, du = torch.empty_like(a), torch.empty_like(a)
    P.plora_swiglu_bwd(dev(da), dev(g), dev(u), dg, du)
    out = torch.empty_like(a)
    P.plora_add(dev(g), dev(u), out)
    torch.cuda.synchronize()
    check_block(host(a), OB.swiglu_fwd(g, u), 1e-2, "swiglu")
    rg, ru = OB.swiglu_bwd(da, g, u)
    check_block(host(dg), rg, 1e-2, "dg")
    check_block(host(du), ru, 1e-2, "du")
    np.testing.assert_array_equal(host(out), rnd(g.astype(np.float64) + u))


# (768, 512): pipelined GEMM (fused epilogue) at both tile widths, a ragged
# token tail, K-sliced shrinks (adapters of <= 128 tokens use dg as scratch);
# (712, 512): a feature tail (712 = 2 x 256 + 200) in the fused epilogue;
# (768, 264): K = 264 is off the pipelined path (GEMM, then the SwiGLU kernel
# in place); n_adapters = 0: the frozen GEMM alone
@pytest.mark.parametrize("d_mlp,d_hid,tile_p,frozen", [(768, 512, "256", False), (768, 512, "128", False),
                                                       (712, 512, "256", False), (712, 512, "128", False),
                                                       (768, 264, "256", False), (768, 512, "256", True)])
def test_backward_dx_swiglu_fused(P, d_mlp, d_hid, tile_p, frozen, monkeypatch):
    """plora_backward_dx_swiglu writes bitwise what plora_backward_dx followed
    by plora_swiglu_bwd writes (dg, du and G), and the oracle's SwiGLU
    backward of the oracle's dX within the bf16 tolerance."""
    import torch
    import oracle
    from parity_utils import to_dev
    monkeypatch.setenv("PLORA_GEMM_TILE_P", tile_p)
    wl = workloads.custom(d_mlp, d_hid, [300, 0, 64, 1, 335], [16, 8, 64, 32, 1], [32.0, 16.0, 8.0, 16.0, 4.0],
                          "bf16", seed=81, name="dx_swiglu")
    log("case %s d_mlp=%d d_hid=%d tile_p=%s frozen=%s" % (wl.name, d_mlp, d_hid, tile_p, frozen))
    inp = workloads.make_inputs(wl)
    d = P.Desc([0], [], [], d_mlp, d_hid, "bf16", n_tokens=wl.T) if frozen else P.Desc.from_workload(wl)
    T = wl.T
    dY, W = to_dev(inp["dY"], "bf16"), to_dev(inp["W"], "bf16")
    A = None if frozen else to_dev(inp["A"], "bf16")
    B = None if frozen else to_dev(inp["B"], "bf16")
    g, u = bf((T, d_mlp), 82, 1, 3.0), bf((T, d_mlp), 82, 2)
    gd, ud = dev(g), dev(u)
    he = P.plora_h_elems(d)
    nan = lambda *shape: torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    G0 = torch.full((max(he, 4),), float("nan"), device="cuda")[:he] if he else None
    G1 = torch.full((max(he, 4),), float("nan"), device="cuda")[:he] if he else None
    dX, dg0, du0 = nan(T, d_mlp), nan(T, d_mlp), nan(T, d_mlp)
    P.plora_backward_dx(d, dY, W, A, B, dX, G0)
    P.plora_swiglu_bwd(dX, gd, ud, dg0, du0)
    dg1, du1 = nan(T, d_mlp), nan(T, d_mlp)
    P.plora_backward_dx_swiglu(d, dY, W, A, B, gd, ud, dg1, du1, G1)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    assert torch.equal(bits(dg1), bits(dg0)), "dg"
    assert torch.equal(bits(du1), bits(du0)), "du"
    if he:
        assert torch.equal(G1.view(torch.int32), G0.view(torch.int32)), "G"
    # against the oracle: its dX (fp64), rounded to bf16 as the GEMM stores it,
    # through its SwiGLU backward
    if frozen:
        dx_ref = inp["dY"].astype(np.float64) @ inp["W"].astype(np.float64)
    else:
        dx_ref = oracle.run_workload(wl, inp)["dX"]
    rg, ru = OB.swiglu_bwd(rnd(dx_ref), g, u)
    check_block(host(dg1), rg, 2e-2, "dg")
    check_block(host(du1), ru, 2e-2, "du")


def attn_inputs(offs, n_q, n_kv, seed):
    T = offs[-1]
    return bf((T, n_q * 128), seed, 1), bf((T, n_kv * 128), seed, 2), bf((T, n_kv * 128), seed, 3)


def check_attention_out(got, ref, offs, n_q, name, tol=2e-2, elementwise=True):
    # blocks whose exact value vanishes (a one-token sequence's dQ) are measured
    # against 1e-3 of the whole output's rms
    floor = 1e-3 * float(np.sqrt(np.mean(np.square(ref))))
    for s, (a, b) in enumerate(zip(offs[:-1], offs[1:])):
        for j in range(n_q):
            hs = slice(j * 128, (j + 1) * 128)
            check_block(got[a:b, hs], ref[a:b, hs], tol, "%s[seq %d, head %d]" % (name, s, j), floor_rms=floor,
                        elementwise=elementwise)


# (the last case has one long and three one-token sequences: its work items
# run sequence by sequence; the others run in rank order)
@pytest.mark.parametrize("offs,n_q,n_kv", [([0, 1, 65, 200, 333], 8, 2), ([0, 1024, 2048], 32, 8),
                                          ([0, 100, 230], 16, 2), ([0, 64, 64, 127, 128], 4, 1),
                                          ([0, 700, 701, 702, 703], 8, 2), ([0, 2500], 8, 2)])
def test_attention_fwd(P, offs, n_q, n_kv):
    import torch
    log("attention fwd offs=%s n_q=%d n_kv=%d" % (offs, n_q, n_kv))
    T = offs[-1]
    q, k, v = attn_inputs(offs, n_q, n_kv, 65)
    o = torch.full((T, n_q * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((n_q, T), float("nan"), dtype=torch.float32, device="cuda")
    P.plora_attention_fwd(dev(q), dev(k), dev(v), o, lse, offs, n_q, n_kv)
    torch.cuda.synchronize()
    o_ref, lse_ref = OB.attention_fwd(q, k, v, offs, n_q, n_kv)
    check_attention_out(host(o), o_ref, offs, n_q, "o")
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("offs,n_q,n_kv", [([0, 1, 65, 200, 333], 8, 2), ([0, 1024, 2048], 32, 8),
                                          ([0, 100, 230], 16, 2), ([0, 64, 64, 127, 128], 4, 1),
                                          ([0, 700, 701, 702, 703], 8, 2), ([0, 2500], 8, 2)])
def test_attention_bwd(P, offs, n_q, n_kv):
    import torch
    log("attention bwd offs=%s n_q=%d n_kv=%d" % (offs, n_q, n_kv))
    T = offs[-1]
    q, k, v = attn_inputs(offs, n_q, n_kv, 66)
    dO = bf((T, n_q * 128), 66, 4)
    o_ref, lse_ref = OB.attention_fwd(q, k, v, offs, n_q, n_kv)
    o16 = rnd(o_ref)                          # the forward's stored output
    lse32 = lse_ref.astype(np.float32)        # and its fp32 statistics
    outs = [torch.full((T, n * 128), float("nan"), dtype=torch.bfloat16, device="cuda") for n in (n_q, n_kv, n_kv)]
    delta = torch.full((n_q, T), float("nan"), dtype=torch.float32, device="cuda")
    P.plora_attention_bwd(dev(q), dev(k), dev(v), dev(o16), dev32(lse32), dev(dO), *outs, delta, offs, n_q, n_kv)
    torch.cuda.synchronize()
    refs = OB.attention_bwd(dO, q, k, v, o16, lse32.astype(np.float64), offs, n_q, n_kv)
    bounds = bwd_rounding_bounds(q, k, v, dO, o16, lse32.astype(np.float64), offs, n_q, n_kv)
    for name, got, ref, nh, bd in zip(("dq", "dk", "dv"), outs, refs, (n_q, n_kv, n_kv), bounds):
        got = host(got)
        # Frobenius per block as for every kernel ...
        check_attention_out(got, ref, offs, nh, name, elementwise=False)
        # ... and elementwise against the rounding model: the kernel feeds P and dS
        # to the matrix cores as bf16 (relative 2^-9 each), so an element may be
        # off by 2^-9 * sum |dS| |K| (dq), sum |dS| |Q| (dk), sum P |dO| (dv),
        # plus the fp32 rounding of S, dP and delta (bwd_rounding_bounds) and its
        # own bf16 rounding; twice that is allowed
        err = np.abs(got - ref)
        lim = 2.0 * (bd + 2.0 ** -9 * np.abs(ref)) + 1e-6
        assert np.all(err <= lim), "%s: %d elements beyond the rounding bound; worst ratio %.2f" % (
            name, int(np.sum(err > lim)), float(np.max(err / lim)))


def bwd_rounding_bounds(q, k, v, dO, o, lse, offs, n_q, n_kv):
    """Per-element size of the bf16 rounding of P and dS in the backward
    products: 2^-9 * (|dS| @ |K|, |dS|^T @ |Q|, P^T @ |dO|), plus the fp32
    rounding of the length-128 dot products behind them (at most
    gamma_128 ~ 2^-17 of the sum of |terms|): the score (an absolute error in
    the exponent, so relative in P) and dP - delta (absolute, which matters
    where dP ~ delta and dS itself is small), in fp64."""
    scale, grp = 1.0 / np.sqrt(128.0), n_q // n_kv
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for a, b in zip(offs[:-1], offs[1:]):
        if b == a:
            continue
        mask = np.tril(np.ones((b - a, b - a), bool))
        for j in range(n_q):
            hs, gs = slice(j * 128, (j + 1) * 128), slice((j // grp) * 128, (j // grp + 1) * 128)
            Q, K, V = (x.astype(np.float64) for x in (q[a:b, hs], k[a:b, gs], v[a:b, gs]))
            dOh, Oh = dO[a:b, hs].astype(np.float64), o[a:b, hs].astype(np.float64)
            Pm = np.where(mask, np.exp(Q @ K.T * scale - lse[j, a:b][:, None]), 0.0)
            dS = Pm * (dOh @ V.T - np.sum(dOh * Oh, axis=1, keepdims=True))
            es = 2.0 ** -17 * scale * (np.abs(Q) @ np.abs(K).T)
            ed = 2.0 ** -17 * (np.abs(dOh) @ np.abs(V).T + np.sum(np.abs(dOh * Oh), axis=1, keepdims=True))
            dS_err = 2.0 ** -9 * np.abs(dS) + Pm * ed + np.abs(dS) * es
            bq[a:b, hs] += scale * dS_err @ np.abs(K)
            bk[a:b, gs] += scale * dS_err.T @ np.abs(Q)
            bv[a:b, gs] += (2.0 ** -9 * Pm + Pm * es).T @ np.abs(dOh)
    return bq, bk, bv


@pytest.mark.slow
def test_attention_full_size_32_sequences(P):
    """Attention forward and backward at the decoder block's full size: 32
    sequences of 1024 tokens, 32 query / 8 key-value heads (the work order of
    many sequences), checked per kernel, as above, on three sampled sequences
    (each sequence's attention depends on its own rows only)."""
    import torch
    n_q, n_kv, L, n = 32, 8, 1024, 32
    offs = [i * L for i in range(n + 1)]
    T = offs[-1]
    log("attention fwd+bwd %d sequences x %d tokens, heads %d/%d" % (n, L, n_q, n_kv))
    q, k, v = attn_inputs(offs, n_q, n_kv, 68)
    dO = bf((T, n_q * 128), 68, 4)
    o = torch.full((T, n_q * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((n_q, T), float("nan"), dtype=torch.float32, device="cuda")
    P.plora_attention_fwd(dev(q), dev(k), dev(v), o, lse, offs, n_q, n_kv)
    outs = [torch.full((T, nh * 128), float("nan"), dtype=torch.bfloat16, device="cuda") for nh in (n_q, n_kv, n_kv)]
    delta = torch.full((n_q, T), float("nan"), dtype=torch.float32, device="cuda")
    # the backward from the GPU's own forward outputs (o, lse)
    P.plora_attention_bwd(dev(q), dev(k), dev(v), o, lse, dev(dO), *outs, delta, offs, n_q, n_kv)
    torch.cuda.synchronize()
    o_h, lse_h = host(o), host(lse)
    outs_h = [host(t) for t in outs]
    for sq in (0, 13, 31):
        a, b = offs[sq], offs[sq + 1]
        log("sequence %d" % sq)
        one = [0, L]
        o_ref, lse_ref = OB.attention_fwd(q[a:b], k[a:b], v[a:b], one, n_q, n_kv)
        check_attention_out(o_h[a:b], o_ref, one, n_q, "o[seq %d]" % sq)
        np.testing.assert_allclose(lse_h[:, a:b], lse_ref, rtol=1e-5, atol=1e-4)
        refs = OB.attention_bwd(dO[a:b], q[a:b], k[a:b], v[a:b], o_h[a:b], lse_h[:, a:b], one, n_q, n_kv)
        bounds = bwd_rounding_bounds(q[a:b], k[a:b], v[a:b], dO[a:b], o_h[a:b], lse_h[:, a:b], one, n_q, n_kv)
        for name, got, ref, nh, bd in zip(("dq", "dk", "dv"), outs_h, refs, (n_q, n_kv, n_kv), bounds):
            got = got[a:b]
            check_attention_out(got, ref, one, nh, "%s[seq %d]" % (name, sq), elementwise=False)
            err = np.abs(got - ref)
            lim = 2.0 * (bd + 2.0 ** -9 * np.abs(ref)) + 1e-6
            assert np.all(err <= lim), "%s[seq %d]: %d elements beyond the rounding bound; worst ratio %.2f" % (
                name, sq, int(np.sum(err > lim)), float(np.max(err / lim)))


def block_params(hidden, n_q, n_kv, mlp, ranks, seed):
    import torch
    from packed_adapter_lora_amd.block import proj_dims
    dims = proj_dims(hidden, n_q, n_kv, mlp)
    R = int(sum(ranks))
    host_p = {"w1": 1.0 + bf((1, hidden), seed, 1, 0.1)[0], "w2": 1.0 + bf((1, hidden), seed, 2, 0.1)[0],
              "W": {}, "A": {}, "B": {}, "dims": dims, "n_q": n_q, "n_kv": n_kv}
    host_p["w1"], host_p["w2"] = rnd(host_p["w1"]), rnd(host_p["w2"])
    for i, (n, (di, do)) in enumerate(sorted(dims.items())):
        host_p["W"][n] = bf((do, di), seed, 10 + i, 1.0 / np.sqrt(di))
        host_p["A"][n] = bf((R, di), seed, 20 + i, 0.25)
        host_p["B"][n] = bf((R, do), seed, 30 + i, 0.1)
    devp = {"w1": dev(host_p["w1"]), "w2": dev(host_p["w2"]),
            "W": {n: dev(v) for n, v in host_p["W"].items()}, "A": {n: dev(v) for n, v in host_p["A"].items()},
            "B": {n: dev(v) for n, v in host_p["B"].items()}}
    return host_p, devp


def test_decoder_block_fwd_bwd(P):
    import torch
    from packed_adapter_lora_amd.block import DecoderBlock, PROJ
    hidden, n_q, n_kv, mlp = 512, 4, 1, 384
    ranks, alphas = [8, 16, 4], [16.0, 16.0, 8.0]
    seg, seq = [0, 150, 150, 256], [0, 100, 150, 256]
    T = seg[-1]
    log("decoder block T=%d hidden=%d heads=%d/%d mlp=%d" % (T, hidden, n_q, n_kv, mlp))
    hp, dp = block_params(hidden, n_q, n_kv, mlp, ranks, 67)
    x, dout = bf((T, hidden), 67, 90), bf((T, hidden), 67, 91)
    blk = DecoderBlock(dp, seg, ranks, alphas, seq, hidden=hidden, n_q=n_q, n_kv=n_kv, mlp=mlp)
    out = blk.forward(dev(x))
    dx, grads = blk.backward(dev(dout))
    torch.cuda.synchronize()
    hp["ranks"], hp["alphas"] = np.array(ranks), np.array(alphas)
    ref_out, cache = OB.block_forward(hp, x, seg, seq, store=rnd)
    ref_dx, ref_grads = OB.block_backward(hp, cache, dout, seg, seq, store=rnd)
    # This test checks the wiring of a chain of ~10 (forward) and ~25
    # (backward) kernels, each verified alone above.  Each rounds to bf16; the
    # oracle rounds at the same points, but a one-ulp difference at one step
    # propagates, so tails of the elementwise error reach ~10 % of the rms
    # while the Frobenius error stays below 1 %.  Held to: Frobenius 2e-2 and
    # elementwise 2e-2 |ref| + 0.15 rms(ref); a wiring mistake (wrong buffer,
    # order or fusion) is off by O(1).
    def chain(got, ref, name):
        got, ref = host(got), np.asarray(ref, np.float64)
        check_block(got, ref, 2e-2, name, elementwise=False)
        rms = float(np.sqrt(np.mean(ref * ref)))
        err = np.abs(got - ref)
        lim = 2e-2 * np.abs(ref) + 0.15 * rms
        log("%s: rel Frobenius %.2e, worst elementwise %.2f of the bound" % (
            name, np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30), float(np.max(err / lim))))
        assert np.all(err <= lim), "%s: %d elements beyond the chained-rounding bound" % (name, int(np.sum(err > lim)))

    chain(out, ref_out, "out")
    chain(dx, ref_dx, "dx")
    for n in PROJ:
        chain(grads[n][0], ref_grads[n][0], "dA[%s]" % n)
        chain(grads[n][1], ref_grads[n][1], "dB[%s]" % n)


# ---------------------------------------------------------------------------
# The decoder block at its full size: hidden 4096, 32 query / 8 key-value
# heads, MLP 14336, 32 adapters (ranks cycling 8..64) of 1024 tokens each, one
# sequence per adapter.  Attention stays inside a sequence and every other
# kernel is row-wise, so a sequence's output and input-gradient rows and its
# adapter's dA/dB on every projection depend on that sequence alone: the fp64
# oracle runs on one sequence (as a one-adapter problem with that adapter's
# A/B rows) and is compared with those rows and gradients of the full-size GPU
# run.
# ---------------------------------------------------------------------------

FULL = dict(hidden=4096, n_q=32, n_kv=8, mlp=14336, n=32, L=1024, seed=71)


def chained_check(got, ref, name, elementwise=True):
    """The chained-rounding bound of test_decoder_block_fwd_bwd: Frobenius
    2e-2 and elementwise 2e-2 |ref| + 0.15 rms(ref)."""
    got = host(got) if hasattr(got, "detach") else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    check_block(got, ref, 2e-2, name, elementwise=False)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    lim = 2e-2 * np.abs(ref) + 0.15 * rms
    if not elementwise:
        log("%s: rel Frobenius %.2e (elementwise: link by link below)" % (
            name, np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)))
        return
    log("%s: rel Frobenius %.2e, worst elementwise %.2f of the bound" % (
        name, np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30), float(np.max(err / lim))))
    assert np.all(err <= lim), "%s: %d elements beyond the chained-rounding bound" % (name, int(np.sum(err > lim)))


@pytest.fixture(scope="module")
def full_block(P):
    import torch
    from packed_adapter_lora_amd.block import DecoderBlock
    f = FULL
    ranks = [(8, 16, 32, 64)[i % 4] for i in range(f["n"])]
    alphas = [(8.0, 16.0, 32.0)[i % 3] for i in range(f["n"])]
    off = [i * f["L"] for i in range(f["n"] + 1)]
    T = off[-1]
    log("full-size decoder block T=%d hidden=%d heads=%d/%d mlp=%d adapters=%d" % (
        T, f["hidden"], f["n_q"], f["n_kv"], f["mlp"], f["n"]))
    hp, dp = block_params(f["hidden"], f["n_q"], f["n_kv"], f["mlp"], ranks, f["seed"])
    x, dout = bf((T, f["hidden"]), f["seed"], 90), bf((T, f["hidden"]), f["seed"], 91)
    blk = DecoderBlock(dp, off, ranks, alphas, off)
    out = blk.forward(dev(x))
    dx, grads = blk.backward(dev(dout), keep=True)
    torch.cuda.synchronize()
    res = {"out": host(out), "dx": host(dx), "grads": {n: (host(a), host(b)) for n, (a, b) in grads.items()}}
    c, cb = blk.cache, blk.cache["bwd"]
    rows = np.concatenate([np.arange(off[i], off[i + 1]) for i in FULL_SEQS])
    rt = torch.from_numpy(rows).cuda()
    # the GPU's own intermediates on the sampled sequences' rows: q and k after
    # the rotary embedding, v, the attention output and statistics, and the
    # backward's attention gradients, dq and dk after the rotary adjoint
    res["mid"] = {k: (rows, host(t[rt])) for k, t in (("q", c["q"]), ("k", c["k"]), ("v", c["v"]),
                                                       ("att", c["att"]), ("datt", cb["datt"]), ("dq", cb["dq"]),
                                                       ("dk", cb["dk"]), ("dv", cb["dv"]), ("dx2", cb["dx2"]))}
    res["mid"]["lse"] = (rows, host(c["lse"][:, rt]))
    res["mid"]["r1"] = (rows, host(c["r1"][rt]))
    del blk, out, dx, grads, dp, c, cb
    torch.cuda.empty_cache()
    return hp, x, dout, ranks, alphas, off, res


FULL_SEQS = (0, 13, 31)


def rope_abs(e, positions):
    """Elementwise bound after the rotary adjoint: each element of a rotated
    pair is at most |cos| e_same + |sin| e_other."""
    T = e.shape[0]
    eh = e.reshape(T, -1, 128)
    ang = OB.rope_angles(positions)[:, None, :]
    c, s = np.abs(np.cos(ang)), np.abs(np.sin(ang))
    lo, hi = eh[..., :64], eh[..., 64:]
    return np.concatenate([lo * c + hi * s, hi * c + lo * s], axis=-1).reshape(T, -1)


def gpu_rows(res, key, a, b):
    """The GPU's intermediate `key` on token rows a..b-1 (kept by the fixture)."""
    rows, vals = res["mid"][key]
    i = int(np.searchsorted(rows, a))
    assert rows[i] == a and rows[i + b - a - 1] == b - 1
    return vals[..., i:i + b - a] if key == "lse" else vals[i:i + b - a]


@pytest.mark.slow
@pytest.mark.parametrize("seq", FULL_SEQS)
def test_decoder_block_full_size(full_block, seq):
    from packed_adapter_lora_amd.block import PROJ
    hp, x, dout, ranks, alphas, off, res = full_block
    a, b = off[seq], off[seq + 1]
    r, ro = ranks[seq], sum(ranks[:seq])
    L = b - a
    log("sequence %d (rank %d, alpha %g): fp64 oracle on tokens %d..%d" % (seq, r, alphas[seq], a, b))
    sub = dict(hp)
    sub["A"] = {n: v[ro:ro + r] for n, v in hp["A"].items()}
    sub["B"] = {n: v[ro:ro + r] for n, v in hp["B"].items()}
    sub["ranks"], sub["alphas"] = np.array([r]), np.array([alphas[seq]])
    ref_out, cache = OB.block_forward(sub, x[a:b], [0, L], [0, L], store=rnd)
    ref_dx, ref_grads = OB.block_backward(sub, cache, dout[a:b], [0, L], [0, L], store=rnd)
    chained_check(res["out"][a:b], ref_out, "out[sequence %d]" % seq)
    # dx lies below both attention kernels, which feed P and dS to the matrix
    # cores in bf16 while the oracle's attention is fp64 by definition; in the
    # block the scores are large (the adapters' branches dominate q and k), so
    # that rounding is amplified.  End to end dx is held to the Frobenius
    # bound; elementwise it is checked link by link from the GPU's own
    # intermediates: attention forward and backward at their per-kernel
    # rounding bounds, then the rest of the chain (rotary adjoint, the q/k/v
    # input gradients, the first RMSNorm's backward) at the chained bound.
    chained_check(res["dx"][a:b], ref_dx, "dx[sequence %d]" % seq, elementwise=False)
    one, n_q, n_kv = [0, L], sub["n_q"], sub["n_kv"]
    q, k, v = (gpu_rows(res, key, a, b) for key in ("q", "k", "v"))
    att, lse, datt = gpu_rows(res, "att", a, b), gpu_rows(res, "lse", a, b), gpu_rows(res, "datt", a, b)
    o_ref, lse_ref = OB.attention_fwd(q, k, v, one, n_q, n_kv)
    check_attention_out(att, o_ref, one, n_q, "attention o[sequence %d]" % seq)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-5, atol=1e-4)
    pos = OB.positions_of(one)
    refs = OB.attention_bwd(datt, q, k, v, att, lse, one, n_q, n_kv)
    bounds = bwd_rounding_bounds(q, k, v, datt, att, lse, one, n_q, n_kv)
    for name, ref, bd, nh in zip(("dq", "dk", "dv"), refs, bounds, (n_q, n_kv, n_kv)):
        got = gpu_rows(res, name, a, b)
        lim = 2.0 * (bd + 2.0 ** -9 * np.abs(ref)) + 1e-6
        if name != "dv":
            # the GPU's dq, dk are kept after the rotary adjoint: an orthogonal
            # map of each pair, whose kernel rounds its output to bf16 again
            ref = OB.rope_bwd(ref, pos)
            lim = rope_abs(lim, pos) + 2.0 * 2.0 ** -9 * np.abs(ref)
        check_attention_out(got, ref, one, nh, "attention %s[sequence %d]" % (name, seq), elementwise=False)
        err = np.abs(got - ref)
        log("attention %s[sequence %d]: worst elementwise %.2f of the rounding bound" % (
            name, seq, float(np.max(err / lim))))
        assert np.all(err <= lim), "attention %s[sequence %d]: %d elements beyond the rounding bound" % (
            name, seq, int(np.sum(err > lim)))
    dh1 = 0.0
    for name in ("q", "k", "v"):
        dh1 = dh1 + rnd(OB._proj(sub, name, one, ("dX",), dY=gpu_rows(res, "d" + name, a, b))["dX"])
    r1 = gpu_rows(res, "r1", a, b)
    tail = rnd(gpu_rows(res, "dx2", a, b) + OB.rmsnorm_bwd(dh1, x[a:b], sub["w1"], r1))
    chained_check(res["dx"][a:b], tail, "dx[sequence %d] from the GPU's attention gradients" % seq)
    for n in PROJ:
        chained_check(res["grads"][n][0][ro:ro + r], ref_grads[n][0], "dA[%s, adapter %d]" % (n, seq))
        chained_check(res["grads"][n][1][ro:ro + r], ref_grads[n][1], "dB[%s, adapter %d]" % (n, seq))
