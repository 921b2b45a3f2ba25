"""GPU parity of the optimizer-side entry points through the C ABI:
per-adapter AdamW against the fp64 oracle, and gradient accumulation of
plora_backward_dAdB_acc (bitwise doubling, micro-batch sums against the
oracle, untouched adapters without tokens)."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import adamw as OA
from parity_utils import TOL, TOL_F32_OUT, check_block, h_blocks, host, log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def _dev32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def _bf16_of(x32):
    return workloads.f32_to_bf16_bits(np.ascontiguousarray(x32, dtype=np.float32))


# AdamW: fp32 arithmetic against fp64.  Relative 1e-6 on values (a few fp32
# roundings) plus an absolute term for the update itself, whose size is about
# lr; moments get an absolute term from the size of g.
def _f32(x):
    """The fp32 value the ABI receives, widened back (the oracle uses exactly that number)."""
    return [float(np.float32(v)) for v in x] if isinstance(x, (list, tuple)) else float(np.float32(x))


def _oracle(ranks, lrs, wds, steps, p, m, v, g, beta1=0.9, beta2=0.999, eps=1e-8):
    return OA.adamw_packed(ranks, _f32(lrs), _f32(wds), steps, p, m, v, g, beta1=_f32(beta1), beta2=_f32(beta2),
                           eps=_f32(eps))


def _check_adamw(name, got, ref, lr_max, gmax):
    atol = {"P": 1e-5 * lr_max + 1e-12, "m": 1e-7 * gmax, "v": 1e-7 * gmax * gmax}[name[0]]
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=atol, err_msg=name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_adamw_parity(P, dtype):
    import torch
    ranks = [1, 8, 16, 33, 64, 128]
    wl = workloads.custom(320, 264, [5, 0, 7, 3, 1, 2], ranks, [1.0] * len(ranks), dtype, seed=41, name="adamw")
    d = P.Desc.from_workload(wl)
    st = workloads.optimizer_state(wl, 43)
    dev = {k: _dev32(v) for k, v in st.items()}
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    A = torch.full((wl.R, wl.d_in), float("nan"), dtype=tdt, device="cuda")
    B = torch.full((wl.R, wl.d_out), float("nan"), dtype=tdt, device="cuda")
    lrs = [1e-3, 2e-2, 5e-4, 1e-1, 3e-3, 1e-2]
    wds = [0.01, 0.0, 0.1, 0.01, 0.5, 0.0]
    rng = np.random.default_rng(5)
    for it in range(3):
        steps = [it + 1, it + 4, 0 if it == 1 else it + 1, it + 1, 1000 + it, it + 2]
        log("adamw %s step set %s" % (dtype, steps))
        before = {k: host(v) for k, v in dev.items()}
        a_before, b_before = A.clone(), B.clone()
        cfg = P.AdamwConfig(lrs, steps, wds, beta1=0.9, beta2=0.999, eps=1e-8)
        P.plora_adamw_step(d, cfg, dev["PA"], dev["PB"], dev["mA"], dev["vA"], dev["mB"], dev["vB"], dev["dA"],
                           dev["dB"], A, B)
        torch.cuda.synchronize()
        for k in ("A", "B"):
            pr, mr, vr = _oracle(ranks, lrs, wds, steps, before["P" + k], before["m" + k], before["v" + k],
                                 before["d" + k])
            gmax = float(np.abs(before["d" + k]).max())
            _check_adamw("P" + k, host(dev["P" + k]), pr, max(lrs), gmax)
            _check_adamw("m" + k, host(dev["m" + k]), mr, max(lrs), gmax)
            _check_adamw("v" + k, host(dev["v" + k]), vr, max(lrs), gmax)
            # the operator copy is the rounding of the updated master, bit for bit
            out = A if k == "A" else B
            prev = a_before if k == "A" else b_before
            pnew = host(dev["P" + k]).astype(np.float32)
            ro = 0
            for i, r in enumerate(ranks):
                rows = slice(ro, ro + r)
                ro += r
                if steps[i] == 0:  # skipped: everything untouched (NaN copy stays NaN on the first pass)
                    for nm in ("P", "m", "v"):
                        np.testing.assert_array_equal(host(dev[nm + k])[rows], before[nm + k][rows])
                    assert torch.equal(out[rows].view(torch.int16 if dtype == "bf16" else torch.int32),
                                       prev[rows].view(torch.int16 if dtype == "bf16" else torch.int32))
                    continue
                if dtype == "bf16":
                    got = out[rows].view(torch.int16).cpu().numpy().view(np.uint16)
                    np.testing.assert_array_equal(got, _bf16_of(pnew[rows]))
                else:
                    np.testing.assert_array_equal(out[rows].cpu().numpy(), pnew[rows])
        # fresh gradients for the next step
        dev["dA"] = _dev32(rng.standard_normal((wl.R, wl.d_in)) * 1e-2)
        dev["dB"] = _dev32(rng.standard_normal((wl.R, wl.d_out)) * 1e-2)


def test_adamw_f32_copy_may_alias_master(P):
    import torch
    wl = workloads.custom(64, 32, [2, 2], [4, 8], [4.0, 8.0], "f32", seed=44, name="adamw_alias")
    d = P.Desc.from_workload(wl)
    st = workloads.optimizer_state(wl, 45)
    dev = {k: _dev32(v) for k, v in st.items()}
    cfg = P.AdamwConfig([1e-2, 1e-3], [1, 7])
    P.plora_adamw_step(d, cfg, dev["PA"], dev["PB"], dev["mA"], dev["vA"], dev["mB"], dev["vB"], dev["dA"], dev["dB"],
                       dev["PA"], dev["PB"])
    torch.cuda.synchronize()
    for k in ("A", "B"):
        pr, _, _ = _oracle([4, 8], [1e-2, 1e-3], [0.01, 0.01], [1, 7], st["P" + k], st["m" + k], st["v" + k],
                           st["d" + k])
        _check_adamw("P" + k, host(dev["P" + k]), pr, 1e-2, float(np.abs(st["d" + k]).max()))


def _dadb(P, wl, dev, H, G, dA, dB, accumulate):
    import torch
    d = P.Desc.from_workload(wl)
    nb = P.plora_workspace_bytes(d)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    P.plora_backward_dAdB(d, dev["X"], dev["dY"], H, G, dA, dB, ws, accumulate=accumulate)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_accumulate_same_batch_doubles_bitwise(P, dtype):
    import torch
    # adapter 0 spans several 1024-token chunks (partials + reduction), adapter
    # 2 is one chunk (direct store), adapter 1 has no tokens
    counts = [2100, 0, 300, 17] if dtype == "bf16" else [40, 0, 30, 7]
    wl = workloads.custom(384, 264, counts, [16, 8, 64, 1], [32.0, 16.0, 8.0, 2.0], dtype, seed=46, name="acc2")
    log("case %s dtype=%s T=%d" % (wl.name, dtype, wl.T))
    inp = workloads.make_inputs(wl)
    dev = {k: to_dev(v, dtype) for k, v in inp.items()}
    out = run_gpu(P, wl, dev)
    dA1, dB1 = out["dA"].clone(), out["dB"].clone()
    _dadb(P, wl, dev, out["H"], out["G"], out["dA"], out["dB"], accumulate=True)
    assert torch.equal(out["dA"], 2 * dA1) and torch.equal(out["dB"], 2 * dB1)


def test_accumulate_two_micro_batches_vs_oracle(P):
    import torch
    ranks, alphas = [16, 8, 64, 32], [32.0, 16.0, 8.0, 64.0]
    wl1 = workloads.custom(384, 640, [1500, 3, 0, 260], ranks, alphas, "bf16", seed=47, name="mb1")
    wl2 = workloads.custom(384, 640, [200, 0, 90, 1100], ranks, alphas, "bf16", seed=48, name="mb2")
    dA = dB = None
    refs = []
    for k, wl in enumerate((wl1, wl2)):
        log("micro-batch %d T=%d" % (k, wl.T))
        inp = workloads.make_inputs(wl)
        if k == 1:  # the same adapters in both micro-batches
            inp["A"], inp["B"], inp["W"] = a_b_w
        a_b_w = (inp["A"], inp["B"], inp["W"])
        dev = {n: to_dev(v, "bf16") for n, v in inp.items()}
        out = run_gpu(P, wl, dev, want=("fwd", "dx"))
        if dA is None:
            dA = torch.full((wl.R, wl.d_in), float("nan"), dtype=torch.float32, device="cuda")
            dB = torch.full((wl.R, wl.d_out), float("nan"), dtype=torch.float32, device="cuda")
        _dadb(P, wl, dev, out["H"], out["G"], dA, dB, accumulate=(k == 1))
        if k == 0:
            first = (dA.clone(), dB.clone())
        refs.append(oracle.run_workload(wl, inp, want=("dA", "dB")))
    gA, gB = host(dA), host(dB)
    for i, _, rr, _, r, _ in h_blocks(wl1):
        check_block(gA[rr], refs[0]["dA"][rr] + refs[1]["dA"][rr], TOL_F32_OUT, "dA[adapter %d]" % i)
        check_block(gB[rr], refs[0]["dB"][rr] + refs[1]["dB"][rr], TOL_F32_OUT, "dB[adapter %d]" % i)
    # adapter 1 has no tokens in the second micro-batch: its rows keep the first micro-batch's values
    rr = h_blocks(wl1)[1][2]
    assert torch.equal(dA[rr], first[0][rr]) and torch.equal(dB[rr], first[1][rr])
