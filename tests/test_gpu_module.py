"""GPU parity of PackedLoRALinear (the PyTorch module over the C ABI) against
the fp64 oracle: loss.backward() through the module gives the oracle's dX,
dA and dB; gradient accumulation runs in the kernel; the operator's bf16
copies follow the fp32 masters (after a change made in PyTorch and after the
library's AdamW step)."""
import numpy as np
import pytest

import oracle
import workloads
from parity_utils import TOL, check_full, host, log, to_dev, tol_of, check_block, h_blocks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def module_case(P, wl, inp):
    import torch
    from packed_adapter_lora_amd.module import PackedLoRALinear
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    W = to_dev(inp["W"], wl.dtype)
    A = torch.from_numpy(inp["A"]).cuda()
    B = torch.from_numpy(inp["B"]).cuda()
    m = PackedLoRALinear(W, wl.ranks, wl.alphas, A=A, B=B, seg_offsets=wl.offsets)
    X = to_dev(inp["X"], wl.dtype).requires_grad_(True)
    dY = to_dev(inp["dY"], wl.dtype)
    assert X.dtype == tdt
    return m, X, dY


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_module_backward_matches_oracle(P, dtype):
    """loss = sum(dY * module(X)): the gradient reaching the operator is dY,
    so X.grad, lora_A.grad and lora_B.grad are the oracle's dX, dA and dB."""
    import torch
    wl = workloads.custom(512, 768, [300, 0, 1, 100, 1200, 57], [16, 8, 33, 64, 1, 128],
                          [32.0, 16.0, 33.0, 16.0, 2.0, 64.0], dtype, seed=51, name="module_" + dtype)
    log("case %s" % wl.name)
    inp = workloads.make_inputs(wl)
    m, X, dY = module_case(P, wl, inp)
    Y = m(X)
    loss = (dY * Y).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle.run_workload(wl, inp)
    got = {"Y": host(Y), "dX": host(X.grad), "dA": host(m.lora_A.grad), "dB": host(m.lora_B.grad)}
    check_full(wl, got, ref, names=("Y", "dX", "dA", "dB"))
    assert m.weight.grad is None


def test_module_grad_accumulation_in_kernel(P):
    """A second backward over the same batch adds in the kernel: .grad becomes
    exactly twice the first (x + x is exact in fp32), and the tensor object is
    the same (no new gradient handed to autograd)."""
    import torch
    wl = workloads.custom(384, 640, [100, 513, 0, 64], [16, 64, 8, 32], [32.0, 16.0, 8.0, 64.0], "bf16", seed=52,
                          name="module_acc")
    log("case %s" % wl.name)
    inp = workloads.make_inputs(wl)
    m, X, dY = module_case(P, wl, inp)
    m(X).backward(dY)
    torch.cuda.synchronize()
    gA, gB = m.lora_A.grad, m.lora_B.grad
    first = (gA.clone(), gB.clone())
    m(X).backward(dY)
    torch.cuda.synchronize()
    assert m.lora_A.grad is gA and m.lora_B.grad is gB
    assert torch.equal(gA, 2 * first[0]) and torch.equal(gB, 2 * first[1])
    # a different micro-batch: the sum matches the oracle's sum
    inp2 = dict(inp)
    inp2["X"] = workloads.draw(53, workloads.TID_X, (wl.T, wl.d_in), 1.0, "bf16")
    inp2["dY"] = workloads.draw(53, workloads.TID_DY, (wl.T, wl.d_out), 1.0, "bf16")
    m.zero_grad(set_to_none=True)
    m(X).backward(dY)
    X2 = to_dev(inp2["X"], "bf16")
    m(X2).backward(to_dev(inp2["dY"], "bf16"))
    torch.cuda.synchronize()
    r1, r2 = oracle.run_workload(wl, inp), oracle.run_workload(wl, inp2)
    for i, rows, rr, hs, r, n in h_blocks(wl):
        check_block(host(m.lora_A.grad)[rr], r1["dA"][rr] + r2["dA"][rr], tol_of("bf16", "dA"), "dA[%d]" % i)
        check_block(host(m.lora_B.grad)[rr], r1["dB"][rr] + r2["dB"][rr], tol_of("bf16", "dB"), "dB[%d]" % i)


def test_module_copies_follow_masters(P):
    """The operator's bf16 copies are the round-to-nearest-even of the fp32
    masters: at construction, after a change made with a PyTorch in-place op
    (version counter), and after the library's AdamW step."""
    import torch
    from packed_adapter_lora_amd.module import PackedLoRALinear
    wl = workloads.custom(256, 512, [40, 0, 300], [8, 16, 64], [16.0, 16.0, 32.0], "bf16", seed=54, name="copies")
    inp = workloads.make_inputs(wl)
    W = to_dev(inp["W"], "bf16")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    m = PackedLoRALinear(W, wl.ranks, wl.alphas, seg_offsets=wl.offsets, generator=g)
    assert torch.count_nonzero(m.lora_B).item() == 0  # B = 0 at the start

    def rne(t):
        return workloads.f32_to_bf16_bits(t.detach().cpu().numpy())

    def check():
        A_op, B_op = m.operator_panels()
        assert np.array_equal(A_op.view(torch.int16).cpu().numpy().view(np.uint16), rne(m.lora_A))
        assert np.array_equal(B_op.view(torch.int16).cpu().numpy().view(np.uint16), rne(m.lora_B))

    check()
    # B = 0: the layer is the frozen one, bit for bit
    X = to_dev(inp["X"], "bf16")
    Y = m(X)
    d0 = P.Desc([0], [], [], wl.d_in, wl.d_out, "bf16", n_tokens=wl.T)
    Y0 = torch.empty_like(Y)
    P.plora_forward(d0, X, W, None, None, Y0, None)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))
    with torch.no_grad():
        m.lora_B.copy_(torch.from_numpy(np.random.default_rng(3).standard_normal((wl.R, wl.d_out)).astype(np.float32)))
    check()
    Y = m(X)
    Y.backward(to_dev(inp["dY"], "bf16"))
    m.adamw_step(lr=[1e-3, 2e-3, 5e-4], weight_decay=0.01)
    torch.cuda.synchronize()
    check()


def test_module_frozen_only(P):
    """No adapters: the module is the frozen layer (plora_forward with N = 0)."""
    import torch
    from packed_adapter_lora_amd.module import PackedLoRALinear
    T, d_in, d_out = 200, 256, 520
    W = to_dev(workloads.draw(55, 1, (d_out, d_in), 1 / 16, "bf16"), "bf16")
    Xh = workloads.draw(55, 4, (T, d_in), 1.0, "bf16")
    dYh = workloads.draw(55, 5, (T, d_out), 1.0, "bf16")
    m = PackedLoRALinear(W, [], [])
    X = to_dev(Xh, "bf16").requires_grad_(True)
    Y = m(X, [0])
    Y.backward(to_dev(dYh, "bf16"))
    torch.cuda.synchronize()
    ref = oracle.packed_lora([0], [], [], d_in, d_out, X=Xh, dY=dYh, W=workloads.draw(55, 1, (d_out, d_in), 1 / 16,
                                                                                        "bf16"), want=("Y", "dX"), T=T)
    check_block(host(Y), ref["Y"], TOL["bf16"], "Y")
    check_block(host(X.grad), ref["dX"], TOL["bf16"], "dX")
