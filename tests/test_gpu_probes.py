"""The ceiling micro-benchmarks (include/plora_probe.h) on the GPU: the
matrix-core probe fed from LDS (shape 2) runs the same instructions on the
same fragments as the register-fed probe (shape 0), so their accumulator
sums are equal bit for bit; the L2 -> LDS probe leaves the bytes it streamed
in LDS (a one-piece span: every slot holds the wave's first KiB)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import packed_adapter_lora_amd as P
    return P


def test_mfma_probe_lds_fed_equals_register_fed(P):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    nb = P.plora_probe_mfma_operand_bytes()
    ops = torch.randn((nb // 2,), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    wg, iters = 8, 5
    outs = []
    for shape in (0, 2):
        out = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
        fl = P.plora_probe_mfma(ops, wg, iters, out, shape=shape)
        assert fl == wg * 4 * iters * 2.0 * 128 * 128 * 32
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


def test_lds_dma_probe_lands_the_bytes(P):
    import torch
    src = torch.arange(4096 // 4, dtype=torch.int32, device="cuda")
    wg = 3
    out = torch.full((wg * 256,), -1, dtype=torch.int32, device="cuda")
    nbytes = P.plora_probe_lds_dma(src, wg, 4, out)
    torch.cuda.synchronize()
    assert nbytes == wg * 4 * 4096
    # thread t reads word t of the ring: wave 0's slot 0 holds src bytes [0, 1 KiB)
    expect = torch.arange(256, dtype=torch.int32, device="cuda").repeat(wg)
    assert torch.equal(out, expect)
