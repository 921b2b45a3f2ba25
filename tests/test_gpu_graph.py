"""GPU tests of the entry points under HIP graph capture.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a caller may capture a whole step into a
graph and replay it.  Each test captures a sequence of calls once, then
replays the graph three times with eager work and synchronisations between
the replays; every replay must reproduce the eager outputs bit for bit.
Outputs are refilled with NaN (by an eager fill kernel) before each replay,
so an element the replay does not write fails the comparison.
"""
import pytest

import workloads
from parity_utils import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_adapter_lora_amd as P  # raises if libplora.so is missing
    return P


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _capture_and_replay(fn, outs, eager_between):
    """Eager fn() -> reference; capture fn() into a graph; replay 3 times."""
    import torch
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(o), _bits(r)), "replay %d, output %d" % (rep, k)
        eager_between()
        torch.cuda.synchronize()


# segments: several 1024-token weight-gradient chunks (partials and their
# reduction), adapters of at most 128 tokens (K-sliced shrink and its slice
# sum), an empty one, a single token
_WL = dict(d_in=512, d_out=768, counts=[1300, 0, 513, 1, 64, 300], ranks=[16, 8, 64, 32, 1, 33],
           alphas=[32.0, 16.0, 8.0, 16.0, 4.0, 66.0])


def _inputs(P, seed, name):
    import torch
    wl = workloads.custom(_WL["d_in"], _WL["d_out"], _WL["counts"], _WL["ranks"], _WL["alphas"], "bf16", seed=seed,
                          name=name)
    inp = workloads.make_inputs(wl)
    dev = {k: to_dev(v, "bf16") for k, v in inp.items()}
    d = P.Desc.from_workload(wl)
    he = P.plora_h_elems(d)
    out = {
        "Y": torch.empty((wl.T, wl.d_out), dtype=torch.bfloat16, device="cuda"),
        "dX": torch.empty((wl.T, wl.d_in), dtype=torch.bfloat16, device="cuda"),
        "H": torch.empty(he, device="cuda"),
        "G": torch.empty(he, device="cuda"),
        "dA": torch.empty((wl.R, wl.d_in), device="cuda"),
        "dB": torch.empty((wl.R, wl.d_out), device="cuda"),
    }
    return wl, d, dev, out


def test_graph_replay_step(P):
    """forward + backward_dx + backward_dAdB (caller workspace) in one graph."""
    import torch
    wl, d, dev, out = _inputs(P, 71, "graph_step")
    log("case %s T=%d" % (wl.name, wl.T))
    ws = torch.empty(max(P.plora_workspace_bytes(d), 16), dtype=torch.uint8, device="cuda")

    def step():
        P.plora_forward(d, dev["X"], dev["W"], dev["A"], dev["B"], out["Y"], out["H"])
        P.plora_backward_dx(d, dev["dY"], dev["W"], dev["A"], dev["B"], out["dX"], out["G"])
        P.plora_backward_dAdB(d, dev["X"], dev["dY"], out["H"], out["G"], out["dA"], out["dB"], ws)

    # eager work between replays: the same step on other inputs, into other outputs
    other = {k: torch.empty_like(v) for k, v in out.items()}
    X2 = dev["X"].flip(0).contiguous()

    def between():
        P.plora_forward(d, X2, dev["W"], dev["A"], dev["B"], other["Y"], other["H"])
        P.plora_backward_dAdB(d, X2, dev["dY"], other["H"], out["G"], other["dA"], other["dB"], ws)

    _capture_and_replay(step, [out[k] for k in ("Y", "dX", "H", "G", "dA", "dB")], between)


def test_graph_replay_noalloc_and_shared(P):
    """The entry point without a workspace (its scratch is a device array that
    earlier calls leave dirty) and the shared-input calls of two projections,
    captured together."""
    import torch
    wl, d, dev, out = _inputs(P, 72, "graph_shared")
    log("case %s T=%d" % (wl.name, wl.T))
    # a second projection on the same X: its own A, B and outputs
    gen = torch.Generator(device="cpu").manual_seed(73)
    A1 = (torch.randn(dev["A"].shape, generator=gen) * 0.1).to("cuda", torch.bfloat16)
    B1 = (torch.randn(dev["B"].shape, generator=gen) * 0.02).to("cuda", torch.bfloat16)
    he = P.plora_h_elems(d)
    H1, G1 = torch.empty(he, device="cuda"), torch.empty(he, device="cuda")
    Y1 = torch.empty_like(out["Y"])
    dA1, dA2 = torch.empty_like(out["dA"]), torch.empty_like(out["dA"])
    ws = torch.empty(max(P.plora_workspace_bytes_dA_shared(d, 2), 16), dtype=torch.uint8, device="cuda")
    # G of both projections from one backward_dx each (eager, before capture)
    P.plora_backward_dx(d, dev["dY"], dev["W"], dev["A"], dev["B"], out["dX"], out["G"])
    P.plora_backward_dx(d, dev["dY"], dev["W"], A1, B1, out["dX"], G1)
    torch.cuda.synchronize()

    def seq():
        P.plora_shrink_shared(d, dev["X"], [dev["A"], A1], [out["H"], H1])
        P.plora_forward_expand(d, dev["X"], dev["W"], dev["B"], out["Y"], out["H"])
        P.plora_forward_expand(d, dev["X"], dev["W"], B1, Y1, H1)
        P.plora_backward_dA_shared(d, dev["X"], [out["G"], G1], [out["dA"], dA1], ws)
        P.plora_backward_dAdB_noalloc(d, dev["X"], dev["dY"], out["H"], out["G"], dA2, out["dB"])

    # eager between replays: a no-alloc call on another problem dirties the scratch
    wl2, d2, dev2, out2 = _inputs(P, 74, "graph_shared_other")

    def between():
        P.plora_forward(d2, dev2["X"], dev2["W"], dev2["A"], dev2["B"], out2["Y"], out2["H"])
        P.plora_backward_dx(d2, dev2["dY"], dev2["W"], dev2["A"], dev2["B"], out2["dX"], out2["G"])
        P.plora_backward_dAdB_noalloc(d2, dev2["X"], dev2["dY"], out2["H"], out2["G"], out2["dA"], out2["dB"])

    _capture_and_replay(seq, [out["H"], H1, out["Y"], Y1, out["dA"], dA1, dA2, out["dB"]], between)
    # the shared pass and the no-alloc pass compute projection 0's dA by the same kernels
    assert torch.equal(_bits(out["dA"]), _bits(dA2))
