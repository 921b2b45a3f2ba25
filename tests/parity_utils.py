"""Helpers for the GPU-vs-oracle parity tests (not collected by pytest).

Tolerance reading: for each output block (the Y and dX rows of one segment,
one adapter's H, G, dA, dB) the error must satisfy both
    ||out - ref||_F <= tol * ||ref||_F
and, elementwise,
    |out - ref| <= tol * (|ref| + rms(ref_block))
with tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 accumulate).

The fp32 outputs of bf16 problems (H, G, dA, dB) are held to 1e-4 as well:
they are fp32 sums of exact bf16 products, and H/G enter the expand and the
weight-gradient products as a bf16 hi/lo pair (about 2^-16 relative), so a
loss of that precision (a single bf16 term, 2^-9) fails them.
"""
from __future__ import annotations

import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_F32_OUT = 1e-4


def tol_of(wl_dtype, name):
    """Tolerance of output `name` for a problem of dtype wl_dtype."""
    return TOL_F32_OUT if name in ("H", "G", "dA", "dB") else TOL[wl_dtype]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    """fp32 numpy (bf16-representable for bf16) -> device tensor of the workload dtype (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def poison(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def run_gpu(P, wl, dev, want=("fwd", "dx", "dadb"), desc=None):
    """Run the three entry points on device inputs ``dev`` (dict of tensors).

    Outputs are NaN-filled first, so an element no kernel writes fails parity.
    Returns a dict of device tensors.
    """
    import torch
    d = desc if desc is not None else P.Desc.from_workload(wl)
    T, R = wl.T, wl.R
    tdt = torch_dtype(wl.dtype)
    he = P.plora_h_elems(d) if wl.n_adapters else 0
    out = {}
    if "fwd" in want:
        out["Y"] = poison((T, wl.d_out), tdt)
        out["H"] = poison((he,), torch.float32)
        P.plora_forward(d, dev["X"], dev["W"], dev.get("A"), dev.get("B"), out["Y"], out["H"] if he else None)
    if "dx" in want:
        out["dX"] = poison((T, wl.d_in), tdt)
        out["G"] = poison((he,), torch.float32)
        P.plora_backward_dx(d, dev["dY"], dev["W"], dev.get("A"), dev.get("B"), out["dX"], out["G"] if he else None)
    if "dadb" in want and wl.n_adapters:
        out["dA"] = poison((R, wl.d_in), torch.float32)
        out["dB"] = poison((R, wl.d_out), torch.float32)
        nb = P.plora_workspace_bytes(d)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
        H = out["H"] if "H" in out else dev["H"]
        G = out["G"] if "G" in out else dev["G"]
        P.plora_backward_dAdB(d, dev["X"], dev["dY"], H, G, out["dA"], out["dB"], ws)
    torch.cuda.synchronize()
    return out


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_block(out, ref, tol, name, floor_rms=0.0, elementwise=True):
    """floor_rms: a scale below which a block's own rms is not used (for blocks
    whose exact value is zero or nearly so, e.g. a one-token sequence's dQ);
    errors are then measured against that scale instead."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (name, out.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(out)), "%s: non-finite output (unwritten element?)" % name
    diff = out - ref
    fro = np.linalg.norm(diff)
    rms = max(np.linalg.norm(ref) / np.sqrt(ref.size), floor_rms)
    rf = rms * np.sqrt(ref.size)
    assert fro <= tol * rf + 1e-30, "%s: ||diff||_F %.3e > tol %.1e * ||ref||_F %.3e" % (name, fro, tol, rf)
    if not elementwise:
        return
    bound = tol * (np.abs(ref) + rms) + 1e-30
    bad = np.abs(diff) > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(np.abs(diff) / bound), diff.shape)
        raise AssertionError("%s: %d elements out of tolerance; worst at %s: out %.6e ref %.6e" %
                             (name, int(bad.sum()), idx, out[idx], ref[idx]))


def h_blocks(wl):
    """(adapter, rows slice, rank-row slice, H/G slice, r, n) per adapter."""
    res, ro, ho = [], 0, 0
    for i, r in enumerate(wl.ranks.tolist()):
        a, b = int(wl.offsets[i]), int(wl.offsets[i + 1])
        res.append((i, slice(a, b), slice(ro, ro + r), slice(ho, ho + (b - a) * r), r, b - a))
        ro += r
        ho += (b - a) * r
    return res


def check_full(wl, gpu, ref, tol=None, names=("Y", "H", "dX", "G", "dA", "dB")):
    """Blockwise comparison of every output of a small problem (tol: one
    tolerance for every output instead of tol_of's)."""
    t = (lambda k: tol_of(wl.dtype, k)) if tol is None else (lambda k: tol)
    if wl.n_adapters == 0:
        for k in ("Y", "dX"):
            if k in names and k in gpu:
                check_block(gpu[k], ref[k], t(k), k)
        return
    for i, rows, rr, hs, r, n in h_blocks(wl):
        for k in ("Y", "dX"):
            if k in names and k in gpu:
                check_block(gpu[k][rows], ref[k][rows], t(k), "%s[segment %d]" % (k, i))
        for k in ("H", "G"):
            if k in names and k in gpu:
                check_block(gpu[k][hs], ref[k][hs], t(k), "%s[adapter %d]" % (k, i))
        for k in ("dA", "dB"):
            if k in names and k in gpu:
                check_block(gpu[k][rr], ref[k][rr], t(k), "%s[adapter %d]" % (k, i))
