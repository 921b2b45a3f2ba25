"""Inputs of the rank-r indexing probe (not collected by pytest).

Every adapter i gets distinct unit vectors as the columns of A_i (rows of the
packed A), B_i = c_i * ones with c_i = i + 1, a power-of-two scale s_i, 0/1
token rows X, one-hot rows of dY and a sparse frozen weight of -1/0/+1.  With
these values every product the operator forms is a small integer times a
power of two, so every fp32 sum is exact whatever its order, and the outputs
have closed forms (``tests/test_oracle_pins.py`` checks the oracle against
them); a token row served by the wrong adapter shows the wrong c_i or the
wrong unit vectors.  This module only draws inputs: it holds none of the
operator's arithmetic.
"""
from __future__ import annotations

import numpy as np

# Two adapter sets.  "le64": ranks <= 64 (the weight-gradient kernels that
# stream transposed H/G, the compact expand), with an adapter of <= 128 tokens
# (its shrink is split along K and summed afterwards), one of > 1024 tokens
# (weight-gradient partials and their reduction), a one-token and an empty
# segment, and segments that cross 256-token tiles.  "r128": a rank-128
# adapter (the general expand and weight-gradient kernels) among small ones.
ADAPTER_SETS = {
    "le64": dict(counts=[300, 0, 1, 100, 2100, 257, 64], ranks=[16, 8, 33, 64, 1, 33, 16],
                 scales=[2.0, 1.0, 0.5, 4.0, 2.0, 1.0, 0.25]),
    "r128": dict(counts=[129, 40, 1500, 0, 700, 3], ranks=[128, 1, 64, 16, 33, 24],
                 scales=[1.0, 4.0, 0.5, 2.0, 1.0, 2.0]),
}


def probe_inputs(counts, ranks, d_in, d_out, seed, x_density=0.25, w_density=1.0 / 32):
    """fp32 arrays W [d_out, d_in], A [R, d_in], B [R, d_out], X [T, d_in],
    dY [T, d_out] (all values exact in bf16), plus the unit-vector columns
    ``ks`` (row R_off[i] + j of A is e_{ks[R_off[i] + j]}), the token's
    one-hot column ``nt`` and ``c``."""
    rng = np.random.default_rng(seed)
    N, T, R = len(counts), int(sum(counts)), int(sum(ranks))
    if R > d_in:
        raise ValueError("distinct unit vectors need sum(ranks) <= d_in")
    ks = rng.choice(d_in, size=R, replace=False)
    A = np.zeros((R, d_in), np.float32)
    A[np.arange(R), ks] = 1.0
    c = np.arange(1, N + 1, dtype=np.float32)
    B = np.repeat(np.repeat(c, ranks)[:, None], d_out, axis=1).astype(np.float32)
    X = (rng.random((T, d_in)) < x_density).astype(np.float32)
    nt = rng.integers(0, d_out, size=T)
    dY = np.zeros((T, d_out), np.float32)
    dY[np.arange(T), nt] = 1.0
    u = rng.random((d_out, d_in))
    W = np.where(u < w_density / 2, -1.0, np.where(u > 1.0 - w_density / 2, 1.0, 0.0)).astype(np.float32)
    return dict(W=W, A=A, B=B, X=X, dY=dY), ks, nt, c
