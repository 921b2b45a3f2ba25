"""Pins for the fp64 oracle: facts the pages and the mathematics fix, none of
which re-types the oracle's own loops.

* B = 0 at initialisation makes the branch vanish, so Y is exactly the frozen
  output [LLM+LoRA微调加速技术原理解析, 深入理解LoRA: A Gaussian, B zero].
* A trained branch can be merged into the frozen weight, W + s A B, with no
  change to the output [same page, advantage 3 of the LoRA summary list]:
  checked against numpy matmul, forward and backward.
* Packed = adapter by adapter [PLoRA technical summary, 方法论 > 2]: the
  concatenated-tensor (block-diagonal, masked dense) form, separate runs per
  adapter, permutation and locality.
* A rank-1 closed form with small integers: exact values.
* Backward = gradient of the forward: central differences of
  L = sum(dY * Y), only A and B (and X) receive gradients
  [LoRA加速集成方案, 四、工作原理 > 3. 反向传播阶段].
* A hand-worked example (tests/golden/hand_example.json).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed, counts=(3, 0, 5, 1), ranks=(2, 3, 1, 4), alphas=(4.0, 3.0, 2.0, 32.0), d_in=7, d_out=6):
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    ranks = np.asarray(ranks, np.int32)
    alphas = np.asarray(alphas, np.float64)
    T, R = int(off[-1]), int(ranks.sum())
    p = dict(offsets=off, ranks=ranks, alphas=alphas, d_in=d_in, d_out=d_out,
             X=rng.standard_normal((T, d_in)), dY=rng.standard_normal((T, d_out)),
             W=rng.standard_normal((d_out, d_in)) / np.sqrt(d_in),
             A=rng.standard_normal((R, d_in)), B=rng.standard_normal((R, d_out)))
    return p


def run(p, want=("Y", "H", "dX", "G", "dA", "dB")):
    return oracle.packed_lora(p["offsets"], p["ranks"], p["alphas"], p["d_in"], p["d_out"],
                              X=p["X"], dY=p["dY"], W=p["W"], A=p["A"], B=p["B"], want=want)


def blocks(p):
    """(i, s_i, rows slice, rank-row slice, H slice) per adapter."""
    out, ro, ho = [], 0, 0
    for i, r in enumerate(p["ranks"].tolist()):
        a, b = int(p["offsets"][i]), int(p["offsets"][i + 1])
        out.append((i, p["alphas"][i] / r, slice(a, b), slice(ro, ro + r), slice(ho, ho + (b - a) * r), r, b - a))
        ro += r
        ho += (b - a) * r
    return out


def close(a, b, rtol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.abs(b).max(initial=0.0)))
    assert np.allclose(a, b, rtol=rtol, atol=rtol * scale), float(np.abs(a - b).max(initial=0.0))


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------

def test_hand_example_exact():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    out = oracle.packed_lora(g["offsets"], g["ranks"], g["alphas"], g["d_in"], g["d_out"],
                             X=g["X"], dY=g["dY"], W=g["W_stored_dout_by_din"], A=g["A_stored_R_by_din"],
                             B=g["B_stored_R_by_dout"])
    for k in ("Y", "H", "dX", "G", "dA", "dB"):
        assert np.array_equal(out[k], np.asarray(g[k], dtype=np.float64)), k


# --------------------------------------------------------------------------
# B = 0: the branch vanishes exactly
# --------------------------------------------------------------------------

def test_b_zero_gives_frozen_output_exactly():
    p = rand_problem(1)
    p["B"] = np.zeros_like(p["B"])
    out = run(p)
    base = oracle.packed_lora([0], [], [], p["d_in"], p["d_out"], X=p["X"], dY=p["dY"],
                              W=p["W"], want=("Y", "dX"), T=p["X"].shape[0])
    # frozen-only (no adapters) covering the same tokens
    assert np.array_equal(out["Y"], base["Y"])
    assert np.array_equal(out["dA"], np.zeros_like(out["dA"]))
    assert np.array_equal(out["G"], np.zeros_like(out["G"]))
    assert np.array_equal(out["dX"], base["dX"])
    # dB is not zero: s * H^T dY
    assert np.abs(out["dB"]).max() > 0
    for i, s, rows, rr, hs, r, n in blocks(p):
        Ai = p["A"][rr].T
        close(out["dB"][rr], s * (p["X"][rows] @ Ai).T @ p["dY"][rows])


def test_frozen_path_matches_numpy():
    p = rand_problem(2, counts=(9,), ranks=(1,), alphas=(0.0,))
    out = run(p)
    close(out["Y"], p["X"] @ p["W"].T)
    close(out["dX"], p["dY"] @ p["W"])
    n0 = oracle.packed_lora([0], [], [], 7, 6, X=p["X"], dY=p["dY"], W=p["W"], want=("Y", "dX"), T=9)
    close(n0["Y"], p["X"] @ p["W"].T)
    close(n0["dX"], p["dY"] @ p["W"])


# --------------------------------------------------------------------------
# merge identity (forward and backward) against numpy matmul
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [3, 4])
def test_merge_identity(seed):
    # adapter 2 uses the PEFT example's r=8, alpha=32 (s = 4)
    p = rand_problem(seed, counts=(4, 6, 5, 0), ranks=(2, 5, 8, 3), alphas=(4.0, 5.0, 32.0, 1.0), d_in=9, d_out=11)
    out = run(p)
    Wm = p["W"].T
    for i, s, rows, rr, hs, r, n in blocks(p):
        Ai = p["A"][rr].T  # d_in x r
        Bi = p["B"][rr]  # r x d_out
        Weff = Wm + s * (Ai @ Bi)
        X, dY = p["X"][rows], p["dY"][rows]
        close(out["Y"][rows], X @ Weff)
        close(out["dX"][rows], dY @ Weff.T)
        XtdY = X.T @ dY  # a different evaluation order than the oracle's
        close(out["dA"][rr], (s * XtdY @ Bi.T).T)
        close(out["dB"][rr], s * Ai.T @ XtdY)
        close(out["H"][hs].reshape(n, r), X @ Ai)
        close(out["G"][hs].reshape(n, r), dY @ Bi.T)


# --------------------------------------------------------------------------
# concatenated (block-diagonal, masked dense) form
# --------------------------------------------------------------------------

def test_block_diagonal_dense_form():
    p = rand_problem(5, counts=(5, 2, 0, 7, 3), ranks=(3, 1, 2, 6, 4), alphas=(6.0, 1.0, 2.0, 12.0, 1.0))
    out = run(p)
    T, R = p["X"].shape[0], int(p["ranks"].sum())
    A_cat, B_cat = p["A"].T, p["B"]  # d_in x R, R x d_out
    M = np.zeros((T, R))
    svec = np.zeros(R)
    for i, s, rows, rr, hs, r, n in blocks(p):
        M[rows, rr] = 1.0
        svec[rr] = s
    S = np.diag(svec)
    Wm = p["W"].T
    HX = M * (p["X"] @ A_cat)
    GX = M * (p["dY"] @ B_cat.T)
    close(out["Y"], p["X"] @ Wm + HX @ S @ B_cat)
    close(out["dX"], p["dY"] @ Wm.T + GX @ S @ A_cat.T)
    close(out["dA"], (p["X"].T @ GX @ S).T)
    close(out["dB"], S @ HX.T @ p["dY"])


# --------------------------------------------------------------------------
# rank-1 closed form: exact small-integer values
# --------------------------------------------------------------------------

def rank1_problem(seed, counts, d_in, d_out, with_w):
    rng = np.random.default_rng(seed)
    N = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    ks = rng.choice(d_in, size=N, replace=False)
    svals = np.array([2.0 ** (i % 3) for i in range(N)])  # 1, 2, 4
    c = np.arange(1, N + 1, dtype=np.float64)
    A = np.zeros((N, d_in))
    A[np.arange(N), ks] = 1.0
    B = np.repeat(c[:, None], d_out, axis=1)
    X = rng.integers(0, 2, size=(T, d_in)).astype(np.float64)
    dY = np.zeros((T, d_out))
    nt = rng.integers(0, d_out, size=T)
    dY[np.arange(T), nt] = 1.0
    W = rng.integers(-2, 3, size=(d_out, d_in)).astype(np.float64) * (rng.random((d_out, d_in)) < 0.2) if with_w \
        else np.zeros((d_out, d_in))
    return dict(offsets=off, ranks=np.ones(N, np.int32), alphas=svals, d_in=d_in, d_out=d_out,
                X=X, dY=dY, W=W, A=A, B=B), ks, svals, c, nt


@pytest.mark.parametrize("with_w", [False, True])
def test_rank1_closed_form(with_w):
    counts = [3, 0, 1, 7, 2, 0, 5]
    p, ks, svals, c, nt = rank1_problem(11, counts, 16, 12, with_w)
    out = run(p)
    T = p["X"].shape[0]
    Y = np.zeros((T, 12))
    dX = np.zeros((T, 16))
    H = np.zeros(T)
    G = np.zeros(T)
    dA = np.zeros((len(counts), 16))
    dB = np.zeros((len(counts), 12))
    for i in range(len(counts)):
        a, b = int(p["offsets"][i]), int(p["offsets"][i + 1])
        for t in range(a, b):
            base_y = [sum(p["X"][t, k] * p["W"][n, k] for k in range(16)) for n in range(12)]
            Y[t] = np.array(base_y) + svals[i] * c[i] * p["X"][t, ks[i]]
            dX[t] = p["W"][nt[t]]  # one-hot dY picks one row of the stored weight
            dX[t, ks[i]] += svals[i] * c[i]
            H[t] = p["X"][t, ks[i]]
            G[t] = c[i]
            dA[i] += svals[i] * c[i] * p["X"][t]
            dB[i, nt[t]] += svals[i] * p["X"][t, ks[i]]
    assert np.array_equal(out["Y"], Y)
    assert np.array_equal(out["dX"], dX)
    assert np.array_equal(out["H"], H)
    assert np.array_equal(out["G"], G)
    assert np.array_equal(out["dA"], dA)
    assert np.array_equal(out["dB"], dB)


# --------------------------------------------------------------------------
# rank-r closed form on the inputs of the GPU indexing probe
# --------------------------------------------------------------------------

@pytest.mark.parametrize("set_name", ["le64", "r128"])
def test_rank_r_probe_closed_form(set_name):
    """With A_i's columns distinct unit vectors e_k (k in K_i), B_i = c_i * ones,
    0/1 rows X, one-hot dY (column n_t) and a -1/0/+1 weight, for t in S_i:
      H[t, j] = X[t, k_ij]             G[t, j] = c_i
      Y[t]    = X[t] W^T + s_i c_i sum_j X[t, k_ij]
      dX[t]   = W[n_t] + s_i c_i on the columns K_i
      dA_i[j] = s_i c_i sum_t X[t]     dB_i[j, n] = s_i * #{t : X[t, k_ij] = 1, n_t = n}
    all exact small integers times powers of two (the GPU probe compares
    against the oracle bit for bit on the same inputs)."""
    from exact_probe import ADAPTER_SETS, probe_inputs
    cfg = ADAPTER_SETS[set_name]
    counts, ranks, svals = cfg["counts"], cfg["ranks"], np.array(cfg["scales"])
    d_in, d_out = 512, 96
    inp, ks, nt, c = probe_inputs(counts, ranks, d_in, d_out, seed=3)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    alphas = svals * np.asarray(ranks)
    out = oracle.packed_lora(off, ranks, alphas, d_in, d_out, **inp)
    X, W = inp["X"].astype(np.float64), inp["W"].astype(np.float64)
    T, R = X.shape[0], sum(ranks)
    Y, dX = np.zeros((T, d_out)), np.zeros((T, d_in))
    H, G = np.zeros(out["H"].shape), np.zeros(out["G"].shape)
    dA, dB = np.zeros((R, d_in)), np.zeros((R, d_out))
    ro, ho = 0, 0
    for i, r in enumerate(ranks):
        cols = ks[ro:ro + r]
        for t in range(int(off[i]), int(off[i + 1])):
            m = X[t, cols]
            Y[t] = X[t] @ W.T + svals[i] * c[i] * m.sum()
            dX[t] = W[nt[t]]
            dX[t, cols] += svals[i] * c[i]
            H[ho:ho + r] = m
            G[ho:ho + r] = c[i]
            ho += r
            dA[ro:ro + r] += svals[i] * c[i] * X[t]
            dB[ro + np.arange(r), nt[t]] += svals[i] * m
        ro += r
    for k, v in (("Y", Y), ("dX", dX), ("H", H), ("G", G), ("dA", dA), ("dB", dB)):
        assert np.array_equal(out[k], v), k


# --------------------------------------------------------------------------
# backward = gradient of the forward (central differences, L affine per entry)
# --------------------------------------------------------------------------

def loss(p):
    y = oracle.packed_lora(p["offsets"], p["ranks"], p["alphas"], p["d_in"], p["d_out"], X=p["X"], W=p["W"],
                           A=p["A"], B=p["B"], want=("Y",))["Y"]
    return float(np.sum(p["dY"] * y))


def test_finite_differences():
    p = rand_problem(7, counts=(2, 0, 5), ranks=(1, 2, 3), alphas=(2.0, 3.0, 6.0), d_in=5, d_out=6)
    out = run(p)
    h = 0.5
    rng = np.random.default_rng(0)
    checks = []
    for name, grad in (("X", out["dX"]), ("A", out["dA"]), ("B", out["dB"])):
        arr = p[name]
        idx = [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(12)]
        for ix in idx:
            q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            q[name][ix] += h
            lp = loss(q)
            q[name][ix] -= 2 * h
            lm = loss(q)
            fd = (lp - lm) / (2 * h)
            checks.append((name, ix, fd, grad[ix]))
    Lscale = max(1.0, abs(loss(p)))
    for name, ix, fd, g in checks:
        assert abs(fd - g) <= 1e-10 * Lscale + 1e-10 * abs(g), (name, ix, fd, g)
    # rows of the empty adapter's A/B get zero gradient
    assert np.array_equal(out["dA"][1:3], np.zeros((2, 5)))
    assert np.array_equal(out["dB"][1:3], np.zeros((2, 6)))


# --------------------------------------------------------------------------
# packed = separate, permutation, locality
# --------------------------------------------------------------------------

def test_packed_equals_separate_bitwise():
    p = rand_problem(8, counts=(4, 0, 3, 6), ranks=(2, 3, 5, 1), alphas=(2.0, 3.0, 10.0, 0.5))
    out = run(p)
    for i, s, rows, rr, hs, r, n in blocks(p):
        q = dict(offsets=np.array([0, n], np.int64), ranks=p["ranks"][i:i + 1], alphas=p["alphas"][i:i + 1],
                 d_in=p["d_in"], d_out=p["d_out"], X=p["X"][rows], dY=p["dY"][rows], W=p["W"],
                 A=p["A"][rr], B=p["B"][rr])
        o1 = run(q)
        assert np.array_equal(out["Y"][rows], o1["Y"])
        assert np.array_equal(out["dX"][rows], o1["dX"])
        assert np.array_equal(out["dA"][rr], o1["dA"])
        assert np.array_equal(out["dB"][rr], o1["dB"])
        assert np.array_equal(out["H"][hs], o1["H"])
        assert np.array_equal(out["G"][hs], o1["G"])


def test_permutation_of_adapters():
    p = rand_problem(9, counts=(4, 2, 0, 6), ranks=(2, 3, 5, 1), alphas=(2.0, 3.0, 10.0, 0.5))
    out = run(p)
    perm = [2, 0, 3, 1]
    bl = blocks(p)
    q = dict(p)
    q["ranks"] = p["ranks"][perm]
    q["alphas"] = p["alphas"][perm]
    q["offsets"] = np.concatenate([[0], np.cumsum([bl[i][6] for i in perm])]).astype(np.int64)
    q["X"] = np.concatenate([p["X"][bl[i][2]] for i in perm])
    q["dY"] = np.concatenate([p["dY"][bl[i][2]] for i in perm])
    q["A"] = np.concatenate([p["A"][bl[i][3]] for i in perm])
    q["B"] = np.concatenate([p["B"][bl[i][3]] for i in perm])
    o2 = run(q)
    assert np.array_equal(o2["Y"], np.concatenate([out["Y"][bl[i][2]] for i in perm]))
    assert np.array_equal(o2["dX"], np.concatenate([out["dX"][bl[i][2]] for i in perm]))
    assert np.array_equal(o2["dA"], np.concatenate([out["dA"][bl[i][3]] for i in perm]))
    assert np.array_equal(o2["dB"], np.concatenate([out["dB"][bl[i][3]] for i in perm]))
    assert np.array_equal(o2["H"], np.concatenate([out["H"][bl[i][4]] for i in perm]))


def test_locality_of_one_adapter():
    p = rand_problem(10, counts=(4, 3, 6), ranks=(2, 3, 4), alphas=(2.0, 3.0, 4.0))
    out = run(p)
    bl = blocks(p)
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    rr = bl[1][3]
    q["A"][rr] += 0.25
    q["B"][rr] *= -1.5
    q["alphas"][1] = 7.0
    o2 = run(q)
    for i, s, rows, rr_i, hs, r, n in bl:
        same = i != 1
        assert np.array_equal(o2["Y"][rows], out["Y"][rows]) == same
        assert np.array_equal(o2["dX"][rows], out["dX"][rows]) == same
        assert np.array_equal(o2["dA"][rr_i], out["dA"][rr_i]) == same
        assert np.array_equal(o2["dB"][rr_i], out["dB"][rr_i]) == same


# --------------------------------------------------------------------------
# degenerate cases and validation
# --------------------------------------------------------------------------

def test_empty_tokens():
    p = rand_problem(12, counts=(0, 0), ranks=(3, 2), alphas=(1.0, 2.0))
    out = run(p)
    assert out["Y"].shape == (0, 6) and out["dX"].shape == (0, 7)
    assert out["H"].shape == (0,)
    assert np.array_equal(out["dA"], np.zeros((5, 7)))
    assert np.array_equal(out["dB"], np.zeros((5, 6)))


def test_validation_errors():
    assert oracle.check([0, 3], [2], [1.0], 4, 4) == 0
    assert oracle.check([0], [], [], 4, 4, T=5) == 0  # no adapters: frozen path only
    assert oracle.check([0, 3], [2], [1.0], 4, 4, T=4) == -2  # o_N != T
    assert oracle.check([1, 3], [2], [1.0], 4, 4) == -2  # o_0 != 0
    assert oracle.check([0, 3, 2], [2, 2], [1.0, 1.0], 4, 4) == -2  # decreasing
    assert oracle.check([0, 3], [0], [1.0], 4, 4) == -3
    assert oracle.check([0, 3], [129], [1.0], 4, 4) == -3
    assert oracle.check([0, 3], [2], [float("nan")], 4, 4) == -4
    assert oracle.check([0, 3], [2], [1.0], 0, 4) == -5
    assert oracle.check([0] * 66, [1] * 65, [1.0] * 65, 4, 4) == -6
    with pytest.raises(oracle.OracleError):
        oracle.packed_lora([0, 2], [1], [1.0], 3, 3, X=np.ones((2, 3)), want=("Y",))  # W, B missing


def test_rows_subproblem_matches_full():
    import workloads
    wl = workloads.custom(24, 20, [5, 0, 9, 3], [2, 3, 4, 1], [2.0, 3.0, 8.0, 1.0], dtype="f32")
    inp = workloads.make_inputs(wl)
    full = oracle.run_workload(wl, inp)
    rows = np.array([0, 4, 5, 11, 13, 16])
    sub = oracle.rows_subproblem(wl, inp, rows)
    assert np.array_equal(sub["Y"], full["Y"][rows])
    assert np.array_equal(sub["dX"], full["dX"][rows])
    # per-row H matches the packed block layout
    hoff = np.concatenate([[0], np.cumsum(np.diff(wl.offsets) * wl.ranks)])
    for u, t in enumerate(rows):
        i = int(np.searchsorted(wl.offsets, t, side="right") - 1)
        r = int(wl.ranks[i])
        pos = hoff[i] + (t - wl.offsets[i]) * r
        assert np.array_equal(sub["H"][u, :r], full["H"][pos:pos + r])
