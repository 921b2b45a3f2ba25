"""Pins of the decoder-block oracle (CPU only).

Every pin comes from outside ``oracle/block.py``: PyTorch's own RMSNorm,
scaled-dot-product attention and SiLU in float64 with autograd for the
gradients, the relative-position property and orthogonality of the rotary
embedding, closed forms (one-token attention returns v; RMSNorm is
scale-invariant), and adjoint identities.  The last test plants mistakes in
copies of ``oracle/block.py`` and checks that each fails a pin.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle import block as OB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
torch = pytest.importorskip("torch")
F = torch.nn.functional


def t64(a, grad=False):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, requires_grad=grad)


def pin_rmsnorm_torch(mod):
    rng = np.random.default_rng(1)
    x, w, dy = rng.standard_normal((5, 24)) * 3, rng.standard_normal(24), rng.standard_normal((5, 24))
    y, rstd = mod.rmsnorm_fwd(x, w, eps=1e-5)
    xt = t64(x, True)
    yt = F.rms_norm(xt, (24,), t64(w), eps=1e-5)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-13)
    yt.backward(t64(dy))
    np.testing.assert_allclose(mod.rmsnorm_bwd(dy, x, w, rstd), xt.grad.numpy(), rtol=1e-11, atol=1e-12)


def pin_rmsnorm_closed_forms(mod):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 16))
    y, _ = mod.rmsnorm_fwd(x, np.ones(16), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-13)  # unit RMS
    y2, _ = mod.rmsnorm_fwd(7.5 * x, np.ones(16), eps=0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13)  # scale invariance
    # scale invariance makes the gradient orthogonal to x
    _, r = mod.rmsnorm_fwd(x, np.ones(16), eps=0.0)
    dx = mod.rmsnorm_bwd(rng.standard_normal((3, 16)), x, np.ones(16), r)
    np.testing.assert_allclose(np.sum(dx * x, axis=1), 0.0, atol=1e-12)


def pin_rope_properties(mod):
    rng = np.random.default_rng(3)
    head, heads = 8, 2
    x = rng.standard_normal((6, heads * head))
    np.testing.assert_allclose(mod.rope_fwd(x[:1], [0], head=head), x[:1], rtol=0, atol=1e-15)  # position 0
    # rotation: norms of every pair are kept, and scores depend only on the position difference
    q, k = rng.standard_normal((1, head)), rng.standard_normal((1, head))
    dots = [float((mod.rope_fwd(q, [m], head=head) @ mod.rope_fwd(k, [n], head=head).T)[0, 0])
            for m, n in ((5, 2), (103, 100), (3, 0))]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)
    y = mod.rope_fwd(x, np.arange(6) * 37, head=head)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # the lower half rotates into the upper one with the documented frequencies: one pair by hand
    th = 11 * 500000.0 ** (-2 * 1 / head)
    e = np.zeros((1, head))
    e[0, 1] = 1.0
    r = mod.rope_fwd(e, [11], head=head)
    np.testing.assert_allclose([r[0, 1], r[0, 1 + head // 2]], [np.cos(th), np.sin(th)], rtol=1e-13)


def pin_rope_adjoint(mod):
    rng = np.random.default_rng(4)
    x, dy = rng.standard_normal((5, 32)), rng.standard_normal((5, 32))
    pos = [0, 1, 7, 500, 1023]
    lhs = np.sum(dy * mod.rope_fwd(x, pos, head=16))
    rhs = np.sum(mod.rope_bwd(dy, pos, head=16) * x)
    assert abs(lhs - rhs) < 1e-12 * (abs(lhs) + 1)
    np.testing.assert_allclose(mod.rope_bwd(mod.rope_fwd(x, pos, head=16), pos, head=16), x, atol=1e-13)


def _sdpa(q, k, v, offs, n_q, n_kv, head):
    """PyTorch's scaled_dot_product_attention per sequence (float64, causal, kv heads repeated)."""
    T = q.shape[0]
    outs = []
    for a, b in zip(offs[:-1], offs[1:]):
        qh = q[a:b].reshape(b - a, n_q, head).transpose(0, 1)
        kh = k[a:b].reshape(b - a, n_kv, head).transpose(0, 1).repeat_interleave(n_q // n_kv, dim=0)
        vh = v[a:b].reshape(b - a, n_kv, head).transpose(0, 1).repeat_interleave(n_q // n_kv, dim=0)
        outs.append(F.scaled_dot_product_attention(qh, kh, vh, is_causal=True).transpose(0, 1).reshape(b - a, -1))
    return torch.cat(outs, 0) if outs else torch.zeros(T, n_q * head, dtype=torch.float64)


def pin_attention_torch(mod):
    rng = np.random.default_rng(5)
    n_q, n_kv, head = 4, 2, 8
    offs = [0, 5, 6, 13]
    T = offs[-1]
    q, k, v = (rng.standard_normal((T, n * head)) for n in (n_q, n_kv, n_kv))
    do = rng.standard_normal((T, n_q * head))
    o, lse = mod.attention_fwd(q, k, v, offs, n_q, n_kv, head)
    qt, kt, vt = t64(q, True), t64(k, True), t64(v, True)
    ot = _sdpa(qt, kt, vt, offs, n_q, n_kv, head)
    np.testing.assert_allclose(o, ot.detach().numpy(), rtol=1e-11, atol=1e-12)
    ot.backward(t64(do))
    dq, dk, dv = mod.attention_bwd(do, q, k, v, o, lse, offs, n_q, n_kv, head)
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-11)
    # log-sum-exp of the scaled causal scores, from torch.logsumexp
    j, a = 3, 6
    S = t64(q[a:, j * head:(j + 1) * head]) @ t64(k[a:, (j // 2) * head:(j // 2 + 1) * head]).T / np.sqrt(head)
    S = S.masked_fill(~torch.ones(7, 7, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(lse[j, a:], torch.logsumexp(S, dim=1).numpy(), rtol=1e-12)


def pin_attention_closed_forms(mod):
    rng = np.random.default_rng(6)
    n_q, n_kv, head = 4, 1, 8
    q, k, v = rng.standard_normal((1, 32)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    o, lse = mod.attention_fwd(q, k, v, [0, 1], n_q, n_kv, head)
    np.testing.assert_allclose(o, np.tile(v, (1, 4)), rtol=1e-14)  # one token: o = v for every head
    # identical keys: uniform weights over the visible prefix -> running mean of v
    T = 5
    q, v = rng.standard_normal((T, 32)), rng.standard_normal((T, 8))
    k = np.tile(rng.standard_normal((1, 8)), (T, 1))
    o, _ = mod.attention_fwd(q, k, v, [0, T], n_q, n_kv, head)
    mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o[:, 16:24], mean, rtol=1e-12)


def pin_swiglu_torch(mod):
    rng = np.random.default_rng(7)
    g, u, da = (rng.standard_normal((4, 9)) * 4 for _ in range(3))
    gt, ut = t64(g, True), t64(u, True)
    at = F.silu(gt) * ut
    np.testing.assert_allclose(mod.swiglu_fwd(g, u), at.detach().numpy(), rtol=1e-13)
    at.backward(t64(da))
    dg, du = mod.swiglu_bwd(da, g, u)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(du, ut.grad.numpy(), rtol=1e-12, atol=1e-14)


def pin_positions(mod):
    np.testing.assert_array_equal(mod.positions_of([0, 3, 3, 5]), [0, 1, 2, 0, 1])


PINS = [pin_rmsnorm_torch, pin_rmsnorm_closed_forms, pin_rope_properties, pin_rope_adjoint, pin_attention_torch,
        pin_attention_closed_forms, pin_swiglu_torch, pin_positions]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_block_oracle_pin(pin):
    pin(OB)


MUTANTS = {
    "rms_mean_to_sum": ("np.mean(x * x, axis=-1) + eps", "np.sum(x * x, axis=-1) + eps"),
    "rms_bwd_drop_term": ("return r * g - x * r ** 3 * np.mean(g * x, axis=-1, keepdims=True)", "return r * g"),
    "rope_sign": ("[lo * c - hi * s, hi * c + lo * s]", "[lo * c + hi * s, hi * c - lo * s]"),
    "rope_freq": ("inv = base ** (-np.arange(0, head, 2, dtype=np.float64) / head)",
                  "inv = base ** (-np.arange(0, head // 2, dtype=np.float64) / head)"),
    "rope_bwd_same_rotation": ("[lo * c + hi * s, hi * c - lo * s]", "[lo * c - hi * s, hi * c + lo * s]"),
    "attn_no_mask": ("S = np.where(mask, Q @ K.T * scale, -np.inf)", "S = Q @ K.T * scale"),
    "attn_no_scale": ("scale = 1.0 / np.sqrt(head)\n    o = np.zeros", "scale = 1.0\n    o = np.zeros"),
    "attn_kv_head": ("            g = j // grp\n            Q = q", "            g = j % n_kv\n            Q = q"),
    "attn_bwd_no_D": ("dS = P * (dP - Dr)", "dS = P * dP"),
    "attn_bwd_dk_transpose": ("dk[a:b, gs] += scale * dS.T @ Q", "dk[a:b, gs] += scale * dS @ Q"),
    "swiglu_bwd_sig": ("(1.0 + g * (1.0 - sg))", "(1.0 + g * sg)"),
    "positions_global": ("pos[a:b] = np.arange(b - a)", "pos[a:b] = np.arange(a, b)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_pins_catch_planted_mistakes(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "block.py")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / ("block_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("block_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, RuntimeError):
            failed += 1
    assert failed > 0, "planted mistake %s passed every pin" % name


# ---------------------------------------------------------------- the composed block
def small_block(seed=9, hidden=512, n_q=4, n_kv=1, mlp=96, ranks=(4, 8, 2), alphas=(8.0, 8.0, 4.0)):
    rng = np.random.default_rng(seed)
    dims = OB.proj_dims(hidden, n_q, n_kv, mlp)
    R = sum(ranks)
    p = {"w1": 1 + 0.1 * rng.standard_normal(hidden), "w2": 1 + 0.1 * rng.standard_normal(hidden),
         "W": {}, "A": {}, "B": {}, "ranks": np.array(ranks), "alphas": np.array(alphas), "dims": dims,
         "n_q": n_q, "n_kv": n_kv}
    for n, (di, do) in dims.items():
        p["W"][n] = rng.standard_normal((do, di)) / np.sqrt(di)
        p["A"][n] = rng.standard_normal((R, di)) / np.sqrt(4)
        p["B"][n] = rng.standard_normal((R, do)) * 0.2
    return p


def torch_block(p, x, seg, seq):
    """The same block written with PyTorch float64 ops (rms_norm, SDPA, silu,
    plain matrix products per adapter segment) for autograd."""
    n_q, n_kv = p["n_q"], p["n_kv"]
    W = {n: t64(p["W"][n]) for n in OB.PROJ}
    A = {n: t64(p["A"][n], True) for n in OB.PROJ}
    B = {n: t64(p["B"][n], True) for n in OB.PROJ}

    def proj(n, X):
        Y = X @ W[n].T
        parts, ro = [], 0
        for i, r in enumerate(p["ranks"]):
            a, b = seg[i], seg[i + 1]
            s = float(p["alphas"][i]) / r
            parts.append(Y[a:b] + s * (X[a:b] @ A[n][ro:ro + r].T) @ B[n][ro:ro + r])
            ro += r
        return torch.cat(parts, 0)

    def rope(t):
        T = t.shape[0]
        pos = torch.tensor(OB.positions_of(seq), dtype=torch.float64)
        inv = 500000.0 ** (-torch.arange(0, 128, 2, dtype=torch.float64) / 128)
        ang = (pos[:, None] * inv[None, :])[:, None, :]
        th = t.reshape(T, -1, 128)
        lo, hi = th[..., :64], th[..., 64:]
        return torch.cat([lo * torch.cos(ang) - hi * torch.sin(ang), hi * torch.cos(ang) + lo * torch.sin(ang)],
                         -1).reshape(T, -1)

    xt = t64(x, True)
    h1 = F.rms_norm(xt, (xt.shape[1],), t64(p["w1"]), eps=1e-5)
    q, k, v = rope(proj("q", h1)), rope(proj("k", h1)), proj("v", h1)
    att = _sdpa(q, k, v, seq, n_q, n_kv, 128)
    x2 = xt + proj("o", att)
    h2 = F.rms_norm(x2, (x2.shape[1],), t64(p["w2"]), eps=1e-5)
    out = x2 + proj("d", F.silu(proj("g", h2)) * proj("u", h2))
    return out, xt, A, B


def test_block_oracle_matches_torch_autograd():
    p = small_block()
    seg, seq = [0, 40, 40, 70], [0, 25, 40, 70]
    rng = np.random.default_rng(10)
    x, dout = rng.standard_normal((70, 512)), rng.standard_normal((70, 512))
    out, cache = OB.block_forward(p, x, seg, seq, store_f32=OB.identity)  # fp64 throughout
    ot, xt, At, Bt = torch_block(p, x, seg, seq)
    np.testing.assert_allclose(out, ot.detach().numpy(), rtol=1e-10, atol=1e-10)
    ot.backward(t64(dout))
    dx, grads = OB.block_backward(p, cache, dout, seg, seq)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-9, atol=1e-10)
    for n in OB.PROJ:
        np.testing.assert_allclose(grads[n][0], At[n].grad.numpy(), rtol=1e-9, atol=1e-10, err_msg="dA " + n)
        np.testing.assert_allclose(grads[n][1], Bt[n].grad.numpy(), rtol=1e-9, atol=1e-10, err_msg="dB " + n)
