"""Pins of the AdamW oracle (CPU only).

Each pin comes from outside the oracle: PyTorch's own AdamW implementation in
float64, closed forms that follow from the update rule, and the skip rule.
The last test plants plausible mistakes in copies of ``oracle/adamw.py`` and
checks that every one of them fails at least one pin.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle import adamw as OA

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _torch_reference(p0, grads, groups, beta1=0.9, beta2=0.999, eps=1e-8):
    """PyTorch's AdamW (single-tensor path, float64) over several steps.
    groups: list of (row slice, lr, weight_decay)."""
    torch = pytest.importorskip("torch")
    params = [torch.nn.Parameter(torch.tensor(p0[sl], dtype=torch.float64)) for sl, _, _ in groups]
    opt = torch.optim.AdamW([{"params": [q], "lr": lr, "weight_decay": wd} for q, (_, lr, wd) in zip(params, groups)],
                            betas=(beta1, beta2), eps=eps, foreach=False)
    for g in grads:
        for q, (sl, _, _) in zip(params, groups):
            q.grad = torch.tensor(g[sl], dtype=torch.float64)
        opt.step()
    out = np.array(p0, dtype=np.float64)
    for q, (sl, _, _) in zip(params, groups):
        out[sl] = q.detach().numpy()
    return out


def _run_oracle(mod, p0, grads, ranks, lrs, wds, first_step=1, **hp):
    p, m, v = np.array(p0), np.zeros_like(p0), np.zeros_like(p0)
    for k, g in enumerate(grads):
        p, m, v = mod.adamw_packed(ranks, lrs, wds, [first_step + k] * len(ranks), p, m, v, g, **hp)
    return p, m, v


def pin_torch(mod):
    rng = np.random.default_rng(11)
    ranks = [3, 5, 2]
    D = 7
    p0 = rng.standard_normal((sum(ranks), D))
    grads = [rng.standard_normal((sum(ranks), D)) * s for s in (1.0, 0.3, 2.0, 1e-3)]
    lrs, wds = [1e-3, 5e-2, 0.2], [0.01, 0.0, 0.1]
    groups, row = [], 0
    for r, lr, wd in zip(ranks, lrs, wds):
        groups.append((slice(row, row + r), lr, wd))
        row += r
    ref = _torch_reference(p0, grads, groups, beta1=0.8, beta2=0.95, eps=1e-6)
    got, _, _ = _run_oracle(mod, p0, grads, ranks, lrs, wds, beta1=0.8, beta2=0.95, eps=1e-6)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def pin_constant_gradient(mod):
    # with a constant gradient the bias-corrected moments are exactly g and g^2,
    # so every step subtracts lr * g / (|g| + eps) after the decay
    g = np.array([[2.0, -0.5, 1e-3, -7.0]])
    p0 = np.array([[1.0, -2.0, 0.5, 3.0]])
    lr, wd, eps = 0.01, 0.1, 1e-8
    p, m, v = np.array(p0), np.zeros_like(p0), np.zeros_like(p0)
    want = np.array(p0)
    for t in range(1, 6):
        p, m, v = mod.adamw_block(p, m, v, g, lr, wd, t, eps=eps)
        want = want * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
        np.testing.assert_allclose(p, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m / (1 - 0.9 ** 5), g, rtol=1e-12)
    np.testing.assert_allclose(v / (1 - 0.999 ** 5), g * g, rtol=1e-12)


def pin_zero_gradient_decay(mod):
    p0 = np.array([[1.5, -4.0], [0.25, 8.0]])
    p, m, v = np.array(p0), np.zeros_like(p0), np.zeros_like(p0)
    for t in range(1, 4):
        p, m, v = mod.adamw_block(p, m, v, np.zeros_like(p0), 0.1, 0.5, t)
    np.testing.assert_allclose(p, p0 * (1 - 0.05) ** 3, rtol=1e-14)
    assert not m.any() and not v.any()


def pin_skip(mod):
    rng = np.random.default_rng(3)
    p0, m0, v0 = rng.standard_normal((5, 4)), rng.standard_normal((5, 4)), rng.random((5, 4))
    g = rng.standard_normal((5, 4))
    p, m, v = mod.adamw_packed([2, 3], [0.1, 0.1], [0.01, 0.01], [0, 4], p0, m0, v0, g)
    np.testing.assert_array_equal(p[:2], p0[:2])
    np.testing.assert_array_equal(m[:2], m0[:2])
    np.testing.assert_array_equal(v[:2], v0[:2])
    assert np.all(p[2:] != p0[2:]) and np.all(m[2:] != m0[2:])


PINS = [pin_torch, pin_constant_gradient, pin_zero_gradient_decay, pin_skip]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_adamw_oracle_pin(pin):
    pin(OA)


MUTANTS = {
    "no_bias_correction_m": ("m_hat = m / (1.0 - beta1 ** step)", "m_hat = m"),
    "no_bias_correction_v": ("v_hat = v / (1.0 - beta2 ** step)", "v_hat = v"),
    "l2_instead_of_decoupled": ("    p = p * (1.0 - lr * weight_decay)\n    m = beta1 * m + (1.0 - beta1) * g",
                                "    g = g + weight_decay * p\n    m = beta1 * m + (1.0 - beta1) * g"),
    "eps_inside_sqrt": ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    "betas_swapped": ("m = beta1 * m + (1.0 - beta1) * g", "m = beta2 * m + (1.0 - beta2) * g"),
    "decay_after_step": ("    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)\n",
                         "    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)\n    p = p * (1.0 - lr * weight_decay)\n"),
    "skip_still_updates_moments": ("    if step == 0:\n        return p, m, v\n", ""),
    "wrong_rows": ("sl = slice(row, row + int(r))", "sl = slice(row, row + int(ranks[0]))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_adamw_pins_catch_planted_mistakes(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "adamw.py")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / ("adamw_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("adamw_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, "planted mistake %s passed every pin" % name
