"""fp64 CPU oracle for the per-adapter AdamW update of packed LoRA panels.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and by the CPU leg of
``bench.py``; the product package never imports it and it imports nothing of
the product.

What it computes.  The fine-tuning loop on the PEFT page trains the LoRA
parameters with ``torch.optim.AdamW`` at lr = 1e-3 and PyTorch's other
defaults [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 5. 设定优化器和正则项];
PLoRA packs jobs whose configurations differ in learning rate among other
things [PLoRA technical summary (gist.science, arXiv 2508.02932), 结果], so
every adapter has its own learning rate, weight decay and step count.  The
update is AdamW with decoupled weight decay (Loshchilov & Hutter, "Decoupled
Weight Decay Regularization", ICLR 2019, Algorithm 2, in the form PyTorch
documents for ``torch.optim.AdamW``), applied to one adapter's rows of the
packed A (or B) panel, all in fp64:

    p <- p (1 - lr wd)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

A step count of 0 means the adapter is not trained in this call: its
parameters and moments are left as they are.

Pins (``tests/test_oracle_adamw.py``): PyTorch's own AdamW in float64 over
several steps with per-group hyper-parameters; the constant-gradient closed
form (bias correction makes m_hat = g and v_hat = g^2 exactly); pure decay under
a zero gradient; the skip rule.  ``tests/test_oracle_adamw.py`` also plants
mistakes in copies of this file and shows each fails a pin.
"""
from __future__ import annotations

import numpy as np


def adamw_block(p, m, v, g, lr, weight_decay, step, beta1=0.9, beta2=0.999, eps=1e-8):
    """One AdamW update of one parameter block; returns new (p, m, v) in fp64."""
    p = np.array(p, dtype=np.float64)
    m = np.array(m, dtype=np.float64)
    v = np.array(v, dtype=np.float64)
    if step == 0:
        return p, m, v
    g = np.asarray(g, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def adamw_packed(ranks, lrs, weight_decays, steps, p, m, v, g, beta1=0.9, beta2=0.999, eps=1e-8):
    """AdamW over a packed panel [R, D]: adapter i owns rows R_off[i] .. R_off[i] + r_i - 1."""
    p = np.array(p, dtype=np.float64)
    m = np.array(m, dtype=np.float64)
    v = np.array(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    row = 0
    for i, r in enumerate(ranks):
        sl = slice(row, row + int(r))
        p[sl], m[sl], v[sl] = adamw_block(p[sl], m[sl], v[sl], g[sl], float(lrs[i]), float(weight_decays[i]),
                                          int(steps[i]), beta1, beta2, eps)
        row += int(r)
    return p, m, v
