"""fp64 CPU oracle for the Llama-3-8B decoder block around the packed LoRA
projections (RMSNorm, rotary embedding, causal grouped-query attention,
SwiGLU, residual adds), forward and backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the CPU leg of
``bench.py``; the product package never imports it.

What the block is.  The pages fine-tune LLaMA-3 and Qwen-2.5 models [PLoRA
technical summary (gist.science, arXiv 2508.02932), 结果], and LoRA puts a
trainable low-rank branch on the weights of every Transformer block
[LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与PEFT实现];
the pages do not print the block, so its layers follow the public Llama 3
architecture (8B: hidden 4096, 32 query heads and 8 key/value heads of
128, MLP width 14336, RMSNorm eps 1e-5, rotary base 500000), written out from
the definitions:

    h1 = rmsnorm(x) * w1
    q, k, v = h1 Wq, h1 Wk, h1 Wv          (+ each projection's LoRA branch)
    q, k = rope(q), rope(k)                  (position = index within the sequence)
    a = softmax(q k^T / sqrt(128), causal) v    (query head j uses key/value head j // 4)
    x2 = x + a Wo                            (+ LoRA)
    h2 = rmsnorm(x2) * w2
    y = x2 + (silu(h2 Wg) * (h2 Wu)) Wd      (+ LoRA on gate, up, down)

Each backward function below is derived by hand from its forward (chain rule,
no automatic differentiation); ``tests/test_oracle_block.py`` pins them to
PyTorch autograd in float64, finite differences and closed forms.

Storage points.  The GPU keeps activations in bf16 between kernels (the LoRA
activations H, G and the per-row statistics in fp32).  The block oracle
(``block_forward`` / ``block_backward``) takes a ``store`` function applied
wherever a kernel writes a bf16 activation, so that it can either keep fp64
throughout (store = identity) or round where the GPU rounds (store = round to
bf16).  The projections are the packed LoRA operator's own oracle
(``oracle.packed_lora``).  The per-kernel functions take and return fp64
arrays.
"""
from __future__ import annotations

import numpy as np

HIDDEN, N_Q, N_KV, HEAD, MLP = 4096, 32, 8, 128, 14336
RMS_EPS, ROPE_BASE = 1e-5, 500000.0


def identity(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- RMSNorm
def rmsnorm_fwd(x, w, eps=RMS_EPS):
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis; returns (y, rstd)."""
    x = np.asarray(x, np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * rstd[..., None] * np.asarray(w, np.float64), rstd


def rmsnorm_bwd(dy, x, w, rstd):
    """dx for y = x * rstd * w with rstd = (mean(x^2) + eps)^(-1/2) (w frozen):
    d rstd / d x_j = -rstd^3 x_j / n, so dx = rstd * g - x * rstd^3 * mean(g * x), g = dy * w."""
    x = np.asarray(x, np.float64)
    g = np.asarray(dy, np.float64) * np.asarray(w, np.float64)
    r = rstd[..., None]
    return r * g - x * r ** 3 * np.mean(g * x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- rotary embedding
def rope_angles(positions, head=HEAD, base=ROPE_BASE):
    """angle[t, i] = pos_t * base^(-2i/head), i < head/2."""
    inv = base ** (-np.arange(0, head, 2, dtype=np.float64) / head)
    return np.asarray(positions, np.float64)[:, None] * inv[None, :]


def rope_fwd(x, positions, head=HEAD, base=ROPE_BASE):
    """Rotate the pairs (i, i + head/2) of every head of x [T, heads * head] by angle[t, i]."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    xh = x.reshape(T, -1, head)
    ang = rope_angles(positions, head, base)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = xh[..., : head // 2], xh[..., head // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1).reshape(T, -1)


def rope_bwd(dy, positions, head=HEAD, base=ROPE_BASE):
    """The rotation is orthogonal: its adjoint is the rotation by the opposite angle."""
    dy = np.asarray(dy, np.float64)
    T = dy.shape[0]
    dh = dy.reshape(T, -1, head)
    ang = rope_angles(positions, head, base)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = dh[..., : head // 2], dh[..., head // 2:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1).reshape(T, -1)


def positions_of(seq_offsets):
    """Index of every token within its sequence."""
    off = np.asarray(seq_offsets, np.int64)
    pos = np.empty(int(off[-1]), np.int64)
    for a, b in zip(off[:-1], off[1:]):
        pos[a:b] = np.arange(b - a)
    return pos


# ---------------------------------------------------------------- attention
def attention_fwd(q, k, v, seq_offsets, n_q=N_Q, n_kv=N_KV, head=HEAD):
    """Causal grouped-query attention per sequence.  q [T, n_q*head], k, v
    [T, n_kv*head]; query head j reads key/value head j // (n_q / n_kv).
    Returns (o [T, n_q*head], lse [n_q, T]) with lse the log-sum-exp of the
    scaled scores of each query row."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    T = q.shape[0]
    grp = n_q // n_kv
    scale = 1.0 / np.sqrt(head)
    o = np.zeros((T, n_q * head))
    lse = np.zeros((n_q, T))
    for a, b in zip(seq_offsets[:-1], seq_offsets[1:]):
        n = b - a
        if n == 0:
            continue
        mask = np.tril(np.ones((n, n), bool))
        for j in range(n_q):
            g = j // grp
            Q = q[a:b, j * head:(j + 1) * head]
            K = k[a:b, g * head:(g + 1) * head]
            V = v[a:b, g * head:(g + 1) * head]
            S = np.where(mask, Q @ K.T * scale, -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            Z = E.sum(axis=1, keepdims=True)
            o[a:b, j * head:(j + 1) * head] = (E / Z) @ V
            lse[j, a:b] = (m + np.log(Z))[:, 0]
    return o, lse


def attention_bwd(do, q, k, v, o, lse, seq_offsets, n_q=N_Q, n_kv=N_KV, head=HEAD):
    """Gradients of attention_fwd: with P = exp(S - lse), dV = P^T dO,
    dP = dO V^T, dS = P * (dP - rowsum(dO * O)), dQ = scale dS K, dK = scale dS^T Q
    (key/value gradients summed over the query heads of their group)."""
    do, q, k, v, o = (np.asarray(a, np.float64) for a in (do, q, k, v, o))
    T = q.shape[0]
    grp = n_q // n_kv
    scale = 1.0 / np.sqrt(head)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a, b in zip(seq_offsets[:-1], seq_offsets[1:]):
        n = b - a
        if n == 0:
            continue
        mask = np.tril(np.ones((n, n), bool))
        for j in range(n_q):
            g = j // grp
            hs, gs = slice(j * head, (j + 1) * head), slice(g * head, (g + 1) * head)
            Q, K, V = q[a:b, hs], k[a:b, gs], v[a:b, gs]
            dO, O = do[a:b, hs], o[a:b, hs]
            P = np.where(mask, np.exp(Q @ K.T * scale - lse[j, a:b][:, None]), 0.0)
            dv[a:b, gs] += P.T @ dO
            dP = dO @ V.T
            Dr = np.sum(dO * O, axis=1, keepdims=True)
            dS = P * (dP - Dr)
            dq[a:b, hs] = scale * dS @ K
            dk[a:b, gs] += scale * dS.T @ Q
    return dq, dk, dv


# ---------------------------------------------------------------- SwiGLU
def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swiglu_fwd(g, u):
    """silu(g) * u with silu(g) = g * sigmoid(g)."""
    g, u = np.asarray(g, np.float64), np.asarray(u, np.float64)
    return g * _sigmoid(g) * u


def swiglu_bwd(da, g, u):
    """d/du = silu(g); d/dg = u * sigmoid(g) * (1 + g (1 - sigmoid(g)))."""
    da, g, u = (np.asarray(a, np.float64) for a in (da, g, u))
    sg = _sigmoid(g)
    return da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg


# ---------------------------------------------------------------- the block
PROJ = ("q", "k", "v", "o", "g", "u", "d")


def proj_dims(hidden, n_q, n_kv, mlp, head=HEAD):
    """(d_in, d_out) of every packed projection."""
    return {"q": (hidden, n_q * head), "k": (hidden, n_kv * head), "v": (hidden, n_kv * head),
            "o": (n_q * head, hidden), "g": (hidden, mlp), "u": (hidden, mlp), "d": (mlp, hidden)}


def _proj(p, name, seg, want, **kw):
    from . import packed_lora
    d_in, d_out = p["dims"][name]
    return packed_lora(seg, p["ranks"], p["alphas"], d_in, d_out, W=p["W"][name], A=p["A"][name], B=p["B"][name],
                       want=want, **kw)


def store32(a):
    """What an fp32 buffer holds."""
    return np.asarray(a, np.float32).astype(np.float64)


def block_forward(p, x, seg, seq, store=identity, eps=RMS_EPS, store_f32=store32):
    """Forward of the block; returns (out, cache).  p: dict with "w1", "w2"
    (norm weights), "W", "A", "B" (per projection: frozen weight [d_out, d_in],
    packed A [R, d_in], packed B [R, d_out]), "ranks", "alphas", "dims",
    "n_q", "n_kv".  seg: adapter segment offsets; seq: sequence offsets.
    store_f32 is applied where the GPU keeps fp32 (H, rstd, lse)."""
    c = {"x": np.asarray(x, np.float64)}
    h1, r1 = rmsnorm_fwd(x, p["w1"], eps)
    c["h1"], c["r1"] = store(h1), store_f32(r1)
    for n in ("q", "k", "v"):
        r = _proj(p, n, seg, ("Y", "H"), X=c["h1"])
        c[n], c["H" + n] = store(r["Y"]), store_f32(r["H"])
    pos = positions_of(seq)
    c["qr"], c["kr"] = store(rope_fwd(c["q"], pos)), store(rope_fwd(c["k"], pos))
    att, lse = attention_fwd(c["qr"], c["kr"], c["v"], seq, p["n_q"], p["n_kv"])
    c["att"], c["lse"] = store(att), store_f32(lse)
    r = _proj(p, "o", seg, ("Y", "H"), X=c["att"])
    c["o"], c["Ho"] = store(r["Y"]), store_f32(r["H"])
    c["x2"] = store(c["x"] + c["o"])
    h2, r2 = rmsnorm_fwd(c["x2"], p["w2"], eps)
    c["h2"], c["r2"] = store(h2), store_f32(r2)
    for n in ("g", "u"):
        r = _proj(p, n, seg, ("Y", "H"), X=c["h2"])
        c[n], c["H" + n] = store(r["Y"]), store_f32(r["H"])
    c["a"] = store(swiglu_fwd(c["g"], c["u"]))
    r = _proj(p, "d", seg, ("Y", "H"), X=c["a"])
    c["dd_out"], c["Hd"] = store(r["Y"]), store_f32(r["H"])
    out = store(c["x2"] + c["dd_out"])
    return out, c


def block_backward(p, c, dout, seg, seq, store=identity, keep=None):
    """Backward of the block from the forward's cache; returns (dx, grads)
    with grads[name] = (dA, dB) for every projection (fp64).  keep: an
    optional dict that receives the gradient entering the attention
    ("datt") and the attention's outputs before the rotary adjoint ("dq",
    "dk", "dv")."""
    dout = np.asarray(dout, np.float64)
    grads = {}

    def bwd(name, X, dY, H):
        dX = store(_proj(p, name, seg, ("dX",), dY=dY)["dX"])
        w = _proj(p, name, seg, ("dA", "dB"), X=X, dY=dY)  # the oracle recomputes H and G itself
        grads[name] = (w["dA"], w["dB"])
        return dX

    da = bwd("d", c["a"], dout, c["Hd"])
    dg, du = swiglu_bwd(da, c["g"], c["u"])
    dg, du = store(dg), store(du)
    dh2 = bwd("g", c["h2"], dg, c["Hg"]) + bwd("u", c["h2"], du, c["Hu"])
    dx2 = store(dout + rmsnorm_bwd(dh2, c["x2"], p["w2"], c["r2"]))
    datt = bwd("o", c["att"], dx2, c["Ho"])
    dq, dk, dv = attention_bwd(datt, c["qr"], c["kr"], c["v"], c["att"], c["lse"], seq, p["n_q"], p["n_kv"])
    if keep is not None:
        keep.update(datt=datt, dq=dq, dk=dk, dv=dv)
    pos = positions_of(seq)
    dq, dk, dv = store(rope_bwd(store(dq), pos)), store(rope_bwd(store(dk), pos)), store(dv)
    dh1 = bwd("q", c["h1"], dq, c["Hq"]) + bwd("k", c["h1"], dk, c["Hk"]) + bwd("v", c["h1"], dv, c["Hv"])
    dx = store(dx2 + rmsnorm_bwd(dh1, c["x"], p["w1"], c["r1"]))
    return dx, grads
