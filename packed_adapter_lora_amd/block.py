"""One Llama-3 decoder block with packed multi-LoRA adapters on all seven
projections, forward and backward, built from the library's kernels.

The pages fine-tune LLaMA-3 models with LoRA on the projections of every
Transformer block [PLoRA technical summary (gist.science, arXiv 2508.02932),
结果; LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与
PEFT实现].  This module only sequences C-ABI calls and allocates their buffers
(torch tensors on the current device); every step runs in the library's
kernels (include/plora.h, include/plora_block.h):

    h1 = rmsnorm(x) w1;  q, k, v = packed projections of h1;  rope(q), rope(k)
    att = causal GQA attention;  x2 = x + proj_o(att);  h2 = rmsnorm(x2) w2
    out = x2 + proj_d(silu(proj_g(h2)) * proj_u(h2))

The adapters are the same on every projection (one rank and alpha per
adapter, as one PEFT LoRA config targets all the modules); each projection has
its own packed A and B.  The projections that read one input (q, k, v from h1;
gate and up from h2) share one pass over it for their LoRA shrinks and their
dA gradients (plora_shrink_shared, plora_backward_dA_shared); their GEMMs and
dB gradients run per projection.  The down projection's dX goes straight
into the SwiGLU backward (plora_backward_dx_swiglu: its GEMM writes the
gradients of gate and up, not dX).
"""
from __future__ import annotations

import numpy as np

from . import (Desc, plora_add, plora_attention_bwd, plora_attention_fwd, plora_backward_dA_shared,
               plora_backward_dAdB, plora_backward_dx, plora_backward_dx_swiglu, plora_forward, plora_forward_expand,
               plora_h_elems, plora_rmsnorm_bwd, plora_rmsnorm_fwd, plora_rope, plora_shrink_shared,
               plora_swiglu_fwd, plora_workspace_bytes, plora_workspace_bytes_dA_shared)

PROJ = ("q", "k", "v", "o", "g", "u", "d")


def proj_dims(hidden, n_q, n_kv, mlp, head=128):
    return {"q": (hidden, n_q * head), "k": (hidden, n_kv * head), "v": (hidden, n_kv * head),
            "o": (n_q * head, hidden), "g": (hidden, mlp), "u": (hidden, mlp), "d": (mlp, hidden)}


class DecoderBlock:
    """params: dict with "w1", "w2" (bf16 [hidden]), "W", "A", "B" (dicts over
    PROJ of bf16 tensors [d_out, d_in], [R, d_in], [R, d_out]).  seg_offsets:
    adapter segments (host int64, N + 1); seq_offsets: sequences (host int64)."""

    def __init__(self, params, seg_offsets, ranks, alphas, seq_offsets, hidden=4096, n_q=32, n_kv=8, mlp=14336,
                 eps=1e-5, rope_base=500000.0):
        import torch
        self.torch = torch
        self.p = params
        self.seg = np.ascontiguousarray(seg_offsets, np.int64)
        self.seq = np.ascontiguousarray(seq_offsets, np.int64)
        self.T = int(self.seg[-1])
        if int(self.seq[-1]) != self.T:
            raise ValueError("sequence and adapter offsets must cover the same tokens")
        self.hidden, self.n_q, self.n_kv, self.mlp = hidden, n_q, n_kv, mlp
        self.eps, self.base = eps, rope_base
        self.dims = proj_dims(hidden, n_q, n_kv, mlp)
        self.desc = {n: Desc(self.seg, ranks, alphas, di, do, "bf16") for n, (di, do) in self.dims.items()}
        self.he = plora_h_elems(self.desc["q"])
        nb = max([plora_workspace_bytes(d) for d in self.desc.values()] +
                 [plora_workspace_bytes_dA_shared(self.desc["q"], 3), plora_workspace_bytes_dA_shared(self.desc["g"], 2)])
        self.ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device="cuda")
        self.cache = {}

    def _bf(self, *shape):
        return self.torch.empty(shape, dtype=self.torch.bfloat16, device="cuda")

    def _f32(self, *shape):
        return self.torch.empty(shape, dtype=self.torch.float32, device="cuda")

    def _shared_forward(self, names, X, c, stream):
        """The projections `names` of one input X: one shrink pass for all
        their H, then each projection's GEMM with its fused expand."""
        p, T = self.p, self.T
        for n in names:
            c[n], c["H" + n] = self._bf(T, self.dims[n][1]), self._f32(max(self.he, 4))[:self.he]
        if self.he:
            plora_shrink_shared(self.desc[names[0]], X, [p["A"][n] for n in names], [c["H" + n] for n in names], stream)
        for n in names:
            plora_forward_expand(self.desc[n], X, p["W"][n], p["B"][n], c[n], c["H" + n], stream)

    def forward(self, x, stream=None):
        """x: bf16 [T, hidden].  Returns the block output; keeps what the backward needs."""
        p, T, c = self.p, self.T, {}
        c["x"] = x
        c["h1"], c["r1"] = self._bf(T, self.hidden), self._f32(T)
        plora_rmsnorm_fwd(x, p["w1"], c["h1"], c["r1"], eps=self.eps, stream=stream)
        self._shared_forward(("q", "k", "v"), c["h1"], c, stream)
        plora_rope(c["q"], self.seq, self.n_q, self.base, stream=stream)  # in place: q and k are now rotated
        plora_rope(c["k"], self.seq, self.n_kv, self.base, stream=stream)
        c["att"], c["lse"] = self._bf(T, self.n_q * 128), self._f32(self.n_q, T)
        plora_attention_fwd(c["q"], c["k"], c["v"], c["att"], c["lse"], self.seq, self.n_q, self.n_kv, stream)
        o, c["Ho"] = self._bf(T, self.hidden), self._f32(max(self.he, 4))[:self.he]
        plora_forward(self.desc["o"], c["att"], p["W"]["o"], p["A"]["o"], p["B"]["o"], o, c["Ho"], stream)
        c["x2"], c["h2"], c["r2"] = self._bf(T, self.hidden), self._bf(T, self.hidden), self._f32(T)
        plora_rmsnorm_fwd(x, p["w2"], c["h2"], c["r2"], res=o, xs_out=c["x2"], eps=self.eps, stream=stream)
        self._shared_forward(("g", "u"), c["h2"], c, stream)
        c["a"] = self._bf(T, self.mlp)
        plora_swiglu_fwd(c["g"], c["u"], c["a"], stream)
        d, c["Hd"] = self._bf(T, self.hidden), self._f32(max(self.he, 4))[:self.he]
        plora_forward(self.desc["d"], c["a"], p["W"]["d"], p["A"]["d"], p["B"]["d"], d, c["Hd"], stream)
        out = self._bf(T, self.hidden)
        plora_add(c["x2"], d, out, stream)
        self.cache = c
        return out

    def backward(self, dout, stream=None, keep=False):
        """dout: bf16 [T, hidden].  Returns (dx, grads) with grads[name] =
        (dA, dB) fp32 for every projection.  keep: also hold the gradient
        entering the attention ("datt"), the attention's input gradients after
        the rotary adjoint ("dq", "dk", "dv") and the residual-stream gradient
        below the MLP ("dx2") in self.cache["bwd"]."""
        p, T, c = self.p, self.T, self.cache
        grads = {}
        R = int(self.desc["q"].R)

        Gs = {}

        def bwd(n, X, dY, H, with_dA=True):
            """dX, G and dB of projection n (and dA unless it is left to a
            shared pass over X)."""
            dX, G = self._bf(T, self.dims[n][0]), self._f32(max(self.he, 4))[:self.he]
            plora_backward_dx(self.desc[n], dY, p["W"][n], p["A"][n], p["B"][n], dX, G, stream)
            dA, dB = self._f32(R, self.dims[n][0]), self._f32(R, self.dims[n][1])
            plora_backward_dAdB(self.desc[n], X if with_dA else None, dY, H, G if with_dA else None,
                                dA if with_dA else None, dB, self.ws, stream)
            grads[n] = (dA, dB)
            Gs[n] = G
            return dX

        def shared_dA(names, X):
            plora_backward_dA_shared(self.desc[names[0]], X, [Gs[n] for n in names], [grads[n][0] for n in names],
                                     self.ws, stream)

        # down projection: its dX goes straight into the SwiGLU backward (dg, du)
        n = "d"
        dg, du, G = self._bf(T, self.mlp), self._bf(T, self.mlp), self._f32(max(self.he, 4))[:self.he]
        plora_backward_dx_swiglu(self.desc[n], dout, p["W"][n], p["A"][n], p["B"][n], c["g"], c["u"], dg, du, G,
                                 stream)
        dA, dB = self._f32(R, self.dims[n][0]), self._f32(R, self.dims[n][1])
        plora_backward_dAdB(self.desc[n], c["a"], dout, c["Hd"], G, dA, dB, self.ws, stream)
        grads[n], Gs[n] = (dA, dB), G
        dh2g = bwd("g", c["h2"], dg, c["Hg"], with_dA=False)
        dh2u = bwd("u", c["h2"], du, c["Hu"], with_dA=False)
        shared_dA(("g", "u"), c["h2"])
        dx2 = self._bf(T, self.hidden)
        plora_rmsnorm_bwd([dh2g, dh2u], c["x2"], p["w2"], c["r2"], dx2, dres=dout, stream=stream)
        datt = bwd("o", c["att"], dx2, c["Ho"])
        dq, dk, dv = self._bf(T, self.n_q * 128), self._bf(T, self.n_kv * 128), self._bf(T, self.n_kv * 128)
        delta = self._f32(self.n_q, T)
        plora_attention_bwd(c["q"], c["k"], c["v"], c["att"], c["lse"], datt, dq, dk, dv, delta, self.seq, self.n_q,
                            self.n_kv, stream)
        plora_rope(dq, self.seq, self.n_q, self.base, inverse=True, stream=stream)
        plora_rope(dk, self.seq, self.n_kv, self.base, inverse=True, stream=stream)
        dh1 = [bwd(n, c["h1"], dn, c["H" + n], with_dA=False) for n, dn in (("q", dq), ("k", dk), ("v", dv))]
        shared_dA(("q", "k", "v"), c["h1"])
        dx = self._bf(T, self.hidden)
        plora_rmsnorm_bwd(dh1, c["x"], p["w1"], c["r1"], dx, dres=dx2, stream=stream)
        if keep:
            c["bwd"] = {"datt": datt, "dq": dq, "dk": dk, "dv": dv, "dx2": dx2}
        return dx, grads
