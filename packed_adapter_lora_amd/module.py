"""PackedLoRALinear: many LoRA adapters on one frozen linear layer, as a
PyTorch module with autograd, over the library's C ABI.

One PEFT LoRA configuration gives an adapter its rank r and scaling alpha
[LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与PEFT实现:
LoraConfig's r and lora_alpha]; the module packs several such adapters, each
serving its own contiguous segment of the token rows, on one frozen weight
[PLoRA technical summary (gist.science, arXiv 2508.02932), 方法论 > 2. LoRA
执行引擎 > 打包 LoRA 算子].  Only the adapters train; the weight is frozen and
gets no gradient [LoRA加速集成方案 (cloud.baidu.com), 四、工作原理 > 3. 反向传播阶段].

This module holds tensors and calls the library; it does no arithmetic of its
own.  Every step runs in the library's kernels:

  forward   plora_forward (writes Y and H; H is saved for the backward)
  backward  plora_backward_dx (dX and G), then plora_backward_dAdB, which
            either writes fresh fp32 gradients (handed to autograd as the
            gradients of the adapter panels) or, when the panels already hold
            .grad, adds to them in place (gradient accumulation in the kernel;
            autograd then receives None for the panels)
  masters   the trainable parameters are fp32 master panels lora_A [R, d_in]
            and lora_B [R, d_out] (row layout of include/plora.h); for bf16
            the operator runs on bf16 copies, written by plora_cast_panels
            when a master has changed (its version counter moved) and by
            plora_adamw_step, which updates masters, moments and copies in one
            pass.

Initialisation follows LoRA's: A Gaussian and B zero, so the branch starts at
zero and the layer starts as the frozen one [深入理解LoRA, same page]; A_i's
draws have variance 1 / r_i.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (AdamwConfig, Desc, plora_adamw_step, plora_backward_dAdB, plora_backward_dx, plora_cast_panels,
               plora_forward, plora_h_elems, plora_workspace_bytes)

__all__ = ["PackedLoRALinear", "PackedLoRAFunction"]


class PackedLoRAFunction(torch.autograd.Function):
    """Y = X W^T + concat_i[ s_i (X[S_i] A_i) B_i ] through the C ABI.

    Inputs: X [T, d_in] (the module's dtype, contiguous), the fp32 master
    panels (autograd routes their gradients; the kernels read the operator
    copies), the module and the descriptor of this call's segments."""

    @staticmethod
    def forward(ctx, X, A_master, B_master, module, desc):
        A_op, B_op = module.operator_panels()
        T, d_out = desc.n_tokens, int(desc.c.d_out)
        Y = torch.empty((T, d_out), dtype=X.dtype, device=X.device)
        he = plora_h_elems(desc) if desc.R else 0
        H = torch.empty((max(he, 4),), dtype=torch.float32, device=X.device)[:he] if desc.R else None
        plora_forward(desc, X, module.weight, A_op, B_op, Y, H)
        ctx.save_for_backward(X, H if H is not None else torch.empty(0, device=X.device))
        ctx.module, ctx.desc, ctx.A_op, ctx.B_op = module, desc, A_op, B_op
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, H = ctx.saved_tensors
        module, desc = ctx.module, ctx.desc
        lora = desc.R > 0
        dY = dY.contiguous()
        dX = torch.empty_like(X)
        G = torch.empty_like(H) if lora else None
        plora_backward_dx(desc, dY, module.weight, ctx.A_op, ctx.B_op, dX, G)
        gA = gB = None
        if lora and (ctx.needs_input_grad[1] or ctx.needs_input_grad[2]):
            nb = plora_workspace_bytes(desc)
            ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=X.device) if nb else None
            pa, pb = module.lora_A, module.lora_B
            if module.fuse_grad_accumulation and (pa.grad is not None or pb.grad is not None):
                # add this call's gradients to .grad in the kernel; a missing
                # one starts from zeros
                for p in (pa, pb):
                    if p.grad is None:
                        p.grad = torch.zeros_like(p)
                plora_backward_dAdB(desc, X, dY, H, G, pa.grad, pb.grad, ws, accumulate=True)
            else:
                gA = torch.empty_like(pa)
                gB = torch.empty_like(pb)
                plora_backward_dAdB(desc, X, dY, H, G, gA, gB, ws)
        return (dX if ctx.needs_input_grad[0] else None), gA, gB, None, None


class PackedLoRALinear(torch.nn.Module):
    """N LoRA adapters (ranks r_i, scalings alpha_i) packed on one frozen linear layer.

    weight   frozen [d_out, d_in] tensor (the nn.Linear weight) on the current
             GPU, bf16 or fp32; it sets the operator's dtype
    ranks    N ranks in 1..128 (N <= 64)
    alphas   N scalings; adapter i's branch is scaled by alpha_i / r_i
    A, B     optional initial panels [R, d_in], [R, d_out] (any float dtype;
             stored as fp32 masters); default: A_i ~ N(0, 1/r_i) drawn with
             `generator`, B = 0
    seg_offsets  optional default segments (N + 1 host ints) for forward()

    forward(x, seg_offsets=None): x [T, d_in] of the weight's dtype, rows of
    adapter i at seg_offsets[i] .. seg_offsets[i+1]-1; returns [T, d_out].

    With fuse_grad_accumulation (default), a backward pass that finds .grad
    already set on the panels adds to it in the kernel instead of returning a
    gradient to autograd; functional torch.autograd.grad() calls on the panels
    therefore need .grad to be None (or fuse_grad_accumulation = False).
    """

    def __init__(self, weight, ranks, alphas, A=None, B=None, seg_offsets=None, generator=None,
                 fuse_grad_accumulation=True):
        super().__init__()
        if weight.dim() != 2 or not weight.is_cuda:
            raise ValueError("weight must be a 2-D tensor on the GPU")
        if weight.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("weight must be bf16 or fp32")
        self.register_buffer("weight", weight.detach().contiguous(), persistent=True)
        self.d_out, self.d_in = (int(v) for v in weight.shape)
        self.ranks = np.ascontiguousarray(ranks, dtype=np.int32).reshape(-1)
        self.alphas = np.ascontiguousarray(alphas, dtype=np.float32).reshape(-1)
        if self.alphas.shape != self.ranks.shape:
            raise ValueError("one alpha per adapter")
        self.dtype_name = "bf16" if weight.dtype == torch.bfloat16 else "f32"
        R = int(self.ranks.sum())
        dev = weight.device
        if A is None:
            A = torch.empty((R, self.d_in), dtype=torch.float32, device=dev)
            ro = 0
            for r in self.ranks.tolist():
                A[ro:ro + r].normal_(0.0, float(1.0 / np.sqrt(r)), generator=generator)
                ro += r
        if B is None:
            B = torch.zeros((R, self.d_out), dtype=torch.float32, device=dev)
        for name, t, d in (("A", A, self.d_in), ("B", B, self.d_out)):
            if tuple(t.shape) != (R, d):
                raise ValueError("%s must be [%d, %d], got %s" % (name, R, d, tuple(t.shape)))
        self.lora_A = torch.nn.Parameter(A.detach().to(device=dev, dtype=torch.float32).contiguous())
        self.lora_B = torch.nn.Parameter(B.detach().to(device=dev, dtype=torch.float32).contiguous())
        self.seg_offsets = None if seg_offsets is None else np.asarray(seg_offsets, np.int64)
        self.fuse_grad_accumulation = fuse_grad_accumulation
        self._copies = None  # (A version, B version, A copy, B copy)
        self._adam = None

    @property
    def n_adapters(self):
        return int(self.ranks.shape[0])

    def desc(self, seg_offsets, n_tokens=None):
        return Desc(seg_offsets, self.ranks, self.alphas, self.d_in, self.d_out, self.dtype_name, n_tokens)

    def operator_panels(self):
        """The A/B panels the kernels read: the fp32 masters themselves for an
        fp32 layer, else bf16 copies refreshed when a master has changed."""
        if self.dtype_name == "f32":
            return self.lora_A, self.lora_B
        va, vb = self.lora_A._version, self.lora_B._version
        c = self._copies
        if c is None or c[0] != va or c[1] != vb:
            A_op = c[2] if c is not None else torch.empty_like(self.lora_A, dtype=torch.bfloat16)
            B_op = c[3] if c is not None else torch.empty_like(self.lora_B, dtype=torch.bfloat16)
            if self.n_adapters:
                plora_cast_panels(self.desc(np.zeros(self.n_adapters + 1, np.int64)), self.lora_A.detach(),
                                  self.lora_B.detach(), A_op, B_op)
            self._copies = (va, vb, A_op, B_op)
        return self._copies[2], self._copies[3]

    def forward(self, x, seg_offsets=None):
        off = self.seg_offsets if seg_offsets is None else np.asarray(seg_offsets, np.int64)
        if off is None:
            raise ValueError("segment offsets are needed (argument or constructor)")
        if x.dim() != 2 or x.shape[1] != self.d_in:
            raise ValueError("x must be [T, %d]" % self.d_in)
        if x.dtype != self.weight.dtype:
            raise ValueError("x must have the weight's dtype %s" % self.weight.dtype)
        T = int(x.shape[0])
        d = self.desc(off if self.n_adapters else np.zeros(1, np.int64), n_tokens=T)
        return PackedLoRAFunction.apply(x.contiguous(), self.lora_A, self.lora_B, self, d)

    @torch.no_grad()
    def adamw_step(self, lr, weight_decay=0.01, betas=(0.9, 0.999), eps=1e-8, step=None):
        """One AdamW step on every adapter in the library's kernel
        (plora_adamw_step): per-adapter lr and weight decay (scalars or N
        values), moments kept by the module, and step counts per adapter
        (default: each adapter's own count, advanced by this call; 0 skips an
        adapter).  Uses .grad of the panels and writes the operator copies."""
        n = self.n_adapters
        if n == 0:
            return
        if self.lora_A.grad is None or self.lora_B.grad is None:
            raise RuntimeError("adamw_step needs .grad on lora_A and lora_B")
        if self._adam is None:
            z = torch.zeros_like
            self._adam = {"mA": z(self.lora_A), "vA": z(self.lora_A), "mB": z(self.lora_B), "vB": z(self.lora_B),
                          "t": np.zeros(n, np.int64)}
        st = self._adam
        if step is None:
            st["t"] = st["t"] + 1
            step = st["t"]
        cfg = AdamwConfig(lr, list(np.asarray(step, np.int64)), weight_decay=weight_decay, beta1=betas[0],
                          beta2=betas[1], eps=eps)
        A_op, B_op = self.operator_panels()
        copies = (A_op, B_op) if self.dtype_name == "bf16" else (None, None)
        plora_adamw_step(self.desc(np.zeros(n + 1, np.int64)), cfg, self.lora_A, self.lora_B, st["mA"], st["vA"],
                         st["mB"], st["vB"], self.lora_A.grad, self.lora_B.grad, copies[0], copies[1])
        # the kernel wrote masters and copies together (through raw pointers,
        # so the version counters did not move): the copies stay current
