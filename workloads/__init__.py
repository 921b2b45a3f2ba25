"""Seeded synthetic workloads for the packed multi-LoRA operator.

This module only describes shapes and draws random numbers.  It holds none of
the operator's arithmetic, so both the fp64 oracle (``oracle/``) and the HIP
path (``packed_adapter_lora_amd``) can take their inputs from it without
sharing any code with each other.

Shapes follow the projections the PLoRA summary evaluates (gist.science,
arXiv 2508.02932, 技术摘要 > 结果: Qwen-2.5 and LLaMA-3 on A100/A10); the
long-tail token mix stands in for the long-tailed multi-tenant length
distribution of the LobRA article (scholat.com, VLDB 2025 LobRA, 背景,
Fig. 1).  No dataset or checkpoint is read: values are normal draws.

Value recipe
------------
* Every tensor is drawn in row chunks.  Chunk ``c`` of tensor ``tid`` uses
  ``numpy.random.default_rng(SeedSequence([seed, tid, c]))`` (PCG64), so the
  draw is independent of the number of threads that fill it.
* A draw is ``standard_normal(float64) * std``, rounded to fp32 (numpy's
  round-to-nearest-even cast) and, for bf16 workloads, to bf16 by
  round-to-nearest-even on the fp32 bit pattern.
* ``N(0, v)`` in the workload descriptions names the variance ``v``
  (``std = sqrt(v)``), so ``X @ W.T`` has unit variance per element.
* Storage layouts: ``W`` is ``[d_out, d_in]`` (``nn.Linear.weight``); the
  packed ``A`` is ``[R, d_in]`` with rows ``R_off[i]..R_off[i+1]`` holding
  adapter i's down-projection transposed; the packed ``B`` is ``[R, d_out]``;
  ``X`` is ``[T, d_in]``; ``dY`` is ``[T, d_out]``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from statistics import NormalDist

import numpy as np

# tensor ids for the per-tensor random streams
TID_W, TID_A, TID_B, TID_X, TID_DY = 1, 2, 3, 4, 5
_ROW_CHUNK = 2048


@dataclass
class Workload:
    """One packed-LoRA problem: shapes, segment offsets, ranks, alphas."""

    name: str
    d_in: int
    d_out: int
    offsets: np.ndarray  # int64 [N+1], o_0 = 0 <= ... <= o_N = T
    ranks: np.ndarray  # int32 [N]
    alphas: np.ndarray  # float32 [N]
    dtype: str  # "f32" or "bf16"
    seed: int
    w_var: float
    x_var: float = 1.0
    b_var: float = 0.02
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_adapters(self) -> int:
        return int(self.ranks.shape[0])

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def R(self) -> int:
        return int(self.ranks.sum())

    @property
    def counts(self) -> np.ndarray:
        return np.diff(self.offsets)


def _offsets(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)


def long_tail_counts(n: int = 16, median: int = 256, cap: int = 16384, sigma: float = 4.65) -> list:
    """Deterministic lognormal quantiles: n_k = clip(round(median*exp(sigma*Phi^-1((k-1/2)/n))), 1, cap).

    With the defaults this gives 16 counts with median ~256, three segments at
    the 16384 cap and a total of 65534 tokens.
    """
    nd = NormalDist()
    return [int(min(cap, max(1, round(median * math.exp(sigma * nd.inv_cdf((k - 0.5) / n))))))
            for k in range(1, n + 1)]


_RANK_CYCLE = (8, 16, 32, 64)
_ALPHA_CYCLE = (8.0, 16.0, 32.0)


def llama_like(d_in: int, d_out: int, n_adapters: int, tokens_each: int, seed: int, name: str) -> Workload:
    ranks = np.array([_RANK_CYCLE[i % 4] for i in range(n_adapters)], dtype=np.int32)
    alphas = np.array([_ALPHA_CYCLE[i % 3] for i in range(n_adapters)], dtype=np.float32)
    return Workload(name, d_in, d_out, _offsets([tokens_each] * n_adapters), ranks, alphas,
                    "bf16", seed, w_var=1.0 / d_in)


def config(name: str, n_adapters: int | None = None, tokens_each: int | None = None) -> Workload:
    """The named synthetic workloads.

    tiny      256->256 fp32, 2 adapters (r 4/8, alpha 8/16), 64 tokens each
    qwen_q    3584->3584 bf16, 8 adapters r16 alpha32, 4x512 tokens each
    llama_sq  4096->4096 bf16, N adapters (default 32), ranks cycle 8..64
    llama_up  4096->14336 bf16, same adapters; 32 x 2048 tokens is the headline
    longtail  4096->14336 bf16, 16 adapters, lognormal token counts
    block_<p> one Llama-3-8B decoder projection p in q,k,v,o,gate,up,down,
              32 adapters x 1024 tokens
    decode_up, decode_sq
              decode-shaped serving batches on the llama_up / llama_sq
              shapes: N adapters (default 64) with 1, 2, 4, 8, 16 tokens
              (cycling; 387 tokens at N = 64), ranks cycle 8..64
    """
    if name == "tiny":
        return Workload("tiny", 256, 256, _offsets([64, 64]), np.array([4, 8], np.int32),
                        np.array([8.0, 16.0], np.float32), "f32", 1, w_var=1.0 / 256)
    if name == "qwen_q":
        n = 8 if n_adapters is None else n_adapters
        te = 4 * 512 if tokens_each is None else tokens_each
        return Workload("qwen_q", 3584, 3584, _offsets([te] * n), np.full(n, 16, np.int32),
                        np.full(n, 32.0, np.float32), "bf16", 2, w_var=1.0 / 3584)
    if name in ("llama_sq", "llama_up"):
        n = 32 if n_adapters is None else n_adapters
        te = 2048 if tokens_each is None else tokens_each
        d_out = 4096 if name == "llama_sq" else 14336
        return llama_like(4096, d_out, n, te, 3, name)
    if name == "longtail":
        seed = 4
        rng = np.random.default_rng(seed)
        ranks = rng.choice(np.array(_RANK_CYCLE, dtype=np.int32), size=16)
        counts = np.array(long_tail_counts(), dtype=np.int64)[rng.permutation(16)]
        alphas = np.array([_ALPHA_CYCLE[i % 3] for i in range(16)], dtype=np.float32)
        return Workload("longtail", 4096, 14336, _offsets(counts), ranks.astype(np.int32), alphas,
                        "bf16", seed, w_var=1.0 / 4096)
    if name in ("decode_up", "decode_sq"):
        n = 64 if n_adapters is None else n_adapters
        d_out = 14336 if name == "decode_up" else 4096
        counts = [[1, 2, 4, 8, 16][i % 5] for i in range(n)] if tokens_each is None else [tokens_each] * n
        ranks = np.array([_RANK_CYCLE[i % 4] for i in range(n)], dtype=np.int32)
        alphas = np.array([_ALPHA_CYCLE[i % 3] for i in range(n)], dtype=np.float32)
        return Workload(name, 4096, d_out, _offsets(counts), ranks, alphas, "bf16", 6, w_var=1.0 / 4096)
    if name.startswith("block_"):
        proj = name[len("block_"):]
        shapes = {"q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024), "o": (4096, 4096),
                  "gate": (4096, 14336), "up": (4096, 14336), "down": (14336, 4096)}
        d_in, d_out = shapes[proj]
        n = 32 if n_adapters is None else n_adapters
        te = 1024 if tokens_each is None else tokens_each
        wl = llama_like(d_in, d_out, n, te, 5, name)
        return wl
    raise KeyError(name)


def custom(d_in: int, d_out: int, counts, ranks, alphas, dtype: str = "bf16", seed: int = 7,
           name: str = "custom") -> Workload:
    """A workload with explicit segment counts, ranks and alphas (for edge-case tests)."""
    return Workload(name, int(d_in), int(d_out), _offsets(counts), np.asarray(ranks, np.int32),
                    np.asarray(alphas, np.float32), dtype, seed, w_var=1.0 / d_in)


# ---------------------------------------------------------------------------
# Rounding helpers: number representation only (fp32 <-> bf16 bit patterns).
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw(seed: int, tid: int, shape, std: float, dtype: str) -> np.ndarray:
    """Draw a [rows, cols] tensor; returns fp32 values (bf16-representable when dtype == 'bf16')."""
    rows, cols = int(shape[0]), int(shape[1])
    out = np.empty((rows, cols), dtype=np.float32)
    n_chunks = (rows + _ROW_CHUNK - 1) // _ROW_CHUNK

    def fill(c):
        r0, r1 = c * _ROW_CHUNK, min(rows, (c + 1) * _ROW_CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([seed, tid, c]))
        v = (rng.standard_normal((r1 - r0, cols)) * std).astype(np.float32)
        if dtype == "bf16":
            v = bf16_bits_to_f32(f32_to_bf16_bits(v)).reshape(v.shape)
        out[r0:r1] = v

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def make_inputs(wl: Workload, which=("W", "A", "B", "X", "dY")) -> dict:
    """fp32 arrays (bf16-representable for bf16 workloads) for the requested tensors.

    A and B are drawn adapter by adapter (adapter i's rows use chunk ids offset
    by 1000*i) with std 1/sqrt(r_i) for A and sqrt(0.02) for B.
    """
    out = {}
    T, R = wl.T, wl.R
    if "W" in which:
        out["W"] = draw(wl.seed, TID_W, (wl.d_out, wl.d_in), math.sqrt(wl.w_var), wl.dtype)
    if "A" in which or "B" in which:
        A = np.empty((R, wl.d_in), np.float32)
        B = np.empty((R, wl.d_out), np.float32)
        ro = 0
        for i, r in enumerate(wl.ranks.tolist()):
            if "A" in which:
                A[ro:ro + r] = draw(wl.seed * 1000 + i, TID_A, (r, wl.d_in), 1.0 / math.sqrt(r), wl.dtype)
            if "B" in which:
                B[ro:ro + r] = draw(wl.seed * 1000 + i, TID_B, (r, wl.d_out), math.sqrt(wl.b_var), wl.dtype)
            ro += r
        if "A" in which:
            out["A"] = A
        if "B" in which:
            out["B"] = B
    if "X" in which:
        out["X"] = draw(wl.seed, TID_X, (T, wl.d_in), math.sqrt(wl.x_var), wl.dtype)
    if "dY" in which:
        out["dY"] = draw(wl.seed, TID_DY, (T, wl.d_out), 1.0, wl.dtype)
    return out


def sample_rows(wl: Workload, per_segment: int = 4, seed: int = 99) -> np.ndarray:
    """Token rows to check at full size: each segment's first and last row, rows
    next to every multiple of 256 inside it, and a few seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for i in range(wl.n_adapters):
        a, b = int(wl.offsets[i]), int(wl.offsets[i + 1])
        if b <= a:
            continue
        rows.update([a, b - 1])
        for m in range((a // 256 + 1) * 256, b, 256 * 4):
            rows.update([m - 1, m])
        rows.update(rng.integers(a, b, size=min(per_segment, b - a)).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < wl.T), dtype=np.int64)


def optimizer_state(wl: Workload, seed: int) -> dict:
    """fp32 optimizer inputs for the packed panels (N(0, v) names the variance):
    master weights PA/PB (the adapters' own draws, full fp32), first moments
    mA/mB ~ N(0, 1e-6), second moments vA/vB = squares of N(0, 1e-6) draws,
    gradients dA/dB ~ N(0, 1e-4)."""
    R, di, do = wl.R, wl.d_in, wl.d_out
    base = make_inputs(custom(di, do, [0] * wl.n_adapters, wl.ranks, wl.alphas, "f32", seed), which=("A", "B"))
    out = {"PA": base["A"], "PB": base["B"]}
    for k, tid, d in (("A", 20, di), ("B", 21, do)):
        out["m" + k] = draw(seed, tid, (R, d), 1e-3, "f32")
        out["v" + k] = np.square(draw(seed, tid + 10, (R, d), 1e-3, "f32"))
        out["d" + k] = draw(seed, tid + 20, (R, d), 1e-2, "f32")
    return out
