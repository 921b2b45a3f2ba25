"""fp64 CPU oracle for the packed multi-LoRA operator (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``.  The product
package never imports it, and it never imports the product package.

``plora_oracle.c`` holds the arithmetic (plain fp64 loops, adapter by adapter,
token by token); this file compiles it with gcc when needed and marshals
numpy arrays.  Inputs are converted to fp64 exactly (bf16 and fp32 values are
exactly representable in fp64).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(B = 0 identity, merge identity against numpy matmul, block-diagonal dense
form, rank-1 closed form, finite differences, permutation, locality, a
hand-worked example).  No function is left unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "plora_oracle.c")
_LIB = os.path.join(_HERE, "libplora_oracle.so")
_lock = threading.Lock()
_lib = None

ERRORS = {0: "ok", -1: "null", -2: "segments", -3: "rank", -4: "alpha", -5: "shape",
          -6: "adapters", -7: "nomem"}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i64p = ctypes.POINTER(ctypes.c_int64)
            i32p = ctypes.POINTER(ctypes.c_int32)
            lib.oracle_packed_lora.restype = ctypes.c_int
            lib.oracle_packed_lora.argtypes = [ctypes.c_int, ctypes.c_int64, i64p, i32p, dp, ctypes.c_int64, ctypes.c_int64] + [dp] * 11
            lib.oracle_check.restype = ctypes.c_int
            lib.oracle_check.argtypes = [ctypes.c_int, ctypes.c_int64, i64p, i32p, dp, ctypes.c_int64, ctypes.c_int64]
            lib.oracle_h_elems.restype = ctypes.c_int64
            lib.oracle_h_elems.argtypes = [ctypes.c_int, i64p, i32p]
            lib.oracle_threads.restype = ctypes.c_int
            lib.oracle_threads.argtypes = []
            lib.oracle_set_threads.restype = None
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


class use_library:
    """Context manager: route calls to another build of the oracle source.

    Used only by the mutation test, which plants mistakes in a copy of
    ``plora_oracle.c`` and checks that the pins reject every such copy."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self._saved = _lib
        lib = ctypes.CDLL(self.path)
        for name in ("oracle_packed_lora", "oracle_check", "oracle_h_elems", "oracle_threads", "oracle_set_threads"):
            f, g = getattr(lib, name), getattr(self._saved, name)
            f.restype, f.argtypes = g.restype, g.argtypes
        _lib = lib
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def threads() -> int:
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads of later oracle calls (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ=ctypes.c_double):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(typ))
    return a.ctypes.data_as(ctypes.POINTER(typ))


class OracleError(RuntimeError):
    pass


def check(offsets, ranks, alphas, d_in, d_out, T=None) -> int:
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    rk = np.ascontiguousarray(ranks, dtype=np.int32)
    al = np.ascontiguousarray(alphas, dtype=np.float64)
    T = int(off[-1]) if T is None else int(T)
    return int(_load().oracle_check(int(rk.shape[0]), T, _ptr(off, ctypes.c_int64), _ptr(rk, ctypes.c_int32),
                                    _ptr(al), int(d_in), int(d_out)))


def packed_lora(offsets, ranks, alphas, d_in, d_out, X=None, dY=None, W=None, A=None, B=None,
                want=("Y", "H", "dX", "G", "dA", "dB"), T=None) -> dict:
    """Run the oracle; returns a dict of fp64 arrays for the names in ``want``.

    ``T`` defaults to the last offset; with no adapters (empty ``ranks``) it
    is the token count of the frozen-only problem.
    Shapes: X [T, d_in], dY [T, d_out], W [d_out, d_in], A [R, d_in],
    B [R, d_out]; Y [T, d_out], dX [T, d_in], H and G flat [sum n_i r_i],
    dA [R, d_in], dB [R, d_out].
    """
    lib = _load()
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    rk = np.ascontiguousarray(ranks, dtype=np.int32)
    al = np.ascontiguousarray(alphas, dtype=np.float64)
    n = int(rk.shape[0])
    T = int(off[-1]) if T is None else int(T)
    R = int(rk.sum())
    X, dY, W, A, B = (_f64(v) for v in (X, dY, W, A, B))
    he = int(lib.oracle_h_elems(n, _ptr(off, ctypes.c_int64), _ptr(rk, ctypes.c_int32))) if n else 0
    shapes = {"Y": (T, d_out), "dX": (T, d_in), "H": (he,), "G": (he,), "dA": (R, d_in), "dB": (R, d_out)}
    outs = {k: np.empty(shapes[k], dtype=np.float64) for k in want}
    rc = lib.oracle_packed_lora(n, T, _ptr(off, ctypes.c_int64), _ptr(rk, ctypes.c_int32), _ptr(al),
                                int(d_in), int(d_out), _ptr(X), _ptr(dY), _ptr(W), _ptr(A), _ptr(B),
                                _ptr(outs.get("Y")), _ptr(outs.get("H")), _ptr(outs.get("dX")),
                                _ptr(outs.get("G")), _ptr(outs.get("dA")), _ptr(outs.get("dB")))
    if rc != 0:
        raise OracleError("oracle_packed_lora: %s (%d)" % (ERRORS.get(rc, "?"), rc))
    return outs


def run_workload(wl, inputs: dict, want=("Y", "H", "dX", "G", "dA", "dB")) -> dict:
    """Oracle on a ``workloads.Workload`` with inputs from ``workloads.make_inputs``."""
    return packed_lora(wl.offsets, wl.ranks, wl.alphas.astype(np.float64), wl.d_in, wl.d_out,
                       X=inputs.get("X"), dY=inputs.get("dY"), W=inputs.get("W"),
                       A=inputs.get("A"), B=inputs.get("B"), want=want)


def rows_subproblem(wl, inputs: dict, rows, want=("Y", "H", "dX", "G")) -> dict:
    """Row outputs (Y, dX and the per-row H, G) for a sorted subset of token rows.

    Rows are independent in the method's definition, so the oracle runs on the
    sub-problem made of just these rows, each kept in its adapter's segment.
    Returned H and G are [len(rows), r_max] arrays padded with NaN.
    """
    rows = np.asarray(rows, dtype=np.int64)
    seg = np.searchsorted(wl.offsets, rows, side="right") - 1
    counts = np.bincount(seg, minlength=wl.n_adapters)
    sub_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sub = {}
    for k in ("X", "dY"):
        if k in inputs and inputs[k] is not None:
            sub[k] = inputs[k][rows]
    for k in ("W", "A", "B"):
        if k in inputs:
            sub[k] = inputs[k]
    out = packed_lora(sub_off, wl.ranks, wl.alphas.astype(np.float64), wl.d_in, wl.d_out,
                      X=sub.get("X"), dY=sub.get("dY"), W=sub.get("W"), A=sub.get("A"),
                      B=sub.get("B"), want=want)
    rmax = int(wl.ranks.max()) if wl.n_adapters else 0
    for k in ("H", "G"):
        if k in out:
            flat = out[k]
            mat = np.full((len(rows), rmax), np.nan)
            pos = 0
            for u in range(len(rows)):
                r = int(wl.ranks[seg[u]])
                mat[u, :r] = flat[pos:pos + r]
                pos += r
            out[k] = mat
    return out
