"""Python binding of libplora.so, the packed multi-LoRA operator for MI355X.

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI declared in ``include/plora.h``.  The functions keep
the C names.  Device buffers are passed as torch tensors (their
``data_ptr()``) or raw integer addresses; the stream defaults to torch's
current stream.  There is no fallback: if ``libplora.so`` is missing, loading
this package raises.

    desc = Desc(offsets, ranks, alphas, d_in, d_out, "bf16")
    plora_forward(desc, X, W, A, B, Y, H)
    plora_backward_dx(desc, dY, W, A, B, dX, G)
    plora_backward_dAdB(desc, X, dY, H, G, dA, dB, ws)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "Desc", "PloraError", "plora_forward", "plora_backward_dx", "plora_backward_dAdB", "plora_h_elems",
    "plora_backward_dx_swiglu",
    "plora_adamw_step", "plora_cast_panels", "AdamwConfig", "plora_backward_dAdB_noalloc",
    "plora_shrink_shared", "plora_forward_expand", "plora_backward_dA_shared", "plora_workspace_bytes_dA_shared",
    "plora_workspace_bytes", "plora_validate", "plora_status_string", "plora_last_error", "plora_version", "plora_source_hash",
    "plora_profile_enable", "plora_profile_read", "plora_profile_reset", "LIB_PATH", "PLORA_F32", "PLORA_BF16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libplora.so")
PLORA_F32, PLORA_BF16 = 0, 1
_DTYPES = {"f32": PLORA_F32, "float32": PLORA_F32, "bf16": PLORA_BF16, "bfloat16": PLORA_BF16}


class plora_desc(ctypes.Structure):
    _fields_ = [
        ("n_adapters", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_out", ctypes.c_int64),
        ("seg_offsets", ctypes.POINTER(ctypes.c_int64)),
        ("ranks", ctypes.POINTER(ctypes.c_int32)),
        ("alphas", ctypes.POINTER(ctypes.c_float)),
    ]


class plora_job(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("mem_bytes", ctypes.c_double), ("ms_per_step", ctypes.c_double)]


class plora_pack_model(ctypes.Structure):
    _fields_ = [("mem_budget", ctypes.c_double), ("fixed_ms", ctypes.c_double), ("mem_quantum", ctypes.c_double)]


class plora_adamw_config(ctypes.Structure):
    _fields_ = [
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("lr", ctypes.POINTER(ctypes.c_float)),
        ("weight_decay", ctypes.POINTER(ctypes.c_float)),
        ("step", ctypes.POINTER(ctypes.c_int64)),
    ]


def _load():
    # Load PyTorch's HIP runtime first when PyTorch is installed: libplora.so
    # then binds to that same runtime.  Loaded the other way round, the process
    # would hold two HIP runtimes (the system one for this library, PyTorch's
    # bundled one for the tensors) and this library's would find no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("libplora.so is not built (run: python packed_adapter_lora_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    # refuse a library built from other sources than the ones beside it
    from .build import source_hash
    lib.plora_source_hash.restype, lib.plora_source_hash.argtypes = ctypes.c_char_p, []
    built, here = lib.plora_source_hash().decode(), source_hash()
    if built != here:
        raise ImportError("libplora.so was built from other sources (hash %s, sources %s); rebuild it with "
                          "python packed_adapter_lora_amd/build.py" % (built, here))
    vp, dp = ctypes.c_void_p, ctypes.POINTER(plora_desc)
    fp = ctypes.c_void_p
    sig = {
        "plora_forward": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, fp, vp]),
        "plora_backward_dx": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, fp, vp]),
        "plora_backward_dAdB": (ctypes.c_int, [dp, vp, vp, fp, fp, fp, fp, vp, ctypes.c_size_t, vp]),
        "plora_backward_dAdB_acc": (ctypes.c_int, [dp, vp, vp, fp, fp, fp, fp, vp, ctypes.c_size_t, ctypes.c_int,
                                                   vp]),
        "plora_backward_dAdB_noalloc": (ctypes.c_int, [dp, vp, vp, fp, fp, fp, fp, ctypes.c_int, vp]),
        "plora_shrink_shared": (ctypes.c_int, [dp, vp, ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), vp]),
        "plora_forward_expand": (ctypes.c_int, [dp, vp, vp, vp, vp, fp, vp]),
        "plora_backward_dA_shared": (ctypes.c_int, [dp, vp, ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                                    ctypes.c_size_t, ctypes.c_int, vp]),
        "plora_workspace_bytes_dA_shared": (ctypes.c_size_t, [dp, ctypes.c_int]),
        "plora_adamw_step": (ctypes.c_int, [dp, ctypes.POINTER(plora_adamw_config)] + [vp] * 11),
        "plora_cast_panels": (ctypes.c_int, [dp, vp, vp, vp, vp, vp]),
        "plora_rmsnorm_fwd": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                             vp]),
        "plora_rmsnorm_bwd": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64] + [vp] * 9),
        "plora_rope": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_float, ctypes.c_int,
                                      vp, vp]),
        "plora_swiglu_fwd": (ctypes.c_int, [ctypes.c_int64, vp, vp, vp, vp]),
        "plora_swiglu_bwd": (ctypes.c_int, [ctypes.c_int64, vp, vp, vp, vp, vp, vp]),
        "plora_backward_dx_swiglu": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, vp, vp, fp, vp]),
        "plora_add": (ctypes.c_int, [ctypes.c_int64, vp, vp, vp, vp]),
        "plora_attention_fwd": (ctypes.c_int, [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32] + [vp] * 6),
        "plora_attention_bwd": (ctypes.c_int, [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32] + [vp] * 11),
        "plora_plan_packs": (ctypes.c_int, [ctypes.POINTER(plora_job), ctypes.c_int32, ctypes.POINTER(plora_pack_model),
                                            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_double)]),
        "plora_plan_makespan": (ctypes.c_double, [ctypes.POINTER(plora_job), ctypes.c_int32,
                                                  ctypes.POINTER(plora_pack_model), ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.c_int32]),
        "plora_probe_mfma_operand_bytes": (ctypes.c_size_t, []),
        "plora_probe_mfma": (ctypes.c_int, [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp,
                                            ctypes.POINTER(ctypes.c_double), vp]),
        "plora_probe_copy": (ctypes.c_int, [vp, vp, ctypes.c_size_t, ctypes.c_int32, vp]),
        "plora_probe_read": (ctypes.c_int, [vp, ctypes.c_size_t, ctypes.c_int32, vp, vp]),
        "plora_probe_lds_dma": (ctypes.c_int, [vp, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, vp,
                                               ctypes.POINTER(ctypes.c_double), vp]),
        "plora_h_elems": (ctypes.c_size_t, [dp]),
        "plora_workspace_bytes": (ctypes.c_size_t, [dp]),
        "plora_validate": (ctypes.c_int, [dp]),
        "plora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "plora_last_error": (ctypes.c_char_p, []),
        "plora_version": (ctypes.c_int, []),
        "plora_source_hash": (ctypes.c_char_p, []),
        "plora_profile_enable": (ctypes.c_int, [ctypes.c_int]),
        "plora_profile_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(ctypes.c_double)]),
        "plora_profile_reset": (None, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()


class PloraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (plora_status_string(status), status, msg))
        self.status = status


class Desc:
    """Owns the host arrays of a ``plora_desc`` (offsets int64, ranks int32, alphas fp32)."""

    def __init__(self, offsets, ranks, alphas, d_in, d_out, dtype="bf16", n_tokens=None):
        self.offsets = np.ascontiguousarray(offsets, dtype=np.int64).reshape(-1)
        self.ranks = np.ascontiguousarray(ranks, dtype=np.int32).reshape(-1)
        self.alphas = np.ascontiguousarray(alphas, dtype=np.float32).reshape(-1)
        n = int(self.ranks.shape[0])
        if n == 0 and self.offsets.shape[0] < 1:
            self.offsets = np.zeros(1, np.int64)
        # the library reads offsets[0..n] and alphas[0..n-1] through raw pointers
        if self.offsets.shape[0] != n + 1:
            raise ValueError("%d adapters need %d segment offsets, got %d" % (n, n + 1, self.offsets.shape[0]))
        if self.alphas.shape[0] != n:
            raise ValueError("%d adapters need %d alphas, got %d" % (n, n, self.alphas.shape[0]))
        T = int(self.offsets[-1]) if n_tokens is None else int(n_tokens)
        self.dtype = _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        self.c = plora_desc(n, self.dtype, T, int(d_in), int(d_out),
                            self.offsets.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                            self.ranks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            self.alphas.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))

    @classmethod
    def from_workload(cls, wl):
        return cls(wl.offsets, wl.ranks, wl.alphas, wl.d_in, wl.d_out, wl.dtype, wl.T)

    @property
    def n_tokens(self):
        return int(self.c.n_tokens)

    @property
    def R(self):
        return int(self.ranks.sum())

    def ref(self):
        return ctypes.byref(self.c)


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != 0:
        raise PloraError(rc, (_lib.plora_last_error() or b"").decode())


def _check_tensor(name, t, shape, dtype):
    """Shape, dtype, layout and device check of a torch tensor against the descriptor."""
    if t is None or isinstance(t, int):
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and str(t.dtype).split(".")[-1] != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    # a host tensor's address handed to a kernel would fault the GPU
    if not t.is_cuda:
        raise ValueError("%s is on %s; the operator needs device memory" % (name, t.device))
    import torch
    if t.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s but the current device is cuda:%d" % (name, t.device,
                                                                          torch.cuda.current_device()))


def _elt(desc):
    return "bfloat16" if desc.dtype == PLORA_BF16 else "float32"


def plora_forward(desc: Desc, X, W, A, B, Y, H, stream=None):
    T, di, do, R = desc.n_tokens, int(desc.c.d_in), int(desc.c.d_out), desc.R
    e = _elt(desc)
    for n, t, s, d in (("X", X, (T, di), e), ("W", W, (do, di), e), ("A", A, (R, di), e), ("B", B, (R, do), e),
                       ("Y", Y, (T, do), e), ("H", H, (plora_h_elems(desc),), "float32")):
        _check_tensor(n, t, s, d)
    _check(_lib.plora_forward(desc.ref(), _addr(X), _addr(W), _addr(A), _addr(B), _addr(Y), _addr(H),
                              _stream(stream)))


def plora_backward_dx(desc: Desc, dY, W, A, B, dX, G, stream=None):
    T, di, do, R = desc.n_tokens, int(desc.c.d_in), int(desc.c.d_out), desc.R
    e = _elt(desc)
    for n, t, s, d in (("dY", dY, (T, do), e), ("W", W, (do, di), e), ("A", A, (R, di), e), ("B", B, (R, do), e),
                       ("dX", dX, (T, di), e), ("G", G, (plora_h_elems(desc),), "float32")):
        _check_tensor(n, t, s, d)
    _check(_lib.plora_backward_dx(desc.ref(), _addr(dY), _addr(W), _addr(A), _addr(B), _addr(dX), _addr(G),
                                  _stream(stream)))


def plora_backward_dx_swiglu(desc: Desc, dY, W, A, B, g, u, dg, du, G, stream=None):
    """The down projection's dX with the SwiGLU backward applied to it: dg, du
    (see plora_block.h); dX itself is not stored."""
    T, di, do, R = desc.n_tokens, int(desc.c.d_in), int(desc.c.d_out), desc.R
    e = _elt(desc)
    for n, t, s, d in (("dY", dY, (T, do), e), ("W", W, (do, di), e), ("A", A, (R, di), e), ("B", B, (R, do), e),
                       ("g", g, (T, di), e), ("u", u, (T, di), e), ("dg", dg, (T, di), e), ("du", du, (T, di), e),
                       ("G", G, (plora_h_elems(desc),), "float32")):
        _check_tensor(n, t, s, d)
    _check(_lib.plora_backward_dx_swiglu(desc.ref(), _addr(dY), _addr(W), _addr(A), _addr(B), _addr(g), _addr(u),
                                         _addr(dg), _addr(du), _addr(G), _stream(stream)))


def plora_backward_dAdB(desc: Desc, X, dY, H, G, dA, dB, workspace=None, stream=None, accumulate=False):
    T, di, do, R = desc.n_tokens, int(desc.c.d_in), int(desc.c.d_out), desc.R
    e = _elt(desc)
    he = plora_h_elems(desc)
    for n, t, s, d in (("X", X, (T, di), e), ("dY", dY, (T, do), e), ("H", H, (he,), "float32"),
                       ("G", G, (he,), "float32"), ("dA", dA, (R, di), "float32"), ("dB", dB, (R, do), "float32")):
        _check_tensor(n, t, s, d)
    nbytes = 0
    if workspace is not None and not isinstance(workspace, int):
        nbytes = workspace.numel() * workspace.element_size()
    elif isinstance(workspace, int):
        nbytes = plora_workspace_bytes(desc)
    _check(_lib.plora_backward_dAdB_acc(desc.ref(), _addr(X), _addr(dY), _addr(H), _addr(G), _addr(dA), _addr(dB),
                                        _addr(workspace), nbytes, 1 if accumulate else 0, _stream(stream)))


def plora_backward_dAdB_noalloc(desc: Desc, X, dY, H, G, dA, dB, accumulate=False, stream=None):
    """plora_backward_dAdB without a workspace (the library's per-device scratch array; see plora.h)."""
    T, di, do, R = desc.n_tokens, int(desc.c.d_in), int(desc.c.d_out), desc.R
    e = _elt(desc)
    he = plora_h_elems(desc)
    for n, t, s, d in (("X", X, (T, di), e), ("dY", dY, (T, do), e), ("H", H, (he,), "float32"),
                       ("G", G, (he,), "float32"), ("dA", dA, (R, di), "float32"), ("dB", dB, (R, do), "float32")):
        _check_tensor(n, t, s, d)
    _check(_lib.plora_backward_dAdB_noalloc(desc.ref(), _addr(X), _addr(dY), _addr(H), _addr(G), _addr(dA),
                                            _addr(dB), 1 if accumulate else 0, _stream(stream)))


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[_addr(t) for t in ts])


def plora_shrink_shared(desc: Desc, X, A_list, H_list, stream=None):
    """H[p] = X A[p] for the 1-3 projections that read X (see plora.h)."""
    T, di, R = desc.n_tokens, int(desc.c.d_in), desc.R
    e = _elt(desc)
    if not 1 <= len(A_list) <= 3 or len(H_list) != len(A_list):
        raise ValueError("1 to 3 panels, one H per panel")
    _check_tensor("X", X, (T, di), e)
    he = plora_h_elems(desc)
    for p, (A, H) in enumerate(zip(A_list, H_list)):
        _check_tensor("A[%d]" % p, A, (R, di), e)
        _check_tensor("H[%d]" % p, H, (he,), "float32")
    _check(_lib.plora_shrink_shared(desc.ref(), _addr(X), len(A_list), _ptr_array(A_list), _ptr_array(H_list),
                                    _stream(stream)))


def plora_forward_expand(desc: Desc, X, W, B, Y, H, stream=None):
    """The forward GEMM with its fused expand, H given (see plora.h)."""
    T, di, do, R = desc.n_tokens, int(desc.c.d_in), int(desc.c.d_out), desc.R
    e = _elt(desc)
    for n, t, s_, d in (("X", X, (T, di), e), ("W", W, (do, di), e), ("B", B, (R, do), e), ("Y", Y, (T, do), e),
                        ("H", H, (plora_h_elems(desc),), "float32")):
        _check_tensor(n, t, s_, d)
    _check(_lib.plora_forward_expand(desc.ref(), _addr(X), _addr(W), _addr(B), _addr(Y), _addr(H), _stream(stream)))


def plora_workspace_bytes_dA_shared(desc: Desc, np_: int) -> int:
    return int(_lib.plora_workspace_bytes_dA_shared(desc.ref(), int(np_)))


def plora_backward_dA_shared(desc: Desc, X, G_list, dA_list, workspace=None, stream=None, accumulate=False):
    """dA[p] = s_i X^T G[p] for the 1-3 projections that read X (see plora.h)."""
    T, di, R = desc.n_tokens, int(desc.c.d_in), desc.R
    e = _elt(desc)
    if not 1 <= len(G_list) <= 3 or len(dA_list) != len(G_list):
        raise ValueError("1 to 3 panels, one dA per G")
    _check_tensor("X", X, (T, di), e)
    he = plora_h_elems(desc)
    for p, (G, dA) in enumerate(zip(G_list, dA_list)):
        _check_tensor("G[%d]" % p, G, (he,), "float32")
        _check_tensor("dA[%d]" % p, dA, (R, di), "float32")
    nbytes = 0
    if workspace is not None and not isinstance(workspace, int):
        nbytes = workspace.numel() * workspace.element_size()
    elif isinstance(workspace, int):
        nbytes = plora_workspace_bytes_dA_shared(desc, len(G_list))
    _check(_lib.plora_backward_dA_shared(desc.ref(), _addr(X), len(G_list), _ptr_array(G_list), _ptr_array(dA_list),
                                         _addr(workspace), nbytes, 1 if accumulate else 0, _stream(stream)))


class AdamwConfig:
    """Host-side AdamW settings for plora_adamw_step: per-adapter learning rate,
    weight decay and step count (0 = skip the adapter), shared betas and eps.
    Defaults are PyTorch's AdamW defaults."""

    def __init__(self, lr, step, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8):
        n = len(step)
        wd = [weight_decay] * n if np.isscalar(weight_decay) else list(weight_decay)
        lr = [lr] * n if np.isscalar(lr) else list(lr)
        if len(lr) != n or len(wd) != n:
            raise ValueError("lr, weight_decay and step need one value per adapter")
        self.lr = np.ascontiguousarray(lr, dtype=np.float32)
        self.wd = np.ascontiguousarray(wd, dtype=np.float32)
        self.step = np.ascontiguousarray(step, dtype=np.int64)
        self.c = plora_adamw_config(beta1, beta2, eps,
                                    self.lr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                    self.wd.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                    self.step.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))

    def ref(self):
        return ctypes.byref(self.c)


def plora_adamw_step(desc: Desc, cfg: AdamwConfig, PA, PB, mA, vA, mB, vB, dA, dB, A=None, B=None, stream=None):
    """One per-adapter AdamW step over the packed panels (see plora.h)."""
    R, di, do = desc.R, int(desc.c.d_in), int(desc.c.d_out)
    if len(cfg.step) != int(desc.c.n_adapters):
        raise ValueError("AdamW configuration has %d adapters, descriptor %d" % (len(cfg.step), desc.c.n_adapters))
    for n, t, shp in (("PA", PA, (R, di)), ("mA", mA, (R, di)), ("vA", vA, (R, di)), ("dA", dA, (R, di)),
                      ("PB", PB, (R, do)), ("mB", mB, (R, do)), ("vB", vB, (R, do)), ("dB", dB, (R, do))):
        _check_tensor(n, t, shp, "float32")
    e = _elt(desc)
    for n, t, shp in (("A", A, (R, di)), ("B", B, (R, do))):
        if t is not None:
            _check_tensor(n, t, shp, e)
    _check(_lib.plora_adamw_step(desc.ref(), cfg.ref(), _addr(PA), _addr(PB), _addr(mA), _addr(vA), _addr(mB),
                                 _addr(vB), _addr(dA), _addr(dB), _addr(A), _addr(B), _stream(stream)))


def plora_cast_panels(desc: Desc, PA, PB, A, B, stream=None):
    """The operator's desc.dtype copies A, B of the fp32 master panels PA, PB (see plora.h)."""
    R, di, do = desc.R, int(desc.c.d_in), int(desc.c.d_out)
    e = _elt(desc)
    for n, t, shp, dt in (("PA", PA, (R, di), "float32"), ("PB", PB, (R, do), "float32"), ("A", A, (R, di), e),
                          ("B", B, (R, do), e)):
        _check_tensor(n, t, shp, dt)
    _check(_lib.plora_cast_panels(desc.ref(), _addr(PA), _addr(PB), _addr(A), _addr(B), _stream(stream)))


# ---------------------------------------------------------------------------
# Ceiling micro-benchmarks (include/plora_probe.h): device buffers as torch
# tensors; each call enqueues one kernel on the stream.
# ---------------------------------------------------------------------------

def plora_probe_mfma_operand_bytes() -> int:
    return int(_lib.plora_probe_mfma_operand_bytes())


def plora_probe_mfma(operands, workgroups, iters, out, shape=0, stream=None) -> float:
    """Enqueues the sustained-MFMA probe (shape 0: 32x32x16, 1: 16x16x32,
    2: 32x32x16 with the operands read from LDS); returns the launch's FLOP
    count."""
    if operands.numel() * operands.element_size() < plora_probe_mfma_operand_bytes():
        raise ValueError("operand buffer smaller than plora_probe_mfma_operand_bytes()")
    if out.numel() < workgroups * 256 or str(out.dtype) != "torch.float32":
        raise ValueError("out needs workgroups * 256 fp32 values")
    for n, t in (("operands", operands), ("out", out)):
        _check_tensor(n, t, tuple(t.shape), None)
    fl = ctypes.c_double(0.0)
    _check(_lib.plora_probe_mfma(_addr(operands), int(shape), int(workgroups), int(iters), _addr(out),
                                 ctypes.byref(fl), _stream(stream)))
    return float(fl.value)


def plora_probe_copy(src, dst, workgroups=2048, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    for n, t in (("src", src), ("dst", dst)):
        _check_tensor(n, t, tuple(t.shape), None)
    _check(_lib.plora_probe_copy(_addr(src), _addr(dst), nbytes, int(workgroups), _stream(stream)))


def plora_probe_read(src, out, workgroups=2048, stream=None):
    if out.numel() < workgroups * 256 or out.element_size() != 4:
        raise ValueError("out needs workgroups * 256 32-bit values")
    for n, t in (("src", src), ("out", out)):
        _check_tensor(n, t, tuple(t.shape), None)
    _check(_lib.plora_probe_read(_addr(src), src.numel() * src.element_size(), int(workgroups), _addr(out),
                                 _stream(stream)))


def plora_probe_lds_dma(src, workgroups, iters, out, stream=None) -> float:
    """Enqueues the L2 -> LDS probe over all of src (a multiple of 4096
    bytes); returns the bytes the launch moves."""
    if out.numel() < workgroups * 256 or out.element_size() != 4:
        raise ValueError("out needs workgroups * 256 32-bit values")
    for n, t in (("src", src), ("out", out)):
        _check_tensor(n, t, tuple(t.shape), None)
    nb = ctypes.c_double(0.0)
    _check(_lib.plora_probe_lds_dma(_addr(src), src.numel() * src.element_size(), int(workgroups), int(iters),
                                    _addr(out), ctypes.byref(nb), _stream(stream)))
    return float(nb.value)


def plora_h_elems(desc: Desc) -> int:
    return int(_lib.plora_h_elems(desc.ref()))


def plora_workspace_bytes(desc: Desc) -> int:
    return int(_lib.plora_workspace_bytes(desc.ref()))


def plora_validate(desc: Desc) -> int:
    return int(_lib.plora_validate(desc.ref()))


def plora_status_string(status: int) -> str:
    return _lib.plora_status_string(int(status)).decode()


def plora_last_error() -> str:
    return (_lib.plora_last_error() or b"").decode()


def plora_version() -> int:
    return int(_lib.plora_version())


def plora_source_hash() -> str:
    return _lib.plora_source_hash().decode()


def plora_profile_enable(on: bool = True):
    _check(_lib.plora_profile_enable(1 if on else 0))


def plora_profile_read(kernel_class: str):
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(_lib.plora_profile_read(kernel_class.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def plora_profile_reset():
    _lib.plora_profile_reset()


# ---------------------------------------------------------------------------
# Decoder-block kernels (include/plora_block.h).  Tensors are bf16 torch
# tensors; sequence tables are host int64 arrays of n_seq + 1 offsets.
# ---------------------------------------------------------------------------

def _seq(seq_offsets):
    off = np.ascontiguousarray(seq_offsets, dtype=np.int64)
    return off, len(off) - 1, off.ctypes.data


def _bf16(name, t, shape=None):
    _check_tensor(name, t, shape if shape is not None else tuple(t.shape), "bfloat16")


def plora_rmsnorm_fwd(x, w, h, rstd, res=None, xs_out=None, eps=1e-5, stream=None):
    T, D = x.shape
    for n, t in (("x", x), ("h", h), ("res", res), ("xs_out", xs_out)):
        if t is not None:
            _bf16(n, t, (T, D))
    _bf16("w", w, (D,))
    _check_tensor("rstd", rstd, (T,), "float32")
    _check(_lib.plora_rmsnorm_fwd(T, D, _addr(x), _addr(res), _addr(w), eps, _addr(xs_out), _addr(h), _addr(rstd),
                                  _stream(stream)))


def plora_rmsnorm_bwd(dys, x, w, rstd, dx, dres=None, stream=None):
    T, D = x.shape
    dys = list(dys) + [None] * (3 - len(dys))
    for n, t in (("dy0", dys[0]), ("dy1", dys[1]), ("dy2", dys[2]), ("x", x), ("dres", dres), ("dx", dx)):
        if t is not None:
            _bf16(n, t, (T, D))
    _bf16("w", w, (D,))
    _check_tensor("rstd", rstd, (T,), "float32")
    _check(_lib.plora_rmsnorm_bwd(T, D, _addr(dys[0]), _addr(dys[1]), _addr(dys[2]), _addr(x), _addr(w), _addr(rstd),
                                  _addr(dres), _addr(dx), _stream(stream)))


def plora_rope(x, seq_offsets, heads, base=500000.0, inverse=False, stream=None):
    off, n, p = _seq(seq_offsets)
    _bf16("x", x, (int(off[-1]), heads * 128))
    _check(_lib.plora_rope(int(off[-1]), heads, n, p, base, 1 if inverse else 0, _addr(x), _stream(stream)))


def plora_swiglu_fwd(g, u, a, stream=None):
    for n, t in (("g", g), ("u", u), ("a", a)):
        _bf16(n, t, tuple(g.shape))
    _check(_lib.plora_swiglu_fwd(g.numel(), _addr(g), _addr(u), _addr(a), _stream(stream)))


def plora_swiglu_bwd(da, g, u, dg, du, stream=None):
    for n, t in (("da", da), ("g", g), ("u", u), ("dg", dg), ("du", du)):
        _bf16(n, t, tuple(g.shape))
    _check(_lib.plora_swiglu_bwd(g.numel(), _addr(da), _addr(g), _addr(u), _addr(dg), _addr(du), _stream(stream)))


def plora_add(x, y, out, stream=None):
    for n, t in (("x", x), ("y", y), ("out", out)):
        _bf16(n, t, tuple(x.shape))
    _check(_lib.plora_add(x.numel(), _addr(x), _addr(y), _addr(out), _stream(stream)))


def plora_attention_fwd(q, k, v, o, lse, seq_offsets, n_q, n_kv, stream=None):
    off, n, p = _seq(seq_offsets)
    T = int(off[-1])
    _bf16("q", q, (T, n_q * 128))
    _bf16("k", k, (T, n_kv * 128))
    _bf16("v", v, (T, n_kv * 128))
    _bf16("o", o, (T, n_q * 128))
    _check_tensor("lse", lse, (n_q, T), "float32")
    _check(_lib.plora_attention_fwd(n, p, n_q, n_kv, _addr(q), _addr(k), _addr(v), _addr(o), _addr(lse),
                                    _stream(stream)))


def plora_attention_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, seq_offsets, n_q, n_kv, stream=None):
    off, n, p = _seq(seq_offsets)
    T = int(off[-1])
    for nm, t, hh in (("q", q, n_q), ("k", k, n_kv), ("v", v, n_kv), ("o", o, n_q), ("dO", dO, n_q), ("dq", dq, n_q),
                      ("dk", dk, n_kv), ("dv", dv, n_kv)):
        _bf16(nm, t, (T, hh * 128))
    _check_tensor("lse", lse, (n_q, T), "float32")
    _check_tensor("delta", delta, (n_q, T), "float32")
    _check(_lib.plora_attention_bwd(n, p, n_q, n_kv, _addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(dO),
                                    _addr(dq), _addr(dk), _addr(dv), _addr(delta), _stream(stream)))


# ---------------------------------------------------------------------------
# Packing planner (include/plora_planner.h), host only.
# ---------------------------------------------------------------------------

def _jobs(steps, mem_bytes, ms_per_step):
    n = len(steps)
    arr = (plora_job * n)()
    for k in range(n):
        arr[k].steps, arr[k].mem_bytes, arr[k].ms_per_step = int(steps[k]), float(mem_bytes[k]), float(ms_per_step[k])
    return arr, n


def plora_plan_packs(steps, mem_bytes, ms_per_step, mem_budget, fixed_ms, mem_quantum):
    """Returns (pack_of_job as an int32 array, n_packs, makespan_ms)."""
    arr, n = _jobs(steps, mem_bytes, ms_per_step)
    model = plora_pack_model(mem_budget, fixed_ms, mem_quantum)
    out = np.empty(n, dtype=np.int32)
    npk, ms = ctypes.c_int32(0), ctypes.c_double(0.0)
    _check(_lib.plora_plan_packs(arr, n, ctypes.byref(model), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 ctypes.byref(npk), ctypes.byref(ms)))
    return out, int(npk.value), float(ms.value)


def plora_plan_makespan(steps, mem_bytes, ms_per_step, mem_budget, fixed_ms, mem_quantum, pack_of_job, n_packs):
    arr, n = _jobs(steps, mem_bytes, ms_per_step)
    model = plora_pack_model(mem_budget, fixed_ms, mem_quantum)
    p = np.ascontiguousarray(pack_of_job, dtype=np.int32)
    v = _lib.plora_plan_makespan(arr, n, ctypes.byref(model), p.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 int(n_packs))
    if v < 0:
        _check(int(v))
    return float(v)


def __getattr__(name):
    # the PyTorch module is imported on first use (the C-ABI binding itself
    # needs only numpy and ctypes)
    if name in ("PackedLoRALinear", "PackedLoRAFunction"):
        from . import module
        return getattr(module, name)
    raise AttributeError(name)
