"""Host-side checks of the C ABI (no GPU needed).

The library loads on a machine without a GPU; validation runs entirely on the
host before anything is enqueued, so every error path is exercised here with
descriptors and pointer values that are never dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def P():
    pkg = pytest.importorskip("packed_adapter_lora_amd")
    return pkg


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(plora_[a-z_A-Z0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("plora_forward", "plora_backward_dx", "plora_backward_dAdB", "plora_h_elems",
              "plora_workspace_bytes", "plora_status_string", "plora_last_error", "plora_version",
              "plora_backward_dAdB_acc", "plora_adamw_step", "plora_rmsnorm_fwd", "plora_rmsnorm_bwd", "plora_rope",
              "plora_swiglu_fwd", "plora_swiglu_bwd", "plora_add", "plora_attention_fwd", "plora_attention_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(P):
    lib = ctypes.CDLL(P.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_version_and_strings(P):
    assert P.plora_version() == 1
    assert P.plora_status_string(0) == "PLORA_OK"
    assert P.plora_status_string(-8) == "PLORA_ERR_WORKSPACE"
    assert P.plora_status_string(12345) == "PLORA_ERR_UNKNOWN"


def desc(P, counts=(3, 0, 5), ranks=(4, 8, 16), alphas=(8.0, 16.0, 32.0), d_in=64, d_out=32, dtype="bf16", T=None):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return P.Desc(off, ranks, alphas, d_in, d_out, dtype, T)


def test_validation_codes(P):
    assert P.plora_validate(desc(P)) == 0
    assert P.plora_validate(desc(P, d_in=12)) == -5
    assert P.plora_validate(desc(P, d_out=0)) == -5
    assert P.plora_validate(desc(P, ranks=(4, 0, 16))) == -3
    assert P.plora_validate(desc(P, ranks=(4, 129, 16))) == -3
    assert P.plora_validate(desc(P, alphas=(8.0, float("inf"), 1.0))) == -4
    assert P.plora_validate(desc(P, T=9)) == -2
    d = desc(P)
    d.offsets[1] = 5  # 0, 5, 3, 8: decreasing
    assert P.plora_validate(d) == -2
    d = desc(P)
    d.c.dtype = 7
    assert P.plora_validate(d) == -7
    d = desc(P)
    d.c.n_adapters = 65
    assert P.plora_validate(d) == -6
    # no adapters: any token count, offsets unused
    d0 = P.Desc([0], [], [], 64, 32, "bf16", n_tokens=17)
    assert P.plora_validate(d0) == 0


def test_sizes(P):
    d = desc(P, counts=(3, 0, 5), ranks=(4, 8, 16))
    assert P.plora_h_elems(d) == 3 * 4 + 0 + 5 * 16
    # workspace = [dA partials][dB partials][G^T hi+lo][H^T hi+lo], each rounded to 256 B;
    # the transposed blocks hold r_i rows of pad64(n_i) bf16 tokens
    r256 = lambda b: (b + 255) // 256 * 256
    pad64 = lambda n: (n + 63) // 64 * 64
    ft = r256((4 * pad64(3) + 8 * pad64(0) + 16 * pad64(5)) * 2 * 2)
    assert P.plora_workspace_bytes(d) == 0 + 0 + 2 * ft
    big = desc(P, counts=(5000, 1, 0), ranks=(64, 8, 16), d_in=4096, d_out=16384)
    # d_in <= 8192: 1024-token chunks; d_out > 8192: 2048-token chunks; only adapter 0 is split
    a = 5 * 64 * 4096 * 4
    b = 3 * 64 * 16384 * 4
    ft = r256((64 * pad64(5000) + 8 * pad64(1) + 16 * pad64(0)) * 2 * 2)
    assert P.plora_workspace_bytes(big) == r256(a) + r256(b) + 2 * ft
    assert P.plora_workspace_bytes(desc(P, d_in=12)) == 0  # invalid -> 0
    assert P.plora_workspace_bytes(desc(P, dtype="f32")) == 0


def raw(lib_fn_name, P, *args):
    return getattr(P._lib, lib_fn_name)(*args)


def test_error_paths_have_no_side_effects(P):
    d = desc(P)
    # NULL required pointers
    rc = P._lib.plora_forward(d.ref(), None, None, None, None, None, None, None)
    assert rc == -1 and "required" in P.plora_last_error()
    # misaligned device pointers are rejected before any launch
    rc = P._lib.plora_forward(d.ref(), 0x1001, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None)
    assert rc == -9
    rc = P._lib.plora_backward_dx(d.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5008, 0x6000, None)
    assert rc == -9
    # invalid descriptor
    bad = desc(P, ranks=(4, 0, 16))
    assert P._lib.plora_backward_dAdB(bad.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 0,
                                      None) == -3
    # workspace too small
    big = desc(P, counts=(5000, 1, 0), ranks=(64, 8, 16), d_in=4096, d_out=16384)
    rc = P._lib.plora_backward_dAdB(big.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 16, None)
    assert rc == -8 and "workspace" in P.plora_last_error()
    # T = 0 forward is a no-op (nothing touched, no GPU needed)
    z = P.Desc([0, 0, 0], [4, 8], [1.0, 1.0], 64, 32, "bf16")
    assert P._lib.plora_forward(z.ref(), None, None, None, None, None, None, None) == 0
    assert P._lib.plora_backward_dx(z.ref(), None, None, None, None, None, None, None) == 0
    # N = 0 backward_dAdB is a no-op
    n0 = P.Desc([0], [], [], 64, 32, "bf16", n_tokens=5)
    assert P._lib.plora_backward_dAdB(n0.ref(), None, None, None, None, None, None, None, 0, None) == 0


def test_python_shape_checks(P):
    torch = pytest.importorskip("torch")
    d = desc(P, counts=(3, 0, 5), d_in=64, d_out=32)
    X = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        P.plora_forward(d, X, torch.zeros(32, 65, dtype=torch.bfloat16), None, None, None, None, stream=0)
    with pytest.raises(ValueError):
        P.plora_forward(d, X.float(), None, None, None, None, None, stream=0)


def test_python_device_checks(P):
    """Host tensors of the right shape and dtype are refused before the call:
    their addresses would reach a kernel as device pointers."""
    torch = pytest.importorskip("torch")
    d = desc(P, counts=(3, 0, 5), d_in=64, d_out=32)
    bf = torch.bfloat16
    X, W = torch.zeros(8, 64, dtype=bf), torch.zeros(32, 64, dtype=bf)
    A, B = torch.zeros(28, 64, dtype=bf), torch.zeros(28, 32, dtype=bf)
    Y, H = torch.zeros(8, 32, dtype=bf), torch.zeros(P.plora_h_elems(d), dtype=torch.float32)
    with pytest.raises(ValueError, match="device memory"):
        P.plora_forward(d, X, W, A, B, Y, H, stream=0)
    dX, G = torch.zeros(8, 64, dtype=bf), torch.zeros(P.plora_h_elems(d), dtype=torch.float32)
    with pytest.raises(ValueError, match="device memory"):
        P.plora_backward_dx(d, Y, W, A, B, dX, G, stream=0)
    dA, dB = torch.zeros(28, 64), torch.zeros(28, 32)
    with pytest.raises(ValueError, match="device memory"):
        P.plora_backward_dAdB(d, X, Y, H, G, dA, dB, None, stream=0)


def test_desc_array_lengths(P):
    """The descriptor's host arrays must have N + 1 offsets and N alphas: the
    library reads them through raw pointers."""
    with pytest.raises(ValueError, match="segment offsets"):
        P.Desc([0, 3, 8], [4, 8, 16], [1.0, 1.0, 1.0], 64, 32)
    with pytest.raises(ValueError, match="segment offsets"):
        P.Desc([0, 3, 3, 8, 9], [4, 8, 16], [1.0, 1.0, 1.0], 64, 32)
    with pytest.raises(ValueError, match="alphas"):
        P.Desc([0, 3, 3, 8], [4, 8, 16], [1.0, 1.0], 64, 32)
    with pytest.raises(ValueError, match="alphas"):
        P.Desc([0, 3, 3, 8], [4, 8, 16], [1.0, 1.0, 1.0, 1.0], 64, 32)
    assert P.plora_validate(P.Desc([0, 3, 3, 8], [4, 8, 16], [1.0, 1.0, 1.0], 64, 32)) == 0
    assert P.plora_validate(P.Desc([], [], [], 64, 32, n_tokens=4)) == 0


def test_profile_read_empty(P):
    P.plora_profile_reset()
    assert P.plora_profile_read("gemm_fwd") == (0, 0.0)


def test_planner_host_only_build(tmp_path):
    """The planner is plain C++: it builds with g++ alone and its tables are checked here."""
    src = os.path.join(ROOT, "packed_adapter_lora_amd", "csrc", "plan.cpp")
    drv = tmp_path / "drv.cpp"
    drv.write_text(r'''
#include "plan.h"
#include <cstdio>
int main() {
  int64_t off[5] = {0, 70, 70, 71, 4171};
  int32_t rk[4] = {8, 16, 3, 64};
  float al[4] = {16.f, 16.f, 6.f, 32.f};
  plora_desc d{4, PLORA_BF16, 4171, 4096, 14336, off, rk, al};
  const char* why;
  if (plora::validate_desc(&d, &why)) return 1;
  plora::SegTable s; plora::build_segtable(&d, &s);
  plora::WorkMap m; int u = plora::build_shrink_map(s, &m);
  plora::WgradPlan pa, pb; plora::build_wgrad_plan(s, 4096, &pa); plora::build_wgrad_plan(s, 14336, &pb);
  std::printf("%d %d %d %d %d %lld %lld %d %d %lld %d %g %g\n", u, m.pre[1], m.pre[2], m.pre[3], s.roff[4],
              (long long)s.hoff[4], (long long)pa.part_elems, pa.chunks.pre[4], pb.chunks.pre[4],
              (long long)pb.part_elems, s.rmax, s.scale[0], s.scale[2]);
  return 0;
}
''')
    exe = tmp_path / "drv"
    import subprocess
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", os.path.join(ROOT, "include"), "-I",
                    os.path.join(ROOT, "packed_adapter_lora_amd", "csrc"), str(drv), src, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True, check=True).stdout.split()
    # shrink tiles of 32 rows: 3 + 0 + 1 + 129
    assert out[:4] == ["133", "3", "3", "4"]
    assert out[4] == "91"  # R
    assert out[5] == str(70 * 8 + 1 * 3 + 4100 * 64)
    # dA (1024-token chunks): adapter 3 has 5 chunks -> partials 5*64*4096
    assert out[6] == str(5 * 64 * 4096) and out[7] == str(1 + 0 + 1 + 5)
    # dB (2048-token chunks): adapter 3 has 3 chunks
    assert out[8] == str(1 + 0 + 1 + 3) and out[9] == str(3 * 64 * 14336)
    assert out[10] == "64" and float(out[11]) == 2.0 and float(out[12]) == 2.0


def test_status_string_hparam(P):
    assert P.plora_status_string(-11) == "PLORA_ERR_HPARAM"


def test_adamw_validation(P):
    d = desc(P, counts=(3, 0, 5), ranks=(4, 8, 16))
    lib = P._lib
    ptrs = [0x1000 * (k + 1) for k in range(8)]  # never dereferenced: every case fails or is a no-op first

    def call(cfg, ps=ptrs, A=None, B=None, dd=d):
        return lib.plora_adamw_step(dd.ref(), cfg.ref() if cfg is not None else None, *ps, A, B, None)

    assert call(None) == -1
    assert call(P.AdamwConfig([1e-3] * 3, [1, 1, 1], beta1=1.0)) == -11
    assert call(P.AdamwConfig([1e-3] * 3, [1, 1, 1], beta2=-0.1)) == -11
    assert call(P.AdamwConfig([1e-3] * 3, [1, 1, 1], eps=0.0)) == -11
    assert call(P.AdamwConfig([1e-3, float("nan"), 1e-3], [1, 1, 1])) == -11
    assert call(P.AdamwConfig([1e-3] * 3, [1, 1, 1], weight_decay=[0.0, -1.0, 0.0])) == -11
    assert call(P.AdamwConfig([1e-3] * 3, [1, -2, 1])) == -11
    assert "step[1]" in P.plora_last_error()
    ok = P.AdamwConfig([1e-3] * 3, [1, 0, 2])
    assert call(ok, ps=[None] + ptrs[1:]) == -1
    assert call(ok, ps=ptrs[:3] + [0x3008] + ptrs[4:]) == -9
    assert call(ok, A=0x7001) == -9
    bad = desc(P, ranks=(4, 0, 16))
    assert call(ok, dd=bad) == -3
    n0 = P.Desc([0], [], [], 64, 32, "bf16", n_tokens=5)
    assert lib.plora_adamw_step(n0.ref(), None, *([None] * 10), None) == 0


def test_adamw_python_checks(P):
    torch = pytest.importorskip("torch")
    d = desc(P, counts=(3, 0, 5), ranks=(4, 8, 16), d_in=64, d_out=32)
    f = lambda *s: torch.zeros(*s, dtype=torch.float32)
    with pytest.raises(ValueError):
        P.AdamwConfig([1e-3, 1e-3], [1, 1, 1])
    with pytest.raises(ValueError):  # wrong number of adapters
        P.plora_adamw_step(d, P.AdamwConfig(1e-3, [1, 1]), f(28, 64), f(28, 32), f(28, 64), f(28, 64), f(28, 32),
                           f(28, 32), f(28, 64), f(28, 32))
    with pytest.raises(ValueError):  # PB with the shape of A
        P.plora_adamw_step(d, P.AdamwConfig(1e-3, [1, 1, 1]), f(28, 64), f(28, 64), f(28, 64), f(28, 64), f(28, 32),
                           f(28, 32), f(28, 64), f(28, 32))


def test_dadb_acc_error_paths(P):
    lib = P._lib
    bad = desc(P, ranks=(4, 0, 16))
    assert lib.plora_backward_dAdB_acc(bad.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 0, 1,
                                       None) == -3
    big = desc(P, counts=(5000, 1, 0), ranks=(64, 8, 16), d_in=4096, d_out=16384)
    assert lib.plora_backward_dAdB_acc(big.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 16, 1,
                                       None) == -8
    n0 = P.Desc([0], [], [], 64, 32, "bf16", n_tokens=5)
    assert lib.plora_backward_dAdB_acc(n0.ref(), None, None, None, None, None, None, None, 0, 1, None) == 0


def test_library_matches_sources(P):
    """The loaded library was built from the sources in this tree (the package
    refuses to load one that was not)."""
    from packed_adapter_lora_amd.build import source_hash
    assert P.plora_source_hash() == source_hash()
    assert len(source_hash()) == 16


def test_noalloc_error_paths(P):
    """The no-allocation entry point validates on the host before it looks up
    its scratch: invalid descriptors and problems whose workspace exceeds the
    scratch array return their codes without touching a GPU."""
    lib = P._lib
    bad = desc(P, ranks=(4, 0, 16))
    assert lib.plora_backward_dAdB_noalloc(bad.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0, None) == -3
    # 200000 tokens of one rank-128 adapter over d_in = 4096: 196 chunks of partials (411 MB)
    huge = desc(P, counts=(200000,), ranks=(128,), alphas=(1.0,), d_in=4096, d_out=16384)
    assert P.plora_workspace_bytes(huge) > (256 << 20)
    rc = lib.plora_backward_dAdB_noalloc(huge.ref(), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0, None)
    assert rc == -8 and "scratch" in P.plora_last_error()
    n0 = P.Desc([0], [], [], 64, 32, "bf16", n_tokens=5)
    assert lib.plora_backward_dAdB_noalloc(n0.ref(), None, None, None, None, None, None, 1, None) == 0


def test_shared_input_error_paths(P):
    """The shared-input entry points check the panel count, their pointers and
    the workspace on the host before anything is enqueued; plora_backward_dAdB
    skips a NULL output but needs one of the two."""
    lib = P._lib
    d = desc(P)
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    for np_ in (0, 4):
        assert lib.plora_shrink_shared(d.ref(), 0x1000, np_, arr(0x2000), arr(0x3000), None) == -5
        assert lib.plora_backward_dA_shared(d.ref(), 0x1000, np_, arr(0x2000), arr(0x3000), None, 0, 0, None) == -5
        assert P.plora_workspace_bytes_dA_shared(d, np_) == 0
    assert lib.plora_shrink_shared(d.ref(), 0x1000, 2, arr(0x2000, None), arr(0x3000, 0x4000), None) == -1
    assert lib.plora_shrink_shared(d.ref(), 0x1000, 2, arr(0x2000, 0x2008), arr(0x3000, 0x4000), None) == -9
    assert lib.plora_backward_dA_shared(d.ref(), 0x1000, 2, arr(0x2000, 0x2100), arr(0x3000, None), None, 0, 0,
                                        None) == -1
    big = desc(P, counts=(5000, 1, 0), ranks=(64, 8, 16), d_in=4096, d_out=16384)
    need3 = P.plora_workspace_bytes_dA_shared(big, 3)
    assert need3 > P.plora_workspace_bytes_dA_shared(big, 1) > 0
    rc = lib.plora_backward_dA_shared(big.ref(), 0x1000, 3, arr(0x2000, 0x2100, 0x2200), arr(0x3000, 0x3100, 0x3200),
                                      0x7000, need3 - 256, 0, None)
    assert rc == -8 and "workspace" in P.plora_last_error()
    assert lib.plora_forward_expand(d.ref(), 0x1000, 0x2000, None, 0x4000, 0x5000, None) == -1
    assert lib.plora_backward_dAdB_acc(d.ref(), 0x1000, 0x2000, 0x3000, 0x4000, None, None, None, 0, 0, None) == -1
    assert lib.plora_backward_dAdB_acc(d.ref(), 0x1000, None, 0x3000, 0x4000, None, 0x6000, None, 0, 0, None) == -1
    # N = 0 and T = 0 are no-ops
    n0 = P.Desc([0], [], [], 64, 32, "bf16", n_tokens=5)
    assert lib.plora_shrink_shared(n0.ref(), None, 3, None, None, None) == 0
    assert lib.plora_backward_dA_shared(n0.ref(), None, 2, None, None, None, 0, 0, None) == 0


def test_dx_swiglu_error_paths(P):
    """The fused down-projection/SwiGLU backward validates on the host: bf16
    only, every pointer it writes or reads, 16-byte alignment; T = 0 is a
    no-op."""
    lib = P._lib
    d = desc(P)
    # pointer values that every case below rejects before anything is enqueued
    args = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 0x8000, 0x9000]
    f32 = desc(P, dtype="f32")
    assert lib.plora_backward_dx_swiglu(f32.ref(), *args, None) == -7
    for k in (0, 1, 4, 5, 6, 7):  # dY, W, g, u, dg, du
        a = list(args)
        a[k] = None
        assert lib.plora_backward_dx_swiglu(d.ref(), *a, None) == -1, k
    a = list(args)
    a[4] += 8  # g misaligned
    assert lib.plora_backward_dx_swiglu(d.ref(), *a, None) == -9
    assert lib.plora_backward_dx_swiglu(desc(P, ranks=(4, 0, 16)).ref(), *args, None) == -3
    n0 = P.Desc([0, 0], [8], [16.0], 64, 32, "bf16")
    assert lib.plora_backward_dx_swiglu(n0.ref(), *([None] * 9), None) == 0


def test_probe_error_paths(P):
    """The ceiling probes reject bad arguments on the host, before any launch."""
    lib = P._lib
    fl = ctypes.c_double(0.0)
    assert lib.plora_probe_mfma(0x1000, 3, 1, 1, 0x2000, ctypes.byref(fl), None) == -5  # shape 0..2
    assert lib.plora_probe_mfma(None, 0, 1, 1, 0x2000, ctypes.byref(fl), None) == -1
    assert lib.plora_probe_mfma(0x1000, 2, 0, 1, 0x2000, ctypes.byref(fl), None) == -5
    assert lib.plora_probe_mfma(0x1008, 2, 1, 1, 0x2000, ctypes.byref(fl), None) == -9
    nb = ctypes.c_double(0.0)
    assert lib.plora_probe_lds_dma(0x1000, 4096 + 16, 1, 1, 0x2000, ctypes.byref(nb), None) == -5
    assert lib.plora_probe_lds_dma(0x1000, 0, 1, 1, 0x2000, ctypes.byref(nb), None) == -5
    assert lib.plora_probe_lds_dma(0x1000, (1 << 30) + 4096, 1, 1, 0x2000, ctypes.byref(nb), None) == -5
    assert lib.plora_probe_lds_dma(0x1000, 4096, 0, 1, 0x2000, ctypes.byref(nb), None) == -5
    assert lib.plora_probe_lds_dma(None, 4096, 1, 1, 0x2000, ctypes.byref(nb), None) == -1
    assert lib.plora_probe_lds_dma(0x1000, 4096, 1, 1, 0x2004, ctypes.byref(nb), None) == -9
    assert "aligned" in P.plora_last_error()
