"""The library's host code and the C oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, built with g++ / gcc here).

Host code: descriptor validation, the per-adapter tables, the shrink and
weight-gradient work maps, the workspace layouts and the packing planner,
driven over seeded random descriptors up to the limits (64 adapters, rank
128, empty and one-token segments) and random job sets.  Oracle: the fp64
reference on small random problems with every output requested, and its
validation paths.  Any out-of-bounds access, overflow or other undefined
behaviour aborts the program, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_adapter_lora_amd", "csrc")
INC = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

HOST_DRIVER = r'''
#include "plan.h"
#include "plora_planner.h"
#include <cstdio>
#include <cstdint>
#include <string>
#include <vector>

namespace plora {
int fail(int status, const std::string&) { return status; }  // (the library's version keeps the message)
}

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(uint32_t n) {  // splitmix64
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((z ^ (z >> 31)) % n);
}

int main() {
    using namespace plora;
    long checks = 0;
    for (int it = 0; it < 400; ++it) {
        const int n = it % 50 == 0 ? PLORA_MAX_ADAPTERS : 1 + (int)rnd(it % 3 == 0 ? PLORA_MAX_ADAPTERS : 40);
        std::vector<int64_t> off(n + 1, 0);
        std::vector<int32_t> rk(n);
        std::vector<float> al(n);
        for (int i = 0; i < n; ++i) {
            const uint32_t kind = rnd(6);
            const int64_t cnt = kind == 0 ? 0 : kind == 1 ? 1 : kind == 2 ? 1 + rnd(128) : 1 + rnd(3000);
            off[i + 1] = off[i] + cnt;
            rk[i] = it % 7 == 0 ? 128 : 1 + (int32_t)rnd(128);
            al[i] = 1.0f + (float)rnd(64);
        }
        const int64_t dims[4] = {64, 768, 4096, 14336};
        const int64_t d_in = dims[rnd(4)], d_out = dims[rnd(4)];
        plora_desc d{n, it % 5 == 0 ? PLORA_F32 : PLORA_BF16, off[n], d_in, d_out, off.data(), rk.data(), al.data()};
        const char* why = nullptr;
        if (validate_desc(&d, &why) != 0) return 10;
        SegTable s;
        build_segtable(&d, &s);
        WorkMap m;
        checks += build_shrink_map(s, &m);
        bool split = false;
        for (int rows : {32, 128})
            for (int row_bytes : {0, (int)(d_out * 2)})
                for (bool all : {false, true}) checks += build_shrink_pipe_map(s, &m, d_in, row_bytes, &split, rows, all);
        WgradPlan pa, pb;
        build_wgrad_plan(s, d_in, &pa);
        build_wgrad_plan(s, d_out, &pb);
        checks += (long)(workspace_bytes(s, d_in, d_out) & 0xff) + pa.chunks.pre[n] + pb.chunks.pre[n];
        for (int np = 1; np <= 3; ++np) checks += (long)(dA_shared_layout(s, d_in, np).total & 0xff);
        // invalid descriptors are rejected, not read past their arrays
        rk[rnd(n)] = 129;
        if (validate_desc(&d, &why) == 0) return 11;
        rk[0] = 0;
        if (validate_desc(&d, &why) == 0) return 12;
    }
    plora_desc bad{PLORA_MAX_ADAPTERS + 1, PLORA_BF16, 0, 64, 64, nullptr, nullptr, nullptr};
    const char* why = nullptr;
    if (validate_desc(&bad, &why) == 0) return 13;
    if (validate_desc(nullptr, &why) == 0) return 14;

    for (int it = 0; it < 200; ++it) {
        const int n = 1 + (int)rnd(it % 10 == 0 ? 2000 : 60);
        std::vector<plora_job> jobs(n);
        for (auto& j : jobs) {
            j.steps = 1 + rnd(5000);
            j.mem_bytes = 1e6 * (1 + rnd(40000));
            j.ms_per_step = 0.01 * rnd(500);
        }
        plora_pack_model model{4.1e10, 2.0, 1e7};
        std::vector<int32_t> pack(n, -1);
        int32_t n_packs = 0;
        double ms = 0.0;
        if (plora_plan_packs(jobs.data(), n, &model, pack.data(), &n_packs, &ms) != 0) return 20;
        if (plora_plan_makespan(jobs.data(), n, &model, pack.data(), n_packs) < 0.0) return 21;
        jobs[rnd(n)].mem_bytes = 5e10;  // larger than the budget: rejected
        if (plora_plan_packs(jobs.data(), n, &model, pack.data(), &n_packs, &ms) == 0) return 22;
        checks += n_packs;
    }
    std::printf("ok %ld\n", checks);
    return 0;
}
'''

ORACLE_DRIVER = r'''
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
int oracle_packed_lora(int n, int64_t T, const int64_t* off, const int32_t* ranks, const double* alphas,
                       int64_t d_in, int64_t d_out, const double* X, const double* dY, const double* W,
                       const double* A, const double* B, double* Y, double* H, double* dX, double* G,
                       double* dA, double* dB);
int64_t oracle_h_elems(int n, const int64_t* off, const int32_t* ranks);
static uint64_t st = 12345;
static double u(void) { st = st * 6364136223846793005ull + 1442695040888963407ull; return (double)(st >> 11) / 9007199254740992.0 - 0.5; }
static double* arr(int64_t k) { double* p = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double)); for (int64_t i = 0; i < k; ++i) p[i] = u(); return p; }
int main(void) {
    for (int it = 0; it < 40; ++it) {
        const int n = 1 + it % 7;
        int64_t off[8] = {0};
        int32_t rk[7];
        double al[7];
        for (int i = 0; i < n; ++i) {
            off[i + 1] = off[i] + (i % 3 == 0 ? 0 : 1 + (it * 7 + i * 5) % 23);
            rk[i] = 1 + (it + 3 * i) % 17;
            al[i] = 1.0 + i;
        }
        const int64_t T = off[n], di = 8 + 8 * (it % 4), dout = 16 + 8 * (it % 3);
        int64_t R = 0;
        for (int i = 0; i < n; ++i) R += rk[i];
        const int64_t he = oracle_h_elems(n, off, rk);
        double *X = arr(T * di), *dY = arr(T * dout), *W = arr(dout * di), *A = arr(R * di), *B = arr(R * dout);
        double *Y = arr(T * dout), *H = arr(he), *dX = arr(T * di), *G = arr(he), *dA = arr(R * di), *dB = arr(R * dout);
        if (oracle_packed_lora(n, T, off, rk, al, di, dout, X, dY, W, A, B, Y, H, dX, G, dA, dB) != 0) return 10;
        rk[0] = 200;  /* invalid: rejected before any array is read */
        if (oracle_packed_lora(n, T, off, rk, al, di, dout, X, dY, W, A, B, Y, H, dX, G, dA, dB) == 0) return 11;
        free(X); free(dY); free(W); free(A); free(B); free(Y); free(H); free(dX); free(G); free(dA); free(dB);
    }
    printf("ok\n");
    return 0;
}
'''


def _run(cmd, **kw):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)


def _sanitizers_work(tmp_path, compiler):
    src = tmp_path / ("probe.c" if compiler == "gcc" else "probe.cpp")
    src.write_text("int main(void) { return 0; }\n")
    exe = tmp_path / "probe"
    if _run([compiler] + SAN + [str(src), "-o", str(exe)]).returncode != 0:
        return False
    return _run([str(exe)]).returncode == 0


def test_host_code_under_asan_ubsan(tmp_path):
    if shutil.which("g++") is None or not _sanitizers_work(tmp_path, "g++"):
        pytest.skip("g++ with ASan/UBSan is not available")
    drv = tmp_path / "host_drv.cpp"
    drv.write_text(HOST_DRIVER)
    exe = tmp_path / "host_drv"
    b = _run(["g++", "-std=c++17"] + SAN + ["-I", INC, "-I", CSRC, str(drv), os.path.join(CSRC, "plan.cpp"),
                                            os.path.join(CSRC, "planner.cpp"), "-o", str(exe)])
    assert b.returncode == 0, b.stdout[-3000:]
    r = _run([str(exe)], timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-3000:]


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None or not _sanitizers_work(tmp_path, "gcc"):
        pytest.skip("gcc with ASan/UBSan is not available")
    drv = tmp_path / "oracle_drv.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_drv"
    b = _run(["gcc", "-std=c11", "-ffp-contract=off"] + SAN + [str(drv), os.path.join(ROOT, "oracle", "plora_oracle.c"),
                                                                "-lm", "-o", str(exe)])
    assert b.returncode == 0, b.stdout[-3000:]
    r = _run([str(exe)], timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-3000:]
