// api.hip -- the C ABI of the packed multi-LoRA operator (see include/plora.h).
//
// Each entry point validates everything on the host first (no side effects on
// failure), builds the per-adapter table and work maps, and enqueues its
// kernels on the caller's stream.  No device memory is allocated and nothing
// is synchronised.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "api_util.h"
#include "block_launch.h"
#include "launch.h"
#include "plan.h"
#include "plora.h"
#include "plora_block.h"

#ifndef PLORA_SOURCE_HASH
#define PLORA_SOURCE_HASH "unstamped"
#endif

namespace plora {

thread_local std::string g_last_error;

int fail(int status, const std::string& why) {
    g_last_error = std::string(plora_status_string(status)) + ": " + why;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PLORA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

Prof g_prof;

hipEvent_t take_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

namespace {

int check_common(const plora_desc* d) {
    const char* why = "";
    const int rc = validate_desc(d, &why);
    if (rc != PLORA_OK) return fail(rc, why);
    return PLORA_OK;
}

}  // namespace
}  // namespace plora

using namespace plora;

extern "C" {

const char* plora_status_string(int s) {
    switch (s) {
        case PLORA_OK: return "PLORA_OK";
        case PLORA_ERR_NULL: return "PLORA_ERR_NULL";
        case PLORA_ERR_SEGMENTS: return "PLORA_ERR_SEGMENTS";
        case PLORA_ERR_RANK: return "PLORA_ERR_RANK";
        case PLORA_ERR_ALPHA: return "PLORA_ERR_ALPHA";
        case PLORA_ERR_SHAPE: return "PLORA_ERR_SHAPE";
        case PLORA_ERR_ADAPTERS: return "PLORA_ERR_ADAPTERS";
        case PLORA_ERR_DTYPE: return "PLORA_ERR_DTYPE";
        case PLORA_ERR_WORKSPACE: return "PLORA_ERR_WORKSPACE";
        case PLORA_ERR_ALIGN: return "PLORA_ERR_ALIGN";
        case PLORA_ERR_HIP: return "PLORA_ERR_HIP";
        case PLORA_ERR_HPARAM: return "PLORA_ERR_HPARAM";
        default: return "PLORA_ERR_UNKNOWN";
    }
}

const char* plora_last_error(void) { return g_last_error.c_str(); }

int plora_version(void) { return PLORA_ABI_VERSION; }

const char* plora_source_hash(void) { return PLORA_SOURCE_HASH; }

int plora_validate(const plora_desc* d) {
    const char* why = "";
    return validate_desc(d, &why);
}

size_t plora_h_elems(const plora_desc* d) {
    if (plora_validate(d) != PLORA_OK) return 0;
    SegTable s;
    build_segtable(d, &s);
    return (size_t)s.hoff[s.n];
}

size_t plora_workspace_bytes(const plora_desc* d) {
    if (plora_validate(d) != PLORA_OK) return 0;
    if (d->dtype == PLORA_F32) return 0;
    SegTable s;
    build_segtable(d, &s);
    return workspace_bytes(s, d->d_in, d->d_out);
}

int plora_forward(const plora_desc* d, const void* X, const void* W, const void* A, const void* B, void* Y,
                  float* H, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->n_tokens == 0) return PLORA_OK;
        const bool lora = d->n_adapters > 0;
        if (!X || !W || !Y) return fail(PLORA_ERR_NULL, "X, W and Y are required");
        if (lora && (!A || !B || !H)) return fail(PLORA_ERR_NULL, "A, B and H are required when n_adapters > 0");
        if (misaligned(X) || misaligned(W) || misaligned(Y) || (lora && (misaligned(A) || misaligned(B) || misaligned(H))))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const bool bf = d->dtype == PLORA_BF16;
        hipError_t e = hipSuccess;
        if (lora) {
            const ShrinkArgs sa{X, A, H, d->d_in, Y, d->d_out * 2, 0};
            if (bf) {
                WorkMap m;
                const int32_t units = build_shrink_map(s, &m);
                e = timed("shrink", st, [&] { return launch_shrink_bf16(sa, s, m, units, st); });
            } else {
                e = timed("shrink", st, [&] { return launch_shrink_f32(sa, s, st); });
            }
            if (e != hipSuccess) return hip_fail(e, "shrink launch");
        }
        const GemmArgs ga{W, X, B, H, Y, d->n_tokens, d->d_in, d->d_out, lora ? 1 : 0};
        e = timed("gemm_fwd", st, [&] { return bf ? launch_gemm_bf16(true, ga, s, st) : launch_gemm_f32(true, ga, s, st); });
        if (e != hipSuccess) return hip_fail(e, "gemm launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_backward_dx(const plora_desc* d, const void* dY, const void* W, const void* A, const void* B, void* dX,
                      float* G, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->n_tokens == 0) return PLORA_OK;
        const bool lora = d->n_adapters > 0;
        if (!dY || !W || !dX) return fail(PLORA_ERR_NULL, "dY, W and dX are required");
        if (lora && (!A || !B || !G)) return fail(PLORA_ERR_NULL, "A, B and G are required when n_adapters > 0");
        if (misaligned(dY) || misaligned(W) || misaligned(dX) ||
            (lora && (misaligned(A) || misaligned(B) || misaligned(G))))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const bool bf = d->dtype == PLORA_BF16;
        hipError_t e = hipSuccess;
        if (lora) {
            const ShrinkArgs sa{dY, B, G, d->d_out, dX, d->d_in * 2, 0};
            if (bf) {
                WorkMap m;
                const int32_t units = build_shrink_map(s, &m);
                e = timed("shrink", st, [&] { return launch_shrink_bf16(sa, s, m, units, st); });
            } else {
                e = timed("shrink", st, [&] { return launch_shrink_f32(sa, s, st); });
            }
            if (e != hipSuccess) return hip_fail(e, "shrink launch");
        }
        // dX[t][k] = sum_n dY[t][n] W[n][k] + ...: P(p = k, kk = n) = W[n][k] is p-contiguous.
        const GemmArgs ga{W, dY, A, G, dX, d->n_tokens, d->d_out, d->d_in, lora ? 1 : 0};
        e = timed("gemm_bwd", st, [&] { return bf ? launch_gemm_bf16(false, ga, s, st) : launch_gemm_f32(false, ga, s, st); });
        if (e != hipSuccess) return hip_fail(e, "gemm launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_backward_dx_swiglu(const plora_desc* d, const void* dY, const void* W, const void* A, const void* B,
                             const void* g, const void* u, void* dg, void* du, float* G, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->dtype != PLORA_BF16) return fail(PLORA_ERR_DTYPE, "the fused SwiGLU backward is bf16 only");
        if (d->n_tokens == 0) return PLORA_OK;
        const bool lora = d->n_adapters > 0;
        if (!dY || !W || !g || !u || !dg || !du) return fail(PLORA_ERR_NULL, "dY, W, g, u, dg and du are required");
        if (lora && (!A || !B || !G)) return fail(PLORA_ERR_NULL, "A, B and G are required when n_adapters > 0");
        if (misaligned(dY) || misaligned(W) || misaligned(g) || misaligned(u) || misaligned(dg) || misaligned(du) ||
            (lora && (misaligned(A) || misaligned(B) || misaligned(G))))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        hipError_t e = hipSuccess;
        if (lora) {
            // dg is the scratch of the shrink's K slices (the GEMM writes it afterwards)
            const ShrinkArgs sa{dY, B, G, d->d_out, dg, d->d_in * 2, 0};
            WorkMap m;
            const int32_t units = build_shrink_map(s, &m);
            e = timed("shrink", st, [&] { return launch_shrink_bf16(sa, s, m, units, st); });
            if (e != hipSuccess) return hip_fail(e, "shrink launch");
        }
        GemmArgs ga{W, dY, A, G, dg, d->n_tokens, d->d_out, d->d_in, lora ? 1 : 0};
        if (gemm_bf16_pipelined(ga, s)) {
            // da never leaves the GEMM: its epilogue writes dg and du
            ga.sw_g = g;
            ga.sw_u = u;
            ga.sw_dg = dg;
            ga.sw_du = du;
            e = timed("gemm_bwd", st, [&] { return launch_gemm_bf16(false, ga, s, st); });
            if (e != hipSuccess) return hip_fail(e, "gemm launch");
        } else {
            // da into dg, then the SwiGLU backward in place (element by element)
            e = timed("gemm_bwd", st, [&] { return launch_gemm_bf16(false, ga, s, st); });
            if (e != hipSuccess) return hip_fail(e, "gemm launch");
            e = timed("swiglu", st, [&] { return launch_swiglu_bwd(dg, g, u, dg, du, d->n_tokens * d->d_in, st); });
            if (e != hipSuccess) return hip_fail(e, "swiglu launch");
        }
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_backward_dAdB(const plora_desc* d, const void* X, const void* dY, const float* H, const float* G, float* dA,
                        float* dB, void* ws, size_t ws_bytes, void* stream) {
    return plora_backward_dAdB_acc(d, X, dY, H, G, dA, dB, ws, ws_bytes, 0, stream);
}

int plora_backward_dAdB_acc(const plora_desc* d, const void* X, const void* dY, const float* H, const float* G,
                            float* dA, float* dB, void* ws, size_t ws_bytes, int accumulate, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->n_adapters == 0) return PLORA_OK;
        if (!dA && !dB) return fail(PLORA_ERR_NULL, "dA or dB is required");
        if (d->n_tokens > 0 && dB && (!dY || !H)) return fail(PLORA_ERR_NULL, "dB needs dY and H");
        if (d->n_tokens > 0 && dA && (!X || !G)) return fail(PLORA_ERR_NULL, "dA needs X and G");
        if (misaligned(X) || misaligned(dY) || misaligned(H) || misaligned(G) || misaligned(dA) || misaligned(dB))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const int32_t acc = accumulate ? 1 : 0;
        hipError_t e = hipSuccess;
        if (d->dtype == PLORA_F32) {
            const WgradArgs wb{dY, H, dB, nullptr, d->d_out, acc};
            const WgradArgs wa{X, G, dA, nullptr, d->d_in, acc};
            if (dB) {
                e = timed("wgrad", st, [&] { return launch_wgrad_f32(wb, s, st); });
                if (e != hipSuccess) return hip_fail(e, "wgrad launch");
            }
            if (dA) {
                e = timed("wgrad", st, [&] { return launch_wgrad_f32(wa, s, st); });
                if (e != hipSuccess) return hip_fail(e, "wgrad launch");
            }
            return PLORA_OK;
        }
        const size_t need = workspace_bytes(s, d->d_in, d->d_out);
        if (ws_bytes < need || (need > 0 && !ws))
            return fail(PLORA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
        if (need > 0 && misaligned(ws)) return fail(PLORA_ERR_ALIGN, "workspace must be 16-byte aligned");
        WgradPlan pa, pb;
        build_wgrad_plan(s, d->d_in, &pa);
        build_wgrad_plan(s, d->d_out, &pb);
        const WorkspaceLayout wl = workspace_layout(s, d->d_in, d->d_out);
        uint8_t* wsb = static_cast<uint8_t*>(ws);
        float* part_a = wsb ? reinterpret_cast<float*>(wsb + wl.part_a) : nullptr;
        float* part_b = wsb ? reinterpret_cast<float*>(wsb + wl.part_b) : nullptr;
        __bf16* g_hi = wsb ? reinterpret_cast<__bf16*>(wsb + wl.ft_g) : nullptr;
        __bf16* h_hi = wsb ? reinterpret_cast<__bf16*>(wsb + wl.ft_h) : nullptr;
        const WgradArgs wb{dY, H, dB, part_b, d->d_out, acc};
        const WgradArgs wa{X, G, dA, part_a, d->d_in, acc};
        // one launch for the transposes of H and G, the two weight-gradient
        // passes, one launch for both passes' chunk reductions
        const bool pipe_b = dB && wgrad_pipe_ok(wb, s, pb, h_hi);
        const bool pipe_a = dA && wgrad_pipe_ok(wa, s, pa, g_hi);
        const float* pf[2];
        __bf16 *phi[2], *plo[2];
        int np = 0;
        if (pipe_b) pf[np] = H, phi[np] = h_hi, plo[np++] = h_hi + pb.ft_elems;
        if (pipe_a) pf[np] = G, phi[np] = g_hi, plo[np++] = g_hi + pa.ft_elems;
        if (np > 0) {
            e = timed("wgrad", st, [&] { return launch_wgrad_prep(np, pf, phi, plo, s, pa, st); });
            if (e != hipSuccess) return hip_fail(e, "wgrad launch");
        }
        const WgradArgs* ra[2];
        const WgradPlan* rp[2];
        int nr = 0;
        if (dB) {
            e = timed("wgrad", st, [&] {
                return pipe_b ? launch_wgrad_bf16_pipe(wb, s, pb, h_hi, h_hi + pb.ft_elems, st)
                              : launch_wgrad_bf16(wb, s, pb, st);
            });
            if (e != hipSuccess) return hip_fail(e, "wgrad launch");
            ra[nr] = &wb, rp[nr++] = &pb;
        }
        if (dA) {
            e = timed("wgrad", st, [&] {
                return pipe_a ? launch_wgrad_bf16_pipe(wa, s, pa, g_hi, g_hi + pa.ft_elems, st)
                              : launch_wgrad_bf16(wa, s, pa, st);
            });
            if (e != hipSuccess) return hip_fail(e, "wgrad launch");
            ra[nr] = &wa, rp[nr++] = &pa;
        }
        e = timed("reduce", st, [&] { return launch_wgrad_reduce(nr, ra, rp, s, st); });
        if (e != hipSuccess) return hip_fail(e, "reduce launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_shrink_shared(const plora_desc* d, const void* X, int np, const void* const* A, float* const* H,
                        void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (np < 1 || np > 3) return fail(PLORA_ERR_SHAPE, "np must be 1, 2 or 3");
        if (d->n_adapters == 0 || d->n_tokens == 0) return PLORA_OK;
        if (!X || !A || !H) return fail(PLORA_ERR_NULL, "X, A and H are required");
        for (int p = 0; p < np; ++p) {
            if (!A[p] || !H[p]) return fail(PLORA_ERR_NULL, "A[" + std::to_string(p) + "] and H[p] are required");
            if (misaligned(A[p]) || misaligned(H[p])) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        }
        if (misaligned(X)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        hipError_t e = hipSuccess;
        if (d->dtype == PLORA_BF16) {
            ShrinkArgs sa{X, A[0], H[0], d->d_in, nullptr, 0, 0};
            sa.P1 = np > 1 ? A[1] : nullptr;
            sa.P2 = np > 2 ? A[2] : nullptr;
            sa.out1 = np > 1 ? H[1] : nullptr;
            sa.out2 = np > 2 ? H[2] : nullptr;
            sa.np = np;
            WorkMap m;
            const int32_t units = build_shrink_map(s, &m);
            e = timed("shrink", st, [&] { return launch_shrink_bf16(sa, s, m, units, st); });
            if (e != hipSuccess) return hip_fail(e, "shrink launch");
        } else {
            for (int p = 0; p < np; ++p) {
                const ShrinkArgs sa{X, A[p], H[p], d->d_in, nullptr, 0, 0};
                e = timed("shrink", st, [&] { return launch_shrink_f32(sa, s, st); });
                if (e != hipSuccess) return hip_fail(e, "shrink launch");
            }
        }
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_forward_expand(const plora_desc* d, const void* X, const void* W, const void* B, void* Y, const float* H,
                         void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->n_tokens == 0) return PLORA_OK;
        const bool lora = d->n_adapters > 0;
        if (!X || !W || !Y) return fail(PLORA_ERR_NULL, "X, W and Y are required");
        if (lora && (!B || !H)) return fail(PLORA_ERR_NULL, "B and H are required when n_adapters > 0");
        if (misaligned(X) || misaligned(W) || misaligned(Y) || (lora && (misaligned(B) || misaligned(H))))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const bool bf = d->dtype == PLORA_BF16;
        const GemmArgs ga{W, X, B, H, Y, d->n_tokens, d->d_in, d->d_out, lora ? 1 : 0};
        const hipError_t e =
            timed("gemm_fwd", st, [&] { return bf ? launch_gemm_bf16(true, ga, s, st) : launch_gemm_f32(true, ga, s, st); });
        if (e != hipSuccess) return hip_fail(e, "gemm launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

size_t plora_workspace_bytes_dA_shared(const plora_desc* d, int np) {
    if (plora_validate(d) != PLORA_OK || np < 1 || np > 3) return 0;
    if (d->dtype == PLORA_F32) return 0;
    SegTable s;
    build_segtable(d, &s);
    return dA_shared_layout(s, d->d_in, np).total;
}

int plora_backward_dA_shared(const plora_desc* d, const void* X, int np, const float* const* G, float* const* dA,
                             void* ws, size_t ws_bytes, int accumulate, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (np < 1 || np > 3) return fail(PLORA_ERR_SHAPE, "np must be 1, 2 or 3");
        if (d->n_adapters == 0) return PLORA_OK;
        if (!dA || (d->n_tokens > 0 && (!X || !G))) return fail(PLORA_ERR_NULL, "X, G and dA are required");
        for (int p = 0; p < np; ++p) {
            if (!dA[p] || (d->n_tokens > 0 && !G[p]))
                return fail(PLORA_ERR_NULL, "G[" + std::to_string(p) + "] and dA[p] are required");
            if (misaligned(dA[p]) || (d->n_tokens > 0 && misaligned(G[p])))
                return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        }
        if (misaligned(X)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        SegTable s;
        build_segtable(d, &s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const int32_t acc = accumulate ? 1 : 0;
        const float* g[3] = {nullptr, nullptr, nullptr};
        for (int p = 0; p < np; ++p) g[p] = d->n_tokens > 0 ? G[p] : nullptr;
        hipError_t e = hipSuccess;
        if (d->dtype == PLORA_F32) {
            for (int p = 0; p < np; ++p) {
                const WgradArgs wa{X, g[p], dA[p], nullptr, d->d_in, acc};
                e = timed("wgrad", st, [&] { return launch_wgrad_f32(wa, s, st); });
                if (e != hipSuccess) return hip_fail(e, "wgrad launch");
            }
            return PLORA_OK;
        }
        const SharedDaLayout wl = dA_shared_layout(s, d->d_in, np);
        if (ws_bytes < wl.total || (wl.total > 0 && !ws))
            return fail(PLORA_ERR_WORKSPACE, "workspace needs " + std::to_string(wl.total) + " bytes");
        if (wl.total > 0 && misaligned(ws)) return fail(PLORA_ERR_ALIGN, "workspace must be 16-byte aligned");
        WgradPlan pa;
        build_wgrad_plan(s, d->d_in, &pa);
        uint8_t* wsb = static_cast<uint8_t*>(ws);
        float* part = wsb ? reinterpret_cast<float*>(wsb) : nullptr;
        __bf16* g_hi = wsb ? reinterpret_cast<__bf16*>(wsb + wl.ft_base) : nullptr;
        WgradArgs wa{X, g[0], dA[0], part, d->d_in, acc};
        wa.F1 = g[1];
        wa.F2 = g[2];
        wa.out1 = np > 1 ? dA[1] : nullptr;
        wa.out2 = np > 2 ? dA[2] : nullptr;
        wa.part_stride = (int64_t)(wl.part_stride / 4);
        wa.ft_stride = (int64_t)(wl.ft_stride / 2);
        wa.np = np;
        const bool pipe = wgrad_pipe_ok(wa, s, pa, g_hi);
        if (pipe) {
            // the np transposes in one launch (panel p's at p * ft_stride)
            __bf16 *phi[3], *plo[3];
            for (int p = 0; p < np; ++p) phi[p] = g_hi + p * wa.ft_stride, plo[p] = phi[p] + pa.ft_elems;
            e = timed("wgrad", st, [&] { return launch_wgrad_prep(np, g, phi, plo, s, pa, st); });
            if (e != hipSuccess) return hip_fail(e, "wgrad launch");
        }
        e = timed("wgrad", st, [&] {
            return pipe ? launch_wgrad_bf16_pipe(wa, s, pa, g_hi, g_hi + pa.ft_elems, st) : launch_wgrad_bf16(wa, s, pa, st);
        });
        if (e != hipSuccess) return hip_fail(e, "wgrad launch");
        // the panels' chunk reductions in one launch
        WgradArgs side[3];
        const WgradArgs* ra[3];
        const WgradPlan* rp[3];
        for (int p = 0; p < np; ++p) {
            side[p] = WgradArgs{X, g[p], dA[p], part ? part + p * wa.part_stride : nullptr, d->d_in, acc};
            ra[p] = &side[p];
            rp[p] = &pa;
        }
        e = timed("reduce", st, [&] { return launch_wgrad_reduce(np, ra, rp, s, st); });
        if (e != hipSuccess) return hip_fail(e, "reduce launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_adamw_step(const plora_desc* d, const plora_adamw_config* cfg, float* PA, float* PB, float* mA, float* vA,
                     float* mB, float* vB, const float* dA, const float* dB, void* A, void* B, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->n_adapters == 0) return PLORA_OK;
        if (!cfg || !cfg->lr || !cfg->weight_decay || !cfg->step)
            return fail(PLORA_ERR_NULL, "the AdamW configuration and its lr, weight_decay and step arrays are required");
        const float b1 = cfg->beta1, b2 = cfg->beta2, eps = cfg->eps;
        if (!(b1 >= 0.0f && b1 < 1.0f) || !(b2 >= 0.0f && b2 < 1.0f))
            return fail(PLORA_ERR_HPARAM, "betas must lie in [0, 1)");
        if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(PLORA_ERR_HPARAM, "eps must be finite and > 0");
        for (int i = 0; i < d->n_adapters; ++i) {
            if (!(cfg->lr[i] >= 0.0f) || !std::isfinite(cfg->lr[i]))
                return fail(PLORA_ERR_HPARAM, "lr[" + std::to_string(i) + "] must be finite and >= 0");
            if (!(cfg->weight_decay[i] >= 0.0f) || !std::isfinite(cfg->weight_decay[i]))
                return fail(PLORA_ERR_HPARAM, "weight_decay[" + std::to_string(i) + "] must be finite and >= 0");
            if (cfg->step[i] < 0) return fail(PLORA_ERR_HPARAM, "step[" + std::to_string(i) + "] must be >= 0");
        }
        if (!PA || !PB || !mA || !vA || !mB || !vB || !dA || !dB)
            return fail(PLORA_ERR_NULL, "PA, PB, mA, vA, mB, vB, dA and dB are required");
        if (misaligned(PA) || misaligned(PB) || misaligned(mA) || misaligned(vA) || misaligned(mB) ||
            misaligned(vB) || misaligned(dA) || misaligned(dB) || misaligned(A) || misaligned(B))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        AdamwTable t{};
        t.n = d->n_adapters;
        t.roff[0] = 0;
        for (int i = 0; i < t.n; ++i) {
            t.roff[i + 1] = t.roff[i] + d->ranks[i];
            const int64_t k = cfg->step[i];
            t.active[i] = k > 0;
            const double lr = cfg->lr[i], wd = cfg->weight_decay[i];
            t.decay[i] = (float)(1.0 - lr * wd);
            t.step_size[i] = k > 0 ? (float)(lr / (1.0 - std::pow((double)b1, (double)k))) : 0.0f;
            t.rs_bc2[i] = k > 0 ? (float)(1.0 / std::sqrt(1.0 - std::pow((double)b2, (double)k))) : 0.0f;
        }
        t.beta1 = b1;
        t.one_minus_beta1 = (float)(1.0 - (double)b1);
        t.beta2 = b2;
        t.one_minus_beta2 = (float)(1.0 - (double)b2);
        t.eps = eps;
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const int32_t bf = d->dtype == PLORA_BF16 ? 1 : 0;
        const AdamwArgs aa{PA, mA, vA, dA, A, bf, d->d_in};
        const AdamwArgs ab{PB, mB, vB, dB, B, bf, d->d_out};
        hipError_t e = timed("adamw", st, [&] { return launch_adamw(aa, t, st); });
        if (e != hipSuccess) return hip_fail(e, "adamw launch");
        e = timed("adamw", st, [&] { return launch_adamw(ab, t, st); });
        if (e != hipSuccess) return hip_fail(e, "adamw launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_cast_panels(const plora_desc* d, const float* PA, const float* PB, void* A, void* B, void* stream) {
    try {
        int rc = check_common(d);
        if (rc) return rc;
        if (d->n_adapters == 0) return PLORA_OK;
        if (!PA || !PB || !A || !B) return fail(PLORA_ERR_NULL, "PA, PB, A and B are required");
        if (misaligned(PA) || misaligned(PB) || misaligned(A) || misaligned(B))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        int64_t R = 0;
        for (int i = 0; i < d->n_adapters; ++i) R += d->ranks[i];
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const int32_t bf = d->dtype == PLORA_BF16 ? 1 : 0;
        hipError_t e = launch_cast_panel(PA, A, bf, R * d->d_in, st);
        if (e != hipSuccess) return hip_fail(e, "cast launch");
        e = launch_cast_panel(PB, B, bf, R * d->d_out, st);
        if (e != hipSuccess) return hip_fail(e, "cast launch");
        return PLORA_OK;
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_profile_enable(int on) {
    g_prof.on = on != 0;
    return PLORA_OK;
}

int plora_profile_read(const char* cls, int* launches, double* total_ms) {
    if (!cls || !launches || !total_ms) return fail(PLORA_ERR_NULL, "profile_read arguments");
    std::lock_guard<std::mutex> lk(g_prof.mu);
    int n = 0;
    double ms = 0.0;
    for (auto& r : g_prof.recs) {
        if (r.cls != cls) continue;
        float t = 0.0f;
        const hipError_t e = hipEventElapsedTime(&t, r.a, r.b);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        ++n;
        ms += t;
    }
    *launches = n;
    *total_ms = ms;
    return PLORA_OK;
}

void plora_profile_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (auto& r : g_prof.recs) {
        g_prof.pool.push_back(r.a);
        g_prof.pool.push_back(r.b);
    }
    g_prof.recs.clear();
}

}  // extern "C"
