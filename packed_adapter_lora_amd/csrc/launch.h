// launch.h -- internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace plora {

// Base GEMM with the fused LoRA term, token-major output:
//   O[q][p] = round( sum_k Q[q][k] P(p,k) + s_i sum_j F_i[q-o_i][j] E[R_off[i]+j][p] )
// for token q in segment i.  Forward: P(p,k) = W[p][k] (K-contiguous),
// E = B, F = H.  Backward-data: P(p,k) = W[k][p] (p-contiguous), E = A, F = G.
struct GemmArgs {
    const void* P;    // frozen weight
    const void* Q;    // X or dY, [T][K]
    const void* E;    // packed B (forward) or A (backward), [R][Pdim]
    const float* F;   // H or G
    void* O;          // Y or dX, [T][Pdim]
    int64_t T, K, Pdim;
    int32_t lora;     // 0: frozen path only
};

// Shrink: out[hoff_i + (t - o_i) r_i + j] = sum_k Q[t][k] P[R_off[i]+j][k]
// (H = X A_i with P = A, K = d_in;  G = dY B_i^T with P = B, K = d_out).
struct ShrinkArgs {
    const void* Q;   // [T][K]
    const void* P;   // [R][K]
    float* out;      // H or G
    int64_t K;
    void* scratch;       // output activation (Y or dX), free until the GEMM writes it
    int64_t scratch_row; // its bytes per token row (0: no K slices)
};

// Weight gradient: out[R_off[i]+j][c] = s_i sum_{t in S_i} F_i[t-o_i][j] Q[t][c]
// (dA: F = G, Q = X, D = d_in;  dB: F = H, Q = dY, D = d_out).
struct WgradArgs {
    const void* Q;     // [T][D]
    const float* F;    // H or G
    float* out;        // dA or dB, [R][D]
    float* part;       // fp32 partials (adapters split over several chunks)
    int64_t D;
    int32_t accumulate;  // nonzero: out += result (adapters without tokens untouched)
};

hipError_t launch_gemm_bf16(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st);
hipError_t launch_shrink_bf16(const ShrinkArgs& a, const SegTable& s, const WorkMap& m, int32_t units,
                              hipStream_t st);
hipError_t launch_wgrad_bf16(const WgradArgs& a, const SegTable& s, const WgradPlan& p, hipStream_t st);
// Pipelined weight gradient: first writes the transposed hi/lo bf16 copy of F
// (plan.ft_elems elements each) into fhi / flo, then reduces over tokens.
hipError_t launch_wgrad_bf16_pipe(const WgradArgs& a, const SegTable& s, const WgradPlan& p, __bf16* fhi, __bf16* flo,
                                  hipStream_t st);
hipError_t launch_wgrad_reduce(const WgradArgs& a, const SegTable& s, const WgradPlan& p, hipStream_t st);

// Per-adapter AdamW over one packed panel [R][D] (fp32 master P, moments m, v,
// gradient g; optional operator copy `out` of dtype out_dtype).  The factors
// are per adapter: decay = 1 - lr wd, step_size = lr / (1 - beta1^t),
// rs_bc2 = 1 / sqrt(1 - beta2^t); active = 0 skips the adapter.
struct AdamwTable {
    int32_t n;
    int32_t roff[kMaxN + 1];
    int32_t active[kMaxN];
    float decay[kMaxN];
    float step_size[kMaxN];
    float rs_bc2[kMaxN];
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps;
};
struct AdamwArgs {
    float* P;
    float* m;
    float* v;
    const float* g;
    void* out;          // nullptr: not written
    int32_t out_bf16;   // 1: bf16 (round to nearest even), 0: fp32
    int64_t D;
};
hipError_t launch_adamw(const AdamwArgs& a, const AdamwTable& t, hipStream_t st);

hipError_t launch_gemm_f32(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st);
hipError_t launch_shrink_f32(const ShrinkArgs& a, const SegTable& s, hipStream_t st);
hipError_t launch_wgrad_f32(const WgradArgs& a, const SegTable& s, hipStream_t st);

}  // namespace plora
