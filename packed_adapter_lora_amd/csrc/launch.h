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
    // feature range [p_begin, p_end) covered by one launch of the pipelined
    // kernel (p_end = 0: up to Pdim); Pdim stays the row length and bound
    int64_t p_begin, p_end;
    // SwiGLU backward fused into the epilogue (dX GEMM, pipelined path only;
    // sw_g = null: plain output O): with da = O's bf16 value, writes
    // sw_dg / sw_du [T][Pdim] from sw_g / sw_u [T][Pdim] instead of O
    const void* sw_g;
    const void* sw_u;
    void* sw_dg;
    void* sw_du;
    int32_t group_q;  // token tiles per L2 group of the tile map (0: 2)
};

// Shrink: out[hoff_i + (t - o_i) r_i + j] = sum_k Q[t][k] P[R_off[i]+j][k]
// (H = X A_i with P = A, K = d_in;  G = dY B_i^T with P = B, K = d_out).
// Shared input: np = 2 or 3 panels P, P1, P2 (same ranks, same segments) read
// one pass over Q and write out, out1, out2 (np = 0 or 1: P and out only).
struct ShrinkArgs {
    const void* Q;   // [T][K]
    const void* P;   // [R][K]
    float* out;      // H or G
    int64_t K;
    void* scratch;       // output activation (Y or dX), free until the GEMM writes it
    int64_t scratch_row; // its bytes per token row (0: no K slices)
    int32_t split_all;   // K slices for every adapter whose partials fit (not only single-tile ones)
    const void* P1;
    const void* P2;
    float* out1;
    float* out2;
    int32_t np;
};

// Weight gradient: out[R_off[i]+j][c] = s_i sum_{t in S_i} F_i[t-o_i][j] Q[t][c]
// (dA: F = G, Q = X, D = d_in;  dB: F = H, Q = dY, D = d_out).
// Shared input: np = 2 or 3 factors F, F1, F2 (same ranks, same segments) and
// outputs out, out1, out2 from one pass over Q; panel p's partials start
// p * part_stride floats after part and its transposed hi/lo factor p *
// ft_stride elements after the first (np = 0 or 1: F and out only).
struct WgradArgs {
    const void* Q;     // [T][D]
    const float* F;    // H or G
    float* out;        // dA or dB, [R][D]
    float* part;       // fp32 partials (adapters split over several chunks)
    int64_t D;
    int32_t accumulate;  // nonzero: out += result (adapters without tokens untouched)
    const float* F1;
    const float* F2;
    float* out1;
    float* out2;
    int64_t part_stride;
    int64_t ft_stride;
    int32_t np;
};

hipError_t launch_gemm_bf16(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st);
// whether launch_gemm_bf16 takes the pipelined kernels for this shape (the
// only ones with the fused SwiGLU epilogue)
bool gemm_bf16_pipelined(const GemmArgs& a, const SegTable& s);
hipError_t launch_shrink_bf16(const ShrinkArgs& a, const SegTable& s, const WorkMap& m, int32_t units,
                              hipStream_t st);
hipError_t launch_wgrad_bf16(const WgradArgs& a, const SegTable& s, const WgradPlan& p, hipStream_t st);
// Whether the pipelined weight-gradient kernel takes this reduction (ranks up
// to 64, the transposed copy of F given, offsets within 32 bits).
bool wgrad_pipe_ok(const WgradArgs& a, const SegTable& s, const WgradPlan& p, const __bf16* fhi);
// The transposed hi/lo bf16 copies of nside (1..3) F's over the same segments
// in one launch: F[k] into hi[k] / lo[k] (p.ft_elems elements each; the layout
// does not depend on the feature width, so any plan of the call will do).
hipError_t launch_wgrad_prep(int nside, const float* const* F, __bf16* const* hi, __bf16* const* lo,
                             const SegTable& s, const WgradPlan& p, hipStream_t st);
// Pipelined weight gradient over the copies launch_wgrad_prep wrote.
hipError_t launch_wgrad_bf16_pipe(const WgradArgs& a, const SegTable& s, const WgradPlan& p, const __bf16* fhi,
                                  const __bf16* flo, hipStream_t st);
// The chunk reductions (and the zero rows of adapters without tokens) of
// nside (1..3) weight-gradient passes of one call in one launch: pass k is a[k]
// (single panel: a[k]->np <= 1) with plan p[k].
hipError_t launch_wgrad_reduce(int nside, const WgradArgs* const* a, const WgradPlan* const* p, const SegTable& s,
                               hipStream_t st);

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
// out[e] = dtype copy of P[e] for e < n (bf16: round to nearest even).
hipError_t launch_cast_panel(const float* P, void* out, int32_t out_bf16, int64_t n, hipStream_t st);

hipError_t launch_gemm_f32(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st);
hipError_t launch_shrink_f32(const ShrinkArgs& a, const SegTable& s, hipStream_t st);
hipError_t launch_wgrad_f32(const WgradArgs& a, const SegTable& s, hipStream_t st);

}  // namespace plora
