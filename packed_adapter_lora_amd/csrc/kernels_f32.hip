// kernels_f32.hip -- fp32 path of the packed multi-LoRA operator (gfx950).
//
// Same contractions as the bf16 path, in true fp32 on the vector ALUs (no
// reduced-precision matrix modes): the frozen GEMM with the LoRA term added
// in its epilogue, the segment-indexed shrink and the weight gradients
// [LLM+LoRA微调加速技术原理解析, 深入理解LoRA; PLoRA technical summary
// (gist.science, arXiv 2508.02932), 方法论 > 2. LoRA 执行引擎].  These are
// simple LDS-tiled kernels for small fp32 problems.
#include "device_common.h"
#include "launch.h"

namespace plora {
namespace {

// O[q][p] = sum_k Q[q][k] P(p,k) + s_i * sum_j F_i[q-o_i][j] E[R_off[i]+j][p]
template <bool P_KMAJOR>
__global__ __launch_bounds__(256) void gemm_lora_f32(GemmArgs a, SegTable seg) {
    __shared__ float qs[16][65];
    __shared__ float ps[16][65];
    const float* __restrict__ P = static_cast<const float*>(a.P);
    const float* __restrict__ Q = static_cast<const float*>(a.Q);
    const int64_t T = a.T, K = a.K, Pdim = a.Pdim;
    const int64_t q0 = (int64_t)blockIdx.y * 64, p0 = (int64_t)blockIdx.x * 64;
    const int tx = (int)threadIdx.x & 15, ty = (int)threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        for (int e = (int)threadIdx.x; e < 16 * 64; e += 256) {
            const int kk = e & 15, rr = e >> 4;
            const int64_t k = k0 + kk, q = q0 + rr, p = p0 + rr;
            qs[kk][rr] = (k < K && q < T) ? Q[q * K + k] : 0.0f;
            float pv = 0.0f;
            if (k < K && p < Pdim) pv = P_KMAJOR ? P[p * K + k] : P[k * Pdim + p];
            ps[kk][rr] = pv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float qv[4], pv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) { qv[u] = qs[kk][ty * 4 + u]; pv[u] = ps[kk][tx * 4 + u]; }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(qv[u], pv[v], acc[u][v]);
        }
        __syncthreads();
    }
    const float* __restrict__ E = static_cast<const float*>(a.E);
    float* __restrict__ O = static_cast<float*>(a.O);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t q = q0 + ty * 4 + u;
        if (q >= T) continue;
        int i = -1;
        if (a.lora && seg.n > 0) i = segment_of(seg, q);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t p = p0 + tx * 4 + v;
            if (p >= Pdim) continue;
            float out = acc[u][v];
            if (i >= 0) {
                const int r = seg.rank[i];
                const float* f = a.F + seg.hoff[i] + (q - seg.off[i]) * r;
                const float* e = E + (int64_t)seg.roff[i] * Pdim + p;
                float d = 0.0f;
                for (int j = 0; j < r; ++j) d = fmaf(f[j], e[(int64_t)j * Pdim], d);
                out = out + seg.scale[i] * d;
            }
            O[q * Pdim + p] = out;
        }
    }
}

// out[hoff_i + (t - o_i) r + j] = sum_k Q[t][k] P[R_off[i]+j][k]; one block per token.
__global__ __launch_bounds__(256) void shrink_f32(ShrinkArgs a, SegTable seg) {
    __shared__ float red[256];
    const int64_t t = blockIdx.x;
    const int i = segment_of(seg, t);
    const int r = seg.rank[i];
    const float* __restrict__ q = static_cast<const float*>(a.Q) + t * a.K;
    const float* __restrict__ P = static_cast<const float*>(a.P) + (int64_t)seg.roff[i] * a.K;
    float* out = a.out + seg.hoff[i] + (t - seg.off[i]) * r;
    for (int j = 0; j < r; ++j) {
        float s = 0.0f;
        for (int64_t k = threadIdx.x; k < a.K; k += 256) s = fmaf(q[k], P[(int64_t)j * a.K + k], s);
        red[threadIdx.x] = s;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) out[j] = red[0];
        __syncthreads();
    }
}

// out[g][c] = s_i * sum_{t in S_i} F_i[t-o_i][j] Q[t][c] for global rank row g = R_off[i] + j.
__global__ __launch_bounds__(256) void wgrad_f32(WgradArgs a, SegTable seg) {
    const int g = (int)blockIdx.y;
    int i = 0;
    while (i + 1 < seg.n && seg.roff[i + 1] <= g) ++i;
    const int j = g - seg.roff[i];
    const int r = seg.rank[i];
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= a.D) return;
    if (a.accumulate && seg.off[i + 1] == seg.off[i]) return;  // no tokens: leave the rows alone
    const float* __restrict__ Q = static_cast<const float*>(a.Q);
    const float* f = a.F + seg.hoff[i];
    float s = 0.0f;
    for (int64_t t = seg.off[i]; t < seg.off[i + 1]; ++t) s = fmaf(f[(t - seg.off[i]) * r + j], Q[t * a.D + c], s);
    const int64_t o = (int64_t)g * a.D + c;
    a.out[o] = a.accumulate ? a.out[o] + seg.scale[i] * s : seg.scale[i] * s;
}

}  // namespace

hipError_t launch_gemm_f32(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st) {
    const dim3 grid((unsigned)((a.Pdim + 63) / 64), (unsigned)((a.T + 63) / 64)), block(256);
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    if (p_kmajor)
        hipLaunchKernelGGL(gemm_lora_f32<true>, grid, block, 0, st, a, s);
    else
        hipLaunchKernelGGL(gemm_lora_f32<false>, grid, block, 0, st, a, s);
    return hipGetLastError();
}

hipError_t launch_shrink_f32(const ShrinkArgs& a, const SegTable& s, hipStream_t st) {
    if (s.T <= 0 || s.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(shrink_f32, dim3((unsigned)s.T), dim3(256), 0, st, a, s);
    return hipGetLastError();
}

hipError_t launch_wgrad_f32(const WgradArgs& a, const SegTable& s, hipStream_t st) {
    const int R = s.roff[s.n];
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(wgrad_f32, dim3((unsigned)((a.D + 255) / 256), (unsigned)R), dim3(256), 0, st, a, s);
    return hipGetLastError();
}

}  // namespace plora
