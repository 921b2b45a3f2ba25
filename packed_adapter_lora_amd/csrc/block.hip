// block.hip -- the element-wise and row-wise kernels of the Llama-3 decoder
// block around the packed LoRA projections: RMSNorm (with the residual add
// fused in front), its backward (with the gradient sum of the projections
// that read its output and the residual gradient fused in), the rotary
// embedding, SwiGLU and a residual add.
//
// LoRA sits on the projections of every Transformer block [LLM+LoRA微调加速技
// 术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与PEFT实现] of the LLaMA-3
// models the pages fine-tune [PLoRA technical summary (gist.science, arXiv
// 2508.02932), 结果]; the layers follow the public Llama 3 definitions.
//
// Activations are bf16 in HBM; every kernel computes in fp32 and rounds its
// outputs to bf16 once.  All of them are bound by HBM: one pass over their
// inputs and outputs, 16-byte accesses.
#include "block_launch.h"
#include "device_common.h"

namespace plora {
namespace {

__device__ __forceinline__ void load8(const bf16* p, float (&f)[8]) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(v[k] << 16);
        f[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
    }
}

// (non-temporal: these row-streaming kernels do not read their outputs again;
// kept out of L2, they leave it to the kernels' inputs; −0.25 % per block step)
__device__ __forceinline__ void store8(bf16* p, const float (&f)[8]) {
    bf16x8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = to_bf16(f[k]);
    __builtin_nontemporal_store(as_u32x4(o), reinterpret_cast<u32x4*>(p));
}

// Sum over the 256 threads of a workgroup (4 waves of 64).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = (int)threadIdx.x >> 6;
    __syncthreads();  // red may still be read from a previous call
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// One workgroup per row.  xs = x (+ res, rounded to bf16, written to xs_out);
// rstd = 1 / sqrt(mean(xs^2) + eps); h = xs * rstd * w.  NC chunks of 2048
// elements per row (the row stays in registers; fewer chunks, more rows in
// flight).
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(RmsFwdArgs a) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int64_t D = a.D;
    const bf16* x = static_cast<const bf16*>(a.x) + row * D;
    const bf16* r = a.res ? static_cast<const bf16*>(a.res) + row * D : nullptr;
    float ss = 0.0f;
    float v[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
        if (e < D) {
            load8(x + e, v[c]);
            if (r) {
                float rv[8];
                load8(r + e, rv);
#pragma unroll
                for (int k = 0; k < 8; ++k) v[c][k] = static_cast<float>(to_bf16(v[c][k] + rv[k]));
                store8(static_cast<bf16*>(a.xs_out) + row * D + e, v[c]);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) ss += v[c][k] * v[c][k];
        }
    }
    const float rstd = 1.0f / sqrtf(block_sum(ss, red) / (float)D + a.eps);
    if (threadIdx.x == 0) a.rstd[row] = rstd;
    const bf16* w = static_cast<const bf16*>(a.w);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
        if (e < D) {
            float wv[8], o[8];
            load8(w + e, wv);
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = v[c][k] * rstd * wv[k];
            store8(static_cast<bf16*>(a.h) + row * D + e, o);
        }
    }
}

// One workgroup per row.  g = (dy0 + dy1 + dy2) * w;
// dx = dres + rstd * g - x * rstd^3 * mean(g * x).  NC chunks as above.
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(RmsBwdArgs a) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int64_t D = a.D;
    const float rstd = a.rstd[row];
    float g[NC][8], xv[NC][8];
    float sgx = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
        if (e < D) {
            float wv[8], t[8];
            load8(static_cast<const bf16*>(a.dy[0]) + row * D + e, g[c]);
#pragma unroll
            for (int m = 1; m < 3; ++m) {
                if (a.dy[m]) {
                    load8(static_cast<const bf16*>(a.dy[m]) + row * D + e, t);
#pragma unroll
                    for (int k = 0; k < 8; ++k) g[c][k] += t[k];
                }
            }
            load8(static_cast<const bf16*>(a.w) + e, wv);
            load8(static_cast<const bf16*>(a.x) + row * D + e, xv[c]);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                g[c][k] *= wv[k];
                sgx += g[c][k] * xv[c][k];
            }
        }
    }
    const float m = block_sum(sgx, red) / (float)D;
    const float r3m = rstd * rstd * rstd * m;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
        if (e < D) {
            float o[8], rv[8];
            if (a.dres)
                load8(static_cast<const bf16*>(a.dres) + row * D + e, rv);
            else
#pragma unroll
                for (int k = 0; k < 8; ++k) rv[k] = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = rv[k] + (rstd * g[c][k] - xv[c][k] * r3m);
            store8(static_cast<bf16*>(a.dx) + row * D + e, o);
        }
    }
}

// Token t of sequence s has position t - off[s].
__device__ __forceinline__ int64_t position_of(const SeqTable& s, int64_t t) {
    int lo = 0, hi = s.n;  // off[lo] <= t < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s.off[mid] <= t) lo = mid; else hi = mid;
    }
    return t - s.off[lo];
}

// Rotary embedding in place: thread handles 8 pairs (i, i + 64) of one token
// in every head (8 threads per token), so each angle's sine and cosine are
// taken once per token; inverse = 1 applies the transpose (backward).
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over T * 8
    if (idx >= a.T * 8) return;
    const int64_t t = idx >> 3;
    const int i0 = (int)(idx & 7) * 8;
    const float pos = (float)position_of(a.seq, t);
    float cs[8], sn[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        sincosf(pos * a.inv_freq[i0 + k], &sn[k], &cs[k]);
        if (a.inverse) sn[k] = -sn[k];
    }
    bf16* row = static_cast<bf16*>(a.x) + t * a.heads * 128 + i0;
#pragma unroll 4
    for (int hd = 0; hd < a.heads; ++hd) {
        bf16* base = row + hd * 128;
        float lo[8], hi[8], olo[8], ohi[8];
        load8(base, lo);
        load8(base + 64, hi);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            olo[k] = lo[k] * cs[k] - hi[k] * sn[k];
            ohi[k] = hi[k] * cs[k] + lo[k] * sn[k];
        }
        store8(base, olo);
        store8(base + 64, ohi);
    }
}

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + __expf(-x)); }

__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const bf16* g, const bf16* u, bf16* out, int64_t n) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e >= n) return;
    float gv[8], uv[8], o[8];
    load8(g + e, gv);
    load8(u + e, uv);
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = gv[k] * sigmoidf(gv[k]) * uv[k];
    store8(out + e, o);
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16* da, const bf16* g, const bf16* u, bf16* dg,
                                                         bf16* du, int64_t n) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e >= n) return;
    float av[8], gv[8], uv[8], og[8], ou[8];
    load8(da + e, av);
    load8(g + e, gv);
    load8(u + e, uv);
#pragma unroll
    for (int k = 0; k < 8; ++k) swiglu_grad(av[k], gv[k], uv[k], og[k], ou[k]);
    store8(dg + e, og);
    store8(du + e, ou);
}

__global__ __launch_bounds__(256) void add_kernel(const bf16* x, const bf16* y, bf16* out, int64_t n) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e >= n) return;
    float a[8], b[8];
    load8(x + e, a);
    load8(y + e, b);
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] += b[k];
    store8(out + e, a);
}

unsigned blocks_for(int64_t n8) { return (unsigned)((n8 + 255) / 256); }

// chunks of 2048 elements a row needs, rounded up to 1, 2, 4 or 8
int rms_chunks(int64_t D) {
    const int64_t c = (D + 2047) / 2048;
    return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 8;
}

}  // namespace

hipError_t launch_rmsnorm_fwd(const RmsFwdArgs& a, int64_t T, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const dim3 grid((unsigned)T), block(256);
    switch (rms_chunks(a.D)) {
        case 1: hipLaunchKernelGGL(rmsnorm_fwd_kernel<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(rmsnorm_fwd_kernel<2>, grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL(rmsnorm_fwd_kernel<4>, grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL(rmsnorm_fwd_kernel<kRmsMaxChunks>, grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const RmsBwdArgs& a, int64_t T, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const dim3 grid((unsigned)T), block(256);
    switch (rms_chunks(a.D)) {
        case 1: hipLaunchKernelGGL(rmsnorm_bwd_kernel<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(rmsnorm_bwd_kernel<2>, grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL(rmsnorm_bwd_kernel<4>, grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL(rmsnorm_bwd_kernel<kRmsMaxChunks>, grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t st) {
    const int64_t n = a.T * 8;
    if (n <= 0 || a.heads <= 0) return hipSuccess;
    hipLaunchKernelGGL(rope_kernel, dim3(blocks_for(n)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const void* g, const void* u, void* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(blocks_for(n / 8)), dim3(256), 0, st, static_cast<const bf16*>(g),
                       static_cast<const bf16*>(u), static_cast<bf16*>(out), n);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* da, const void* g, const void* u, void* dg, void* du, int64_t n,
                             hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(blocks_for(n / 8)), dim3(256), 0, st, static_cast<const bf16*>(da),
                       static_cast<const bf16*>(g), static_cast<const bf16*>(u), static_cast<bf16*>(dg),
                       static_cast<bf16*>(du), n);
    return hipGetLastError();
}

hipError_t launch_add(const void* x, const void* y, void* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(add_kernel, dim3(blocks_for(n / 8)), dim3(256), 0, st, static_cast<const bf16*>(x),
                       static_cast<const bf16*>(y), static_cast<bf16*>(out), n);
    return hipGetLastError();
}

}  // namespace plora
