// optim.hip -- per-adapter AdamW over the packed LoRA panels.
//
// Adapter i owns rows R_off[i] .. R_off[i]+r_i-1 of the packed A [R][d_in]
// and B [R][d_out] panels.  Each element is updated with AdamW (decoupled
// weight decay; Loshchilov & Hutter, ICLR 2019), the optimizer of the PEFT
// fine-tuning loop [LLM+LoRA微调加速技术原理解析 (m.youleyou.com),
// 5. 设定优化器和正则项], with the learning rate, weight decay and step count
// of its own adapter, since packed jobs differ in learning rate [PLoRA
// technical summary (gist.science, arXiv 2508.02932), 结果].
//
// The update is elementwise and bound by HBM: per element it reads the fp32
// master value, both moments and the gradient and writes back the master
// value, the moments and the operator's bf16 (or fp32) copy: 30 bytes for a
// bf16 copy.  One workgroup covers 1024 consecutive elements of one row, so
// the adapter (and its factors) is uniform per workgroup, and every access is
// a 16-byte vector.
#include "device_common.h"
#include "launch.h"

namespace plora {
namespace {

__global__ __launch_bounds__(256) void adamw_panel(AdamwArgs a, AdamwTable t) {
    const int row = (int)blockIdx.y;
    int i = 0;
    while (i + 1 < t.n && t.roff[i + 1] <= row) ++i;
    if (!t.active[i]) return;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= a.D) return;  // D is a multiple of 8: a row holds whole groups of 4
    const int64_t o = (int64_t)row * a.D + e;
    const float decay = t.decay[i], step_size = t.step_size[i], rs_bc2 = t.rs_bc2[i];
    f32x4 p = *reinterpret_cast<const f32x4*>(a.P + o);
    f32x4 m = *reinterpret_cast<const f32x4*>(a.m + o);
    f32x4 v = *reinterpret_cast<const f32x4*>(a.v + o);
    const f32x4 g = *reinterpret_cast<const f32x4*>(a.g + o);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float pk = p[k] * decay;
        const float mk = t.beta1 * m[k] + t.one_minus_beta1 * g[k];
        const float vk = t.beta2 * v[k] + t.one_minus_beta2 * (g[k] * g[k]);
        pk = pk - step_size * (mk / (sqrtf(vk) * rs_bc2 + t.eps));
        p[k] = pk;
        m[k] = mk;
        v[k] = vk;
    }
    *reinterpret_cast<f32x4*>(a.P + o) = p;
    *reinterpret_cast<f32x4*>(a.m + o) = m;
    *reinterpret_cast<f32x4*>(a.v + o) = v;
    if (a.out) {
        if (a.out_bf16) {
            bf16x4 b;
            b[0] = to_bf16(p[0]);
            b[1] = to_bf16(p[1]);
            b[2] = to_bf16(p[2]);
            b[3] = to_bf16(p[3]);
            *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.out) + o) = b;
        } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = p;
        }
    }
}

// out = dtype copy of the fp32 panel P (bf16: round to nearest even), 16-byte
// accesses; one workgroup per 1024 elements.
__global__ __launch_bounds__(256) void cast_panel(const float* __restrict__ P, void* __restrict__ out, int32_t out_bf16,
                                                  int64_t n) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= n) return;  // n is a multiple of 8
    const f32x4 p = *reinterpret_cast<const f32x4*>(P + e);
    if (out_bf16) {
        bf16x4 b;
        b[0] = to_bf16(p[0]);
        b[1] = to_bf16(p[1]);
        b[2] = to_bf16(p[2]);
        b[3] = to_bf16(p[3]);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(out) + e) = b;
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + e) = p;
    }
}

}  // namespace

hipError_t launch_cast_panel(const float* P, void* out, int32_t out_bf16, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t wg = (n + 1023) / 1024;
    if (wg > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cast_panel, dim3((unsigned)wg), dim3(256), 0, st, P, out, out_bf16, n);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamwArgs& a, const AdamwTable& t, hipStream_t st) {
    const int R = t.roff[t.n];
    if (R <= 0 || a.D <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.D + 1023) / 1024), (unsigned)R), block(256);
    hipLaunchKernelGGL(adamw_panel, grid, block, 0, st, a, t);
    return hipGetLastError();
}

}  // namespace plora
