// probes.hip -- micro-benchmarks that measure the ceilings the operator's
// kernels are held against: sustained bf16 matrix-core throughput with random
// register operands, and HBM bandwidth of a plain copy and a plain read.
//
// mfma_probe: every wave keeps 8 A and 8 B fragments of random bf16 values in
// registers (from the caller's operand buffer, a different slice per wave)
// and issues v_mfma_f32_32x32x16_bf16 back to back over four independent
// accumulators, each instruction on a different pair of fragments, so the
// multipliers see fresh data every instruction as in a GEMM's inner loop (the
// chip's clock under load depends on how much the operands toggle).  No
// memory traffic inside the loop.  Each lane writes the sum of its
// accumulators at the end, so nothing is optimised away.
//
// copy_probe / read_probe: 16-byte accesses, grid-stride over the buffer.
#include <string>

#include "api_util.h"
#include "device_common.h"
#include "plora.h"
#include "plora_probe.h"

namespace plora {
namespace {

constexpr int kProbeSlots = 1024;  // wave slices of the operand buffer (16 fragments x 64 lanes x 16 B each)

__global__ __launch_bounds__(256) void mfma_probe(const u32x4* __restrict__ ops, int32_t iters, float* __restrict__ out) {
    const int l = lane_id();
    const int slot = (int)(((int64_t)blockIdx.x * 4 + wave_id()) % kProbeSlots);
    const u32x4* p = ops + (int64_t)slot * 16 * 64 + l;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = as_bf16x8(p[k * 64]);
        b[k] = as_bf16x8(p[(8 + k) * 64]);
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            acc[k & 3] = mfma32x32x16(a[k], b[k], acc[k & 3]);
            acc[(k + 2) & 3] = mfma32x32x16(a[k], b[(k + 3) & 7], acc[(k + 2) & 3]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_probe(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) dst[e] = src[e];
}

__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ src, int64_t n, uint32_t* __restrict__ out) {
    u32x4 x = {0u, 0u, 0u, 0u};
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) x ^= src[e];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace

}  // namespace plora

using namespace plora;

extern "C" {

size_t plora_probe_mfma_operand_bytes(void) { return (size_t)kProbeSlots * 16 * 64 * 16; }

int plora_probe_mfma(const void* operands, int32_t workgroups, int32_t iters, float* out, double* flops,
                     void* stream) {
    if (!operands || !out || !flops) return fail(PLORA_ERR_NULL, "operands, out and flops are required");
    if (workgroups <= 0 || iters <= 0) return fail(PLORA_ERR_SHAPE, "workgroups and iters must be positive");
    if (misaligned(operands) || misaligned(out)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
    *flops = (double)workgroups * 4.0 * (double)iters * 16.0 * (2.0 * 32 * 32 * 16);
    hipLaunchKernelGGL(mfma_probe, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(operands), iters, out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLORA_OK : hip_fail(e, "mfma probe launch");
}

int plora_probe_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, void* stream) {
    if (!src || !dst) return fail(PLORA_ERR_NULL, "src and dst are required");
    if (bytes % 16 != 0 || workgroups <= 0) return fail(PLORA_ERR_SHAPE, "bytes must be a multiple of 16");
    if (misaligned(src) || misaligned(dst)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
    hipLaunchKernelGGL(copy_probe, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), (int64_t)(bytes / 16));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLORA_OK : hip_fail(e, "copy probe launch");
}

int plora_probe_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* out, void* stream) {
    if (!src || !out) return fail(PLORA_ERR_NULL, "src and out are required");
    if (bytes % 16 != 0 || workgroups <= 0) return fail(PLORA_ERR_SHAPE, "bytes must be a multiple of 16");
    if (misaligned(src) || misaligned(out)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
    hipLaunchKernelGGL(read_probe, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), (int64_t)(bytes / 16), out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLORA_OK : hip_fail(e, "read probe launch");
}

}  // extern "C"
