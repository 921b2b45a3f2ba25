// probes.hip -- micro-benchmarks that measure the ceilings the operator's
// kernels are held against: sustained bf16 matrix-core throughput with random
// register operands, and HBM bandwidth of a plain copy and a plain read.
//
// mfma probes: every wave keeps 8 A and 8 B fragments of random bf16 values
// in registers (from the caller's operand buffer, a different slice per wave)
// and issues matrix-core instructions back to back over a 128 x 128 block of
// accumulators, the operands changing from instruction to instruction as in a
// GEMM's inner loop (the chip is power-capped, and its clock under load
// depends on how much the operands toggle).  No memory traffic inside the
// loop.  Each lane writes the sum of its accumulators at the end, so nothing
// is optimised away.
//
// Shape 2 of the mfma probe: the same loop with the fragments read from LDS
// at every step, as the GEMM's K loop does (8 fragment reads of 16 bytes per
// lane for 16 instructions), each wave from its own 16 KiB copy of its
// fragments.
//
// copy_probe / read_probe: 16-byte accesses, grid-stride over the buffer.
//
// lds_dma_probe: every wave streams a small (L2-resident) buffer into LDS with
// 16-byte buffer loads that write LDS directly (the path the operator's
// pipelined kernels stage their tiles through), up to kDmaInFlight loads in
// flight per wave; nothing reads the data back except one word at the end.
#include <string>

#include "api_util.h"
#include "device_common.h"
#include "plora.h"
#include "plora_probe.h"

namespace plora {
namespace {

constexpr int kProbeSlots = 1024;  // wave slices of the operand buffer (16 fragments x 64 lanes x 16 B each)

// shape 0: v_mfma_f32_32x32x16_bf16 on a 4 x 4 block of accumulators (a
// 128 x 128 wave tile) in serpentine order (consecutive instructions share one
// operand), as in the GEMM's K loop, two sets of fragments alternating; shape
// 1: v_mfma_f32_16x16x32_bf16 on 8 x 8 (the same tile), row by row (in
// serpentine order the compiler shuffles these accumulators between
// registers at every instruction).
__device__ __forceinline__ void probe_frags(const u32x4* ops, bf16x8 (&a)[8], bf16x8 (&b)[8]) {
    const int slot = (int)(((int64_t)blockIdx.x * 4 + wave_id()) % kProbeSlots);
    const u32x4* p = ops + (int64_t)slot * 16 * 64 + lane_id();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = as_bf16x8(p[k * 64]);
        b[k] = as_bf16x8(p[(8 + k) * 64]);
    }
}

__global__ __launch_bounds__(256) void mfma_probe32(const u32x4* __restrict__ ops, int32_t iters,
                                                    float* __restrict__ out) {
    bf16x8 a[8], b[8];
    probe_frags(ops, a, b);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j0 = 0; j0 < 4; ++j0) {
                    const int j = (i & 1) ? 3 - j0 : j0;
                    acc[i][j] = mfma32x32x16(a[4 * h + i], b[4 * h + j], acc[i][j]);
                }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) s += acc[i][j][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_probe16(const u32x4* __restrict__ ops, int32_t iters,
                                                    float* __restrict__ out) {
    bf16x8 a[8], b[8];
    probe_frags(ops, a, b);
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) s += acc[i][j][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_probe32_lds(const u32x4* __restrict__ ops, int32_t iters,
                                                        float* __restrict__ out) {
    __shared__ u32x4 sh[4 * 16 * 64];  // per wave: 16 fragments x 64 lanes
    const int w = wave_id(), l = lane_id();
    {
        const int slot = (int)(((int64_t)blockIdx.x * 4 + w) % kProbeSlots);
        const u32x4* p = ops + (int64_t)slot * 16 * 64 + l;
#pragma unroll
        for (int k = 0; k < 16; ++k) sh[(w * 16 + k) * 64 + l] = p[k * 64];
    }
    // (each wave reads back only what it wrote itself)
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // fragments 4h .. 4h+3 (A) and 8+4h .. 8+4h+3 (B), as in shape 0,
            // so both shapes compute the same sums; an opaque offset keeps
            // the reads inside the loop
            int o = (w * 16 + 4 * h) * 64 + l;
            asm volatile("" : "+v"(o));
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = as_bf16x8(sh[o + i * 64]);
                b[i] = as_bf16x8(sh[o + (8 + i) * 64]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j0 = 0; j0 < 4; ++j0) {
                    const int j = (i & 1) ? 3 - j0 : j0;
                    acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
                }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) s += acc[i][j][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kDmaSlots = 8;     // 1 KiB LDS slots per wave
constexpr int kDmaInFlight = 6;  // loads in flight per wave

__global__ __launch_bounds__(256) void lds_dma_probe(const void* __restrict__ src, int32_t span, int32_t iters,
                                                     uint32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * kDmaSlots * 1024];
    const int w = wave_id(), l = lane_id();
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), 0, span, kRsrcWord3);
    uint8_t* const mine = ring + wu * kDmaSlots * 1024;
    // wave wu reads 1 KiB pieces wu, wu + 4, ... of the span (span a multiple of 4 KiB)
    const int pieces = span / 4096;
    int n = 0;
    for (int it = 0; it < iters; ++it) {
        for (int q = 0; q < pieces; ++q, ++n) {
            if (n >= kDmaInFlight) wait_vmcnt<kDmaInFlight - 1>();
            const uint32_t vo = (uint32_t)(q * 4096 + wu * 1024 + l * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(mine + (n % kDmaSlots) * 1024), 16, vo, 0, 0, 0);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = reinterpret_cast<const uint32_t*>(ring)[threadIdx.x];
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

int plora_probe_mfma(const void* operands, int32_t shape, int32_t workgroups, int32_t iters, float* out, double* flops,
                     void* stream) {
    if (!operands || !out || !flops) return fail(PLORA_ERR_NULL, "operands, out and flops are required");
    if (workgroups <= 0 || iters <= 0) return fail(PLORA_ERR_SHAPE, "workgroups and iters must be positive");
    if (shape < 0 || shape > 2)
        return fail(PLORA_ERR_SHAPE, "shape must be 0 (32x32x16), 1 (16x16x32) or 2 (32x32x16 fed from LDS)");
    if (misaligned(operands) || misaligned(out)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
    // both shapes: 128 x 128 x 32 multiply-adds per wave and iteration
    *flops = (double)workgroups * 4.0 * (double)iters * (2.0 * 128 * 128 * 32);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (shape == 0)
        hipLaunchKernelGGL(mfma_probe32, dim3((unsigned)workgroups), dim3(256), 0, st,
                           static_cast<const u32x4*>(operands), iters, out);
    else if (shape == 1)
        hipLaunchKernelGGL(mfma_probe16, dim3((unsigned)workgroups), dim3(256), 0, st,
                           static_cast<const u32x4*>(operands), iters, out);
    else
        hipLaunchKernelGGL(mfma_probe32_lds, dim3((unsigned)workgroups), dim3(256), 0, st,
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

int plora_probe_lds_dma(const void* src, size_t span_bytes, int32_t workgroups, int32_t iters, uint32_t* out,
                        double* bytes, void* stream) {
    if (!src || !out || !bytes) return fail(PLORA_ERR_NULL, "src, out and bytes are required");
    if (span_bytes == 0 || span_bytes % 4096 != 0 || span_bytes > ((size_t)1 << 30) || workgroups <= 0 || iters <= 0)
        return fail(PLORA_ERR_SHAPE, "span must be a positive multiple of 4096 up to 1 GiB; workgroups, iters positive");
    if (misaligned(src) || misaligned(out)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
    *bytes = (double)workgroups * (double)iters * (double)span_bytes;
    hipLaunchKernelGGL(lds_dma_probe, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), src,
                       (int32_t)span_bytes, iters, out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLORA_OK : hip_fail(e, "lds dma probe launch");
}

}  // extern "C"
