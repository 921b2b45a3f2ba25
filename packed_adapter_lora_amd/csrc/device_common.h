// device_common.h -- gfx950 device helpers shared by the packed-LoRA kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace plora {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// D[32x32] += A[32x16] * B[16x32] on the matrix cores (bf16 in, fp32 out).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each as the 8
// consecutive k of slot (l / 32).  Lane l receives column (l % 32) of D,
// rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Round fp32 to bf16 (nearest, ties to even; gfx950 converts in hardware).
__device__ __forceinline__ bf16 to_bf16(float f) { return static_cast<bf16>(f); }

// Two-term bf16 split of an fp32 value: v ~= hi + lo with |v - hi - lo| <= 2^-16 |v|.
__device__ __forceinline__ void split_bf16(float v, bf16& hi, bf16& lo) {
    hi = static_cast<bf16>(v);
    lo = static_cast<bf16>(v - static_cast<float>(hi));
}

// 16-byte global load that yields zero when pred is false.
__device__ __forceinline__ u32x4 load16_or_zero(const void* p, bool pred) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (pred) z = *reinterpret_cast<const u32x4*>(p);
    return z;
}

// Adapter owning token t: the i with off[i] <= t < off[i+1] (N <= 64, linear).
__device__ __forceinline__ int segment_of(const SegTable& s, int64_t t) {
    int i = 0;
    while (i + 1 < s.n && s.off[i + 1] <= t) ++i;
    return i;
}

// Work map lookup: the i with pre[i] <= w < pre[i+1].
__device__ __forceinline__ int adapter_of_unit(const WorkMap& m, int n, int32_t w) {
    int i = 0;
    while (i + 1 < n && m.pre[i + 1] <= w) ++i;
    return i;
}

}  // namespace plora
