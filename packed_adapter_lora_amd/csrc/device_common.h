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

// SwiGLU a = silu(g) * u: the gradients of g and u for one element given da,
// s = sigmoid(g).  One definition for every kernel that applies it (the
// SwiGLU backward kernel and the dX GEMM's fused epilogue), so both give the
// same bits.
__device__ __forceinline__ void swiglu_grad(float da, float g, float u, float& dg, float& du) {
    const float s = 1.0f / (1.0f + __expf(-g));
    dg = da * u * s * (1.0f + g * (1.0f - s));
    du = da * g * s;
}

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

// Adapter owning token t: the last i with off[i] <= t, i.e. off[i] <= t <
// off[i+1] with empty segments skipped (binary search: with uniform t the
// table reads are a short chain of scalar loads).
__device__ __forceinline__ int segment_of(const SegTable& s, int64_t t) {
    int lo = 0, hi = s.n;  // off[lo] <= t, and off[hi] > t or hi == n
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s.off[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Work map lookup: the i with pre[i] <= w < pre[i+1].
__device__ __forceinline__ int adapter_of_unit(const WorkMap& m, int n, int32_t w) {
    int i = 0;
    while (i + 1 < n && m.pre[i + 1] <= w) ++i;
    return i;
}

// ---- LDS DMA pipelines (shared by the GEMM, shrink and weight-gradient kernels)

typedef __attribute__((address_space(3))) void lds_void;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

// Byte offset of 16-byte chunk c of row r in a tile of 128-byte rows.  The XOR
// keeps any 16 (or 8) consecutive rows read at one chunk on distinct banks.
__device__ __forceinline__ int kofs128(int r, int c) { return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Byte offset of 16-byte chunk c of row k in a tile of 512-byte rows read
// transposed: chunk c of row k is stored at c ^ 4*(k%4), so the 16 lanes of a
// transposed read (4 rows x 32 bytes) and the next 16 hit distinct banks.
__device__ __forceinline__ int tofs(int k, int c) { return k * 512 + ((c ^ ((k & 3) << 2)) << 4); }

typedef __bf16 bf16x4v __attribute__((vector_size(8)));

// 8 consecutive rows k of column p from a tile of ROWB-byte rows (512 or 256;
// 16-byte chunk c of row k stored at chunk c ^ 4 (k % 4), the tofs layout), as
// one MFMA operand, with two transposed LDS reads (ds_read_b64_tr_b16).
// Within each 16-lane group, lane L supplies the address of row kb + L/4,
// columns pc + 4*(L%4) .. +3, and lane i gets back rows kb..kb+3 of column
// pc + i.  Lane l receives column p0 + l%32, rows kb + 8*(l/32) .. +7.
template <int ROWB = 512>
__device__ __forceinline__ bf16x8 pfrag_tr(const uint8_t* tile, int p0, int kb) {
    const int l = lane_id(), L = l & 15, g = l >> 4;
    const int p = p0 + 16 * (g & 1) + 4 * (L & 3);
    const int k = kb + 8 * (g >> 1) + (L >> 2);
    const uint8_t* a0 = tile + k * ROWB + ((((p >> 3) ^ ((k & 3) << 2))) << 4) + (p & 7) * 2;
    const uint8_t* a1 = tile + (k + 4) * ROWB + ((((p >> 3) ^ (((k + 4) & 3) << 2))) << 4) + (p & 7) * 2;
    typedef __attribute__((address_space(3))) bf16x4v lds_v4;
    const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a0));
    const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a1));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// (vmcnt is 6 bits: at most 63; a wave stalls issuing beyond that, so
// waiting for "all but the newest N" stays exact for N <= 63)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// workgroup barrier for LDS only: wait for this wave's LDS reads, then s_barrier
// (no vmcnt drain, so in-flight prefetches stay in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace plora
