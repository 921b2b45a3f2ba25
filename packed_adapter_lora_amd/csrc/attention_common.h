// attention_common.h -- LDS layout and matrix-core operand helpers shared by
// the attention kernels (forward, dQ, dK/dV).
#pragma once

#include "block_launch.h"
#include "device_common.h"

namespace plora {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Tiles of 128-wide bf16 rows (256 bytes) in LDS, `stride` bytes apart; the
// 16-byte chunk c of row r sits at chunk c ^ (r % 16), so 16 consecutive rows
// read at one chunk hit distinct banks.
__device__ __forceinline__ int swz(int r, int c, int stride) { return r * stride + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int swz256(int r, int c) { return swz(r, c, 256); }

// MFMA operand of row r: dims 16*(c/2) + 8*(c%2) .. +7 (chunk c)
template <int STRIDE = 256>
__device__ __forceinline__ bf16x8 frag_row(const uint8_t* tile, int r, int c) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + swz(r, c, STRIDE)));
}

// Transposed read: lane l gets column d0 + l%32 of rows k0 + 4h .. +3 and
// k0 + 8 + 4h .. +3 (h = l/32), the row order of a score block's lane.
template <int STRIDE = 256>
__device__ __forceinline__ bf16x8 frag_tr(const uint8_t* tile, int d0, int k0) {
    const int l = lane_id(), L = l & 15, g = l >> 4;
    const int d = d0 + 16 * (g & 1) + 4 * (L & 3);
    const int k = k0 + 4 * (g >> 1) + (L >> 2);
    typedef __attribute__((address_space(3))) bf16x4v lds_v4;
    const bf16x4v lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(tile + swz(k, d >> 3, STRIDE) + (d & 7) * 2));
    const bf16x4v hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(tile + swz(k + 8, d >> 3, STRIDE) + (d & 7) * 2));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Values 8j .. 8j+7 of a 32x32 block as bf16: the B operand over the block's
// rows 16j .. 16j+15 in the lane's own row order.
__device__ __forceinline__ bf16x8 rows_as_b(const f32x16& a, int j) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = to_bf16(a[8 * j + e]);
    return r;
}

// Work item -> (sequence, tile within it); reverse = 1 walks the tiles from
// the last (the heaviest query tiles of a causal mask) to the first.
__device__ __forceinline__ void tile_of(const SeqTable& s, int item, int& seq, int& tile, bool reverse = true) {
    const int w = reverse ? s.tiles[s.n] - 1 - item : item;
    int lo = 0, hi = s.n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s.tiles[mid] <= w) lo = mid; else hi = mid;
    }
    seq = lo;
    tile = w - s.tiles[lo];
}

}  // namespace
}  // namespace plora
