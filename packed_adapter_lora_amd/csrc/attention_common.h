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
// 16-byte chunk c of row r sits at chunk c ^ rowkey(r), rowkey(r) = 4 (r % 4)
// + (r / 4) % 4.  The LDS serves 256 bytes per cycle from 64 banks, so reads
// are conflict-free when the 16-byte chunks served together are distinct
// modulo 256 bytes: 16 consecutive rows at one chunk (row reads: rowkey is a
// bijection on 16 rows), and 4 rows from a multiple of 4 at 4 chunks from a
// multiple of 4 (transposed reads: rowkey's high bits follow r % 4).
__device__ __forceinline__ int rowkey(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz(int r, int c, int stride) { return r * stride + ((c ^ rowkey(r)) << 4); }
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

// Stores a wave's 32 x 128 block of o (lane: row l%32, columns db*32 +
// 8*(v/4) + 4*(l/32) + v%4 in o[db][v]) times mul as bf16 rows: the lane's
// values go through the wave's own 8 KiB of LDS (swizzled 256-byte rows),
// then each store writes 16 bytes per lane, 16 lanes per 256-byte row.  Row r
// goes to base + r * row_stride (elements) when r < nrows.
__device__ __forceinline__ void store_rows_via_lds(const f32x16 (&o)[4], float mul, uint8_t* tile, bf16* base,
                                                   int64_t row_stride, int nrows) {
    const int l = lane_id(), l32 = l & 31, lh = l >> 5;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = to_bf16(o[db][4 * g4 + e] * mul);
            *reinterpret_cast<bf16x4*>(tile + swz256(l32, 4 * db + g4) + 8 * lh) = v4;
        }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (l >> 4), c = l & 15;
        const u32x4 x = *reinterpret_cast<const u32x4*>(tile + swz256(r, c));
        if (r < nrows) *reinterpret_cast<u32x4*>(base + r * row_stride + 8 * c) = x;
    }
}

// Work item -> (sequence, tile within it, head group).  Level order (s.lmax >
// 0): item (r * n + seq) * ngroups + group is the tile of rank r of its
// sequence, rank 0 the heaviest (the last tile when last_first, else the
// first), so equally heavy tiles of all sequences and groups run together and
// the lightest run last; a sequence with fewer tiles leaves the items of its
// missing ranks empty (false).  Otherwise blockIdx.x walks the tiles sequence
// by sequence (each heaviest first) and blockIdx.y is the group.
__device__ __forceinline__ bool work_item(const SeqTable& s, int ngroups, bool last_first, int& seq, int& tile,
                                          int& group) {
    const int item = (int)blockIdx.x;
    if (s.lmax > 0) {
        const int per = s.n * ngroups;
        const int r = item / per, rem = item - r * per;
        seq = rem / ngroups;
        group = rem - seq * ngroups;
        const int nt = s.tiles[seq + 1] - s.tiles[seq];
        tile = last_first ? nt - 1 - r : r;
        return r < nt;
    }
    group = (int)blockIdx.y;
    const int w = last_first ? s.tiles[s.n] - 1 - item : item;
    int lo = 0, hi = s.n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s.tiles[mid] <= w) lo = mid; else hi = mid;
    }
    seq = lo;
    tile = w - s.tiles[lo];
    return true;
}

// Work item -> (sequence, tile, head group) in sequence order with the head
// groups fastest: item t * ngroups + group is tile t of the sequence-major
// tile list (first tile first).  Consecutive work items go to different XCDs,
// so with 8 groups each XCD takes one group (one key/value head) and runs
// the tiles of one or two sequences at a time: their shared query rows stay
// in its L2.
__device__ __forceinline__ void work_item_grouped(const SeqTable& s, int ngroups, int& seq, int& tile, int& group) {
    const int t = (int)blockIdx.x / ngroups;
    group = (int)blockIdx.x - t * ngroups;
    int lo = 0, hi = s.n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s.tiles[mid] <= t) lo = mid; else hi = mid;
    }
    seq = lo;
    tile = t - s.tiles[lo];
}

// Fills s.tiles with ceil(len / per) items per sequence for work_item_grouped;
// returns the grid.
inline dim3 attention_grid_grouped(SeqTable& s, int per, int ngroups) {
    s.tiles[0] = 0;
    for (int i = 0; i < s.n; ++i) s.tiles[i + 1] = s.tiles[i] + (s.off[i + 1] - s.off[i] + per - 1) / per;
    s.lmax = 0;
    return dim3((unsigned)((int64_t)s.tiles[s.n] * ngroups), 1);
}

// Fills s.tiles with ceil(len / per) items per sequence and picks the order:
// level order unless it would launch more than twice as many (partly empty)
// items.  Returns the grid.
inline dim3 attention_grid(SeqTable& s, int per, int ngroups) {
    s.tiles[0] = 0;
    int lmax = 0;
    for (int i = 0; i < s.n; ++i) {
        const int nt = (s.off[i + 1] - s.off[i] + per - 1) / per;
        s.tiles[i + 1] = s.tiles[i] + nt;
        lmax = nt > lmax ? nt : lmax;
    }
    const int64_t level_items = (int64_t)lmax * s.n;
    if (level_items <= 2 * (int64_t)s.tiles[s.n] && level_items * ngroups < (1LL << 31)) {
        s.lmax = lmax;
        return dim3((unsigned)(level_items * ngroups), 1);
    }
    s.lmax = 0;
    return dim3((unsigned)s.tiles[s.n], (unsigned)ngroups);
}

}  // namespace
}  // namespace plora
