// gemm_bf16.hip -- frozen-base GEMM with the packed LoRA expand fused into
// its accumulators (gfx950, bf16 in, fp32 accumulate, one bf16 rounding).
//
//   forward        Y[t]  = X[t] W_m       + s_i H_i[t] B_i      (t in S_i)
//   backward-data  dX[t] = dY[t] W_m^T    + s_i G_i[t] A_i^T
//
// The base product carries almost all of the operator's arithmetic, so it
// runs on the matrix cores (v_mfma_f32_32x32x16_bf16).  The LoRA expand is
// the same contraction with K = r_i, so it is appended to the K loop of every
// output tile: after the frozen weight's K loop, each adapter whose segment
// overlaps the tile's tokens adds K = r_i more MFMA steps into the same fp32
// accumulators, with s_i folded into H/G and the fp32 H/G values split into
// two bf16 terms (hi + lo, ~16 significant bits) so the branch is not
// truncated to bf16.  The result is rounded to bf16 once.  This is the expand
// of the packed operators, tiled along tokens and hidden features rather than
// rank [PLoRA technical summary (gist.science, arXiv 2508.02932),
// 方法论 > 2. LoRA 执行引擎 > 算子设计], applied to the LoRA definition
// Y = XW + (alpha/r) X A B [LLM+LoRA微调加速技术原理解析, 深入理解LoRA].
//
// Tiling: 256 (features p) x 256 (tokens q) x 64 (k) per workgroup of 4
// waves; each wave owns a 128 x 128 quarter as 4 x 4 MFMA tiles of 32 x 32.
// MFMA A = weight side (rows p), MFMA B = token side (columns q), so a lane
// ends up holding 4 consecutive features of one token: 8-byte stores.
// LDS: two stages (global loads of stage k+1 are in flight while stage k is
// multiplied).  K-contiguous tiles use 128-byte rows with an XOR swizzle of
// the 16-byte chunks; p-contiguous tiles (backward weight, expand operand)
// keep the global row order with a 16-byte pad per row and are read
// transposed, 2 bytes per lane.
#include "device_common.h"
#include "launch.h"

namespace plora {
namespace {

constexpr int kBP = 256;   // features per tile
constexpr int kBQ = 256;   // tokens per tile
constexpr int kBK = 64;    // k per stage
constexpr int kThreads = 256;
constexpr int kKRow = kBK * 2;                 // bytes per K-contiguous row
constexpr int kKTile = 256 * kKRow;            // 32 KiB
constexpr int kPRow = kBP * 2 + 16;            // bytes per p-contiguous row (padded)
constexpr int kPTile = kBK * kPRow;            // 33792 B
constexpr int kStage = kPTile + kKTile;        // P tile (either layout) + Q tile
constexpr int kLds = 2 * kStage;               // 132 KiB
constexpr int kGroupQ = 2;                     // token tiles per L2 group

// Byte offset of 16-byte chunk c of row r in a K-contiguous tile.  The XOR
// keeps the 16 rows read by any 16 lanes (and any 8) on distinct bank groups.
__device__ __forceinline__ int kmaj(int r, int c) { return r * kKRow + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Workgroup -> output tile.  Workgroups are dealt round-robin to the 8 XCDs;
// renumber so each XCD gets a contiguous range of tiles, and walk that range
// in groups of kGroupQ token tiles: the ~32 workgroups an XCD runs at once then
// cover 2 token tiles x 16 feature tiles, so the two X/dY panels (2 x 2 MiB at
// K = 4096) stay in that XCD's 4 MB L2 and the weight panels, re-read more
// often, come from the 256 MB Infinity Cache (measured best of 1, 2, 4, 8).
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_q, int tiles_p, int& tq, int& tp) {
    const int base = nwg / 8, extra = nwg % 8;
    const int xcd = bid % 8, slot = bid / 8;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int per_group = kGroupQ * tiles_p;
    const int group = logical / per_group;
    const int first = group * kGroupQ;
    const int gsize = min(tiles_q - first, kGroupQ);
    const int in = logical - group * per_group;
    tq = first + in % gsize;
    tp = in / gsize;
}


// Fragment of a p-contiguous tile: 8 consecutive k of feature p, read
// transposed from rows k..k+7 (2 bytes per lane per row).
__device__ __forceinline__ bf16x8 pfrag_rows(const uint8_t* base, int row_bytes, int p, int k) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const uint16_t*>(base + (k + e) * row_bytes + p * 2);
    return __builtin_bit_cast(bf16x8, v);
}

// LoRA expand appended to the K loop of one 256 x 256 tile: for every adapter
// whose segment overlaps the tile's tokens, K = r_i more MFMA steps with
// A = E rows (B_i or A_i^T, p-contiguous) and B = s_i * F_i split into bf16
// hi + lo, zero outside the segment.  se: >= 64 rows of se_row bytes;
// shi/slo: 32 KiB K-contiguous tiles.  Must be called by the whole workgroup
// once the LDS used by the K loop is free.
__device__ __forceinline__ void lora_expand(f32x16 (&acc)[4][4], const GemmArgs& a, const SegTable& seg,
                                            int64_t q0, int64_t p0, uint8_t* se, int se_row, uint8_t* shi,
                                            uint8_t* slo) {
    const bf16* __restrict__ E = static_cast<const bf16*>(a.E);
    const float* __restrict__ F = a.F;
    const int64_t T = a.T, Pdim = a.Pdim;
    const int tid = (int)threadIdx.x, l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;
    const int64_t tq1 = q0 + kBQ < T ? q0 + kBQ : T;
    for (int i = segment_of(seg, q0); i < seg.n && seg.off[i] < tq1; ++i) {
        const int64_t s0 = seg.off[i], s1 = seg.off[i + 1];
        if (s1 <= s0 || s1 <= q0) continue;
        const int r = seg.rank[i];
        const float sc = seg.scale[i];
        const int64_t rbase = seg.roff[i];
        const float* Fi = F + seg.hoff[i];
        for (int jb = 0; jb < r; jb += 64) {
            const int rc = r - jb < 64 ? r - jb : 64;
            const int nkk = (rc + 15) >> 4;
            // issue every global load of this chunk before touching LDS: one
            // round trip.  E: 16*nkk rows x 32 chunks of 16 B (8 per thread at
            // most); F: thread tid owns token row q0 + tid (rc fp32 values).
            u32x4 ev[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int id = tid + u * kThreads;
                const int j = id >> 5, pc = id & 31;
                const int64_t p = p0 + pc * 8;
                ev[u] = load16_or_zero(E + (rbase + jb + j) * Pdim + p, j < rc && p < Pdim);
            }
            const int64_t t = q0 + tid;
            const bool in = t >= s0 && t < s1;
            const float* frow = Fi + (in ? (t - s0) * r + jb : 0);
            float fv[64];
            if (((seg.hoff[i] + jb) & 3) == 0 && (r & 3) == 0) {
                // rows start on 16-byte boundaries: 4 values per load (rc is a multiple of 4)
#pragma unroll
                for (int j4 = 0; j4 < 16; ++j4) {
                    f32x4 v = {0.f, 0.f, 0.f, 0.f};
                    if (in && 4 * j4 < rc) v = *reinterpret_cast<const f32x4*>(frow + 4 * j4);
                    fv[4 * j4 + 0] = v[0];
                    fv[4 * j4 + 1] = v[1];
                    fv[4 * j4 + 2] = v[2];
                    fv[4 * j4 + 3] = v[3];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 64; ++j) fv[j] = (in && j < rc) ? frow[j] : 0.0f;
            }
            __syncthreads();  // the K loop / previous chunk is done with LDS
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int id = tid + u * kThreads;
                const int j = id >> 5, pc = id & 31;
                if (j < 16 * nkk) *reinterpret_cast<u32x4*>(se + j * se_row + pc * 16) = ev[u];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (c >= 2 * nkk) break;
                u16x8 hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16 h, o;
                    split_bf16(sc * fv[c * 8 + e], h, o);
                    hi[e] = __builtin_bit_cast(uint16_t, h);
                    lo[e] = __builtin_bit_cast(uint16_t, o);
                }
                *reinterpret_cast<u16x8*>(shi + kmaj(tid, c)) = hi;
                *reinterpret_cast<u16x8*>(slo + kmaj(tid, c)) = lo;
            }
            __syncthreads();
            // only this wave's 32-token blocks that hold tokens of the segment
            // have nonzero F rows: the others skip their MFMAs (many adapters
            // with few tokens each share a tile at serving shapes)
            bool live[4];
            bool any = false;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int64_t b0 = q0 + wq * 128 + nt * 32;
                live[nt] = b0 < s1 && b0 + 32 > s0;
                any |= live[nt];
            }
            for (int kk = 0; any && kk < nkk; ++kk) {
                bf16x8 fa[4], fh[4], fl[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    fa[mt] = pfrag_rows(se, se_row, wp * 128 + mt * 32 + l32, 16 * kk + 8 * lh);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (!live[nt]) continue;
                    const int row = wq * 128 + nt * 32 + l32;
                    fh[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(shi + kmaj(row, 2 * kk + lh)));
                    fl[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(slo + kmaj(row, 2 * kk + lh)));
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (!live[nt]) continue;
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        acc[mt][nt] = mfma32x32x16(fa[mt], fh[nt], acc[mt][nt]);
                        acc[mt][nt] = mfma32x32x16(fa[mt], fl[nt], acc[mt][nt]);
                    }
                }
            }
        }
    }
}

// One rounding to bf16, token-major stores: lane holds features
// p .. p+3 (p = 8*(v/4) + 4*(l/32)) of token q = l%32 in each 32 x 32 block.
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], const GemmArgs& a, int64_t q0, int64_t p0) {
    bf16* __restrict__ O = static_cast<bf16*>(a.O);
    const int64_t T = a.T, Pdim = a.Pdim;
    const int l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int64_t t = q0 + wq * 128 + nt * 32 + l32;
        if (t >= T) continue;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t p = p0 + wp * 128 + mt * 32 + 8 * g + 4 * lh;
                if (p < Pdim) {
                    bf16x4 o;
                    o[0] = to_bf16(acc[mt][nt][4 * g + 0]);
                    o[1] = to_bf16(acc[mt][nt][4 * g + 1]);
                    o[2] = to_bf16(acc[mt][nt][4 * g + 2]);
                    o[3] = to_bf16(acc[mt][nt][4 * g + 3]);
                    *reinterpret_cast<bf16x4*>(O + t * Pdim + p) = o;
                }
            }
        }
    }
}

// The same rounding and output, staged through LDS so that global stores are
// whole 16-byte chunks of contiguous 256-byte row pieces (one instruction = 4
// token rows x 256 bytes) instead of 8-byte pieces of 32 rows.  Each wave
// writes its own 128 x 128 quarter into its own 32 KiB buffer `sb` (token rows
// of 256 bytes); 8-byte slot s of row q is stored at slot s ^ (q % 32), which
// keeps both the 8-byte writes (32 rows, one slot) and the 16-byte reads (one
// row, 16 chunks) free of bank conflicts.  No workgroup barrier: a wave only
// reads what it wrote.
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[4][4], const GemmArgs& a, int64_t q0, int64_t p0,
                                               uint8_t* sb) {
    bf16* __restrict__ O = static_cast<bf16*>(a.O);
    const int64_t T = a.T, Pdim = a.Pdim;
    const int l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int q = nt * 32 + l32;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 o;
                o[0] = to_bf16(acc[mt][nt][4 * g + 0]);
                o[1] = to_bf16(acc[mt][nt][4 * g + 1]);
                o[2] = to_bf16(acc[mt][nt][4 * g + 2]);
                o[3] = to_bf16(acc[mt][nt][4 * g + 3]);
                const int slot = (mt * 8 + 2 * g + lh) ^ (q & 31);
                *reinterpret_cast<bf16x4*>(sb + q * 256 + slot * 8) = o;
            }
        }
    }
    const int k = l & 15;
    const int64_t pc = p0 + wp * 128 + 8 * k;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
        const int row = it * 4 + (l >> 4);
        const int x = row & 31;
        u32x4 v = *reinterpret_cast<const u32x4*>(sb + row * 256 + ((k ^ (x >> 1)) << 4));
        if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        const int64_t t = q0 + wq * 128 + row;
        if (t < T && pc < Pdim) *reinterpret_cast<u32x4*>(O + t * Pdim + pc) = v;
    }
}

template <bool P_KMAJOR>
__global__ __launch_bounds__(kThreads, 1) void gemm_lora_bf16(GemmArgs a, SegTable seg) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
    const bf16* __restrict__ P = static_cast<const bf16*>(a.P);
    const bf16* __restrict__ Q = static_cast<const bf16*>(a.Q);
    const int64_t T = a.T, K = a.K, Pdim = a.Pdim;
    const int tiles_q = (int)((T + kBQ - 1) / kBQ);
    const int tiles_p = (int)((Pdim + kBP - 1) / kBP);
    int tq, tp;
    tile_of((int)blockIdx.x, (int)gridDim.x, tiles_q, tiles_p, tq, tp);
    const int64_t q0 = (int64_t)tq * kBQ, p0 = (int64_t)tp * kBP;

    const int tid = (int)threadIdx.x, l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1;
    const int l32 = l & 31, lh = l >> 5;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // ---- global -> register prefetch of one k stage -------------------------
    u32x4 pf[16];
    const int krow_r = tid >> 3, krow_c = tid & 7;      // K-contiguous: 32 rows x 8 chunks per pass
    const int prow_r = tid >> 5, prow_c = tid & 31;     // p-contiguous: 8 rows x 32 chunks per pass
    auto gload = [&](int kt) {
        const int64_t k0 = (int64_t)kt * kBK;
        if constexpr (P_KMAJOR) {
            const int64_t k = k0 + krow_c * 8;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                int64_t p = p0 + it * 32 + krow_r;
                p = p < Pdim ? p : Pdim - 1;
                pf[it] = load16_or_zero(P + p * K + k, k < K);
            }
        } else {
            const int64_t p = p0 + prow_c * 8;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int64_t k = k0 + it * 8 + prow_r;
                pf[it] = load16_or_zero(P + k * Pdim + p, k < K && p < Pdim);
            }
        }
        const int64_t k = k0 + krow_c * 8;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            int64_t t = q0 + it * 32 + krow_r;
            t = t < T ? t : T - 1;
            pf[8 + it] = load16_or_zero(Q + t * K + k, k < K);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* sp = smem + buf * kStage;
        uint8_t* sq = sp + kPTile;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            if constexpr (P_KMAJOR)
                *reinterpret_cast<u32x4*>(sp + kmaj(it * 32 + krow_r, krow_c)) = pf[it];
            else
                *reinterpret_cast<u32x4*>(sp + (it * 8 + prow_r) * kPRow + prow_c * 16) = pf[it];
        }
#pragma unroll
        for (int it = 0; it < 8; ++it)
            *reinterpret_cast<u32x4*>(sq + kmaj(it * 32 + krow_r, krow_c)) = pf[8 + it];
    };

    // Fragment of a p-contiguous tile: 8 consecutive k of feature p, read
    // transposed from rows k..k+7 (2 bytes per lane per row).
    auto pfrag_t = [&](const uint8_t* base, int p, int k) -> bf16x8 {
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const uint16_t*>(base + (k + e) * kPRow + p * 2);
        return __builtin_bit_cast(bf16x8, v);
    };

    auto compute = [&](int buf) {
        const uint8_t* sp = smem + buf * kStage;
        const uint8_t* sq = sp + kPTile;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = wp * 128 + mt * 32 + l32;
                if constexpr (P_KMAJOR)
                    fa[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(sp + kmaj(row, 2 * kk + lh)));
                else
                    fa[mt] = pfrag_t(sp, row, 16 * kk + 8 * lh);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                fb[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(sq + kmaj(wq * 128 + nt * 32 + l32, 2 * kk + lh)));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma32x32x16(fa[mt], fb[nt], acc[mt][nt]);
        }
    };

    // ---- frozen-weight K loop ------------------------------------------------
    const int KT = (int)((K + kBK - 1) / kBK);
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        compute(cur);
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---- LoRA expand, then one rounding to bf16 -------------------------------
    if (a.lora && seg.n > 0) lora_expand(acc, a, seg, q0, p0, smem, kPRow, smem + kPTile, smem + kPTile + kKTile);
    store_tile(acc, a, q0, p0);
}


// ===========================================================================
// Pipelined kernel (K a multiple of 128).
//
// Global -> LDS without registers: buffer_load_dwordx4 ... lds (gfx950 LDS
// DMA, 16 bytes per lane, 1 KiB per instruction = 8 rows x 128 bytes or 2
// rows x 512 bytes, i.e. whole cache lines).  Tiles are BK = 64 deep, 32 KiB
// each.  The token tile is triple-buffered and loaded two stages ahead: it is
// shared by the 16 or so feature tiles an XCD runs at once, so every one of
// them waits on the same L2 miss, and that wait is the one worth hiding.  The
// weight tile is double-buffered and loaded one stage ahead.  5 x 32 KiB = all
// 160 KiB of LDS.  Each buffer is its own __shared__ array so the compiler can
// tell which LDS DMA a fragment read depends on; the 6-stage rotation is
// unrolled so every buffer choice is static.  Rows past the tensor's end fall
// outside the buffer resource's range and read as zero.  Per stage: four k16
// steps of 16 MFMAs per wave; the fragments of step s+1 are read while step s
// runs; one barrier per stage, before the last step.
// ===========================================================================
constexpr int kPipeTile = 256 * kKRow;           // 32 KiB: 256 rows x 128 B (or 64 rows x 512 B)

__shared__ __attribute__((aligned(1024))) uint8_t g_t0[kPipeTile];  // token tiles (3)
__shared__ __attribute__((aligned(1024))) uint8_t g_t1[kPipeTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_t2[kPipeTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_w0[kPipeTile];  // weight tiles (2)
__shared__ __attribute__((aligned(1024))) uint8_t g_w1[kPipeTile];


// LoRA expand of the pipelined kernel.  The adapters whose segments overlap
// the tile are expanded together, over their ranks laid out in a 16-aligned
// rank space (adapter i owns virtual ranks voff[i] .. voff[i]+r_i-1, the rest
// of its 16-rank groups is zero), in chunks of 64 virtual ranks, however many
// adapters share the tile.  A 16-rank k-step therefore always holds ranks of
// one adapter in the same grouping as when that adapter runs alone, so the
// packed result equals the separate one bit for bit.  E rows of a chunk (p-
// contiguous, 512 bytes) arrive by LDS DMA, double-buffered, read transposed;
// F is block-diagonal: thread tid fills token row q0 + tid with s_i * H_i of
// its own adapter where the chunk covers that adapter's ranks and zero
// elsewhere (bf16 hi/lo).  The next chunk's loads are in flight during the
// current chunk's MFMAs, and per 16-rank k-step only the 32-token blocks
// holding tokens of the k-step's adapter multiply.  e0/e1 (E), shi/slo (F),
// tab (virtual rank -> E row table, at most 8192 entries): 32 KiB each, free.
__device__ __forceinline__ void lora_expand_pipe(f32x16 (&acc)[4][4], const GemmArgs& a, const SegTable& seg,
                                                 int64_t q0, int64_t p0, uint8_t* e0, uint8_t* e1, uint8_t* shi,
                                                 uint8_t* slo, uint8_t* tab) {
    const int64_t T = a.T, Pdim = a.Pdim;
    const int tid = (int)threadIdx.x, l = lane_id(), w = wave_id();
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;
    const int64_t tlast = (q0 + kBQ < T ? q0 + kBQ : T) - 1;
    const int i_first = segment_of(seg, q0), i_last = segment_in(seg, i_first, seg.n - 1, tlast);
    const int vlo = seg.voff[i_first], vhi = seg.voff[i_last + 1];
    const int nch = (vhi - vlo + 63) >> 6;
    if (nch <= 0) return;

    // E rows: buffer from column p0; row j at j * Pdim * 2 bytes; rows past R read zero
    const int R = seg.roff[seg.n];
    const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.E) + p0), 0, (int)(((int64_t)R * Pdim - p0) * 2), kRsrcWord3);
    const int tr = l >> 5;
    const uint32_t lane_t0 = (uint32_t)(((l & 31) ^ (tr << 2)) << 4);
    const uint32_t lane_t1 = (uint32_t)(((l & 31) ^ ((2 + tr) << 2)) << 4);
    // virtual rank rows j0 .. j0+63 (those below vhi); wave: 1 KiB blocks 8w .. 8w+7 of 2
    // rows v, v+1 (same adapter: adapters start at multiples of 16).  Padding rows read zero.
    // Table: byte offset of the E row of virtual rank vlo + i (0x80000000 for padding: reads zero)
    const int* rowtab = reinterpret_cast<const int*>(tab);
    for (int i = i_first; i <= i_last; ++i) {
        const int vb = seg.voff[i] - vlo, vn = seg.voff[i + 1] - seg.voff[i], r = seg.rank[i], rb = seg.roff[i];
        for (int k = tid; k < vn; k += kThreads)
            reinterpret_cast<int*>(tab)[vb + k] = k < r ? (int)((int64_t)(rb + k) * Pdim * 2) : (int)0x80000000u;
    }
    auto issue_e = [&](uint8_t* buf, int j0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int blk = 8 * wu + j;
            const int v = j0 + 2 * blk;
            if (v >= vhi) break;
            const uint32_t vo = ((j & 1) ? lane_t1 : lane_t0) + (uint32_t)rowtab[v + tr - vlo];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
    };

    // this thread's token row: adapter, its virtual rank range, its H row and scale.
    // The search runs over the tile's adapters with uniform indices (table reads
    // stay scalar); each lane keeps the entry that holds its token.
    const int64_t t = q0 + tid;
    int va = 0, rt = 0;
    float sc = 0.0f;
    int64_t hbase = 0;
    for (int i = i_first; i <= i_last; ++i) {
        if (t >= seg.off[i] && t < seg.off[i + 1]) {
            va = seg.voff[i];
            rt = seg.rank[i];
            sc = seg.scale[i];
            hbase = seg.hoff[i] + (t - seg.off[i]) * seg.rank[i];
        }
    }
    const float* hrow = a.F + hbase;
    // 16-byte loads need every 4-rank group to be inside or outside the row
    const bool vec = (hbase & 3) == 0 && (rt & 3) == 0;
    float fv[64];
    auto gather = [&](int j0) {  // fv[j] = H of virtual rank j0 + j when this row's adapter owns it, else 0
        if (vec) {
#pragma unroll
            for (int j4 = 0; j4 < 16; ++j4) {
                const int vv = j0 + 4 * j4;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (vv >= va && vv < va + rt) x = *reinterpret_cast<const f32x4*>(hrow + (vv - va));
                fv[4 * j4 + 0] = x[0];
                fv[4 * j4 + 1] = x[1];
                fv[4 * j4 + 2] = x[2];
                fv[4 * j4 + 3] = x[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                const int vv = j0 + j;
                fv[j] = (vv >= va && vv < va + rt) ? hrow[vv - va] : 0.0f;
            }
        }
    };
    auto stage_f = [&]() {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 h, o;
                split_bf16(sc * fv[c * 8 + e], h, o);
                hi[e] = __builtin_bit_cast(uint16_t, h);
                lo[e] = __builtin_bit_cast(uint16_t, o);
            }
            *reinterpret_cast<u16x8*>(shi + kmaj(tid, c)) = hi;
            *reinterpret_cast<u16x8*>(slo + kmaj(tid, c)) = lo;
        }
    };
    // virtual rank range of the adapters of each of this wave's 32-token blocks:
    // tokens are sorted by adapter, so it runs from the first token's adapter
    // start to the last token's adapter end (exchanged through shi, which the
    // first chunk's F overwrites after a barrier)
    int* vr = reinterpret_cast<int*>(shi);
    vr[tid] = va;
    vr[kThreads + tid] = va + ((rt + 15) & ~15);
    lds_barrier();  // also orders the table writes before the first E loads
    int blo[4], bhi[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int64_t b0 = q0 + (wu >> 1) * 128 + nt * 32;
        if (b0 > tlast) {
            blo[nt] = 1;
            bhi[nt] = 0;
        } else {
            const int f = (int)(b0 - q0), e = (int)((b0 + 31 < tlast ? b0 + 31 : tlast) - q0);
            blo[nt] = vr[f];
            bhi[nt] = vr[kThreads + e];
        }
    }
    auto chunk = [&](const uint8_t* eb, int j0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // virtual ranks j0 + 16 kk ..: the blocks whose adapters own some of them
            const int k0 = j0 + 16 * kk;
            bool live[4];
            bool any = false;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                live[nt] = blo[nt] < k0 + 16 && bhi[nt] > k0;
                any |= live[nt];
            }
            if (!any) continue;
            bf16x8 fa[4], fh[4], fl[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) fa[mt] = pfrag_tr(eb, wp * 128 + mt * 32, 16 * kk);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                if (!live[nt]) continue;
                const int row = wq * 128 + nt * 32 + l32;
                fh[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(shi + kmaj(row, 2 * kk + lh)));
                fl[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(slo + kmaj(row, 2 * kk + lh)));
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                if (!live[nt]) continue;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    acc[mt][nt] = mfma32x32x16(fa[mt], fh[nt], acc[mt][nt]);
                    acc[mt][nt] = mfma32x32x16(fa[mt], fl[nt], acc[mt][nt]);
                }
            }
        }
    };
    // one chunk: stage F (its values are in fv), make E(c) visible, start the
    // next chunk's loads, multiply
    auto step = [&](uint8_t* eb, uint8_t* en, int c) {
        const int j0 = vlo + 64 * c;
        lds_barrier();  // every wave is done with chunk c-1 (its F tiles and the buffer en)
        stage_f();  // its wait for fv (loaded after E(c) was issued) also covers E(c)
        if (c + 1 < nch) {
            issue_e(en, j0 + 64);
            wait_vmcnt<8>();  // at most 8 loads (E(c+1)) may stay in flight
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        if (c + 1 < nch) gather(j0 + 64);
        chunk(eb, j0);
    };
    issue_e(e0, vlo);
    gather(vlo);
    for (int c = 0; c < nch; c += 2) {
        step(e0, e1, c);
        if (c + 1 >= nch) break;
        step(e1, e0, c + 1);
    }
}

template <bool P_KMAJOR>
__global__ __launch_bounds__(kThreads, 1) void gemm_lora_bf16_pipe(GemmArgs a, SegTable seg) {
    const int64_t T = a.T, K = a.K, Pdim = a.Pdim;
    const int tiles_q = (int)((T + kBQ - 1) / kBQ);
    const int tiles_p = (int)((Pdim + kBP - 1) / kBP);
    int tq, tp;
    tile_of((int)blockIdx.x, (int)gridDim.x, tiles_q, tiles_p, tq, tp);
    const int64_t q0 = (int64_t)tq * kBQ, p0 = (int64_t)tp * kBP;
    const int l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;

    const int64_t prow = Pdim - p0 < kBP ? Pdim - p0 : kBP;
    const int64_t qrow = T - q0 < kBQ ? T - q0 : kBQ;
    // weight tile: K-contiguous rows p0.. (forward) or p-contiguous rows k.. of
    // columns p0.. (backward; columns past Pdim read neighbouring data that only
    // feeds output columns that are never stored)
    const __amdgpu_buffer_rsrc_t rp =
        P_KMAJOR ? __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const bf16*>(a.P) + p0 * K), 0,
                                                     (int)(prow * K * 2), kRsrcWord3)
                 : __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const bf16*>(a.P) + p0), 0,
                                                     (int)((K * Pdim - p0) * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.Q) + q0 * K), 0, (int)(qrow * K * 2), kRsrcWord3);
    // LDS DMA block b (1 KiB).  K-contiguous tiles: 8 rows x 128 B, lane l fills
    // row 8b + l/8, physical chunk l%8.  p-contiguous tile: 2 k-rows x 512 B, lane
    // l fills k-row 2b + l/32, physical chunk l%32.  Wave w owns blocks 8w..8w+7.
    // (row = 8b + l/8, so its swizzle (row ^ row/8) % 8 = (l/8 ^ b) % 8 = (l/8 ^ j) % 8)
    const int r0 = l >> 3;
    const uint32_t lane_row = (uint32_t)(r0 * K * 2);
    const uint32_t blk_stride = (uint32_t)(8 * K * 2);  // 8 rows
    // (row k = 2b + l/32, so k%4 = 2*(b%2) + l/32: one lane offset per block parity)
    const int tr = l >> 5;
    const uint32_t lane_off_t0 = (uint32_t)(tr * Pdim * 2) + (uint32_t)(((l & 31) ^ (tr << 2)) << 4);
    const uint32_t lane_off_t1 = (uint32_t)(tr * Pdim * 2) + (uint32_t)(((l & 31) ^ ((2 + tr) << 2)) << 4);
    const uint32_t blk_stride_t = (uint32_t)(2 * Pdim * 2);  // 2 k-rows
    const int KT = (int)(K / 64);
    const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform: LDS DMA bases stay scalar
    // past the last stage: push the offset beyond the resource's range (all
    // ranges are < 2^31 bytes), so the load writes zeros; no branch
    auto oob = [&](int kt) { return kt < KT ? 0u : 0x80000000u; };
    // this wave's 8 loads of stage kt's weight tile / token tile
    auto issue_w = [&](uint8_t* buf, int kt) {
        const uint32_t kb = (uint32_t)kt * 128u + oob(kt);
        const uint32_t kbt = (uint32_t)kt * (uint32_t)(64 * Pdim * 2) + oob(kt);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int blk = 8 * wu + j;
            const uint32_t vo =
                P_KMAJOR ? lane_row + (uint32_t)(((l & 7) ^ ((r0 ^ j) & 7)) << 4) + (uint32_t)blk * blk_stride + kb
                         : ((j & 1) ? lane_off_t1 : lane_off_t0) + (uint32_t)blk * blk_stride_t + kbt;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
    };
    auto issue_t = [&](uint8_t* buf, int kt) {
        const uint32_t kb = (uint32_t)kt * 128u + oob(kt);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int blk = 8 * wu + j;
            const uint32_t vo = lane_row + (uint32_t)(((l & 7) ^ ((r0 ^ j) & 7)) << 4) + (uint32_t)blk * blk_stride + kb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][4], fb[2][4];
    auto rd = [&](const uint8_t* bw, const uint8_t* bt, int kk, int s) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if constexpr (P_KMAJOR)
                fa[s][m] = as_bf16x8(*reinterpret_cast<const u32x4*>(bw + kmaj(wp * 128 + m * 32 + l32, 2 * kk + lh)));
            else
                fa[s][m] = pfrag_tr(bw, wp * 128 + m * 32, 16 * kk);  // p-contiguous weight tile
        }
#pragma unroll
        for (int n = 0; n < 4; ++n)
            fb[s][n] = as_bf16x8(*reinterpret_cast<const u32x4*>(bt + kmaj(wq * 128 + n * 32 + l32, 2 * kk + lh)));
    };
    auto mm = [&](int s) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[m][n] = mfma32x32x16(fa[s][m], fb[s][n], acc[m][n]);
    };
    // 16 MFMAs interleaved with 8 fragment reads (and `dma` LDS DMA loads)
    auto sched = [&](int dma) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            if (i < dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // LDS DMA load
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Stage kt: token tile in tc, weight tile in wc; stage kt+1 landing in tn /
    // wn; tf (free since the previous barrier) receives the token tile of stage
    // kt+2.  In flight at the barrier: tokens kt+2 only (8 loads).
    auto stage = [&](uint8_t* tc, uint8_t* wc, uint8_t* tn, uint8_t* wn, uint8_t* tf, int kt) {
        issue_t(tf, kt + 2);
        rd(wc, tc, 1, 1);
        mm(0);
        sched(8);
        rd(wc, tc, 2, 0);
        mm(1);
        sched(0);
        rd(wc, tc, 3, 1);
        mm(0);
        sched(0);
        wait_vmcnt<8>();  // stage kt+1 landed (tokens kt+2 may still be in flight)
        lds_barrier();    // and every wave is done reading wc / tc
        __builtin_amdgcn_sched_barrier(0);
        issue_w(wc, kt + 2);
        rd(wn, tn, 0, 0);
        mm(1);
        sched(8);
    };

    issue_t(g_t0, 0);
    issue_w(g_w0, 0);
    issue_t(g_t1, 1);
    issue_w(g_w1, 1);
    wait_vmcnt<16>();
    lds_barrier();
    rd(g_w0, g_t0, 0, 0);
    int kt = 0;
    for (; kt + 6 <= KT; kt += 6) {
        stage(g_t0, g_w0, g_t1, g_w1, g_t2, kt);
        stage(g_t1, g_w1, g_t2, g_w0, g_t0, kt + 1);
        stage(g_t2, g_w0, g_t0, g_w1, g_t1, kt + 2);
        stage(g_t0, g_w1, g_t1, g_w0, g_t2, kt + 3);
        stage(g_t1, g_w0, g_t2, g_w1, g_t0, kt + 4);
        stage(g_t2, g_w1, g_t0, g_w0, g_t1, kt + 5);
    }
    // KT is even: 0, 2 or 4 stages remain, continuing the same rotation
    if (kt + 2 <= KT) {
        stage(g_t0, g_w0, g_t1, g_w1, g_t2, kt);
        stage(g_t1, g_w1, g_t2, g_w0, g_t0, kt + 1);
    }
    if (kt + 4 <= KT) {
        stage(g_t2, g_w0, g_t0, g_w1, g_t1, kt + 2);
        stage(g_t0, g_w1, g_t1, g_w0, g_t2, kt + 3);
    }
    wait_vmcnt<0>();
    lds_barrier();

    if (a.lora && seg.n > 0) {
        lora_expand_pipe(acc, a, seg, q0, p0, g_t0, g_t1, g_w0, g_w1, g_t2);
        __syncthreads();  // the expand's LDS reads are done before the staging writes
    }
    store_tile_lds(acc, a, q0, p0, wu == 0 ? g_t0 : wu == 1 ? g_t1 : wu == 2 ? g_t2 : g_w0);
}
}  // namespace

hipError_t launch_gemm_bf16(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st) {
    const int64_t tq = (a.T + kBQ - 1) / kBQ, tp = (a.Pdim + kBP - 1) / kBP;
    const int64_t nwg = tq * tp;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg), block(kThreads);
    // 32-bit buffer ranges: one tile's token rows (256 x K elements), the
    // weight and the expand's E rows all stay below 2^31 bytes
    const bool pipelined = a.K % 128 == 0 && a.K < (int64_t(1) << 22) && a.Pdim < (int64_t(1) << 22) &&
                           a.K * a.Pdim * 2 < (int64_t(1) << 31) &&
                           (int64_t)(s.roff[s.n] + 64) * a.Pdim * 2 < (int64_t(1) << 31);  // expand's E range
    if (pipelined && p_kmajor)
        hipLaunchKernelGGL(gemm_lora_bf16_pipe<true>, grid, block, 0, st, a, s);
    else if (pipelined)
        hipLaunchKernelGGL(gemm_lora_bf16_pipe<false>, grid, block, 0, st, a, s);
    else if (p_kmajor)
        hipLaunchKernelGGL(gemm_lora_bf16<true>, grid, block, 0, st, a, s);
    else
        hipLaunchKernelGGL(gemm_lora_bf16<false>, grid, block, 0, st, a, s);
    return hipGetLastError();
}

}  // namespace plora
