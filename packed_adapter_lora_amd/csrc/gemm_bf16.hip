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

#include <atomic>
#include <cstdlib>

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

// Byte offset of 16-byte chunk c of row r in a K-contiguous tile.  The XOR
// keeps the 16 rows read by any 16 lanes (and any 8) on distinct bank groups.
__device__ __forceinline__ int kmaj(int r, int c) { return r * kKRow + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Workgroup -> output tile.  Workgroups are dealt round-robin to the 8 XCDs;
// renumber so each XCD gets a contiguous range of tiles, and walk that range
// in groups of gq token tiles: the ~32 workgroups an XCD runs at once then
// cover gq token tiles x 32/gq feature tiles, so their X/dY panels stay in
// that XCD's 4 MB L2 and the weight panels, re-read more often, come from the
// 256 MB Infinity Cache.  The launcher picks gq (2 or 4) per shape.
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_q, int tiles_p, int gq, int& tq, int& tp) {
    const int base = nwg / 8, extra = nwg % 8;
    const int xcd = bid % 8, slot = bid / 8;
    const int logical = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int per_group = gq * tiles_p;
    const int group = logical / per_group;
    const int first = group * gq;
    const int gsize = min(tiles_q - first, gq);
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
// whole 16-byte chunks of contiguous row pieces (one instruction = 1 KiB of
// token rows) instead of 8-byte pieces of 32 rows.  Each wave writes its own
// 128 (tokens) x 32*NM (features) quarter into its own 32 KiB buffer `sb`
// (token rows of 64*NM bytes, NS = 8*NM slots of 8 bytes); slot s of row q is
// stored at slot s ^ (q % NS), which keeps the 8-byte writes (rows x one slot)
// and the 16-byte reads (one row, NS/2 chunks) free of bank conflicts.  No
// workgroup barrier: a wave only reads what it wrote.  The stores are
// non-temporal: the output is not read again by this launch, and leaving it
// out of L2 keeps the token and weight panels there (1 % on the Y GEMM of
// the 4096 -> 14336 shape, same bits).  SWI: the row pieces
// are SwiGLU's da; the g and u pieces at the same place are read (eight row
// pieces' loads issued together) and dg, du written in place of O.
template <int NM = 4, bool SWI = false>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[NM][4], const GemmArgs& a, int64_t q0, int64_t p0,
                                               uint8_t* sb) {
    constexpr int NS = 8 * NM, RB = 8 * NS, CH = NS / 2, RPI = 64 / CH;  // slots, row bytes, chunks, rows/instr
    constexpr int NIT = 128 / RPI;                                         // row-piece stores per lane
    bf16* __restrict__ O = static_cast<bf16*>(a.O);
    const int64_t T = a.T, Pdim = a.Pdim;
    const int l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;
    const int k = l % CH;
    const int64_t pc = p0 + wp * (32 * NM) + 8 * k;
    // SWI: the g and u pieces of 8 row pieces per batch, two batches in
    // flight (rows past T and columns past Pdim load a valid piece instead;
    // their results are not stored)
    constexpr int BT = 8, NB = NIT / BT;
    u32x4 gv[2][BT], uv[2][BT];
    auto load_batch = [&](int b, int sl) {
        const bf16* __restrict__ gp = static_cast<const bf16*>(a.sw_g);
        const bf16* __restrict__ up = static_cast<const bf16*>(a.sw_u);
        const int64_t pcc = pc < Pdim ? pc : Pdim - 8;
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            const int64_t t = q0 + wq * 128 + (b * BT + j) * RPI + l / CH;
            const int64_t e = (t < T ? t : T - 1) * Pdim + pcc;
            gv[sl][j] = *reinterpret_cast<const u32x4*>(gp + e);
            uv[sl][j] = *reinterpret_cast<const u32x4*>(up + e);
        }
    };
    if constexpr (SWI) load_batch(0, 0);  // (in flight during the staging writes)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int q = nt * 32 + l32;
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 o;
                o[0] = to_bf16(acc[mt][nt][4 * g + 0]);
                o[1] = to_bf16(acc[mt][nt][4 * g + 1]);
                o[2] = to_bf16(acc[mt][nt][4 * g + 2]);
                o[3] = to_bf16(acc[mt][nt][4 * g + 3]);
                const int slot = (mt * 8 + 2 * g + lh) ^ (q & (NS - 1));
                *reinterpret_cast<bf16x4*>(sb + q * RB + slot * 8) = o;
            }
        }
    }
    if constexpr (SWI) {
        bf16* __restrict__ dgp = static_cast<bf16*>(a.sw_dg);
        bf16* __restrict__ dup = static_cast<bf16*>(a.sw_du);
        // bf16 element e of a 16-byte piece, as fp32
        auto elt = [](const u32x4& v, int e) {
            return __builtin_bit_cast(float, (v[e >> 1] >> (16 * (e & 1))) << 16);
        };
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b + 1 < NB) load_batch(b + 1, (b + 1) & 1);
#pragma unroll
            for (int j = 0; j < BT; ++j) {
                const int row = (b * BT + j) * RPI + l / CH;
                const int x = row & (NS - 1);
                u32x4 v = *reinterpret_cast<const u32x4*>(sb + row * RB + ((k ^ (x >> 1)) << 4));
                if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
                bf16x8 og, ou;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float dg, du;
                    swiglu_grad(elt(v, e), elt(gv[b & 1][j], e), elt(uv[b & 1][j], e), dg, du);
                    og[e] = to_bf16(dg);
                    ou[e] = to_bf16(du);
                }
                const int64_t t = q0 + wq * 128 + row;
                if (t < T && pc < Pdim) {
                    __builtin_nontemporal_store(as_u32x4(og), reinterpret_cast<u32x4*>(dgp + t * Pdim + pc));
                    __builtin_nontemporal_store(as_u32x4(ou), reinterpret_cast<u32x4*>(dup + t * Pdim + pc));
                }
            }
        }
    } else {
#pragma unroll 4
        for (int it = 0; it < NIT; ++it) {
            const int row = it * RPI + l / CH;
            const int x = row & (NS - 1);
            u32x4 v = *reinterpret_cast<const u32x4*>(sb + row * RB + ((k ^ (x >> 1)) << 4));
            if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            const int64_t t = q0 + wq * 128 + row;
            if (t < T && pc < Pdim) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(O + t * Pdim + pc));
        }
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
    tile_of((int)blockIdx.x, (int)gridDim.x, tiles_q, tiles_p, a.group_q > 0 ? a.group_q : 2, tq, tp);
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

// Tiles of p-contiguous rows (the dX weight tile, the expand's E rows) are
// 2*BP bytes wide for a tile of BP = 64*NM features: 512 (NM = 4) or 256
// (NM = 2) bytes.  One 1 KiB LDS DMA block holds kRowsPerBlk rows; lane l
// fills row l / (chunks per row) of the block at physical chunk l % (chunks
// per row), holding logical chunk (physical ^ 4 (row % 4)) -- the layout
// pfrag_tr<2*BP> reads.
template <int NM>
struct PRows {
    static_assert(NM == 4 || NM == 2, "tiles of 256 or 128 features");
    static constexpr int kBytes = 128 * NM;               // bytes per row
    static constexpr int kChunks = kBytes / 16;           // 16-byte chunks per row
    static constexpr int kRowsPerBlk = 1024 / kBytes;     // 2 or 4
    static constexpr int kShift = NM == 4 ? 5 : 4;         // log2(kChunks)
    // row of the block this lane fills, and its byte offset within the row
    // for a block whose first row is r0 (r0 % 4 = 0, or 2 with 2-row blocks)
    __device__ static int lane_row(int l) { return l >> kShift; }
    __device__ static uint32_t lane_col(int l, int r0) {
        return (uint32_t)(((l & (kChunks - 1)) ^ ((r0 + (l >> kShift)) << 2)) << 4);
    }
};

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
// F is block-diagonal: token row t holds s_i * H_i[t] (bf16 hi + lo) at its
// own adapter's virtual ranks and zero elsewhere.  Per 16-rank k-step only
// the 32-token blocks holding tokens of the k-step's adapter multiply.
//
// F comes from one of two LDS layouts, with the same fragment values and
// MFMA order (so the same bits):
//  - compact (every adapter of the tile has r_i <= 64): staged once, one row
//    per token over the token's own ranks (zero from r_i on); an MFMA lane
//    reads the 8 ranks it needs at the adapter's local offset, or zero.  The
//    chunks then only stream E, and each 128-token half of the tile streams
//    its own: chunks of its own adapters' ranks (32 rows of 512 bytes, or 64
//    of 256 with 128-feature tiles: 16 KiB) into its own half of each E
//    buffer (the halves share at most one adapter), so both halves multiply
//    in every step.  One barrier per step; the next step's rows are in flight
//    during the current step's MFMAs.
//  - per chunk (some r_i > 64): the 64 virtual ranks of the chunk for every
//    token, restaged each chunk from registers gathered during the previous
//    chunk.
// A tile of one adapter with r_i <= 64 (every tile of long segments) takes
// the compact layout with a uniform setup: the adapter's fields are scalar
// loads, its E rows are addressed without the row table, and the first E
// step is in flight while F is staged.
// e0/e1 (E), shi/slo (F hi/lo), tab (virtual rank -> E row table, at most
// 8192 entries): 32 KiB each, free.  e1 first holds a per-token table.
template <int NM>
__device__ __forceinline__ void lora_expand_pipe(f32x16 (&acc)[NM][4], const GemmArgs& a, const SegTable& seg,
                                                 int64_t q0, int64_t p0, uint8_t* e0, uint8_t* e1, uint8_t* shi,
                                                 uint8_t* slo, uint8_t* tab) {
    using PR = PRows<NM>;
    constexpr int RPB = PR::kRowsPerBlk;
    const int64_t T = a.T, Pdim = a.Pdim;
    const int tid = (int)threadIdx.x, l = lane_id(), w = wave_id();
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;
    const int64_t tlast = (q0 + kBQ < T ? q0 + kBQ : T) - 1;
    // The tile's adapters: the first whose segment ends past q0, the first
    // whose segment ends past tlast (lane j tests adapter j; at most 64)
    const int64_t endl = l < seg.n ? seg.off[l + 1] : INT64_MAX;
    const int i_first = (int)__popcll(__ballot(endl <= q0));
    const int i_last = (int)__popcll(__ballot(endl <= tlast));
    const int vlo = seg.voff[i_first], vhi = seg.voff[i_last + 1];
    const int nch = (vhi - vlo + 63) >> 6;
    if (nch <= 0) return;

    // E rows: buffer from column p0; row j at j * Pdim * 2 bytes; rows past R read zero
    const int R = seg.roff[seg.n];
    const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.E) + p0), 0, (int)(((int64_t)R * Pdim - p0) * 2), kRsrcWord3);
    const int tr = PR::lane_row(l);
    const uint32_t lane_t0 = PR::lane_col(l, 0);
    const uint32_t lane_t1 = PR::lane_col(l, 2);  // (blocks of 2 rows starting at 2 mod 4)
    // virtual rank rows j0 .. j0+63 (those below vhi); wave: 1 KiB blocks of RPB rows
    // (same adapter: adapters start at multiples of 16).  Padding rows read zero.
    // Table: byte offset of the E row of virtual rank vlo + i (0x80000000 for padding: reads zero)
    const int* rowtab = reinterpret_cast<const int*>(tab);
    auto issue_e = [&](uint8_t* buf, int j0) {
        constexpr int NB = 16 / RPB;  // blocks per wave: 64 rows / RPB / 4 waves
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int blk = NB * wu + j;
            const int v = j0 + RPB * blk;
            if (v >= vhi) break;
            const uint32_t vo = ((RPB == 2 && (j & 1)) ? lane_t1 : lane_t0) + (uint32_t)rowtab[v + tr - vlo];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
    };

    // The tile's adapter when it is one of rank <= 64 (the common case): its
    // fields are wave-uniform (scalar loads), its E rows are addressed without
    // the row table, and the first E rows are in flight with the H loads.
    const int na = i_last - i_first + 1;
    const int r_first = seg.rank[i_first];
    const bool single = na == 1 && r_first <= 64;
    const int rb_first = seg.roff[i_first];
    const uint32_t row_bytes = (uint32_t)(Pdim * 2);

    // this thread's token row: its adapter, the adapter's virtual rank range,
    // its H row and scale (zero for rows past the last token)
    const int64_t t = q0 + tid;
    int va = 0, rt = 0, rmax = r_first;
    float sc = 0.0f;
    int64_t hbase = 0;
    if (single) {
        if (t <= tlast) {
            va = vlo;
            rt = r_first;
            sc = seg.scale[i_first];
            hbase = seg.hoff[i_first] + (t - seg.off[i_first]) * rt;
        }
    } else {
        // Per-adapter records of the tile's adapters (in e1 past the token
        // table, free until the E loads of step 1): lane j of wave 0 takes
        // adapter i_first + j, writes its E row table entries (virtual rank ->
        // byte offset, at most 128 per adapter) and its record; the largest
        // rank goes into the record area too.
        int64_t* rec_off = reinterpret_cast<int64_t*>(e1 + 4096);  // 64 x 8 B
        int64_t* rec_hoff = rec_off + 64;                          // 64 x 8 B
        int* rec_voff = reinterpret_cast<int*>(rec_hoff + 64);     // 64 x 4 B
        int* rec_rank = rec_voff + 64;
        float* rec_scale = reinterpret_cast<float*>(rec_rank + 64);
        int* rec_rmax = reinterpret_cast<int*>(rec_scale + 64);
        if (wu == 0) {
            const int i = i_first + l;
            int r = 0;
            if (l < na) {
                const int v0 = seg.voff[i], vn = seg.voff[i + 1] - v0, rb = seg.roff[i];
                r = seg.rank[i];
                // (16 entries per iteration: vn and v0 - vlo are multiples of 16)
                for (int k = 0; k < vn; k += 16) {
                    u32x4 e[4];
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        e[q >> 2][q & 3] = k + q < r ? (uint32_t)((int64_t)(rb + k + q) * Pdim * 2) : 0x80000000u;
#pragma unroll
                    for (int q = 0; q < 4; ++q) reinterpret_cast<u32x4*>(tab)[(v0 - vlo + k) / 4 + q] = e[q];
                }
                rec_off[l] = seg.off[i];
                rec_hoff[l] = seg.hoff[i];
                rec_voff[l] = v0;
                rec_rank[l] = r;
                rec_scale[l] = seg.scale[i];
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const int o = __shfl_xor(r, d);
                r = o > r ? o : r;
            }
            if (l == 0) *rec_rmax = r;
        }
        lds_barrier();
        rmax = __builtin_amdgcn_readfirstlane(*rec_rmax);
        if (t <= tlast) {
            // the last record starting at or before t
            int lo = 0, hi = na;  // rec_off[lo] <= t < rec_off[hi] (or hi == na)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (rec_off[mid] <= t) lo = mid; else hi = mid;
            }
            va = rec_voff[lo];
            rt = rec_rank[lo];
            sc = rec_scale[lo];
            hbase = rec_hoff[lo] + (t - rec_off[lo]) * rt;
        }
    }
    const bool compact = rmax <= 64;
    const float* hrow = a.F + hbase;
    // 16-byte loads need every 4-rank group to be inside or outside the row
    const bool vec = (hbase & 3) == 0 && (rt & 3) == 0;
    float fv[64];
    // fv[j] = H of virtual rank j0 + j when this row's adapter owns it, else 0
    // (compact layout: j0 = va, the row's own ranks)
    auto gather = [&](int j0) {
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
    // row tid of shi/slo (128-byte kmaj rows) = s * fv split into bf16 hi + lo
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
    // 16 zero bytes past the row table (compact: at most 64 x 64 entries = 16 KiB):
    // the F fragment of lanes whose token does not own the k-step's ranks
    const uint8_t* zero16 = tab + 32768 - 16;
    if (compact) gather(va);
    // per MFMA lane and token block nt: the range of token wq*128 + nt*32 + l%32
    // (compact layout); per block: the range of its adapters (tokens are sorted
    // by adapter: first token's start to last token's end).  Per 128-token half
    // (compact layout): its virtual rank range (its first block's start to its
    // last valid block's end), as HR-rank chunks.
    constexpr int HR = 16384 / PR::kBytes;  // 32 or 64 rows: 16 KiB per half
    int tva[4], tve[4], blo[4], bhi[4];
    int hlo[2], hn[2];
    if (single) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const bool in = q0 + wq * 128 + nt * 32 + l32 <= tlast;
            tva[nt] = in ? vlo : 0;
            tve[nt] = in ? vhi : 0;
            const bool bin = q0 + (wu >> 1) * 128 + nt * 32 <= tlast;
            blo[nt] = bin ? vlo : 1;
            bhi[nt] = bin ? vhi : 0;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool hin = q0 + h * 128 <= tlast;
            hlo[h] = hin ? vlo : 0;
            hn[h] = hin ? (vhi - vlo + HR - 1) / HR : 0;
        }
    } else {
        // token table: first virtual rank of each token's adapter and the end of
        // its 16-rank groups
        int* ti = reinterpret_cast<int*>(e1);
        ti[tid] = va;
        ti[kThreads + tid] = va + ((rt + 15) & ~15);
        lds_barrier();  // also orders the row table writes before the first E loads
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int row = wq * 128 + nt * 32 + l32;
            tva[nt] = ti[row];
            tve[nt] = ti[kThreads + row];
            const int64_t b0 = q0 + (wu >> 1) * 128 + nt * 32;
            if (b0 > tlast) {
                blo[nt] = 1;
                bhi[nt] = 0;
            } else {
                const int f = (int)(b0 - q0), e = (int)((b0 + 31 < tlast ? b0 + 31 : tlast) - q0);
                blo[nt] = __builtin_amdgcn_readfirstlane(ti[f]);  // (wave-uniform: scalar tests below)
                bhi[nt] = __builtin_amdgcn_readfirstlane(ti[kThreads + e]);
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t b0 = q0 + h * 128;
            if (b0 > tlast) {
                hlo[h] = 0;
                hn[h] = 0;
            } else {
                const int f = h * 128, e = (int)((b0 + 127 < tlast ? b0 + 127 : tlast) - q0);
                hlo[h] = __builtin_amdgcn_readfirstlane(ti[f]);
                hn[h] = (__builtin_amdgcn_readfirstlane(ti[kThreads + e]) - hlo[h] + HR - 1) / HR;
            }
        }
    }
    // k-steps in pairs: both steps' fragments are read before the first
    // step's MFMAs, so the second step's reads overlap them
    auto chunk = [&](const uint8_t* eb, int j0, int nkk) {
#pragma unroll
        for (int kp = 0; kp < 4; kp += 2) {
            if (kp >= nkk) break;
            bool live[2][4], any[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                // virtual ranks k0 ..: the blocks whose adapters own some of them
                const int k0 = j0 + 16 * (kp + s2);
                any[s2] = false;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    live[s2][nt] = blo[nt] < k0 + 16 && bhi[nt] > k0;
                    any[s2] |= live[s2][nt];
                }
            }
            bf16x8 fa[2][NM], fh[2][4], fl[2][4];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (!any[s2]) continue;
                const int kk = kp + s2, k0 = j0 + 16 * kk;
#pragma unroll
                for (int mt = 0; mt < NM; ++mt)
                    fa[s2][mt] = pfrag_tr<PR::kBytes>(eb, wp * (32 * NM) + mt * 32, 16 * kk);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (!live[s2][nt]) continue;
                    // ranks k0 + 8*lh .. +7 of this lane's token: 8-rank group (v - va)/8
                    // of its compact row, or group 2*kk + lh of the chunk's rows
                    // (lanes that do not own them read 16 zero bytes)
                    const int v = k0 + 8 * lh;
                    const bool own = !compact || (v >= tva[nt] && v < tve[nt]);
                    const int col = compact ? (own ? (v - tva[nt]) >> 3 : 0) : 2 * kk + lh;
                    const int off = kmaj(wq * 128 + nt * 32 + l32, col);
                    fh[s2][nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(own ? shi + off : zero16));
                    fl[s2][nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(own ? slo + off : zero16));
                }
            }
            // per accumulator: k-steps in order, hi then lo (the order of the
            // separate expand); the four accumulators of a block interleaved
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (!any[s2]) continue;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (!live[s2][nt]) continue;
#pragma unroll
                    for (int mt = 0; mt < NM; ++mt)
                        acc[mt][nt] = mfma32x32x16(fa[s2][mt], fh[s2][nt], acc[mt][nt]);
#pragma unroll
                    for (int mt = 0; mt < NM; ++mt)
                        acc[mt][nt] = mfma32x32x16(fa[s2][mt], fl[s2][nt], acc[mt][nt]);
                }
            }
        }
    };
    const int wqu = wu >> 1;  // (this wave's half, wave-uniform)
    const int own_lo = wqu ? hlo[1] : hlo[0], own_n = wqu ? hn[1] : hn[0];
    const int nstep = compact ? (hn[0] > hn[1] ? hn[0] : hn[1]) : nch;
    // this wave's loads of its half's chunk from virtual rank j0 (HR rows, split
    // over the wave pair: 1 KiB blocks HB*wp .. +HB-1 of RPB rows), into buf
    // (16 KiB)
    const int own_hi = own_lo + HR * own_n;
    constexpr int HB = 8;
    // (all row offsets first, then the loads; rows past the range or the
    // adapter's rank read zero)
    auto issue_half = [&](uint8_t* buf, int j0) {
        uint32_t ro[HB];
#pragma unroll
        for (int j = 0; j < HB; ++j) {
            const int v = j0 + RPB * (HB * wp + j);
            const bool in = v < own_hi && v < vhi;
            if (single) {
                const int k = v + tr - vlo;
                ro[j] = in && k < r_first ? (uint32_t)(rb_first + k) * row_bytes : 0x80000000u;
            } else {
                ro[j] = in ? (uint32_t)rowtab[(in ? v : vlo) + tr - vlo] : 0x80000000u;
            }
        }
#pragma unroll
        for (int j = 0; j < HB; ++j) {
            const int blk = HB * wp + j;
            const uint32_t vo = ((RPB == 2 && (j & 1)) ? lane_t1 : lane_t0) + ro[j];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
    };
    // One chunk.  Per-chunk layout: stage F of chunk c (its values are in fv),
    // make E(c) visible, start the next chunk's loads, multiply.  Compact
    // layout: start the next chunk's loads, multiply, make E(c+1) visible.
    auto step = [&](uint8_t* eb, uint8_t* en, int c) {
        // (one chunk() call for both layouts: the accumulators stay on one path;
        // its E buffer is eb plus an offset, so the compiler still sees which
        // LDS DMA it depends on and need not wait for the next step's)
        const uint8_t* ec = eb + (compact ? wqu * 16384 : 0);
        const int jc = compact ? own_lo + HR * c : vlo + 64 * c;
        const int nkk = compact ? (c < own_n ? HR / 16 : 0) : 4;
        if (compact) {
            if (c + 1 < own_n) issue_half(en + wqu * 16384, own_lo + HR * (c + 1));
        } else {
            const int j0 = vlo + 64 * c;
            lds_barrier();  // every wave is done with chunk c-1 (its F tiles and the buffer en)
            stage_f();      // its wait for fv (loaded after E(c) was issued) also covers E(c)
            if (c + 1 < nch) {
                issue_e(en, j0 + 64);
                wait_vmcnt<8>();  // at most 8 loads (E(c+1)) may stay in flight
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
            if (c + 1 < nch) gather(j0 + 64);
        }
        chunk(ec, jc, nkk);
        if (compact) {
            wait_vmcnt<0>();
            lds_barrier();  // step c+1 landed everywhere; every wave is done with eb
        }
    };
    if (compact) {
        // E of step 0 in flight while F is staged (its H rows were loaded first)
        if (own_n > 0) issue_half(e0 + wqu * 16384, own_lo);
        stage_f();
        if (tid == 0) *reinterpret_cast<u32x4*>(tab + 32768 - 16) = u32x4{0u, 0u, 0u, 0u};
        wait_vmcnt<0>();
        lds_barrier();  // step 0 and F landed; the token table is read before step 1 overwrites it
    } else {
        issue_e(e0, vlo);
        gather(vlo);
    }
    for (int c = 0; c < nstep; c += 2) {
        step(e0, e1, c);
        if (c + 1 >= nstep) break;
        step(e1, e0, c + 1);
    }
}

// NM = 32-feature MFMA blocks per wave: tiles of 64*NM features x 256 tokens
// (NM = 4: 256 x 256; NM = 2: 128 x 256, twice the tiles for shapes whose
// 256-wide tiles leave most of the chip idle or a last partial wave).
template <bool P_KMAJOR, int NM, bool SWI = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_lora_bf16_pipe(GemmArgs a, SegTable seg) {
    constexpr int BP = 64 * NM;          // features per tile
    constexpr int WL = 2 * NM;           // weight-tile loads per wave and stage
    using PR = PRows<NM>;
    const int64_t T = a.T, K = a.K, Pdim = a.Pdim;
    const int64_t pb = a.p_begin, pe = a.p_end > 0 ? a.p_end : Pdim;
    const int tiles_q = (int)((T + kBQ - 1) / kBQ);
    const int tiles_p = (int)((pe - pb + BP - 1) / BP);
    int tq, tp;
    tile_of((int)blockIdx.x, (int)gridDim.x, tiles_q, tiles_p, a.group_q > 0 ? a.group_q : 2, tq, tp);
    const int64_t q0 = (int64_t)tq * kBQ, p0 = pb + (int64_t)tp * BP;
    const int l = lane_id(), w = wave_id();
    const int wp = w & 1, wq = w >> 1, l32 = l & 31, lh = l >> 5;

    const int64_t prow = Pdim - p0 < BP ? Pdim - p0 : BP;
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
    // row 8b + l/8, physical chunk l%8.  p-contiguous weight tile: RPB k-rows of
    // 2*BP bytes (PRows).  The token tile's blocks 8w..8w+7 and the weight
    // tile's WL*w .. WL*w+WL-1 belong to wave w.
    // (row = 8b + l/8, so its swizzle (row ^ row/8) % 8 = (l/8 ^ b) % 8)
    const int r0 = l >> 3;
    const uint32_t lane_row = (uint32_t)(r0 * K * 2);
    const uint32_t blk_stride = (uint32_t)(8 * K * 2);  // 8 rows
    // (k-row = RPB b + row of the lane; with RPB = 2 the swizzle depends on b's parity)
    const int tr = PR::lane_row(l);
    const uint32_t lane_off_t0 = (uint32_t)(tr * Pdim * 2) + PR::lane_col(l, 0);
    const uint32_t lane_off_t1 = (uint32_t)(tr * Pdim * 2) + PR::lane_col(l, 2);
    const uint32_t blk_stride_t = (uint32_t)(PR::kRowsPerBlk * Pdim * 2);
    const int KT = (int)(K / 64);
    const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform: LDS DMA bases stay scalar
    // past the last stage: push the offset beyond the resource's range (all
    // ranges are < 2^31 bytes), so the load writes zeros; no branch
    auto oob = [&](int kt) { return kt < KT ? 0u : 0x80000000u; };
    // this wave's WL (weight) / 8 (token) loads of stage kt
    auto issue_w = [&](uint8_t* buf, int kt) {
        const uint32_t kb = (uint32_t)kt * 128u + oob(kt);
        const uint32_t kbt = (uint32_t)kt * (uint32_t)(64 * Pdim * 2) + oob(kt);
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const int blk = WL * wu + j;
            const uint32_t vo =
                P_KMAJOR ? lane_row + (uint32_t)(((l & 7) ^ ((r0 ^ blk) & 7)) << 4) + (uint32_t)blk * blk_stride + kb
                         : ((PR::kRowsPerBlk == 2 && (j & 1)) ? lane_off_t1 : lane_off_t0) +
                               (uint32_t)blk * blk_stride_t + kbt;
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

    f32x16 acc[NM][4];
#pragma unroll
    for (int i = 0; i < NM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][NM], fb[2][4];
    auto rd = [&](const uint8_t* bw, const uint8_t* bt, int kk, int s) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if constexpr (P_KMAJOR)
                fa[s][m] =
                    as_bf16x8(*reinterpret_cast<const u32x4*>(bw + kmaj(wp * (32 * NM) + m * 32 + l32, 2 * kk + lh)));
            else
                fa[s][m] = pfrag_tr<PR::kBytes>(bw, wp * (32 * NM) + m * 32, 16 * kk);  // p-contiguous weight tile
        }
#pragma unroll
        for (int n = 0; n < 4; ++n)
            fb[s][n] = as_bf16x8(*reinterpret_cast<const u32x4*>(bt + kmaj(wq * 128 + n * 32 + l32, 2 * kk + lh)));
    };
    // serpentine order: consecutive instructions share one operand (the chip is
    // power-capped and its clock follows how much the operands toggle), here
    // the token fragment for NM instructions in a row (0.1-0.3 % faster than
    // holding the weight fragment); every accumulator still sees its k-steps
    // in order, so the bits do not change
    auto mm = [&](int s) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int m0 = 0; m0 < NM; ++m0) {
                const int m = (n & 1) ? NM - 1 - m0 : m0;
                acc[m][n] = mfma32x32x16(fa[s][m], fb[s][n], acc[m][n]);
            }
    };
    // 4*NM MFMAs interleaved with NM + 4 fragment reads (and `dma` LDS DMA loads)
    auto sched = [&](int dma) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (2 * i < 4 * NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (i < NM + 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
            if (i < dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // LDS DMA load
            if (2 * i + 1 < 4 * NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
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
        sched(WL);
    };

    issue_t(g_t0, 0);
    issue_w(g_w0, 0);
    issue_t(g_t1, 1);
    issue_w(g_w1, 1);
    wait_vmcnt<8 + WL>();  // stage 0 landed (stage 1 may be in flight)
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
        lora_expand_pipe<NM>(acc, a, seg, q0, p0, g_t0, g_t1, g_w0, g_w1, g_t2);
        __syncthreads();  // the expand's LDS reads are done before the staging writes
    }
    store_tile_lds<NM, SWI>(acc, a, q0, p0, wu == 0 ? g_t0 : wu == 1 ? g_t1 : wu == 2 ? g_t2 : g_w0);
}
}  // namespace

// Compute units of the current device (cached per device id; atomic, since
// calls may come from several host threads at once).
static int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// 32-bit buffer ranges: one tile's token rows (256 x K elements), the weight
// and the expand's E rows all stay below 2^31 bytes
bool gemm_bf16_pipelined(const GemmArgs& a, const SegTable& s) {
    return a.K % 128 == 0 && a.K < (int64_t(1) << 22) && a.Pdim < (int64_t(1) << 22) &&
           a.K * a.Pdim * 2 < (int64_t(1) << 31) &&
           (int64_t)(s.roff[s.n] + 64) * a.Pdim * 2 < (int64_t(1) << 31);  // expand's E range
}

hipError_t launch_gemm_bf16(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st) {
    const int64_t tq = (a.T + kBQ - 1) / kBQ, tp = (a.Pdim + kBP - 1) / kBP;
    const int64_t nwg = tq * tp;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x3fffffff) return hipErrorInvalidValue;
    const dim3 block(kThreads);
    const bool pipelined = gemm_bf16_pipelined(a, s);
    // the fused SwiGLU epilogue exists for the pipelined dX GEMM only
    const bool swi = a.sw_g != nullptr;
    if (swi && (p_kmajor || !pipelined)) return hipErrorInvalidValue;
    if (pipelined) {
        // Tile widths.  A 128-wide tile takes ~0.57 of a 256-wide tile's time.
        // All 128-wide when they fit on the chip at once (a few hundred tokens).
        // Otherwise the feature range is split: 256-wide tiles over the first
        // f columns of 256 features, 128-wide over the rest, as two launches,
        // with f chosen by counting waves (one unit per wave of 256-wide tiles,
        // 0.57 per wave of 128-wide): a grid of 3.5 waves of 256-wide tiles
        // becomes 3 waves plus one wave of 128-wide tiles.  Each output element
        // sees the same MFMA sequence at either width, so the split does not
        // change any bit.  PLORA_GEMM_TILE_P=128 or 256 forces one width.
        // L2 groups of 4 token tiles when K is at most 8192, else 2 (llama
        // 4096 -> 14336: Y GEMM -0.9 % with 4, the K = 14336 dX GEMM +2.1 %;
        // 4096 -> 4096: -1.7 % / -1.1 %).  PLORA_GEMM_GROUP_Q=1, 2, 4 or 8
        // forces it.  The tile a workgroup computes changes, no output bit does.
        GemmArgs ag = a;
        const char* fgq = getenv("PLORA_GEMM_GROUP_Q");
        const int fg = fgq ? atoi(fgq) : 0;
        ag.group_q = fg == 1 || fg == 2 || fg == 4 || fg == 8 ? fg : (a.K <= 8192 ? 4 : 2);
        const int64_t cus = cu_count(), tp2 = (a.Pdim + 127) / 128, nwg2 = tq * tp2;
        const char* force = getenv("PLORA_GEMM_TILE_P");
        const int fw = force ? atoi(force) : 0;
        int64_t f = tp;  // 256-wide feature columns
        if (fw == 128 || (fw != 256 && nwg2 <= cus)) {
            f = 0;
        } else if (fw != 256) {
            auto waves = [&](int64_t n) { return (n + cus - 1) / cus; };
            double best = (double)waves(nwg);
            for (int64_t g = tp - 1; g >= 0; --g) {
                const int64_t rest = (a.Pdim - 256 * g + 127) / 128;
                const double c = (double)waves(tq * g) + 0.57 * (double)waves(tq * rest);
                if (c < best - 1e-9) {
                    best = c;
                    f = g;
                }
            }
        }
        if (f > 0) {
            GemmArgs w = ag;
            w.p_begin = 0;
            w.p_end = f == tp ? 0 : 256 * f;
            const dim3 grid((unsigned)(tq * f));
            if (p_kmajor)
                hipLaunchKernelGGL((gemm_lora_bf16_pipe<true, 4>), grid, block, 0, st, w, s);
            else if (swi)
                hipLaunchKernelGGL((gemm_lora_bf16_pipe<false, 4, true>), grid, block, 0, st, w, s);
            else
                hipLaunchKernelGGL((gemm_lora_bf16_pipe<false, 4>), grid, block, 0, st, w, s);
        }
        if (f < tp) {
            GemmArgs h = ag;
            h.p_begin = 256 * f;
            h.p_end = 0;
            const dim3 grid((unsigned)(tq * ((a.Pdim - 256 * f + 127) / 128)));
            if (p_kmajor)
                hipLaunchKernelGGL((gemm_lora_bf16_pipe<true, 2>), grid, block, 0, st, h, s);
            else if (swi)
                hipLaunchKernelGGL((gemm_lora_bf16_pipe<false, 2, true>), grid, block, 0, st, h, s);
            else
                hipLaunchKernelGGL((gemm_lora_bf16_pipe<false, 2>), grid, block, 0, st, h, s);
        }
    } else {
        const dim3 grid((unsigned)nwg);
        if (p_kmajor)
            hipLaunchKernelGGL(gemm_lora_bf16<true>, grid, block, 0, st, a, s);
        else
            hipLaunchKernelGGL(gemm_lora_bf16<false>, grid, block, 0, st, a, s);
    }
    return hipGetLastError();
}

}  // namespace plora
