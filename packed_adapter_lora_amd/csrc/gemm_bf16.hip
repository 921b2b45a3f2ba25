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
constexpr int kGroupQ = 8;                     // token tiles per L2 group

// Byte offset of 16-byte chunk c of row r in a K-contiguous tile.  The XOR
// keeps the 16 rows read by any 16 lanes (and any 8) on distinct bank groups.
__device__ __forceinline__ int kmaj(int r, int c) { return r * kKRow + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Workgroup -> output tile.  Workgroups are dealt round-robin to the 8 XCDs;
// renumber so each XCD gets a contiguous range of tiles, and walk that range
// in groups of kGroupQ token tiles so concurrent workgroups on one XCD share
// X/dY and W panels in that XCD's L2.
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

    // ---- LoRA expand: K = r_i more steps per overlapping adapter -------------
    if (a.lora && seg.n > 0) {
        const bf16* __restrict__ E = static_cast<const bf16*>(a.E);
        const float* __restrict__ F = a.F;
        const int64_t tq1 = q0 + kBQ < T ? q0 + kBQ : T;
        uint8_t* se = smem;                 // [j][p] p-contiguous, up to 64 rows
        uint8_t* shi = smem + kPTile;       // [q][j] K-contiguous (hi terms)
        uint8_t* slo = shi + kKTile;        // [q][j] K-contiguous (lo terms)
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
                __syncthreads();
                for (int id = tid; id < 16 * nkk * 32; id += kThreads) {
                    const int j = id >> 5, pc = id & 31;
                    const int64_t p = p0 + pc * 8;
                    *reinterpret_cast<u32x4*>(se + j * kPRow + pc * 16) =
                        load16_or_zero(E + (rbase + jb + j) * Pdim + p, j < rc && p < Pdim);
                }
                const int nch = 2 * nkk;
                for (int id = tid; id < kBQ * nch; id += kThreads) {
                    const int q = id / nch, c = id - q * nch;
                    const int64_t t = q0 + q;
                    const bool in = t >= s0 && t < s1;
                    u16x8 hi, lo;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = c * 8 + e;
                        const float v = (in && j < rc) ? sc * Fi[(t - s0) * r + jb + j] : 0.0f;
                        bf16 h, o;
                        split_bf16(v, h, o);
                        hi[e] = __builtin_bit_cast(uint16_t, h);
                        lo[e] = __builtin_bit_cast(uint16_t, o);
                    }
                    *reinterpret_cast<u16x8*>(shi + kmaj(q, c)) = hi;
                    *reinterpret_cast<u16x8*>(slo + kmaj(q, c)) = lo;
                }
                __syncthreads();
                for (int kk = 0; kk < nkk; ++kk) {
                    bf16x8 fa[4], fh[4], fl[4];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) fa[mt] = pfrag_t(se, wp * 128 + mt * 32 + l32, 16 * kk + 8 * lh);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const int row = wq * 128 + nt * 32 + l32;
                        fh[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(shi + kmaj(row, 2 * kk + lh)));
                        fl[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(slo + kmaj(row, 2 * kk + lh)));
                    }
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 4; ++nt) {
                            acc[mt][nt] = mfma32x32x16(fa[mt], fh[nt], acc[mt][nt]);
                            acc[mt][nt] = mfma32x32x16(fa[mt], fl[nt], acc[mt][nt]);
                        }
                }
            }
        }
    }

    // ---- one rounding to bf16, token-major stores ----------------------------
    bf16* __restrict__ O = static_cast<bf16*>(a.O);
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

}  // namespace

hipError_t launch_gemm_bf16(bool p_kmajor, const GemmArgs& a, const SegTable& s, hipStream_t st) {
    const int64_t tq = (a.T + kBQ - 1) / kBQ, tp = (a.Pdim + kBP - 1) / kBP;
    const int64_t nwg = tq * tp;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg), block(kThreads);
    if (p_kmajor)
        hipLaunchKernelGGL(gemm_lora_bf16<true>, grid, block, 0, st, a, s);
    else
        hipLaunchKernelGGL(gemm_lora_bf16<false>, grid, block, 0, st, a, s);
    return hipGetLastError();
}

}  // namespace plora
