// lora_bf16.hip -- segment-indexed LoRA kernels that are not fused into the
// base GEMM (gfx950, bf16 in, fp32 out).
//
//   shrink   H_i = X[S_i] A_i          G_i = dY[S_i] B_i^T           (n_i x r_i)
//   wgrad    dA_i = s_i X[S_i]^T G_i   dB_i = s_i H_i^T dY[S_i]      (reduce over tokens)
//
// These are the down-projection and the two weight-gradient cases of the
// packed operators [PLoRA technical summary (gist.science, arXiv
// 2508.02932), 方法论 > 2. LoRA 执行引擎 > 算子设计: tile the concatenated
// LoRA tensors along tokens or hidden features, not rank; balance load across
// heterogeneous adapters], for the LoRA branch X A B scaled by alpha/r with
// gradients only for A and B [LLM+LoRA微调加速技术原理解析, 深入理解LoRA;
// LoRA加速集成方案, 四、工作原理 > 3. 反向传播阶段].
//
// Both stream one large activation (X or dY) once from HBM and are bound by
// HBM bandwidth (about r flop per byte).  Work is cut into equal token tiles
// per adapter (32 rows for shrink, a fixed token chunk x 256 features for the
// weight gradients), so adapters with 16x more tokens get 16x more work items
// rather than a 16x longer one.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <cstdlib>

namespace plora {
namespace {

// ---------------------------------------------------------------------------
// shrink: one wavefront per 32-token tile of one adapter; MFMA A = token rows,
// MFMA B = rank rows of the packed panel (r padded to 32 with zeros).  Lane l
// reads k = kb + 32*(l/32) + 8*s (s = 0..3) of its row, so the two half-waves
// together read each row's 128-byte block.  No LDS, no barriers.
// ---------------------------------------------------------------------------
template <int MAXJT>
__global__ __launch_bounds__(256) void shrink_bf16(ShrinkArgs a, SegTable seg, WorkMap m, int32_t units) {
    const int gw = (int)blockIdx.x * 4 + wave_id();
    if (gw >= units) return;
    const bf16* __restrict__ Q = static_cast<const bf16*>(a.Q);
    const bf16* __restrict__ P = static_cast<const bf16*>(a.P);
    const int64_t K = a.K;
    const int i = adapter_of_unit(m, seg.n, gw);
    const int64_t s0 = seg.off[i], s1 = seg.off[i + 1];
    const int64_t t0 = s0 + (int64_t)(gw - m.pre[i]) * kShrinkRows;
    const int nrows = (int)(s1 - t0 < kShrinkRows ? s1 - t0 : kShrinkRows);
    const int r = seg.rank[i];
    const int ntj = (r + 31) >> 5;
    const int l = lane_id(), l32 = l & 31, lh = l >> 5;

    const bf16* qrow = Q + (t0 + (l32 < nrows ? l32 : nrows - 1)) * K + 32 * lh;
    const bf16* prow[MAXJT];
    bool pv[MAXJT];
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) {
        const int j = jt * 32 + l32;
        pv[jt] = j < r;
        prow[jt] = P + ((int64_t)seg.roff[i] + (pv[jt] ? j : 0)) * K + 32 * lh;
    }

    f32x16 acc[MAXJT];
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) acc[jt] = f32x16{};

    // three register buffers of one 64-k block each: two blocks stay in flight
    // while one is multiplied (HBM streaming needs many loads outstanding)
    u32x4 xq[3][4], ap[3][MAXJT][4];
    auto load = [&](int buf, int64_t kb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bool ok = kb + 32 * lh + 8 * s < K;
            xq[buf][s] = load16_or_zero(qrow + kb + 8 * s, ok);
#pragma unroll
            for (int jt = 0; jt < MAXJT; ++jt)
                ap[buf][jt][s] = load16_or_zero(prow[jt] + kb + 8 * s, ok && pv[jt] && jt < ntj);
        }
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int jt = 0; jt < MAXJT; ++jt)
                if (jt < ntj) acc[jt] = mfma32x32x16(as_bf16x8(xq[buf][s]), as_bf16x8(ap[buf][jt][s]), acc[jt]);
    };
    // unrolled by three so every buffer index is a constant
    load(0, 0);
    if (64 < K) load(1, 64);
    for (int64_t kb = 0; kb < K; kb += 192) {
        if (kb + 128 < K) load(2, kb + 128);
        mma(0);
        if (kb + 64 >= K) break;
        if (kb + 192 < K) load(0, kb + 192);
        mma(1);
        if (kb + 128 >= K) break;
        if (kb + 256 < K) load(1, kb + 256);
        mma(2);
    }

    float* __restrict__ out = a.out + seg.hoff[i] + (t0 - s0) * r;
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) {
        const int j = jt * 32 + l32;
        if (jt >= ntj || j >= r) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + 4 * lh + (v & 3);
            if (row < nrows) out[(int64_t)row * r + j] = acc[jt][v];
        }
    }
}

// ---------------------------------------------------------------------------
// Pipelined shrink (K a multiple of 64): one workgroup of WPG waves per tile
// of 32*WPG tokens of one adapter, or per K slice of it (shrink_slices:
// adapters of a few tokens, whose single tile would otherwise walk all of K
// on one CU).  Each 64-k stage brings the tile's token rows of X/dY and the
// adapter's 32*MAXJT panel rows into LDS with LDS DMA (1 KiB per instruction
// = 8 rows x 128 B, whole cache lines), five stages deep so four stay in
// flight; wavefront w multiplies its 32 token rows against the panel.  Rows
// past the segment, the tensor or the rank read as zero (outside the buffer
// range).  A wave's MFMA sequence for its 32 rows is the same for any WPG,
// so both tile sizes give the same bits: WPG = 4 (128-token tiles) normally,
// WPG = 1 when the 128-token tiles would leave most CUs idle (a CU's own
// stream of loads, not its arithmetic, bounds this kernel).
// ---------------------------------------------------------------------------
constexpr int kShRowB = 128;                     // bytes per LDS row (64 bf16 of k)

// NP = 2 or 3: panels P, P1, P2 that share the input (the q/k/v or gate/up
// projections of one layer) in one pass over X; each panel's accumulators see
// the MFMA sequence of the single-panel kernel, so the bits match separate
// calls.  Stages: as many of the 160 KiB as fit, at most five.
template <int NP>
__device__ __forceinline__ const void* shrink_panel(const ShrinkArgs& a, int p) {
    return p == 0 ? a.P : p == 1 ? a.P1 : a.P2;
}
template <int NP>
__device__ __forceinline__ float* shrink_out(const ShrinkArgs& a, int p) {
    return p == 0 ? a.out : p == 1 ? a.out1 : a.out2;
}

template <int MAXJT, int WPG, int NP>
__global__ __launch_bounds__(64 * WPG, 1) void shrink_bf16_pipe(ShrinkArgs a, SegTable seg, WorkMap m) {
    constexpr int TR = 32 * WPG;                                // token rows per tile
    constexpr int kShX = TR * kShRowB;                          // token rows per stage
    constexpr int kShPan = 32 * MAXJT * kShRowB;                // one panel's rows per stage
    constexpr int kShStage = kShX + NP * kShPan;
    constexpr int NST = (163840 / kShStage) < 5 ? (163840 / kShStage) : 5;  // LDS stages
    static_assert(NST >= 3, "three stages at least");
    // one LDS object per stage buffer: the compiler tracks in-flight LDS DMA
    // per object, so reads of one stage wait only for that stage's loads (one
    // array for all stages made every LDS read wait for every load); buffers
    // past NST are never referenced and take no LDS
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh0[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh1[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh2[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh3[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh4[kShStage];
    uint8_t* const g_sh[5] = {g_sh0, g_sh1, g_sh2, g_sh3, g_sh4};
    const int unit = (int)blockIdx.x;
    const int64_t K = a.K;
    const int i = adapter_of_unit(m, seg.n, unit);
    const int64_t s0 = seg.off[i], s1 = seg.off[i + 1];
    const int nsl = shrink_slices(s1 - s0, seg.rank[i], K, a.scratch_row, a.split_all != 0);
    const int u = unit - m.pre[i], slice = u % nsl;
    const int64_t t0 = s0 + (int64_t)(u / nsl) * TR;
    const int nrows = (int)(s1 - t0 < TR ? s1 - t0 : TR);
    const int r = seg.rank[i];
    const int ntj = (r + 31) >> 5;
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.Q) + t0 * K), 0, (int)(nrows * K * 2), kRsrcWord3);
    __amdgpu_buffer_rsrc_t ra[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
        ra[p] = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const bf16*>(shrink_panel<NP>(a, p)) + (int64_t)seg.roff[i] * K), 0, (int)(r * K * 2),
            kRsrcWord3);
    // DMA block b: rows 8b .. 8b+7; lane l -> row 8b + l/8, physical chunk l%8
    const int r0 = l >> 3;
    const uint32_t lane_row = (uint32_t)(r0 * K * 2);
    // this work item's stages: [kt0, kt1) of the K / 64 (one K quarter per slice)
    const int KT = (int)(K / 64), kt0 = slice * KT / nsl, kt1 = (slice + 1) * KT / nsl;
    const int nq = shrink_quarters(K);
    // token tile: blocks 4w .. 4w+3 (32 rows per wave); each panel: 4*MAXJT
    // blocks, PB per wave
    constexpr int PB = 4 * MAXJT / WPG;
    auto issue = [&](uint8_t* buf, int kt) {
        const uint32_t oob = kt < kt1 ? 0u : 0x80000000u;
        const uint32_t kb = (uint32_t)kt * 128u + oob;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int blk = 4 * wu + j;
            const uint32_t vo = lane_row + (uint32_t)(((l & 7) ^ ((r0 ^ blk) & 7)) << 4) + (uint32_t)blk * (8u * K * 2) + kb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            // (a scalar copy: an array element passed straight to the LDS DMA
            // builtin leaves the kernel's host stub undefined)
            const __amdgpu_buffer_rsrc_t rp = ra[p];
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                const int blk = PB * wu + j;
                const uint32_t vo =
                    lane_row + (uint32_t)(((l & 7) ^ ((r0 ^ blk) & 7)) << 4) + (uint32_t)blk * (8u * K * 2) + kb;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_void*)(buf + kShX + p * kShPan + blk * 1024), 16, vo, 0,
                                                         0, 0);
            }
        }
    };
    f32x16 acc[NP][MAXJT], tot[NP][MAXJT];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int jt = 0; jt < MAXJT; ++jt) acc[p][jt] = tot[p][jt] = f32x16{};
    int q = nsl == 1 ? 0 : slice;  // the K quarter being accumulated
    // after stage kt: at the end of quarter q, total = q0 (or this slice's
    // quarter) or total + q, and the accumulator restarts from zero
    auto fold = [&](int kt) {
        if (kt + 1 != (q + 1) * KT / nq) return;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int jt = 0; jt < MAXJT; ++jt) {
                if (q == 0 || nsl > 1) tot[p][jt] = acc[p][jt];
                else tot[p][jt] += acc[p][jt];
                acc[p][jt] = f32x16{};
            }
        ++q;
    };
    auto compute = [&](const uint8_t* buf) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 xa = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kofs128(32 * w + l32, 2 * kk + lh)));
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int jt = 0; jt < MAXJT; ++jt) {
                    if (jt >= ntj) continue;
                    const bf16x8 pb = as_bf16x8(
                        *reinterpret_cast<const u32x4*>(buf + kShX + p * kShPan + kofs128(32 * jt + l32, 2 * kk + lh)));
                    acc[p][jt] = mfma32x32x16(xa, pb, acc[p][jt]);
                }
        }
    };
    constexpr int kPer = 4 + NP * PB;  // DMA loads per wave per stage
    // stage kt in cur; stages kt+1 .. kt+NST-2 in flight; refill prv (stage
    // kt-1, done) with stage kt+NST-1
    auto step = [&](uint8_t* cur, uint8_t* prv, int kt) {
        // stage kt landed, the next NST-2 may be in flight (or fewer, where
        // their loads outnumber what vmcnt can count)
        wait_vmcnt<((NST - 2) * kPer < 63 ? (NST - 2) * kPer : 63)>();
        lds_barrier();                   // and every wave is done with stage kt-1
        issue(prv, kt + NST - 1);
        compute(cur);
        fold(kt);
    };
#pragma unroll
    for (int b = 0; b < NST - 1; ++b) issue(g_sh[b], kt0 + b);
    // whole rotations in the loop, the rest after it: a conditional exit
    // inside the unrolled rotation makes the compiler lose track of which
    // buffer each in-flight load fills, and wait for all of them at the
    // first step of every rotation
    int kt = kt0;
    for (; kt + NST <= kt1; kt += NST) {
#pragma unroll
        for (int b = 0; b < NST; ++b) step(g_sh[b], g_sh[(b + NST - 1) % NST], kt + b);
    }
#pragma unroll
    for (int b = 0; b < NST - 1; ++b) {
        if (kt + b >= kt1) break;
        step(g_sh[b], g_sh[(b + NST - 1) % NST], kt + b);
    }
    wait_vmcnt<0>();

    // D[t][j]: lane holds rank column j, token rows 8*(v/4) + 4*(l/32) + v%4 of its wave's 32.
    // K slices (single panel only): slice s of the adapter's [n_i][r_i] block
    // goes to its own rows of the scratch activation, s * n_i * r_i floats in
    // (shrink_slice_sum adds them)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        float* __restrict__ out =
            (nsl == 1 ? shrink_out<NP>(a, p) + seg.hoff[i]
                      : reinterpret_cast<float*>(static_cast<uint8_t*>(a.scratch) + s0 * a.scratch_row) +
                            (int64_t)slice * (s1 - s0) * r) +
            (t0 - s0) * r;
#pragma unroll
        for (int jt = 0; jt < MAXJT; ++jt) {
            const int j = jt * 32 + l32;
            if (jt >= ntj || j >= r) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 32 * w + 8 * (v >> 2) + 4 * lh + (v & 3);
                if (row < nrows) out[(int64_t)row * r + j] = tot[p][jt][v];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// wgrad: one workgroup per (adapter token chunk, 256 features).  MFMA
// A = rank rows (from fp32 H/G, s folded in later, split into bf16 hi + lo),
// MFMA B = feature columns of X/dY, K = tokens, 32 tokens per stage.
// ---------------------------------------------------------------------------
constexpr int kWgTok = 32;                   // tokens per stage
constexpr int kWgCols = 256;                 // features per workgroup
constexpr int kQRow = kWgCols * 2 + 16;      // LDS row of the activation tile (padded)
constexpr int kQTile = kWgTok * kQRow;       // 16896 B
constexpr int kFRow = kWgTok * 2;            // LDS row of the H/G tile: 32 tokens bf16
constexpr int kFTile = 128 * kFRow;          // up to 128 rank rows: 8 KiB
constexpr int kWgStage = kQTile + 2 * kFTile;

__device__ __forceinline__ int fofs(int j, int c) { return j * kFRow + ((c ^ ((j >> 1) & 3)) << 4); }

template <int MAXJT>
__global__ __launch_bounds__(256) void wgrad_bf16(WgradArgs a, SegTable seg, WgradPlan plan) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kWgStage];
    const bf16* __restrict__ Q = static_cast<const bf16*>(a.Q);
    const int64_t D = a.D;
    const int w = (int)blockIdx.x;
    const int64_t c0 = (int64_t)blockIdx.y * kWgCols;
    const int i = adapter_of_unit(plan.chunks, seg.n, w);
    const int u = w - plan.chunks.pre[i];
    const int nchunks = plan.chunks.pre[i + 1] - plan.chunks.pre[i];
    const int64_t s0 = seg.off[i], s1 = seg.off[i + 1];
    const int64_t ta = s0 + (int64_t)u * plan.chunk_tokens;
    const int64_t tb = ta + plan.chunk_tokens < s1 ? ta + plan.chunk_tokens : s1;
    const int r = seg.rank[i];
    const int ntj = (r + 31) >> 5;
    const int rp = ntj * 32;
    const float* __restrict__ Fi = a.F + seg.hoff[i];

    const int tid = (int)threadIdx.x, l = lane_id(), wv = wave_id();
    const int l32 = l & 31, lh = l >> 5;

    f32x16 acc[MAXJT][2];
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) acc[jt][0] = acc[jt][1] = f32x16{};

    // staging registers: 4 activation chunks + up to 2 H/G tasks per thread
    u32x4 qv[4];
    u16x8 fh[2], fl[2];
    const int q_row = tid >> 5, q_pc = tid & 31;
    auto gload = [&](int64_t tt) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int64_t t = tt + it * 8 + q_row;
            const int64_t c = c0 + q_pc * 8;
            qv[it] = load16_or_zero(Q + t * D + c, t < tb && c < D);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int task = tid + it * 256;      // (rank row j, 8-token chunk tc)
            const int j = task >> 2, tc = task & 3;
            u16x8 h, o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t t = tt + tc * 8 + e;
                const float v = (j < r && t < tb) ? Fi[(t - s0) * r + j] : 0.0f;
                bf16 hb, lb;
                split_bf16(v, hb, lb);
                h[e] = __builtin_bit_cast(uint16_t, hb);
                o[e] = __builtin_bit_cast(uint16_t, lb);
            }
            fh[it] = h;
            fl[it] = o;
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* sq = smem + buf * kWgStage;
        uint8_t* sh = sq + kQTile;
        uint8_t* sl = sh + kFTile;
#pragma unroll
        for (int it = 0; it < 4; ++it) *reinterpret_cast<u32x4*>(sq + (it * 8 + q_row) * kQRow + q_pc * 16) = qv[it];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int task = tid + it * 256;
            const int j = task >> 2, tc = task & 3;
            if (j < rp) {
                *reinterpret_cast<u16x8*>(sh + fofs(j, tc)) = fh[it];
                *reinterpret_cast<u16x8*>(sl + fofs(j, tc)) = fl[it];
            }
        }
    };
    auto compute = [&](int buf) {
        const uint8_t* sq = smem + buf * kWgStage;
        const uint8_t* sh = sq + kQTile;
        const uint8_t* sl = sh + kFTile;
#pragma unroll
        for (int kk = 0; kk < kWgTok / 16; ++kk) {
            bf16x8 qf[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int c = wv * 64 + ct * 32 + l32;
                u16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = *reinterpret_cast<const uint16_t*>(sq + (16 * kk + 8 * lh + e) * kQRow + c * 2);
                qf[ct] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int jt = 0; jt < MAXJT; ++jt) {
                if (jt >= ntj) continue;
                const int j = jt * 32 + l32;
                const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4*>(sh + fofs(j, 2 * kk + lh)));
                const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(sl + fofs(j, 2 * kk + lh)));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    acc[jt][ct] = mfma32x32x16(ah, qf[ct], acc[jt][ct]);
                    acc[jt][ct] = mfma32x32x16(al, qf[ct], acc[jt][ct]);
                }
            }
        }
    };

    const int nst = (int)((tb - ta + kWgTok - 1) / kWgTok);
    gload(ta);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int cur = st & 1;
        if (st + 1 < nst) gload(ta + (int64_t)(st + 1) * kWgTok);
        compute(cur);
        if (st + 1 < nst) lstore(cur ^ 1);
        __syncthreads();
    }

    // D[j][c]: lane holds feature column c, rank rows 8*(v/4) + 4*(l/32) + v%4.
    const bool direct = nchunks == 1;
    const float sc = seg.scale[i];
    float* __restrict__ dst = direct ? a.out + (int64_t)seg.roff[i] * D
                                     : a.part + plan.part_off[i] + (int64_t)u * r * D;
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) {
        if (jt >= ntj) continue;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int64_t c = c0 + wv * 64 + ct * 32 + l32;
            if (c >= D) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = jt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                if (j < r) {
                    float val = direct ? sc * acc[jt][ct][v] : acc[jt][ct][v];
                    if (direct && a.accumulate) val += dst[(int64_t)j * D + c];
                    dst[(int64_t)j * D + c] = val;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pipelined weight gradient.
//
// wgrad_prep writes the fp32 H_i (or G_i) block [n_i][r_i] transposed as two
// bf16 arrays hi = bf16(v), lo = bf16(v - hi), row j of length pad64(n_i)
// (zero-padded), so the main kernel can stream it as whole 128-byte lines.
// One workgroup per (64-token block, adapter, side): the block's 64 rows of
// r_i values are contiguous in H, so they are read whole, transposed in LDS,
// and leave as r_i pieces of 128 bytes per array.  The sides (H and G of one
// call, or the G's of a shared-input pass) share one launch.
//
// wgrad_bf16_pipe: one workgroup per (adapter token chunk, 256 features), the
// feature tiles fastest so the workgroups running together read whole rows.
// Each 64-token stage brings the chunk's X/dY rows (64 x 512 B, read
// transposed: MFMA B = features, K = tokens) and the adapter's hi/lo rank
// panels (32*MAXJT rows x 128 B each, MFMA A = rank rows) into LDS with LDS
// DMA; three stages, two in flight (ranks up to 64; larger ranks use the
// register-staged kernel above).  Tokens past the chunk read as zero
// (outside the buffer range or zero padding).
// ---------------------------------------------------------------------------
struct PrepSides {
    const float* F[3];
    bf16* hi[3];
    bf16* lo[3];
};

__global__ __launch_bounds__(256) void wgrad_prep(PrepSides ps, SegTable seg, WgradPlan plan) {
    const int z = (int)blockIdx.z;
    const float* const F = z == 0 ? ps.F[0] : z == 1 ? ps.F[1] : ps.F[2];
    bf16* const hi = z == 0 ? ps.hi[0] : z == 1 ? ps.hi[1] : ps.hi[2];
    bf16* const lo = z == 0 ? ps.lo[0] : z == 1 ? ps.lo[1] : ps.lo[2];
    const int i = (int)blockIdx.y;
    const int64_t n = seg.off[i + 1] - seg.off[i];
    const int64_t u0 = (int64_t)blockIdx.x * 64;
    if (u0 >= n) return;  // (u0 is a multiple of 64: the block holding token n-1 also writes the padding)
    const int r = seg.rank[i];  // <= 64 on this path
    const int64_t np = pad64(n);
    __shared__ float tile[64 * 65];  // [token][rank], rows of 65 floats: the column reads below hit 64 banks
    const float* __restrict__ Fi = F + seg.hoff[i] + u0 * r;
    const int valid = (int)((n - u0 < 64 ? n - u0 : 64) * r);
    for (int e = (int)threadIdx.x; e < 64 * r; e += 256) {
        const int t = e / r, j = e - t * r;
        tile[t * 65 + j] = e < valid ? Fi[e] : 0.0f;
    }
    __syncthreads();
    // thread task e: rank row j = e / 8, tokens u0 + 8q .. +7 (q = e % 8): 16 bytes per array
    for (int e = (int)threadIdx.x; e < 8 * r; e += 256) {
        const int j = e >> 3, q = e & 7;
        u16x8 h8, l8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            bf16 hb, lb;
            split_bf16(tile[(8 * q + k) * 65 + j], hb, lb);
            h8[k] = __builtin_bit_cast(uint16_t, hb);
            l8[k] = __builtin_bit_cast(uint16_t, lb);
        }
        const int64_t o = plan.ft_off[i] + (int64_t)j * np + u0 + 8 * q;
        *reinterpret_cast<u16x8*>(hi + o) = h8;
        *reinterpret_cast<u16x8*>(lo + o) = l8;
    }
}

// NCT = 32-feature MFMA column tiles per wave: workgroups of 128 * NCT
// features (NCT = 2: 256, NCT = 1: 128, for grids too small to fill the CUs;
// an element's token sum does not depend on the width, so neither do the bits)
template <int NCT>
struct WqTile {
    static constexpr int kCols = 128 * NCT;          // features per workgroup
    static constexpr int kRowB = 2 * kCols;          // bytes per token row of the tile
    static constexpr int kBytes = 64 * kRowB;        // 64 tokens
    static constexpr int kRowsPerBlk = 1024 / kRowB; // 2 or 4 token rows per 1 KiB DMA block
    static constexpr int kLanesPerRow = 64 / kRowsPerBlk;
    static constexpr int kBlkPerWave = 64 / kRowsPerBlk / 4;
    static constexpr int kStages = NCT == 2 ? 3 : 4; // LDS stages (kStages - 1 in flight)
};

// NP = 2 or 3: factors F, F1, F2 of projections that share the input (dA of
// the q/k/v or gate/up projections) against one pass over X; each output
// element sees the MFMA sequence of the single-panel kernel (same bits).
// With NP panels a 64-token stage would leave room for two stages only, so
// these stages hold 32 tokens (rank rows of 64 bytes per hi / lo panel, 16
// rows per DMA block) and four of them fit (three in flight); the k-steps of
// 16 tokens and their order stay the same.
__device__ __forceinline__ float* wgrad_out(const WgradArgs& a, int p) {
    return p == 0 ? a.out : p == 1 ? a.out1 : a.out2;
}

template <int MAXJT, int NCT, int NP>
__global__ __launch_bounds__(256, 1) void wgrad_bf16_pipe(WgradArgs a, SegTable seg, WgradPlan plan, const bf16* fhi,
                                                          const bf16* flo) {
    using WT = WqTile<NCT>;
    constexpr int TS = NP > 1 ? 32 : 64;                     // tokens per stage
    constexpr int kXBytes = TS * WT::kRowB;                  // activation tile
    constexpr int kXBlkPerWave = TS / WT::kRowsPerBlk / 4;   // its DMA blocks per wave
    constexpr int kFRow = 2 * TS;                            // bytes of a rank row in one stage
    constexpr int kF = 32 * MAXJT * kFRow;                   // one of the hi / lo panels
    constexpr int kFBlkPerWave = NP * 2 * (kF / 1024) / 4;   // hi / lo DMA blocks per wave
    constexpr int kStage = kXBytes + NP * 2 * kF;
    constexpr int kMaxSt = TS == 64 ? WT::kStages : 4;
    constexpr int NST = (163840 / kStage) < kMaxSt ? (163840 / kStage) : kMaxSt;
    static_assert(NST >= 3, "three stages at least");
    static_assert(NP * 2 * (kF / 1024) % 4 == 0 && MAXJT <= 2, "whole DMA blocks per wave");
    // one LDS object per stage buffer (see the shrink); unreferenced ones take no LDS
    __shared__ __attribute__((aligned(1024))) uint8_t g_b0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_b1[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_b2[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_b3[kStage];
    uint8_t* const g_b[4] = {g_b0, g_b1, g_b2, g_b3};
    const int64_t D = a.D;
    const int w = (int)blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * WT::kCols;  // (feature tiles fastest: a chunk's rows are read whole)
    const int i = adapter_of_unit(plan.chunks, seg.n, w);
    const int u = w - plan.chunks.pre[i];
    const int nchunks = plan.chunks.pre[i + 1] - plan.chunks.pre[i];
    const int64_t s0 = seg.off[i], s1 = seg.off[i + 1];
    const int TK = plan.chunk_tokens;
    const int64_t ta = s0 + (int64_t)u * TK;
    const int64_t tb = ta + TK < s1 ? ta + TK : s1;
    const int64_t np = pad64(s1 - s0);
    const int r = seg.rank[i];
    const int ntj = (r + 31) >> 5;
    const int l = lane_id(), wv = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(wv);

    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.Q) + ta * D + c0), 0, (int)(((tb - ta - 1) * D + (D - c0)) * 2), kRsrcWord3);
    __amdgpu_buffer_rsrc_t rh[NP], rl[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int64_t fo = p * a.ft_stride + plan.ft_off[i] + (int64_t)u * TK;
        rh[p] = __builtin_amdgcn_make_buffer_rsrc((void*)(fhi + fo), 0, (int)((r * np - (int64_t)u * TK) * 2), kRsrcWord3);
        rl[p] = __builtin_amdgcn_make_buffer_rsrc((void*)(flo + fo), 0, (int)((r * np - (int64_t)u * TK) * 2), kRsrcWord3);
    }
    // activation tile: block b = kRowsPerBlk token rows of kRowB bytes; lane l
    // -> row RPB*b + l/(lanes per row), physical chunk l % (lanes per row),
    // holding logical chunk physical ^ 4 (row % 4) (the layout pfrag_tr reads).
    // With 2-row blocks the row's parity within 4 alternates with the block.
    const int tr = l / WT::kLanesPerRow, tc = l % WT::kLanesPerRow;
    const uint32_t q_off0 = (uint32_t)(tr * D * 2) + (uint32_t)((tc ^ (tr << 2)) << 4);
    const uint32_t q_off1 = (uint32_t)(tr * D * 2) + (uint32_t)((tc ^ ((2 + tr) << 2)) << 4);
    // rank panels: block b = 8 rank rows x 128 B; lane l -> row 8b + l/8, physical chunk l%8
    const int r0 = l >> 3;
    const uint32_t f_row = (uint32_t)(r0 * np * 2);
    const int nst = (int)((tb - ta + TS - 1) / TS);
    // 32-token stages: rank panel blocks of 16 rows x 64 B; lane l -> row 16b + l/4,
    // physical chunk l%4, holding logical chunk (l%4) ^ (row/4 % 4) (kofs64)
    const int r0q = l >> 2;
    auto issue = [&](uint8_t* buf, int st) {
        const uint32_t oob = st < nst ? 0u : 0x80000000u;
#pragma unroll
        for (int j = 0; j < kXBlkPerWave; ++j) {
            const int blk = kXBlkPerWave * wu + j;
            const uint32_t vo = ((WT::kRowsPerBlk == 2 && (j & 1)) ? q_off1 : q_off0) +
                                (uint32_t)blk * (uint32_t)(WT::kRowsPerBlk * D * 2) + (uint32_t)st * (uint32_t)(TS * D * 2) +
                                oob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
        if constexpr (TS == 64) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const __amdgpu_buffer_rsrc_t rhp = rh[p], rlp = rl[p];  // (scalar copies, as in the shrink)
#pragma unroll
                for (int j = 0; j < MAXJT; ++j) {
                    const int blk = MAXJT * wu + j;
                    const uint32_t vo = f_row + (uint32_t)(((l & 7) ^ ((r0 ^ blk) & 7)) << 4) +
                                        (uint32_t)blk * (uint32_t)(8 * np * 2) + (uint32_t)st * 128u + oob;
                    uint8_t* fb = buf + kXBytes + p * 2 * kF;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rhp, (lds_void*)(fb + blk * 1024), 16, vo, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rlp, (lds_void*)(fb + kF + blk * 1024), 16, vo, 0, 0, 0);
                }
            }
        } else {
            // each hi / lo panel is 2 * MAXJT blocks; the panel index is fixed by
            // j (unrolled), the block (and with MAXJT = 1 the half) by the wave
#pragma unroll
            for (int j = 0; j < kFBlkPerWave; ++j) {
                const int pp = MAXJT == 2 ? j >> 1 : j;
                const int hl = MAXJT == 2 ? (j & 1) : (wu >> 1);
                const int b = MAXJT == 2 ? wu : (wu & 1);
                const int row = 16 * b + r0q;
                const uint32_t vo = (uint32_t)(row * np * 2) + (uint32_t)(((l & 3) ^ ((row >> 2) & 3)) << 4) +
                                    (uint32_t)st * 64u + oob;
                const __amdgpu_buffer_rsrc_t rhp = rh[pp], rlp = rl[pp];
                const __amdgpu_buffer_rsrc_t rf = hl ? rlp : rhp;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rf, (lds_void*)(buf + kXBytes + (2 * pp + hl) * kF + b * 1024), 16,
                                                         vo, 0, 0, 0);
            }
        }
    };
    // logical chunk c of rank row j in a 64-byte-row panel (32-token stages)
    auto kofs64 = [](int j, int c) { return j * 64 + ((c ^ ((j >> 2) & 3)) << 4); };
    f32x16 acc[NP][MAXJT][NCT];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int jt = 0; jt < MAXJT; ++jt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[p][jt][ct] = f32x16{};
    auto compute = [&](const uint8_t* buf) {
#pragma unroll
        for (int kk = 0; kk < TS / 16; ++kk) {
            bf16x8 qf[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) qf[ct] = pfrag_tr<WT::kRowB>(buf, 32 * NCT * wv + 32 * ct, 16 * kk);
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int jt = 0; jt < MAXJT; ++jt) {
                    if (jt >= ntj) continue;
                    const int row = 32 * jt + l32;
                    const uint8_t* fb = buf + kXBytes + p * 2 * kF;
                    const int fo = TS == 64 ? kofs128(row, 2 * kk + lh) : kofs64(row, 2 * kk + lh);
                    const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4*>(fb + fo));
                    const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(fb + kF + fo));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        acc[p][jt][ct] = mfma32x32x16(ah, qf[ct], acc[p][jt][ct]);
                        acc[p][jt][ct] = mfma32x32x16(al, qf[ct], acc[p][jt][ct]);
                    }
                }
        }
    };
    constexpr int kPer = kXBlkPerWave + (TS == 64 ? 2 * NP * MAXJT : kFBlkPerWave);  // DMA loads per wave per stage
    constexpr int kAhead = NST - 1;                          // stages in flight
    constexpr int kWait = (kAhead - 1) * kPer < 63 ? (kAhead - 1) * kPer : 63;
    auto step = [&](uint8_t* cur, uint8_t* prv, int st) {
        wait_vmcnt<kWait>();  // stage st landed, the next kAhead-1 may be in flight
        lds_barrier();        // every wave is done with stage st-1
        issue(prv, st + kAhead);
        compute(cur);
    };
#pragma unroll
    for (int b = 0; b < kAhead; ++b) issue(g_b[b], b);
    // (whole rotations in the loop, as in the shrink)
    int st = 0;
    for (; st + NST <= nst; st += NST) {
#pragma unroll
        for (int b = 0; b < NST; ++b) step(g_b[b], g_b[(b + NST - 1) % NST], st + b);
    }
#pragma unroll
    for (int b = 0; b < NST - 1; ++b) {
        if (st + b >= nst) break;
        step(g_b[b], g_b[(b + NST - 1) % NST], st + b);
    }
    wait_vmcnt<0>();

    // D[j][c]: lane holds feature column c, rank rows 8*(v/4) + 4*(l/32) + v%4.
    const bool direct = nchunks == 1;
    const float sc = seg.scale[i];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        float* __restrict__ dst = direct ? wgrad_out(a, p) + (int64_t)seg.roff[i] * D
                                         : a.part + p * a.part_stride + plan.part_off[i] + (int64_t)u * r * D;
#pragma unroll
        for (int jt = 0; jt < MAXJT; ++jt) {
            if (jt >= ntj) continue;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int64_t c = c0 + 32 * NCT * wv + ct * 32 + l32;
                if (c >= D) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = jt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    if (j < r) {
                        float val = direct ? sc * acc[p][jt][ct][v] : acc[p][jt][ct][v];
                        if (direct && a.accumulate) val += dst[(int64_t)j * D + c];
                        dst[(int64_t)j * D + c] = val;
                    }
                }
            }
        }
    }
}

// out rows of adapters whose tokens span 0 or >= 2 chunks:
// out = s_i * sum_u partial[u] in chunk order (0 for an empty adapter), or
// out += that when accumulating (an empty adapter is then left alone).
// Side z (blockIdx.z) is one weight-gradient pass of the call (dB, dA, or a
// panel of a shared-input pass); only the per-adapter fields the reduction
// reads travel as kernel arguments.
struct ReduceSide {
    float* out;
    const float* part;
    int64_t D;
    int64_t part_off[kMaxN + 1];
    int32_t pre[kMaxN + 1];
};
struct ReduceArgs {
    ReduceSide side[3];
    int32_t rank[kMaxN];
    int32_t roff[kMaxN];
    float scale[kMaxN];
    int32_t accumulate;
};
static_assert(sizeof(ReduceArgs) <= 4096, "kernel arguments");

__global__ __launch_bounds__(256) void wgrad_reduce(ReduceArgs ra) {
    const int i = (int)blockIdx.y;
    const ReduceSide& sd = ra.side[blockIdx.z];
    const int nch = sd.pre[i + 1] - sd.pre[i];
    if (nch == 1 || (nch == 0 && ra.accumulate)) return;
    const int64_t n = (int64_t)ra.rank[i] * sd.D;  // multiple of 8
    const float sc = ra.scale[i];
    float* __restrict__ out = sd.out + (int64_t)ra.roff[i] * sd.D;
    const float* __restrict__ part = sd.part + sd.part_off[i];
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < n; e += (int64_t)gridDim.x * 1024) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        for (int u = 0; u < nch; ++u) s += *reinterpret_cast<const f32x4*>(part + (int64_t)u * n + e);
        f32x4 o = s * sc;
        if (ra.accumulate) o += *reinterpret_cast<const f32x4*>(out + e);
        *reinterpret_cast<f32x4*>(out + e) = o;
    }
}

// Sum of the K slices of the shrink (fixed order 0, 1, ...) into H / G: one
// workgroup per adapter; adapters that were not sliced return at once.
__global__ __launch_bounds__(256) void shrink_slice_sum(ShrinkArgs a, SegTable seg) {
    const int i = (int)blockIdx.y;
    const int64_t n = seg.off[i + 1] - seg.off[i];
    const int r = seg.rank[i];
    const int nsl = shrink_slices(n, r, a.K, a.scratch_row, a.split_all != 0);
    if (nsl == 1) return;
    const int64_t ne = n * r;
    const float* __restrict__ part =
        reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.scratch) + seg.off[i] * a.scratch_row);
    float* __restrict__ out = a.out + seg.hoff[i];
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < ne; e += (int64_t)gridDim.x * 256) {
        float v = part[e];
        for (int sl = 1; sl < nsl; ++sl) v += part[sl * ne + e];
        out[e] = v;
    }
}

}  // namespace

namespace {

// Panel p of a shared-input call as a single-panel call.
ShrinkArgs shrink_single(const ShrinkArgs& a, int p) {
    ShrinkArgs o = a;
    o.P = p == 0 ? a.P : p == 1 ? a.P1 : a.P2;
    o.out = p == 0 ? a.out : p == 1 ? a.out1 : a.out2;
    o.P1 = o.P2 = nullptr;
    o.out1 = o.out2 = nullptr;
    o.np = 1;
    return o;
}
WgradArgs wgrad_single(const WgradArgs& a, int p) {
    WgradArgs o = a;
    o.F = p == 0 ? a.F : p == 1 ? a.F1 : a.F2;
    o.out = p == 0 ? a.out : p == 1 ? a.out1 : a.out2;
    o.part = a.part ? a.part + p * a.part_stride : nullptr;
    o.F1 = o.F2 = nullptr;
    o.out1 = o.out2 = nullptr;
    o.np = 1;
    return o;
}

// (kernel templates are launched from non-template code: a kernel template
// first referenced inside a function template left its host stub undefined)
#define PLORA_SHRINK_NP(MAXJT, WPG)                                                                          \
    do {                                                                                                    \
        if (np == 3)                                                                                        \
            hipLaunchKernelGGL((shrink_bf16_pipe<MAXJT, WPG, 3>), grid, block, 0, st, a, s, mp);              \
        else if (np == 2)                                                                                   \
            hipLaunchKernelGGL((shrink_bf16_pipe<MAXJT, WPG, 2>), grid, block, 0, st, a, s, mp);              \
        else                                                                                                \
            hipLaunchKernelGGL((shrink_bf16_pipe<MAXJT, WPG, 1>), grid, block, 0, st, a, s, mp);              \
    } while (0)

}  // namespace

hipError_t launch_shrink_bf16(const ShrinkArgs& a_in, const SegTable& s, const WorkMap& m, int32_t units,
                              hipStream_t st) {
    if (units <= 0) return hipSuccess;
    const int np = a_in.np > 1 ? a_in.np : 1;
    const bool pipe = a_in.K % 64 == 0 && (int64_t)kShrinkTileRows * a_in.K * 2 < (int64_t(1) << 31) &&
                      (int64_t)s.roff[s.n] * a_in.K * 2 < (int64_t(1) << 31);
    if (np > 1 && (!pipe || s.rmax > 64)) {
        // shared input with ranks beyond 64 (or no pipelined shape): one pass per panel
        for (int p = 0; p < np; ++p) {
            const hipError_t e = launch_shrink_bf16(shrink_single(a_in, p), s, m, units, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (pipe) {
        ShrinkArgs a = a_in;
        if (!a.scratch || np > 1) a.scratch_row = 0;  // (shared input: no K slices; the K order is the same)
        WorkMap mp;
        bool split = false;
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        // K slices for every adapter when the 128-token tiles number at most a
        // quarter of the CUs (a CU's own stream of loads bounds this kernel, so
        // few work items leave most of HBM's bandwidth unused; with more, the
        // one-wave tiles below spread better); the K order is the same either
        // way.  PLORA_SHRINK_SPLIT=0 or 1 forces the choice.
        a.split_all = 0;
        int32_t items = build_shrink_pipe_map(s, &mp, a.K, a.scratch_row, &split, kShrinkTileRows, false);
        const char* fsplit = getenv("PLORA_SHRINK_SPLIT");
        const int fs = fsplit ? atoi(fsplit) : -1;
        if (a.scratch_row > 0 && (fs == 1 || (fs != 0 && 4 * (int64_t)items <= cus))) {
            a.split_all = 1;
            items = build_shrink_pipe_map(s, &mp, a.K, a.scratch_row, &split, kShrinkTileRows, true);
        }
        // 32-token tiles (one wave each) when the 128-token grid fills at most
        // half of the CUs: four times the workgroups, same results
        // (PLORA_SHRINK_TILE_ROWS=32 or 128 forces the tile size)
        const char* force = getenv("PLORA_SHRINK_TILE_ROWS");
        const int fr = force ? atoi(force) : 0;
        const bool small = fr == 32 || (fr != 128 && 2 * (int64_t)items <= cus);
        if (small) items = build_shrink_pipe_map(s, &mp, a.K, a.scratch_row, &split, 32, a.split_all != 0);
        const dim3 grid((unsigned)items), block(small ? 64 : 256);
        switch (((s.rmax + 31) / 32) * 2 + (small ? 1 : 0)) {
            case 2: PLORA_SHRINK_NP(1, 4); break;
            case 3: PLORA_SHRINK_NP(1, 1); break;
            case 4: PLORA_SHRINK_NP(2, 4); break;
            case 5: PLORA_SHRINK_NP(2, 1); break;
            case 6: hipLaunchKernelGGL((shrink_bf16_pipe<3, 4, 1>), grid, block, 0, st, a, s, mp); break;
            case 7: hipLaunchKernelGGL((shrink_bf16_pipe<3, 1, 1>), grid, block, 0, st, a, s, mp); break;
            case 8: hipLaunchKernelGGL((shrink_bf16_pipe<4, 4, 1>), grid, block, 0, st, a, s, mp); break;
            default: hipLaunchKernelGGL((shrink_bf16_pipe<4, 1, 1>), grid, block, 0, st, a, s, mp); break;
        }
        if (split) {
            int64_t ne = 0;  // the largest adapter's n_i * r_i: 1024 values per workgroup (at most 64 per adapter)
            for (int i = 0; i < s.n; ++i) ne = std::max(ne, (int64_t)(s.off[i + 1] - s.off[i]) * s.rank[i]);
            const int64_t bx = std::min<int64_t>((ne + 1023) / 1024, 64);
            hipLaunchKernelGGL(shrink_slice_sum, dim3((unsigned)bx, (unsigned)s.n), dim3(256), 0, st, a, s);
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((units + 3) / 4)), block(256);
    const int jt = (s.rmax + 31) / 32;
    switch (jt) {
        case 1: hipLaunchKernelGGL(shrink_bf16<1>, grid, block, 0, st, a_in, s, m, units); break;
        case 2: hipLaunchKernelGGL(shrink_bf16<2>, grid, block, 0, st, a_in, s, m, units); break;
        case 3: hipLaunchKernelGGL(shrink_bf16<3>, grid, block, 0, st, a_in, s, m, units); break;
        default: hipLaunchKernelGGL(shrink_bf16<4>, grid, block, 0, st, a_in, s, m, units); break;
    }
    return hipGetLastError();
}

hipError_t launch_wgrad_bf16(const WgradArgs& a, const SegTable& s, const WgradPlan& p, hipStream_t st) {
    const int32_t units = p.chunks.pre[s.n];
    if (units <= 0) return hipSuccess;
    if (a.np > 1) {
        for (int q = 0; q < a.np; ++q) {
            const hipError_t e = launch_wgrad_bf16(wgrad_single(a, q), s, p, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const dim3 grid((unsigned)units, (unsigned)p.col_tiles), block(256);
    const int jt = (s.rmax + 31) / 32;
    switch (jt) {
        case 1: hipLaunchKernelGGL(wgrad_bf16<1>, grid, block, 0, st, a, s, p); break;
        case 2: hipLaunchKernelGGL(wgrad_bf16<2>, grid, block, 0, st, a, s, p); break;
        case 3: hipLaunchKernelGGL(wgrad_bf16<3>, grid, block, 0, st, a, s, p); break;
        default: hipLaunchKernelGGL(wgrad_bf16<4>, grid, block, 0, st, a, s, p); break;
    }
    return hipGetLastError();
}

#define PLORA_WGRAD_NP(MAXJT, NCT)                                                                        \
    do {                                                                                                \
        if (np == 3)                                                                                    \
            hipLaunchKernelGGL((wgrad_bf16_pipe<MAXJT, NCT, 3>), grid, block, 0, st, a, s, p, fhi, flo);  \
        else if (np == 2)                                                                               \
            hipLaunchKernelGGL((wgrad_bf16_pipe<MAXJT, NCT, 2>), grid, block, 0, st, a, s, p, fhi, flo);  \
        else                                                                                            \
            hipLaunchKernelGGL((wgrad_bf16_pipe<MAXJT, NCT, 1>), grid, block, 0, st, a, s, p, fhi, flo);  \
    } while (0)

bool wgrad_pipe_ok(const WgradArgs& a, const SegTable& s, const WgradPlan& p, const bf16* fhi) {
    // (the pipelined grid puts the chunks in y: at most 65535 of them)
    return s.rmax <= 64 && fhi != nullptr && (int64_t)p.chunk_tokens * a.D * 2 < (int64_t(1) << 31) &&
           p.chunks.pre[s.n] <= 65535;
}

hipError_t launch_wgrad_prep(int nside, const float* const* F, bf16* const* hi, bf16* const* lo, const SegTable& s,
                             const WgradPlan& p, hipStream_t st) {
    if (nside < 1 || nside > 3) return hipErrorInvalidValue;
    int64_t maxnp = 0;
    for (int i = 0; i < s.n; ++i) maxnp = maxnp > pad64(s.off[i + 1] - s.off[i]) ? maxnp : pad64(s.off[i + 1] - s.off[i]);
    if (maxnp == 0 || s.roff[s.n] == 0) return hipSuccess;
    PrepSides ps{};
    for (int k = 0; k < nside; ++k) {
        ps.F[k] = F[k];
        ps.hi[k] = hi[k];
        ps.lo[k] = lo[k];
    }
    // (hi/lo offsets are multiples of 64 elements and the arrays start 16-byte aligned)
    hipLaunchKernelGGL(wgrad_prep, dim3((unsigned)(maxnp / 64), (unsigned)s.n, (unsigned)nside), dim3(256), 0, st, ps,
                       s, p);
    return hipGetLastError();
}

hipError_t launch_wgrad_bf16_pipe(const WgradArgs& a, const SegTable& s, const WgradPlan& p, const bf16* fhi,
                                  const bf16* flo, hipStream_t st) {
    const int np = a.np > 1 ? a.np : 1;
    const int32_t units = p.chunks.pre[s.n];
    if (units <= 0) return hipSuccess;
    // 128-feature workgroups when the 256-feature grid would not give every CU
    // two (PLORA_WGRAD_COLS=128 or 256 forces the width; same results)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const char* force = getenv("PLORA_WGRAD_COLS");
    const int fc = force ? atoi(force) : 0;
    const bool narrow = fc == 128 || (fc != 256 && (int64_t)p.col_tiles * units < 2 * (int64_t)cus);
    const dim3 grid((unsigned)(narrow ? (a.D + 127) / 128 : p.col_tiles), (unsigned)units), block(256);
    if (s.rmax <= 32 && narrow)
        PLORA_WGRAD_NP(1, 1);
    else if (s.rmax <= 32)
        PLORA_WGRAD_NP(1, 2);
    else if (narrow)
        PLORA_WGRAD_NP(2, 1);
    else
        PLORA_WGRAD_NP(2, 2);
    return hipGetLastError();
}

hipError_t launch_wgrad_reduce(int nside, const WgradArgs* const* a, const WgradPlan* const* p, const SegTable& s,
                               hipStream_t st) {
    if (nside < 0 || nside > 3) return hipErrorInvalidValue;
    ReduceArgs ra{};
    int z = 0;
    int64_t dmax = 0;
    for (int k = 0; k < nside; ++k) {
        bool any = false;  // a side with nothing to reduce or zero is left out
        for (int i = 0; i < s.n; ++i) any |= (p[k]->chunks.pre[i + 1] - p[k]->chunks.pre[i]) != 1;
        if (!any) continue;
        ReduceSide& sd = ra.side[z++];
        sd.out = a[k]->out;
        sd.part = a[k]->part;
        sd.D = a[k]->D;
        for (int i = 0; i <= s.n; ++i) {
            sd.part_off[i] = p[k]->part_off[i];
            sd.pre[i] = p[k]->chunks.pre[i];
        }
        dmax = dmax > sd.D ? dmax : sd.D;
        ra.accumulate = a[k]->accumulate;
    }
    if (z == 0 || s.n == 0) return hipSuccess;
    for (int i = 0; i < s.n; ++i) {
        ra.rank[i] = s.rank[i];
        ra.roff[i] = s.roff[i];
        ra.scale[i] = s.scale[i];
    }
    const int64_t n = (int64_t)s.rmax * dmax;
    int64_t bx = (n / 4 + 255) / 256;
    if (bx > 1024) bx = 1024;
    hipLaunchKernelGGL(wgrad_reduce, dim3((unsigned)bx, (unsigned)s.n, (unsigned)z), dim3(256), 0, st, ra);
    return hipGetLastError();
}

}  // namespace plora
