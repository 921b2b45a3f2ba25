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

template <int MAXJT, int WPG>
__global__ __launch_bounds__(64 * WPG, 1) void shrink_bf16_pipe(ShrinkArgs a, SegTable seg, WorkMap m) {
    constexpr int TR = 32 * WPG;                           // token rows per tile
    constexpr int kShX = TR * kShRowB;                     // token rows per stage
    constexpr int kShStage = kShX + 32 * MAXJT * kShRowB;  // + the panel rows
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh0[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh1[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh2[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh3[kShStage];
    __shared__ __attribute__((aligned(1024))) uint8_t g_sh4[kShStage];
    const int unit = (int)blockIdx.x;
    const int64_t K = a.K;
    const int i = adapter_of_unit(m, seg.n, unit);
    const int64_t s0 = seg.off[i], s1 = seg.off[i + 1];
    const int nsl = shrink_slices(s1 - s0, seg.rank[i], K, a.scratch_row);
    const int u = unit - m.pre[i], slice = u % nsl;
    const int64_t t0 = s0 + (int64_t)(u / nsl) * TR;
    const int nrows = (int)(s1 - t0 < TR ? s1 - t0 : TR);
    const int r = seg.rank[i];
    const int ntj = (r + 31) >> 5;
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.Q) + t0 * K), 0, (int)(nrows * K * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.P) + (int64_t)seg.roff[i] * K), 0, (int)(r * K * 2), kRsrcWord3);
    // DMA block b: rows 8b .. 8b+7; lane l -> row 8b + l/8, physical chunk l%8
    const int r0 = l >> 3;
    const uint32_t lane_row = (uint32_t)(r0 * K * 2);
    // this work item's stages: [kt0, kt1) of the K / 64
    const int KT = (int)(K / 64), kt0 = slice * KT / nsl, kt1 = (slice + 1) * KT / nsl;
    // token tile: blocks 4w .. 4w+3 (32 rows per wave); panel: 4*MAXJT blocks,
    // PB per wave
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
        for (int j = 0; j < PB; ++j) {
            const int blk = PB * wu + j;
            const uint32_t vo = lane_row + (uint32_t)(((l & 7) ^ ((r0 ^ blk) & 7)) << 4) + (uint32_t)blk * (8u * K * 2) + kb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(buf + kShX + blk * 1024), 16, vo, 0, 0, 0);
        }
    };
    f32x16 acc[MAXJT];
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) acc[jt] = f32x16{};
    auto compute = [&](const uint8_t* buf) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 xa = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kofs128(32 * w + l32, 2 * kk + lh)));
#pragma unroll
            for (int jt = 0; jt < MAXJT; ++jt) {
                if (jt >= ntj) continue;
                const bf16x8 pb = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kShX + kofs128(32 * jt + l32, 2 * kk + lh)));
                acc[jt] = mfma32x32x16(xa, pb, acc[jt]);
            }
        }
    };
    constexpr int kPer = 4 + PB;  // DMA loads per wave per stage
    // stage kt in cur; stages kt+1 .. kt+3 in flight; refill prv (stage kt-1,
    // done) with stage kt+4
    auto step = [&](uint8_t* cur, uint8_t* prv, int kt) {
        wait_vmcnt<3 * kPer>();  // stage kt landed, stages kt+1 .. kt+3 may be in flight
        lds_barrier();           // and every wave is done with stage kt-1
        issue(prv, kt + 4);
        compute(cur);
    };
    issue(g_sh0, kt0);
    issue(g_sh1, kt0 + 1);
    issue(g_sh2, kt0 + 2);
    issue(g_sh3, kt0 + 3);
    for (int kt = kt0; kt < kt1; kt += 5) {
        step(g_sh0, g_sh4, kt);
        if (kt + 1 >= kt1) break;
        step(g_sh1, g_sh0, kt + 1);
        if (kt + 2 >= kt1) break;
        step(g_sh2, g_sh1, kt + 2);
        if (kt + 3 >= kt1) break;
        step(g_sh3, g_sh2, kt + 3);
        if (kt + 4 >= kt1) break;
        step(g_sh4, g_sh3, kt + 4);
    }
    wait_vmcnt<0>();

    // D[t][j]: lane holds rank column j, token rows 8*(v/4) + 4*(l/32) + v%4 of its wave's 32.
    // K slices: slice s of the adapter's [n_i][r_i] block goes to its own rows of
    // the scratch activation, s * n_i * r_i floats in (shrink_slice_sum adds them)
    float* __restrict__ out =
        (nsl == 1 ? a.out + seg.hoff[i]
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
            if (row < nrows) out[(int64_t)row * r + j] = acc[jt][v];
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
// One workgroup per (64-token block, adapter): the block's 64 rows of r_i
// values are contiguous in H, so they are read whole, transposed in LDS, and
// leave as r_i pieces of 128 bytes per array.
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
__global__ __launch_bounds__(256) void wgrad_prep(const float* F, bf16* hi, bf16* lo, SegTable seg, WgradPlan plan) {
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

constexpr int kWqTile = 64 * 512;  // 64 tokens x 256 features bf16

template <int MAXJT>
__global__ __launch_bounds__(256, 1) void wgrad_bf16_pipe(WgradArgs a, SegTable seg, WgradPlan plan, const bf16* fhi,
                                                          const bf16* flo) {
    constexpr int kF = 32 * MAXJT * 128;       // one of the hi / lo panels
    constexpr int kStage = kWqTile + 2 * kF;
    __shared__ __attribute__((aligned(1024))) uint8_t b0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[kStage];
    const int64_t D = a.D;
    const int w = (int)blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * kWgCols;  // (feature tiles fastest: a chunk's rows are read whole)
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
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(fhi + plan.ft_off[i] + (int64_t)u * TK), 0, (int)((r * np - (int64_t)u * TK) * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(flo + plan.ft_off[i] + (int64_t)u * TK), 0, (int)((r * np - (int64_t)u * TK) * 2), kRsrcWord3);
    // activation tile: block b = 2 token rows x 512 B; lane l -> row 2b + l/32, physical chunk l%32
    // (row % 4 = 2*(b%2) + l/32: one lane offset per block parity)
    const int tr = l >> 5;
    const uint32_t q_off0 = (uint32_t)(tr * D * 2) + (uint32_t)(((l & 31) ^ (tr << 2)) << 4);
    const uint32_t q_off1 = (uint32_t)(tr * D * 2) + (uint32_t)(((l & 31) ^ ((2 + tr) << 2)) << 4);
    // rank panels: block b = 8 rank rows x 128 B; lane l -> row 8b + l/8, physical chunk l%8
    const int r0 = l >> 3;
    const uint32_t f_row = (uint32_t)(r0 * np * 2);
    const int nst = (int)((tb - ta + 63) / 64);
    auto issue = [&](uint8_t* buf, int st) {
        const uint32_t oob = st < nst ? 0u : 0x80000000u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int blk = 8 * wu + j;
            const uint32_t vo = ((j & 1) ? q_off1 : q_off0) + (uint32_t)blk * (uint32_t)(2 * D * 2) +
                                (uint32_t)st * (uint32_t)(64 * D * 2) + oob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(buf + blk * 1024), 16, vo, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < MAXJT; ++j) {
            const int blk = MAXJT * wu + j;
            const uint32_t vo = f_row + (uint32_t)(((l & 7) ^ ((r0 ^ blk) & 7)) << 4) + (uint32_t)blk * (uint32_t)(8 * np * 2) +
                                (uint32_t)st * 128u + oob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void*)(buf + kWqTile + blk * 1024), 16, vo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(buf + kWqTile + kF + blk * 1024), 16, vo, 0, 0, 0);
        }
    };
    f32x16 acc[MAXJT][2];
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) acc[jt][0] = acc[jt][1] = f32x16{};
    auto compute = [&](const uint8_t* buf) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 qf[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) qf[ct] = pfrag_tr(buf, 64 * wv + 32 * ct, 16 * kk);
#pragma unroll
            for (int jt = 0; jt < MAXJT; ++jt) {
                if (jt >= ntj) continue;
                const int row = 32 * jt + l32;
                const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kWqTile + kofs128(row, 2 * kk + lh)));
                const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kWqTile + kF + kofs128(row, 2 * kk + lh)));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    acc[jt][ct] = mfma32x32x16(ah, qf[ct], acc[jt][ct]);
                    acc[jt][ct] = mfma32x32x16(al, qf[ct], acc[jt][ct]);
                }
            }
        }
    };
    constexpr int kPer = 8 + 2 * MAXJT;  // DMA loads per wave per stage
    auto step = [&](uint8_t* cur, uint8_t* prv, int st) {
        wait_vmcnt<kPer>();  // stage st landed, st+1 may be in flight
        lds_barrier();       // every wave is done with stage st-1
        issue(prv, st + 2);
        compute(cur);
    };
    issue(b0, 0);
    issue(b1, 1);
    for (int st = 0; st < nst; st += 3) {
        step(b0, b2, st);
        if (st + 1 >= nst) break;
        step(b1, b0, st + 1);
        if (st + 2 >= nst) break;
        step(b2, b1, st + 2);
    }
    wait_vmcnt<0>();

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

// out rows of adapters whose tokens span 0 or >= 2 chunks:
// out = s_i * sum_u partial[u] in chunk order (0 for an empty adapter), or
// out += that when accumulating (an empty adapter is then left alone).
__global__ __launch_bounds__(256) void wgrad_reduce(WgradArgs a, SegTable seg, WgradPlan plan) {
    const int i = (int)blockIdx.y;
    const int nch = plan.chunks.pre[i + 1] - plan.chunks.pre[i];
    if (nch == 1 || (nch == 0 && a.accumulate)) return;
    const int64_t n = (int64_t)seg.rank[i] * a.D;  // multiple of 8
    const float sc = seg.scale[i];
    float* __restrict__ out = a.out + (int64_t)seg.roff[i] * a.D;
    const float* __restrict__ part = a.part + plan.part_off[i];
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < n; e += (int64_t)gridDim.x * 1024) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        for (int u = 0; u < nch; ++u) s += *reinterpret_cast<const f32x4*>(part + (int64_t)u * n + e);
        f32x4 o = s * sc;
        if (a.accumulate) o += *reinterpret_cast<const f32x4*>(out + e);
        *reinterpret_cast<f32x4*>(out + e) = o;
    }
}

// Sum of the K slices of the shrink (fixed order 0, 1, ...) into H / G: one
// workgroup per adapter; adapters that were not sliced return at once.
__global__ __launch_bounds__(256) void shrink_slice_sum(ShrinkArgs a, SegTable seg) {
    const int i = (int)blockIdx.y;
    const int64_t n = seg.off[i + 1] - seg.off[i];
    const int r = seg.rank[i];
    const int nsl = shrink_slices(n, r, a.K, a.scratch_row);
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

hipError_t launch_shrink_bf16(const ShrinkArgs& a_in, const SegTable& s, const WorkMap& m, int32_t units,
                              hipStream_t st) {
    if (units <= 0) return hipSuccess;
    if (a_in.K % 64 == 0 && (int64_t)kShrinkTileRows * a_in.K * 2 < (int64_t(1) << 31) &&
        (int64_t)s.roff[s.n] * a_in.K * 2 < (int64_t(1) << 31)) {
        ShrinkArgs a = a_in;
        if (!a.scratch) a.scratch_row = 0;
        WorkMap mp;
        bool split = false;
        int32_t items = build_shrink_pipe_map(s, &mp, a.K, a.scratch_row, &split, kShrinkTileRows);
        // 32-token tiles (one wave each) when the 128-token ones fill at most
        // half of the CUs: four times the workgroups, same results
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        // (PLORA_SHRINK_TILE_ROWS=32 or 128 forces the tile size)
        const char* force = getenv("PLORA_SHRINK_TILE_ROWS");
        const int fr = force ? atoi(force) : 0;
        const bool small = fr == 32 || (fr != 128 && 2 * (int64_t)items <= cus);
        if (small) items = build_shrink_pipe_map(s, &mp, a.K, a.scratch_row, &split, 32);
        const dim3 grid((unsigned)items), block(small ? 64 : 256);
        switch (((s.rmax + 31) / 32) * 2 + (small ? 1 : 0)) {
            case 2: hipLaunchKernelGGL((shrink_bf16_pipe<1, 4>), grid, block, 0, st, a, s, mp); break;
            case 3: hipLaunchKernelGGL((shrink_bf16_pipe<1, 1>), grid, block, 0, st, a, s, mp); break;
            case 4: hipLaunchKernelGGL((shrink_bf16_pipe<2, 4>), grid, block, 0, st, a, s, mp); break;
            case 5: hipLaunchKernelGGL((shrink_bf16_pipe<2, 1>), grid, block, 0, st, a, s, mp); break;
            case 6: hipLaunchKernelGGL((shrink_bf16_pipe<3, 4>), grid, block, 0, st, a, s, mp); break;
            case 7: hipLaunchKernelGGL((shrink_bf16_pipe<3, 1>), grid, block, 0, st, a, s, mp); break;
            case 8: hipLaunchKernelGGL((shrink_bf16_pipe<4, 4>), grid, block, 0, st, a, s, mp); break;
            default: hipLaunchKernelGGL((shrink_bf16_pipe<4, 1>), grid, block, 0, st, a, s, mp); break;
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

hipError_t launch_wgrad_bf16_pipe(const WgradArgs& a, const SegTable& s, const WgradPlan& p, bf16* fhi, bf16* flo,
                                  hipStream_t st) {
    const int64_t tk = p.chunk_tokens;
    // (the pipelined grid puts the chunks in y: at most 65535 of them)
    if (s.rmax > 64 || fhi == nullptr || tk * a.D * 2 >= (int64_t(1) << 31) || p.chunks.pre[s.n] > 65535)
        return launch_wgrad_bf16(a, s, p, st);
    const int R = s.roff[s.n];
    if (R > 0) {
        int64_t maxnp = 0;
        for (int i = 0; i < s.n; ++i) maxnp = maxnp > pad64(s.off[i + 1] - s.off[i]) ? maxnp : pad64(s.off[i + 1] - s.off[i]);
        if (maxnp > 0) {
            // (hi/lo offsets are multiples of 64 elements and the arrays start 16-byte aligned)
            hipLaunchKernelGGL(wgrad_prep, dim3((unsigned)(maxnp / 64), (unsigned)s.n), dim3(256), 0, st, a.F, fhi, flo,
                               s, p);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    const int32_t units = p.chunks.pre[s.n];
    if (units <= 0) return hipSuccess;
    const dim3 grid((unsigned)p.col_tiles, (unsigned)units), block(256);
    if (s.rmax <= 32)
        hipLaunchKernelGGL((wgrad_bf16_pipe<1>), grid, block, 0, st, a, s, p, fhi, flo);
    else
        hipLaunchKernelGGL((wgrad_bf16_pipe<2>), grid, block, 0, st, a, s, p, fhi, flo);
    return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const WgradArgs& a, const SegTable& s, const WgradPlan& p, hipStream_t st) {
    bool any = false;
    for (int i = 0; i < s.n; ++i) any |= (p.chunks.pre[i + 1] - p.chunks.pre[i]) != 1;
    if (!any || s.n == 0) return hipSuccess;
    const int64_t n = (int64_t)s.rmax * a.D;
    int64_t bx = (n / 4 + 255) / 256;
    if (bx > 1024) bx = 1024;
    const dim3 grid((unsigned)bx, (unsigned)s.n), block(256);
    hipLaunchKernelGGL(wgrad_reduce, grid, block, 0, st, a, s, p);
    return hipGetLastError();
}

}  // namespace plora
