// attention_dkv.hip -- the dK/dV pass of the causal grouped-query attention
// backward (head size 128) on the matrix cores.
//
// With P = exp(S - lse) from the forward's statistics and dS = P * (dP -
// delta), dP = dO V^T: dV_j = sum over the query heads of key/value head j of
// P^T dO, dK_j = scale * sum of dS^T Q, over the queries at or after each key
// [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与PEFT实现:
// the attention layer of the Transformer blocks that LoRA adapts].
//
// Work items in sequence order, the key/value heads fastest (one per XCD
// with 8 of them), so the items sharing a sequence's query rows run together.
// Work item: (sequence, key/value head, 64 keys); 8 waves = (query head of a
// head quad, 32-key block), two per SIMD.  Orientation S = Q K^T: a lane owns
// one key of its block and 16 query rows, so P^T and dS^T feed the dV and dK
// products straight from registers, with dO^T and Q^T read transposed
// (ds_read_b64_tr_b16) in the lane's query order.
//  - K rows of the 64 keys sit in LDS for the whole item; V enters the dP
//    product as the B operand, so each lane keeps its key's V row in
//    registers.
//  - Query tiles of 32 rows x 4 heads (Q and dO, 1 KiB per token) and their
//    lse/delta stream through LDS by DMA, double-buffered, one tile in flight
//    while the other is used: each tile serves 64 keys.
//  - Each wave's dK/dV accumulators (4 column blocks x 2) stay in registers
//    for the whole item; the 4 heads' partials of a key block are summed
//    through LDS at the end in a fixed order.
#include "attention_common.h"

namespace plora {
namespace {

constexpr int kDkvKeys = kAttnKTileB;             // keys per work item (64)
constexpr int kDkvQRows = 32;                     // query rows per stage
constexpr int kDkvRow = 1024;                     // 4 heads x 256 bytes per token
constexpr int kDkvTile = kDkvQRows * kDkvRow;     // 32 KiB
static_assert(kDkvKeys == 64, "two 32-key blocks");

__shared__ __attribute__((aligned(1024))) uint8_t g_tq0[kDkvTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_tq1[kDkvTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_td0[kDkvTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_td1[kDkvTile];
__shared__ __attribute__((aligned(16))) float g_tl0[2 * 4 * kDkvQRows];  // lse rows, then delta rows
__shared__ __attribute__((aligned(16))) float g_tl1[2 * 4 * kDkvQRows];
__shared__ __attribute__((aligned(1024))) uint8_t g_tk[kDkvKeys * 256];  // the item's K rows

__global__ __launch_bounds__(512, 1) void attn_bwd_dkv_kernel(AttnArgs a, SeqTable s) {
    int seq, kt, kvh;
    work_item_grouped(s, a.n_kv, seq, kt, kvh);
    const int l = lane_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(wave_id());
    const int hw = wu & 3, kb = wu >> 2;  // this wave's head within the quad, key block
    const int grp = a.n_q / a.n_kv, nquads = grp / 4;
    const int64_t t0 = s.off[seq];
    const int len = s.off[seq + 1] - s.off[seq];
    const int k0 = kt * kDkvKeys;  // the item's first key
    const int64_t qstride = (int64_t)a.n_q * kHeadDim, kstride = (int64_t)a.n_kv * kHeadDim;

    // K rows of the 64 keys into g_tk (swizzled 256-byte rows; keys past the
    // sequence read as zero): 1024 chunks of 16 bytes, 2 per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = (int)threadIdx.x + 512 * i, row = idx >> 4, ch = idx & 15;
        const int kr = k0 + row;
        const bf16* src = static_cast<const bf16*>(a.k) + (t0 + (kr < len ? kr : 0)) * kstride + kvh * kHeadDim + 8 * ch;
        *reinterpret_cast<u32x4*>(g_tk + swz256(row, ch)) = load16_or_zero(src, kr < len);
    }
    // V of this lane's key as the B operand of dP = dO V^T, one per k-step of
    // 16 dims: key k0 + 32 kb + l%32, dims 16 kk + 8 (l/32) .. +7
    const int key = k0 + 32 * kb + l32;
    bf16x8 vf[8];
    {
        const bf16* row = static_cast<const bf16*>(a.v) + (t0 + (key < len ? key : 0)) * kstride + kvh * kHeadDim + 8 * lh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) vf[kk] = as_bf16x8(load16_or_zero(row + 16 * kk, key < len));
    }

    // query rows of this sequence; rows past it read as zero
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.q) + t0 * qstride), 0, (int)((int64_t)len * qstride * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.dO) + t0 * qstride), 0, (int)((int64_t)len * qstride * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.lse, 0, (int)(a.T * a.n_q * 4), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.delta, 0, (int)(a.T * a.n_q * 4), kRsrcWord3);
    const int qt0 = k0 / kDkvQRows;                      // first query tile that can see these keys
    const int nqt = (len + kDkvQRows - 1) / kDkvQRows;   // query tiles of the sequence
    const int nst = (nqt - qt0) * nquads;                // stages: (query tile, head quad)
    const int hsh = l >> 4, hpc = l & 15;                // DMA lane: head of the row, physical chunk
    // stage z: query tile qt0 + z / nquads, heads kvh*grp + 4*(z % nquads) + 0..3.
    // Wave w loads token rows 4w .. 4w+3 of Q and of dO; waves 0-3 also one of
    // the four lse/delta pieces (4-byte loads: 2 heads x 32 queries each).
    // In flight per wave: 8 or 9 loads.
    auto issue = [&](uint8_t* qbuf, uint8_t* dbuf, float* lbuf, int z) {
        const int qt = qt0 + z / nquads;
        const int hq0 = kvh * grp + 4 * (z % nquads);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * wu + j;  // token row of the tile
            const uint32_t vo = (uint32_t)((int64_t)(qt * kDkvQRows + r) * qstride * 2) +
                                (uint32_t)((hq0 + hsh) * 256) + (uint32_t)((hpc ^ rowkey(r)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(qbuf + r * kDkvRow), 16, vo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(dbuf + r * kDkvRow), 16, vo, 0, 0, 0);
        }
        if (wu < 4) {
            // piece wu: lse (wu < 2) or delta rows of heads 2*(wu%2) .. +1, 32 queries each.
            // The lane terms come from an opaque copy of the lane id: a head
            // offset held across the loop was spilled, and its reload's wait
            // also waited for the stage in flight.
            int lo = lane_id();
            asm volatile("" : "+v"(lo));
            const int hh = 2 * (wu & 1) + (lo >> 5);
            const int64_t e = (int64_t)(hq0 + hh) * a.T + t0 + qt * kDkvQRows + (lo & 31);
            const uint32_t vo = (uint32_t)(e * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wu < 2 ? rl : rt,
                                                     (lds_void*)(lbuf + (wu >> 1) * 128 + 64 * (wu & 1)), 4, vo,
                                                     0, 0, 0);
        }
    };

    // wait until only the next stage's loads (9 for waves 0-3, else 8) are in flight
    auto wait_stage = [&]() {
        if (wu < 4) wait_vmcnt<9>(); else wait_vmcnt<8>();
    };

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dk[db] = dv[db] = f32x16{};
    const float c = a.scale * kLog2e;

    auto stage = [&](const uint8_t* qbuf, const uint8_t* dbuf, const float* lbuf, int z) {
        const int qt = qt0 + z / nquads;
        const uint8_t* qh = qbuf + hw * 256;  // this wave's head within the 1 KiB rows
        const uint8_t* dh = dbuf + hw * 256;
        // S = Q K^T and dP = dO V^T; lane: key column, query rows
        // 8*(v/4) + 4*lh + v%4 of the tile
        f32x16 st = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            st = mfma32x32x16(frag_row<kDkvRow>(qh, l32, 2 * kk + lh), frag_row(g_tk, 32 * kb + l32, 2 * kk + lh), st);
            dp = mfma32x32x16(frag_row<kDkvRow>(dh, l32, 2 * kk + lh), vf[kk], dp);
        }
        // Masks: the causal one on the first two query tiles (the only ones
        // holding queries before some of the keys), rows past the sequence
        // (zero Q and dO rows, but the lse and delta of other tokens) on the
        // last.  Keys past the sequence are not stored.
        if (qt < qt0 + 2 || (qt + 1) * kDkvQRows > len) {
            const int lim = key - qt * kDkvQRows - 4 * lh, end = len - qt * kDkvQRows - 4 * lh;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 8 * (v >> 2) + (v & 3);
                if (r < lim || r >= end) st[v] = kNegInf;
            }
        }
        // P = 2^(c S - lse log2 e), dS = P (dP - delta)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int r0 = 8 * g4 + 4 * lh;
            const f32x4 ls = *reinterpret_cast<const f32x4*>(lbuf + hw * 32 + r0);
            const f32x4 dl = *reinterpret_cast<const f32x4*>(lbuf + 128 + hw * 32 + r0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * g4 + e;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], c, -ls[e] * kLog2e));
                st[v] = p;
                dp[v] = p * (dp[v] - dl[e]);
            }
        }
        const bf16x8 p0 = rows_as_b(st, 0), p1 = rows_as_b(st, 1);
        const bf16x8 s0 = rows_as_b(dp, 0), s1 = rows_as_b(dp, 1);
        // dV += P^T dO and dK += dS^T Q
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            dv[db] = mfma32x32x16(p0, frag_tr<kDkvRow>(dh, db * 32, 0), dv[db]);
            dv[db] = mfma32x32x16(p1, frag_tr<kDkvRow>(dh, db * 32, 16), dv[db]);
            dk[db] = mfma32x32x16(s0, frag_tr<kDkvRow>(qh, db * 32, 0), dk[db]);
            dk[db] = mfma32x32x16(s1, frag_tr<kDkvRow>(qh, db * 32, 16), dk[db]);
        }
    };

    if (nst > 0) {
        issue(g_tq0, g_td0, g_tl0, 0);
        for (int z = 0; z < nst; z += 2) {
            if (z + 1 < nst) {
                issue(g_tq1, g_td1, g_tl1, z + 1);
                wait_stage();  // stage z landed (stage z+1 in flight)
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();  // (the first one also makes g_tk visible)
            stage(g_tq0, g_td0, g_tl0, z);
            lds_barrier();
            if (z + 1 >= nst) break;
            if (z + 2 < nst) {
                issue(g_tq0, g_td0, g_tl0, z + 2);
                wait_stage();
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
            stage(g_tq1, g_td1, g_tl1, z + 1);
            lds_barrier();
        }
    }

    // Sum the 4 heads' partials of each key block through LDS (free now; a
    // partial is 128 values per lane, stored [value][lane]: 32 KiB): heads
    // 2, 3 -> 0, 1, then 1 -> 0, so every sum is (h0 + h2) + (h1 + h3).
    auto slot = [&](int i) -> float* {
        return reinterpret_cast<float*>(i == 0 ? g_tq0 : i == 1 ? g_tq1 : i == 2 ? g_td0 : g_td1);
    };
    auto put = [&](float* b) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                b[(db * 16 + e) * 64 + l] = dk[db][e];
                b[(64 + db * 16 + e) * 64 + l] = dv[db][e];
            }
    };
    auto take = [&](const float* b) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                dk[db][e] += b[(db * 16 + e) * 64 + l];
                dv[db][e] += b[(64 + db * 16 + e) * 64 + l];
            }
    };
    if (hw >= 2) put(slot(2 * kb + hw - 2));
    __syncthreads();
    if (hw < 2) take(slot(2 * kb + hw));
    __syncthreads();
    if (hw == 1) put(slot(kb));
    __syncthreads();
    if (hw != 0) return;
    take(slot(kb));

    // lane: dim db*32 + l%32, keys 8*(v/4) + 4*lh + v%4 of the key block
    bf16* DK = static_cast<bf16*>(a.out2);
    bf16* DV = static_cast<bf16*>(a.out3);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int kr = k0 + 32 * kb + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (kr >= len) continue;
        const int64_t ro = (t0 + kr) * kstride + kvh * kHeadDim + l32;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            DK[ro + db * 32] = to_bf16(dk[db][e] * a.scale);
            DV[ro + db * 32] = to_bf16(dv[db][e]);
        }
    }
}

}  // namespace

hipError_t launch_attention_dkv(const AttnArgs& a, const SeqTable& s0, hipStream_t st) {
    SeqTable s = s0;
    const dim3 grid = attention_grid_grouped(s, kDkvKeys, a.n_kv);
    if (s.tiles[s.n] == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_bwd_dkv_kernel, grid, dim3(512), 0, st, a, s);
    return hipGetLastError();
}

}  // namespace plora
