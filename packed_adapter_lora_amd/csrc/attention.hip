// attention.hip -- causal grouped-query attention of the Llama-3 decoder block
// (head size 128), forward and backward, on the matrix cores.
//
// The attention layer belongs to every Transformer block that LoRA adapts
// [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与PEFT实现]
// in the LLaMA-3 models the pages fine-tune [PLoRA technical summary
// (gist.science, arXiv 2508.02932), 结果].  For every sequence, query head j
// attends to key/value head j / (n_q / n_kv) over the keys at or before its
// own position: o = softmax(q k^T / sqrt(128)) v.
//
// The scores never reach HBM: each work item keeps one tile of queries and
// streams the keys in tiles, with the running maximum and sum of the softmax
// kept per query (the online softmax).  Orientation: the score tile is
// computed transposed, S^T = K Q^T, so a lane of a 32x32 matrix-core block
// owns one query and 16 keys; row statistics need one exchange between the
// two lanes that share a query, and P^T feeds the next product (O^T += V^T
// P^T) straight from registers.  That product's k index (the key) runs over
// the keys a lane holds in the order the matrix core left them; V^T is read
// with the same key order by transposed LDS reads (ds_read_b64_tr_b16).
//
// Work item: one sequence, 4 query heads that share one key/value head, 64
// queries; 8 waves, one per (query head, 32-query block), so all of them
// share each K/V tile in LDS and two waves share each SIMD.
// K/V tiles (64 keys x 256 bytes) arrive by LDS DMA, double-buffered, rows
// XOR-swizzled in 16-byte chunks.  Keys past the sequence read as zero (the
// buffer range ends with the sequence) and are masked.
#include "attention_common.h"

namespace plora {
namespace {

__shared__ __attribute__((aligned(1024))) uint8_t g_k0[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_k1[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_k2[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_v0[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_v1[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_v2[kAttnKTile * 256];

__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnArgs a, SeqTable s) {
    int seq, qt, hg;
    if (!work_item(s, a.n_q / 4, true, seq, qt, hg)) return;
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int head = 4 * hg + (w & 3);
    const int qb = w >> 2;  // this wave's 32-query block of the tile
    const int grp = a.n_q / a.n_kv;
    const int kvh = (4 * hg) / grp;
    const int64_t t0 = s.off[seq];
    const int len = s.off[seq + 1] - s.off[seq];
    const int qi = qt * kAttnQTile + qb * 32 + l32;  // this lane's query, within the sequence
    const int64_t qstride = (int64_t)a.n_q * kHeadDim, kstride = (int64_t)a.n_kv * kHeadDim;

    // this lane's query as B operands, one per k step of 16 dims
    bf16x8 qf[8];
    {
        const bool ok = qi < len;
        const bf16* row = static_cast<const bf16*>(a.q) + (t0 + (ok ? qi : 0)) * qstride + head * kHeadDim + 8 * lh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qf[kk] = as_bf16x8(load16_or_zero(row + 16 * kk, ok));
    }

    // K/V rows of this sequence and key/value head; rows past the sequence read as zero
    const uint32_t bytes = (uint32_t)((int64_t)len * kstride * 2);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.k) + t0 * kstride + kvh * kHeadDim), 0, (int)bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.v) + t0 * kstride + kvh * kHeadDim), 0, (int)bytes, kRsrcWord3);
    // DMA block b (1 KiB) = rows 4b .. 4b+3; lane l -> row 4b + l/16, physical chunk l%16;
    // wave w loads blocks 2w, 2w+1 of K and of V
    const int rr = l >> 4, pc = l & 15;
    auto issue = [&](uint8_t* kb, uint8_t* vb, int kt) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int b = 2 * wu + j;
            const int r = 4 * b + rr;
            const uint32_t vo = (uint32_t)((int64_t)(kt * kAttnKTile + r) * kstride * 2) +
                                (uint32_t)((pc ^ rowkey(r)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kb + b * 1024), 16, vo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vb + b * 1024), 16, vo, 0, 0, 0);
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    // Online softmax with a lazily moved reference: p = 2^(c s - mref), where
    // mref (shared by the two lanes of a query) only moves when some query of
    // the wave sees a score more than 2^8 above it; o and the lane's part of
    // the denominator are rescaled then.  In between, p <= 2^8.
    float mref = kNegInf, lpart = 0.0f;
    const float c = a.scale * kLog2e;

    // one 64-key tile from LDS, as two halves of 32 keys: both score blocks
    // first, so the second one's products run during the first one's softmax
    auto tile = [&](const uint8_t* kb, const uint8_t* vb, int kt) {
        f32x16 st[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            st[hb] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                st[hb] = mfma32x32x16(frag_row(kb, hb * 32 + l32, 2 * kk + lh), qf[kk], st[hb]);
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            // causal mask on the diagonal tile: key hb*32 + 8*(v/4) + 4*lh + v%4
            // of the tile against the query (keys past the sequence only occur
            // there, after every valid query)
            if (kt == qt) {
                const int lim = qi - kt * kAttnKTile - hb * 32 - 4 * lh;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (8 * (v >> 2) + (v & 3) > lim) st[hb][v] = kNegInf;
            }
            float mx = st[hb][0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, st[hb][v]);
            const float mxs = mx * c;
            if (__ballot(mxs > mref + 8.0f)) {
                const float mn = fmaxf(mref, fmaxf(mxs, __shfl_xor(mxs, 32)));
                // (a query with no visible key yet keeps -inf; its o and lpart are 0)
                const float alpha = mn == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(mref - mn);
                lpart *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) o[db] *= alpha;
                mref = mn;
            }
            const float sh = mref == kNegInf ? 0.0f : mref;
            float ps = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[hb][v], c, -sh));
                st[hb][v] = p;
                ps += p;
            }
            lpart += ps;
            const bf16x8 p0 = rows_as_b(st[hb], 0), p1 = rows_as_b(st[hb], 1);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                o[db] = mfma32x32x16(frag_tr(vb, db * 32, hb * 32), p0, o[db]);
                o[db] = mfma32x32x16(frag_tr(vb, db * 32, hb * 32 + 16), p1, o[db]);
            }
        }
    };

    // causal: key tiles 0 .. qt.  Each wave waits for its own loads, then the
    // barrier makes every wave's loads visible (no vmcnt drain at the barrier).
    const int nkt = qt + 1;
    // three buffers: tiles kt+1 and kt+2 in flight while tile kt is used; one
    // barrier per tile (after it, every wave's loads of tile kt are visible
    // and every wave is done with tile kt-1, whose buffer receives kt+2)
    auto step = [&](uint8_t* kb, uint8_t* vb, uint8_t* kn, uint8_t* vn, int kt) {
        if (kt + 1 < nkt) wait_vmcnt<4>(); else wait_vmcnt<0>();  // tile kt landed (kt+1 in flight)
        lds_barrier();
        if (kt + 2 < nkt) issue(kn, vn, kt + 2);
        tile(kb, vb, kt);
    };
    issue(g_k0, g_v0, 0);
    if (nkt > 1) issue(g_k1, g_v1, 1);
    for (int kt = 0; kt < nkt; kt += 3) {
        step(g_k0, g_v0, g_k2, g_v2, kt);
        if (kt + 1 >= nkt) break;
        step(g_k1, g_v1, g_k0, g_v0, kt + 1);
        if (kt + 2 >= nkt) break;
        step(g_k2, g_v2, g_k1, g_v1, kt + 2);
    }
    lds_barrier();  // every wave is done with the last tile

    // normalise and store (the K/V buffers are free: 8 KiB per wave); lane
    // holds query qi, dims db*32 + 8*(v/4) + 4*lh + v%4
    const float lsum = lpart + __shfl_xor(lpart, 32);
    const int q0b = qt * kAttnQTile + qb * 32;  // this wave's first query
    store_rows_via_lds(o, 1.0f / lsum, (wu < 2 ? g_k0 : wu < 4 ? g_k1 : wu < 6 ? g_v0 : g_v1) + (wu & 1) * 8192,
                       static_cast<bf16*>(a.out) + (t0 + q0b) * qstride + head * kHeadDim, qstride, len - q0b);
    if (qi < len && lh == 0) a.lse[(int64_t)head * a.T + t0 + qi] = (mref + log2f(lsum)) / kLog2e;
}

// ===========================================================================
// Backward.  With P = exp(S - lse) (lse from the forward), dV = P^T dO,
// dP = dO V^T, dS = P * (dP - delta), delta = rowsum(dO * O), dQ = scale dS K,
// dK = scale dS^T Q.  Two kernels: dQ (the forward's orientation, one work
// item per query tile, streaming key tiles; it also writes delta), then dK
// and dV (attention_dkv.hip: the other orientation, S = Q K^T with one key
// per lane, one work item per 64-key tile of one key/value head, streaming
// query tiles of all its query heads).
// ===========================================================================

// dQ: work item = (sequence, 4 query heads of one key/value head, 64 queries);
// 8 waves = (query head, 32-query block), key tiles streamed as in the forward.
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_kernel(AttnArgs a, SeqTable s) {
    int seq, qt, hg;
    if (!work_item(s, a.n_q / 4, true, seq, qt, hg)) return;
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int head = 4 * hg + (w & 3);
    const int qb = w >> 2;
    const int grp = a.n_q / a.n_kv;
    const int kvh = (4 * hg) / grp;
    const int64_t t0 = s.off[seq];
    const int len = s.off[seq + 1] - s.off[seq];
    const int qi = qt * kAttnQTile + qb * 32 + l32;
    const bool qok = qi < len;
    const int64_t qstride = (int64_t)a.n_q * kHeadDim, kstride = (int64_t)a.n_kv * kHeadDim;

    // this lane's query row of Q and dO as B operands, and delta = rowsum(dO * O)
    // (the two lanes of a query hold 64 of its dims each; the dK/dV pass reads
    // delta from here)
    bf16x8 qf[8], df[8];
    float dlt;
    {
        const int64_t ro = (t0 + (qok ? qi : 0)) * qstride + head * kHeadDim + 8 * lh;
        float dp = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            qf[kk] = as_bf16x8(load16_or_zero(static_cast<const bf16*>(a.q) + ro + 16 * kk, qok));
            const u32x4 dv = load16_or_zero(static_cast<const bf16*>(a.dO) + ro + 16 * kk, qok);
            const u32x4 ov = load16_or_zero(static_cast<const bf16*>(a.o) + ro + 16 * kk, qok);
            df[kk] = as_bf16x8(dv);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dp += __uint_as_float(dv[e] << 16) * __uint_as_float(ov[e] << 16) +
                      __uint_as_float(dv[e] & 0xffff0000u) * __uint_as_float(ov[e] & 0xffff0000u);
        }
        dlt = dp + __shfl_xor(dp, 32);
        if (qok && lh == 0) a.delta[(int64_t)head * a.T + t0 + qi] = dlt;
    }
    const float c = a.scale * kLog2e;
    // (a row past the sequence gets lse = +inf: its p is 0 without a mask)
    const float lse2 = qok ? a.lse[(int64_t)head * a.T + t0 + qi] * kLog2e : __builtin_inff();

    const uint32_t bytes = (uint32_t)((int64_t)len * kstride * 2);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.k) + t0 * kstride + kvh * kHeadDim), 0, (int)bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.v) + t0 * kstride + kvh * kHeadDim), 0, (int)bytes, kRsrcWord3);
    auto issue = [&](uint8_t* kb, uint8_t* vb, int kt) {
        // (the lane's row and chunk are taken from an opaque copy of the lane
        // id at every call: held across the loop, the offsets were spilled,
        // and each reload's wait for it also waited for the K/V tile in
        // flight; −1.4 % for the backward)
        int lo = lane_id();
        asm volatile("" : "+v"(lo));
        const int rr = lo >> 4, pc = lo & 15;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int b = 2 * wu + j;
            const int r = 4 * b + rr;
            const uint32_t vo = (uint32_t)((int64_t)(kt * kAttnKTile + r) * kstride * 2) +
                                (uint32_t)((pc ^ rowkey(r)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kb + b * 1024), 16, vo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vb + b * 1024), 16, vo, 0, 0, 0);
        }
    };

    f32x16 dq[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[db] = f32x16{};
    auto tile = [&](const uint8_t* kb, const uint8_t* vb, int kt) {
        const bool diag = kt == qt;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            f32x16 st = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                st = mfma32x32x16(frag_row(kb, hb * 32 + l32, 2 * kk + lh), qf[kk], st);
                dp = mfma32x32x16(frag_row(vb, hb * 32 + l32, 2 * kk + lh), df[kk], dp);
            }
            // causal mask on the diagonal tile: key hb*32 + 8*(v/4) + 4*lh + v%4
            // of the tile against the query (keys past the sequence only occur
            // there, after every valid query)
            if (diag) {
                const int lim = qi - kt * kAttnKTile - hb * 32 - 4 * lh;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (8 * (v >> 2) + (v & 3) > lim) st[v] = kNegInf;
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], c, -lse2));
                st[v] = p * (dp[v] - dlt);  // dS^T
            }
            const bf16x8 s0 = rows_as_b(st, 0), s1 = rows_as_b(st, 1);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                dq[db] = mfma32x32x16(frag_tr(kb, db * 32, hb * 32), s0, dq[db]);
                dq[db] = mfma32x32x16(frag_tr(kb, db * 32, hb * 32 + 16), s1, dq[db]);
            }
        }
    };

    const int nkt = qt + 1;
    issue(g_k0, g_v0, 0);
    for (int kt = 0; kt < nkt; kt += 2) {
        if (kt + 1 < nkt) {
            issue(g_k1, g_v1, kt + 1);
            wait_vmcnt<4>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        tile(g_k0, g_v0, kt);
        lds_barrier();
        if (kt + 1 >= nkt) break;
        if (kt + 2 < nkt) {
            issue(g_k0, g_v0, kt + 2);
            wait_vmcnt<4>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        tile(g_k1, g_v1, kt + 1);
        lds_barrier();
    }

    // (the K/V buffers are free: 8 KiB per wave)
    const int q0b = qt * kAttnQTile + qb * 32;  // this wave's first query
    store_rows_via_lds(dq, a.scale, (wu < 2 ? g_k0 : wu < 4 ? g_k1 : wu < 6 ? g_v0 : g_v1) + (wu & 1) * 8192,
                       static_cast<bf16*>(a.out) + (t0 + q0b) * qstride + head * kHeadDim, qstride, len - q0b);
}

}  // namespace

hipError_t launch_attention_fwd(const AttnArgs& a, const SeqTable& s0, hipStream_t st) {
    SeqTable s = s0;
    const dim3 grid = attention_grid(s, kAttnQTile, a.n_q / 4);
    if (s.tiles[s.n] == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_fwd_kernel, grid, dim3(512), 0, st, a, s);
    return hipGetLastError();
}

hipError_t launch_attention_bwd(const AttnArgs& a, const SeqTable& s0, hipStream_t st) {
    SeqTable s = s0;
    const dim3 grid = attention_grid(s, kAttnQTile, a.n_q / 4);
    if (s.tiles[s.n] == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_bwd_dq_kernel, grid, dim3(512), 0, st, a, s);  // (also writes delta)
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attention_dkv(a, s0, st);
}

}  // namespace plora
