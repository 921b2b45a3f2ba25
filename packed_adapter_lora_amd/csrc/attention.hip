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

__shared__ __attribute__((aligned(1024))) uint8_t g_k0[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_k1[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_v0[kAttnKTile * 256];
__shared__ __attribute__((aligned(1024))) uint8_t g_v1[kAttnKTile * 256];

__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnArgs a, SeqTable s) {
    int seq, qt;
    tile_of(s, (int)blockIdx.x, seq, qt);
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int head = 4 * (int)blockIdx.y + (w & 3);
    const int qb = w >> 2;  // this wave's 32-query block of the tile
    const int grp = a.n_q / a.n_kv;
    const int kvh = (4 * (int)blockIdx.y) / grp;
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
                                (uint32_t)((pc ^ (r & 15)) << 4);
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

    // causal: key tiles 0 .. qt.  Tile kt+1 is in flight while tile kt is
    // used; each wave waits for its own loads, then the barrier makes every
    // wave's loads visible (no vmcnt drain at the barrier).
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
        lds_barrier();  // every wave is done with buffer 0
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

    // normalise and store: lane holds query qi, dims db*32 + 8*(v/4) + 4*lh + v%4
    const float lsum = lpart + __shfl_xor(lpart, 32);
    if (qi < len) {
        const float inv = 1.0f / lsum;
        bf16* row = static_cast<bf16*>(a.out) + (t0 + qi) * qstride + head * kHeadDim;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = to_bf16(o[db][4 * g4 + e] * inv);
                *reinterpret_cast<bf16x4*>(row + db * 32 + 8 * g4 + 4 * lh) = v4;
            }
        }
        if (lh == 0) a.lse[(int64_t)head * a.T + t0 + qi] = (mref + log2f(lsum)) / kLog2e;
    }
}

// ===========================================================================
// Backward.  With P = exp(S - lse) (lse from the forward), dV = P^T dO,
// dP = dO V^T, dS = P * (dP - delta), delta = rowsum(dO * O), dQ = scale dS K,
// dK = scale dS^T Q.  Three kernels: delta; dQ (the forward's orientation,
// one work item per query tile, streaming key tiles); dK and dV (the other
// orientation, S = Q K^T with one key per lane, one work item per 64-key tile
// of one key/value head, streaming query tiles of all its query heads).
// ===========================================================================

// delta[h][t] = sum_d dO[t][h][d] * O[t][h][d]: 16 lanes per (token, head)
__global__ __launch_bounds__(256) void attn_delta_kernel(AttnArgs a) {
    const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // token * n_q + head
    const int part = threadIdx.x & 15;
    const bool ok = item < a.T * a.n_q;
    float acc = 0.0f;
    if (ok) {
        const int64_t off = item * kHeadDim + part * 8;
        const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.dO) + off);
        const u32x4 y = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.o) + off);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            acc += __uint_as_float(x[k] << 16) * __uint_as_float(y[k] << 16) +
                   __uint_as_float(x[k] & 0xffff0000u) * __uint_as_float(y[k] & 0xffff0000u);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (ok && part == 0) {
        const int64_t t = item / a.n_q, h = item - t * a.n_q;
        a.delta[h * a.T + t] = acc;
    }
}

// dQ: work item = (sequence, 4 query heads of one key/value head, 64 queries);
// 8 waves = (query head, 32-query block), key tiles streamed as in the forward.
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_kernel(AttnArgs a, SeqTable s) {
    int seq, qt;
    tile_of(s, (int)blockIdx.x, seq, qt);
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int head = 4 * (int)blockIdx.y + (w & 3);
    const int qb = w >> 2;
    const int grp = a.n_q / a.n_kv;
    const int kvh = (4 * (int)blockIdx.y) / grp;
    const int64_t t0 = s.off[seq];
    const int len = s.off[seq + 1] - s.off[seq];
    const int qi = qt * kAttnQTile + qb * 32 + l32;
    const bool qok = qi < len;
    const int64_t qstride = (int64_t)a.n_q * kHeadDim, kstride = (int64_t)a.n_kv * kHeadDim;

    bf16x8 qf[8], df[8];
    {
        const int64_t ro = (t0 + (qok ? qi : 0)) * qstride + head * kHeadDim + 8 * lh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            qf[kk] = as_bf16x8(load16_or_zero(static_cast<const bf16*>(a.q) + ro + 16 * kk, qok));
            df[kk] = as_bf16x8(load16_or_zero(static_cast<const bf16*>(a.dO) + ro + 16 * kk, qok));
        }
    }
    const float c = a.scale * kLog2e;
    // (a row past the sequence gets lse = +inf: its p is 0 without a mask)
    const float lse2 = qok ? a.lse[(int64_t)head * a.T + t0 + qi] * kLog2e : __builtin_inff();
    const float dlt = qok ? a.delta[(int64_t)head * a.T + t0 + qi] : 0.0f;

    const uint32_t bytes = (uint32_t)((int64_t)len * kstride * 2);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.k) + t0 * kstride + kvh * kHeadDim), 0, (int)bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const bf16*>(a.v) + t0 * kstride + kvh * kHeadDim), 0, (int)bytes, kRsrcWord3);
    const int rr = l >> 4, pc = l & 15;
    auto issue = [&](uint8_t* kb, uint8_t* vb, int kt) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int b = 2 * wu + j;
            const int r = 4 * b + rr;
            const uint32_t vo = (uint32_t)((int64_t)(kt * kAttnKTile + r) * kstride * 2) +
                                (uint32_t)((pc ^ (r & 15)) << 4);
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

    if (qok) {
        bf16* row = static_cast<bf16*>(a.out) + (t0 + qi) * qstride + head * kHeadDim;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = to_bf16(dq[db][4 * g4 + e] * a.scale);
                *reinterpret_cast<bf16x4*>(row + db * 32 + 8 * g4 + 4 * lh) = v4;
            }
        }
    }
}

// dK, dV: work item = (sequence, key/value head, 32 keys); 4 waves = the 4
// query heads of the key/value head.  Query tiles of 32 rows stream through
// LDS for the 4 heads at a time (one token's 4 head rows are 1 KiB
// contiguous): Q, dO, and the rows' lse and delta, double-buffered.  The
// keys' K and V rows sit in LDS for the whole item (in registers they crowd
// out the fragment prefetches); each wave accumulates partial dK and dV for
// its query head, and the 4 partials are summed through LDS at the end.
constexpr int kBwdQRows = 32;
constexpr int kBwdKTile = 32;                    // keys per dK/dV work item
constexpr int kBwdRow = 1024;                    // 4 heads x 256 bytes per token
constexpr int kBwdTile = kBwdQRows * kBwdRow;    // 32 KiB
__shared__ __attribute__((aligned(1024))) uint8_t g_bq0[kBwdTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_bq1[kBwdTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_bd0[kBwdTile];
__shared__ __attribute__((aligned(1024))) uint8_t g_bd1[kBwdTile];
__shared__ __attribute__((aligned(16))) float g_bl0[2 * 4 * kBwdQRows];  // lse*log2e rows, then delta rows
__shared__ __attribute__((aligned(16))) float g_bl1[2 * 4 * kBwdQRows];
__shared__ __attribute__((aligned(1024))) uint8_t g_bkv[2 * kBwdKTile * 256];  // the keys' K rows, then V rows

// (4 waves of 512 registers each: the K/V fragments and both accumulators
// stay in registers, so nothing is spilled inside the query loop)
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(AttnArgs a, SeqTable s) {
    int seq, kt;
    tile_of(s, (int)blockIdx.x, seq, kt, false);  // early key tiles see the most queries: first
    const int l = lane_id(), w = wave_id(), l32 = l & 31, lh = l >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int kb = 0, hw = w;
    const int kvh = (int)blockIdx.y;
    const int grp = a.n_q / a.n_kv, nquads = grp / 4;
    const int64_t t0 = s.off[seq];
    const int len = s.off[seq + 1] - s.off[seq];
    const int key = kt * kBwdKTile + kb * 32 + l32;  // this lane's key (column of S)
    const int64_t qstride = (int64_t)a.n_q * kHeadDim, kstride = (int64_t)a.n_kv * kHeadDim;

    // K and V rows of the 32 keys into g_bkv (swizzled 256-byte rows; keys past
    // the sequence read as zero): 1024 chunks of 16 bytes, 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = (int)threadIdx.x + 256 * i, ten = idx >> 9, row = (idx >> 4) & 31, ch = idx & 15;
        const int kr = kt * kBwdKTile + row;
        const bf16* src = static_cast<const bf16*>(ten ? a.v : a.k) +
                          (t0 + (kr < len ? kr : 0)) * kstride + kvh * kHeadDim + 8 * ch;
        *reinterpret_cast<u32x4*>(g_bkv + ten * (kBwdKTile * 256) + swz256(row, ch)) = load16_or_zero(src, kr < len);
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
    const int qt0 = (kt * kBwdKTile) / kBwdQRows;       // first query tile that can see these keys
    const int nqt = (len + kBwdQRows - 1) / kBwdQRows;   // query tiles of the sequence
    const int nst = (nqt - qt0) * nquads;                // stages: (query tile, head quad)
    const int hsh = l >> 4, hpc = l & 15;                // DMA lane: head of the row, physical chunk
    // stage z: query tile qt0 + z / nquads, heads kvh*grp + 4*(z % nquads) + 0..3.
    // Wave w loads token rows 8w .. 8w+7 of Q and of dO, and one of the four
    // lse/delta pieces (4-byte loads: 2 heads x 32 queries each): 17 loads.
    auto issue = [&](uint8_t* qbuf, uint8_t* dbuf, float* lbuf, int z) {
        const int qt = qt0 + z / nquads;
        const int hq0 = kvh * grp + 4 * (z % nquads);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * wu + j;  // token row of the tile
            const uint32_t vo = (uint32_t)((int64_t)(qt * kBwdQRows + r) * qstride * 2) +
                                (uint32_t)((hq0 + hsh) * 256) + (uint32_t)((hpc ^ (r & 15)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(qbuf + r * kBwdRow), 16, vo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(dbuf + r * kBwdRow), 16, vo, 0, 0, 0);
        }
        {
            // piece wu: lse (wu < 2) or delta rows of heads 2*(wu%2) .. +1, 32 queries each
            const int hh = 2 * (wu & 1) + (l >> 5);
            const int64_t e = (int64_t)(hq0 + hh) * a.T + t0 + qt * kBwdQRows + (l & 31);
            const uint32_t vo = (uint32_t)(e * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wu < 2 ? rl : rt,
                                                     (lds_void*)(lbuf + (wu >> 1) * 128 + 64 * (wu & 1)), 4, vo,
                                                     0, 0, 0);
        }
    };

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dk[db] = dv[db] = f32x16{};
    const float c = a.scale * kLog2e;

    auto stage = [&](const uint8_t* qbuf, const uint8_t* dbuf, const float* lbuf, int z) {
        const int qt = qt0 + z / nquads;
        // (an opaque zero in the bases: the fragment addresses are formed per
        // stage instead of occupying registers across the loop)
        int oz;
        asm volatile("s_mov_b32 %0, 0" : "=s"(oz));
        const uint8_t* qh = qbuf + hw * 256 + oz;  // this wave's head within the 1 KiB rows
        const uint8_t* dh = dbuf + hw * 256 + oz;
        f32x16 st = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            st = mfma32x32x16(frag_row<kBwdRow>(qh, l32, 2 * kk + lh), frag_row(g_bkv, l32, 2 * kk + lh), st);
            dp = mfma32x32x16(frag_row<kBwdRow>(dh, l32, 2 * kk + lh),
                              frag_row(g_bkv + kBwdKTile * 256, l32, 2 * kk + lh), dp);
        }
        // lane: key column, query rows 8*(v/4) + 4*lh + v%4 of the tile.  Only
        // the diagonal tile and the sequence's last tile need a mask: the
        // causal one, and rows past the sequence (zero Q and dO rows, but the
        // lse and delta of other tokens).  Keys past the sequence are not stored.
        if (qt == kt || (qt + 1) * kBwdQRows > len) {
            const int lim = key - qt * kBwdQRows - 4 * lh, end = len - qt * kBwdQRows - 4 * lh;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 8 * (v >> 2) + (v & 3);
                if (r < lim || r >= end) st[v] = kNegInf;
            }
        }
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
                dp[v] = p * (dp[v] - dl[e]);  // dS
            }
        }
        const bf16x8 p0 = rows_as_b(st, 0), p1 = rows_as_b(st, 1);
        const bf16x8 s0 = rows_as_b(dp, 0), s1 = rows_as_b(dp, 1);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            dv[db] = mfma32x32x16(p0, frag_tr<kBwdRow>(dh, db * 32, 0), dv[db]);
            dv[db] = mfma32x32x16(p1, frag_tr<kBwdRow>(dh, db * 32, 16), dv[db]);
            dk[db] = mfma32x32x16(s0, frag_tr<kBwdRow>(qh, db * 32, 0), dk[db]);
            dk[db] = mfma32x32x16(s1, frag_tr<kBwdRow>(qh, db * 32, 16), dk[db]);
        }
    };

    if (nst > 0) {
        issue(g_bq0, g_bd0, g_bl0, 0);
        for (int z = 0; z < nst; z += 2) {
            if (z + 1 < nst) {
                issue(g_bq1, g_bd1, g_bl1, z + 1);
                wait_vmcnt<17>();  // stage z landed (stage z+1 in flight)
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
            stage(g_bq0, g_bd0, g_bl0, z);
            lds_barrier();
            if (z + 1 >= nst) break;
            if (z + 2 < nst) {
                issue(g_bq0, g_bd0, g_bl0, z + 2);
                wait_vmcnt<17>();
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
            stage(g_bq1, g_bd1, g_bl1, z + 1);
            lds_barrier();
        }
    }

    // Sum the 4 query-head partials of each key block through LDS (free now):
    // heads 2, 3 -> 0, 1, then 1 -> 0.  A partial is 128 values per lane,
    // stored [value][lane] (32 KiB, one of the four 32 KiB buffers).
    auto slot = [&](int i) -> float* {
        return reinterpret_cast<float*>(i == 0 ? g_bq0 : i == 1 ? g_bq1 : i == 2 ? g_bd0 : g_bd1);
    };
    auto put = [&](float* b) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                b[(db * 16 + v) * 64 + l] = dk[db][v];
                b[(64 + db * 16 + v) * 64 + l] = dv[db][v];
            }
    };
    auto take = [&](const float* b) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                dk[db][v] += b[(db * 16 + v) * 64 + l];
                dv[db][v] += b[(64 + db * 16 + v) * 64 + l];
            }
    };
    const int hwu = wu & 3, kbu = wu >> 2;
    if (hwu >= 2) put(slot(2 * kbu + hwu - 2));
    __syncthreads();
    if (hwu < 2) take(slot(2 * kbu + hwu));
    __syncthreads();
    if (hwu == 1) put(slot(kbu));
    __syncthreads();
    if (hwu != 0) return;
    take(slot(kbu));

    // lane: dim db*32 + l%32, keys 8*(v/4) + 4*lh + v%4 of the key block
    bf16* DK = static_cast<bf16*>(a.out2);
    bf16* DV = static_cast<bf16*>(a.out3);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int kr = kt * kBwdKTile + kb * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (kr >= len) continue;
        const int64_t ro = (t0 + kr) * kstride + kvh * kHeadDim + l32;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            DK[ro + db * 32] = to_bf16(dk[db][v] * a.scale);
            DV[ro + db * 32] = to_bf16(dv[db][v]);
        }
    }
}

}  // namespace

hipError_t launch_attention_fwd(const AttnArgs& a, const SeqTable& s0, hipStream_t st) {
    SeqTable s = s0;
    s.tiles[0] = 0;
    for (int i = 0; i < s.n; ++i) s.tiles[i + 1] = s.tiles[i] + (s.off[i + 1] - s.off[i] + kAttnQTile - 1) / kAttnQTile;
    if (s.tiles[s.n] == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)s.tiles[s.n], (unsigned)(a.n_q / 4)), dim3(512), 0, st, a, s);
    return hipGetLastError();
}

hipError_t launch_attention_bwd(const AttnArgs& a, const SeqTable& s0, hipStream_t st) {
    SeqTable s = s0;
    s.tiles[0] = 0;
    for (int i = 0; i < s.n; ++i) s.tiles[i + 1] = s.tiles[i] + (s.off[i + 1] - s.off[i] + kAttnQTile - 1) / kAttnQTile;
    if (s.tiles[s.n] == 0) return hipSuccess;
    const int64_t lanes = a.T * a.n_q * 16;
    hipLaunchKernelGGL(attn_delta_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)s.tiles[s.n], (unsigned)(a.n_q / 4)), dim3(512), 0, st, a,
                       s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    SeqTable sk = s0;
    sk.tiles[0] = 0;
    for (int i = 0; i < sk.n; ++i)
        sk.tiles[i + 1] = sk.tiles[i] + (sk.off[i + 1] - sk.off[i] + kBwdKTile - 1) / kBwdKTile;
    hipLaunchKernelGGL(attn_bwd_dkv_kernel, dim3((unsigned)sk.tiles[sk.n], (unsigned)a.n_kv), dim3(256), 0, st, a,
                       sk);
    return hipGetLastError();
}

}  // namespace plora
