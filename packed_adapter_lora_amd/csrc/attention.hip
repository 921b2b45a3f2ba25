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

// byte offset of 16-byte chunk c of row r in a tile of 256-byte rows
__device__ __forceinline__ int swz256(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

__device__ __forceinline__ bf16x8 frag_row(const uint8_t* tile, int r, int c) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + swz256(r, c)));
}

// Transposed read: lane l gets column d0 + l%32 of rows k0 + 4h .. +3 and
// k0 + 8 + 4h .. +3 (h = l/32), the key order of a score block's lane.
__device__ __forceinline__ bf16x8 frag_tr(const uint8_t* tile, int d0, int k0) {
    const int l = lane_id(), L = l & 15, g = l >> 4;
    const int d = d0 + 16 * (g & 1) + 4 * (L & 3);
    const int k = k0 + 4 * (g >> 1) + (L >> 2);
    typedef __attribute__((address_space(3))) bf16x4v lds_v4;
    const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(tile + swz256(k, d >> 3) + (d & 7) * 2));
    const bf16x4v hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(tile + swz256(k + 8, d >> 3) + (d & 7) * 2));
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

// Work item -> (sequence, tile within it), heaviest tiles first.
__device__ __forceinline__ void tile_of(const SeqTable& s, int item, int& seq, int& tile) {
    const int w = s.tiles[s.n] - 1 - item;
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
    float m = kNegInf, lsum = 0.0f;
    const float c = a.scale * kLog2e;

    // one 64-key tile from LDS, as two halves of 32 keys
    auto tile = [&](const uint8_t* kb, const uint8_t* vb, int kt) {
        const bool diag = kt == qt;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            f32x16 st = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) st = mfma32x32x16(frag_row(kb, hb * 32 + l32, 2 * kk + lh), qf[kk], st);
            float mx = kNegInf;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = kt * kAttnKTile + hb * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                float x = st[v] * c;
                if ((diag && key > qi) || key >= len) x = kNegInf;
                st[v] = x;
                mx = fmaxf(mx, x);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m, mx);
            // a row with no visible key yet keeps mn = -inf: shift by 0 instead
            const float sh = mn == kNegInf ? 0.0f : mn;
            const float alpha = exp2f(m - sh);
            float ps = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2f(st[v] - sh);
                st[v] = p;
                ps += p;
            }
            ps += __shfl_xor(ps, 32);
            lsum = lsum * alpha + ps;
            m = mn;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
            const bf16x8 p0 = rows_as_b(st, 0), p1 = rows_as_b(st, 1);
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
        if (lh == 0) a.lse[(int64_t)head * a.T + t0 + qi] = (m + log2f(lsum)) / kLog2e;
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

hipError_t launch_attention_bwd(const AttnArgs&, const SeqTable&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace plora
