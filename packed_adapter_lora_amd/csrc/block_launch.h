// block_launch.h -- internal launch interface of the decoder-block kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace plora {

constexpr int kMaxSeq = 256;       // sequences per call (the table travels as kernel arguments)
constexpr int kRmsMaxChunks = 8;   // RMSNorm rows up to 8 * 256 * 8 = 16384 elements
constexpr int kHeadDim = 128;      // attention head size
constexpr int kAttnQTile = 64;     // query rows per attention work item
constexpr int kAttnKTile = 64;     // keys per attention step (forward and dQ)
constexpr int kAttnKTileB = 64;    // keys per work item of the dK/dV pass

// Sequence table: tokens off[s] .. off[s+1]-1 form sequence s; tiles[s] is the
// prefix of per-sequence work-item counts (filled per kernel); lmax > 0 (the
// most items of one sequence) selects the attention kernels' level order.
struct SeqTable {
    int32_t n;
    int32_t lmax;
    int32_t off[kMaxSeq + 1];
    int32_t tiles[kMaxSeq + 1];
};

struct RmsFwdArgs {
    const void* x;     // [T][D] bf16
    const void* res;   // optional [T][D] bf16 added to x first
    const void* w;     // [D] bf16
    void* xs_out;      // [T][D] bf16: x + res (when res is given)
    void* h;           // [T][D] bf16
    float* rstd;       // [T]
    int64_t D;
    float eps;
};

struct RmsBwdArgs {
    const void* dy[3];  // up to three [T][D] bf16 gradients of h, summed (dy[1], dy[2] may be null)
    const void* x;      // [T][D] bf16: the normalised input
    const void* w;      // [D] bf16
    const float* rstd;  // [T]
    const void* dres;   // optional [T][D] bf16 gradient added to dx (residual branch)
    void* dx;           // [T][D] bf16
    int64_t D;
};

struct RopeArgs {
    void* x;  // [T][heads][128] bf16, rotated in place
    int64_t T;
    int32_t heads;
    int32_t inverse;     // 1: apply the transpose (backward)
    float inv_freq[64];  // base^(-2i/128)
    SeqTable seq;
};

struct AttnArgs {
    const void* q;   // [T][n_q][128] bf16
    const void* k;   // [T][n_kv][128] bf16
    const void* v;   // [T][n_kv][128] bf16
    const void* o;   // forward output / backward input [T][n_q][128] bf16
    const void* dO;  // [T][n_q][128] bf16 (backward)
    void* out;       // forward: O; dQ pass: dQ
    void* out2;      // dK/dV pass: dK
    void* out3;      // dK/dV pass: dV
    float* lse;      // [n_q][T] log-sum-exp (natural log) of the scaled scores
    float* delta;    // [n_q][T] rowsum(dO * O) (backward)
    int64_t T;
    int32_t n_q, n_kv;
    float scale;     // 1 / sqrt(128)
};

hipError_t launch_rmsnorm_fwd(const RmsFwdArgs& a, int64_t T, hipStream_t st);
hipError_t launch_rmsnorm_bwd(const RmsBwdArgs& a, int64_t T, hipStream_t st);
hipError_t launch_rope(const RopeArgs& a, hipStream_t st);
hipError_t launch_swiglu_fwd(const void* g, const void* u, void* out, int64_t n, hipStream_t st);
hipError_t launch_swiglu_bwd(const void* da, const void* g, const void* u, void* dg, void* du, int64_t n,
                             hipStream_t st);
hipError_t launch_add(const void* x, const void* y, void* out, int64_t n, hipStream_t st);
hipError_t launch_attention_fwd(const AttnArgs& a, const SeqTable& s, hipStream_t st);
hipError_t launch_attention_bwd(const AttnArgs& a, const SeqTable& s, hipStream_t st);
// (the dK/dV pass alone; part of launch_attention_bwd, after delta)
hipError_t launch_attention_dkv(const AttnArgs& a, const SeqTable& s, hipStream_t st);

}  // namespace plora
