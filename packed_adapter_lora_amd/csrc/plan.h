// plan.h -- host-side planning for the packed multi-LoRA operator.
//
// Plain C++ (no HIP headers): descriptor validation, the per-adapter tables
// every kernel receives by value (segment offsets, rank prefix, H/G block
// offsets, scales), and the work maps that cut each adapter's tokens into
// fixed-size tiles so that a launch covers all adapters at once and no tile
// straddles two adapters.  Tiling runs along tokens and hidden features,
// never along the small rank dimension [PLoRA technical summary (gist.science,
// arXiv 2508.02932), 方法论 > 2. LoRA 执行引擎 > 算子设计].
#pragma once

#include <cstddef>
#include <cstdint>

#include "plora.h"

namespace plora {

constexpr int kMaxN = PLORA_MAX_ADAPTERS;
constexpr int kMaxRank = PLORA_MAX_RANK;

// Token rows per shrink work unit: 32 (one wavefront) in the general kernel,
// 128 (one workgroup of four wavefronts) in the pipelined one.
constexpr int kShrinkRows = 32;
constexpr int kShrinkTileRows = 128;

// Per-adapter table, passed to kernels by value (about 1.8 KiB of kernel
// arguments; N <= 64 keeps it well under the 4 KiB argument limit, so no
// device-side metadata buffer or host-to-device copy is needed).
struct SegTable {
    int32_t n;       // adapters
    int32_t rmax;    // largest rank
    int64_t T;       // tokens
    int64_t off[kMaxN + 1];   // segment offsets o_i
    int64_t hoff[kMaxN + 1];  // H/G block offsets: sum_{j<i} n_j r_j
    int32_t roff[kMaxN + 1];  // rank prefix R_off[i]
    int32_t voff[kMaxN + 1];  // prefix of ranks rounded up to 16: adapter i's ranks in a
                              // 16-aligned rank space (a k-step of 16 never spans two adapters)
    int32_t rank[kMaxN];
    float scale[kMaxN];       // alpha_i / r_i (fp32)
};

// Prefix sums of per-adapter work units (tiles or token chunks).
struct WorkMap {
    int32_t pre[kMaxN + 1];
};

// Weight-gradient plan for one reduction (dA over d_in or dB over d_out).
struct WgradPlan {
    int32_t chunk_tokens;      // tokens per work item (fixed per feature width)
    int32_t col_tiles;         // ceil(D / 256)
    WorkMap chunks;            // token chunks per adapter
    int64_t part_off[kMaxN + 1];  // fp32 element offset of adapter i's partials
    int64_t part_elems;        // total partial elements
    int64_t ft_off[kMaxN + 1];    // bf16 element offset of adapter i's transposed H/G block
    int64_t ft_elems;          // sum_i r_i * pad64(n_i): one of the hi / lo arrays
};

// Tokens of adapter i rounded up to a multiple of 64 (rows of the transposed
// bf16 H/G blocks the weight-gradient kernel streams).
constexpr int64_t pad64(int64_t n) { return (n + 63) & ~int64_t(63); }

// Returns a plora_status; checks only the descriptor (no pointers to data).
int validate_desc(const plora_desc* d, const char** why);

// Fills the segment table of a validated descriptor.
void build_segtable(const plora_desc* d, SegTable* s);

// Shrink tiles: ceil(n_i / rows) per adapter.  Returns the total.
int32_t build_shrink_map(const SegTable& s, WorkMap* m, int rows = kShrinkRows);

// K order of the pipelined shrink.  Every H/G element is the sum of kShrinkSlices
// K quarters, each accumulated in k order from zero, combined as
// ((q0 + q1) + q2) + q3 in fp32 (K / 64 >= 4 stages; fewer stages: one
// sequential sum).  Whether the quarters run one after another in one
// wavefront or in four workgroups (K slices, whose fp32 partials go to the
// adapter's own rows of the output activation, which the GEMM overwrites
// afterwards, and are then added in slice order) therefore changes no bit, so
// the split can follow the size of the grid.
//
// K slices of the pipelined shrink for adapter i (n tokens, rank r) over K:
// kShrinkSlices when the split is wanted (split_all, or a single 128-token
// tile) and the slices' fp32 partials (kShrinkSlices x n x r) fit in the
// adapter's rows of the scratch activation (row_bytes bytes per token; 0 = no
// scratch), else 1.
constexpr int kShrinkSlices = 4;
constexpr int shrink_quarters(int64_t K) { return K / 64 >= kShrinkSlices ? kShrinkSlices : 1; }
constexpr int shrink_slices(int64_t n, int r, int64_t K, int64_t row_bytes, bool split_all) {
    return (row_bytes > 0 && n >= 1 && (split_all || n <= kShrinkTileRows) && K % 64 == 0 &&
            K / 64 >= 2 * kShrinkSlices && (int64_t)4 * kShrinkSlices * r <= row_bytes)
               ? kShrinkSlices
               : 1;
}

// Work items of the pipelined shrink: tiles of `rows` tokens x shrink_slices()
// per adapter.  Returns the total; *any_split tells whether a partial sum
// pass is needed.
int32_t build_shrink_pipe_map(const SegTable& s, WorkMap* m, int64_t K, int64_t row_bytes, bool* any_split,
                              int rows, bool split_all);

// Token-chunk size of the weight-gradient reduction over a feature width D.
// It depends only on D, so an adapter's reduction order is the same whether
// it is packed with others or run alone.
int32_t wgrad_chunk_tokens(int64_t D);

// Plan one weight-gradient reduction over feature width D.  Adapters whose
// tokens span more than one chunk get fp32 partials (chunks * r_i * D
// elements); the rest are written directly.
void build_wgrad_plan(const SegTable& s, int64_t D, WgradPlan* p);

// Workspace of plora_backward_dAdB, each region rounded up to 256 bytes:
// [dA partials fp32][dB partials fp32][G^T hi, lo bf16][H^T hi, lo bf16].
struct WorkspaceLayout {
    size_t part_a, part_b, ft_g, ft_h, total;  // byte offsets and total
};
WorkspaceLayout workspace_layout(const SegTable& s, int64_t d_in, int64_t d_out);
size_t workspace_bytes(const SegTable& s, int64_t d_in, int64_t d_out);

// Workspace of the shared-input dA pass over np projections: np blocks of
// partials (part_stride bytes apart, from 0), then np hi/lo transposes of
// the G's (ft_stride bytes apart, from ft_base).
struct SharedDaLayout {
    size_t part_stride, ft_base, ft_stride, total;
};
SharedDaLayout dA_shared_layout(const SegTable& s, int64_t d_in, int np);

}  // namespace plora
