// plan.cpp -- host-side planning for the packed multi-LoRA operator.
#include "plan.h"

#include <cmath>
#include <cstring>

namespace plora {

int validate_desc(const plora_desc* d, const char** why) {
    const char* dummy;
    if (!why) why = &dummy;
    *why = "";
    if (!d) { *why = "descriptor is NULL"; return PLORA_ERR_NULL; }
    if (d->n_adapters < 0 || d->n_adapters > kMaxN) {
        *why = "n_adapters must be in 0..64";
        return PLORA_ERR_ADAPTERS;
    }
    if (d->dtype != PLORA_F32 && d->dtype != PLORA_BF16) { *why = "unknown dtype"; return PLORA_ERR_DTYPE; }
    if (d->n_tokens < 0) { *why = "n_tokens must be >= 0"; return PLORA_ERR_SHAPE; }
    if (d->d_in <= 0 || d->d_out <= 0 || (d->d_in % 8) != 0 || (d->d_out % 8) != 0) {
        *why = "d_in and d_out must be positive multiples of 8";
        return PLORA_ERR_SHAPE;
    }
    if (d->d_in > (int64_t(1) << 30) || d->d_out > (int64_t(1) << 30)) {
        *why = "d_in/d_out too large";
        return PLORA_ERR_SHAPE;
    }
    const int n = d->n_adapters;
    if (n == 0) return PLORA_OK;
    if (!d->seg_offsets || !d->ranks || !d->alphas) {
        *why = "seg_offsets, ranks and alphas are required when n_adapters > 0";
        return PLORA_ERR_NULL;
    }
    if (d->seg_offsets[0] != 0 || d->seg_offsets[n] != d->n_tokens) {
        *why = "seg_offsets must start at 0 and end at n_tokens";
        return PLORA_ERR_SEGMENTS;
    }
    for (int i = 0; i < n; ++i) {
        if (d->seg_offsets[i + 1] < d->seg_offsets[i]) {
            *why = "seg_offsets must be non-decreasing";
            return PLORA_ERR_SEGMENTS;
        }
        if (d->ranks[i] < 1 || d->ranks[i] > kMaxRank) { *why = "rank must be in 1..128"; return PLORA_ERR_RANK; }
        if (!std::isfinite(d->alphas[i])) { *why = "alpha must be finite"; return PLORA_ERR_ALPHA; }
    }
    return PLORA_OK;
}

void build_segtable(const plora_desc* d, SegTable* s) {
    std::memset(s, 0, sizeof(*s));
    s->n = d->n_adapters;
    s->T = d->n_tokens;
    int64_t h = 0;
    int32_t r = 0, v = 0;
    int32_t rmax = 0;
    for (int i = 0; i < s->n; ++i) {
        s->off[i] = d->seg_offsets[i];
        s->hoff[i] = h;
        s->roff[i] = r;
        s->voff[i] = v;
        v += (d->ranks[i] + 15) & ~15;
        s->rank[i] = d->ranks[i];
        s->scale[i] = d->alphas[i] / (float)d->ranks[i];
        h += (d->seg_offsets[i + 1] - d->seg_offsets[i]) * (int64_t)d->ranks[i];
        r += d->ranks[i];
        if (d->ranks[i] > rmax) rmax = d->ranks[i];
    }
    s->off[s->n] = d->n_tokens;
    s->hoff[s->n] = h;
    s->roff[s->n] = r;
    s->voff[s->n] = v;
    s->rmax = rmax;
}

int32_t build_shrink_map(const SegTable& s, WorkMap* m, int rows) {
    int32_t t = 0;
    for (int i = 0; i < s.n; ++i) {
        m->pre[i] = t;
        const int64_t ni = s.off[i + 1] - s.off[i];
        t += (int32_t)((ni + rows - 1) / rows);
    }
    m->pre[s.n] = t;
    return t;
}

int32_t build_shrink_pipe_map(const SegTable& s, WorkMap* m, int64_t K, int64_t row_bytes, bool* any_split,
                              int rows, bool split_all) {
    int32_t t = 0;
    *any_split = false;
    for (int i = 0; i < s.n; ++i) {
        m->pre[i] = t;
        const int64_t ni = s.off[i + 1] - s.off[i];
        const int sl = shrink_slices(ni, s.rank[i], K, row_bytes, split_all);
        *any_split = *any_split || sl > 1;
        t += (int32_t)((ni + rows - 1) / rows) * sl;
    }
    m->pre[s.n] = t;
    return t;
}

int32_t wgrad_chunk_tokens(int64_t D) { return D > 8192 ? 2048 : 1024; }

void build_wgrad_plan(const SegTable& s, int64_t D, WgradPlan* p) {
    std::memset(p, 0, sizeof(*p));
    p->chunk_tokens = wgrad_chunk_tokens(D);
    p->col_tiles = (int32_t)((D + 255) / 256);
    int32_t c = 0;
    int64_t po = 0, fo = 0;
    for (int i = 0; i < s.n; ++i) {
        const int64_t ni = s.off[i + 1] - s.off[i];
        const int32_t ci = (int32_t)((ni + p->chunk_tokens - 1) / p->chunk_tokens);
        p->chunks.pre[i] = c;
        p->part_off[i] = po;
        p->ft_off[i] = fo;
        c += ci;
        if (ci > 1) po += (int64_t)ci * s.rank[i] * D;
        fo += (int64_t)s.rank[i] * pad64(ni);
    }
    p->chunks.pre[s.n] = c;
    p->part_off[s.n] = po;
    p->part_elems = po;
    p->ft_off[s.n] = fo;
    p->ft_elems = fo;
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(const SegTable& s, int64_t d_in, int64_t d_out) {
    WgradPlan a, b;
    build_wgrad_plan(s, d_in, &a);
    build_wgrad_plan(s, d_out, &b);
    WorkspaceLayout w;
    w.part_a = 0;
    w.part_b = w.part_a + round256((size_t)a.part_elems * 4);
    w.ft_g = w.part_b + round256((size_t)b.part_elems * 4);
    w.ft_h = w.ft_g + round256((size_t)a.ft_elems * 2 * 2);
    w.total = w.ft_h + round256((size_t)b.ft_elems * 2 * 2);
    return w;
}

size_t workspace_bytes(const SegTable& s, int64_t d_in, int64_t d_out) {
    return workspace_layout(s, d_in, d_out).total;
}

SharedDaLayout dA_shared_layout(const SegTable& s, int64_t d_in, int np) {
    WgradPlan a;
    build_wgrad_plan(s, d_in, &a);
    SharedDaLayout w;
    w.part_stride = round256((size_t)a.part_elems * 4);
    w.ft_base = (size_t)np * w.part_stride;
    w.ft_stride = round256((size_t)a.ft_elems * 2 * 2);
    w.total = w.ft_base + (size_t)np * w.ft_stride;
    return w;
}

}  // namespace plora
