// api_block.hip -- C ABI of the decoder-block kernels (see include/plora_block.h).
//
// Every entry point validates its arguments on the host before anything is
// enqueued, then launches on the caller's stream.  Nothing is allocated.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "api_util.h"
#include "block_launch.h"
#include "plora.h"
#include "plora_block.h"

namespace plora {
namespace {

int bad_shape(const std::string& why) { return fail(PLORA_ERR_SHAPE, why); }

// Validates a host sequence table and copies it into the kernel-argument form.
int seq_table(int32_t n_seq, const int64_t* off, int64_t* T, SeqTable* s) {
    if (!off) return fail(PLORA_ERR_NULL, "seq_offsets is required");
    if (n_seq < 1 || n_seq > kMaxSeq) return fail(PLORA_ERR_SEGMENTS, "n_seq must be in 1..256");
    if (off[0] != 0) return fail(PLORA_ERR_SEGMENTS, "seq_offsets[0] must be 0");
    for (int i = 0; i < n_seq; ++i)
        if (off[i + 1] < off[i]) return fail(PLORA_ERR_SEGMENTS, "seq_offsets must be non-decreasing");
    if (off[n_seq] >= (int64_t(1) << 31)) return fail(PLORA_ERR_SEGMENTS, "T must be below 2^31");
    s->n = n_seq;
    for (int i = 0; i <= n_seq; ++i) s->off[i] = (int32_t)off[i];
    for (int i = 0; i <= n_seq; ++i) s->tiles[i] = 0;
    *T = off[n_seq];
    return PLORA_OK;
}

int heads_ok(int32_t n_q, int32_t n_kv, int64_t T) {
    if (n_q <= 0 || n_kv <= 0 || n_q % n_kv != 0 || (n_q / n_kv) % 4 != 0)
        return bad_shape("n_q must be a positive multiple of n_kv with n_q / n_kv a multiple of 4");
    if (T * (int64_t)n_q * kHeadDim * 2 >= (int64_t(1) << 40)) return bad_shape("tensor too large");
    return PLORA_OK;
}

}  // namespace
}  // namespace plora

using namespace plora;

extern "C" {

int plora_rmsnorm_fwd(int64_t T, int64_t D, const void* x, const void* res, const void* w, float eps, void* xs_out,
                      void* h, float* rstd, void* stream) {
    try {
        if (T < 0 || D <= 0 || D % 8 != 0 || D > kRmsMaxChunks * 256 * 8)
            return bad_shape("D must be a positive multiple of 8 up to 16384, T >= 0");
        if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(PLORA_ERR_HPARAM, "eps must be finite and >= 0");
        if (T == 0) return PLORA_OK;
        if (!x || !w || !h || !rstd || (res && !xs_out)) return fail(PLORA_ERR_NULL, "x, w, h, rstd (and xs_out with res)");
        if (misaligned(x) || misaligned(res) || misaligned(w) || misaligned(xs_out) || misaligned(h) || misaligned(rstd))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        const RmsFwdArgs a{x, res, w, xs_out, h, rstd, D, eps};
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("norm", st, [&] { return launch_rmsnorm_fwd(a, T, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "rmsnorm launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_rmsnorm_bwd(int64_t T, int64_t D, const void* dy0, const void* dy1, const void* dy2, const void* x,
                      const void* w, const float* rstd, const void* dres, void* dx, void* stream) {
    try {
        if (T < 0 || D <= 0 || D % 8 != 0 || D > kRmsMaxChunks * 256 * 8)
            return bad_shape("D must be a positive multiple of 8 up to 16384, T >= 0");
        if (T == 0) return PLORA_OK;
        if (!dy0 || !x || !w || !rstd || !dx) return fail(PLORA_ERR_NULL, "dy0, x, w, rstd and dx are required");
        if (misaligned(dy0) || misaligned(dy1) || misaligned(dy2) || misaligned(x) || misaligned(w) ||
            misaligned(rstd) || misaligned(dres) || misaligned(dx))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        const RmsBwdArgs a{{dy0, dy1, dy2}, x, w, rstd, dres, dx, D};
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("norm", st, [&] { return launch_rmsnorm_bwd(a, T, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "rmsnorm launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_rope(int64_t T, int32_t heads, int32_t n_seq, const int64_t* seq_offsets, float base, int inverse, void* x,
               void* stream) {
    try {
        RopeArgs a{};
        int64_t Ts = 0;
        int rc = seq_table(n_seq, seq_offsets, &Ts, &a.seq);
        if (rc) return rc;
        if (Ts != T) return fail(PLORA_ERR_SEGMENTS, "seq_offsets must end at T");
        if (heads <= 0) return bad_shape("heads must be positive");
        if (!(base > 1.0f) || !std::isfinite(base)) return fail(PLORA_ERR_HPARAM, "base must be finite and > 1");
        if (T == 0) return PLORA_OK;
        if (!x) return fail(PLORA_ERR_NULL, "x is required");
        if (misaligned(x)) return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        a.x = x;
        a.T = T;
        a.heads = heads;
        a.inverse = inverse ? 1 : 0;
        for (int i = 0; i < 64; ++i) a.inv_freq[i] = (float)std::pow((double)base, -2.0 * i / kHeadDim);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("rope", st, [&] { return launch_rope(a, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "rope launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_swiglu_fwd(int64_t n, const void* g, const void* u, void* a, void* stream) {
    try {
        if (n < 0 || n % 8 != 0) return bad_shape("n must be a non-negative multiple of 8");
        if (n == 0) return PLORA_OK;
        if (!g || !u || !a) return fail(PLORA_ERR_NULL, "g, u and a are required");
        if (misaligned(g) || misaligned(u) || misaligned(a))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("swiglu", st, [&] { return launch_swiglu_fwd(g, u, a, n, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "swiglu launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_swiglu_bwd(int64_t n, const void* da, const void* g, const void* u, void* dg, void* du, void* stream) {
    try {
        if (n < 0 || n % 8 != 0) return bad_shape("n must be a non-negative multiple of 8");
        if (n == 0) return PLORA_OK;
        if (!da || !g || !u || !dg || !du) return fail(PLORA_ERR_NULL, "da, g, u, dg and du are required");
        if (misaligned(da) || misaligned(g) || misaligned(u) || misaligned(dg) || misaligned(du))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("swiglu", st, [&] { return launch_swiglu_bwd(da, g, u, dg, du, n, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "swiglu launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_add(int64_t n, const void* x, const void* y, void* out, void* stream) {
    try {
        if (n < 0 || n % 8 != 0) return bad_shape("n must be a non-negative multiple of 8");
        if (n == 0) return PLORA_OK;
        if (!x || !y || !out) return fail(PLORA_ERR_NULL, "x, y and out are required");
        if (misaligned(x) || misaligned(y) || misaligned(out))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("add", st, [&] { return launch_add(x, y, out, n, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "add launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_attention_fwd(int32_t n_seq, const int64_t* seq_offsets, int32_t n_q, int32_t n_kv, const void* q,
                        const void* k, const void* v, void* o, float* lse, void* stream) {
    try {
        SeqTable s{};
        int64_t T = 0;
        int rc = seq_table(n_seq, seq_offsets, &T, &s);
        if (rc) return rc;
        if ((rc = heads_ok(n_q, n_kv, T))) return rc;
        for (int i = 0; i < n_seq; ++i)
            if ((int64_t)(s.off[i + 1] - s.off[i]) * n_kv * kHeadDim * 2 >= (int64_t(1) << 31))
                return bad_shape("a sequence's keys exceed 2 GiB");
        if (T == 0) return PLORA_OK;
        if (!q || !k || !v || !o || !lse) return fail(PLORA_ERR_NULL, "q, k, v, o and lse are required");
        if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        AttnArgs a{};
        a.q = q;
        a.k = k;
        a.v = v;
        a.out = o;
        a.lse = lse;
        a.T = T;
        a.n_q = n_q;
        a.n_kv = n_kv;
        a.scale = (float)(1.0 / std::sqrt((double)kHeadDim));
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("attn_fwd", st, [&] { return launch_attention_fwd(a, s, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "attention launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

int plora_attention_bwd(int32_t n_seq, const int64_t* seq_offsets, int32_t n_q, int32_t n_kv, const void* q,
                        const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
                        void* dk, void* dv, float* delta, void* stream) {
    try {
        SeqTable s{};
        int64_t T = 0;
        int rc = seq_table(n_seq, seq_offsets, &T, &s);
        if (rc) return rc;
        if ((rc = heads_ok(n_q, n_kv, T))) return rc;
        for (int i = 0; i < n_seq; ++i)
            if ((int64_t)(s.off[i + 1] - s.off[i]) * n_q * kHeadDim * 2 >= (int64_t(1) << 31))
                return bad_shape("a sequence's queries exceed 2 GiB");
        if (T * (int64_t)n_q * 4 >= (int64_t(1) << 31)) return bad_shape("lse and delta exceed 2 GiB");
        if (T == 0) return PLORA_OK;
        if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !delta)
            return fail(PLORA_ERR_NULL, "q, k, v, o, lse, dO, dq, dk, dv and delta are required");
        if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) || misaligned(dO) ||
            misaligned(dq) || misaligned(dk) || misaligned(dv) || misaligned(delta))
            return fail(PLORA_ERR_ALIGN, "device pointers must be 16-byte aligned");
        AttnArgs a{};
        a.q = q;
        a.k = k;
        a.v = v;
        a.o = o;
        a.dO = dO;
        a.out = dq;
        a.out2 = dk;
        a.out3 = dv;
        a.lse = const_cast<float*>(lse);
        a.delta = delta;
        a.T = T;
        a.n_q = n_q;
        a.n_kv = n_kv;
        a.scale = (float)(1.0 / std::sqrt((double)kHeadDim));
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = timed("attn_bwd", st, [&] { return launch_attention_bwd(a, s, st); });
        return e == hipSuccess ? PLORA_OK : hip_fail(e, "attention launch");
    } catch (...) {
        return fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

}  // extern "C"
