/*
 * plora_oracle.c -- fp64 CPU oracle for the packed multi-LoRA linear operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes, and where the pages define it
 * -----------------------------------------------
 *  - LoRA branch: a down-projection A (d -> r) and an up-projection B (r -> d)
 *    run beside the frozen weight; the branch output is scaled by alpha/r and
 *    summed with the frozen layer's output.  A starts Gaussian, B starts at
 *    zero.  [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), section
 *    深入理解LoRA：基本原理与PEFT实现]
 *  - Only A and B receive gradients; W stays frozen, so no dW is produced.
 *    [LoRA加速集成方案 (cloud.baidu.com), 四、工作原理 > 3. 反向传播阶段]
 *  - Packed execution: many adapters train at once on one shared frozen base;
 *    the packed operators batch what the naive method computes adapter by
 *    adapter, so each adapter's result is its own computation on its own
 *    tokens.  [PLoRA technical summary (gist.science, arXiv 2508.02932),
 *    方法论 and 方法论 > 2. LoRA 执行引擎 > 打包 LoRA 算子]
 *
 * Adapter i owns the token segment S_i = [o_i, o_{i+1}) and has rank r_i and
 * scale s_i = alpha_i / r_i.  With W_m = W^T the math-orientation weight
 * (d_in x d_out) and A_i (d_in x r_i), B_i (r_i x d_out):
 *
 *   H_i[t-o_i] = X[t] A_i                    (1 x r_i)     for t in S_i
 *   Y[t]       = X[t] W_m + s_i H_i[t-o_i] B_i
 *   G_i[t-o_i] = dY[t] B_i^T                 (1 x r_i)
 *   dX[t]      = dY[t] W_m^T + s_i G_i[t-o_i] A_i^T
 *   dA_i       = s_i X[S_i]^T G_i            (d_in x r_i)
 *   dB_i       = s_i H_i^T dY[S_i]           (r_i x d_out)
 *
 * These are the exact derivatives of L = sum(dY * Y) with respect to X, A_i
 * and B_i.
 *
 * Storage (all row-major, fp64):
 *   X [T, d_in], dY [T, d_out], W [d_out, d_in] (nn.Linear weight, = W_m^T),
 *   A [R, d_in] with row R_off[i]+j holding column j of A_i,
 *   B [R, d_out] with row R_off[i]+j holding row j of B_i,
 *   dA, dB like A, B;  H, G: block i at H_off[i] = sum_{j<i} n_j r_j is
 *   [n_i, r_i].
 *
 * Evaluation order: plain loops, one adapter and one token at a time; every
 * sum runs over its index in ascending order (k for X W, n for dY W^T, j for
 * the rank sums, t for dA/dB).  Sums that a reader might write as a dot
 * product over a strided operand are written as running row accumulations
 * (acc[k] += a * w[k]); the order of additions per element is the same.  The
 * scale is applied after the rank sum (Y = base + s * (h B)) and after the
 * token sum (dA = s * (X^T G)).  OpenMP only splits independent rows or
 * independent output columns across threads; it never changes the order of
 * additions, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_NULL -1
#define ORACLE_ERR_SEGMENTS -2
#define ORACLE_ERR_RANK -3
#define ORACLE_ERR_ALPHA -4
#define ORACLE_ERR_SHAPE -5
#define ORACLE_ERR_ADAPTERS -6
#define ORACLE_ERR_NOMEM -7

#define ORACLE_MAX_ADAPTERS 64
#define ORACLE_MAX_RANK 128

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of threads later calls may use (n >= 1); results do not depend on it
 * (threads split independent rows and output columns only). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Mathematical preconditions of the problem: a partition of the T tokens
 * into N contiguous, possibly empty, segments (o_0 = 0, o_N = T); ranks in
 * 1..128; finite alphas.  With N = 0 there is no adapter and every token takes
 * the frozen path only. */
int oracle_check(int n, int64_t T, const int64_t* off, const int32_t* ranks, const double* alphas,
                 int64_t d_in, int64_t d_out) {
    if (n < 0 || n > ORACLE_MAX_ADAPTERS) return ORACLE_ERR_ADAPTERS;
    if (n > 0 && (!off || !ranks || !alphas)) return ORACLE_ERR_NULL;
    if (d_in <= 0 || d_out <= 0 || T < 0) return ORACLE_ERR_SHAPE;
    if (n == 0) return ORACLE_OK; /* no adapters: every token takes the frozen path only */
    if (off[0] != 0 || off[n] != T) return ORACLE_ERR_SEGMENTS;
    for (int i = 0; i < n; ++i) {
        if (off[i + 1] < off[i]) return ORACLE_ERR_SEGMENTS;
        if (ranks[i] < 1 || ranks[i] > ORACLE_MAX_RANK) return ORACLE_ERR_RANK;
        if (!isfinite(alphas[i])) return ORACLE_ERR_ALPHA;
    }
    return ORACLE_OK;
}

int64_t oracle_h_elems(int n, const int64_t* off, const int32_t* ranks) {
    int64_t s = 0;
    for (int i = 0; i < n; ++i) s += (off[i + 1] - off[i]) * (int64_t)ranks[i];
    return s;
}

/* h[j] = sum_k x[k] * A[j][k], k ascending (one token's down-projection). */
static void down_proj(const double* x, const double* Ai, int r, int64_t d, double* h) {
    for (int j = 0; j < r; ++j) {
        const double* a = Ai + (int64_t)j * d;
        double acc = 0.0;
        for (int64_t k = 0; k < d; ++k) acc += x[k] * a[k];
        h[j] = acc;
    }
}

/* out[c] = sum_j h[j] * P[j][c], j ascending (one token's up-projection). */
static void up_proj(const double* h, const double* Pi, int r, int64_t d, double* out) {
    for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
    for (int j = 0; j < r; ++j) {
        const double hj = h[j];
        const double* p = Pi + (int64_t)j * d;
        for (int64_t c = 0; c < d; ++c) out[c] += hj * p[c];
    }
}

/*
 * Computes any subset of {Y, H, dX, G, dA, dB}: pass NULL for outputs that are
 * not wanted.  Inputs that no requested output needs may be NULL
 * (Y: X, W, A, B;  H: X, A;  dX: dY, W, A, B;  G: dY, B;  dA: X, dY, B;
 * dB: X, A, dY).  Returns 0 or a negative error code.
 */
int oracle_packed_lora(int n, int64_t T, const int64_t* off, const int32_t* ranks,
                       const double* alphas, int64_t d_in, int64_t d_out,
                       const double* X, const double* dY, const double* W,
                       const double* A, const double* B,
                       double* Y, double* H, double* dX, double* G, double* dA, double* dB) {
    int rc = oracle_check(n, T, off, ranks, alphas, d_in, d_out);
    if (rc) return rc;
    const int need_h = (n > 0 && (Y || H || dB)) ? 1 : 0;
    const int need_g = (n > 0 && (dX || G || dA)) ? 1 : 0;
    if ((need_h && (!X || !A)) || (need_g && (!dY || !B)) || ((Y || dX) && !W) ||
        (Y && !X) || (dX && !dY) || (n > 0 && ((Y && !B) || (dX && !A))) ||
        (dA && !X) || (dB && !dY))
        return ORACLE_ERR_NULL;

    /* Frozen path for every token, whichever adapter it belongs to:
     * Y[t][c] = sum_k X[t][k] W_m[k][c] = sum_k X[t][k] W[c][k];
     * dX[t][k] = sum_c dY[t][c] W[c][k], accumulated c ascending. */
    if (Y) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* x = X + t * d_in;
            for (int64_t c = 0; c < d_out; ++c) {
                const double* w = W + c * d_in;
                double acc = 0.0;
                for (int64_t k = 0; k < d_in; ++k) acc += x[k] * w[k];
                Y[t * d_out + c] = acc;
            }
        }
    }
    if (dX) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            double* dx = dX + t * d_in;
            const double* dy = dY + t * d_out;
            for (int64_t k = 0; k < d_in; ++k) dx[k] = 0.0;
            for (int64_t c = 0; c < d_out; ++c) {
                const double g = dy[c];
                const double* w = W + c * d_in;
                for (int64_t k = 0; k < d_in; ++k) dx[k] += g * w[k];
            }
        }
    }

    int64_t r_off = 0, h_off = 0;
    for (int i = 0; i < n; ++i) {
        const int r = ranks[i];
        const double s = alphas[i] / (double)r;
        const int64_t o0 = off[i], ni = off[i + 1] - off[i];
        const double* Ai = A ? A + r_off * d_in : NULL;   /* r rows of d_in */
        const double* Bi = B ? B + r_off * d_out : NULL;  /* r rows of d_out */
        double* Hi = NULL;
        double* Gi = NULL;
        double* h_tmp = NULL;
        double* g_tmp = NULL;
        if (ni > 0 && need_h) {
            if (H) Hi = H + h_off;
            else { h_tmp = (double*)malloc(sizeof(double) * (size_t)(ni * r)); Hi = h_tmp; }
            if (!Hi) return ORACLE_ERR_NOMEM;
        }
        if (ni > 0 && need_g) {
            if (G) Gi = G + h_off;
            else { g_tmp = (double*)malloc(sizeof(double) * (size_t)(ni * r)); Gi = g_tmp; }
            if (!Gi) { free(h_tmp); return ORACLE_ERR_NOMEM; }
        }

        /* Per-token branch work for the tokens of this adapter. */
        if (ni > 0) {
#pragma omp parallel
            {
                double* row = (double*)malloc(sizeof(double) * (size_t)(d_in > d_out ? d_in : d_out));
#pragma omp for schedule(static)
                for (int64_t u = 0; u < ni; ++u) {
                    const int64_t t = o0 + u;
                    if (need_h) down_proj(X + t * d_in, Ai, r, d_in, Hi + u * r);
                    if (need_g) down_proj(dY + t * d_out, Bi, r, d_out, Gi + u * r);
                    if (Y) {
                        up_proj(Hi + u * r, Bi, r, d_out, row);
                        for (int64_t c = 0; c < d_out; ++c) Y[t * d_out + c] += s * row[c];
                    }
                    if (dX) {
                        up_proj(Gi + u * r, Ai, r, d_in, row);
                        for (int64_t k = 0; k < d_in; ++k) dX[t * d_in + k] += s * row[k];
                    }
                }
                free(row);
            }
        }

        /* Weight gradients: sums over this adapter's tokens, t ascending.
         * dA_i[k][j] lives at dA[(r_off + j) * d_in + k];
         * dB_i[j][c] lives at dB[(r_off + j) * d_out + c]. */
        if (dA) {
            double* dAi = dA + r_off * d_in;
#pragma omp parallel for schedule(static)
            for (int64_t k0 = 0; k0 < d_in; k0 += 64) {
                const int64_t k1 = k0 + 64 < d_in ? k0 + 64 : d_in;
                for (int j = 0; j < r; ++j)
                    for (int64_t k = k0; k < k1; ++k) dAi[(int64_t)j * d_in + k] = 0.0;
                for (int64_t u = 0; u < ni; ++u) {
                    const double* x = X + (o0 + u) * d_in;
                    for (int j = 0; j < r; ++j) {
                        const double g = Gi[u * r + j];
                        double* acc = dAi + (int64_t)j * d_in;
                        for (int64_t k = k0; k < k1; ++k) acc[k] += x[k] * g;
                    }
                }
                for (int j = 0; j < r; ++j)
                    for (int64_t k = k0; k < k1; ++k) dAi[(int64_t)j * d_in + k] *= s;
            }
        }
        if (dB) {
            double* dBi = dB + r_off * d_out;
#pragma omp parallel for schedule(static)
            for (int64_t c0 = 0; c0 < d_out; c0 += 64) {
                const int64_t c1 = c0 + 64 < d_out ? c0 + 64 : d_out;
                for (int j = 0; j < r; ++j)
                    for (int64_t c = c0; c < c1; ++c) dBi[(int64_t)j * d_out + c] = 0.0;
                for (int64_t u = 0; u < ni; ++u) {
                    const double* dy = dY + (o0 + u) * d_out;
                    for (int j = 0; j < r; ++j) {
                        const double h = Hi[u * r + j];
                        double* acc = dBi + (int64_t)j * d_out;
                        for (int64_t c = c0; c < c1; ++c) acc[c] += h * dy[c];
                    }
                }
                for (int j = 0; j < r; ++j)
                    for (int64_t c = c0; c < c1; ++c) dBi[(int64_t)j * d_out + c] *= s;
            }
        }
        free(h_tmp);
        free(g_tmp);
        r_off += r;
        h_off += ni * r;
    }
    return ORACLE_OK;
}
