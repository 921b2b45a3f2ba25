/*
 * plora_block.h -- C ABI of the kernels of the Llama-3 decoder block that
 * surrounds the packed LoRA projections (see plora.h): RMSNorm, rotary
 * embedding, causal grouped-query attention, SwiGLU and the residual add,
 * forward and backward.
 *
 * LoRA puts a trainable low-rank branch on the weights of every Transformer
 * block [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理
 * 与PEFT实现] of the LLaMA-3 models the pages fine-tune [PLoRA technical
 * summary (gist.science, arXiv 2508.02932), 结果].  The pages do not print the
 * block; its layers follow the public Llama 3 definitions (8B: hidden 4096,
 * 32 query heads and 8 key/value heads of 128, MLP 14336, RMSNorm eps 1e-5,
 * rotary base 500000):
 *
 *   rmsnorm      h = x / sqrt(mean(x^2) + eps) * w          (per row of D)
 *   rope         pairs (i, i+64) of every 128-wide head rotated by
 *                pos * base^(-2i/128), pos = index within the sequence
 *   attention    o = softmax(q k^T / sqrt(128), causal within each sequence) v,
 *                query head j reads key/value head j / (n_q / n_kv)
 *   swiglu       a = silu(g) * u,  silu(g) = g / (1 + exp(-g))
 *
 * Conventions (all entry points).  Tensors are bf16, row-major, contiguous,
 * device memory, 16-byte aligned, unless stated; per-row statistics are fp32.
 * Kernels compute in fp32 and round each output element to bf16 once (round
 * to nearest even).  Sequence tables (seq_offsets) are HOST arrays of
 * n_seq + 1 int64: 0 = o_0 <= ... <= o_n_seq = T, 1 <= n_seq <= 256, T < 2^31.
 * The library allocates nothing, never synchronises and enqueues only on
 * `stream`; validation happens before anything is enqueued.  Return values and
 * plora_last_error() as in plora.h.
 */
#ifndef PLORA_BLOCK_H
#define PLORA_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#include "plora.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PLORA_MAX_SEQUENCES 256

/* RMSNorm forward over rows of D (a multiple of 8, <= 16384), T rows.
 *   res == NULL: xs = x.  Otherwise xs = bf16(x + res) is written to xs_out
 *   (the residual stream) and normalised.  h = xs * rstd * w and
 *   rstd = 1 / sqrt(mean(xs^2) + eps) (fp32 [T]) are written. */
int plora_rmsnorm_fwd(int64_t T, int64_t D, const void* x, const void* res, const void* w, float eps,
                      void* xs_out, void* h, float* rstd, void* stream);

/* RMSNorm backward (w frozen): with g = (dy0 + dy1 + dy2) * w (dy1, dy2 may be
 * NULL: the gradients of every projection that reads h, summed in fp32),
 *   dx = dres + rstd * g - x * rstd^3 * mean(g * x)
 * (dres may be NULL: the gradient arriving through the residual branch).  x
 * and rstd are the forward's xs and rstd. */
int plora_rmsnorm_bwd(int64_t T, int64_t D, const void* dy0, const void* dy1, const void* dy2, const void* x,
                      const void* w, const float* rstd, const void* dres, void* dx, void* stream);

/* Rotary embedding in place on x [T, heads, 128]; inverse != 0 applies the
 * transpose (the backward of the forward rotation). */
int plora_rope(int64_t T, int32_t heads, int32_t n_seq, const int64_t* seq_offsets, float base, int inverse,
               void* x, void* stream);

/* a = silu(g) * u over n elements (n a multiple of 8). */
int plora_swiglu_fwd(int64_t n, const void* g, const void* u, void* a, void* stream);

/* dg = da * u * s * (1 + g (1 - s)), du = da * silu(g), s = sigmoid(g). */
int plora_swiglu_bwd(int64_t n, const void* da, const void* g, const void* u, void* dg, void* du, void* stream);

/* The MLP's down projection backward with the SwiGLU backward behind it:
 * da = dY W_m^T + concat_i[ s_i G_i A_i^T ] (the packed operator's dX, as
 * plora_backward_dx computes it [PLoRA technical summary, 方法论 › 2],
 * rounded to bf16), then dg and du from da, g and u as plora_swiglu_bwd
 * computes them; da itself is never stored.  desc describes the down
 * projection (d_in = the MLP width, d_out = hidden; bf16 only, else
 * PLORA_ERR_DTYPE); g and u [T][d_in] are the forward's gate and up
 * activations; dg and du [T][d_in] are overwritten and must not overlap any
 * input or each other (dg is also the shrink's scratch, as dX is for
 * plora_backward_dx);
 * G as for plora_backward_dx.  dg and du are bitwise what plora_backward_dx
 * followed by plora_swiglu_bwd writes: on shapes with the pipelined GEMM the
 * GEMM's epilogue applies the SwiGLU backward to its rounded output, on the
 * others the two kernels run one after the other. */
int plora_backward_dx_swiglu(const plora_desc* desc, const void* dY, const void* W, const void* A, const void* B,
                             const void* g, const void* u, void* dg, void* du, float* G, void* stream);

/* out = x + y over n elements (n a multiple of 8); out may alias x or y. */
int plora_add(int64_t n, const void* x, const void* y, void* out, void* stream);

/* Causal grouped-query attention forward.  q [T, n_q, 128], k and v
 * [T, n_kv, 128]; n_q a multiple of 4 and of n_kv, (n_q / n_kv) a multiple of
 * 4.  Writes o [T, n_q, 128] and lse (fp32 [n_q, T]: the natural log-sum-exp
 * of each query's scaled scores, kept for the backward). */
int plora_attention_fwd(int32_t n_seq, const int64_t* seq_offsets, int32_t n_q, int32_t n_kv, const void* q,
                        const void* k, const void* v, void* o, float* lse, void* stream);

/* Causal grouped-query attention backward: from dO (and the forward's q, k,
 * v, o, lse) writes dq, dk, dv (shapes of q, k, v).  `delta` is fp32
 * scratch of n_q * T floats (contents on entry do not matter; it holds
 * rowsum(dO * o) afterwards).  PLORA_ERR_SHAPE when a sequence's queries
 * exceed 2 GiB or n_q * T * 4 bytes reach 2 GiB. */
int plora_attention_bwd(int32_t n_seq, const int64_t* seq_offsets, int32_t n_q, int32_t n_kv, const void* q,
                        const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
                        void* dk, void* dv, float* delta, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PLORA_BLOCK_H */
