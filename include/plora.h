/*
 * plora.h -- C ABI of the packed multi-LoRA linear operator for AMD MI355X
 * (gfx950).
 *
 * The operator.  Many LoRA adapters, each with its own rank r_i, scale
 * s_i = alpha_i / r_i and token segment S_i = [o_i, o_{i+1}), train together
 * on one frozen linear layer W.  The LoRA branch is a down-projection A_i
 * (d_in -> r_i) followed by an up-projection B_i (r_i -> d_out), scaled by
 * alpha_i / r_i and added to the frozen layer's output
 * [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 深入理解LoRA：基本原理与PEFT实现];
 * W is frozen and only A and B receive gradients
 * [LoRA加速集成方案 (cloud.baidu.com), 四、工作原理 > 3. 反向传播阶段];
 * the adapters are packed on one shared base and their work is batched
 * instead of run adapter by adapter, covering the forward and the backward
 * gradient cases [PLoRA technical summary (gist.science, arXiv 2508.02932),
 * 方法论 > 2. LoRA 执行引擎 > 打包 LoRA 算子 / 算子设计].
 *
 * For a token t in S_i (math orientation: W_m = W^T is d_in x d_out,
 * A_i is d_in x r_i, B_i is r_i x d_out):
 *
 *   plora_forward        Y[t]  = X[t] W_m + s_i (X[t] A_i) B_i,  H_i[t] = X[t] A_i
 *   plora_backward_dx    dX[t] = dY[t] W_m^T + s_i (dY[t] B_i^T) A_i^T,
 *                        G_i[t] = dY[t] B_i^T
 *   plora_backward_dAdB  dA_i = s_i X[S_i]^T G_i,  dB_i = s_i H_i^T dY[S_i]
 *
 * Storage (row-major, contiguous, device memory, 16-byte aligned):
 *   X, dX  [T, d_in]        element type = desc.dtype
 *   Y, dY  [T, d_out]       element type = desc.dtype
 *   W      [d_out, d_in]    element type = desc.dtype (the nn.Linear weight;
 *                           W_m = W^T)
 *   A      [R, d_in]        rows R_off[i] .. R_off[i]+r_i-1 hold A_i^T
 *                           (column j of A_i is row R_off[i]+j), R = sum r_i,
 *                           R_off[i] = sum_{j<i} r_j
 *   B      [R, d_out]       rows R_off[i] .. hold B_i
 *   dA, dB fp32, laid out like A and B
 *   H, G   fp32, plora_h_elems() elements; block i starts at
 *          H_off[i] = sum_{j<i} n_j r_j and is [n_i, r_i] row-major
 *
 * Precision.  bf16: products of bf16 inputs are accumulated in fp32; H and G
 * are fp32; each element of Y and dX is rounded once (round to nearest even)
 * to bf16 from its fp32 accumulator; dA and dB are fp32.  f32: fp32 inputs,
 * fp32 arithmetic throughout (no reduced-precision matrix modes).
 *
 * Ownership and side effects.  The caller owns every buffer.  The library
 * allocates no device memory, keeps no per-call state, never synchronises and
 * enqueues work only on `stream` (a hipStream_t; NULL means the null stream):
 * kernels and nothing else (no memset, no copy), so a caller may capture a
 * sequence of calls into a HIP graph and replay it; the kernel arguments,
 * buffer addresses included, are those of the captured calls.
 * Host arrays in the descriptor are read during the call only.  Inputs are
 * never written.  Outputs (Y, H, dX, G, dA, dB) are overwritten, not
 * accumulated (plora_backward_dAdB_acc can accumulate dA and dB).  One
 * training step calls plora_forward (writes H), then plora_backward_dx
 * (writes G), then plora_backward_dAdB (reads H and G), then, to update the
 * adapters, plora_adamw_step.
 *
 * Errors.  Every entry point returns PLORA_OK (0) or a negative plora_status.
 * All arguments are validated before anything is enqueued, so a call that
 * fails validation has no side effects.  After PLORA_ERR_HIP the stream may
 * hold part of the call's work.  plora_last_error() gives a message for the
 * last failure on the calling thread.  No C++ exception crosses this ABI.
 * Calls are reentrant; calls that share output buffers on overlapping
 * streams race, as any two kernels writing one buffer would.
 *
 * Environment.  PLORA_GEMM_TILE_P=128 or 256 forces the feature width of the
 * bf16 GEMM tiles of plora_forward / plora_backward_dx (by default a launch
 * mixes 256- and 128-wide tiles by a wave count), PLORA_SHRINK_TILE_ROWS=32 or
 * 128 the token rows of their shrink tiles, PLORA_SHRINK_SPLIT=0 or 1 whether
 * every adapter's shrink is split along K (not only single-tile adapters),
 * PLORA_WGRAD_COLS=128 or 256 the feature width of the weight-gradient
 * work items, and PLORA_GEMM_GROUP_Q=1, 2, 4 or 8 the token tiles per L2 group in
 * the GEMM's tile order (by default all are chosen per shape and device).
 * Results are bitwise the same either way.
 */
#ifndef PLORA_H
#define PLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLORA_ABI_VERSION 1
#define PLORA_MAX_ADAPTERS 64
#define PLORA_MAX_RANK 128

typedef enum {
    PLORA_OK = 0,
    PLORA_ERR_NULL = -1,      /* a required pointer is NULL */
    PLORA_ERR_SEGMENTS = -2,  /* offsets not 0 = o_0 <= ... <= o_N = n_tokens */
    PLORA_ERR_RANK = -3,      /* a rank outside 1..PLORA_MAX_RANK */
    PLORA_ERR_ALPHA = -4,     /* a non-finite alpha */
    PLORA_ERR_SHAPE = -5,     /* d_in/d_out not positive multiples of 8, n_tokens < 0 */
    PLORA_ERR_ADAPTERS = -6,  /* n_adapters outside 0..PLORA_MAX_ADAPTERS */
    PLORA_ERR_DTYPE = -7,     /* dtype not a plora_dtype */
    PLORA_ERR_WORKSPACE = -8, /* workspace smaller than plora_workspace_bytes() */
    PLORA_ERR_ALIGN = -9,     /* a device pointer not 16-byte aligned */
    PLORA_ERR_HIP = -10,      /* a HIP runtime call or kernel launch failed */
    PLORA_ERR_HPARAM = -11    /* an optimizer hyper-parameter out of range */
} plora_status;

typedef enum { PLORA_F32 = 0, PLORA_BF16 = 1 } plora_dtype;

/* Problem descriptor.  All pointers are HOST pointers.
 *   n_adapters   N, 0..64.  N = 0 runs the frozen path only (Y = X W_m,
 *                dX = dY W_m^T); H, G, A, B may then be NULL.
 *   dtype        plora_dtype of X, W, A, B, Y, dY, dX.
 *   n_tokens     T >= 0.  With T = 0 plora_forward and plora_backward_dx do
 *                nothing and plora_backward_dAdB writes dA = dB = 0.
 *   d_in, d_out  positive multiples of 8.
 *   seg_offsets  N+1 int64: o_0 = 0, non-decreasing, o_N = T; empty
 *                segments are allowed (that adapter gets dA_i = dB_i = 0).
 *   ranks        N int32 in 1..128.
 *   alphas       N finite floats; s_i = alphas[i] / ranks[i] in fp32. */
typedef struct {
    int32_t n_adapters;
    int32_t dtype;
    int64_t n_tokens;
    int64_t d_in;
    int64_t d_out;
    const int64_t* seg_offsets;
    const int32_t* ranks;
    const float* alphas;
} plora_desc;

/* Forward: Y = X W_m + concat_i[ s_i (X[S_i] A_i) B_i ], and H (fp32) for the
 * weight-gradient pass.  Y and H are overwritten; Y must not overlap any
 * input, since the call may first use an adapter's own rows of Y as scratch
 * (partial sums of H) before writing the result there. */
int plora_forward(const plora_desc* desc, const void* X, const void* W, const void* A,
                  const void* B, void* Y, float* H, void* stream);

/* Backward through the activations: dX = dY W_m^T + concat_i[ s_i G_i A_i^T ]
 * with G_i = dY[S_i] B_i^T, and G (fp32) for the weight-gradient pass.  dX
 * and G are overwritten; dX must not overlap any input (scratch as for Y). */
int plora_backward_dx(const plora_desc* desc, const void* dY, const void* W, const void* A,
                      const void* B, void* dX, float* G, void* stream);

/* Backward to the adapters: dA_i = s_i X[S_i]^T G_i and dB_i = s_i H_i^T dY[S_i]
 * (fp32, layouts of A and B), reducing over each adapter's tokens.  H and G are
 * the buffers written by plora_forward and plora_backward_dx.  `workspace`
 * must hold plora_workspace_bytes(desc) bytes (it may be NULL when that is
 * 0); its contents on entry do not matter.  The reduction order is fixed, so
 * results are bitwise reproducible run to run. */
int plora_backward_dAdB(const plora_desc* desc, const void* X, const void* dY, const float* H,
                        const float* G, float* dA, float* dB, void* workspace,
                        size_t workspace_bytes, void* stream);

/* plora_backward_dAdB with a choice of write mode.  accumulate = 0 behaves
 * exactly like plora_backward_dAdB.  accumulate != 0 adds this call's
 * gradients to dA and dB instead of overwriting them: each element becomes
 * old + (s_i-scaled gradient of this call) in fp32, and adapters with no
 * tokens in this call are left unchanged.  This sums the micro-batches of one
 * optimizer step (gradient accumulation); the caller zeroes dA and dB, or
 * passes accumulate = 0, for the first micro-batch.  Either output may be
 * skipped: dA = NULL (G is then not read) computes dB only, dB = NULL (H not
 * read) dA only; not both. */
int plora_backward_dAdB_acc(const plora_desc* desc, const void* X, const void* dY, const float* H,
                            const float* G, float* dA, float* dB, void* workspace,
                            size_t workspace_bytes, int accumulate, void* stream);

/* Projections that read the same input.  In a Transformer block that carries
 * LoRA on every projection [LLM+LoRA微调加速技术原理解析 (m.youleyou.com),
 * 深入理解LoRA：基本原理与PEFT实现], the query, key and value projections read
 * one activation X, and the gate and up projections another; with the same
 * adapters (segments, ranks, alphas) on each, their shrinks H_p = X A_p and
 * their gradients dA_p = s_i X^T G_p can share one pass over X, which is most
 * of their memory traffic (the packed operators are tiled for memory-access
 * efficiency [PLoRA technical summary (gist.science, arXiv 2508.02932),
 * 方法论 > 2. LoRA 执行引擎 > 算子设计]).  np = 1, 2 or 3 projections; `desc`
 * describes each of them (only d_in, the segments, ranks, alphas and dtype are
 * used); A[p], H[p], G[p], dA[p] are the per-projection buffers with the
 * layouts above (HOST arrays of np device pointers).  Every output element is
 * bitwise the value the single-projection entry points give.
 *
 * plora_shrink_shared: H[p] = X A[p] (fp32, overwritten), p < np. */
int plora_shrink_shared(const plora_desc* desc, const void* X, int np, const void* const* A, float* const* H,
                        void* stream);

/* The forward of one projection whose H was computed already (by
 * plora_shrink_shared or plora_forward): Y = X W_m + concat_i[ s_i H_i B_i ].
 * Y is overwritten (bitwise what plora_forward writes); H is read only. */
int plora_forward_expand(const plora_desc* desc, const void* X, const void* W, const void* B, void* Y,
                         const float* H, void* stream);

/* dA[p]_i = s_i X[S_i]^T G[p]_i for p < np (fp32, layout of A; overwritten, or
 * accumulated as in plora_backward_dAdB_acc).  `workspace` must hold
 * plora_workspace_bytes_dA_shared(desc, np) bytes (NULL when that is 0); its
 * contents on entry do not matter. */
int plora_backward_dA_shared(const plora_desc* desc, const void* X, int np, const float* const* G,
                             float* const* dA, void* workspace, size_t workspace_bytes, int accumulate,
                             void* stream);

/* Workspace bytes of plora_backward_dA_shared (0 for PLORA_F32, np outside
 * 1..3 or an invalid descriptor). */
size_t plora_workspace_bytes_dA_shared(const plora_desc* desc, int np);

/* plora_backward_dAdB_acc without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * or training loops, harnesses that forbid hipMalloc.  Nothing is allocated
 * per call: the workspace lives in a library-owned device array of
 * PLORA_NOALLOC_SCRATCH_BYTES (256 MiB), one per device, held from the
 * library's first use of that device until the process ends.  A descriptor
 * whose plora_workspace_bytes() exceeds that size returns PLORA_ERR_WORKSPACE
 * before anything is enqueued.  The array is not cleared between calls (the
 * kernels write whatever they read from it).  All calls on one device share
 * the array: calls that overlap on one GPU (other streams, or threads
 * without ordering between their calls) race.  Otherwise the arguments,
 * results and errors are those of plora_backward_dAdB_acc; the device is the
 * current one. */
#define PLORA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int plora_backward_dAdB_noalloc(const plora_desc* desc, const void* X, const void* dY, const float* H,
                                const float* G, float* dA, float* dB, int accumulate, void* stream);

/* Per-adapter AdamW over the packed adapter panels.
 *
 * The fine-tuning loop that trains the LoRA parameters uses AdamW with
 * PyTorch's defaults (lr 1e-3, betas 0.9 / 0.999, eps 1e-8, weight decay
 * 0.01) [LLM+LoRA微调加速技术原理解析 (m.youleyou.com), 5. 设定优化器和正则项];
 * packed jobs differ in learning rate among other settings [PLoRA technical
 * summary (gist.science, arXiv 2508.02932), 结果], so the learning rate, the
 * weight decay and the step count are per adapter.  For every element of
 * adapter i's rows (R_off[i] .. R_off[i]+r_i-1) of both panels, in fp32,
 * with t = step[i] (decoupled weight decay; Loshchilov & Hutter, ICLR 2019):
 *
 *   p <- p (1 - lr_i wd_i)
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - (lr_i / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 *
 * The per-adapter factors (1 - lr wd, lr / (1 - beta1^t), 1 / sqrt(1 -
 * beta2^t)) are formed in double on the host and rounded to fp32.
 * step[i] = 0 leaves adapter i's parameters and moments untouched. */
typedef struct {
    float beta1;                /* 0 <= beta1 < 1 */
    float beta2;                /* 0 <= beta2 < 1 */
    float eps;                  /* finite, > 0 */
    const float* lr;            /* HOST, N values: finite, >= 0 */
    const float* weight_decay;  /* HOST, N values: finite, >= 0 */
    const int64_t* step;        /* HOST, N values: >= 0 (1-based step count; 0 = skip) */
} plora_adamw_config;

/* One AdamW step for all adapters of `desc` (only n_adapters, ranks, dtype,
 * d_in and d_out are used; the descriptor must still be valid).
 *   PA, mA, vA  fp32 [R, d_in]: master copy of A and its moments, updated in place
 *   PB, mB, vB  fp32 [R, d_out]: the same for B
 *   dA, dB      fp32 gradients (layouts of A and B), read only
 *   A, B        desc.dtype copies of the updated PA / PB for the operator
 *               (bf16: round to nearest even; f32: a copy); either may be NULL
 *               (not written) and, for f32, may be the same buffer as PA / PB.
 * All device pointers 16-byte aligned.  N = 0 is a no-op. */
int plora_adamw_step(const plora_desc* desc, const plora_adamw_config* cfg, float* PA, float* PB, float* mA,
                     float* vA, float* mB, float* vB, const float* dA, const float* dB, void* A, void* B,
                     void* stream);

/* The operator's copies of fp32 master panels: A = PA and B = PB in
 * desc.dtype (bf16: each element rounded to nearest even; f32: a copy).
 * Mixed-precision training keeps the adapters as fp32 masters and runs the
 * operator on their bf16 copies [LoRA加速集成方案 (cloud.baidu.com), 三、核心组件
 * > 2. 硬件加速 (mixed precision) and 七、使用建议]; plora_adamw_step writes the
 * copies itself, this call is for masters changed by anything else.
 *   PA  fp32 [R, d_in], PB fp32 [R, d_out] (read only)
 *   A   desc.dtype [R, d_in], B desc.dtype [R, d_out] (overwritten; must not
 *       overlap PA / PB)
 * Only n_adapters, ranks, dtype, d_in and d_out of `desc` are used (it must
 * still be valid).  All pointers 16-byte aligned.  N = 0 is a no-op. */
int plora_cast_panels(const plora_desc* desc, const float* PA, const float* PB, void* A, void* B, void* stream);

/* Number of fp32 elements of H (and of G): sum_i n_i r_i.  Returns 0 for an
 * invalid descriptor. */
size_t plora_h_elems(const plora_desc* desc);

/* Bytes of workspace plora_backward_dAdB needs for this descriptor: the fp32
 * partial sums of adapters whose tokens are split across work items and the
 * bf16 hi/lo transposes of H and G (bf16 only; 0 for PLORA_F32 and when no
 * adapter has tokens).  Returns 0 for an invalid descriptor. */
size_t plora_workspace_bytes(const plora_desc* desc);

/* Validates a descriptor without touching the GPU; returns a plora_status. */
int plora_validate(const plora_desc* desc);

/* Human-readable name of a plora_status. */
const char* plora_status_string(int status);

/* Message for the last failed call on this thread ("" if none). */
const char* plora_last_error(void);

/* PLORA_ABI_VERSION of the loaded library. */
int plora_version(void);

/* Hash of the sources and compile flags the library was built from (16 hex
 * digits, or "unstamped" for a build that did not pass one), so a caller can
 * tell whether a prebuilt library matches the sources beside it. */
const char* plora_source_hash(void);

/* Kernel timing.  With profiling on, the library records a HIP event pair
 * on the call's stream around every kernel it launches (kernel classes:
 * "shrink", "gemm_fwd", "gemm_bwd", "wgrad", "reduce", "adamw").  After the caller has
 * synchronised the stream, plora_profile_read returns the number of launches
 * and their summed duration in milliseconds for one class.  Profiling is a
 * process-wide switch meant for benchmarks: while it is on, the launches of
 * every thread are recorded, one call at a time under a process-wide lock. */
int plora_profile_enable(int on);
int plora_profile_read(const char* kernel_class, int* launches, double* total_ms);
void plora_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* PLORA_H */
