/*
 * plora_planner.h -- C ABI of the packing planner: which LoRA fine-tuning
 * jobs to train together on one GPU.
 *
 * The planner of the pages groups heterogeneous LoRA configurations into
 * packed tasks so as to minimise the total completion time (makespan) on a
 * fixed pool of GPUs; it treats the choice as a 0-1 knapsack variant (NP-hard)
 * and picks, one task after another, the group that packs the most work,
 * using a cost model of memory and throughput measured on the first
 * iterations [PLoRA technical summary (gist.science, arXiv 2508.02932),
 * 方法论 > 1. LoRA 打包规划器].  Here the pool is one GPU (parallelism 1), the
 * knapsack is solved exactly by dynamic programming instead of an ILP solver,
 * and the cost model is the one measured for the packed operator:
 *
 *   one step of a pack P costs  fixed_ms + sum_{k in P, still running} ms_per_step[k]
 *
 * (fixed_ms is the per-step cost that packing amortises: launches and the
 * tails of under-filled kernels; ms_per_step[k] is job k's own share, which
 * grows with its tokens per step).  A pack runs until its longest job is done,
 * so its cost is fixed_ms * max_k steps[k] + sum_k steps[k] * ms_per_step[k],
 * and the makespan is the sum over the packs, run one after another.
 *
 * Algorithm: sort jobs by steps (longest first); the longest unplanned job
 * opens a pack; a 0-1 knapsack over the memory left in the pack (item weight:
 * the job's memory rounded up to mem_quantum; value: its steps) chooses which
 * of the remaining jobs join it; repeat until every job is planned.
 */
#ifndef PLORA_PLANNER_H
#define PLORA_PLANNER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t steps;       /* optimizer steps the job runs (>= 1) */
    double mem_bytes;    /* device memory the job adds to a pack (> 0): adapter weights, optimizer
                            state, activations of its tokens */
    double ms_per_step;  /* the job's own share of a packed step (>= 0) */
} plora_job;

typedef struct {
    double mem_budget;   /* bytes one pack may use besides the shared frozen model (> 0) */
    double fixed_ms;     /* per-step cost shared by the jobs of a pack (>= 0) */
    double mem_quantum;  /* knapsack resolution in bytes (> 0; budget / quantum <= 2^20) */
} plora_pack_model;

/* Plans n jobs (1 <= n <= 65536).  Writes pack_of_job[k] (pack index, packs
 * numbered in the order they run, from 0), *n_packs and *makespan_ms (the
 * cost model's total).  Returns 0, or PLORA_ERR_NULL / PLORA_ERR_SHAPE /
 * PLORA_ERR_HPARAM (a job larger than the budget, a bad field) with a message
 * in plora_last_error(); nothing is written on failure.  Host only. */
int plora_plan_packs(const plora_job* jobs, int32_t n, const plora_pack_model* model, int32_t* pack_of_job,
                     int32_t* n_packs, double* makespan_ms);

/* The cost model's makespan of a given assignment (pack_of_job[k] in
 * 0 .. n_packs-1, every pack non-empty, each within the memory budget), or a
 * negative plora_status. */
double plora_plan_makespan(const plora_job* jobs, int32_t n, const plora_pack_model* model,
                           const int32_t* pack_of_job, int32_t n_packs);

#ifdef __cplusplus
}
#endif

#endif /* PLORA_PLANNER_H */
