// planner.cpp -- packing planner for LoRA fine-tuning jobs on one GPU (see
// include/plora_planner.h).  Plain C++, host only.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <string>
#include <vector>

#include "plora.h"
#include "plora_planner.h"

namespace plora {
int fail(int status, const std::string& why);  // api.hip
}

namespace {

int check(const plora_job* jobs, int32_t n, const plora_pack_model* m) {
    using plora::fail;
    if (!jobs || !m) return fail(PLORA_ERR_NULL, "jobs and model are required");
    if (n < 1 || n > 65536) return fail(PLORA_ERR_SHAPE, "n must be in 1..65536");
    if (!(m->mem_budget > 0) || !std::isfinite(m->mem_budget) || !(m->fixed_ms >= 0) || !std::isfinite(m->fixed_ms) ||
        !(m->mem_quantum > 0) || !std::isfinite(m->mem_quantum) || m->mem_budget / m->mem_quantum > double(1 << 20))
        return fail(PLORA_ERR_HPARAM, "model: budget > 0, fixed_ms >= 0, quantum > 0, budget / quantum <= 2^20");
    for (int k = 0; k < n; ++k) {
        const plora_job& j = jobs[k];
        if (j.steps < 1 || !(j.mem_bytes > 0) || !std::isfinite(j.mem_bytes) || !(j.ms_per_step >= 0) ||
            !std::isfinite(j.ms_per_step))
            return fail(PLORA_ERR_HPARAM, "job " + std::to_string(k) + ": steps >= 1, mem_bytes > 0, ms_per_step >= 0");
        if (j.mem_bytes > m->mem_budget)
            return fail(PLORA_ERR_HPARAM, "job " + std::to_string(k) + " needs more memory than the budget");
    }
    return PLORA_OK;
}

// Memory in quanta, rounded up (a job never takes less than it needs).
int64_t quanta(double bytes, double q) { return (int64_t)std::ceil(bytes / q - 1e-9); }

}  // namespace

extern "C" {

int plora_plan_packs(const plora_job* jobs, int32_t n, const plora_pack_model* m, int32_t* pack_of_job,
                     int32_t* n_packs, double* makespan_ms) {
    try {
        int rc = check(jobs, n, m);
        if (rc) return rc;
        if (!pack_of_job || !n_packs || !makespan_ms) return plora::fail(PLORA_ERR_NULL, "outputs are required");
        std::vector<int32_t> order(n);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
            if (jobs[a].steps != jobs[b].steps) return jobs[a].steps > jobs[b].steps;
            return jobs[a].mem_bytes > jobs[b].mem_bytes;
        });
        std::vector<int32_t> assign(n, -1);
        std::vector<char> done(n, 0);
        const int64_t cap_total = (int64_t)std::floor(m->mem_budget / m->mem_quantum + 1e-9);
        int packs = 0;
        double total = 0.0;
        for (int oi = 0; oi < n; ++oi) {
            const int anchor = order[oi];
            if (done[anchor]) continue;
            // candidates: unplanned jobs after the anchor (none runs longer than it)
            std::vector<int> cand;
            for (int oj = oi + 1; oj < n; ++oj)
                if (!done[order[oj]]) cand.push_back(order[oj]);
            const int64_t cap = cap_total - quanta(jobs[anchor].mem_bytes, m->mem_quantum);
            // 0-1 knapsack: best[c] = most steps packed within c quanta; keep[i][c] for reconstruction
            const size_t nc = cand.size();
            std::vector<int64_t> best((size_t)std::max<int64_t>(cap, 0) + 1, 0);
            std::vector<std::vector<char>> keep(nc);
            for (size_t i = 0; i < nc; ++i) {
                const int64_t w = quanta(jobs[cand[i]].mem_bytes, m->mem_quantum);
                const int64_t v = jobs[cand[i]].steps;
                keep[i].assign(best.size(), 0);
                for (int64_t c = (int64_t)best.size() - 1; c >= w; --c) {
                    if (best[(size_t)(c - w)] + v > best[(size_t)c]) {
                        best[(size_t)c] = best[(size_t)(c - w)] + v;
                        keep[i][(size_t)c] = 1;
                    }
                }
            }
            double cost = m->fixed_ms * (double)jobs[anchor].steps + jobs[anchor].ms_per_step * jobs[anchor].steps;
            assign[anchor] = packs;
            done[anchor] = 1;
            for (int64_t c = (int64_t)best.size() - 1, i = (int64_t)nc - 1; i >= 0 && c >= 0; --i) {
                if (!keep[(size_t)i][(size_t)c]) continue;
                const int k = cand[(size_t)i];
                assign[k] = packs;
                done[k] = 1;
                cost += jobs[k].ms_per_step * (double)jobs[k].steps;
                c -= quanta(jobs[k].mem_bytes, m->mem_quantum);
            }
            total += cost;
            ++packs;
        }
        for (int k = 0; k < n; ++k) pack_of_job[k] = assign[k];
        *n_packs = packs;
        *makespan_ms = total;
        return PLORA_OK;
    } catch (...) {
        return plora::fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

double plora_plan_makespan(const plora_job* jobs, int32_t n, const plora_pack_model* m, const int32_t* pack_of_job,
                           int32_t n_packs) {
    try {
        int rc = check(jobs, n, m);
        if (rc) return rc;
        if (!pack_of_job) return plora::fail(PLORA_ERR_NULL, "pack_of_job is required");
        if (n_packs < 1 || n_packs > n) return plora::fail(PLORA_ERR_SHAPE, "n_packs must be in 1..n");
        std::vector<int64_t> longest(n_packs, 0);
        std::vector<double> mem(n_packs, 0.0), own(n_packs, 0.0);
        for (int k = 0; k < n; ++k) {
            const int p = pack_of_job[k];
            if (p < 0 || p >= n_packs) return plora::fail(PLORA_ERR_SHAPE, "pack index out of range");
            longest[p] = std::max(longest[p], jobs[k].steps);
            mem[p] += (double)quanta(jobs[k].mem_bytes, m->mem_quantum);
            own[p] += jobs[k].ms_per_step * (double)jobs[k].steps;
        }
        double total = 0.0;
        const double cap = std::floor(m->mem_budget / m->mem_quantum + 1e-9);
        for (int p = 0; p < n_packs; ++p) {
            if (longest[p] == 0) return plora::fail(PLORA_ERR_SHAPE, "empty pack");
            if (mem[p] > cap) return plora::fail(PLORA_ERR_HPARAM, "a pack exceeds the memory budget");
            total += m->fixed_ms * (double)longest[p] + own[p];
        }
        return total;
    } catch (...) {
        return plora::fail(PLORA_ERR_HIP, "unexpected exception");
    }
}

}  // extern "C"
