// Rimuru's adjuster (the digest's section "The adjuster: when to evict an
// expert, and which one?"): host-side policy, run once per scheduling round.
//
// Amounts: an expert holds three expert pages (W1, W3, W2).  A shortfall of
// R_b pages evicts ceil((R_b + 1) / 3) experts (one page to spare); with no
// shortfall, fewer than 2 free pages evict one expert; more than 9 free pages
// add min(5, floor((F_b - 9) / 3)); in between nothing changes, so that free
// memory hovering at a threshold does not flip an expert out and back.
//
// Which experts: each layer has an offline ranking of its experts by routing
// probability and keeps the top slice of it resident.  Growing, every layer
// nominates its first expert outside the slice and the most probable
// nomination wins; shrinking, every layer nominates the last expert of its
// slice and the least probable wins, except layers that already offload
// offload_limit experts.  One expert is decided at a time (the chosen layer
// then nominates its next); equal probabilities go to the lower layer.
#include "internal.h"
#include "moe.h"

#include <algorithm>
#include <string>
#include <vector>

namespace {
constexpr int kPagesPerExpert = 3;
}

extern "C" {

int moe_adjust_amounts(int32_t short_pages, int32_t free_pages, int32_t *n_evict, int32_t *n_add)
{
    if (!n_evict || !n_add)
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "n_evict / n_add is null");
    if (short_pages < 0 || free_pages < 0)
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "page counts must be non-negative");
    *n_evict = 0;
    *n_add = 0;
    if (short_pages > 0) {
        const int64_t need = (int64_t)short_pages + 1;
        *n_evict = (int32_t)((need + kPagesPerExpert - 1) / kPagesPerExpert);
    } else if (free_pages < 2) {
        *n_evict = 1;
    } else if (free_pages > 9) {
        *n_add = std::min(5, (free_pages - 9) / kPagesPerExpert);
    }
    return MOE_OK;
}

int moe_rank_experts(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E, int32_t *ranking, float *prob)
{
    if (!ranking || !prob || (T > 0 && !topk_ids))
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "null pointer");
    if (T < 0 || k < 0 || E <= 0)
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "T, k must be >= 0 and E > 0");
    std::vector<int64_t> count(E, 0);
    for (int64_t i = 0; i < T * (int64_t)k; i++) {
        const int32_t e = topk_ids[i];
        if (e >= 0 && e < E) // the shared expert (id E) and invalid ids are not ranked
            count[e]++;
    }
    std::vector<int32_t> order(E);
    for (int32_t e = 0; e < E; e++)
        order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return count[a] > count[b]; });
    for (int32_t i = 0; i < E; i++) {
        ranking[i] = order[i];
        prob[i] = T > 0 ? (float)((double)count[order[i]] / (double)T) : 0.f;
    }
    return MOE_OK;
}

int moe_adjust_select(int32_t L, int32_t E, const int32_t *ranking, const float *prob, int32_t *resident,
                      int32_t offload_limit, int32_t n_evict, int32_t n_add, int32_t *out_layer,
                      int32_t *out_expert, int32_t *out_add, int32_t *n_out)
{
    if (!ranking || !prob || !resident || !n_out || ((n_evict > 0 || n_add > 0) && (!out_layer || !out_expert || !out_add)))
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "null pointer");
    if (L <= 0 || E <= 0 || n_evict < 0 || n_add < 0 || offload_limit < 0)
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "L, E must be > 0; counts and limit >= 0");
    if (n_evict > 0 && n_add > 0)
        return pmoe::set_error(MOE_ERR_INVALID_ARG, "a round either evicts or adds");
    std::vector<char> seen(E);
    for (int32_t l = 0; l < L; l++) {
        if (resident[l] < 0 || resident[l] > E)
            return pmoe::set_error(MOE_ERR_INVALID_ARG, ("resident[" + std::to_string(l) + "] out of [0, E]").c_str());
        std::fill(seen.begin(), seen.end(), 0);
        for (int32_t i = 0; i < E; i++) {
            const int32_t e = ranking[(int64_t)l * E + i];
            if (e < 0 || e >= E || seen[e])
                return pmoe::set_error(MOE_ERR_INVALID_ARG,
                                       ("ranking row " + std::to_string(l) + " is not a permutation of [0, E)").c_str());
            seen[e] = 1;
        }
    }
    int32_t n = 0;
    for (int32_t j = 0; j < n_add; j++) {
        int32_t best = -1;
        float bp = 0.f;
        for (int32_t l = 0; l < L; l++) {
            if (resident[l] >= E)
                continue;
            const float p = prob[(int64_t)l * E + resident[l]];
            if (best < 0 || p > bp) {
                best = l;
                bp = p;
            }
        }
        if (best < 0)
            break;
        out_layer[n] = best;
        out_expert[n] = ranking[(int64_t)best * E + resident[best]];
        out_add[n] = 1;
        resident[best]++;
        n++;
    }
    for (int32_t j = 0; j < n_evict; j++) {
        int32_t best = -1;
        float bp = 0.f;
        for (int32_t l = 0; l < L; l++) {
            if (resident[l] <= 0 || E - resident[l] >= offload_limit)
                continue;
            const float p = prob[(int64_t)l * E + resident[l] - 1];
            if (best < 0 || p < bp) {
                best = l;
                bp = p;
            }
        }
        if (best < 0)
            break;
        resident[best]--;
        out_layer[n] = best;
        out_expert[n] = ranking[(int64_t)best * E + resident[best]];
        out_add[n] = 0;
        n++;
    }
    *n_out = n;
    return MOE_OK;
}

} // extern "C"
