"""CPU oracle of Rimuru's adjuster: how many experts to evict or add in a
round, and which ones (the digest "Rimuru: Unified Memory Management for
Modern LLM Serving via Elastic Expert Offloading", section "The adjuster: when
to evict an expert, and which one?").

TEST INFRASTRUCTURE.  Only tests/ may import this module.  The library's own
adjuster (paged_expert_weight_amd/csrc/adjuster.cpp) shares no code with it.

Plain Python, written step by step from the section's rules:
  * amounts: an expert takes 3 expert pages (W1, W3, W2).  Short of R_b pages
    -> evict ceil((R_b + 1) / 3) experts.  Otherwise fewer than 2 free pages
    F_b -> evict 1.  Otherwise more than 9 free -> add min(5, floor((F_b - 9) / 3)).
    Otherwise no change.
  * ranking: per layer, experts sorted by routing probability measured on
    sample routing.
  * selection: to grow, every layer nominates the next expert of its ranking
    that is not resident and the highest probability wins; to shrink, every
    layer nominates the last expert it keeps and the lowest wins.  A layer that
    already offloads offload_limit experts is left out of shrinking.

Readings where the section leaves a step open (listed in the design notes):
  * the routing probability of expert e is the fraction of sample tokens
    whose top-k contains e (count_e / T); ranking ties go to the lower id;
  * one expert is chosen at a time, and the chosen layer then nominates its
    next expert; equal probabilities go to the lower layer index;
  * a round either evicts or adds, never both (the three rules are exclusive).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

PAGES_PER_EXPERT = 3  # W1, W3 and W2 each take one expert page


def adjust_amounts(short_pages: int, free_pages: int) -> Tuple[int, int]:
    """(experts to evict, experts to add) for one round."""
    if short_pages < 0 or free_pages < 0:
        raise ValueError("page counts are non-negative")
    if short_pages > 0:
        need = short_pages + 1                      # cover the shortfall plus one page
        return -(-need // PAGES_PER_EXPERT), 0     # ceil
    if free_pages < 2:
        return 1, 0
    if free_pages > 9:
        return 0, min(5, (free_pages - 9) // PAGES_PER_EXPERT)
    return 0, 0


def rank_experts(topk_ids: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """Ranking of one layer from sample routing: (expert ids by descending
    routing probability, their probabilities).  topk_ids [T, k] int."""
    ids = np.asarray(topk_ids)
    T = ids.shape[0]
    counts = [0] * E
    for row in ids:
        for e in row:
            if 0 <= e < E:
                counts[int(e)] += 1
    order = sorted(range(E), key=lambda e: (-counts[e], e))
    prob = np.array([counts[e] / T if T else 0.0 for e in order], dtype=np.float32)
    return np.array(order, dtype=np.int32), prob


def select(ranking: np.ndarray, prob: np.ndarray, resident: Sequence[int], offload_limit: int,
           n_evict: int, n_add: int) -> Tuple[List[Tuple[int, int, int]], List[int]]:
    """Change list [(layer, expert, 1 add / 0 evict)] in decision order, and the
    new resident counts.  ranking/prob [L][E] in ranking order; resident[l] =
    size of layer l's resident top slice."""
    L, E = ranking.shape
    res = [int(r) for r in resident]
    out = []
    for _ in range(n_add):
        best_l, best_p = -1, None
        for l in range(L):
            if res[l] < E:
                p = float(prob[l][res[l]])
                if best_l < 0 or p > best_p:
                    best_l, best_p = l, p
        if best_l < 0:
            break
        out.append((best_l, int(ranking[best_l][res[best_l]]), 1))
        res[best_l] += 1
    for _ in range(n_evict):
        best_l, best_p = -1, None
        for l in range(L):
            if res[l] > 0 and E - res[l] < offload_limit:
                p = float(prob[l][res[l] - 1])
                if best_l < 0 or p < best_p:
                    best_l, best_p = l, p
        if best_l < 0:
            break
        res[best_l] -= 1
        out.append((best_l, int(ranking[best_l][res[best_l]]), 0))
    return out, res
