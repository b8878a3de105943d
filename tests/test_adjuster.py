"""Adjuster rules and hot-expert ranking (the Rimuru digest's section "The
adjuster: when to evict an expert, and which one?").

CPU only: the oracle (oracle/adjuster.py) against the section's printed cases,
the rules' thresholds and closed forms of the greedy choices; then the
library's C++ adjuster against the oracle, bit for bit (integer change lists).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import adjuster as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adjuster_examples.json")


# ----------------------------------------------------------------------------- oracle pins

def test_printed_examples():
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        ev, add = ora.adjust_amounts(c["short_pages"], c["free_pages"])
        assert (ev, add) == (c["evict"], c["add"])
        if "pages_freed" in c:
            assert ev * g["pages_per_expert"] == c["pages_freed"]
            assert c["pages_freed"] - c["short_pages"] == c["cushion"]


@pytest.mark.parametrize("free,expect", [(0, (1, 0)), (1, (1, 0)), (2, (0, 0)), (5, (0, 0)), (9, (0, 0)),
                                         (10, (0, 0)), (11, (0, 0)), (12, (0, 1)), (15, (0, 2)), (24, (0, 5)),
                                         (30, (0, 5)), (1000, (0, 5))])
def test_free_page_thresholds(free, expect):
    """Shrink below 2 free pages, grow above 9, at most 5 per round, nothing in between."""
    assert ora.adjust_amounts(0, free) == expect


def test_shortfall_is_covered_with_one_spare_page_by_the_fewest_experts():
    for short in range(1, 200):
        for free in (0, 1, 5, 50):
            ev, add = ora.adjust_amounts(short, free)
            assert add == 0
            # brute force: the least n whose 3n pages cover the shortfall plus one
            n = next(m for m in range(1, 1000) if 3 * m >= short + 1)
            assert ev == n


def test_rejects_negative_counts():
    with pytest.raises(ValueError):
        ora.adjust_amounts(-1, 0)


def _rankings(seed, L, E, ties=False):
    g = np.random.default_rng(seed)
    ranking = np.stack([g.permutation(E) for _ in range(L)]).astype(np.int32)
    if ties:
        p = g.integers(0, 4, size=(L, E)).astype(np.float32) / 8
    else:
        p = g.random((L, E)).astype(np.float32)
    prob = -np.sort(-p, axis=1)  # each layer's list in descending probability
    return ranking, prob


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("ties", [False, True])
def test_grow_takes_the_most_probable_missing_experts(seed, ties):
    """Greedy nominations = the n_add best non-resident (layer, position) entries."""
    L, E = 5, 9
    ranking, prob = _rankings(seed, L, E, ties)
    g = np.random.default_rng(100 + seed)
    resident = g.integers(0, E + 1, size=L)
    for n_add in range(0, 12):
        out, res = ora.select(ranking, prob, resident, E, 0, n_add)
        cands = sorted(((-float(prob[l][i]), l, i) for l in range(L) for i in range(resident[l], E)))
        want = [(l, int(ranking[l][i]), 1) for _, l, i in cands[:n_add]]
        assert out == want
        assert all(res[l] - resident[l] == sum(1 for o in out if o[0] == l) for l in range(L))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("ties", [False, True])
def test_shrink_takes_the_least_probable_resident_experts(seed, ties):
    """Without an offload limit in the way: the n_evict lowest resident entries,
    each layer giving up the tail of its resident slice."""
    L, E = 4, 7
    ranking, prob = _rankings(seed, L, E, ties)
    g = np.random.default_rng(200 + seed)
    resident = g.integers(0, E + 1, size=L)
    for n_ev in range(0, 10):
        out, res = ora.select(ranking, prob, resident, E + 1, n_ev, 0)
        cands = sorted(((float(prob[l][i]), l, -i) for l in range(L) for i in range(resident[l])))
        want = [(l, int(ranking[l][-ni]), 0) for _, l, ni in cands[:n_ev]]
        assert out == want


def test_shrink_respects_the_offload_limit():
    L, E, limit = 6, 8, 3
    ranking, prob = _rankings(7, L, E)
    resident = [8, 7, 6, 5, 8, 8]  # layer 3 already offloads 3 experts
    out, res = ora.select(ranking, prob, resident, limit, 20, 0)
    for l in range(L):
        offloaded = E - res[l]
        assert offloaded <= max(limit, E - resident[l])
        evicted = [o[1] for o in out if o[0] == l]
        assert evicted == [int(ranking[l][i]) for i in range(resident[l] - 1, res[l] - 1, -1)]
    assert res[3] == 5 and all(E - res[l] == limit for l in (0, 1, 2, 4, 5))


def test_rank_experts_by_routing_frequency():
    g = np.random.default_rng(3)
    T, E, k = 500, 12, 3
    ids = np.stack([g.choice(E, k, replace=False, p=np.arange(1, E + 1) / np.arange(1, E + 1).sum())
                    for _ in range(T)]).astype(np.int32)
    ranking, prob = ora.rank_experts(ids, E)
    counts = np.bincount(ids.ravel(), minlength=E)
    want = np.lexsort((np.arange(E), -counts))
    assert np.array_equal(ranking, want)
    np.testing.assert_array_equal(prob, (counts[want] / T).astype(np.float32))
    assert math.isclose(float(prob.sum()), k, rel_tol=1e-5)


def test_rank_experts_ties_go_to_the_lower_id():
    ids = np.array([[3, 1], [1, 3], [0, 2]], dtype=np.int32)  # counts 1, 2, 1, 2, 0
    ranking, prob = ora.rank_experts(ids, 5)
    assert ranking.tolist() == [1, 3, 0, 2, 4]
    np.testing.assert_array_equal(prob, np.array([2, 2, 1, 1, 0], dtype=np.float32) / 3)


# ----------------------------------------------------------------------------- library vs oracle

@pytest.fixture(scope="module")
def lib_adj():
    import paged_expert_weight_amd as pm
    try:
        pm.lib()
    except (RuntimeError, OSError) as e:  # the library has not been built
        pytest.skip(str(e))
    return pm


def test_library_amounts_match_oracle(lib_adj):
    for short in range(0, 60):
        for free in range(0, 60):
            if short and free % 7:
                continue
            assert lib_adj.adjust_amounts(short, free) == ora.adjust_amounts(short, free)
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        assert lib_adj.adjust_amounts(c["short_pages"], c["free_pages"]) == (c["evict"], c["add"])


@pytest.mark.parametrize("seed", range(8))
def test_library_ranking_matches_oracle(lib_adj, seed):
    g = np.random.default_rng(seed)
    T, E, k = int(g.integers(1, 400)), int(g.integers(1, 70)), int(g.integers(1, 6))
    k = min(k, E)
    w = g.random(E) ** 3 + 1e-3
    ids = np.stack([g.choice(E, k, replace=False, p=w / w.sum()) for _ in range(T)]).astype(np.int32)
    if seed % 2:  # a shared expert column (id E) is not ranked
        ids = np.concatenate([ids, np.full((T, 1), E, np.int32)], axis=1)
    r_lib, p_lib = lib_adj.rank_experts(ids, E)
    r_ora, p_ora = ora.rank_experts(ids, E)
    assert np.array_equal(r_lib, r_ora)
    np.testing.assert_array_equal(p_lib, p_ora)


@pytest.mark.parametrize("seed", range(12))
def test_library_selection_matches_oracle(lib_adj, seed):
    g = np.random.default_rng(1000 + seed)
    L, E = int(g.integers(1, 9)), int(g.integers(1, 40))
    ranking, prob = _rankings(seed, L, E, ties=bool(seed % 3 == 0))
    resident = g.integers(0, E + 1, size=L).tolist()
    limit = int(g.integers(0, E + 2))
    for n_ev, n_add in ((0, 0), (0, 1), (0, 5), (1, 0), (3, 0), (7, 0), (0, 40), (40, 0)):
        got = lib_adj.adjust_select(ranking, prob, resident, limit, n_ev, n_add)
        assert got == ora.select(ranking, prob, resident, limit, n_ev, n_add), (n_ev, n_add)


def test_library_rejects_bad_inputs(lib_adj):
    from paged_expert_weight_amd import MoeError
    with pytest.raises(MoeError):
        lib_adj.adjust_amounts(-1, 3)
    ranking, prob = _rankings(0, 2, 4)
    bad = ranking.copy()
    bad[1, 0] = bad[1, 1]
    with pytest.raises(MoeError):
        lib_adj.adjust_select(bad, prob, [2, 2], 4, 1, 0)
    with pytest.raises(MoeError):
        lib_adj.adjust_select(ranking, prob, [5, 2], 4, 1, 0)
    with pytest.raises(MoeError):
        lib_adj.adjust_select(ranking, prob, [2, 2], 4, 1, 1)
