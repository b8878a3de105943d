"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something independent of its code: the
address formula printed in the Rimuru digest's kernel section (hand-evaluated
golden cases and a brute-force check against whole-page pool images), library
routines (numpy's stable argsort, scipy's softmax, torch's SiLU and matmul),
closed forms and invariants.  A plausible slip in the oracle (swapped W1/W3,
a wrong page for a column half, an unstable sort, a missing renormalisation,
ties broken upward, W2 read transposed) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------- routing

def test_route_golden():
    for c in _gold("route_small.json")["cases"]:
        logits = np.array([c["logits"]], dtype=np.float32)
        ids, w = oracle.route(logits, c["k"], c["S"])
        assert ids[0].tolist() == c["ids"], c["why"]
        np.testing.assert_allclose(w[0], c["w"], rtol=1e-12, atol=0, err_msg=c["why"])


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (128, 60, 4), (32, 512, 10), (16, 7, 7)])
def test_route_matches_stable_argsort(T, E, k):
    g = np.random.default_rng(T * 1000 + E)
    logits = g.standard_normal((T, E)).astype(np.float32)
    # coarse values force many exact ties
    logits[: T // 2] = np.round(logits[: T // 2] * 2) / 2
    ids, w = oracle.route(logits, k)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_k1_weight_exactly_one():
    logits = np.random.default_rng(3).standard_normal((100, 60)).astype(np.float32)
    ids, w = oracle.route(logits, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))


def test_route_k_equals_E_is_full_softmax():
    logits = (np.random.default_rng(4).standard_normal((50, 9)) * 3).astype(np.float32)
    ids, w = oracle.route(logits, 9)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, axis=1), rtol=1e-12, atol=1e-15)


def test_route_shared_expert_appended():
    logits = np.random.default_rng(5).standard_normal((20, 16)).astype(np.float32)
    ids, w = oracle.route(logits, 3, S=1)
    ids0, w0 = oracle.route(logits, 3, S=0)
    assert np.all(ids[:, 3] == 16) and np.all(w[:, 3] == 1.0)
    assert np.array_equal(ids[:, :3], ids0) and np.array_equal(w[:, :3], w0)


def test_route_invariant_to_logit_shift():
    logits = np.random.default_rng(6).standard_normal((40, 12)).astype(np.float32)
    ids, w = oracle.route(logits, 4)
    ids2, w2 = oracle.route(logits + np.float32(8.0), 4)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-5)


# ----------------------------------------------------------------------------- alignment

def test_align_golden():
    g = _gold("align_small.json")
    ids = np.array(g["ids"], dtype=np.int32)
    for c in g["cases"]:
        s, b, n = oracle.align(ids, g["E_tot"], c["BM"])
        assert s.tolist() == c["sorted_ids"]
        assert b.tolist() == c["block_expert"]
        assert n == c["num_padded"]


def _check_alignment(flat, E_tot, BM, s, b, npad):
    n = flat.size
    counts = np.bincount(flat, minlength=E_tot)
    assert npad == int(sum(-(-c // BM) * BM for c in counts))
    assert npad % BM == 0 and s.size == npad and b.size == npad // BM
    real = s[s != n]
    # every flat index exactly once, in the order of a stable sort by expert
    assert np.array_equal(real, np.argsort(flat, kind="stable"))
    # each block is one expert; its real rows belong to it; sentinels trail
    for blk in range(npad // BM):
        rows = s[blk * BM:(blk + 1) * BM]
        e = b[blk]
        r = rows[rows != n]
        assert np.all(flat[r] == e)
        if r.size < BM:
            assert np.all(rows[r.size:] == n)
    assert np.all(np.diff(b) >= 0)
    # experts with no tokens own no block; others own exactly ceil(c/BM)
    for e in range(E_tot):
        assert int(np.sum(b == e)) == -(-int(counts[e]) // BM)


@pytest.mark.parametrize("T,E_tot,k,BM", [(16, 8, 2, 16), (1024, 60, 4, 64), (37, 513, 11, 32),
                                          (5, 60, 4, 128), (300, 9, 3, 1)])
def test_align_invariants(T, E_tot, k, BM):
    g = np.random.default_rng(T + E_tot + BM)
    ids = np.stack([g.permutation(E_tot)[:k] for _ in range(T)]).astype(np.int32)
    s, b, npad = oracle.align(ids, E_tot, BM)
    _check_alignment(ids.reshape(-1), E_tot, BM, s, b, npad)


def test_align_empty_and_rejects_bad_id():
    s, b, npad = oracle.align(np.zeros((0, 2), np.int32), 8, 16)
    assert npad == 0 and s.size == 0 and b.size == 0
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 8]], np.int32), 8, 16)


# ----------------------------------------------------------------------------- addresses

def test_addr_golden():
    g = _gold("addr_formula.json")
    locs = np.array([tuple([r[0], r[1:]]) for r in g["locs"]], dtype=synth.LOC_DTYPE)
    for c in g["cases"]:
        off, base = oracle.addr(locs, g["f"], g["d"], g["num_pages"], g["slots"], c["active"],
                                [c["e"]], [c["which"]], [c["row"]], [c["col"]])
        assert (int(off[0]), int(base[0])) == (c["off"], c["base"]), c["why"]
    for c in g["rejects"]:
        with pytest.raises(ValueError):
            oracle.addr(locs, g["f"], g["d"], g["num_pages"], g["slots"], 0,
                        [c["e"]], [c["which"]], [c["row"]], [c["col"]])


def test_addr_rejects_page_out_of_range():
    locs = np.zeros(1, dtype=synth.LOC_DTYPE)
    locs[0]["idx"] = (0, 1, 4)
    with pytest.raises(ValueError):
        oracle.addr(locs, 2, 2, 4, 0, 0, [0], [1], [0], [0])


@pytest.mark.parametrize("name", ["tiny"])
@pytest.mark.parametrize("active", [0, 1])
def test_addr_brute_force_against_pool_image(name, active):
    """Every weight of every expert, found through the formula, in page images
    built by whole-matrix copies."""
    s = synth.SPECS[name]
    L = synth.make_layer(s)
    pl = L.placement
    pool = synth.build_pool_image(s, L.w13, L.w2, pl).reshape(-1)
    buf = synth.build_loadbuf_image(s, L.w13, L.w2, pl).reshape(-1)
    bases = {0: pool, 1 + active: buf}
    for e in range(s.E_tot):
        for which, (R, C) in ((0, (2 * s.f, s.d)), (1, (s.d, s.f))):
            rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
            rr, cc = rr.reshape(-1), cc.reshape(-1)
            # sample a strided subset to keep the pure-Python loop short, plus all corners
            sel = np.unique(np.concatenate([np.arange(0, rr.size, 97), [0, C - 1, rr.size - C, rr.size - 1]]))
            off, base = oracle.addr(pl.locs, s.f, s.d, s.pool_pages, s.loadbuf_slots, active,
                                    [e] * sel.size, [which] * sel.size, rr[sel], cc[sel])
            want = (L.w13[e] if which == 0 else L.w2[e])[rr[sel], cc[sel]]
            assert np.unique(base).size == 1
            img = bases[int(base[0])]
            assert np.array_equal(img[off], want)


def test_addr_full_brute_force_tiny_pool():
    """Exhaustive on a pool small enough to enumerate every (e, n, t)."""
    s = synth.spec("tiny", d=8, f=4, E=4, k=2, pool_pages=16, loadbuf_experts=(3,), loadbuf_slots=2)
    L = synth.make_layer(s)
    pool = synth.build_pool_image(s, L.w13, L.w2, L.placement).reshape(-1)
    buf = synth.build_loadbuf_image(s, L.w13, L.w2, L.placement).reshape(-1)
    for e in range(s.E_tot):
        for which, M, (R, C) in ((0, L.w13[e], (2 * s.f, s.d)), (1, L.w2[e], (s.d, s.f))):
            for r in range(R):
                for c in range(C):
                    off, base = oracle.addr(L.placement.locs, s.f, s.d, s.pool_pages,
                                            s.loadbuf_slots, 0, [e], [which], [r], [c])
                    img = pool if base[0] == 0 else buf
                    assert img[off[0]] == M[r, c]


# ----------------------------------------------------------------------------- layer output

def _swiglu_torch(x, w1, w3, w2):
    """SwiGLU MLP through torch library routines, fp64: W2 (silu(W1 x) * (W3 x))."""
    h = torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)
    return h @ w2.T


def _f64(bits):
    return torch.from_numpy(synth.bf16_bits_to_f32(bits).astype(np.float64))


def _small_layer(E, k, S=0, T=6, d=32, f=16, seed=0):
    s = synth.spec("tiny", T=T, d=d, f=f, E=E, k=k, S=S, pool_pages=3 * (E + S),
                   loadbuf_experts=(), loadbuf_slots=0, seed=seed)
    return s, synth.make_layer(s)


def test_moe_single_expert_is_swiglu_mlp():
    s, L = _small_layer(E=1, k=1, T=9)
    y, ids, w = oracle.layer(L.x, L.logits, L.w13, L.w2, 1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    ref = _swiglu_torch(_f64(L.x), _f64(L.w13[0, : s.f]), _f64(L.w13[0, s.f:]), _f64(L.w2[0]))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_moe_is_routing_weighted_sum_of_expert_mlps():
    s, L = _small_layer(E=5, k=2, S=1, T=7)
    y, ids, w = oracle.layer(L.x, L.logits, L.w13, L.w2, 2, 1)
    x = _f64(L.x)
    per_e = [_swiglu_torch(x, _f64(L.w13[e, : s.f]), _f64(L.w13[e, s.f:]), _f64(L.w2[e])).numpy()
             for e in range(s.E_tot)]
    ref = np.zeros_like(y)
    for t in range(s.T):
        for j in range(3):
            ref[t] += w[t, j] * per_e[ids[t, j]][t]
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13)


def test_moe_gate_is_w1_closed_form():
    """x = e_0, W1 row c = g_c e_0, W3 row c = u_c e_0, W2 = identity-like:
    y_r = sum_c W2[r,c] * silu(g_c) * u_c; swapping gate and up changes it."""
    d = f = 4
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 1.0
    g = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    u = np.array([2.0, 1.0, -1.0, 0.25], np.float32)
    w13 = np.zeros((1, 2 * f, d), np.float32)
    w13[0, :f, 0] = g
    w13[0, f:, 0] = u
    w2 = np.eye(d, f, dtype=np.float32)[None]
    y = oracle.moe(synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w13), synth.f32_to_bf16_bits(w2),
                   np.zeros((1, 1), np.int32), np.ones((1, 1)))
    want = [gc / (1 + math.exp(-gc)) * uc for gc, uc in zip(g.tolist(), u.tolist())]
    np.testing.assert_allclose(y[0], want, rtol=1e-14)
    swapped = [uc / (1 + math.exp(-uc)) * gc for gc, uc in zip(g.tolist(), u.tolist())]
    assert not np.allclose(y[0], swapped)


def test_moe_zero_routed_down_leaves_shared_expert():
    s, L = _small_layer(E=4, k=2, S=1, T=5)
    w2 = L.w2.copy()
    w2[: s.E] = 0
    y, ids, w = oracle.layer(L.x, L.logits, L.w13, w2, 2, 1)
    ref = _swiglu_torch(_f64(L.x), _f64(L.w13[s.E, : s.f]), _f64(L.w13[s.E, s.f:]), _f64(L.w2[s.E]))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_moe_down_scaling_is_exact():
    s, L = _small_layer(E=4, k=2, T=5)
    y, _, _ = oracle.layer(L.x, L.logits, L.w13, L.w2, 2)
    w2x2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(L.w2) * 2)
    y2, _, _ = oracle.layer(L.x, L.logits, L.w13, w2x2, 2)
    assert np.array_equal(y2, 2 * y)


def test_moe_token_subset_matches_full():
    s, L = _small_layer(E=6, k=2, T=11)
    y, ids, w = oracle.layer(L.x, L.logits, L.w13, L.w2, 2)
    sub = [10, 0, 4]
    ys = oracle.moe(L.x, L.w13, L.w2, ids, w, tokens=sub)
    assert np.array_equal(ys, y[sub])


# ----------------------------------------------------------------------------- generator

def test_generator_is_deterministic_and_poisons_non_expert_pages():
    s = synth.SPECS["tiny"]
    a, b = synth.make_layer(s), synth.make_layer(s)
    for f in ("x", "logits", "w13", "w2"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    pool = synth.build_pool_image(s, a.w13, a.w2, a.placement)
    used = set(a.placement.expert_pages.tolist())
    for p in range(s.pool_pages):
        if p not in used:
            assert np.all(pool[p] == synth.BF16_NAN)
    assert np.all(synth.build_loadbuf_image(s, a.w13, a.w2, a.placement)[a.placement.slot_expert < 0]
                  == synth.BF16_NAN)


def test_generator_kv_pages_divide_expert_page():
    for name in ("mixtral", "qwen3n"):
        s = synth.SPECS[name]
        pl = synth.make_placement(s)
        assert (s.f * s.d * 2) % s.kv_pages_per_hole == 0
        assert pl.hole_pages.size + pl.expert_pages.size == s.pool_pages


def test_generator_zipf_top1_frequency():
    """Gumbel-max over log p gives top-1 choices distributed exactly as p."""
    s = synth.spec("qwen3n", T=8192)
    logits = synth.make_logits(s)
    rank = synth.zipf_rank(s)
    top1 = np.argmax(logits, axis=1)
    p = rank.astype(np.float64) ** (-s.zipf_s)
    p /= p.sum()
    hottest = int(np.argmin(rank))
    frac = np.mean(top1 == hottest)
    assert abs(frac - p[hottest]) < 4 * math.sqrt(p[hottest] * (1 - p[hottest]) / s.T)
