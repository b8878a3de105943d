"""Seeded random layers through the C ABI against the oracle.

Each case draws a layer shape and placement: expert count, top-k, with or
without the shared expert, d and f (multiples of 64 up to 768), token count
(one to 3000 tokens, so that the decode forms, the one-workgroup routing
forms, the tile forms and the multi-chunk alignment all occur), uniform or
Zipf-skewed routing, some
routed experts in the load buffer and the rest on permuted pool pages.  At
the tile height moe_suggest_block_m picks and at one drawn at random:
routing ids bit for bit and weights to 1e-6 relative against the oracle, the
aligned order and block map bit for bit, y within 2e-2 * max|ref|, the paged
forward equal bit for bit to the contiguous twin, and moe_route_forward (one
call) equal bit for bit to moe_route + moe_paged_forward."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm
from workloads import synth

from gpu_cases import Case, max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2
N_CASES = 64
MAX_WEIGHT_ELEMS = 48 << 20  # keeps each drawn layer's host weights and oracle work small


def draw_spec(i: int) -> synth.LayerSpec:
    g = np.random.default_rng(9000 + i)
    d = 64 * int(g.integers(1, 13))
    f = 64 * int(g.integers(1, 13))
    E = int(g.choice([1, 2, 3, 5, 8, 16, 33, 60, 64, 65, 128, 200, 257]))
    S = int(g.integers(0, 2))
    while E > 1 and (E + S) * 3 * d * f > MAX_WEIGHT_ELEMS:
        E //= 2
    k = int(g.integers(1, min(E, 12) + 1))
    T = int(g.choice([1, 2, 3, 4, 5, 8, 13, 31, 64, 100, 200, 257, 400, 700, 1500, 3000]))
    n_lb = int(g.integers(0, min(E, 8) + 1))
    lb = tuple(sorted(int(e) for e in g.choice(E, n_lb, replace=False))) if n_lb else ()
    slots = n_lb + int(g.integers(0, 3)) if n_lb else 0
    pool_pages = 3 * (E + S - n_lb) + int(g.integers(0, 20))
    zipf = None if g.random() < 0.5 else float(g.choice([0.8, 1.1, 1.5]))
    return dataclasses.replace(synth.SPECS["tiny"], name=f"random{i}", T=T, d=d, f=f, E=E, k=k, S=S,
                               pool_pages=pool_pages, loadbuf_experts=lb, loadbuf_slots=slots, zipf_s=zipf,
                               kv_pages_per_hole=0, seed=9000 + i)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer_matches_oracle(i):
    spec = draw_spec(i)
    layer = synth.make_layer(spec)
    c = Case(layer)
    s, T = c.s, layer.T
    ids, w = oracle.route(layer.logits, s.k, s.S)
    ref = oracle.moe(layer.x, layer.w13, layer.w2, ids, w)
    g = np.random.default_rng(9500 + i)
    block_ms = sorted({pm.moe_suggest_block_m(c.pool, T), int(g.choice([16, 32, 64, 128, 256]))})
    for bm in block_ms:
        case = f"{spec} block_m {bm}"
        y, r = c.forward(bm)
        yc, _ = c.contiguous(bm)
        ws = pm.workspace(c.pool, T, bm)
        y1, r1 = pm.route_forward(c.pool, c.dev.logits, c.dev.x, c.active, ws, bm,
                                  y=torch.full_like(c.dev.x, float("nan")))
        torch.cuda.synchronize()
        assert np.array_equal(r.topk_ids.cpu().numpy(), ids), case
        np.testing.assert_allclose(r.topk_w.cpu().numpy(), w, rtol=1e-6, atol=0, err_msg=case)
        s_ids, blk, npad = oracle.align(ids, s.E_tot, bm)
        assert int(r.num_padded.item()) == npad, case
        assert np.array_equal(r.sorted_ids[:npad].cpu().numpy(), s_ids), case
        assert np.array_equal(r.block_expert[: npad // bm].cpu().numpy(), blk), case
        got = y_f64(y)
        assert np.all(np.isfinite(got)), case
        assert max_rel_err(got, ref) <= TOL, case
        assert torch.equal(y, yc), case
        assert torch.equal(r1.topk_ids, r.topk_ids) and torch.equal(r1.topk_w, r.topk_w), case
        assert int(r1.num_padded.item()) == npad, case
        assert torch.equal(r1.sorted_ids[:npad], r.sorted_ids[:npad]), case
        assert torch.equal(y1, y), case
    c.pool.close()
