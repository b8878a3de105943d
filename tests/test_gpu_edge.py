"""Degenerate and extreme layers on the GPU, through the C ABI, against the
oracle: one expert with k = 1, k = E, every token on one expert (one expert
owning many blocks at every tile height), the smallest shapes (d = f = 64, and
d not a multiple of 128), a ragged token count, a shared expert beside two
routed ones, the largest expert count (E + S = 1024), batches with enough
128-row blocks for the 512-column down tiles (one of them with experts whose
blocks run in pairs as 256-row tiles), and the empty batch (T = 0).  Routing ids,
aligned order and block map are compared bit for bit, y within the bar, and
paged against contiguous weights bit for bit."""
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
BLOCK_MS = (16, 32, 64, 128, 256)


def _spec(name, **kw):
    return dataclasses.replace(synth.SPECS["tiny"], name=name, **kw)


EDGE = {
    "one_expert": _spec("one_expert", T=37, E=1, k=1, S=0, pool_pages=4, loadbuf_experts=(), loadbuf_slots=0,
                        seed=4001),
    "k_equals_E": _spec("k_equals_E", T=29, E=4, k=4, pool_pages=16, loadbuf_experts=(3,), loadbuf_slots=1,
                        seed=4002),
    "shared_beside_two": _spec("shared_beside_two", T=45, E=2, k=1, S=1, pool_pages=12, loadbuf_experts=(1,),
                               loadbuf_slots=1, seed=4003),
    "d64_f64": _spec("d64_f64", T=19, d=64, f=64, seed=4004),
    "d192_ragged": _spec("d192_ragged", T=1000, d=192, f=192, E=16, k=3, pool_pages=64,
                         loadbuf_experts=(13, 14, 15), loadbuf_slots=4, seed=4005),
    "max_experts": _spec("max_experts", T=40, d=64, f=64, E=1023, k=8, S=1, pool_pages=3 * 1024 + 8,
                         loadbuf_experts=tuple(range(1000, 1023)), loadbuf_slots=24, seed=4006),
    # enough 128-row blocks (1800 picks over 1024 experts: up to 1038 blocks) for the 512-column down
    # tiles, with f not a multiple of 256 (64-column gate/up tiles beside them)
    "wide_down": _spec("wide_down", T=600, d=512, f=192, E=1023, k=2, S=1, pool_pages=3 * 1024 + 5,
                       loadbuf_experts=tuple(range(1010, 1023)), loadbuf_slots=16, seed=4009),
    # the same with f a multiple of 256 (256 + 256-column gate/up tiles) and skewed routing, so
    # that experts with several 128-row blocks run pairs of them as 256-row tiles (the shared
    # expert's 2000 rows are 16 blocks), beside single-block experts and odd last blocks
    "wide_pairs": _spec("wide_pairs", T=2000, d=512, f=256, E=1023, k=2, S=1, pool_pages=3 * 1024 + 5,
                        loadbuf_experts=tuple(range(1010, 1023)), loadbuf_slots=16, zipf_s=1.1, seed=4010),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


def _check_layer(layer, block_ms=BLOCK_MS):
    c = Case(layer)
    s = c.s
    ids, w = oracle.route(layer.logits, s.k, s.S)
    ref = oracle.moe(layer.x, layer.w13, layer.w2, ids, w)
    for bm in block_ms:
        y, r = c.forward(bm)
        yc, _ = c.contiguous(bm)
        torch.cuda.synchronize()
        assert np.array_equal(r.topk_ids.cpu().numpy(), ids), f"block_m {bm}: routing ids"
        np.testing.assert_allclose(r.topk_w.cpu().numpy(), w, rtol=1e-6, atol=0)
        s_ids, blk, npad = oracle.align(ids, s.E_tot, bm)
        assert int(r.num_padded.item()) == npad
        assert np.array_equal(r.sorted_ids[:npad].cpu().numpy(), s_ids), f"block_m {bm}: sorted order"
        assert np.array_equal(r.block_expert[: npad // bm].cpu().numpy(), blk), f"block_m {bm}: block map"
        got = y_f64(y)
        assert np.all(np.isfinite(got)), f"block_m {bm}: non-finite output"
        assert max_rel_err(got, ref) <= TOL, f"block_m {bm}: y off the oracle"
        assert torch.equal(y, yc), f"block_m {bm}: paged and contiguous differ"
    c.pool.close()


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_layer_matches_oracle(name):
    _check_layer(synth.make_layer(EDGE[name]))


def test_every_token_on_one_expert():
    """Expert 0 wins every token's first pick: it owns T rows, many blocks at
    every tile height (and the 256-row launch's split last wave)."""
    spec = _spec("one_hot_expert", T=700, E=8, k=2, pool_pages=32, seed=4007)
    layer = synth.make_layer(spec)
    # +50 puts expert 0 first for all 700 tokens (the other logits are N(0, 1)),
    # so every second pick's weight is about exp(-50): the routing weights must
    # keep the 1e-6 relative bar at that gap
    layer.logits[:, 0] += 50.0
    ids, _ = oracle.route(layer.logits, spec.k, spec.S)
    assert np.all(ids[:, 0] == 0)
    _check_layer(layer)


def test_expert_segment_longer_than_64_blocks():
    """256-row tiles group an expert's blocks from its first block, found by
    reading the block map 64 entries at a time around a tile's block: with
    every token's first pick on expert 0 (40000 rows, 157 blocks) the search
    must walk several windows in both directions for the blocks in the middle
    of that segment.  d = 256 and f = 128 select the 256 x 256 tiles; the 314
    tiles of each GEMM are one full wave and a split last wave on 256 CUs."""
    spec = _spec("long_segment", T=40000, d=256, f=128, E=4, k=2, pool_pages=16, loadbuf_experts=(3,),
                 loadbuf_slots=1, seed=4008)
    layer = synth.make_layer(spec)
    layer.logits[:, 0] += 50.0  # second picks at weights near exp(-50), as in test_every_token_on_one_expert
    ids, _ = oracle.route(layer.logits, spec.k, spec.S)
    assert np.all(ids[:, 0] == 0)
    _check_layer(layer, block_ms=(256,))


@pytest.mark.parametrize("T", [1, 3])
def test_edge_decode_steps(T):
    """The decode forms on the degenerate layers (one expert, k = E, shared beside two)."""
    for name in ("one_expert", "k_equals_E", "shared_beside_two", "max_experts"):
        layer = synth.make_layer(EDGE[name], T)
        c = Case(layer)
        s = c.s
        assert pm.moe_forward_form(c.pool, T) == pm.MOE_FORM_DECODE
        ids, w = oracle.route(layer.logits, s.k, s.S)
        ref = oracle.moe(layer.x, layer.w13, layer.w2, ids, w)
        y1, _ = c.forward(16)
        ws = pm.workspace(c.pool, T, 16)
        y2, r2 = pm.route_forward(c.pool, c.dev.logits, c.dev.x, c.active, ws, 16)
        torch.cuda.synchronize()
        assert np.array_equal(r2.topk_ids.cpu().numpy(), ids), name
        assert torch.equal(y1, y2), name
        assert max_rel_err(y_f64(y1), ref) <= TOL, name
        c.pool.close()


def test_empty_batch_is_a_no_op():
    """T = 0 at every entry point (route, paged, contiguous, one-call and
    allocation-free forward): success, nothing written (the caller's buffers
    keep their sentinels), and the next batch on the same handle and
    workspace is unaffected."""
    layer = synth.make_layer(EDGE["shared_beside_two"])
    c = Case(layer)
    s = c.s
    logits0, x0 = c.dev.logits[:0], c.dev.x[:0]
    for bm in (16, 128):
        ws = pm.workspace(c.pool, 0, bm)
        r = pm.RouteOut(c.pool, 0, bm)
        r.num_padded.fill_(-7)
        r.sorted_ids.fill_(-7)
        r.block_expert.fill_(-7)
        pm.moe_route(c.pool, logits0, bm, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded, ws)
        y = pm.paged_forward(c.pool, x0, r, c.active, ws)
        yc = pm.contiguous_forward(c.pool, c.dev.w13, c.dev.w2, x0, r, ws)
        y1, r1 = pm.route_forward(c.pool, logits0, x0, c.active, ws, bm)
        r1.num_padded.fill_(-7)
        pm.moe_route_forward_noalloc(c.pool, logits0, x0, bm, r1.topk_ids, r1.topk_w, r1.sorted_ids,
                                     r1.block_expert, r1.num_padded, c.active, y1)
        torch.cuda.synchronize()
        assert y.shape[0] == yc.shape[0] == y1.shape[0] == 0
        for t in (r.num_padded, r.sorted_ids, r.block_expert, r1.num_padded):
            assert bool(torch.all(t == -7)), f"block_m {bm}: an empty batch wrote a routing output"
    # a batch after the empty calls, on a workspace an empty call used
    ids, w = oracle.route(layer.logits, s.k, s.S)
    ref = oracle.moe(layer.x, layer.w13, layer.w2, ids, w)
    bm = 16
    ws = pm.workspace(c.pool, layer.T, bm)
    pm.moe_route(c.pool, logits0, bm, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded, ws)
    y, r2 = pm.route_forward(c.pool, c.dev.logits, c.dev.x, c.active, ws, bm)
    torch.cuda.synchronize()
    assert np.array_equal(r2.topk_ids.cpu().numpy(), ids)
    assert max_rel_err(y_f64(y), ref) <= TOL
    c.pool.close()
