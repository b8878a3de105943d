"""The layer step (moe_route_forward) captured in a HIP graph through
torch.cuda.graph and replayed.  The step launches kernels only (no memset
node, no allocation); with the active load buffer's fill complete and its
read mark deferred (MOE_FLAG_DEFER_READ_DONE) it records no stream event
either.  Every replay, with eager work of the program's own and host
synchronisations between replays, must give the eager step's routing outputs
and y bit for bit, for the decode forms (routing inside the gate/up launch at
1-4 tokens, the decode kernels up to 8) and the tiled form (routing,
alignment, both GEMMs and the ordered combine).  The allocation-free variant
(moe_route_forward_noalloc, its workspace in the library's own device array)
is captured and replayed the same way."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm

from gpu_cases import Case, host_layer, max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


def _outputs(rt, y, bm):
    npad = int(rt.num_padded.item())
    return dict(topk_ids=rt.topk_ids.clone(), topk_w=rt.topk_w.clone(), num_padded=rt.num_padded.clone(),
                sorted_ids=rt.sorted_ids[:npad].clone(), block_expert=rt.block_expert[: npad // bm].clone(),
                y=y.clone())


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 3), ("decode", 8), ("decode", 64), ("tiny", 16),
                                    ("qwen15", 1024)])
def test_graph_replay_matches_eager(name, T):
    c = Case(host_layer(name, T if name == "decode" else None))
    assert c.layer.T == T
    bm = pm.moe_suggest_block_m(c.pool, T)
    ws = pm.workspace(c.pool, T, bm)
    rt = pm.RouteOut(c.pool, T, bm)
    y = torch.empty_like(c.dev.x)
    flags = pm.MOE_FLAG_DEFER_READ_DONE

    def step(stream):
        pm.moe_route_forward(c.pool, c.dev.logits, c.dev.x, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids,
                             rt.block_expert, rt.num_padded, c.active, y, ws, flags, stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = _outputs(rt, y, bm)
    ids, w = oracle.route(c.layer.logits, c.s.k, c.s.S)
    assert np.array_equal(ref["topk_ids"].cpu().numpy(), ids)
    assert max_rel_err(y_f64(ref["y"]), oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)) <= TOL

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        step(side)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        # eager work between replays: poison every output the step writes
        y.fill_(float("nan"))
        rt.topk_ids.fill_(-7)
        rt.topk_w.fill_(float("nan"))
        rt.sorted_ids.fill_(-7)
        rt.block_expert.fill_(-7)
        rt.num_padded.fill_(-7)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(rt, y, bm)
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k}"
    del g
    c.pool.close()


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 8), ("qwen15", 1024)])
def test_graph_replay_of_the_allocation_free_call(name, T):
    """moe_route_forward_noalloc (workspace in the library's static device
    array) captured and replayed: every replay gives the eager call's outputs
    bit for bit."""
    c = Case(host_layer(name, T if name == "decode" else None))
    bm = pm.moe_suggest_block_m(c.pool, T)
    rt = pm.RouteOut(c.pool, T, bm)
    y = torch.empty_like(c.dev.x)
    flags = pm.MOE_FLAG_DEFER_READ_DONE

    def step(stream):
        pm.moe_route_forward_noalloc(c.pool, c.dev.logits, c.dev.x, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids,
                                     rt.block_expert, rt.num_padded, c.active, y, flags, stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = _outputs(rt, y, bm)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        step(side)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        y.fill_(float("nan"))
        rt.topk_ids.fill_(-7)
        rt.topk_w.fill_(float("nan"))
        rt.sorted_ids.fill_(-7)
        rt.block_expert.fill_(-7)
        rt.num_padded.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(rt, y, bm)
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k}"
    del g
    c.pool.close()
