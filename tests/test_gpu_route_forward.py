"""moe_route_forward (routing and the layer in one call) through the C ABI.

For a decode step (T <= 4) the routing runs inside the gate/up launch; every
output must equal, bit for bit, what moe_route followed by moe_paged_forward
writes (routing ids and weights, aligned order, block map, num_padded, y), and
y must match the oracle.  Larger batches run the two-call path and must equal
it too.  The contiguous twin must equal the paged call.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm
from workloads import synth

from gpu_cases import Case, host_layer, max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


# a Qwen3-Next-like layer scaled down: 512 routed experts top-10 plus the
# shared expert, Zipf routing, load-buffer experts
SMALL_512 = synth.spec("qwen3n", T=8, d=512, f=256, kv_pages_per_hole=8, seed=3005)


def _two_calls(c: Case, bm: int, flags: int = 0):
    ws = torch.zeros(pm.moe_workspace_bytes(c.pool, c.layer.T, bm, flags), dtype=torch.uint8, device="cuda")
    r = pm.route(c.pool, c.dev.logits, bm, ws)
    y = pm.paged_forward(c.pool, c.dev.x, r, c.active, ws, flags)
    return y, r


def _one_call(c: Case, bm: int, flags: int = 0):
    ws = torch.zeros(pm.moe_workspace_bytes(c.pool, c.layer.T, bm, flags), dtype=torch.uint8, device="cuda")
    # poison the outputs: every entry the call must write is checked
    y, r = pm.route_forward(c.pool, c.dev.logits, c.dev.x, c.active, ws, bm, flags,
                            y=torch.full_like(c.dev.x, float("nan")))
    return y, r


def _same_routing(r1, r2, bm):
    assert torch.equal(r1.topk_ids, r2.topk_ids)
    assert torch.equal(r1.topk_w, r2.topk_w)
    npad = int(r1.num_padded.item())
    assert npad == int(r2.num_padded.item())
    assert torch.equal(r1.sorted_ids[:npad], r2.sorted_ids[:npad])
    assert torch.equal(r1.block_expert[: npad // bm], r2.block_expert[: npad // bm])


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("bm", [16, 64])
def test_decode_step_equals_two_calls(T, bm):
    c = Case(host_layer("decode", T))
    assert pm.moe_forward_form(c.pool, T) == pm.MOE_FORM_DECODE
    y2, r2 = _two_calls(c, bm)
    y1, r1 = _one_call(c, bm)
    torch.cuda.synchronize()
    _same_routing(r1, r2, bm)
    assert torch.equal(y1, y2)
    ids, w = oracle.route(c.layer.logits, c.s.k, c.s.S)
    assert np.array_equal(r1.topk_ids.cpu().numpy(), ids)
    s_ids, blk, npad = oracle.align(ids, c.s.E_tot, bm)
    assert int(r1.num_padded.item()) == npad
    assert np.array_equal(r1.sorted_ids[:npad].cpu().numpy(), s_ids)
    assert np.array_equal(r1.block_expert[: npad // bm].cpu().numpy(), blk)
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)
    assert max_rel_err(y_f64(y1), ref) <= TOL
    c.pool.close()


# One-token steps across the expert counts that pick how the launch reads the
# chosen expert's table entry: one entry per lane loaded beside the logits
# (E + S <= 64, or <= 128 in two registers), else a table read after the
# routing; load-buffer experts among them (the slot form of the entry).
@pytest.mark.parametrize("E,S", [(8, 0), (63, 1), (64, 1), (100, 0), (127, 1), (128, 1), (200, 0)])
def test_one_token_step_across_expert_counts(E, S):
    s = synth.spec("tiny", T=1, E=E, k=4, S=S, pool_pages=3 * (E + S), loadbuf_experts=(0, 1, E // 2, E - 1),
                   loadbuf_slots=4, seed=3300 + E)
    L = synth.make_layer(s)
    # the load-buffer experts are among the picks of the token
    L.logits[0, [0, E // 2, E - 1]] += 6.0
    c = Case(L)
    assert pm.moe_route_forward_form(c.pool, 1) == pm.MOE_FORM_DECODE_ROUTED
    y2, r2 = _two_calls(c, 16)
    y1, r1 = _one_call(c, 16)
    ws = torch.zeros(pm.moe_workspace_bytes(c.pool, 1, 16, 0), dtype=torch.uint8, device="cuda")
    r3 = pm.RouteOut(c.pool, 1, 16)
    y3 = torch.full_like(c.dev.x, float("nan"))
    pm.moe_route_contiguous_forward(c.pool, c.dev.w13, c.dev.w2, c.dev.logits, c.dev.x, 16, r3.topk_ids, r3.topk_w,
                                    r3.sorted_ids, r3.block_expert, r3.num_padded, y3, ws)
    torch.cuda.synchronize()
    _same_routing(r1, r2, 16)
    _same_routing(r1, r3, 16)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    ids, w = oracle.route(c.layer.logits, c.s.k, c.s.S)
    assert np.array_equal(r1.topk_ids.cpu().numpy(), ids)
    assert {0, E // 2, E - 1} <= set(ids[0].tolist())
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)
    assert max_rel_err(y_f64(y1), ref) <= TOL
    c.pool.close()


@pytest.mark.parametrize("T", [1, 3, 4, 8])
def test_decode_step_512_experts_and_shared(T):
    """E = 512 (eight logits per lane), k = 10 and the shared expert, Zipf routing."""
    c = Case(synth.make_layer(SMALL_512, T))
    assert pm.moe_forward_form(c.pool, T) == pm.MOE_FORM_DECODE
    y2, r2 = _two_calls(c, 16)
    y1, r1 = _one_call(c, 16)
    torch.cuda.synchronize()
    _same_routing(r1, r2, 16)
    assert torch.equal(y1, y2)
    ids, w = oracle.route(c.layer.logits, c.s.k, c.s.S)
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)
    assert max_rel_err(y_f64(y1), ref) <= TOL
    c.pool.close()


@pytest.mark.parametrize("T", [1, 2, 4])
def test_decode_steps_reuse_one_workspace(T):
    """Back-to-back one-call steps on one workspace that starts as 0xFF bytes,
    with the routing changing from step to step: nothing left in the workspace
    by the previous step (or garbage) may leak into the next one."""
    c = Case(host_layer("decode", T))
    bm = 16
    assert pm.moe_route_forward_form(c.pool, T) == pm.MOE_FORM_DECODE_ROUTED
    ws = torch.full((pm.moe_workspace_bytes(c.pool, T, bm, 0),), 255, dtype=torch.uint8, device="cuda")
    steps = []
    for rep in range(5):
        logits = torch.roll(c.dev.logits, shifts=7 * rep, dims=1).contiguous()
        y, _ = pm.route_forward(c.pool, logits, c.dev.x, c.active, ws, bm, 0,
                                y=torch.full_like(c.dev.x, float("nan")))
        steps.append((logits, y))
    torch.cuda.synchronize()
    for logits, y in steps:
        ws2 = torch.zeros(pm.moe_workspace_bytes(c.pool, T, bm, 0), dtype=torch.uint8, device="cuda")
        r2 = pm.route(c.pool, logits, bm, ws2)
        y2 = pm.paged_forward(c.pool, c.dev.x, r2, c.active, ws2, 0)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
    c.pool.close()


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", 32)])
def test_larger_batches_take_the_two_call_path(name, T):
    c = Case(host_layer(name, T))
    for bm in (16, 32):
        y2, r2 = _two_calls(c, bm)
        y1, r1 = _one_call(c, bm)
        torch.cuda.synchronize()
        _same_routing(r1, r2, bm)
        assert torch.equal(y1, y2)
    c.pool.close()


@pytest.mark.parametrize("T", [1, 4, 8, 32])
def test_contiguous_twin_equals_paged(T):
    c = Case(host_layer("decode", T))
    bm = 16
    y1, r1 = _one_call(c, bm)
    ws = torch.zeros(pm.moe_workspace_bytes(c.pool, T, bm, 0), dtype=torch.uint8, device="cuda")
    r3 = pm.RouteOut(c.pool, T, bm)
    y3 = torch.full_like(c.dev.x, float("nan"))
    pm.moe_route_contiguous_forward(c.pool, c.dev.w13, c.dev.w2, c.dev.logits, c.dev.x, bm, r3.topk_ids, r3.topk_w,
                                    r3.sorted_ids, r3.block_expert, r3.num_padded, y3, ws)
    torch.cuda.synchronize()
    _same_routing(r1, r3, bm)
    assert torch.equal(y1, y3)
    c.pool.close()


def test_zero_tokens_and_errors():
    c = Case(host_layer("tiny"))
    s = c.s
    x = torch.empty((0, s.d), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((0, s.E), dtype=torch.float32, device="cuda")
    ws = pm.workspace(c.pool, 0, 16)
    y, r = pm.route_forward(c.pool, logits, x, 0, ws, 16)
    torch.cuda.synchronize()
    assert y.shape == (0, s.d)
    # null logits, bad buffer index
    ws = pm.workspace(c.pool, s.T, 16)
    r = pm.RouteOut(c.pool, s.T, 16)
    y = torch.empty_like(c.dev.x)
    with pytest.raises(pm.MoeError) as ei:
        pm.moe_route_forward(c.pool, None, c.dev.x, 16, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert,
                             r.num_padded, 0, y, ws)
    assert ei.value.code == pm.MOE_ERR_INVALID_ARG
    with pytest.raises(pm.MoeError) as ei:
        pm.moe_route_forward(c.pool, c.dev.logits, c.dev.x, 16, r.topk_ids, r.topk_w, r.sorted_ids,
                             r.block_expert, r.num_padded, 2, y, ws)
    assert ei.value.code == pm.MOE_ERR_INVALID_ARG
    c.pool.close()


def test_route_forward_form():
    c = Case(host_layer("decode", 1))
    forms = {T: pm.moe_route_forward_form(c.pool, T) for T in (1, 2, 4, 5, 8, 32)}
    assert forms[1] == forms[2] == forms[4] == pm.MOE_FORM_DECODE_ROUTED
    assert forms[5] == forms[8] == pm.MOE_FORM_DECODE
    assert forms[32] == pm.MOE_FORM_TILES == pm.moe_forward_form(c.pool, 32)
    c.pool.close()
