"""The allocation-free route + forward (moe_route_forward_noalloc) through the C ABI.

Its workspace is the library's static scratch array instead of a caller's
allocation; the kernels and launches are those of moe_route_forward, so every
output (routing ids and weights, aligned order, block map, num_padded, y) must
equal moe_route_forward's with a caller workspace bit for bit (y with the
fp32-atomic combine, whose order of additions is not fixed, within the layer's
bar max |y - y_ref| <= 2e-2 * max |y_ref|).  Two calls in a
row share the array: the second, with a smaller batch, must not see what the
first left there.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_expert_weight_amd as pm

from gpu_cases import Case, host_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


@pytest.fixture(scope="module")
def qwen15():
    c = Case(host_layer("qwen15"))
    yield c
    c.pool.close()


def _noalloc(c, T, bm, flags):
    x, logits = c.dev.x[:T], c.dev.logits[:T]
    r = pm.RouteOut(c.pool, T, bm)
    y = torch.empty_like(x)
    pm.moe_route_forward_noalloc(c.pool, logits, x, bm, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert,
                                 r.num_padded, c.active, y, flags)
    return y, r


def _with_workspace(c, T, bm, flags):
    ws = pm.workspace(c.pool, T, bm, flags)
    return pm.route_forward(c.pool, c.dev.logits[:T], c.dev.x[:T], c.active, ws, bm, flags)


def _same(a, b, bm, what, exact_y=True):
    (ya, ra), (yb, rb) = a, b
    if exact_y:
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), f"{what}: y"
    else:  # fp32 atomics add in no fixed order: y to the layer's tolerance bar
        err = float((ya.float() - yb.float()).abs().max() / yb.float().abs().max())
        assert err <= 2e-2, f"{what}: y off by {err:.3e} of max|y|"
    assert torch.equal(ra.topk_ids, rb.topk_ids), f"{what}: routing ids"
    assert torch.equal(ra.topk_w.view(torch.int32), rb.topk_w.view(torch.int32)), f"{what}: routing weights"
    npad = int(ra.num_padded.item())
    assert npad == int(rb.num_padded.item()), f"{what}: num_padded"
    assert torch.equal(ra.sorted_ids[:npad], rb.sorted_ids[:npad]), f"{what}: sorted order"
    assert torch.equal(ra.block_expert[: npad // bm], rb.block_expert[: npad // bm]), f"{what}: block map"


@pytest.mark.parametrize("flags", [0, pm.MOE_FLAG_ATOMIC_COMBINE])
def test_noalloc_matches_workspace_call_twice(qwen15, flags):
    c = qwen15
    # 1024 tokens at block_m 128 (about 50 MB of the 64 MiB array), then 32
    # tokens at block_m 16 and a one-token step (the routed decode form) in the
    # array the first call filled
    for T, bm in ((1024, 128), (32, 16), (1, 16)):
        got = _noalloc(c, T, bm, flags)
        ref = _with_workspace(c, T, bm, flags)
        torch.cuda.synchronize()
        _same(got, ref, bm, f"T={T} block_m={bm}", exact_y=not flags & pm.MOE_FLAG_ATOMIC_COMBINE)
        y = got[0].float()
        assert torch.isfinite(y).all() and y.abs().max() > 0


def test_noalloc_rejects_a_workspace_beyond_the_array(qwen15):
    c = qwen15
    need = pm.moe_workspace_bytes(c.pool, 1024, 256, 0)
    assert need > pm.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(pm.MoeError) as ei:
        _noalloc(c, 1024, 256, 0)
    assert ei.value.code == pm.MOE_ERR_WORKSPACE
    # the refused call launched nothing; the next one still matches
    _same(_noalloc(c, 64, 32, 0), _with_workspace(c, 64, 32, 0), 32, "after a refusal")
