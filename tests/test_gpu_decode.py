"""The decode form of the two GEMMs (1..8 tokens), through the C ABI.

Every weight row is read once and dotted on the vector ALUs with the x rows of
the picks of its expert block; the down projection adds a token's picks in
slot order and writes y directly.  Bars: y within the oracle bar
(max |y - y_oracle| <= 2e-2 * max |y_oracle|); bit-identical for every tile
height and with the atomic-combine flag (the form does not depend on either);
paged bit-identical to contiguous; pools NaN-poisoned outside expert pages,
so a stray read shows up as NaN.
"""
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

SPECS = {
    # the Qwen1.5-shaped decode layer: half the experts in the load buffer
    "decode": synth.SPECS["decode"],
    # 512 routed experts top-10 plus a shared one, Zipf(1.1) popularity, 64 via the load buffer
    "wide": synth.spec("qwen3n", T=8, E=512, k=10, S=1, pool_pages=3 * 449, loadbuf_slots=64, seed=6100),
    # d = 4096: the widest register tile of the gate/up form
    "deep": synth.spec("qwen15", T=8, d=4096, f=512, E=16, k=2, pool_pages=48, loadbuf_experts=(14, 15),
                       loadbuf_slots=2, seed=6200),
    "tiny": synth.SPECS["tiny"],
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


_cases = {}


def case(name, T) -> Case:
    key = (name, T)
    if key not in _cases:
        _cases.clear()
        torch.cuda.empty_cache()
        _cases[key] = Case(synth.make_layer(SPECS[name], T))
    return _cases[key]


def _bits(y):
    return y.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 2), ("decode", 3), ("decode", 5), ("decode", 8),
                                    ("wide", 1), ("wide", 8), ("deep", 1), ("deep", 8), ("tiny", 1),
                                    ("tiny", 8)])
def test_decode_form(name, T):
    c = case(name, T)
    assert pm.moe_forward_form(c.pool, T) == pm.MOE_FORM_DECODE
    ids, w = oracle.route(c.layer.logits, c.s.k, c.s.S)
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)
    first = None
    for bm in BLOCK_MS:
        y, _ = c.forward(bm)
        yc, _ = c.contiguous(bm)
        ya, _ = c.forward(bm, pm.MOE_FLAG_ATOMIC_COMBINE)
        torch.cuda.synchronize()
        got = y_f64(y)
        assert np.all(np.isfinite(got)), f"NaN in y (block_m={bm})"
        err = max_rel_err(got, ref)
        assert err <= TOL, f"block_m={bm}: {err}"
        b = _bits(y)
        assert np.array_equal(b, _bits(yc)), f"paged != contiguous (block_m={bm})"
        assert np.array_equal(b, _bits(ya)), f"atomic flag changed y (block_m={bm})"
        if first is None:
            first = b
        assert np.array_equal(b, first), f"block_m={bm} changed y"


def test_decode_form_limits():
    """Nine tokens, zero tokens, f above 2048 and d above 4096 take the tile GEMMs."""
    c = case("decode", 8)
    assert pm.moe_forward_form(c.pool, 9) == pm.MOE_FORM_TILES
    assert pm.moe_forward_form(c.pool, 0) == pm.MOE_FORM_TILES
    for d, f in ((4096, 14336), (8192, 512)):
        big = pm.moe_pool_create(0x1000, 8, d, f, 8, 2, 0, 0)
        assert pm.moe_forward_form(big, 1) == pm.MOE_FORM_TILES
        big.close()
    ok = pm.moe_pool_create(0x1000, 8, 4096, 2048, 8, 2, 0, 0)
    assert pm.moe_forward_form(ok, 8) == pm.MOE_FORM_DECODE
    ok.close()
