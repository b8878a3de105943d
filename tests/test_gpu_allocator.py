"""The layer on a pool shaped by the three-tier allocator: a seeded serving
churn (KV requests arriving and finishing, experts evicted and brought back)
is replayed through moe_alloc_*, and the expert pages it hands out become the
location table.  Expert pages end up in runs between expert pages split into
KV pages; every page that holds no expert matrix is bf16 NaN.  Bars: y against
the oracle (max |y - y_oracle| <= 2e-2 * max |y_oracle|) and bit-identical to
the same layer placed by a plain page permutation (same kernels, same K order)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm
from paged_expert_weight_amd import placement
from workloads import churn, synth

from gpu_cases import Case, max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


def allocator_layer(s: synth.LayerSpec, kv_bytes: int, seed: int, arrivals: float):
    base = synth.make_layer(s)
    slots = {int(e): int(base.placement.locs[e]["idx"][0]) for e in range(s.E_tot)
             if base.placement.locs[e]["kind"] == synth.LOC_LOADBUF}
    pool_experts = [e for e in range(s.E_tot) if e not in slots]
    e_bytes = s.f * s.d * 2
    alloc = pm.PageAllocator(s.pool_pages * e_bytes, e_bytes, kv_bytes)
    r = placement.replay(alloc, pool_experts, churn.events(seed, len(pool_experts), 300, arrivals=arrivals))
    locs = placement.location_table(s.E_tot, r["pages"], slots)
    per = e_bytes // kv_bytes
    holes = sorted({q // per for v in r["kv"].values() for q in v})
    used = sorted(p for v in r["pages"].values() for p in v)
    free = sorted(set(range(s.pool_pages)) - set(used) - set(holes))
    pl = synth.Placement(locs, np.asarray(used, np.int64), np.asarray(holes, np.int64),
                         np.asarray(free, np.int64), base.placement.slot_expert)
    return base, synth.Layer(s, base.x, base.logits, base.w13, base.w2, pl), alloc.stats()


SPEC = synth.spec("qwen3n", T=256, d=512, f=256, E=128, k=8, S=1, pool_pages=420, loadbuf_experts=(),
                  loadbuf_slots=16, zipf_s=1.1, kv_pages_per_hole=16, seed=5100)


@pytest.mark.parametrize("block_m", (16, 64))
def test_layer_on_allocator_pool(block_m):
    base, L, st = allocator_layer(SPEC, (SPEC.f * SPEC.d * 2) // 16, seed=11, arrivals=6.0)
    locs = L.placement.locs
    pages = sorted(int(p) for e in range(SPEC.E_tot) if locs[e]["kind"] == synth.LOC_POOL for p in locs[e]["idx"])
    runs = 1 + sum(1 for a, b in zip(pages, pages[1:]) if b != a + 1)
    print(f"expert pages in {runs} runs, {len(L.placement.hole_pages)} pages split into KV pages, "
          f"{st['trapped_bytes']} trapped bytes", flush=True)
    assert runs > 4 and len(L.placement.hole_pages) > 0
    c = Case(L)
    y, r = c.forward(block_m)
    torch.cuda.synchronize()
    ids, w = oracle.route(L.logits, SPEC.k, SPEC.S)
    ref = oracle.moe(L.x, L.w13, L.w2, ids, w)
    assert max_rel_err(y_f64(y), ref) <= TOL
    c0 = Case(base)
    y0, _ = c0.forward(block_m)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy(), y0.view(torch.int16).cpu().numpy())
