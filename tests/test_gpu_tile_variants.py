"""Every GEMM tile configuration the forward chooses, each selected by a small
layer shaped for it: y against the oracle (within 2e-2 * max|ref|) and the
paged forward equal bit for bit to the contiguous twin.

The forward picks its tile configuration from the block height and the
divisibility of d and f (and, for 128-row blocks with d a multiple of 512,
from how many 512-column down tiles the batch can produce); each case names
the configuration its shape selects.  The two 512-column-down configurations
need over a thousand blocks and are covered by the Qwen3-Next-shaped layer
(all tokens against the oracle) and the wide_down edge layer.  Skewed routing
with a shared expert leaves some experts with a last block that is mostly
padding, so the 128-row tiles also run waves whose rows are all padding, and
the few tiles of the 256-row cases all take the split last wave."""
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

# (configuration, block_m, d, f, T, E, k, S)
CASES = [
    ("16-row tiles", 16, 128, 64, 40, 8, 2, 0),
    ("32-row tiles", 32, 128, 64, 70, 8, 2, 1),
    ("64-row tiles, 256-column down (d % 256 == 0)", 64, 256, 128, 150, 8, 2, 1),
    ("64-row tiles (d % 256 != 0)", 64, 192, 128, 150, 8, 2, 0),
    ("128 x 256 gate/up, 256-column down (d, f % 256 == 0)", 128, 256, 256, 300, 8, 2, 1),
    ("128 x 64 gate/up, 256-column down (f % 256 != 0)", 128, 256, 192, 300, 8, 2, 1),
    ("128 x 64 gate/up, 128-column down (d % 256 != 0)", 128, 384, 128, 300, 8, 2, 1),
    ("128 x 64 gate/up, 64-column down (d % 128 != 0)", 128, 192, 128, 300, 8, 2, 1),
    ("256-row tiles (f % 128 == 0, d % 256 == 0)", 256, 256, 128, 700, 4, 2, 1),
    ("256-row tiles, 64 columns (f % 128 != 0)", 256, 256, 192, 700, 4, 2, 0),
    # experts whose last 256-row block holds 129 rows (one past the second
    # pair of waves) and exactly 128 (the last two waves padding only)
    ("256-row tiles, a last block of 129 rows", 256, 512, 256, 1500, 8, 2, 1, 7111),
    ("256-row tiles, a last block of 128 rows", 256, 512, 256, 1500, 8, 2, 1, 7113),
]


def _layer(i, bm, d, f, T, E, k, S, seed=None):
    spec = dataclasses.replace(synth.SPECS["tiny"], name=f"tiles{i}", T=T, d=d, f=f, E=E, k=k, S=S,
                               pool_pages=3 * (E + S) + 5, loadbuf_experts=(E - 1,), loadbuf_slots=1,
                               zipf_s=1.2, kv_pages_per_hole=0, seed=7100 + i if seed is None else seed)
    return synth.make_layer(spec)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_tile_configuration_matches_oracle(i):
    label, bm, d, f, T, E, k, S = CASES[i][:8]
    layer = _layer(i, *CASES[i][1:])
    c = Case(layer)
    assert pm.moe_forward_form(c.pool, T) == pm.MOE_FORM_TILES, label
    ids, w = oracle.route(layer.logits, k, S)
    ref = oracle.moe(layer.x, layer.w13, layer.w2, ids, w)
    counts = np.bincount(ids.ravel(), minlength=E + S)
    last = counts[counts > 0] % bm
    if bm == 128:  # some expert's last block has a wave of padding rows only
        assert np.any((last > 0) & (last <= 64)), label
    if "a last block of" in label:
        assert np.any(last == int(label.split()[-2])), label
    y, r = c.forward(bm)
    yc, _ = c.contiguous(bm)
    torch.cuda.synchronize()
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids), label
    got = y_f64(y)
    assert np.all(np.isfinite(got)), label
    err = max_rel_err(got, ref)
    print(f"  {label}: block_m {bm}, max|err|/max|ref| = {err:.3e}")
    assert err <= TOL, label
    assert torch.equal(y.view(torch.int16), yc.view(torch.int16)), label
    c.pool.close()
