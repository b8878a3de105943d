"""Expert views behind remapped virtual addresses (moe_vmm_*), through the C ABI.

Every pool page and load-buffer matrix is its own physical allocation, mapped
into the pool / load-buffer views (which the paged kernels read through the
location table) and into the expert views w13 / w2 (which the contiguous
kernels read unchanged).  Pages that hold no expert are bf16 NaN.  Before any
kernel reads a view, plain copies read every mapped expert page back and
compare it with the matrix it should show.  Bars: y of the remapped views
bit-identical to the paged forward over the same physical pages and to the
contiguous forward over ordinary allocations, and within the oracle bar
(max |y - y_oracle| <= 2e-2 * max |y_oracle|); after each remap (an eviction
into a free slot, a load-buffer expert cached into free pages, a load-buffer
swap) the views show the new placement and y stays bit-identical.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm
from workloads import synth

from gpu_cases import max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2
BF16_NAN = 0x7FC0
H2D, D2H = 1, 2

SPEC = synth.spec("qwen3n", T=256, d=2048, f=512, E=32, k=4, S=1, pool_pages=120, loadbuf_experts=(),
                  loadbuf_slots=8, zipf_s=1.1, kv_pages_per_hole=0, seed=5200)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    h.hipMemsetD16.argtypes = [ctypes.c_void_p, ctypes.c_uint16, ctypes.c_size_t]
    return h


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


class VmmLayer:
    def __init__(self, s: synth.LayerSpec):
        self.s = s
        self.hip = _hip()
        self.L = L = synth.make_layer(s)
        self.P = P = s.f * s.d * 2
        self.fd = s.f * s.d
        try:
            self.ev = pm.ExpertViews(P, s.pool_pages, s.loadbuf_slots, s.E_tot)
        except pm.MoeError as e:
            if e.code == pm.MOE_ERR_UNSUPPORTED:
                pytest.skip(str(e))
            raise
        v = self.v = self.ev.views()
        assert v["w13"] is None and v["w2"] is None
        torch.cuda.synchronize()
        assert self.hip.hipMemsetD16(v["pool"], BF16_NAN, s.pool_pages * self.fd) == 0
        for b in (0, 1):
            assert self.hip.hipMemsetD16(v[f"loadbuf{b}"], BF16_NAN, s.loadbuf_slots * 3 * self.fd) == 0
        self.locs = L.placement.locs.copy()
        for e in range(s.E_tot):
            if self.locs[e]["kind"] == synth.LOC_POOL:
                self.write_pages(e, [int(p) for p in self.locs[e]["idx"]])
        self.blobs = {}
        for e in range(s.E_tot):
            b = torch.empty(3 * self.fd, dtype=torch.bfloat16, pin_memory=True)
            b.view(torch.int16).copy_(torch.from_numpy(synth.expert_blob(s, L.w13, L.w2, e).view(np.int16)))
            self.blobs[e] = b
        self.pool = pm.moe_pool_create(v["pool"], s.pool_pages, s.d, s.f, s.E, s.k, s.S, s.loadbuf_slots,
                                       (v["loadbuf0"], v["loadbuf1"]))
        pm.moe_set_expert_locs(self.pool, self.locs)
        self.fill(0)
        self.x = _bf16(L.x)
        self.w13 = _bf16(L.w13)
        self.w2 = _bf16(L.w2)
        self.logits = torch.from_numpy(L.logits).cuda()
        torch.cuda.synchronize()

    def mats(self, e):
        s, L = self.s, self.L
        return [L.w13[e, : s.f], L.w13[e, s.f:], L.w2[e]]

    def write_pages(self, e, pages):
        for m, p in zip(self.mats(e), pages):
            a = np.ascontiguousarray(m)
            assert self.hip.hipMemcpy(self.v["pool"] + p * self.P, a.ctypes.data, self.P, H2D) == 0

    def fill(self, buf):
        lb = [e for e in range(self.s.E_tot) if self.locs[e]["kind"] == synth.LOC_LOADBUF]
        slots = [int(self.locs[e]["idx"][0]) for e in lb]
        pm.moe_loadbuf_fill(self.pool, buf, slots, [self.blobs[e] for e in lb])
        torch.cuda.synchronize()

    def check_views(self):
        """Copy every expert-view page back and compare it with its matrix."""
        v = self.ev.views()
        assert v["w13"] and v["w2"]
        out = np.empty(self.fd, dtype=np.uint16)
        for e in range(self.s.E_tot):
            for m, want in enumerate(self.mats(e)):
                src = v["w13"] + (2 * e + m) * self.P if m < 2 else v["w2"] + e * self.P
                assert self.hip.hipMemcpy(out.ctypes.data, src, self.P, D2H) == 0
                assert np.array_equal(out, want.reshape(-1)), f"expert {e} matrix {m}"

    def forwards(self, block_m, active):
        ws = pm.workspace(self.pool, self.s.T, block_m)
        r = pm.route(self.pool, self.logits, block_m, ws)
        yp = pm.paged_forward(self.pool, self.x, r, active, ws)
        yv = self.ev.forward(self.pool, self.x, r, ws)
        yc = pm.contiguous_forward(self.pool, self.w13, self.w2, self.x, r, ws)
        torch.cuda.synchronize()
        return [t.view(torch.int16).cpu().numpy() for t in (yp, yv, yc)], yv

    def close(self):
        self.pool.close()
        self.ev.close()


@pytest.fixture(scope="module")
def vl():
    v = VmmLayer(SPEC)
    yield v
    v.close()


def test_views_before_mapping(vl):
    ws = pm.workspace(vl.pool, SPEC.T, 16)
    r = pm.route(vl.pool, vl.logits, 16, ws)
    with pytest.raises(pm.MoeError) as ei:
        vl.ev.forward(vl.pool, vl.x, r, ws)
    assert ei.value.code == pm.MOE_ERR_STATE
    bad = vl.locs.copy()
    bad[0]["idx"] = bad[1]["idx"] if bad[1]["kind"] == synth.LOC_POOL else bad[0]["idx"]
    if bad[0]["kind"] == synth.LOC_POOL and bad[1]["kind"] == synth.LOC_POOL:
        with pytest.raises(pm.MoeError) as ei:
            vl.ev.map_experts(bad, 0)
        assert ei.value.code == pm.MOE_ERR_PAGE_ALIAS
    with pytest.raises(pm.MoeError) as ei:
        vl.ev.map_experts(vl.locs[:-1], 0)
    assert ei.value.code == pm.MOE_ERR_INVALID_ARG
    assert vl.ev.views()["w13"] is None


@pytest.mark.parametrize("block_m", (16, 64))
def test_remapped_views_match_paged_and_contiguous(vl, block_m):
    n = vl.ev.map_experts(vl.locs, 0)
    assert n in (0, 3 * SPEC.E_tot)
    vl.check_views()
    (yp, yv, yc), y = vl.forwards(block_m, 0)
    assert np.array_equal(yv, yp) and np.array_equal(yv, yc)
    ids, w = oracle.route(vl.L.logits, SPEC.k, SPEC.S)
    assert max_rel_err(y_f64(y), oracle.moe(vl.L.x, vl.L.w13, vl.L.w2, ids, w)) <= TOL


def test_remap_after_placement_changes(vl):
    vl.ev.map_experts(vl.locs, 0)
    (yp0, _, _), _ = vl.forwards(16, 0)
    s = SPEC
    locs = vl.locs.copy()
    pool_e = [e for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_POOL and e != s.E]  # keep the shared one
    lb_e = [e for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_LOADBUF]
    used = {int(p) for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_POOL for p in locs[e]["idx"]}
    free = [p for p in range(s.pool_pages) if p not in used]
    # evict one pool expert into the slot a load-buffer expert leaves when it is cached in free pages
    ev_e, add_e = pool_e[0], lb_e[0]
    slot_used = {int(locs[e]["idx"][0]) for e in lb_e if e != add_e}
    locs[add_e]["kind"] = synth.LOC_POOL
    locs[add_e]["idx"] = free[:3]
    vl.write_pages(add_e, free[:3])
    locs[ev_e]["kind"] = synth.LOC_LOADBUF
    locs[ev_e]["idx"] = (min(set(range(s.loadbuf_slots)) - slot_used), 0, 0)
    vl.locs = locs
    pm.moe_set_expert_locs(vl.pool, locs)
    vl.fill(0)
    assert vl.ev.map_experts(locs, 0) == 6
    vl.check_views()
    (yp, yv, yc), _ = vl.forwards(16, 0)
    assert np.array_equal(yp, yp0) and np.array_equal(yv, yp0) and np.array_equal(yc, yp0)
    # the other load buffer: only load-buffer experts move
    vl.fill(1)
    n_lb = sum(1 for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_LOADBUF)
    assert vl.ev.map_experts(locs, 1) == 3 * n_lb
    vl.check_views()
    (yp, yv, yc), _ = vl.forwards(16, 1)
    assert np.array_equal(yp, yp0) and np.array_equal(yv, yp0)
    assert vl.ev.map_experts(locs, 1) == 0


def test_forward_rejects_other_layer_shape(vl):
    vl.ev.map_experts(vl.locs, 0)
    other = pm.moe_pool_create(vl.v["pool"], SPEC.pool_pages, SPEC.d, SPEC.f // 2, SPEC.E, SPEC.k, SPEC.S,
                               SPEC.loadbuf_slots, (vl.v["loadbuf0"], vl.v["loadbuf1"]))
    ws = pm.workspace(vl.pool, SPEC.T, 16)
    r = pm.route(vl.pool, vl.logits, 16, ws)
    with pytest.raises(pm.MoeError) as ei:
        vl.ev.forward(other, vl.x, r, ws)
    assert ei.value.code == pm.MOE_ERR_INVALID_ARG
    other.close()


@pytest.mark.parametrize("flags", [0, pm.MOE_FLAG_DEFER_READ_DONE])
def test_fill_waits_for_a_queued_vmm_forward(vl, flags):
    """A forward over the expert views that reads load buffer 0 is held back on
    its stream behind a sleep kernel; a fill of buffer 0 with NaN pages is
    enqueued after it on a copy stream.  The fill must wait for that forward
    (write after read), so y matches the oracle; a forward after the fill
    reads the NaN pages through the views (read after write)."""
    s = SPEC
    vl.fill(0)
    vl.ev.map_experts(vl.locs, 0)
    lb = [e for e in range(s.E_tot) if vl.locs[e]["kind"] == synth.LOC_LOADBUF]
    assert lb, "the table must place experts in the load buffer"
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    ws = pm.workspace(vl.pool, s.T, 16)
    r = pm.route(vl.pool, vl.logits, 16, ws)
    torch.cuda.synchronize()
    with torch.cuda.stream(comp):
        torch.cuda._sleep(50_000_000)
        y = vl.ev.forward(vl.pool, vl.x, r, ws, flags=flags, stream=comp)
    held = not comp.query()
    nan = torch.full((3 * vl.fd,), float("nan"), dtype=torch.bfloat16).pin_memory()
    slots = [int(vl.locs[e]["idx"][0]) for e in lb]
    pm.moe_loadbuf_fill(vl.pool, 0, slots, [nan] * len(slots), copy)
    torch.cuda.synchronize()
    assert held, "the forward had finished before the fill was enqueued; the test shows nothing"
    ids, w = oracle.route(vl.L.logits, s.k, s.S)
    got = y_f64(y)
    assert np.all(np.isfinite(got)) and max_rel_err(got, oracle.moe(vl.L.x, vl.L.w13, vl.L.w2, ids, w)) <= TOL
    assert np.isin(ids, lb).any()
    with torch.cuda.stream(comp):
        y2 = vl.ev.forward(vl.pool, vl.x, r, ws, flags=flags, stream=comp)
    torch.cuda.synchronize()
    assert np.isnan(y_f64(y2)).any(), "the forward after the NaN fill did not read it"
    vl.fill(0)  # the real experts back in buffer 0
