"""GPU tests of the multi-layer pipeline (moe_pipeline_*) through the C ABI.

Three layers share one pool and the two load buffers; layer l reads buffer
l % 2.  Every pool page that holds no expert, every load-buffer slot not yet
filled and every page the test hands back after a reclaim is bf16 NaN, so a
read of a page before its copy has landed, or after it was given away, puts
NaN into y.  Bars: y against the oracle as in the single-layer parity tests
(max |y - y_oracle| <= 2e-2 * max |y_oracle|), and y of every later pass
bit-identical to the first pass (a placement change moves where the kernels
read an expert, never how they add it up).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm
from workloads import synth

from gpu_cases import max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2
L = 3
D, F, E, K, T = 512, 256, 16, 4, 96
SLOTS = 8   # slots per load buffer
N_LB = 4    # experts each layer starts with in the load buffer
SPARE = 36  # pages no table names at the start
# cycles of the sleep kernel that holds the copy stream (a bounded spin that
# ends on its own, some hundreds of milliseconds: far longer than enqueuing a pass)
HOLD_CYCLES = 400_000_000


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


class Stack:
    """L layers over one NaN-poisoned pool, each with its table set."""

    def __init__(self, seed: int, block_m: int = 16):
        dev = "cuda"
        nan = float("nan")
        self.fd = fd = F * D
        self.specs = [synth.spec("tiny", T=T, d=D, f=F, E=E, k=K, S=0, pool_pages=3 * E, loadbuf_experts=(),
                                 loadbuf_slots=0, seed=seed + l) for l in range(L)]
        self.layers = [synth.make_layer(s) for s in self.specs]
        self.P = L * 3 * (E - N_LB) + SPARE
        g = synth.rng_for(seed, "stack_pages")
        order = [int(p) for p in g.permutation(self.P)]
        self.pool = torch.full((self.P, fd), nan, dtype=torch.bfloat16, device=dev)
        self.lbuf = [torch.full((SLOTS, 3 * fd), nan, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        self.blobs = []
        for l, Ly in enumerate(self.layers):
            bl = []
            for e in range(E):
                b = torch.empty(3 * fd, dtype=torch.bfloat16, pin_memory=True)
                b.view(torch.int16).copy_(torch.from_numpy(
                    synth.expert_blob(self.specs[l], Ly.w13, Ly.w2, e).view(np.int16)))
                bl.append(b)
            self.blobs.append(bl)
        self.tables = []
        nxt = 0
        for l in range(L):
            lb = sorted(int(e) for e in g.permutation(E)[:N_LB])
            t = np.zeros(E, dtype=synth.LOC_DTYPE)
            for e in range(E):
                if e in lb:
                    t[e]["kind"] = synth.LOC_LOADBUF
                    t[e]["idx"] = (lb.index(e), 0, 0)
                else:
                    t[e]["kind"] = synth.LOC_POOL
                    t[e]["idx"] = order[nxt: nxt + 3]
                    nxt += 3
                    self.write_pages(l, e, t[e]["idx"])
            self.tables.append(t)
        self.free = order[nxt:]
        self.handles = [pm.moe_pool_create(self.pool, self.P, D, F, E, K, 0, SLOTS, tuple(self.lbuf))
                        for _ in range(L)]
        for h, t in zip(self.handles, self.tables):
            pm.moe_set_expert_locs(h, t)
        self.block_m = block_m
        self.ws = pm.workspace(self.handles[0], T, block_m)
        self.x = [torch.from_numpy(Ly.x.view(np.int16)).to(dev).view(torch.bfloat16) for Ly in self.layers]
        self.r = [pm.route(h, torch.from_numpy(Ly.logits).to(dev), block_m, self.ws)
                  for h, Ly in zip(self.handles, self.layers)]
        self.ref = [oracle.layer(Ly.x, Ly.logits, Ly.w13, Ly.w2, K)[0] for Ly in self.layers]
        torch.cuda.synchronize()

    def write_pages(self, l, e, pages):
        b = self.blobs[l][e]
        for m, p in enumerate(pages):
            self.pool[int(p)].copy_(b[m * self.fd: (m + 1) * self.fd])

    def fill_args(self, l, table):
        lb = [e for e in range(E) if table[e]["kind"] == synth.LOC_LOADBUF]
        return [int(table[e]["idx"][0]) for e in lb], [self.blobs[l][e] for e in lb]

    def close(self):
        for h in self.handles:
            h.close()


def run_pass(pipe, st: Stack, tables, after_first_fill=None, stream=None):
    """prefetch(0); [hook]; then prefetch(l + 1) ahead of forward(l) for every layer."""
    ys = []
    pipe.prefetch(0, *st.fill_args(0, tables[0]))
    if after_first_fill is not None:
        after_first_fill()
    for l in range(L):
        if l + 1 < L:
            pipe.prefetch(l + 1, *st.fill_args(l + 1, tables[l + 1]))
        ys.append(pipe.forward(l, st.x[l], st.r[l], st.ws, stream=stream))
    return ys


def _pages(t, e):
    return [int(p) for p in t[e]["idx"]]


def change_list(st: Stack):
    """New tables, per-layer copy lists and the dropped pages: layer 0 evicts
    two experts into free slots and caches one load-buffer expert; layer 1
    caches two; layer 2 evicts three."""
    new = [t.copy() for t in st.tables]
    copies = [[] for _ in range(L)]
    dropped = []
    free = list(st.free)

    def used_slots(t):
        return {int(t[e]["idx"][0]) for e in range(E) if t[e]["kind"] == synth.LOC_LOADBUF}

    def evict(l, e):
        t = new[l]
        dropped.extend(_pages(t, e))
        slot = min(set(range(SLOTS)) - used_slots(t))
        t[e]["kind"] = synth.LOC_LOADBUF
        t[e]["idx"] = (slot, 0, 0)

    def add(l, e):
        t = new[l]
        pg = [free.pop(0) for _ in range(3)]
        t[e]["kind"] = synth.LOC_POOL
        t[e]["idx"] = pg
        copies[l].append((e, st.blobs[l][e]))

    pool_e = [[e for e in range(E) if t[e]["kind"] == synth.LOC_POOL] for t in st.tables]
    lb_e = [[e for e in range(E) if t[e]["kind"] == synth.LOC_LOADBUF] for t in st.tables]
    evict(0, pool_e[0][0])
    evict(0, pool_e[0][1])
    add(0, lb_e[0][0])
    add(1, lb_e[1][0])
    add(1, lb_e[1][1])
    for e in pool_e[2][:3]:
        evict(2, e)
    return new, copies, sorted(dropped), free


def _check_oracle(st, ys):
    for l in range(L):
        err = max_rel_err(y_f64(ys[l]), st.ref[l])
        assert err <= TOL, f"layer {l}: {err}"


@pytest.mark.parametrize("block_m", (16, 64))
def test_pipeline_passes_copy_before_switch(block_m):
    st = Stack(4100, block_m)
    copy = torch.cuda.Stream()
    pipe = pm.MoePipeline(st.handles, copy)
    y1 = run_pass(pipe, st, st.tables)
    torch.cuda.synchronize()
    _check_oracle(st, y1)
    b1 = [_bits(y) for y in y1]

    new, copies, dropped, free = change_list(st)
    ev_hold = torch.cuda.Event()

    def stage():
        # hold the copy stream so that the page copies land long after layer 0 could start
        with torch.cuda.stream(copy):
            torch.cuda._sleep(HOLD_CYCLES)
            ev_hold.record(copy)
        for l in range(L):
            pipe.stage_table(l, new[l], copies[l])

    y2 = run_pass(pipe, st, new, after_first_fill=stage)
    pending = not ev_hold.query()
    torch.cuda.synchronize()
    assert pending, "the copy stream was no longer held when the pass had been enqueued; the test shows nothing"
    _check_oracle(st, y2)
    for l in range(L):
        assert np.array_equal(_bits(y2[l]), b1[l]), f"layer {l} differs from the first pass"

    got = pipe.reclaim()
    assert sorted(got) == dropped
    assert pipe.reclaim() == []
    named = {p for t in new for e in range(E) if t[e]["kind"] == synth.LOC_POOL for p in _pages(t, e)}
    assert not named & set(got)
    # the reclaimed pages go to someone else: poison them, run again
    for p in got:
        st.pool[p].fill_(float("nan"))
    y3 = run_pass(pipe, st, new)
    torch.cuda.synchronize()
    for l in range(L):
        assert np.array_equal(_bits(y3[l]), b1[l]), f"layer {l} read a reclaimed page"
    pipe.close()
    st.close()


def test_pipeline_reclaim_waits_for_running_pass():
    st = Stack(4200)
    copy = torch.cuda.Stream()
    pipe = pm.MoePipeline(st.handles, copy)
    ev_hold = torch.cuda.Event()
    with torch.cuda.stream(copy):
        torch.cuda._sleep(HOLD_CYCLES)  # pass 1 waits for its fills behind this
        ev_hold.record(copy)
    y1 = run_pass(pipe, st, st.tables)
    new = st.tables[2].copy()
    ev = [e for e in range(E) if new[e]["kind"] == synth.LOC_POOL][0]
    dropped = _pages(new, ev)
    new[ev]["kind"] = synth.LOC_LOADBUF
    new[ev]["idx"] = (N_LB, 0, 0)
    pipe.stage_table(2, new)
    tables = list(st.tables)
    tables[2] = new
    y2 = run_pass(pipe, st, tables)
    # the dropped pages may not be named again before they are reclaimed
    t1 = st.tables[1].copy()
    e1 = [e for e in range(E) if t1[e]["kind"] == synth.LOC_LOADBUF][0]
    t1[e1]["kind"] = synth.LOC_POOL
    t1[e1]["idx"] = (dropped[0], st.free[0], st.free[1])
    with pytest.raises(pm.MoeError) as ei:
        pipe.stage_table(1, t1, [(e1, st.blobs[1][e1])])
    assert ei.value.code == pm.MOE_ERR_PAGE_ALIAS
    early = pipe.reclaim()
    still_running = not ev_hold.query()
    assert still_running, "pass 1 was no longer held at the reclaim; the test shows nothing"
    assert early == [], "pages reported while the pass reading them had not finished"
    torch.cuda.synchronize()
    got = sorted(early + pipe.reclaim())
    assert got == sorted(dropped)
    _check_oracle(st, y1)
    for l in range(L):
        assert np.array_equal(_bits(y2[l]), _bits(y1[l]))
    pipe.close()
    st.close()


def _code(fn, *a, **kw):
    with pytest.raises(pm.MoeError) as ei:
        fn(*a, **kw)
    return ei.value.code


def test_pipeline_ordering_errors():
    st = Stack(4300)
    copy = torch.cuda.Stream()
    pipe = pm.MoePipeline(st.handles, copy)
    # a layer that reads a buffer nobody filled for it
    assert _code(pipe.forward, 0, st.x[0], st.r[0], st.ws) == pm.MOE_ERR_STATE
    pipe.prefetch(0, *st.fill_args(0, st.tables[0]))
    # buffer 0 holds layer 0's experts until layer 0 runs
    assert _code(pipe.prefetch, 2, *st.fill_args(2, st.tables[2])) == pm.MOE_ERR_STATE
    pipe.prefetch(1, *st.fill_args(1, st.tables[1]))
    # layer 2 reads buffer 0, filled for layer 0
    assert _code(pipe.forward, 2, st.x[2], st.r[2], st.ws) == pm.MOE_ERR_STATE
    y0 = pipe.forward(0, st.x[0], st.r[0], st.ws)
    other = torch.cuda.Stream()
    assert _code(pipe.forward, 1, st.x[1], st.r[1], st.ws, stream=other) == pm.MOE_ERR_INVALID_ARG
    y1 = pipe.forward(1, st.x[1], st.r[1], st.ws)

    t0 = st.tables[0]
    pe = [e for e in range(E) if t0[e]["kind"] == synth.LOC_POOL]
    le = [e for e in range(E) if t0[e]["kind"] == synth.LOC_LOADBUF]
    # copy into a page the current table reads: swap two pool experts' pages
    t = t0.copy()
    t[pe[0]]["idx"], t[pe[1]]["idx"] = t0[pe[1]]["idx"].copy(), t0[pe[0]]["idx"].copy()
    assert _code(pipe.stage_table, 0, t, [(pe[0], st.blobs[0][pe[0]])]) == pm.MOE_ERR_PAGE_ALIAS
    # a page of another layer's table
    t = t0.copy()
    t[le[0]]["kind"] = synth.LOC_POOL
    t[le[0]]["idx"] = st.tables[1][[e for e in range(E) if st.tables[1][e]["kind"] == synth.LOC_POOL][0]]["idx"]
    assert _code(pipe.stage_table, 0, t, [(le[0], st.blobs[0][le[0]])]) == pm.MOE_ERR_PAGE_ALIAS
    # copies from pageable memory, or of an expert the new table does not put in the pool
    t = t0.copy()
    t[le[0]]["kind"] = synth.LOC_POOL
    t[le[0]]["idx"] = st.free[:3]
    pageable = torch.empty(3 * st.fd, dtype=torch.bfloat16)
    assert _code(pipe.stage_table, 0, t, [(le[0], pageable)]) == pm.MOE_ERR_INVALID_ARG
    assert _code(pipe.stage_table, 0, t, [(le[1], st.blobs[0][le[1]])]) == pm.MOE_ERR_INVALID_ARG
    # one change per layer until it is applied
    pipe.stage_table(0, t, [(le[0], st.blobs[0][le[0]])])
    assert _code(pipe.stage_table, 0, t, []) == pm.MOE_ERR_STATE
    # the copied pages now belong to layer 0's staged table
    t2 = st.tables[2].copy()
    l2 = [e for e in range(E) if t2[e]["kind"] == synth.LOC_LOADBUF][0]
    t2[l2]["kind"] = synth.LOC_POOL
    t2[l2]["idx"] = st.free[:3]
    assert _code(pipe.stage_table, 2, t2, [(l2, st.blobs[2][l2])]) == pm.MOE_ERR_PAGE_ALIAS
    pipe.prefetch(2, *st.fill_args(2, st.tables[2]))
    y2 = pipe.forward(2, st.x[2], st.r[2], st.ws)
    torch.cuda.synchronize()
    _check_oracle(st, [y0, y1, y2])
    pipe.close()

    # creation: tables that share a page, handles over different buffers
    h = pm.moe_pool_create(st.pool, st.P, D, F, E, K, 0, SLOTS, tuple(st.lbuf))
    pm.moe_set_expert_locs(h, st.tables[0])
    assert _code(pm.MoePipeline, [st.handles[0], h], copy) == pm.MOE_ERR_PAGE_ALIAS
    assert _code(pm.MoePipeline, [st.handles[0], st.handles[0]], copy) == pm.MOE_ERR_INVALID_ARG
    h2 = pm.moe_pool_create(st.pool, st.P, D, F, E, K, 0, SLOTS, (st.lbuf[1], st.lbuf[0]))
    pm.moe_set_expert_locs(h2, st.tables[1])
    assert _code(pm.MoePipeline, [st.handles[0], h2], copy) == pm.MOE_ERR_INVALID_ARG
    h3 = pm.moe_pool_create(st.pool, st.P, D, F, E, K, 0, SLOTS, tuple(st.lbuf))
    assert _code(pm.MoePipeline, [st.handles[0], h3], copy) == pm.MOE_ERR_STATE
    for x in (h, h2, h3):
        x.close()
    st.close()
