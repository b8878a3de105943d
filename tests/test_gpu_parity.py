"""GPU parity of the paged fused-MoE path against the CPU oracle, through the C ABI.

Bars:
  * routing indices, sorted token order, block map and resolved weight
    addresses: bit-exact;
  * routing weights: relative 1e-6 (fp64 on both sides, rounded once to fp32
    on the GPU; the summation order of the k terms differs);
  * layer output y: max |y - y_oracle| <= 2e-2 * max |y_oracle| (bf16 inputs,
    fp32 accumulation, h and y rounded to bf16 on the GPU; the oracle is fp64);
  * paged vs contiguous weights, page permutations, tile heights: bit-identical
    (same kernels, same K order; only the per-tile base address differs).
Every pool holds bf16 NaN outside expert pages, and the load buffer that is not
active is NaN as well, so a stray read shows up as NaN in y.
"""
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_expert_weight_amd as pm
from workloads import synth

from gpu_cases import Case, host_layer, max_rel_err, y_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2
BLOCK_MS = (16, 32, 64, 128, 256)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pm.lib()


_cases = {}


def case(name, T=None) -> Case:
    key = (name, T)
    if key not in _cases:
        _cases.clear()  # keep at most one large layer resident
        torch.cuda.empty_cache()
        _cases[key] = Case(host_layer(name, T))
    return _cases[key]


def _oracle_routing(c: Case):
    return oracle.route(c.layer.logits, c.s.k, c.s.S)


def _check_routing(c: Case, r, block_m):
    ids, w = _oracle_routing(c)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids)
    np.testing.assert_allclose(r.topk_w.cpu().numpy(), w, rtol=1e-6, atol=0)
    s_ids, blk, npad = oracle.align(ids, c.s.E_tot, block_m)
    assert int(r.num_padded.item()) == npad
    assert np.array_equal(r.sorted_ids[:npad].cpu().numpy(), s_ids)
    assert np.array_equal(r.block_expert[: npad // block_m].cpu().numpy(), blk)


# ----------------------------------------------------------------------------- routing / alignment

@pytest.mark.parametrize("name,T", [("tiny", None), ("qwen15", None), ("decode", 1), ("decode", 8),
                                    ("decode", 32), ("decode", 128), ("decode", 512)])
@pytest.mark.parametrize("block_m", BLOCK_MS)
def test_route_align_bitexact(name, T, block_m):
    c = case(name, T)
    r, _ = c.route(block_m)
    torch.cuda.synchronize()
    _check_routing(c, r, block_m)


@pytest.mark.parametrize("name", ["mixtral", "qwen3n"])
@pytest.mark.parametrize("block_m", (64, 128, 256))
def test_route_align_bitexact_large(name, block_m):
    c = case(name)
    r, _ = c.route(block_m)
    torch.cuda.synchronize()
    _check_routing(c, r, block_m)


# Batches past 48 alignment chunks of 2048 picks (120000 and 132000 picks): the
# scatter workgroups read the per-chunk count table in two batches of columns.
@pytest.mark.parametrize("S", (0, 1))
@pytest.mark.parametrize("block_m", (16, 128))
def test_route_align_bitexact_many_chunks(S, block_m):
    s = synth.spec("tiny", T=12000, E=64, k=10, S=S, pool_pages=3 * (64 + S), loadbuf_experts=(), loadbuf_slots=0,
                   seed=3200 + S)
    c = Case(synth.make_layer(s))
    r, _ = c.route(block_m)
    torch.cuda.synchronize()
    _check_routing(c, r, block_m)


# The one-workgroup routing forms at their limits: many experts with a shared
# one (lanes hold 8 logits each), the largest expert count (E+S = 1024) with
# k = 32 and the most picks the smallest form takes (T*(k+S) = 495), and the
# first batch sizes past it.
@pytest.mark.parametrize("E,k,S,T", [(512, 10, 1, 1), (512, 10, 1, 16), (512, 10, 1, 32), (1023, 32, 1, 15),
                                     (1023, 32, 1, 16), (60, 4, 0, 33), (8, 2, 0, 64)])
@pytest.mark.parametrize("block_m", (16, 256))
def test_route_align_small_batch_forms(E, k, S, T, block_m):
    s = synth.spec("tiny", T=T, E=E, k=k, S=S, pool_pages=3 * (E + S), loadbuf_experts=(), loadbuf_slots=0,
                   seed=3000 + E + T)
    c = Case(synth.make_layer(s))
    r, _ = c.route(block_m)
    torch.cuda.synchronize()
    _check_routing(c, r, block_m)


def test_route_weights_at_large_logit_gaps():
    """Picks 50 and 80 below the first one: the weights keep the 1e-6 relative
    bar (exp(-80) is still a normal fp32 value)."""
    s = synth.spec("tiny", T=256, E=60, k=4, pool_pages=3 * 60, loadbuf_experts=(), loadbuf_slots=0, seed=3100)
    L = synth.make_layer(s)
    g = np.random.default_rng(31)
    lg = (-200.0 - np.abs(g.standard_normal((s.T, s.E)))).astype(np.float32)
    for t in range(s.T):
        ids = g.choice(s.E, 4, replace=False)
        lg[t, ids] = np.array([0.0, -20.0, -50.0, -80.0]) + g.uniform(-1, 1, 4)
    L.logits = lg
    c = Case(L)
    for bm in (16, 64):
        r, _ = c.route(bm)
        torch.cuda.synchronize()
        _check_routing(c, r, bm)
    ids, w = _oracle_routing(c)
    assert w[:, 3].min() < 1e-33  # the smallest weights are tiny but normal fp32 values


def test_route_ties_and_edge_logits():
    """Exact ties everywhere: the lower expert id must win."""
    s = synth.spec("tiny", T=300, E=40, k=6, pool_pages=3 * 40, loadbuf_experts=(), loadbuf_slots=0)
    L = synth.make_layer(s)
    L.logits = np.round(L.logits * 2).astype(np.float32) / 2
    L.logits[:7] = 0.0
    c = Case(L)
    for bm in (16, 64):
        r, _ = c.route(bm)
        torch.cuda.synchronize()
        _check_routing(c, r, bm)


# ----------------------------------------------------------------------------- addresses

def _resolve(c: Case, active, e, which, row, col):
    dev = "cuda"
    te = torch.tensor(e, dtype=torch.int32, device=dev)
    tw = torch.tensor(which, dtype=torch.int32, device=dev)
    tr = torch.tensor(row, dtype=torch.int64, device=dev)
    tc = torch.tensor(col, dtype=torch.int64, device=dev)
    off = torch.empty(len(e), dtype=torch.int64, device=dev)
    base = torch.empty(len(e), dtype=torch.int32, device=dev)
    pm.moe_resolve_addrs(c.pool, active, te, tw, tr, tc, off, base)
    torch.cuda.synchronize()
    return off.cpu().numpy(), base.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "qwen15"])
@pytest.mark.parametrize("active", [0, 1])
def test_resolve_addrs_bitexact(name, active):
    c = case(name)
    s = c.s
    g = np.random.default_rng(7)
    qs = []
    for e in range(s.E_tot):
        for which, R, C in ((0, 2 * s.f, s.d), (1, s.d, s.f)):
            rows = np.concatenate([[0, R - 1, s.f - 1, s.f] if which == 0 else [0, R - 1], g.integers(0, R, 6)])
            cols = np.concatenate([[0, C - 1], g.integers(0, C, rows.size - 2)])
            for r_, c_ in zip(rows, cols):
                qs.append((e, which, int(r_), int(c_)))
    e, which, row, col = (list(v) for v in zip(*qs))
    off, base = _resolve(c, active, e, which, row, col)
    ref_off, ref_base = oracle.addr(c.layer.placement.locs, s.f, s.d, s.pool_pages, s.loadbuf_slots, active,
                                    e, which, row, col)
    assert np.array_equal(base, ref_base)
    assert np.array_equal(off, ref_off)


def test_resolve_addrs_rejects_out_of_range():
    c = case("tiny")
    s = c.s
    off, base = _resolve(c, 0, [s.E_tot, 0, 0, -1], [0, 2, 0, 0], [0, 0, 2 * s.f, 0], [0, 0, 0, 0])
    assert np.all(off == -1) and np.all(base == -1)


# ----------------------------------------------------------------------------- layer output

def _check_y(c: Case, y, tokens=None):
    torch.cuda.synchronize()
    ids, w = _oracle_routing(c)
    toks = np.arange(c.layer.T) if tokens is None else np.asarray(tokens)
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w, tokens=toks)
    got = y_f64(y)[toks]
    assert np.all(np.isfinite(got)), "NaN/Inf in y: a stray read of a poisoned page"
    err = max_rel_err(got, ref)
    print(f"  {c.s.name} T={c.layer.T}: max|err|/max|ref| = {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name,T", [("tiny", None), ("qwen15", None), ("decode", 1), ("decode", 8),
                                    ("decode", 32), ("decode", 128), ("decode", 512)])
def test_forward_matches_oracle(name, T):
    c = case(name, T)
    bm = pm.moe_suggest_block_m(c.pool, c.layer.T)
    y, _ = c.forward(bm)
    _check_y(c, y)


# The two large layers against the oracle on every token, at the block height
# the layer runs with (Mixtral-shaped: 256, Qwen3-Next-shaped: 128).  y is
# computed once per layer and compared in chunks of 512 tokens, a few seconds
# of oracle time each; the bar is checked per chunk (max|ref| of a chunk is at
# most that of the whole y, so this is the stricter form).
LARGE_CHUNK = 512
_large_y = {}


def large_y(name):
    if name not in _large_y:
        _large_y.clear()
        c = case(name)
        bm = pm.moe_suggest_block_m(c.pool, c.layer.T)
        y, _ = c.forward(bm)
        torch.cuda.synchronize()
        _large_y[name] = (bm, y_f64(y))
    return _large_y[name]


@pytest.mark.parametrize("name,chunk", [("mixtral", i) for i in range(4096 // LARGE_CHUNK)] +
                         [("qwen3n", i) for i in range(8192 // LARGE_CHUNK)])
def test_forward_large_all_tokens(name, chunk):
    bm, got_all = large_y(name)
    c = case(name)
    toks = np.arange(chunk * LARGE_CHUNK, min(c.layer.T, (chunk + 1) * LARGE_CHUNK))
    ids, w = _oracle_routing(c)
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w, tokens=toks)
    got = got_all[toks]
    assert np.all(np.isfinite(got)), "NaN/Inf in y: a stray read of a poisoned page"
    err = max_rel_err(got, ref)
    print(f"  {name} block_m={bm} tokens {toks[0]}..{toks[-1]}: max|err|/max|ref| = {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name", ["mixtral", "qwen3n"])
def test_large_paged_equals_contiguous_bitwise(name):
    c = case(name)
    bm = pm.moe_suggest_block_m(c.pool, c.layer.T)
    y, _ = c.forward(bm)
    yc, _ = c.contiguous(bm)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yc.view(torch.int16)), f"block_m={bm}"


@pytest.mark.parametrize("name", ["tiny", "qwen15"])
def test_forward_atomic_combine_matches_oracle(name):
    c = case(name)
    y, _ = c.forward(64, pm.MOE_FLAG_ATOMIC_COMBINE)
    _check_y(c, y)


# ----------------------------------------------------------------------------- bit identities

@pytest.mark.parametrize("name", ["tiny", "qwen15", "decode"])
def test_paged_equals_contiguous_bitwise(name):
    c = case(name)
    for bm in (16, 64, 128):
        y, _ = c.forward(bm)
        yc, _ = c.contiguous(bm)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), yc.view(torch.int16)), f"block_m={bm}"


# Tile heights 32..256 share one K summation order (32-wide MFMA steps in K
# order); the 16-row decode tile splits K over four waves and adds the partial
# sums in wave order, so it is held to the oracle tolerance instead, and so is
# a 256-row launch whose last partial wave is cut into K ranges (the layers
# below).  qwen15 and tiny never take that path: their last waves are more
# than half full (qwen15) or use the 64-column 256-row tiles (tiny).
SAME_K_ORDER = (32, 64, 128, 256)


@pytest.mark.parametrize("name", ["tiny", "qwen15"])
def test_tile_height_does_not_change_y(name):
    c = case(name)
    ys = [c.forward(bm)[0] for bm in SAME_K_ORDER]
    torch.cuda.synchronize()
    for bm, y in zip(SAME_K_ORDER[1:], ys[1:]):
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16)), f"block_m={bm}"


@pytest.mark.parametrize("name,T", [("tiny", None), ("qwen15", None), ("decode", 8)])
def test_every_tile_height_matches_oracle(name, T):
    c = case(name, T)
    for bm in BLOCK_MS:
        y, _ = c.forward(bm)
        _check_y(c, y)


# Layers whose 256-row GEMM launches split their last wave into K ranges on a
# 256-CU device (one 256-row tile per CU): in "split_all" every tile is split
# (fewer tiles than half the CUs); in "split_tail" the gate/up launch has one
# whole wave of 256 tiles and a tail of about 64 split tiles.
SPLIT_SPECS = {
    "split_all": synth.LayerSpec("split_all", 512, 512, 512, 4, 2, 0, 16, (3,), 1, None, 0, 2001),
    "split_tail": synth.LayerSpec("split_tail", 3840, 1024, 1280, 8, 2, 0, 24, (7,), 1, None, 0, 2002),
}


@functools.lru_cache(maxsize=1)
def split_case(name):
    return Case(synth.make_layer(SPLIT_SPECS[name]))


@pytest.mark.parametrize("name,ntok", [("split_all", None), ("split_tail", 96)])
def test_split_last_wave_matches_oracle(name, ntok):
    c = split_case(name)
    toks = None
    if ntok:
        g = np.random.default_rng(5)
        toks = np.unique(np.concatenate([[0, c.layer.T - 1], g.choice(c.layer.T, ntok, replace=False)]))
    for flags in (0, pm.MOE_FLAG_ATOMIC_COMBINE):
        y, _ = c.forward(256, flags)
        _check_y(c, y, toks)


@pytest.mark.parametrize("name", ["split_all", "split_tail"])
def test_split_last_wave_paged_equals_contiguous(name):
    c = split_case(name)
    y, _ = c.forward(256)
    yc, _ = c.contiguous(256)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yc.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "qwen15"])
def test_page_permutations_bitwise(name):
    """Five other seeded page assignments (and slot orders) give the same y bit for bit."""
    base = host_layer(name)
    ref = None
    for i in range(6):
        L = synth.Layer(base.spec, base.x, base.logits, base.w13, base.w2,
                        synth.make_placement(base.spec, seed_name=f"pages{i}" if i else "pages"))
        c = Case(L, active_buf=i % 2)
        y, _ = c.forward(64)
        torch.cuda.synchronize()
        if ref is None:
            ref = y
        else:
            assert torch.equal(ref.view(torch.int16), y.view(torch.int16)), f"permutation {i}"
        del c
    _cases.clear()


def test_down_projection_scaling_exact():
    """Doubling every W2 weight (exact in bf16) doubles y exactly."""
    base = host_layer("tiny")
    c1 = Case(base)
    y1, _ = c1.forward(16)
    w2x2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(base.w2) * 2)
    c2 = Case(synth.Layer(base.spec, base.x, base.logits, base.w13, w2x2, base.placement))
    y2, _ = c2.forward(16)
    torch.cuda.synchronize()
    assert torch.equal((y1.float() * 2).view(torch.int32), y2.float().view(torch.int32))


def test_swapping_gate_and_up_pages_changes_y_as_predicted():
    """Pointing W1 at the W3 page and back swaps the roles of gate and up:
    the result equals the oracle run on weights with the two halves swapped."""
    base = host_layer("tiny")
    s = base.spec
    pl = synth.make_placement(s)
    locs = pl.locs.copy()
    for e in range(s.E_tot):
        if locs[e]["kind"] == synth.LOC_POOL:
            p1, p3, p2 = locs[e]["idx"]
            locs[e]["idx"] = (p3, p1, p2)
    c = Case(synth.Layer(s, base.x, base.logits, base.w13, base.w2, pl))
    pm.moe_set_expert_locs(c.pool, locs)
    y, _ = c.forward(16)
    torch.cuda.synchronize()
    w13s = base.w13.copy()
    for e in range(s.E_tot):
        if locs[e]["kind"] == synth.LOC_POOL:
            w13s[e] = np.concatenate([base.w13[e, s.f:], base.w13[e, : s.f]])
    ids, w = oracle.route(base.logits, s.k, s.S)
    ref = oracle.moe(base.x, w13s, base.w2, ids, w)
    assert max_rel_err(y_f64(y), ref) <= TOL


# ----------------------------------------------------------------------------- double buffer protocol

def test_double_buffer_alternation():
    """Layer A reads buffer 0 while layer B's experts are copied into buffer 1
    on a side stream; then the roles swap.  Both outputs match the oracle."""
    sA = synth.SPECS["tiny"]
    sB = synth.spec("tiny", seed=2001)
    LA, LB = synth.make_layer(sA), synth.make_layer(sB)
    from workloads import device as wdev
    dA, dB = wdev.to_device(LA), wdev.to_device(LB)
    bufs = dA.loadbuf  # both layers share the two load buffers
    pool = pm.moe_pool_create(dA.pool, sA.pool_pages, sA.d, sA.f, sA.E, sA.k, sA.S, sA.loadbuf_slots, tuple(bufs))
    poolB = dB.pool
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    slots = sorted(dA.host_blobs)
    pm.moe_set_expert_locs(pool, LA.placement.locs)
    pm.moe_loadbuf_fill(pool, 0, slots, [dA.host_blobs[k] for k in slots], copy)
    ws = pm.workspace(pool, sA.T, 16)
    r = pm.route(pool, dA.logits, 16, ws)
    yA = pm.paged_forward(pool, dA.x, r, 0, ws)
    # next layer: its experts go to buffer 1 while layer A may still be computing
    pm.moe_loadbuf_fill(pool, 1, slots, [dB.host_blobs[k] for k in slots], copy)
    # layer B's resident experts: copy its pool pages in after A finished (stream-ordered on comp)
    comp.synchronize()
    dA.pool.copy_(poolB)
    pm.moe_set_expert_locs(pool, LB.placement.locs)
    rB = pm.route(pool, dB.logits, 16, ws)
    yB = pm.paged_forward(pool, dB.x, rB, 1, ws)
    torch.cuda.synchronize()
    for L, y in ((LA, yA), (LB, yB)):
        ids, w = oracle.route(L.logits, L.spec.k, L.spec.S)
        ref = oracle.moe(L.x, L.w13, L.w2, ids, w)
        assert max_rel_err(y_f64(y), ref) <= TOL
    pool.close()


@pytest.mark.parametrize("flags", [0, pm.MOE_FLAG_DEFER_READ_DONE])
def test_fill_waits_for_a_queued_forward_of_its_buffer(flags):
    """A forward reading load buffer 0 is held back on its stream behind a
    sleep kernel; a fill of buffer 0 with NaN pages is enqueued after it on a
    copy stream.  The fill must wait for that forward (write after read), so
    y matches the oracle; a forward after the fill reads the NaN pages.  With
    the deferred flag the forward records nothing on its stream, and the fill
    marks the stream instead; destroy waits for a deferred forward too."""
    c = Case(host_layer("tiny"))
    s = c.s
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    ws = pm.workspace(c.pool, s.T, 16)
    torch.cuda.synchronize()
    with torch.cuda.stream(comp):
        torch.cuda._sleep(50_000_000)
        r = pm.route(c.pool, c.dev.logits, 16, ws, stream=comp)
        y = torch.empty_like(c.dev.x)
        pm.moe_paged_forward(c.pool, c.dev.x, 16, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded,
                             0, y, ws, flags, comp)
    held = not comp.query()
    slots = sorted(c.dev.host_blobs)
    nan = torch.full((3 * s.f * s.d,), float("nan"), dtype=torch.bfloat16).pin_memory()
    pm.moe_loadbuf_fill(c.pool, 0, slots, [nan] * len(slots), copy)
    torch.cuda.synchronize()
    assert held, "the forward had finished before the fill was enqueued; the test shows nothing"
    ids, w = _oracle_routing(c)
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)
    got = y_f64(y)
    assert np.all(np.isfinite(got)) and max_rel_err(got, ref) <= TOL
    picks_loadbuf = np.isin(ids, synth.loadbuf_experts(s)).any()
    with torch.cuda.stream(comp):
        y2 = torch.empty_like(c.dev.x)
        pm.moe_paged_forward(c.pool, c.dev.x, 16, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert,
                             r.num_padded, 0, y2, ws, flags, comp)
    c.pool.close()  # waits for the forward above, also when it was deferred
    assert picks_loadbuf and np.isnan(y_f64(y2)).any()


@pytest.mark.parametrize("flags", [0, pm.MOE_FLAG_DEFER_READ_DONE])
def test_fill_waits_for_forwards_on_two_streams(flags):
    """Two forwards read load buffer 0 on two streams: the first is held back
    behind a sleep kernel, the second runs at once (and, without the deferred
    flag, re-records the buffer's "read" event on its own stream after the
    first one's).  A fill of buffer 0 with NaN pages enqueued after both must
    wait for both, so both outputs match the oracle."""
    c = Case(host_layer("tiny"))
    s = c.s
    held, free, copy = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    ys = []
    torch.cuda.synchronize()
    for st, sleep in ((held, True), (free, False)):
        ws = pm.workspace(c.pool, s.T, 16)
        with torch.cuda.stream(st):
            if sleep:
                torch.cuda._sleep(50_000_000)
            r = pm.route(c.pool, c.dev.logits, 16, ws, stream=st)
            y = torch.empty_like(c.dev.x)
            pm.moe_paged_forward(c.pool, c.dev.x, 16, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert,
                                 r.num_padded, 0, y, ws, flags, st)
        ys.append((y, ws, r))
    free.synchronize()
    still_held = not held.query()
    slots = sorted(c.dev.host_blobs)
    nan = torch.full((3 * s.f * s.d,), float("nan"), dtype=torch.bfloat16).pin_memory()
    pm.moe_loadbuf_fill(c.pool, 0, slots, [nan] * len(slots), copy)
    torch.cuda.synchronize()
    assert still_held, "the held forward had finished before the fill was enqueued; the test shows nothing"
    ids, w = _oracle_routing(c)
    assert np.isin(ids, synth.loadbuf_experts(s)).any(), "no token reads the load buffer"
    ref = oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)
    for y, _, _ in ys:
        got = y_f64(y)
        assert np.all(np.isfinite(got)) and max_rel_err(got, ref) <= TOL
    c.pool.close()


def test_state_errors():
    c = case("tiny")
    s = c.s
    # a fresh handle with no table
    p2 = pm.moe_pool_create(c.dev.pool, s.pool_pages, s.d, s.f, s.E, s.k, s.S, s.loadbuf_slots, tuple(c.dev.loadbuf))
    ws = pm.workspace(p2, s.T, 16)
    r, _ = c.route(16)
    with pytest.raises(pm.MoeError) as ei:
        pm.paged_forward(p2, c.dev.x, r, 0, ws)
    assert ei.value.code == pm.MOE_ERR_STATE
    # table names load-buffer experts but buffer 1 was never filled
    pm.moe_set_expert_locs(p2, c.layer.placement.locs)
    with pytest.raises(pm.MoeError) as ei:
        pm.paged_forward(p2, c.dev.x, r, 1, ws)
    assert ei.value.code == pm.MOE_ERR_STATE
    # workspace too small: the forward's own error is reported (the load buffer's
    # read mark, recorded after a failed forward too, does not replace it), and
    # the buffer can be filled and read again afterwards
    for flags in (0, pm.MOE_FLAG_DEFER_READ_DONE):
        with pytest.raises(pm.MoeError) as ei:
            pm.paged_forward(c.pool, c.dev.x, r, 0, ws[:256], flags)
        assert ei.value.code == pm.MOE_ERR_WORKSPACE
        assert "workspace" in str(ei.value)
    slots = sorted(c.dev.host_blobs)
    pm.moe_loadbuf_fill(c.pool, 0, slots, [c.dev.host_blobs[k] for k in slots])
    y, _ = c.forward(16)
    torch.cuda.synchronize()
    ids, w = oracle.route(c.layer.logits, s.k, s.S)
    assert max_rel_err(y_f64(y), oracle.moe(c.layer.x, c.layer.w13, c.layer.w2, ids, w)) <= TOL
    # pageable host memory is refused for a fill
    pageable = torch.empty(3 * s.f * s.d, dtype=torch.bfloat16)
    with pytest.raises(pm.MoeError) as ei:
        pm.moe_loadbuf_fill(p2, 0, [0], [pageable])
    assert ei.value.code == pm.MOE_ERR_INVALID_ARG
    p2.close()


def test_zero_tokens_is_noop():
    c = case("tiny")
    s = c.s
    x = torch.empty((0, s.d), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((0, s.E), dtype=torch.float32, device="cuda")
    ws = pm.workspace(c.pool, 0, 16)
    r = pm.route(c.pool, logits, 16, ws)
    y = pm.paged_forward(c.pool, x, r, 0, ws)
    torch.cuda.synchronize()
    assert y.shape == (0, s.d)
