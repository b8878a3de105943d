"""Seeded synthetic inputs for the paged fused-MoE layer.

This module draws random numbers and lays them out in memory; it holds none of
the layer's arithmetic (no routing, no sorting, no address formula, no FFN).
Both the CPU oracle and the HIP path take their inputs from here.

Workloads (shapes and distributions follow the five layer configurations the
Rimuru digest's kernel section is evaluated against):

  tiny     T=16,   d=128,  f=64,    E=8,   k=2        uniform logits
  qwen15   T=1024, d=2048, f=1408,  E=60,  k=4        uniform logits
  decode   T in {1,8,32,128,512} of the qwen15 layer (first T rows of a 512-row draw)
  mixtral  T=4096, d=4096, f=14336, E=8,   k=2        Zipf(1.2) expert popularity
  qwen3n   T=8192, d=2048, f=512,   E=512, k=10, +1 shared expert, Zipf(1.1)

Memory objects produced for a layer:
  * ``w13``  uint16 (bf16 bits) [E+S, 2f, d]: rows [0,f) are W1 (gate), rows
    [f,2f) are W3 (up) of each expert.
  * ``w2``   uint16 [E+S, d, f]: the down projection of each expert.
  * ``x``    uint16 [T, d] hidden states; ``logits`` float32 [T, E].
  * a page assignment: for experts resident in the pool, the three page
    numbers (W1, W3, W2); for the rest, a slot in the load buffer.
  * the pool image is whole pages: page p holds one matrix copied as a block
    (``pool[p] = matrix.reshape(-1)``); every page that holds no expert matrix
    is filled with bf16 NaN so that a stray read poisons the output.
"""
from __future__ import annotations

import concurrent.futures as _fut
import dataclasses
import os
import zlib
from typing import Dict, List, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# kind codes of one location-table entry (int32 kind, int32 idx[3])
LOC_POOL = 0
LOC_LOADBUF = 1

LOC_DTYPE = np.dtype([("kind", "<i4"), ("idx", "<i4", (3,))])


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    S: int                       # shared experts (0 or 1)
    pool_pages: int
    loadbuf_experts: tuple       # routed expert ids served from the load buffer
    loadbuf_slots: int           # slots per load buffer
    zipf_s: Optional[float]      # None: logits ~ N(0,1)
    kv_pages_per_hole: int       # small KV pages carved from one non-expert page (0: plain free pages)
    seed: int

    @property
    def E_tot(self) -> int:
        return self.E + self.S

    @property
    def k_eff(self) -> int:
        return self.k + self.S


def _spec_table() -> Dict[str, LayerSpec]:
    t = {}
    t["tiny"] = LayerSpec("tiny", 16, 128, 64, 8, 2, 0, 32, (6, 7), 2, None, 0, 1001)
    t["qwen15"] = LayerSpec("qwen15", 1024, 2048, 1408, 60, 4, 0, 256,
                            tuple(range(48, 60)), 12, None, 0, 1002)
    t["decode"] = LayerSpec("decode", 512, 2048, 1408, 60, 4, 0, 256,
                            tuple(range(30, 60)), 30, None, 0, 1003)
    # 112 MiB expert pages, 8 of 32 pages carved into 64 KiB KV pages
    t["mixtral"] = LayerSpec("mixtral", 4096, 4096, 14336, 8, 2, 0, 32, (), 0, 1.2,
                             (14336 * 4096 * 2) // (64 * 1024), 1004)
    # 2 MiB expert pages; 64 coldest experts via the load buffer; 16-token KV pages of 32 KiB
    t["qwen3n"] = LayerSpec("qwen3n", 8192, 2048, 512, 512, 10, 1, 2048, (), 64, 1.1,
                            (512 * 2048 * 2) // (32 * 1024), 1005)
    return t


SPECS = _spec_table()
DECODE_T = (1, 8, 32, 128, 512)


def spec(name: str, **override) -> LayerSpec:
    return dataclasses.replace(SPECS[name], **override)


def rng_for(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream per (seed, array name)."""
    ss = np.random.SeedSequence([seed, zlib.crc32(name.encode())])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even), returned as uint16 bits."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> 16
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    u += r
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 20   # elements per independent random stream


def _normal_tasks(seed: int, name: str, out: np.ndarray, std: float):
    """Work items that fill ``out`` (any shape, contiguous uint16) with N(0, std)
    rounded to bf16.  The array is cut into fixed chunks of _CHUNK elements,
    each drawn from its own stream (seed, name#i), so the values do not depend on
    how many threads draw them."""
    flat = out.reshape(-1)
    n = flat.size

    def draw(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        a = rng_for(seed, f"{name}#{i}").standard_normal(size=hi - lo, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        flat[lo:hi] = f32_to_bf16_bits(a)

    return [(draw, i) for i in range((n + _CHUNK - 1) // _CHUNK)]


def _run(tasks):
    if len(tasks) == 1:
        fn, i = tasks[0]
        fn(i)
        return
    with _fut.ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(lambda t: t[0](t[1]), tasks))


def _normal_bf16(seed: int, name: str, shape, std: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    _run(_normal_tasks(seed, name, out, std))
    return out


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def zipf_rank(s: LayerSpec) -> np.ndarray:
    """rank[e] in 1..E: seeded permutation of expert ids (rank 1 = hottest)."""
    perm = rng_for(s.seed, "zipf_rank").permutation(s.E)
    rank = np.empty(s.E, dtype=np.int64)
    rank[perm] = np.arange(1, s.E + 1)
    return rank


def loadbuf_experts(s: LayerSpec) -> List[int]:
    """Routed experts that are not resident in the pool (served from a load buffer)."""
    if s.zipf_s is not None and s.loadbuf_slots > 0 and not s.loadbuf_experts:
        rank = zipf_rank(s)
        coldest = np.argsort(-rank, kind="stable")[: s.loadbuf_slots]
        return sorted(int(e) for e in coldest)
    return list(s.loadbuf_experts)


def make_logits(s: LayerSpec, T: Optional[int] = None) -> np.ndarray:
    """Router logits float32 [T, E].  N(0,1), or log-Zipf bias + Gumbel(0,1) noise."""
    T = s.T if T is None else T
    g = rng_for(s.seed, "logits")
    if s.zipf_s is None:
        return g.standard_normal(size=(s.T, s.E), dtype=np.float32)[:T].copy()
    rank = zipf_rank(s).astype(np.float64)
    p = rank ** (-s.zipf_s)
    p /= p.sum()
    bias = np.log(p)
    noise = g.gumbel(size=(s.T, s.E))
    return (bias[None, :] + noise).astype(np.float32)[:T].copy()


def make_x(s: LayerSpec, T: Optional[int] = None) -> np.ndarray:
    T = s.T if T is None else T
    return _normal_bf16(s.seed, "x", (s.T, s.d), 1.0)[:T].copy()


def _expert_tasks(s: LayerSpec, e: int, w13: np.ndarray, w2: np.ndarray):
    return (_normal_tasks(s.seed, f"w1_{e}", w13[: s.f], 0.02)
            + _normal_tasks(s.seed, f"w3_{e}", w13[s.f:], 0.02)
            + _normal_tasks(s.seed, f"w2_{e}", w2, 0.02))


def make_expert(s: LayerSpec, e: int):
    """(w13 [2f, d], w2 [d, f]) bf16 bits of expert e; every weight ~ N(0, 0.02)."""
    w13 = np.empty((2 * s.f, s.d), dtype=np.uint16)
    w2 = np.empty((s.d, s.f), dtype=np.uint16)
    _run(_expert_tasks(s, e, w13, w2))
    return w13, w2


def make_weights(s: LayerSpec):
    """All experts: w13 [E+S, 2f, d] and w2 [E+S, d, f] (bf16 bits)."""
    w13 = np.empty((s.E_tot, 2 * s.f, s.d), dtype=np.uint16)
    w2 = np.empty((s.E_tot, s.d, s.f), dtype=np.uint16)
    tasks = []
    for e in range(s.E_tot):
        tasks += _expert_tasks(s, e, w13[e], w2[e])
    _run(tasks)
    return w13, w2


@dataclasses.dataclass
class Placement:
    """Where each expert lives.  ``locs`` is the location table (LOC_DTYPE [E+S])."""
    locs: np.ndarray
    expert_pages: np.ndarray      # int64 [n_pool_experts*3] pages holding expert matrices
    hole_pages: np.ndarray        # pages carved into KV pages (poisoned)
    free_pages: np.ndarray        # other non-expert pages (poisoned)
    slot_expert: np.ndarray       # int32 [slots]: expert id in each load-buffer slot, -1 = empty


def make_placement(s: LayerSpec, seed_name: str = "pages") -> Placement:
    lb = set(loadbuf_experts(s))
    pool_experts = [e for e in range(s.E_tot) if e not in lb]
    need = 3 * len(pool_experts)
    if need > s.pool_pages:
        raise ValueError(f"{s.name}: {need} expert pages do not fit a {s.pool_pages}-page pool")
    g = rng_for(s.seed, seed_name)
    order = g.permutation(s.pool_pages)
    locs = np.zeros(s.E_tot, dtype=LOC_DTYPE)
    for i, e in enumerate(pool_experts):
        locs[e]["kind"] = LOC_POOL
        locs[e]["idx"] = order[3 * i: 3 * i + 3]
    rest = order[need:]
    if s.kv_pages_per_hole > 0:
        # small pages must tile an expert page exactly (three-tier page sizes)
        if (s.f * s.d * 2) % s.kv_pages_per_hole:
            raise ValueError("KV page size does not divide the expert page")
        holes, free = rest, rest[:0]
    else:
        holes, free = rest[:0], rest
    slot_perm = g.permutation(s.loadbuf_slots) if s.loadbuf_slots else np.zeros(0, np.int64)
    slot_expert = np.full(s.loadbuf_slots, -1, dtype=np.int32)
    for i, e in enumerate(sorted(lb)):
        slot = int(slot_perm[i])
        locs[e]["kind"] = LOC_LOADBUF
        locs[e]["idx"] = (slot, 0, 0)
        slot_expert[slot] = e
    return Placement(locs, order[:need].astype(np.int64), np.sort(holes), np.sort(free), slot_expert)


def build_pool_image(s: LayerSpec, w13: np.ndarray, w2: np.ndarray, pl: Placement) -> np.ndarray:
    """Pool as uint16 pages [pool_pages, f*d]; whole matrices copied page by page."""
    pool = np.full((s.pool_pages, s.f * s.d), BF16_NAN, dtype=np.uint16)
    for e in range(s.E_tot):
        if pl.locs[e]["kind"] != LOC_POOL:
            continue
        p1, p3, p2 = (int(v) for v in pl.locs[e]["idx"])
        pool[p1] = w13[e, : s.f].reshape(-1)
        pool[p3] = w13[e, s.f:].reshape(-1)
        pool[p2] = w2[e].reshape(-1)
    return pool


def expert_blob(s: LayerSpec, w13: np.ndarray, w2: np.ndarray, e: int) -> np.ndarray:
    """One expert as it travels to a load-buffer slot: W1, W3, W2 back to back (3*f*d)."""
    return np.concatenate([w13[e, : s.f].reshape(-1), w13[e, s.f:].reshape(-1), w2[e].reshape(-1)])


def build_loadbuf_image(s: LayerSpec, w13: np.ndarray, w2: np.ndarray, pl: Placement) -> np.ndarray:
    """The filled load buffer [slots, 3*f*d]; empty slots poisoned."""
    buf = np.full((s.loadbuf_slots, 3 * s.f * s.d), BF16_NAN, dtype=np.uint16)
    for slot, e in enumerate(pl.slot_expert):
        if e >= 0:
            buf[slot] = expert_blob(s, w13, w2, int(e))
    return buf


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    x: np.ndarray
    logits: np.ndarray
    w13: np.ndarray
    w2: np.ndarray
    placement: Placement

    @property
    def T(self) -> int:
        return self.x.shape[0]


def make_layer(name_or_spec, T: Optional[int] = None, with_weights: bool = True) -> Layer:
    s = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    x = make_x(s, T)
    logits = make_logits(s, T)
    if with_weights:
        w13, w2 = make_weights(s)
    else:
        w13 = w2 = None
    return Layer(s, x, logits, w13, w2, make_placement(s))
