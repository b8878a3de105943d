"""Place a layer's experts in a shared page pool through the three-tier
allocator (moe_alloc_*), as a serving system would: expert pages and KV pages
come out of the same pool, and evicted experts come back wherever the
allocator finds room.  Host-side only.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Tuple

from . import MOE_ERR_NO_SPACE, MOE_PAGE_KV, MoeError, PageAllocator


def replay(alloc: PageAllocator, experts: Iterable[int], events: Iterable[Tuple]) -> Dict[str, object]:
    """Allocate 3 expert pages (W1, W3, W2) per expert in order, then replay
    churn events: ("req", id, n) takes n KV pages for request id (skipped when
    the pool is full), ("grow", id, n) adds n pages to a running request,
    ("done", id) frees them, ("evict", e) frees expert e's
    pages, ("add", e) brings it back (skipped when there is no room).  At the
    end every evicted expert comes back, finishing the oldest requests until it
    fits.  Returns {"pages": {e: (w1, w3, w2)}, "kv": {id: [pages]},
    "refused": count of refused requests}."""
    pages: Dict[int, Tuple[int, int, int]] = {}
    for e in experts:
        pages[e] = tuple(alloc.alloc_expert(3))
    kv: Dict[int, List[int]] = {}
    out = []
    refused = 0

    def try_add(e):
        try:
            pages[e] = tuple(alloc.alloc_expert(3))
            return True
        except MoeError as err:
            if err.code != MOE_ERR_NO_SPACE:
                raise
            return False

    for ev in events:
        if ev[0] == "req":
            try:
                kv[ev[1]] = alloc.alloc_small(MOE_PAGE_KV, ev[1], ev[2])
            except MoeError as err:
                if err.code != MOE_ERR_NO_SPACE:
                    raise
                refused += 1
        elif ev[0] == "grow":
            if ev[1] in kv:
                try:
                    kv[ev[1]] += alloc.alloc_small(MOE_PAGE_KV, ev[1], ev[2])
                except MoeError as err:
                    if err.code != MOE_ERR_NO_SPACE:
                        raise
                    refused += 1
        elif ev[0] == "done":
            if kv.pop(ev[1], None) is not None:
                alloc.free_request(ev[1])
        elif ev[0] == "evict":
            if ev[1] in pages:
                alloc.free_expert(list(pages.pop(ev[1])))
                out.append(ev[1])
        elif ev[0] == "add":
            if ev[1] in out and try_add(ev[1]):
                out.remove(ev[1])
    for e in list(out):
        while not try_add(e):
            oldest = min(kv)
            kv.pop(oldest)
            alloc.free_request(oldest)
        out.remove(e)
    return {"pages": pages, "kv": kv, "refused": refused}


def location_table(n_total: int, pages: Dict[int, Tuple[int, int, int]], slots: Dict[int, int]):
    """The location table (moe_expert_loc layout as a numpy structured array)
    of n_total experts: pool experts at their (W1, W3, W2) pages, the others
    in load-buffer slots.  Every expert must be placed exactly once."""
    import numpy as np

    from . import MOE_LOC_LOADBUF, MOE_LOC_POOL
    t = np.zeros(n_total, dtype=np.dtype([("kind", "<i4"), ("idx", "<i4", (3,))]))
    if set(pages) & set(slots) or set(pages) | set(slots) != set(range(n_total)):
        raise ValueError("every expert needs exactly one location")
    for e, pg in pages.items():
        t[e]["kind"] = MOE_LOC_POOL
        t[e]["idx"] = pg
    for e, s in slots.items():
        t[e]["kind"] = MOE_LOC_LOADBUF
        t[e]["idx"] = (s, 0, 0)
    return t
