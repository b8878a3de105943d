"""Seeded serving churn for the page pool: KV requests that arrive and finish,
and experts that are evicted and brought back.  Random events only; the
allocation rules live in the allocator that replays them.

Request sizes follow a log-normal length mix (ShareGPT-like conversations:
median about 300 tokens, long tail), converted to KV pages of a fixed number of
tokens.  A real benchmark trace is not available here; this mix stands in for
one.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .synth import rng_for


def kv_pages_for(tokens: int, tokens_per_page: int) -> int:
    return max(1, math.ceil(tokens / tokens_per_page))


def events(seed: int, n_experts: int, steps: int, tokens_per_page: int = 16, arrivals: float = 3.0,
           mean_life: float = 20.0, evict_rate: float = 0.15, len_median: float = 300.0,
           len_sigma: float = 1.0) -> List[Tuple]:
    """Per step (one decode step of every live request): Poisson(arrivals) new
    requests whose prompts take ("req", id, kv pages); every live request
    generates one token and takes one more KV page each time it crosses a page
    boundary ("grow", id, 1); each live request finishes with probability
    1/mean_life ("done", id); with probability evict_rate one resident expert
    is evicted ("evict", e) and, with the same rate, one evicted expert comes
    back ("add", e)."""
    g = rng_for(seed, "churn")
    ev: List[Tuple] = []
    live: List[int] = []
    tokens = {}
    evicted: List[int] = []
    resident = list(range(n_experts))
    rid = 0
    for _ in range(steps):
        for _ in range(g.poisson(arrivals)):
            n = int(np.clip(g.lognormal(math.log(len_median), len_sigma), 16, 32768))
            ev.append(("req", rid, kv_pages_for(n, tokens_per_page)))
            tokens[rid] = n
            live.append(rid)
            rid += 1
        keep = []
        for r in live:
            if g.random() < 1.0 / mean_life:
                ev.append(("done", r))
                del tokens[r]
            else:
                if tokens[r] % tokens_per_page == 0:
                    ev.append(("grow", r, 1))
                tokens[r] += 1
                keep.append(r)
        live = keep
        if resident and g.random() < evict_rate:
            e = resident.pop(int(g.integers(len(resident))))
            evicted.append(e)
            ev.append(("evict", e))
        if evicted and g.random() < evict_rate:
            e = evicted.pop(int(g.integers(len(evicted))))
            resident.append(e)
            ev.append(("add", e))
    return ev
