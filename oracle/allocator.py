"""CPU oracle of Rimuru's three-tier page pool (the digest "Rimuru: Unified
Memory Management for Modern LLM Serving via Elastic Expert Offloading",
section "One pool for data whose sizes differ by orders of magnitude").

TEST INFRASTRUCTURE.  Only tests/ and the benchmark may import this module.
The library's own allocator (paged_expert_weight_amd/csrc/allocator.cpp)
shares no code with it.

What the section fixes, and this model follows step by step:
  * views: the pool is one byte range; every kind of page indexes it with its
    own page size, so page i of a kind of size B covers bytes [i*B, (i+1)*B);
  * tiers: huge pages of lcm(expert page, SSM page) bytes (the expert page
    when the model has no SSM layers); middle pages (expert and SSM pages);
    small pages (KV and convolution-state pages), whose sizes divide the
    huge page;
  * allocation splits downward: a KV request first takes a free small page
    that is already split off, then splits a free expert page, and only then
    turns a free huge page into expert pages; a huge page is never cut
    straight into small pages;
  * reclamation merges upward: when every small page of an expert page is
    free it is an expert page again, and when every page under a huge page is
    free the huge page returns to the pool;
  * same-request packing: small pages of one expert page go to one request
    where possible, so that they are freed together.

Readings where the section leaves a step open (listed in the design notes):
  * small pages are carved from expert pages only, so their sizes must divide
    the expert page (which implies that they divide the huge page); one
    split expert page holds small pages of one kind;
  * a huge page is split into middle pages of one kind;
  * among candidates of equal rank the lowest page index wins (free pages,
    split pages, slots within a page);
  * packing order for a small page of request r: a free slot in an expert
    page that already holds r's pages, then a free slot in any split page of
    that kind, then a fresh split; switching packing off drops the first rank;
  * a request for n pages is all or nothing, and is served one page at a time
    by the rules above.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

KV, CONV = 0, 1
KIND_NAMES = ("kv", "conv")


class AllocError(Exception):
    """The pool cannot serve the request (nothing was changed)."""


class Pool:
    def __init__(self, pool_bytes: int, expert_bytes: int, kv_bytes: int, ssm_bytes: int = 0,
                 conv_bytes: int = 0, packing: bool = True):
        if min(pool_bytes, expert_bytes, kv_bytes) <= 0 or ssm_bytes < 0 or conv_bytes < 0:
            raise ValueError("sizes must be positive (ssm and conv may be 0)")
        self.huge_bytes = math.lcm(expert_bytes, ssm_bytes) if ssm_bytes else expert_bytes
        for b in (kv_bytes, conv_bytes):
            if b and expert_bytes % b:
                raise ValueError("small page sizes must divide the expert page")
        if pool_bytes % self.huge_bytes:
            raise ValueError("the pool must hold a whole number of huge pages")
        self.expert_bytes, self.ssm_bytes = expert_bytes, ssm_bytes
        self.small_bytes = (kv_bytes, conv_bytes)
        self.packing = packing
        self.n_huge = pool_bytes // self.huge_bytes
        self.e_per_huge = self.huge_bytes // expert_bytes
        self.s_per_huge = self.huge_bytes // ssm_bytes if ssm_bytes else 0
        # huge page -> None (free, whole) | "expert" | "ssm"
        self.huge: List[Optional[str]] = [None] * self.n_huge
        # expert page -> "free" | "used" | ("split", kind); present while its huge page is split into expert pages
        self.mid: Dict[int, object] = {}
        # ssm page -> "free" | "used"
        self.ssm: Dict[int, str] = {}
        # (kind, small page) -> owner request, or None when free; present while its expert page is split
        self.small: Dict[tuple, Optional[int]] = {}

    # ------------------------------------------------------------ geometry
    def per_mid(self, kind: int) -> int:
        return self.expert_bytes // self.small_bytes[kind]

    def mid_of_small(self, kind: int, q: int) -> int:
        return q // self.per_mid(kind)

    def huge_of_mid(self, p: int) -> int:
        return p // self.e_per_huge

    def huge_of_ssm(self, s: int) -> int:
        return s // self.s_per_huge

    # ------------------------------------------------------------ splitting
    def _split_huge(self, kind: str) -> None:
        h = self.huge.index(None)  # lowest free huge page
        self.huge[h] = kind
        if kind == "expert":
            for p in range(h * self.e_per_huge, (h + 1) * self.e_per_huge):
                self.mid[p] = "free"
        else:
            for s in range(h * self.s_per_huge, (h + 1) * self.s_per_huge):
                self.ssm[s] = "free"

    def _split_mid(self, p: int, kind: int) -> None:
        self.mid[p] = ("split", kind)
        n = self.per_mid(kind)
        for q in range(p * n, (p + 1) * n):
            self.small[(kind, q)] = None

    # ------------------------------------------------------------ merging
    def _merge_huge(self, h: int) -> None:
        if self.huge[h] == "expert":
            ps = range(h * self.e_per_huge, (h + 1) * self.e_per_huge)
            if all(self.mid[p] == "free" for p in ps):
                for p in ps:
                    del self.mid[p]
                self.huge[h] = None
        elif self.huge[h] == "ssm":
            ss = range(h * self.s_per_huge, (h + 1) * self.s_per_huge)
            if all(self.ssm[s] == "free" for s in ss):
                for s in ss:
                    del self.ssm[s]
                self.huge[h] = None

    def _merge_mid(self, p: int, kind: int) -> None:
        n = self.per_mid(kind)
        qs = range(p * n, (p + 1) * n)
        if all(self.small[(kind, q)] is None for q in qs):
            for q in qs:
                del self.small[(kind, q)]
            self.mid[p] = "free"
            self._merge_huge(self.huge_of_mid(p))

    # ------------------------------------------------------------ capacity
    def free_huge(self) -> int:
        return self.huge.count(None)

    def free_mid(self) -> int:
        return sum(1 for v in self.mid.values() if v == "free")

    def expert_pages_available(self) -> int:
        return self.free_mid() + self.free_huge() * self.e_per_huge

    # ------------------------------------------------------------ middle tier
    def alloc_expert(self, n: int) -> List[int]:
        if n < 0:
            raise ValueError("n < 0")
        if self.expert_pages_available() < n:
            raise AllocError("not enough expert pages")
        out = []
        for _ in range(n):
            free = sorted(p for p, v in self.mid.items() if v == "free")
            if not free:
                self._split_huge("expert")
                free = sorted(p for p, v in self.mid.items() if v == "free")
            p = free[0]
            self.mid[p] = "used"
            out.append(p)
        return out

    def free_expert(self, pages: List[int]) -> None:
        if len(set(pages)) != len(pages) or any(self.mid.get(p) != "used" for p in pages):
            raise ValueError("not an allocated expert page")
        for p in pages:
            self.mid[p] = "free"
            self._merge_huge(self.huge_of_mid(p))

    def alloc_ssm(self, n: int) -> List[int]:
        if not self.ssm_bytes:
            raise ValueError("the pool has no SSM pages")
        avail = sum(1 for v in self.ssm.values() if v == "free") + self.free_huge() * self.s_per_huge
        if n < 0 or avail < n:
            raise AllocError("not enough SSM pages")
        out = []
        for _ in range(n):
            free = sorted(s for s, v in self.ssm.items() if v == "free")
            if not free:
                self._split_huge("ssm")
                free = sorted(s for s, v in self.ssm.items() if v == "free")
            s = free[0]
            self.ssm[s] = "used"
            out.append(s)
        return out

    def free_ssm(self, pages: List[int]) -> None:
        if len(set(pages)) != len(pages) or any(self.ssm.get(s) != "used" for s in pages):
            raise ValueError("not an allocated SSM page")
        for s in pages:
            self.ssm[s] = "free"
            self._merge_huge(self.huge_of_ssm(s))

    # ------------------------------------------------------------ small tier
    def _free_slots(self, kind: int) -> List[int]:
        return sorted(q for (k, q), o in self.small.items() if k == kind and o is None)

    def alloc_small(self, kind: int, request: int, n: int) -> List[int]:
        if not self.small_bytes[kind]:
            raise ValueError("the pool has no pages of this kind")
        if n < 0:
            raise ValueError("n < 0")
        if len(self._free_slots(kind)) + self.expert_pages_available() * self.per_mid(kind) < n:
            raise AllocError("not enough small pages")
        out = []
        for _ in range(n):
            slots = self._free_slots(kind)
            pick = None
            if self.packing:
                mine = {self.mid_of_small(kind, q) for (k, q), o in self.small.items()
                        if k == kind and o == request}
                own = [q for q in slots if self.mid_of_small(kind, q) in mine]
                if own:
                    pick = own[0]
            if pick is None and slots:
                pick = slots[0]
            if pick is None:
                free = sorted(p for p, v in self.mid.items() if v == "free")
                if not free:
                    self._split_huge("expert")
                    free = sorted(p for p, v in self.mid.items() if v == "free")
                self._split_mid(free[0], kind)
                pick = free[0] * self.per_mid(kind)
            self.small[(kind, pick)] = request
            out.append(pick)
        return out

    def free_small(self, kind: int, pages: List[int]) -> None:
        if len(set(pages)) != len(pages) or any(self.small.get((kind, q)) is None for q in pages):
            raise ValueError("not an allocated small page")
        for q in pages:
            self.small[(kind, q)] = None
            self._merge_mid(self.mid_of_small(kind, q), kind)

    def free_request(self, request: int) -> int:
        """Free every small page of one request (kinds in order, pages ascending)."""
        n = 0
        for kind in (KV, CONV):
            qs = sorted(q for (k, q), o in self.small.items() if k == kind and o == request)
            self.free_small(kind, qs)
            n += len(qs)
        return n

    # ------------------------------------------------------------ state
    def stats(self) -> dict:
        used_small = [0, 0]
        free_small = [0, 0]
        for (k, q), o in self.small.items():
            (free_small if o is None else used_small)[k] += 1
        split = [sum(1 for v in self.mid.values() if v == ("split", k)) for k in (KV, CONV)]
        return {
            "free_huge": self.free_huge(),
            "free_expert": self.free_mid(),
            "used_expert": sum(1 for v in self.mid.values() if v == "used"),
            "free_ssm": sum(1 for v in self.ssm.values() if v == "free"),
            "used_ssm": sum(1 for v in self.ssm.values() if v == "used"),
            "split": split,
            "used_small": used_small,
            "free_small": free_small,
            "expert_available": self.expert_pages_available(),
            "trapped_bytes": sum(free_small[k] * self.small_bytes[k] for k in (KV, CONV)),
        }

    def byte_ranges(self) -> List[tuple]:
        """(start, end, what) of every allocated page, through its own view."""
        r = []
        for p, v in self.mid.items():
            if v == "used":
                r.append((p * self.expert_bytes, (p + 1) * self.expert_bytes, ("expert", p)))
        for s, v in self.ssm.items():
            if v == "used":
                r.append((s * self.ssm_bytes, (s + 1) * self.ssm_bytes, ("ssm", s)))
        for (k, q), o in self.small.items():
            if o is not None:
                b = self.small_bytes[k]
                r.append((q * b, (q + 1) * b, (KIND_NAMES[k], q, o)))
        return sorted(r)
