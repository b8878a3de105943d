"""CPU oracle of the paged fused-MoE layer (ctypes wrapper over moe_oracle.c).

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``paged_expert_weight_amd``) never imports it and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 accumulation, OpenMP
over tokens only).  This wrapper only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_threads.restype = i32
    lib.oracle_route.argtypes = [P, i64, i32, i32, i32, P, P]
    lib.oracle_route.restype = i32
    lib.oracle_align.argtypes = [P, i64, i32, i32, P, i64, P, i64, P]
    lib.oracle_align.restype = i32
    lib.oracle_addr.argtypes = [P, i32, i64, i64, i64, i32, i32, i32, i32, i64, i64, P, P]
    lib.oracle_addr.restype = i32
    lib.oracle_moe.argtypes = [P, P, P, P, P, i64, i64, i64, i32, i32, P, i64, P]
    lib.oracle_moe.restype = i32
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    return int(_load().oracle_threads())


def route(logits: np.ndarray, k: int, S: int = 0):
    """Top-k softmax routing: (ids int32 [T, k+S], w float64 [T, k+S])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k + S), dtype=np.int32)
    w = np.zeros((T, k + S), dtype=np.float64)
    rc = _load().oracle_route(_p(logits), T, E, k, S, _p(ids), _p(w))
    if rc:
        raise ValueError(f"oracle_route rc={rc}")
    return ids, w


def align(ids: np.ndarray, E_tot: int, block_m: int):
    """Stable counting sort by expert, segments padded to block_m.

    Returns (sorted_ids int32 [num_padded], block_expert int32 [num_padded/block_m],
    num_padded)."""
    flat = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    n = flat.size
    cap = n + E_tot * (block_m - 1)
    sorted_ids = np.full(cap, -1, dtype=np.int32)
    block_expert = np.full(max(1, cap // block_m), -1, dtype=np.int32)
    num = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_align(_p(flat), n, E_tot, block_m, _p(sorted_ids), cap,
                              _p(block_expert), block_expert.size, _p(num))
    if rc:
        raise ValueError(f"oracle_align rc={rc}")
    npad = int(num[0])
    return sorted_ids[:npad].copy(), block_expert[: npad // block_m].copy(), npad


def addr(locs: np.ndarray, f: int, d: int, num_pages: int, slots: int, active_buf: int,
         e: Sequence[int], which: Sequence[int], row: Sequence[int], col: Sequence[int]):
    """Address formula per query: (off int64 [n], base int32 [n]).

    base 0 = pool, 1 = load buffer 0, 2 = load buffer 1.  Raises on a query out
    of range."""
    L = np.ascontiguousarray(locs).view(np.int32).reshape(-1, 4)
    lib = _load()
    n = len(e)
    off = np.zeros(n, dtype=np.int64)
    base = np.zeros(n, dtype=np.int32)
    o = np.zeros(1, dtype=np.int64)
    b = np.zeros(1, dtype=np.int32)
    for q in range(n):
        rc = lib.oracle_addr(_p(L), L.shape[0], f, d, num_pages, slots, active_buf,
                             int(e[q]), int(which[q]), int(row[q]), int(col[q]), _p(o), _p(b))
        if rc:
            raise ValueError(f"oracle_addr rc={rc} for query {q}")
        off[q], base[q] = o[0], b[0]
    return off, base


def moe(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, ids: np.ndarray, w: np.ndarray,
        tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """y (float64) for the listed tokens (all tokens by default)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w13 = np.ascontiguousarray(w13, dtype=np.uint16)
    w2 = np.ascontiguousarray(w2, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, d = x.shape
    E_tot, f2, d2 = w13.shape
    f = f2 // 2
    assert d2 == d and w2.shape == (E_tot, d, f) and ids.shape == w.shape and ids.shape[0] == T
    toks = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    y = np.zeros((toks.size, d), dtype=np.float64)
    rc = _load().oracle_moe(_p(x), _p(w13), _p(w2), _p(ids), _p(w), T, d, f, E_tot,
                            ids.shape[1], _p(toks), toks.size, _p(y))
    if rc:
        raise ValueError(f"oracle_moe rc={rc}")
    return y


def layer(x, logits, w13, w2, k: int, S: int = 0, tokens=None):
    """Full layer: routing then the per-token expert sum.  Returns (y, ids, w)."""
    ids, w = route(logits, k, S)
    return moe(x, w13, w2, ids, w, tokens), ids, w
