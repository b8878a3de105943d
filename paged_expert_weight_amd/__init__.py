"""Paged fused-MoE layer for MI355X: Python binding of the HIP C-ABI library.

Every function here marshals arguments for the entry point of the same name in
``include/moe.h`` and checks its return code; all computation runs in the HIP
kernels of ``libpmoe.so``.  PyTorch is used for device memory and streams only.
If the library is missing, importing works but the first call raises: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_PAGE_RANGE = -2
MOE_ERR_PAGE_ALIAS = -3
MOE_ERR_SLOT_RANGE = -4
MOE_ERR_ALIGN = -5
MOE_ERR_WORKSPACE = -6
MOE_ERR_STATE = -7
MOE_ERR_HIP = -8
MOE_ERR_UNSUPPORTED = -9
MOE_ERR_NO_SPACE = -10

MOE_LOC_POOL = 0
MOE_LOC_LOADBUF = 1
MOE_FLAG_ATOMIC_COMBINE = 1
MOE_FLAG_DEFER_READ_DONE = 2
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static workspace of moe_route_forward_noalloc, per device
MOE_FORM_TILES = 0
MOE_FORM_DECODE = 1
MOE_FORM_DECODE_ROUTED = 2
MOE_PAGE_KV = 0
MOE_PAGE_CONV = 1
MOE_ALLOC_NO_PACKING = 1

# every function moe.h declares
EXPORTS = (
    "moe_pool_create", "moe_pool_destroy", "moe_validate_locs", "moe_set_expert_locs",
    "moe_route_capacity", "moe_workspace_bytes", "moe_route", "moe_paged_forward", "moe_route_forward",
    "moe_route_contiguous_forward", "moe_forward_form", "moe_route_forward_form",
    "moe_contiguous_forward", "moe_loadbuf_fill", "moe_resolve_addrs", "moe_suggest_block_m",
    "moe_stage_timing", "moe_stage_times", "moe_last_error", "moe_version",
    "moe_adjust_amounts", "moe_rank_experts", "moe_adjust_select",
    "moe_pipeline_create", "moe_pipeline_destroy", "moe_pipeline_stage_table", "moe_pipeline_prefetch",
    "moe_pipeline_forward", "moe_pipeline_reclaim",
    "moe_alloc_create", "moe_alloc_destroy", "moe_alloc_expert_pages", "moe_free_expert_pages",
    "moe_alloc_ssm_pages", "moe_free_ssm_pages", "moe_alloc_small_pages", "moe_free_small_pages",
    "moe_free_request", "moe_alloc_get_stats",
    "moe_vmm_create", "moe_vmm_destroy", "moe_vmm_views", "moe_vmm_granularity", "moe_vmm_map_experts",
    "moe_vmm_forward", "moe_route_forward_noalloc",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class moe_pool_desc(ctypes.Structure):
    _fields_ = [
        ("pool_base", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("f", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("num_shared", ctypes.c_int32),
        ("loadbuf_slots", ctypes.c_int32),
        ("loadbuf_base", ctypes.c_void_p * 2),
    ]


class moe_alloc_desc(ctypes.Structure):
    _fields_ = [("pool_bytes", ctypes.c_int64), ("expert_page_bytes", ctypes.c_int64),
                ("ssm_page_bytes", ctypes.c_int64), ("kv_page_bytes", ctypes.c_int64),
                ("conv_page_bytes", ctypes.c_int64), ("flags", ctypes.c_uint32)]


class moe_alloc_stats(ctypes.Structure):
    _fields_ = [("huge_bytes", ctypes.c_int64), ("n_huge", ctypes.c_int64), ("free_huge", ctypes.c_int64),
                ("free_expert", ctypes.c_int64), ("used_expert", ctypes.c_int64), ("free_ssm", ctypes.c_int64),
                ("used_ssm", ctypes.c_int64), ("split", ctypes.c_int64 * 2), ("used_small", ctypes.c_int64 * 2),
                ("free_small", ctypes.c_int64 * 2), ("expert_available", ctypes.c_int64),
                ("trapped_bytes", ctypes.c_int64)]


class moe_expert_loc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("idx", ctypes.c_int32 * 3)]


_lib = None


def lib():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run paged_expert_weight_amd/build.py (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    L.moe_pool_create.argtypes = [ctypes.POINTER(moe_pool_desc), ctypes.POINTER(P)]
    L.moe_pool_destroy.argtypes = [P]
    L.moe_validate_locs.argtypes = [ctypes.POINTER(moe_pool_desc), P, i32]
    L.moe_set_expert_locs.argtypes = [P, P, i32, P]
    L.moe_route_capacity.argtypes = [P, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.moe_workspace_bytes.argtypes = [P, i64, i32, u32, ctypes.POINTER(sz)]
    L.moe_route.argtypes = [P, P, i64, i32, P, P, P, P, P, P, sz, P]
    L.moe_paged_forward.argtypes = [P, P, i64, i32, P, P, P, P, P, i32, P, P, sz, u32, P]
    L.moe_contiguous_forward.argtypes = [P, P, P, P, i64, i32, P, P, P, P, P, P, P, sz, u32, P]
    L.moe_route_forward.argtypes = [P, P, P, i64, i32, P, P, P, P, P, i32, P, P, sz, u32, P]
    L.moe_route_forward_noalloc.argtypes = [P, P, P, i64, i32, P, P, P, P, P, i32, P, u32, P]
    L.moe_route_contiguous_forward.argtypes = [P, P, P, P, P, i64, i32, P, P, P, P, P, P, P, sz, u32, P]
    L.moe_loadbuf_fill.argtypes = [P, i32, i32, P, P, P]
    L.moe_resolve_addrs.argtypes = [P, i32, i64, P, P, P, P, P, P, P]
    L.moe_stage_timing.argtypes = [P, i32]
    L.moe_stage_times.argtypes = [P, P, P]
    L.moe_adjust_amounts.argtypes = [i32, i32, P, P]
    L.moe_rank_experts.argtypes = [P, i64, i32, i32, P, P]
    L.moe_adjust_select.argtypes = [i32, i32, P, P, P, i32, i32, i32, P, P, P, P]
    L.moe_pipeline_create.argtypes = [i32, P, P, ctypes.POINTER(P)]
    L.moe_pipeline_destroy.argtypes = [P]
    L.moe_pipeline_stage_table.argtypes = [P, i32, P, i32, i32, P, P]
    L.moe_pipeline_prefetch.argtypes = [P, i32, i32, P, P]
    L.moe_pipeline_forward.argtypes = [P, i32, P, i64, i32, P, P, P, P, P, P, P, sz, u32, P]
    L.moe_pipeline_reclaim.argtypes = [P, P, i32, P]
    L.moe_alloc_create.argtypes = [ctypes.POINTER(moe_alloc_desc), ctypes.POINTER(P)]
    L.moe_alloc_destroy.argtypes = [P]
    for nm in ("moe_alloc_expert_pages", "moe_free_expert_pages", "moe_alloc_ssm_pages", "moe_free_ssm_pages"):
        getattr(L, nm).argtypes = [P, i32, P]
    L.moe_alloc_small_pages.argtypes = [P, i32, i64, i32, P]
    L.moe_free_small_pages.argtypes = [P, i32, i32, P]
    L.moe_free_request.argtypes = [P, i64, ctypes.POINTER(i64)]
    L.moe_alloc_get_stats.argtypes = [P, ctypes.POINTER(moe_alloc_stats)]
    L.moe_vmm_create.argtypes = [i64, i64, i32, i32, ctypes.POINTER(P)]
    L.moe_vmm_destroy.argtypes = [P]
    L.moe_vmm_views.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                                ctypes.POINTER(P)]
    L.moe_vmm_map_experts.argtypes = [P, P, i32, i32, P, ctypes.POINTER(i32)]
    L.moe_vmm_granularity.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.moe_vmm_forward.argtypes = [P, P, P, i64, i32, P, P, P, P, P, P, P, sz, u32, P]
    L.moe_suggest_block_m.argtypes = [P, i64]
    L.moe_suggest_block_m.restype = i32
    L.moe_forward_form.argtypes = [P, i64]
    L.moe_forward_form.restype = i32
    L.moe_route_forward_form.argtypes = [P, i64]
    L.moe_route_forward_form.restype = i32
    L.moe_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("moe_last_error", "moe_suggest_block_m", "moe_forward_form", "moe_route_forward_form"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_desc(pool, num_pages: int, d: int, f: int, num_experts: int, top_k: int, num_shared: int = 0,
              loadbuf_slots: int = 0, loadbuf=(None, None)) -> moe_pool_desc:
    desc = moe_pool_desc()
    desc.pool_base = _ptr(pool) if not isinstance(pool, int) else pool
    desc.num_pages = num_pages
    desc.d, desc.f = d, f
    desc.num_experts, desc.top_k, desc.num_shared = num_experts, top_k, num_shared
    desc.loadbuf_slots = loadbuf_slots
    desc.loadbuf_base[0] = _ptr(loadbuf[0]) if loadbuf[0] is not None and not isinstance(loadbuf[0], int) else loadbuf[0]
    desc.loadbuf_base[1] = _ptr(loadbuf[1]) if loadbuf[1] is not None and not isinstance(loadbuf[1], int) else loadbuf[1]
    return desc


def locs_array(locs: np.ndarray) -> np.ndarray:
    """Location table as a contiguous int32 [n, 4] array (kind, idx0, idx1, idx2)."""
    a = np.ascontiguousarray(np.asarray(locs).view(np.int32).reshape(-1, 4), dtype=np.int32)
    return a


def moe_validate_locs(desc: moe_pool_desc, locs: np.ndarray) -> None:
    a = locs_array(locs)
    _check(lib().moe_validate_locs(ctypes.byref(desc), a.ctypes.data, a.shape[0]))


class MoePool:
    """Owner of one moe_pool handle.  ``desc`` keeps the device pointers it names;
    the tensors behind them must outlive the handle."""

    def __init__(self, desc: moe_pool_desc, keep=()):
        self.desc = desc
        self._keep = keep
        h = ctypes.c_void_p()
        _check(lib().moe_pool_create(ctypes.byref(desc), ctypes.byref(h)))
        self.handle = h

    @property
    def keff(self) -> int:
        return self.desc.top_k + self.desc.num_shared

    @property
    def E_tot(self) -> int:
        return self.desc.num_experts + self.desc.num_shared

    def close(self):
        if self.handle:
            _check(lib().moe_pool_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_pool_create(pool, num_pages, d, f, num_experts, top_k, num_shared=0, loadbuf_slots=0,
                    loadbuf=(None, None)) -> MoePool:
    desc = make_desc(pool, num_pages, d, f, num_experts, top_k, num_shared, loadbuf_slots, loadbuf)
    return MoePool(desc, keep=(pool, loadbuf))


def moe_pool_destroy(p: MoePool) -> None:
    p.close()


def moe_set_expert_locs(p: MoePool, locs: np.ndarray, stream=None) -> None:
    a = locs_array(locs)
    _check(lib().moe_set_expert_locs(p.handle, a.ctypes.data, a.shape[0], _stream(stream)))


def moe_route_capacity(p: MoePool, T: int, block_m: int):
    s, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().moe_route_capacity(p.handle, T, block_m, ctypes.byref(s), ctypes.byref(b)))
    return s.value, b.value


def moe_workspace_bytes(p: MoePool, T: int, block_m: int, flags: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(p.handle, T, block_m, flags, ctypes.byref(n)))
    return n.value


def moe_suggest_block_m(p: MoePool, T: int) -> int:
    return int(lib().moe_suggest_block_m(p.handle, T))


def moe_route(p: MoePool, logits, block_m: int, topk_ids, topk_w, sorted_ids, block_expert, num_padded,
              workspace, stream=None) -> None:
    T = logits.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().moe_route(p.handle, _ptr(logits), T, block_m, _ptr(topk_ids), _ptr(topk_w), _ptr(sorted_ids),
                           _ptr(block_expert), _ptr(num_padded), _ptr(workspace), ws_bytes, _stream(stream)))


def moe_paged_forward(p: MoePool, x, block_m: int, topk_ids, topk_w, sorted_ids, block_expert, num_padded,
                      active_buf: int, y, workspace, flags: int = 0, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_paged_forward(p.handle, _ptr(x), x.shape[0], block_m, _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded), active_buf, _ptr(y),
                                   _ptr(workspace), ws_bytes, flags, _stream(stream)))


def moe_contiguous_forward(p: MoePool, w13, w2, x, block_m: int, topk_ids, topk_w, sorted_ids, block_expert,
                           num_padded, y, workspace, flags: int = 0, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_contiguous_forward(p.handle, _ptr(w13), _ptr(w2), _ptr(x), x.shape[0], block_m,
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(sorted_ids), _ptr(block_expert),
                                        _ptr(num_padded), _ptr(y), _ptr(workspace), ws_bytes, flags,
                                        _stream(stream)))


def moe_route_forward(p: MoePool, logits, x, block_m: int, topk_ids, topk_w, sorted_ids, block_expert, num_padded,
                      active_buf: int, y, workspace, flags: int = 0, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_route_forward(p.handle, _ptr(logits), _ptr(x), x.shape[0], block_m, _ptr(topk_ids),
                                   _ptr(topk_w), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
                                   active_buf, _ptr(y), _ptr(workspace), ws_bytes, flags, _stream(stream)))


def moe_route_forward_noalloc(p: MoePool, logits, x, block_m: int, topk_ids, topk_w, sorted_ids, block_expert,
                              num_padded, active_buf: int, y, flags: int = 0, stream=None) -> None:
    _check(lib().moe_route_forward_noalloc(p.handle, _ptr(logits), _ptr(x), x.shape[0], block_m, _ptr(topk_ids),
                                           _ptr(topk_w), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
                                           active_buf, _ptr(y), flags, _stream(stream)))


def moe_route_contiguous_forward(p: MoePool, w13, w2, logits, x, block_m: int, topk_ids, topk_w, sorted_ids,
                                 block_expert, num_padded, y, workspace, flags: int = 0, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_route_contiguous_forward(p.handle, _ptr(w13), _ptr(w2), _ptr(logits), _ptr(x), x.shape[0],
                                              block_m, _ptr(topk_ids), _ptr(topk_w), _ptr(sorted_ids),
                                              _ptr(block_expert), _ptr(num_padded), _ptr(y), _ptr(workspace),
                                              ws_bytes, flags, _stream(stream)))


def moe_loadbuf_fill(p: MoePool, buf: int, slots: Sequence[int], host_src: Sequence, copy_stream=None) -> None:
    n = len(slots)
    s = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
    srcs = (ctypes.c_void_p * max(1, n))(*[_ptr(t) if not isinstance(t, int) else t for t in host_src])
    _check(lib().moe_loadbuf_fill(p.handle, buf, n, s.ctypes.data if n else None, srcs, _stream(copy_stream)))


def _ptr_array(ts: Sequence):
    n = len(ts)
    return (ctypes.c_void_p * max(1, n))(*[_ptr(t) if not isinstance(t, int) else t for t in ts])


class MoePipeline:
    """Owner of one moe_pipeline handle over the layers' MoePool objects (kept
    alive by it)."""

    def __init__(self, layers: Sequence[MoePool], copy_stream=None):
        self.layers = list(layers)
        hs = (ctypes.c_void_p * len(self.layers))(*[p.handle.value for p in self.layers])
        h = ctypes.c_void_p()
        self._copy = copy_stream
        _check(lib().moe_pipeline_create(len(self.layers), hs, _stream(copy_stream), ctypes.byref(h)))
        self.handle = h
        self._keep = []  # host sources of copies that may still be in flight

    def close(self):
        if self.handle:
            _check(lib().moe_pipeline_destroy(self.handle))
            self.handle = None
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stage_table(self, layer: int, locs: np.ndarray, copies=()) -> None:
        """copies: [(expert, pinned host tensor of 3*f*d bf16)]."""
        a = locs_array(locs)
        n = len(copies)
        e = np.ascontiguousarray(np.asarray([c[0] for c in copies], dtype=np.int32))
        srcs = _ptr_array([c[1] for c in copies])
        _check(lib().moe_pipeline_stage_table(self.handle, layer, a.ctypes.data, a.shape[0], n,
                                              e.ctypes.data if n else None, srcs))
        self._keep.append([c[1] for c in copies])

    def prefetch(self, layer: int, slots: Sequence[int], host_src: Sequence) -> None:
        n = len(slots)
        s = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
        _check(lib().moe_pipeline_prefetch(self.handle, layer, n, s.ctypes.data if n else None,
                                           _ptr_array(host_src)))

    def forward(self, layer: int, x, r: "RouteOut", ws, flags: int = 0, y=None, stream=None):
        import torch
        if y is None:
            y = torch.empty_like(x)
        _check(lib().moe_pipeline_forward(self.handle, layer, _ptr(x), x.shape[0], r.block_m, _ptr(r.topk_ids),
                                          _ptr(r.topk_w), _ptr(r.sorted_ids), _ptr(r.block_expert),
                                          _ptr(r.num_padded), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                          flags, _stream(stream)))
        return y

    def reclaim(self, cap: int = 4096):
        out = np.zeros(max(1, cap), dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().moe_pipeline_reclaim(self.handle, out.ctypes.data, cap, ctypes.byref(n)))
        return [int(v) for v in out[: n.value]]


def moe_resolve_addrs(p: MoePool, active_buf: int, e, which, row, col, off, base, stream=None) -> None:
    _check(lib().moe_resolve_addrs(p.handle, active_buf, e.numel(), _ptr(e), _ptr(which), _ptr(row), _ptr(col),
                                   _ptr(off), _ptr(base), _stream(stream)))


def moe_stage_timing(p: MoePool, enable: bool) -> None:
    _check(lib().moe_stage_timing(p.handle, 1 if enable else 0))


def moe_stage_times(p: MoePool):
    """(summed ms per stage [gate/up, down, combine], number of forwards timed)."""
    ms = (ctypes.c_float * 3)()
    n = ctypes.c_int32()
    _check(lib().moe_stage_times(p.handle, ctypes.addressof(ms), ctypes.addressof(n)))
    return [float(v) for v in ms], n.value


def moe_forward_form(p: MoePool, T: int) -> int:
    """MOE_FORM_TILES or MOE_FORM_DECODE: the GEMM form a forward of T tokens takes."""
    v = int(lib().moe_forward_form(p.handle, T))
    if v < 0:
        _check(v)
    return v


def moe_route_forward_form(p: MoePool, T: int) -> int:
    """MOE_FORM_DECODE_ROUTED when moe_route_forward routes inside the gate/up launch, else moe_forward_form's."""
    v = int(lib().moe_route_forward_form(p.handle, T))
    if v < 0:
        _check(v)
    return v


def moe_version() -> int:
    return int(lib().moe_version())


# ----------------------------------------------------------------------------- allocation helpers (torch plumbing)

class RouteOut:
    """Device buffers moe_route writes for T tokens at tile height block_m."""

    def __init__(self, p: MoePool, T: int, block_m: int, device="cuda"):
        import torch
        sorted_cap, blocks_cap = moe_route_capacity(p, T, block_m)
        self.block_m = block_m
        self.topk_ids = torch.empty((T, p.keff), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, p.keff), dtype=torch.float32, device=device)
        self.sorted_ids = torch.empty(max(1, sorted_cap), dtype=torch.int32, device=device)
        self.block_expert = torch.empty(max(1, blocks_cap), dtype=torch.int32, device=device)
        self.num_padded = torch.zeros(1, dtype=torch.int32, device=device)


def workspace(p: MoePool, T: int, block_m: int, flags: int = 0, device="cuda"):
    import torch
    n = moe_workspace_bytes(p, T, block_m, flags)
    return torch.empty(max(256, n), dtype=torch.uint8, device=device)


def route(p: MoePool, logits, block_m: int, ws, stream=None) -> RouteOut:
    r = RouteOut(p, logits.shape[0], block_m, device=logits.device)
    moe_route(p, logits, block_m, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded, ws, stream)
    return r


def paged_forward(p: MoePool, x, r: RouteOut, active_buf: int, ws, flags: int = 0, y=None, stream=None):
    import torch
    if y is None:
        y = torch.empty_like(x)
    moe_paged_forward(p, x, r.block_m, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded,
                      active_buf, y, ws, flags, stream)
    return y


def route_forward(p: MoePool, logits, x, active_buf: int, ws, block_m: int, flags: int = 0, y=None, stream=None):
    """Routing and the layer output in one call; returns (y, RouteOut)."""
    import torch
    r = RouteOut(p, logits.shape[0], block_m, device=logits.device)
    if y is None:
        y = torch.empty_like(x)
    moe_route_forward(p, logits, x, block_m, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded,
                      active_buf, y, ws, flags, stream)
    return y, r


def contiguous_forward(p: MoePool, w13, w2, x, r: RouteOut, ws, flags: int = 0, y=None, stream=None):
    import torch
    if y is None:
        y = torch.empty_like(x)
    moe_contiguous_forward(p, w13, w2, x, r.block_m, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert,
                           r.num_padded, y, ws, flags, stream)
    return y


# ----------------------------------------------------------------------------- adjuster (host policy)

def adjust_amounts(short_pages: int, free_pages: int):
    """(experts to evict, experts to add) for one scheduling round."""
    import numpy as np
    out = np.zeros(2, dtype=np.int32)
    _check(lib().moe_adjust_amounts(int(short_pages), int(free_pages), out[0:].ctypes.data,
                                    out[1:].ctypes.data))
    return int(out[0]), int(out[1])


def rank_experts(topk_ids, E: int):
    """(ranking, prob) of one layer from sample routing topk_ids [T][k] (host array)."""
    import numpy as np
    ids = np.ascontiguousarray(np.asarray(topk_ids, dtype=np.int32))
    T, k = (ids.shape[0], ids.shape[1]) if ids.ndim == 2 else (0, 0)
    ranking = np.empty(E, dtype=np.int32)
    prob = np.empty(E, dtype=np.float32)
    _check(lib().moe_rank_experts(ids.ctypes.data, T, k, int(E), ranking.ctypes.data, prob.ctypes.data))
    return ranking, prob


def adjust_select(ranking, prob, resident, offload_limit: int, n_evict: int, n_add: int):
    """Change list [(layer, expert, 1 add / 0 evict)] and the new resident counts."""
    import numpy as np
    rk = np.ascontiguousarray(np.asarray(ranking, dtype=np.int32))
    pr = np.ascontiguousarray(np.asarray(prob, dtype=np.float32))
    L, E = rk.shape
    res = np.ascontiguousarray(np.asarray(resident, dtype=np.int32)).copy()
    cap = max(1, int(n_evict) + int(n_add))
    ol, oe, oa = (np.zeros(cap, dtype=np.int32) for _ in range(3))
    n = np.zeros(1, dtype=np.int32)
    _check(lib().moe_adjust_select(L, E, rk.ctypes.data, pr.ctypes.data, res.ctypes.data, int(offload_limit),
                                   int(n_evict), int(n_add), ol.ctypes.data, oe.ctypes.data, oa.ctypes.data,
                                   n.ctypes.data))
    m = int(n[0])
    return [(int(ol[i]), int(oe[i]), int(oa[i])) for i in range(m)], [int(v) for v in res]


# ----------------------------------------------------------------------------- three-tier page pool (host)

class PageAllocator:
    """Owner of one moe_alloc: the three-tier page pool over one byte range."""

    def __init__(self, pool_bytes: int, expert_bytes: int, kv_bytes: int, ssm_bytes: int = 0, conv_bytes: int = 0,
                 packing: bool = True):
        d = moe_alloc_desc(pool_bytes, expert_bytes, ssm_bytes, kv_bytes, conv_bytes,
                           0 if packing else MOE_ALLOC_NO_PACKING)
        h = ctypes.c_void_p()
        _check(lib().moe_alloc_create(ctypes.byref(d), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _check(lib().moe_alloc_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _pages(n):
        return np.zeros(max(1, n), dtype=np.int64)

    def alloc_expert(self, n: int):
        out = self._pages(n)
        _check(lib().moe_alloc_expert_pages(self.handle, n, out.ctypes.data))
        return [int(v) for v in out[:n]]

    def free_expert(self, pages):
        a = np.ascontiguousarray(np.asarray(pages, dtype=np.int64))
        _check(lib().moe_free_expert_pages(self.handle, a.size, a.ctypes.data if a.size else None))

    def alloc_ssm(self, n: int):
        out = self._pages(n)
        _check(lib().moe_alloc_ssm_pages(self.handle, n, out.ctypes.data))
        return [int(v) for v in out[:n]]

    def free_ssm(self, pages):
        a = np.ascontiguousarray(np.asarray(pages, dtype=np.int64))
        _check(lib().moe_free_ssm_pages(self.handle, a.size, a.ctypes.data if a.size else None))

    def alloc_small(self, kind: int, request: int, n: int):
        out = self._pages(n)
        _check(lib().moe_alloc_small_pages(self.handle, kind, request, n, out.ctypes.data))
        return [int(v) for v in out[:n]]

    def free_small(self, kind: int, pages):
        a = np.ascontiguousarray(np.asarray(pages, dtype=np.int64))
        _check(lib().moe_free_small_pages(self.handle, kind, a.size, a.ctypes.data if a.size else None))

    def free_request(self, request: int) -> int:
        n = ctypes.c_int64()
        _check(lib().moe_free_request(self.handle, request, ctypes.byref(n)))
        return n.value

    def stats(self) -> dict:
        s = moe_alloc_stats()
        _check(lib().moe_alloc_get_stats(self.handle, ctypes.byref(s)))
        return {"free_huge": s.free_huge, "free_expert": s.free_expert, "used_expert": s.used_expert,
                "free_ssm": s.free_ssm, "used_ssm": s.used_ssm, "split": list(s.split),
                "used_small": list(s.used_small), "free_small": list(s.free_small),
                "expert_available": s.expert_available, "trapped_bytes": s.trapped_bytes,
                "huge_bytes": s.huge_bytes, "n_huge": s.n_huge}


# ----------------------------------------------------------------------------- remapped expert views

class ExpertViews:
    """Owner of one moe_vmm: physical pages, the pool / load-buffer views over
    them, and the remappable expert views w13 / w2."""

    def __init__(self, page_bytes: int, num_pages: int, loadbuf_slots: int, n_experts_total: int):
        h = ctypes.c_void_p()
        _check(lib().moe_vmm_create(page_bytes, num_pages, loadbuf_slots, n_experts_total, ctypes.byref(h)))
        self.handle = h
        self.page_bytes, self.num_pages, self.slots, self.E_tot = page_bytes, num_pages, loadbuf_slots, n_experts_total

    def close(self):
        if self.handle:
            _check(lib().moe_vmm_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def views(self):
        """{"pool", "loadbuf0", "loadbuf1", "w13", "w2"}: device addresses (None where unset)."""
        ps = [ctypes.c_void_p() for _ in range(5)]
        _check(lib().moe_vmm_views(self.handle, *[ctypes.byref(p) for p in ps]))
        return dict(zip(("pool", "loadbuf0", "loadbuf1", "w13", "w2"), [p.value for p in ps]))

    def granularity(self):
        """(minimum, recommended) mapping granularity in bytes."""
        a, b = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().moe_vmm_granularity(self.handle, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def map_experts(self, locs: np.ndarray, active_buf: int = 0, stream=None) -> int:
        a = locs_array(locs)
        n = ctypes.c_int32()
        _check(lib().moe_vmm_map_experts(self.handle, a.ctypes.data, a.shape[0], active_buf, _stream(stream),
                                         ctypes.byref(n)))
        return n.value

    def forward(self, p: MoePool, x, r: "RouteOut", ws, flags: int = 0, y=None, stream=None):
        import torch
        if y is None:
            y = torch.empty_like(x)
        _check(lib().moe_vmm_forward(self.handle, p.handle, _ptr(x), x.shape[0], r.block_m, _ptr(r.topk_ids),
                                     _ptr(r.topk_w), _ptr(r.sorted_ids), _ptr(r.block_expert), _ptr(r.num_padded),
                                     _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), flags, _stream(stream)))
        return y
