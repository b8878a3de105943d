"""C-ABI library checks that need no GPU: it loads, exports every entry point
include/moe.h declares, and rejects bad arguments on the host before touching
the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_expert_weight_amd as pm
from workloads import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pm.LIB_PATH):
        from paged_expert_weight_amd import build
        build.build()
    return pm.lib()


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text))
    return names


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert {"moe_pool_create", "moe_route", "moe_paged_forward"} <= declared
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert declared == set(pm.EXPORTS)
    assert lib.moe_version() == 103


def _desc(**kw):
    base = dict(pool=0x10000, num_pages=32, d=128, f=64, num_experts=8, top_k=2, num_shared=0,
                loadbuf_slots=2, loadbuf=(0x20000, 0x30000))
    base.update(kw)
    return pm.make_desc(**base)


def _rc(fn, *a):
    return fn(*a)


def test_validate_locs_accepts_generated_table(lib):
    s = synth.SPECS["tiny"]
    pl = synth.make_placement(s)
    pm.moe_validate_locs(_desc(), pl.locs)


@pytest.mark.parametrize("mutate,code", [
    (lambda L: L.__setitem__(0, (0, [32, 1, 2])), pm.MOE_ERR_PAGE_RANGE),
    (lambda L: L.__setitem__(0, (0, [-1, 1, 2])), pm.MOE_ERR_PAGE_RANGE),
    (lambda L: L.__setitem__(1, (0, [L[0]["idx"][2], 30, 31])), pm.MOE_ERR_PAGE_ALIAS),
    (lambda L: L.__setitem__(0, (0, [5, 5, 6])), pm.MOE_ERR_PAGE_ALIAS),
    (lambda L: L.__setitem__(6, (1, [2, 0, 0])), pm.MOE_ERR_SLOT_RANGE),
    (lambda L: L.__setitem__(6, (1, [int(L[7]["idx"][0]), 0, 0])), pm.MOE_ERR_SLOT_RANGE),
    (lambda L: L.__setitem__(3, (7, [0, 0, 0])), pm.MOE_ERR_INVALID_ARG),
])
def test_validate_locs_rejects(lib, mutate, code):
    s = synth.SPECS["tiny"]
    locs = synth.make_placement(s).locs.copy()
    # free pages 0..31 not used by the generated table are fine targets; make
    # sure the mutation's own pages do not collide by accident
    mutate(locs)
    with pytest.raises(pm.MoeError) as ei:
        pm.moe_validate_locs(_desc(), locs)
    assert ei.value.code == code


def test_validate_locs_wrong_count_and_no_loadbuf(lib):
    s = synth.SPECS["tiny"]
    locs = synth.make_placement(s).locs
    with pytest.raises(pm.MoeError) as ei:
        pm.moe_validate_locs(_desc(), locs[:-1])
    assert ei.value.code == pm.MOE_ERR_INVALID_ARG
    with pytest.raises(pm.MoeError) as ei:
        pm.moe_validate_locs(_desc(loadbuf_slots=0, loadbuf=(None, None)), locs)
    assert ei.value.code == pm.MOE_ERR_SLOT_RANGE


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), pm.MOE_ERR_UNSUPPORTED),
    (dict(f=96), pm.MOE_ERR_UNSUPPORTED),
    (dict(top_k=9), pm.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), pm.MOE_ERR_INVALID_ARG),
    (dict(num_shared=2), pm.MOE_ERR_INVALID_ARG),
    (dict(num_experts=1024, num_shared=1), pm.MOE_ERR_UNSUPPORTED),
    (dict(pool=0x10008), pm.MOE_ERR_ALIGN),
    (dict(pool=0), pm.MOE_ERR_INVALID_ARG),
    (dict(num_pages=0), pm.MOE_ERR_INVALID_ARG),
    (dict(loadbuf=(0x20000, None)), pm.MOE_ERR_INVALID_ARG),
    (dict(loadbuf=(0x20004, 0x30000)), pm.MOE_ERR_ALIGN),
    (dict(d=16384, f=65536), pm.MOE_ERR_UNSUPPORTED),
])
def test_pool_create_rejects_bad_desc_before_any_device_call(lib, kw, code):
    desc = _desc(**kw)
    h = ctypes.c_void_p()
    rc = lib.moe_pool_create(ctypes.byref(desc), ctypes.byref(h))
    assert rc == code, lib.moe_last_error()
    assert not h.value
    assert lib.moe_last_error()


def test_null_handles_rejected(lib):
    s, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.moe_route_capacity(None, 4, 16, ctypes.byref(s), ctypes.byref(b)) == pm.MOE_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(None, 4, 16, 0, ctypes.byref(n)) == pm.MOE_ERR_INVALID_ARG
    assert lib.moe_paged_forward(None, None, 1, 16, None, None, None, None, None, 0, None, None, 0, 0,
                                 None) == pm.MOE_ERR_INVALID_ARG
    assert lib.moe_route_forward(None, None, None, 1, 16, None, None, None, None, None, 0, None, None, 0, 0,
                                 None) == pm.MOE_ERR_INVALID_ARG
    assert lib.moe_route_contiguous_forward(None, None, None, None, None, 1, 16, None, None, None, None, None,
                                            None, None, 0, 0, None) == pm.MOE_ERR_INVALID_ARG
    assert lib.moe_pool_destroy(None) == pm.MOE_OK


def test_pipeline_host_checks(lib):
    """Argument errors of the pipeline entry points are caught before any device call."""
    E = pm.MOE_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.moe_pipeline_create(0, None, None, ctypes.byref(h)) == E
    assert lib.moe_pipeline_create(1, None, None, None) == E
    two_null = (ctypes.c_void_p * 2)(None, None)
    assert lib.moe_pipeline_create(2, two_null, None, ctypes.byref(h)) == E
    assert not h.value
    assert lib.moe_pipeline_destroy(None) == pm.MOE_OK
    n = ctypes.c_int32()
    assert lib.moe_pipeline_reclaim(None, None, 0, ctypes.byref(n)) == E
    assert lib.moe_pipeline_stage_table(None, 0, None, 0, 0, None, None) == E
    assert lib.moe_pipeline_prefetch(None, 0, 0, None, None) == E
    assert lib.moe_pipeline_forward(None, 0, None, 1, 16, None, None, None, None, None, None, None, 0, 0,
                                    None) == E


def test_library_has_no_oracle_dependency():
    """The product library links no oracle code and the package does not import it."""
    import sys
    import subprocess
    code = ("import sys, paged_expert_weight_amd as pm; pm.lib(); "
            "assert 'oracle' not in sys.modules, 'product imported the oracle'")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
    out = subprocess.run(["nm", "-D", pm.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle_" not in out


def _prototypes():
    """name -> (return kind, [parameter kinds]) of every prototype in include/."""
    out = {}
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for ret, name, params in re.findall(r"^(int32_t|int|const char \*|void)\s*\b(moe_[a-z_0-9]+)\s*\(([^)]*)\)\s*;",
                                            text, flags=re.M):
            kinds = []
            for p in params.split(","):
                p = " ".join(p.split())
                if p in ("", "void"):
                    continue
                kinds.append(_kind(p.rsplit(" ", 1)[0] if "*" not in p else "*"))
            out[name] = (_kind(ret.strip()), kinds)
    return out


def _kind(t: str) -> str:
    if "*" in t:
        return "ptr"
    return {"int": "i32", "int32_t": "i32", "int64_t": "i64", "size_t": "sz", "uint32_t": "u32"}[t]


def _ctype_kind(c) -> str:
    if c in (ctypes.c_void_p, ctypes.c_char_p) or issubclass(c, ctypes._Pointer):
        return "ptr"
    for k, ct in (("i32", ctypes.c_int32), ("i64", ctypes.c_int64), ("sz", ctypes.c_size_t),
                  ("u32", ctypes.c_uint32)):
        if c is ct:
            return k
    raise AssertionError(f"unexpected ctypes type {c}")


def test_binding_signatures_match_the_header(lib):
    """Every binding's ctypes argument and result types against its prototype
    in include/: the same count, and pointer / int32 / int64 / size_t /
    uint32 in each position (a wrong width would truncate a size or a
    pointer without an error)."""
    protos = _prototypes()
    assert set(protos) == set(pm.EXPORTS)
    for name, (ret, kinds) in sorted(protos.items()):
        f = getattr(lib, name)
        got = [_ctype_kind(a) for a in (f.argtypes or [])]
        assert got == kinds, f"{name}: binding {got}, header {kinds}"
        r = f.restype
        assert (r is ctypes.c_char_p and ret == "ptr") or (r in (ctypes.c_int, ctypes.c_int32) and ret == "i32"), \
            f"{name}: result {r}, header {ret}"
