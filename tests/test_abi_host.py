"""Host-only checks of the C ABI: the library loads, exports every function
include/lychee.h declares, sizes workspaces, and rejects bad arguments before
touching a device.  Pointers here are fake integers: the validator compares
address ranges and never dereferences them."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import hybrid_head_sparse_amd as hhs
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lychee.h")
TRACE_HEADER = os.path.join(ROOT, "include", "lychee_trace.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hhs.LIB_PATH):
        from hybrid_head_sparse_amd import build
        build.build(verbose=False)
    return hhs.load()


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lychee_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(hhs.EXPORTED)


def test_trace_header_is_exported_by_the_trace_build_only(lib):
    """include/lychee_trace.h declares what the trace build adds; the
    product library does not carry it."""
    from hybrid_head_sparse_amd import build
    if not os.path.exists(build.TRACE_LIB):
        build.build(verbose=False, trace=True)
    tlib = ctypes.CDLL(build.TRACE_LIB)
    extra = _declared_functions(TRACE_HEADER)
    assert extra == ["lychee_set_trace"]
    for name in extra:
        assert hasattr(tlib, name), name
        assert not hasattr(lib, name), name
    for name in _declared_functions():
        assert hasattr(tlib, name), name


def _dims(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, max_ctx=131072, k_max=4096, dtype="bf16")
    base.update(kw)
    return hhs.make_dims(**base)


def test_workspace_bytes_for_every_workload(lib):
    for w in synth.WORKLOADS.values():
        d = hhs.make_dims(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_ctx, w.k, w.dtype)
        n = hhs.workspace_bytes(d)
        # at least the selection-candidate buffer of every head (key + index per token)
        assert n >= w.batch * w.n_kv_heads * w.max_ctx * 8
        assert n % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), hhs.LYCHEE_ERR_UNSUPPORTED),
    (dict(n_q_heads=24), hhs.LYCHEE_ERR_UNSUPPORTED),        # G = 3
    (dict(n_q_heads=30), hhs.LYCHEE_ERR_INVALID_ARG),        # not a multiple
    (dict(n_kv_heads=128, n_q_heads=128), hhs.LYCHEE_ERR_UNSUPPORTED),
    (dict(max_ctx=1 << 19), hhs.LYCHEE_ERR_UNSUPPORTED),
    (dict(batch=0), hhs.LYCHEE_ERR_INVALID_ARG),
    (dict(k_max=200000), hhs.LYCHEE_ERR_INVALID_ARG),
    (dict(batch=200), hhs.LYCHEE_ERR_UNSUPPORTED),           # B * Hkv > 1024
])
def test_bad_dims_are_rejected(lib, kw, status):
    d = _dims(**kw)
    assert lib.lychee_workspace_bytes(ctypes.byref(d)) == 0
    st = hhs.validate_layer(d, 1 << 40, 2 << 40, 3 << 40, [1] * d.n_kv_heads, None, 5 << 40, 6 << 40, 7 << 40, 1)
    assert st == status
    assert lib.lychee_last_error()


def _good_ptrs():
    return dict(q=1 << 40, k_cache=2 << 40, v_cache=3 << 40, S_in=4 << 40, S_out=5 << 40, out=6 << 40,
                n_ctx=7 << 40)


def _validate(d, role=None, k=64, **over):
    p = _good_ptrs()
    p.update(over)
    role = [0, 1] + [0] * (d.n_kv_heads - 2) if role is None else role
    return hhs.validate_layer(d, p["q"], p["k_cache"], p["v_cache"], role, p["S_in"], p["S_out"], p["out"],
                              p["n_ctx"], k)


def test_valid_arguments_pass(lib):
    d = _dims()
    assert _validate(d) == hhs.LYCHEE_OK
    assert _validate(d, S_out=4 << 40) == hhs.LYCHEE_OK                   # in place
    assert _validate(d, role=[1] * 8, S_in=None) == hhs.LYCHEE_OK          # layer 0


@pytest.mark.parametrize("over,k,reason", [
    (dict(q=None), 64, "null q"),
    (dict(S_out=None), 64, "null S_out"),
    (dict(S_in=None), 64, "sparse head without S_in"),
    (dict(S_out=(4 << 40) + 64), 64, "S_out partially overlaps S_in"),
    (dict(out=(1 << 40) + 256), 64, "out overlaps q"),
    (dict(S_out=(6 << 40) + 4), 64, "S_out overlaps out"),
    (dict(k_cache=(2 << 40) + 8), 64, "misaligned cache"),
    ({}, 0, "k = 0"),
    ({}, 4097, "k > k_max"),
])
def test_bad_layer_arguments_are_rejected(lib, over, k, reason):
    d = _dims()
    assert _validate(d, k=k, **over) == hhs.LYCHEE_ERR_INVALID_ARG, reason
    assert lib.lychee_last_error().decode()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.lychee_status_str(code).decode()
    assert lib.lychee_status_str(-99).decode() == "unknown status"


def test_null_handle_is_rejected(lib):
    assert lib.lychee_decode_layer(None, None, None, None, None, None, None, None, None, 1) == hhs.LYCHEE_ERR_INVALID_ARG
    assert lib.lychee_check_device_errors(None) == hhs.LYCHEE_ERR_INVALID_ARG
    lib.lychee_destroy(None)


@pytest.mark.parametrize("rule, param, needle", [
    (3, 0.0, "rule"),
    (-1, 0.0, "rule"),
    (hhs.SELECT_RULES["ratio"], 0.0, "theta"),
    (hhs.SELECT_RULES["ratio"], 1.5, "theta"),
    (hhs.SELECT_RULES["ratio"], float("nan"), "theta"),
    (hhs.SELECT_RULES["threshold"], float("nan"), "tau"),
    (hhs.SELECT_RULES["topp"], 0.0, "p must"),
    (hhs.SELECT_RULES["topp"], 1.0000001, "p must"),
    (5, 0.5, "rule"),
    (hhs.SELECT_RULES["block"], 48.0, "block size"),
    (hhs.SELECT_RULES["block"], 512.0, "block size"),
    (hhs.SELECT_RULES["block"], 64.5, "block size"),
])
def test_bad_selection_rules_are_rejected(lib, rule, param, needle):
    # the rule is checked before the handle, so a NULL handle still reports it
    st = lib.lychee_decode_layer_select(None, None, None, None, None, None, None, None, None, 1, rule, param)
    assert st == hhs.LYCHEE_ERR_INVALID_ARG
    assert needle in lib.lychee_last_error().decode()


@pytest.mark.parametrize("rule, param", [(0, 0.0), (1, 1.0), (1, 1e-9), (2, float("inf")), (2, -float("inf")),
                                         (2, -3.5), (3, 1.0), (3, 1e-12), (4, 64.0), (4, 16.0)])
def test_valid_selection_rules_reach_the_handle_check(lib, rule, param):
    st = lib.lychee_decode_layer_select(None, None, None, None, None, None, None, None, None, 4096, rule, param)
    assert st == hhs.LYCHEE_ERR_INVALID_ARG
    assert "handle" in lib.lychee_last_error().decode()


def test_block_rule_needs_k_of_at_least_one_block(lib):
    st = lib.lychee_decode_layer_select(None, None, None, None, None, None, None, None, None, 32, 4, 64.0)
    assert st == hhs.LYCHEE_ERR_INVALID_ARG and "block" in lib.lychee_last_error().decode()


def test_static_entry_rejects_dims_beyond_its_scratch(lib):
    """The allocation-free entry point checks its arguments and its scratch
    limit on the host, before anything touches a device."""
    p = _good_ptrs()
    big = _dims(batch=16, max_ctx=131072)                      # 128 heads x 128K rows: > 64 MiB
    role = (ctypes.c_uint8 * 8)(*([1] * 8))
    st = lib.lychee_decode_layer_static(ctypes.byref(big), None, p["q"], p["k_cache"], p["v_cache"], role, None,
                                        p["S_out"], p["out"], p["n_ctx"], 64)
    assert st == hhs.LYCHEE_ERR_WORKSPACE
    assert "64" in lib.lychee_last_error().decode() or "scratch" in lib.lychee_last_error().decode()
    bad = _dims()
    st = lib.lychee_decode_layer_static(ctypes.byref(bad), None, None, p["k_cache"], p["v_cache"], role, None,
                                        p["S_out"], p["out"], p["n_ctx"], 64)
    assert st == hhs.LYCHEE_ERR_INVALID_ARG
