"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/zha.h declares, computes sizes, and rejects bad arguments before it
would enqueue anything (no compute call is made here)."""
import ctypes
import math
import os
import re

import pytest

import hierarchical_tree_indexed_build_amd as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"ZHA_API\s+[\w\s\*]+?\b(zha_\w+)\s*\(", txt)))


def test_header_declares_the_abi():
    names = _declared()
    assert set(names) == set(Z.EXPORTED), names


def test_library_exports_every_declared_symbol():
    L = Z.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings():
    L = Z.lib()
    for code in range(7):
        assert L.zha_status_string(code)
    assert L.zha_status_string(99) == b"unknown status"


def _geom(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, branching=32, n_levels=4,
                capacity=(1 << 20) + 256, kv_dtype="bf16")
    base.update(kw)
    return Z.make_geom(**base)


def test_sizes_match_layout_arithmetic():
    g = _geom()
    s = Z.query_sizes(g, 1)
    cap = (1 << 20) + 256
    nodes = [cap // 32 ** l for l in range(1, 5)]
    assert list(s.level_nodes)[:4] == nodes and list(s.level_nodes)[4:] == [0] * 4
    off = 0
    for l in range(4):
        assert s.level_offset[l] == off
        off += 8 * nodes[l] * 128
    assert s.summaries_bytes == off * 4
    assert s.level_sel_offset[1] == nodes[0]
    assert s.max_rows == 1
    # the workspace grows with the number of query rows
    assert Z.query_sizes(g, 64).workspace_bytes > s.workspace_bytes


def test_tangent_scoring_layout_and_validation():
    g = _geom(n_refs=4, scoring="tangent")
    s = Z.query_sizes(g, 1)
    cap = (1 << 20) + 256
    nodes = [cap // 32 ** l for l in range(1, 5)]
    off = 0
    for l in range(4):                       # keys: R rows of d per node
        assert s.level_offset[l] == off
        off += 8 * nodes[l] * 4 * 128
    for l in range(4):                       # then the offsets: R per node
        assert s.level_bias_offset[l] == off
        off += 8 * nodes[l] * 4
    assert s.summaries_bytes == off * 4
    for kw in (dict(n_refs=2), dict(n_refs=17, scoring="tangent"), dict(n_refs=-1, scoring="tangent"),
               dict(scoring=7)):
        with pytest.raises(Z.ZhaError) as e:
            Z.query_sizes(_geom(**kw), 1)
        assert e.value.code == Z.ZHA_ERR_UNSUPPORTED, kw


def test_value_summaries_layout_and_validation():
    g = _geom(value_summaries=True)
    s = Z.query_sizes(g, 1)
    cap = (1 << 20) + 256
    nodes = [cap // 32 ** l for l in range(1, 5)]
    keys = sum(8 * n * 128 for n in nodes)
    off = keys
    for l in range(4):                       # value summaries follow the keys: d floats per node
        assert s.level_value_offset[l] == off
        off += 8 * nodes[l] * 128
    assert s.summaries_bytes == off * 4
    assert s.workspace_bytes > Z.query_sizes(_geom(), 1).workspace_bytes     # the pseudo-token partials
    with pytest.raises(Z.ZhaError) as e:
        Z.query_sizes(_geom(value_summaries=True, n_refs=4, scoring="tangent"), 1)
    assert e.value.code == Z.ZHA_ERR_UNSUPPORTED


def test_level_schedule_is_validated():
    assert Z.query_sizes(_geom(level_p=[0.9, 1.0, 0.5, 0.0]), 1).max_rows == 1
    for bad in ([1.5, 0, 0, 0], [-0.1, 0, 0, 0], [0.9, 0.9, 0.9, 0.9, 0.9], [float("nan"), 0, 0, 0]):
        with pytest.raises(Z.ZhaError) as e:
            Z.query_sizes(_geom(level_p=bad), 1)
        assert e.value.code == Z.ZHA_ERR_SHAPE and b"level_p" in Z.lib().zha_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv_heads=6), Z.ZHA_ERR_SHAPE),
    (dict(n_q_heads=24, n_kv_heads=8), Z.ZHA_ERR_UNSUPPORTED),      # group of 3
    (dict(head_dim=96), Z.ZHA_ERR_UNSUPPORTED),
    (dict(branching=24), Z.ZHA_ERR_UNSUPPORTED),
    (dict(branching=512), Z.ZHA_ERR_UNSUPPORTED),
    (dict(branching=96), Z.ZHA_ERR_UNSUPPORTED),
    (dict(n_levels=0), Z.ZHA_ERR_SHAPE),
    (dict(n_levels=9), Z.ZHA_ERR_SHAPE),
    (dict(capacity=0), Z.ZHA_ERR_SHAPE),
    (dict(capacity=1 << 31), Z.ZHA_ERR_SHAPE),
    (dict(kv_dtype=7), Z.ZHA_ERR_UNSUPPORTED),
    (dict(batch=0), Z.ZHA_ERR_SHAPE),
])
def test_bad_geometry_is_rejected(kw, code):
    with pytest.raises(Z.ZhaError) as e:
        Z.query_sizes(_geom(**kw), 1)
    assert e.value.code == code


def test_null_and_workspace_errors_return_before_launch():
    L = Z.lib()
    g = _geom()
    gp = ctypes.byref(g)
    fake = ctypes.c_void_p(1 << 40)          # never dereferenced: validation fails first
    assert L.zha_build_tree(gp, None, None, None, None, None, None, 0, None) == Z.ZHA_ERR_NULL
    assert L.zha_build_tree(None, fake, fake, fake, fake, fake, fake, 1 << 20, None) == Z.ZHA_ERR_NULL
    gv = _geom(value_summaries=True)
    assert L.zha_build_tree(ctypes.byref(gv), fake, None, fake, fake, fake, fake, 1 << 20, None) == Z.ZHA_ERR_NULL
    need = Z.query_sizes(g, 1).workspace_bytes
    rc = L.zha_route(gp, fake, 1, None, fake, fake, ctypes.c_float(0.95), 16, fake, fake, None, None, fake,
                     need - 1, None)
    assert rc == Z.ZHA_ERR_WORKSPACE
    assert b"needed" in L.zha_last_error()
    rc = L.zha_route(gp, fake, 1, None, fake, fake, ctypes.c_float(1.5), 16, fake, fake, None, None, fake, need, None)
    assert rc == Z.ZHA_ERR_SHAPE
    rc = L.zha_route(gp, fake, 1, None, fake, fake, ctypes.c_float(0.9), 0, fake, fake, None, None, fake, need, None)
    assert rc == Z.ZHA_ERR_SHAPE
    rc = L.zha_route(gp, fake, 0, None, fake, fake, ctypes.c_float(0.9), 4, fake, fake, None, None, fake, need, None)
    assert rc == Z.ZHA_ERR_SHAPE
    misaligned = ctypes.c_void_p((1 << 40) + 8)
    rc = L.zha_dense_attend(gp, fake, 1, None, fake, fake, fake, fake, fake, misaligned, need, None)
    assert rc == Z.ZHA_ERR_SHAPE
    rc = L.zha_append(gp, fake, fake, fake, fake, 0, fake, fake, fake, fake, 1 << 20, None)
    assert rc == Z.ZHA_ERR_SHAPE
    rc = L.zha_sparse_attend(gp, fake, 1, None, fake, fake, fake, None, fake, 4, fake, fake, fake, need, None)
    assert rc == Z.ZHA_ERR_NULL
    rc = L.zha_read_device_status(None, None, None, 0)
    assert rc == Z.ZHA_ERR_NULL


def test_binding_refuses_to_run_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(Z, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(Z, "_lib", None)
    with pytest.raises(ImportError):
        Z.lib()
