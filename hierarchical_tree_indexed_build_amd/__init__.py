"""Python binding of libzha, the MI355X (gfx950) ZHA decode hot path.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libzha.so``; PyTorch supplies device memory and the current stream. The
names mirror the C ABI in ``include/zha.h``. Importing this package does not
need a GPU; calling anything that enqueues work does. If the library has not
been built, :func:`lib` raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libzha.so")

ZHA_OK, ZHA_ERR_NULL, ZHA_ERR_SHAPE, ZHA_ERR_UNSUPPORTED, ZHA_ERR_WORKSPACE, ZHA_ERR_CAPACITY, ZHA_ERR_HIP = range(7)
ZHA_DEV_SEL_OVERFLOW = 1
ZHA_DEV_APPEND_OVERFLOW = 2
ZHA_KV_BF16, ZHA_KV_F32 = 0, 1
ZHA_SCORE_SUMMARY, ZHA_SCORE_TANGENT = 0, 1
ZHA_MAX_LEVELS = 8

EXPORTED = ("zha_query_sizes", "zha_build_tree", "zha_append", "zha_route", "zha_sparse_attend", "zha_attend",
            "zha_attend_noalloc", "zha_dense_attend", "zha_read_device_status", "zha_profile_start", "zha_profile_collect",
            "zha_status_string", "zha_last_error")


class Geom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("branching", ctypes.c_int32), ("n_levels", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("kv_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("level_p", ctypes.c_float * ZHA_MAX_LEVELS), ("n_refs", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("value_summaries", ctypes.c_int32)]


class Sizes(ctypes.Structure):
    _fields_ = [("summaries_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
                ("level_nodes", ctypes.c_int64 * ZHA_MAX_LEVELS), ("level_offset", ctypes.c_int64 * ZHA_MAX_LEVELS),
                ("level_bias_offset", ctypes.c_int64 * ZHA_MAX_LEVELS),
                ("level_value_offset", ctypes.c_int64 * ZHA_MAX_LEVELS),
                ("level_sel_offset", ctypes.c_int64 * ZHA_MAX_LEVELS), ("level_sel_bytes", ctypes.c_size_t),
                ("max_rows", ctypes.c_int32), ("tile_rows", ctypes.c_int32), ("workspace_bytes_tiled", ctypes.c_size_t)]


class ZhaError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded libzha.so; raises if it is missing (build it with build_lib.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run hierarchical_tree_indexed_build_amd.build_lib")
        L = ctypes.CDLL(LIB_PATH)
        GP = ctypes.POINTER(Geom)
        i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        sig = {
            "zha_query_sizes": [GP, i32, ctypes.POINTER(Sizes)],
            "zha_build_tree": [GP, _P, _P, _P, _P, _P, _P, sz, _P],
            "zha_append": [GP, _P, _P, _P, _P, i32, _P, _P, _P, _P, sz, _P],
            "zha_route": [GP, _P, i32, _P, _P, _P, f32, i32, _P, _P, _P, _P, _P, sz, _P],
            "zha_sparse_attend": [GP, _P, i32, _P, _P, _P, _P, _P, _P, i32, _P, _P, _P, sz, _P],
            "zha_attend": [GP, _P, i32, _P, _P, _P, _P, _P, f32, i32, _P, _P, _P, _P, _P, _P, _P, sz, _P],
            "zha_attend_noalloc": [GP, _P, i32, _P, _P, _P, _P, _P, f32, i32, _P, _P, _P, _P, _P, _P, _P, _P],
            "zha_dense_attend": [GP, _P, i32, _P, _P, _P, _P, _P, _P, _P, sz, _P],
            "zha_read_device_status": [_P, _P, ctypes.POINTER(ctypes.c_uint32), i32],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        L.zha_profile_start.argtypes = [ctypes.c_char_p]
        L.zha_profile_start.restype = ctypes.c_int32
        L.zha_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64)]
        L.zha_profile_collect.restype = ctypes.c_int32
        L.zha_status_string.argtypes = [ctypes.c_int32]
        L.zha_status_string.restype = ctypes.c_char_p
        L.zha_last_error.argtypes = []
        L.zha_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != ZHA_OK:
        L = lib()
        raise ZhaError(code, where, f"{L.zha_status_string(code).decode()}: {L.zha_last_error().decode()}")


def make_geom(batch, n_q_heads, n_kv_heads, head_dim, branching, n_levels, capacity, kv_dtype="bf16",
              scale=0.0, level_p=None, n_refs=0, scoring="summary", value_summaries=False) -> Geom:
    """A zha_geom. level_p (optional, n_levels floats, level 1 first): the cut
    fraction of each level, overriding a call's top_p where non-zero. scoring
    "summary" (one reference query, q . summary) or "tangent" (n_refs
    reference queries, the maximum of the node's tangents). value_summaries:
    pruned subtrees join zha_attend's softmax as pseudo-tokens."""
    kd = {"bf16": ZHA_KV_BF16, "fp32": ZHA_KV_F32}[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    lp = (ctypes.c_float * ZHA_MAX_LEVELS)(*([float(x) for x in level_p] if level_p is not None else []))
    sc = {"summary": ZHA_SCORE_SUMMARY, "tangent": ZHA_SCORE_TANGENT}[scoring] if isinstance(scoring, str) \
        else int(scoring)
    return Geom(batch, n_q_heads, n_kv_heads, head_dim, branching, n_levels, capacity, kd, scale, lp, n_refs, sc,
                1 if value_summaries else 0)


def query_sizes(geom: Geom, max_t: int) -> Sizes:
    out = Sizes()
    _check(lib().zha_query_sizes(ctypes.byref(geom), max_t, ctypes.byref(out)), "zha_query_sizes")
    return out


# ----------------------------------------------------------------------------
# tensor plumbing (torch owns memory and streams)
# ----------------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libzha must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def build_tree(geom, K, ref_q, seq_lens, summaries, ws, stream=None, V=None):
    """V is read only for value summaries."""
    _check(lib().zha_build_tree(ctypes.byref(geom), _ptr(K), _ptr(V), _ptr(ref_q), _ptr(seq_lens), _ptr(summaries),
                                _ptr(ws), _nbytes(ws), _stream(stream)), "zha_build_tree")


def append(geom, K, V, k_new, v_new, seq_lens, ref_q, summaries, ws, stream=None):
    t_new = k_new.shape[-2]
    _check(lib().zha_append(ctypes.byref(geom), _ptr(K), _ptr(V), _ptr(k_new), _ptr(v_new), t_new, _ptr(seq_lens),
                            _ptr(ref_q), _ptr(summaries), _ptr(ws), _nbytes(ws), _stream(stream)), "zha_append")


def route(geom, q, q_pos, summaries, seq_lens, top_p, sel_blocks, n_sel, ws, level_stats=None, level_sel=None,
          stream=None):
    t = q.shape[1]
    _check(lib().zha_route(ctypes.byref(geom), _ptr(q), t, _ptr(q_pos), _ptr(summaries), _ptr(seq_lens),
                           float(top_p), sel_blocks.shape[-1], _ptr(sel_blocks), _ptr(n_sel), _ptr(level_stats),
                           _ptr(level_sel), _ptr(ws), _nbytes(ws), _stream(stream)), "zha_route")


def sparse_attend(geom, q, q_pos, K, V, seq_lens, sel_blocks, n_sel, out, lse, ws, stream=None):
    t = q.shape[1]
    _check(lib().zha_sparse_attend(ctypes.byref(geom), _ptr(q), t, _ptr(q_pos), _ptr(K), _ptr(V), _ptr(seq_lens),
                                   _ptr(sel_blocks), _ptr(n_sel), sel_blocks.shape[-1], _ptr(out), _ptr(lse),
                                   _ptr(ws), _nbytes(ws), _stream(stream)), "zha_sparse_attend")


def attend(geom, q, q_pos, K, V, summaries, seq_lens, top_p, sel_blocks, n_sel, out, lse, ws, level_stats=None,
           level_sel=None, stream=None):
    t = q.shape[1]
    _check(lib().zha_attend(ctypes.byref(geom), _ptr(q), t, _ptr(q_pos), _ptr(K), _ptr(V), _ptr(summaries),
                            _ptr(seq_lens), float(top_p), sel_blocks.shape[-1], _ptr(sel_blocks), _ptr(n_sel),
                            _ptr(level_stats), _ptr(level_sel), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws),
                            _stream(stream)), "zha_attend")


def attend_noalloc(geom, q, q_pos, K, V, summaries, seq_lens, top_p, sel_blocks, n_sel, out, lse, level_stats=None,
                   level_sel=None, dev_status=None, stream=None):
    """zha_attend with the library's static scratch instead of a workspace (no allocation)."""
    t = q.shape[1]
    _check(lib().zha_attend_noalloc(ctypes.byref(geom), _ptr(q), t, _ptr(q_pos), _ptr(K), _ptr(V), _ptr(summaries),
                                    _ptr(seq_lens), float(top_p), sel_blocks.shape[-1], _ptr(sel_blocks), _ptr(n_sel),
                                    _ptr(level_stats), _ptr(level_sel), _ptr(out), _ptr(lse), _ptr(dev_status),
                                    _stream(stream)), "zha_attend_noalloc")


def dense_attend(geom, q, q_pos, K, V, seq_lens, out, lse, ws, stream=None):
    t = q.shape[1]
    _check(lib().zha_dense_attend(ctypes.byref(geom), _ptr(q), t, _ptr(q_pos), _ptr(K), _ptr(V), _ptr(seq_lens),
                                  _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)), "zha_dense_attend")


def read_device_status(ws, clear: bool = False, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().zha_read_device_status(_ptr(ws), _stream(stream), ctypes.byref(v), 1 if clear else 0),
           "zha_read_device_status")
    return int(v.value)


def profile_start(label: Optional[str]):
    """Time every launch of kernel `label` ("name" or "name@level") with HIP events; None stops."""
    _check(lib().zha_profile_start(label.encode() if label else None), "zha_profile_start")


def profile_collect():
    """(summed kernel ms, launches timed, launches dropped) since the last collect."""
    ms, n, d = ctypes.c_double(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().zha_profile_collect(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(d)), "zha_profile_collect")
    return ms.value, int(n.value), int(d.value)


def level_sel_view(level_sel, sizes: Sizes, geom: Geom, rows: int, level: int):
    """View of one level inside a level_sel buffer: [rows, H_q, level_nodes]."""
    n = sizes.level_nodes[level - 1]
    off = rows * geom.n_q_heads * sizes.level_sel_offset[level - 1]
    return level_sel[off:off + rows * geom.n_q_heads * n].view(rows, geom.n_q_heads, n)


def summaries_view(summaries, sizes: Sizes, geom: Geom, level: int):
    """View of one level of the summary buffer: [B, H_kv, level_nodes, d], or
    [B, H_kv, level_nodes, R, d] (the tangents' keys) with tangent scoring."""
    n = sizes.level_nodes[level - 1]
    off = sizes.level_offset[level - 1]
    R = max(1, geom.n_refs)
    cnt = geom.batch * geom.n_kv_heads * n * R * geom.head_dim
    v = summaries[off:off + cnt]
    if geom.scoring == ZHA_SCORE_TANGENT:
        return v.view(geom.batch, geom.n_kv_heads, n, R, geom.head_dim)
    return v.view(geom.batch, geom.n_kv_heads, n, geom.head_dim)


def values_view(summaries, sizes: Sizes, geom: Geom, level: int):
    """The value summaries of one level (value summaries on): [B, H_kv, level_nodes, d]."""
    n = sizes.level_nodes[level - 1]
    off = sizes.level_value_offset[level - 1]
    cnt = geom.batch * geom.n_kv_heads * n * geom.head_dim
    return summaries[off:off + cnt].view(geom.batch, geom.n_kv_heads, n, geom.head_dim)


def offsets_view(summaries, sizes: Sizes, geom: Geom, level: int):
    """The tangents' offsets of one level (tangent scoring): [B, H_kv, level_nodes, R]."""
    n = sizes.level_nodes[level - 1]
    off = sizes.level_bias_offset[level - 1]
    R = max(1, geom.n_refs)
    return summaries[off:off + geom.batch * geom.n_kv_heads * n * R].view(geom.batch, geom.n_kv_heads, n, R)


class Cache:
    """Device buffers for one geometry: K, V, summaries, seq_lens, workspace (torch-allocated)."""

    def __init__(self, geom: Geom, max_t: int = 1, device: str = "cuda", tiled: bool = False):
        """tiled: a workspace for row tiles (zha_sizes.workspace_bytes_tiled) instead of every row at once."""
        import torch
        self.geom = geom
        self.sizes = query_sizes(geom, max_t)
        kdt = torch.bfloat16 if geom.kv_dtype == ZHA_KV_BF16 else torch.float32
        shape = (geom.batch, geom.n_kv_heads, geom.capacity, geom.head_dim)
        self.K = torch.zeros(shape, dtype=kdt, device=device)
        self.V = torch.zeros(shape, dtype=kdt, device=device)
        self.summaries = torch.zeros(max(1, self.sizes.summaries_bytes // 4), dtype=torch.float32, device=device)
        self.seq_lens = torch.zeros(geom.batch, dtype=torch.int32, device=device)
        wsb = self.sizes.workspace_bytes_tiled if tiled else self.sizes.workspace_bytes
        self.ws = torch.zeros(max(256, wsb) // 4 + 64, dtype=torch.int32, device=device)

    def level(self, level: int):
        return summaries_view(self.summaries, self.sizes, self.geom, level)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
