"""Helpers for the GPU parity tests: stage a workload on the device through the
binding, and compare the HIP path with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import hierarchical_tree_indexed_build_amd as Z
import workloads as W
from oracle import zha_oracle as O

EPS32 = float(np.finfo(np.float32).eps)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def kv_tensor(w, arr):
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(arr))
    if w.kv_dtype == "bf16":
        x = x.view(t.bfloat16)
    return x.cuda()


class Staged:
    """A workload's cache, tree and buffers on cuda:0, plus host copies for the oracle."""

    def __init__(self, w, max_t=None, build=True, n_tokens=None):
        t = torch()
        self.w = w
        self.T = w.queries_per_step if max_t is None else max_t
        self.geom = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels,
                                w.capacity, w.kv_dtype)
        self.cache = Z.Cache(self.geom, self.T)
        self.K_np, self.V_np = W.kv_cache(w)
        self.cache.K.copy_(kv_tensor(w, self.K_np))
        self.cache.V.copy_(kv_tensor(w, self.V_np))
        self.R = W.ref_queries(w)
        self.ref_q = t.from_numpy(self.R).cuda()
        n = w.n_tokens if n_tokens is None else n_tokens
        self.cache.seq_lens.copy_(t.full((w.batch,), n, dtype=t.int32))
        self.Kf = W.as_f32(w, self.K_np)
        self.Vf = W.as_f32(w, self.V_np)
        if build:
            Z.build_tree(self.geom, self.cache.K, self.ref_q, self.cache.seq_lens, self.cache.summaries,
                         self.cache.ws)
            t.cuda.synchronize()

    @property
    def sizes(self):
        return self.cache.sizes

    def gpu_level(self, level):
        return self.cache.level(level).cpu().numpy()

    def oracle_trees(self, n_tokens=None):
        w = self.w
        lens = [w.n_tokens if n_tokens is None else n_tokens] * w.batch
        return O.build_all(self.Kf, self.R, lens, w.branching)

    def route_buffers(self, rows, sel_cap=None):
        t = torch()
        g = self.geom
        cap = self.sizes.level_nodes[0] if sel_cap is None else sel_cap
        T = rows // g.batch
        sel = t.full((g.batch, T, g.n_q_heads, max(1, cap)), -1, dtype=t.int32, device="cuda")
        nsel = t.zeros((g.batch, T, g.n_q_heads), dtype=t.int32, device="cuda")
        stats = t.zeros((g.batch, T, g.n_q_heads, g.n_levels, 2), dtype=t.int32, device="cuda")
        sizes = Z.query_sizes(g, T)
        lsel = t.full((max(1, sizes.level_sel_bytes // 4),), -1, dtype=t.int32, device="cuda")
        return sel, nsel, stats, lsel

    def queries(self, step=0, rows=None):
        t = torch()
        q = W.queries(self.w, step, rows=rows)
        return q, t.from_numpy(q).cuda()


def level_kept(st, lsel, stats, rows, level):
    """GPU kept ids per (row, head) at `level` from level_sel / level_stats (host arrays)."""
    v = Z.level_sel_view(lsel, st.sizes, st.geom, rows, level).cpu().numpy()
    cnt = stats[..., level - 1, 1].reshape(rows, -1).cpu().numpy()
    cand = stats[..., level - 1, 0].reshape(rows, -1).cpu().numpy()
    return v, cnt, cand


def summary_tol(children, r, scale):
    """Bound on |GPU - oracle| for one level: fp32 accumulation over d + b terms.

    The pooling logits z = scale * r . c carry a rounding error of about
    d * eps * scale * |r| |c|; a softmax weight then moves by that much
    relatively, and the weighted mean of children bounded by max|c| moves by
    (2 + max|z|) of those errors plus the b-term accumulation of the sum. The
    factor 64 covers d <= 128 and b <= 64 with room.
    """
    c = np.abs(children).max() if children.size else 1.0
    z = scale * np.abs(children @ r).max() if children.size else 1.0
    return 64 * EPS32 * (2.0 + z) * max(1.0, c)


def check_sets(gpu_ids, cut, p, where=""):
    """North-star set parity: symmetric difference within the 1e-5 margin exemptions."""
    g = set(int(x) for x in gpu_ids)
    o = set(int(x) for x in cut.selected)
    diff = g ^ o
    if not diff:
        return 0
    ex = set(int(x) for x in O.cut_exemptions(cut, p))
    bad = diff - ex
    assert not bad, f"{where}: {len(bad)} ids differ outside the margin exemptions: {sorted(bad)[:10]}"
    return len(diff)


def attn_tol(w):
    return 1e-5 if w.kv_dtype == "fp32" else 2e-3
