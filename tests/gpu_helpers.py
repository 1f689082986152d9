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
SUMMARY_FACTOR = 4.0        # units of eps32 * (2 + max|z|) * max|c| in summary_tol


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

    def __init__(self, w, max_t=None, build=True, n_tokens=None, level_p=None, n_refs=None, values=False):
        """n_refs: tangent scoring with that many reference queries per (level, kv head);
        values: compressed value summaries."""
        t = torch()
        self.w = w
        self.T = w.queries_per_step if max_t is None else max_t
        self.tangent = n_refs is not None
        self.geom = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels,
                                w.capacity, w.kv_dtype, level_p=level_p, n_refs=n_refs or 0,
                                scoring="tangent" if self.tangent else "summary", value_summaries=values)
        self.cache = Z.Cache(self.geom, self.T)
        self.K_np, self.V_np = W.kv_cache(w)
        self.cache.K.copy_(kv_tensor(w, self.K_np))
        self.cache.V.copy_(kv_tensor(w, self.V_np))
        self.R = W.ref_queries(w, n_refs)
        self.ref_q = t.from_numpy(self.R).cuda()
        n = w.n_tokens if n_tokens is None else n_tokens
        self.cache.seq_lens.copy_(t.full((w.batch,), n, dtype=t.int32))
        self.Kf = W.as_f32(w, self.K_np)
        self.Vf = W.as_f32(w, self.V_np)
        if build:
            Z.build_tree(self.geom, self.cache.K, self.ref_q, self.cache.seq_lens, self.cache.summaries,
                         self.cache.ws, V=self.cache.V)
            t.cuda.synchronize()

    @property
    def sizes(self):
        return self.cache.sizes

    def gpu_level(self, level):
        return self.cache.level(level).cpu().numpy()

    def gpu_offsets(self, level):
        return Z.offsets_view(self.cache.summaries, self.sizes, self.geom, level).cpu().numpy()

    def oracle_trees(self, n_tokens=None, slab=None):
        w = self.w
        lens = [w.n_tokens if n_tokens is None else n_tokens] * w.batch
        if self.tangent:
            return [[O.build_tangent_tree(self.Kf[s, h, :lens[s]], self.R[:, h], w.branching, slab=slab)
                     for h in range(w.n_kv_heads)] for s in range(w.batch)]
        return O.build_all(self.Kf, self.R, lens, w.branching, slab=slab)

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
    factor is SUMMARY_FACTOR: the largest error seen on the GPU over the
    parity, full-size and geometry workloads (d = 128, b up to 256, up to six
    levels) is 0.12 of this bound, so it leaves a margin of about 8 and still
    fails a summary that is wrong in its last few bits of a dozen-term sum.
    """
    c = np.abs(children).max() if children.size else 1.0
    z = scale * np.abs(children @ r).max() if children.size else 1.0
    return SUMMARY_FACTOR * EPS32 * (2.0 + z) * max(1.0, c)


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
    # bf16 caches: the logits are fp32 dot products of the bf16 keys with q (q
    # goes to the matrix cores as three bf16 parts that sum to it to about
    # 2^-25), so what is left is fp32 rounding in the logits, the softmax and
    # the accumulation; worst seen 1.7e-5. The bar is ten times that, tighter
    # than the 2e-3 the method's tolerance allows for bf16 KV.
    return 1e-5 if w.kv_dtype == "fp32" else 2e-4


def teacher_forced(st, qn, qpos_np, stats, lsel, p, trees, pairs=None):
    """Check every level's kept set of each (row, query head), teacher-forced: the
    oracle cuts the candidates of the GPU's own kept parents (p: one fraction, or
    a per-level schedule, level 1 first). Candidate counts
    must be exact, kept ids ascending, and the sets equal up to the margin
    exemptions. ``pairs`` (a list of (sequence, query head)) restricts the check
    to a sample. Returns the number of exempt differences."""
    w = st.w
    rows = qn.shape[0] * qn.shape[1]
    kept = {l: level_kept(st, lsel, stats, rows, l) for l in range(1, w.n_levels + 1)}
    todo = pairs if pairs is not None else [(s, h) for s in range(w.batch) for h in range(w.n_q_heads)]
    flips = 0
    for s, hq in todo:
        for t_ in range(qn.shape[1]):
            r = s * qn.shape[1] + t_
            N = int(qpos_np[s, t_]) + 1
            kv = hq // w.group
            tree = trees[s][kv]
            parents = None
            for level in range(w.n_levels, 0, -1):
                v, cnt, cand = kept[level]
                gpu_ids = v[r, hq, :cnt[r, hq]]
                pl = O.level_fraction(p, level)
                cut = O.route_level(qn[s, t_, hq], tree[level - 1], level, parents, N, w.branching,
                                    w.n_levels, pl, w.scale)
                assert cand[r, hq] == len(cut.ids), (s, t_, hq, level, cand[r, hq], len(cut.ids))
                assert np.all(np.diff(gpu_ids) > 0), "kept ids must be ascending"
                flips += check_sets(gpu_ids, cut, pl, f"row {r} head {hq} level {level}")
                parents = gpu_ids
    return flips


def check_tree(st, trees, n_tokens, pairs=None):
    """GPU summaries of every level against the oracle's tree (summary_tol per level)."""
    w = st.w
    worst = 0.0
    todo = pairs if pairs is not None else [(s, h) for s in range(w.batch) for h in range(w.n_kv_heads)]
    for level in range(1, w.n_levels + 1):
        gpu = st.gpu_level(level)
        for s, h in todo:
            ref = trees[s][h][level - 1]
            n = ref.shape[0]
            assert n == n_tokens // w.branching ** level
            if n == 0:
                continue
            children = st.Kf[s, h, :n_tokens] if level == 1 else trees[s][h][level - 2]
            tol = summary_tol(children.astype(np.float64), st.R[level - 1, h].astype(np.float64), w.scale)
            err = np.abs(gpu[s, h, :n].astype(np.float64) - ref).max()
            assert err <= tol, (level, s, h, err, tol)
            worst = max(worst, err / tol)
    return worst


def check_attention(st, qn, qpos_np, out, lse, sel, nsel, pairs=None):
    """GPU attention of each (row, head) against the oracle over the GPU's own index set."""
    w = st.w
    o_np, l_np = out.cpu().numpy(), lse.cpu().numpy()
    s_np, n_np = sel.cpu().numpy(), nsel.cpu().numpy()
    tol = attn_tol(w)
    worst = 0.0
    todo = pairs if pairs is not None else [(s, h) for s in range(w.batch) for h in range(w.n_q_heads)]
    for s, hq in todo:
        for t_ in range(qn.shape[1]):
            N = int(qpos_np[s, t_]) + 1
            kv = hq // w.group
            I = O.index_set(s_np[s, t_, hq, :n_np[s, t_, hq]], N, w.branching)
            o, l = O.attend(qn[s, t_, hq], st.Kf[s, kv], st.Vf[s, kv], I, w.scale)
            e = max(np.abs(o_np[s, t_, hq] - o).max(), abs(l_np[s, t_, hq] - l))
            worst = max(worst, e)
            assert e <= tol, (s, t_, hq, e)
    return worst

