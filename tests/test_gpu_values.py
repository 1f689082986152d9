"""Compressed value summaries on the GPU ("Subquadratic Attention with a
Hierarchical Tree-Structured Indexer", Future Directions: pruned subtrees
contribute coarse attention outputs) against the CPU oracle.

* the tree: turning value summaries on leaves the key summaries' bits as they
  are; the value summaries match the oracle's within the summaries' fp32 bound;
* zha_attend: out and lse match the oracle's softmax over the exact tokens of
  the GPU's own index set and one pseudo-token per pruned candidate of every
  level, the candidates and kept sets taken from the GPU's route
  (teacher-forced), the logits from the oracle's scores; within 2e-4 (bf16
  KV) and 1e-5 (fp32 KV);
* on keys and values repeated over every top-level span, every pruned subtree
  is uniform and the output equals the dense kernel's;
* p = 1 prunes nothing: the output has the bits of the plain zha_attend;
* appends (fused single-token path and multi-token path) give the value
  summaries of a fresh build.
"""
import dataclasses

import numpy as np
import pytest

import hierarchical_tree_indexed_build_amd as Z
import workloads as W
from oracle import zha_oracle as O
from tests.gpu_helpers import Staged, attn_tol, kv_tensor, level_kept, say, summary_tol, torch

pytestmark = pytest.mark.gpu


def _check_values(st):
    """Value summaries against the oracle's, and the key summaries against a
    build without value summaries (bit for bit)."""
    t = torch()
    w = st.w
    plain = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels, w.capacity,
                        w.kv_dtype)
    ref = Z.Cache(plain, 1)
    ref.K.copy_(st.cache.K)
    ref.seq_lens.copy_(st.cache.seq_lens)
    Z.build_tree(plain, ref.K, st.ref_q, ref.seq_lens, ref.summaries, ref.ws)
    t.cuda.synchronize()
    worst = 0.0
    for level in range(1, w.n_levels + 1):
        m = w.n_tokens // w.branching ** level
        assert t.equal(st.cache.level(level)[:, :, :m], ref.level(level)[:, :, :m]), level
        gv = Z.values_view(st.cache.summaries, st.sizes, st.geom, level).cpu().numpy()
        for s in range(w.batch):
            for h in range(w.n_kv_heads):
                kt = O.build_tree(st.Kf[s, h, :w.n_tokens], st.R[:, h], w.branching)
                vt = O.build_value_tree(st.Kf[s, h, :w.n_tokens], st.Vf[s, h, :w.n_tokens], st.R[:, h], w.branching)
                if m == 0:
                    continue
                children_k = st.Kf[s, h, :w.n_tokens] if level == 1 else kt[level - 2]
                children_v = st.Vf[s, h, :w.n_tokens] if level == 1 else vt[level - 2]
                tol = summary_tol(children_k.astype(np.float64), st.R[level - 1, h].astype(np.float64), w.scale) \
                    * max(1.0, float(np.abs(children_v).max()))
                err = np.abs(gv[s, h, :m].astype(np.float64) - vt[level - 1]).max()
                assert err <= tol, (level, s, h, err, tol)
                worst = max(worst, err / tol)
    return worst


def _oracle_compressed(st, qn, qpos_np, stats, lsel, sel, nsel, trees, vtrees, p):
    """The oracle's compressed output of every (row, head), on the GPU's own
    candidates and kept sets (teacher-forced)."""
    w = st.w
    rows = qn.shape[0] * qn.shape[1]
    kept = {l: level_kept(st, lsel, stats, rows, l) for l in range(1, w.n_levels + 1)}
    s_np, n_np = sel.cpu().numpy(), nsel.cpu().numpy()
    outs = {}
    for s in range(w.batch):
        for t_ in range(qn.shape[1]):
            r = s * qn.shape[1] + t_
            N = int(qpos_np[s, t_]) + 1
            for hq in range(w.n_q_heads):
                kv = hq // w.group
                parents, cuts = None, [None] * w.n_levels
                for level in range(w.n_levels, 0, -1):
                    v, cnt, cand = kept[level]
                    gpu_ids = np.sort(v[r, hq, :cnt[r, hq]]).astype(np.int64)
                    cut = O.route_level(qn[s, t_, hq], trees[s][kv][level - 1], level, parents, N, w.branching,
                                        w.n_levels, p, w.scale)
                    assert cand[r, hq] == len(cut.ids)
                    cuts[level - 1] = dataclasses.replace(cut, selected=gpu_ids)
                    parents = gpu_ids
                rr = O.RouteResult(cuts, [c.selected for c in cuts])
                lg, pv = O.pseudo_tokens(rr, vtrees[s][kv], N, w.branching)
                I = O.index_set(s_np[s, t_, hq, :n_np[s, t_, hq]], N, w.branching)
                outs[(s, t_, hq)] = O.attend_compressed(qn[s, t_, hq], st.Kf[s, kv], st.Vf[s, kv], I, lg, pv,
                                                        w.scale) + (len(lg),)
    return outs


def _attend(st, q, q_pos, p, stats=None, lsel=None, rows=None):
    t = torch()
    w = st.w
    sel, nsel, st_, ls_ = st.route_buffers(w.batch * (rows or q.shape[1]))
    out = t.zeros_like(q)
    lse = t.zeros(q.shape[:3], dtype=t.float32, device="cuda")
    Z.attend(st.geom, q, q_pos, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, p, sel, nsel, out,
             lse, st.cache.ws, level_stats=st_ if stats is None else stats, level_sel=ls_ if lsel is None else lsel)
    t.cuda.synchronize()
    return sel, nsel, st_ if stats is None else stats, ls_ if lsel is None else lsel, out, lse


# (workload, shrink, batch, rows): the split cut (one row, b = 32), the per-pair
# cut (batch 8), fp32 with 16 rows, 64 causal rows (every level scored on the
# matrix cores), a deep geometry whose upper levels are cut in the fused kernel
CASES = [("decode1m", 1, 1, 1), ("gqa128k", 2, 8, 1), ("tiny", 0, None, 16), ("gqa128k", 1, 1, 64),
         ("c4l6", 0, 1, 1)]
IDS = ["decode1m-s1", "gqa128k-s2-b8", "tiny-16rows", "gqa128k-s1-64rows", "c4l6"]


def _workload(name, shrink, batch, rows):
    if name == "c4l6":
        w = W.get_workload("gqa128k", batch=1)
        w.n_tokens = w.capacity = 1 << 16
        w.branching, w.n_levels = 4, 6
    else:
        w = W.get_workload(name, shrink=shrink, batch=batch)
    w.queries_per_step = rows
    return w


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_value_summaries_parity(case):
    t = torch()
    w = _workload(*case)
    rows = w.queries_per_step
    say(f"[values] {w.name}: N={w.n_tokens} b={w.branching} L={w.n_levels}, batch {w.batch}, {rows} row(s)")
    st = Staged(w, values=True)
    worst_v = _check_values(st)
    trees = st.oracle_trees()
    vtrees = [[O.build_value_tree(st.Kf[s, h, :w.n_tokens], st.Vf[s, h, :w.n_tokens], st.R[:, h], w.branching)
               for h in range(w.n_kv_heads)] for s in range(w.batch)]
    qn, q = st.queries(0, rows=rows)
    qpos_np = (w.n_tokens - rows + np.arange(rows, dtype=np.int32))[None, :].repeat(w.batch, 0)
    q_pos = t.from_numpy(np.ascontiguousarray(qpos_np)).cuda()
    sel, nsel, stats, lsel, out, lse = _attend(st, q, q_pos, w.top_p)
    assert Z.read_device_status(st.cache.ws) == 0
    ref = _oracle_compressed(st, qn, qpos_np, stats, lsel, sel, nsel, trees, vtrees, w.top_p)
    o_np, l_np = out.cpu().numpy(), lse.cpu().numpy()
    tol = attn_tol(w)
    worst, pseudo = 0.0, 0
    for (s, t_, hq), (o, l, n_ps) in ref.items():
        e = max(np.abs(o_np[s, t_, hq] - o).max(), abs(l_np[s, t_, hq] - l))
        assert e <= tol, (s, t_, hq, e)
        worst, pseudo = max(worst, e), pseudo + n_ps
    assert pseudo > 0
    say(f"  value summaries {worst_v:.3g} of the bound; {pseudo} pseudo-tokens; worst output error {worst:.3g}")
    # p = 1: nothing pruned, the plain zha_attend's bits
    plain = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels, w.capacity,
                        w.kv_dtype)
    _, _, _, _, out1, lse1 = _attend(st, q, q_pos, 1.0)
    st.geom, g_v = plain, st.geom
    pc = Z.Cache(plain, rows)
    sel2, nsel2, stats2, lsel2 = st.route_buffers(w.batch * rows)
    out2, lse2 = t.zeros_like(q), t.zeros_like(lse)
    Z.attend(plain, q, q_pos, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, 1.0, sel2, nsel2, out2,
             lse2, pc.ws)
    t.cuda.synchronize()
    st.geom = g_v
    assert t.equal(out1, out2) and t.equal(lse1, lse2)


def test_value_summaries_exact_on_uniform_subtrees():
    """Keys and values repeated over every top-level span (fp32, b = 4, L = 3):
    every pruned subtree is uniform, so the compressed output equals the dense
    kernel's."""
    t = torch()
    w = W.get_workload("tiny")
    w.branching, w.n_levels = 4, 3
    w.n_tokens, w.capacity = 64 * 40 + 3, 64 * 40 + 3
    rows = 8
    w.queries_per_step = rows
    st = Staged(w, build=False, values=True)
    rng = np.random.default_rng(5)
    d = w.head_dim
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    tops = np.arange(w.capacity) // 64
    a = (rng.standard_normal(tops.max() + 1) * 4).astype(np.float32)
    vals = rng.standard_normal((tops.max() + 1, d)).astype(np.float32)
    K = (a[tops, None] * u[None, :]).astype(np.float32)[None, None]
    V = vals[tops][None, None].astype(np.float32)
    st.cache.K.copy_(t.from_numpy(K))
    st.cache.V.copy_(t.from_numpy(V))
    Z.build_tree(st.geom, st.cache.K, st.ref_q, st.cache.seq_lens, st.cache.summaries, st.cache.ws, V=st.cache.V)
    q = t.from_numpy((rng.standard_normal((1, rows, 1, d)) * 3).astype(np.float32)).cuda()
    q_pos = t.from_numpy((w.n_tokens - rows + np.arange(rows, dtype=np.int32))[None]).cuda()
    for p in (0.3, 0.7):
        sel, nsel, stats, lsel, out, lse = _attend(st, q, q_pos, p)
        od, ld = t.zeros_like(out), t.zeros_like(lse)
        Z.dense_attend(st.geom, q, q_pos, st.cache.K, st.cache.V, st.cache.seq_lens, od, ld, st.cache.ws)
        t.cuda.synchronize()
        kept1 = stats[..., 0, 1].float().mean().item()
        e = max((out - od).abs().max().item(), (lse - ld).abs().max().item())
        say(f"[values uniform] p={p}: kept leaves {kept1:.1f} of {w.n_tokens // 4}, |compressed - dense| {e:.3g}")
        assert e <= 2e-5, (p, e)


def test_value_summaries_append_matches_build():
    t = torch()
    w = W.get_workload("decode1m", shrink=2)      # b = 32, L = 2, bf16, 8 kv heads
    w.capacity = 1400
    n0 = 1000
    st = Staged(w, n_tokens=n0, values=True)
    say("[values append] decode1m shrink 2: 60 single-token appends from 1000, then 200 tokens")
    K_host, V_host = st.K_np.copy(), st.V_np.copy()
    n = n0
    for step in range(60):
        kn, vn = W.appended_tokens(w, step, 1)
        K_host[:, :, n:n + 1], V_host[:, :, n:n + 1] = kn, vn
        Z.append(st.geom, st.cache.K, st.cache.V, kv_tensor(w, kn), kv_tensor(w, vn), st.cache.seq_lens, st.ref_q,
                 st.cache.summaries, st.cache.ws)
        n += 1
    kn, vn = W.appended_tokens(w, 999, 200)
    K_host[:, :, n:n + 200], V_host[:, :, n:n + 200] = kn, vn
    Z.append(st.geom, st.cache.K, st.cache.V, kv_tensor(w, kn), kv_tensor(w, vn), st.cache.seq_lens, st.ref_q,
             st.cache.summaries, st.cache.ws)
    n += 200
    t.cuda.synchronize()
    assert Z.read_device_status(st.cache.ws) == 0
    ref = Z.Cache(st.geom, 1)
    ref.K.copy_(kv_tensor(w, K_host))
    ref.V.copy_(kv_tensor(w, V_host))
    ref.seq_lens.fill_(n)
    Z.build_tree(st.geom, ref.K, st.ref_q, ref.seq_lens, ref.summaries, ref.ws, V=ref.V)
    t.cuda.synchronize()
    for level in range(1, w.n_levels + 1):
        m = n // w.branching ** level
        assert t.equal(st.cache.level(level)[:, :, :m], ref.level(level)[:, :, :m]), level
        a = Z.values_view(st.cache.summaries, st.sizes, st.geom, level)[:, :, :m]
        b = Z.values_view(ref.summaries, ref.sizes, st.geom, level)[:, :, :m]
        assert t.equal(a, b), level
