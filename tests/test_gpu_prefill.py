"""Chunked causal prefill on the GPU against the oracle.

A chunk of new tokens is appended to a built cache (the tree grows by every
node the chunk completes), then every row of the chunk is routed and attended
at once, each row seeing the tokens up to its own position. With this many
rows per sequence every level's node scores come from one contraction per
(sequence, kv head) on the fp32 matrix cores; the cuts read them per
(row, head).

Checks, on sampled rows (every head): each level's kept set against the
oracle's cut of the same candidates (teacher forcing, margin exemptions as in
the decode tests), the candidate counts, and the attention output over the
GPU's own index set within the bf16 tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest

import hierarchical_tree_indexed_build_amd as Z
import workloads as W
from oracle import zha_oracle as O
from tests.gpu_helpers import Staged, attn_tol, check_sets, kv_tensor, level_kept, say, torch

pytestmark = pytest.mark.gpu

# (workload, shrink, chunk): shrink 1 is a 16384-token cache + 512-row chunk
# (16 row tiles per kv head, 9 node tiles at level 1, the last one ragged);
# shrink 2 with 200 rows has a ragged row tile; shrink 0 is the full
# 262144-token cache + 8192-row chunk.
PREFILL = [("prefill256k", 2, 200), ("prefill256k", 1, None), ("prefill256k", 0, None)]


def _sample_rows(T, k):
    rows = set(range(0, T, max(1, T // k)))
    rows.update({0, 1, T // 2, T - 2, T - 1})
    return sorted(r for r in rows if 0 <= r < T)


def _run_prefill(w, sel_cap):
    t = torch()
    n0, T = w.n_tokens, w.prefill_chunk
    st = Staged(w, max_t=T)
    kn, vn = W.prefill_chunk_kv(w)
    Z.append(st.geom, st.cache.K, st.cache.V, kv_tensor(w, kn), kv_tensor(w, vn), st.cache.seq_lens, st.ref_q,
             st.cache.summaries, st.cache.ws)
    qn, q = st.queries(0, rows=T)
    q_pos = (n0 + t.arange(T, dtype=t.int32, device="cuda")).view(1, T).repeat(w.batch, 1).contiguous()
    sizes = Z.query_sizes(st.geom, T)
    sel = t.full((w.batch, T, w.n_q_heads, sel_cap), -1, dtype=t.int32, device="cuda")
    nsel = t.zeros((w.batch, T, w.n_q_heads), dtype=t.int32, device="cuda")
    stats = t.zeros((w.batch, T, w.n_q_heads, w.n_levels, 2), dtype=t.int32, device="cuda")
    lsel = t.full((sizes.level_sel_bytes // 4,), -1, dtype=t.int32, device="cuda")
    out = t.zeros_like(q)
    lse = t.zeros(q.shape[:3], dtype=t.float32, device="cuda")
    Z.attend(st.geom, q, q_pos, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, w.top_p, sel, nsel,
             out, lse, st.cache.ws, level_stats=stats, level_sel=lsel)
    t.cuda.synchronize()
    assert int(st.cache.seq_lens[0].item()) == n0 + T
    Kf = np.concatenate([st.Kf[:, :, :n0], W.as_f32(w, kn)], axis=2)
    Vf = np.concatenate([st.Vf[:, :, :n0], W.as_f32(w, vn)], axis=2)
    return st, qn, q_pos, sel, nsel, stats, lsel, out, lse, Kf, Vf


@pytest.mark.parametrize("case", PREFILL, ids=[f"{n}-s{s}" + (f"-c{c}" if c else "") for n, s, c in PREFILL])
def test_prefill_chunk_parity(case):
    name, shrink, chunk = case
    w = W.get_workload(name, shrink=shrink, chunk=chunk)
    T = w.prefill_chunk
    say(f"[prefill] {w.name}: {w.n_tokens} cached tokens + {T}-row causal chunk, L={w.n_levels}")
    full = shrink == 0
    sel_cap = 4096 if full else None
    st, qn, q_pos, sel, nsel, stats, lsel, out, lse, Kf, Vf = _run_prefill(
        w, sel_cap if sel_cap else (w.capacity // w.branching))
    assert Z.read_device_status(st.cache.ws, clear=True) & ~Z.ZHA_DEV_SEL_OVERFLOW == 0
    rows = _sample_rows(T, 12 if full else 48)
    say(f"  checking rows {rows[:6]}... ({len(rows)} rows x {w.n_q_heads} heads)")
    trees = O.build_all(Kf, st.R, [w.n_tokens + T] * w.batch, w.branching)
    g = st.geom
    ridx = torch().tensor(rows, dtype=torch().int64, device="cuda")
    # per level: kept ids of the sampled rows only (the full buffers are large)
    kept = {}
    for level in range(1, w.n_levels + 1):
        v = Z.level_sel_view(lsel, st.sizes, g, w.batch * T, level)
        kept[level] = v.view(w.batch, T, w.n_q_heads, -1).index_select(1, ridx).cpu().numpy()
    st_np = stats.index_select(1, ridx).cpu().numpy()
    o_np = out.index_select(1, ridx).cpu().numpy()
    l_np = lse.index_select(1, ridx).cpu().numpy()
    tol = attn_tol(w)
    flips = 0
    worst = 0.0
    for s in range(w.batch):
        for i, t_ in enumerate(rows):
            N = w.n_tokens + t_ + 1
            for hq in range(w.n_q_heads):
                kv = hq // w.group
                parents = None
                for level in range(w.n_levels, 0, -1):
                    cand, cnt = st_np[s, i, hq, level - 1]
                    gpu_ids = kept[level][s, i, hq, :cnt]
                    cut = O.route_level(qn[s, t_, hq], trees[s][kv][level - 1], level, parents, N, w.branching,
                                        w.n_levels, w.top_p, w.scale)
                    assert cand == len(cut.ids), (s, t_, hq, level, cand, len(cut.ids))
                    assert np.all(np.diff(gpu_ids) > 0), "kept ids must be ascending"
                    flips += check_sets(gpu_ids, cut, w.top_p, f"row {t_} head {hq} level {level}")
                    parents = gpu_ids
                I = O.index_set(parents, N, w.branching)
                o, l = O.attend(qn[s, t_, hq], Kf[s, kv], Vf[s, kv], I, w.scale)
                e = max(np.abs(o_np[s, i, hq] - o).max(), abs(l_np[s, i, hq] - l))
                worst = max(worst, e)
                assert e <= tol, (s, t_, hq, e)
    say(f"  margin-exempt differences: {flips}; worst |gpu - oracle| attention {worst:.3g} (tol {tol})")


# crowded scores through the one-wave-per-pair cut: identical keys (every
# score equal: one bin, ties broken by node id) and keys within a narrow band
# (crowded bins resolved by radix select)
CROWDED = [("equal", 0.0), ("band", 1e-3), ("band", 3e-2)]


@pytest.mark.parametrize("kind,noise", CROWDED, ids=[f"{k}-{e:g}" for k, e in CROWDED])
def test_many_rows_crowded_scores(kind, noise):
    t = torch()
    w = W.get_workload("gqa128k", shrink=1, batch=1)
    T = 64
    say(f"[many rows crowded] {kind} noise {noise:g}: {w.n_tokens} tokens, {T} causal rows")
    st = Staged(w, max_t=T, build=False)
    rng = np.random.default_rng(20261204)
    B, H, C, D = st.K_np.shape
    base = rng.standard_normal((B, H, 1, D)).astype(np.float32)
    K = np.broadcast_to(base, (B, H, C, D)).copy()
    if noise:
        K += noise * rng.standard_normal(K.shape).astype(np.float32)
    st.K_np = W.f32_to_bf16_bits(K)
    st.Kf = W.as_f32(w, st.K_np)
    st.cache.K.copy_(kv_tensor(w, st.K_np))
    Z.build_tree(st.geom, st.cache.K, st.ref_q, st.cache.seq_lens, st.cache.summaries, st.cache.ws)
    qn, q = st.queries(0, rows=T)
    q_pos = (w.n_tokens - T + t.arange(T, dtype=t.int32, device="cuda")).view(1, T).contiguous()
    sel, nsel, stats, lsel = st.route_buffers(T)
    Z.route(st.geom, q, q_pos, st.cache.summaries, st.cache.seq_lens, w.top_p, sel, nsel, st.cache.ws,
            level_stats=stats, level_sel=lsel)
    t.cuda.synchronize()
    trees = st.oracle_trees()
    kept = {level: level_kept(st, lsel, stats, T, level) for level in range(1, w.n_levels + 1)}
    flips = 0
    for t_ in range(T):
        N = w.n_tokens - T + t_ + 1
        for hq in range(w.n_q_heads):
            kv = hq // w.group
            parents = None
            for level in range(w.n_levels, 0, -1):
                v, cnt, cand = kept[level]
                gpu_ids = v[t_, hq, :cnt[t_, hq]]
                cut = O.route_level(qn[0, t_, hq], trees[0][kv][level - 1], level, parents, N, w.branching,
                                    w.n_levels, w.top_p, w.scale)
                assert cand[t_, hq] == len(cut.ids), (t_, hq, level, cand[t_, hq], len(cut.ids))
                assert np.all(np.diff(gpu_ids) > 0), "kept ids must be ascending"
                flips += check_sets(gpu_ids, cut, w.top_p, f"row {t_} head {hq} level {level}")
                parents = gpu_ids
    say(f"  margin-exempt differences: {flips}")


# exact ties at the cut boundary through the one-wave cut: every chunk of
# the cache repeats one of 256 key patterns, so the nodes of a pattern score
# identically and the index rule splits a boundary tie group. The cache of
# 131072 tokens puts 8192 nodes at level 1 (the variant that re-reads
# scores); peaked scores (amplitude 2) keep few leaves, so the kept set comes
# from the boundary bin's members and the list of earlier bins, flat ones
# (amplitude 0.5) keep hundreds and take the compaction over all candidates.
TIES = [2.0, 0.5]


@pytest.mark.parametrize("amp", TIES, ids=[f"amp{a:g}" for a in TIES])
def test_many_rows_boundary_ties(amp):
    t = torch()
    w = W.get_workload("gqa128k", shrink=0, batch=1)
    T, M = 64, 256
    say(f"[many rows ties] amplitude {amp:g}, {M} chunk patterns: {w.n_tokens} tokens, {T} causal rows")
    st = Staged(w, max_t=T, build=False)
    rng = np.random.default_rng(20261205)
    B, H, C, D = st.K_np.shape
    pat = (amp * rng.standard_normal((H, M, D))).astype(np.float32)
    chunk = np.arange(C) // w.branching
    st.K_np = W.f32_to_bf16_bits(np.ascontiguousarray(pat[:, chunk % M][None]))
    st.Kf = W.as_f32(w, st.K_np)
    st.cache.K.copy_(kv_tensor(w, st.K_np))
    Z.build_tree(st.geom, st.cache.K, st.ref_q, st.cache.seq_lens, st.cache.summaries, st.cache.ws)
    qn, q = st.queries(0, rows=T)
    q_pos = (w.n_tokens - T + t.arange(T, dtype=t.int32, device="cuda")).view(1, T).contiguous()
    sel, nsel, stats, lsel = st.route_buffers(T)
    Z.route(st.geom, q, q_pos, st.cache.summaries, st.cache.seq_lens, w.top_p, sel, nsel, st.cache.ws,
            level_stats=stats, level_sel=lsel)
    t.cuda.synchronize()
    trees = st.oracle_trees()
    kept = {level: level_kept(st, lsel, stats, T, level) for level in range(1, w.n_levels + 1)}
    flips = split_ties = 0
    leaf_kept = []
    for t_ in _sample_rows(T, 16):
        N = w.n_tokens - T + t_ + 1
        for hq in range(w.n_q_heads):
            kv = hq // w.group
            parents = None
            for level in range(w.n_levels, 0, -1):
                v, cnt, cand = kept[level]
                gpu_ids = v[t_, hq, :cnt[t_, hq]]
                cut = O.route_level(qn[0, t_, hq], trees[0][kv][level - 1], level, parents, N, w.branching,
                                    w.n_levels, w.top_p, w.scale)
                assert cand[t_, hq] == len(cut.ids), (t_, hq, level, cand[t_, hq], len(cut.ids))
                assert np.all(np.diff(gpu_ids) > 0), "kept ids must be ascending"
                flips += check_sets(gpu_ids, cut, w.top_p, f"row {t_} head {hq} level {level}")
                last = cut.scores64[cut.order[cut.m - 1]]
                split_ties += int(np.sum(cut.scores64 == last) > np.sum(cut.scores64[cut.order[:cut.m]] == last))
                if level == 1:
                    leaf_kept.append(len(gpu_ids))
                parents = gpu_ids
    leaf_kept = np.array(leaf_kept)
    say(f"  margin-exempt differences: {flips}; cuts splitting a tie group: {split_ties}; "
        f"leaves kept min/median/max {leaf_kept.min()}/{int(np.median(leaf_kept))}/{leaf_kept.max()}")
    assert split_ties > 0, "no cut split a tie group"
    if amp > 1:
        assert np.median(leaf_kept) <= 128, "peaked scores should keep few leaves"
    else:
        assert np.median(leaf_kept) > 128, "flat scores should keep many leaves"


def test_many_rows_deep_levels():
    """b = 2 puts levels of 32768 and 16384 nodes under 64 causal rows: the
    one-wave cut re-reads their scores from global memory, and the larger
    one keeps its kept bitmap in global memory."""
    t = torch()
    w = W.get_workload("tiny")
    w.n_tokens = 65536
    w.capacity = 65536
    w.branching = 2
    w.n_levels = 5
    w.top_p = 0.9
    T = 64
    say(f"[many rows deep] b=2 L=5 N=65536, {T} causal rows")
    st = Staged(w, max_t=T)
    qn, q = st.queries(0, rows=T)
    q_pos = (w.n_tokens - T + t.arange(T, dtype=t.int32, device="cuda")).view(1, T).contiguous()
    sel, nsel, stats, lsel = st.route_buffers(T)
    Z.route(st.geom, q, q_pos, st.cache.summaries, st.cache.seq_lens, w.top_p, sel, nsel, st.cache.ws,
            level_stats=stats, level_sel=lsel)
    t.cuda.synchronize()
    trees = st.oracle_trees()
    kept = {level: level_kept(st, lsel, stats, T, level) for level in range(1, w.n_levels + 1)}
    flips = 0
    for t_ in range(T):
        N = w.n_tokens - T + t_ + 1
        parents = None
        for level in range(w.n_levels, 0, -1):
            v, cnt, cand = kept[level]
            gpu_ids = v[t_, 0, :cnt[t_, 0]]
            cut = O.route_level(qn[0, t_, 0], trees[0][0][level - 1], level, parents, N, w.branching,
                                w.n_levels, w.top_p, w.scale)
            assert cand[t_, 0] == len(cut.ids), (t_, level, cand[t_, 0], len(cut.ids))
            assert np.all(np.diff(gpu_ids) > 0), "kept ids must be ascending"
            flips += check_sets(gpu_ids, cut, w.top_p, f"row {t_} level {level}")
            parents = gpu_ids
        # the leaf level's kept ids also arrive as sel_blocks / n_sel
        n1 = int(nsel[0, t_, 0].item())
        assert n1 == len(parents)
        assert np.array_equal(np.sort(sel[0, t_, 0, :n1].cpu().numpy()), parents)
    say(f"  margin-exempt differences: {flips}")


@pytest.mark.parametrize("shrink", [1, 0], ids=["s1", "full"])
def test_prefill_row_tiles_match_one_pass(shrink):
    """A workspace that holds only a tile of rows: zha_attend runs the chunk in
    row tiles. Kept leaves, counts per level and the positions the rows see are
    those of one pass over every row (each row's route is its own); the
    attention differs only by the split-K partition's fp32 rounding."""
    t = torch()
    w = W.get_workload("prefill256k", shrink=shrink)
    n0, T = w.n_tokens, w.prefill_chunk
    st = Staged(w, max_t=T)
    kn, vn = W.prefill_chunk_kv(w)
    Z.append(st.geom, st.cache.K, st.cache.V, kv_tensor(w, kn), kv_tensor(w, vn), st.cache.seq_lens, st.ref_q,
             st.cache.summaries, st.cache.ws)
    qn, q = st.queries(0, rows=T)
    sizes = Z.query_sizes(st.geom, T)
    tile = 128 if shrink else sizes.tile_rows
    small = Z.query_sizes(st.geom, tile).workspace_bytes
    say(f"[prefill tiles] {w.name}: {T} rows; one pass {sizes.workspace_bytes / 2**30:.2f} GiB, "
        f"tiles of {tile} rows {small / 2**30:.3f} GiB (tile_rows {sizes.tile_rows})")
    ws_small = t.zeros(small // 4 + 64, dtype=t.int32, device="cuda")
    cap = 4096
    res = []
    for ws in (st.cache.ws, ws_small):
        sel = t.full((1, T, w.n_q_heads, cap), -1, dtype=t.int32, device="cuda")
        nsel = t.zeros((1, T, w.n_q_heads), dtype=t.int32, device="cuda")
        stats = t.zeros((1, T, w.n_q_heads, w.n_levels, 2), dtype=t.int32, device="cuda")
        out = t.zeros_like(q)
        lse = t.zeros(q.shape[:3], dtype=t.float32, device="cuda")
        # no q_pos: the rows are the last T positions, which the tiles must reproduce
        Z.attend(st.geom, q, None, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, w.top_p, sel,
                 nsel, out, lse, ws, level_stats=stats)
        t.cuda.synchronize()
        res.append((sel, nsel, stats, out, lse))
    (s1, n1, a1, o1, l1), (s2, n2, a2, o2, l2) = res
    assert t.equal(n1, n2) and t.equal(a1, a2)
    m = n1.clamp(max=cap)
    keep = t.arange(cap, device="cuda")[None, None, None, :] < m[..., None]
    assert t.equal(t.where(keep, s1, -1), t.where(keep, s2, -1))
    e = max((o1 - o2).abs().max().item(), (l1 - l2).abs().max().item())
    say(f"  kept sets and counts identical; |tiled - one pass| = {e:.3g}")
    assert e <= 1e-4
