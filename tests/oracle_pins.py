"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Every pin is a plain function of the oracle module so that the same checks can
be run against deliberately broken copies of the oracle (see
``test_oracle_mutants.py``): each plausible mistake must trip at least one pin.

What pins what:
* geometry       - spans and node counts printed on the pages (golden file).
* summaries      - torch's scaled_dot_product_attention in fp64 with the chunk as
                   keys and values (the pages define the summary as exactly that
                   attention); closed forms (zero reference query -> mean,
                   identical children -> the child, huge reference query -> the
                   arg-max child); permutation invariance; append order.
* cut            - hand-worked cases (golden file), brute force over all subsets
                   for small candidate sets, the uniform-mass closed form ceil(p n).
* routing        - hand-worked trees (golden file); an independent mask-based
                   formulation; causal prefixes.
* attention      - torch SDPA with a boolean mask; p = 1 equals dense; the
                   top-p decomposition identity; split-and-merge by LSE.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa64(q, k, v):
    """torch SDPA in fp64, single query: q (d,), k/v (n, d) -> (d,)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


def _sdpa64_masked(q, k, v, mask):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    mt = torch.from_numpy(np.asarray(mask, bool))[None, None, None, :]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt)[0, 0, 0].numpy()


def _ranges(rs):
    out = []
    for a, b in rs:
        out.extend(range(a, b))
    return np.array(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------
def pin_geometry(orc):
    g = _load("geometry_pages.json")
    for c in g["cases"]:
        if "spans_top_down" in c:
            spans = [orc.node_span(c["b"], l) for l in range(c["levels"], 0, -1)]
            assert spans == c["spans_top_down"], (spans, c)
        elif "pairs" in c:
            for b, L in c["pairs"]:
                assert orc.node_span(b, L) == c["span"]
        elif "n_top" in c:
            assert orc.complete_nodes(c["n_tokens"], c["b"], c["levels"])[-1] == c["n_top"]
        else:
            assert orc.node_span(c["b"], c["levels"]) == c["span"]
    # complete nodes only: 4095 tokens leave the last leaf of b=16 and the top node incomplete
    assert orc.complete_nodes(4095, 16, 3) == [255, 15, 0]
    assert orc.complete_nodes(4096, 16, 3) == [256, 16, 1]


# ----------------------------------------------------------------------------
# summaries
# ----------------------------------------------------------------------------
def pin_summary_sdpa(orc):
    rng = np.random.default_rng(11)
    for b, d, L, n in [(4, 8, 3, 200), (16, 64, 2, 600), (3, 5, 2, 40)]:
        K = rng.standard_normal((n, d)).astype(np.float32)
        R = rng.standard_normal((L, d)).astype(np.float32)
        tree = orc.build_tree(K, R, b)
        X = K.astype(np.float64)
        for l in range(L):
            m = X.shape[0] // b
            assert tree[l].shape == (m, d), (tree[l].shape, m, d)
            assert tree[l].dtype == np.float32
            ref = np.stack([_sdpa64(R[l], X[i * b:(i + 1) * b], X[i * b:(i + 1) * b]) for i in range(m)]) \
                if m else np.zeros((0, d))
            err = np.abs(tree[l].astype(np.float64) - ref).max() if m else 0.0
            tol = 4 * np.finfo(np.float32).eps * max(1.0, np.abs(ref).max() if m else 1.0)
            assert err <= tol, (b, d, l, err, tol)
            X = tree[l].astype(np.float64)      # the next level is built from stored (fp32) summaries


def pin_summary_closed_forms(orc):
    rng = np.random.default_rng(12)
    b, d = 8, 16
    C = rng.standard_normal((b, d)).astype(np.float32)
    # zero reference query: plain mean
    s0 = orc.pool_children(C, np.zeros(d, np.float32), b, 1 / math.sqrt(d))[0]
    assert np.abs(s0 - C.astype(np.float64).mean(0)).max() < 1e-6
    # identical children: the child itself
    same = np.repeat(C[:1], b, axis=0)
    s1 = orc.pool_children(same, rng.standard_normal(d).astype(np.float32), b, 1 / math.sqrt(d))[0]
    assert np.array_equal(s1, C[0])
    # a huge reference query along e_0 picks the child with the largest e_0 component
    r = np.zeros(d, np.float32)
    r[0] = 1e5
    s2 = orc.pool_children(C, r, b, 1 / math.sqrt(d))[0]
    assert np.abs(s2 - C[np.argmax(C[:, 0])]).max() < 1e-6
    # and the smallest one for the opposite direction (sign of the pooling logits)
    s3 = orc.pool_children(C, -r, b, 1 / math.sqrt(d))[0]
    assert np.abs(s3 - C[np.argmin(C[:, 0])]).max() < 1e-6
    # permutation of the children does not change the summary
    rr = rng.standard_normal(d).astype(np.float32)
    perm = rng.permutation(b)
    a1 = orc.pool_children(C, rr, b, 1 / math.sqrt(d))[0]
    a2 = orc.pool_children(C[perm], rr, b, 1 / math.sqrt(d))[0]
    assert np.abs(a1.astype(np.float64) - a2).max() < 1e-6
    # one summary per group of b consecutive rows; a partial group makes no summary
    K = rng.standard_normal((3 * b + 5, d)).astype(np.float32)
    out = orc.pool_children(K, rr, b, 1 / math.sqrt(d))
    assert out.shape == (3, d)
    assert np.abs(out[1] - orc.pool_children(K[b:2 * b], rr, b, 1 / math.sqrt(d))[0]).max() == 0


def pin_incremental_equals_batch(orc):
    rng = np.random.default_rng(13)
    for b, L, n in [(4, 3, 150), (2, 5, 77), (8, 2, 130)]:
        K = rng.standard_normal((n, 8)).astype(np.float32)
        R = rng.standard_normal((L, 8)).astype(np.float32)
        t1 = orc.build_tree(K, R, b)
        t2 = orc.build_tree_incremental(K, R, b)
        t3 = orc.build_tree(K, R, b, slab=3 * b)      # level 1 pooled a few leaves at a time
        for a, c, e in zip(t1, t2, t3):
            assert a.shape == c.shape and np.array_equal(a, c), (b, L, n)
            assert a.shape == e.shape and np.array_equal(a, e), (b, L, n)


# ----------------------------------------------------------------------------
# cut
# ----------------------------------------------------------------------------
def _parse_score(s):
    return math.log(float(s[2:])) if s.startswith("ln") else float(s)


def pin_cut_golden(orc):
    for c in _load("cut_cases.json")["cases"]:
        s = np.array([_parse_score(x) for x in c["scores"]])
        r = orc.topp_cut(np.array(c["ids"]), s, c["p"])
        assert list(r.selected) == c["kept"], (c, list(r.selected))


def pin_cut_bruteforce(orc):
    rng = np.random.default_rng(14)
    checked = 0
    for trial in range(400):
        n = int(rng.integers(1, 10))
        if trial % 3 == 0:
            s = rng.integers(-2, 3, size=n).astype(np.float64) * 0.7     # many exact ties
        else:
            s = rng.standard_normal(n) * rng.choice([0.3, 1.0, 4.0])
        ids = rng.permutation(50)[:n]
        p = float(rng.choice([0.05, 0.3, 0.5, 0.77, 0.9, 0.95, 0.999]))
        w = np.exp(s - s.max())
        w = w / w.sum()
        masses = {}
        best = None
        near = False
        for k in range(1, n + 1):
            for sub in itertools.combinations(range(n), k):
                m = w[list(sub)].sum()
                if abs(m - p) < 1e-9:
                    near = True
                if m >= p and best is None:
                    best = k
            if best is not None:
                break
        if near:
            continue
        r = orc.topp_cut(ids, s, p)
        kept = set(int(i) for i in r.selected)
        pos = {int(i): j for j, i in enumerate(ids)}
        assert len(kept) == best, (s, p, kept, best)
        assert w[[pos[i] for i in kept]].sum() >= p
        out = [j for j in range(n) if int(ids[j]) not in kept]
        inn = [pos[i] for i in kept]
        if out:
            lo_in = min(s[j] for j in inn)
            hi_out = max(s[j] for j in out)
            assert lo_in >= hi_out, (s, kept)
            if lo_in == hi_out:       # a tie straddles the cut: lower ids must be inside
                tie_in = max(int(ids[j]) for j in inn if s[j] == lo_in)
                tie_out = min(int(ids[j]) for j in out if s[j] == hi_out)
                assert tie_in < tie_out, (s, ids, kept)
        checked += 1
    assert checked > 300


def pin_cut_exemptions(orc):
    """The margin rule's exempt sets on hand-worked cases (golden file); then, on
    random cuts with many exact ties, the oracle's set (which only pairs the
    candidates nearest the boundary) equals a pass over every pair."""
    for c in _load("exemption_cases.json")["cases"]:
        s = np.array([_parse_score(x) for x in c["scores"]])
        r = orc.topp_cut(np.array(c["ids"]), s, c["p"])
        got = [int(x) for x in orc.cut_exemptions(r, c["p"])]
        assert got == c["exempt"], (c["name"], got, c["exempt"])
    rng = np.random.default_rng(22)
    for _ in range(200):
        n = int(rng.integers(2, 30))
        s = np.round(rng.standard_normal(n) * 0.5, 3)
        ids = rng.permutation(1000)[:n]
        p = float(rng.choice([0.3, 0.6, 0.9, 0.95]))
        r = orc.topp_cut(ids, s, p)
        ex = set(int(x) for x in orc.cut_exemptions(r, p))
        w = np.exp(s - s.max())
        w = w / w.sum()
        order = np.lexsort((ids, -s))
        before = np.concatenate([[0.0], np.cumsum(w[order])])
        rank = {int(ids[j]): k for k, j in enumerate(order)}
        kept = set(int(x) for x in r.selected)
        pos = {int(i): j for j, i in enumerate(ids)}
        want = set()
        for i in map(int, ids):
            if abs(before[rank[i]] - p) < 1e-5:
                want.add(i)
            for o in map(int, ids):
                if (i in kept) != (o in kept) and s[pos[i]] != s[pos[o]] and abs(w[pos[i]] - w[pos[o]]) < 1e-5:
                    want.add(i)
        assert ex == want, (sorted(ex), sorted(want))


def pin_cut_uniform(orc):
    for n in [1, 2, 3, 7, 16, 100, 240, 257]:
        for p in [0.1, 0.33, 0.5, 0.91, 0.95, 0.999]:
            if abs(p * n - round(p * n)) < 1e-6:
                continue
            r = orc.topp_cut(np.arange(n)[::-1].copy(), np.full(n, 0.25), p)
            assert list(r.selected) == list(range(math.ceil(p * n))), (n, p, r.m)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def _golden_inputs(c):
    b, L, N, d = c["b"], c["L"], c["N"], c["d"]
    u = np.zeros(d, np.float32)
    u[0] = 1.0
    if c["keys"] == "identical":
        rng = np.random.default_rng(15)
        k0 = rng.standard_normal(d).astype(np.float32)
        K = np.repeat(k0[None], N, axis=0)
        R = rng.standard_normal((L, d)).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
    else:
        K = np.zeros((N, d), np.float32)
        for leaf, val in c["values"].items():
            i = int(leaf)
            K[i * b:(i + 1) * b] = np.float32(val) * u
        R = np.zeros((L, d), np.float32)
        q = (np.float32(c["qscale"] * math.sqrt(d)) * u).astype(np.float32)
    return K, R, q


def pin_route_golden(orc):
    for c in _load("route_closed_forms.json")["cases"]:
        K, R, q = _golden_inputs(c)
        tree = orc.build_tree(K, R, c["b"])
        r = orc.route(q, tree, c["N"], c["b"], c["p_levels"] if "p_levels" in c else c["p"])
        for lvl, rs in c["kept"].items():
            got = list(r.selected[int(lvl) - 1])
            assert got == list(_ranges(rs)), (c["name"], lvl, got)
        I = orc.index_set(r.selected[0], c["N"], c["b"])
        assert list(I) == list(_ranges(c["I"])), (c["name"], list(I))


def route_by_masks(q, tree, N, b, p, scale):
    """Independent formulation: score every complete node, restrict by masks.

    A node is allowed at level l if it is complete and either l is the top level,
    or its parent is kept, or its parent is not complete.
    """
    L = len(tree)
    nc = [N // b ** l for l in range(1, L + 1)]
    kept = [None] * L
    parent_kept = None
    for level in range(L, 0, -1):
        n = nc[level - 1]
        allowed = []
        for i in range(n):
            par = i // b
            if level == L or par >= nc[level] or par in parent_kept:
                allowed.append(i)
        s64 = scale * (tree[level - 1][:n].astype(np.float64) @ q.astype(np.float64)) if n else np.zeros(0)
        s = s64.astype(np.float32).astype(np.float64)
        if not allowed:
            kept[level - 1] = []
            parent_kept = set()
            continue
        pairs = sorted(allowed, key=lambda i: (-s[i], i))
        mx = max(s[i] for i in allowed)
        tot = sum(math.exp(s[i] - mx) for i in allowed)
        acc, take = 0.0, []
        for i in pairs:
            if p < 1.0 and acc >= p * tot:
                break
            take.append(i)
            acc += math.exp(s[i] - mx)
        kept[level - 1] = sorted(take)
        parent_kept = set(take)
    return kept


def pin_route_dense_mask(orc):
    rng = np.random.default_rng(16)
    for b, L, N, d, p in [(4, 3, 203, 8, 0.8), (3, 4, 250, 6, 0.9), (8, 2, 500, 16, 0.95), (2, 5, 61, 4, 0.7)]:
        K = rng.standard_normal((N, d)).astype(np.float32)
        R = rng.standard_normal((L, d)).astype(np.float32)
        tree = orc.build_tree(K, R, b)
        for _ in range(6):
            q = (rng.standard_normal(d) * 2).astype(np.float32)
            r = orc.route(q, tree, N, b, p)
            want = route_by_masks(q, tree, N, b, p, 1 / math.sqrt(d))
            for l in range(L):
                assert list(r.selected[l]) == want[l], (b, L, N, l, list(r.selected[l]), want[l])


def pin_causal_prefix(orc):
    rng = np.random.default_rng(17)
    b, L, N, d = 4, 3, 180, 8
    K = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((L, d)).astype(np.float32)
    full = orc.build_tree(K, R, b)
    for t in [0, 3, 4, 15, 16, 63, 64, 65, 130, 179]:
        q = rng.standard_normal(d).astype(np.float32) * 3
        part = orc.build_tree(K[:t + 1], R, b)
        a = orc.route(q, full, t + 1, b, 0.85)
        c = orc.route(q, part, t + 1, b, 0.85)
        for l in range(L):
            assert list(a.selected[l]) == list(c.selected[l]), (t, l)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def pin_attend_sdpa(orc):
    rng = np.random.default_rng(18)
    for N, d in [(50, 8), (300, 64), (1, 16)]:
        K = rng.standard_normal((N, d)).astype(np.float32)
        V = rng.standard_normal((N, d)).astype(np.float32)
        q = (rng.standard_normal(d) * 2).astype(np.float32)
        idx = np.sort(rng.choice(N, size=max(1, N // 3), replace=False))
        o, lse = orc.attend(q, K, V, idx)
        mask = np.zeros(N, bool)
        mask[idx] = True
        ref = _sdpa64_masked(q, K, V, mask)
        assert np.abs(o - ref).max() < 1e-12
        z = (K[idx].astype(np.float64) @ q.astype(np.float64)) / math.sqrt(d)
        assert abs(lse - logsumexp(z)) < 1e-12
        od, _ = orc.dense_attend(q, K, V, N)
        assert np.abs(od - _sdpa64(q, K, V)).max() < 1e-12


def pin_p1_dense(orc):
    rng = np.random.default_rng(19)
    for b, L, N, d in [(16, 3, 4096, 16), (4, 3, 203, 8), (32, 2, 2000, 8)]:
        K = (rng.standard_normal((N, d)) / math.sqrt(d)).astype(np.float32)
        V = rng.standard_normal((N, d)).astype(np.float32)
        R = rng.standard_normal((L, d)).astype(np.float32)
        tree = orc.build_tree(K, R, b)
        q = (rng.standard_normal(d) * 3).astype(np.float32)
        r = orc.route(q, tree, N, b, 1.0)
        I = orc.index_set(r.selected[0], N, b)
        assert list(I) == list(range(N))
        o, lse = orc.attend(q, K, V, I)
        od, lsed = orc.dense_attend(q, K, V, N)
        assert np.abs(o - od).max() / np.abs(od).max() <= 1e-6
        assert abs(lse - lsed) <= 1e-6 * max(1.0, abs(lsed))


def pin_eq1_identity(orc):
    """Top-p decomposition: o_dense = P_S o_S + (1 - P_S) o_rest with P_S the mass of S."""
    rng = np.random.default_rng(20)
    b, L, N, d, p = 8, 2, 700, 16, 0.9
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((L, d)).astype(np.float32)
    tree = orc.build_tree(K, R, b)
    for _ in range(4):
        q = (rng.standard_normal(d) * 3).astype(np.float32)
        od, _ = orc.dense_attend(q, K, V, N)
        r = orc.route(q, tree, N, b, p)
        for S in (orc.index_set(r.selected[0], N, b), orc.topp_key_set(q, K, N, p)):
            rest = np.setdiff1d(np.arange(N), S)
            P = orc.realised_mass(q, K, N, S)
            oS, _ = orc.attend(q, K, V, S)
            mix = P * oS
            if len(rest):
                oR, _ = orc.attend(q, K, V, rest)
                mix = mix + (1 - P) * oR
            assert np.abs(mix - od).max() <= 1e-6 * max(1.0, np.abs(od).max())
        Kp = orc.topp_key_set(q, K, N, p)
        assert orc.realised_mass(q, K, N, Kp) >= p
        if len(Kp) > 1:   # minimal: dropping its smallest member falls below p
            pr = orc.key_probs(q, K, N)
            assert pr[Kp].sum() - pr[Kp].min() < p


def pin_split_merge(orc):
    rng = np.random.default_rng(21)
    N, d = 400, 32
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    q = (rng.standard_normal(d) * 2).astype(np.float32)
    I = np.sort(rng.choice(N, size=150, replace=False))
    o, lse = orc.attend(q, K, V, I)
    parts = np.array_split(I[rng.permutation(len(I))], 4)
    os_, ls = zip(*[orc.attend(q, K, V, np.sort(pp)) for pp in parts])
    M = logsumexp(ls)
    merged = sum(math.exp(l - M) * x for l, x in zip(ls, os_))
    assert np.abs(merged - o).max() < 1e-12
    assert abs(M - lse) < 1e-12


# ----------------------------------------------------------------------------
# the full scoring rule: tangents, offsets, max over R reference queries
# ----------------------------------------------------------------------------
def _entropy(z):
    w = np.exp(z - z.max())
    w = w / w.sum()
    return float(-(w[w > 0] * np.log(w[w > 0])).sum())


def pin_tangent_golden(orc):
    """Hand-worked one-dimensional trees (d = 1, scale 1) where the offset, the
    maximum over reference queries and the child offsets each change the answer."""
    K = np.array([[0.0], [0.0], [1.0], [-1.0]], np.float32)     # chunk 0 = {0, 0}, chunk 1 = {1, -1}
    th = math.tanh(10.0)
    H = math.log(math.exp(10) + math.exp(-10)) - 10 * th         # entropy of softmax(+-10): chunk 1's offset
    # one reference query q_hat = 10: chunk 0 is (k_hat 0, b_hat ln 2), chunk 1 is (tanh 10, H)
    t1 = orc.build_tangent_tree(K, np.array([[[10.0]]], np.float32), 2, scale=1.0)
    assert abs(float(t1[0].keys[0, 0, 0])) < 1e-7 and abs(float(t1[0].offs[0, 0]) - math.log(2)) < 1e-7
    assert abs(float(t1[0].keys[1, 0, 0]) - th) < 1e-7 and abs(float(t1[0].offs[1, 0]) - H) < 1e-7
    # q = 0.5: scores ln 2 (chunk 0) vs 0.5 tanh 10 + H (chunk 1); chunk 0 alone holds 2 / (2 + e^0.5) = 0.548
    r = orc.route(np.array([0.5], np.float32), t1, 4, 2, 0.5, scale=1.0)
    assert list(r.selected[0]) == [0], list(r.selected[0])
    # the summary rule without offsets keeps chunk 1 (scores 0 and 0.5 tanh 10)
    m = orc.build_tree(K, np.array([[10.0]], np.float32), 2, scale=1.0)
    assert list(orc.route(np.array([0.5], np.float32), m, 4, 2, 0.5, scale=1.0).selected[0]) == [1]
    # two reference queries +-10: chunk 1 scores max(+-q tanh 10) + H = 0.5 + H at q = -0.5, so at p = 0.6
    # chunk 0 (mass 2 / (2 + e^0.5) = 0.548) no longer suffices; with q_hat = 10 alone chunk 1 scores
    # -0.5 + H and chunk 0 holds 2 / (2 + e^-0.5) = 0.767
    t2 = orc.build_tangent_tree(K, np.array([[[10.0], [-10.0]]], np.float32), 2, scale=1.0)
    assert list(orc.route(np.array([-0.5], np.float32), t2, 4, 2, 0.6, scale=1.0).selected[0]) == [0, 1]
    assert list(orc.route(np.array([-0.5], np.float32), t1, 4, 2, 0.6, scale=1.0).selected[0]) == [0]
    # a parent over the two chunks with q_hat = 0: logits are the children's offsets (ln 2, H), so
    # w = (2, e^H) / (2 + e^H), k_hat = tanh(10) e^H / (2 + e^H) and b_hat = ln(2 + e^H)
    t3 = orc.build_tangent_tree(K, np.array([[[10.0]], [[0.0]]], np.float32), 2, scale=1.0)
    eH = math.exp(H)
    assert abs(float(t3[1].keys[0, 0, 0]) - th * eH / (2 + eH)) < 1e-7
    assert abs(float(t3[1].offs[0, 0]) - math.log(2 + eH)) < 1e-7


def pin_tangent_level1(orc):
    """Level 1 against the definitions: b_hat is the entropy of the pooling weights
    (0 <= b_hat <= ln b); every tangent lies below the chunk's log-sum-exp F_C and
    touches it at its reference query (convexity); identical keys give the key
    itself with offset ln b, a tangent exact everywhere."""
    rng = np.random.default_rng(31)
    b, d, R = 8, 16, 3
    K = rng.standard_normal((20 * b, d)).astype(np.float32)
    refs = rng.standard_normal((1, R, d)).astype(np.float32)
    sc = 1 / math.sqrt(d)
    t = orc.build_tangent_tree(K, refs, b)[0]
    for i in range(20):
        C = K[i * b:(i + 1) * b].astype(np.float64)
        for r in range(R):
            z = sc * (C @ refs[0, r].astype(np.float64))
            assert abs(float(t.offs[i, r]) - _entropy(z)) < 1e-6
            assert -1e-6 <= float(t.offs[i, r]) <= math.log(b) + 1e-6
            tr = sc * float(t.keys[i, r].astype(np.float64) @ refs[0, r]) + float(t.offs[i, r])
            assert abs(tr - logsumexp(z)) < 2e-6
        for _ in range(5):
            q = rng.standard_normal(d) * 2
            F = logsumexp(sc * (C @ q))
            assert np.all(sc * (t.keys[i].astype(np.float64) @ q) + t.offs[i] <= F + 2e-6)
    same = np.repeat(K[:1], b, axis=0)
    ts = orc.build_tangent_tree(same, refs, b)[0]
    assert np.array_equal(ts.keys[0, 0], K[0]) and abs(float(ts.offs[0, 0]) - math.log(b)) < 1e-6


def pin_tangent_upper_levels(orc):
    """Levels above: every node's estimate max_r t_r(q) stays below the true
    log-sum-exp of the keys it spans (each level of lower bounds, combined by a
    monotone LSE); a parent's tangent touches the log-sum-exp of its children's
    estimates at its reference query, and its key is that function's gradient
    there (central differences, scale included)."""
    rng = np.random.default_rng(32)
    b, d, R, L = 4, 8, 3, 3
    K = (rng.standard_normal((b ** L * 2, d)) * 1.5).astype(np.float32)
    refs = rng.standard_normal((L, R, d)).astype(np.float32)
    sc = 1 / math.sqrt(d)
    tree = orc.build_tangent_tree(K, refs, b)
    Kd = K.astype(np.float64)
    for _ in range(6):
        q = rng.standard_normal(d) * 2
        for l in range(L):
            est = orc.tangent_logmass(q, tree[l], np.arange(len(tree[l])), sc)
            span = b ** (l + 1)
            true = np.array([logsumexp(sc * (Kd[i * span:(i + 1) * span] @ q)) for i in range(len(tree[l]))])
            assert np.all(est <= true + 1e-5), (l, (est - true).max())

    def children_lse(l, i, x):
        ch = tree[l - 1]
        idx = np.arange(i * b, (i + 1) * b)
        v = sc * (ch.keys[idx].astype(np.float64) @ x) + ch.offs[idx]
        return logsumexp(v.max(axis=1))

    for l in (1, 2):
        for i in range(len(tree[l])):
            for r in range(R):
                x0 = refs[l, r].astype(np.float64)
                tr = sc * float(tree[l].keys[i, r].astype(np.float64) @ x0) + float(tree[l].offs[i, r])
                assert abs(tr - children_lse(l, i, x0)) < 1e-5
                if tree[l].gap[i, r] < 1e-3:
                    continue                                    # a child's best tangent is near a switch
                eps = 1e-5
                g = np.array([(children_lse(l, i, x0 + eps * e) - children_lse(l, i, x0 - eps * e)) / (2 * eps)
                              for e in np.eye(d)])
                assert np.abs(g - sc * tree[l].keys[i, r].astype(np.float64)).max() < 1e-4


def pin_tangent_duplicate_refs(orc):
    """A repeated reference query adds a tangent equal to an existing one: the
    node estimates and the routing do not change."""
    rng = np.random.default_rng(33)
    b, d, L, N = 4, 8, 3, 200
    K = rng.standard_normal((N, d)).astype(np.float32)
    a = rng.standard_normal((L, 2, d)).astype(np.float32)
    dup = np.concatenate([a, a[:, :1]], axis=1)
    t1, t2 = orc.build_tangent_tree(K, a, b), orc.build_tangent_tree(K, dup, b)
    sc = 1 / math.sqrt(d)
    for _ in range(4):
        q = (rng.standard_normal(d) * 2).astype(np.float32)
        for l in range(L):
            ids = np.arange(len(t1[l]))
            # equal up to fp64 rounding (BLAS may round a repeated row differently by its position)
            assert np.abs(orc.tangent_logmass(q, t1[l], ids, sc) - orc.tangent_logmass(q, t2[l], ids, sc)).max() < 1e-12
        r1, r2 = orc.route(q, t1, N, b, 0.9), orc.route(q, t2, N, b, 0.9)
        assert all(np.array_equal(x, y) for x, y in zip(r1.selected, r2.selected))


def pin_tangent_route_golden(orc):
    """With zero reference queries every node's offset is the same at a level
    (l ln b: uniform weights all the way up), so the tangent tree routes the
    hand-worked cases exactly as the summary rule does."""
    for c in _load("route_closed_forms.json")["cases"]:
        K, R, q = _golden_inputs(c)
        if c["keys"] != "leafconst":
            continue
        tree = orc.build_tangent_tree(K, R[:, None, :], c["b"])
        r = orc.route(q, tree, c["N"], c["b"], c["p_levels"] if "p_levels" in c else c["p"])
        for lvl, rs in c["kept"].items():
            assert list(r.selected[int(lvl) - 1]) == list(_ranges(rs)), (c["name"], lvl)


# ----------------------------------------------------------------------------
# compressed value summaries: pruned subtrees as pseudo-tokens
# ----------------------------------------------------------------------------
def pin_value_summaries(orc):
    """A value summary pools the children's values with the key summary's
    weights: zero reference query -> the plain mean of the values; a huge
    reference query along e_0 -> the value of the child with the largest e_0
    key component; children permuted together -> the same summary."""
    rng = np.random.default_rng(41)
    b, d = 8, 16
    C = rng.standard_normal((b, d)).astype(np.float32)
    Y = rng.standard_normal((b, d)).astype(np.float32)
    sc = 1 / math.sqrt(d)
    v0 = orc.pool_values(C, Y, np.zeros(d, np.float32), b, sc)[0]
    assert np.abs(v0 - Y.astype(np.float64).mean(0)).max() < 1e-6
    r = np.zeros(d, np.float32)
    r[0] = 1e5
    assert np.abs(orc.pool_values(C, Y, r, b, sc)[0] - Y[np.argmax(C[:, 0])]).max() < 1e-6
    rr = rng.standard_normal(d).astype(np.float32)
    perm = rng.permutation(b)
    a1 = orc.pool_values(C, Y, rr, b, sc)[0]
    a2 = orc.pool_values(C[perm], Y[perm], rr, b, sc)[0]
    assert np.abs(a1.astype(np.float64) - a2).max() < 1e-6
    # values = keys: the value summary is the key summary
    K = rng.standard_normal((17 * b, d)).astype(np.float32)
    R = rng.standard_normal((2, d)).astype(np.float32)
    kt, vt = orc.build_tree(K, R, b), orc.build_value_tree(K, K, R, b)
    for x, y in zip(kt, vt):
        assert x.shape == y.shape and (x.size == 0 or np.abs(x.astype(np.float64) - y).max() < 1e-6)


def _uniform_spans(rng, b, L, N, d):
    """Keys and values constant over every span of b^L tokens: every subtree a
    cut can prune holds one repeated key and value."""
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    n_top = N // b ** L + 1
    a = rng.standard_normal(n_top) * 3
    vals = rng.standard_normal((n_top, d))
    t = np.arange(N) // b ** L
    return (a[t, None] * u[None, :]).astype(np.float32), vals[t].astype(np.float32)


def pin_compressed_exact_on_uniform_subtrees(orc):
    """Where every pruned subtree repeats one key and one value, the pseudo-token
    of a pruned node carries exactly its tokens' mass and value, so the output
    equals dense attention; this needs the right logit offset (the log of the
    node's tokens outside the sink and the current chunk), the right value and
    every pruned candidate of every level."""
    rng = np.random.default_rng(42)
    for b, L, N, d in [(4, 3, 64 * 5 + 3, 8), (4, 3, 64 * 5, 8), (2, 4, 80, 4), (8, 2, 64 * 3 + 7, 16)]:
        K, V = _uniform_spans(rng, b, L, N, d)
        R = rng.standard_normal((L, d)).astype(np.float32)
        tree, vals = orc.build_tree(K, R, b), orc.build_value_tree(K, V, R, b)
        pruned_total = 0
        for p in (0.3, 0.6, 0.9):
            for _ in range(3):
                q = (rng.standard_normal(d) * 3).astype(np.float32)
                r = orc.route(q, tree, N, b, p)
                I = orc.index_set(r.selected[0], N, b)
                lg, pv = orc.pseudo_tokens(r, vals, N, b)
                pruned_total += len(lg)
                o, l = orc.attend_compressed(q, K, V, I, lg, pv)
                od, ld = orc.dense_attend(q, K, V, N)
                assert np.abs(o - od).max() < 1e-9 and abs(l - ld) < 1e-9, (b, L, N, p, np.abs(o - od).max())
        assert pruned_total > 10


def pin_compressed_p1_and_sdpa(orc):
    """p = 1 prunes nothing: the compressed output is exact attention over I
    (= dense). For p < 1 the combination equals torch's SDPA in fp64 over the
    exact keys plus one zero key per pseudo-token whose logit enters as an
    additive mask, with the value summaries as its values."""
    rng = np.random.default_rng(43)
    b, L, N, d = 4, 3, 203, 8
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((L, d)).astype(np.float32)
    tree, vals = orc.build_tree(K, R, b), orc.build_value_tree(K, V, R, b)
    for _ in range(4):
        q = (rng.standard_normal(d) * 2).astype(np.float32)
        r = orc.route(q, tree, N, b, 1.0)
        lg, pv = orc.pseudo_tokens(r, vals, N, b)
        assert len(lg) == 0
        o, l = orc.attend_compressed(q, K, V, orc.index_set(r.selected[0], N, b), lg, pv)
        od, ld = orc.dense_attend(q, K, V, N)
        assert np.abs(o - od).max() < 1e-12 and abs(l - ld) < 1e-12
        r = orc.route(q, tree, N, b, 0.7)
        I = orc.index_set(r.selected[0], N, b)
        lg, pv = orc.pseudo_tokens(r, vals, N, b)
        assert len(lg) > 0
        o, _ = orc.attend_compressed(q, K, V, I, lg, pv)
        keys = np.concatenate([K[I].astype(np.float64), np.zeros((len(lg), d))])
        vv = np.concatenate([V[I].astype(np.float64), pv])
        bias = np.concatenate([np.zeros(len(I)), lg])
        qt = torch.from_numpy(q.astype(np.float64))[None, None, None, :]
        ref = F.scaled_dot_product_attention(qt, torch.from_numpy(keys)[None, None], torch.from_numpy(vv)[None, None],
                                             attn_mask=torch.from_numpy(bias)[None, None, None, :])[0, 0, 0].numpy()
        assert np.abs(o - ref).max() < 1e-12


ALL_PINS = [
    pin_geometry, pin_summary_sdpa, pin_summary_closed_forms, pin_incremental_equals_batch,
    pin_cut_golden, pin_cut_bruteforce, pin_cut_exemptions, pin_cut_uniform,
    pin_route_golden, pin_route_dense_mask, pin_causal_prefix,
    pin_attend_sdpa, pin_p1_dense, pin_eq1_identity, pin_split_merge,
    pin_tangent_golden, pin_tangent_level1, pin_tangent_upper_levels, pin_tangent_duplicate_refs,
    pin_tangent_route_golden,
    pin_value_summaries, pin_compressed_exact_on_uniform_subtrees, pin_compressed_p1_and_sdpa,
]
