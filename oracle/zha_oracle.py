"""CPU oracle for the Zyphra Hierarchical Attention (ZHA) decode path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
The product path (the HIP library and its Python binding) never touches it and
shares no code with it.

Plain, slow, obviously correct NumPy. Arithmetic is fp64 unless stated. Inputs
are fp32 arrays (bf16 caches are widened exactly before they get here).

Sources (cited by title and section; formulas are restated, not quoted):

* [SAHTI] "Subquadratic Attention with a Hierarchical Tree-Structured Indexer"
  (summary page of the technical report):
    - §Key Insight, eq. (1): top-p decomposition of attention.
    - §Tree Construction: chunk log-mass F_C, the reference-query summary
      k_hat_r = Attn(q_hat_r, K_C, K_C), recursion over children.
    - §Routing: the per-level cut m_l(q), the index set I(q), o(q).
* [ZHA-END] "Zyphra Hierarchical Attention: The End of Quadratic Attention?":
    - §How the tree is built and searched: contiguous chunks, recursive
      grouping, full KV kept at the leaves, top-p per level, token 0 kept as a
      sink.
    - §A query's path through the tree: level spans (4096/1024/.../4 for C4-L6).

Readings where the pages leave a step open (each restated where used):

* R-1 summary: a node's summary is the softmax(r_l . c / sqrt(d))-weighted mean
  of its children c (raw keys at level 1, child summaries above), one reference
  query r_l per (level, kv head); no tangent offset enters the score.
* R-2 score: s_i = q . x_i / sqrt(d); the cut runs on scores rounded to fp32
  (the precision fixed for scoring), masses exp(s - max) are fp64.
* R-3 cut: order by (score desc, node index asc); keep the smallest prefix whose
  cumulative mass is >= p times the candidates' total; p >= 1 keeps all.
* R-4 geometry: only complete nodes exist (node i of level l covers tokens
  [i b^l, (i+1) b^l) and exists once all of them are present). Complete nodes
  whose parent is not complete ("orphans") enter as candidates at their own
  level; at the top level every complete node is a candidate.
* R-5 current chunk: C_cur = [b floor((N-1)/b), N) for a query that sees N
  tokens (its own token included); token 0 is always attended; I(q) is a set.
* R-6 causal rows: a query at position t sees N = t + 1 tokens and only nodes
  complete within them.
* R-7 the full scoring rule (the tangent tree, an option beside R-1/R-2): each
  node keeps R tangents t_r(q) = q . k_hat_r / sqrt(d) + b_hat_r, one per
  reference query of its level, and scores max_r t_r(q). At level 1 the
  tangents are the page's: k_hat_r is the attention of q_hat_r over the chunk
  with the keys as values, b_hat_r = F_C(q_hat_r) - q_hat_r . k_hat_r / sqrt(d).
  Above, a node's log-mass is read as the log-sum-exp of its children's
  estimates, F(q) = LSE_j max_r' t_{j,r'}(q), and its tangents are the
  first-order expansion of that function at the level's reference queries: at
  q_hat_r each child enters with its best tangent there (lowest r' on ties),
  the logits z_j = t_{j,r*}(q_hat_r) include the child offsets, w =
  softmax(z), k_hat_r = sum_j w_j k_hat_{j,r*}, b_hat_r = LSE(z) - q_hat_r .
  k_hat_r / sqrt(d). Keys and offsets are stored in fp32.
* R-8 compressed value summaries (an option beside exact attention over I):
  a node also stores a value summary, its children's values (raw values at
  level 1) pooled with the weights of its key summary. After routing, every
  candidate a level's cut did not keep joins the attention as one
  pseudo-token: value its value summary, logit its routing score plus the log
  of the number of tokens it stands for, i.e. its span b^l less the tokens of
  it the exact part already attends (the sink and the current chunk), so no
  token is counted twice. The output is the softmax over the exact tokens of
  I and these pseudo-tokens. It is exact when every pruned subtree holds one
  repeated key and value, and it equals exact attention over I when nothing is
  pruned (p = 1).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

F64 = np.float64
F32 = np.float32


# ----------------------------------------------------------------------------
# Geometry [ZHA-END §How the tree is built and searched; SAHTI §Tree Construction]
# ----------------------------------------------------------------------------
def node_span(b: int, level: int) -> int:
    """Tokens covered by one node of ``level`` (level 1 = leaf chunk of b keys)."""
    return b ** level


def complete_nodes(n_tokens: int, b: int, n_levels: int) -> List[int]:
    """[n_1, ..., n_L]: complete nodes per level among the first ``n_tokens`` tokens (R-4)."""
    return [n_tokens // (b ** l) for l in range(1, n_levels + 1)]


# ----------------------------------------------------------------------------
# Tree build [SAHTI §Tree Construction: k_hat_r; recursion over children]
# ----------------------------------------------------------------------------
def pool_weights(children: np.ndarray, r: np.ndarray, b: int, scale: float):
    """softmax(scale * C r) over each group C of b consecutive children (R-1):
    returns the weights (m, b) and the groups (m, b, d), fp64."""
    X = np.asarray(children, dtype=F64)
    m = X.shape[0] // b
    X = X[: m * b].reshape(m, b, X.shape[-1])
    z = scale * (X @ np.asarray(r, dtype=F64))           # (m, b)
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    return w, X


def pool_children(children: np.ndarray, r: np.ndarray, b: int, scale: float) -> np.ndarray:
    """Summaries of consecutive groups of ``b`` rows of ``children`` (R-1).

    For each group C: weights w = softmax(scale * C r) and summary sum_j w_j C_j,
    i.e. single-query attention of r over C with C as both keys and values.
    Returned in fp32, the storage precision of summaries.
    """
    w, X = pool_weights(children, r, b, scale)
    s = np.einsum("mj,mjd->md", w, X)
    return s.astype(F32)


def pool_values(children: np.ndarray, child_values: np.ndarray, r: np.ndarray, b: int, scale: float) -> np.ndarray:
    """Value summaries of consecutive groups of b children (R-8): the children's
    values pooled with the weights of the key summary."""
    w, _ = pool_weights(children, r, b, scale)
    Y = np.asarray(child_values, dtype=F64)
    Y = Y[: w.shape[0] * b].reshape(w.shape[0], b, Y.shape[-1])
    return np.einsum("mj,mjd->md", w, Y).astype(F32)


def build_value_tree(K: np.ndarray, V: np.ndarray, R: np.ndarray, b: int, scale: Optional[float] = None,
                     slab: Optional[int] = None) -> List[np.ndarray]:
    """Every level's value summaries for one (sequence, kv head) (R-8), beside
    the key summaries of build_tree (whose weights they reuse)."""
    d = K.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    keys = build_tree(K, R, b, scale, slab)
    vals = []
    n1 = K.shape[0] // b
    step = n1 * b if slab is None else slab
    for l in range(R.shape[0]):
        if l == 0:
            parts = [pool_values(K[t0:min(t0 + step, n1 * b)], V[t0:min(t0 + step, n1 * b)], R[0], b, scale)
                     for t0 in range(0, n1 * b, max(step, 1))]
            vals.append(np.concatenate(parts) if parts else np.zeros((0, d), F32))
        else:
            vals.append(pool_values(keys[l - 1], vals[l - 1], R[l], b, scale))
    return vals


def build_tree(K: np.ndarray, R: np.ndarray, b: int, scale: Optional[float] = None,
               slab: Optional[int] = None) -> List[np.ndarray]:
    """All levels for one (sequence, kv head).

    K: (N, d) keys of the visible tokens. R: (L, d) reference queries of this kv
    head. Returns [X_1, ..., X_L] with X_l of shape (floor(N / b^l), d), fp32.
    With ``slab`` (a multiple of b), level 1 is pooled ``slab`` keys at a time,
    which bounds the fp64 copy of K for very long caches; a leaf never spans
    two slabs, so the nodes are the same.
    """
    d = K.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    levels = []
    if slab is None or R.shape[0] == 0:
        X = np.asarray(K, dtype=F64)
    else:
        assert slab % b == 0, "a slab must hold whole leaf chunks"
        n1 = K.shape[0] // b
        X = np.concatenate([pool_children(K[t0:min(t0 + slab, n1 * b)], R[0], b, scale)
                            for t0 in range(0, n1 * b, slab)] or [np.zeros((0, d), F32)])
        levels.append(X)
    for l in range(len(levels), R.shape[0]):
        X = pool_children(X, R[l], b, scale)
        levels.append(X)
    return levels


def build_tree_incremental(K: np.ndarray, R: np.ndarray, b: int, scale: Optional[float] = None) -> List[np.ndarray]:
    """Same tree, grown one appended token at a time [ZHA-END §A query's path: built on the fly].

    After token t arrives (N = t + 1 tokens), every node that N completes is
    summarised once from its children, lowest level first; nothing is ever
    rewritten.
    """
    d = K.shape[-1]
    L = R.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    levels: List[List[np.ndarray]] = [[] for _ in range(L)]
    for t in range(K.shape[0]):
        n = t + 1
        for l in range(1, L + 1):
            span = b ** l
            if n % span:
                break
            i = n // span - 1
            if l == 1:
                ch = np.asarray(K[i * b:(i + 1) * b], dtype=F64)
            else:
                ch = np.stack(levels[l - 2][i * b:(i + 1) * b]).astype(F64)
            levels[l - 1].append(pool_children(ch, R[l - 1], b, scale)[0])
    return [np.stack(v) if v else np.zeros((0, d), F32) for v in levels]


# ----------------------------------------------------------------------------
# The full scoring rule: R tangents per node [SAHTI §Tree Construction; R-7]
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class TangentLevel:
    """One level of a tangent tree (R-7)."""
    keys: np.ndarray     # (n, R, d) fp32: k_hat of each reference query
    offs: np.ndarray     # (n, R) fp32: b_hat
    gap: np.ndarray      # (n, R) fp64: smallest lead of a child's chosen tangent over its runner-up (inf at level 1)

    @property
    def shape(self):
        return self.keys.shape[:1] + self.keys.shape[2:]

    def __len__(self):
        return self.keys.shape[0]


def tangent_pool(child_keys: np.ndarray, child_offs: np.ndarray, refs: np.ndarray, b: int,
                 scale: float) -> TangentLevel:
    """Tangents of consecutive groups of b children, at reference queries refs (R, d).

    child_keys (n, Rc, d) and child_offs (n, Rc) are the children's tangents:
    raw keys with offset 0 at level 1 (Rc = 1). For reference query r, child j
    enters with its tangent of largest value at refs[r] (lowest index on ties):
    z_j = refs[r] . key * scale + off; w = softmax(z); k_hat = sum_j w_j key_j;
    b_hat = LSE(z) - refs[r] . k_hat * scale.
    """
    X = np.asarray(child_keys, dtype=F64)
    O = np.asarray(child_offs, dtype=F64)
    n, Rc, d = X.shape
    m = n // b
    X = X[:m * b].reshape(m, b, Rc, d)
    O = O[:m * b].reshape(m, b, Rc)
    R = refs.shape[0]
    keys = np.zeros((m, R, d), F32)
    offs = np.zeros((m, R), F32)
    gap = np.full((m, R), np.inf)
    for r in range(R):
        q = np.asarray(refs[r], dtype=F64)
        t = scale * (X @ q) + O                          # (m, b, Rc): every child tangent at refs[r]
        best = np.argmax(t, axis=2)                      # first maximum: lowest index on ties
        z = np.take_along_axis(t, best[..., None], axis=2)[..., 0]
        if Rc > 1:
            runner = np.sort(t, axis=2)[..., -2]
            gap[:, r] = (z - runner).min(axis=1) if m else gap[:, r]
        ksel = np.take_along_axis(X, best[..., None, None], axis=2)[:, :, 0, :]   # (m, b, d)
        zm = z.max(axis=1, keepdims=True)
        e = np.exp(z - zm)
        w = e / e.sum(axis=1, keepdims=True)
        kh = np.einsum("mj,mjd->md", w, ksel)
        lse = zm[:, 0] + np.log(e.sum(axis=1))
        keys[:, r] = kh.astype(F32)
        offs[:, r] = (lse - scale * (kh @ q)).astype(F32)
    return TangentLevel(keys, offs, gap)


def build_tangent_tree(K: np.ndarray, R: np.ndarray, b: int, scale: Optional[float] = None,
                       slab: Optional[int] = None) -> List[TangentLevel]:
    """Every level's tangents for one (sequence, kv head) (R-7).

    K: (N, d) keys. R: (L, R, d) reference queries of this kv head. With
    ``slab`` (a multiple of b), level 1 is pooled ``slab`` keys at a time."""
    d = K.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    L = R.shape[0]
    levels: List[TangentLevel] = []
    if L == 0:
        return levels
    n1 = K.shape[0] // b
    step = n1 * b if slab is None else slab
    assert step == 0 or step % b == 0, "a slab must hold whole leaf chunks"
    parts = []
    for t0 in range(0, n1 * b, max(step, 1)):
        Kc = np.asarray(K[t0:min(t0 + step, n1 * b)])
        parts.append(tangent_pool(Kc[:, None, :], np.zeros((Kc.shape[0], 1)), R[0], b, scale))
    if not parts:
        parts = [tangent_pool(np.zeros((0, 1, d)), np.zeros((0, 1)), R[0], b, scale)]
    levels.append(TangentLevel(np.concatenate([x.keys for x in parts]), np.concatenate([x.offs for x in parts]),
                               np.concatenate([x.gap for x in parts])))
    for l in range(1, L):
        up = levels[-1]
        levels.append(tangent_pool(up.keys, up.offs, R[l], b, scale))
    return levels


def tangent_logmass(q: np.ndarray, level: TangentLevel, ids: np.ndarray, scale: float) -> np.ndarray:
    """max_r t_r(q) of nodes ``ids``, fp64 (R-7)."""
    k = np.asarray(level.keys[ids], dtype=F64)            # (n, R, d)
    o = np.asarray(level.offs[ids], dtype=F64)            # (n, R)
    return (scale * (k @ np.asarray(q, dtype=F64)) + o).max(axis=1) if len(ids) else np.zeros(0)


# ----------------------------------------------------------------------------
# Top-p cut [SAHTI §Routing, m_l(q); R-3]
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class CutResult:
    ids: np.ndarray          # candidate node ids, as enumerated
    scores: np.ndarray       # decision scores (fp32 values held in fp64)
    scores64: np.ndarray     # exact fp64 scores (ties are judged on these)
    masses: np.ndarray       # normalised masses, fp64, aligned with ids
    order: np.ndarray        # positions into ids in (score desc, id asc) order
    prefix: np.ndarray       # prefix[k] = mass of the first k in order (prefix[0] = 0)
    m: int                   # number kept
    selected: np.ndarray     # kept ids, ascending


def topp_cut(ids: np.ndarray, scores: np.ndarray, p: float, scores64: Optional[np.ndarray] = None) -> CutResult:
    """Smallest (score desc, id asc)-prefix holding at least fraction p of the mass."""
    ids = np.asarray(ids, dtype=np.int64)
    s = np.asarray(scores, dtype=F64)
    s64 = s if scores64 is None else np.asarray(scores64, dtype=F64)
    n = len(ids)
    if n == 0:
        z = np.zeros(0)
        return CutResult(ids, s, s64, z, np.zeros(0, np.int64), np.zeros(1), 0, ids.copy())
    order = np.lexsort((ids, -s))
    e = np.exp(s - s.max())
    E = e.sum()
    masses = e / E
    c = np.cumsum(e[order])
    prefix = np.concatenate([[0.0], np.cumsum(masses[order])])
    if p >= 1.0:
        m = n
    else:
        hit = np.nonzero(c >= p * E)[0]
        m = int(hit[0]) + 1 if len(hit) else n
    sel = np.sort(ids[order[:m]])
    return CutResult(ids, s, s64, masses, order, prefix, m, sel)


def cut_exemptions(cut: CutResult, p: float, margin: float = 1e-5) -> np.ndarray:
    """Ids whose membership may legitimately differ from this cut at precision ``margin``.

    A candidate at sorted rank k is exempt when (i) the mass before it is within
    ``margin`` of p (its inclusion hinges on less than ``margin`` of mass), or
    (ii) a candidate on the other side of the cut has a different exact score and
    a mass within ``margin`` of its own (the two could swap places). Exact ties
    are never exempt: the index rule decides them.
    """
    n = len(cut.ids)
    if n == 0 or p >= 1.0:
        return np.zeros(0, np.int64)
    ex = set()
    for k in range(n):
        if abs(cut.prefix[k] - p) < margin:
            ex.add(int(cut.ids[cut.order[k]]))
    inside = cut.order[: cut.m]
    outside = cut.order[cut.m:]
    if len(inside) and len(outside):
        wi, wo = cut.masses[inside], cut.masses[outside]
        si, so = cut.scores64[inside], cut.scores64[outside]
        # only the candidates nearest the boundary can be within margin of the other side
        lo_in = wi.min()
        hi_out = wo.max()
        cand_in = inside[wi < hi_out + margin]
        cand_out = outside[wo > lo_in - margin]
        for x in cand_in:
            close = np.abs(cut.masses[cand_out] - cut.masses[x]) < margin
            diff = cut.scores64[cand_out] != cut.scores64[x]
            if np.any(close & diff):
                ex.add(int(cut.ids[x]))
                for y in cand_out[close & diff]:
                    ex.add(int(cut.ids[y]))
    return np.array(sorted(ex), dtype=np.int64)


# ----------------------------------------------------------------------------
# Routing [SAHTI §Routing; ZHA-END §How the tree is built and searched; R-4]
# ----------------------------------------------------------------------------
def level_candidates(level: int, parents: Optional[np.ndarray], n_visible: int, b: int, n_levels: int) -> np.ndarray:
    """Candidates at ``level``: children of the kept parents, then the level's orphans.

    ``parents`` are kept ids at level + 1 (ignored at the top level). Orphans are
    the complete nodes [b * nc_{l+1}, nc_l) whose parent is not complete; at the
    top level nc_{L+1} = 0 so every complete node is a candidate.
    """
    nc = complete_nodes(n_visible, b, n_levels) + [0]
    out = []
    if level < n_levels and parents is not None:
        for pnode in np.sort(np.asarray(parents, dtype=np.int64)):
            out.append(np.arange(pnode * b, pnode * b + b, dtype=np.int64))
    lo = b * nc[level] if level < n_levels else 0
    out.append(np.arange(lo, nc[level - 1], dtype=np.int64))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def score_nodes(q: np.ndarray, X, ids: np.ndarray, scale: float):
    """(fp32-rounded scores, exact fp64 scores) of nodes ``ids`` of one level:
    q . x / sqrt(d) (R-2), or max_r t_r(q) for a tangent level (R-7)."""
    if isinstance(X, TangentLevel):
        s64 = tangent_logmass(q, X, ids, scale)
    else:
        s64 = scale * (np.asarray(X[ids], dtype=F64) @ np.asarray(q, dtype=F64))
    return s64.astype(F32).astype(F64), s64


@dataclasses.dataclass
class RouteResult:
    levels: List[CutResult]          # levels[l - 1] is level l
    selected: List[np.ndarray]       # selected[l - 1]: kept ids at level l (ascending)


def route_level(q, X_level, level, parents, n_visible, b, n_levels, p, scale, score_dtype=F32) -> CutResult:
    ids = level_candidates(level, parents, n_visible, b, n_levels)
    if len(ids) == 0:
        return topp_cut(ids, np.zeros(0), p)
    s, s64 = score_nodes(q, X_level, ids, scale)
    if score_dtype == F64:
        s = s64
    return topp_cut(ids, s, p, s64)


def level_fraction(p, level: int) -> float:
    """The cut fraction at ``level``: p itself, or p[level - 1] for a per-level
    schedule [SAHTI §Future Directions: scaling p with depth]."""
    return float(p) if np.ndim(p) == 0 else float(p[level - 1])


def route(q: np.ndarray, tree: Sequence[np.ndarray], n_visible: int, b: int, p,
          scale: Optional[float] = None, score_dtype=F32) -> RouteResult:
    """Top-down routing of one query through one (sequence, kv head) tree.

    ``p`` is one fraction for every level or a schedule [p_1, ..., p_L]."""
    L = len(tree)
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    cuts: List[Optional[CutResult]] = [None] * L
    parents = None
    for level in range(L, 0, -1):
        c = route_level(q, tree[level - 1], level, parents, n_visible, b, L, level_fraction(p, level), scale,
                        score_dtype)
        cuts[level - 1] = c
        parents = c.selected
    return RouteResult(cuts, [c.selected for c in cuts])


def index_set(leaf_ids: np.ndarray, n_visible: int, b: int) -> np.ndarray:
    """I(q) = {0} U (union of kept leaf chunks) U C_cur, ascending token ids (R-5)."""
    if n_visible <= 0:
        return np.zeros(0, np.int64)
    toks = np.zeros(n_visible, dtype=bool)
    toks[0] = True
    for i in np.asarray(leaf_ids, dtype=np.int64):
        toks[i * b:(i + 1) * b] = True
    toks[b * ((n_visible - 1) // b):n_visible] = True
    return np.nonzero(toks)[0]


# ----------------------------------------------------------------------------
# Attention [SAHTI §Routing, o(q); §The Quadratic Bottleneck (dense decode)]
# ----------------------------------------------------------------------------
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray, scale: Optional[float] = None):
    """Exact softmax attention of q over tokens ``idx``: returns (o (d,), lse)."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    idx = np.asarray(idx, dtype=np.int64)
    k = np.asarray(K[idx], dtype=F64)
    v = np.asarray(V[idx], dtype=F64)
    z = scale * (k @ np.asarray(q, dtype=F64))
    mx = z.max()
    e = np.exp(z - mx)
    l = e.sum()
    return (e @ v) / l, mx + math.log(l)


def dense_attend(q, K, V, n_visible, scale=None):
    return attend(q, K, V, np.arange(n_visible), scale)


def pseudo_tokens(route_res: "RouteResult", values: Sequence[np.ndarray], n_visible: int, b: int):
    """The pruned candidates of every level as (logit, value summary) pairs (R-8):
    logit = routing score (exact fp64) + ln(the node's tokens outside the sink
    and the current chunk); nodes with no such token are left out."""
    cur = b * ((n_visible - 1) // b) if n_visible > 0 else 0
    logits, vals = [], []
    for level, cut in enumerate(route_res.levels, start=1):
        if cut is None or len(cut.ids) == 0:
            continue
        kept = set(int(x) for x in cut.selected)
        span = b ** level
        for j, node in enumerate(cut.ids):
            node = int(node)
            if node in kept:
                continue
            lo, hi = node * span, (node + 1) * span
            count = span - (1 if lo == 0 else 0) - max(0, min(n_visible, hi) - max(cur, lo))
            if lo == 0 and cur == 0:
                count += 1                              # the sink lies in the current chunk: counted once
            if count <= 0:
                continue
            logits.append(float(cut.scores64[j]) + math.log(count))
            vals.append(np.asarray(values[level - 1][node], dtype=F64))
    return np.array(logits, dtype=F64), (np.stack(vals) if vals else np.zeros((0, 0)))


def attend_compressed(q, K, V, idx, logits, pvals, scale=None):
    """Softmax attention over the exact tokens idx and the pseudo-tokens (logit,
    value) of the pruned subtrees (R-8): returns (o (d,), lse)."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    idx = np.asarray(idx, dtype=np.int64)
    z = scale * (np.asarray(K[idx], dtype=F64) @ np.asarray(q, dtype=F64))
    vv = np.asarray(V[idx], dtype=F64)
    if len(logits):
        z = np.concatenate([z, logits])
        vv = np.concatenate([vv, pvals])
    mx = z.max()
    e = np.exp(z - mx)
    l = e.sum()
    return (e @ vv) / l, mx + math.log(l)


# ----------------------------------------------------------------------------
# Diagnostics (not parity) [SAHTI §Key Insight, eq. (1)]
# ----------------------------------------------------------------------------
def key_probs(q, K, n_visible, scale=None) -> np.ndarray:
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    z = scale * (np.asarray(K[:n_visible], dtype=F64) @ np.asarray(q, dtype=F64))
    e = np.exp(z - z.max())
    return e / e.sum()


def topp_key_set(q, K, n_visible, p, scale=None) -> np.ndarray:
    """Exact key-level top-p set K_p: smallest set of keys with probability >= p."""
    pr = key_probs(q, K, n_visible, scale)
    order = np.lexsort((np.arange(n_visible), -pr))
    c = np.cumsum(pr[order])
    m = int(np.nonzero(c >= p)[0][0]) + 1 if p < 1 else n_visible
    return np.sort(order[:m])


def realised_mass(q, K, n_visible, idx, scale=None) -> float:
    return float(key_probs(q, K, n_visible, scale)[np.asarray(idx, dtype=np.int64)].sum())


# ----------------------------------------------------------------------------
# Whole-batch helpers (GQA: query head h uses kv head h // (H_q / H_kv))
# ----------------------------------------------------------------------------
def build_all(K: np.ndarray, R: np.ndarray, seq_lens: Sequence[int], b: int, scale=None, slab=None):
    """trees[s][h] for K [B, H_kv, N_cap, d] (fp32 values) and R [L, H_kv, d]."""
    B, H = K.shape[:2]
    return [[build_tree(K[s, h, :int(seq_lens[s])], R[:, h], b, scale, slab) for h in range(H)] for s in range(B)]
