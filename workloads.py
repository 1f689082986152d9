"""Seeded synthetic inputs for the ZHA decode path.

This module only draws random numbers and lays them out. It holds none of
the method's arithmetic (no summaries, scores, softmax or selection), so both
the CPU oracle (through the tests) and the HIP path (through the tests and the
benchmark) can consume the very same bits.

Five workloads are defined, each reproducing the shapes, value distributions
and structure named for it:

* ``tiny``      4096 fp32 keys, one head, d=64, b=16, three levels, eight
                planted needle keys, queries built from pairs of needles.
* ``gqa128k``   batch 8, 32 query / 8 kv heads, d=128, bf16, 131072 tokens,
                b=16, 64 clusters of 32 adjacent tokens per sequence.
* ``decode1m``  batch 1, 32/8 heads, d=128, bf16, 1048576 tokens, b=32,
                power-law cluster layout (count grows as sqrt(N), Zipf(1.2)
                sizes), one appended token per decode step.
* ``prefill256k`` a 262144-token cache with the ``gqa128k`` layout plus an
                8192-token chunk processed causally.
* ``decode16m`` batch 1, 8/1 heads, d=128, bf16, 16777216 tokens, b=32, the
                power-law layout of ``decode1m``.

Conventions (stated once, used everywhere):
* N(mu, s) means a normal law with standard deviation s.
* Every tensor draws from its own ``SeedSequence(seed, spawn_key=...)`` so that
  chunked generation is deterministic and independent of chunk order.
* bf16 values are produced from fp32 by round-to-nearest-even and kept as raw
  ``uint16`` bit patterns; :func:`bf16_bits_to_f32` widens them exactly.
* Layouts: K, V ``[B, H_kv, N_cap, d]``; reference queries ``[L, H_kv, d]``
  fp32; queries ``[B, T, H_q, d]`` fp32; positions ``[B, T]`` int32.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

# Token chunk used when drawing K/V so that huge caches can be produced piecewise
# with results independent of how the caller slices them.
_GEN_CHUNK = 1 << 16

_TAG_K, _TAG_V, _TAG_R, _TAG_LAYOUT, _TAG_DIR, _TAG_Q, _TAG_APPEND = range(7)


# ----------------------------------------------------------------------------
# bf16 helpers (input representation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))))


# ----------------------------------------------------------------------------
# Workload description
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    branching: int
    n_levels: int
    top_p: float
    kv_dtype: str            # "bf16" or "fp32"
    n_tokens: int            # initial cache length per sequence
    capacity: int            # allocated tokens per sequence (>= n_tokens + appended)
    steps: int               # decode steps (or 1 for the prefill chunk)
    append_per_step: int     # tokens appended before each decode step (0 = fixed cache)
    queries_per_step: int    # T: query rows per sequence per step
    # cluster layout per sequence: list of (start, length) arrays
    cluster_mode: str        # "needles", "uniform", "powerlaw"
    n_clusters: int
    cluster_len: int         # for "uniform"
    prefill_chunk: int = 0   # >0: causal chunk appended and queried at once
    description: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _base(name: str) -> Workload:
    if name == "tiny":
        return Workload("tiny", 1, 1, 1, 1, 64, 16, 3, 0.9, "fp32", 4096, 4096, 1, 0, 16,
                        "needles", 8, 1,
                        description="4096 fp32 keys, 1 head, d=64, b=16, L=3, p=0.9, 8 needles, 16 queries")
    if name == "gqa128k":
        return Workload("gqa128k", 2, 8, 32, 8, 128, 16, 4, 0.95, "bf16", 131072, 131072, 16, 0, 1,
                        "uniform", 64, 32,
                        description="batch 8, 32/8 heads, d=128, bf16, 131072 tokens, b=16, L=4, p=0.95")
    if name == "decode1m":
        n = 1 << 20
        return Workload("decode1m", 3, 1, 32, 8, 128, 32, 4, 0.95, "bf16", n, n + 256, 256, 1, 1,
                        "powerlaw", int(round(64 * math.sqrt(n / 131072))), 0,
                        description="batch 1, 32/8 heads, d=128, bf16, 1048576 tokens, b=32, L=4, p=0.95, "
                                    "256 steps with one appended token each")
    if name == "prefill256k":
        n = 1 << 18
        return Workload("prefill256k", 4, 1, 32, 8, 128, 16, 4, 0.9, "bf16", n, n + 8192, 1, 0, 8192,
                        "uniform", 64, 32, prefill_chunk=8192,
                        description="262144-token cache + 8192-token causal chunk, 32/8 heads, d=128, bf16, "
                                    "b=16, L=4, p=0.9")
    if name == "decode16m":
        n = 1 << 24
        return Workload("decode16m", 5, 1, 8, 1, 128, 32, 5, 0.95, "bf16", n, n, 64, 0, 1,
                        "powerlaw", int(round(64 * math.sqrt(n / 131072))), 0,
                        description="batch 1, 8/1 heads, d=128, bf16, 16777216 tokens, b=32, L=5, p=0.95, "
                                    "64 steps on a fixed cache")
    raise KeyError(name)


WORKLOAD_NAMES = ("tiny", "gqa128k", "decode1m", "prefill256k", "decode16m")


def get_workload(name: str, shrink: int = 0, batch: Optional[int] = None,
                 steps: Optional[int] = None, chunk: Optional[int] = None) -> Workload:
    """Return a workload, optionally shrunk by ``branching**shrink`` tokens and ``shrink`` levels.

    Shrinking keeps b, the heads, d and the value distributions; the cluster
    count scales as the full workload's rule prescribes for the smaller N.
    """
    w = _base(name)
    if shrink:
        f = w.branching ** shrink
        n = max(w.n_tokens // f, w.branching)
        extra = w.capacity - w.n_tokens
        w.n_tokens = n
        w.n_levels = max(1, w.n_levels - shrink)
        if w.cluster_mode == "powerlaw":
            w.n_clusters = max(1, int(round(64 * math.sqrt(n / 131072))))
        elif w.cluster_mode == "uniform":
            w.n_clusters = max(1, min(w.n_clusters, n // (4 * w.cluster_len)))
        if w.prefill_chunk:
            w.prefill_chunk = max(w.branching, w.prefill_chunk // f)
            w.queries_per_step = w.prefill_chunk
            extra = w.prefill_chunk
        w.capacity = n + extra
        w.name = f"{name}/shrink{shrink}"
    if batch is not None:
        w.batch = batch
    if steps is not None:
        w.steps = steps
        if w.append_per_step:
            w.capacity = w.n_tokens + steps * w.append_per_step
    if chunk is not None and w.prefill_chunk:
        w.prefill_chunk = chunk
        w.queries_per_step = chunk
        w.capacity = w.n_tokens + chunk
    return w


# ----------------------------------------------------------------------------
# Cluster layout
# ----------------------------------------------------------------------------
def _place_nonoverlapping(rng: np.random.Generator, lengths: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Uniform start positions in [lo, hi - len) such that no two clusters overlap."""
    starts = np.empty(len(lengths), dtype=np.int64)
    taken: List[Tuple[int, int]] = []
    for i, ln in enumerate(lengths):
        for _attempt in range(10000):
            s = int(rng.integers(lo, max(lo + 1, hi - int(ln))))
            e = s + int(ln)
            if all(e <= a or s >= b for a, b in taken):
                break
        else:  # pragma: no cover - only reachable with absurd densities
            raise RuntimeError("could not place clusters without overlap")
        taken.append((s, e))
        starts[i] = s
    return starts


def cluster_layout(w: Workload, seq: int) -> Tuple[np.ndarray, np.ndarray]:
    """(starts, lengths) of the planted clusters of sequence ``seq`` (shared by its kv heads)."""
    rng = _rng(w.seed, _TAG_LAYOUT, seq)
    n = w.n_tokens
    if w.cluster_mode == "needles":
        pos = rng.choice(np.arange(1, n), size=w.n_clusters, replace=False)
        return np.sort(pos).astype(np.int64), np.ones(w.n_clusters, dtype=np.int64)
    if w.cluster_mode == "uniform":
        lengths = np.full(w.n_clusters, w.cluster_len, dtype=np.int64)
    else:
        lengths = np.clip(rng.zipf(1.2, size=w.n_clusters), 1, 4096).astype(np.int64)
        # never let the clusters crowd more than half the cache
        while lengths.sum() > n // 2:
            lengths = np.maximum(1, lengths // 2)
    starts = _place_nonoverlapping(rng, lengths, 1, n)
    order = np.argsort(starts)
    return starts[order], lengths[order]


def cluster_directions(w: Workload, seq: int, kv: int) -> np.ndarray:
    """Cluster directions u ~ N(0, I_d), one per cluster, for (sequence, kv head)."""
    rng = _rng(w.seed, _TAG_DIR, seq, kv)
    return rng.standard_normal((w.n_clusters, w.head_dim), dtype=np.float32)


# ----------------------------------------------------------------------------
# K / V / reference queries
# ----------------------------------------------------------------------------
def _background_chunk(w: Workload, tag: int, seq: int, kv: int, c0: int, c1: int) -> np.ndarray:
    """fp32 background draws for tokens [c0, c1) of (seq, kv); chunk-order independent."""
    out = np.empty((c1 - c0, w.head_dim), dtype=np.float32)
    k = c0 // _GEN_CHUNK
    pos = c0
    while pos < c1:
        g0 = k * _GEN_CHUNK
        g1 = g0 + _GEN_CHUNK
        rng = _rng(w.seed, tag, seq, kv, k)
        block = rng.standard_normal((_GEN_CHUNK, w.head_dim), dtype=np.float32)
        a, b = max(pos, g0), min(c1, g1)
        out[a - c0:b - c0] = block[a - g0:b - g0]
        pos = b
        k += 1
    return out


def keys_f32(w: Workload, seq: int, kv: int, t0: int = 0, t1: Optional[int] = None,
             layout=None) -> np.ndarray:
    """fp32 keys of tokens [t0, t1) for (seq, kv), before any bf16 rounding."""
    t1 = w.n_tokens if t1 is None else t1
    k = _background_chunk(w, _TAG_K, seq, kv, t0, t1)
    if w.cluster_mode == "needles":
        k *= np.float32(1.0 / math.sqrt(w.head_dim))       # N(0,1)/sqrt(d); needles are plain keys
        return k
    starts, lengths = cluster_layout(w, seq) if layout is None else layout
    dirs = cluster_directions(w, seq, kv)
    for ci, (s, ln) in enumerate(zip(starts, lengths)):
        a, b = max(s, t0), min(s + ln, t1)
        if a < b:
            # cluster key = direction + N(0, 0.2): reuse the background draw as the noise
            k[a - t0:b - t0] = dirs[ci] + np.float32(0.2) * k[a - t0:b - t0]
    return k


def values_f32(w: Workload, seq: int, kv: int, t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    t1 = w.n_tokens if t1 is None else t1
    return _background_chunk(w, _TAG_V, seq, kv, t0, t1)


def _to_kv_dtype(w: Workload, x: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x) if w.kv_dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def kv_chunk(w: Workload, seq: int, kv: int, t0: int, t1: int, layout=None) -> Tuple[np.ndarray, np.ndarray]:
    """K and V rows [t0, t1) in the storage dtype (uint16 bf16 bits or fp32)."""
    return (_to_kv_dtype(w, keys_f32(w, seq, kv, t0, t1, layout)),
            _to_kv_dtype(w, values_f32(w, seq, kv, t0, t1)))


def host_threads() -> int:
    """Threads for host-side generation: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def kv_cache(w: Workload, threads: Optional[int] = None, slab: int = 1 << 20) -> Tuple[np.ndarray, np.ndarray]:
    """Whole initial cache [B, H_kv, capacity, d]; rows past n_tokens are zero.

    Slabs of ``slab`` tokens of every (sequence, kv head) are drawn on a thread
    pool (NumPy's generators release the GIL); each slab seeds its own streams,
    so the bits do not depend on the slab size or the thread count.
    """
    dt = np.uint16 if w.kv_dtype == "bf16" else np.float32
    K = np.zeros((w.batch, w.n_kv_heads, w.capacity, w.head_dim), dtype=dt)
    V = np.zeros_like(K)
    lays = [cluster_layout(w, s) if w.cluster_mode != "needles" else None for s in range(w.batch)]
    tasks = [(s, h, t0, min(t0 + slab, w.n_tokens)) for s in range(w.batch) for h in range(w.n_kv_heads)
             for t0 in range(0, w.n_tokens, slab)]

    def fill(task):
        s, h, t0, t1 = task
        K[s, h, t0:t1], V[s, h, t0:t1] = kv_chunk(w, s, h, t0, t1, lays[s])

    n = host_threads() if threads is None else max(1, threads)
    if n == 1 or len(tasks) == 1:
        for task in tasks:
            fill(task)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(fill, tasks))
    return K, V


def as_f32(w: Workload, x: np.ndarray) -> np.ndarray:
    """Storage-dtype array -> fp32 values (exact widening for bf16)."""
    return bf16_bits_to_f32(x) if w.kv_dtype == "bf16" else np.asarray(x, dtype=np.float32)


def ref_queries(w: Workload, n_refs: Optional[int] = None) -> np.ndarray:
    """Per-level, per-kv-head reference queries: [L, H_kv, d] fp32, or with
    ``n_refs`` = R, [L, H_kv, R, d] whose first query of each (level, kv head)
    is the one drawn without n_refs (the others from a stream of their own)."""
    rng = _rng(w.seed, _TAG_R)
    r = rng.standard_normal((w.n_levels, w.n_kv_heads, w.head_dim), dtype=np.float32)
    if n_refs is not None:
        more = _rng(w.seed, _TAG_R, 1).standard_normal((w.n_levels, w.n_kv_heads, max(0, n_refs - 1), w.head_dim),
                                                       dtype=np.float32)
        r = np.concatenate([r[:, :, None, :], more], axis=2)
    if w.cluster_mode == "needles":
        r *= np.float32(1.0 / math.sqrt(w.head_dim))
    return r


# ----------------------------------------------------------------------------
# Queries and appended tokens
# ----------------------------------------------------------------------------
def queries(w: Workload, step: int, rows: Optional[int] = None, row0: int = 0) -> np.ndarray:
    """Query rows for one step: [B, T, H_q, d] fp32 (T = rows or queries_per_step)."""
    T = w.queries_per_step if rows is None else rows
    out = np.empty((w.batch, T, w.n_q_heads, w.head_dim), dtype=np.float32)
    for s in range(w.batch):
        if w.cluster_mode == "needles":
            starts, _ = cluster_layout(w, s)
            keys = keys_f32(w, s, 0, 0, w.n_tokens)
            kv_vals = as_f32(w, _to_kv_dtype(w, keys))
            for t in range(T):
                rng = _rng(w.seed, _TAG_Q, step, s, row0 + t)
                a, b = rng.choice(len(starts), size=2, replace=False)
                noise = rng.standard_normal(w.head_dim).astype(np.float32) * np.float32(0.1)
                q = np.float32(3.0) * (kv_vals[starts[a]] + kv_vals[starts[b]]) + noise
                out[s, t, :] = q
            continue
        dirs = [cluster_directions(w, s, h) for h in range(w.n_kv_heads)]
        for t in range(T):
            rng = _rng(w.seed, _TAG_Q, step, s, row0 + t)
            for hq in range(w.n_q_heads):
                kv = hq // w.group
                j = int(rng.integers(1, 5))
                pick = rng.choice(w.n_clusters, size=min(j, w.n_clusters), replace=False)
                q = np.float32(4.0) * dirs[kv][pick].sum(axis=0)
                q = q + rng.standard_normal(w.head_dim).astype(np.float32)
                out[s, t, hq] = q
    return out


def appended_tokens(w: Workload, step: int, count: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Background tokens appended before a step: K, V [B, H_kv, count, d] in storage dtype."""
    n = (w.append_per_step if count is None else count)
    rng = _rng(w.seed, _TAG_APPEND, step)
    k = rng.standard_normal((w.batch, w.n_kv_heads, n, w.head_dim), dtype=np.float32)
    v = rng.standard_normal((w.batch, w.n_kv_heads, n, w.head_dim), dtype=np.float32)
    return _to_kv_dtype(w, k), _to_kv_dtype(w, v)


def prefill_chunk_kv(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """The causal chunk's new K/V rows [B, H_kv, chunk, d] (background distribution)."""
    return appended_tokens(w, 0, w.prefill_chunk)


def seq_lens(w: Workload) -> np.ndarray:
    return np.full(w.batch, w.n_tokens, dtype=np.int32)


def summary(w: Workload) -> Dict[str, object]:
    d = dataclasses.asdict(w)
    d["group"] = w.group
    return d
