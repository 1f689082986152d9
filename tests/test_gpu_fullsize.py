"""Parity of the HIP path with the CPU oracle at the workloads' full sizes, in the
launch configuration the benchmark times (one query row per sequence, the
timed step's calls).

* decode1m: 1,048,576 bf16 tokens, 32/8 heads, b = 32, L = 4. Every level of
  the tree against the oracle's own tree built from the host keys; then decode
  steps (append one token per kv head, route, attend), each checked
  teacher-forced for all 32 heads, with the appended rows against the host
  tokens and the attention against the oracle over the GPU's index set.
* decode16m: 16,777,216 bf16 tokens (4 GiB of K and 4 GiB of V, so K/V byte
  offsets pass 2^32), one kv head, 8 query heads, b = 32, L = 5 (a 524,288-node
  leaf level cut over 256 slices). The oracle pools level 1 in slabs. Two decode
  steps on the fixed cache; the dense kernel on two heads against the oracle's
  dense attention merged from per-slab partial results (the LSE merge is exact,
  see the oracle's split-and-merge pin).
* gqa128k at batch 8: 131,072 tokens per sequence, 256 (row, head) pairs, so
  the per-pair cut kernel runs with thousands of candidates; checked on a
  sample of (sequence, head) pairs.

Bars as in test_gpu_parity: summaries within the fp32 accumulation bound, kept
sets equal up to the 1e-5 margin exemptions with exact candidate counts,
attention within 2e-4 max-abs (bf16 KV).
"""
import math

import numpy as np
import pytest

import hierarchical_tree_indexed_build_amd as Z
import workloads as W
from oracle import zha_oracle as O
from tests.gpu_helpers import (Staged, attn_tol, check_attention, check_tree, kv_tensor, say, teacher_forced,
                               torch)

pytestmark = pytest.mark.gpu


def _decode_steps(st, steps, append, pairs=None, check=True):
    """Run `steps` decode steps through zha_append + zha_attend (the timed step),
    checking each one; returns the per-step level_stats."""
    t = torch()
    w = st.w
    trees = st.oracle_trees(slab=1 << 20)
    worst = check_tree(st, trees, w.n_tokens, pairs=None if pairs is None else
                       sorted({(s, h // w.group) for s, h in pairs}))
    say(f"  tree parity: worst error {worst:.3g} of the bound")
    n = w.n_tokens
    out_stats = []
    for step in range(steps):
        if append:
            kn, vn = W.appended_tokens(w, step)
            Z.append(st.geom, st.cache.K, st.cache.V, kv_tensor(w, kn), kv_tensor(w, vn), st.cache.seq_lens,
                     st.ref_q, st.cache.summaries, st.cache.ws)
            st.K_np[:, :, n:n + 1], st.V_np[:, :, n:n + 1] = kn, vn
            st.Kf[:, :, n:n + 1], st.Vf[:, :, n:n + 1] = W.as_f32(w, kn), W.as_f32(w, vn)
            n += 1
            for s in range(w.batch):
                for h in range(w.n_kv_heads):
                    # a leaf (and above) completes when n is a multiple of b: extend the oracle's tree
                    for level in range(1, w.n_levels + 1):
                        span = w.branching ** level
                        if n % span:
                            break
                        i = n // span - 1
                        ch = st.Kf[s, h, i * w.branching:(i + 1) * w.branching] if level == 1 else \
                            trees[s][h][level - 2][i * w.branching:(i + 1) * w.branching]
                        node = O.pool_children(ch, st.R[level - 1, h], w.branching, w.scale)
                        trees[s][h][level - 1] = np.concatenate([trees[s][h][level - 1], node])
        qn, q = st.queries(step)
        sel, nsel, stats, lsel = st.route_buffers(w.batch)
        out = t.zeros_like(q)
        lse = t.zeros(q.shape[:3], dtype=t.float32, device="cuda")
        Z.attend(st.geom, q, None, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, w.top_p, sel,
                 nsel, out, lse, st.cache.ws, level_stats=stats, level_sel=lsel)
        t.cuda.synchronize()
        assert Z.read_device_status(st.cache.ws) == 0
        assert np.all(st.cache.seq_lens.cpu().numpy() == n)
        if append:
            got = st.cache.K.view(t.uint16)[:, :, n - 1].cpu().numpy()
            assert np.array_equal(got, st.K_np[:, :, n - 1]), "appended K row"
            got = st.cache.V.view(t.uint16)[:, :, n - 1].cpu().numpy()
            assert np.array_equal(got, st.V_np[:, :, n - 1]), "appended V row"
        qpos = np.full((w.batch, 1), n - 1, dtype=np.int64)
        if check:
            flips = teacher_forced(st, qn, qpos, stats, lsel, w.top_p, trees, pairs=pairs)
            worst = check_attention(st, qn, qpos, out, lse, sel, nsel, pairs=pairs)
            st_np = stats.cpu().numpy()
            say(f"  step {step}: N={n}, exempt differences {flips}, worst attention error {worst:.3g}, "
                f"level-1 candidates {int(st_np[..., 0, 0].max())} max, kept leaves {int(nsel.max().item())} max")
        out_stats.append(stats.cpu().numpy())
    return out_stats


def test_decode1m_full_size():
    w = W.get_workload("decode1m", steps=3)
    say(f"[full] decode1m: N={w.n_tokens}, capacity {w.capacity}")
    st = Staged(w)
    say("  staged and built")
    _decode_steps(st, 3, append=True)


def test_gqa128k_batch8_full_size():
    w = W.get_workload("gqa128k")
    assert w.batch == 8
    say(f"[full] gqa128k batch 8: N={w.n_tokens}")
    st = Staged(w)
    say("  staged and built")
    rng = np.random.default_rng(7)
    # every head of two sequences, plus two random heads of each other sequence
    pairs = [(s, h) for s in (0, 5) for h in range(w.n_q_heads)]
    pairs += [(s, int(h)) for s in range(w.batch) if s not in (0, 5) for h in rng.choice(w.n_q_heads, 2, False)]
    stats = _decode_steps(st, 1, append=False, pairs=pairs)
    # the per-pair cut ran with thousands of candidates per pair
    assert int(stats[0][..., 0, 0].max()) > 2048


def test_decode16m_full_size():
    t = torch()
    w = W.get_workload("decode16m")
    assert w.n_tokens == 1 << 24 and w.n_kv_heads == 1
    say(f"[full] decode16m: N={w.n_tokens}")
    st = Staged(w)
    say("  staged and built")
    assert st.cache.K.numel() * st.cache.K.element_size() >= 1 << 32
    _decode_steps(st, 2, append=False)
    # dense over all 16,777,216 tokens on two heads: the oracle's attention over
    # slabs, merged by their log-sum-exp
    qn, q = st.queries(0)
    out = t.zeros_like(q)
    lse = t.zeros(q.shape[:3], dtype=t.float32, device="cuda")
    Z.dense_attend(st.geom, q, None, st.cache.K, st.cache.V, st.cache.seq_lens, out, lse, st.cache.ws)
    t.cuda.synchronize()
    o_np, l_np = out.cpu().numpy(), lse.cpu().numpy()
    N, slab = w.n_tokens, 1 << 21
    for hq in (0, 5):
        parts = [O.attend(qn[0, 0, hq], st.Kf[0, 0], st.Vf[0, 0], np.arange(a, min(a + slab, N)), w.scale)
                 for a in range(0, N, slab)]
        M = max(l for _, l in parts)
        wts = [math.exp(l - M) for _, l in parts]
        o = sum(wi * oi for wi, (oi, _) in zip(wts, parts)) / sum(wts)
        l = M + math.log(sum(wts))
        e = max(np.abs(o_np[0, 0, hq] - o).max(), abs(l_np[0, 0, hq] - l))
        say(f"  dense head {hq}: error {e:.3g}")
        assert e <= attn_tol(w), (hq, e)
