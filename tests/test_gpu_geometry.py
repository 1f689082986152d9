"""The two tree geometries the pages evaluate, against the CPU oracle:

* C4-L6 (deep): b = 4, six levels, 4096 tokens per top node. At 262,144 tokens
  the top level holds 64 nodes and the levels below span 1024, 256, 64, 16 and 4
  tokens ("Zyphra Hierarchical Attention: The End of Quadratic Attention?",
  §A query's path through the tree, step by step).
* C256-L1 (wide): b = 256, one level, so routing is a single top-p cut over
  the 1024 chunks of 256 tokens ("Subquadratic Attention with a Hierarchical
  Tree-Structured Indexer", §Reasoning and Retrieval Performance).

Both on the c2 key distribution (64 planted clusters of 32 tokens), 32/8 heads,
d = 128, bf16, p = 0.95: the tree against the oracle's, every level's kept set
teacher-forced (1e-5 margin exemptions, exact candidate counts), attention over
the GPU's index set within 2e-4. One decode row, then 64 causal rows (the
many-rows path: every level scored at once on the matrix cores).
"""
import numpy as np
import pytest

import hierarchical_tree_indexed_build_amd as Z
import workloads as W
from tests.gpu_helpers import Staged, check_attention, check_tree, say, teacher_forced, torch

pytestmark = pytest.mark.gpu

GEOMETRIES = [("c4l6", 4, 6), ("c256l1", 256, 1)]


def _workload(b, L, rows):
    w = W.get_workload("gqa128k", batch=1)
    w.n_tokens = 1 << 18
    w.capacity = w.n_tokens
    w.branching, w.n_levels = b, L
    w.queries_per_step = rows
    w.name = f"gqa128k-c{b}-l{L}"
    return w


@pytest.mark.parametrize("rows", [1, 64], ids=["decode", "64rows"])
@pytest.mark.parametrize("geo", GEOMETRIES, ids=[g[0] for g in GEOMETRIES])
def test_geometry_parity(geo, rows):
    t = torch()
    _, b, L = geo
    w = _workload(b, L, rows)
    say(f"[geometry] {w.name}: N={w.n_tokens}, {rows} row(s)")
    st = Staged(w)
    trees = st.oracle_trees()
    worst = check_tree(st, trees, w.n_tokens)
    say(f"  tree parity: worst error {worst:.3g} of the bound")
    qn, q = st.queries(0, rows=rows)
    qpos_np = (w.n_tokens - rows + np.arange(rows, dtype=np.int32))[None, :].repeat(w.batch, 0)
    q_pos = t.from_numpy(qpos_np).cuda()
    sel, nsel, stats, lsel = st.route_buffers(w.batch * rows)
    out = t.zeros_like(q)
    lse = t.zeros(q.shape[:3], dtype=t.float32, device="cuda")
    Z.attend(st.geom, q, q_pos, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, w.top_p, sel, nsel,
             out, lse, st.cache.ws, level_stats=stats, level_sel=lsel)
    t.cuda.synchronize()
    assert Z.read_device_status(st.cache.ws) == 0
    st_np = stats.cpu().numpy()
    if L == 6:
        # the top level of the last row holds the 64 nodes of 4096 tokens
        assert int(st_np[0, -1, 0, L - 1, 0]) == (1 << 18) // 4 ** 6 == 64
    flips = teacher_forced(st, qn, qpos_np, stats, lsel, w.top_p, trees)
    worst = check_attention(st, qn, qpos_np, out, lse, sel, nsel)
    say(f"  exempt differences {flips}, worst attention error {worst:.3g}; candidates per level "
        f"{[int(st_np[..., l, 0].max()) for l in range(L)]}, kept {[int(st_np[..., l, 1].max()) for l in range(L)]}")
