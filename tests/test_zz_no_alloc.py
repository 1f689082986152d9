"""zha_attend_noalloc, the entry point for callers that cannot allocate: the same
route and attention as zha_attend, run in the library's static scratch instead
of a caller workspace. Checked through the C ABI against zha_attend on the same
inputs, bit for bit (same kernels, same order of arithmetic), on consecutive
calls whose second input is smaller than the first (the scratch keeps the last
call's contents), and for the device status it reports per call."""
import numpy as np
import pytest

import hierarchical_tree_indexed_build_amd as Z
import workloads as W
from tests.gpu_helpers import Staged, say, torch

pytestmark = pytest.mark.gpu


def _both(st, rows_per_seq, sel_cap=None):
    """zha_attend (caller workspace) and zha_attend_noalloc on the same query rows."""
    t = torch()
    w = st.w
    qn, q = st.queries(0, rows=rows_per_seq)
    q_pos = t.full((w.batch, rows_per_seq), w.n_tokens - 1, dtype=t.int32, device="cuda")
    res = []
    for noalloc in (False, True):
        sel, nsel, stats, lsel = st.route_buffers(w.batch * rows_per_seq, sel_cap)
        out = t.full_like(q, float("nan"))
        lse = t.full(q.shape[:3], float("nan"), dtype=t.float32, device="cuda")
        if noalloc:
            status = t.full((1,), 0xFFFF, dtype=t.int32, device="cuda")
            Z.attend_noalloc(st.geom, q, q_pos, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens,
                             w.top_p, sel, nsel, out, lse, level_stats=stats, level_sel=lsel, dev_status=status)
            t.cuda.synchronize()
            dev = int(status.item())
        else:
            Z.read_device_status(st.cache.ws, clear=True)
            Z.attend(st.geom, q, q_pos, st.cache.K, st.cache.V, st.cache.summaries, st.cache.seq_lens, w.top_p,
                     sel, nsel, out, lse, st.cache.ws, level_stats=stats, level_sel=lsel)
            dev = Z.read_device_status(st.cache.ws, clear=True)
        res.append(dict(out=out, lse=lse, sel=sel, nsel=nsel, stats=stats, lsel=lsel, dev=dev))
    a, b = res
    for k in ("out", "lse", "nsel", "stats", "lsel"):
        assert t.equal(a[k], b[k]), k
    cap = a["sel"].shape[-1]
    n = a["nsel"].clamp(max=cap)
    for idx in np.ndindex(*a["nsel"].shape):
        m = int(n[idx].item())
        assert t.equal(a["sel"][idx][:m], b["sel"][idx][:m]), idx
    assert a["dev"] == b["dev"], (a["dev"], b["dev"])
    return a


def test_noalloc_matches_attend_on_consecutive_calls():
    # a 32768-token bf16 cache (32/8 heads, b = 32, three levels: the split cut)
    w1 = W.get_workload("decode1m", shrink=1)
    say(f"[noalloc] call 1: {w1.name} N={w1.n_tokens}")
    st1 = Staged(w1)
    r = _both(st1, 1)
    assert r["dev"] == 0
    # a smaller input: the 4096-token fp32 cache, 16 rows, with a kept list that overflows
    w2 = W.get_workload("tiny")
    say(f"[noalloc] call 2: {w2.name} N={w2.n_tokens}, sel_capacity 50")
    st2 = Staged(w2)
    r = _both(st2, 16, sel_cap=50)
    assert int(r["nsel"].max().item()) > 50 and r["dev"] & Z.ZHA_DEV_SEL_OVERFLOW
    # the status word starts every call at zero
    say("[noalloc] call 3: the same input, no overflow")
    r = _both(st2, 16)
    assert r["dev"] == 0
    # and the first input again, after the smaller ones
    say("[noalloc] call 4: the first input again")
    r = _both(st1, 1)
    assert r["dev"] == 0


def test_noalloc_rejects_a_layout_past_the_scratch():
    t = torch()
    w = W.get_workload("decode16m")
    g = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels, w.capacity, w.kv_dtype)
    assert Z.query_sizes(g, 1).workspace_bytes > 64 << 20
    x = t.zeros(64, dtype=t.float32, device="cuda")
    i = t.zeros(64, dtype=t.int32, device="cuda")
    with pytest.raises(Z.ZhaError) as e:
        Z.attend_noalloc(g, x.view(1, 1, 8, 8), None, x, x, x, i, w.top_p, i.view(1, 1, 8, 8), i[:8].view(1, 1, 8),
                         x.view(1, 1, 8, 8), x[:8].view(1, 1, 8))
    assert e.value.code == Z.ZHA_ERR_WORKSPACE and "static scratch" in str(e.value)
