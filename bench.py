"""Benchmark of the ZHA decode hot path on one MI355X.

One step = one decode token for every sequence: append its K/V row (completing
any tree nodes it closes), route its query through the tree and attend exactly
over the selected keys (zha_append + zha_attend). Default workload: 1,048,576
bf16 tokens, batch 1, 32 query / 8 kv heads, d=128, b=32, 4 levels, p=0.95.

Printed: one JSON line with queries/s, the dominant kernel's roofline, the
in-run dense kernel on the same cache and queries, and the CPU oracle timed on
the host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps 256] [--warmup 8] [--workload decode1m]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hierarchical_tree_indexed_build_amd as Z  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode1m_attend_traffic.json")
KERNEL_SOURCES = {"attend": "attend.hip", "route_score": "route.hip", "route_cut": "route.hip"}
METRIC = "ZHA decode queries/sec at 1M-token KV; % HBM roofline; speedup vs dense"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="decode1m", choices=["decode1m", "gqa128k", "decode16m", "prefill256k"])
    ap.add_argument("--kernel", default="attend", help="kernel label timed live for the roofline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="copy a buffer of this many MiB once before the timed steps (calibrates byte counters)")
    ap.add_argument("--timed-only", action="store_true",
                    help="run the warmup and timed steps only (for profiler runs), print a short line")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-flushed run")
    ap.add_argument("--cold", action="store_true",
                    help="with --timed-only: read a 512 MiB buffer before every timed step (counter runs of "
                         "the cache-flushed steps)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the kernel's HBM traffic per launch from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of --timed-only --copy-probe-mib M, then exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# staging
# ----------------------------------------------------------------------------
class Bench:
    def __init__(self, w, steps, warmup, K_host, V_host, q_host, kv_new):
        import torch
        self.t = torch
        self.w = w
        self.steps, self.warmup = steps, warmup
        self.geom = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels,
                                w.capacity, w.kv_dtype)
        self.c = Z.Cache(self.geom, 1)
        self.sizes = self.c.sizes
        t0 = time.time()
        kdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
        self.K_host, self.V_host = K_host, V_host
        self.c.K.copy_(torch.from_numpy(self.K_host).view(kdt))
        self.c.V.copy_(torch.from_numpy(self.V_host).view(kdt))
        log(f"[bench] uploaded the {w.n_tokens}-token cache in {time.time() - t0:.1f}s")
        self.R = W.ref_queries(w)
        self.ref_q = torch.from_numpy(self.R).cuda()
        self.c.seq_lens.fill_(w.n_tokens)
        # per-step inputs, resident in HBM before any timing
        self.q = torch.from_numpy(q_host).cuda()                          # [S, B, 1, Hq, d]
        self.q_host = q_host
        if w.append_per_step:
            self.k_new = torch.stack([torch.from_numpy(k).view(kdt) for k, _ in kv_new]).cuda()
            self.v_new = torch.stack([torch.from_numpy(v).view(kdt) for _, v in kv_new]).cuda()
            self.kv_host = kv_new
        n1 = self.sizes.level_nodes[0]
        self.sel = torch.zeros((w.batch, 1, w.n_q_heads, n1), dtype=torch.int32, device="cuda")
        self.nsel = torch.zeros((w.batch, 1, w.n_q_heads), dtype=torch.int32, device="cuda")
        self.out = torch.zeros((w.batch, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        self.lse = torch.zeros((w.batch, 1, w.n_q_heads), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.time()
        Z.build_tree(self.geom, self.c.K, self.ref_q, self.c.seq_lens, self.c.summaries, self.c.ws)
        torch.cuda.synchronize()
        self.build_s = time.time() - t0
        log(f"[bench] tree built in {self.build_s * 1e3:.1f} ms (first call, includes module load)")

    def step(self, i, level_stats=None, level_sel=None):
        w, c = self.w, self.c
        if w.append_per_step:
            Z.append(self.geom, c.K, c.V, self.k_new[i], self.v_new[i], c.seq_lens, self.ref_q, c.summaries, c.ws)
        Z.attend(self.geom, self.q[i], None, c.K, c.V, c.summaries, c.seq_lens, w.top_p, self.sel, self.nsel,
                 self.out, self.lse, c.ws, level_stats=level_stats, level_sel=level_sel)

    def snapshot(self):
        return self.c.summaries.clone(), self.c.seq_lens.clone()

    def restore(self, snap):
        self.c.summaries.copy_(snap[0])
        self.c.seq_lens.copy_(snap[1])


# ----------------------------------------------------------------------------
# algorithmic bytes (each unique byte the method must move, once)
# ----------------------------------------------------------------------------
def _lsel_level(b: Bench, lsel: np.ndarray, rows: int, level: int) -> np.ndarray:
    n = b.sizes.level_nodes[level - 1]
    off = rows * b.geom.n_q_heads * b.sizes.level_sel_offset[level - 1]
    return lsel[off:off + rows * b.geom.n_q_heads * n].reshape(rows, b.geom.n_q_heads, n)


def step_bytes(b: Bench, stats, lsel, sel, nsel, N):
    """Algorithmic bytes per kernel family for one decode step.

    route_score@l: every summary row of level l scored for a kv group, read once
      (4d bytes), plus one fp32 score per (query head, row) written.
    route_cut@l: every candidate score read once (4 B) plus kept ids written (4 B).
    attend: K and V rows of the union of the group's index sets, read once
      (2 d s_kv bytes per token), plus the query (4d) and partial writes.
    append: one K and one V row per kv head.
    """
    w = b.w
    d, g, bb, L = w.head_dim, w.group, w.branching, w.n_levels
    skv = 2 if w.kv_dtype == "bf16" else 4
    rows = w.batch
    out = {}
    nc = [N // bb ** l for l in range(1, L + 1)] + [0]
    stats = stats.reshape(rows, w.n_q_heads, L, 2)
    for level in range(L, 0, -1):
        scored = 0
        for s in range(rows):
            for kv in range(w.n_kv_heads):
                if level == L:
                    scored += nc[L - 1]
                    continue
                v = _lsel_level(b, lsel, rows, level + 1)
                par = set()
                for h in range(kv * g, kv * g + g):
                    cnt = int(stats[s, h, level, 1])
                    par.update(v[s, h, :cnt].tolist())
                scored += len(par) * bb + (nc[level - 1] - nc[level] * bb)
        out[f"route_score@{level}"] = scored * (4 * d + 4 * g) + rows * w.n_q_heads * 4 * d
        cands = int(stats[:, :, level - 1, 0].sum())
        kept = int(stats[:, :, level - 1, 1].sum())
        out[f"route_cut@{level}"] = 4 * cands + 4 * kept
    toks = 0
    for s in range(rows):
        for kv in range(w.n_kv_heads):
            blocks = {0, (N - 1) // bb}
            for h in range(kv * g, kv * g + g):
                blocks.update(sel[s, 0, h, :nsel[s, 0, h]].tolist())
            toks += sum(min(bb, N - x * bb) for x in blocks)
    out["attend"] = toks * 2 * d * skv + rows * w.n_q_heads * 4 * d
    out["append"] = rows * w.n_kv_heads * 2 * d * skv if w.append_per_step else 0
    return out


# ----------------------------------------------------------------------------
# CPU oracle baseline
# ----------------------------------------------------------------------------
_CPU = {}     # the oracle leg's inputs, set before its worker processes fork (they inherit it)


def cpu_workers() -> int:
    """Worker processes for the oracle leg: the cores this process may run on,
    at most 16 (one GPU's share of a host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_query(task):
    """One (step, sequence, query head) through the oracle: route, then exact
    attention over the index set. Runs in a worker with one BLAS thread."""
    from oracle import zha_oracle as O
    step, s, hq = task
    d = _CPU
    w = d["w"]
    kv = hq // w.group
    N = d["N"][step]
    q = d["q"][step][s, 0, hq]
    r = O.route(q, d["trees"][s][kv], N, w.branching, d["top_p"])
    I = O.index_set(r.selected[0], N, w.branching)
    o, lse = O.attend(q, d["Kf"][s][kv], d["Vf"][s][kv], I)
    return step, s, hq, r.selected[0].astype(np.int32), o, lse


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def cpu_baseline(w, K_host, V_host, q_host, kv_new, first_step, last_step, budget_s):
    """The oracle's per-query work (route + exact attention of every head) timed on
    the host's cores before the GPU is touched: a process pool (fork) with one
    BLAS thread per worker, one decode step's queries per round, steps
    first_step, first_step + 1, ... until about budget_s seconds have passed.
    The oracle builds its own tree from the host keys (not timed: it is built
    once per cache). Returns the record and the outputs per (step, s, hq)."""
    import multiprocessing as mp
    from concurrent.futures import ThreadPoolExecutor
    from oracle import zha_oracle as O
    app = w.append_per_step
    n_last = w.n_tokens + (last_step + 1) * app
    Kh, Vh = K_host, V_host
    if app:
        Kh, Vh = K_host.copy(), V_host.copy()
        for i, (k, v) in enumerate(kv_new[:last_step + 1]):
            Kh[:, :, w.n_tokens + i * app:w.n_tokens + (i + 1) * app] = k
            Vh[:, :, w.n_tokens + i * app:w.n_tokens + (i + 1) * app] = v
    Kf = [[W.as_f32(w, Kh[s, h, :n_last]) for h in range(w.n_kv_heads)] for s in range(w.batch)]
    Vf = [[W.as_f32(w, Vh[s, h, :n_last]) for h in range(w.n_kv_heads)] for s in range(w.batch)]
    R = W.ref_queries(w)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(W.host_threads()) as ex:
        flat = list(ex.map(lambda sh: O.build_tree(Kf[sh[0]][sh[1]], R[:, sh[1]], w.branching, slab=1 << 20),
                           [(s, h) for s in range(w.batch) for h in range(w.n_kv_heads)]))
    trees = [flat[s * w.n_kv_heads:(s + 1) * w.n_kv_heads] for s in range(w.batch)]
    log(f"[bench] oracle tree built from the host keys in {time.perf_counter() - t0:.1f}s")
    _CPU.update(w=w, trees=trees, Kf=Kf, Vf=Vf, q=q_host, top_p=w.top_p,
                N={i: w.n_tokens + (i + 1) * app for i in range(last_step + 1)})
    n = cpu_workers()
    outs = {}
    done = 0
    ctx = mp.get_context("fork")
    with ctx.Pool(n, initializer=_one_blas_thread) as pool:
        t0 = time.perf_counter()
        for step in range(first_step, last_step + 1):
            tasks = [(step, s, hq) for s in range(w.batch) for hq in range(w.n_q_heads)]
            for res in pool.map(_oracle_query, tasks, chunksize=1):
                outs[res[:3]] = res[3:]
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
    _CPU.clear()
    rec = {"value": round(done * w.batch / el, 3), "unit": "queries/s", "cores": n, "kind": "oracle",
           "sample": f"{done} decode steps (steps {first_step}..{first_step + done - 1} of the timed run) x "
                     f"{w.batch} sequence(s) x {w.n_q_heads} heads: route + exact attention per head, NumPy "
                     f"fp64, {n} worker processes with one BLAS thread each, the oracle's own tree built from "
                     f"the host keys; {el:.1f}s"}
    return rec, outs


def cpu_parity(w, outs, gpu):
    """End-to-end agreement of the GPU's timed steps with the oracle leg's outputs
    on the same queries: kept leaf sets, then attention on the heads whose sets
    are equal (other heads differ by a margin flip upstream, which the
    teacher-forced parity tests cover)."""
    equal, worst, n = 0, 0.0, 0
    for (step, s, hq), (ids, o, lse) in outs.items():
        if step not in gpu:
            continue
        sel, nsel, out, l = gpu[step]
        n += 1
        g_ids = sel[s, 0, hq, :nsel[s, 0, hq]]
        if len(g_ids) == len(ids) and np.array_equal(np.sort(g_ids), ids):
            equal += 1
            worst = max(worst, float(np.abs(out[s, 0, hq] - o).max()), abs(float(l[s, 0, hq]) - lse))
    tol = 2e-4 if w.kv_dtype == "bf16" else 1e-5
    return {"heads": n, "index_sets_equal": equal, "max_abs_err_on_equal_sets": round(worst, 7), "tol": tol,
            "ok": bool(n and worst <= tol)}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter runs (FETCH_SIZE, WRITE_SIZE,
    each scaled by its reading for a copy of known size), or None when no counters were taken
    for this workload or the kernel's source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    name = kernel.split("@")[0]
    src = os.path.join(ROOT, "hierarchical_tree_indexed_build_amd", "csrc", KERNEL_SOURCES.get(name, ""))
    if rec.get("kernel") != kernel or rec.get("workload") != workload or not os.path.isfile(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("source_sha256"):
            return None
    return int(rec["traffic_bytes_per_launch"])


KERNEL_SYMBOLS = {"attend": ("attend_kernel<", "attend_mfma_kernel<"), "route_score": ("route_score_kernel<",),
                  "route_cut": ("route_cut_kernel", "route_split_hist_kernel", "route_split_emit_kernel")}


def _counter_rows(run_dir: str, counter: str):
    """(dispatch id, kernel name, value) of every dispatch in a rocprofv3 --pmc csv run."""
    import csv
    paths = []
    for dp, _, fs in os.walk(run_dir):
        paths += [os.path.join(dp, f) for f in fs if f.endswith("counter_collection.csv")]
    if len(paths) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {run_dir}, found {len(paths)}")
    acc = {}
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = acc.get(d, (r["Kernel_Name"], 0.0))
            acc[d] = (name, v + float(r["Counter_Value"]))     # summed over agents/instances
    return [(d, n, v) for d, (n, v) in sorted(acc.items())]


def write_traffic(fetch_dir: str, write_dir: str, kernel: str, workload: str, probe_mib: int, steps: int,
                  cold: bool = False):
    """Turn two counter runs of `bench.py --timed-only --copy-probe-mib M` (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch) into HBM bytes per launch of `kernel`: each counter is
    scaled by (copy size / its reading for the copy probe) and averaged over the last `steps`
    launches, which are the timed ones."""
    sym = KERNEL_SYMBOLS[kernel.split("@")[0]]
    probe = probe_mib << 20
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copies = [v for _, n, v in rows if "copyBuffer" in n]
        if not copies:
            raise SystemExit(f"{counter}: no copy kernel found in {d}")
        factor = probe / (max(copies) * 1024.0)
        vals = [v * 1024.0 * factor for _, n, v in rows if any(x in n for x in sym)][-steps:]
        if len(vals) < steps:
            raise SystemExit(f"{counter}: {len(vals)} launches of {sym} in {d}, expected {steps}")
        per[counter] = {"factor": round(factor, 4), "bytes_per_launch": sum(vals) / len(vals),
                        "copy_probe_kib": max(copies)}
    name = kernel.split("@")[0]
    with open(os.path.join(ROOT, "hierarchical_tree_indexed_build_amd", "csrc", KERNEL_SOURCES[name]), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    rec = {"kernel": kernel, "workload": workload, "source_sha256": sha, "launches": steps,
           "cold": cold, "copy_probe_bytes": probe,
           "fetch": per["FETCH_SIZE"], "write": per["WRITE_SIZE"],
           "traffic_bytes_per_launch": int(round(per["FETCH_SIZE"]["bytes_per_launch"]
                                                 + per["WRITE_SIZE"]["bytes_per_launch"]))}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


# ----------------------------------------------------------------------------
# chunked prefill: append a causal chunk, then route and attend all its rows
# ----------------------------------------------------------------------------
FP32_MFMA_PEAK = 157.3e12   # MI355X dense fp32 matrix FLOP/s
PREFILL_METRIC = "ZHA chunked-prefill rows/sec at 256K-token KV (8192-row causal chunk)"


def prefill_main(args, w):
    """One step = seq_lens reset to the cache length, zha_append of the chunk
    (summarising every node it completes), zha_attend of its T causal rows.
    Re-appending the same chunk at the same place rewrites identical bits, so
    every step does the same work."""
    import torch
    steps = args.steps if args.steps is not None else 5
    warm = min(args.warmup, 2)
    T, n0 = w.prefill_chunk, w.n_tokens
    log(f"[bench] workload {w.name}: {w.description}; steps {steps}, warmup {warm}")
    K_host, V_host = W.kv_cache(w)
    kn, vn = W.prefill_chunk_kv(w)
    q_host = W.queries(w, 0, rows=T)
    cpu, cpu_outs = None, {}
    if not (args.no_cpu or args.timed_only):
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f}s on {cpu_workers()} worker processes")
        cpu, cpu_outs = prefill_cpu_baseline(w, q_host, K_host, V_host, kn, vn, args.cpu_seconds)
    import torch
    geom = Z.make_geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.branching, w.n_levels, w.capacity,
                       w.kv_dtype)
    c = Z.Cache(geom, T, tiled=True)         # row tiles: the workspace of one tile, not of all T rows
    log(f"[bench] workspace {c.ws.numel() * 4 / 2**30:.2f} GiB (rows in tiles of {c.sizes.tile_rows}; "
        f"{c.sizes.workspace_bytes / 2**30:.1f} GiB for every row at once)")
    kdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    c.K.copy_(torch.from_numpy(K_host).view(kdt))
    c.V.copy_(torch.from_numpy(V_host).view(kdt))
    k_new = torch.from_numpy(kn).view(kdt).cuda()
    v_new = torch.from_numpy(vn).view(kdt).cuda()
    ref_q = torch.from_numpy(W.ref_queries(w)).cuda()
    q = torch.from_numpy(q_host).cuda()
    q_pos = (n0 + torch.arange(T, dtype=torch.int32, device="cuda")).view(1, T).repeat(w.batch, 1).contiguous()
    lens0 = torch.full((w.batch,), n0, dtype=torch.int32, device="cuda")
    c.seq_lens.copy_(lens0)
    Z.build_tree(geom, c.K, ref_q, c.seq_lens, c.summaries, c.ws)
    sel_cap = 4096
    sel = torch.zeros((w.batch, T, w.n_q_heads, sel_cap), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((w.batch, T, w.n_q_heads), dtype=torch.int32, device="cuda")
    out = torch.zeros((w.batch, T, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.zeros((w.batch, T, w.n_q_heads), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(level_stats=None):
        c.seq_lens.copy_(lens0)
        Z.append(geom, c.K, c.V, k_new, v_new, c.seq_lens, ref_q, c.summaries, c.ws)
        Z.attend(geom, q, q_pos, c.K, c.V, c.summaries, c.seq_lens, w.top_p, sel, nsel, out, lse, c.ws,
                 level_stats=level_stats)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    if Z.read_device_status(c.ws, clear=True) & ~Z.ZHA_DEV_SEL_OVERFLOW:
        raise RuntimeError("device status raised during warmup")
    kernel = "route_dense" if args.kernel == "attend" else args.kernel
    Z.profile_start(kernel)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms, k_launch, _ = Z.profile_collect()
    Z.profile_start(None)
    if args.timed_only:
        print(json.dumps({"workload": w.name, "steps": steps, "warmup": warm, "ms_per_step": wall * 1e3 / steps,
                          "kernel": kernel, "kernel_avg_us": k_ms / max(1, k_launch) * 1e3,
                          "launches": k_launch}), flush=True)
        return
    # per-step time of each kernel family, one family per pass
    fam_ms = {}
    for fam in ("append_rows", "build_level", "advance_seq", "route_dense", "route_cut", "attn_items", "attn_plan",
                "attend", "attend_combine"):
        Z.profile_start(fam)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        ms, _, _ = Z.profile_collect()
        fam_ms[fam] = round(ms / 2, 4)
    Z.profile_start(None)
    stats = torch.zeros((w.batch, T, w.n_q_heads, w.n_levels, 2), dtype=torch.int32, device="cuda")
    step(level_stats=stats)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()

    # algorithmic work of the dense scores: every node each row sees, for each of its heads
    d, g, bb = w.head_dim, w.group, w.branching
    Nv = n0 + 1 + np.arange(T, dtype=np.int64)
    seen = sum(int((Nv // bb ** l).sum()) for l in range(1, w.n_levels + 1))
    flops = 2.0 * d * seen * w.batch * w.n_q_heads
    k_avg_s = (k_ms / 1e3) / max(1, k_launch)
    # a row tile per launch: the chunk's flops over the launches of its steps
    flops_launch = flops * steps / max(1, k_launch)
    achieved = flops_launch / k_avg_s if (kernel == "route_dense" and k_avg_s > 0) else 0.0

    if cpu is not None:
        # the GPU's rows against the oracle leg's, end to end
        s_np, n_np, o_np, l_np = sel.cpu().numpy(), nsel.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
        gpu = {t_: (s_np[:, t_:t_ + 1], n_np[:, t_:t_ + 1], o_np[:, t_:t_ + 1], l_np[:, t_:t_ + 1])
               for t_ in {k[0] for k in cpu_outs}}
        cpu["parity"] = cpu_parity(w, cpu_outs, gpu)
    ms_step = wall * 1e3 / steps
    res = {
        "metric": PREFILL_METRIC,
        "value": round(w.batch * T * steps / wall, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_tokens": n0, "chunk": T, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": d, "branching": bb, "levels": w.n_levels,
                   "top_p": w.top_p, "kv_cache": w.kv_dtype},
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": FP32_MFMA_PEAK / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / FP32_MFMA_PEAK, 4), "traffic": None,
                     "kernel": kernel, "flops_per_launch": flops_launch, "avg_launch_us": round(k_avg_s * 1e6, 3),
                     "launches": k_launch},
        "cpu_baseline": cpu,
        "ms_by_kernel_family": fam_ms,
        "workspace_bytes": int(c.ws.numel() * 4),
        "row_tile": int(c.sizes.tile_rows),
        "workspace_bytes_one_pass": int(c.sizes.workspace_bytes),
        "candidates_per_row_head": [round(float(st[..., l, 0].mean()), 1) for l in range(w.n_levels)],
        "kept_per_row_head": [round(float(st[..., l, 1].mean()), 2) for l in range(w.n_levels)],
    }
    print(json.dumps(res), flush=True)


def prefill_cpu_baseline(w, q_host, K_host, V_host, kn, vn, budget_s):
    """The oracle routes and attends the chunk's rows in order (every head), each
    row seeing the tokens up to its own position, on the same process pool as
    the decode leg (run before the GPU is touched), against its own tree built
    from the host keys, until the budget is spent. Returns the record and the
    outputs per (row, 0, head)."""
    import multiprocessing as mp
    from concurrent.futures import ThreadPoolExecutor
    from oracle import zha_oracle as O
    T, n0 = w.prefill_chunk, w.n_tokens
    Kf = np.concatenate([W.as_f32(w, K_host[:, :, :n0]), W.as_f32(w, kn)], axis=2)
    Vf = np.concatenate([W.as_f32(w, V_host[:, :, :n0]), W.as_f32(w, vn)], axis=2)
    R = W.ref_queries(w)
    with ThreadPoolExecutor(W.host_threads()) as ex:
        flat = list(ex.map(lambda sh: O.build_tree(Kf[sh[0], sh[1]], R[:, sh[1]], w.branching),
                           [(s, h) for s in range(w.batch) for h in range(w.n_kv_heads)]))
    trees = [flat[s * w.n_kv_heads:(s + 1) * w.n_kv_heads] for s in range(w.batch)]
    # a row of the chunk plays the part of a decode step: its query and the tokens it sees
    qsteps = [q_host[:, t:t + 1] for t in range(T)]
    _CPU.update(w=w, trees=trees, Kf=[[Kf[s, h] for h in range(w.n_kv_heads)] for s in range(w.batch)],
                Vf=[[Vf[s, h] for h in range(w.n_kv_heads)] for s in range(w.batch)], q=qsteps, top_p=w.top_p,
                N={t: n0 + t + 1 for t in range(T)})
    n = cpu_workers()
    done = 0
    outs = {}
    with mp.get_context("fork").Pool(n, initializer=_one_blas_thread) as pool:
        t0 = time.perf_counter()
        while done < T and time.perf_counter() - t0 < budget_s:
            tasks = [(done, s, hq) for s in range(w.batch) for hq in range(w.n_q_heads)]
            for res in pool.map(_oracle_query, tasks, chunksize=1):
                outs[res[:3]] = res[3:]
            done += 1
        el = time.perf_counter() - t0
    _CPU.clear()
    rec = {"value": round(done * w.batch / el, 3), "unit": "rows/s", "cores": n, "kind": "oracle",
           "sample": f"the chunk's first {done} rows x {w.batch} sequence(s) x {w.n_q_heads} heads: route + exact "
                     f"attention per head, NumPy fp64, {n} worker processes with one BLAS thread each, the oracle's "
                     f"own tree built from the host keys; {el:.1f}s"}
    return rec, outs


# ----------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this build has no "
              f"multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        w = W.get_workload(args.workload)
        write_traffic(*args.traffic_from, args.kernel, w.name, args.copy_probe_mib,
                      args.steps if args.steps is not None else w.steps, cold=args.cold)
        return
    w = W.get_workload(args.workload)
    if w.prefill_chunk:
        prefill_main(args, w)
        return
    steps = args.steps if args.steps is not None else w.steps
    warm = args.warmup
    total = steps + warm
    if w.append_per_step:
        w.capacity = w.n_tokens + total * w.append_per_step
    log(f"[bench] workload {w.name}: {w.description}; steps {steps}, warmup {warm}")
    t0 = time.time()
    K_host, V_host = W.kv_cache(w)
    q_host = np.stack([W.queries(w, i) for i in range(total)])            # [S, B, 1, Hq, d]
    kv_new = [W.appended_tokens(w, i) for i in range(total)] if w.append_per_step else []
    log(f"[bench] generated the {w.n_tokens}-token cache and {total} steps of inputs in {time.time() - t0:.1f}s")
    # the CPU oracle runs first, in worker processes forked before the GPU is touched
    cpu, cpu_outs = None, {}
    if not (args.no_cpu or args.timed_only):
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f}s on {cpu_workers()} worker processes")
        cpu, cpu_outs = cpu_baseline(w, K_host, V_host, q_host, kv_new, warm, warm + steps - 1, args.cpu_seconds)
    import torch
    b = Bench(w, steps, warm, K_host, V_host, q_host, kv_new)

    # ---- warmup ----
    for i in range(warm):
        b.step(i)
    torch.cuda.synchronize()
    if Z.read_device_status(b.c.ws):
        raise RuntimeError("device status raised during warmup")
    snap = b.snapshot()

    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- timed pass: product calls only, one kernel family timed with events ----
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda") if (args.timed_only and args.cold) else None
    fsum = torch.zeros((), dtype=torch.float32, device="cuda")
    Z.profile_start(args.kernel)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warm, warm + steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=fsum)          # reads 512 MiB: clean lines evict the step's bytes
        b.step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del flush
    k_ms, k_launch, k_drop = Z.profile_collect()
    Z.profile_start(None)
    out_timed = b.out.clone()
    status = Z.read_device_status(b.c.ws)
    if args.timed_only:
        print(json.dumps({"workload": w.name, "steps": steps, "warmup": warm, "ms_per_step": wall * 1e3 / steps,
                          "kernel": args.kernel, "kernel_avg_us": k_ms / max(1, k_launch) * 1e3,
                          "launches": k_launch, "device_status": status, "cold": bool(args.cold)}), flush=True)
        return
    log(f"[bench] timed {steps} steps in {wall * 1e3:.2f} ms; {args.kernel}: {k_launch} launches, "
        f"{k_ms / max(1, k_launch) * 1e3:.2f} us avg")

    # ---- replay for byte accounting (deterministic: identical routing) ----
    b.restore(snap)
    L = w.n_levels
    rows = w.batch
    stats = torch.zeros((w.batch, 1, w.n_q_heads, L, 2), dtype=torch.int32, device="cuda")
    lsel = torch.zeros(max(1, b.sizes.level_sel_bytes // 4), dtype=torch.int32, device="cuda")
    totals = {}
    kept1 = []
    gpu_steps = {}
    for i in range(warm, warm + steps):
        b.step(i, level_stats=stats, level_sel=lsel)
        N = int(b.c.seq_lens[0].item())
        by = step_bytes(b, stats.cpu().numpy(), lsel.cpu().numpy(), b.sel.cpu().numpy(), b.nsel.cpu().numpy(), N)
        for k, v in by.items():
            totals[k] = totals.get(k, 0) + v
        kept1.append(b.nsel.cpu().numpy().reshape(-1))
        if any(k[0] == i for k in cpu_outs):
            gpu_steps[i] = (b.sel.cpu().numpy(), b.nsel.cpu().numpy(), b.out.cpu().numpy(), b.lse.cpu().numpy())
        if i == warm:
            st0 = stats.cpu().numpy().reshape(w.batch, w.n_q_heads, L, 2)[0]      # the first sequence
    torch.cuda.synchronize()
    replay_same = bool(torch.equal(out_timed, b.out))
    step_total = sum(totals.values())

    # ---- attend-only and dense on the final cache, same queries ----
    qs = [b.q[i] for i in range(warm, warm + steps)]
    c = b.c
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for q in qs:
        Z.attend(b.geom, q, None, c.K, c.V, c.summaries, c.seq_lens, w.top_p, b.sel, b.nsel, b.out, b.lse, c.ws)
    torch.cuda.synchronize()
    zha_ms = (time.perf_counter() - t0) * 1e3 / steps
    od = torch.zeros_like(b.out)
    ld = torch.zeros_like(b.lse)
    ndense = min(steps, 64)
    for q in qs[:4]:
        Z.dense_attend(b.geom, q, None, c.K, c.V, c.seq_lens, od, ld, c.ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for q in qs[:ndense]:
        Z.dense_attend(b.geom, q, None, c.K, c.V, c.seq_lens, od, ld, c.ws)
    torch.cuda.synchronize()
    dense_ms = (time.perf_counter() - t0) * 1e3 / ndense
    Nf = int(c.seq_lens[0].item())
    skv = 2 if w.kv_dtype == "bf16" else 4
    dense_bytes = w.batch * w.n_kv_heads * Nf * 2 * w.head_dim * skv
    # dense vs zha outputs for the last query: sparse attention is an approximation
    Z.attend(b.geom, qs[-1], None, c.K, c.V, c.summaries, c.seq_lens, w.top_p, b.sel, b.nsel, b.out, b.lse, c.ws)
    Z.dense_attend(b.geom, qs[-1], None, c.K, c.V, c.seq_lens, od, ld, c.ws)
    torch.cuda.synchronize()
    approx_err = float((b.out - od).abs().max().item())

    # ---- cold run: flush MALL / L2 between steps, time each step with events ----
    cold_qps = None
    cold_ms = ck_ms = 0.0
    ck_launch = 0
    if not args.no_cold:
        b.restore(snap)
        flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        fsum = torch.zeros((), dtype=torch.float32, device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        Z.profile_start(args.kernel)
        for j, i in enumerate(range(warm, warm + steps)):
            torch.sum(flush, dim=0, out=fsum)          # reads 512 MiB: clean lines evict the step's bytes
            ev[j][0].record()
            b.step(i)
            ev[j][1].record()
        torch.cuda.synchronize()
        ck_ms, ck_launch, _ = Z.profile_collect()
        Z.profile_start(None)
        cold_ms = sum(a.elapsed_time(z) for a, z in ev) / steps
        cold_qps = w.batch / (cold_ms / 1e3)
        del flush

    if cpu is not None:
        cpu["parity"] = cpu_parity(w, cpu_outs, gpu_steps)

    ms_step = wall * 1e3 / steps
    kb = sum(v for k, v in totals.items() if k == args.kernel or k.split("@")[0] == args.kernel)
    k_avg_s = (k_ms / 1e3) / max(1, k_launch)
    achieved = (kb / steps) / k_avg_s if k_avg_s > 0 else 0.0
    ck_avg_s = (ck_ms / 1e3) / max(1, ck_launch)
    cold_achieved = (kb / steps) / ck_avg_s if ck_avg_s > 0 else 0.0
    res = {
        "metric": METRIC,
        "value": round(w.batch * steps / wall, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "precision": {"kv_cache": w.kv_dtype, "summaries_scores_softmax": "f32",
                      "attention_logits": ("f32 dot products of the bf16 keys with q, which goes to the matrix "
                                           "cores as three bf16 parts summing to it within about 2^-25, "
                                           "f32 accumulation") if w.kv_dtype == "bf16" else "f32"},
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_tokens": w.n_tokens, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "branching": w.branching,
                   "levels": w.n_levels, "top_p": w.top_p, "kv_cache": w.kv_dtype,
                   "append_per_step": w.append_per_step},
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 2), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4), "traffic": measured_traffic(args.kernel, w.name),
                     "kernel": args.kernel, "bytes_per_launch": int(kb / steps),
                     "avg_launch_us": round(k_avg_s * 1e6, 3), "launches": k_launch,
                     "cold": ({"achieved": round(cold_achieved / 1e9, 2), "frac": round(cold_achieved / HBM_PEAK, 4),
                               "avg_launch_us": round(ck_avg_s * 1e6, 3), "launches": ck_launch,
                               "note": "a 512 MiB buffer is read between steps, so the 256 MB Infinity Cache "
                                       "holds none of the step's bytes"} if ck_launch else None)},
        "cpu_baseline": cpu,
        "step_hbm_frac": round((step_total / steps) / (ms_step / 1e3) / HBM_PEAK, 4),
        "step_hbm_frac_cold": round((step_total / steps) / (cold_ms / 1e3) / HBM_PEAK, 4) if cold_ms else None,
        "step_bytes": int(step_total / steps),
        "bytes_by_kernel": {k: int(v / steps) for k, v in sorted(totals.items())},
        "zha_attend_ms": round(zha_ms, 5),
        "dense_ms": round(dense_ms, 5),
        "dense_hbm_frac": round(dense_bytes / (dense_ms / 1e3) / HBM_PEAK, 4),
        "speedup_vs_dense": round(dense_ms / zha_ms, 3),
        "cold_queries_per_s": round(cold_qps, 2) if cold_qps else None,
        "keys_attended_frac": round(float(totals.get("attend", 0) / steps /
                                          (w.batch * w.n_kv_heads * Nf * 2 * w.head_dim * skv)), 6),
        "kept_leaves_mean": round(float(np.mean(np.concatenate(kept1))), 2),
        "level_counts_first_step": st0.tolist(),
        "max_abs_sparse_vs_dense": round(approx_err, 5),
        "replay_identical": replay_same,
        "device_status": status,
        "tree_build_ms": round(b.build_s * 1e3, 3),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
