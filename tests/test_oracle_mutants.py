"""Plant plausible mistakes in copies of the oracle and check that some pin catches each one.

The mistakes are planted on the CPU, in throwaway module copies built from the
oracle's source text; the real oracle is never modified.
"""
import os
import sys
import types

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "zha_oracle.py")

MUTANTS = {
    "pool-logit-sign": ("z = scale * (X @ np.asarray(r, dtype=F64))", "z = -scale * (X @ np.asarray(r, dtype=F64))"),
    "pool-norm-axis": ("w = w / w.sum(axis=1, keepdims=True)", "w = w / w.sum(axis=0, keepdims=True)"),
    "pool-no-scale": ("z = scale * (X @ np.asarray(r, dtype=F64))", "z = (X @ np.asarray(r, dtype=F64))"),
    "same-ref-every-level": ("X = pool_children(X, R[l], b, scale)", "X = pool_children(X, R[0], b, scale)"),
    "levels-from-raw-keys": ("X = pool_children(X, R[l], b, scale)\n        levels.append(X)",
                             "levels.append(pool_children(np.asarray(K, dtype=F64), R[l], b ** (l + 1), scale))"),
    "tie-index-desc": ("order = np.lexsort((ids, -s))", "order = np.lexsort((-ids, -s))"),
    "order-ascending": ("order = np.lexsort((ids, -s))", "order = np.lexsort((ids, s))"),
    "cut-strict": ("hit = np.nonzero(c >= p * E)[0]", "hit = np.nonzero(c > p * E)[0]"),
    "cut-off-by-one": ("m = int(hit[0]) + 1 if len(hit) else n", "m = int(hit[0]) if len(hit) else n"),
    "cut-no-max-shift": ("e = np.exp(s - s.max())", "e = np.exp(s)"),
    "no-orphans": ("out.append(np.arange(lo, nc[level - 1], dtype=np.int64))", "out.append(np.arange(lo, lo, dtype=np.int64))"),
    "children-short": ("np.arange(pnode * b, pnode * b + b, dtype=np.int64)", "np.arange(pnode * b, pnode * b + b - 1, dtype=np.int64)"),
    "expand-all-candidates": ("parents = c.selected", "parents = c.ids"),
    "ceil-complete-nodes": ("return [n_tokens // (b ** l) for l in range(1, n_levels + 1)]",
                            "return [-(-n_tokens // (b ** l)) for l in range(1, n_levels + 1)]"),
    "no-sink": ("toks[0] = True", "toks[0] = toks[0]"),
    "cur-chunk-off": ("toks[b * ((n_visible - 1) // b):n_visible] = True", "toks[b * (n_visible // b):n_visible] = True"),
    "score-no-scale": ("s64 = scale * (np.asarray(X[ids], dtype=F64) @ np.asarray(q, dtype=F64))",
                       "s64 = (np.asarray(X[ids], dtype=F64) @ np.asarray(q, dtype=F64))"),
    "attend-no-scale": ("z = scale * (k @ np.asarray(q, dtype=F64))", "z = (k @ np.asarray(q, dtype=F64))"),
    "attend-unnormalised": ("return (e @ v) / l, mx + math.log(l)", "return (e @ v) / e.max(), mx + math.log(l)"),
    "lse-no-max": ("return (e @ v) / l, mx + math.log(l)", "return (e @ v) / l, math.log(l)"),
    "span-off": ("return b ** level", "return b ** (level + 1)"),
    "level-p-reversed": ("return float(p) if np.ndim(p) == 0 else float(p[level - 1])",
                         "return float(p) if np.ndim(p) == 0 else float(p[-level])"),
    "level-p-first-only": ("return float(p) if np.ndim(p) == 0 else float(p[level - 1])",
                           "return float(p) if np.ndim(p) == 0 else float(p[0])"),
    "tangent-offset-sign": ("offs[:, r] = (lse - scale * (kh @ q)).astype(F32)",
                            "offs[:, r] = (scale * (kh @ q) - lse).astype(F32)"),
    "tangent-score-no-offset": ("return (scale * (k @ np.asarray(q, dtype=F64)) + o).max(axis=1)",
                                "return (scale * (k @ np.asarray(q, dtype=F64))).max(axis=1)"),
    "tangent-mean-over-refs": ("return (scale * (k @ np.asarray(q, dtype=F64)) + o).max(axis=1)",
                               "return (scale * (k @ np.asarray(q, dtype=F64)) + o).mean(axis=1)"),
    "tangent-child-offsets-dropped": ("t = scale * (X @ q) + O", "t = scale * (X @ q) + 0 * O"),
    "tangent-first-child-tangent": ("best = np.argmax(t, axis=2)", "best = np.zeros_like(np.argmax(t, axis=2))"),
    "tangent-lse-no-max": ("lse = zm[:, 0] + np.log(e.sum(axis=1))", "lse = np.log(e.sum(axis=1))"),
    "tangent-same-ref-every-level": ("levels.append(tangent_pool(up.keys, up.offs, R[l], b, scale))",
                                     "levels.append(tangent_pool(up.keys, up.offs, R[0], b, scale))"),
    "values-uniform-weights": ("w, _ = pool_weights(children, r, b, scale)",
                               "w, _ = pool_weights(children, 0 * np.asarray(r), b, scale)"),
    "pseudo-no-count-offset": ("logits.append(float(cut.scores64[j]) + math.log(count))",
                               "logits.append(float(cut.scores64[j]))"),
    "pseudo-whole-span": ("count = span - (1 if lo == 0 else 0) - max(0, min(n_visible, hi) - max(cur, lo))",
                          "count = span"),
    "pseudo-includes-kept": ("            if node in kept:\n                continue\n", ""),
    "pseudo-level-span-off": ("span = b ** level\n        for j, node", "span = b ** (level - 1)\n        for j, node"),
    "exempt-all": ("return np.array(sorted(ex), dtype=np.int64)",
                   "return np.array(sorted(int(i) for i in cut.ids), dtype=np.int64)"),
    "exempt-none": ("return np.array(sorted(ex), dtype=np.int64)", "return np.array([], dtype=np.int64)"),
    "exempt-ties": ("diff = cut.scores64[cand_out] != cut.scores64[x]",
                    "diff = cut.scores64[cand_out] == cut.scores64[cand_out]"),
    "exempt-same-side": ("cand_out = outside[wo > lo_in - margin]", "cand_out = inside[wi > lo_in - margin]"),
    "exempt-prefix-after": ("if abs(cut.prefix[k] - p) < margin:", "if abs(cut.prefix[k + 1] - p) < margin:"),
    "exempt-margin-wide": ("margin: float = 1e-5", "margin: float = 1e-4"),
    "exempt-no-rule-i": ("ex.add(int(cut.ids[cut.order[k]]))", "pass"),
    "exempt-one-sided": ("                for y in cand_out[close & diff]:\n                    ex.add(int(cut.ids[y]))\n",
                         ""),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"pattern for {name} must occur exactly once"
    modname = f"zha_oracle_mutant_{name.replace('-', '_')}"
    mod = types.ModuleType(modname)
    sys.modules[modname] = mod          # dataclasses look their module up here
    exec(compile(src.replace(old, new), SRC + f"[{name}]", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
