"""Test helpers: graphs written out in the golden JSON files, and path checks."""

from __future__ import annotations

import json
import os

import numpy as np

from synth import Graph

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(x):
    if isinstance(x, str):
        if x == "-inf":
            return F32(-np.inf)
        return np.array(int(x, 16), dtype=np.uint32).view(np.float32)[()]
    return F32(x)


def graph_from_states(spec) -> Graph:
    """Build a Graph from ``{"start", "vocab", "epsilon_id", "states": [[[dest, il, ol, w], ...], ...]}``."""
    rs = [0]
    dest, il, ol, w = [], [], [], []
    for arcs in spec["states"]:
        for d, i, o, x in arcs:
            dest.append(d); il.append(i); ol.append(o); w.append(_f32(x))
        rs.append(len(dest))
    return Graph(num_states=len(spec["states"]), start=int(spec["start"]), vocab=int(spec["vocab"]),
                 epsilon_id=int(spec["epsilon_id"]), row_splits=np.array(rs, dtype=np.int32),
                 dest=np.array(dest, dtype=np.int32), ilabel=np.array(il, dtype=np.int32),
                 olabel=np.array(ol, dtype=np.int32), weight=np.array(w, dtype=np.float32))


def f32_value(x):
    return _f32(x)


def arc_src(g):
    return np.repeat(np.arange(g.num_states), np.diff(g.row_splits)).astype(np.int64)


def check_path(g, lp_lane, length, arcs, words, score, reached_final):
    """Invariants of a returned best path, from the page's section 1 (relaxation,
    backtrack to words) and section 5.3 (fp32 add order): re-summing the arcs in
    order gives the score bit for bit; the running score never increases; the
    words are the non-zero olabels; the path has `length` emitting arcs then one
    final arc; consecutive arcs chain from the start state."""
    arcs = np.asarray(arcs, dtype=np.int64)
    src = arc_src(g)
    il = g.ilabel
    eps = (il == g.epsilon_id) if g.epsilon_id >= 0 else np.zeros(il.shape, bool)
    if len(arcs) == 0:
        assert len(words) == 0
        return
    s = F32(0.0)
    t = 0
    state = g.start
    prev = s
    for k, a in enumerate(arcs):
        assert src[a] == state, f"arc {a} does not leave state {state}"
        if il[a] == -1:
            assert k == len(arcs) - 1, "final arc must be last"
            s = F32(s + g.weight[a])
        elif eps[a]:
            s = F32(s + g.weight[a])
        else:
            s = F32(F32(s + g.weight[a]) + F32(lp_lane[t, il[a]]))
            t += 1
        assert s <= prev, "score increased along the path"
        prev = s
        state = int(g.dest[a])
    assert t == length, f"path has {t} emitting arcs, expected {length}"
    if reached_final:
        assert il[arcs[-1]] == -1 and state == g.num_states - 1
    assert s == F32(score) or (np.isneginf(s) and np.isneginf(score)), f"resummed {s!r} != {score!r}"
    ol = g.olabel[arcs]
    assert np.array_equal(ol[ol != 0], np.asarray(words)), "words are not the path's olabels"
