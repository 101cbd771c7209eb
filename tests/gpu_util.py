"""GPU-test helpers: run the HIP decoder through the C ABI and compare it with the
oracle lane by lane (arc ids and words bit-exact, scores within 1e-4 and in
practice bit-equal, and the per-step counters equal)."""

from __future__ import annotations

import os

import numpy as np

import oracle
import wfst_beam_search_amd as wb

ORACLE_THREADS = min(16, os.cpu_count() or 1)
SCORE_TOL = 1e-4
OIDX = {name: i for i, name in enumerate(oracle.FIELDS)}
GIDX = {name: i for i, name in enumerate(wb.STEP_FIELDS)}


def gpu_decode(graph, lp, lengths, beam, max_active, min_active=0, allow_partial=False,
               eps_iterations=0, use_graphs=True, max_lanes=None, max_frames=None, dgraph=None,
               with_steps=True, **caps):
    import torch
    B, T, V = lp.shape
    own = dgraph is None
    g = wb.Graph(graph) if own else dgraph
    dec = wb.Decoder(g, beam, max_active, min_active=min_active, allow_partial=allow_partial,
                     max_lanes=max_lanes or B, max_frames=max_frames or max(T, 1),
                     lp_dtype="f16" if lp.dtype == np.float16 else "f32",
                     eps_iterations=eps_iterations, use_graphs=use_graphs,
                     **caps)
    x = torch.from_numpy(np.ascontiguousarray(lp)).cuda()
    r = dec.decode(x, lengths)
    steps = [dec.step_stats(b) for b in range(B)] if with_steps else None
    stats = dec.stats()
    dec.close()
    if own:
        g.release()
    return r, steps, stats


def oracle_lanes(graph, lp, lengths, beam, max_active, min_active=0, allow_partial=False,
                 eps_iterations=0, lanes=None):
    og = oracle.OracleGraph(graph)
    return oracle.decode_batch(og, lp, lengths, beam, max_active, min_active, allow_partial,
                               eps_iterations, lanes=lanes, threads=ORACLE_THREADS)


def _f(bits):
    return np.array(int(bits) & 0xFFFFFFFF, dtype=np.uint32).view(np.float32)[()]


def compare_lane(b, r, steps, o, check_steps=True):
    """Assert GPU lane b equals the oracle's result o."""
    tag = f"lane {b}"
    assert int(r.meta[b, 2]) == 0, f"{tag}: overflow bits {r.meta[b, 2]}"
    assert int(r.meta[b, 0]) == 1, f"{tag}: ok = 0"
    assert int(r.meta[b, 1]) == o["reached_final"], f"{tag}: reached_final"
    assert np.array_equal(r.arcs[b], o["arcs"]), f"{tag}: arc ids differ"
    assert np.array_equal(r.words[b], o["words"]), f"{tag}: words differ"
    gs, os_ = np.float32(r.scores[b]), np.float32(o["score"])
    if np.isneginf(os_):
        assert np.isneginf(gs), f"{tag}: score {gs} vs -inf"
    else:
        assert abs(float(gs) - float(os_)) <= SCORE_TOL, f"{tag}: score {gs!r} vs {os_!r}"
    if not check_steps or steps is None:
        return
    st = steps[b]
    ost = o["steps"]
    sc = o["start_closure"]
    assert list(st[0, [GIDX[k] for k in ("eps_arcs", "eps_admitted", "eps_distinct", "eps_new",
                                           "eps_replaced", "eps_passes")]]) == list(sc[:6]), f"{tag}: start closure"
    for t in range(ost.shape[0]):
        g = st[t + 1]
        oo = ost[t]
        for k in ("n", "arcs", "admitted", "distinct", "eps_arcs", "eps_admitted", "eps_distinct",
                  "eps_new", "eps_replaced", "eps_passes", "phase"):
            assert g[GIDX[k]] == oo[OIDX[k]], f"{tag} step {t}: {k} {g[GIDX[k]]} vs {oo[OIDX[k]]}"
        for k in ("beam", "max"):
            assert (int(g[GIDX[k]]) & 0xFFFFFFFF) == (int(oo[OIDX[k]]) & 0xFFFFFFFF), \
                f"{tag} step {t}: {k} {_f(g[GIDX[k]])!r} vs {_f(oo[OIDX[k]])!r}"
    for t in range(ost.shape[0] + 1, st.shape[0]):
        assert st[t, GIDX["phase"]] == -1, f"{tag}: step {t - 1} ran after the lane ended"


def compare_batch(r, steps, ors, lanes=None, check_steps=True):
    lanes = list(range(len(ors))) if lanes is None else list(lanes)
    for b, o in zip(lanes, ors):
        compare_lane(b, r, steps, o, check_steps)
