"""Exhaustive references that pin the CPU oracle on tiny inputs (test-only).

Both functions are written independently of the oracle (no pruning, no frontier,
no hash): they follow the plain definition of the best path score of a weighted
automaton against CTC frames, in the max-plus semiring, with the fp32 addition
order of the page "GPU WFST Beam-Search Decoder", section 5.3 (an emitting arc
adds its weight and then the frame's log-prob; epsilon and final arcs add only
their weight).

* ``viterbi_exact``: a full trellis dynamic program that updates every state at
  every frame (infinite beam), with the epsilon closure computed to a fixpoint.
* ``viterbi_partial``: the same trellis stopped after T frames, best state
  without a final arc (the partial hypothesis of a stream).
* ``complete_paths``: every complete path of an epsilon-free graph with its
  score (the lattice pins compare kept arcs with them).
* ``enumerate_paths``: lists every path (at most ``max_eps`` epsilon arcs
  between frames) and takes the maximum.
* ``complete_paths_framed``: every complete path (at most ``max_eps`` epsilon
  arcs between frames) with its score and each arc tagged with the frame it
  runs in (an epsilon arc: the number of emitting arcs before it; an emitting
  arc: its frame; the final arc: T).
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
NEG = F32(-np.inf)


def _arc_src(g):
    return np.repeat(np.arange(g.num_states), np.diff(g.row_splits))


def _classes(g):
    il = g.ilabel
    final = il == -1
    eps = (il == g.epsilon_id) if g.epsilon_id >= 0 else np.zeros_like(final)
    emit = ~final & ~eps
    return final, eps, emit


def _trellis(g, lp, T):
    """Scores, one best path and tie flags of every state after T frames of the
    full trellis (epsilon closure to a fixpoint after the start and every frame)."""
    src = _arc_src(g)
    final, eps, emit = _classes(g)
    S = g.num_states
    score = [NEG] * S
    path = [None] * S
    tie = [False] * S
    score[g.start] = F32(0.0)
    path[g.start] = []

    def closure():
        changed = True
        while changed:
            changed = False
            for a in np.nonzero(eps)[0]:
                s, d = int(src[a]), int(g.dest[a])
                if path[s] is None:
                    continue
                c = F32(score[s] + g.weight[a])
                if path[d] is None or c > score[d]:
                    score[d], path[d], tie[d] = c, path[s] + [int(a)], tie[s]
                    changed = True
                elif c == score[d] and path[s] + [int(a)] != path[d]:
                    tie[d] = True

    closure()
    for t in range(T):
        ns, npth, ntie = [NEG] * S, [None] * S, [False] * S
        for a in np.nonzero(emit)[0]:
            s, d = int(src[a]), int(g.dest[a])
            if path[s] is None:
                continue
            c = F32(F32(score[s] + g.weight[a]) + F32(lp[t, g.ilabel[a]]))
            if npth[d] is None or c > ns[d]:
                ns[d], npth[d], ntie[d] = c, path[s] + [int(a)], tie[s]
            elif c == ns[d]:
                ntie[d] = True
        score, path, tie = ns, npth, ntie
        closure()
    return score, path, tie


def viterbi_exact(g, lp, T):
    """Best score and one best path over the full graph x frames trellis.

    Returns (score, arcs, tied) where ``tied`` says whether any maximum on the
    returned path was reached by more than one candidate (then the path is not
    unique and only the score is meaningful).
    """
    src = _arc_src(g)
    final, _, _ = _classes(g)
    score, path, tie = _trellis(g, lp, T)
    best, bpath, btie = None, None, False
    for a in np.nonzero(final)[0]:
        s = int(src[a])
        if path[s] is None:
            continue
        c = F32(score[s] + g.weight[a])
        if bpath is None or c > best:
            best, bpath, btie = c, path[s] + [int(a)], tie[s]
        elif c == best:
            btie = True
    if bpath is None:
        return NEG, [], False
    return best, bpath, btie


def viterbi_partial(g, lp, T):
    """Best state of the trellis after T frames (no final arc): its score and path.

    Returns (score, arcs, tied); ``tied`` is set when another state reaches the
    same score or the path itself was tied."""
    score, path, tie = _trellis(g, lp, T)
    best, bpath, btie = None, None, False
    for s in range(g.num_states):
        if path[s] is None:
            continue
        if bpath is None or score[s] > best:
            best, bpath, btie = score[s], path[s], tie[s]
        elif score[s] == best:
            btie = True
    if bpath is None:
        return NEG, [], False
    return best, bpath, btie


def enumerate_paths(g, lp, T, max_eps):
    """Maximum over every path of the form e* (x e*)^T f with at most ``max_eps``
    epsilon arcs per e* run. Returns (score, arcs, number of paths at the max)."""
    final, eps, emit = _classes(g)
    rs = g.row_splits
    best = [NEG, None, 0]

    def rec(s, t, sc, arcs, eps_left):
        for a in range(rs[s], rs[s + 1]):
            if eps[a] and eps_left > 0:
                rec(int(g.dest[a]), t, F32(sc + g.weight[a]), arcs + [a], eps_left - 1)
            elif emit[a] and t < T:
                c = F32(F32(sc + g.weight[a]) + F32(lp[t, g.ilabel[a]]))
                rec(int(g.dest[a]), t + 1, c, arcs + [a], max_eps)
            elif final[a] and t == T:
                c = F32(sc + g.weight[a])
                if best[1] is None or c > best[0]:
                    best[0], best[1], best[2] = c, arcs + [a], 1
                elif c == best[0]:
                    best[2] += 1

    rec(g.start, 0, F32(0.0), [], max_eps)
    return best[0], (best[1] or []), best[2]


def complete_paths(g, lp, T):
    """Every path x^T f of an epsilon-free graph from the start state: a list of
    (score, arcs) with the fp32 left-to-right score of section 5.3."""
    final, _, emit = _classes(g)
    rs = g.row_splits
    out = []

    def rec(s, t, sc, arcs):
        for a in range(rs[s], rs[s + 1]):
            if emit[a] and t < T:
                rec(int(g.dest[a]), t + 1, F32(F32(sc + g.weight[a]) + F32(lp[t, g.ilabel[a]])), arcs + [a])
            elif final[a] and t == T:
                out.append((F32(sc + g.weight[a]), arcs + [a]))

    rec(g.start, 0, F32(0.0), [])
    return out


def complete_paths_framed(g, lp, T, max_eps):
    """Every path e* (x e*)^T f from the start state, at most ``max_eps`` epsilon
    arcs per e* run: a list of (score, [(frame, arc), ...]) with the fp32
    left-to-right score of section 5.3."""
    final, eps, emit = _classes(g)
    rs = g.row_splits
    out = []

    def rec(s, t, sc, arcs, eps_left):
        for a in range(rs[s], rs[s + 1]):
            if eps[a] and eps_left > 0:
                rec(int(g.dest[a]), t, F32(sc + g.weight[a]), arcs + [(t, int(a))], eps_left - 1)
            elif emit[a] and t < T:
                c = F32(F32(sc + g.weight[a]) + F32(lp[t, g.ilabel[a]]))
                rec(int(g.dest[a]), t + 1, c, arcs + [(t, int(a))], max_eps)
            elif final[a] and t == T:
                out.append((F32(sc + g.weight[a]), arcs + [(t, int(a))]))

    rec(g.start, 0, F32(0.0), [], max_eps)
    return out
