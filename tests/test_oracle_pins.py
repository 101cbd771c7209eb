"""Pins of the CPU oracle against things other than itself (no GPU needed).

* hand-traced golden cases (tests/golden/*.json, each citing its passage);
* the exact Viterbi score of a full trellis DP and exhaustive path enumeration on
  tiny graphs at infinite beam (the beam search reduces to them exactly);
* closed forms: greedy CTC on a one-state graph (numpy argmax / running sum) and
  forced alignment on a linear chain;
* invariants of every returned path on the five workloads.
"""

import numpy as np
import pytest

import oracle
import synth
from bruteforce import complete_paths, complete_paths_framed, enumerate_paths, viterbi_exact, viterbi_partial
from cases import check_path, f32_value, graph_from_states, load_golden

F32 = np.float32
IDX = {name: i for i, name in enumerate(oracle.FIELDS)}


def _bits(x):
    return int(np.array(F32(x)).view(np.uint32))


def _decode(g, lp, T, beam, max_active, min_active=0, allow_partial=False, eps=0,
            online=False, partial=False):
    return oracle.decode_lane(g, lp, T, beam, max_active, min_active, allow_partial, eps,
                              online=online, partial=partial)


def _const_lp(frames, vocab, value):
    return np.full((frames, vocab), value, dtype=np.float32)


# ---------------------------------------------------------------- golden cases

@pytest.mark.parametrize("case", load_golden("beam_schedule.json")["cases"], ids=lambda c: c["name"])
def test_golden_beam_schedule(case):
    spec = load_golden("beam_schedule.json")["graphs"][case["graph"]]
    g = graph_from_states(spec)
    lp = _const_lp(case["frames"], g.vocab, case["lp_value"])
    r = _decode(g, lp, case["frames"], case["beam"], case["max_active"], case["min_active"])
    st = r["steps"]
    assert list(st[:, IDX["n"]]) == case["expect_n"]
    assert [hex(int(x)) for x in st[:, IDX["beam"]]] == case["expect_beam_hex"]
    got_max = np.array(st[:, IDX["max"]], dtype=np.uint32).view(np.float32)
    assert list(got_max) == [F32(x) for x in case["expect_max"]]
    assert list(r["arcs"]) == case["expect_arcs"]
    assert r["score"] == F32(case["expect_score"])
    assert r["reached_final"] == 1


def test_golden_tie_chain():
    case = load_golden("tie_chain.json")
    g = graph_from_states(case["graph"])
    lp = _const_lp(case["frames"], g.vocab, case["lp_value"])
    r = _decode(g, lp, case["frames"], case["beam"], case["max_active"], case["min_active"])
    assert list(r["arcs"]) == case["expect_arcs"]
    assert list(r["words"]) == case["expect_words"]
    assert r["score"] == F32(case["expect_score"])
    assert r["reached_final"] == case["expect_reached_final"]


def test_golden_eps_closure():
    case = load_golden("eps_closure.json")
    g = graph_from_states(case["graph"])
    lp = np.array(case["lp_rows"], dtype=np.float32)
    r = _decode(g, lp, case["frames"], case["beam"], case["max_active"], case["min_active"],
                eps=case["eps_iterations"])
    assert list(r["arcs"]) == case["expect_arcs"]
    assert list(r["words"]) == case["expect_words"]
    assert r["score"] == F32(case["expect_score"])
    sc = case["expect_start_closure"]
    assert list(r["start_closure"][:7]) == [sc["eps_arcs"], sc["admitted"], sc["distinct"], sc["new"],
                                            sc["replaced"], sc["passes"], sc["n_after"]]
    s0 = r["steps"][0]
    for k, v in case["expect_step0"].items():
        got = s0[IDX[k]]
        if k in ("beam", "max", "cutoff"):
            assert got == _bits(v), k
        else:
            assert got == v, k


@pytest.mark.parametrize("case", load_golden("edge_cases.json")["cases"], ids=lambda c: c["name"])
def test_golden_edge_cases(case):
    g = graph_from_states(case["graph"])
    lp = np.array(case["lp_rows"], dtype=np.float32).reshape(case["frames"], g.vocab)
    r = _decode(g, lp, case["frames"], case["beam"], case["max_active"], case["min_active"],
                allow_partial=bool(case["allow_partial"]), eps=case.get("eps_iterations", 0))
    assert list(r["arcs"]) == case["expect_arcs"]
    assert list(r["words"]) == case["expect_words"]
    exp = f32_value(case["expect_score"])
    assert (r["score"] == exp) or (np.isneginf(exp) and np.isneginf(r["score"]))
    assert r["reached_final"] == case["expect_reached_final"]
    assert r["dead"] == case["expect_dead"]
    for k, v in case.get("expect_step0", {}).items():
        assert r["steps"][0][IDX[k]] == v, k


# ----------------------------------------------------- exact search at infinite beam

INF_BEAM = 1e10


def _tiny(seed, eps):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 9))
    vocab = int(rng.integers(2, 6))
    g = synth.random_graph(seed, n=n, deg=(1, 3), vocab=vocab, epsilon=eps, eps_levels=3,
                           self_loop=0.3 if seed % 2 else 0.0)
    T = int(rng.integers(0, 7))
    lp = synth.random_logprobs(seed + 7, 1, max(T, 1), vocab)[0]
    return g, lp, T


@pytest.mark.parametrize("eps", [False, True])
def test_infinite_beam_equals_exact_viterbi(eps):
    compared_paths = 0
    for seed in range(120):
        g, lp, T = _tiny(seed, eps)
        P = 2 if eps else 0
        r = _decode(g, lp, T, INF_BEAM, 1 << 20, eps=P)
        best, path, tied = viterbi_exact(g, lp, T)
        assert r["reached_final"] == 1
        assert r["score"] == best, (seed, r["score"], best)
        if not tied:
            assert list(r["arcs"]) == path, seed
            compared_paths += 1
        check_path(g, lp, T, r["arcs"], r["words"], r["score"], 1)
    assert compared_paths > 80


@pytest.mark.parametrize("eps", [False, True])
def test_infinite_beam_equals_path_enumeration(eps):
    unique = 0
    for seed in range(200, 260):
        rng = np.random.default_rng(seed)
        n = int(rng.integers(2, 7))
        vocab = int(rng.integers(2, 5))
        g = synth.random_graph(seed, n=n, deg=(1, 3), vocab=vocab, epsilon=eps, eps_levels=3)
        T = int(rng.integers(0, 6))
        lp = synth.random_logprobs(seed, 1, max(T, 1), vocab)[0]
        P = 2 if eps else 0
        r = _decode(g, lp, T, INF_BEAM, 1 << 20, eps=P)
        best, path, count = enumerate_paths(g, lp, T, P)
        assert r["score"] == best, seed
        if count == 1:
            assert list(r["arcs"]) == path, seed
            unique += 1
    assert unique > 40


def test_deeper_closure_needs_more_passes():
    """A 3-arc epsilon chain 0 -> 1 -> 2 -> 3 (only state 3 final) is closed by
    3 passes and not by 2: each pass extends chains by one arc."""
    spec = {"start": 0, "vocab": 2, "epsilon_id": 0,
            "states": [[[1, 0, 0, -0.5]], [[2, 0, 0, -0.25]], [[3, 0, 0, -0.125]],
                       [[3, 1, 0, 0.0], [4, -1, 0, 0.0]], []]}
    g = graph_from_states(spec)
    for T in (0, 1, 3):
        lp = synth.random_logprobs(T, 1, max(T, 1), 2)[0]
        best, path, _ = viterbi_exact(g, lp, T)
        r3 = _decode(g, lp, T, 10.0, 100, eps=3)
        assert r3["score"] == best and list(r3["arcs"]) == path
        r2 = _decode(g, lp, T, 10.0, 100, eps=2)
        if T == 0:
            assert r2["reached_final"] == 0 and np.isneginf(r2["score"])
        else:
            assert r2["score"] <= best


def test_pruned_score_never_beats_exact():
    for seed in range(400, 480):
        g, lp, T = _tiny(seed, seed % 3 == 0)
        best, _, _ = viterbi_exact(g, lp, T)
        r = _decode(g, lp, T, 1.5, 2, eps=2 if seed % 3 == 0 else 0)
        if r["reached_final"]:
            assert r["score"] <= best
            check_path(g, lp, T, r["arcs"], r["words"], r["score"], 1)


# ------------------------------------------------------------------ closed forms

def _greedy_graph(vocab):
    """One state with a self-loop per label (arc id = label, weight 0) and a final arc."""
    spec = {"start": 0, "vocab": vocab, "epsilon_id": -1,
            "states": [[[0, v, v + 1, 0.0] for v in range(vocab)] + [[1, -1, 0, 0.0]], []]}
    return graph_from_states(spec)


@pytest.mark.parametrize("vocab,frames", [(5, 12), (32, 50), (500, 30)])
def test_greedy_ctc_closed_form(vocab, frames):
    g = _greedy_graph(vocab)
    lp = synth.random_logprobs(vocab * 7 + frames, 1, frames, vocab, sigma=3.0)[0]
    r = _decode(g, lp, frames, 10.0, 100)
    expect_arcs = list(np.argmax(lp, axis=1)) + [vocab]
    s = F32(0.0)
    for t in range(frames):
        s = F32(s + lp[t].max())
    assert list(r["arcs"]) == expect_arcs
    assert r["score"] == s
    assert list(r["words"]) == [a + 1 for a in expect_arcs[:-1]]


def test_greedy_ctc_ties_take_smallest_label():
    g = _greedy_graph(6)
    lp = _const_lp(9, 6, -1.75)
    r = _decode(g, lp, 9, 10.0, 100)
    assert list(r["arcs"]) == [0] * 9 + [6]


def test_forced_alignment_closed_form():
    rng = np.random.default_rng(5)
    T, V = 40, 17
    labels = rng.integers(0, V, size=T)
    w = np.log(rng.uniform(0.1, 1.0, size=T)).astype(np.float32)
    states = [[[k + 1, int(labels[k]), k + 1, float(w[k])]] for k in range(T)]
    states.append([[T + 1, -1, 0, 0.0]])
    states.append([])
    g = graph_from_states({"start": 0, "vocab": V, "epsilon_id": -1, "states": states})
    lp = synth.random_logprobs(9, 1, T, V)[0]
    r = _decode(g, lp, T, 10.0, 100)
    s = F32(0.0)
    for k in range(T):
        s = F32(F32(s + w[k]) + lp[k, labels[k]])
    assert r["score"] == s
    assert list(r["arcs"]) == list(range(T)) + [T]


# ------------------------------------------------------ dynamic beam consistency

def _recompute_beams(steps, length, beam, max_active, min_active, online=False):
    out, bp = [], F32(beam)
    for t, n in enumerate(steps[:, IDX["n"]]):
        if t == length:
            out.append(F32(1e10)); continue
        mina = max(min_active, max_active // 2) if (length - t <= 5 and not online) else min_active
        if n > max_active:
            b = F32(min(bp, F32(beam)) * F32(0.8))
        elif n < mina:
            b = F32(max(bp, F32(beam)) * F32(1.25))
        else:
            b = F32(F32(F32(0.8) * bp) + F32(F32(0.2) * F32(beam)))
        out.append(b); bp = b
    return np.array(out, dtype=np.float32)


@pytest.mark.parametrize("cid", [1, 2])
def test_logged_beams_follow_the_update_rule(cid):
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    for b in range(min(wl.batch, 3)):
        r = _decode(g, lp[b], int(L[b]), wl.beam, wl.max_active)
        st = r["steps"]
        got = np.array(st[:, IDX["beam"]], dtype=np.uint32).view(np.float32)
        assert np.array_equal(got, _recompute_beams(st, int(L[b]), wl.beam, wl.max_active, 0))
        # soft cap: the frontier is allowed to exceed max_active
        cut = np.array(st[:, IDX["cutoff"]], dtype=np.uint32).view(np.float32)
        mx = np.array(st[:, IDX["max"]], dtype=np.uint32).view(np.float32)
        assert np.array_equal(cut[:-1], (mx - got)[:-1])


# ------------------------------------------------------ invariants on workloads

@pytest.mark.parametrize("cid,lanes", [(1, [0]), (2, list(range(8))), (5, [0, 1]), (4, [0]), (3, [0])])
def test_workload_paths_are_consistent(cid, lanes):
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    og = oracle.OracleGraph(g)
    rs = oracle.decode_batch(og, lp, L, wl.beam, wl.max_active, eps_iterations=wl.eps_iterations,
                             lanes=lanes, threads=len(lanes))
    for b, r in zip(lanes, rs):
        assert r["reached_final"] == 1 and r["dead"] == 0
        check_path(g, lp[b].astype(np.float32), int(L[b]), r["arcs"], r["words"], r["score"], 1)
        st = r["steps"]
        assert st.shape[0] == int(L[b]) + 1
        assert np.all(st[:, IDX["distinct"]] <= st[:, IDX["admitted"]])
        assert np.all(st[:, IDX["admitted"]] <= st[:, IDX["arcs"]])
        if not wl.epsilon:
            assert np.array_equal(st[:-1, IDX["n_next"]], st[1:, IDX["n"]])
            assert np.array_equal(st[:, IDX["n_next"]], st[:, IDX["distinct"]])


# ------------------------------------------- streaming: online beam, partial results

@pytest.mark.parametrize("eps", [False, True])
def test_partial_at_infinite_beam_equals_trellis_best(eps):
    """Page section 8: a partial hypothesis is the path of the best current token.
    At infinite beam the frontier is the whole trellis column, so it is the best
    state of the exact trellis after T frames."""
    compared = 0
    for seed in range(500, 620):
        g, lp, T = _tiny(seed, eps)
        P = 2 if eps else 0
        r = _decode(g, lp, T, INF_BEAM, 1 << 20, eps=P, online=True, partial=True)
        best, path, tied = viterbi_partial(g, lp, T)
        assert r["reached_final"] == 0
        assert r["score"] == best, (seed, r["score"], best)
        if not tied:
            assert list(r["arcs"]) == path, seed
            compared += 1
    assert compared > 60


def _no_final_spec(seed):
    """A random graph whose states have no final arc (the super-final state is
    unreachable), so an offline decode with allow_partial always redirects."""
    rng = np.random.default_rng(seed)
    n, vocab = int(rng.integers(2, 8)), int(rng.integers(2, 5))
    states = []
    for _ in range(n):
        arcs = [[int(rng.integers(0, n)), int(rng.integers(0, vocab)), int(rng.integers(0, 3)),
                 float(rng.normal())] for _ in range(int(rng.integers(1, 4)))]
        arcs.sort(key=lambda a: a[1])
        states.append(arcs)
    states.append([])
    return {"start": 0, "vocab": vocab, "epsilon_id": -1, "states": states}, vocab


def test_partial_equals_redirect_without_final_arcs():
    """Section 3: with no final arc and allow_partial the final step hands the
    result to the best token (key over score + 0); the partial hypothesis takes
    the best token too. With distinct scores both name the same token, and with
    min_active >= max_active / 2 the offline "last frames" clause changes nothing."""
    checked = 0
    for seed in range(700, 780):
        spec, vocab = _no_final_spec(seed)
        g = graph_from_states(spec)
        T = int(np.random.default_rng(seed).integers(1, 8))
        lp = synth.random_logprobs(seed, 1, T, vocab)[0]
        off = _decode(g, lp, T, 3.0, 6, min_active=3, allow_partial=True)
        on = _decode(g, lp, T, 3.0, 6, min_active=3, online=True, partial=True)
        if off["dead"]:
            assert on["dead"] == 1
            continue
        assert off["steps"][-1, IDX["phase"]] == oracle.PHASE_REDIRECT
        assert on["score"] == off["score"] and list(on["arcs"]) == list(off["arcs"]), seed
        assert list(on["words"]) == list(off["words"])
        checked += 1
    assert checked > 50


@pytest.mark.parametrize("cid", [1, 2])
def test_online_beams_skip_the_final_window(cid):
    """Section 3: a stream's length is unknown until it ends, so the raise of
    min_active over the last frames never happens; every other beam rule holds."""
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    differs = 0
    for b in range(min(wl.batch, 3)):
        r = _decode(g, lp[b], int(L[b]), wl.beam, wl.max_active, online=True)
        st = r["steps"]
        got = np.array(st[:, IDX["beam"]], dtype=np.uint32).view(np.float32)
        assert np.array_equal(got, _recompute_beams(st, int(L[b]), wl.beam, wl.max_active, 0, online=True))
        off = _decode(g, lp[b], int(L[b]), wl.beam, wl.max_active)
        differs += int(not np.array_equal(off["steps"], st))
    assert differs > 0   # the clause matters on these lanes, so the test can fail


def test_online_equals_offline_when_the_final_window_is_inert():
    for seed in range(800, 860):
        g, lp, T = _tiny(seed, seed % 2 == 1)
        P = 2 if seed % 2 else 0
        kw = dict(eps=P, min_active=2)
        a = _decode(g, lp, T, 1.5, 4, **kw)
        b = _decode(g, lp, T, 1.5, 4, online=True, **kw)
        assert a["score"] == b["score"] or (np.isneginf(a["score"]) and np.isneginf(b["score"]))
        assert list(a["arcs"]) == list(b["arcs"]) and np.array_equal(a["steps"], b["steps"])


def test_partial_prefix_of_final_steps():
    """A partial result after t frames is the search state after those frames:
    its records are the first t records of the whole (online) decode."""
    g, lp, L = synth.workload_inputs(2)
    wl = synth.WORKLOADS[2]
    T = int(L[0])
    full = _decode(g, lp[0], T, wl.beam, wl.max_active, online=True)
    for t in (0, 1, 17, T // 2, T):
        part = _decode(g, lp[0], t, wl.beam, wl.max_active, online=True, partial=True)
        assert np.array_equal(part["steps"], full["steps"][:t])
        check_path(g, lp[0].astype(np.float32), t, part["arcs"], part["words"], part["score"], 0)


# ------------------------------------------------ lattice: backward pass and prune

LF = {name: i for i, name in enumerate(oracle.LAT_FIELDS)}


def _lat(g, lp, T, beam, max_active, output_beam, **kw):
    return oracle.decode_lane(g, lp, T, beam, max_active, output_beam=output_beam, **kw)


EPS_FLAG = 4    # lattice record flag of an epsilon arc (it stays in its frame)


def _next_node(r):
    """The lattice node an arc record enters: (frame + 1, dst), or (frame, dst)
    for an epsilon arc, which runs inside its frame."""
    f = int(r[LF["frame"]])
    return (f if int(r[LF["flags"]]) == EPS_FLAG else f + 1, int(r[LF["dst"]]))


def _continuations(lat, sf):
    """Best right-folded continuation score of every lattice node (frame, state),
    by listing every continuation path to the super-final state explicitly."""
    out_arcs = {}
    for k, r in enumerate(lat["lattice"]):
        out_arcs.setdefault((int(r[LF["frame"]]), int(r[LF["src"]])), []).append(k)
    vals = lat["lattice_vals"]

    def paths(node):
        res = []
        for k in out_arcs.get(node, []):
            r = lat["lattice"][k]
            s = F32(vals[k, 1])
            if int(r[LF["dst"]]) == sf:
                res.append([s])
            else:
                for p in paths(_next_node(r)):
                    res.append([s] + p)
        return res

    def fold(p):
        acc = F32(0.0)
        for s in reversed(p):
            acc = F32(s + acc)
        return acc

    best = {}
    for node in out_arcs:
        ps = paths(node)
        best[node] = max((fold(p) for p in ps), default=F32(-np.inf))
    return best


def test_lattice_backward_scores_are_best_continuations():
    """Section 3 / 7 "Lattice": bwd(dst) of every arc is the best score of a
    continuation from its destination to the super-final state, each path's score
    folded from its last arc back (its own recursion, written out as lists)."""
    checked = 0
    for seed in range(900, 960):
        g, lp, T = _tiny(seed, False)
        r = _lat(g, lp, T, 4.0, 50, 3.0)
        if r["reached_final"] != 1:
            continue
        sf = g.num_states - 1
        best = _continuations(r, sf)
        for k, rr in enumerate(r["lattice"]):
            dst = int(rr[LF["dst"]])
            want = F32(0.0) if dst == sf else best.get((int(rr[LF["frame"]]) + 1, dst), F32(-np.inf))
            assert r["lattice_vals"][k, 2] == want, (seed, k)
            checked += 1
    assert checked > 300


def test_lattice_keep_rule_and_best_path():
    """Section 3: output_beam acts only in the backward prune,
    forward[src] + arc + backward[dst] >= best - output_beam; the best path itself
    always survives a positive output_beam."""
    for cid, lanes in ((1, [0]), (2, [0, 3])):
        g, lp, L = synth.workload_inputs(cid)
        wl = synth.WORKLOADS[cid]
        for b in lanes:
            for ob in (0.5, 4.0):
                r = _lat(g, lp[b].astype(np.float32), int(L[b]), wl.beam, wl.max_active, ob)
                v = r["lattice_vals"]
                thr = (v[:, 0] + v[:, 1]).astype(np.float32) + v[:, 2]
                keep = (thr.astype(np.float32) >= np.float32(r["score"] - np.float32(ob))).astype(np.int32)
                assert np.array_equal(keep, r["lattice"][:, LF["keep"]])
                kept = {(int(x[LF["frame"]]), int(x[LF["arc"]])) for x in r["lattice"] if x[LF["keep"]]}
                assert all((t, int(a)) in kept for t, a in enumerate(r["arcs"]))
                st = r["steps"]
                per_frame = np.bincount(r["lattice"][:, LF["frame"]], minlength=st.shape[0])
                assert np.array_equal(per_frame, st[:, IDX["admitted"]])   # every admitted arc is an arc


def test_lattice_at_infinite_beam_is_every_complete_path():
    """At infinite search beam every candidate is admitted; with a wide output beam
    the kept (frame, arc) pairs are exactly the arc occurrences of complete paths,
    and with a narrow one those on a path within output_beam of the best (pairs
    within 1e-4 of the threshold are not checked)."""
    checked = 0
    for seed in range(1000, 1060):
        g, lp, T = _tiny(seed, False)
        paths = complete_paths(g, lp, T)
        if not paths:
            continue
        best = max(p[0] for p in paths)
        for ob in (1e6, 1.0):
            r = _lat(g, lp, T, INF_BEAM, 1 << 20, ob)
            assert r["score"] == best
            kept = {(int(x[LF["frame"]]), int(x[LF["arc"]])) for x in r["lattice"] if x[LF["keep"]]}
            through = {}
            for sc, arcs in paths:
                for t, a in enumerate(arcs):
                    through[(t, a)] = max(through.get((t, a), F32(-np.inf)), sc)
            for key, sc in through.items():
                margin = float(sc) - (float(best) - ob)
                if abs(margin) < 1e-4:
                    continue
                assert (key in kept) == (margin > 0), (seed, ob, key)
                checked += 1
            assert kept <= set(through), seed
    assert checked > 500


def test_lattice_keep_at_exact_ties():
    """Section 3 on output_beam (keep at >=, reading R26), where equality
    happens: with weights and log-probs on a 1/8 grid every sum is exact, so an
    arc occurrence of a complete path scoring sc has (fwd(src) + s) + bwd(dst) at
    least sc, with equality on the best such path. Output beam 0 then keeps
    exactly the arc occurrences of the best-scoring complete paths (ties
    included), output beam 0.5 those of paths within 0.5 of the best."""
    checked = 0
    for seed in range(1100, 1160):
        g, lp, T = _tiny(seed, False)
        if T == 0:
            continue
        rng = np.random.default_rng(seed)
        g.weight = (-rng.integers(0, 9, size=len(g.weight)) / 8.0).astype(np.float32)
        lp = (-rng.integers(0, 17, size=lp.shape) / 8.0).astype(np.float32)
        paths = complete_paths(g, lp, T)
        if not paths:
            continue
        best = max(p[0] for p in paths)
        for ob in (0.0, 0.5):
            r = _lat(g, lp, T, INF_BEAM, 1 << 20, ob)
            assert r["score"] == best
            kept = {(int(x[LF["frame"]]), int(x[LF["arc"]])) for x in r["lattice"] if x[LF["keep"]]}
            want = {(t, a) for sc, arcs in paths if sc >= best - F32(ob) for t, a in enumerate(arcs)}
            assert kept == want, (seed, ob)
            checked += len(want)
    assert checked > 200


def _grid(g, lp, seed):
    """Weights and log-probs on a 1/8 grid (every fp32 sum of a tiny case exact)."""
    rng = np.random.default_rng(seed)
    g.weight = (-rng.integers(0, 9, size=len(g.weight)) / 8.0).astype(np.float32)
    return g, (-rng.integers(0, 17, size=lp.shape) / 8.0).astype(np.float32)


def test_eps_lattice_at_infinite_beam_is_every_path_within_output_beam():
    """Section 5.5 (the candidate set persisted after the closure, epsilon arcs
    tagged), reading R31: at infinite search beam every candidate of every step
    and closure pass is admitted, and with epsilon chains at most P arcs long P
    passes reach every state an epsilon path reaches. With weights and
    log-probs on a 1/8 grid every sum is exact, so the kept (frame, arc) pairs at
    output beam ob are exactly the arc occurrences of complete paths scoring at
    least best - ob, epsilon arcs counted in the frame they run in; each epsilon
    arc is one record per frame (never repeated when several passes admit it),
    tagged with the epsilon id and flag 4."""
    checked = 0
    for seed in range(1200, 1290):
        g, lp, T = _tiny(seed, True)
        if T == 0 or g.epsilon_id < 0:
            continue
        g, lp = _grid(g, lp, seed)
        P = 2   # _tiny's epsilon levels: chains of at most 2 arcs
        paths = complete_paths_framed(g, lp, T, P)
        if not paths:
            continue
        best = max(p[0] for p in paths)
        for ob in (0.0, 0.5, 1e6):
            r = _lat(g, lp, T, INF_BEAM, 1 << 20, ob, eps_iterations=P)
            assert r["score"] == best, seed
            recs = r["lattice"]
            keys = [(int(x[LF["frame"]]), int(x[LF["arc"]])) for x in recs]
            assert len(keys) == len(set(keys)), f"seed {seed}: an arc recorded twice in one frame"
            epsr = recs[recs[:, LF["flags"]] == EPS_FLAG]
            assert np.all(g.ilabel[epsr[:, LF["arc"]]] == g.epsilon_id)
            assert np.all(epsr[:, LF["ilabel"]] == g.epsilon_id)
            kept = {k for k, x in zip(keys, recs) if x[LF["keep"]]}
            want = {fa for sc, arcs in paths if sc >= best - F32(ob) for fa in arcs}
            assert kept == want, (seed, ob)
            checked += sum(1 for f, a in want if g.ilabel[a] == g.epsilon_id)
    assert checked > 100


def test_eps_lattice_backward_scores_are_best_continuations():
    """Reading R31: an epsilon arc's backward term is its destination's best
    continuation inside the same frame (epsilon arcs again, then the frame's step)
    and an emitting arc's that of its destination in the next frame, each
    continuation folded from its last arc back; pruned search (finite beam),
    listing every continuation explicitly."""
    checked = 0
    for seed in range(1300, 1380):
        g, lp, T = _tiny(seed, True)
        r = _lat(g, lp, T, 3.0, 50, 2.0, eps_iterations=2)
        if r["reached_final"] != 1:
            continue
        sf = g.num_states - 1
        best = _continuations(r, sf)
        for k, rr in enumerate(r["lattice"]):
            dst = int(rr[LF["dst"]])
            want = F32(0.0) if dst == sf else best.get(_next_node(rr), F32(-np.inf))
            assert r["lattice_vals"][k, 2] == want, (seed, k)
            checked += int(rr[LF["flags"]]) == EPS_FLAG
    assert checked > 100


def test_eps_lattice_refuses_positive_epsilon_weights():
    """Reading R31: a best continuation needs epsilon weights <= 0 (a positive
    epsilon cycle would raise it without bound), so lattice mode refuses them."""
    g, lp, T = _tiny(1201, True)
    eps = g.ilabel == g.epsilon_id
    assert eps.any()
    g.weight = np.where(eps, np.float32(0.25), g.weight).astype(np.float32)
    with pytest.raises(RuntimeError):
        _lat(g, lp, max(T, 1), 5.0, 50, 1.0, eps_iterations=2)


def _kept(r):
    return {(int(x[LF["frame"]]), int(x[LF["arc"]])) for x in r["lattice"] if x[LF["keep"]]}


@pytest.mark.parametrize("eps", [False, True])
def test_interval_prune_keeps_the_final_keep_set(eps):
    """Section 7 (lat_prune_interval: a window-loose interval prune, the exact
    final pass unchanged), reading R32: on a 1/8 grid every sum is exact, so an
    arc the interval prune removes fails the final test whatever the future
    holds; the final kept set, records and values included, is the same with
    pruning every 1, 2 or 3 steps as without, on pruned searches (finite beam)
    and at every output beam tried; arcs are only ever removed."""
    compared = 0
    for seed in range(1400, 1480):
        g, lp, T = _tiny(seed, eps)
        if T < 2:
            continue
        g, lp = _grid(g, lp, seed)
        P = 2 if eps else 0
        for beam, ob in ((2.0, 0.0), (4.0, 0.5), (INF_BEAM, 1.0)):
            base = _lat(g, lp, T, beam, 50, ob, eps_iterations=P)
            if base["reached_final"] != 1:
                continue
            keep0 = base["lattice"][base["lattice"][:, LF["keep"]] == 1]
            for n in (1, 2, 3):
                r = _lat(g, lp, T, beam, 50, ob, eps_iterations=P, lat_prune_interval=n)
                assert r["score"] == base["score"] and np.array_equal(r["arcs"], base["arcs"])
                keep = r["lattice"][r["lattice"][:, LF["keep"]] == 1]
                o0 = np.lexsort((keep0[:, LF["arc"]], keep0[:, LF["frame"]]))
                o1 = np.lexsort((keep[:, LF["arc"]], keep[:, LF["frame"]]))
                assert np.array_equal(keep[o1], keep0[o0]), (seed, beam, ob, n)
                assert r["lattice"].shape[0] <= base["lattice"].shape[0]
                compared += keep.shape[0]
    assert compared > 300


def test_interval_prune_bounds_the_live_lattice():
    """Reading R32: with pruning every N steps the arcs held at once grow with
    the utterance only about as fast as the arcs within output_beam of the
    local best do, a fraction of the growth without pruning (every admitted
    arc); the kept set is the same (pruned search on random graphs, lanes of 200
    and 400 frames)."""
    for gs in (5, 7):
        g = synth.random_graph(gs, n=30, deg=(1, 6), vocab=6, self_loop=0.3)
        lp = synth.random_logprobs(6, 1, 400, g.vocab, sigma=2.0)[0]
        live = {}
        for T in (200, 400):
            for n in (0, 8):
                r = _lat(g, lp, T, 6.0, 100, 2.0, lat_prune_interval=n)
                assert r["reached_final"] == 1
                live[T, n] = r["lattice_max_live"]
                if n:
                    assert _kept(r) == _kept(_lat(g, lp, T, 6.0, 100, 2.0)), (gs, T)
        assert live[400, 8] < live[400, 0] / 4, gs
        assert live[400, 8] - live[200, 8] < (live[400, 0] - live[200, 0]) / 4, gs


# ------------------------------------------------------------ blank-skip slicing

def _blank_lp(case, V=3):
    n = len(case["blank_logprob"])
    lp = np.full((1, max(n, 1), V), -5.0, dtype=np.float32)
    for t, x in enumerate(case["blank_logprob"]):
        lp[0, t, 0] = np.float32(x)
        lp[0, t, 1] = np.float32(-1.0 - t)      # marks the row
    return lp


@pytest.mark.parametrize("case", load_golden("blank_skip.json")["cases"], ids=lambda c: c["name"])
def test_golden_blank_skip(case):
    fx = load_golden("blank_skip.json")
    assert hex(int(np.array(np.float32(np.log(np.float64(np.float32(fx["threshold"]))))).view(np.uint32))) == fx["lthr_float32_bits"]
    lp = _blank_lp(case)
    out, n = oracle.blank_skip(lp, [case["length"]], fx["blank_id"], fx["threshold"])
    assert int(n[0]) == len(case["expect_kept"])
    assert np.array_equal(out[0, :n[0]], lp[0, case["expect_kept"]])
    assert not out[0, n[0]:].any()


def test_blank_skip_threshold_one_keeps_everything():
    """Log-probs are <= 0, so no blank probability exceeds a threshold of 1."""
    lp = synth.random_logprobs(31, 3, 40, 7, boost=8.0)
    L = np.array([40, 13, 0], np.int32)
    out, n = oracle.blank_skip(lp, L, 0, 1.0)
    assert np.array_equal(n, L)
    for b in range(3):
        assert np.array_equal(out[b, :L[b]], lp[b, :L[b]])
