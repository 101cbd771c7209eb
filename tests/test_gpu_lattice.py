"""GPU parity of lattice mode (page section 1 "Lattice mode", section 3 on
output_beam, section 5.5 on the candidate set persisted after the closure with
epsilon arcs tagged, section 7 "Lattice"): the kept lattice arcs of every lane,
as flat records, equal the oracle's kept arcs bit for bit (frame, states,
labels, arc ids, arc-score bits, flags), on epsilon-free graphs and on graphs
with epsilon arcs; the 1-best results stay those of a plain decode."""

import numpy as np
import pytest

import oracle
import synth
import wfst_beam_search_amd as wb
from gpu_util import compare_batch, oracle_lanes

pytestmark = pytest.mark.gpu

OF = {name: i for i, name in enumerate(oracle.LAT_FIELDS)}


def _say(*a):
    print(*a, flush=True)


def _oracle_kept(g, lp_lane, T, beam, max_active, min_active, allow_partial, ob, lane, eps_iterations=0,
                 lat_prune_interval=0):
    r = oracle.decode_lane(g, lp_lane.astype(np.float32), T, beam, max_active, min_active, allow_partial,
                           eps_iterations=eps_iterations, output_beam=ob, lat_prune_interval=lat_prune_interval)
    lat = r["lattice"]
    k = lat[lat[:, OF["keep"]] == 1]
    out = np.stack([k[:, OF["frame"]], k[:, OF["src"]], k[:, OF["dst"]], k[:, OF["ilabel"]], k[:, OF["arc"]],
                    k[:, OF["score_bits"]], np.full(k.shape[0], lane, np.int32), k[:, OF["flags"]]], 1) \
        if k.shape[0] else np.zeros((0, 8), np.int32)
    out = out.astype(np.int32)
    return out[np.lexsort((out[:, 4], out[:, 1], out[:, 0]))] if out.shape[0] else out, r


def lattice_case(g, lp, L, beam, ma, mi, ap, ob, dgraph=None, eps_iterations=0, lanes=None, **caps):
    import torch
    B, T, V = lp.shape
    own = dgraph is None
    dg = wb.Graph(g) if own else dgraph
    dec = wb.Decoder(dg, beam, ma, min_active=mi, allow_partial=ap, max_lanes=B, max_frames=max(T, 1),
                     lp_dtype="f16" if lp.dtype == np.float16 else "f32", lattice=True, output_beam=ob,
                     eps_iterations=eps_iterations, **caps)
    r = dec.decode(torch.from_numpy(np.ascontiguousarray(lp)).cuda(), L)
    lanes = list(range(B)) if lanes is None else list(lanes)
    lats = [dec.lattice(b) for b in lanes]
    dec.close()
    if own:
        dg.release()
    o = oracle_lanes(g, lp, L, beam, ma, mi, ap, eps_iterations=eps_iterations, lanes=lanes)
    compare_batch(r, None, o, lanes=lanes, check_steps=False)
    for j, b in enumerate(lanes):
        want, _ = _oracle_kept(g, lp[b], int(L[b]), beam, ma, mi, ap, ob, b, eps_iterations,
                               caps.get("lat_prune_interval", 0))
        got = lats[j]
        assert got.shape == want.shape, f"lane {b}: {got.shape[0]} kept arcs vs {want.shape[0]}"
        assert np.array_equal(got, want), f"lane {b}: lattice records differ"
    return r, lats


def _random_case(seed):
    rng = np.random.default_rng(70_000 + seed)
    n = int(rng.integers(3, 40))
    vocab = int(rng.integers(2, 10))
    g = synth.random_graph(seed + 11, n=n, deg=(1, int(rng.integers(2, 8))), vocab=vocab,
                           self_loop=float(rng.choice([0.0, 0.3])))
    B = int(rng.integers(1, 5))
    T = int(rng.integers(0, 20))
    lp = synth.random_logprobs(seed + 5, B, max(T, 1), vocab, sigma=float(rng.uniform(0.5, 3.0)))
    if T == 0:
        lp = lp[:, :0, :]
    L = rng.integers(0, T + 1, size=B).astype(np.int32)
    beam = float(rng.choice([1.0, 3.0, 8.0, 1e10]))
    ma = int(rng.choice([2, 5, 50, 1000]))
    mi = int(rng.choice([0, 0, 3]))
    ap = bool(rng.integers(0, 2))
    ob = float(rng.choice([0.0, 0.5, 2.0, 10.0]))
    return g, lp, L, beam, ma, mi, ap, ob


def test_lattice_random_small_graphs():
    kept = 0
    for seed in range(60):
        g, lp, L, beam, ma, mi, ap, ob = _random_case(seed)
        _say("lattice random", seed, lp.shape, beam, ma, mi, ap, ob)
        _, lats = lattice_case(g, lp, L, beam, ma, mi, ap, ob)
        kept += sum(x.shape[0] for x in lats)
    assert kept > 500


@pytest.mark.parametrize("ob", [0.5, 4.0])
def test_lattice_workload(ob):
    cid = 2
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    lanes = [0, 5]
    lp2 = np.ascontiguousarray(lp[lanes, :120])
    L2 = np.minimum(L[lanes], 120).astype(np.int32)
    _say("lattice workload", ob, lp2.shape)
    _, lats = lattice_case(g, lp2, L2, wl.beam, wl.max_active, 0, False, ob)
    assert all(x.shape[0] > L2[b] for b, x in enumerate(lats))


def _random_tlg_case(seed):
    rng = np.random.default_rng(71_000 + seed)
    n = int(rng.integers(3, 40))
    vocab = int(rng.integers(3, 10))
    levels = int(rng.integers(2, 5))
    g = synth.random_graph(seed + 13, n=n, deg=(1, int(rng.integers(2, 8))), vocab=vocab, epsilon=True,
                           eps_levels=levels, eps_share=float(rng.choice([0.2, 0.4])))
    B = int(rng.integers(1, 5))
    T = int(rng.integers(0, 20))
    lp = synth.random_logprobs(seed + 6, B, max(T, 1), vocab, sigma=float(rng.uniform(0.5, 3.0)))
    if T == 0:
        lp = lp[:, :0, :]
    L = rng.integers(0, T + 1, size=B).astype(np.int32)
    beam = float(rng.choice([1.0, 3.0, 8.0, 1e10]))
    ma = int(rng.choice([2, 5, 50, 1000]))
    mi = int(rng.choice([0, 0, 3]))
    ap = bool(rng.integers(0, 2))
    ob = float(rng.choice([0.0, 0.5, 2.0, 10.0]))
    P = int(rng.integers(1, 5))
    return g, lp, L, beam, ma, mi, ap, ob, P


def test_lattice_random_tlg_graphs():
    """Graphs with epsilon arcs (levels 2-4, 1-4 closure passes): epsilon arcs
    persisted by every closure pass, kept records equal the oracle's."""
    kept = eps_kept = 0
    for seed in range(60):
        g, lp, L, beam, ma, mi, ap, ob, P = _random_tlg_case(seed)
        _say("lattice tlg random", seed, lp.shape, beam, ma, mi, ap, ob, P)
        _, lats = lattice_case(g, lp, L, beam, ma, mi, ap, ob, eps_iterations=P)
        kept += sum(x.shape[0] for x in lats)
        eps_kept += sum(int((x[:, 7] == 4).sum()) for x in lats)
    assert kept > 500 and eps_kept > 100


def test_lattice_tlg_workload_full_size():
    """The TLG workload at full size (1M states, 16 x 400 frames, 4 closure
    passes), lattice mode with output beam 4: every lane's 1-best result and,
    on sampled lanes, the kept records equal the oracle's bit for bit."""
    cid = 4
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    _say("lattice tlg workload", lp.shape)
    _, lats = lattice_case(g, lp, L, wl.beam, wl.max_active, 0, False, 4.0, eps_iterations=wl.eps_iterations,
                           lanes=[0, 9], arena_entries=16 << 20)
    assert all(int((x[:, 7] == 4).sum()) > 0 for x in lats)


def test_lattice_interval_prune_random():
    """Section 7's interval prune (reading R32), every 1, 2, 3 or 5 steps, on
    random epsilon-free and TLG graphs: the kept records equal the oracle's with
    the same interval bit for bit."""
    kept = 0
    for seed in range(40):
        n = (1, 2, 3, 5)[seed % 4]
        if seed % 2:
            g, lp, L, beam, ma, mi, ap, ob, P = _random_tlg_case(200 + seed)
        else:
            g, lp, L, beam, ma, mi, ap, ob = _random_case(200 + seed)
            P = 0
        _say("lattice interval prune", seed, n, lp.shape, beam, ma, ob, P)
        _, lats = lattice_case(g, lp, L, beam, ma, mi, ap, ob, eps_iterations=P, lat_prune_interval=n)
        kept += sum(x.shape[0] for x in lats)
    assert kept > 300


def _large_frame_case(levels):
    g = synth.random_graph(77, n=60000, deg=(4, 14), vocab=8, epsilon=True, eps_levels=levels, eps_share=0.3)
    lp = synth.random_logprobs(78, 2, 5, g.vocab, sigma=1.0)
    return g, lp, np.array([5, 4], dtype=np.int32)


@pytest.mark.parametrize("interval,levels,passes", [(0, 4, 3), (2, 4, 3), (0, 8, 1), (2, 8, 2)])
def test_lattice_large_epsilon_frames(interval, levels, passes):
    """Frames of up to 60k tokens with up to 160k epsilon records (an unbounded
    beam on a 60k-state graph with epsilon arcs): the final pass's flat epsilon
    rounds, and, with epsilon chains longer than the rounds settle (8 levels, 1
    or 2 closure passes), the per-lane finish of the fixpoint, in LDS for a
    small frame and on the scores in memory for a large one; the interval
    prune's per-lane fixpoint likewise. The kept records equal the oracle's."""
    g, lp, L = _large_frame_case(levels)
    _say("lattice large epsilon frames", interval, levels, passes, lp.shape)
    _, lats = lattice_case(g, lp, L, 1e10, 10**6, 0, False, 2.0, eps_iterations=passes, frontier_cap=1 << 17,
                           slot_cap=1 << 21, claims_cap=1 << 21, arena_entries=4 << 20, lattice_cap=4 << 20,
                           lat_prune_interval=interval)
    assert all(int((x[:, 7] == 4).sum()) > 0 for x in lats)


@pytest.mark.parametrize("interval", [0, 3])
def test_lattice_large_frames(interval):
    """Frames growing to 60k tokens and 530k lattice arcs on an epsilon-free
    graph (an unbounded beam on a 60k-state graph): with the interval prune
    every 3 steps, the second prune's sweep holds its small frames' backward
    scores in LDS and its large ones in memory, with a step between the two.
    The kept records equal the oracle's."""
    g = synth.random_graph(79, n=60000, deg=(4, 14), vocab=8)
    lp = synth.random_logprobs(80, 2, 7, g.vocab, sigma=1.0)
    L = np.array([7, 6], dtype=np.int32)
    _say("lattice large frames", interval, lp.shape)
    _, lats = lattice_case(g, lp, L, 1e10, 10**6, 0, False, 2.0, frontier_cap=1 << 17, slot_cap=1 << 21,
                           claims_cap=1 << 21, arena_entries=4 << 20, lattice_cap=4 << 20,
                           lat_prune_interval=interval)
    assert all(x.shape[0] > 0 for x in lats)


def test_lattice_deep_epsilon_chains():
    """Small graphs whose epsilon chains run up to 7 arcs, 1 or 2 closure passes:
    the final pass's flat rounds leave chains unsettled, and the per-lane finish
    of the fixpoint completes them; kept records equal the oracle's."""
    kept = eps_kept = 0
    for seed in range(30):
        rng = np.random.default_rng(72_000 + seed)
        g = synth.random_graph(seed + 900, n=int(rng.integers(20, 60)), deg=(1, int(rng.integers(3, 8))),
                               vocab=int(rng.integers(3, 8)), epsilon=True, eps_levels=8, eps_share=0.5)
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 12))
        lp = synth.random_logprobs(seed + 901, B, T, g.vocab, sigma=float(rng.uniform(0.5, 2.0)))
        L = rng.integers(1, T + 1, size=B).astype(np.int32)
        P = int(rng.integers(1, 3))
        _say("lattice deep epsilon", seed, lp.shape, P)
        _, lats = lattice_case(g, lp, L, 1e10, 1000, 0, True, float(rng.choice([1.0, 5.0])), eps_iterations=P)
        kept += sum(x.shape[0] for x in lats)
        eps_kept += sum(int((x[:, 7] == 4).sum()) for x in lats)
    assert kept > 100 and eps_kept > 50


def _long_case():
    g = synth.random_graph(5, n=30, deg=(1, 6), vocab=6, self_loop=0.3)
    lp = synth.random_logprobs(6, 2, 400, g.vocab, sigma=2.0)
    return g, lp, np.array([400, 371], dtype=np.int32)


def test_lattice_interval_prune_bounds_the_arena():
    """A 400-frame lane admits ~11k lattice arcs; with lattice_cap 4000 the
    lattice overflows without the interval prune (arena bit, no records) and
    fits with a prune every 8 steps, its kept records equal to the oracle's."""
    import torch
    g, lp, L = _long_case()
    dg = wb.Graph(g)
    try:
        dec = wb.Decoder(dg, 6.0, 100, max_lanes=2, max_frames=400, lattice=True, output_beam=2.0, lattice_cap=4000)
        r = dec.decode(torch.from_numpy(lp).cuda(), L)
        assert all(int(r.meta[b, 2]) & 4 for b in range(2)) and dec.lattice(0).shape[0] == 0
        dec.close()
        _, lats = lattice_case(g, lp, L, 6.0, 100, 0, False, 2.0, dgraph=dg, lattice_cap=4000, lat_prune_interval=8)
        assert all(x.shape[0] > 400 for x in lats)
    finally:
        dg.release()


def test_lattice_interval_prune_longest_window():
    """The largest interval (512 steps): 1100-frame lanes pruned after steps
    511 and 1023 over windows reaching back to frame 0 (1025 step offsets in
    the sweep's table, 1024 slots in the work-record pass); kept records equal
    the oracle's with the same interval."""
    g = synth.random_graph(15, n=30, deg=(1, 5), vocab=6, self_loop=0.3)
    lp = synth.random_logprobs(16, 2, 1100, g.vocab, sigma=2.0)
    L = np.array([1100, 1030], dtype=np.int32)
    _say("lattice longest prune window", lp.shape)
    _, lats = lattice_case(g, lp, L, 6.0, 100, 0, False, 2.0, lattice_cap=1 << 16, lat_prune_interval=512)
    assert all(x.shape[0] > 1000 for x in lats)


def test_lattice_final_pass_windows():
    """Lanes of 2100, 1500, 1025 and 1024 frames on an epsilon-free graph
    without the interval prune: the final pass's sweep walks each lane in
    windows of 1024 frames, each starting from the scores the one above left;
    kept records equal the oracle's."""
    g = synth.random_graph(17, n=30, deg=(1, 5), vocab=6, self_loop=0.3)
    lp = synth.random_logprobs(18, 4, 2100, g.vocab, sigma=2.0)
    L = np.array([2100, 1500, 1025, 1024], dtype=np.int32)
    _say("lattice final-pass windows", lp.shape)
    _, lats = lattice_case(g, lp, L, 6.0, 100, 0, False, 2.0, lattice_cap=1 << 18)
    assert all(x.shape[0] > L[b] for b, x in enumerate(lats))


@pytest.mark.parametrize("grid", [1, 7])
def test_lattice_grid_sizes(grid):
    """Lattice mode with one and with seven workgroups per frame-loop launch
    (grid_blocks), with and without the interval prune, on random
    epsilon-free and TLG graphs: kept records equal the oracle's."""
    for seed in range(8):
        if seed % 2:
            g, lp, L, beam, ma, mi, ap, ob, P = _random_tlg_case(600 + seed)
        else:
            g, lp, L, beam, ma, mi, ap, ob = _random_case(600 + seed)
            P = 0
        n = (0, 0, 2, 3)[seed % 4]
        _say("lattice grid", grid, seed, lp.shape, P, n)
        lattice_case(g, lp, L, beam, ma, mi, ap, ob, eps_iterations=P, grid_blocks=grid, lat_prune_interval=n)


def test_lattice_with_log_compaction():
    """Log compaction rounds in lattice mode (section 6.3): lattice nodes are
    frame positions, never winners-log entries, so rounds every 16 steps leave
    the kept records and the 1-best results those of the oracle, with and
    without the interval prune, while a winners log of 3000 entries per lane
    (the whole decode appends about 6300) suffices."""
    g, lp, L = _long_case()
    for n in (0, 8):
        _say("lattice with compaction", n)
        r, lats = lattice_case(g, lp, L, 6.0, 100, 0, False, 2.0, gc_interval=16, arena_entries=3000,
                               lat_prune_interval=n)
        assert all(int(r.meta[b, 2]) == 0 for b in range(2))
        assert all(x.shape[0] > 400 for x in lats)


def test_lattice_capacity_and_rejections():
    import torch
    g, lp, L, beam, ma, mi, ap, _ = _random_case(3)
    lp = synth.random_logprobs(9, 1, 12, g.vocab)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 8.0, 1000, max_lanes=1, max_frames=12, lattice=True, output_beam=5.0, lattice_cap=4)
    r = dec.decode(torch.from_numpy(lp).cuda(), [12])
    assert int(r.meta[0, 2]) & 4 and int(r.meta[0, 0]) == 0      # arena bit: lattice full
    assert dec.stats()["regrows"] == 0                           # (not the log: no re-run)
    with pytest.raises(wb.WfstError):
        dec.create_stream()                                          # no streams in lattice mode
    dec.close()
    with pytest.raises(wb.WfstError):
        wb.Decoder(dg, 8.0, 100, lattice=True, output_beam=float("inf"))
    # a positive epsilon weight: no best continuation inside a frame
    eg = synth.random_graph(4, n=6, deg=(1, 3), vocab=4, epsilon=True, eps_levels=3)
    eps = eg.ilabel == eg.epsilon_id
    assert eps.any()
    eg.weight = np.where(eps, np.float32(0.5), eg.weight).astype(np.float32)
    deg_ = wb.Graph(eg)
    with pytest.raises(wb.WfstError, match="epsilon weight"):
        wb.Decoder(deg_, 8.0, 100, eps_iterations=2, lattice=True, output_beam=1.0)
    wb.Decoder(deg_, 8.0, 100, eps_iterations=2).close()       # (1-best decoding takes it)
    deg_.release()
    dg.release()


def test_lattice_with_the_recombination_hash():
    """Lattice mode over the open-addressing recombination hash (64 slots per
    lane: long probe chains) on random epsilon-free and TLG graphs, with and
    without the interval prune: kept records equal the oracle's."""
    kept = 0
    for seed in range(24):
        if seed % 2:
            g, lp, L, beam, ma, mi, ap, ob, P = _random_tlg_case(400 + seed)
        else:
            g, lp, L, beam, ma, mi, ap, ob = _random_case(400 + seed)
            P = 0
        n = (0, 2, 0, 3)[seed % 4]
        _say("lattice hash", seed, lp.shape, P, n)
        _, lats = lattice_case(g, lp, L, beam, ma, mi, ap, ob, eps_iterations=P, recomb_slots=64,
                               lat_prune_interval=n)
        kept += sum(x.shape[0] for x in lats)
    assert kept > 100


def test_lattice_tlg_workload_interval_prune():
    """The TLG workload at full size with the interval prune every 32 steps
    (output beam 4): sampled lanes' kept records equal the oracle's with the
    same interval, epsilon records among them."""
    cid = 4
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    _say("lattice tlg workload prune", lp.shape)
    _, lats = lattice_case(g, lp, L, wl.beam, wl.max_active, 0, False, 4.0, eps_iterations=wl.eps_iterations,
                           lanes=[3, 12], arena_entries=16 << 20, lat_prune_interval=32)
    assert all(int((x[:, 7] == 4).sum()) > 0 for x in lats)


def test_lattice_hlg_workload_interval_prune():
    """The HLG workload at full size in lattice mode with output beam 8 and the
    interval prune every 64 steps, as its benchmark runs it: sampled lanes'
    kept records equal the oracle's with the same interval."""
    cid = 3
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    _say("lattice hlg workload prune", lp.shape)
    _, lats = lattice_case(g, lp, L, wl.beam, wl.max_active, 0, False, 8.0, lanes=[1, 17, 30],
                           lat_prune_interval=64)
    assert all(x.shape[0] > 0 for x in lats)


def test_lattice_epsilon_graph_with_log_compaction():
    """A 300-frame TLG-style decode in lattice mode with log compaction every
    16 steps and the interval prune every 8: kept records and 1-best results
    equal the oracle's while a winners log of 4000 entries per lane suffices."""
    g = synth.random_graph(7, n=40, deg=(1, 6), vocab=6, epsilon=True, eps_levels=3, eps_share=0.3)
    lp = synth.random_logprobs(8, 2, 300, g.vocab, sigma=2.0)
    L = np.array([300, 277], dtype=np.int32)
    r, lats = lattice_case(g, lp, L, 6.0, 100, 0, False, 2.0, eps_iterations=2, gc_interval=16,
                           arena_entries=4000, lat_prune_interval=8)
    assert all(int(r.meta[b, 2]) == 0 for b in range(2))
    assert all(int((x[:, 7] == 4).sum()) > 0 for x in lats)
