"""GPU tests of the winners log's memory: compaction (page section 8.1: a GC
round keeps the entries live tokens still reach; memory bounded, results
identical) and lazily committed regions (section 6.2: address space reserved
once, memory mapped as the logs grow, a decode that outgrows it run again).
Decodes and streams with compaction rounds equal the oracle (arc ids and words
bit-exact, scores and every per-step record), a winners-log region too small for
an uncompacted decode or stream suffices once rounds run, and a decoder whose
regions start nearly empty returns the fully committed decoder's results."""

import numpy as np
import pytest

import oracle
import synth
import wfst_beam_search_amd as wb
from gpu_util import compare_batch, gpu_decode, oracle_lanes
from test_gpu_stream import check_stream, stream_run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _case(seed, eps):
    rng = np.random.default_rng(120_000 + seed)
    n = int(rng.integers(3, 50))
    vocab = int(rng.integers(2, 10))
    g = synth.random_graph(seed + 500, n=n, deg=(1, int(rng.integers(2, 8))), vocab=vocab, epsilon=eps,
                           eps_levels=int(rng.integers(2, 5)), self_loop=float(rng.choice([0.0, 0.3])))
    B = int(rng.integers(1, 5))
    T = int(rng.integers(1, 40))
    lp = synth.random_logprobs(seed + 9, B, T, vocab, sigma=float(rng.uniform(0.5, 3.0)))
    L = rng.integers(0, T + 1, size=B).astype(np.int32)
    beam = float(rng.choice([1.0, 4.0, 10.0, 1e10]))
    ma = int(rng.choice([2, 5, 30, 1000]))
    ap = bool(rng.integers(0, 2))
    P = int(rng.integers(1, 4)) if eps else 0
    gi = int(rng.choice([1, 2, 3, 7]))
    return g, lp, L, beam, ma, ap, P, gi


@pytest.mark.parametrize("eps", [False, True])
def test_gc_random_graphs(eps):
    for seed in range(50):
        g, lp, L, beam, ma, ap, P, gi = _case(seed + (300 if eps else 0), eps)
        _say("gc random", eps, seed, lp.shape, beam, ma, ap, P, "interval", gi)
        r, steps, _ = gpu_decode(g, lp, L, beam, ma, 0, ap, P, gc_interval=gi,
                                 use_graphs=bool(seed % 2))
        o = oracle_lanes(g, lp, L, beam, ma, 0, ap, P)
        compare_batch(r, steps, o)


@pytest.mark.parametrize("cid", [2, 4])
def test_gc_workload_bounds_the_log(cid):
    """mid-hlg-50k and the TLG: the same results with rounds every 8 steps, and
    the compacted log holds a small fraction of the uncompacted one."""
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    lanes = [0, 1] if cid == 4 else [0, 3, 6]
    lp2 = np.ascontiguousarray(lp[lanes])
    L2 = L[lanes]
    dg = wb.Graph(g)
    try:
        r0, _, s0 = gpu_decode(g, lp2, L2, wl.beam, wl.max_active, 0, False, wl.eps_iterations, dgraph=dg)
        r1, steps, s1 = gpu_decode(g, lp2, L2, wl.beam, wl.max_active, 0, False, wl.eps_iterations, dgraph=dg,
                                   gc_interval=8)
    finally:
        dg.release()
    _say("log entries", s0["log_entries"], "->", s1["log_entries"])
    o = oracle_lanes(g, lp2, L2, wl.beam, wl.max_active, 0, False, wl.eps_iterations)
    compare_batch(r1, steps, o)
    for b in range(len(lanes)):
        assert np.array_equal(r0.arcs[b], r1.arcs[b])
    assert s1["log_entries"] * 5 < s0["log_entries"]


def test_gc_small_arena_decode():
    """A region that an uncompacted decode overflows (arena bit) holds a
    compacted one, with the oracle's result."""
    g, lp, L = synth.workload_inputs(2)
    wl = synth.WORKLOADS[2]
    lp1 = np.ascontiguousarray(lp[:2])
    L1 = L[:2]
    dg = wb.Graph(g)
    try:
        arena = 60_000
        r0, _, _ = gpu_decode(g, lp1, L1, wl.beam, wl.max_active, 0, False, 0, dgraph=dg, with_steps=False,
                              arena_entries=arena)
        assert all(int(m[2]) & 4 for m in r0.meta)
        r1, steps, _ = gpu_decode(g, lp1, L1, wl.beam, wl.max_active, 0, False, 0, dgraph=dg,
                                  arena_entries=arena, gc_interval=4)
    finally:
        dg.release()
    compare_batch(r1, steps, oracle_lanes(g, lp1, L1, wl.beam, wl.max_active))


@pytest.mark.parametrize("eps", [False, True])
def test_gc_streams(eps):
    for seed in range(15):
        g, lp, L, beam, ma, ap, P, gi = _case(seed + (700 if eps else 0), eps)
        chunk = int(np.random.default_rng(seed).choice([1, 3, 8, 16]))
        _say("gc stream", eps, seed, lp.shape, chunk, "interval", gi)
        check_stream(g, lp, L, chunk, beam, ma, 0, ap, P, gc_interval=gi, use_graphs=bool(seed % 2))


def test_gc_long_stream_in_a_small_region():
    """A 600-frame stream through a winners-log region of 60k entries: without
    rounds it overflows; with them it ends with the oracle's online result."""
    g, lp, L = synth.workload_inputs(2)
    wl = synth.WORKLOADS[2]
    T = 600
    lp1 = np.ascontiguousarray(np.concatenate([lp[0, :200], lp[1, :200], lp[2, :200]])[None])
    L1 = np.array([T], np.int32)
    dg = wb.Graph(g)
    try:
        _, _, _, fin0 = stream_run(g, lp1, L1, 32, wl.beam, wl.max_active, dgraph=dg, partial_every=1000,
                                   arena_entries=60_000)
        assert int(fin0[0][3][2]) & 4
        _, _, _, fin = stream_run(g, lp1, L1, 32, wl.beam, wl.max_active, dgraph=dg, partial_every=1000,
                                  arena_entries=60_000, gc_interval=4)
    finally:
        dg.release()
    o = oracle.decode_lane(g, lp1[0], T, wl.beam, wl.max_active, online=True)
    words, arcs, score, meta, _ = fin[0]
    assert int(meta[2]) == 0 and list(arcs) == list(o["arcs"]) and list(words) == list(o["words"])
    assert np.float32(score) == np.float32(o["score"])


def test_lazy_region_commits_on_demand():
    """A first commitment of 4096 entries per lane: the first decode outgrows it,
    commits more and runs again; its result is the oracle's and the fully
    committed decoder's, and the next decode runs once."""
    import torch
    g, lp, L = synth.workload_inputs(2)
    wl = synth.WORKLOADS[2]
    lanes = [0, 3, 6]
    lp2 = np.ascontiguousarray(lp[lanes])
    L2 = L[lanes]
    dg = wb.Graph(g)
    try:
        dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=3, max_frames=lp2.shape[1], arena_commit=4096)
        x = torch.from_numpy(lp2).cuda()
        r1 = dec.decode(x, L2)
        s1 = dec.stats()
        r2 = dec.decode(x, L2)
        s2 = dec.stats()
        steps = [dec.step_stats(b) for b in range(3)]
        ms = dec.mem_stats()
        dec.close()
        rf, _, sf = gpu_decode(g, lp2, L2, wl.beam, wl.max_active, dgraph=dg, with_steps=False, arena_commit=-1)
    finally:
        dg.release()
    _say("lazy", s1["regrows"], s1["log_committed_bytes"], "of", s1["log_reserved_bytes"], "entries", s1["log_entries"])
    assert s1["regrows"] >= 1 and s2["regrows"] == 0
    assert ms["reserved"] == ms["fixed"] + s2["log_reserved_bytes"]
    assert ms["committed"] == ms["fixed"] + s2["log_committed_bytes"] < ms["reserved"]
    assert 0 < ms["log_high_water"] <= s2["log_committed_bytes"] // 3 and ms["log_high_water"] * 3 >= s2["log_entries"] * 8
    assert s1["log_entries"] * 8 <= s1["log_committed_bytes"] < s1["log_reserved_bytes"]
    assert sf["log_committed_bytes"] >= sf["log_reserved_bytes"] and sf["regrows"] == 0
    compare_batch(r2, steps, oracle_lanes(g, lp2, L2, wl.beam, wl.max_active))
    for b in range(3):
        for r in (r1, rf):
            assert np.array_equal(r.arcs[b], r2.arcs[b]) and np.array_equal(r.words[b], r2.words[b])
            assert np.float32(r.scores[b]) == np.float32(r2.scores[b]) and np.array_equal(r.meta[b], r2.meta[b])


@pytest.mark.parametrize("gi", [0, 3])
def test_lazy_region_streams(gi):
    """Streams on a decoder whose regions start with 2048 committed entries per
    lane: opening a stream commits the whole region, results are the oracle's."""
    for seed in range(4):
        g, lp, L, beam, ma, ap, P, _ = _case(seed + 900, bool(seed % 2))
        _say("lazy stream", seed, lp.shape, "interval", gi)
        check_stream(g, lp, L, 5, beam, ma, 0, ap, P, gc_interval=gi, arena_commit=2048)


def test_stream_commit_tracks_open_channels():
    """Page section 6.2 (a channel's slice committed at CreateStream): with
    lazily committed regions of 2^21 entries per lane (16 MiB, 4 MiB chunks), each
    stream opened commits its own lane's region, the same amount per lane, and
    nothing when a released channel opens again; a decode after the streams
    (kernels' bound back to the decode's committed size) equals the oracle."""
    import torch
    g = synth.random_graph(2024, n=50, deg=(1, 6), vocab=8, self_loop=0.3)
    lp = synth.random_logprobs(2025, 4, 30, g.vocab, sigma=2.0)
    L = np.array([30, 22, 17, 30], dtype=np.int32)
    dg = wb.Graph(g)
    try:
        dec = wb.Decoder(dg, 8.0, 200, max_lanes=8, max_frames=30, arena_entries=1 << 21, arena_commit=4096)
        m0 = dec.mem_stats()
        chans, seen = [], [m0["committed"]]
        for k in range(3):
            chans.append(dec.create_stream())
            seen.append(dec.mem_stats()["committed"])
        per = seen[1] - seen[0]
        _say("committed per opened stream", per, seen)
        assert per >= (1 << 21) * 8 - (4 << 20)
        assert all(seen[k + 1] - seen[k] == per for k in range(3))
        assert dec.mem_stats()["reserved"] == m0["reserved"]
        # a stream on those lanes decodes (its whole region is usable)
        x = torch.from_numpy(np.ascontiguousarray(lp[:1])).cuda()
        dec.advance_chunk([chans[0]], x, [30])
        fin = dec.finalize_stream(chans[0])
        o = oracle.decode_lane(g, lp[0], 30, 8.0, 200, online=True)
        assert np.array_equal(fin.arcs[0], o["arcs"]) and np.float32(fin.scores[0]) == np.float32(o["score"])
        for c in chans:
            dec.release_stream(c)
        again = dec.create_stream()
        assert again in chans and dec.mem_stats()["committed"] == seen[-1]
        dec.release_stream(again)
        r = dec.decode(torch.from_numpy(lp).cuda(), L)
        compare_batch(r, None, oracle_lanes(g, lp, L, 8.0, 200), check_steps=False)
        dec.close()
    finally:
        dg.release()
