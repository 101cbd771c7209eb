"""GPU parity of streams (page section 8 "Streaming Lifecycle"; section 3 on the
online beam): the HIP decoder fed in chunks through the C ABI against the CPU
oracle's online mode. Per chunk, the partial hypothesis (best current token's
path) and the chunk's per-step records equal the oracle's after the same frames;
at the end, the final result equals the oracle's online decode of all frames.
Arc ids and words bit-exact, scores bit-equal (within 1e-4 by contract)."""

import numpy as np
import pytest

import oracle
import synth
import wfst_beam_search_amd as wb
from cases import check_path
from gpu_util import GIDX, OIDX, SCORE_TOL

pytestmark = pytest.mark.gpu

STEP_KEYS = ("n", "arcs", "admitted", "distinct", "eps_arcs", "eps_admitted", "eps_distinct",
             "eps_new", "eps_replaced", "eps_passes", "phase")


def _say(*a):
    print(*a, flush=True)


def _same_score(a, b):
    a, b = np.float32(a), np.float32(b)
    if np.isneginf(b):
        return bool(np.isneginf(a))
    return abs(float(a) - float(b)) <= SCORE_TOL


def _check_records(tag, got, ost, first, count):
    """GPU records of one call that ran `count` steps of the lane (row t + 1 = the
    call's step t) against the oracle's records of the same steps (its step
    first + t); the row after them shows a step that did not run."""
    assert got.shape[0] >= count + 1, tag
    if got.shape[0] > count + 1:
        assert got[count + 1, GIDX["phase"]] == -1, f"{tag}: step {first + count} ran past the chunk"
    for t in range(count):
        g = got[t + 1]
        if first + t >= ost.shape[0]:
            assert g[GIDX["phase"]] == -1, f"{tag}: step {first + t} ran after the lane ended"
            continue
        oo = ost[first + t]
        for k in STEP_KEYS:
            assert g[GIDX[k]] == oo[OIDX[k]], f"{tag} step {first + t}: {k} {g[GIDX[k]]} vs {oo[OIDX[k]]}"
        for k in ("beam", "max"):
            assert (int(g[GIDX[k]]) & 0xFFFFFFFF) == (int(oo[OIDX[k]]) & 0xFFFFFFFF), f"{tag} step {first + t}: {k}"


def stream_run(g, lp, lengths, chunk, beam, max_active, min_active=0, allow_partial=False, eps=0,
               partial_every=1, dgraph=None, max_lanes=None, open_at=None, use_graphs=False, batch_finalize=False,
               batch_open=False, **caps):
    """Streams each lane of ``lp`` [B, T, V] in chunks of ``chunk`` frames (lane b
    opened before chunk open_at[b]); returns (channels, partials, records, finals),
    partials[b] = [(frames so far, words, arcs, score, meta)], records[b] = [(first
    step, steps, records of that call)]."""
    import torch
    B, T, V = lp.shape
    own = dgraph is None
    dg = wb.Graph(g) if own else dgraph
    # a stream's path and winners log span all its frames, not one chunk
    caps.setdefault("path_cap", (T + 2) * (1 + eps))
    caps.setdefault("arena_entries", min(max(1 << 20, 4 * max_active * (T + 2) * (1 + eps)),
                                         ((1 << 31) - 1) // (max_lanes or B)))
    dec = wb.Decoder(dg, beam, max_active, min_active=min_active, allow_partial=allow_partial,
                     max_lanes=max_lanes or B, max_frames=max(chunk, 1),
                     lp_dtype="f16" if lp.dtype == np.float16 else "f32", eps_iterations=eps,
                     use_graphs=use_graphs, **caps)
    open_at = open_at or [0] * B
    chans = [-1] * B
    done = [0] * B
    partials = [[] for _ in range(B)]
    records = [[] for _ in range(B)]
    n_chunks = max(1, -(-max(int(x) for x in lengths) // max(chunk, 1))) + max(open_at)
    for ci in range(n_chunks + 1):
        if batch_open and ci == 0:
            first = [b for b in range(B) if open_at[b] == 0]
            got = dec.create_streams(len(first))
            assert len(got) == len(first) and len(set(got)) == len(got)
            for b, ch in zip(first, got):
                chans[b] = ch
        for b in range(B):
            if open_at[b] == ci and chans[b] < 0:
                chans[b] = dec.create_stream()
                assert chans[b] >= 0
        live = [b for b in range(B) if chans[b] >= 0 and done[b] < int(lengths[b])]
        if not live:
            if ci >= max(open_at):
                break
            continue
        x = np.zeros((len(live), max(chunk, 1), V), dtype=lp.dtype)
        lens = []
        for j, b in enumerate(live):
            n = min(chunk, int(lengths[b]) - done[b])
            x[j, :n] = lp[b, done[b]:done[b] + n]
            lens.append(n)
        want = ci % partial_every == 0
        res = dec.advance_chunk([chans[b] for b in live], torch.from_numpy(x).cuda(), lens, want_partial=want)
        for j, b in enumerate(live):
            records[b].append((done[b], lens[j], dec.step_stats(chans[b])))
            done[b] += lens[j]
            if want:
                partials[b].append((done[b], res.words[j], res.arcs[j], res.scores[j], res.meta[j].copy()))
    finals = []
    if batch_finalize:
        # every stream ended by one call, the channels listed in a scrambled order
        for b in range(B):
            if chans[b] < 0:
                chans[b] = dec.create_stream()
        order = list(np.random.default_rng(B).permutation(B))
        r = dec.finalize_streams([chans[b] for b in order])
        row = {b: j for j, b in enumerate(order)}
        for b in range(B):
            j = row[b]
            finals.append((r.words[j], r.arcs[j], r.scores[j], r.meta[j].copy(), dec.step_stats(chans[b])))
    for b in range(B if not batch_finalize else 0):
        if chans[b] < 0:
            chans[b] = dec.create_stream()
        r = dec.finalize_stream(chans[b])
        fin_rec = dec.step_stats(chans[b])
        finals.append((r.words[0], r.arcs[0], r.scores[0], r.meta[0].copy(), fin_rec))
    for b in range(B):
        dec.release_stream(chans[b])
    dec.close()
    if own:
        dg.release()
    return chans, partials, records, finals


def check_stream(g, lp, lengths, chunk, beam, max_active, min_active=0, allow_partial=False, eps=0,
                 partial_every=1, partial_lanes=None, **kw):
    B = lp.shape[0]
    _, partials, records, finals = stream_run(g, lp, lengths, chunk, beam, max_active, min_active,
                                              allow_partial, eps, partial_every, **kw)
    og = oracle.OracleGraph(g)
    for b in range(B):
        Tb = int(lengths[b])
        lpb = lp[b].astype(np.float32)
        o = oracle.decode_lane(og, lpb, Tb, beam, max_active, min_active, allow_partial, eps, online=True)
        tag = f"lane {b}"
        words, arcs, score, meta, fin_rec = finals[b]
        assert int(meta[2]) == 0, f"{tag}: overflow {meta}"
        assert int(meta[1]) == o["reached_final"], tag
        assert list(arcs) == list(o["arcs"]), f"{tag}: final arcs differ"
        assert list(words) == list(o["words"]), f"{tag}: final words differ"
        assert _same_score(score, o["score"]), f"{tag}: final score {score} vs {o['score']}"
        ost = o["steps"]
        for first, count, rec in records[b]:
            _check_records(tag, rec, ost, first, count)
        _check_records(tag, fin_rec, ost, Tb, 1)
        if partial_lanes is not None and b not in partial_lanes:
            continue
        for t, pw, pa, ps, pm in partials[b]:
            p = oracle.decode_lane(og, lpb, t, beam, max_active, min_active, allow_partial, eps,
                                   online=True, partial=True)
            assert int(pm[1]) == 0 and int(pm[2]) == 0, f"{tag} t={t}: meta {pm}"
            assert list(pa) == list(p["arcs"]), f"{tag} t={t}: partial arcs differ"
            assert list(pw) == list(p["words"]), f"{tag} t={t}: partial words differ"
            assert _same_score(ps, p["score"]), f"{tag} t={t}: partial score {ps} vs {p['score']}"
            if not p["dead"]:
                check_path(g, lpb, t, pa, pw, ps, 0)


# ------------------------------------------------------------ random small graphs

def _random_stream_case(seed, eps):
    rng = np.random.default_rng(50_000 + seed)
    n = int(rng.integers(3, 50))
    vocab = int(rng.integers(2, 10))
    g = synth.random_graph(seed + 77, n=n, deg=(1, int(rng.integers(2, 8))), vocab=vocab, epsilon=eps,
                           eps_levels=int(rng.integers(2, 5)), self_loop=float(rng.choice([0.0, 0.3])))
    B = int(rng.integers(1, 5))
    T = int(rng.integers(1, 30))
    lp = synth.random_logprobs(seed + 3, B, T, vocab, sigma=float(rng.uniform(0.5, 3.0)))
    lengths = rng.integers(0, T + 1, size=B).astype(np.int32)
    chunk = int(rng.choice([1, 2, 3, 7, 16, 32]))
    beam = float(rng.choice([0.5, 2.0, 5.0, 12.0]))
    max_active = int(rng.choice([1, 2, 5, 20, 1000]))
    min_active = int(rng.choice([0, 0, 3]))
    allow_partial = bool(rng.integers(0, 2))
    P = int(rng.integers(1, 4)) if eps else 0
    return g, lp, lengths, chunk, beam, max_active, min_active, allow_partial, P


@pytest.mark.parametrize("eps", [False, True])
def test_stream_random_small_graphs(eps):
    for seed in range(40):
        g, lp, L, chunk, beam, ma, mi, ap, P = _random_stream_case(seed + (500 if eps else 0), eps)
        graphs = seed % 2 == 1   # captured chunk sequences on odd seeds
        # epoch wraps every few rounds on most seeds: a sequence's first or
        # last round offsets may be unused, and the wipe must still come
        # before the first round used past each multiple of the period
        ep = (0, 2, 3, 5, 7)[seed % 5]
        _say("stream random", eps, seed, lp.shape, chunk, beam, ma, mi, ap, P, "graphs" if graphs else "eager", ep)
        check_stream(g, lp, L, chunk, beam, ma, mi, ap, P, use_graphs=graphs, epoch_period=ep)


def test_stream_epoch_wrap_on_an_unused_round():
    """Without epsilon arcs an open uses none of its one round number and a
    chunk of c frames uses rounds 1..c of its c + 1, so with B streams opened one
    by one and an epoch period of B + c + 1 the second chunk starts exactly at a
    multiple of the period, on its unused round 0: the table must still be wiped
    before its first used round (older entries carry larger epochs)."""
    B, T = 2, 30
    for seed, chunk in ((3, 4), (8, 5)):
        g = synth.random_graph(seed + 900, n=40, deg=(2, 6), vocab=6, self_loop=0.3)
        lp = synth.random_logprobs(seed + 901, B, T, 6, sigma=1.5)
        L = np.array([T, T - 3], np.int32)
        # B opens (one round number each, none used), then chunks of c + 1
        # rounds: the second chunk begins at round B + chunk + 1
        _say("stream wrap on an unused round", seed, lp.shape, chunk)
        for graphs in (False, True):
            check_stream(g, lp, L, chunk, 8.0, 1000, 0, False, 0, use_graphs=graphs,
                         epoch_period=B + chunk + 1)


def test_stream_staggered_open_with_epsilon():
    """A stream opened while another is mid-utterance: the start closure of the
    new one must not touch the other (page section 8, last paragraphs)."""
    g, lp, L, _, beam, ma, mi, ap, P = _random_stream_case(901, True)
    lp = synth.random_logprobs(902, 3, 24, g.vocab, sigma=2.0)
    L = np.array([24, 19, 24], np.int32)
    check_stream(g, lp, L, 5, 6.0, 50, 0, False, 3, open_at=[0, 2, 3])


def test_stream_chunkings_agree_on_a_workload():
    """mid-hlg-50k: the same utterances streamed in chunks of 1, 13 and 64 frames
    give one result, the oracle's online decode."""
    cid = 2
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    lanes = [0, 3, 6]
    lp3 = np.ascontiguousarray(lp[lanes, :120])
    L3 = np.minimum(L[lanes], 120).astype(np.int32)
    dg = wb.Graph(g)
    try:
        finals = []
        for chunk, graphs in ((1, False), (13, True), (64, False)):
            _say("workload stream chunk", chunk, "graphs" if graphs else "eager")
            _, _, _, fin = stream_run(g, lp3, L3, chunk, wl.beam, wl.max_active, dgraph=dg,
                                      partial_every=1000, use_graphs=graphs)
            finals.append(fin)
        check_stream(g, lp3, L3, 13, wl.beam, wl.max_active, partial_every=2, partial_lanes=[0],
                     dgraph=dg, use_graphs=True)
    finally:
        dg.release()
    for fin in finals[1:]:
        for b in range(len(lanes)):
            assert list(fin[b][1]) == list(finals[0][b][1])
            assert np.float32(fin[b][2]).view(np.uint32) == np.float32(finals[0][b][2]).view(np.uint32)


def test_stream_lifecycle_and_decode_exclusion():
    import torch
    g, lp, L, _, beam, ma, mi, ap, P = _random_stream_case(3, False)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 8.0, 100, max_lanes=2, max_frames=8)
    a, b = dec.create_stream(), dec.create_stream()
    assert sorted([a, b]) == [0, 1]
    assert dec.create_stream() == -1                       # every lane holds a stream
    x = torch.zeros((1, 4, g.vocab), device="cuda")
    with pytest.raises(wb.WfstError):
        dec.decode(x, [4])                                  # streams open
    with pytest.raises(wb.WfstError):
        dec.advance_chunk([a, a], torch.zeros((2, 4, g.vocab), device="cuda"), [1, 1])   # repeated
    with pytest.raises(wb.WfstError):
        dec.advance_chunk([a], torch.zeros((1, 9, g.vocab), device="cuda"), [9])         # chunk > max_frames
    r1 = dec.finalize_stream(a)
    r2 = dec.finalize_stream(a)                             # the same result again
    assert list(r1.arcs[0]) == list(r2.arcs[0]) and r1.scores[0] == r2.scores[0]
    dec.release_stream(a)
    with pytest.raises(wb.WfstError):
        dec.release_stream(a)
    c = dec.create_stream()
    assert c == a
    dec.release_stream(b)
    dec.release_stream(c)
    # offline decoding works again once every stream is released
    T = lp.shape[1]
    xx = torch.from_numpy(np.ascontiguousarray(lp[:1, :min(T, 8)])).cuda()
    r = dec.decode(xx, [min(int(L[0]), 8)])
    o = oracle.decode_lane(g, lp[0, :min(T, 8)], min(int(L[0]), 8), 8.0, 100)
    assert list(r.arcs[0]) == list(o["arcs"])
    dec.close()
    dg.release()


def test_stream_arena_overflow_is_reported():
    """A stream's path lives in its lane's winners-log region: a stream longer
    than the region sets the arena bit (page section 7 meanings)."""
    import torch
    V, T = 4, 40
    g = synth.random_graph(5, n=6, deg=(2, 3), vocab=V)
    lp = synth.random_logprobs(6, 1, T, V)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 10.0, 1000, max_lanes=1, max_frames=8, arena_entries=64, use_graphs=False)
    ch = dec.create_stream()
    for s in range(0, T, 8):
        dec.advance_chunk([ch], torch.from_numpy(np.ascontiguousarray(lp[:, s:s + 8])).cuda(), [8])
    r = dec.finalize_stream(ch)
    assert int(r.meta[0, 2]) & 4 and int(r.meta[0, 0]) == 0
    dec.release_stream(ch)
    dec.close()
    dg.release()


@pytest.mark.parametrize("eps", [False, True])
def test_streams_ended_together(eps):
    """wfst_finalize_streams: every stream of a batch ended by one call, in any
    channel order, gives each the oracle's online result and final records."""
    for seed in range(12):
        g, lp, L, chunk, beam, ma, mi, ap, P = _random_stream_case(seed + (800 if eps else 0), eps)
        _say("streams ended together", eps, seed, lp.shape, chunk)
        check_stream(g, lp, L, chunk, beam, ma, mi, ap, P, batch_finalize=True, batch_open=True,
                     use_graphs=bool(seed % 2))


def test_create_streams_grants_the_free_lanes():
    """wfst_create_streams opens at most the free lanes, lowest first; a full
    decoder grants none (no error)."""
    g = synth.random_graph(61, n=8, deg=(1, 3), vocab=4)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 6.0, 50, max_lanes=4, max_frames=4)
    a = dec.create_stream()
    got = dec.create_streams(6)
    assert a == 0 and got == [1, 2, 3]
    assert dec.create_streams(2) == [] and dec.create_stream() == -1
    assert dec.create_streams(0) == []
    with pytest.raises(wb.WfstError):
        dec.create_streams(-1)
    dec.release_stream(2)
    assert dec.create_streams(3) == [2]
    for ch in range(4):
        dec.release_stream(ch)
    dec.close()
    dg.release()
