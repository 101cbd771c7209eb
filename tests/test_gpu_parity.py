"""GPU parity: the HIP decoder (through the C ABI) against the CPU oracle on the
same seeded inputs. Arc ids and words must be bit-exact, scores within 1e-4
(they come out bit-equal), and every per-step counter (frontier size, beam,
exact max, arcs expanded, admitted, distinct, epsilon counters) equal."""

import numpy as np
import pytest

import synth
import wfst_beam_search_amd as wb
from cases import check_path, graph_from_states, load_golden
from gpu_util import compare_batch, compare_lane, gpu_decode, oracle_lanes

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ golden

def _golden_cases():
    out = []
    bs = load_golden("beam_schedule.json")
    for c in bs["cases"]:
        out.append(("beam_" + c["name"], graph_from_states(bs["graphs"][c["graph"]]),
                    np.full((c["frames"], 1), c["lp_value"], np.float32), c, 0, 0))
    tc = load_golden("tie_chain.json")
    g = graph_from_states(tc["graph"])
    out.append(("tie_chain", g, np.full((tc["frames"], g.vocab), tc["lp_value"], np.float32), tc, 0, 0))
    ec = load_golden("eps_closure.json")
    out.append(("eps_closure", graph_from_states(ec["graph"]), np.array(ec["lp_rows"], np.float32), ec,
                ec["eps_iterations"], 0))
    for c in load_golden("edge_cases.json")["cases"]:
        g = graph_from_states(c["graph"])
        out.append(("edge_" + c["name"], g,
                    np.array(c["lp_rows"], np.float32).reshape(c["frames"], g.vocab), c, c.get("eps_iterations", 0),
                    c["allow_partial"]))
    return out


# table keys: ties by in-rank (default on these graphs), by arc id (plain_keys
# 2), plain keys (1); epoch wraps forced every few rounds (epoch_period);
# recombination through the open-addressing hash (recomb_slots: 64 slots on the
# small graphs, so probe chains run long, a quarter million on the workloads)
MODES = {"graph": dict(use_graphs=True), "eager": dict(use_graphs=False),
         "plain": dict(use_graphs=True, plain_keys=1), "arcid": dict(use_graphs=True, plain_keys=2),
         "wrap": dict(use_graphs=True, epoch_period=3), "wrap_eager": dict(use_graphs=False, epoch_period=2),
         "hash": dict(use_graphs=True, recomb_slots=64), "hash_wrap": dict(use_graphs=False, recomb_slots=64,
                                                                            epoch_period=3, plain_keys=2),
         "hash_big": dict(use_graphs=True, recomb_slots=1 << 18)}


@pytest.mark.parametrize("name,g,lp,case,eps,ap", _golden_cases(), ids=lambda x: x if isinstance(x, str) else "")
@pytest.mark.parametrize("mode", list(MODES))
def test_golden(name, g, lp, case, eps, ap, mode):
    _say("golden", name, mode)
    T = lp.shape[0]
    lpb = lp.reshape(1, T, g.vocab)
    r, steps, _ = gpu_decode(g, lpb, [T], case["beam"], case["max_active"], case.get("min_active", 0),
                             bool(ap), eps, **MODES[mode])
    assert list(r.arcs[0]) == case["expect_arcs"]
    if "expect_words" in case:
        assert list(r.words[0]) == case["expect_words"]
    exp = case["expect_score"]
    if exp == "-inf":
        assert np.isneginf(r.scores[0])
    else:
        assert r.scores[0] == np.float32(exp)
    o = oracle_lanes(g, lpb, [T], case["beam"], case["max_active"], case.get("min_active", 0), bool(ap), eps)
    compare_lane(0, r, steps, o[0])


# --------------------------------------------------------- random small graphs

def _random_case(seed, eps):
    rng = np.random.default_rng(10_000 + seed)
    n = int(rng.integers(3, 60))
    vocab = int(rng.integers(2, 12))
    g = synth.random_graph(seed, n=n, deg=(1, int(rng.integers(2, 9))), vocab=vocab, epsilon=eps,
                           eps_levels=int(rng.integers(2, 5)), self_loop=float(rng.choice([0.0, 0.3])))
    B = int(rng.integers(1, 6))
    T = int(rng.integers(0, 24))
    lp = synth.random_logprobs(seed, B, max(T, 1), vocab, sigma=float(rng.uniform(0.5, 3.0)))
    if T == 0:
        lp = lp[:, :0, :]
    lengths = rng.integers(0, T + 1, size=B).astype(np.int32)
    beam = float(rng.choice([0.5, 2.0, 5.0, 12.0, 1e10]))
    max_active = int(rng.choice([1, 2, 5, 20, 1000]))
    min_active = int(rng.choice([0, 0, 3]))
    allow_partial = bool(rng.integers(0, 2))
    P = int(rng.integers(1, 5)) if eps else 0
    return g, lp, lengths, beam, max_active, min_active, allow_partial, P


@pytest.mark.parametrize("eps", [False, True])
def test_random_small_graphs(eps):
    for seed in range(150):
        g, lp, L, beam, ma, mi, ap, P = _random_case(seed + (1000 if eps else 0), eps)
        _say("random", eps, seed, lp.shape, beam, ma, mi, ap, P)
        mode = ("graph", "eager", "plain", "arcid", "wrap", "wrap_eager", "hash", "hash_wrap")[seed % 8]
        r, steps, _ = gpu_decode(g, lp, L, beam, ma, mi, ap, P, **MODES[mode])
        o = oracle_lanes(g, lp, L, beam, ma, mi, ap, P)
        compare_batch(r, steps, o)


@pytest.mark.parametrize("grid", [1, 3, 8, 1000])
def test_grid_sizes(grid):
    """Any workgroup count of the frame-loop kernels (grid_blocks): one, a
    prime, a multiple of the XCD count, more workgroups than work. The
    per-wavefront shares, the bookkeeping of workgroup 0 and the XCD-aware
    block order change with it; random graphs with and without epsilon arcs
    and the mid-size workload's first lanes equal the oracle's results and
    per-step records."""
    for seed in range(12):
        eps = bool(seed % 2)
        g, lp, L, beam, ma, mi, ap, P = _random_case(3000 + seed, eps)
        _say("grid", grid, seed, lp.shape, P)
        r, steps, _ = gpu_decode(g, lp, L, beam, ma, mi, ap, P, grid_blocks=grid)
        compare_batch(r, steps, oracle_lanes(g, lp, L, beam, ma, mi, ap, P))
    g, lp, L = synth.workload_inputs(2)
    wl = synth.WORKLOADS[2]
    lp2 = np.ascontiguousarray(lp[:3, :60])
    L2 = np.minimum(L[:3], 60).astype(np.int32)
    r, steps, _ = gpu_decode(g, lp2, L2, wl.beam, wl.max_active, grid_blocks=grid)
    compare_batch(r, steps, oracle_lanes(g, lp2, L2, wl.beam, wl.max_active))


def test_greedy_closed_form_gpu():
    V, T = 500, 60
    spec = {"start": 0, "vocab": V, "epsilon_id": -1,
            "states": [[[0, v, v + 1, 0.0] for v in range(V)] + [[1, -1, 0, 0.0]], []]}
    g = graph_from_states(spec)
    lp = synth.random_logprobs(77, 3, T, V, sigma=3.0)
    r, _, _ = gpu_decode(g, lp, [T, T - 7, 0], 10.0, 100)
    for b, Tb in enumerate([T, T - 7, 0]):
        exp = list(np.argmax(lp[b, :Tb], axis=1)) + [V]
        s = np.float32(0.0)
        for t in range(Tb):
            s = np.float32(s + lp[b, t].max())
        assert list(r.arcs[b]) == exp
        assert r.scores[b] == s


def test_graph_from_arrays():
    """A graph uploaded from plain arrays decodes to the oracle's result."""
    g = synth.random_graph(77, n=40, deg=(1, 6), vocab=7, self_loop=0.3)
    lp = synth.random_logprobs(78, 3, 25, g.vocab)
    L = np.array([25, 11, 0], np.int32)
    dg = wb.Graph.from_arrays(g.row_splits, g.dest, g.ilabel, g.olabel, g.weight, start=g.start, vocab=g.vocab,
                              epsilon_id=g.epsilon_id)
    try:
        r, steps, _ = gpu_decode(g, lp, L, 8.0, 50, dgraph=dg)
    finally:
        dg.release()
    compare_batch(r, steps, oracle_lanes(g, lp, L, 8.0, 50))


# ------------------------------------------------------------- workloads

WORKLOAD_IDS = [1, 2, 5, 4, 3]


@pytest.fixture(scope="module")
def workload_graphs():
    return {}


@pytest.mark.parametrize("cid", WORKLOAD_IDS)
def test_workload_parity(cid, workload_graphs):
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    _say("workload", cid, lp.shape, lp.dtype)
    dg = wb.Graph(g)
    runs = {}
    try:
        extra = {2: ("plain", "wrap", "hash_big"), 3: ("arcid", "hash_big"), 4: ("plain", "wrap", "hash_big"),
                 5: ("hash_big",)}.get(cid, ())
        for mode in ("graph", "eager") + extra:
            runs[mode] = gpu_decode(g, lp, L, wl.beam, wl.max_active, 0, False, wl.eps_iterations,
                                    dgraph=dg, **MODES[mode])
            _say("  gpu", mode, "done; stats", runs[mode][2])
    finally:
        dg.release()
    o = oracle_lanes(g, lp, L, wl.beam, wl.max_active, 0, False, wl.eps_iterations)
    _say("  oracle done")
    for mode, (r, steps, stats) in runs.items():
        _say("  compare", mode)
        compare_batch(r, steps, o)
        for b in range(lp.shape[0]):
            check_path(g, lp[b].astype(np.float32), int(L[b]), r.arcs[b], r.words[b], r.scores[b], 1)
        assert stats["arcs"] == sum(int(x["steps"][:, 4].sum()) for x in o)


def test_graph_replay_equals_eager_and_is_idempotent():
    cid = 2
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    import torch
    dg = wb.Graph(g)
    dec_g = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=wl.batch, max_frames=wl.frames, use_graphs=True)
    dec_e = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=wl.batch, max_frames=wl.frames, use_graphs=False)
    # rounds number on across decodes; with a period of 500 rounds they pass a
    # wrap every second decode (then the decode starts at the next multiple
    # with the table wiped)
    dec_p = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=wl.batch, max_frames=wl.frames, use_graphs=True,
                       epoch_period=500)
    x = torch.from_numpy(lp).cuda()
    runs = [dec_g.decode(x, L), dec_g.decode(x, L), dec_e.decode(x, L), dec_g.decode(x, L)]
    runs += [dec_p.decode(x, L) for _ in range(4)]
    for rr in runs[1:]:
        for b in range(wl.batch):
            assert np.array_equal(rr.arcs[b], runs[0].arcs[b])
            assert np.array_equal(rr.words[b], runs[0].words[b])
        assert np.array_equal(rr.scores.view(np.uint32), runs[0].scores.view(np.uint32))
        assert np.array_equal(rr.meta, runs[0].meta)
    dec_g.close(); dec_e.close(); dec_p.close(); dg.release()


def test_lane_result_independent_of_batchmates():
    cid = 2
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    import torch
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=wl.batch, max_frames=wl.frames)
    full = dec.decode(torch.from_numpy(lp).cuda(), L)
    for b in (0, 5):
        one = dec.decode(torch.from_numpy(np.ascontiguousarray(lp[b:b + 1])).cuda(), L[b:b + 1])
        assert np.array_equal(one.arcs[0], full.arcs[b])
        assert one.scores[0].view(np.uint32) == full.scores[b].view(np.uint32)
    # a shorter batch after a longer one reuses the same decoder
    part = dec.decode(torch.from_numpy(np.ascontiguousarray(lp[2:5, :100])).cuda(), np.minimum(L[2:5], 100))
    o = oracle_lanes(g, np.ascontiguousarray(lp[2:5, :100]), np.minimum(L[2:5], 100), wl.beam, wl.max_active)
    for b in range(3):
        compare_lane(b, part, None, o[b], check_steps=False)
    dec.close(); dg.release()


# ------------------------------------------------------------ errors, overflow

def test_decode_argument_errors():
    import torch
    g = graph_from_states(load_golden("tie_chain.json")["graph"])
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 10.0, 100, max_lanes=2, max_frames=4)
    x = torch.zeros((2, 4, g.vocab), device="cuda")
    with pytest.raises(wb.WfstError):
        dec.decode(x, [5, 1])                      # length > T
    with pytest.raises(wb.WfstError):
        dec.decode(torch.zeros((3, 4, g.vocab), device="cuda"), [1, 1, 1])   # B > max_lanes
    with pytest.raises(wb.WfstError):
        dec.decode(torch.zeros((1, 5, g.vocab), device="cuda"), [1])         # T > max_frames
    with pytest.raises(wb.WfstError):
        dec.decode(torch.zeros((1, 4, g.vocab + 1), device="cuda"), [1])     # V mismatch
    with pytest.raises(wb.WfstError):
        dec.decode(torch.zeros((0, 4, g.vocab), device="cuda"), [])          # an empty batch
    r = dec.decode(x, [0, 3])
    assert r.meta[0, 0] == 1
    dec.close(); dg.release()
    with pytest.raises(wb.WfstError):
        wb.Decoder(wb.Graph(g), -1.0, 10)
    dg = wb.Graph(g)
    for bad in (dict(plain_keys=3), dict(epoch_period=1), dict(epoch_period=-1), dict(epoch_period=65536)):
        with pytest.raises(wb.WfstError):
            wb.Decoder(dg, 10.0, 100, max_lanes=2, max_frames=4, **bad)
    wb.Decoder(dg, 10.0, 100, max_lanes=2, max_frames=4, epoch_period=2).close()
    dg.release()


@pytest.mark.parametrize("cid,cap,bit", [(2, "frontier_cap", 16), (2, "arena_entries", 4),
                                         (2, "claims_cap", 8), (2, "slot_cap", 1), (2, "recomb_slots", 2),
                                         (4, "frontier_cap", 16), (4, "arena_entries", 4), (4, "recomb_slots", 2)])
def test_capacity_overflow_is_flagged(cid, cap, bit):
    import torch
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    _say("overflow", cid, cap)
    caps = {"frontier_cap": {"frontier_cap": 2000 if cid == 4 else 64, "claims_cap": 1000000},
            "arena_entries": {"arena_entries": 40000 if cid == 4 else 4096},
            "claims_cap": {"frontier_cap": 100000, "claims_cap": 64},
            "slot_cap": {"slot_cap": 256},
            "recomb_slots": {"recomb_slots": 64}}[cap]
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=2, max_frames=wl.frames,
                     eps_iterations=wl.eps_iterations, **caps)
    x = torch.from_numpy(np.ascontiguousarray(lp[:2])).cuda()
    r = dec.decode(x, L[:2])
    assert all(int(r.meta[b, 2]) & bit for b in range(2))
    assert all(int(r.meta[b, 0]) == 0 for b in range(2))
    # the same decoder recovers on a decode that fits (a claims overflow leaves
    # stale recombination-table entries that the next decode clears first)
    short = np.array([1, 2], dtype=np.int32)
    r2 = dec.decode(x, short)
    o = oracle_lanes(g, lp[:2], short, wl.beam, wl.max_active, eps_iterations=wl.eps_iterations)
    for b in range(2):
        compare_lane(b, r2, None, o[b], check_steps=False)
    dec.close(); dg.release()


def test_threads_and_streams():
    """Two threads sharing one decoder (its calls are serial), then two decoders
    running at once on streams of their own: every result equals a sequential
    decode's."""
    import threading
    import torch
    cid = 2
    g, lp, L = synth.workload_inputs(cid)
    wl = synth.WORKLOADS[cid]
    halves = [(np.ascontiguousarray(lp[:4]), L[:4]), (np.ascontiguousarray(lp[4:]), L[4:])]
    dg = wb.Graph(g)
    got, errs = {}, []
    try:
        want = [gpu_decode(g, x, n, wl.beam, wl.max_active, dgraph=dg, with_steps=False)[0] for x, n in halves]
        decs = [wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=4, max_frames=lp.shape[1]) for _ in range(2)]
        xs = [torch.from_numpy(x).cuda() for x, _ in halves]
        torch.cuda.synchronize()

        def run(tag, dec, i, stream):
            try:
                with torch.cuda.stream(stream):
                    for rep in range(3):
                        got[(tag, i, rep)] = dec.decode(xs[i], halves[i][1])
            except Exception as e:      # reported below, in the test's thread
                errs.append(e)

        for tag, pick in (("shared", lambda i: decs[0]), ("own", lambda i: decs[i])):
            _say("threads", tag)
            ths = [threading.Thread(target=run, args=(tag, pick(i), i, torch.cuda.Stream())) for i in range(2)]
            for th in ths:
                th.start()
            for th in ths:
                th.join()
        for dec in decs:
            dec.close()
    finally:
        dg.release()
    assert not errs, errs
    assert len(got) == 12
    for (tag, i, rep), r in got.items():
        w = want[i]
        for b in range(4):
            assert np.array_equal(r.arcs[b], w.arcs[b]) and np.array_equal(r.words[b], w.words[b]), (tag, i, rep, b)
            assert np.float32(r.scores[b]) == np.float32(w.scores[b]) and np.array_equal(r.meta[b], w.meta[b])


def test_buffers_not_on_the_device_are_rejected():
    """log_prob in pinned host memory (readable by the GPU, so no access can
    fault) is refused by the C ABI with WFST_EINVAL before any launch: decode,
    blank-skip input and output."""
    import ctypes
    import torch
    g = synth.random_graph(31, n=10, deg=(1, 4), vocab=5)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 8.0, 100, max_lanes=2, max_frames=10)
    host = torch.zeros((2, 10, g.vocab), dtype=torch.float32, pin_memory=True)
    dev = torch.zeros((2, 10, g.vocab), dtype=torch.float32, device="cuda")
    lens = np.array([10, 5], np.int32)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out_words, wl, out_arcs, al, sc, meta = dec._outputs(2, 12, 12)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = wb._lib.wfst_decode(dec.handle, ctypes.c_void_p(host.data_ptr()), 2, 10, g.vocab, p(lens), s,
                             p(out_words), 12, p(wl), p(out_arcs), 12, p(al), p(sc), p(meta))
    assert rc == -1 and b"device memory" in wb._lib.wfst_last_error()
    outl = np.zeros(2, np.int32)
    for src, dst in ((host, dev), (dev, host)):
        rc = wb._lib.wfst_blank_skip(dec.handle, ctypes.c_void_p(src.data_ptr()), 2, 10, g.vocab, p(lens), 0,
                                     ctypes.c_float(0.98), ctypes.c_void_p(dst.data_ptr()), p(outl), s)
        assert rc == -1 and b"device memory" in wb._lib.wfst_last_error()
    r = dec.decode(dev, lens)                  # the decoder still works
    assert r.meta.shape == (2, 3)
    dec.close()
    dg.release()


def test_profiled_decode_matches_and_times_every_step_kernel():
    """With per-launch timing on (plain launches, an event pair per dispatch) a
    decode returns the same results; every step launches the two step kernels."""
    import torch
    g, lp, L = synth.workload_inputs(2)
    wl = synth.WORKLOADS[2]
    lp2, L2 = np.ascontiguousarray(lp[:3]), L[:3]
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=3, max_frames=lp.shape[1])
    x = torch.from_numpy(lp2).cuda()
    r0 = dec.decode(x, L2)
    dec.profile(True)
    r1 = dec.decode(x, L2)
    kt = dec.kernel_times()
    dec.profile(False)
    r2 = dec.decode(x, L2)
    dec.close()
    dg.release()
    steps = int(L2.max()) + 1
    assert kt["max"][1] == steps and kt["finalize"][1] == steps and kt["max"][0] > 0.0
    for r in (r1, r2):
        for b in range(3):
            assert np.array_equal(r.arcs[b], r0.arcs[b]) and np.float32(r.scores[b]) == np.float32(r0.scores[b])
