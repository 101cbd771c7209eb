"""GPU test of wfst_decode_noalloc, the decode for callers that cannot allocate
device memory: its workspace lives in the library's static device scratch.
Through the C ABI its results must equal wfst_decode's (a decoder object with
the same graph, configuration and inputs) to the parity bar: arc ids, words,
reached-final and overflow bits equal, scores bit-equal. Two calls run in a row,
the second on a smaller batch, so the second finds the first one's leftovers
in the scratch; a call on a graph with epsilon arcs in between, and the oracle
beside them."""

import numpy as np
import pytest
import torch

import synth
import wfst_beam_search_amd as wb
from gpu_util import oracle_lanes, compare_batch

pytestmark = pytest.mark.gpu

# capacities that fit the scratch (the derived defaults are sized for decoder
# objects and do not)
CAPS = dict(frontier_cap=4096, claims_cap=16384, slot_cap=65536, arena_entries=1 << 16)


def _both(g, dg, lp, lengths, beam, max_active, eps_iterations=0, max_lanes=4, max_frames=48):
    lp_dtype = "f16" if lp.dtype == np.float16 else "f32"
    cfg = dict(max_lanes=max_lanes, max_frames=max_frames, lp_dtype=lp_dtype, eps_iterations=eps_iterations, **CAPS)
    x = torch.from_numpy(np.ascontiguousarray(lp)).cuda()
    print(f"noalloc case: B={lp.shape[0]} T={lp.shape[1]} V={lp.shape[2]} states={g.num_states} "
          f"eps={eps_iterations}", flush=True)
    got = wb.decode_noalloc(dg, x, lengths, beam, max_active, **cfg)
    dec = wb.Decoder(dg, beam, max_active, **cfg)
    ref = dec.decode(x, lengths)
    dec.close()
    return got, ref


def _same(got, ref, B):
    for b in range(B):
        assert np.array_equal(got.arcs[b], ref.arcs[b]), f"lane {b}: arc ids differ"
        assert np.array_equal(got.words[b], ref.words[b]), f"lane {b}: words differ"
        assert np.float32(got.scores[b]).tobytes() == np.float32(ref.scores[b]).tobytes(), f"lane {b}: score bits"
        assert np.array_equal(got.meta[b], ref.meta[b]), f"lane {b}: meta {got.meta[b]} vs {ref.meta[b]}"
        assert int(got.word_lens[b]) == int(ref.word_lens[b]) and int(got.arc_lens[b]) == int(ref.arc_lens[b])


def test_noalloc_equals_decode_two_calls_second_smaller():
    g = synth.random_graph(501, n=300, deg=(1, 8), vocab=9, self_loop=0.3)
    ge = synth.random_graph(502, n=200, deg=(1, 6), vocab=9, epsilon=True, eps_levels=4)
    dg, dge = wb.Graph(g), wb.Graph(ge)
    try:
        # first call: 4 lanes of up to 40 frames
        lp1 = synth.random_logprobs(503, 4, 40, g.vocab, sigma=2.5)
        L1 = np.array([40, 33, 0, 17], dtype=np.int32)
        got, ref = _both(g, dg, lp1, L1, 8.0, 150)
        _same(got, ref, 4)
        compare_batch(got, None, oracle_lanes(g, lp1, L1, 8.0, 150), check_steps=False)
        # a graph with epsilon arcs in between (its position maps and closure lists)
        lpe = synth.random_logprobs(504, 3, 30, ge.vocab, sigma=2.0)
        Le = np.array([30, 12, 25], dtype=np.int32)
        got, ref = _both(ge, dge, lpe, Le, 7.0, 120, eps_iterations=3)
        _same(got, ref, 3)
        compare_batch(got, None, oracle_lanes(ge, lpe, Le, 7.0, 120, eps_iterations=3), check_steps=False)
        # second call on the first graph: a smaller batch, shorter frames, fp16
        lp2 = synth.random_logprobs(505, 2, 20, g.vocab, sigma=2.5, dtype="f16")
        L2 = np.array([20, 9], dtype=np.int32)
        got, ref = _both(g, dg, lp2, L2, 8.0, 150)
        _same(got, ref, 2)
        compare_batch(got, None, oracle_lanes(g, lp2, L2, 8.0, 150), check_steps=False)
    finally:
        dg.release()
        dge.release()


def test_noalloc_tiny_workload():
    g, lp, L = synth.workload_inputs(1)
    wl = synth.WORKLOADS[1]
    dg = wb.Graph(g)
    try:
        got, ref = _both(g, dg, lp, L, wl.beam, wl.max_active, max_lanes=1, max_frames=wl.frames)
        _same(got, ref, 1)
        compare_batch(got, None, oracle_lanes(g, lp, L, wl.beam, wl.max_active), check_steps=False)
    finally:
        dg.release()


def test_noalloc_refuses_a_workspace_larger_than_the_scratch():
    g = synth.random_graph(506, n=50, deg=(1, 4), vocab=5)
    dg = wb.Graph(g)
    try:
        x = torch.zeros((1, 4, g.vocab), dtype=torch.float32, device="cuda")
        with pytest.raises(wb.WfstError, match="bytes"):
            wb.decode_noalloc(dg, x, [4], 5.0, 100, max_lanes=8, max_frames=4, arena_entries=1 << 24)
        with pytest.raises(wb.WfstError, match="lattice"):
            wb.decode_noalloc(dg, x, [4], 5.0, 100, max_lanes=1, max_frames=4, lattice=True, **CAPS)
    finally:
        dg.release()
