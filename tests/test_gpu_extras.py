"""GPU parity of the steps around the search: blank-skip frame pre-slicing done
before the decoder runs (page "GPU WFST Beam-Search Decoder", section 3) against the oracle's slicing
bit for bit, a decode of the sliced frames against the oracle's decode of its
own slicing, and graphs with sparse final arcs (allow_partial on and off,
section 3 "Final step") against the oracle, per-step records included."""

import numpy as np
import pytest

import oracle
import synth
import wfst_beam_search_amd as wb
from cases import load_golden
from gpu_util import compare_batch, gpu_decode, oracle_lanes

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("vocab", [9, 64])      # (rows 16-byte aligned only at 64: the vector copy)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_blank_skip_matches_oracle(dtype, vocab):
    import torch
    g = synth.random_graph(41, n=30, deg=(1, 5), vocab=vocab, self_loop=0.3)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 8.0, 200, max_lanes=6, max_frames=300, lp_dtype=dtype)
    for seed, (B, T, boost, thr) in enumerate([(6, 300, 6.0, 0.98), (3, 77, 4.0, 0.9), (5, 1, 9.0, 0.98),
                                               (2, 129, 0.0, 0.5)]):
        lp = synth.random_logprobs(600 + seed, B, T, g.vocab, boost=boost, dtype=dtype)
        L = np.random.default_rng(seed).integers(0, T + 1, size=B).astype(np.int32)
        x = torch.from_numpy(lp).cuda()
        out, n = dec.blank_skip(x, L, 0, thr)
        want, wn = oracle.blank_skip(lp, L, 0, thr)
        _say("blank skip", dtype, B, T, boost, thr, n, wn)
        assert np.array_equal(n, wn)
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint16 if dtype == "f16" else np.uint32),
                              want.view(np.uint16 if dtype == "f16" else np.uint32))
        r = dec.decode(out, n)
        o = oracle_lanes(g, want, wn, 8.0, 200)
        compare_batch(r, None, o, check_steps=False)
    dec.close()
    dg.release()


def test_blank_skip_golden_on_gpu():
    import torch
    fx = load_golden("blank_skip.json")
    g = synth.random_graph(42, n=5, deg=(1, 3), vocab=3)
    dg = wb.Graph(g)
    dec = wb.Decoder(dg, 8.0, 100, max_lanes=1, max_frames=8)
    for case in fx["cases"]:
        n = len(case["blank_logprob"])
        lp = np.full((1, max(n, 1), 3), -5.0, dtype=np.float32)
        for t, v in enumerate(case["blank_logprob"]):
            lp[0, t, 0] = np.float32(v)
            lp[0, t, 1] = np.float32(-1.0 - t)
        out, k = dec.blank_skip(torch.from_numpy(lp).cuda(), [case["length"]], fx["blank_id"], fx["threshold"])
        got = out.cpu().numpy()
        assert int(k[0]) == len(case["expect_kept"]), case["name"]
        assert np.array_equal(got[0, :k[0]], lp[0, case["expect_kept"]]), case["name"]
    dec.close()
    dg.release()


@pytest.mark.parametrize("keep", [0.0, 0.15, 0.5])
def test_sparse_final_arcs(keep):
    checked = 0
    for seed in range(30):
        rng = np.random.default_rng(90_000 + seed)
        g = synth.drop_finals(synth.random_graph(seed + 300, n=int(rng.integers(3, 40)),
                                                 deg=(1, int(rng.integers(2, 7))), vocab=int(rng.integers(2, 8)),
                                                 self_loop=0.3), seed, keep)
        B = int(rng.integers(1, 5))
        T = int(rng.integers(1, 20))
        lp = synth.random_logprobs(seed + 900, B, T, g.vocab)
        L = rng.integers(0, T + 1, size=B).astype(np.int32)
        ap = bool(seed % 2)
        beam = float(rng.choice([2.0, 6.0, 1e10]))
        ma = int(rng.choice([3, 30, 1000]))
        _say("sparse finals", keep, seed, lp.shape, ap, beam, ma)
        r, steps, _ = gpu_decode(g, lp, L, beam, ma, 0, ap, 0)
        o = oracle_lanes(g, lp, L, beam, ma, 0, ap, 0)
        compare_batch(r, steps, o)
        checked += sum(1 for x in o if x["reached_final"] == 0)
    if keep < 0.5:
        assert checked > 0    # some lanes ended without a final arc


def test_largest_vocabulary():
    """The largest vocabulary the 16-bit labels hold (65534 symbols, labels up to
    65533 beside the final-arc label): arcs on the top labels, rows the top
    labels win, results equal to the oracle's."""
    V = 65534
    g = synth.random_graph(51, n=25, deg=(1, 5), vocab=V, self_loop=0.3)
    il = np.asarray(g.ilabel).copy()
    emit = np.flatnonzero(il >= 0)
    il[emit[::3]] = V - 1
    il[emit[1::3]] = V - 2
    g.ilabel = il
    lp = synth.random_logprobs(52, 3, 30, V, sigma=2.0)
    lp[:, ::2, V - 1] = np.float32(-0.05)
    lp[:, 1::2, V - 2] = np.float32(-0.05)
    L = np.array([30, 17, 1], np.int32)
    _say("vocab", V, lp.shape)
    for dtype in ("f32", "f16"):
        x = lp if dtype == "f32" else lp.astype(np.float16)
        r, steps, _ = gpu_decode(g, x, L, 10.0, 200)
        o = oracle_lanes(g, x, L, 10.0, 200)
        compare_batch(r, steps, o)
        assert any((a >= 0).any() and (il[a[a < il.shape[0]]] >= V - 2).any() for a in r.arcs)


def test_long_utterance():
    """3000 frames (a 3008-step graph bucket), with and without compaction
    rounds: the oracle's path, arc for arc."""
    g = synth.random_graph(53, n=60, deg=(1, 6), vocab=12, self_loop=0.3)
    T = 3000
    lp = synth.random_logprobs(54, 2, T, g.vocab, sigma=2.5)
    L = np.array([T, 1777], np.int32)
    o = oracle_lanes(g, lp, L, 8.0, 300)
    for gi in (0, 64):
        _say("long", T, "interval", gi)
        r, steps, st = gpu_decode(g, lp, L, 8.0, 300, gc_interval=gi)
        compare_batch(r, steps, o)
        assert len(r.arcs[0]) == T + 1
