"""Seeded synthetic inputs for the WFST beam-search decoder: graphs, log-probs, lengths.

This module is shared by the CPU oracle (under ``oracle/``), the tests and the
benchmark. It holds none of the decoder's arithmetic: it only draws random CSR
graphs, CTC log-posteriors and utterance lengths with the shapes and value
distributions of the five workloads listed below, from numpy's PCG64 generator.

Graph conventions (the same ones the decoder's C ABI validates):

* states ``0 .. N-1`` are real states; state ``N`` is an added super-final state
  with no out-arcs, so ``num_states = N + 1``;
* arc id = CSR index; per state the arcs are ordered
  ``[epsilon arcs][emitting arcs][final arcs]``;
* a final arc has ``ilabel = -1``, ``olabel = 0``, ``weight = 0.0f`` and goes to
  state ``N``; every real state has exactly one (every state is final);
* ``weight`` is a log-score ``log U(lo, 1) <= 0`` (drawn in float64, rounded to
  float32): the pages state the weights as ``-log U`` costs, and the decoder adds
  them to log-probabilities, so the generator stores the log-score;
* on the TLG workload ``epsilon_id = 0``: an arc with ``ilabel == 0`` is an
  epsilon arc, emitting ilabels lie in ``[1, 100)``.

Draw order (fixed, so a seed names one input exactly):

* graph, seed ``1000 + c``: out-degrees; [TLG only: levels, epsilon flags,
  epsilon destinations]; [self-loop flags when the workload has them];
  uniform destinations; ilabels; word-arc flags; word ids; weights;
* log-probs, seed ``2000 + c``: one ``normal(0, sigma, (T, V))`` draw per lane,
  lane by lane; ``+boost`` on column 0 (the CTC blank); log-softmax in float64;
  clamp to ``<= 0``; rounding to the workload's dtype (float32 or float16);
* lengths, seed ``3000 + c``: ``integers(lo, hi + 1, size=B)``.
"""

from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "Graph", "make_graph", "make_logprobs", "make_lengths",
    "workload_inputs", "random_graph", "random_logprobs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: graph family, log-prob shape and search settings."""
    cid: int
    name: str
    num_states: int            # real states N (the super-final state is extra)
    degree: tuple              # ("uniform", lo, hi) | ("geom", p, cap) | ("power", alpha, lo, hi)
    vocab: int                 # V, width of the log-prob rows
    ilabel_range: tuple        # emitting ilabels are uniform on [lo, hi)
    word_prob: float           # probability that a non-final arc carries a word id
    word_vocab: int            # word ids are uniform on [1, word_vocab)
    weight_lo: float           # weights are log U(weight_lo, 1)
    self_loop: float           # probability that an emitting arc is a self-loop
    epsilon: bool              # TLG-style epsilon arcs (20% of arcs, acyclic, depth <= 4)
    batch: int                 # B
    frames: int                # T
    lengths: tuple             # lengths uniform on [lo, hi]
    sigma: float               # logits ~ N(0, sigma)
    blank_boost: float         # added to the blank logit (column 0)
    dtype: str                 # "f32" | "f16"
    beam: float
    max_active: int

    @property
    def epsilon_id(self) -> int:
        return 0 if self.epsilon else -1

    @property
    def eps_iterations(self) -> int:
        return 4 if self.epsilon else 0


WORKLOADS = {
    1: Workload(1, "tiny-200", 200, ("uniform", 1, 10), 32, (0, 32), 0.20, 100, 0.05, 0.0,
                False, 1, 50, (50, 50), 2.0, 3.0, "f32", 10.0, 1000),
    2: Workload(2, "mid-hlg-50k", 50_000, ("geom", 0.1, 200), 500, (0, 500), 0.15, 10_000,
                0.01, 0.3, False, 8, 200, (150, 200), 3.0, 4.0, "f32", 15.0, 7000),
    3: Workload(3, "hlg-2M", 2_000_000, ("power", 2.1, 2, 5000), 5000, (0, 5000), 0.10,
                200_000, 0.001, 0.0, False, 32, 500, (300, 500), 4.0, 5.0, "f16", 20.0, 10000),
    4: Workload(4, "tlg-1M-eps", 1_000_000, ("geom", 0.1, 200), 100, (1, 100), 0.12, 50_000,
                0.01, 0.0, True, 16, 400, (400, 400), 3.0, 4.0, "f32", 16.0, 8000),
    5: Workload(5, "wide-200k", 200_000, ("geom", 0.1, 200), 500, (0, 500), 0.15, 10_000,
                0.01, 0.3, False, 64, 1000, (600, 1000), 3.0, 4.0, "f16", 12.0, 4000),
}


@dataclasses.dataclass
class Graph:
    """A CSR decoding graph in the decoder's conventions (see the module docstring)."""
    num_states: int            # N + 1 (includes the super-final state, the last one)
    start: int
    vocab: int
    epsilon_id: int
    row_splits: np.ndarray     # int32 [num_states + 1]
    dest: np.ndarray           # int32 [A]
    ilabel: np.ndarray         # int32 [A]
    olabel: np.ndarray         # int32 [A]
    weight: np.ndarray         # float32 [A]

    @property
    def num_arcs(self) -> int:
        return int(self.dest.shape[0])


def _degrees(rng, n, spec):
    kind = spec[0]
    if kind == "uniform":
        return rng.integers(spec[1], spec[2] + 1, size=n)
    if kind == "geom":
        return np.minimum(rng.geometric(spec[1], size=n), spec[2])
    if kind == "power":
        d = np.arange(spec[2], spec[3] + 1)
        p = d.astype(np.float64) ** (-float(spec[1]))
        p /= p.sum()
        return rng.choice(d, size=n, p=p)
    raise ValueError(f"unknown degree law {spec!r}")


def _build(rng, n, degree, ilabel_range, word_prob, word_vocab, weight_lo, self_loop,
           epsilon, eps_levels=5, eps_share=0.2, start=0, vocab=None):
    """Draw one graph (the draw order is the module docstring's)."""
    deg = _degrees(rng, n, degree).astype(np.int64)
    a_nf = int(deg.sum())
    src = np.repeat(np.arange(n, dtype=np.int64), deg)
    is_eps = np.zeros(a_nf, dtype=bool)
    dest = np.empty(a_nf, dtype=np.int64)
    if epsilon:
        levels = rng.integers(0, eps_levels, size=n)
        order = np.argsort(levels, kind="stable")
        first_of_level = np.searchsorted(levels[order], np.arange(eps_levels + 1))
        # an arc can be epsilon only if some state sits on a strictly higher level
        low = first_of_level[levels[src] + 1] < n
        q = eps_share * a_nf / max(1, int(low.sum()))
        is_eps = low & (rng.random(a_nf) < q)
        e_idx = np.nonzero(is_eps)[0]
        lo = first_of_level[levels[src[e_idx]] + 1]
        dest[e_idx] = order[rng.integers(lo, n)]
    m_idx = np.nonzero(~is_eps)[0]
    n_emit = m_idx.shape[0]
    if self_loop > 0.0:
        loop = rng.random(n_emit) < self_loop
        uni = rng.integers(0, n, size=n_emit)
        dest[m_idx] = np.where(loop, src[m_idx], uni)
    else:
        dest[m_idx] = rng.integers(0, n, size=n_emit)
    il = np.zeros(a_nf, dtype=np.int64)
    il[m_idx] = rng.integers(ilabel_range[0], ilabel_range[1], size=n_emit)
    has_word = rng.random(a_nf) < word_prob
    word = rng.integers(1, word_vocab, size=a_nf)
    ol = np.where(has_word, word, 0)
    w = np.log(rng.uniform(weight_lo, 1.0, size=a_nf)).astype(np.float32)

    # epsilon arcs first inside each state's range (stable: arcs were drawn state-major)
    perm = np.lexsort((~is_eps, src))
    src, dest, il, ol, w = src[perm], dest[perm], il[perm], ol[perm], w[perm]

    a = a_nf + n
    row_splits = np.zeros(n + 2, dtype=np.int64)
    row_splits[1:n + 1] = np.cumsum(deg + 1)
    row_splits[n + 1] = a
    pos = np.arange(a_nf, dtype=np.int64) + src          # each earlier state adds one final arc
    fin = row_splits[1:n + 1] - 1
    g_dest = np.empty(a, dtype=np.int32)
    g_il = np.empty(a, dtype=np.int32)
    g_ol = np.empty(a, dtype=np.int32)
    g_w = np.empty(a, dtype=np.float32)
    g_dest[pos], g_il[pos], g_ol[pos], g_w[pos] = dest, il, ol, w
    g_dest[fin], g_il[fin], g_ol[fin], g_w[fin] = n, -1, 0, np.float32(0.0)
    if vocab is None:
        vocab = int(ilabel_range[1])
    return Graph(num_states=n + 1, start=start, vocab=vocab,
                 epsilon_id=0 if epsilon else -1,
                 row_splits=row_splits.astype(np.int32), dest=g_dest, ilabel=g_il,
                 olabel=g_ol, weight=g_w)


def make_graph(cid: int) -> Graph:
    """The graph of workload ``cid`` (seed ``1000 + cid``)."""
    wl = WORKLOADS[cid]
    rng = np.random.Generator(np.random.PCG64(1000 + cid))
    return _build(rng, wl.num_states, wl.degree, wl.ilabel_range, wl.word_prob,
                  wl.word_vocab, wl.weight_lo, wl.self_loop, wl.epsilon, vocab=wl.vocab)


def _logsoftmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=-1, keepdims=True)
    z = np.log(np.exp(logits - m).sum(axis=-1, keepdims=True))
    return logits - m - z


def _draw_logprobs(rng, batch, frames, vocab, sigma, boost, dtype):
    out = np.empty((batch, frames, vocab), dtype=np.float16 if dtype == "f16" else np.float32)
    for b in range(batch):
        x = rng.normal(0.0, sigma, size=(frames, vocab))
        x[:, 0] += boost
        lp = np.minimum(_logsoftmax_rows(x), 0.0)
        out[b] = lp.astype(out.dtype)
    return out


def make_logprobs(cid: int) -> np.ndarray:
    """log_prob[B, T, V] of workload ``cid`` (seed ``2000 + cid``), float32 or float16."""
    wl = WORKLOADS[cid]
    rng = np.random.Generator(np.random.PCG64(2000 + cid))
    return _draw_logprobs(rng, wl.batch, wl.frames, wl.vocab, wl.sigma, wl.blank_boost, wl.dtype)


def make_lengths(cid: int) -> np.ndarray:
    """Per-utterance lengths (int32 [B]) of workload ``cid`` (seed ``3000 + cid``)."""
    wl = WORKLOADS[cid]
    rng = np.random.Generator(np.random.PCG64(3000 + cid))
    return rng.integers(wl.lengths[0], wl.lengths[1] + 1, size=wl.batch).astype(np.int32)


_CACHE: dict = {}


def workload_inputs(cid: int):
    """(graph, log_prob, lengths) of workload ``cid``; memoised in-process."""
    if cid not in _CACHE:
        _CACHE[cid] = (make_graph(cid), make_logprobs(cid), make_lengths(cid))
    return _CACHE[cid]


def random_graph(seed: int, n: int = 6, deg=(1, 3), vocab: int = 4, word_prob: float = 0.5,
                 weight_lo: float = 0.05, self_loop: float = 0.0, epsilon: bool = False,
                 eps_levels: int = 3, eps_share: float = 0.3, word_vocab: int = 20) -> Graph:
    """A small random graph of the same family, for tests (seed ``seed``).

    With ``epsilon`` the emitting ilabels lie in [1, vocab) and epsilon arcs (ilabel 0)
    go from a state's level to a strictly higher one, so epsilon chains have at most
    ``eps_levels - 1`` arcs.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    il_range = (1, vocab) if epsilon else (0, vocab)
    return _build(rng, n, ("uniform", deg[0], deg[1]), il_range, word_prob, word_vocab,
                  weight_lo, self_loop, epsilon, eps_levels=eps_levels, eps_share=eps_share,
                  vocab=vocab)


def random_logprobs(seed: int, batch: int, frames: int, vocab: int, sigma: float = 2.0,
                    boost: float = 3.0, dtype: str = "f32") -> np.ndarray:
    """Small random log_prob[B, T, V] of the workloads' family, for tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw_logprobs(rng, batch, frames, vocab, sigma, boost, dtype)


def drop_finals(g: Graph, seed: int, keep: float) -> Graph:
    """``g`` with the final arc of each real state kept with probability ``keep``
    (seed ``seed``; the start state's too): graphs with sparse finals, where a
    lane may end without a final arc."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = g.num_states - 1
    rs = np.asarray(g.row_splits, dtype=np.int64)
    drop_state = rng.random(n) >= keep
    src = np.repeat(np.arange(g.num_states), np.diff(rs))
    drop = (np.asarray(g.ilabel) == -1) & np.concatenate([drop_state, [False]])[src]
    keep_arc = ~drop
    counts = np.bincount(src[keep_arc], minlength=g.num_states)
    row_splits = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return Graph(num_states=g.num_states, start=g.start, vocab=g.vocab, epsilon_id=g.epsilon_id,
                 row_splits=row_splits, dest=np.asarray(g.dest)[keep_arc].astype(np.int32),
                 ilabel=np.asarray(g.ilabel)[keep_arc].astype(np.int32),
                 olabel=np.asarray(g.olabel)[keep_arc].astype(np.int32),
                 weight=np.asarray(g.weight)[keep_arc].astype(np.float32))
