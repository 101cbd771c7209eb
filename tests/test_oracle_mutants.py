"""The oracle's pins catch planted mistakes. Each mutant is a copy of the
oracle's C source with one plausible mistake in the arithmetic or rule of a
page passage (page "GPU WFST Beam-Search Decoder"), built in a temporary
directory; the pin tests of tests/test_oracle_pins.py run against it and at
least one of them must fail. The unmutated copy, built the same way, passes
them all. The committed oracle is never modified."""

import ctypes
import inspect
import os
import subprocess
import textwrap

import pytest

import oracle
import test_oracle_pins as pins
from cases import load_golden

SRC = os.path.join(os.path.dirname(oracle.__file__), "wfst_oracle.c")

_ADMIT = ("if (!is_final) end = end + row[g->ilabel[a]];\n                if (end > cutoff) {",
          "if (!is_final) end = end + row[g->ilabel[a]];\n                if (end >= cutoff) {")
_CAND = ("float end = cur.score[i] + g->weight[a];\n                if (!is_final) end = end + row[g->ilabel[a]];")

# name (and the passage it breaks): [(text, replacement, occurrences)]
MUTANTS = {
    # section 3 "Admit test": strict
    "admit_not_strict": [(_ADMIT[0], _ADMIT[1], 1)],
    # section 5.3: (score + weight) + log-prob, in that order
    "add_order": [(_CAND, "float end = is_final ? cur.score[i] + g->weight[a]\n"
                          "                                          : cur.score[i] + (g->weight[a] + row[g->ilabel[a]]);", 2)],
    # section 3 "Dynamic beam": the decay, relaxation and widening constants
    "beam_decay": [("b = (b_prev < cfg->beam ? b_prev : cfg->beam) * 0.8f;",
                    "b = (b_prev < cfg->beam ? b_prev : cfg->beam) * 0.75f;", 1)],
    "beam_relax": [("float y = 0.2f * cfg->beam;", "float y = 0.25f * cfg->beam;", 1)],
    "beam_widen": [("b = (b_prev > cfg->beam ? b_prev : cfg->beam) * 1.25f;",
                    "b = (b_prev > cfg->beam ? b_prev : cfg->beam) * 1.5f;", 1)],
    # section 3: min_active raised over the last frames
    "last_frames": [("!cfg->online && T - t <= 5", "!cfg->online && T - t < 5", 1)],
    "max_active_bound": [("if (n > cfg->max_active) {", "if (n >= cfg->max_active) {", 1)],
    # ties: the smaller arc id wins (encoded and decoded consistently the other way)
    "ties_reversed": [("(uint64_t)(0xffffffffu - (uint32_t)arc);", "(uint64_t)(uint32_t)arc;", 1),
                      ("(int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffu));", "(int32_t)(uint32_t)(k & 0xffffffffu);", 2)],
    # section 3, last paragraph: a stream's T is unbounded, so no last-frames rule
    "online_final_window": [("!cfg->online && T - t <= 5", "T - t <= 5", 1)],
    # section 5.5: closure candidates pass the frame cutoff strictly
    "closure_admit_not_strict": [("float end = snap_sc[j] + g->weight[a];\n                stat[0]++;\n                if (end > cutoff) {",
                                  "float end = snap_sc[j] + g->weight[a];\n                stat[0]++;\n                if (end >= cutoff) {", 1)],
    # section 5.5: eps_iterations closure passes
    "closure_one_pass_short": [("for (int32_t pass = 0; pass < passes_max && src.n > 0; pass++)",
                                "for (int32_t pass = 0; pass < passes_max - 1 && src.n > 0; pass++)", 1)],
    # section 3 "Final step": a final arc's weight counts
    "final_weight_dropped": [(_CAND, "float end = is_final ? cur.score[i] : cur.score[i] + g->weight[a];\n"
                                     "                if (!is_final) end = end + row[g->ilabel[a]];", 2)],
    # section 3 on output_beam: keep at >=, and the backward score adds the arc's
    "lattice_keep_strict": [("r[6] = thr >= thresh ? 1 : 0;", "r[6] = thr > thresh ? 1 : 0;", 2)],
    "lattice_backward_drops_arc": [("const float v = sa + bd;", "const float v = bd;", 2)],
    # section 5.5 lattice persistence, reading R31: a frame's epsilon arcs relaxed
    # to a fixpoint, each recorded once per frame
    "lattice_eps_one_round": [("for (int changed = 1; changed;) {", "for (int changed = 1; changed; changed = 0) {", 2)],
    "lattice_eps_no_dedupe": [("if (sc->lat && sc->eps_seen[a] != sc->frame + 1) {", "if (sc->lat) {", 1)],
    # section 7 interval prune, reading R32: the frontier's continuation bound is
    # -fwd, and an arc exactly at the loose threshold stays
    "interval_prune_zero_bound": [("for (int64_t i = 0; i < cur.n; i++) bnext[i] = -cur.score[i];",
                                   "for (int64_t i = 0; i < cur.n; i++) bnext[i] = 0.0f;", 1)],
    "interval_prune_strict": [("keep_e[k - ea0] = ((lt_score.v[fa + i] + sa) + bd) >= thr_loose;",
                               "keep_e[k - ea0] = ((lt_score.v[fa + i] + sa) + bd) > thr_loose;", 1)],
}


# the blank-skip slicing (section 3, WeNet-style; reading R27) is numpy: its
# mutants edit the function's own source
PY_MUTANTS = {
    "blank_drop_at_threshold": ("if not (np.float32(lp[b, t, blank_id]) > lthr)",
                                "if not (np.float32(lp[b, t, blank_id]) >= lthr)"),
    "blank_threshold_binary64": ("lthr = np.float32(np.log(np.float64(np.float32(threshold))))",
                                 "lthr = np.float32(np.log(np.float64(threshold)))"),
}


def _blank_pin_calls():
    return [("blank:" + c["name"], lambda c=c: pins.test_golden_blank_skip(c))
            for c in load_golden("blank_skip.json")["cases"]] + \
           [("blank_threshold_one", pins.test_blank_skip_threshold_one_keeps_everything)]


def _pin_calls():
    calls = []
    for c in load_golden("beam_schedule.json")["cases"]:
        calls.append(("beam_schedule:" + c["name"], lambda c=c: pins.test_golden_beam_schedule(c)))
    for c in load_golden("edge_cases.json")["cases"]:
        calls.append(("edge:" + c["name"], lambda c=c: pins.test_golden_edge_cases(c)))
    calls += [
        ("tie_chain", pins.test_golden_tie_chain),
        ("eps_closure", pins.test_golden_eps_closure),
        ("viterbi", lambda: pins.test_infinite_beam_equals_exact_viterbi(False)),
        ("viterbi_eps", lambda: pins.test_infinite_beam_equals_exact_viterbi(True)),
        ("enumeration", lambda: pins.test_infinite_beam_equals_path_enumeration(False)),
        ("enumeration_eps", lambda: pins.test_infinite_beam_equals_path_enumeration(True)),
        ("closure_depth", pins.test_deeper_closure_needs_more_passes),
        ("greedy", lambda: pins.test_greedy_ctc_closed_form(32, 50)),
        ("greedy_ties", pins.test_greedy_ctc_ties_take_smallest_label),
        ("forced_alignment", pins.test_forced_alignment_closed_form),
        ("beam_rule", lambda: pins.test_logged_beams_follow_the_update_rule(1)),
        ("online_window", lambda: pins.test_online_beams_skip_the_final_window(1)),
        ("partial", lambda: pins.test_partial_at_infinite_beam_equals_trellis_best(False)),
        ("redirect", pins.test_partial_equals_redirect_without_final_arcs),
        ("lattice_bwd", pins.test_lattice_backward_scores_are_best_continuations),
        ("lattice_keep", pins.test_lattice_keep_rule_and_best_path),
        ("lattice_paths", pins.test_lattice_at_infinite_beam_is_every_complete_path),
        ("lattice_ties", pins.test_lattice_keep_at_exact_ties),
        ("eps_lattice_paths", pins.test_eps_lattice_at_infinite_beam_is_every_path_within_output_beam),
        ("eps_lattice_bwd", pins.test_eps_lattice_backward_scores_are_best_continuations),
        ("interval_prune", lambda: pins.test_interval_prune_keeps_the_final_keep_set(False)),
        ("interval_prune_eps", lambda: pins.test_interval_prune_keeps_the_final_keep_set(True)),
    ]
    return calls


def _build(tmp, edits):
    src = open(SRC).read()
    for old, new, count in edits:
        assert src.count(old) == count, f"mutation anchor found {src.count(old)} times, not {count}: {old[:60]!r}"
        src = src.replace(old, new)
    c = os.path.join(tmp, "mutant.c")
    so = os.path.join(tmp, "mutant.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-o", so, c, "-lm"])
    lib = ctypes.CDLL(so)
    ref = oracle._load()
    lib.wo_decode.restype = ref.wo_decode.restype
    lib.wo_decode.argtypes = ref.wo_decode.argtypes
    return lib


def _failing_pins(lib):
    saved = oracle._lib
    oracle._lib = lib
    failed = []
    try:
        for name, call in _pin_calls():
            try:
                call()
            except AssertionError:
                failed.append(name)
    finally:
        oracle._lib = saved
    return failed


def test_unmutated_copy_passes_every_pin(tmp_path):
    assert _failing_pins(_build(str(tmp_path), [])) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    failed = _failing_pins(_build(str(tmp_path), MUTANTS[name]))
    assert failed, f"mutant {name} passes every pin"


def _py_mutant(old, new):
    src = textwrap.dedent(inspect.getsource(oracle.blank_skip))
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<blank_skip mutant>", "exec"), ns)
    return ns["blank_skip"]


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_planted_blank_skip_mistake_is_caught(name):
    saved = oracle.blank_skip
    oracle.blank_skip = _py_mutant(*PY_MUTANTS[name])
    failed = []
    try:
        for pin, call in _blank_pin_calls():
            try:
                call()
            except AssertionError:
                failed.append(pin)
    finally:
        oracle.blank_skip = saved
    assert failed, f"mutant {name} passes every pin"


def test_unmutated_blank_skip_passes_its_pins():
    for _, call in _blank_pin_calls():
        call()
