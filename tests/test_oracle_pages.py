"""The oracle against the worked example printed on the pages.

Pingala-8 blog post, the 1-bit toy trellis.  Data of the example: the cosets
{-1.5, 0.5} (state 0) and {-0.5, 1.5} (state 1), the weights [-0.4, 0.1, 1.5] and the
start state 0.  Its rule, restated: the coded bit selects the smaller (0) or larger (1)
member of the current coset, and that same bit is the state for the next weight.  The
page gives 1.42 as the score of plain 1-bit rounding, and orders the methods: greedy
coding along the trellis scores worse than 1.42, the Viterbi search better.
"""
import json
import os

import numpy as np
import pytest

import brute_force as bf

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def toy():
    with open(os.path.join(HERE, "golden", "toy_trellis.json")) as f:
        return json.load(f)


def _toy_inputs(toy):
    r = toy["bitshift_reading"]
    C = np.array(r["codebook_by_state"], dtype=np.float32).reshape(-1, 1)
    w = np.array(toy["what_the_page_states"]["weights"], dtype=np.float32)
    return w, C, r["L"], r["k"], r["V"], r["T"]


def test_toy_codebook_matches_cosets(toy):
    # the bitshift reading reproduces the page's cosets and "lower/higher" bit rule
    w, C, L, k, V, T = _toy_inputs(toy)
    page = toy["what_the_page_states"]
    for prev in (0, 1):
        rows = [((prev << 1) | b) & 3 for b in (0, 1)]
        vals = [float(C[r, 0]) for r in rows]
        assert vals == page[f"coset_of_state_{prev}"]
        assert vals[0] < vals[1]
    assert sorted(C[:, 0].tolist()) == page["levels"]


def test_toy_scalar_rounding_is_printed_value(oracle_lib, toy):
    # Plain 1-bit rounding to {-1, 1} is the memoryless trellis L = 1, k = 1 (every
    # step may choose freely); the page prints its score as 1.42.
    page = toy["what_the_page_states"]
    w = np.array(page["weights"], dtype=np.float32)
    C = np.array(page["plain_1bit_rounding_to"], dtype=np.float32).reshape(-1, 1)
    bits, s0, cost = oracle_lib.encode_block(w, None, C, 1, 1, 1, 3)
    assert abs(float(cost) - page["plain_1bit_rounding_score"]) < 1e-6


def test_toy_viterbi_beats_rounding_and_greedy_loses(oracle_lib, toy):
    w, C, L, k, V, T = _toy_inputs(toy)
    page = toy["what_the_page_states"]
    scalar = page["plain_1bit_rounding_score"]
    bits, s0, cost = oracle_lib.encode_block(w, None, C, L, k, V, T,
                                             fixed_s0=page["start_state"])
    # greedy: at each step take the closer of the two allowed values
    s, greedy = page["start_state"], 0.0
    for x in w:
        opts = [((s << 1) | b) & 3 for b in (0, 1)]
        errs = [(float(x) - float(C[o, 0])) ** 2 for o in opts]
        b = int(np.argmin(errs))
        greedy += errs[b]
        s = opts[b]
    assert greedy > scalar > float(cost)        # the ordering the page states
    derived = toy["derived_by_enumerating_all_8_paths"]
    assert abs(float(cost) - derived["viterbi_fixed_start_0"]["cost"]) < 1e-6
    assert abs(greedy - derived["greedy_fixed_start_0"]["cost"]) < 1e-6
    dec = oracle_lib.decode_block(bits, s0, C, L, k, V, T)
    assert dec.tolist() == derived["viterbi_fixed_start_0"]["values"]
    # the enumeration agrees
    best = bf.best_path(w, None, C, L, k, V, T, fixed_s0=0)[0]
    assert best == cost


def test_toy_free_start(oracle_lib, toy):
    w, C, L, k, V, T = _toy_inputs(toy)
    derived = toy["derived_by_enumerating_all_8_paths"]["viterbi_free_start"]
    bits, s0, cost = oracle_lib.encode_block(w, None, C, L, k, V, T)
    assert s0 == derived["start_state"]
    assert abs(float(cost) - derived["cost"]) < 1e-6
    dec = oracle_lib.decode_block(bits, s0, C, L, k, V, T)
    assert dec.tolist() == derived["values"]
    # bits 0,1,1 packed MSB-first into the first word
    assert int(bits[0]) == 0b011 << 29
