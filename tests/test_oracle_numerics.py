"""Pins for the scalar emulation of the four decode programs (oracle/emulate).

- In exact arithmetic every program, at every platform's geometry, must give
  the exact output the post prints for its 27,525-token input: a dropped
  correction factor, a wrong weight or a lost group fails this.
- The FlashAttention 2 program reproduces the printed fp32/bf16 outputs (in
  test_oracle_pins); the other programs share its group summary.
- The group counts the post states (16 segments, XQA's 33 and 47 groups) and
  the geometry rules: every token exactly once, tiles dealt round robin,
  FlashAttention 2's groups walked last block first.
- Merges: a single group returns its own normalized output; an empty group is
  ignored by the ordered recurrence; all four merges agree in exact
  arithmetic on arbitrary group records.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import emulate as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PROGRAMS = ("segments16", "fa2", "xqa", "trt")


def _gold():
    with open(os.path.join(GOLD, "worked_example.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("name", PROGRAMS)
def test_every_program_is_exact_in_real_arithmetic(name):
    g = _gold()
    tol = 0.5 * 10.0 ** -g["exact_output_printed_decimals"]
    s, v = synth.worked_example_scores_values()
    for row in g["platforms"]:
        r = E.run_program(name, s, v, row["sm_count"], exact=True)
        assert abs(r.out32 - g["exact_output"]) <= tol, (name, row["platform"], r.out32)


def test_group_counts_stated_by_the_post():
    g = _gold()
    d = g["decode_programs"]
    s, v = synth.worked_example_scores_values()
    sm = {row["platform"]: row["sm_count"] for row in g["platforms"]}
    assert E.run_program("segments16", s, v, sm["H200"]).groups == d["segments"]
    for plat, n in d["xqa_groups"].items():
        assert E.xqa_group_count(g["tokens"], sm[plat], tile_tokens=d["xqa_tile_tokens"]) == n
        assert E.run_program("xqa", s, v, sm[plat]).groups == n
    assert E.run_program("trt", s, v, sm["B200"]).groups == -(-g["tokens"] // d["trt_tile_tokens"])
    for row in g["platforms"]:
        assert E.run_program("fa2", s, v, row["sm_count"]).groups == row["splits"]


@pytest.mark.parametrize("T", [1, 15, 16, 255, 256, 257, 1000, 27525])
def test_geometries_cover_every_token_once(T):
    def check(groups):
        allt = np.sort(np.concatenate(groups))
        assert np.array_equal(allt, np.arange(T))
        assert all(len(g) > 0 for g in groups)
    for S in (1, 3, 54, 87):
        check(E.fa2_groups(T, S))
    check(E.segment_groups(T))
    for P in (1, 5, 33, 47):
        check(E.round_robin_groups(T, P))
    check(E.tile_groups(T))


def test_round_robin_deals_tiles_in_turn():
    groups = E.round_robin_groups(27525, 33)
    for gi, g in enumerate(groups):
        tiles = np.unique(g // 256)
        assert np.all(tiles % 33 == gi)
        assert np.all(np.diff(g) > 0)
    # the last tile is partial: 27525 - 107 * 256 tokens, in group 107 mod 33
    assert len(groups[107 % 33]) == 3 * 256 + (27525 - 107 * 256)


def test_fa2_groups_walk_blocks_backward_and_segments_are_whole_tiles():
    g = E.fa2_groups(1000, 3)        # 16 blocks, 6 per group
    assert list(g[0][:64]) == list(range(320, 384))
    assert list(g[0][-64:]) == list(range(0, 64))
    seg = E.segment_groups(27525)
    assert len(seg[0]) == 108 * 16 and all(len(x) % 16 == 0 for x in seg[:-1])


def _random_parts(rng, n, exact=True):
    A = E.Arithmetic(exact)
    s = rng.standard_normal(40 * n) * 3
    v = rng.standard_normal(40 * n)
    idx = np.array_split(np.arange(40 * n), n)
    return A, s, v, [E.summarize(A, s, v, i) for i in idx]


def test_merges_agree_in_exact_arithmetic_and_match_the_definition():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7):
        A, s, v, parts = _random_parts(rng, n)
        want = math.fsum(math.exp(x - s.max()) * y for x, y in zip(s, v)) / \
            math.fsum(math.exp(x - s.max()) for x in s)
        for merge in (E.merge_lse, E.merge_numerators, E.merge_normalizer_weighted, E.merge_ordered):
            assert abs(merge(A, parts) - want) < 1e-12, merge.__name__


def test_single_group_merges_return_its_output():
    rng = np.random.default_rng(4)
    A, s, v, parts = _random_parts(rng, 1, exact=False)
    p = parts[0]
    assert E.merge_lse(A, parts) == p.out
    assert E.merge_numerators(A, parts) == float(np.float32(np.float32(p.num) / np.float32(p.l)))
    assert E.merge_normalizer_weighted(A, parts) == float(np.float32(np.float32(p.out) * np.float32(p.l))
                                                          / np.float32(p.l))


def test_ordered_merge_skips_empty_groups():
    rng = np.random.default_rng(5)
    A, s, v, parts = _random_parts(rng, 4, exact=False)
    empty = E.Summary(0, -math.inf, 0.0, 0.0, 0.0, -math.inf)
    base = E.merge_ordered(A, parts)
    assert E.merge_ordered(A, [empty] + parts) == base
    assert E.merge_ordered(A, parts[:2] + [empty] + parts[2:]) == base


def test_rounding_points_move_the_result():
    # the bf16 rounding points are live: with them the fp32 outputs differ
    # from the exact value, and the XQA program's differ from FlashAttention 2's
    g = _gold()
    s, v = synth.worked_example_scores_values()
    outs = {n: E.run_program(n, s, v, 132).out32 for n in PROGRAMS}
    assert all(o != g["exact_output"] for o in outs.values())
    assert len(set(outs.values())) == 4
    # every program lands within a few bf16 steps of the exact value
    assert all(abs(o - g["exact_output"]) < 2 ** -6 for o in outs.values())
