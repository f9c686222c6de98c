"""Pins for the fp64 oracle: values printed on the pages, closed forms, special
cases, brute force and invariances. None of these re-types the oracle's formula:
each compares it with something fixed independently of it."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import emulate as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- pages' numbers
def test_worked_example_exact_value_all_forms():
    g = _gold("worked_example.json")
    tol = 0.5 * 10.0 ** -g["exact_output_printed_decimals"]
    s, v = synth.worked_example_scores_values()
    assert len(s) == g["tokens"]
    # pure-Python exactly-rounded form
    o_b, _ = oracle.decode_brute(s, v)
    assert abs(o_b - g["exact_output"]) <= tol
    # the same input as a real paged decode problem (q = e0, k = s e0, v = val e0)
    case = synth.worked_example_decode(head_dim=64)
    q, kc, vc = case.as_f64()
    O, L = oracle.decode_dense(q, kc, vc, case.block_table, case.seq_lens, case.scale)
    assert abs(O[0, 0, 0] - g["exact_output"]) <= tol
    assert np.all(O[0, 0, 1:] == 0.0)
    assert abs(L[0, 0] - (max(s) + math.log(sum(math.exp(x - max(s)) for x in s)))) < 1e-12
    # split form with the page-aligned geometry, merged by log-sum-exp
    for S in (54, 62, 87):
        po, pl = oracle.decode_split_partials(q, kc, vc, case.block_table, case.seq_lens, case.scale, S)
        Oc, Lc = oracle.combine_partials(po, pl)
        assert abs(Oc[0, 0] - g["exact_output"]) <= tol
        assert abs(Lc[0] - L[0, 0]) < 1e-12


def test_worked_example_shuffled_pages_same_result():
    case = synth.worked_example_decode(head_dim=16, shuffle=True)
    q, kc, vc = case.as_f64()
    O, _ = oracle.decode_dense(q, kc, vc, case.block_table, case.seq_lens, case.scale)
    assert abs(O[0, 0, 0] - 1.325056137248) < 5e-13


def test_fa2_split_table():
    g = _gold("worked_example.json")
    for row in g["platforms"]:
        s, nb, bps = E.fa2_split_count(g["tokens"], row["sm_count"])
        assert (s, nb, bps) == (row["splits"], g["key_value_blocks"], row["blocks_per_split"])


def test_page_aligned_groups_reproduce_fa2_boundaries():
    # 16-token pages split into ceil(pages/S) per group land on the same
    # token boundaries as FlashAttention 2's 64-token blocks for S = 54/62/87.
    g = _gold("worked_example.json")
    n_pages = -(-g["tokens"] // 16)
    for row in g["platforms"]:
        rng = oracle.page_split_ranges(n_pages, row["splits"])
        assert (rng[0][1] - rng[0][0]) * 16 == row["first_group_tokens"]
        assert rng[1][0] * 16 == row["first_group_tokens"]


def test_fa2_like_emulation_reproduces_printed_outputs():
    g = _gold("worked_example.json")
    tol = 0.5 * 10.0 ** -g["fp32_output_printed_decimals"]
    s, v = synth.worked_example_scores_values()
    s, v = list(s), list(v)
    for row in g["platforms"]:
        out32, out16, first_n, first_max = E.fa2_like_decode(s, v, row["splits"])
        assert abs(out32 - row["fp32_output"]) <= tol
        assert out16 == row["bf16_output"]
        assert first_n == row["first_group_tokens"]
        assert first_max == row["first_local_max"]


def test_reduction_order_example():
    g = _gold("reduction_order.json")
    a, b = E.reduction_order_example()
    assert a == g["left_first"] and b == g["small_pair_first"]
    assert 2.0 ** -24 == g["half_unit"]


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seqlens,Hq,Hkv,D,causal", [
    ([7], 2, 1, 8, True),
    ([5, 3, 1], 4, 2, 4, True),
    ([6, 4], 2, 2, 8, False),
    ([9], 3, 1, 5, False),
])
def test_dense_matches_brute_force(seqlens, Hq, Hkv, D, causal):
    c = synth.make_prefill(101, 3, seqlens, Hq, Hkv, D, 0.37, causal, "fp32")
    q, k, v = c.as_f64()
    Od, Ld = oracle.attention_dense(q, k, v, c.cu_seqlens, Hq, Hkv, c.scale, causal)
    Ob, Lb = oracle.attention_brute(q, k, v, c.cu_seqlens, Hq, Hkv, c.scale, causal)
    assert np.max(np.abs(Od - Ob)) <= 1e-13
    assert np.max(np.abs(Ld - Lb)) <= 1e-13


def test_decode_matches_brute_force():
    c = synth.make_decode(102, 1, [37, 16, 5], 4, 2, 8, 0.3, shuffle=True)
    q, kc, vc = c.as_f64()
    O, L = oracle.decode_dense(q, kc, vc, c.block_table, c.seq_lens, c.scale)
    for b in range(c.batch):
        n = int(c.seq_lens[b])
        toks = [(int(c.block_table[b, t // 16]), t % 16) for t in range(n)]
        for h in range(4):
            g = h // 2
            for d in range(8):
                sc = [c.scale * math.fsum(q[b, h, e] * kc[p, s, g, e] for e in range(8)) for p, s in toks]
                vals = [vc[p, s, g, d] for p, s in toks]
                o, lse = oracle.decode_brute(sc, vals)
                assert abs(O[b, h, d] - o) < 1e-13
                assert abs(L[b, h] - lse) < 1e-13


# ---------------------------------------------------------------- closed forms
def test_identical_keys_give_mean_of_values():
    T, Hq, Hkv, D = 9, 2, 1, 6
    rng = np.random.default_rng(5)
    q = rng.standard_normal((T, Hq, D))
    k = np.tile(rng.standard_normal((1, Hkv, D)), (T, 1, 1))
    v = rng.standard_normal((T, Hkv, D))
    scale = 0.5
    for causal in (False, True):
        O, L = oracle.attention_dense(q, k, v, [0, T], Hq, Hkv, scale, causal)
        for i in range(T):
            n = i + 1 if causal else T
            for h in range(Hq):
                s = scale * float(np.dot(q[i, h], k[0, 0]))
                assert np.allclose(O[i, h], v[:n, 0].mean(axis=0), atol=1e-14, rtol=0)
                assert abs(L[h, i] - (s + math.log(n))) < 1e-13


def test_one_hot_scores_select_one_value():
    T, D = 6, 4
    q = np.zeros((T, 1, D)); q[:, 0, 0] = 1.0
    k = np.zeros((T, 1, D)); k[:, 0, 0] = np.arange(T) * 0.25
    star = 3
    k[star, 0, 0] = 1000.0          # beats every other score by > 800: exp underflows to 0
    v = np.random.default_rng(1).standard_normal((T, 1, D))
    O, L = oracle.attention_dense(q, k, v, [0, T], 1, 1, 1.0, False)
    assert np.array_equal(O[:, 0], np.tile(v[star, 0], (T, 1)))
    assert np.array_equal(L[0], np.full(T, 1000.0))


def test_causal_row_zero_is_first_value():
    c = synth.make_prefill(103, 0, [11, 4], 4, 2, 8, 0.25, True, "bf16")
    q, k, v = c.as_f64()
    O, L = oracle.attention_dense(q, k, v, c.cu_seqlens, 4, 2, c.scale, True)
    for s0 in c.cu_seqlens[:-1]:
        for h in range(4):
            g = h // 2
            assert np.array_equal(O[s0, h], v[s0, g])
            assert L[h, s0] == c.scale * float(np.dot(q[s0, h], k[s0, g]))


# ---------------------------------------------------------------- invariances
def test_split_count_invariance_and_empty_splits():
    c = synth.make_decode(104, 2, [100, 33, 16, 1], 8, 2, 16, 0.25, shuffle=True)
    q, kc, vc = c.as_f64()
    O, L = oracle.decode_dense(q, kc, vc, c.block_table, c.seq_lens, c.scale)
    for S in (1, 2, 3, 5, 7, 16, 40):
        po, pl = oracle.decode_split_partials(q, kc, vc, c.block_table, c.seq_lens, c.scale, S)
        Oc, Lc = oracle.combine_partials(po, pl)
        assert np.max(np.abs(Oc.reshape(O.shape) - O)) <= 1e-12
        assert np.max(np.abs(Lc.reshape(L.shape) - L)) <= 1e-12
        if S == 40:   # more groups than pages: trailing groups are empty
            assert np.isneginf(pl).any()


def test_score_shift_invariance():
    c = synth.make_prefill(105, 0, [13, 7], 4, 2, 8, 0.25, True, "bf16")
    q, k, v = c.as_f64()
    O, L = oracle.attention_dense(q, k, v, c.cu_seqlens, 4, 2, c.scale, True)
    shift = 3.0
    q2 = np.concatenate([q, np.full(q.shape[:2] + (1,), shift)], axis=2)
    k2 = np.concatenate([k, np.ones(k.shape[:2] + (1,))], axis=2)
    O2, L2 = oracle.attention_dense(q2, k2, v, c.cu_seqlens, 4, 2, c.scale, True)
    assert np.max(np.abs(O2 - O)) <= 1e-12
    assert np.max(np.abs(L2 - (L + c.scale * shift))) <= 1e-12


def test_gqa_equals_repeated_head_mha():
    c = synth.make_prefill(106, 0, [10, 6], 8, 2, 8, 0.3, True, "bf16")
    q, k, v = c.as_f64()
    O, L = oracle.attention_dense(q, k, v, c.cu_seqlens, 8, 2, c.scale, True)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    Or, Lr = oracle.attention_dense(q, kr, vr, c.cu_seqlens, 8, 8, c.scale, True)
    assert np.array_equal(O, Or) and np.array_equal(L, Lr)


def test_packed_varlen_equals_separate_sequences():
    c = synth.make_prefill(107, 0, [5, 12, 1, 8], 4, 1, 8, 0.3, True, "bf16")
    q, k, v = c.as_f64()
    O, L = oracle.attention_dense(q, k, v, c.cu_seqlens, 4, 1, c.scale, True)
    cu = c.cu_seqlens
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        Ob, Lb = oracle.attention_dense(q[s0:s1], k[s0:s1], v[s0:s1], [0, s1 - s0], 4, 1, c.scale, True)
        assert np.array_equal(O[s0:s1], Ob) and np.array_equal(L[:, s0:s1], Lb)


def test_decode_equals_last_row_of_causal_prefill():
    # one decode step over a shuffled paged cache is the last row of a causal
    # prefill over the same tokens: two independent paths through the oracle
    L_ = 45
    pc = synth.make_prefill(108, 0, [L_], 4, 2, 8, 0.3, True, "bf16")
    q, k, v = pc.as_f64()
    O, L = oracle.attention_dense(q, k, v, pc.cu_seqlens, 4, 2, pc.scale, True)
    P = 16
    n_pages = -(-L_ // P)
    perm = np.random.default_rng(0).permutation(n_pages + 3)
    kc = np.full((n_pages + 3, P, 2, 8), np.nan)
    vc = np.full((n_pages + 3, P, 2, 8), np.nan)
    for p in range(n_pages):
        n = min(P, L_ - p * P)
        kc[perm[p], :n] = k[p * P: p * P + n]
        vc[perm[p], :n] = v[p * P: p * P + n]
    bt = perm[:n_pages][None, :].astype(np.int32)
    Od, Ld = oracle.decode_dense(q[L_ - 1][None], kc, vc, bt, np.array([L_]), pc.scale)
    assert np.max(np.abs(Od[0] - O[L_ - 1])) <= 1e-13
    assert np.max(np.abs(Ld[0] - L[:, L_ - 1])) <= 1e-13


# ---------------------------------------------------------------- degenerate cases
def test_combine_empty_rows_and_splits():
    po, pl = synth.random_partials(0, 6, 5, 4, empty_frac=0.4)
    pl[2, :] = -np.inf
    po[2, :] = 0.0
    O, L = oracle.combine_partials(po.astype(np.float64), pl.astype(np.float64))
    assert np.array_equal(O[2], np.zeros(4)) and np.isneginf(L[2])
    # a single non-empty split passes straight through
    po1 = np.zeros((1, 3, 4)); pl1 = np.full((1, 3), -np.inf)
    po1[0, 1] = [1.0, -2.0, 0.5, 3.0]; pl1[0, 1] = 7.25
    O1, L1 = oracle.combine_partials(po1, pl1)
    assert np.array_equal(O1[0], po1[0, 1]) and L1[0] == 7.25


def test_zero_length_decode_sequence():
    c = synth.make_decode(109, 0, [20, 3], 2, 1, 4, 0.5, shuffle=False)
    q, kc, vc = c.as_f64()
    O, L = oracle.decode_dense(q, kc, vc, c.block_table, np.array([0, 3]), c.scale)
    assert np.array_equal(O[0], np.zeros((2, 4))) and np.all(np.isneginf(L[0]))
    assert np.all(np.isfinite(O[1]))


def test_nan_page_tails_never_reach_results():
    c = synth.make_decode(110, 0, [17, 31, 5], 4, 2, 8, 0.3, shuffle=True, tail="nan")
    q, kc, vc = c.as_f64()
    assert np.isnan(kc).any()
    O, L = oracle.decode_dense(q, kc, vc, c.block_table, c.seq_lens, c.scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    po, pl = oracle.decode_split_partials(q, kc, vc, c.block_table, c.seq_lens, c.scale, 3)
    assert np.all(np.isfinite(po))


def test_row_sampler_matches_dense():
    c = synth.make_prefill(111, 0, [40, 9, 23], 4, 2, 8, 0.3, True, "bf16")
    q, k, v = c.as_f64()
    O, L = oracle.attention_dense(q, k, v, c.cu_seqlens, 4, 2, c.scale, True)
    rows = [0, 39, 40, 48, 49, 71, 5]
    Or, Lr = oracle.attention_rows(q, k, v, c.cu_seqlens, 4, 2, c.scale, True, rows)
    assert np.max(np.abs(Or - O[rows])) <= 1e-14
    assert np.max(np.abs(Lr - L[:, rows])) <= 1e-14
    On, Ln = oracle.attention_rows(q, k, v, c.cu_seqlens, 4, 2, c.scale, False, rows)
    Od, Ld = oracle.attention_dense(q, k, v, c.cu_seqlens, 4, 2, c.scale, False)
    assert np.max(np.abs(On - Od[rows])) <= 1e-14
