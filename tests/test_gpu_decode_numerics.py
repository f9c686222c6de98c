"""Numerics variants of the paged split-KV decode (attn_decode_paged_numerics).

Every record kind, rounding point and group geometry must meet the decode's
parity bar against the fp64 oracle (bf16 max-abs 1e-2, mean-abs 1e-3; LSE
1e-3), except the LSE of variants whose normaliser sums rounded weights: each
weight then carries a relative rounding error of up to 2^-8 (bf16) or 2^-11
(fp16), and so can the normaliser, whose log moves by as much; their LSE bar is
that bound plus 1e-4. Beyond that:
- the LSE record with contiguous groups is the fast path, bit for bit;
- round-robin tiles that give each group exactly one tile are the contiguous
  geometry with the same groups, bit for bit, for every record kind;
- the bf16 output is the round-to-nearest-even of the fp32 output;
- on the worked example of "Why your local LLM feels dumber than it is"
  ("Plugging in actual numbers") every variant lands on one of the two bf16
  neighbours of the exact result;
- fixed inputs and split count give bitwise identical results; empty
  sequences give (0, -inf).
test_distance_from_the_fp64_centre prints the study table: each variant's
distance from the fp64 result and from the centre of all variants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as mi
import oracle
import synth
from gpu_util import (assert_bf16_close, assert_lse_close, bf16_dev, bitwise_equal, errors, host, i32_dev)

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")

R_LSE, R_NUM, R_NRM16, R_NUM16 = (mi.RECORD_LSE, mi.RECORD_NUMERATOR_F32, mi.RECORD_NORMALIZED_BF16,
                                  mi.RECORD_NUMERATOR_BF16)
RL, PF16 = mi.NUMERICS_ROUNDED_NORMALIZER, mi.NUMERICS_P_FP16
ALL_NUMERICS = [r | f for r in (R_LSE, R_NUM, R_NRM16, R_NUM16) for f in (0, RL, PF16, RL | PF16)]


def lse_tol(numerics):
    if not numerics & RL:
        return 1e-3
    return (2.0 ** -11 if numerics & PF16 else 2.0 ** -8) + 1e-4


def to_dev(case):
    return (bf16_dev(case.q), bf16_dev(case.k_cache), bf16_dev(case.v_cache), i32_dev(case.block_table),
            i32_dev(case.seq_lens))


def run(args, case, S, numerics, tile_pages=0, out_dtype=torch.bfloat16, **kw):
    o, l = mi.attn_decode_paged_numerics(*args, scale=case.scale, num_splits=S, numerics=numerics,
                                         tile_pages=tile_pages, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return o, l


def reference(case):
    q, kc, vc = case.as_f64()
    return oracle.decode_dense(q, kc, vc, case.block_table, case.seq_lens, case.scale)


def name(numerics, tile_pages):
    rec = {R_LSE: "lse", R_NUM: "num32", R_NRM16: "norm16", R_NUM16: "num16-ordered"}[numerics & 3]
    fl = ("+rl" if numerics & RL else "") + ("+pf16" if numerics & PF16 else "")
    return f"{rec}{fl}/{'rr' + str(tile_pages) if tile_pages else 'contig'}"


def test_lse_record_is_the_fast_path_bitwise():
    case = synth.make_decode(3, 1, [1, 15, 16, 17, 100, 300, 33, 64], 32, 8, 128, 1 / math.sqrt(128),
                             shuffle=True, tail="nan", name="small_nan_tails")
    args = to_dev(case)
    for S in (1, 3, 16):
        o0, l0 = mi.attn_decode_paged(*args, scale=case.scale, num_splits=S)
        o1, l1 = run(args, case, S, R_LSE)
        assert bitwise_equal(o0, o1) and bitwise_equal(l0, l1), S


@pytest.mark.parametrize("tile_pages", [0, 2, 4])
@pytest.mark.parametrize("numerics", ALL_NUMERICS)
def test_small_batch_against_oracle(numerics, tile_pages):
    case = synth.make_decode(3, 1, [1, 15, 16, 17, 100, 300, 33, 64], 32, 8, 128, 1 / math.sqrt(128),
                             shuffle=True, tail="nan", name="small_nan_tails")
    args = to_dev(case)
    O, L = reference(case)
    for S in (1, 3, 7):
        what = f"{name(numerics, tile_pages)} S={S}"
        print(f"[decode-numerics] {case.name} {what}", flush=True)
        o, l = run(args, case, S, numerics, tile_pages)
        assert not torch.isnan(o.float()).any()
        assert_bf16_close(host(o), O, what)
        assert_lse_close(host(l), L, what, lse_tol(numerics))


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 8, 8), (256, 16, 4), (128, 6, 3)])
def test_head_dims(D, Hq, Hkv):
    case = synth.make_decode(30, 2, [50, 1, 129, 400, 1000], Hq, Hkv, D, 1 / math.sqrt(D), shuffle=True,
                             tail="nan")
    args = to_dev(case)
    O, L = reference(case)
    for numerics in (R_NUM, R_NRM16 | RL, R_NUM16, R_LSE | PF16):
        for tp in (0, 4):
            what = f"D={D} {name(numerics, tp)}"
            print(f"[decode-numerics] {what}", flush=True)
            o, l = run(args, case, 5, numerics, tp)
            assert_bf16_close(host(o), O, what)
            assert_lse_close(host(l), L, what, lse_tol(numerics))


def test_paged_decode_full_size():
    case = synth.config3(seed=0)
    args = to_dev(case)
    O, L = reference(case)
    for numerics in (R_NUM, R_NRM16 | RL, R_NUM16, R_LSE | PF16, R_NRM16 | RL | PF16):
        for S, tp in ((4, 0), (16, 0), (8, 4), (32, 8)):
            what = f"config3 {name(numerics, tp)} S={S}"
            print(f"[decode-numerics] {what}", flush=True)
            o, l = run(args, case, S, numerics, tp)
            assert_bf16_close(host(o), O, what)
            assert_lse_close(host(l), L, what, lse_tol(numerics))


@pytest.mark.parametrize("ctx", [16384, 131072])
def test_long_context(ctx):
    case = synth.config4(ctx=ctx, seed=0)
    args = to_dev(case)
    O, L = reference(case)
    for numerics in (R_NUM, R_NRM16 | RL, R_NUM16, R_LSE | PF16):
        for S, tp in ((16, 0), (256, 0), (64, 16), (ctx // 128, 8)):
            what = f"ctx={ctx} {name(numerics, tp)} S={S}"
            print(f"[decode-numerics] {what}", flush=True)
            o, l = run(args, case, S, numerics, tp)
            assert_bf16_close(host(o), O, what)
            assert_lse_close(host(l), L, what, lse_tol(numerics))
            o2, l2 = run(args, case, S, numerics, tp)
            assert bitwise_equal(o, o2) and bitwise_equal(l, l2), what


@pytest.mark.parametrize("numerics", [R_LSE, R_NUM, R_NRM16 | RL, R_NUM16, R_NUM | PF16])
def test_one_tile_per_group_is_the_contiguous_geometry(numerics):
    # 300 pages, tiles of 4 pages: 75 groups of one tile each = contiguous
    # groups of ceil(300 / 75) = 4 pages
    case = synth.make_decode(33, 0, [4800, 4000, 1], 16, 4, 128, 0.09, shuffle=True, tail="nan")
    assert case.block_table.shape[1] == 300
    args = to_dev(case)
    o1, l1 = run(args, case, 75, numerics, 4)
    o2, l2 = run(args, case, 75, numerics, 0)
    assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)


@pytest.mark.parametrize("numerics", [R_LSE, R_NUM, R_NRM16 | RL, R_NUM16 | PF16])
def test_bf16_output_is_the_rounded_fp32_output(numerics):
    case = synth.make_decode(34, 1, [700, 33, 256], 32, 8, 128, 0.088, shuffle=True, tail="zero")
    args = to_dev(case)
    for S, tp in ((3, 0), (5, 2)):
        o32, l32 = run(args, case, S, numerics, tp, out_dtype=torch.float32)
        o16, l16 = run(args, case, S, numerics, tp)
        assert o32.dtype == torch.float32
        assert bitwise_equal(o32.to(torch.bfloat16), o16) and bitwise_equal(l32, l16)


def test_empty_sequences_and_more_groups_than_tiles():
    case = synth.make_decode(31, 0, [40, 3, 90], 8, 2, 128, 0.1, shuffle=True)
    dev = list(to_dev(case))
    dev[4] = i32_dev(np.array([0, 3, 90], np.int32))
    for numerics in ALL_NUMERICS:
        for S, tp in ((7, 0), (9, 1), (5, 2)):
            o, l = run(tuple(dev), case, S, numerics, tp)
            oh, lh = host(o), host(l)
            assert np.all(oh[0] == 0) and np.all(np.isneginf(lh[0])), name(numerics, tp)
            assert np.all(np.isfinite(lh[1:])) and not np.isnan(oh).any(), name(numerics, tp)


def test_caller_workspace_agrees_with_library_workspace():
    case = synth.config4(ctx=16384, seed=2)
    args = to_dev(case)
    for numerics, S, tp in ((R_NUM16, 128, 8), (R_NRM16 | RL, 64, 16)):
        n = mi.decode_numerics_workspace_bytes(case.batch, case.num_q_heads, case.head_dim, S)
        ws = torch.full((n // 4,), float("nan"), dtype=torch.float32, device=args[0].device)
        o1, l1 = run(args, case, S, numerics, tp, workspace=ws)
        o2, l2 = run(args, case, S, numerics, tp)
        assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)


def _worked_example_variants():
    # the split geometries of the post's four programs, expressed in 16-token
    # pages, plus this library's policy
    n_pages = -(-27525 // 16)
    v = [("fa2-like H200 (54 contiguous)", R_LSE, 54, 0), ("fa2-like B200 (62 contiguous)", R_LSE, 62, 0),
         ("fa2-like SM120 (87 contiguous)", R_LSE, 87, 0),
         ("16 segments, fp32 numerators", R_NUM, 16, 0),
         ("xqa-like H200 (33 groups of 256-token tiles)", R_NRM16 | RL, 33, 16),
         ("xqa-like SM120 (47 groups of 256-token tiles)", R_NRM16 | RL, 47, 16),
         ("trt-like (one group per 128-token tile)", R_NUM16, -(-n_pages // 8), 8),
         ("library policy, LSE record", R_LSE, 0, 0),
         ("library policy, LSE record, fp16 P", R_LSE | PF16, 0, 0)]
    return v


def test_worked_example_every_variant():
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    allowed = {row["bf16_output"] for row in g["platforms"]}
    case = synth.worked_example_decode(head_dim=256, num_q_heads=16, num_kv_heads=4)
    args = to_dev(case)
    for label, numerics, S, tp in _worked_example_variants():
        o32, _ = run(args, case, S, numerics, tp, out_dtype=torch.float32)
        o16, _ = run(args, case, S, numerics, tp)
        v32 = host(o32)[0, :, 0]
        v16 = host(o16)[0, :, 0]
        print(f"  worked example {label}: fp32 {v32[0]:.10f} bf16 {v16[0]!r}", flush=True)
        assert np.all(v32 == v32[0]) and np.all(v16 == v16[0]), label   # every head sees the same input
        assert v16[0] in allowed, label
        assert abs(v32[0] - g["exact_output"]) <= 2.0 ** -8, label
        assert torch.count_nonzero(o16[0, :, 1:].float()) == 0


def _study_rows(case, variants, out_dtype=torch.float32):
    args = to_dev(case)
    O, _ = reference(case)
    outs = {}
    for label, numerics, S, tp in variants:
        o, _ = run(args, case, S, numerics, tp, out_dtype=out_dtype)
        outs[label] = host(o)
    centre = np.mean(np.stack(list(outs.values())), axis=0)
    rows = []
    for label, x in outs.items():
        mx, mean = errors(x, O)
        cmx, cmean = errors(x, centre)
        rows.append((label, mx, mean, float(np.sqrt(np.mean((x - O) ** 2))), cmx, cmean))
    return rows, outs, O


def _print_table(title, rows):
    print(f"\n[numerics study] {title}")
    print(f"  {'variant':52s} {'max|x-fp64|':>12s} {'mean|x-fp64|':>13s} {'rms':>10s} "
          f"{'max|x-ctr|':>11s} {'mean|x-ctr|':>12s}")
    for label, mx, mean, rms, cmx, cmean in rows:
        print(f"  {label:52s} {mx:12.3e} {mean:13.3e} {rms:10.3e} {cmx:11.3e} {cmean:12.3e}")


def test_distance_from_the_fp64_centre():
    """The comparison of "Nobody's Right When Everybody's Wrong" run on this
    kernel's variants: distance of each variant's fp32 output (before the final
    bf16 rounding) from the fp64 result and from the mean of all variants."""
    we = synth.worked_example_decode(head_dim=256, num_q_heads=16, num_kv_heads=4)
    rows, _, _ = _study_rows(we, _worked_example_variants())
    _print_table("worked example, 27,525 tokens (one value channel)", rows)
    for mx in (r[1] for r in rows):
        assert mx <= 2.0 ** -8

    c3 = synth.config3(seed=0)
    pol3 = mi.decode_pick_splits(c3.batch, c3.num_kv_heads, c3.max_pages * 16)
    v3 = [("LSE record, policy splits", R_LSE, pol3, 0), ("LSE record, 16 splits", R_LSE, 16, 0),
          ("fp32 numerators, 16 contiguous", R_NUM, 16, 0),
          ("bf16 normalised + rounded l, round robin 16 pages", R_NRM16 | RL, 4, 16),
          ("bf16 numerators ordered, one group per 8 pages", R_NUM16, 32, 8),
          ("LSE record, fp16 P, policy splits", R_LSE | PF16, pol3, 0)]
    rows, _, _ = _study_rows(c3, v3)
    _print_table("paged decode, 64 sequences, ctx U[512,4096], Hq=32 Hkv=8 D=128", rows)
    for r in rows:
        assert r[1] <= 1e-2 and r[2] <= 1e-3, r

    c4 = synth.config4(ctx=32768, seed=0)
    pol4 = mi.decode_pick_splits(1, c4.num_kv_heads, c4.max_pages * 16)
    v4 = [("LSE record, policy splits", R_LSE, pol4, 0), ("LSE record, 16 splits", R_LSE, 16, 0),
          ("fp32 numerators, 16 contiguous", R_NUM, 16, 0),
          ("bf16 normalised + rounded l, 64 groups of 16-page tiles", R_NRM16 | RL, 64, 16),
          ("bf16 numerators ordered, one group per 8 pages", R_NUM16, 256, 8),
          ("LSE record, fp16 P, policy splits", R_LSE | PF16, pol4, 0)]
    rows, _, _ = _study_rows(c4, v4)
    _print_table("long decode, ctx 32768, Hq=16 Hkv=4 D=256, 4 outlier K channels", rows)
    for r in rows:
        assert r[1] <= 1e-2 and r[2] <= 1e-3, r
