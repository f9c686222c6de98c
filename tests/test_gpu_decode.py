"""Paged split-KV decode parity against the fp64 oracle, split-count
agreement, bitwise repeatability and layout invariances."""
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


def to_dev(case):
    return (bf16_dev(case.q), bf16_dev(case.k_cache), bf16_dev(case.v_cache), i32_dev(case.block_table),
            i32_dev(case.seq_lens))


def run(case, S, dev_args=None, **kw):
    args = dev_args or to_dev(case)
    o, l = mi.attn_decode_paged(*args, scale=case.scale, num_splits=S, **kw)
    torch.cuda.synchronize()
    return o, l


def reference(case):
    q, kc, vc = case.as_f64()
    return oracle.decode_dense(q, kc, vc, case.block_table, case.seq_lens, case.scale)


@pytest.mark.parametrize("S", [1, 2, 5, 0])
def test_small_batch_nan_tails(S):
    case = synth.make_decode(3, 1, [1, 15, 16, 17, 100, 300, 33, 64], 32, 8, 128, 1 / math.sqrt(128),
                             shuffle=True, tail="nan", name="small_nan_tails")
    print(f"[decode] {case.name} S={S}", flush=True)
    o, l = run(case, S)
    O, L = reference(case)
    assert_bf16_close(host(o), O, f"S={S}")
    assert_lse_close(host(l), L, f"S={S}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_paged_decode_full_size(seed):
    case = synth.config3(seed=seed)
    print(f"[decode] {case.name} seed={seed} policy split={mi.decode_pick_splits(64, 8, case.max_pages * 16)}",
          flush=True)
    dev = to_dev(case)
    O, L = reference(case)
    for S in (0, 1, 4):
        o, l = run(case, S, dev)
        assert_bf16_close(host(o), O, f"S={S}")
        assert_lse_close(host(l), L, f"S={S}")


@pytest.mark.parametrize("ctx", [16384, 32768, 65536, 131072])
def test_long_context_split_agreement(ctx):
    # every context of the long-decode workload at every split count: oracle
    # parity, a bitwise repeat per split count and pairwise agreement
    case = synth.config4(ctx=ctx, seed=0)
    print(f"[decode] {case.name}", flush=True)
    dev = to_dev(case)
    O, L = reference(case)
    outs = {}
    for S in (1, 16, 64, 256):
        o, l = run(case, S, dev)
        assert_bf16_close(host(o), O, f"ctx={ctx} S={S}")
        assert_lse_close(host(l), L, f"ctx={ctx} S={S}")
        o2, l2 = run(case, S, dev)
        assert bitwise_equal(o, o2) and bitwise_equal(l, l2), f"not bitwise repeatable at S={S}"
        outs[S] = host(o)
    for a in outs:
        for b in outs:
            if a < b:
                mx, mean = errors(outs[a], outs[b])
                assert mx <= 1e-2 and mean <= 1e-3, (a, b, mx, mean)


@pytest.mark.parametrize("ctx", [32768, 65536])
def test_long_context_policy_split(ctx):
    case = synth.config4(ctx=ctx, seed=1)
    dev = to_dev(case)
    O, L = reference(case)
    o, l = run(case, 0, dev)
    assert_bf16_close(host(o), O, f"ctx={ctx} policy")
    assert_lse_close(host(l), L, f"ctx={ctx} policy")


@pytest.mark.parametrize("which,S", [("paged", 4), ("paged", 16), ("long32k", 16), ("long32k", 64)])
def test_split_partials_match_oracle(which, S):
    # the per-split records themselves (contiguous groups of ceil(table width
    # / S) pages, normalised fp32 partial and its LSE; trailing groups of
    # short sequences empty), read back from a caller workspace after the
    # call, against the oracle's split form
    case = synth.config3(seed=2) if which == "paged" else synth.config4(ctx=32768, seed=2)
    print(f"[decode] {case.name} per-split records S={S}", flush=True)
    dev = to_dev(case)
    B, Hq, D = case.q.shape
    ws = torch.empty(mi.decode_workspace_bytes(B, Hq, D, S), dtype=torch.uint8, device="cuda")
    run(case, S, dev, workspace=ws)
    rows = B * Hq
    flat = ws.view(torch.float32)
    po = host(flat[:rows * S * D].view(rows, S, D))
    plse = host(flat[rows * S * D:rows * S * D + rows * S].view(rows, S))
    q, kc, vc = case.as_f64()
    PO, PL = oracle.decode_split_partials(q, kc, vc, case.block_table, case.seq_lens, case.scale, S)
    empty = ~np.isfinite(PL)
    print(f"  {int(empty.sum())} of {empty.size} records empty", flush=True)
    assert np.array_equal(~np.isfinite(plse), empty)
    assert np.all(plse[empty] == -np.inf) and np.all(po[empty] == 0.0)
    assert_bf16_close(po[~empty], PO[~empty], f"partials S={S}")
    mx, _ = errors(plse[~empty], PL[~empty])
    print(f"  partial lse max-abs {mx:.3e}", flush=True)
    assert mx <= 1e-3


def test_worked_example():
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    case = synth.worked_example_decode(head_dim=64)
    dev = to_dev(case)
    allowed = {row["bf16_output"] for row in g["platforms"]}
    for S in (1, 54, 62, 87):
        o, l = run(case, S, dev)
        val = float(o[0, 0, 0].float().cpu())
        print(f"  worked example S={S}: {val!r}", flush=True)
        assert val in allowed
        assert abs(val - g["exact_output"]) <= 1e-2
        assert torch.count_nonzero(o[0, 0, 1:].float()) == 0


def test_shuffled_equals_identity_table():
    ident = synth.make_decode(3, 4, [700, 33, 256], 32, 8, 128, 0.088, shuffle=False, tail="zero")
    shuf = synth.make_decode(3, 4, [700, 33, 256], 32, 8, 128, 0.088, shuffle=True, tail="zero")
    for S in (1, 3):
        oi, li = run(ident, S)
        os_, ls = run(shuf, S)
        assert bitwise_equal(oi, os_) and bitwise_equal(li, ls)


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 128), (8, 1, 64), (16, 2, 256), (6, 3, 128),
                                      (16, 1, 128), (24, 2, 64), (32, 2, 256), (96, 8, 128)])   # G = 12, 16
def test_shapes(Hq, Hkv, D):
    case = synth.make_decode(30, 0, [50, 1, 129, 400], Hq, Hkv, D, 1 / math.sqrt(D), shuffle=True)
    O, L = reference(case)
    for S in (1, 3):
        o, l = run(case, S)
        assert_bf16_close(host(o), O, f"{Hq}x{Hkv} D={D} S={S}")
        assert_lse_close(host(l), L, f"{Hq}x{Hkv} D={D} S={S}")


def test_empty_sequence_and_more_splits_than_pages():
    case = synth.make_decode(31, 0, [40, 3], 8, 2, 128, 0.1, shuffle=True)
    dev = list(to_dev(case))
    dev[4] = i32_dev(np.array([0, 3], np.int32))
    o, l = run(case, 7, tuple(dev))
    O, L = oracle.decode_dense(*case.as_f64(), case.block_table, np.array([0, 3]), case.scale)
    assert torch.count_nonzero(o[0].float()) == 0
    assert torch.all(torch.isneginf(l[0]))
    assert_bf16_close(host(o), O, "empty seq")
    assert_lse_close(host(l), L, "empty seq")


def test_decode_matches_last_row_of_prefill():
    L_ = 333
    pc = synth.make_prefill(32, 0, [L_], 32, 8, 128, 1 / math.sqrt(128), True, "bf16")
    op, lp = mi.attn_fwd(bf16_dev(pc.q), bf16_dev(pc.k), bf16_dev(pc.v), i32_dev(pc.cu_seqlens), L_,
                         scale=pc.scale, causal=True)
    n_pages = (L_ + 15) // 16
    kc = np.zeros((n_pages * 16, 8, 128), np.uint16); vc = np.zeros_like(kc)
    kc[:L_] = pc.k; vc[:L_] = pc.v
    kc = kc.reshape(n_pages, 16, 8, 128); vc = vc.reshape(n_pages, 16, 8, 128)
    od, ld = mi.attn_decode_paged(bf16_dev(pc.q[L_ - 1:L_]), bf16_dev(kc), bf16_dev(vc),
                                  i32_dev(np.arange(n_pages)[None]), i32_dev(np.array([L_])), scale=pc.scale,
                                  num_splits=3)
    torch.cuda.synchronize()
    assert_bf16_close(host(od[0]), host(op[L_ - 1]), "decode vs prefill last row")
    assert np.max(np.abs(host(ld[0]) - host(lp[:, L_ - 1]))) <= 1e-3


def test_caller_workspace():
    case = synth.make_decode(33, 0, [500, 200], 32, 8, 128, 0.09, shuffle=True)
    n = mi.decode_workspace_bytes(2, 32, 128, 4)
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    o1, l1 = run(case, 4, workspace=ws)
    o2, l2 = run(case, 4)
    assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)
    small = torch.empty(8, dtype=torch.float32, device="cuda")
    with pytest.raises(mi.MiattnError):
        run(case, 4, workspace=small)


@pytest.mark.parametrize("S", [0, 2, 4, 16])
def test_library_and_caller_workspace_agree(S):
    case = synth.make_decode(3, 11, [1, 900, 37, 2048, 513, 64, 17, 1500], 32, 8, 128, 1 / math.sqrt(128),
                             shuffle=True, tail="nan", name="workspace_paths")
    dev = to_dev(case)
    O, L = reference(case)
    of, lf = run(case, S, dev)
    ws = torch.empty(mi.decode_workspace_bytes(case.batch, case.num_q_heads, case.head_dim, S),
                     dtype=torch.uint8, device=dev[0].device)
    oc, lc = run(case, S, dev, workspace=ws)
    assert_bf16_close(host(of), O, f"S={S}")
    assert_lse_close(host(lf), L, f"S={S}")
    assert bitwise_equal(of, oc) and bitwise_equal(lf, lc)


def test_repeatable_with_other_shapes_in_between():
    # the library workspace is regrown and reused across shapes; results of a
    # fixed problem keep their bits
    a = synth.make_decode(3, 12, [700, 33, 256, 1000], 32, 8, 128, 0.088, shuffle=True, tail="zero")
    b = synth.make_decode(3, 13, [50] * 17, 16, 4, 64, 0.125, shuffle=True, tail="zero")
    da, db = to_dev(a), to_dev(b)
    o1, l1 = run(a, 3, da)
    for S in (2, 40, 7):
        ob, lb = run(b, S, db)
        o2, l2 = run(a, 3, da)
        assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)
    Ob, Lb = reference(b)
    assert_bf16_close(host(ob), Ob, "interleaved batch")
    assert_lse_close(host(lb), Lb, "interleaved batch")


def test_policy_groups_follow_lengths():
    # num_splits = 0 on a batch the split-count policy splits and large enough
    # for the length-proportional plan (batch x table width >= 2^17 tokens):
    # an empty sequence, a one-token one; parity, repeatability, and agreement
    # with fixed contiguous splits
    lens = [8192, 512, 0, 1, 6000, 700, 8191, 16, 4096, 1500] * 4
    case = synth.make_decode(3, 14, lens, 32, 8, 128, 1 / math.sqrt(128), shuffle=True, tail="nan",
                             name="policy_groups")
    assert mi.decode_pick_splits(case.batch, 8, case.max_pages * 16) > 1
    assert case.batch * case.max_pages * 16 >= 1 << 17
    dev = to_dev(case)
    O, L = reference(case)
    o1, l1 = run(case, 0, dev)
    assert_bf16_close(host(o1), O, "policy groups")
    assert_lse_close(host(l1), L, "policy groups")
    o2, l2 = run(case, 0, dev)
    assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)
    o4, _ = run(case, 4, dev)
    mx, mean = errors(host(o1), host(o4))
    assert mx <= 1e-2 and mean <= 1e-3


def test_group_of_16_query_heads_with_policy_groups():
    # G = 16 (128 query heads on 8 kv heads) on a batch large enough for the
    # length-proportional groups, and at a fixed split count
    lens = [3000, 17, 0, 2048, 1500, 4096, 700, 2500] * 4
    case = synth.make_decode(3, 16, lens, 128, 8, 128, 1 / math.sqrt(128), shuffle=True, tail="nan",
                             name="g16_policy")
    assert case.batch * case.max_pages * 16 >= 1 << 17
    dev = to_dev(case)
    O, L = reference(case)
    for S in (0, 3):
        o, l = run(case, S, dev)
        assert_bf16_close(host(o), O, f"G=16 S={S}")
        assert_lse_close(host(l), L, f"G=16 S={S}")


def test_policy_groups_of_one_sequence_are_the_contiguous_splits():
    # one sequence: the policy's 256 groups are exactly the 256 contiguous
    # splits of the table width, so the bits agree
    case = synth.config4(ctx=16384, seed=3)
    assert mi.decode_pick_splits(1, case.num_kv_heads, case.max_pages * 16) == 256
    dev = to_dev(case)
    o0, l0 = run(case, 0, dev)
    o1, l1 = run(case, 256, dev)
    assert bitwise_equal(o0, o1) and bitwise_equal(l0, l1)


def test_policy_small_launch_contiguous_within_workspace_bound():
    # num_splits = 0 below the plan's size threshold: the policy's contiguous
    # count (256 here) capped at 1 + 256 / batch, so the workspace size
    # published for num_splits = 0 suffices
    case = synth.make_decode(3, 15, [4096, 4000, 100], 8, 1, 128, 1 / math.sqrt(128), shuffle=True,
                             tail="nan", name="small_launch_policy")
    assert mi.decode_pick_splits(case.batch, 1, case.max_pages * 16) > 1 + 256 // case.batch
    dev = to_dev(case)
    O, L = reference(case)
    ws = torch.empty(mi.decode_workspace_bytes(case.batch, case.num_q_heads, case.head_dim, 0),
                     dtype=torch.uint8, device=dev[0].device)
    oc, lc = run(case, 0, dev, workspace=ws)
    assert_bf16_close(host(oc), O, "small launch, caller workspace")
    assert_lse_close(host(lc), L, "small launch, caller workspace")
    ol, ll = run(case, 0, dev)
    assert bitwise_equal(oc, ol) and bitwise_equal(lc, ll)


def test_policy_groups_long_rows_beside_short_ones():
    # length-proportional groups where one sequence takes far more than the
    # 16 splits one wave merges alone (about 80 groups) beside short and empty
    # ones, with 6 query heads per sequence so that some merge workgroups' four
    # rows belong to two sequences: those merge row by row with the whole
    # workgroup, the rest one wave per row
    lens = [40000, 100, 3000, 17, 0, 20000] * 2
    case = synth.make_decode(3, 17, lens, 6, 2, 128, 1 / math.sqrt(128), shuffle=True, tail="nan",
                             name="policy_long_rows")
    assert mi.decode_pick_splits(case.batch, 2, case.max_pages * 16) > 1
    assert case.batch * case.max_pages * 16 >= 1 << 17
    dev = to_dev(case)
    O, L = reference(case)
    o1, l1 = run(case, 0, dev)
    assert_bf16_close(host(o1), O, "policy groups, long rows")
    assert_lse_close(host(l1), L, "policy groups, long rows")
    o2, l2 = run(case, 0, dev)
    assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)
    o4, _ = run(case, 4, dev)
    mx, mean = errors(host(o1), host(o4))
    assert mx <= 1e-2 and mean <= 1e-3
