"""The no-allocation decode entry point (miattn_attn_decode_paged_noalloc):
called through the C ABI, it gives bitwise the outputs of
miattn_attn_decode_paged on the same inputs, on calls in a row that share its
static per-GPU scratch (the second with a smaller input), and refuses a
problem whose split partials exceed that scratch before enqueuing anything."""
import ctypes
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as mi
import oracle
import synth
from gpu_util import assert_bf16_close, assert_lse_close, bf16_dev, bitwise_equal, host, i32_dev

pytestmark = pytest.mark.gpu


def to_dev(case):
    return (bf16_dev(case.q), bf16_dev(case.k_cache), bf16_dev(case.v_cache), i32_dev(case.block_table),
            i32_dev(case.seq_lens))


def noalloc_c(dev_args, scale, S, o, lse):
    """Direct C-ABI call of the no-allocation entry point (outputs given)."""
    q, kc, vc, bt, sl = dev_args
    B, Hq, D = q.shape
    num_pages, page, Hkv, _ = kc.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return mi.lib.miattn_attn_decode_paged_noalloc(
        p(q), p(kc), p(vc), p(bt), p(sl), B, bt.shape[1], page, num_pages, Hq, Hkv, D, float(scale), int(S),
        p(o), p(lse), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def both(case, S, dev_args):
    q = dev_args[0]
    o_ref, l_ref = mi.attn_decode_paged(*dev_args, scale=case.scale, num_splits=S)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device)
    rc = noalloc_c(dev_args, case.scale, S, o, lse)
    assert rc == mi.OK, mi.last_error()
    torch.cuda.synchronize()
    return o_ref, l_ref, o, lse


@pytest.mark.parametrize("S_big,S_small", [(0, 0), (4, 3)])
def test_noalloc_matches_decode_on_two_calls(S_big, S_small):
    # first call: the 64-sequence paged workload (the library plan at S = 0);
    # second call, smaller: 5 sequences of mixed length, NaN page tails
    big = synth.config3(seed=0)
    small = synth.make_decode(3, 7, [1, 100, 513, 16, 2000], 32, 8, 128, 1 / math.sqrt(128), shuffle=True,
                              tail="nan", name="noalloc_small")
    for case, S in ((big, S_big), (small, S_small)):
        print(f"[noalloc] {case.name} S={S}", flush=True)
        dev = to_dev(case)
        o_ref, l_ref, o, l = both(case, S, dev)
        assert bitwise_equal(o, o_ref) and bitwise_equal(l, l_ref), f"{case.name} S={S}"
        if case is small:
            q, kc, vc = case.as_f64()
            O, L = oracle.decode_dense(q, kc, vc, case.block_table, case.seq_lens, case.scale)
            assert_bf16_close(host(o), O, f"noalloc S={S}")
            assert_lse_close(host(l), L, f"noalloc S={S}")


def test_noalloc_long_context_then_short():
    # 256 splits of one 128K-token sequence (the largest partials of the
    # decode workloads), then 16 splits of a 16K one
    for ctx, S in ((131072, 256), (16384, 16)):
        case = synth.config4(ctx=ctx, seed=0)
        print(f"[noalloc] {case.name} S={S}", flush=True)
        dev = to_dev(case)
        o_ref, l_ref, o, l = both(case, S, dev)
        assert bitwise_equal(o, o_ref) and bitwise_equal(l, l_ref), f"ctx={ctx} S={S}"


def test_noalloc_refuses_partials_beyond_scratch():
    # 64 sequences x 256 splits x 32 heads x 129 floats = 270 MB of partials
    B, Hq, Hkv, D, pages = 64, 32, 8, 128, 256
    need = mi.decode_workspace_bytes(B, Hq, D, 256)
    assert need > mi.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((pages, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, pages), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), 16 * pages, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq), 7.0, dtype=torch.float32, device="cuda")
    rc = noalloc_c((q, kc, kc, bt, sl), 0.1, 256, o, lse)
    assert rc == mi.ERR_WORKSPACE
    assert "static scratch" in mi.last_error()
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all()) and bool((lse == 7.0).all())   # nothing was enqueued
    # and the entry point still works after the refusal
    case = synth.make_decode(3, 8, [300, 40], 32, 8, 128, 0.088, shuffle=True, tail="zero")
    o_ref, l_ref, o2, l2 = both(case, 2, to_dev(case))
    assert bitwise_equal(o2, o_ref) and bitwise_equal(l2, l_ref)
