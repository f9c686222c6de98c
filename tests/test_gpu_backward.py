"""Attention backward (attn_bwd) against the fp64 oracle.

Two comparisons:
- given inputs: attn_bwd is handed Q, K, V, dO and the forward's stored output
  and log-sum-exp as the oracle's own forward produces them (O rounded to
  bf16, LSE to fp32); the reference is oracle.attention_bwd_given on the same
  tensors, i.e. exactly what a recomputing backward defines from its inputs;
- the pipeline: attn_fwd then attn_bwd on the GPU, against the same
  reference and against the exact gradients of oracle.attention_bwd_dense.
Bar for the given-input comparison: the bf16 bar of the forward (max-abs 1e-2,
mean-abs 1e-3) on dQ, dK and dV, with the max-abs part applied to the error
beyond each element's own rounding to bf16: gradients are unbounded sums
(magnitudes up to ~9 here), and half a bf16 ulp is already 0.0156 from 4 up.
Bar for the pipeline: mean-abs 1e-3 against both references, and max-abs
2e-2 on the error beyond each element's own bf16 rounding. The pipeline adds
two error sources, each held to 1e-2 by its own bar: the backward's (the
given-input comparison above) and the forward's output error, which enters
through the stored O (the row term dO . O sums it over the head dimension);
their sum is the pipeline's bound. Beyond parity: bitwise
repeatability, and the closed forms the oracle is pinned with (the keys' dV
sum to the queries' dO sum, the keys' dK sum to zero) on every head at the
full 4096-token size.
"""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as mi
import oracle
import synth
from gpu_util import assert_bf16_close_beyond_rounding as assert_grad_close
from gpu_util import bf16_dev, bitwise_equal, errors, f32_dev, half_ulp_bf16, host, i32_dev

pytestmark = pytest.mark.gpu


def f64(bits):
    return synth.bf16_to_f64(bits)


def inputs(c, seed):
    dout = synth.output_gradient(9, seed, c.total_tokens, c.num_q_heads, c.head_dim)
    return f64(c.q), f64(c.k), f64(c.v), f64(dout), dout


def stored_forward(c, q, k, v):
    """The oracle's forward outputs in their storage formats: O as bf16 bits,
    LSE as float32."""
    O, LSE = oracle.attention_dense(q, k, v, c.cu_seqlens, c.num_q_heads, c.num_kv_heads, c.scale, c.causal)
    return synth.bf16_bits(O.astype(np.float32)), LSE.astype(np.float32)


def max_len(c):
    return int(max(c.seqlens)) if len(c.seqlens) else 1


def gpu_bwd(c, o_dev, lse_dev, dout_bits):
    dq, dk, dv = mi.attn_bwd(bf16_dev(c.q), bf16_dev(c.k), bf16_dev(c.v), o_dev, lse_dev, bf16_dev(dout_bits),
                             i32_dev(c.cu_seqlens), max_len(c), scale=c.scale, causal=c.causal)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def gpu_pipeline(c, dout_bits):
    q, k, v, cu = bf16_dev(c.q), bf16_dev(c.k), bf16_dev(c.v), i32_dev(c.cu_seqlens)
    o, lse = mi.attn_fwd(q, k, v, cu, max_len(c), scale=c.scale, causal=c.causal)
    dq, dk, dv = mi.attn_bwd(q, k, v, o, lse, bf16_dev(dout_bits), cu, max_len(c), scale=c.scale, causal=c.causal)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(got, want, tag):
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        assert_grad_close(g, w, f"{tag} {name}")


def check(c, seed=0, pipeline=True):
    print(f"[bwd] {c.name} lens={list(c.seqlens)[:8]} Hq={c.num_q_heads} Hkv={c.num_kv_heads} D={c.head_dim} "
          f"causal={c.causal}", flush=True)
    q, k, v, do, dout = inputs(c, seed)
    o_bits, lse32 = stored_forward(c, q, k, v)
    ref = oracle.attention_bwd_given(q, k, v, f64(o_bits), lse32.astype(np.float64), do, c.cu_seqlens,
                                     c.num_q_heads, c.num_kv_heads, c.scale, c.causal)
    compare(gpu_bwd(c, bf16_dev(o_bits), f32_dev(lse32), dout), ref, f"{c.name} given")
    if pipeline:
        got = [host(x) for x in gpu_pipeline(c, dout)]
        exact = oracle.attention_bwd_dense(q, k, v, do, c.cu_seqlens, c.num_q_heads, c.num_kv_heads, c.scale,
                                           c.causal)
        for what, want in (("given-form reference", ref), ("exact gradients", exact)):
            for name, g, w in zip(("dQ", "dK", "dV"), got, want):
                mx, mean = errors(g, w)
                excess = float(np.max(np.abs(g - w) - half_ulp_bf16(w))) if g.size else 0.0
                print(f"  {c.name} pipeline vs {what} {name}: max-abs {mx:.3e} (beyond rounding {excess:.3e}) "
                      f"mean-abs {mean:.3e}", flush=True)
                assert mean <= 1e-3, (what, name, mean)
                assert excess <= 2e-2, (what, name, excess)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 8), (128, 8, 4), (128, 4, 2), (64, 16, 2),
                                      (128, 24, 8), (64, 12, 2), (128, 5, 1),    # G = 3, 6, 5 too
                                      (256, 16, 4), (256, 4, 4), (256, 6, 2)])   # head_dim 256
def test_small_varlen(D, Hq, Hkv, causal):
    # ragged lengths: a single token, tiles of 32 / 128 plus tails, several blocks
    lens = [1, 33, 128, 200, 7, 300]
    check(synth.make_prefill(9, D + Hq, lens, Hq, Hkv, D, 1 / math.sqrt(D), causal, "bf16", "bwd_small"))


def test_empty_sequence_in_the_packing():
    check(synth.make_prefill(9, 5, [64, 0, 100], 8, 2, 128, 0.088, True, "bf16", "bwd_empty_seq"))


@pytest.mark.parametrize("S", [1024, 2048])
def test_causal_gqa_full_heads(S):
    check(synth.config2(S=S, seed=0))


def test_causal_gqa_4096():
    # the 4096-token causal GQA geometry (G = 4, D = 128) on 8 query heads so
    # the fp64 oracle stays quick
    check(synth.make_prefill(2, 1, [4096], 8, 2, 128, 1.0 / math.sqrt(128.0), True, "bf16", "bwd_causal_s4096"))


def test_varlen_d256():
    # the head_dim-256 varlen geometry (Hq = 16, Hkv = 4, scale 2^-4): packed
    # causal sequences spanning many 64-key blocks and 32-query tiles
    check(synth.make_prefill(5, 3, [700, 1, 1500, 2300], 16, 4, 256, 2.0 ** -4, True, "bf16", "bwd_varlen_d256"))


def test_d256_repeatable_and_overestimate_bitwise():
    c = synth.make_prefill(5, 4, [300, 64, 777], 8, 2, 256, 2.0 ** -4, True, "bf16", "bwd_d256_rep")
    dout = synth.output_gradient(9, 4, c.total_tokens, c.num_q_heads, c.head_dim)
    q, k, v, cu = bf16_dev(c.q), bf16_dev(c.k), bf16_dev(c.v), i32_dev(c.cu_seqlens)
    o, lse = mi.attn_fwd(q, k, v, cu, max_len(c), scale=c.scale, causal=True)
    do = bf16_dev(dout)
    a = mi.attn_bwd(q, k, v, o, lse, do, cu, max_len(c), scale=c.scale, causal=True)
    b = mi.attn_bwd(q, k, v, o, lse, do, cu, max_len(c), scale=c.scale, causal=True)
    d = mi.attn_bwd(q, k, v, o, lse, do, cu, 2 * max_len(c) + 9, scale=c.scale, causal=True)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, d):
        assert bitwise_equal(x, y) and bitwise_equal(x, z)


def test_closed_forms_on_every_head_at_4096():
    c = synth.config2(S=4096, seed=1)
    dout = synth.output_gradient(9, 1, c.total_tokens, c.num_q_heads, c.head_dim)
    dq, dk, dv = gpu_pipeline(c, dout)
    do = f64(dout)
    G = c.num_q_heads // c.num_kv_heads
    dvh, dkh = host(dv), host(dk)
    for g in range(c.num_kv_heads):
        # sum_j dV_j = sum of the group's dO; sum_j dK_j = 0 (4096 bf16 terms)
        want = do[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        assert np.max(np.abs(dvh[:, g].sum(axis=0) - want)) < 0.5
        assert np.max(np.abs(dkh[:, g].sum(axis=0))) < 0.5


def test_repeatable_bitwise():
    c = synth.make_prefill(9, 7, [500, 77, 1000], 32, 8, 128, 0.088, True, "bf16", "bwd_rep")
    dout = synth.output_gradient(9, 7, c.total_tokens, c.num_q_heads, c.head_dim)
    a = gpu_pipeline(c, dout)
    b = gpu_pipeline(c, dout)
    for x, y in zip(a, b):
        assert bitwise_equal(x, y)


def test_max_seqlen_overestimate_gives_same_bits():
    c = synth.make_prefill(9, 8, [300, 77, 1000, 1], 8, 2, 128, 0.088, True, "bf16", "bwd_overestimate")
    dout = synth.output_gradient(9, 8, c.total_tokens, c.num_q_heads, c.head_dim)
    q, k, v, cu = bf16_dev(c.q), bf16_dev(c.k), bf16_dev(c.v), i32_dev(c.cu_seqlens)
    o, lse = mi.attn_fwd(q, k, v, cu, max_len(c), scale=c.scale, causal=True)
    do = bf16_dev(dout)
    a = mi.attn_bwd(q, k, v, o, lse, do, cu, max_len(c), scale=c.scale, causal=True)
    b = mi.attn_bwd(q, k, v, o, lse, do, cu, 3 * max_len(c) + 5, scale=c.scale, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert bitwise_equal(x, y)
