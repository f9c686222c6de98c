"""Chunked prefill against a paged cache: the HIP kernel against the fp64
oracle (bf16: max-abs 1e-2, mean-abs 1e-3; LSE: 1e-3), plus the properties
that tie it to the contiguous prefill."""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as mi
import oracle
import synth
from gpu_util import assert_bf16_close, assert_lse_close, bf16_dev, bitwise_equal, host, i32_dev

pytestmark = pytest.mark.gpu


def run(c, causal=True):
    o, l = mi.attn_fwd_paged(bf16_dev(c.q), bf16_dev(c.k_cache), bf16_dev(c.v_cache), i32_dev(c.block_table),
                             i32_dev(c.cu_seqlens_q), i32_dev(c.seq_lens_k), c.max_seqlen_q, scale=c.scale,
                             causal=causal)
    torch.cuda.synchronize()
    return o, l


def reference(c, causal=True):
    return oracle.prefill_paged_dense(synth.bf16_to_f64(c.q), synth.bf16_to_f64(c.k_cache),
                                      synth.bf16_to_f64(c.v_cache), c.block_table, c.cu_seqlens_q, c.seq_lens_k,
                                      c.num_q_heads, c.num_kv_heads, c.scale, causal)


def check(c, causal=True):
    print(f"[prefill-paged] q_lens={c.q_lens[:8]} k_lens={c.seq_lens_k.tolist()[:8]} Hq={c.num_q_heads} "
          f"Hkv={c.num_kv_heads} D={c.head_dim} causal={causal}", flush=True)
    o, l = run(c, causal)
    O, L = reference(c, causal)
    assert_bf16_close(host(o), O, c.name)
    assert_lse_close(host(l), L, c.name)
    return o, l


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 8), (256, 16, 4), (128, 8, 4), (128, 16, 2),
                                      (128, 24, 8), (64, 12, 2)])   # G = 3 and 6 as well
def test_chunks_against_oracle(D, Hq, Hkv, causal):
    # prefixes crossing the 64-page block-table window, a chunk longer than a
    # prefix, ragged chunk and cache ends, a one-token chunk
    q_lens = [200, 97, 1, 64, 130]
    k_lens = [1200 + 200, 97 + 33, 1 + 2100, 64, 130 + 511]
    c = synth.make_chunked_prefill(6, D + Hq, q_lens, k_lens, Hq, Hkv, D, D ** -0.5, shuffle=True, tail="nan")
    o, _ = check(c, causal)
    assert not torch.isnan(o.float()).any()


def test_config6_shape_against_oracle():
    # the chunked-prefill workload's sequence geometry (chunks of 1024 after
    # prefixes up to 6144) with 8 query heads so the oracle stays quick
    pre = synth.varlen_lengths(6, 0, 3, 0, 6144)
    c = synth.make_chunked_prefill(6, 0, [1024] * 3, [p + 1024 for p in pre], 8, 2, 128, 128 ** -0.5,
                                   shuffle=True, tail="nan")
    check(c, True)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 4, 64), (4, 4, 128)])
def test_whole_sequence_chunk_equals_contiguous_prefill_bitwise(Hq, Hkv, D):
    # Lq == Lk with pages in order: the paged kernel and the dense one (a
    # different kernel at D <= 128) visit the same tiles with the same
    # accumulation orders and softmax rule, so the bits agree
    lens = [700, 33, 256]
    p = synth.make_prefill(2, 3, lens, Hq, Hkv, D, D ** -0.5, True, "bf16")
    T = sum(lens)
    k = p.k.reshape(T, Hkv, D)
    v = p.v.reshape(T, Hkv, D)
    total = sum((L + 15) // 16 for L in lens)
    kc = np.zeros((total, 16, Hkv, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    bt = np.full((len(lens), max((L + 15) // 16 for L in lens)), -1, dtype=np.int32)
    page, off = 0, 0
    for b, L in enumerate(lens):
        for j in range((L + 15) // 16):
            n = min(16, L - 16 * j)
            kc[page, :n] = k[off + 16 * j: off + 16 * j + n]
            vc[page, :n] = v[off + 16 * j: off + 16 * j + n]
            bt[b, j] = page
            page += 1
        off += L
    for causal in (True, False):
        o1, l1 = mi.attn_fwd(bf16_dev(p.q), bf16_dev(p.k), bf16_dev(p.v), i32_dev(p.cu_seqlens), p.max_seqlen,
                             scale=p.scale, causal=causal)
        o2, l2 = mi.attn_fwd_paged(bf16_dev(p.q), bf16_dev(kc), bf16_dev(vc), i32_dev(bt), i32_dev(p.cu_seqlens),
                                   i32_dev(np.asarray(lens, dtype=np.int32)), p.max_seqlen, scale=p.scale,
                                   causal=causal)
        torch.cuda.synchronize()
        assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)


def test_queries_before_any_key_are_empty():
    # 40 queries, 10 cached keys: causal rows 0..29 see nothing
    c = synth.make_chunked_prefill(6, 9, [40], [10], 8, 2, 128, 0.09, shuffle=False, tail="nan")
    o, l = check(c, True)
    oh, lh = host(o), host(l)
    assert np.all(oh[:30] == 0) and np.all(np.isneginf(lh[:, :30]))
    assert np.all(np.isfinite(lh[:, 30:]))


def test_repeatable_bitwise():
    c = synth.make_chunked_prefill(6, 4, [300, 77], [1000, 77], 32, 8, 128, 0.088, shuffle=True, tail="zero")
    o1, l1 = run(c)
    o2, l2 = run(c)
    assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)


def test_max_seqlen_overestimate_gives_same_bits():
    c = synth.make_chunked_prefill(6, 5, [200, 1, 64], [900, 1, 64], 8, 2, 128, 0.088, shuffle=True, tail="zero")
    args = (bf16_dev(c.q), bf16_dev(c.k_cache), bf16_dev(c.v_cache), i32_dev(c.block_table),
            i32_dev(c.cu_seqlens_q), i32_dev(c.seq_lens_k))
    o1, l1 = mi.attn_fwd_paged(*args, c.max_seqlen_q, scale=c.scale, causal=True)
    o2, l2 = mi.attn_fwd_paged(*args, 4 * c.max_seqlen_q + 3, scale=c.scale, causal=True)
    torch.cuda.synchronize()
    assert bitwise_equal(o1, o2) and bitwise_equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128])
def test_rising_scores_take_every_softmax_path(D):
    # channel 0 (q = 1, k = r_p) adds scale * r_p to the score of cached key
    # p, rising ~0.1 (kv head 0) and ~0.6 (head 1) log2 units per key: tiles
    # kept, rescaled, and above the tile-sum bound without a rescale; head 1
    # rises by ~600 log2 units over 1000 keys (fp32 overflow without every
    # rescale)
    c = synth.make_chunked_prefill(6, 40 + D, [300, 64], [1000, 700], 4, 2, D, D ** -0.5, shuffle=True,
                                   tail="zero")
    cl = c.scale * math.log2(math.e)
    for b, L in enumerate(c.seq_lens_k.tolist()):
        pos = np.arange(L)
        pages, slots = c.block_table[b, pos // 16], pos % 16
        for h, slope in enumerate((0.1, 0.6)):
            c.k_cache[pages, slots, h, 0] = synth.bf16_bits((slope / cl * pos).astype(np.float32))
    c.q[:, :, 0] = synth.bf16_bits(np.float32(1.0))
    # peaky attention copies single V rows: V / 4 (exact) keeps |O| below 1
    c.v_cache[:] = synth.bf16_bits((synth.bf16_to_f64(c.v_cache) / 4).astype(np.float32))
    o, l = check(c, True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
