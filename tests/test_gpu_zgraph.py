"""The entry points under HIP graph capture: a stream's library-owned state
(the fp16 copy of V and the work queues of the head_dim-256 prefill, the
decode workspace) is created by eager calls on that stream first; the graph
then replays the same kernels on it. Every replay, with eager calls on the
same stream and synchronisations between replays, must give the bits of the
eager calls."""
import math

import pytest
import torch

import attention_attn_fwd_03_amd as mi
import synth
from gpu_util import bf16_dev, bitwise_equal, i32_dev

pytestmark = pytest.mark.gpu


def prefill_inputs(case):
    return (bf16_dev(case.q), bf16_dev(case.k), bf16_dev(case.v), i32_dev(case.cu_seqlens))


def decode_inputs(case):
    return (bf16_dev(case.q), bf16_dev(case.k_cache), bf16_dev(case.v_cache), i32_dev(case.block_table),
            i32_dev(case.seq_lens))


def test_graph_replays_match_eager_calls():
    p128 = synth.config2(S=4096, seed=3)                       # eight-wave prefill
    p256 = synth.make_prefill(41, 0, [700, 1, 1900, 0, 333], 16, 4, 256, 2.0 ** -4, True, "bf16", "graph_d256")
    dec = synth.make_decode(41, 1, [4000, 17, 2500, 1024, 3333, 1], 32, 8, 128, 1 / math.sqrt(128),
                            shuffle=True, tail="zero", name="graph_decode")
    other = synth.make_prefill(41, 2, [1200, 64], 16, 4, 256, 2.0 ** -4, True, "bf16", "graph_other")
    a128, a256, ad, ao = prefill_inputs(p128), prefill_inputs(p256), decode_inputs(dec), prefill_inputs(other)
    torch.cuda.synchronize()

    def calls():
        r = []
        r += mi.attn_fwd(*a128, p128.max_seqlen, scale=p128.scale, causal=True)
        r += mi.attn_fwd(*a256, p256.max_seqlen, scale=p256.scale, causal=True)
        r += mi.attn_decode_paged(*ad, scale=dec.scale, num_splits=0)
        r += mi.attn_decode_paged(*ad, scale=dec.scale, num_splits=5)
        r += mi.attn_decode_paged_noalloc(*ad, scale=dec.scale, num_splits=0)
        return r

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = calls()            # also creates the stream's library-owned state
        other_ref = mi.attn_fwd(*ao, other.max_seqlen, scale=other.scale, causal=True)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        captured = calls()
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(captured, eager)):
            assert bitwise_equal(x, y), f"replay {rep}, output {i}"
        # eager work on the same stream between replays: it shares the fp16
        # V copy, the work queues and the decode workspace with the graph
        with torch.cuda.stream(s):
            o2 = mi.attn_fwd(*ao, other.max_seqlen, scale=other.scale, causal=True)
        s.synchronize()
        assert bitwise_equal(o2[0], other_ref[0]) and bitwise_equal(o2[1], other_ref[1])
