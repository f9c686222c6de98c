"""Algorithmic work of one call, used for throughput and roofline figures.

Only the work the method must do is counted: query/key pairs a query may see
(causal: j <= i), 4*D flops per pair (a multiply-add for q.k and one for p.v),
and each byte of Q, K, V that a call must read plus the O and LSE it writes,
once ("GPU Datapath: Where Every Byte Moves", sections C and D, count the
theoretical minimum the same way: Q+K+V+O for prefill, every cached K/V byte
plus Q and O for decode). Padding, masked halves of diagonal tiles,
partial-page tails and split partials are not credited.
"""
from __future__ import annotations


def prefill_flops(seqlens, num_q_heads: int, head_dim: int, causal: bool) -> float:
    pairs = 0
    for L in seqlens:
        L = int(L)
        pairs += L * (L + 1) // 2 if causal else L * L
    return 4.0 * head_dim * num_q_heads * pairs


def prefill_bytes(total_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  elem_bytes: int = 2, with_lse: bool = True) -> float:
    qo = 2 * total_tokens * num_q_heads * head_dim * elem_bytes
    kv = 2 * total_tokens * num_kv_heads * head_dim * elem_bytes
    lse = total_tokens * num_q_heads * 4 if with_lse else 0
    return float(qo + kv + lse)


def decode_bytes(seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2,
                 with_lse: bool = True, with_block_table: bool = True, page_size: int = 16) -> float:
    toks = sum(int(x) for x in seq_lens)
    B = len(seq_lens)
    kv = 2 * toks * num_kv_heads * head_dim * elem_bytes
    qo = 2 * B * num_q_heads * head_dim * elem_bytes
    lse = B * num_q_heads * 4 if with_lse else 0
    bt = sum((int(x) + page_size - 1) // page_size for x in seq_lens) * 4 if with_block_table else 0
    return float(kv + qo + lse + bt)


def decode_flops(seq_lens, num_q_heads: int, head_dim: int) -> float:
    return 4.0 * head_dim * num_q_heads * sum(int(x) for x in seq_lens)


def chunked_prefill_flops(q_lens, k_lens, num_q_heads: int, head_dim: int, causal: bool) -> float:
    """A chunk of Lq queries against Lk cached keys, queries aligned to the end
    of the sequence: causal query i sees min(Lk, max(0, i + Lk - Lq + 1)) keys."""
    pairs = 0
    for Lq, Lk in zip(q_lens, k_lens):
        Lq, Lk = int(Lq), int(Lk)
        if not causal:
            pairs += Lq * Lk
            continue
        off = Lk - Lq
        for i in range(Lq):
            pairs += min(Lk, max(0, i + off + 1))
    return 4.0 * head_dim * num_q_heads * pairs


def chunked_prefill_bytes(q_lens, k_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          elem_bytes: int = 2, with_lse: bool = True, page_size: int = 16) -> float:
    """Q and O of the chunk, every cached K/V byte once, LSE, block-table entries."""
    tq = sum(int(x) for x in q_lens)
    tk = sum(int(x) for x in k_lens)
    qo = 2 * tq * num_q_heads * head_dim * elem_bytes
    kv = 2 * tk * num_kv_heads * head_dim * elem_bytes
    lse = tq * num_q_heads * 4 if with_lse else 0
    bt = sum((int(x) + page_size - 1) // page_size for x in k_lens) * 4
    return float(qo + kv + lse + bt)


def backward_flops(seqlens, num_q_heads: int, head_dim: int, causal: bool) -> float:
    """Backward by recomputation: five products per admissible pair (S = Q K^T,
    dP = dO V^T, dV += P^T dO, dK += dS^T Q, dQ += dS K), 2 D flops each, i.e.
    2.5 times the forward's count. Recomputing S and dP a second time for dQ
    (as a deterministic implementation without atomics may) is not credited."""
    return 2.5 * prefill_flops(seqlens, num_q_heads, head_dim, causal)


def backward_bytes(total_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   elem_bytes: int = 2) -> float:
    """Bytes the backward must move once: Q, O, dO read and dQ written per
    query head; K, V read and dK, dV written per kv head; the LSE read."""
    q_side = 4 * total_tokens * num_q_heads * head_dim * elem_bytes
    kv_side = 4 * total_tokens * num_kv_heads * head_dim * elem_bytes
    return float(q_side + kv_side + total_tokens * num_q_heads * 4)
