"""Scalar fp32/bf16 emulation of a split-KV decode (test infrastructure).

Used only to pin the split geometry, the log-sum-exp merge and the rounding
helpers against the numbers printed in "Why your local LLM feels dumber than it
is", sections "Why FlashAttention 2 selects 54, 62, or 87 groups" and
"Plugging in actual numbers", and the reduction-order example of "GPU specific
lowering in Triton". It is written from the pages' prose: each group finds its
local maximum, forms fp32 exponential weights, sums the unrounded fp32 weights
for the normalizer and the bf16-rounded weights times values for the numerator
(section "Why the calculation is split into groups"), stores the normalized
fp32 partial and its fp32 log-sum-exp, and the groups are merged with weights
exp(LSE_s - max LSE) (FlashAttention 2 entry of "Backend names expand into four
decode algorithms"). Inside a group, FlashAttention 2 walks its contiguous
64-token blocks from the last one back to the first.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32


def f32(x) -> float:
    """Round a real number to the nearest float32 (ties to even)."""
    return float(np.float32(x))


def bf16(x) -> float:
    """Round to float32 then to bfloat16, ties to even."""
    u = int(np.array([np.float32(x)], dtype=np.float32).view(np.uint32)[0])
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return float(np.array([u], dtype=np.uint32).view(np.float32)[0])


def add32(a, b) -> float:
    return float(F32(a) + F32(b))


def mul32(a, b) -> float:
    return float(F32(a) * F32(b))


def div32(a, b) -> float:
    return float(F32(a) / F32(b))


def exp32(x) -> float:
    """float32 of the (correctly rounded in fp64) exponential."""
    return f32(math.exp(float(x)))


def log32(x) -> float:
    return f32(math.log(float(x)))


def fa2_split_count(total_tokens: int, sm_count: int, kv_heads: int = 4, batch: int = 1,
                    block_tokens: int = 64, max_splits: int = 128, blocks_per_sm: int = 2,
                    threshold: float = 0.85):
    """The split-count rule described in "Why FlashAttention 2 selects 54, 62,
    or 87 groups": capacity = 2 work blocks per streaming multiprocessor; a
    candidate count s gives work ratio batch*kv_heads*s / capacity and
    efficiency ratio / ceil(ratio); counts that do not change the number of
    64-token blocks per split are skipped; the smallest count reaching 85% of
    the best efficiency wins (`threshold` generalizes the 85%). Returns
    (splits, key_value_blocks, blocks_per_split)."""
    n_blocks = -(-total_tokens // block_tokens)
    capacity = blocks_per_sm * sm_count
    work = batch * kv_heads
    top = min(max_splits, capacity, n_blocks)
    cands = []
    for s in range(1, top + 1):
        if s > 1 and -(-n_blocks // s) == -(-n_blocks // (s - 1)):
            continue
        ratio = work * s / capacity
        cands.append((s, ratio / math.ceil(ratio)))
    best = max(e for _, e in cands)
    s = next(c for c, e in cands if e >= threshold * best)
    return s, n_blocks, -(-n_blocks // s)


def fa2_groups(total_tokens: int, splits: int, block_tokens: int = 64):
    """Token index lists of the contiguous groups, each walked block-backward."""
    n_blocks = -(-total_tokens // block_tokens)
    bps = -(-n_blocks // splits)
    groups = []
    for s in range(splits):
        b0 = s * bps
        b1 = min(b0 + bps, n_blocks)
        toks = []
        for blk in range(b1 - 1, b0 - 1, -1):
            toks.extend(range(blk * block_tokens, min((blk + 1) * block_tokens, total_tokens)))
        if toks:
            groups.append(toks)
    return groups


def group_partial(scores, values, toks):
    """One group's (local max, fp32 normalizer, fp32 numerator, normalized
    partial, fp32 LSE) with the FlashAttention 2 rounding points."""
    m = f32(max(scores[t] for t in toks))
    l = 0.0
    acc = 0.0
    for t in toks:
        e = exp32(f32(scores[t] - m))
        l = add32(l, e)
        acc = add32(acc, mul32(bf16(e), bf16(values[t])))
    out = div32(acc, l)
    lse = f32(m + log32(l))
    return m, l, acc, out, lse


def merge_by_lse(partials):
    """Normalized partials weighted by exp(LSE_s - max LSE), in fp32."""
    M = f32(max(p[4] for p in partials))
    W = 0.0
    A = 0.0
    for p in partials:
        w = exp32(f32(p[4] - M))
        W = add32(W, w)
        A = add32(A, mul32(p[3], w))
    return div32(A, W)


def fa2_like_decode(scores, values, splits: int):
    """Returns (fp32 output, bf16 output, first group size, first local max)."""
    groups = fa2_groups(len(scores), splits)
    parts = [group_partial(scores, values, g) for g in groups]
    out = merge_by_lse(parts)
    return out, bf16(out), len(groups[0]), parts[0][0]


def reduction_order_example():
    """(1 + 2^-24) + 2^-24 versus 1 + (2^-24 + 2^-24), each step in fp32."""
    h = 2.0 ** -24
    return add32(add32(1.0, h), h), add32(1.0, add32(h, h))
