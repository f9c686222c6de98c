"""Scalar fp32/bf16 emulation of split-KV decode programs (test infrastructure).

Part of the oracle package: only tests, the smoke check and the CPU baseline
may use it. It emulates, one scalar per token, the decode programs that "Why
your local LLM feels dumber than it is" compares, so that their geometry,
rounding points and merges can be checked against the numbers the post prints
and so that the GPU library's numerics variants can be set beside them.

What a program is made of, from the post's prose:
- a partition of the context into groups ("Why the calculation is split into
  groups"; the geometries of "Backend names expand into four decode
  algorithms": 16 contiguous segments, FlashAttention 2's contiguous 64-token
  blocks walked last-to-first inside a group, round-robin 256-token tiles,
  one group per 128-token tile);
- per group, the local maximum, fp32 exponential weights relative to it, an
  fp32 normalizer summed from the unrounded weights (or from the bf16-rounded
  ones), an fp32 numerator summed from bf16 weight times bf16 value, the
  normalized partial (optionally rounded to bf16) and the fp32 log-sum-exp;
- a merge of the group records: log-sum-exp weights (FlashAttention 2),
  max-corrected fp32 numerators and normalizers (the 16-segment program),
  normalized bf16 partials weighted by their corrected normalizers (XQA), or an
  ordered running recurrence over bf16 numerators that ignores an empty
  running state (the TensorRT-LLM reducer).
Every step of a program rounds to float32 in the order written; sums are taken
strictly left to right (the post does not give the reduction trees: the
plainest reading). ``Arithmetic(exact=True)`` turns every rounding into the
identity so that each program reduces to the real-number definition: that is
what pins the merge algebra, independently of the printed outputs.

Pinned against the post: the FlashAttention 2 split table and its fp32/bf16
outputs ("Why FlashAttention 2 selects 54, 62, or 87 groups", "Plugging in
actual numbers"), the XQA group counts 33 and 47, the reduction-order example
("GPU specific lowering in Triton"), and, in exact arithmetic, the printed
exact output for all four programs. The rounding points that only the XQA and
TensorRT-LLM programs use (bf16 weights in the normalizer, bf16 partials, the
bf16 numerator at the merge) have no printed output: parity unpinned for those
rounding points.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = np.float32


# --------------------------------------------------------------- scalar helpers
def f32(x) -> float:
    """Round a real number to the nearest float32 (ties to even)."""
    return float(np.float32(x))


def _bf16_bits_round(u: np.ndarray) -> np.ndarray:
    # round-to-nearest-even on the upper 16 bits of float32 bit patterns
    return (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)


def bf16(x) -> float:
    """Round to float32 then to bfloat16, ties to even."""
    u = np.array([np.float32(x)], dtype=np.float32).view(np.uint32)
    return float(_bf16_bits_round(u).view(np.float32)[0])


def bf16_array(x) -> np.ndarray:
    """Element-wise bf16 rounding of a float32 array (returned as float32)."""
    a = np.array(x, dtype=np.float32)
    return _bf16_bits_round(a.reshape(-1).view(np.uint32)).view(np.float32).reshape(a.shape)


def add32(a, b) -> float:
    return float(F32(a) + F32(b))


def reduction_order_example():
    """(1 + 2^-24) + 2^-24 versus 1 + (2^-24 + 2^-24), each step in fp32."""
    h = 2.0 ** -24
    return add32(add32(1.0, h), h), add32(1.0, add32(h, h))


# ------------------------------------------------------------------ arithmetic
class Arithmetic:
    """Where a program rounds. Default: every step in float32, bf16 where a
    program says so. ``exact=True``: float64 everywhere and bf16 rounding the
    identity, i.e. the same program in (nearly) real arithmetic."""

    def __init__(self, exact: bool = False):
        self.exact = exact
        self.dtype = np.float64 if exact else np.float32

    def r(self, x):
        return np.asarray(x, dtype=np.float64).astype(self.dtype)

    def half(self, x):
        return self.r(x) if self.exact else bf16_array(x)

    def exp(self, x):
        # exponential of the rounded argument, computed in fp64 and rounded
        return self.r(np.exp(np.asarray(x, dtype=np.float64)))

    def log(self, x):
        return self.r(np.log(np.asarray(x, dtype=np.float64)))

    def total(self, x):
        """Left-to-right sum, every partial sum rounded."""
        x = self.r(x)
        return np.add.accumulate(x)[-1] if x.size else self.dtype(0)


# ------------------------------------------------------------------ geometries
def fa2_split_count(total_tokens: int, sm_count: int, kv_heads: int = 4, batch: int = 1,
                    block_tokens: int = 64, max_splits: int = 128, blocks_per_sm: int = 2,
                    threshold: float = 0.85):
    """The split-count rule described in "Why FlashAttention 2 selects 54, 62,
    or 87 groups". The key/value blocks (64 tokens) are dealt out in equal
    runs, so a split count only matters through the run length it gives; for
    every run length that some count up to min(max_splits, capacity, blocks)
    can give, the count in play is the smallest one giving it. Each such count
    s is scored by its estimated efficiency, the filled fraction of the last
    wave when batch*kv_heads*s work units meet a capacity of 2 work blocks per
    streaming multiprocessor; the smallest count scoring at least 85% of the
    best score is chosen (`threshold` generalizes the 85%). Scores are exact
    fractions. Returns (splits, key_value_blocks, blocks_per_split)."""
    from fractions import Fraction
    n_blocks = -(-total_tokens // block_tokens)
    capacity = blocks_per_sm * sm_count
    units = batch * kv_heads
    limit = min(max_splits, capacity, n_blocks)
    # run length -> smallest split count that produces it
    first_count = {}
    for s in range(limit, 0, -1):
        first_count[-(-n_blocks // s)] = s
    counts = sorted(first_count.values())

    def efficiency(s):
        waves = Fraction(units * s, capacity)
        return waves / math.ceil(waves)

    scores = {s: efficiency(s) for s in counts}
    best = max(scores.values())
    chosen = min(s for s in counts if scores[s] >= Fraction(threshold).limit_denominator(10 ** 6) * best)
    return chosen, n_blocks, -(-n_blocks // chosen)


def fa2_groups(total_tokens: int, splits: int, block_tokens: int = 64):
    """Contiguous groups of whole 64-token blocks, ceil(blocks/splits) each,
    every group walked from its last block back to its first."""
    n_blocks = -(-total_tokens // block_tokens)
    bps = -(-n_blocks // splits)
    groups = []
    for first in range(0, n_blocks, bps):
        blocks = range(min(first + bps, n_blocks) - 1, first - 1, -1)
        groups.append(np.concatenate([np.arange(b * block_tokens, min((b + 1) * block_tokens, total_tokens))
                                      for b in blocks]))
    return groups


def segment_groups(total_tokens: int, segments: int = 16, tile_tokens: int = 16):
    """`segments` contiguous groups, each a whole number of tiles: the first
    groups take ceil(T / (segments * tile)) tiles each, the last what is left."""
    span = -(-total_tokens // (segments * tile_tokens)) * tile_tokens
    return [np.arange(a, min(a + span, total_tokens)) for a in range(0, total_tokens, span)]


def round_robin_groups(total_tokens: int, groups: int, tile_tokens: int = 256):
    """Tiles of `tile_tokens` dealt to `groups` in turn: tile j goes to group
    j mod groups; a group visits its tiles in increasing order."""
    n_tiles = -(-total_tokens // tile_tokens)
    out = []
    for g in range(min(groups, n_tiles)):
        out.append(np.concatenate([np.arange(j * tile_tokens, min((j + 1) * tile_tokens, total_tokens))
                                   for j in range(g, n_tiles, groups)]))
    return out


def tile_groups(total_tokens: int, tile_tokens: int = 128):
    """One group per tile of `tile_tokens`."""
    return [np.arange(a, min(a + tile_tokens, total_tokens)) for a in range(0, total_tokens, tile_tokens)]


def xqa_group_count(total_tokens: int, sm_count: int, kv_heads: int = 4, batch: int = 1,
                    tile_tokens: int = 256) -> int:
    """XQA's group count: the processing units shared out over batch x kv heads,
    at least 1, at most the number of 256-token tiles."""
    return min(max(1, sm_count // (batch * kv_heads)), -(-total_tokens // tile_tokens))


# ----------------------------------------------------------- group summaries
@dataclass
class Summary:
    tokens: int
    m: float        # local maximum score
    l: float        # normalizer
    num: float      # numerator (weighted-value sum)
    out: float      # normalized partial as stored for the merge
    lse: float      # m + log(l)


def summarize(A: Arithmetic, scores: np.ndarray, values: np.ndarray, idx: np.ndarray,
              rounded_normalizer: bool = False, bf16_partial: bool = False) -> Summary:
    """One group: weights exp(score - local max) in fp32; the numerator sums
    bf16(weight) * bf16(value); the normalizer sums the fp32 weights, or the
    bf16-rounded ones when `rounded_normalizer`."""
    s = A.r(scores[idx])
    m = s.max()
    w = A.exp(A.r(s - m))
    wh = A.half(w)
    l = A.total(wh if rounded_normalizer else w)
    num = A.total(A.r(wh * A.half(A.r(values[idx]))))
    out = A.r(num / l)
    if bf16_partial:
        out = A.half(out)
    lse = A.r(m + A.log(l))
    return Summary(len(idx), float(m), float(l), float(num), float(out), float(lse))


# ----------------------------------------------------------------- merges
def merge_lse(A: Arithmetic, parts) -> float:
    """Normalized partials weighted by exp(LSE_g - max LSE)."""
    L = np.array([p.lse for p in parts])
    top = A.r(L.max())
    w = A.exp(A.r(A.r(L) - top))
    out = A.r([p.out for p in parts])
    return float(A.r(A.total(A.r(out * w)) / A.total(w)))


def merge_numerators(A: Arithmetic, parts) -> float:
    """Numerators and normalizers brought to the largest local maximum."""
    m = A.r([p.m for p in parts])
    c = A.exp(A.r(m - m.max()))
    den = A.total(A.r(A.r([p.l for p in parts]) * c))
    num = A.total(A.r(A.r([p.num for p in parts]) * c))
    return float(A.r(num / den))


def merge_normalizer_weighted(A: Arithmetic, parts) -> float:
    """Normalized partials weighted by their normalizers brought to the
    largest local maximum."""
    m = A.r([p.m for p in parts])
    c = A.exp(A.r(m - m.max()))
    wl = A.r(A.r([p.l for p in parts]) * c)
    num = A.total(A.r(A.r([p.out for p in parts]) * wl))
    return float(A.r(num / A.total(wl)))


def merge_ordered(A: Arithmetic, parts, bf16_numerator: bool = True) -> float:
    """The ordered running recurrence of the TensorRT-LLM reducer ("Backend
    names expand into four decode algorithms"): a state (max, normalizer,
    numerator) absorbs the group records one at a time in group order. To
    absorb a record, both sides are brought to the larger of the two maxima
    and added; a state that is still empty (max -inf) contributes nothing, and
    an empty record (max -inf) leaves the state as it is. The numerator of a
    record enters rounded to bf16 when `bf16_numerator`."""
    from functools import reduce

    def absorb(state, p):
        m_run, l_run, n_run = state
        if p.m == -math.inf:
            return state
        top = max(m_run, p.m)
        w_run = A.dtype(0) if m_run == -math.inf else A.exp(A.r(m_run - top))
        w_new = A.exp(A.r(p.m - top))
        num = A.half(p.num) if bf16_numerator else A.r(p.num)
        return (top,
                A.r(A.r(l_run * w_run) + A.r(A.r(p.l) * w_new)),
                A.r(A.r(n_run * w_run) + A.r(num * w_new)))

    _, l_fin, n_fin = reduce(absorb, parts, (-math.inf, A.dtype(0), A.dtype(0)))
    return float(A.r(n_fin / l_fin))


# ----------------------------------------------------------- the four programs
@dataclass
class ProgramResult:
    name: str
    groups: int
    out32: float
    out16: float
    parts: list


def run_program(name: str, scores, values, sm_count: int, exact: bool = False,
                kv_heads: int = 4, batch: int = 1) -> ProgramResult:
    """One of the four decode programs of "Backend names expand into four
    decode algorithms" on a single (query head, value channel):
    'segments16' (16 contiguous segments, fp32 split state, numerator merge),
    'fa2' (platform split count, contiguous 64-token blocks, LSE merge),
    'xqa' (round-robin 256-token tiles, bf16 weights in the normalizer, bf16
    partials, normalizer-weighted merge), 'trt' (one group per 128-token tile,
    ordered running merge over bf16 numerators)."""
    A = Arithmetic(exact)
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    T = len(scores)
    if name == "segments16":
        groups = segment_groups(T)
        parts = [summarize(A, scores, values, g) for g in groups]
        out = merge_numerators(A, parts)
    elif name == "fa2":
        groups = fa2_groups(T, fa2_split_count(T, sm_count, kv_heads, batch)[0])
        parts = [summarize(A, scores, values, g) for g in groups]
        out = merge_lse(A, parts)
    elif name == "xqa":
        groups = round_robin_groups(T, xqa_group_count(T, sm_count, kv_heads, batch))
        parts = [summarize(A, scores, values, g, rounded_normalizer=True, bf16_partial=True) for g in groups]
        out = merge_normalizer_weighted(A, parts)
    elif name == "trt":
        groups = tile_groups(T)
        parts = [summarize(A, scores, values, g) for g in groups]
        out = merge_ordered(A, parts)
    else:
        raise ValueError(name)
    return ProgramResult(name, len(groups), out, out if exact else bf16(out), parts)


def fa2_like_decode(scores, values, splits: int):
    """FlashAttention 2's program at a given split count. Returns (fp32
    output, bf16 output, first group size, first local max)."""
    A = Arithmetic()
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    parts = [summarize(A, s, v, g) for g in fa2_groups(len(s), splits)]
    out = merge_lse(A, parts)
    return out, bf16(out), parts[0].tokens, parts[0].m
