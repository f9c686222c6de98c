"""fp64 CPU reference for tiled attention with an online softmax (test infrastructure).

This package is the oracle that the GPU library is checked against. It is test
infrastructure, not part of the product: only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it. It
shares no code with the HIP library or its Python binding and imports neither.

What it computes is the plain definition of attention given in "Why your local
LLM feels dumber than it is" (section "What attention is trying to calculate"):
score = scale * dot(query, key), weight = exp(score), normalized over the keys a
query may see, output = weighted sum of values. The tiled, online-softmax GPU
method ("Streaming process", steps 3-8 and its code snippet) reaches the same
result up to rounding order, so the oracle is that definition written out, in
float64, on the exact upcasts of the bits the GPU receives.

Forms:
- ``attention_dense`` / ``decode_dense``: materialized scores per (sequence,
  head), the naive form of "GPU Datapath", section C, harmless on a CPU.
- ``prefill_paged_dense``: the same materialized form for a chunk of query
  rows against a paged cache holding the whole sequence (queries aligned to
  the end of the sequence for causal masking).
- ``attention_bwd_dense``: the gradients of the same definition (dQ, dK, dV of
  sum(dO * O)), with scores recomputed in fp64, for the backward pass;
  ``attention_bwd_given``: the same products as a function of the forward's
  stored output and log-sum-exp, as a recomputing backward receives them.
- ``attention_brute`` / ``decode_brute``: pure-Python loops with ``math.fsum``
  for tiny inputs and the worked example.
- ``decode_split_partials`` + ``combine_partials``: the split-into-groups form
  of "Why the calculation is split into groups" with the log-sum-exp merge of
  the FlashAttention 2 style described under "Backend names expand into four
  decode algorithms"; also the combine oracle for arbitrary partials.
- ``emulate``: fp32/bf16 scalar emulation of the four decode programs of "Why
  your local LLM feels dumber than it is" (their geometries, rounding points and
  merges), pinned against the numbers printed under "Plugging in actual
  numbers" and, in exact arithmetic, against the printed exact output.

Every function is pinned by ``tests/test_oracle_*.py`` against values printed
on the pages (``tests/golden/``), closed forms, special cases, brute force and
invariances. Readings of points the pages leave open are listed in the
project's design notes.
"""
from .reference import (  # noqa: F401
    attention_dense,
    attention_brute,
    attention_bwd_dense,
    attention_bwd_given,
    attention_rows,
    decode_dense,
    decode_brute,
    prefill_paged_dense,
    gather_sequence_kv,
    page_split_ranges,
    decode_split_partials,
    combine_partials,
)
from . import emulate  # noqa: F401
