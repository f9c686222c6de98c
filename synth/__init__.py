"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no attention arithmetic: it draws numbers, rounds them to the
storage format the kernels read (bf16 bits, or fp32), lays them out in the
documented buffer layouts and builds the integer structure (sequence lengths,
cu_seqlens, shuffled page tables). Both the fp64 reference and the GPU path
consume exactly these arrays, so they see the same bits.

Workload shapes follow the pages' measured cells:
- "GPU Datapath: Where Every Byte Moves", section C (FlashAttention prefill,
  causal, GQA 32:8, s in {1024, 2048, 4096}) and section D (paged decode, batch
  64, 16-token pages, shuffled block table);
- "Why your local LLM feels dumber than it is", sections "What attention is
  trying to calculate" (head width 256, scale 2^-4) and "Why FlashAttention 2
  selects 54, 62, or 87 groups" (four key/value heads, long contexts).

RNG recipe: values come from ``numpy.random.default_rng([cfg, seed, 0])``
drawn as float32 standard normals in the order Q, K, V; structure (lengths,
permutations, outlier channels) from ``default_rng([cfg, seed, 1])``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16. NaN stays a quiet NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, (u >> 16).astype(np.uint32) | 0x40, r)
    return (r & 0xFFFF).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


# --------------------------------------------------------------------------
# prefill inputs  (q [T,Hq,D], k/v [T,Hkv,D], cu_seqlens int32 [n+1])
# --------------------------------------------------------------------------
@dataclass
class PrefillCase:
    name: str
    q: np.ndarray            # uint16 bf16 bits, or float32
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: np.ndarray   # int32 [num_seqs + 1]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float             # float32 value handed to the kernel
    causal: bool
    dtype: str               # "bf16" or "fp32"

    @property
    def seqlens(self):
        return np.diff(self.cu_seqlens).astype(np.int64)

    @property
    def total_tokens(self):
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self):
        s = self.seqlens
        return int(s.max()) if len(s) else 0

    def as_f64(self):
        f = bf16_to_f64 if self.dtype == "bf16" else f32_to_f64
        return f(self.q), f(self.k), f(self.v)


def make_prefill(cfg: int, seed: int, seqlens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, scale: float, causal: bool, dtype: str = "bf16",
                 name: str = "") -> PrefillCase:
    seqlens = [int(s) for s in seqlens]
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens, dtype=np.int64).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng([cfg, seed, 0])
    q = _normal(rng, (T, num_q_heads, head_dim))
    k = _normal(rng, (T, num_kv_heads, head_dim))
    v = _normal(rng, (T, num_kv_heads, head_dim))
    if dtype == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return PrefillCase(name or f"cfg{cfg}", q, k, v, cu, num_q_heads, num_kv_heads,
                       head_dim, float(np.float32(scale)), causal, dtype)


def output_gradient(cfg: int, seed: int, total_tokens: int, num_q_heads: int, head_dim: int) -> np.ndarray:
    """Upstream gradient dO [T, Hq, D] for a backward pass over a prefill case:
    standard normals from its own stream default_rng([cfg, seed, 2]) (so the
    case's Q/K/V draws are unchanged), rounded to bf16 bits."""
    rng = np.random.default_rng([cfg, seed, 2])
    return bf16_bits(_normal(rng, (total_tokens, num_q_heads, head_dim)))


def config1(seed: int = 0, S: int = 256, D: int = 64) -> PrefillCase:
    """Single-head dense fp32 attention, Sq=Sk=256, D=64, non-causal, scale 1/8."""
    return make_prefill(1, seed, [S], 1, 1, D, 0.125, False, "fp32", f"dense_fp32_s{S}_d{D}")


def config2(S: int = 4096, seed: int = 0) -> PrefillCase:
    """Causal GQA prefill, Hq=32, Hkv=8, D=128, one sequence of S tokens."""
    return make_prefill(2, seed, [S], 32, 8, 128, 1.0 / math.sqrt(128.0), True, "bf16",
                        f"causal_gqa32x8_d128_s{S}")


def varlen_lengths(cfg: int, seed: int, n: int, lo: int, hi: int):
    rng = np.random.default_rng([cfg, seed, 1])
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def config5(seed: int = 0, n: int = 8, lo: int = 256, hi: int = 8192) -> PrefillCase:
    """Varlen packed causal prefill: n lengths uniform in [lo,hi], Hq=16, Hkv=4, D=256."""
    lens = varlen_lengths(5, seed, n, lo, hi)
    return make_prefill(5, seed, lens, 16, 4, 256, 2.0 ** -4, True, "bf16",
                        f"varlen_causal_{n}seq_d256")


# --------------------------------------------------------------------------
# paged decode inputs
#   q [B,Hq,D]; k_cache/v_cache [num_pages, 16, Hkv, D]; block_table int32
#   [B, max_pages]; seq_lens int32 [B]
# --------------------------------------------------------------------------
@dataclass
class DecodeCase:
    name: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    page_size: int = PAGE_SIZE
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.q.shape[0])

    @property
    def max_pages(self):
        return int(self.block_table.shape[1])

    @property
    def num_pages(self):
        return int(self.k_cache.shape[0])

    def as_f64(self):
        return bf16_to_f64(self.q), bf16_to_f64(self.k_cache), bf16_to_f64(self.v_cache)


def _fill_pages(k_tok, v_tok, ctx_lens, phys, total_pages: int, tail: str):
    """Scatter each sequence's token rows (concatenated in k_tok / v_tok) into
    16-token physical pages in the order given by ``phys``; returns the caches
    and the block table (-1 past each sequence's last page)."""
    P = PAGE_SIZE
    B = len(ctx_lens)
    Hkv, D = k_tok.shape[1], k_tok.shape[2]
    pages_per = [(c + P - 1) // P for c in ctx_lens]
    max_pages = max(pages_per) if B else 0
    fill = np.float32(np.nan) if tail == "nan" else np.float32(0.0)
    kc = np.full((total_pages, P, Hkv, D), fill, dtype=np.float32)
    vc = np.full((total_pages, P, Hkv, D), fill, dtype=np.float32)
    bt = np.full((B, max(max_pages, 1)), -1, dtype=np.int32)
    nxt = 0
    off = 0
    for b, c in enumerate(ctx_lens):
        for p in range(pages_per[b]):
            pp = int(phys[nxt])
            nxt += 1
            bt[b, p] = pp
            lo = p * P
            hi = min(c, lo + P)
            kc[pp, : hi - lo] = k_tok[off + lo: off + hi]
            vc[pp, : hi - lo] = v_tok[off + lo: off + hi]
        off += c
    return kc, vc, bt


def make_decode(cfg: int, seed: int, ctx_lens, num_q_heads: int, num_kv_heads: int,
                head_dim: int, scale: float, shuffle: bool = True, tail: str = "nan",
                outlier_channels: int = 0, outlier_factor: float = 8.0,
                extra_pages: int = 0, name: str = "") -> DecodeCase:
    """Build a paged KV cache holding each sequence's keys/values.

    Token t of sequence b lives in logical page t // 16, slot t % 16; the block
    table maps logical pages to physical pages. With ``shuffle`` the physical
    pages are a seeded random permutation; otherwise they are laid out in
    order (the identity table of a contiguous [T,Hkv,D] cache). Slots past
    ``seq_len`` in a sequence's last page hold ``tail`` ("nan" or "zero"), which
    no correct kernel may let into a result. ``block_table`` entries past a
    sequence's last page are -1.
    """
    ctx_lens = [int(c) for c in ctx_lens]
    B = len(ctx_lens)
    P = PAGE_SIZE
    pages_per = [(c + P - 1) // P for c in ctx_lens]
    total_pages = sum(pages_per) + extra_pages
    max_pages = max(pages_per) if B else 0
    srng = np.random.default_rng([cfg, seed, 1])
    out_ch = None
    if outlier_channels:
        out_ch = np.sort(srng.choice(head_dim, size=outlier_channels, replace=False))
    phys = srng.permutation(total_pages) if shuffle else np.arange(total_pages)
    vrng = np.random.default_rng([cfg, seed, 0])
    q = _normal(vrng, (B, num_q_heads, head_dim))
    T = sum(ctx_lens)
    k_tok = _normal(vrng, (T, num_kv_heads, head_dim))
    v_tok = _normal(vrng, (T, num_kv_heads, head_dim))
    if out_ch is not None:
        k_tok[:, :, out_ch] *= np.float32(outlier_factor)
    kc, vc, bt = _fill_pages(k_tok, v_tok, ctx_lens, phys, total_pages, tail)
    return DecodeCase(name or f"cfg{cfg}", bf16_bits(q), bf16_bits(kc), bf16_bits(vc), bt,
                      np.asarray(ctx_lens, dtype=np.int32), num_q_heads, num_kv_heads,
                      head_dim, float(np.float32(scale)), P,
                      {"outlier_channels": None if out_ch is None else out_ch.tolist(),
                       "shuffled": shuffle, "tail": tail})


@dataclass
class ChunkedCase:
    """Chunked prefill: query chunks packed by cu_seqlens_q against a paged
    cache holding every sequence's seq_lens_k tokens (the chunk's own last)."""
    name: str
    q: np.ndarray                # [Tq, Hq, D] bf16 bits
    k_cache: np.ndarray          # [pages, 16, Hkv, D] bf16 bits
    v_cache: np.ndarray
    block_table: np.ndarray      # [n, max_pages] int32
    cu_seqlens_q: np.ndarray     # [n + 1] int32
    seq_lens_k: np.ndarray       # [n] int32
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def q_lens(self):
        return [int(x) for x in np.diff(self.cu_seqlens_q)]

    @property
    def total_q(self):
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self):
        return max(self.q_lens) if len(self.q_lens) else 0


def make_chunked_prefill(cfg: int, seed: int, q_lens, k_lens, num_q_heads: int, num_kv_heads: int,
                         head_dim: int, scale: float, shuffle: bool = True, tail: str = "nan",
                         name: str = "") -> ChunkedCase:
    """Query chunk b has q_lens[b] rows; sequence b caches k_lens[b] tokens in
    16-token pages (seeded permutation with ``shuffle``). Values are drawn in
    the order Q (all chunks), K, V (all cached tokens) from the value stream;
    the page permutation from the structure stream. The generator does not
    tie a chunk's queries to its cached keys: the cache is an arbitrary one."""
    q_lens = [int(x) for x in q_lens]
    k_lens = [int(x) for x in k_lens]
    P = PAGE_SIZE
    total_pages = sum((c + P - 1) // P for c in k_lens)
    srng = np.random.default_rng([cfg, seed, 1])
    phys = srng.permutation(total_pages) if shuffle else np.arange(total_pages)
    vrng = np.random.default_rng([cfg, seed, 0])
    q = _normal(vrng, (sum(q_lens), num_q_heads, head_dim))
    k_tok = _normal(vrng, (sum(k_lens), num_kv_heads, head_dim))
    v_tok = _normal(vrng, (sum(k_lens), num_kv_heads, head_dim))
    kc, vc, bt = _fill_pages(k_tok, v_tok, k_lens, phys, total_pages, tail)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return ChunkedCase(name or f"cfg{cfg}", bf16_bits(q), bf16_bits(kc), bf16_bits(vc), bt, cu,
                       np.asarray(k_lens, dtype=np.int32), num_q_heads, num_kv_heads, head_dim,
                       float(np.float32(scale)), {"shuffled": shuffle, "tail": tail})


def config6(seed: int = 0, n: int = 8, chunk: int = 1024, lo: int = 0, hi: int = 6144,
            tail: str = "nan") -> ChunkedCase:
    """Chunked prefill: n sequences, each a chunk of `chunk` new tokens after a
    cached prefix uniform in [lo, hi] tokens; Hq=32, Hkv=8, D=128 (the causal
    GQA prefill shape), shuffled 16-token pages."""
    prefix = varlen_lengths(6, seed, n, lo, hi)
    return make_chunked_prefill(6, seed, [chunk] * n, [p + chunk for p in prefix], 32, 8, 128,
                                1.0 / math.sqrt(128.0), shuffle=True, tail=tail,
                                name=f"chunked_prefill_n{n}_chunk{chunk}_prefix{lo}-{hi}")


def config3(seed: int = 0, B: int = 64, lo: int = 512, hi: int = 4096, tail: str = "nan") -> DecodeCase:
    """Paged decode: B sequences, contexts uniform in [lo,hi], Hq=32, Hkv=8, D=128, shuffled pages."""
    lens = varlen_lengths(3, seed, B, lo, hi)
    return make_decode(3, seed, lens, 32, 8, 128, 1.0 / math.sqrt(128.0), shuffle=True,
                       tail=tail, name=f"paged_decode_b{B}_ctx{lo}-{hi}")


def config4(ctx: int = 131072, seed: int = 0) -> DecodeCase:
    """Long-context decode: B=1, Hq=16, Hkv=4, D=256, scale 2^-4, four K channels x8, identity pages."""
    return make_decode(4, seed, [ctx], 16, 4, 256, 2.0 ** -4, shuffle=False, tail="zero",
                       outlier_channels=4, name=f"long_decode_d256_ctx{ctx}")


# --------------------------------------------------------------------------
# the 27,525-token teaching input of "Why your local LLM feels dumber than it
# is" (section "Plugging in actual numbers"): a 12-periodic list of scores and
# values plus an offset of 0.125 times (64-token block index mod 9) on scores.
# Every score and value is a short binary fraction, exact in bf16.
# --------------------------------------------------------------------------
_WE_SCORES = (0.5, 1.0, 0.75, -2.0, -1.25, -0.75, -0.5, -3.0, -0.25, -2.25, 0.75, 0.5)
_WE_VALUES = (1.875, 3.5, -0.5, 6.0, 0.0, -1.0, 5.5, -0.5, -3.5, 0.5, 4.0, -2.5)
WORKED_EXAMPLE_TOKENS = 27525


def worked_example_scores_values(n: int = WORKED_EXAMPLE_TOKENS):
    t = np.arange(n)
    base = np.asarray(_WE_SCORES, dtype=np.float64)[t % 12]
    off = ((t // 64) % 9) * 0.125
    scores = base + off
    values = np.asarray(_WE_VALUES, dtype=np.float64)[t % 12]
    return scores, values


def worked_example_decode(head_dim: int = 64, num_q_heads: int = 1, num_kv_heads: int = 1,
                          shuffle: bool = False) -> DecodeCase:
    """The teaching input as a real decode problem: q = e0, k_t = score_t * e0,
    v_t = value_t * e0, scale 1, so every score and every value reaches the
    kernel exactly (all are bf16-representable)."""
    s, vals = worked_example_scores_values()
    n = len(s)
    q = np.zeros((1, num_q_heads, head_dim), dtype=np.float32)
    q[:, :, 0] = 1.0
    P = PAGE_SIZE
    pages = (n + P - 1) // P
    k_tok = np.zeros((n, num_kv_heads, head_dim), dtype=np.float32)
    v_tok = np.zeros((n, num_kv_heads, head_dim), dtype=np.float32)
    k_tok[:, :, 0] = s[:, None]
    v_tok[:, :, 0] = vals[:, None]
    kc = np.zeros((pages * P, num_kv_heads, head_dim), dtype=np.float32)
    vc = np.zeros_like(kc)
    kc[:n] = k_tok
    vc[:n] = v_tok
    kc[n:] = np.nan
    vc[n:] = np.nan
    kc = kc.reshape(pages, P, num_kv_heads, head_dim)
    vc = vc.reshape(pages, P, num_kv_heads, head_dim)
    order = np.arange(pages)
    if shuffle:
        order = np.random.default_rng([99, 0, 1]).permutation(pages)
    kcs = np.empty_like(kc)
    vcs = np.empty_like(vc)
    kcs[order] = kc
    vcs[order] = vc
    bt = order.astype(np.int32)[None, :]
    return DecodeCase("worked_example_27525", bf16_bits(q), bf16_bits(kcs), bf16_bits(vcs), bt,
                      np.asarray([n], dtype=np.int32), num_q_heads, num_kv_heads, head_dim,
                      1.0, P, {"shuffled": shuffle})


def random_partials(seed: int, rows: int, num_splits: int, head_dim: int, empty_frac: float = 0.2):
    """Arbitrary split partials for the combine step: fp32 normalized outputs
    [rows, S, D] and fp32 log-sum-exps [rows, S]; a fraction of splits is empty
    (LSE = -inf, output 0), and some rows are entirely empty."""
    rng = np.random.default_rng([77, seed, 0])
    po = rng.standard_normal((rows, num_splits, head_dim), dtype=np.float32)
    plse = (rng.standard_normal((rows, num_splits), dtype=np.float32) * np.float32(4.0)
            + np.float32(3.0)).astype(np.float32)
    srng = np.random.default_rng([77, seed, 1])
    empty = srng.random((rows, num_splits)) < empty_frac
    if rows >= 3:
        empty[srng.integers(0, rows)] = True
    plse[empty] = -np.inf
    po[empty] = 0.0
    return po, plse
