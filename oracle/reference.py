"""fp64 attention reference (test infrastructure; see the package docstring).

Notation (from "Why your local LLM feels dumber than it is", section "What
attention is trying to calculate", and the FlashAttention loop of "Streaming
process", code snippet): for query row i of head h and admissible keys J(i),
    s_ij = scale * sum_d q[i,h,d] * k[j,g,d]
    m_i  = max_{j in J(i)} s_ij
    w_ij = exp(s_ij - m_i)
    l_i  = sum_{j in J(i)} w_ij
    O[i,h,:] = sum_j w_ij * v[j,g,:] / l_i
    LSE[i,h] = m_i + ln l_i            (natural log, scaled-score units)
Subtracting m_i changes nothing in exact arithmetic (section "Why the
calculation is split into groups"); it only keeps exp finite.
Readings where the pages are silent:
- GQA: query head h uses key/value head g = h // (Hq / Hkv) (contiguous groups).
- causal: key j is admissible for query i when j <= i, positions counted from
  the start of each sequence (Sq = Sk per sequence).
- decode: the one query token sees every cached token, seq_lens[b] of them.
- chunked prefill (a query chunk of Lq tokens against a cache of Lk >= Lq
  tokens that already holds the chunk's own keys): the chunk is the last Lq
  positions of the sequence, so with causal masking query i sees keys
  j <= i + (Lk - Lq) ("bottom-right" alignment); without it, all Lk keys.
- an empty key set gives O = 0 and LSE = -inf.
Inputs are float64 arrays (exact upcasts of bf16/fp32 storage).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def _softmax_rows(S: np.ndarray, V: np.ndarray):
    """Return (O, LSE) for score rows S [n, L] (with -inf for inadmissible
    keys) against values V [L, D]. Rows with no admissible key give (0, -inf)."""
    n = S.shape[0]
    D = V.shape[1]
    O = np.zeros((n, D), dtype=np.float64)
    lse = np.full(n, NEG_INF, dtype=np.float64)
    if n == 0 or S.shape[1] == 0:
        return O, lse
    m = S.max(axis=1)
    ok = np.isfinite(m)
    if not ok.any():
        return O, lse
    Sm = S[ok]
    mm = m[ok]
    W = np.exp(Sm - mm[:, None])          # exp(-inf) = 0 for masked keys
    l = W.sum(axis=1)
    O[ok] = (W @ V) / l[:, None]
    lse[ok] = mm + np.log(l)
    return O, lse


def attention_dense(q, k, v, cu_seqlens, num_q_heads: int, num_kv_heads: int,
                    scale: float, causal: bool):
    """Materialized attention over packed variable-length sequences.

    q [T, Hq, D], k/v [T, Hkv, D] float64; cu_seqlens int [n+1].
    Returns O [T, Hq, D] float64 and LSE [Hq, T] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, D = q.shape
    assert Hq == num_q_heads and k.shape[1] == num_kv_heads
    assert num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    O = np.zeros((T, Hq, v.shape[2]), dtype=np.float64)
    LSE = np.full((Hq, T), NEG_INF, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        L = s1 - s0
        if L <= 0:
            continue
        mask = np.triu(np.ones((L, L), dtype=bool), 1) if causal else None
        for h in range(Hq):
            g = h // group
            S = scale * (q[s0:s1, h, :] @ k[s0:s1, g, :].T)
            if mask is not None:
                S[mask] = NEG_INF
            o, l = _softmax_rows(S, v[s0:s1, g, :])
            O[s0:s1, h] = o
            LSE[h, s0:s1] = l
    return O, LSE


def attention_bwd_dense(q, k, v, dout, cu_seqlens, num_q_heads: int, num_kv_heads: int,
                        scale: float, causal: bool):
    """Gradients of L = sum(dout * O) for O = attention_dense(q, k, v, ...).

    The backward pass the ELI5 of "Why your local LLM feels dumber than it is"
    describes recomputes the scores instead of storing them; what it computes
    is the derivative of the definition above, by the chain rule through
    s = scale q.k, P = softmax_j(s) and O = P V:
        dV_j = sum_i P_ij dO_i
        dP_ij = dO_i . V_j
        dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
        dQ_i = scale sum_j dS_ij K_j,    dK_j = scale sum_i dS_ij Q_i
    (masked pairs have P = 0 and contribute nothing). With GQA a kv head's
    dK/dV sum the contributions of every query head reading it. Scores are
    recomputed here in fp64 from the inputs; the forward's LSE is not used.
    Returns dq [T, Hq, D], dk [T, Hkv, D], dv [T, Hkv, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    T, Hq, D = q.shape
    assert Hq == num_q_heads and k.shape[1] == num_kv_heads
    assert num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    dq = np.zeros_like(q)
    dk = np.zeros((T, num_kv_heads, D), dtype=np.float64)
    dv = np.zeros((T, num_kv_heads, v.shape[2]), dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        L = s1 - s0
        if L <= 0:
            continue
        mask = np.triu(np.ones((L, L), dtype=bool), 1) if causal else None
        for h in range(Hq):
            g = h // group
            Q, K, V, dO = q[s0:s1, h], k[s0:s1, g], v[s0:s1, g], do[s0:s1, h]
            S = scale * (Q @ K.T)
            if mask is not None:
                S[mask] = NEG_INF
            m = S.max(axis=1, keepdims=True)
            W = np.exp(S - m)
            P = W / W.sum(axis=1, keepdims=True)
            dv[s0:s1, g] += P.T @ dO
            dP = dO @ V.T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[s0:s1, h] = scale * (dS @ K)
            dk[s0:s1, g] += scale * (dS.T @ Q)
    return dq, dk, dv


def attention_bwd_given(q, k, v, o, lse, dout, cu_seqlens, num_q_heads: int, num_kv_heads: int,
                        scale: float, causal: bool):
    """The backward pass as a function of the tensors it is handed: the
    forward's stored output o and log-sum-exp lse besides q, k, v and dout.
    The probabilities are rebuilt from lse, P_ij = exp(scale q_i.k_j - lse_i),
    and the row term from the stored output, Delta_i = dout_i . o_i; then
    dS = P (dP - Delta) and the same products as attention_bwd_dense. With the
    exact forward outputs the two functions agree; with o rounded to its
    storage format (bf16) this is what a recomputing backward computes, and
    it differs from the exact gradients by the rounding of o.
    Returns dq [T, Hq, D], dk [T, Hkv, D], dv [T, Hkv, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    T, Hq, D = q.shape
    assert Hq == num_q_heads and k.shape[1] == num_kv_heads and lse.shape == (Hq, T)
    group = num_q_heads // num_kv_heads
    dq = np.zeros_like(q)
    dk = np.zeros((T, num_kv_heads, D), dtype=np.float64)
    dv = np.zeros((T, num_kv_heads, v.shape[2]), dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        L = s1 - s0
        if L <= 0:
            continue
        mask = np.triu(np.ones((L, L), dtype=bool), 1) if causal else np.zeros((L, L), dtype=bool)
        for h in range(Hq):
            g = h // group
            Q, K, V, dO, Oh = q[s0:s1, h], k[s0:s1, g], v[s0:s1, g], do[s0:s1, h], o[s0:s1, h]
            S = scale * (Q @ K.T)
            P = np.exp(S - lse[h, s0:s1, None])
            P[mask] = 0.0
            dv[s0:s1, g] += P.T @ dO
            dS = P * (dO @ V.T - np.sum(dO * Oh, axis=1, keepdims=True))
            dq[s0:s1, h] = scale * (dS @ K)
            dk[s0:s1, g] += scale * (dS.T @ Q)
    return dq, dk, dv


def attention_brute(q, k, v, cu_seqlens, num_q_heads: int, num_kv_heads: int,
                    scale: float, causal: bool):
    """The same definition with scalar Python loops and exactly rounded sums
    (math.fsum); meant for a few dozen rows. Returns lists shaped like
    attention_dense's outputs (as float64 arrays)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, D = q.shape
    group = num_q_heads // num_kv_heads
    O = np.zeros((T, Hq, v.shape[2]))
    LSE = np.full((Hq, T), NEG_INF)
    cu = [int(x) for x in cu_seqlens]
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        for h in range(Hq):
            g = h // group
            for i in range(s0, s1):
                keys = range(s0, i + 1) if causal else range(s0, s1)
                scores = [scale * math.fsum(float(q[i, h, d]) * float(k[j, g, d]) for d in range(D))
                          for j in keys]
                if not scores:
                    continue
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                l = math.fsum(w)
                for d in range(v.shape[2]):
                    O[i, h, d] = math.fsum(wj * float(v[j, g, d]) for wj, j in zip(w, keys)) / l
                LSE[h, i] = m + math.log(l)
    return O, LSE


def attention_rows(q, k, v, cu_seqlens, num_q_heads: int, num_kv_heads: int,
                   scale: float, causal: bool, token_rows):
    """The same definition evaluated only for the listed packed token rows
    (for spot checks of problems too large to materialize). Returns
    O [n, Hq, D] and LSE [Hq, n] for the rows in the order given."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    group = num_q_heads // num_kv_heads
    rows = [int(t) for t in token_rows]
    O = np.zeros((len(rows), num_q_heads, v.shape[2]))
    LSE = np.full((num_q_heads, len(rows)), NEG_INF)
    for n, t in enumerate(rows):
        b = int(np.searchsorted(cu, t, side="right")) - 1
        s0, s1 = int(cu[b]), int(cu[b + 1])
        hi = t + 1 if causal else s1
        for h in range(num_q_heads):
            g = h // group
            Kb = np.asarray(k[s0:hi, g, :], dtype=np.float64)
            S = (scale * (Kb @ np.asarray(q[t, h, :], dtype=np.float64)))[None, :]
            o, l = _softmax_rows(S, np.asarray(v[s0:hi, g, :], dtype=np.float64))
            O[n, h] = o[0]
            LSE[h, n] = l[0]
    return O, LSE


# --------------------------------------------------------------------------
# paged decode ("GPU Datapath", section D: one query token per sequence, the
# KV cache read through a block table of 16-token pages)
# --------------------------------------------------------------------------
def gather_sequence_kv(k_cache, v_cache, block_table, seq_len: int, b: int):
    """Logical token t of sequence b sits in physical page block_table[b, t//P],
    slot t % P. Returns K, V [seq_len, Hkv, D] for that sequence."""
    P = k_cache.shape[1]
    n_pages = (seq_len + P - 1) // P
    pages = [int(x) for x in block_table[b, :n_pages]]
    if n_pages == 0:
        shp = (0,) + tuple(k_cache.shape[2:])
        return np.zeros(shp), np.zeros(shp)
    K = np.concatenate([k_cache[p] for p in pages], axis=0)[:seq_len]
    V = np.concatenate([v_cache[p] for p in pages], axis=0)[:seq_len]
    return np.asarray(K, dtype=np.float64), np.asarray(V, dtype=np.float64)


def prefill_paged_dense(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k,
                        num_q_heads: int, num_kv_heads: int, scale: float, causal: bool):
    """Chunked prefill against a paged cache: sequence b has the query rows
    q[cu_seqlens_q[b]:cu_seqlens_q[b+1]] (Lq of them) and Lk = seq_lens_k[b]
    cached keys/values (pages through block_table[b], as in
    gather_sequence_kv). With causal masking query i sees keys
    j <= i + (Lk - Lq); a query that sees no key gets O = 0, LSE = -inf.
    q [Tq, Hq, D]; returns O [Tq, Hq, D] and LSE [Hq, Tq] float64."""
    q = np.asarray(q, dtype=np.float64)
    Tq, Hq, D = q.shape
    assert Hq == num_q_heads and k_cache.shape[2] == num_kv_heads
    group = num_q_heads // num_kv_heads
    O = np.zeros((Tq, Hq, v_cache.shape[3]), dtype=np.float64)
    LSE = np.full((Hq, Tq), NEG_INF, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens_q]
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        Lq, Lk = s1 - s0, int(seq_lens_k[b])
        if Lq <= 0:
            continue
        K, V = gather_sequence_kv(k_cache, v_cache, block_table, Lk, b)
        if causal:
            i = np.arange(Lq)[:, None]
            j = np.arange(Lk)[None, :]
            mask = j > i + (Lk - Lq)
        else:
            mask = None
        for h in range(Hq):
            g = h // group
            S = scale * (q[s0:s1, h, :] @ K[:, g, :].T)
            if mask is not None:
                S[mask] = NEG_INF
            o, l = _softmax_rows(S, V[:, g, :])
            O[s0:s1, h] = o
            LSE[h, s0:s1] = l
    return O, LSE


def decode_dense(q, k_cache, v_cache, block_table, seq_lens, scale: float):
    """q [B, Hq, D]; caches [pages, P, Hkv, D]; returns O [B, Hq, D], LSE [B, Hq]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    O = np.zeros((B, Hq, v_cache.shape[3]))
    LSE = np.full((B, Hq), NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K, V = gather_sequence_kv(k_cache, v_cache, block_table, L, b)
        for h in range(Hq):
            g = h // group
            S = (scale * (K[:, g, :] @ q[b, h, :]))[None, :]
            o, l = _softmax_rows(S, V[:, g, :])
            O[b, h] = o[0]
            LSE[b, h] = l[0]
    return O, LSE


def decode_brute(scores, values):
    """Exact scalar softmax-weighted mean for one query: the max-subtracted,
    exactly rounded form (section "Plugging in actual numbers" gives this
    shape of reference). scores, values: 1-D sequences. Returns (o, lse)."""
    scores = [float(s) for s in scores]
    if not scores:
        return 0.0, NEG_INF
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    l = math.fsum(w)
    return math.fsum(wi * float(vi) for wi, vi in zip(w, values)) / l, m + math.log(l)


# --------------------------------------------------------------------------
# split-KV partials and their log-sum-exp merge
# ("Why the calculation is split into groups"; the FlashAttention 2 merge of
#  normalized fp32 partial outputs weighted by exp(LSE_s - max LSE) described
#  under "Backend names expand into four decode algorithms")
# --------------------------------------------------------------------------
def page_split_ranges(n_pages: int, num_splits: int, table_pages: int = None):
    """Contiguous, page-aligned groups of ceil(table_pages / num_splits) pages
    each (table_pages defaults to n_pages, the sequence's own page count);
    groups past the sequence's end are empty. With one sequence that fills its
    block table this is the equal-count partition of "Why the calculation is
    split into groups"; in a batch the group size comes from the table width,
    so every sequence is cut into groups of the same size."""
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    basis = n_pages if table_pages is None else table_pages
    pps = -(-basis // num_splits) if basis > 0 else 0
    return [(min(s * pps, n_pages), min((s + 1) * pps, n_pages)) for s in range(num_splits)]


def decode_split_partials(q, k_cache, v_cache, block_table, seq_lens, scale: float,
                          num_splits: int):
    """Per (sequence, q-head, split): the normalized partial output
    O_s = sum w v / l over the split's keys and LSE_s = m_s + ln l_s, with
    (0, -inf) for an empty split; groups are page_split_ranges with the block
    table width as the basis. Returns po [B*Hq, S, D], plse [B*Hq, S]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    P = k_cache.shape[1]
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    po = np.zeros((B * Hq, num_splits, v_cache.shape[3]))
    plse = np.full((B * Hq, num_splits), NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K, V = gather_sequence_kv(k_cache, v_cache, block_table, L, b)
        n_pages = (L + P - 1) // P
        for s, (p0, p1) in enumerate(page_split_ranges(n_pages, num_splits, block_table.shape[1])):
            t0, t1 = p0 * P, min(p1 * P, L)
            if t1 <= t0:
                continue
            for h in range(Hq):
                g = h // group
                S = (scale * (K[t0:t1, g, :] @ q[b, h, :]))[None, :]
                o, l = _softmax_rows(S, V[t0:t1, g, :])
                po[b * Hq + h, s] = o[0]
                plse[b * Hq + h, s] = l[0]
    return po, plse


def combine_partials(po, plse):
    """Merge split partials: M = max over non-empty splits of LSE_s,
    w_s = exp(LSE_s - M), O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s.
    A row whose splits are all empty gives (0, -inf).
    po [rows, S, D], plse [rows, S] -> O [rows, D], LSE [rows]."""
    po = np.asarray(po, dtype=np.float64)
    plse = np.asarray(plse, dtype=np.float64)
    rows, S, D = po.shape
    O = np.zeros((rows, D))
    LSE = np.full(rows, NEG_INF)
    for r in range(rows):
        ne = np.isfinite(plse[r])
        if not ne.any():
            continue
        M = plse[r, ne].max()
        w = np.exp(plse[r, ne] - M)
        W = w.sum()
        O[r] = (w[:, None] * po[r, ne]).sum(axis=0) / W
        LSE[r] = M + math.log(W)
    return O, LSE
