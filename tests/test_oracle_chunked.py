"""Pins for the oracle's chunked-prefill form (a query chunk against a paged
cache holding the whole sequence; queries aligned to the end of the sequence).

Each pin ties prefill_paged_dense to a differently built, already pinned form
or to a property the definition forces:
- a chunk that is the whole sequence, read from an in-order cache, is the
  plain causal / non-causal prefill (attention_dense);
- cutting a causal prefill into consecutive chunks, each against the cache of
  everything up to its end, reproduces the full prefill's rows (this is what
  end-alignment of the causal mask means);
- a one-token chunk is the decode query (decode_dense), causal or not;
- the physical page order does not matter;
- with fewer cached keys than queries, the leading queries see nothing.
"""
import numpy as np
import pytest

import oracle
import synth

TOL = 1e-12


def _pages_for(k_tok, v_tok, lens, shuffle, seed=0):
    """Paged caches holding consecutive runs of k_tok / v_tok rows."""
    total = sum((c + 15) // 16 for c in lens)
    rng = np.random.default_rng([77, seed])
    phys = rng.permutation(total) if shuffle else np.arange(total)
    return synth._fill_pages(k_tok.astype(np.float32), v_tok.astype(np.float32), lens, phys, total, "nan")


def _case(L, Hq=4, Hkv=2, D=16, seed=0):
    # float32-exact values: the paged caches are stored as float32
    rng = np.random.default_rng([78, seed])
    f = lambda shape: rng.standard_normal(shape).astype(np.float32).astype(np.float64)
    return f((L, Hq, D)), f((L, Hkv, D)), f((L, Hkv, D))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shuffle", [False, True])
def test_whole_sequence_chunk_is_prefill(causal, shuffle):
    lens = [37, 1, 64, 19]
    Hq, Hkv, D = 4, 2, 16
    qs, ks, vs = zip(*[_case(L, Hq, Hkv, D, seed=i) for i, L in enumerate(lens)])
    q, k, v = np.concatenate(qs), np.concatenate(ks), np.concatenate(vs)
    cu = np.concatenate([[0], np.cumsum(lens)])
    O, L = oracle.attention_dense(q, k, v, cu, Hq, Hkv, 0.3, causal)
    kc, vc, bt = _pages_for(k, v, lens, shuffle)
    Op, Lp = oracle.prefill_paged_dense(q, kc, vc, bt, cu, np.array(lens), Hq, Hkv, 0.3, causal)
    assert np.max(np.abs(Op - O)) <= TOL
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(Lp), fin)
    assert np.max(np.abs(Lp[fin] - L[fin])) <= TOL


def test_chunks_reproduce_the_full_causal_prefill():
    Lfull, Hq, Hkv, D = 90, 4, 1, 8
    q, k, v = _case(Lfull, Hq, Hkv, D, seed=3)
    O, LSE = oracle.attention_dense(q, k, v, [0, Lfull], Hq, Hkv, 0.25, True)
    cuts = [0, 17, 18, 50, 90]
    for a, b in zip(cuts[:-1], cuts[1:]):
        # the cache of sequence "b" holds tokens [0, b); the chunk is rows [a, b)
        kc, vc, bt = _pages_for(k[:b], v[:b], [b], shuffle=True, seed=a)
        Oc, Lc = oracle.prefill_paged_dense(q[a:b], kc, vc, bt, [0, b - a], np.array([b]), Hq, Hkv, 0.25, True)
        assert np.max(np.abs(Oc - O[a:b])) <= TOL
        assert np.max(np.abs(Lc - LSE[:, a:b])) <= TOL


@pytest.mark.parametrize("causal", [False, True])
def test_one_token_chunk_is_decode(causal):
    lens = [5, 40, 16]
    Hq, Hkv, D = 8, 2, 16
    rng = np.random.default_rng(5)
    f = lambda shape: rng.standard_normal(shape).astype(np.float32).astype(np.float64)
    k = f((sum(lens), Hkv, D))
    v = f((sum(lens), Hkv, D))
    qd = f((len(lens), Hq, D))
    kc, vc, bt = _pages_for(k, v, lens, shuffle=True)
    Od, Ld = oracle.decode_dense(qd, kc, vc, bt, np.array(lens), 0.2)
    cu = np.arange(len(lens) + 1)
    Op, Lp = oracle.prefill_paged_dense(qd, kc, vc, bt, cu, np.array(lens), Hq, Hkv, 0.2, causal)
    assert np.max(np.abs(Op - Od)) <= TOL
    assert np.max(np.abs(Lp.T - Ld)) <= TOL


def test_queries_before_the_first_key_are_empty():
    # 6 queries, 4 cached keys: causal query i sees keys j <= i - 2
    Hq, Hkv, D = 2, 1, 8
    q, k, v = _case(6, Hq, Hkv, D, seed=9)
    kc, vc, bt = _pages_for(k[:4], v[:4], [4], shuffle=False)
    O, L = oracle.prefill_paged_dense(q, kc, vc, bt, [0, 6], np.array([4]), Hq, Hkv, 0.5, True)
    assert np.all(O[:2] == 0) and np.all(np.isneginf(L[:, :2]))
    # query 2 sees exactly key 0: its output is v[0] and its LSE the one score
    assert np.max(np.abs(O[2, 0] - v[0, 0])) <= TOL
    assert abs(L[0, 2] - 0.5 * float(q[2, 0] @ k[0, 0])) <= TOL
    # query 5 sees every key: the non-causal row
    On, Ln = oracle.prefill_paged_dense(q, kc, vc, bt, [0, 6], np.array([4]), Hq, Hkv, 0.5, False)
    assert np.max(np.abs(O[5] - On[5])) <= TOL


def test_chunked_generator_matches_its_description():
    c = synth.make_chunked_prefill(6, 1, [3, 20], [3, 50], 4, 2, 16, 0.25, shuffle=True, tail="nan")
    assert c.q.shape == (23, 4, 16) and list(c.cu_seqlens_q) == [0, 3, 23]
    assert list(c.seq_lens_k) == [3, 50]
    # every used page appears once; tails past each sequence are NaN
    used = c.block_table[c.block_table >= 0]
    assert len(set(used.tolist())) == len(used) == 1 + 4
    kc = synth.bf16_to_f64(c.k_cache)
    assert np.isnan(kc[c.block_table[0, 0], 3:]).all()
    assert not np.isnan(kc[c.block_table[0, 0], :3]).any()
