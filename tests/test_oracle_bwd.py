"""Pins for the oracle's backward pass (attention_bwd_dense).

- central finite differences of the forward oracle on tiny packed inputs
  (causal and not, GQA): every element of dQ, dK, dV;
- an independent implementation: torch's CPU autograd (float64) through
  softmax(scale Q K^T) V written with torch ops;
- closed forms: the keys' dV sum to the queries' dO sum (softmax rows sum to
  1), the keys' dK sum to zero (the rows of dS sum to zero), and a
  one-token sequence has dQ = dK = 0 and dV = the dO of its query heads.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(seqlens, Hq, Hkv, D, seed):
    rng = np.random.default_rng([91, seed])
    T = sum(seqlens)
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    do = rng.standard_normal((T, Hq, D))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    return q, k, v, do, cu


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences(causal):
    seqlens, Hq, Hkv, D, scale = [5, 3, 1], 4, 2, 3, 0.7
    q, k, v, do, cu = _case(seqlens, Hq, Hkv, D, 0)

    def loss(q_, k_, v_):
        O, _ = oracle.attention_dense(q_, k_, v_, cu, Hq, Hkv, scale, causal)
        return float(np.sum(O * do))

    dq, dk, dv = oracle.attention_bwd_dense(q, k, v, do, cu, Hq, Hkv, scale, causal)
    h = 1e-6
    for which, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[which]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[which]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(num - g)) < 1e-7, which


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_autograd(causal):
    seqlens, Hq, Hkv, D, scale = [37, 64, 1, 20], 8, 2, 16, 0.25
    q, k, v, do, cu = _case(seqlens, Hq, Hkv, D, 1)
    dq, dk, dv = oracle.attention_bwd_dense(q, k, v, do, cu, Hq, Hkv, scale, causal)
    G = Hq // Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    outs = []
    for b in range(len(seqlens)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        Q = tq[s0:s1].transpose(0, 1)                                   # [Hq, L, D]
        K = tk[s0:s1].transpose(0, 1).repeat_interleave(G, dim=0)       # [Hq, L, D]
        V = tv[s0:s1].transpose(0, 1).repeat_interleave(G, dim=0)
        S = scale * torch.matmul(Q, K.transpose(1, 2).contiguous())
        if causal:
            L = s1 - s0
            S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        outs.append(torch.matmul(torch.softmax(S, dim=-1), V).transpose(0, 1))
    O = torch.cat(outs, dim=0)
    (O * torch.tensor(do)).sum().backward()
    assert np.max(np.abs(tq.grad.numpy() - dq)) < 1e-12
    assert np.max(np.abs(tk.grad.numpy() - dk)) < 1e-12
    assert np.max(np.abs(tv.grad.numpy() - dv)) < 1e-12


def test_closed_forms():
    seqlens, Hq, Hkv, D, scale = [50, 1, 17], 6, 3, 8, 0.4
    q, k, v, do, cu = _case(seqlens, Hq, Hkv, D, 2)
    G = Hq // Hkv
    for causal in (True, False):
        dq, dk, dv = oracle.attention_bwd_dense(q, k, v, do, cu, Hq, Hkv, scale, causal)
        for b in range(len(seqlens)):
            s0, s1 = int(cu[b]), int(cu[b + 1])
            for g in range(Hkv):
                dsum = do[s0:s1, g * G:(g + 1) * G].sum(axis=(0, 1))
                assert np.max(np.abs(dv[s0:s1, g].sum(axis=0) - dsum)) < 1e-12
                assert np.max(np.abs(dk[s0:s1, g].sum(axis=0))) < 1e-12
        # the one-token sequence (rows 50): its softmax is the constant 1
        assert np.all(dq[50] == 0) and np.all(dk[50] == 0)
        for g in range(Hkv):
            assert np.max(np.abs(dv[50, g] - do[50, g * G:(g + 1) * G].sum(axis=0))) < 1e-15


@pytest.mark.parametrize("causal", [True, False])
def test_given_form_with_exact_forward_outputs_is_the_gradient(causal):
    seqlens, Hq, Hkv, D, scale = [37, 64, 1, 20], 8, 2, 16, 0.25
    q, k, v, do, cu = _case(seqlens, Hq, Hkv, D, 3)
    O, LSE = oracle.attention_dense(q, k, v, cu, Hq, Hkv, scale, causal)
    want = oracle.attention_bwd_dense(q, k, v, do, cu, Hq, Hkv, scale, causal)
    got = oracle.attention_bwd_given(q, k, v, O, LSE, do, cu, Hq, Hkv, scale, causal)
    for w, g in zip(want, got):
        assert np.max(np.abs(w - g)) < 1e-12


def test_given_form_sees_the_stored_output():
    # shifting the stored output of one row by e moves Delta of that row by
    # dO . e and changes only that query's dQ and the keys it sees
    seqlens, Hq, Hkv, D, scale = [12], 2, 1, 4, 0.5
    q, k, v, do, cu = _case(seqlens, Hq, Hkv, D, 4)
    O, LSE = oracle.attention_dense(q, k, v, cu, Hq, Hkv, scale, True)
    O2 = O.copy()
    O2[5, 1] += 0.25
    a = oracle.attention_bwd_given(q, k, v, O, LSE, do, cu, Hq, Hkv, scale, True)
    b = oracle.attention_bwd_given(q, k, v, O2, LSE, do, cu, Hq, Hkv, scale, True)
    dq_diff = np.abs(a[0] - b[0]).sum(axis=2)
    assert np.count_nonzero(dq_diff > 1e-15) == 1 and dq_diff[5, 1] > 0
    assert np.all(a[2] == b[2])                                   # dV does not use Delta
    assert np.all(np.abs(a[1] - b[1])[6:] < 1e-15)                 # keys after query 5 unaffected
