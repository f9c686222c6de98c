"""Helpers for the GPU parity tests (test side only)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
FP32_MAX_ABS = 1e-5
LSE_MAX_ABS = 1e-3


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def i32_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def errors(got, want):
    e = np.abs(got - want)
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def assert_bf16_close(got, want, what=""):
    mx, mean = errors(got, want)
    print(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (what, mx, mean)


def assert_bf16_rounding_of(got, want, slop=2e-5, what=""):
    """got is a bf16 result whose exact value is `want`: allow half a bf16 ulp
    of |want| (round to nearest) plus the fp32 arithmetic slop."""
    a = np.maximum(np.abs(want), np.abs(got))
    ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 0.0)
    bad = np.abs(got - want) > 0.5 * ulp + slop
    print(f"  {what}: {int(bad.sum())} elements beyond half a bf16 ulp", flush=True)
    assert not bad.any(), what


def half_ulp_bf16(x):
    """Half the spacing of bf16 numbers at |x| (the most a correctly rounded
    bf16 result can differ from x)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def assert_bf16_close_beyond_rounding(got, want, what=""):
    """The bf16 bar applied to what a bf16 output can reach: the error beyond
    each element's own rounding to bf16 (half an ulp of the exact value) within
    max-abs 1e-2, and the plain error within mean-abs 1e-3."""
    err = np.abs(got - want)
    excess = float(np.max(err - half_ulp_bf16(want))) if err.size else 0.0
    mx, mean = errors(got, want)
    print(f"  {what}: max-abs {mx:.3e} (beyond rounding {excess:.3e}) mean-abs {mean:.3e}", flush=True)
    assert excess <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (what, mx, excess, mean)


def assert_lse_close(got, want, what="", tol=LSE_MAX_ABS):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), what
    assert np.array_equal(got[~fin], want[~fin]), what
    mx, _ = errors(got[fin], want[fin])
    print(f"  {what} lse: max-abs {mx:.3e}", flush=True)
    assert mx <= tol, (what, mx, tol)


def bitwise_equal(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def dense_oracle_parallel(q, k, v, cu_seqlens, num_q_heads, num_kv_heads, scale, causal, workers=None):
    """oracle.attention_dense on the whole problem, computed as independent
    sub-problems (one sequence, one kv head and its query heads) on a thread
    pool; each sub-problem is the oracle's own call, so the result is the
    oracle's, only sooner on a many-core host."""
    T, Hq, _ = q.shape
    G = num_q_heads // num_kv_heads
    O = np.zeros((T, Hq, v.shape[2]), dtype=np.float64)
    L = np.full((Hq, T), -np.inf, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    jobs = [(b, g) for b in range(len(cu) - 1) for g in range(num_kv_heads)]
    jobs.sort(key=lambda j: -(cu[j[0] + 1] - cu[j[0]]))   # longest first

    def one(job):
        b, g = job
        s0, s1 = cu[b], cu[b + 1]
        o, l = oracle.attention_dense(q[s0:s1, g * G:(g + 1) * G], k[s0:s1, g:g + 1], v[s0:s1, g:g + 1],
                                      np.array([0, s1 - s0]), G, 1, scale, causal)
        O[s0:s1, g * G:(g + 1) * G] = o
        L[g * G:(g + 1) * G, s0:s1] = l

    n = workers or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(one, jobs))
    return O, L
