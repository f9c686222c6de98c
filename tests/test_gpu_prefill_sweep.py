"""A fixed, seeded sweep of 180 prefill problems against the fp64 oracle:
120 dense (1-4 packed sequences of 0-1299 tokens, G in {1, 2, 4, 8}, Hkv in
{1, 2, 4}, head_dim in {64, 128, 256}, causal or not) and 60 chunked ones
(query chunks of 1-399 tokens after cached prefixes of 0-1499, shuffled pages,
NaN page tails).

The bar here is the bf16 bar as a bf16 output can meet it: mean-abs 1e-3 and
max-abs 1e-2 on the error beyond each element's own rounding to bf16 (half an
ulp of the exact value). Rows that average two or three keys copy single V
values, and where such an output has |O| >= 4 half an ulp is already 0.0156, so
no bf16 result meets a plain 1e-2 there; the plain max-abs is printed. The
workload configurations keep the plain 1e-2 in their own tests."""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as mi
import oracle
import synth
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, LSE_MAX_ABS, bf16_dev, half_ulp_bf16, host, i32_dev

pytestmark = pytest.mark.gpu


def _stats(o, O, l, L):
    err = np.abs(o - O)
    excess = float(np.max(err - half_ulp_bf16(O))) if err.size else 0.0
    fin = np.isfinite(L)
    lerr = float(np.max(np.abs(l[fin] - L[fin]))) if fin.any() else 0.0
    same_inf = bool(np.array_equal(np.isneginf(l), np.isneginf(L)))
    return float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0, excess, lerr, same_inf


def _specs():
    """The 180 problem specifications, drawn in one fixed order."""
    rng = np.random.default_rng(123)
    out = []
    for i in range(180):
        D = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        causal = bool(rng.integers(0, 2))
        if i < 120:
            ns = int(rng.integers(1, 5))
            lens = [int(x) for x in rng.integers(0, 1300, ns)]
            if sum(lens) == 0:
                lens[0] = 1
            out.append(("dense", i, D, Hkv * G, Hkv, causal, lens, None))
        else:
            ns = int(rng.integers(1, 4))
            ql = [int(x) for x in rng.integers(1, 400, ns)]
            kl = [a + int(x) for a, x in zip(ql, rng.integers(0, 1500, ns))]
            out.append(("chunked", i, D, Hkv * G, Hkv, causal, ql, kl))
    return out


def _run(spec):
    kind, i, D, Hq, Hkv, causal, a, b = spec
    if kind == "dense":
        c = synth.make_prefill(40, i, a, Hq, Hkv, D, 1 / math.sqrt(D), causal, "bf16", "sweep")
        o, l = mi.attn_fwd(bf16_dev(c.q), bf16_dev(c.k), bf16_dev(c.v), i32_dev(c.cu_seqlens), c.max_seqlen,
                           scale=c.scale, causal=causal)
        torch.cuda.synchronize()
        q, k, v = c.as_f64()
        O, L = oracle.attention_dense(q, k, v, c.cu_seqlens, Hq, Hkv, c.scale, causal)
    else:
        c = synth.make_chunked_prefill(41, i, a, b, Hq, Hkv, D, D ** -0.5, shuffle=True, tail="nan")
        o, l = mi.attn_fwd_paged(bf16_dev(c.q), bf16_dev(c.k_cache), bf16_dev(c.v_cache), i32_dev(c.block_table),
                                 i32_dev(c.cu_seqlens_q), i32_dev(c.seq_lens_k), c.max_seqlen_q, scale=c.scale,
                                 causal=causal)
        torch.cuda.synchronize()
        O, L = oracle.prefill_paged_dense(synth.bf16_to_f64(c.q), synth.bf16_to_f64(c.k_cache),
                                          synth.bf16_to_f64(c.v_cache), c.block_table, c.cu_seqlens_q,
                                          c.seq_lens_k, Hq, Hkv, c.scale, causal)
    return _stats(host(o), O, host(l), L)


@pytest.mark.parametrize("part", range(6))
def test_prefill_sweep(part):
    """Problems 30 part .. 30 part + 29 of the sweep."""
    bad, worst_plain, worst_excess, worst_mean = [], 0.0, -1.0, 0.0
    for spec in _specs()[30 * part:30 * part + 30]:
        what = "{} {} D={} Hq={} Hkv={} causal={} lens={} {}".format(spec[0], spec[1], spec[2], spec[3], spec[4],
                                                                     spec[5], spec[6], spec[7] or "")
        print(f"[sweep] {what}", flush=True)
        mx, mean, excess, lerr, same_inf = _run(spec)
        worst_plain, worst_excess, worst_mean = max(worst_plain, mx), max(worst_excess, excess), max(worst_mean,
                                                                                                     mean)
        if not (mean <= BF16_MEAN_ABS and excess <= BF16_MAX_ABS and lerr <= LSE_MAX_ABS and same_inf):
            bad.append((what, mx, mean, excess, lerr, same_inf))
    print(f"  part {part}: plain max-abs {worst_plain:.4e}, max beyond bf16 rounding {worst_excess:.4e}, "
          f"worst mean-abs {worst_mean:.3e}", flush=True)
    assert not bad, bad
