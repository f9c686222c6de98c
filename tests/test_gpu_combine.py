"""The combine kernel against the oracle's merge on arbitrary partials."""
import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as mi
import oracle
import synth
from gpu_util import FP32_MAX_ABS, assert_bf16_rounding_of, errors, f32_dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,S,D", [(37, 1, 64), (37, 3, 128), (16, 256, 256), (5, 300, 128), (9, 64, 4),
                                      (3, 2, 1024)])
def test_combine_matches_oracle(rows, S, D):
    po, pl = synth.random_partials(S + D, rows, S, D)
    O, L = oracle.combine_partials(po, pl)
    for dt in (torch.float32, torch.bfloat16):
        o, l = mi.attn_combine(f32_dev(po), f32_dev(pl), out_dtype=dt)
        torch.cuda.synchronize()
        lo = host(l)
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(lo), fin)
        assert np.max(np.abs(lo[fin] - L[fin]), initial=0) <= 1e-5
        if dt == torch.float32:
            mx, _ = errors(host(o), O)
            assert mx <= FP32_MAX_ABS, mx
        else:
            # arbitrary partials reach |O| ~ 3, where bf16 rounding alone exceeds the
            # attention tolerances: check the output is the bf16 rounding of the merge
            assert_bf16_rounding_of(host(o), O, what=f"combine {rows}x{S}x{D}")
        assert np.all(host(o)[~fin] == 0)
