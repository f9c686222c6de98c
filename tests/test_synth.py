"""Input generators: bf16 rounding against torch, cache layout, determinism."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38, 1e-40,
                                  np.inf, -np.inf], dtype=np.float32)])
    # exact ties of the bf16 grid: x = bf16 + half-ulp
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.isnan(synth.bf16_to_f64(synth.bf16_bits(np.array([np.nan], np.float32))))[0]


def test_generators_are_seeded():
    a = synth.config2(S=64, seed=1)
    b = synth.config2(S=64, seed=1)
    c = synth.config2(S=64, seed=2)
    assert np.array_equal(a.q, b.q) and not np.array_equal(a.q, c.q)


def test_paged_cache_holds_each_token_once():
    c = synth.make_decode(9, 0, [33, 16, 1], 4, 2, 8, 0.5, shuffle=True, tail="nan")
    k = synth.bf16_to_f64(c.k_cache)
    used = c.block_table[c.block_table >= 0]
    assert len(set(used.tolist())) == len(used)           # each physical page used once
    for b, L in enumerate(c.seq_lens):
        n = (L + 15) // 16
        last = c.block_table[b, n - 1]
        tail = L - 16 * (n - 1)
        assert np.all(np.isnan(k[last, tail:]))            # tail slots poisoned
        assert np.all(np.isfinite(k[last, :tail]))


def test_identity_table_is_contiguous_cache():
    c = synth.config4(ctx=256, seed=0)
    assert np.array_equal(c.block_table[0], np.arange(16))
    assert c.meta["outlier_channels"] is not None and len(c.meta["outlier_channels"]) == 4
    k = synth.bf16_to_f64(c.k_cache).reshape(256, 4, 256)
    ch = c.meta["outlier_channels"]
    other = [i for i in range(256) if i not in ch]
    assert np.abs(k[:, :, ch]).mean() > 5 * np.abs(k[:, :, other]).mean()


def test_worked_example_inputs_are_bf16_exact():
    s, v = synth.worked_example_scores_values()
    assert np.array_equal(synth.bf16_to_f64(synth.bf16_bits(s.astype(np.float32))), s)
    assert np.array_equal(synth.bf16_to_f64(synth.bf16_bits(v.astype(np.float32))), v)


def test_output_gradient_stream_is_separate():
    c = synth.make_prefill(2, 0, [100, 28], 4, 2, 64, 0.125, True)
    d1 = synth.output_gradient(2, 0, c.total_tokens, 4, 64)
    d2 = synth.output_gradient(2, 0, c.total_tokens, 4, 64)
    assert d1.shape == (128, 4, 64) and d1.dtype == np.uint16 and np.array_equal(d1, d2)
    assert not np.array_equal(d1, c.q)
    x = synth.bf16_to_f64(d1)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
