"""CPU checks of the seeded input generators (formats and determinism)."""
import numpy as np
import torch

from workloads import (CONFIGS, bf16_bits_from_f32, e4m3_bits_from_f32, make_config, make_inputs,
                       quantize_blocks_128x128, quantize_rows_1x128)


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    v = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10 ** g.uniform(-5, 5, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.4e38, 1e-40], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits_from_f32(v), ref)


def test_e4m3_rounding_matches_torch_in_range():
    g = np.random.default_rng(1)
    v = (g.standard_normal(200000) * 10 ** g.uniform(-4, 2.6, 200000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    v = np.concatenate([v, np.array([0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -11], np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_bits_from_f32(v), ref)


def test_e4m3_saturates():
    codes = e4m3_bits_from_f32(np.array([460.0, 470.0, 1e6, -1e6], np.float32))
    assert codes.tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def test_block_quantisers_scale_is_amax_over_448():
    g = np.random.default_rng(2)
    a = g.standard_normal((4, 256)).astype(np.float32)
    q, s = quantize_rows_1x128(a)
    np.testing.assert_allclose(s, np.abs(a.reshape(4, 2, 128)).max(2) / 448, rtol=1e-7)
    assert q.shape == a.shape and s.shape == (4, 2)
    w = g.standard_normal((256, 384)).astype(np.float32)
    q, s = quantize_blocks_128x128(w)
    assert q.shape == w.shape and s.shape == (2, 3)


def test_generation_is_deterministic_and_shaped():
    a = make_inputs(64, 128, 256, 8, 2, seed=0)
    b = make_inputs(64, 128, 256, 8, 2, seed=0)
    c = make_inputs(64, 128, 256, 8, 2, seed=1)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.W1, b.W1) and np.array_equal(a.logits, b.logits)
    assert not np.array_equal(a.x, c.x)
    assert a.x.shape == (64, 128) and a.W1.shape == (8, 128, 512) and a.W2.shape == (8, 256, 128)
    assert a.logits.dtype == np.float32 and a.logits.shape == (64, 8)
    t = make_config("tiny")
    assert t.dy is None and (t.T, t.d, t.f, t.E, t.k) == (64, 128, 256, 8, 2)


def test_skew_bias_is_zipf_like():
    c = CONFIGS["skewed"]
    inp = make_inputs(2048, 128, 128, c["E"], c["k"], seed=3, skew=3.0)
    rank = inp.meta["expert_rank"]
    assert sorted(rank.tolist()) == list(range(1, c["E"] + 1))


def test_fp8_sparse_case_has_empty_experts():
    # the sparse pre-routed fp8 parity case (64 global experts, 6 local, 24 tokens, top-2,
    # seed 31) exercises experts that receive no token, whose weight gradients must be zero
    from workloads import make_prerouted_fp8
    inp = make_prerouted_fp8(24, 64, 6, 256, 256, 2, 31)
    counts = np.bincount(inp.topk_ids[inp.topk_ids >= 0], minlength=6)
    assert (counts == 0).any() and counts.sum() > 0
