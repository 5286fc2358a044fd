"""The seeded input generators (shared by the oracle and the GPU path)."""
import numpy as np
import pytest

from nc_synth import (bf16_bits, bf16_from_bits, bf16_round, get_config,
                      make_params, make_tokens, param_shapes, zipf_probs)


@pytest.mark.parametrize("name,top1", [("gpt2", 0.1389), ("d20", 0.1373)])
def test_zipf_top1_frequency_matches_harmonic_closed_form(name, top1):
    cfg = get_config(name)
    V, s = cfg["vocab"], cfg["zipf_s"]
    h = np.sum(np.arange(1, V + 1, dtype=np.float64) ** -s)
    assert 1.0 / h == pytest.approx(top1, abs=5e-4)
    tokens, targets = make_tokens(cfg)
    n = tokens.size
    p = 1.0 / h
    freq = np.mean(tokens == 0)
    assert abs(freq - p) < 4 * np.sqrt(p * (1 - p) / n)
    assert tokens.min() >= 0 and tokens.max() < V
    np.testing.assert_array_equal(tokens[:, 1:], targets[:, :-1])


def test_uniform_tokens_and_determinism():
    cfg = get_config("tiny")
    a = make_tokens(cfg)
    b = make_tokens(cfg)
    np.testing.assert_array_equal(a[0], b[0])
    assert a[0].dtype == np.int32 and a[0].shape == (2, 64)
    assert make_tokens(cfg, seed=5)[0].tolist() != a[0].tolist()


def test_params_shapes_std_and_bf16_exactness():
    cfg = get_config("tiny", dtype="bf16")
    p = make_params(cfg)
    for name, shape, std in param_shapes(cfg):
        w = p[name]
        assert w.shape == shape and w.dtype == np.float32
        np.testing.assert_array_equal(bf16_round(w), w)
        assert np.std(w) == pytest.approx(std, rel=0.05)
    p2 = make_params(cfg)
    assert all(np.array_equal(p[k], p2[k]) for k in p)


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.1415927],
                 dtype=np.float32)
    r = bf16_round(x)
    # 1 + 2^-8 is the halfway point between 1 and 1 + 2^-7: ties to even -> 1
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -6 and r[3] == 1.0
    assert r[4] == -2.5
    assert abs(r[5] - 3.140625) == 0
    np.testing.assert_array_equal(bf16_from_bits(bf16_bits(r)), r)


def test_param_counts_match_closed_form():
    expect = {"tiny": 491520, "gpt2": 149153280, "d20": 502005760,
              "d30": 1372323840, "long": 502005760}
    for name, n in expect.items():
        cfg = get_config(name)
        assert sum(r * c for _, (r, c), _ in param_shapes(cfg)) == n
