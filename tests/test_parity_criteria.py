"""The comparison criteria of the full-size forward checks, shown on the CPU to
be able to fail.

The full-size GPU tests compare per-token losses with the oracle's through
their deviation from ln V (tests/gpu_helpers.loss_deviation_errors), with an
unembedding of std 0.05 so that the logits carry the features' information
(at the workloads' own std of 0.001 every logit is ~0.04 and every loss sits
within a few hundredths of ln V).  These tests use only the oracle: a feature
set unrelated to the right one, and forward passes with planted mistakes, must
fail the criterion that the GPU passes.
"""
import numpy as np
import pytest

import oracle
import oracle.model as om
from nc_synth import bf16_round, get_config, make_params, make_tokens
from tests.gpu_helpers import DEV_COS, DEV_REL_L2, loss_deviation_errors, rel_l2


def _unit_rows(a):
    return a / np.sqrt(np.mean(a * a, axis=-1, keepdims=True))


def test_unrelated_features_pass_the_plain_loss_bar_but_fail_the_deviation_bar():
    """Softcap-CE at the d20 head shape (V = 65536, D = 1280) over 128 tokens
    for two unrelated unit-RMS feature sets."""
    V, D, n = 65536, 1280, 128
    rng = np.random.default_rng(11)
    y = rng.integers(0, V, n)
    f1 = _unit_rows(rng.standard_normal((n, D)))
    f2 = _unit_rows(rng.standard_normal((n, D)))
    # at the workloads' unembedding std (0.001) the plain bar cannot tell them apart
    w_small = bf16_round((rng.standard_normal((V, D)) * 0.001).astype(np.float32)).astype(np.float64)
    l1, _ = oracle.softcap_cross_entropy(f1 @ w_small.T, y, 15.0)
    l2, _ = oracle.softcap_cross_entropy(f2 @ w_small.T, y, 15.0)
    assert rel_l2(l2, l1) < 1e-2
    # with std 0.05 the deviation bar rejects them by a wide margin
    w = bf16_round((rng.standard_normal((V, D)) * 0.05).astype(np.float32)).astype(np.float64)
    l1, _ = oracle.softcap_cross_entropy(f1 @ w.T, y, 15.0)
    l2, _ = oracle.softcap_cross_entropy(f2 @ w.T, y, 15.0)
    e, c = loss_deviation_errors(l2, l1, V)
    assert e > 10 * DEV_REL_L2 and c < DEV_COS
    # and accepts a feature set ~1% (relative) off the right one, the size of
    # the bf16 path's error
    f3 = _unit_rows(f1 + 0.01 * rng.standard_normal((n, D)))
    l3, _ = oracle.softcap_cross_entropy(f3 @ w.T, y, 15.0)
    e, c = loss_deviation_errors(l3, l1, V)
    assert e < DEV_REL_L2 and c >= DEV_COS


def _forward_tok_loss(cfg, params, tokens, targets):
    return oracle.forward_loss(cfg, params, tokens, targets)[1]


@pytest.fixture(scope="module")
def d20_small():
    cfg = get_config("d20", n_layer=2, seq_len=128, batch=1, vocab=4096)
    params = make_params(cfg)
    params["wlm"] = bf16_round((np.random.default_rng(3).standard_normal(params["wlm"].shape)
                                * 0.05).astype(np.float32))
    tokens, targets = make_tokens(cfg)
    return cfg, params, tokens, targets, _forward_tok_loss(cfg, params, tokens, targets)


def _rotary_off(u, cos, sin):
    return u


def _relu_not_squared(u):
    return np.maximum(u, 0.0)


def _no_causal_mask(qn, kn, v):
    T, H, hd = qn.shape
    s = np.einsum("thd,sd->hts", qn, kn) / np.sqrt(hd)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    return np.einsum("hts,sd->thd", p, v)


@pytest.mark.parametrize("name,target,wrong", [
    ("no rotary", "rotary", _rotary_off),
    ("relu instead of relu^2", "relu_squared", _relu_not_squared),
    ("no causal mask", "causal_mqa_attention", _no_causal_mask),
])
def test_planted_forward_mistakes_fail_the_deviation_bar(d20_small, monkeypatch, name, target,
                                                         wrong):
    """A d20-shaped forward (2 layers, 128 positions, V 4096) with one planted
    mistake in the oracle fails the bar against the correct oracle."""
    cfg, params, tokens, targets, right = d20_small
    monkeypatch.setattr(om, target, wrong)
    bad = _forward_tok_loss(cfg, params, tokens, targets)
    e, c = loss_deviation_errors(bad, right, cfg["vocab"])
    assert e > DEV_REL_L2 or c < DEV_COS, (name, e, c)
