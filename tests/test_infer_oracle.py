"""Pins of the oracle's generation reference, forward_logits: the logits a
KV-cache engine must reproduce position by position."""
import numpy as np
import pytest

import oracle
from nc_synth import get_config, make_params, make_tokens


@pytest.fixture(scope="module")
def small():
    cfg = get_config("tiny", seq_len=64, batch=2)
    params = make_params(cfg)
    params["wlm"] = (np.random.default_rng(5).standard_normal(params["wlm"].shape) * 0.05)
    tokens, targets = make_tokens(cfg)
    return cfg, params, tokens, targets


def test_cross_entropy_of_the_logits_is_the_token_loss(small):
    cfg, params, tokens, targets = small
    c = oracle.forward_logits(cfg, params, tokens)
    _, tl = oracle.forward_loss(cfg, params, tokens, targets)
    m = c.max(-1, keepdims=True)
    lse = m[..., 0] + np.log(np.exp(c - m).sum(-1))
    y = np.take_along_axis(c, targets[..., None], -1)[..., 0]
    np.testing.assert_allclose(lse - y, tl, rtol=1e-13, atol=1e-13)


def test_logits_of_a_prefix_are_the_prefix_positions(small):
    """Causality, the premise of the cache: position t's logits depend on
    tokens 0..t only, so a prefix gives the same logits at its positions."""
    cfg, params, tokens, _ = small
    full = oracle.forward_logits(cfg, params, tokens)
    for t in (0, 1, 17, 40, 63):
        pre = oracle.forward_logits(cfg, params, tokens[:, :t + 1], positions=[t])
        np.testing.assert_allclose(pre[:, 0], full[:, t], rtol=1e-11, atol=1e-12)


def test_logits_bound_positions_and_zero_unembedding(small):
    cfg, params, tokens, _ = small
    c = oracle.forward_logits(cfg, params, tokens)
    assert np.all(np.abs(c) <= cfg["softcap"])
    sel = oracle.forward_logits(cfg, params, tokens, positions=[3, 60])
    np.testing.assert_allclose(sel, c[:, [3, 60]], rtol=1e-13, atol=1e-14)
    p0 = dict(params)
    p0["wlm"] = np.zeros_like(params["wlm"])
    assert not np.any(oracle.forward_logits(cfg, p0, tokens))
