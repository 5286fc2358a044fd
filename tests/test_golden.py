"""The oracle against the stored fixtures under tests/golden/."""
import math
import os

import numpy as np
import pytest

import oracle
from nc_synth import get_config, make_params, make_tokens

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


@pytest.mark.parametrize("vocab,lnv", [(int(a), float(b)) for a, b in _rows("zero_unembedding_loss.txt")])
def test_zero_unembedding_loss_is_ln_vocab(vocab, lnv):
    assert lnv == math.log(vocab)
    cfg = get_config("tiny", vocab=vocab, seq_len=8, batch=1, tokens="zipf")
    params = make_params(cfg)
    params["wlm"][:] = 0.0
    tokens, targets = make_tokens(cfg)
    loss, _ = oracle.forward_loss(cfg, params, tokens, targets)
    assert loss == pytest.approx(lnv, rel=1e-14)


def test_oracle_matches_its_stored_tiny_run():
    rows = _rows("oracle_tiny.txt")
    cfg = get_config("tiny")
    loss, grads = oracle.forward_backward(cfg, make_params(cfg), *make_tokens(cfg))
    for r in rows:
        if r[0] == "loss":
            assert loss == pytest.approx(float(r[1]), rel=1e-12)
        else:
            assert float(np.linalg.norm(grads[r[1]])) == pytest.approx(float(r[2]), rel=1e-10)
