"""The activation-recompute step (nc_forward_backward_recompute) against the
step that keeps every layer's tensors: the same kernels on the same inputs,
so the loss and every gradient must agree bit for bit; and against the oracle
through that equality.  Its workspace must be the smaller one."""
import numpy as np
import pytest

from nc_synth import get_config, make_params, make_tokens
from tests.gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def _both(cfg, params=None, device_init=False):
    from dense_gpt_pretraining_amd import Model
    torch = require_gpu()
    m = Model(cfg)
    p = m.init_params(cfg["seed_params"]) if device_init else m.pack(params)
    tokens, targets = make_tokens(cfg)
    l1, g1 = m.forward_backward(p, tokens, targets)
    torch.cuda.synchronize()
    m.free_workspaces()
    l2, g2 = m.forward_backward(p, tokens, targets, recompute=True)
    torch.cuda.synchronize()
    return m, l1, g1, l2, g2


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("d20", dict(n_layer=3, seq_len=256, batch=2)),
    ("gpt2", dict(n_layer=3, seq_len=128, batch=4)),
])
def test_recompute_is_bitwise_the_stored_step(name, over):
    from dense_gpt_pretraining_amd import binding as b
    torch = require_gpu()
    cfg = get_config(name, **over)
    m, l1, g1, l2, g2 = _both(cfg, make_params(cfg))
    assert float(l1.item()) == float(l2.item())
    for t, off, r, c in m.layout:
        assert bool(torch.equal(g1[off:off + r * c], g2[off:off + r * c])), t
    assert b.nc_workspace_size_recompute(m.c) < b.nc_workspace_size(m.c, True)


@pytest.mark.timeout(600)
def test_recompute_at_full_d20_size():
    """The d20 step in the benchmark's launch configuration."""
    torch = require_gpu()
    cfg = get_config("d20")
    m, l1, g1, l2, g2 = _both(cfg, device_init=True)
    assert float(l1.item()) == float(l2.item())
    # every parameter tensor (padding excluded) agrees bit for bit
    for name, off, r, c in m.layout:
        assert bool(torch.equal(g1[off:off + r * c], g2[off:off + r * c])), name
