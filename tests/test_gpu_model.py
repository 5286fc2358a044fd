"""GPU parity of the whole step (nc_forward_loss / nc_forward_backward) with
the float64 oracle on identical seeded inputs.

Bar: the fp32 configuration matches in loss and every gradient tensor within
1e-4 relative L2; bf16 configurations match the loss within 1e-2 relative and
every gradient tensor within 3e-2 relative L2 with cosine >= 0.999.  The
per-token losses are held to the gradient bar through their deviation from
ln V.
"""
import math

import numpy as np
import pytest

import oracle
from nc_synth import get_config, make_params, make_tokens
from tests.gpu_helpers import cosine, from_dev, loss_deviation_errors, rel_l2, require_gpu

pytestmark = pytest.mark.gpu


def _model(cfg):
    from dense_gpt_pretraining_amd import Model
    return Model(cfg)


def _compare(cfg, params, tokens, targets, loss_tol, grad_tol, cos_min, label):
    torch = require_gpu()
    m = _model(cfg)
    p = m.pack(params)
    loss, grads = m.forward_backward(p, tokens, targets)
    torch.cuda.synchronize()
    g = m.unpack(grads)
    want_loss, want = oracle.forward_backward(cfg, params, tokens, targets)
    got_loss = float(loss.item())
    print(f"[{label}] loss gpu {got_loss:.7f} oracle {want_loss:.7f}")
    assert abs(got_loss - want_loss) <= loss_tol * abs(want_loss)
    worst = []
    for k in want:
        e = rel_l2(g[k], want[k])
        c = cosine(g[k], want[k])
        worst.append((e, k, c))
        assert e < grad_tol, (k, e)
        assert c >= cos_min, (k, c)
    worst.sort(reverse=True)
    print(f"[{label}] worst grads: " + ", ".join(f"{k}:{e:.2e}/cos {c:.6f}" for e, k, c in worst[:4]))
    # forward-only entry points agree with the fused one
    l2 = m.forward_loss(p, tokens, targets)
    l3, tl = m.forward_loss(p, tokens, targets, token_loss=True)
    torch.cuda.synchronize()
    assert abs(float(l2.item()) - got_loss) <= 1e-6 * abs(got_loss)
    assert float(l3.item()) == float(l2.item())
    # per-token losses through their deviation from ln V (the mean loss alone
    # sits near ln V for any finite forward pass at small logits)
    _, want_tl = oracle.forward_loss(cfg, params, tokens, targets)
    e, c = loss_deviation_errors(from_dev(tl), want_tl, cfg["vocab"])
    print(f"[{label}] per-token loss deviation from ln V: rel-L2 {e:.2e} cos {c:.6f}")
    assert e < grad_tol and c >= cos_min, (e, c)
    return m, p, g


def test_tiny_fp32_config():
    cfg = get_config("tiny")
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    _compare(cfg, params, tokens, targets, 1e-4, 1e-4, 0.9999, "tiny f32")


def test_tiny_fp32_large_unembedding():
    # an unembedding of std 0.05 gives the blocks gradients far from zero
    cfg = get_config("tiny")
    params = make_params(cfg)
    params["wlm"] = (np.random.default_rng(7).standard_normal(params["wlm"].shape) * 0.05
                     ).astype(np.float32)
    tokens, targets = make_tokens(cfg)
    _compare(cfg, params, tokens, targets, 1e-4, 1e-4, 0.9999, "tiny f32 lm0.05")


@pytest.mark.parametrize("name,over", [
    ("gpt2", dict(n_layer=2, seq_len=256, batch=2)),
    ("d20", dict(n_layer=2, seq_len=128, batch=2)),
    ("d30", dict(n_layer=2, seq_len=128, batch=1)),
])
def test_bf16_reduced_depth(name, over):
    cfg = get_config(name, **over)
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    _compare(cfg, params, tokens, targets, 1e-2, 3e-2, 0.999, f"{name} {over}")


def test_bf16_large_unembedding():
    cfg = get_config("gpt2", n_layer=3, seq_len=128, batch=2)
    params = make_params(cfg)
    from nc_synth import bf16_round
    params["wlm"] = bf16_round((np.random.default_rng(8).standard_normal(params["wlm"].shape)
                                * 0.05).astype(np.float32))
    tokens, targets = make_tokens(cfg)
    _compare(cfg, params, tokens, targets, 1e-2, 3e-2, 0.999, "gpt2 lm0.05")


def test_zero_unembedding_closed_form_on_gpu():
    torch = require_gpu()
    cfg = get_config("gpt2", n_layer=2, seq_len=128, batch=2)
    params = make_params(cfg)
    params["wlm"][:] = 0.0
    tokens, targets = make_tokens(cfg)
    m = _model(cfg)
    loss, grads = m.forward_backward(m.pack(params), tokens, targets)
    torch.cuda.synchronize()
    assert float(loss.item()) == pytest.approx(math.log(cfg["vocab"]), rel=1e-6)
    g = m.unpack(grads)
    for k, v in g.items():
        if k != "wlm":
            assert np.all(v == 0.0), k


def test_determinism_and_overwrite():
    torch = require_gpu()
    cfg = get_config("d20", n_layer=1, seq_len=128, batch=2)
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    m = _model(cfg)
    p = m.pack(params)
    g1 = torch.full((m.n_params,), 7.0, dtype=torch.float32, device="cuda")
    g2 = torch.full((m.n_params,), -3.0, dtype=torch.float32, device="cuda")
    l1, _ = m.forward_backward(p, tokens, targets, grads=g1)
    l2, _ = m.forward_backward(p, tokens, targets, grads=g2)
    torch.cuda.synchronize()
    assert float(l1.item()) == float(l2.item())
    a, b = m.unpack(g1), m.unpack(g2)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_causality_on_gpu():
    torch = require_gpu()
    cfg = get_config("gpt2", n_layer=2, seq_len=128, batch=1)
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    m = _model(cfg)
    p = m.pack(params)
    _, tl0 = m.forward_loss(p, tokens, targets, token_loss=True)
    tok2 = tokens.copy()
    t0 = 77
    tok2[0, t0] = (tok2[0, t0] + 1) % cfg["vocab"]
    _, tl1 = m.forward_loss(p, tok2, targets, token_loss=True)
    torch.cuda.synchronize()
    a, b = tl0.cpu().numpy(), tl1.cpu().numpy()
    np.testing.assert_array_equal(a[0, :t0], b[0, :t0])
    assert np.any(a[0, t0:] != b[0, t0:])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("over", [
    # one query head (MQA degenerates to single-head attention), the shortest
    # sequence the bf16 kernels take, a vocabulary off the 256-column padding
    dict(n_layer=1, d_model=64, n_head=1, head_dim=64, d_mlp=256, vocab=300, seq_len=64,
         batch=1),
    # heads whose QKV width (H + 2) hd = 576 is no multiple of the 256-wide tile, d_model
    # != H hd, odd batch, vocabulary just past a padding multiple
    dict(n_layer=2, d_model=192, n_head=7, head_dim=64, d_mlp=320, vocab=513, seq_len=128,
         batch=3),
])
def test_degenerate_and_ragged_shapes(dtype, over):
    """Shapes the method allows but the named configurations never reach:
    a single query head, d_model different from H hd, ragged GEMM tiles in
    every product and a padded vocabulary, at fp32 and bf16, against the
    oracle with the unembedding at std 0.05 so the blocks' gradients matter."""
    cfg = get_config("tiny", dtype=dtype, **over)
    params = make_params(cfg)
    w = np.random.default_rng(11).standard_normal(params["wlm"].shape).astype(np.float32) * 0.05
    if dtype == "bf16":
        from nc_synth import bf16_round
        w = bf16_round(w)
    params["wlm"] = w
    tokens, targets = make_tokens(cfg)
    tol = (1e-4, 1e-4, 0.9999) if dtype == "f32" else (1e-2, 3e-2, 0.999)
    _compare(cfg, params, tokens, targets, *tol, f"{dtype} {over['n_head']}x{over['head_dim']}")
