"""Pins of the optimizer oracle (oracle/optim.py) against what its published
definitions and the mathematics fix: an independent AdamW implementation
(torch.optim.AdamW in float64), closed forms of Adam's bias correction and of
decoupled weight decay, the Newton-Schulz map through the singular value
decomposition, the momentum recursions unrolled by hand, the schedule's
closed-form values, and gradient accumulation against the loss's own batch
structure.  Planted mistakes in the oracle must fail a pin."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.optim as oo
from nc_synth import get_config, make_params, make_tokens


def _rng(s):
    return np.random.default_rng(s)


# ----------------------------------------------------------------- AdamW
def test_adamw_matches_torch_adamw_float64():
    rng = _rng(1)
    theta0 = rng.standard_normal((7, 5))
    grads = [rng.standard_normal((7, 5)) for _ in range(4)]
    lr, b1, b2, eps, wd = 3e-3, 0.8, 0.95, 1e-8, 0.1
    p = torch.nn.Parameter(torch.tensor(theta0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    th, m, v = theta0, np.zeros_like(theta0), np.zeros_like(theta0)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, m, v = oo.adamw(th, g, m, v, t, lr, b1, b2, eps, wd)
        np.testing.assert_allclose(th, p.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_first_step_moves_every_weight_by_lr():
    """t = 1, eps = 0, no decay: m_hat = g and v_hat = g^2, so the step is
    exactly -lr sign(g)."""
    g = _rng(2).standard_normal(100)
    th, _, _ = oo.adamw(np.zeros(100), g, np.zeros(100), np.zeros(100), 1, 0.01, 0.9, 0.999,
                        0.0, 0.0)
    np.testing.assert_allclose(th, -0.01 * np.sign(g), rtol=1e-15)


def test_adamw_bias_correction_with_a_constant_gradient():
    """With the same gradient at every step the corrected moments are exactly
    g and g^2 at every t, so every step is -lr g / (|g| + eps)."""
    g = _rng(3).standard_normal(50)
    th, m, v = np.zeros(50), np.zeros(50), np.zeros(50)
    lr, eps = 1e-3, 1e-3
    for t in range(1, 8):
        prev = th
        th, m, v = oo.adamw(th, g, m, v, t, lr, 0.9, 0.99, eps, 0.0)
        np.testing.assert_allclose(th - prev, -lr * g / (np.abs(g) + eps), rtol=1e-10, atol=1e-16)


def test_adamw_weight_decay_acts_on_theta_alone():
    """A zero gradient leaves the moments at zero; decoupled decay then gives
    theta_t = theta_0 (1 - lr wd)^t."""
    th0 = _rng(4).standard_normal(30)
    th, m, v = th0, np.zeros(30), np.zeros(30)
    lr, wd = 0.05, 0.2
    for t in range(1, 6):
        th, m, v = oo.adamw(th, np.zeros(30), m, v, t, lr, 0.9, 0.95, 1e-8, wd)
    np.testing.assert_allclose(th, th0 * (1 - lr * wd) ** 5, rtol=1e-14)
    assert not np.any(m) and not np.any(v)


# ----------------------------------------------------------------- Newton-Schulz
def _ns_by_svd(G, steps=5, eps=1e-7):
    """X0 = G/(|G|+eps) has singular values s; each iteration maps every
    singular value through p(x) = a x + b x^3 + c x^5 and keeps the singular
    vectors, so the result is U p^(steps)(s) V^T."""
    a, b, c = oo.NS_COEFFS
    U, s, Vt = np.linalg.svd(np.asarray(G, dtype=np.float64), full_matrices=False)
    s = s / (np.linalg.norm(G) + eps)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


@pytest.mark.parametrize("shape", [(24, 24), (8, 40), (40, 8), (16, 33)])
def test_newton_schulz_equals_the_singular_value_map(shape):
    G = _rng(5).standard_normal(shape)
    np.testing.assert_allclose(oo.newton_schulz(G), _ns_by_svd(G), rtol=1e-9, atol=1e-11)


def test_newton_schulz_orientation_and_output_spectrum():
    G = _rng(6).standard_normal((12, 64))
    np.testing.assert_allclose(oo.newton_schulz(G.T), oo.newton_schulz(G).T, rtol=1e-13,
                               atol=1e-15)
    # a wide Gaussian matrix has every normalised singular value far from 0,
    # and five iterations bring each into the band the coefficients aim at
    s = np.linalg.svd(oo.newton_schulz(G), compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.25


# ----------------------------------------------------------------- Muon
def test_muon_without_momentum_is_the_scaled_orthogonalised_gradient():
    rng = _rng(7)
    th0, g = rng.standard_normal((20, 8)), rng.standard_normal((20, 8))
    th, buf = oo.muon(th0, g, np.zeros_like(g), 0.02, 0.0, True, 5, 0.0)
    np.testing.assert_allclose(th, th0 - 0.02 * math.sqrt(20 / 8) * _ns_by_svd(g), rtol=1e-9,
                               atol=1e-11)
    np.testing.assert_array_equal(buf, g)


@pytest.mark.parametrize("nesterov", [True, False])
def test_muon_momentum_unrolled_over_two_steps(nesterov):
    rng = _rng(8)
    th0 = rng.standard_normal((6, 10))
    g1, g2 = rng.standard_normal((6, 10)), rng.standard_normal((6, 10))
    mu, lr, wd = 0.9, 0.01, 0.05
    th, buf = oo.muon(th0, g1, np.zeros_like(g1), lr, mu, nesterov, 5, wd)
    th, buf = oo.muon(th, g2, buf, lr, mu, nesterov, 5, wd)
    b2 = mu * g1 + g2
    u1 = g1 + mu * g1 if nesterov else g1
    u2 = g2 + mu * b2 if nesterov else b2
    want = (th0 * (1 - lr * wd) - lr * _ns_by_svd(u1)) * (1 - lr * wd) - lr * _ns_by_svd(u2)
    np.testing.assert_allclose(buf, b2, rtol=1e-15)
    np.testing.assert_allclose(th, want, rtol=1e-9, atol=1e-11)


# ----------------------------------------------------------------- schedule, accumulation, clipping
def test_lr_schedule_closed_form_values():
    f = 0.1
    assert oo.lr_multiplier(0, 100, 10, f) == pytest.approx(0.1, rel=1e-15)
    assert oo.lr_multiplier(9, 100, 10, f) == 1.0
    assert oo.lr_multiplier(10, 100, 10, f) == 1.0
    assert oo.lr_multiplier(55, 100, 10, f) == pytest.approx(f + (1 - f) * 0.5, rel=1e-14)
    assert oo.lr_multiplier(100, 100, 10, f) == f
    assert oo.lr_multiplier(250, 100, 10, f) == f
    m = [oo.lr_multiplier(s, 100, 10, f) for s in range(10, 101)]
    assert all(a >= b for a, b in zip(m, m[1:]))
    assert oo.lr_multiplier(0, 50, 0, 0.0) == 1.0


def test_accumulated_micro_batch_gradients_equal_the_batch_gradient():
    """The loss is a mean over tokens, so with equal micro-batches the mean of
    their gradients is the gradient of the whole batch."""
    cfg = get_config("tiny", batch=4)
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    _, full = oracle.forward_backward(cfg, params, tokens, targets)
    micro = [oracle.forward_backward(get_config("tiny", batch=2), params, tokens[i:i + 2],
                                     targets[i:i + 2])[1] for i in (0, 2)]
    acc = oo.accumulate(micro)
    for k in full:
        np.testing.assert_allclose(acc[k], full[k], rtol=1e-10, atol=1e-15)


def test_clipping_brings_the_norm_to_the_bound():
    rng = _rng(9)
    g = {"a": rng.standard_normal((5, 3)), "b": rng.standard_normal(7)}
    n = oo.global_norm(g)
    assert n == pytest.approx(math.sqrt(sum(float((x ** 2).sum()) for x in g.values())),
                              rel=1e-15)
    s = oo.clip_scale(n, 0.5)
    assert oo.global_norm({k: v * s for k, v in g.items()}) == pytest.approx(0.5, rel=1e-5)
    assert oo.clip_scale(n, 10 * n) == 1.0 and oo.clip_scale(n, 0.0) == 1.0


def test_step_applies_the_parameter_split():
    """wte and wlm move by AdamW, block matrices by Muon, each from its own
    state, and the returned norm is the global norm before clipping."""
    cfg = get_config("tiny")
    params = make_params(cfg)
    rng = _rng(10)
    grads = {k: rng.standard_normal(v.shape) for k, v in params.items()}
    oc = dict(adam_lr=1e-3, adam_beta1=0.8, adam_beta2=0.95, adam_eps=1e-10,
              adam_weight_decay=0.0, muon_lr=0.02, muon_momentum=0.95, muon_nesterov=1,
              muon_ns_steps=5, muon_weight_decay=0.0, grad_clip=1.0)
    st = oo.init_state(params)
    norm = oo.step(oc, st, grads, 1, 0.5)
    assert norm == pytest.approx(oo.global_norm(grads), rel=1e-15)
    s = 1.0 / (norm + 1e-6)
    want_te, _, _ = oo.adamw(params["wte"], grads["wte"] * s, 0, 0, 1, 5e-4, 0.8, 0.95, 1e-10,
                             0.0)
    np.testing.assert_allclose(st["master"]["wte"], want_te, rtol=1e-13)
    want_q, _ = oo.muon(params["h1.wq"], grads["h1.wq"] * s, 0, 0.01, 0.95, True, 5, 0.0)
    np.testing.assert_allclose(st["master"]["h1.wq"], want_q, rtol=1e-12, atol=1e-15)
    assert set(st["m"]) == {"wte", "wlm"} and "wte" not in st["buf"]


# ----------------------------------------------------------------- planted mistakes
def _fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def test_planted_optimizer_mistakes_are_caught(monkeypatch):
    # a wrong sign of one coefficient inside the iteration
    monkeypatch.setattr(oo, "newton_schulz", _wrong_ns)
    assert _fails(test_newton_schulz_equals_the_singular_value_map, (24, 24))
    monkeypatch.undo()
    # a sign flipped in the published coefficients: the spectrum leaves the band
    for coeffs in ((3.4445, 4.7750, 2.0315), (-3.4445, -4.7750, 2.0315),
                   (3.4445, -4.7750, -2.0315)):
        monkeypatch.setattr(oo, "NS_COEFFS", coeffs)
        assert _fails(test_newton_schulz_orientation_and_output_spectrum), coeffs
    monkeypatch.undo()
    # Adam without bias correction
    monkeypatch.setattr(oo, "adamw", _adamw_no_correction)
    assert _fails(test_adamw_bias_correction_with_a_constant_gradient)
    assert _fails(test_adamw_matches_torch_adamw_float64)
    monkeypatch.undo()
    # weight decay coupled into the gradient (L2 regularisation, not AdamW)
    monkeypatch.setattr(oo, "adamw", _adam_l2)
    assert _fails(test_adamw_weight_decay_acts_on_theta_alone)


def _wrong_ns(G, steps=5, eps=1e-7):
    a, b, c = 3.4445, 4.7750, 2.0315
    X = np.asarray(G, dtype=np.float64) / (np.linalg.norm(G) + eps)
    tall = X.shape[0] > X.shape[1]
    X = X.T if tall else X
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * A @ A) @ X
    return X.T if tall else X


def _adamw_no_correction(theta, g, m, v, t, lr, b1, b2, eps, wd):
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    return theta * (1 - lr * wd) - lr * m / (np.sqrt(v) + eps), m, v


def _adam_l2(theta, g, m, v, t, lr, b1, b2, eps, wd):
    g = g + wd * theta
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    return theta - lr * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + eps), m, v


def test_stored_training_curves_are_the_oracle_s():
    """tests/golden/training_curves.json (the GPU training-loop test's
    reference) holds what the oracle computes: the tiny run is recomputed
    here in full; both runs start at the loss of an all-but-zero unembedding
    (std 0.001), within 1e-2 of ln V, and fall to a few percent of it."""
    import json
    import math
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "training_curves.json")) as f:
        cur = json.load(f)
    for r in cur["runs"]:
        V = get_config(r["config"], **r["over"])["vocab"]
        assert abs(r["losses"][0] - math.log(V)) < 1e-2
        assert r["losses"][-1] < 0.05 * r["losses"][0]
    r = cur["runs"][0]
    assert r["config"] == "tiny"
    cfg = get_config("tiny")
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    st = oo.init_state(params)
    for t in range(1, r["steps"] + 1):
        loss, grads = oracle.forward_backward(cfg, {k: st["master"][k] for k in params}, tokens,
                                              targets)
        assert loss == pytest.approx(r["losses"][t - 1], rel=1e-12, abs=1e-12)
        oo.step(cur["optimizer"], st, grads, t,
                oo.lr_multiplier(t - 1, r["steps"], cur["warmup"], cur["final_frac"]))
