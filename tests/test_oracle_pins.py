"""Pins of the oracle against things other than itself.

Every check here is a closed form, an invariant the mathematics fixes, a
library routine (torch CPU float64: rms_norm, scaled_dot_product_attention,
cross_entropy, complex multiplication, autograd), or finite differences.  The
planted-mistake tests at the end patch one oracle function with a plausible
error and assert that some pin then fails.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import model as om
from nc_synth import get_config, make_params, make_tokens

F64 = np.float64


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_rms_and_eps_closed_form():
    u = _rng(1).standard_normal((7, 96)) * 3.0
    y, r = oracle.rms_norm(u, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-13)
    eps = 0.3
    y, r = oracle.rms_norm(u, eps)
    ms = np.mean(u * u, -1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)),
                               np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_rmsnorm_matches_torch():
    u = _rng(2).standard_normal((5, 64))
    y, _ = oracle.rms_norm(u, 1e-6)
    ref = F.rms_norm(torch.from_numpy(u), (64,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_rmsnorm_backward_finite_difference_and_scale_invariance():
    rng = _rng(3)
    u = rng.standard_normal((3, 32))
    dy = rng.standard_normal((3, 32))
    eps = 1e-2
    y, r = oracle.rms_norm(u, eps)
    dx = oracle.rms_norm_backward(dy, y, r)
    h = 1e-6
    fd = np.zeros_like(u)
    for i in range(u.shape[0]):
        for j in range(u.shape[1]):
            up, um = u.copy(), u.copy()
            up[i, j] += h
            um[i, j] -= h
            fd[i, j] = (np.sum(dy * oracle.rms_norm(up, eps)[0])
                        - np.sum(dy * oracle.rms_norm(um, eps)[0])) / (2 * h)
    np.testing.assert_allclose(dx, fd, rtol=1e-7, atol=1e-9)
    # at eps = 0 the norm is scale invariant, so the gradient is orthogonal to u
    y0, r0 = oracle.rms_norm(u, 0.0)
    dx0 = oracle.rms_norm_backward(dy, y0, r0)
    inner = np.sum(dx0 * u, -1) / (np.linalg.norm(dx0, axis=-1) * np.linalg.norm(u, axis=-1))
    assert np.max(np.abs(inner)) < 1e-12


# ----------------------------------------------------------------- rotary
def _rotary_complex(u, T, hd, base):
    """Rotary as complex multiplication: z_i = u_i + 1j*u_{i+hd/2} times
    exp(1j * t * base^(-2i/hd)) (torch complex arithmetic)."""
    half = hd // 2
    t = torch.arange(T, dtype=torch.float64)
    inv = base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64), torch.outer(t, inv))
    ut = torch.from_numpy(u)
    z = torch.complex(ut[..., :half], ut[..., half:]) * rot
    return torch.cat([z.real, z.imag], -1).numpy()


def test_rotary_matches_complex_rotation():
    T, hd = 50, 64
    u = _rng(4).standard_normal((T, hd))
    cos, sin = oracle.rotary_tables(T, hd, 10000.0)
    np.testing.assert_allclose(oracle.rotary(u, cos, sin),
                               _rotary_complex(u, T, hd, 10000.0),
                               rtol=1e-13, atol=1e-13)


def test_rotary_invariants():
    T, hd = 40, 128
    rng = _rng(5)
    u = rng.standard_normal((T, hd))
    w = rng.standard_normal((T, hd))
    cos, sin = oracle.rotary_tables(T, hd, 10000.0)
    ru = oracle.rotary(u, cos, sin)
    # norm preserved, R_0 = I, R^T R = I
    np.testing.assert_allclose(np.linalg.norm(ru, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(ru[0], u[0])
    np.testing.assert_allclose(oracle.rotary_backward(ru, cos, sin), u, rtol=1e-12, atol=1e-13)
    # relative position: <R_t a, R_s b> depends only on t - s
    a, b = u[3], w[5]
    dots = []
    for shift in (0, 7, 20):
        A = np.tile(a, (T, 1))
        Bm = np.tile(b, (T, 1))
        ra = oracle.rotary(A, cos, sin)[10 + shift]
        rb = oracle.rotary(Bm, cos, sin)[4 + shift]
        dots.append(ra @ rb)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)


def test_rotary_commutes_with_norm():
    T, hd = 30, 64
    u = _rng(6).standard_normal((T, hd))
    cos, sin = oracle.rotary_tables(T, hd, 10000.0)
    lhs = oracle.rms_norm(oracle.rotary(u, cos, sin), 1e-6)[0]
    rhs = oracle.rotary(oracle.rms_norm(u, 1e-6)[0], cos, sin)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- attention
def test_attention_matches_sdpa_with_repeated_kv():
    T, H, hd = 37, 3, 16
    rng = _rng(7)
    q = rng.standard_normal((T, H, hd))
    k = rng.standard_normal((T, hd))
    v = rng.standard_normal((T, hd))
    o = oracle.causal_mqa_attention(q, k, v)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k)[None, None].expand(1, H, T, hd)
    vt = torch.from_numpy(v)[None, None].expand(1, H, T, hd)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_first_row_and_uniform_weights():
    T, H, hd = 20, 2, 8
    rng = _rng(8)
    q = rng.standard_normal((T, H, hd))
    k = rng.standard_normal((T, hd))
    v = rng.standard_normal((T, hd))
    o = oracle.causal_mqa_attention(q, k, v)
    for j in range(H):
        np.testing.assert_allclose(o[0, j], v[0], rtol=1e-14)
    o0 = oracle.causal_mqa_attention(q, np.zeros_like(k), v)
    mean = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    for j in range(H):
        np.testing.assert_allclose(o0[:, j], mean, rtol=1e-13)


def test_attention_backward_matches_autograd_sdpa():
    T, H, hd = 29, 3, 16
    rng = _rng(9)
    q = rng.standard_normal((T, H, hd))
    k = rng.standard_normal((T, hd))
    v = rng.standard_normal((T, hd))
    do = rng.standard_normal((T, H, hd))
    dq, dk, dv = oracle.causal_mqa_attention_backward(q, k, v, do)
    qt = torch.from_numpy(q).requires_grad_()
    kt = torch.from_numpy(k).requires_grad_()
    vt = torch.from_numpy(v).requires_grad_()
    o = F.scaled_dot_product_attention(
        qt.permute(1, 0, 2)[None], kt[None, None].expand(1, H, T, hd),
        vt[None, None].expand(1, H, T, hd), is_causal=True)[0].permute(1, 0, 2)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_attention_query_chunking_is_exact(monkeypatch):
    T, H, hd = 70, 2, 8
    rng = _rng(10)
    q, k, v = rng.standard_normal((T, H, hd)), rng.standard_normal((T, hd)), rng.standard_normal((T, hd))
    full = oracle.causal_mqa_attention(q, k, v)
    do = rng.standard_normal((T, H, hd))
    full_b = oracle.causal_mqa_attention_backward(q, k, v, do)
    monkeypatch.setattr(om, "ATTN_QUERY_CHUNK", 16)
    np.testing.assert_allclose(oracle.causal_mqa_attention(q, k, v), full, rtol=1e-14, atol=1e-15)
    # the backward's key-side sums over chunks (run on the thread pool, added
    # in chunk order) equal the single-chunk result
    for a, b in zip(oracle.causal_mqa_attention_backward(q, k, v, do), full_b):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- softcap / CE
def test_embedding_gradient_matches_one_hot_product_and_torch():
    """dW_te of the lookup e_t = W_te[x_t]: the same as the product
    onehot(x)^T de (a matmul, another route to the same sum) and as torch
    autograd through an embedding lookup; ids no token uses get zero rows,
    and the column sums equal those of de."""
    rng = np.random.default_rng(5)
    V, D = 37, 6
    tok = rng.integers(0, 30, (3, 11))          # ids 30..36 never occur
    tok[0, :5] = 7                              # one id several times
    de = rng.standard_normal((3, 11, D))
    got = oracle.embedding_gradient(tok, de, V)
    onehot = np.zeros((tok.size, V))
    onehot[np.arange(tok.size), tok.reshape(-1)] = 1.0
    np.testing.assert_allclose(got, onehot.T @ de.reshape(-1, D), rtol=0, atol=1e-13)
    w = torch.zeros(V, D, dtype=torch.float64, requires_grad=True)
    F.embedding(torch.from_numpy(tok), w).backward(torch.from_numpy(de))
    np.testing.assert_allclose(got, w.grad.numpy(), rtol=0, atol=1e-13)
    assert not got[30:].any()
    np.testing.assert_allclose(got.sum(0), de.reshape(-1, D).sum(0), rtol=1e-13, atol=1e-13)


def test_softcap_bound_and_series():
    s = 15.0
    z = np.linspace(-500, 500, 10001)
    c = oracle.softcap(z, s)
    assert np.all(np.abs(c) <= s)
    small = np.linspace(-0.3, 0.3, 61)
    np.testing.assert_allclose(oracle.softcap(small, s), small - small ** 3 / (3 * s * s),
                               atol=1e-10)


def test_cross_entropy_matches_torch_and_gradient_sums_to_zero():
    rng = _rng(11)
    n, V, s = 9, 300, 15.0
    z = rng.standard_normal((n, V)) * 20
    y = rng.integers(0, V, n)
    loss, dz = oracle.softcap_cross_entropy(z, y, s)
    zt = torch.from_numpy(z).requires_grad_()
    ref = F.cross_entropy(s * torch.tanh(zt / s), torch.from_numpy(y), reduction="none")
    np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-13)
    ref.sum().backward()
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-12, atol=1e-15)
    # dl/dc sums to zero over the vocabulary: divide out the softcap factor
    c = oracle.softcap(z, s)
    dc = dz / (1 - (c / s) ** 2)
    np.testing.assert_allclose(dc.sum(-1), 0.0, atol=1e-12)


# ----------------------------------------------------------------- whole model
def _cfg(name="tiny", **kw):
    return get_config(name, **kw)


def _f64_params(cfg, seed=None, lm_std=None):
    p = make_params(cfg, seed)
    if lm_std is not None:
        rng = np.random.default_rng(123)
        p["wlm"] = (rng.standard_normal(p["wlm"].shape) * lm_std).astype(np.float32)
    return {k: v.astype(F64) for k, v in p.items()}


def _torch_loss(cfg, params, tokens, targets):
    """The model rebuilt from torch library pieces, for autograd."""
    D, H, hd, eps, s = cfg["d_model"], cfg["n_head"], cfg["head_dim"], cfg["rms_eps"], cfg["softcap"]
    B, T = tokens.shape
    tok = torch.from_numpy(tokens.astype(np.int64))
    tgt = torch.from_numpy(targets.astype(np.int64))
    half = hd // 2
    inv = cfg["rope_base"] ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = torch.outer(torch.arange(T, dtype=torch.float64), inv)
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope(u):
        z = torch.complex(u[..., :half], u[..., half:]) * rot
        return torch.cat([z.real, z.imag], -1)

    h = F.rms_norm(F.embedding(tok, params["wte"]), (D,), eps=eps)
    for layer in range(cfg["n_layer"]):
        p = f"h{layer}."
        a = F.rms_norm(h, (D,), eps=eps)
        q = F.linear(a, params[p + "wq"]).view(B, T, H, hd)
        k = F.linear(a, params[p + "wk"]).view(B, T, 1, hd)
        v = F.linear(a, params[p + "wv"]).view(B, T, 1, hd)
        q = F.rms_norm(rope(q), (hd,), eps=eps)
        k = F.rms_norm(rope(k), (hd,), eps=eps)
        o = F.scaled_dot_product_attention(
            q.transpose(1, 2), k.transpose(1, 2).expand(B, H, T, hd),
            v.transpose(1, 2).expand(B, H, T, hd), is_causal=True)
        h = h + F.linear(o.transpose(1, 2).reshape(B, T, H * hd), params[p + "wo"])
        m = F.rms_norm(h, (D,), eps=eps)
        h = h + F.linear(torch.relu(F.linear(m, params[p + "wfc"])).square(), params[p + "wproj"])
    f = F.rms_norm(h, (D,), eps=eps)
    c = s * torch.tanh(F.linear(f, params["wlm"]) / s)
    return F.cross_entropy(c.reshape(B * T, -1), tgt.reshape(-1))


def _torch_grads(cfg, params, tokens, targets):
    pt = {k: torch.from_numpy(np.array(v, dtype=F64)).requires_grad_() for k, v in params.items()}
    loss = _torch_loss(cfg, pt, tokens, targets)
    loss.backward()
    return float(loss), {k: v.grad.numpy() for k, v in pt.items()}


def _rel_l2(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


@pytest.mark.parametrize("variant", ["tiny", "tiny_big_lm", "two_layer_256"])
def test_whole_model_matches_torch_autograd(variant):
    if variant == "two_layer_256":
        cfg = _cfg("tiny", d_model=256, n_head=4, d_mlp=1024, seq_len=128, vocab=700,
                   tokens="zipf")
        params = _f64_params(cfg, lm_std=0.02)
    elif variant == "tiny_big_lm":
        cfg = _cfg("tiny")
        params = _f64_params(cfg, lm_std=0.05)
    else:
        cfg = _cfg("tiny")
        params = _f64_params(cfg)
    tokens, targets = make_tokens(cfg)
    loss, grads = oracle.forward_backward(cfg, params, tokens, targets)
    tloss, tgrads = _torch_grads(cfg, params, tokens, targets)
    assert abs(loss - tloss) <= 1e-12 * abs(tloss)
    for k in params:
        assert _rel_l2(grads[k], tgrads[k]) < 1e-10, k
    l2, tok_loss = oracle.forward_loss(cfg, params, tokens, targets)
    assert abs(l2 - loss) <= 1e-13 * loss
    assert tok_loss.shape == tokens.shape


def _loss_only(cfg, params, tokens, targets):
    return oracle.forward_loss(cfg, params, tokens, targets)[0]


@pytest.mark.parametrize("lm_std", [None, 0.02])
def test_whole_backward_finite_differences(lm_std):
    cfg = _cfg("tiny", seq_len=16, batch=2)
    params = _f64_params(cfg, lm_std=lm_std)
    tokens, targets = make_tokens(cfg)
    _, grads = oracle.forward_backward(cfg, params, tokens, targets)
    rng = np.random.default_rng(99)
    h = 1e-5
    for name, w in params.items():
        g = grads[name]
        flat = np.abs(g).ravel()
        idx = list(np.argsort(flat)[-8:]) + list(rng.integers(0, flat.size, 8))
        for i in idx:
            pos = np.unravel_index(i, w.shape)
            orig = w[pos]
            w[pos] = orig + h
            lp = _loss_only(cfg, params, tokens, targets)
            w[pos] = orig - h
            lm = _loss_only(cfg, params, tokens, targets)
            w[pos] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[pos]) <= 1e-6 * abs(g[pos]) + 1e-9 * max(1.0, np.max(flat)), (name, pos, fd, g[pos])
    # three random directions over all parameters at once
    for d_i in range(3):
        dirs = {k: rng.standard_normal(v.shape) for k, v in params.items()}
        nrm = math.sqrt(sum(float(np.sum(d * d)) for d in dirs.values()))
        dd = sum(float(np.sum(grads[k] * dirs[k])) for k in params) / nrm
        plus = {k: v + h * dirs[k] / nrm for k, v in params.items()}
        minus = {k: v - h * dirs[k] / nrm for k, v in params.items()}
        fd = (_loss_only(cfg, plus, tokens, targets) - _loss_only(cfg, minus, tokens, targets)) / (2 * h)
        assert abs(fd - dd) <= 1e-6 * abs(dd) + 1e-10, (fd, dd)


def test_zero_unembedding_closed_form():
    for name, V in (("tiny", 512), ("tiny", 50257), ("tiny", 65536)):
        cfg = _cfg(name, vocab=V, seq_len=16, batch=2, tokens="zipf")
        params = _f64_params(cfg)
        params["wlm"][:] = 0.0
        tokens, targets = make_tokens(cfg)
        loss, grads = oracle.forward_backward(cfg, params, tokens, targets)
        assert loss == pytest.approx(math.log(V), rel=1e-14)
        for k, g in grads.items():
            if k != "wlm":
                assert np.all(g == 0.0), k
        # dW_lm = (1/N) sum_t (1/V - onehot(y_t)) f_t^T with f the final-norm output
        f = _final_features(cfg, params, tokens)
        N = tokens.size
        onehot = np.zeros((N, V))
        onehot[np.arange(N), targets.reshape(-1)] = 1.0
        expect = (1.0 / V - onehot).T @ f / N
        assert _rel_l2(grads["wlm"], expect) < 1e-12


def _final_features(cfg, params, tokens):
    """Final-norm features via the torch rebuild (independent of the oracle)."""
    D = cfg["d_model"]
    pt = {k: torch.from_numpy(np.array(v, dtype=F64)) for k, v in params.items()}
    captured = {}
    orig = F.linear

    def spy(x, w, *a, **kw):
        if w is pt["wlm"]:
            captured["f"] = x.detach().reshape(-1, D).numpy().copy()
        return orig(x, w, *a, **kw)

    F.linear = spy
    try:
        _torch_loss(cfg, pt, tokens, np.zeros_like(tokens))
    finally:
        F.linear = orig
    return captured["f"]


def test_scale_invariances_at_zero_eps():
    cfg = _cfg("tiny", rms_eps=0.0, seq_len=32)
    params = _f64_params(cfg, lm_std=0.02)
    tokens, targets = make_tokens(cfg)
    _, g = oracle.forward_backward(cfg, params, tokens, targets)
    hd = cfg["head_dim"]

    def cosine(a, b):
        return abs(float(np.sum(a * b))) / (np.linalg.norm(a) * np.linalg.norm(b))

    used = np.unique(tokens)
    for v in used:
        assert cosine(g["wte"][v], params["wte"][v]) < 1e-10
    for layer in range(cfg["n_layer"]):
        p = f"h{layer}."
        for j in range(cfg["n_head"]):
            sl = slice(j * hd, (j + 1) * hd)
            assert cosine(g[p + "wq"][sl], params[p + "wq"][sl]) < 1e-10
        assert cosine(g[p + "wk"], params[p + "wk"]) < 1e-10


def test_causality_bitwise():
    cfg = _cfg("tiny", seq_len=32, batch=1)
    params = _f64_params(cfg, lm_std=0.02)
    tokens, targets = make_tokens(cfg)
    _, base = oracle.forward_loss(cfg, params, tokens, targets)
    t0 = 19
    tok2 = tokens.copy()
    tok2[0, t0] = (tok2[0, t0] + 1) % cfg["vocab"]
    _, pert = oracle.forward_loss(cfg, params, tok2, targets)
    np.testing.assert_array_equal(base[0, :t0], pert[0, :t0])
    assert np.any(base[0, t0:] != pert[0, t0:])


def test_batch_structure():
    cfg = _cfg("tiny", seq_len=16, batch=3)
    params = _f64_params(cfg, lm_std=0.02)
    tokens, targets = make_tokens(cfg)
    loss, g = oracle.forward_backward(cfg, params, tokens, targets)
    perm = [2, 0, 1]
    loss_p, g_p = oracle.forward_backward(cfg, params, tokens[perm], targets[perm])
    assert loss_p == pytest.approx(loss, rel=1e-13)
    for k in g:
        assert _rel_l2(g_p[k], g[k]) < 1e-12
    per = [oracle.forward_backward(cfg, params, tokens[b:b + 1], targets[b:b + 1]) for b in range(3)]
    assert np.mean([p[0] for p in per]) == pytest.approx(loss, rel=1e-13)
    for k in g:
        assert _rel_l2(sum(p[1][k] for p in per) / 3, g[k]) < 1e-12


# ----------------------------------------------------------------- planted mistakes
def _pins_fail(check):
    try:
        check()
    except AssertionError:
        return True
    return False


def test_planted_rotary_sign_error_is_caught(monkeypatch):
    def wrong(u, cos, sin):
        half = u.shape[-1] // 2
        a, b = u[..., :half], u[..., half:]
        return np.concatenate([a * cos + b * sin, -a * sin + b * cos], axis=-1)
    monkeypatch.setattr(oracle, "rotary", wrong)
    assert _pins_fail(test_rotary_matches_complex_rotation)


def test_planted_missing_qk_norm_is_caught(monkeypatch):
    real = om.rms_norm

    def no_qk_norm(u, eps):
        if u.shape[-1] == 64 and u.ndim >= 3:       # head vectors (hd = 64)
            return u, np.ones(u.shape[:-1] + (1,))
        return real(u, eps)
    monkeypatch.setattr(om, "rms_norm", no_qk_norm)
    assert _pins_fail(test_scale_invariances_at_zero_eps)


def test_planted_missing_mask_is_caught(monkeypatch):
    def unmasked(qn, kn, v):
        T, H, hd = qn.shape
        s = np.einsum("thd,sd->hts", qn, kn) / np.sqrt(hd)
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        return np.einsum("hts,sd->thd", p, v)
    monkeypatch.setattr(om, "causal_mqa_attention", unmasked)
    assert _pins_fail(test_causality_bitwise)


def test_planted_backward_errors_are_caught(monkeypatch):
    check = lambda: test_whole_model_matches_torch_autograd("tiny_big_lm")
    # a dropped term in the norm backward
    monkeypatch.setattr(om, "rms_norm_backward", lambda dy, y, r: r * dy)
    assert _pins_fail(check)
    monkeypatch.undo()
    # relu^2 differentiated as if it were relu
    monkeypatch.setattr(om, "relu_squared_backward", lambda dg, u: dg * (u > 0))
    assert _pins_fail(check)
    monkeypatch.undo()
    # the softcap's chain-rule factor (1 - (c/s)^2) dropped
    monkeypatch.setattr(om, "softcap_cross_entropy", _ce_no_cap_factor)
    assert _pins_fail(check)
    monkeypatch.undo()
    # a transposed rotation in the backward (R instead of R^T)
    monkeypatch.setattr(om, "rotary_backward", om.rotary)
    assert _pins_fail(check)


def _ce_no_cap_factor(z, targets, s):
    c = s * np.tanh(z / s)
    m = c.max(-1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(c - m).sum(-1))
    rows = np.arange(z.shape[0])
    dz = np.exp(c - lse[:, None])
    dz[rows, targets] -= 1.0
    return lse - c[rows, targets], dz
