"""GPU parity of generation with the KV cache (include/nc_infer.h) against the
oracle's logits at the same positions (oracle.forward_logits over the whole
sequence, which causality makes equal to generating it position by
position).

Bars: fp32 logits within 1e-4 relative L2 per position; bf16 within 3e-2
relative L2 with cosine >= 0.999 (the bf16 bar of the training step; the
unembedding is drawn with std 0.05 so that the logits reflect the features).
"""
import numpy as np
import pytest

import oracle
from nc_synth import bf16_round, get_config, make_params, make_tokens
from tests.gpu_helpers import cosine, from_dev, rel_l2, require_gpu

pytestmark = pytest.mark.gpu


def _setup(cfg, seq, lm_std=0.05):
    from dense_gpt_pretraining_amd import Model
    params = make_params(cfg)
    w = np.random.default_rng(9).standard_normal(params["wlm"].shape).astype(np.float32) * lm_std
    params["wlm"] = bf16_round(w) if cfg["dtype"] == "bf16" else w
    tokens, _ = make_tokens(cfg, batch=cfg["batch"])
    # a longer stream than the configuration's sequence, when asked
    if seq > tokens.shape[1]:
        tokens = make_tokens(get_config(cfg["name"], seq_len=seq), batch=cfg["batch"])[0]
    m = Model(cfg)
    return m, m.pack(params), params, tokens[:, :seq]


def _check(got, want, fp32, label):
    if fp32:
        e = rel_l2(got, want)
        assert e < 1e-4, (label, e)
        return e, 1.0
    e, c = rel_l2(got, want), cosine(got, want)
    assert e < 3e-2 and c >= 0.999, (label, e, c)
    return e, c


@pytest.mark.parametrize("name,over,t0,seq", [
    ("tiny", dict(batch=2), 64, 128),
    ("d20", dict(n_layer=2, batch=4), 128, 320),
    ("gpt2", dict(n_layer=2, batch=3), 192, 256),
])
def test_prefill_then_decode_matches_the_oracle(name, over, t0, seq):
    from dense_gpt_pretraining_amd import Generator
    torch = require_gpu()
    cfg = get_config(name, **over)
    fp32 = cfg["dtype"] == "f32"
    m, p, params, tokens = _setup(cfg, seq)
    want = oracle.forward_logits(get_config(name, **{**over, "seq_len": seq}), params, tokens,
                                 positions=list(range(t0 - 1, seq)))
    gen = Generator(m, max_seq=seq + 64, max_prefill=t0)
    got = from_dev(gen.prefill(p, tokens[:, :t0]))
    worst = [_check(got, want[:, 0], fp32, "prefill")]
    for pos in range(t0, seq):
        got = from_dev(gen.decode(p, tokens[:, pos], pos))
        worst.append(_check(got, want[:, pos - t0 + 1], fp32, f"decode {pos}"))
    torch.cuda.synchronize()
    e = max(w[0] for w in worst)
    print(f"[{name} {over}] prefill {t0} + decode to {seq}: worst logits rel-L2 {e:.2e}")


def test_decode_from_an_empty_cache():
    """Every position by decode steps alone (no prefill), bf16, hd 128."""
    from dense_gpt_pretraining_amd import Generator
    require_gpu()
    cfg = get_config("d30", n_layer=2, batch=2)
    m, p, params, tokens = _setup(cfg, 40)
    want = oracle.forward_logits(get_config("d30", n_layer=2, batch=2, seq_len=40), params,
                                 tokens)
    gen = Generator(m, max_seq=40)
    for pos in range(40):
        got = from_dev(gen.decode(p, tokens[:, pos], pos))
        _check(got, want[:, pos], False, f"decode {pos}")


@pytest.mark.timeout(900)
def test_generation_at_the_d20_workload_shape():
    """d20 with its batch of 32 sequences: prefill 1984 positions, decode the
    last 64 of the 2048; the oracle runs the last sequence's 2048 positions
    and every decoded position of it is compared."""
    from dense_gpt_pretraining_amd import Generator
    torch = require_gpu()
    cfg = get_config("d20")
    m, p, params, tokens = _setup(cfg, 2048)
    gen = Generator(m, max_seq=2048, max_prefill=1984)
    gen.prefill(p, tokens[:, :1984])
    got = []
    for pos in range(1984, 2048):
        got.append(from_dev(gen.decode(p, tokens[:, pos], pos))[-1])
    torch.cuda.synchronize()
    b = cfg["batch"] - 1
    print("[d20 generation] gpu done; oracle forward of the last sequence", flush=True)
    want = oracle.forward_logits(get_config("d20", batch=1), params, tokens[b:b + 1],
                                 positions=list(range(1984, 2048)))[0]
    errs = [_check(g, w, False, f"decode {1984 + i}") for i, (g, w) in enumerate(zip(got, want))]
    print(f"[d20 generation] 64 decoded positions: worst logits rel-L2 "
          f"{max(e for e, _ in errs):.2e}, lowest cosine {min(c for _, c in errs):.6f}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_generation_on_small_ragged_shapes(dtype):
    """Prefill then decode on shapes whose products are too small to split
    over k, so bf16 decode takes its unfused path (separate rotary / QK-norm
    and RMS kernels; the named configurations all take the fused one), with
    one query head and a padded vocabulary; and a seven-head model with
    d_model != H hd."""
    from dense_gpt_pretraining_amd import Generator
    require_gpu()
    for over in (dict(n_layer=1, d_model=64, n_head=1, head_dim=64, d_mlp=256, vocab=300,
                      batch=2),
                 dict(n_layer=2, d_model=192, n_head=7, head_dim=64, d_mlp=320, vocab=513,
                      batch=3)):
        from dense_gpt_pretraining_amd import Model
        cfg = get_config("tiny", dtype=dtype, seq_len=64, **over)
        cfg96 = get_config("tiny", dtype=dtype, seq_len=96, **over)
        params = make_params(cfg)
        w = np.random.default_rng(9).standard_normal(params["wlm"].shape).astype(np.float32)
        params["wlm"] = bf16_round(w * 0.05) if dtype == "bf16" else w * 0.05
        tokens = make_tokens(cfg96, batch=cfg["batch"])[0]
        m = Model(cfg)
        p = m.pack(params)
        want = oracle.forward_logits(cfg96, params, tokens, positions=list(range(63, 96)))
        gen = Generator(m, max_seq=100, max_prefill=64)
        _check(from_dev(gen.prefill(p, tokens[:, :64])), want[:, 0], dtype == "f32", "prefill")
        for pos in range(64, 96):
            got = from_dev(gen.decode(p, tokens[:, pos], pos))
            _check(got, want[:, pos - 63], dtype == "f32", f"decode {pos}")
