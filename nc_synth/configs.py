"""Model configurations of the nanochat-style dense decoder.

The architecture list of the nanochat article (vpshk.cn page, section on the
hand-written ~8000-line code base) fixes the model family: dense transformer,
rotary positions only, QK-norm, untied embedding/unembedding, a normalised
token embedding, relu^2 MLP, RMSNorm without learnable parameters, no biases,
multi-query attention and a logit softcap.  The five workloads below give the
sizes: a tiny fp32 model, a GPT-2-124M-shaped model (12 layers, 12 heads,
d_model 768, seq 1024, the shape the llm.c article on qian.cx trains, with the
GPT-2 vocabulary of 50257 from the tianqi.csdn.net tokenizer section), the
depth-20 model the speedrun trains (vocabulary 2^16 from the same tokenizer
section), the depth-30 model, and a depth-20 variant at sequence length 8192.

Scalars that the pages leave open are fixed here and used identically by the
oracle and the GPU library: rotary base 10000, softcap 15, RMSNorm epsilon
1e-6, init N(0, 0.02) for every matrix except the unembedding, N(0, 0.001).
"""
from __future__ import annotations

import copy

_COMMON = dict(
    n_kv_head=1,          # multi-query attention: one shared K/V head
    rope_base=10000.0,
    softcap=15.0,
    rms_eps=1e-6,
    init_std=0.02,
    lm_init_std=0.001,
    zipf_s=1.1,
    seed_data=0,
    seed_params=1,
)

CONFIGS = {
    "tiny": dict(n_layer=2, d_model=128, n_head=2, head_dim=64, d_mlp=512,
                 vocab=512, seq_len=64, batch=2, dtype="f32", tokens="uniform"),
    "gpt2": dict(n_layer=12, d_model=768, n_head=12, head_dim=64, d_mlp=3072,
                 vocab=50257, seq_len=1024, batch=16, dtype="bf16", tokens="zipf"),
    "d20": dict(n_layer=20, d_model=1280, n_head=10, head_dim=128, d_mlp=5120,
                vocab=65536, seq_len=2048, batch=32, dtype="bf16", tokens="zipf"),
    "d30": dict(n_layer=30, d_model=1920, n_head=15, head_dim=128, d_mlp=7680,
                vocab=65536, seq_len=2048, batch=16, dtype="bf16", tokens="zipf"),
    "long": dict(n_layer=20, d_model=1280, n_head=10, head_dim=128, d_mlp=5120,
                 vocab=65536, seq_len=8192, batch=8, dtype="bf16", tokens="zipf"),
}
for _c in CONFIGS.values():
    for _k, _v in _COMMON.items():
        _c.setdefault(_k, _v)


def get_config(name: str, **overrides) -> dict:
    """A copy of a named configuration with fields overridden."""
    cfg = copy.deepcopy(CONFIGS[name])
    cfg["name"] = name
    for k, v in overrides.items():
        if k not in cfg:
            raise KeyError(f"unknown config field {k!r}")
        cfg[k] = v
    return cfg


def param_shapes(cfg: dict) -> list[tuple[str, tuple[int, int], float]]:
    """(name, (rows, cols), init std) of every weight matrix, in storage order.

    Every linear layer is stored [out_features, in_features] and has no bias.
    The three attention input projections are listed next to each other so a
    packed layout can treat them as one [(H+2)*hd, D] matrix.
    """
    D, H, hd, F, V = (cfg["d_model"], cfg["n_head"], cfg["head_dim"],
                      cfg["d_mlp"], cfg["vocab"])
    std, lm_std = cfg["init_std"], cfg["lm_init_std"]
    out = [("wte", (V, D), std)]
    for layer in range(cfg["n_layer"]):
        p = f"h{layer}."
        out += [
            (p + "wq", (H * hd, D), std),
            (p + "wk", (hd, D), std),
            (p + "wv", (hd, D), std),
            (p + "wo", (D, H * hd), std),
            (p + "wfc", (F, D), std),
            (p + "wproj", (D, F), std),
        ]
    out.append(("wlm", (V, D), lm_std))
    return out
