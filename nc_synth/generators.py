"""Seeded generators for parameters and token batches.

Everything is drawn with NumPy's PCG64 so the same seed gives the same arrays
on every machine.  Nothing here computes any part of the model.

Token ids.  The pages train on FineWeb / FineWeb-EDU text (llm.c article on
qian.cx; tokenizer section of the tianqi.csdn.net article).  Those corpora are
not used; a finite Zipf law with exponent 1.1 over the vocabulary stands in for
their heavy-headed unigram statistics: P(id = k-1) is proportional to k^-1.1
for k = 1..V, drawn by inverse-CDF sampling.  Each row is a stream of T+1 ids;
tokens are the first T, targets the last T (next-token prediction).
"""
from __future__ import annotations

import numpy as np

from .configs import param_shapes


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs are finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


def make_params(cfg: dict, seed: int | None = None) -> dict[str, np.ndarray]:
    """Every weight matrix as a float32 array, keyed by name.

    Matrix i is drawn from its own PCG64 stream seeded with (seed, i), so a
    single matrix can be regenerated without drawing the others.  For bf16
    configurations the values are rounded to bfloat16, so the GPU (which
    stores bf16) and the oracle (which upcasts) see identical numbers.
    """
    seed = cfg["seed_params"] if seed is None else seed
    out = {}
    for i, (name, shape, std) in enumerate(param_shapes(cfg)):
        rng = np.random.Generator(np.random.PCG64([seed, i]))
        w = rng.standard_normal(shape, dtype=np.float32)
        w *= np.float32(std)
        if cfg["dtype"] == "bf16":
            w = bf16_round(w)
        out[name] = w
    return out


def zipf_probs(vocab: int, s: float) -> np.ndarray:
    """Finite Zipf probabilities over ids 0..V-1 (id = rank - 1), float64."""
    k = np.arange(1, vocab + 1, dtype=np.float64)
    w = k ** (-s)
    return w / w.sum()


def make_tokens(cfg: dict, seed: int | None = None, batch: int | None = None
                ) -> tuple[np.ndarray, np.ndarray]:
    """(tokens, targets), each int32 [batch, seq_len].

    Uniform ids for configurations marked "uniform", Zipf(s) otherwise.
    """
    seed = cfg["seed_data"] if seed is None else seed
    B = cfg["batch"] if batch is None else batch
    T, V = cfg["seq_len"], cfg["vocab"]
    rng = np.random.Generator(np.random.PCG64([seed, 0x70C]))
    if cfg["tokens"] == "uniform":
        stream = rng.integers(0, V, size=(B, T + 1), dtype=np.int64)
    else:
        cdf = np.cumsum(zipf_probs(V, cfg["zipf_s"]))
        cdf[-1] = 1.0
        u = rng.random((B, T + 1))
        stream = np.searchsorted(cdf, u, side="right")
        np.minimum(stream, V - 1, out=stream)
    stream = stream.astype(np.int32)
    return (np.ascontiguousarray(stream[:, :T]),
            np.ascontiguousarray(stream[:, 1:]))
