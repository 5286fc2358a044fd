"""Oracle of the optimizer step: plain float64 NumPy.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
CPU-baseline leg of the benchmark may import this module.  The GPU library
neither imports nor links it and shares no code with it.

What the pages fix: the nanochat article on vpshk.cn (section on the
hand-written ~8000-line code base, optimizer paragraph) names the optimizer as
Muon combined with AdamW, after modded-nanoGPT; the llm.c article on qian.cx
(training-command paragraph) configures gradient accumulation, a learning-rate
schedule after GPT-3's, and weight decay, and reports the gradient norm.  The
pages define none of these, so each follows its published definition:

* AdamW: Adam's moment estimates with bias correction (Kingma & Ba, ICLR 2015)
  and weight decay decoupled from the gradient step (Loshchilov & Hutter,
  ICLR 2019), the decay applied as theta <- theta (1 - lr wd) before the
  Adam step;
* Muon (K. Jordan et al., "Muon: an optimizer for hidden layers in neural
  networks", 2024): a momentum buffer B <- mu B + G, the Nesterov form
  G + mu B (or B itself), orthogonalised by five iterations of a quintic
  Newton-Schulz map X <- a X + (b A + c A^2) X with A = X X^T and
  (a, b, c) = (3.4445, -4.7750, 2.0315), started from the matrix divided by
  its Frobenius norm and run on the orientation whose Gram matrix is the
  smaller one; the step is -lr * sqrt(max(1, rows / cols)) times the result.
  Muon is stated for the 2-D weights of hidden layers; the embedding and the
  unembedding take AdamW (the same split modded-nanoGPT makes);
* the schedule: linear warm-up, then cosine decay to a final fraction of the
  peak (GPT-3's schedule decays to 10 percent);
* gradient accumulation: the mean of the micro-batch gradients;
* gradient clipping by the global L2 norm.

Parity unpinned: the choice of these published forms and of the parameter
split (the pages name the optimizers and nothing more).
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64

# quintic Newton-Schulz coefficients of the published Muon iteration
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def lr_multiplier(step: int, total: int, warmup: int, final_frac: float) -> float:
    """Learning-rate multiplier of (0-based) step `step` of `total`: linear
    warm-up over `warmup` steps ((step+1)/warmup), then a cosine from 1 down
    to final_frac at step `total`; final_frac after that."""
    if step < warmup:
        return (step + 1) / warmup
    if step >= total:
        return final_frac
    p = (step - warmup) / max(1, total - warmup)
    return final_frac + (1.0 - final_frac) * 0.5 * (1.0 + math.cos(math.pi * p))


def accumulate(micro_grads: list[dict]) -> dict:
    """Gradient of the mean loss over micro-batches: the mean of their
    gradients (every micro-batch has the same number of tokens)."""
    n = len(micro_grads)
    return {k: sum(np.asarray(g[k], dtype=F64) for g in micro_grads) / n for k in micro_grads[0]}


def global_norm(grads: dict) -> float:
    """L2 norm over every gradient element."""
    return math.sqrt(sum(float(np.sum(np.asarray(g, dtype=F64) ** 2)) for g in grads.values()))


def clip_scale(norm: float, max_norm: float) -> float:
    """Factor that brings a gradient of global norm `norm` to at most
    `max_norm` (1 when clipping is off, max_norm <= 0)."""
    if max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + 1e-6))


def adamw(theta, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float,
          wd: float):
    """One AdamW step at step number t >= 1.  Returns (theta, m, v)."""
    theta = np.asarray(theta, dtype=F64)
    g = np.asarray(g, dtype=F64)
    m = beta1 * np.asarray(m, dtype=F64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=F64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    theta = theta * (1.0 - lr * wd) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta, m, v


def newton_schulz(G, steps: int = 5, eps: float = 1e-7):
    """The quintic Newton-Schulz orthogonalisation of Muon: X0 = G/(|G|_F +
    eps) in the orientation with rows <= cols, then `steps` times
    X <- a X + (b A + c A A) X with A = X X^T."""
    a, b, c = NS_COEFFS
    X = np.asarray(G, dtype=F64)
    X = X / (np.linalg.norm(X) + eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def muon(theta, g, buf, lr: float, momentum: float, nesterov: bool, steps: int, wd: float):
    """One Muon step of a 2-D weight.  Returns (theta, buf)."""
    theta = np.asarray(theta, dtype=F64)
    g = np.asarray(g, dtype=F64)
    buf = momentum * np.asarray(buf, dtype=F64) + g
    u = g + momentum * buf if nesterov else buf
    o = newton_schulz(u, steps)
    rows, cols = theta.shape
    scale = math.sqrt(max(1.0, rows / cols))
    theta = theta * (1.0 - lr * wd) - lr * scale * o
    return theta, buf


def is_adamw_tensor(name: str) -> bool:
    """The embedding and the unembedding take AdamW, every block matrix Muon."""
    return name in ("wte", "wlm")


def init_state(params: dict) -> dict:
    """Optimizer state: an fp64 master copy of every weight, AdamW's two
    moments for its tensors and Muon's momentum buffer for the others."""
    st = {"master": {k: np.asarray(v, dtype=F64).copy() for k, v in params.items()},
          "m": {}, "v": {}, "buf": {}}
    for k, v in params.items():
        if is_adamw_tensor(k):
            st["m"][k] = np.zeros(v.shape, dtype=F64)
            st["v"][k] = np.zeros(v.shape, dtype=F64)
        else:
            st["buf"][k] = np.zeros(v.shape, dtype=F64)
    return st


def step(ocfg: dict, state: dict, grads: dict, t: int, lr_mult: float) -> float:
    """One optimizer step (t >= 1) on every tensor, in place on `state`.

    ocfg keys: adam_lr, adam_beta1, adam_beta2, adam_eps, adam_weight_decay,
    muon_lr, muon_momentum, muon_nesterov, muon_ns_steps, muon_weight_decay,
    grad_clip.  Returns the global gradient norm before clipping."""
    norm = global_norm(grads)
    s = clip_scale(norm, ocfg["grad_clip"])
    for k, g in grads.items():
        g = np.asarray(g, dtype=F64) * s
        if is_adamw_tensor(k):
            state["master"][k], state["m"][k], state["v"][k] = adamw(
                state["master"][k], g, state["m"][k], state["v"][k], t,
                ocfg["adam_lr"] * lr_mult, ocfg["adam_beta1"], ocfg["adam_beta2"],
                ocfg["adam_eps"], ocfg["adam_weight_decay"])
        else:
            state["master"][k], state["buf"][k] = muon(
                state["master"][k], g, state["buf"][k], ocfg["muon_lr"] * lr_mult,
                ocfg["muon_momentum"], bool(ocfg["muon_nesterov"]), ocfg["muon_ns_steps"],
                ocfg["muon_weight_decay"])
    return norm
