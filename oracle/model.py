"""Oracle: a plain, slow, float64 CPU forward and backward pass of the
nanochat-style dense decoder.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
CPU-baseline leg of the benchmark may import this module.  The GPU library
neither imports nor links it, and it shares no code with the GPU library: the
two meet only in the seeded inputs of ``nc_synth``.

What is computed (nanochat article, vpshk.cn, section on the ~8000-line code
base, architecture list):
  * dense decoder, every token uses every weight;
  * token embedding followed by a normalisation of the embedded token;
  * RMSNorm with no learnable parameters, n(u) = u / sqrt(mean(u^2) + eps);
  * per block, bias-free linear maps for Q, K and V, with multi-query
    attention: H query heads share one key head and one value head;
  * rotary position embedding as the only position information, then QK-norm
    (the same parameter-free RMSNorm over each head's vector);
  * causal softmax attention with scale 1/sqrt(head_dim);
  * bias-free output projection, relu^2 MLP;
  * untied unembedding (its own matrix, not the embedding's);
  * logit softcap c = s * tanh(z / s);
  * mean token cross-entropy (natural log), the pretraining objective named
    on the tianqi.csdn.net and vpshk.cn pages.

Readings where the pages are silent (each also listed in the design notes):
  * norm placement: pre-norm before attention and before the MLP, a final
    norm before the unembedding, plus the embedding norm (the vpshk page
    compares the architecture to Llama);
  * rotary pairs element i with element i + hd/2, angle t * base^(-2i/hd),
    positions restart at 0 in every sequence;
  * rotary is applied before QK-norm (they commute exactly);
  * relu^2 MLP of width d_mlp; loss is the plain mean over all B*T tokens.

Backward: the chain rule written out by hand, one block at a time, recomputing
the block's forward from its stored input (only block inputs are kept).
All arithmetic is float64; parameters arrive as float32 arrays (bf16-exact for
bf16 configurations) and are upcast on use.

Query rows of attention and token rows of the cross-entropy are processed in
chunks only to bound memory; every row is computed exactly as its definition
states and rows never interact.  The query chunks of one sequence's attention
run on a small thread pool; the key-side sums of the backward are then added
in chunk order, so the result does not depend on the pool.  The forward-only
cross-entropy runs its token chunks on the same pool.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F64 = np.float64
ATTN_QUERY_CHUNK = 1024
CE_TOKEN_CHUNK = 2048
ATTN_THREADS = max(1, min(4, len(os.sched_getaffinity(0))))


def _chunks(n: int, size: int, fn):
    """fn(t0, t1) for every chunk [t0, t1) of `size` rows out of n, on the
    thread pool; the results are returned in chunk order."""
    bounds = [(t0, min(n, t0 + size)) for t0 in range(0, n, size)]
    if len(bounds) == 1 or ATTN_THREADS == 1:
        return [fn(a, b) for a, b in bounds]
    with ThreadPoolExecutor(max_workers=ATTN_THREADS) as ex:
        return list(ex.map(lambda ab: fn(*ab), bounds))


def _query_chunks(T: int, fn):
    """fn(t0, t1) for every query chunk [t0, t1) of a length-T sequence."""
    return _chunks(T, ATTN_QUERY_CHUNK, fn)


# ---------------------------------------------------------------- primitives
def rms_norm(u: np.ndarray, eps: float):
    """Parameter-free RMSNorm over the last axis (nanochat architecture list:
    RMSNorm without learnable parameters).  Returns (n(u), r) with
    r = 1/sqrt(mean(u^2) + eps) of shape u.shape[:-1] + (1,)."""
    ms = np.mean(u * u, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    return u * r, r


def rms_norm_backward(dy: np.ndarray, y: np.ndarray, r: np.ndarray):
    """Gradient of y = r*u through the norm: dx = r * (dy - y * mean(dy*y))."""
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rotary_tables(seq_len: int, head_dim: int, base: float):
    """cos and sin of the rotary angles, [T, hd/2] float64.

    Pair i (of hd/2) turns at frequency base^(-2i/hd); position t turns it by
    t * base^(-2i/hd) radians.
    """
    half = head_dim // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=F64) / head_dim)
    ang = np.arange(seq_len, dtype=F64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rotary(u: np.ndarray, cos: np.ndarray, sin: np.ndarray):
    """Rotate pairs (u_i, u_{i+hd/2}) by their angles (rotary embedding, the
    only position encoding in the architecture list).  u is [..., T, hd] or
    [..., T, H, hd] with cos/sin broadcast over the head axis by the caller."""
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def rotary_backward(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray):
    """Transpose of the rotation (R_t^T dy), the gradient of rotary()."""
    half = dy.shape[-1] // 2
    a, b = dy[..., :half], dy[..., half:]
    return np.concatenate([a * cos + b * sin, -a * sin + b * cos], axis=-1)


def relu_squared(u: np.ndarray):
    """MLP activation relu(u)^2 (architecture list: relu squared in the MLP)."""
    return np.maximum(u, 0.0) ** 2


def relu_squared_backward(dg: np.ndarray, u: np.ndarray):
    """Gradient of relu(u)^2: dg * 2 * relu(u)."""
    return dg * 2.0 * np.maximum(u, 0.0)


def softcap(z: np.ndarray, s: float):
    """Logit softcap c = s * tanh(z/s) (architecture list: logit softcap)."""
    return s * np.tanh(z / s)


def _softmax_rows(x: np.ndarray):
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_mqa_attention(qn: np.ndarray, kn: np.ndarray, v: np.ndarray):
    """Causal multi-query attention of one sequence.

    qn [T, H, hd] (H query heads), kn [T, hd] and v [T, hd] (the one shared
    key/value head).  o[t, j] = sum_{tau <= t} softmax_tau(qn[t,j].kn[tau] /
    sqrt(hd)) v[tau].  Returns o [T, H, hd].
    """
    T, H, hd = qn.shape
    scale = 1.0 / np.sqrt(hd)
    qh = np.ascontiguousarray(qn.transpose(1, 0, 2))          # [H, T, hd]
    o = np.empty((H, T, hd), dtype=F64)

    def chunk(t0, t1):
        # keys past the chunk's last query (tau >= t1) take no part in the
        # causal sum of any of its rows, so only keys 0 .. t1-1 are formed
        s = (qh[:, t0:t1, :] @ kn[:t1].T) * scale              # [H, tq, t1]
        future = np.arange(t1)[None, :] > np.arange(t0, t1)[:, None]
        s[:, future] = -np.inf
        p = _softmax_rows(s)
        o[:, t0:t1, :] = p @ v[:t1]

    _query_chunks(T, chunk)
    return np.ascontiguousarray(o.transpose(1, 0, 2))


def causal_mqa_attention_backward(qn, kn, v, do):
    """Gradients (dqn, dkn, dv) of causal_mqa_attention for output grad do.

    With P the attention weights of head j: dv = sum_j P^T do_j;
    dP = do_j v^T; dS = P * (dP - rowsum(dP * P)); dq_j = dS kn / sqrt(hd);
    dkn = sum_j dS^T q_j / sqrt(hd).  P is recomputed from its definition.
    """
    T, H, hd = qn.shape
    scale = 1.0 / np.sqrt(hd)
    qh = np.ascontiguousarray(qn.transpose(1, 0, 2))
    doh = np.ascontiguousarray(do.transpose(1, 0, 2))
    dq = np.empty((H, T, hd), dtype=F64)
    dk = np.zeros((T, hd), dtype=F64)
    dv = np.zeros((T, hd), dtype=F64)

    def chunk(t0, t1):
        # as in the forward, keys tau >= t1 get no weight from these rows
        s = (qh[:, t0:t1, :] @ kn[:t1].T) * scale
        future = np.arange(t1)[None, :] > np.arange(t0, t1)[:, None]
        s[:, future] = -np.inf
        p = _softmax_rows(s)                                   # [H, tq, t1]
        d_o = doh[:, t0:t1, :]                                 # [H, tq, hd]
        dv_c = np.einsum("hqk,hqd->kd", p, d_o, optimize=True)
        dp = d_o @ v[:t1].T                                    # [H, tq, t1]
        ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
        dq[:, t0:t1, :] = (ds @ kn[:t1]) * scale
        dk_c = np.einsum("hqk,hqd->kd", ds, qh[:, t0:t1, :], optimize=True) * scale
        return t1, dk_c, dv_c

    for t1, dk_c, dv_c in _query_chunks(T, chunk):
        dk[:t1] += dk_c
        dv[:t1] += dv_c
    return np.ascontiguousarray(dq.transpose(1, 0, 2)), dk, dv


def softcap_cross_entropy(z: np.ndarray, targets: np.ndarray, s: float):
    """Per-token loss l = logsumexp(c) - c[y] with c = s*tanh(z/s), and the
    gradient dl/dz = (softmax(c) - onehot(y)) * (1 - (c/s)^2).
    z [n, V] float64, targets [n] int.  Returns (loss [n], dl_dz [n, V])."""
    c = softcap(z, s)
    m = np.max(c, axis=-1, keepdims=True)
    lse = m[:, 0] + np.log(np.sum(np.exp(c - m), axis=-1))
    rows = np.arange(z.shape[0])
    loss = lse - c[rows, targets]
    dc = np.exp(c - lse[:, None])
    dc[rows, targets] -= 1.0
    dz = dc * (1.0 - (c / s) ** 2)
    return loss, dz


# ---------------------------------------------------------------- the model
def _w(params, name):
    return np.asarray(params[name], dtype=F64)


def _block_forward(cfg, params, layer, h, cos, sin):
    """One pre-norm block over the whole batch.  h [B, T, D].  Returns the
    block output and every intermediate its backward needs."""
    B, T, D = h.shape
    H, hd, eps = cfg["n_head"], cfg["head_dim"], cfg["rms_eps"]
    p = f"h{layer}."
    wq, wk, wv = _w(params, p + "wq"), _w(params, p + "wk"), _w(params, p + "wv")
    wo, wfc, wproj = _w(params, p + "wo"), _w(params, p + "wfc"), _w(params, p + "wproj")

    a, r1 = rms_norm(h, eps)
    q = (a @ wq.T).reshape(B, T, H, hd)
    k = a @ wk.T                                               # [B, T, hd]
    v = a @ wv.T
    qr = rotary(q, cos[None, :, None, :], sin[None, :, None, :])
    kr = rotary(k, cos[None], sin[None])
    qn, rq = rms_norm(qr, eps)
    kn, rk = rms_norm(kr, eps)
    o = np.stack([causal_mqa_attention(qn[b], kn[b], v[b]) for b in range(B)])
    of = o.reshape(B, T, H * hd)
    h1 = h + of @ wo.T
    m, r2 = rms_norm(h1, eps)
    u = m @ wfc.T
    g = relu_squared(u)
    h2 = h1 + g @ wproj.T
    saved = dict(a=a, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk, v=v, of=of, h1=h1,
                 m=m, r2=r2, u=u, g=g)
    return h2, saved


def _block_backward(cfg, params, layer, h, dh2, cos, sin, grads):
    """Backward of one block given its input h and output gradient dh2.
    Writes the block's weight gradients into grads and returns dh."""
    B, T, D = h.shape
    H, hd = cfg["n_head"], cfg["head_dim"]
    p = f"h{layer}."
    wq, wk, wv = _w(params, p + "wq"), _w(params, p + "wk"), _w(params, p + "wv")
    wo, wfc, wproj = _w(params, p + "wo"), _w(params, p + "wfc"), _w(params, p + "wproj")
    _, s = _block_forward(cfg, params, layer, h, cos, sin)

    def flat(x):
        return x.reshape(-1, x.shape[-1])

    # MLP: h2 = h1 + relu(n(h1) wfc^T)^2 wproj^T
    dg = dh2 @ wproj
    grads[p + "wproj"] = flat(dh2).T @ flat(s["g"])
    du = relu_squared_backward(dg, s["u"])
    dm = du @ wfc
    grads[p + "wfc"] = flat(du).T @ flat(s["m"])
    dh1 = dh2 + rms_norm_backward(dm, s["m"], s["r2"])

    # attention: h1 = h + attn(n(h)) wo^T
    dof = dh1 @ wo
    grads[p + "wo"] = flat(dh1).T @ flat(s["of"])
    do = dof.reshape(B, T, H, hd)
    dqn = np.empty_like(s["qn"])
    dkn = np.empty_like(s["kn"])
    dv = np.empty_like(s["v"])
    for b in range(B):
        dqn[b], dkn[b], dv[b] = causal_mqa_attention_backward(
            s["qn"][b], s["kn"][b], s["v"][b], do[b])
    dqr = rms_norm_backward(dqn, s["qn"], s["rq"])
    dkr = rms_norm_backward(dkn, s["kn"], s["rk"])
    dq = rotary_backward(dqr, cos[None, :, None, :], sin[None, :, None, :])
    dk = rotary_backward(dkr, cos[None], sin[None])
    dq = dq.reshape(B, T, H * hd)
    da = dq @ wq + dk @ wk + dv @ wv
    grads[p + "wq"] = flat(dq).T @ flat(s["a"])
    grads[p + "wk"] = flat(dk).T @ flat(s["a"])
    grads[p + "wv"] = flat(dv).T @ flat(s["a"])
    return dh1 + rms_norm_backward(da, s["a"], s["r1"])


def _embed(cfg, params, tokens):
    """h0 = n(W_te[x]) (architecture list: normalised token embedding)."""
    e = np.asarray(params["wte"][tokens], dtype=F64)            # [B, T, D]
    h0, r0 = rms_norm(e, cfg["rms_eps"])
    return e, h0, r0


def embedding_gradient(tokens: np.ndarray, de: np.ndarray, vocab: int):
    """dW_te: row v is the sum of de_t over the positions t whose token is v
    (the embedding lookup's backward; a row no token uses is zero).  tokens
    int [...], de [..., D]; float64 [vocab, D]."""
    de = np.asarray(de, dtype=F64)
    dwte = np.zeros((vocab, de.shape[-1]), dtype=F64)
    np.add.at(dwte, np.asarray(tokens).reshape(-1), de.reshape(-1, de.shape[-1]))
    return dwte


def _head_loss(cfg, params, h, targets, want_grad):
    """Final norm, untied unembedding, softcap and cross-entropy.

    Returns (per-token loss [B, T], dh [B, T, D] or None, dW_lm or None); the
    gradients are those of the mean loss over all B*T tokens.
    """
    B, T, D = h.shape
    n = B * T
    f, rf = rms_norm(h, cfg["rms_eps"])
    ff = f.reshape(n, D)
    y = targets.reshape(n)
    wlm = _w(params, "wlm")
    loss = np.empty(n, dtype=F64)
    df = np.empty((n, D), dtype=F64) if want_grad else None
    dwlm = np.zeros_like(wlm) if want_grad else None
    if not want_grad:
        # token chunks are independent: the forward alone runs them on the pool
        def chunk(t0, t1):
            loss[t0:t1] = softcap_cross_entropy(ff[t0:t1] @ wlm.T, y[t0:t1], cfg["softcap"])[0]

        _chunks(n, CE_TOKEN_CHUNK, chunk)
        return loss.reshape(B, T), None, None
    for t0 in range(0, n, CE_TOKEN_CHUNK):
        t1 = min(n, t0 + CE_TOKEN_CHUNK)
        z = ff[t0:t1] @ wlm.T
        l, dz = softcap_cross_entropy(z, y[t0:t1], cfg["softcap"])
        loss[t0:t1] = l
        if want_grad:
            dz /= n
            df[t0:t1] = dz @ wlm
            dwlm += dz.T @ ff[t0:t1]
    if not want_grad:
        return loss.reshape(B, T), None, None
    dh = rms_norm_backward(df.reshape(B, T, D), f, rf)
    return loss.reshape(B, T), dh, dwlm


def forward_loss(cfg: dict, params: dict, tokens: np.ndarray,
                 targets: np.ndarray):
    """Mean cross-entropy of a batch and the per-token losses [B, T]."""
    B, T = tokens.shape
    cos, sin = rotary_tables(T, cfg["head_dim"], cfg["rope_base"])
    _, h, _ = _embed(cfg, params, tokens)
    for layer in range(cfg["n_layer"]):
        h, _ = _block_forward(cfg, params, layer, h, cos, sin)
    tok_loss, _, _ = _head_loss(cfg, params, h, targets, want_grad=False)
    return float(np.mean(tok_loss)), tok_loss


def forward_backward(cfg: dict, params: dict, tokens: np.ndarray,
                     targets: np.ndarray):
    """Mean loss and the gradient of every weight matrix (float64 arrays of
    the parameters' shapes, keyed like the parameters)."""
    B, T = tokens.shape
    L = cfg["n_layer"]
    cos, sin = rotary_tables(T, cfg["head_dim"], cfg["rope_base"])
    e, h, r0 = _embed(cfg, params, tokens)
    h0 = h
    inputs = []
    for layer in range(L):
        inputs.append(h)
        h, _ = _block_forward(cfg, params, layer, h, cos, sin)
    tok_loss, dh, dwlm = _head_loss(cfg, params, h, targets, want_grad=True)
    grads = {"wlm": dwlm}
    for layer in reversed(range(L)):
        dh = _block_backward(cfg, params, layer, inputs[layer], dh, cos, sin,
                             grads)
        inputs[layer] = None
    de = rms_norm_backward(dh, h0, r0)
    grads["wte"] = embedding_gradient(tokens, de, params["wte"].shape[0])
    return float(np.mean(tok_loss)), grads


def forward_logits(cfg: dict, params: dict, tokens: np.ndarray, positions=None):
    """Softcapped logits c = s*tanh(z/s) of every sequence at the given
    positions (all positions if None): [B, P, V] float64.

    This is what generation reads: the next-token distribution at position t
    is softmax(c_t).  It is the forward pass of forward_loss without the
    cross-entropy; causality makes c_t a function of tokens[:, :t+1] alone,
    which is what an inference engine with a key/value cache computes one
    position at a time (inference feature of the nanochat pages: a KV cache
    with prefill and decode)."""
    B, T = tokens.shape
    cos, sin = rotary_tables(T, cfg["head_dim"], cfg["rope_base"])
    _, h, _ = _embed(cfg, params, tokens)
    for layer in range(cfg["n_layer"]):
        h, _ = _block_forward(cfg, params, layer, h, cos, sin)
    pos = np.arange(T) if positions is None else np.asarray(positions)
    f, _ = rms_norm(h[:, pos, :], cfg["rms_eps"])
    z = f @ _w(params, "wlm").T
    return softcap(z, cfg["softcap"])
