"""ctypes binding of the step library (include/nc.h, include/nc_ops.h).

Functions keep the C names and marshal arguments only: device pointers are
passed as integers (``tensor.data_ptr()``), streams as the integer value of a
hipStream_t (``torch.cuda.current_stream().cuda_stream``).  Every non-zero
status raises NcError.  The compute happens in libnc.so; if it is missing the
import fails loudly -- there is no fallback.

``Model`` is a convenience wrapper that uses PyTorch only to allocate device
memory and to obtain the current stream.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnc.so")

NC_F32, NC_BF16 = 0, 1


class NcError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str, hip: int | None = None):
        extra = f" (hipError {hip})" if hip else ""
        super().__init__(f"{fn} failed: {code} {msg}{extra}")
        self.code = code


class nc_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layer", "d_model", "n_head", "head_dim", "n_kv_head", "d_mlp", "vocab",
        "seq_len", "batch")] + [
        ("rope_base", C.c_float), ("softcap", C.c_float), ("rms_eps", C.c_float),
        ("dtype", C.c_int32)]


class nc_kernel_stat(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int32), ("total_ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double)]


class nc_optim_config(C.Structure):
    _fields_ = [(n, C.c_float) for n in (
        "adam_lr", "adam_beta1", "adam_beta2", "adam_eps", "adam_weight_decay", "muon_lr",
        "muon_momentum", "muon_weight_decay")] + [
        ("muon_nesterov", C.c_int32), ("muon_ns_steps", C.c_int32), ("grad_clip", C.c_float)]


class nc_tensor_info(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("offset", C.c_int64), ("rows", C.c_int32),
                ("cols", C.c_int32)]


def _load():
    # PyTorch ships its own HIP runtime (libamdhip64, libhsa-runtime64) under
    # the same soname as the system one libnc.so is linked against.  Loading
    # torch first makes the dynamic loader bind libnc.so to torch's copy, so
    # the process drives the GPU through one runtime; loading libnc.so first
    # would map both runtimes into the process, with two instances of the
    # runtime's state for one device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m dense_gpt_pretraining_amd.build` "
            "or `python -c 'import __graft_entry__; __graft_entry__.build()'`")
    return C.CDLL(LIB_PATH)


_lib = _load()
_P = C.c_void_p
_sigs = {
    "nc_param_count": (C.c_int, [C.POINTER(nc_config), C.POINTER(C.c_int64)]),
    "nc_param_layout": (C.c_int, [C.POINTER(nc_config), C.POINTER(nc_tensor_info), C.c_int32,
                                  C.POINTER(C.c_int32)]),
    "nc_workspace_size": (C.c_int, [C.POINTER(nc_config), C.c_int32, C.POINTER(C.c_size_t)]),
    "nc_init_params": (C.c_int, [C.POINTER(nc_config), C.c_uint64, _P, _P]),
    "nc_forward_loss": (C.c_int, [C.POINTER(nc_config), _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "nc_forward_token_loss": (C.c_int, [C.POINTER(nc_config), _P, _P, _P, _P, _P, _P,
                                        C.c_size_t, _P]),
    "nc_forward_backward": (C.c_int, [C.POINTER(nc_config), _P, _P, _P, _P, _P, _P,
                                      C.c_size_t, _P]),
    "nc_workspace_size_recompute": (C.c_int, [C.POINTER(nc_config), C.POINTER(C.c_size_t)]),
    "nc_forward_backward_recompute": (C.c_int, [C.POINTER(nc_config), _P, _P, _P, _P, _P, _P,
                                                C.c_size_t, _P]),
    "nc_forward_backward_timed": (C.c_int, [C.POINTER(nc_config), _P, _P, _P, _P, _P, _P,
                                            C.c_size_t, _P, C.POINTER(nc_kernel_stat),
                                            C.c_int32, C.POINTER(C.c_int32)]),
    "nc_validate_tokens": (C.c_int, [C.POINTER(nc_config), _P, _P, _P, _P]),
    "nc_status_string": (C.c_char_p, [C.c_int]),
    "nc_last_hip_error": (C.c_int, []),
    "nc_optim_state_size": (C.c_int, [C.POINTER(nc_config), C.POINTER(C.c_size_t)]),
    "nc_optim_workspace_size": (C.c_int, [C.POINTER(nc_config), C.POINTER(C.c_size_t)]),
    "nc_optim_init": (C.c_int, [C.POINTER(nc_config), _P, _P, _P]),
    "nc_optim_step": (C.c_int, [C.POINTER(nc_config), C.POINTER(nc_optim_config), C.c_int64,
                                C.c_float, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "nc_grad_accumulate": (C.c_int, [_P, _P, C.c_int64, C.c_float, C.c_int32, _P]),
    "nc_lr_multiplier": (C.c_double, [C.c_int64, C.c_int64, C.c_int64, C.c_double]),
    "nc_kv_cache_size": (C.c_int, [C.POINTER(nc_config), C.c_int32, C.POINTER(C.c_size_t)]),
    "nc_infer_workspace_size": (C.c_int, [C.POINTER(nc_config), C.c_int32, C.c_int32,
                                          C.POINTER(C.c_size_t)]),
    "nc_prefill": (C.c_int, [C.POINTER(nc_config), _P, _P, C.c_int32, C.c_int32, _P, _P, _P,
                             C.c_size_t, _P]),
    "nc_decode_step": (C.c_int, [C.POINTER(nc_config), _P, _P, C.c_int32, C.c_int32, _P, _P, _P,
                                 C.c_size_t, _P]),
    "nc_decode_step_noalloc": (C.c_int, [C.POINTER(nc_config), _P, _P, C.c_int32, C.c_int32,
                                         _P, _P, _P]),
    "nc_op_matmul": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P, C.c_int64,
                               C.c_int32, _P, C.c_int64, C.c_int32, _P, C.c_int64, _P,
                               C.c_size_t, _P]),
    "nc_op_matmul_epilogue": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P,
                                        C.c_int64, C.c_int32, _P, C.c_int64, C.c_int32, _P,
                                        C.c_int64, C.c_int32, _P, _P, _P]),
    "nc_op_attention_fwd": (C.c_int, [C.c_int32] * 5 + [_P, _P, _P, C.c_int64, C.c_int64, _P, _P,
                                                          C.c_int32, _P]),
    "nc_op_attention_bwd": (C.c_int, [C.c_int32] * 5 + [_P, _P, _P, C.c_int64, C.c_int64, _P, _P,
                                                          _P, _P, C.c_size_t, _P, _P, _P, _P]),
    "nc_op_attention_bwd_scratch_bytes": (C.c_int, [C.c_int32] * 4 + [C.POINTER(C.c_size_t)]),
    "nc_op_softcap_ce": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int64, _P, _P, C.c_float,
                                   _P, C.c_float, _P, C.c_int32, _P]),
    "nc_op_rope_qknorm_fwd": (C.c_int, [C.c_int32] * 5 + [_P, C.c_float, C.c_float, _P, _P, _P]),
    "nc_op_embedding_grad": (C.c_int, [C.c_int32] * 3 + [_P, _P, _P, _P, C.c_size_t, _P]),
    "nc_op_embedding_grad_ws_bytes": (C.c_int, [C.c_int32] * 3 + [C.POINTER(C.c_size_t)]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(fn: str, rc: int):
    if rc != 0:
        hip = _lib.nc_last_hip_error() if rc == -6 else None
        raise NcError(fn, rc, _lib.nc_status_string(rc).decode(), hip)


def make_config(cfg: dict) -> nc_config:
    """nc_config from a configuration dict (fields named as in nc.h; dtype
    "f32" or "bf16")."""
    c = nc_config()
    for k in ("n_layer", "d_model", "n_head", "head_dim", "n_kv_head", "d_mlp", "vocab",
              "seq_len", "batch"):
        setattr(c, k, int(cfg[k]))
    c.rope_base = float(cfg["rope_base"])
    c.softcap = float(cfg["softcap"])
    c.rms_eps = float(cfg["rms_eps"])
    d = cfg["dtype"]
    c.dtype = {"f32": NC_F32, "bf16": NC_BF16}[d] if isinstance(d, str) else int(d)
    return c


# ------------------------------------------------------------------ C names
def nc_param_count(cfg: nc_config) -> int:
    n = C.c_int64()
    _check("nc_param_count", _lib.nc_param_count(C.byref(cfg), C.byref(n)))
    return n.value


def nc_param_layout(cfg: nc_config) -> list[tuple[str, int, int, int]]:
    n = C.c_int32()
    rc = _lib.nc_param_layout(C.byref(cfg), None, 0, C.byref(n))
    if rc not in (0, -8):
        _check("nc_param_layout", rc)
    arr = (nc_tensor_info * n.value)()
    _check("nc_param_layout", _lib.nc_param_layout(C.byref(cfg), arr, n.value, C.byref(n)))
    return [(a.name.decode(), a.offset, a.rows, a.cols) for a in arr]


def nc_workspace_size(cfg: nc_config, with_backward: bool) -> int:
    b = C.c_size_t()
    _check("nc_workspace_size", _lib.nc_workspace_size(C.byref(cfg), int(with_backward),
                                                       C.byref(b)))
    return b.value


def nc_init_params(cfg: nc_config, seed: int, params: int, stream: int):
    _check("nc_init_params", _lib.nc_init_params(C.byref(cfg), seed, params, stream))


def nc_forward_loss(cfg, params, tokens, targets, loss, ws, ws_bytes, stream):
    _check("nc_forward_loss", _lib.nc_forward_loss(C.byref(cfg), params, tokens, targets, loss,
                                                   ws, ws_bytes, stream))


def nc_forward_token_loss(cfg, params, tokens, targets, loss, token_loss, ws, ws_bytes, stream):
    _check("nc_forward_token_loss", _lib.nc_forward_token_loss(
        C.byref(cfg), params, tokens, targets, loss, token_loss, ws, ws_bytes, stream))


def nc_forward_backward(cfg, params, tokens, targets, loss, grads, ws, ws_bytes, stream):
    _check("nc_forward_backward", _lib.nc_forward_backward(
        C.byref(cfg), params, tokens, targets, loss, grads, ws, ws_bytes, stream))


def nc_workspace_size_recompute(cfg: nc_config) -> int:
    b = C.c_size_t()
    _check("nc_workspace_size_recompute", _lib.nc_workspace_size_recompute(C.byref(cfg),
                                                                           C.byref(b)))
    return b.value


def nc_forward_backward_recompute(cfg, params, tokens, targets, loss, grads, ws, ws_bytes,
                                  stream):
    _check("nc_forward_backward_recompute", _lib.nc_forward_backward_recompute(
        C.byref(cfg), params, tokens, targets, loss, grads, ws, ws_bytes, stream))


def nc_forward_backward_timed(cfg, params, tokens, targets, loss, grads, ws, ws_bytes, stream,
                              cap: int = 64) -> list[dict]:
    """Runs the step with per-launch events; returns one dict per kernel label."""
    arr = (nc_kernel_stat * cap)()
    n = C.c_int32()
    _check("nc_forward_backward_timed", _lib.nc_forward_backward_timed(
        C.byref(cfg), params, tokens, targets, loss, grads, ws, ws_bytes, stream, arr, cap,
        C.byref(n)))
    return [dict(name=a.name.decode(), launches=a.launches, ms=a.total_ms, flops=a.flops,
                 bytes=a.bytes) for a in arr[:n.value]]


def nc_validate_tokens(cfg, tokens, targets, n_bad, stream):
    _check("nc_validate_tokens", _lib.nc_validate_tokens(C.byref(cfg), tokens, targets, n_bad,
                                                         stream))


def make_optim_config(ocfg: dict) -> nc_optim_config:
    """nc_optim_config from a dict with the field names of nc_optim.h."""
    o = nc_optim_config()
    for name, typ in nc_optim_config._fields_:
        setattr(o, name, int(ocfg[name]) if typ is C.c_int32 else float(ocfg[name]))
    return o


def nc_optim_state_size(cfg: nc_config) -> int:
    b = C.c_size_t()
    _check("nc_optim_state_size", _lib.nc_optim_state_size(C.byref(cfg), C.byref(b)))
    return b.value


def nc_optim_workspace_size(cfg: nc_config) -> int:
    b = C.c_size_t()
    _check("nc_optim_workspace_size", _lib.nc_optim_workspace_size(C.byref(cfg), C.byref(b)))
    return b.value


def nc_optim_init(cfg, params, state, stream):
    _check("nc_optim_init", _lib.nc_optim_init(C.byref(cfg), params, state, stream))


def nc_optim_step(cfg, ocfg, step, lr_mult, grads, params, state, grad_norm, ws, ws_bytes,
                  stream):
    _check("nc_optim_step", _lib.nc_optim_step(C.byref(cfg), C.byref(ocfg), step, lr_mult,
                                               grads, params, state, grad_norm, ws, ws_bytes,
                                               stream))


def nc_grad_accumulate(acc, grads, n, scale, overwrite, stream):
    _check("nc_grad_accumulate", _lib.nc_grad_accumulate(acc, grads, n, scale, int(overwrite),
                                                         stream))


def nc_lr_multiplier(step: int, total: int, warmup: int, final_frac: float) -> float:
    v = _lib.nc_lr_multiplier(step, total, warmup, final_frac)
    if v < 0:
        raise NcError("nc_lr_multiplier", -2, "a schedule argument is out of range")
    return v


def nc_kv_cache_size(cfg: nc_config, max_seq: int) -> int:
    b = C.c_size_t()
    _check("nc_kv_cache_size", _lib.nc_kv_cache_size(C.byref(cfg), max_seq, C.byref(b)))
    return b.value


def nc_infer_workspace_size(cfg: nc_config, max_seq: int, t0: int) -> int:
    b = C.c_size_t()
    _check("nc_infer_workspace_size", _lib.nc_infer_workspace_size(C.byref(cfg), max_seq, t0,
                                                                   C.byref(b)))
    return b.value


def nc_prefill(cfg, params, tokens, t0, max_seq, cache, logits, ws, ws_bytes, stream):
    _check("nc_prefill", _lib.nc_prefill(C.byref(cfg), params, tokens, t0, max_seq, cache, logits,
                                         ws, ws_bytes, stream))


def nc_decode_step(cfg, params, tokens, pos, max_seq, cache, logits, ws, ws_bytes, stream):
    _check("nc_decode_step", _lib.nc_decode_step(C.byref(cfg), params, tokens, pos, max_seq,
                                                 cache, logits, ws, ws_bytes, stream))


def nc_decode_step_noalloc(cfg, params, tokens, pos, max_seq, cache, logits, stream):
    _check("nc_decode_step_noalloc", _lib.nc_decode_step_noalloc(
        C.byref(cfg), params, tokens, pos, max_seq, cache, logits, stream))


def nc_status_string(code: int) -> str:
    return _lib.nc_status_string(code).decode()


def nc_last_hip_error() -> int:
    return _lib.nc_last_hip_error()


def nc_op_matmul(dtype, M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, Cp, ldc, ws, ws_bytes,
                 stream):
    _check("nc_op_matmul", _lib.nc_op_matmul(dtype, M, N, K, A, lda, int(a_kmajor), B, ldb,
                                             int(b_kmajor), Cp, ldc, ws, ws_bytes, stream))


def nc_op_matmul_epilogue(dtype, M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, Cp, ldc, mode,
                          rowscale, aux, stream):
    _check("nc_op_matmul_epilogue", _lib.nc_op_matmul_epilogue(
        dtype, M, N, K, A, lda, int(a_kmajor), B, ldb, int(b_kmajor), Cp, ldc, mode, rowscale, aux,
        stream))


def nc_op_attention_fwd(dtype, B, T, H, hd, q, k, v, ldq, ldkv, o, lse, stream, qk_normed=0):
    _check("nc_op_attention_fwd", _lib.nc_op_attention_fwd(dtype, B, T, H, hd, q, k, v, ldq,
                                                           ldkv, o, lse, qk_normed, stream))


def nc_op_attention_bwd(dtype, B, T, H, hd, q, k, v, ldq, ldkv, o, dout, lse, scratch,
                        scratch_bytes, dq, dk, dv, stream):
    _check("nc_op_attention_bwd", _lib.nc_op_attention_bwd(
        dtype, B, T, H, hd, q, k, v, ldq, ldkv, o, dout, lse, scratch, scratch_bytes, dq, dk, dv,
        stream))


def nc_op_attention_bwd_scratch_bytes(B, T, H, hd) -> int:
    n = C.c_size_t()
    _check("nc_op_attention_bwd_scratch_bytes",
           _lib.nc_op_attention_bwd_scratch_bytes(B, T, H, hd, C.byref(n)))
    return n.value


def nc_op_softcap_ce(dtype, N, V, ldz, z, targets, softcap, rowscale, inv_n, tok_loss,
                     want_grad, stream):
    _check("nc_op_softcap_ce", _lib.nc_op_softcap_ce(dtype, N, V, ldz, z, targets, softcap,
                                                     rowscale, inv_n, tok_loss, int(want_grad),
                                                     stream))


def nc_op_rope_qknorm_fwd(dtype, B, T, H, hd, qkv, base, eps, rqk, tables, stream):
    _check("nc_op_rope_qknorm_fwd", _lib.nc_op_rope_qknorm_fwd(dtype, B, T, H, hd, qkv, base,
                                                               eps, rqk, tables, stream))


def nc_op_embedding_grad_ws_bytes(N, D, V) -> int:
    n = C.c_size_t()
    _check("nc_op_embedding_grad_ws_bytes",
           _lib.nc_op_embedding_grad_ws_bytes(N, D, V, C.byref(n)))
    return n.value


def nc_op_embedding_grad(N, D, V, de, tokens, dwte, ws, ws_bytes, stream):
    _check("nc_op_embedding_grad", _lib.nc_op_embedding_grad(N, D, V, de, tokens, dwte, ws,
                                                             ws_bytes, stream))


def _bf16_bits_rne(w: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (the
    library's own fp32 -> bf16 conversion; inputs are finite)."""
    b = w.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


# ------------------------------------------------------------------ torch helper
class Model:
    """Owns nothing but the config; allocates caller-side buffers with torch."""

    def __init__(self, cfg: dict, device: str = "cuda"):
        import torch
        self.torch = torch
        self.cfg = dict(cfg)
        self.c = make_config(cfg)
        self.device = device
        self.bf16 = self.c.dtype == NC_BF16
        self.tdtype = torch.bfloat16 if self.bf16 else torch.float32
        self.n_params = nc_param_count(self.c)
        self.layout = nc_param_layout(self.c)
        self._ws = {}

    def stream(self) -> int:
        return self.torch.cuda.current_stream().cuda_stream

    # host <-> device parameter packing (marshalling only)
    def pack(self, params: dict) -> "torch.Tensor":
        torch = self.torch
        if self.bf16:
            flat = np.zeros(self.n_params, dtype=np.uint16)
            for name, off, r, c in self.layout:
                w = np.ascontiguousarray(params[name], dtype=np.float32).reshape(-1)
                flat[off:off + r * c] = _bf16_bits_rne(w)
            t = torch.from_numpy(flat.view(np.int16)).to(self.device)
            return t.view(torch.bfloat16)
        flat = np.zeros(self.n_params, dtype=np.float32)
        for name, off, r, c in self.layout:
            flat[off:off + r * c] = np.asarray(params[name], dtype=np.float32).reshape(-1)
        return torch.from_numpy(flat).to(self.device)

    def unpack(self, flat) -> dict:
        """fp32 host arrays per tensor from a flat device buffer (params or grads)."""
        torch = self.torch
        if flat.dtype == torch.bfloat16:
            host = flat.view(torch.int16).cpu().numpy().view(np.uint16)
            host = (host.astype(np.uint32) << np.uint32(16)).view(np.float32)
        else:
            host = flat.float().cpu().numpy()
        return {name: host[off:off + r * c].reshape(r, c) for name, off, r, c in self.layout}

    def workspace(self, with_backward: bool, recompute: bool = False):
        key = ("recompute" if recompute else bool(with_backward))
        if key not in self._ws:
            n = (nc_workspace_size_recompute(self.c) if recompute
                 else nc_workspace_size(self.c, bool(with_backward)))
            self._ws[key] = self.torch.empty(max(n, 256), dtype=self.torch.uint8,
                                             device=self.device)
        return self._ws[key]

    def free_workspaces(self):
        self._ws = {}

    def init_params(self, seed: int):
        p = self.torch.empty(self.n_params, dtype=self.tdtype, device=self.device)
        nc_init_params(self.c, seed, p.data_ptr(), self.stream())
        return p

    def _tok(self, a):
        torch = self.torch
        if isinstance(a, np.ndarray):
            a = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
        return a.to(self.device, torch.int32).contiguous()

    def forward_loss(self, params, tokens, targets, token_loss: bool = False):
        torch = self.torch
        tok, tgt = self._tok(tokens), self._tok(targets)
        loss = torch.empty(1, dtype=torch.float32, device=self.device)
        tl = torch.empty(tok.shape, dtype=torch.float32, device=self.device) if token_loss else None
        ws = self.workspace(False)
        if tl is None:
            nc_forward_loss(self.c, params.data_ptr(), tok.data_ptr(), tgt.data_ptr(),
                            loss.data_ptr(), ws.data_ptr(), ws.numel(), self.stream())
            return loss
        nc_forward_token_loss(self.c, params.data_ptr(), tok.data_ptr(), tgt.data_ptr(),
                              loss.data_ptr(), tl.data_ptr(), ws.data_ptr(), ws.numel(),
                              self.stream())
        return loss, tl

    def forward_backward(self, params, tokens, targets, grads=None, recompute: bool = False):
        torch = self.torch
        tok, tgt = self._tok(tokens), self._tok(targets)
        loss = torch.empty(1, dtype=torch.float32, device=self.device)
        if grads is None:
            grads = torch.empty(self.n_params, dtype=torch.float32, device=self.device)
        ws = self.workspace(True, recompute)
        fn = nc_forward_backward_recompute if recompute else nc_forward_backward
        fn(self.c, params.data_ptr(), tok.data_ptr(), tgt.data_ptr(), loss.data_ptr(),
           grads.data_ptr(), ws.data_ptr(), ws.numel(), self.stream())
        return loss, grads


class Optimizer:
    """Muon + AdamW state for a Model's parameters (device buffers from torch)."""

    def __init__(self, model: Model, ocfg: dict):
        torch = model.torch
        self.m = model
        self.o = make_optim_config(ocfg)
        self.state = torch.empty(nc_optim_state_size(model.c), dtype=torch.uint8,
                                 device=model.device)
        self.ws = torch.empty(max(nc_optim_workspace_size(model.c), 256), dtype=torch.uint8,
                              device=model.device)
        self.norm = torch.empty(1, dtype=torch.float32, device=model.device)

    def init(self, params):
        nc_optim_init(self.m.c, params.data_ptr(), self.state.data_ptr(), self.m.stream())

    def step(self, params, grads, step: int, lr_mult: float = 1.0):
        """One step (step >= 1); returns the device tensor holding the global
        gradient norm before clipping."""
        nc_optim_step(self.m.c, self.o, step, lr_mult, grads.data_ptr(), params.data_ptr(),
                      self.state.data_ptr(), self.norm.data_ptr(), self.ws.data_ptr(),
                      self.ws.numel(), self.m.stream())
        return self.norm

    def master(self):
        """fp32 master weights, unpacked per tensor (host arrays)."""
        n = self.m.n_params
        return self.m.unpack(self.state.view(self.m.torch.float32)[:n])

    def moments(self):
        """(first array, second array) of the state, unpacked per tensor."""
        torch = self.m.torch
        n = self.m.n_params
        arr = ((n * 4 + 255) // 256) * 256 // 4
        f = self.state.view(torch.float32)
        return self.m.unpack(f[arr:arr + n]), self.m.unpack(f[2 * arr:2 * arr + n])


class Generator:
    """KV cache and workspace for prefill + decode of a Model (torch buffers)."""

    def __init__(self, model: Model, max_seq: int, max_prefill: int = 0):
        torch = model.torch
        self.m = model
        self.max_seq = max_seq
        self.cache = torch.empty(nc_kv_cache_size(model.c, max_seq), dtype=torch.uint8,
                                 device=model.device)
        self.ws = torch.empty(max(nc_infer_workspace_size(model.c, max_seq, max_prefill), 256),
                              dtype=torch.uint8, device=model.device)
        self.logits = torch.empty((model.c.batch, model.c.vocab), dtype=torch.float32,
                                  device=model.device)

    def prefill(self, params, tokens):
        """tokens [B, t0] (t0 a multiple of 64); returns the logits at t0-1."""
        tok = self.m._tok(tokens)
        nc_prefill(self.m.c, params.data_ptr(), tok.data_ptr(), tok.shape[1], self.max_seq,
                   self.cache.data_ptr(), self.logits.data_ptr(), self.ws.data_ptr(),
                   self.ws.numel(), self.m.stream())
        return self.logits

    def decode(self, params, tokens, pos: int):
        """tokens [B] at position pos; returns the logits at pos."""
        tok = self.m._tok(tokens)
        nc_decode_step(self.m.c, params.data_ptr(), tok.data_ptr(), pos, self.max_seq,
                       self.cache.data_ptr(), self.logits.data_ptr(), self.ws.data_ptr(),
                       self.ws.numel(), self.m.stream())
        return self.logits
