"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the headers declare, validates configurations and pointers
before any device work, and reports the documented parameter layout."""
import ctypes
import os
import re

import numpy as np
import pytest

from nc_synth import get_config, param_shapes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _b():
    from dense_gpt_pretraining_amd import binding
    return binding


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        with open(os.path.join(ROOT, "include", h)) as f:
            text = f.read()
        names |= set(re.findall(r"\b(nc_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    b = _b()
    lib = ctypes.CDLL(b.LIB_PATH)
    names = _declared()
    assert {"nc_init_params", "nc_forward_loss", "nc_forward_backward"} <= names
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", ["tiny", "gpt2", "d20", "d30", "long"])
def test_layout_matches_parameter_shapes(name):
    b = _b()
    cfg = get_config(name)
    c = b.make_config(cfg)
    lay = b.nc_param_layout(c)
    shapes = param_shapes(cfg)
    assert [x[0] for x in lay] == [s[0] for s in shapes]
    for (n, off, r, k), (_, shp, _) in zip(lay, shapes):
        assert (r, k) == shp
    # offsets increase, tensors do not overlap, wq|wk|wv are contiguous
    ends = [off + r * k for _, off, r, k in lay]
    assert all(lay[i + 1][1] >= ends[i] for i in range(len(lay) - 1))
    for i, (n, off, r, k) in enumerate(lay):
        if n.endswith(".wq"):
            assert lay[i + 1][1] == ends[i] and lay[i + 2][1] == ends[i + 1]
        if not (n.endswith(".wk") or n.endswith(".wv")):
            assert off % 128 == 0
    total = b.nc_param_count(c)
    assert total >= ends[-1]
    assert sum(r * k for _, _, r, k in lay) == sum(r * k for _, (r, k), _ in shapes)


def test_workspace_sizes_are_monotone():
    b = _b()
    c = b.make_config(get_config("d20"))
    assert b.nc_workspace_size(c, True) > b.nc_workspace_size(c, False) > 0


@pytest.mark.parametrize("field,value,code", [
    ("n_layer", 0, -2), ("vocab", 1, -2), ("batch", 0, -2), ("d_model", 4, -2),
    ("head_dim", 96, -7), ("n_kv_head", 2, -7), ("seq_len", 100, -7), ("dtype", 5, -3),
    ("softcap", 0.0, -2), ("softcap", 100.0, -7), ("rms_eps", -1.0, -2), ("d_mlp", 12, -7), ("d_model", 136, -7),
])
def test_bad_configs_are_rejected(field, value, code):
    b = _b()
    cfg = get_config("tiny")
    cfg[field] = value
    c = b.make_config(cfg) if field != "dtype" else b.make_config({**cfg, "dtype": 5})
    with pytest.raises(b.NcError) as ei:
        b.nc_param_count(c)
    assert ei.value.code == code


def test_null_and_alignment_and_workspace_errors_before_device_work():
    b = _b()
    c = b.make_config(get_config("tiny"))
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_loss(c, None, 256, 256, 256, 256, 1 << 20, None)
    assert ei.value.code == -1
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_loss(c, 0x1000 + 8, 256, 256, 256, 512, 1 << 30, None)
    assert ei.value.code == -5
    need = b.nc_workspace_size(c, False)
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_loss(c, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, need - 1, None)
    assert ei.value.code == -4
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_token_loss(c, 0x1000, 0x2000, 0x3000, 0x4000, 0x6000 + 4, 0x5000, need,
                                None)
    assert ei.value.code == -5
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_token_loss(c, 0x1000, 0x2000, 0x3000, 0x4000, 0x6000, 0x5000, need - 1,
                                None)
    assert ei.value.code == -4
    need_b = b.nc_workspace_size(c, True)
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_backward(c, 0x1000, 0x2000, 0x3000, 0x4000, 0x6000, 0x5000, need_b - 1,
                              None)
    assert ei.value.code == -4
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_backward(c, 0x1000, 0x2000, 0x3000, 0x4000, None, 0x5000, need_b, None)
    assert ei.value.code == -1
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_backward(c, 0x1000, 0x2000, 0x3000, 0x4000, 0x6000 + 16, 0x5000, need_b,
                              None)
    assert ei.value.code == -5


def test_step_calls_have_the_three_call_boundary_signatures():
    """nc_init_params, nc_forward_loss and nc_forward_backward take exactly the
    arguments of the three-call boundary: (cfg, seed, params, stream),
    (cfg, params, tokens, targets, loss, ws, ws_bytes, stream) and
    (cfg, params, tokens, targets, loss, grads, ws, ws_bytes, stream)."""
    with open(os.path.join(ROOT, "include", "nc.h")) as f:
        text = " ".join(f.read().split())

    def args(fn):
        m = re.search(r"int " + fn + r"\(([^)]*)\);", text)
        assert m, fn
        return [a.strip().split()[-1].lstrip("*") for a in m.group(1).split(",")]

    assert args("nc_init_params") == ["cfg", "seed", "params", "stream"]
    assert args("nc_forward_loss") == ["cfg", "params", "tokens", "targets", "loss", "ws",
                                       "ws_bytes", "stream"]
    assert args("nc_forward_backward") == ["cfg", "params", "tokens", "targets", "loss",
                                           "grads", "ws", "ws_bytes", "stream"]


def test_pack_rounds_to_nearest_even():
    """Model.pack converts fp32 to bf16 the way the library does (round to
    nearest, ties to even), checked on values whose rounding is known."""
    b = _b()
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9,
                  -(1.0 + 2.0 ** -8 + 2.0 ** -12), 3.0e-3], dtype=np.float32)
    bits = b._bf16_bits_rne(x.copy())
    back = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: even wins (1 + 2^-6)
    assert back[0] == 1.0
    assert back[1] == 1.0
    assert back[2] == 1.0 + 2.0 ** -6
    assert back[3] == 1.0
    assert back[4] == -(1.0 + 2.0 ** -7)
    assert abs(back[5] - np.float32(3.0e-3)) <= 2.0 ** -8 * 3.0e-3


def test_layout_capacity_error():
    b = _b()
    c = b.make_config(get_config("tiny"))
    n = ctypes.c_int32()
    rc = b._lib.nc_param_layout(ctypes.byref(c), None, 0, ctypes.byref(n))
    assert rc == -8 and n.value == 2 + 6 * 2


def test_status_strings():
    b = _b()
    for code in range(-8, 1):
        assert isinstance(b.nc_status_string(code), str) and b.nc_status_string(code)


def test_ops_validation():
    b = _b()
    # bf16 (mn-major A, k-major B) is not built; K must be a multiple of 64
    with pytest.raises(b.NcError) as ei:
        b.nc_op_matmul(1, 8, 8, 64, 0x1000, 8, 0, 0x2000, 64, 1, 0x3000, 8, None, 0, None)
    assert ei.value.code == -7
    with pytest.raises(b.NcError) as ei:
        b.nc_op_matmul(1, 8, 8, 8, 0x1000, 8, 1, 0x2000, 8, 0, 0x3000, 8, None, 0, None)
    assert ei.value.code == -7
    with pytest.raises(b.NcError) as ei:
        b.nc_op_attention_fwd(1, 1, 64, 2, 96, 0x1000, 0x2000, 0x3000, 512, 128, 0x4000, 0x5000,
                              None)
    assert ei.value.code == -7
    with pytest.raises(b.NcError) as ei:
        b.nc_op_softcap_ce(1, 4, 100, 96, 0x1000, 0x2000, 15.0, 0x3000, 0.25, 0x4000, 1, None)
    assert ei.value.code == -2
    # the widest row the cross-entropy kernel holds: 131072 bf16 / 65536 fp32
    # columns (the step's own vocabulary cap); one chunk more is refused
    for dtype, cap in ((1, 131072), (0, 65536)):
        with pytest.raises(b.NcError) as ei:
            b.nc_op_softcap_ce(dtype, 4, 100, cap + 8, 0x1000, 0x2000, 15.0, 0x3000, 0.25,
                               0x4000, 1, None)
        assert ei.value.code == -7
    # the attention flag does not relax the shape checks
    with pytest.raises(b.NcError) as ei:
        b.nc_op_attention_fwd(1, 1, 48, 2, 64, 0x1000, 0x2000, 0x3000, 128, 64, 0x4000, 0x5000,
                              None, qk_normed=1)
    assert ei.value.code == -7
    for dtype, vocab in (("bf16", 131072), ("f32", 65536)):
        c = b.make_config({**get_config("tiny"), "dtype": dtype, "vocab": vocab})
        assert b.nc_param_count(c) > 0
        c = b.make_config({**get_config("tiny"), "dtype": dtype, "vocab": vocab + 1})
        with pytest.raises(b.NcError) as ei:
            b.nc_param_count(c)
        assert ei.value.code == -7


def test_embedding_grad_validation_before_device_work():
    """Shape, pointer, alignment and workspace checks of the embedding
    gradient entry point, all before any device work."""
    b = _b()
    need = b.nc_op_embedding_grad_ws_bytes(1000, 132, 700)
    assert need > 0
    assert b.nc_op_embedding_grad_ws_bytes(2000, 132, 700) > need   # grows with N
    cases = [
        ((0, 132, 700, 0x1000, 0x2000, 0x3000, 0x10000, need), -2),       # N < 1: config
        ((1000, 130, 700, 0x1000, 0x2000, 0x3000, 0x10000, need), -7),    # D % 4: unsupported
        ((1000, 132, 0, 0x1000, 0x2000, 0x3000, 0x10000, need), -2),      # V < 1
        ((1000, 132, 700, 0, 0x2000, 0x3000, 0x10000, need), -1),         # null de
        ((1000, 132, 700, 0x1000, 0x2000, 0x3000, 0, need), -1),          # null workspace
        ((1000, 132, 700, 0x1004, 0x2000, 0x3000, 0x10000, need), -5),    # de not 16-aligned
        ((1000, 132, 700, 0x1000, 0x2000, 0x3000, 0x10010, need), -5),    # ws not 256-aligned
        ((1000, 132, 700, 0x1000, 0x2000, 0x3000, 0x10000, need - 1), -4),  # ws too small
    ]
    for args, code in cases:
        with pytest.raises(b.NcError) as ei:
            b.nc_op_embedding_grad(*args, None)
        assert ei.value.code == code, (args, ei.value.code)


def test_matmul_epilogue_validation_before_device_work():
    """Every argument check of the fused-epilogue product fails before a launch,
    so none of these fake addresses is ever dereferenced."""
    b = _b()
    A, B, C, RS, AUX = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000

    def call(**kw):
        a = dict(dtype=1, M=8, N=8, K=64, A=A, lda=64, a_kmajor=1, B=B, ldb=64, b_kmajor=1,
                 Cp=C, ldc=8, mode=5, rowscale=None, aux=None, stream=None)
        a.update(kw)
        with pytest.raises(b.NcError) as ei:
            b.nc_op_matmul_epilogue(**a)
        return ei.value.code

    assert call(dtype=7) == -3
    assert call(M=0) == -2 and call(N=0) == -2 and call(K=0) == -2
    assert call(mode=0) == -2 and call(mode=6) == -2
    # the row-scaled modes need rowscale, the residual and relu^2 backward need aux
    for mode in (1, 2, 4):
        assert call(mode=mode, aux=AUX) == -1
    for mode in (3, 4):
        assert call(mode=mode, rowscale=RS) == -1
    assert call(A=None) == -1 and call(B=None) == -1 and call(Cp=None) == -1
    assert call(A=A + 8) == -5 and call(Cp=C + 4) == -5
    assert call(mode=3, aux=AUX + 8) == -5
    # leading dimensions shorter than the rows they hold
    assert call(ldc=4) == -2
    assert call(lda=32) == -2 and call(a_kmajor=0, lda=4) == -2
    assert call(ldb=32) == -2 and call(b_kmajor=0, ldb=4) == -2
    # bf16: an mn-major A is not built; an mn-major B only with the
    # data-gradient modes; K a multiple of 64
    assert call(a_kmajor=0, lda=8) == -7
    for mode in (1, 2, 3):
        assert call(mode=mode, b_kmajor=0, ldb=8, rowscale=RS, aux=AUX) == -7
    assert call(K=96, lda=96, ldb=96) == -7
    assert call(lda=68) == -7
    # fp32 runs every operand-major pair, so only the generic checks apply
    assert call(dtype=0, A=None, a_kmajor=0, lda=8) == -1


OCFG = dict(adam_lr=3e-3, adam_beta1=0.8, adam_beta2=0.95, adam_eps=1e-10,
            adam_weight_decay=0.0, muon_lr=0.02, muon_momentum=0.95, muon_weight_decay=0.0,
            muon_nesterov=1, muon_ns_steps=5, grad_clip=1.0)


def test_lr_multiplier_matches_the_oracle_schedule():
    """The library's host-side schedule against the oracle's, step by step."""
    import oracle.optim as oo
    b = _b()
    for total, warmup, f in ((100, 10, 0.1), (50, 0, 0.0), (7, 7, 1.0), (1000, 37, 0.25)):
        for step in list(range(0, total + 3)) + [10 * total]:
            assert b.nc_lr_multiplier(step, total, warmup, f) == pytest.approx(
                oo.lr_multiplier(step, total, warmup, f), rel=1e-14, abs=1e-15)
    for args in ((0, 0, 0, 0.1), (0, 10, -1, 0.1), (0, 10, 1, 1.5), (-1, 10, 1, 0.1)):
        with pytest.raises(b.NcError):
            b.nc_lr_multiplier(*args)


def test_optimizer_validation_before_device_work():
    b = _b()
    c = b.make_config(get_config("tiny"))
    ws = b.nc_optim_workspace_size(c)
    st = b.nc_optim_state_size(c)
    n = b.nc_param_count(c)
    assert st == 3 * (((n * 4 + 255) // 256) * 256)
    assert ws > 0
    o = b.make_optim_config(OCFG)
    args = lambda **kw: dict(dict(step=1, lr_mult=1.0, grads=0x1000, params=0x2000, state=0x3000,
                                  norm=None, ws=0x4000, wsb=ws), **kw)

    def call(oc=o, **kw):
        a = args(**kw)
        b.nc_optim_step(c, oc, a["step"], a["lr_mult"], a["grads"], a["params"], a["state"],
                        a["norm"], a["ws"], a["wsb"], None)

    for kw, code in ((dict(step=0), -2), (dict(lr_mult=-1.0), -2), (dict(grads=None), -1),
                     (dict(params=0x2000 + 16), -5), (dict(norm=0x5002), -5),
                     (dict(wsb=ws - 1), -4)):
        with pytest.raises(b.NcError) as ei:
            call(**kw)
        assert ei.value.code == code, kw
    for field, value in (("adam_beta1", 1.0), ("adam_eps", 0.0), ("muon_momentum", -0.1),
                         ("muon_ns_steps", 17), ("grad_clip", -1.0), ("muon_nesterov", 2),
                         ("adam_lr", float("nan"))):
        with pytest.raises(b.NcError) as ei:
            call(oc=b.make_optim_config({**OCFG, field: value}))
        assert ei.value.code == -2, field
    with pytest.raises(b.NcError) as ei:
        b.nc_grad_accumulate(0x1000 + 4, 0x2000, 10, 0.5, 0, None)
    assert ei.value.code == -5


def test_binding_and_torch_share_one_hip_runtime():
    """Importing the binding before torch must not map a second HIP runtime
    (torch bundles its own copy under the system runtime's soname)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import dense_gpt_pretraining_amd.binding\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(libs))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_generation_validation_before_device_work():
    b = _b()
    cfg = get_config("d20", batch=4)
    c = b.make_config(cfg)
    cache = b.nc_kv_cache_size(c, 320)
    assert cache == 2 * 20 * 4 * 320 * 128 * 2
    ws_dec = b.nc_infer_workspace_size(c, 320, 0)
    ws_pre = b.nc_infer_workspace_size(c, 320, 256)
    assert ws_pre >= ws_dec > 0
    for t0, code in ((100, -2), (0, -2), (384, -2)):
        with pytest.raises(b.NcError) as ei:
            b.nc_prefill(c, 0x1000, 0x2000, t0, 320, 0x3000, 0x4000, 0x5000, ws_pre, None)
        assert ei.value.code == code, t0
    with pytest.raises(b.NcError) as ei:
        b.nc_prefill(c, 0x1000, 0x2000, 256, 320, 0x3000, 0x4000, 0x5000, ws_pre - 1, None)
    assert ei.value.code == -4
    for pos, code in ((-1, -2), (320, -2)):
        with pytest.raises(b.NcError) as ei:
            b.nc_decode_step(c, 0x1000, 0x2000, pos, 320, 0x3000, 0x4000, 0x5000, ws_dec, None)
        assert ei.value.code == code, pos
    with pytest.raises(b.NcError) as ei:
        b.nc_decode_step(c, 0x1000, 0x2000, 5, 320, 0x3000 + 64, 0x4000, 0x5000, ws_dec, None)
    assert ei.value.code == -5
    big = b.make_config({**cfg, "batch": 33})
    with pytest.raises(b.NcError) as ei:
        b.nc_decode_step(big, 0x1000, 0x2000, 5, 320, 0x3000, 0x4000, 0x5000, 1 << 40, None)
    assert ei.value.code == -7
    heads = b.make_config({**cfg, "n_head": 17})
    with pytest.raises(b.NcError) as ei:
        b.nc_kv_cache_size(heads, 320)
    assert ei.value.code == -7
