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
    for h in ("nc.h", "nc_ops.h"):
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
        b.nc_forward_loss(c, None, 256, 256, 256, None, 256, 1 << 20, None)
    assert ei.value.code == -1
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_loss(c, 0x1000 + 8, 256, 256, 256, None, 512, 1 << 30, None)
    assert ei.value.code == -5
    need = b.nc_workspace_size(c, False)
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_loss(c, 0x1000, 0x2000, 0x3000, 0x4000, None, 0x5000, need - 1, None)
    assert ei.value.code == -4
    need_b = b.nc_workspace_size(c, True)
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_backward(c, 0x1000, 0x2000, 0x3000, 0x4000, None, 0x6000, 0x5000,
                              need_b - 1, None)
    assert ei.value.code == -4
    with pytest.raises(b.NcError) as ei:
        b.nc_forward_backward(c, 0x1000, 0x2000, 0x3000, 0x4000, None, None, 0x5000, need_b, None)
    assert ei.value.code == -1


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
