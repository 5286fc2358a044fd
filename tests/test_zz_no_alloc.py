"""nc_decode_step_noalloc (the decode step with its workspace in the
library's own per-GPU array) against nc_decode_step with a caller workspace:
bitwise the same logits and cache rows, on two calls in a row, the second
with a smaller input, and the over-limit case refused."""
import numpy as np
import pytest

from nc_synth import get_config, make_params, make_tokens
from tests.gpu_helpers import require_gpu, stream

pytestmark = pytest.mark.gpu


def _case(name, over, t0, positions, max_seq):
    from dense_gpt_pretraining_amd import Generator, Model, binding as b
    torch = require_gpu()
    cfg = get_config(name, **over)
    m = Model(cfg)
    p = m.pack(make_params(cfg))
    tokens = make_tokens(get_config(name, seq_len=max_seq), batch=cfg["batch"])[0]
    gen = Generator(m, max_seq=max_seq, max_prefill=t0)
    if t0:
        gen.prefill(p, tokens[:, :t0])
    cache2 = gen.cache.clone()
    logits2 = torch.empty_like(gen.logits)
    for pos in positions:
        tok = torch.from_numpy(np.ascontiguousarray(tokens[:, pos])).cuda()
        want = gen.decode(p, tok, pos).clone()
        b.nc_decode_step_noalloc(m.c, p.data_ptr(), tok.data_ptr(), pos, max_seq,
                                 cache2.data_ptr(), logits2.data_ptr(), stream())
        torch.cuda.synchronize()
        assert bool(torch.equal(want, logits2)), (name, pos)
        assert bool(torch.equal(gen.cache, cache2)), (name, pos)


def test_no_alloc_decode_matches_the_workspace_decode_on_two_calls():
    # first call: bf16, 8 sequences, a 512-position cache after a prefill;
    # every position after the prompt is decoded in turn (the cache must hold
    # the sequence so far)
    _case("d20", dict(n_layer=2, batch=8), 256, list(range(256, 301)), 512)
    # second call, smaller: 2 sequences, one layer, 128 positions, from empty
    _case("d20", dict(n_layer=1, batch=2), 0, list(range(0, 64)), 128)


def test_no_alloc_decode_refuses_workspaces_beyond_the_array():
    from dense_gpt_pretraining_amd import Model, binding as b
    require_gpu()
    cfg = get_config("d20", batch=32)
    m = Model(cfg)
    big = 1 << 17                      # the step's workspace outgrows 32 MiB
    assert b.nc_infer_workspace_size(m.c, big, 0) > (32 << 20)
    with pytest.raises(b.NcError) as ei:
        b.nc_decode_step_noalloc(m.c, 0x1000, 0x2000, 0, big, 0x3000, 0x4000, stream())
    assert ei.value.code == -4
