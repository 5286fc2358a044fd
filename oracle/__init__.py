"""The oracle: plain float64 CPU reference of the nanochat-style dense decoder
forward and backward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The GPU library never imports, links or calls anything here.
"""
from .model import (
    causal_mqa_attention,
    causal_mqa_attention_backward,
    embedding_gradient,
    forward_backward,
    forward_logits,
    forward_loss,
    rms_norm,
    rms_norm_backward,
    rotary,
    rotary_backward,
    rotary_tables,
    softcap,
    softcap_cross_entropy,
)

__all__ = [
    "causal_mqa_attention", "causal_mqa_attention_backward", "embedding_gradient",
    "forward_backward", "forward_logits", "forward_loss", "rms_norm", "rms_norm_backward",
    "rotary", "rotary_backward", "rotary_tables", "softcap",
    "softcap_cross_entropy",
]
