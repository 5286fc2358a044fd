"""Writes tests/golden/oracle_tiny.txt from the oracle alone.

The file records the oracle's loss and per-tensor gradient norms on the tiny
configuration with the seeded inputs, so a later change to the oracle's
arithmetic shows up as a diff.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from nc_synth import get_config, make_params, make_tokens  # noqa: E402


def main():
    cfg = get_config("tiny")
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    loss, grads = oracle.forward_backward(cfg, params, tokens, targets)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.txt")
    with open(out, "w") as f:
        f.write("# oracle float64 on the tiny configuration, seeds data=0 params=1\n")
        f.write("# written by tests/golden/make_golden.py (calls only oracle/ and nc_synth)\n")
        f.write(f"loss {loss!r}\n")
        for k in sorted(grads):
            f.write(f"gradnorm {k} {float(np.linalg.norm(grads[k]))!r}\n")


if __name__ == "__main__":
    main()
