"""Writes tests/golden/training_curves.json from the oracle alone.

A short training run on one fixed batch: the oracle's forward+backward
(float64) followed by its optimizer step (Muon on the block matrices, AdamW on
the embeddings, global-norm clipping, warm-up + cosine schedule), repeated.
The file records the settings and the loss before every step, for the tiny
configuration (30 steps) and a two-layer d20-shaped configuration (20 steps,
sequence 256, batch 2; about five minutes).  The GPU test runs the same loop
through the library and compares its losses with these.  Run from the
repository root:
    python tests/golden/make_training_curves.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import oracle.optim as oo  # noqa: E402
from nc_synth import get_config, make_params, make_tokens  # noqa: E402

OCFG = dict(adam_lr=1e-2, adam_beta1=0.8, adam_beta2=0.95, adam_eps=1e-10,
            adam_weight_decay=0.01, muon_lr=0.02, muon_momentum=0.95, muon_weight_decay=0.01,
            muon_nesterov=1, muon_ns_steps=5, grad_clip=1.0)
RUNS = [("tiny", {}, 30), ("d20", {"n_layer": 2, "seq_len": 256, "batch": 2}, 20)]
WARMUP, FINAL = 3, 0.1


def curve(name, over, steps):
    cfg = get_config(name, **over)
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg)
    st = oo.init_state(params)
    losses = []
    for t in range(1, steps + 1):
        cur = {k: st["master"][k] for k in params}
        loss, grads = oracle.forward_backward(cfg, cur, tokens, targets)
        losses.append(float(loss))
        oo.step(OCFG, st, grads, t, oo.lr_multiplier(t - 1, steps, WARMUP, FINAL))
    return losses


def main():
    out = {"written_by": "tests/golden/make_training_curves.py (calls only oracle/ and nc_synth)",
           "optimizer": OCFG, "warmup": WARMUP, "final_frac": FINAL, "runs": []}
    for name, over, steps in RUNS:
        out["runs"].append({"config": name, "over": over, "steps": steps,
                            "losses": curve(name, over, steps)})
        print(name, out["runs"][-1]["losses"][::5], flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "training_curves.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
