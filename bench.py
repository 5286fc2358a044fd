#!/usr/bin/env python3
"""Throughput of one forward+backward pretraining step of the depth-20
nanochat-style decoder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d20]

A step is nc_forward_backward over one batch of synthetic tokens (Zipf(1.1)
ids, seeded) with parameters drawn on the device by nc_init_params; all
inputs are resident in HBM before timing starts.  W untimed steps run first,
then K steps are timed between two device synchronisations (HIP events on the
stream the library launches on).  value = tokens per second; MFU uses the
causal flop count 6*N_matmul + 6*L*H*hd*(T+1) per token against the bf16
dense MFMA peak of 2516.6 TFLOP/s.

roofline: the kernel with the largest share of the step (by summed duration)
from nc_forward_backward_timed, which brackets each kernel with HIP events on
the stream it runs on; achieved = its algorithmic flops (or bytes) per launch
over its mean launch duration.  traffic = HBM bytes per launch measured with
rocprofv3 counters (profiles/<config>_hbm_traffic.md), null when that record
does not match the kernel's current sources.

cpu_baseline: the float64 oracle (test infrastructure, unchanged) timed on
this host for a forward+backward over one sequence of the same workload;
tokens/s of that sample.  A baseline, not the target.

Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec and bf16 MFU, fwd+bwd step, depth-20 model on 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def step_flops(cfg):
    """Causal algorithmic flops of one fwd+bwd step (recompute not counted)."""
    D, H, hd, F, V, L = (cfg[k] for k in ("d_model", "n_head", "head_dim", "d_mlp", "vocab",
                                          "n_layer"))
    T, B = cfg["seq_len"], cfg["batch"]
    n_mm = L * ((H + 2) * hd * D + D * H * hd + 2 * F * D) + V * D
    per_tok = 6 * n_mm + 6 * L * H * hd * (T + 1)
    return per_tok * B * T, 6 * n_mm * B * T + 12 * L * H * hd * T * B * T


def workload_name(name, cfg):
    return (f"{name}: nanochat decoder L{cfg['n_layer']} D{cfg['d_model']} "
            f"H{cfg['n_head']}x{cfg['head_dim']} MQA F{cfg['d_mlp']} V{cfg['vocab']}, "
            f"seq {cfg['seq_len']} x batch {cfg['batch']}, fwd+bwd")


def timed_kernels(model, params, tok, tgt, reps):
    """Per-kernel stats from the timed step variant, averaged over reps."""
    import torch
    from dense_gpt_pretraining_amd import binding as b

    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    grads = torch.empty(model.n_params, dtype=torch.float32, device="cuda")
    ws = model.workspace(True)
    acc = {}
    for _ in range(reps):
        stats = b.nc_forward_backward_timed(model.c, params.data_ptr(), tok.data_ptr(),
                                            tgt.data_ptr(), loss.data_ptr(), grads.data_ptr(),
                                            ws.data_ptr(), ws.numel(), model.stream())
        for st in stats:
            a = acc.setdefault(st["name"], [0, 0.0, 0.0, 0.0])
            a[0] += st["launches"]
            a[1] += st["ms"]
            a[2] += st["flops"]
            a[3] += st["bytes"]
    return {k: dict(launches=v[0] / reps, ms=v[1] / reps, flops=v[2] / reps, bytes=v[3] / reps)
            for k, v in acc.items()}


def measured_traffic(config_name, label):
    """HBM bytes per launch of kernel `label` from the committed rocprofv3 PMC
    summary (FETCH_SIZE and WRITE_SIZE runs scaled by a copy-kernel
    calibration), or None when there is no record or the kernel's sources
    have changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{config_name}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get("kernels", {}).get(label)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        fp = os.path.join(ROOT, f)
        if not os.path.exists(fp):
            return None
        with open(fp, "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return float(rec["bytes_per_launch"])


def cpu_baseline(cfg):
    """The oracle's fwd+bwd on one sequence of the workload, on host cores."""
    import numpy as np

    import oracle
    from nc_synth import make_params, make_tokens
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    params = make_params(cfg)
    tokens, targets = make_tokens(cfg, batch=1)
    t0 = time.perf_counter()
    loss, _ = oracle.forward_backward(cfg, params, tokens, targets)
    dt = time.perf_counter() - t0
    assert math.isfinite(loss)
    ntok = tokens.size
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one sequence ({ntok} tokens, batch 1) of the same workload, float64 "
                      f"NumPy fwd+bwd, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d20")
    ap.add_argument("--profile-reps", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dense_gpt_pretraining_amd import Model
    from nc_synth import get_config, make_tokens

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = get_config(args.config)
    model = Model(cfg)
    params = model.init_params(cfg["seed_params"])
    tokens, targets = make_tokens(cfg)
    tok = torch.from_numpy(tokens).cuda()
    tgt = torch.from_numpy(targets).cuda()
    grads = torch.empty(model.n_params, dtype=torch.float32, device="cuda")
    ntok = tokens.size
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        loss, _ = model.forward_backward(params, tok, tgt, grads=grads)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        loss, _ = model.forward_backward(params, tok, tgt, grads=grads)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    lval = float(loss.item())
    assert math.isfinite(lval), lval

    flops, flops_noncausal = step_flops(cfg)
    tps = ntok / (ms / 1e3)
    mfu = flops / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12)

    kern = timed_kernels(model, params, tok, tgt, args.profile_reps)
    total_k = sum(v["ms"] for v in kern.values())
    dom_name, dom = max(kern.items(), key=lambda kv: kv[1]["ms"])
    per_launch_ms = dom["ms"] / max(dom["launches"], 1)
    if dom["flops"] > 0:
        bound = "mfma" if cfg["dtype"] == "bf16" else "alu"
        peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_FP32_TFLOPS
        achieved = dom["flops"] / (dom["ms"] / 1e3) / 1e12
        unit = "TFLOP/s"
    else:
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        achieved = dom["bytes"] / (dom["ms"] / 1e3) / 1e9
    traffic = measured_traffic(args.config, dom_name)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": round(dom["bytes"] / max(dom["launches"], 1)),
                "kernel": dom_name,
                "launches_per_step": dom["launches"], "mean_launch_ms": round(per_launch_ms, 4),
                "share_of_step": round(dom["ms"] / total_k, 4)}
    kernels = []
    for k, v in sorted(kern.items(), key=lambda kv: -kv[1]["ms"]):
        e = {"name": k, "launches": v["launches"], "ms": round(v["ms"], 3)}
        if v["flops"] > 0:
            e["tflops"] = round(v["flops"] / (v["ms"] / 1e3) / 1e12, 1)
        e["gbs"] = round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1)
        kernels.append(e)

    cpu = cpu_baseline(cfg)

    out = {
        "metric": METRIC,
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "mfu": round(mfu, 4),
        "mfu_noncausal_count": round(flops_noncausal / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "step_tflop": round(flops / 1e12, 2),
        "loss": round(lval, 6),
        "wall_s": round(wall, 3),
        "config": {"workload": workload_name(args.config, cfg), "global_batch": cfg["batch"],
                   "seq_len": cfg["seq_len"], "tokens_per_step": ntok,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
