#!/usr/bin/env python3
"""Throughput of one forward+backward pretraining step of the depth-20
nanochat-style decoder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d20] [--batch B]
                    [--gemm-comparison 0|1]

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


OPTIM = dict(adam_lr=3e-3, adam_beta1=0.8, adam_beta2=0.95, adam_eps=1e-10,
             adam_weight_decay=0.0, muon_lr=0.02, muon_momentum=0.95, muon_weight_decay=0.0,
             muon_nesterov=1, muon_ns_steps=5, grad_clip=1.0)


def optimizer_work(cfg, ns_steps):
    """Algorithmic work of one optimizer step: Newton-Schulz flops (three
    products per iteration per block matrix) and the HBM bytes of the
    elementwise passes (AdamW: g, master, m, v read, master, m, v, param
    written; Muon: momentum, X0 and update passes; the global norm reads g)."""
    D, H, hd, F, V, L = (cfg[k] for k in ("d_model", "n_head", "head_dim", "d_mlp", "vocab",
                                          "n_layer"))
    es = 2 if cfg["dtype"] == "bf16" else 4
    flops, muon_elems = 0.0, 0
    for r, c in ((H * hd, D), (hd, D), (hd, D), (D, H * hd), (F, D), (D, F)):
        m, n = min(r, c), max(r, c)
        flops += L * ns_steps * (2.0 * m * m * n + 2.0 * m * m * m + 2.0 * m * m * n)
        muon_elems += L * r * c
    adam_elems = 2 * V * D
    nbytes = (adam_elems + muon_elems) * 4                       # global norm
    nbytes += adam_elems * (4 + 3 * 8 + es)                      # AdamW
    nbytes += muon_elems * ((4 + 8) + (4 + 4 + es) + (es + 8 + es))  # momentum, X0, update
    return flops, nbytes


def optimizer_timing(model, params, grads, cfg, steps):
    """Mean duration of nc_optim_step (Muon + AdamW) on the workload's
    parameters and the gradients of the last timed step."""
    import torch

    from dense_gpt_pretraining_amd import Optimizer
    opt = Optimizer(model, OPTIM)
    opt.init(params)
    for t in range(1, 3):
        opt.step(params, grads, t, 1.0)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for t in range(3, 3 + steps):
        opt.step(params, grads, t, 1.0)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    flops, nbytes = optimizer_work(cfg, OPTIM["muon_ns_steps"])
    return {"ms_per_step": round(ms, 3), "newton_schulz_tflop": round(flops / 1e12, 3),
            "elementwise_gb": round(nbytes / 1e9, 3),
            "note": "Muon (5 Newton-Schulz iterations, bf16 matrix cores) on every block matrix, "
                    "AdamW on wte and wlm, global-norm clipping; not part of the fwd+bwd metric"}


def generation_timing(model, params, cfg, tokens):
    """Prefill of the batch's first T-64 positions, then 64 decode steps (one
    token per sequence each) up to position T-1; HBM bytes of a decode step:
    every matrix weight read once, the embedding rows and the cache rows the
    step reads (keys and values of every earlier position, all layers)."""
    import torch

    from dense_gpt_pretraining_amd import Generator
    B, T = tokens.shape
    t0 = T - 64
    gen = Generator(model, max_seq=T, max_prefill=t0)
    tok = torch.from_numpy(tokens).cuda()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    gen.prefill(params, tok[:, :t0])          # warm-up of the prefill path
    torch.cuda.synchronize()
    ev[0].record()
    gen.prefill(params, tok[:, :t0])
    ev[1].record()
    for pos in range(t0, T):
        gen.decode(params, tok[:, pos], pos)
    ev[2].record()
    torch.cuda.synchronize()
    pre_ms = ev[0].elapsed_time(ev[1])
    dec_ms = ev[1].elapsed_time(ev[2]) / (T - t0)
    D, H, hd, F, V, L = (cfg[k] for k in ("d_model", "n_head", "head_dim", "d_mlp", "vocab",
                                          "n_layer"))
    es = 2 if cfg["dtype"] == "bf16" else 4
    w_bytes = (L * ((H + 2) * hd * D + D * H * hd + 2 * F * D) + V * D) * es + B * D * es
    mean_pos = (t0 + T - 1) / 2.0 + 1
    kv_bytes = 2 * L * B * mean_pos * hd * es
    return {"prefill_ms": round(pre_ms, 3), "prefill_tokens_per_s": round(B * t0 / pre_ms * 1e3, 1),
            "decode_ms_per_step": round(dec_ms, 4),
            "decode_tokens_per_s": round(B / dec_ms * 1e3, 1),
            "decode_hbm_gb_per_step": round((w_bytes + kv_bytes) / 1e9, 4),
            "decode_hbm_gbs": round((w_bytes + kv_bytes) / (dec_ms / 1e3) / 1e9, 1),
            "shape": f"batch {B}, prefill {t0} positions, decode positions {t0}..{T - 1}"}


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


def gemm_comparison(cfg):
    """The step's plain GEMM shapes timed twice on the same device: the
    library's kernel through its unit entry points (bf16 output for the
    forward and data-gradient layouts, fp32 with its k-split for the weight
    gradients, as in the step) and torch.mm (the vendor BLAS) on contiguous
    row-major operands.  A reference point for the kernels' rates, not part
    of the metric."""
    import torch

    from dense_gpt_pretraining_amd import binding as b
    D, hd, H, F, V = (cfg[k] for k in ("d_model", "head_dim", "n_head", "d_mlp", "vocab"))
    N_tok = cfg["batch"] * cfg["seq_len"]
    Wq = (H + 2) * hd
    # (name, M, N, K, layout): "fwd" = X W^T, "dgrad" = dY W, "wgrad" = dY^T X
    shapes = [("fc forward", N_tok, F, D, "fwd"), ("qkv forward", N_tok, Wq, D, "fwd"),
              ("proj forward", N_tok, D, F, "fwd"), ("unembedding forward", N_tok, V, D, "fwd"),
              ("fc data gradient", N_tok, D, F, "dgrad"),
              ("fc weight gradient", F, D, N_tok, "wgrad"), ("qkv weight gradient", Wq, D, N_tok, "wgrad")]
    stream = torch.cuda.current_stream().cuda_stream
    out = []

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for name, M, N, K, lay in shapes:
        reps = 3 if 2.0 * M * N * K > 5e12 else 10
        g = torch.Generator(device="cuda").manual_seed(1)
        if lay == "fwd":       # A = X [M, K], B = W [N, K], both k-major
            A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
            Bm = torch.randn(N, K, device="cuda", generator=g).to(torch.bfloat16)
            C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            ours = lambda: b.nc_op_matmul_epilogue(1, M, N, K, A.data_ptr(), K, 1, Bm.data_ptr(),
                                                   K, 1, C.data_ptr(), N, 5, None, None, stream)
        elif lay == "dgrad":   # A = dY [M, K] k-major, B = W [K, N] mn-major
            A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
            Bm = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
            C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            ours = lambda: b.nc_op_matmul_epilogue(1, M, N, K, A.data_ptr(), K, 1, Bm.data_ptr(),
                                                   N, 0, C.data_ptr(), N, 5, None, None, stream)
        else:                  # A = dY [K, M], B = X [K, N], both mn-major; fp32 out
            A = torch.randn(K, M, device="cuda", generator=g).to(torch.bfloat16)
            Bm = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
            C = torch.empty(M, N, device="cuda", dtype=torch.float32)
            ws = torch.empty(32 * M * N, device="cuda", dtype=torch.float32)
            ours = lambda: b.nc_op_matmul(1, M, N, K, A.data_ptr(), M, 0, Bm.data_ptr(), N, 0,
                                          C.data_ptr(), N, ws.data_ptr(), ws.numel() * 4, stream)
        t_ours = timed(ours, reps)
        del A, Bm, C
        torch.cuda.empty_cache()
        # the vendor BLAS on contiguous row-major operands: [M, K] @ [K, N]
        X = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        Y = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
        Z = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        t_mm = timed(lambda: torch.mm(X, Y, out=Z), reps)
        del X, Y, Z
        torch.cuda.empty_cache()
        fl = 2.0 * M * N * K
        out.append({"shape": name, "M": M, "N": N, "K": K,
                    "library_ms": round(t_ours, 4), "library_tflops": round(fl / t_ours / 1e9, 1),
                    "torch_mm_ms": round(t_mm, 4), "torch_mm_tflops": round(fl / t_mm / 1e9, 1)})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d20")
    ap.add_argument("--profile-reps", type=int, default=3)
    ap.add_argument("--generation", type=int, default=1,
                    help="also time prefill and KV-cache decode steps (1) or not (0)")
    ap.add_argument("--optimizer", type=int, default=1,
                    help="also time one Muon + AdamW optimizer step (1) or not (0)")
    ap.add_argument("--cpu-baseline", type=int, default=1,
                    help="also time the oracle on one sequence of the workload (1) or not (0)")
    ap.add_argument("--gemm-comparison", type=int, default=0,
                    help="also time the step's GEMM shapes with the library's kernels and with "
                         "torch.mm (1) or not (0)")
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences per step instead of the configuration's (0: keep it); e.g. "
                         "4 for one GPU's share of d20's 32 sequences over 8 GPUs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dense_gpt_pretraining_amd import Model
    from nc_synth import get_config, make_tokens

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = get_config(args.config, **({"batch": args.batch} if args.batch > 0 else {}))
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
    # the counters were read at the configuration's own batch
    traffic = measured_traffic(args.config, dom_name) if args.batch <= 0 else None
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

    gen = generation_timing(model, params, cfg, tokens) if args.generation else None
    optim = optimizer_timing(model, params, grads, cfg, 5) if args.optimizer else None

    cpu = cpu_baseline(cfg) if args.cpu_baseline else None
    gemms = gemm_comparison(cfg) if args.gemm_comparison and cfg["dtype"] == "bf16" else None

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
        "optimizer_step": optim,
        "generation": gen,
        "kernels": kernels,
    }
    if gemms is not None:
        out["gemm_comparison"] = gemms
    print(json.dumps(out))


if __name__ == "__main__":
    main()
