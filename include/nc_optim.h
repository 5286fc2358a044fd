/*
 * nc_optim.h -- the optimizer step that follows nc_forward_backward: Muon for
 * the block matrices and AdamW for the embedding and the unembedding, with
 * gradient accumulation, a learning-rate schedule and clipping by the global
 * gradient norm.
 *
 * The nanochat article (vpshk.cn, section on the ~8000-line code base,
 * optimizer paragraph) names Muon combined with AdamW; the llm.c article
 * (qian.cx, training-command paragraph) adds gradient accumulation, a
 * GPT-3-style learning-rate schedule, weight decay and the gradient norm.
 * The pages define none of them; each follows its published definition:
 *   AdamW  Kingma & Ba (ICLR 2015) with weight decay decoupled as in
 *          Loshchilov & Hutter (ICLR 2019):
 *            m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *            theta = theta (1 - lr wd) - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)
 *   Muon   K. Jordan et al. (2024): B = mu B + g; U = g + mu B (Nesterov) or
 *          B; X = U / (|U|_F + 1e-7) in the orientation with rows <= cols;
 *          `ns_steps` times X = a X + (b A + c A^2) X with A = X X^T and
 *          (a, b, c) = (3.4445, -4.7750, 2.0315);
 *          theta = theta (1 - lr wd) - lr sqrt(max(1, rows/cols)) X.
 *          bf16 configurations run the iteration on the matrix cores with
 *          bf16 operands and fp32 accumulation; fp32 ones in fp32.
 * Muon takes every block matrix (wq, wk, wv, wo, wfc, wproj, each a matrix
 * of its own); AdamW takes wte and wlm.
 *
 * Conventions are those of nc.h (device pointers except cfg / ocfg, caller-
 * owned buffers, stream order, host-side validation before any device work,
 * NC_* status codes).  Gradients are fp32 in the parameter layout; padding
 * between tensors is never read.
 */
#ifndef NC_OPTIM_H
#define NC_OPTIM_H

#include <stddef.h>
#include <stdint.h>

#include "nc.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nc_optim_config {
    float adam_lr;            /* peak learning rate of wte and wlm (>= 0) */
    float adam_beta1;         /* [0, 1) */
    float adam_beta2;         /* [0, 1) */
    float adam_eps;           /* > 0 */
    float adam_weight_decay;  /* >= 0, decoupled */
    float muon_lr;            /* peak learning rate of the block matrices (>= 0) */
    float muon_momentum;      /* mu in [0, 1) */
    float muon_weight_decay;  /* >= 0, decoupled */
    int32_t muon_nesterov;    /* 1: U = g + mu B; 0: U = B */
    int32_t muon_ns_steps;    /* Newton-Schulz iterations, 0 .. 16 (5 in the published method) */
    float grad_clip;          /* > 0: gradients scaled by min(1, grad_clip / (|g| + 1e-6)),
                                 |g| the global L2 norm; 0: no clipping */
} nc_optim_config;

/*
 * Optimizer state: three fp32 arrays in the parameter layout (nc_param_count
 * elements each): the fp32 master weights, then for AdamW tensors the first
 * and second moments, for Muon tensors the momentum buffer and an unused
 * array.  256-byte aligned.
 */
int nc_optim_state_size(const nc_config* cfg, size_t* bytes);

/* Scratch of nc_optim_step (norm partials, the iteration's matrices). */
int nc_optim_workspace_size(const nc_config* cfg, size_t* bytes);

/* state: master = params (as fp32), moments and momentum = 0. */
int nc_optim_init(const nc_config* cfg, const void* params, void* state,
                  void* stream);

/*
 * One optimizer step with step number `step` >= 1 (Adam's bias correction
 * uses it) and learning rates ocfg's peaks times lr_mult.  Reads grads (fp32,
 * the gradient of the mean loss), updates state and writes params (cfg's
 * dtype, rounded from the fp32 master to nearest even).  grad_norm: optional
 * (NULL to skip) device fp32 that receives the global L2 norm of grads before
 * clipping.  ws: ws_bytes >= nc_optim_workspace_size.
 */
int nc_optim_step(const nc_config* cfg, const nc_optim_config* ocfg, int64_t step,
                  float lr_mult, const float* grads, void* params, void* state,
                  float* grad_norm, void* ws, size_t ws_bytes, void* stream);

/*
 * Gradient accumulation over micro-batches of equal size:
 * acc = (overwrite ? 0 : acc) + scale * grads over n fp32 elements (with
 * scale = 1 / number of micro-batches, acc ends as the gradient of the mean
 * loss over all of them).  16-byte aligned pointers.
 */
int nc_grad_accumulate(float* acc, const float* grads, int64_t n, float scale,
                       int32_t overwrite, void* stream);

/*
 * Learning-rate multiplier of 0-based step `step` out of `total`: linear
 * warm-up (step+1)/warmup over the first `warmup` steps, then a cosine from 1
 * to final_frac at step `total`, final_frac afterwards (GPT-3's schedule
 * decays to 0.1).  Host function; returns -1 for total < 1, warmup < 0 or
 * final_frac outside [0, 1].
 */
double nc_lr_multiplier(int64_t step, int64_t total, int64_t warmup, double final_frac);

#ifdef __cplusplus
}
#endif
#endif /* NC_OPTIM_H */
