/*
 * nc_infer.h -- generation with a key/value cache: prefill of a prompt and
 * one-token decode steps of the same model.
 *
 * The nanochat pages list an inference engine with a KV cache and prefill /
 * decode among the project's parts (tianqi.csdn.net feature list; vpshk.cn,
 * section on the $100 run).  What it computes follows from the model: by
 * causality the softcapped logits c_t = s tanh(z_t / s) at position t depend
 * only on tokens 0..t, and the only state position t hands to later
 * positions is, per layer, its rotated and normalised key and its value (one
 * K/V head under multi-query attention, so the cache is 1/H the size a
 * multi-head model needs).  Prefill runs the training forward over a prompt
 * and stores those rows; a decode step runs the model on one new token per
 * sequence, appends its rows, and attends over the cache.
 *
 * Conventions are those of nc.h.  B = cfg->batch sequences; cfg->seq_len is
 * not used (max_seq sizes the cache).  Every sequence of a call is at the
 * same position.
 */
#ifndef NC_INFER_H
#define NC_INFER_H

#include <stddef.h>
#include <stdint.h>

#include "nc.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Cache bytes for max_seq positions: for every layer l a key block then a
 * value block, each [B][max_seq][head_dim] of cfg's dtype (key rows rotated
 * and normalised, as attention reads them).  256-byte aligned.
 */
int nc_kv_cache_size(const nc_config* cfg, int32_t max_seq, size_t* bytes);

/*
 * Workspace of nc_prefill for a prompt of t0 positions and of nc_decode_step
 * (ws_bytes of either call >= this; t0 = 0 sizes decode alone).
 */
int nc_infer_workspace_size(const nc_config* cfg, int32_t max_seq, int32_t t0,
                            size_t* bytes);

/*
 * Prefill: tokens int32 [B, t0] (t0 a multiple of 64, 64 <= t0 <= max_seq).
 * Writes cache positions 0 .. t0-1 of every layer and logits fp32 [B, V]:
 * the softcapped logits at position t0-1 (the next token's distribution is
 * their softmax).  A prompt whose length is not a multiple of 64 is
 * prefilled to the largest multiple and continued with decode steps.
 */
int nc_prefill(const nc_config* cfg, const void* params, const int32_t* tokens,
               int32_t t0, int32_t max_seq, void* cache, float* logits, void* ws,
               size_t ws_bytes, void* stream);

/*
 * Decode step at position pos (0 <= pos < max_seq; positions 0 .. pos-1 of
 * the cache must hold the sequence so far): tokens int32 [B], the token at
 * position pos of each sequence, B <= 32.  Writes cache position pos and
 * logits fp32 [B, V] at position pos.  The step allocates nothing and does
 * not synchronise.
 */
int nc_decode_step(const nc_config* cfg, const void* params, const int32_t* tokens,
                   int32_t pos, int32_t max_seq, void* cache, float* logits, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * nc_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step with its workspace in a 32 MiB array the library holds on
 * every GPU it runs on until the process ends, instead of a `ws` argument.
 * Its kernels are nc_decode_step's and the results are bitwise the same.
 * NC_ERR_WORKSPACE when the step needs more than 32 MiB (nc_infer_workspace_
 * size(cfg, max_seq, 0) > 32 MiB; the depth-20 shapes need about 18 MiB at
 * batch 32 and max_seq 8192).  The array holds the last call's values (the
 * step writes every byte it reads); calls that overlap on one GPU, on any
 * streams, race on it.
 */
int nc_decode_step_noalloc(const nc_config* cfg, const void* params, const int32_t* tokens,
                           int32_t pos, int32_t max_seq, void* cache, float* logits,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NC_INFER_H */
