/*
 * nc.h -- C ABI of the MI355X (gfx950) library that runs one forward+backward
 * pretraining step of the nanochat-style dense decoder.
 *
 * The model (nanochat article on vpshk.cn, section on the ~8000-line code
 * base, architecture list): token embedding followed by a parameter-free
 * RMSNorm; per block a pre-norm, bias-free Q/K/V projections, rotary
 * embedding then QK-norm, causal multi-query attention (one shared K/V head),
 * a bias-free output projection added to the residual, a pre-norm relu^2 MLP
 * added to the residual; then a final norm, an untied unembedding, the logit
 * softcap c = s*tanh(z/s) and the mean token cross-entropy.  RMSNorm is
 * n(u) = u / sqrt(mean(u^2) + eps) everywhere, with no learnable gain.
 *
 * Conventions shared by every function:
 *   - Every pointer except `cfg`, `n_elems`, `bytes`, `out`/`stats`/`n_out`
 *     (host structs and counters) is a DEVICE pointer.  params, grads and ws
 *     must be 256-byte aligned, tokens, targets and token_loss 16-byte
 *     aligned, loss and n_bad 4-byte aligned (torch allocations are);
 *     otherwise NC_ERR_ALIGN.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no mutable global state, so calls on different streams with
 *     different workspaces may run concurrently.
 *   - Calls are stream-ordered and asynchronous: they return once the work is
 *     enqueued on `stream` (a hipStream_t; NULL means the null stream).
 *     Outputs are valid after the stream has been synchronised.
 *   - All validation happens on the host before any device work.  A function
 *     that returns an error has enqueued nothing.  NC_ERR_HIP means a launch
 *     failed after work may have been enqueued; nc_last_hip_error() returns
 *     the HIP error code of the calling thread's last such failure.
 *   - Token and target ids are int32 [batch, seq_len], row-major.  Ids must
 *     lie in [0, vocab); nc_validate_tokens checks this on the device.
 */
#ifndef NC_H
#define NC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of the parameter buffer (and of the activations) */
enum { NC_F32 = 0, NC_BF16 = 1 };

/* status codes */
enum {
    NC_OK = 0,
    NC_ERR_NULL = -1,        /* a required pointer is NULL */
    NC_ERR_CONFIG = -2,      /* a config field is out of range */
    NC_ERR_DTYPE = -3,       /* unknown dtype */
    NC_ERR_WORKSPACE = -4,   /* workspace smaller than nc_workspace_size */
    NC_ERR_ALIGN = -5,       /* a device pointer is not 256-byte aligned */
    NC_ERR_HIP = -6,         /* a HIP call or kernel launch failed */
    NC_ERR_UNSUPPORTED = -7, /* valid model, but a shape the library does not run */
    NC_ERR_CAPACITY = -8     /* output array too small (nc_param_layout) */
};

/*
 * Model and batch description.
 *   n_layer    number of blocks (>= 1)
 *   d_model    width D of the residual stream (multiple of 64; at most 8192
 *              for NC_BF16, 4096 for NC_F32)
 *   n_head     H, query heads; n_head * head_dim is the attention width
 *   head_dim   hd, 64 or 128
 *   n_kv_head  must be 1: multi-query attention (one K head, one V head)
 *   d_mlp      F, hidden width of the relu^2 MLP (multiple of 64)
 *   vocab      V >= 2 (padded to a multiple of 256: at most 131072 for NC_BF16,
 *              65536 for NC_F32)
 *   seq_len    T, a multiple of 64
 *   batch      B >= 1 sequences; tokens per step N = B*T
 *   rope_base  rotary base (angle of pair i at position t: t*base^(-2i/hd))
 *   softcap    s > 0 of the logit softcap s*tanh(z/s)
 *   rms_eps    epsilon of every RMSNorm (>= 0)
 *   dtype      NC_F32 or NC_BF16: storage type of parameters and activations.
 *              NC_BF16 computes products in bf16 on the matrix cores with fp32
 *              accumulation and keeps every statistic (norms, softmax, loss)
 *              in fp32.  NC_F32 computes everything in fp32.
 */
typedef struct nc_config {
    int32_t n_layer, d_model, n_head, head_dim, n_kv_head, d_mlp, vocab,
            seq_len, batch;
    float rope_base, softcap, rms_eps;
    int32_t dtype;
} nc_config;

/* one weight matrix inside the flat parameter buffer */
typedef struct nc_tensor_info {
    char name[32];   /* "wte", "h<l>.wq", "h<l>.wk", "h<l>.wv", "h<l>.wo",
                        "h<l>.wfc", "h<l>.wproj", "wlm" */
    int64_t offset;  /* element offset into the parameter (and gradient) buffer */
    int32_t rows;    /* out_features (vocab for wte/wlm) */
    int32_t cols;    /* in_features (d_model for wte/wlm) */
} nc_tensor_info;

/*
 * Parameter layout.  One flat buffer of cfg->dtype elements holds every
 * matrix row-major as [rows, cols] (the [out, in] convention of a linear
 * layer; no biases exist).  Order: wte [V, D]; for each layer wq [H*hd, D],
 * wk [hd, D], wv [hd, D] (adjacent, so together they are one [(H+2)*hd, D]
 * matrix), wo [D, H*hd], wfc [F, D], wproj [D, F]; then wlm [V, D].  Every
 * offset is a multiple of 128 elements; the gaps are padding the library
 * neither reads nor writes.  The fp32 gradient buffer uses the same element
 * offsets.
 *
 * nc_param_count: total elements of the flat buffer (including padding).
 * nc_param_layout: fills out[0 .. n-1] (n = 2 + 6*n_layer) if cap >= n and
 *   sets *n_out = n; returns NC_ERR_CAPACITY (with *n_out = n) if cap < n.
 */
int nc_param_count(const nc_config* cfg, int64_t* n_elems);
int nc_param_layout(const nc_config* cfg, nc_tensor_info* out, int32_t cap,
                    int32_t* n_out);

/*
 * Bytes of device workspace a step needs.  with_backward = 0 sizes
 * nc_forward_loss, 1 sizes nc_forward_backward (which also suffices for
 * nc_forward_loss).  The workspace holds the saved activations of every
 * layer, the logits and all scratch; its contents are undefined between calls.
 */
int nc_workspace_size(const nc_config* cfg, int32_t with_backward,
                      size_t* bytes);

/*
 * Fill the parameter buffer: every matrix N(0, 0.02^2) except wlm,
 * N(0, 0.001^2) (the workloads' stated initialisation), drawn on the device
 * from a counter-based Philox4x32-10 stream keyed by `seed` (Salmon et al.,
 * SC'11) through the Box-Muller transform.  Deterministic per seed.
 * Padding elements are set to 0.
 */
int nc_init_params(const nc_config* cfg, uint64_t seed, void* params,
                   void* stream);

/*
 * Forward pass and mean loss.  params: dtype per cfg, laid out as above.
 * tokens, targets: int32 [B, T].  loss: one fp32, the mean cross-entropy
 * over all B*T tokens (natural log).  ws: workspace of ws_bytes >=
 * nc_workspace_size(cfg, 0).
 */
int nc_forward_loss(const nc_config* cfg, const void* params,
                    const int32_t* tokens, const int32_t* targets, float* loss,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * nc_forward_loss that also writes the per-token losses: token_loss fp32
 * [B, T], l_t = logsumexp(c_t) - c_t[y_t] (NULL to skip, which is
 * nc_forward_loss).  The mean loss is the mean of these values.
 */
int nc_forward_token_loss(const nc_config* cfg, const void* params,
                          const int32_t* tokens, const int32_t* targets,
                          float* loss, float* token_loss, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Forward and backward pass.  As nc_forward_loss, and `grads` (fp32, same
 * element offsets as params, nc_param_count elements) is OVERWRITTEN with the
 * gradient of the mean loss for every parameter (rows of wte whose id does
 * not occur in `tokens` get zeros).  ws_bytes >= nc_workspace_size(cfg, 1).
 */
int nc_forward_backward(const nc_config* cfg, const void* params,
                        const int32_t* tokens, const int32_t* targets,
                        float* loss, float* grads, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * Activation recompute (the llm.c article on qian.cx names it among its
 * training options): the same step as nc_forward_backward with a workspace
 * that keeps only the block inputs of every layer plus one layer's other
 * saved tensors; before each block's backward pass the block's forward is run
 * again from its input (everything but the block output).  That costs about
 * one more forward pass of the blocks and cuts the workspace by the other
 * per-layer tensors (about 23 GB of the d20 step's 60 GB), so longer
 * sequences or larger batches fit.  The kernels are the step's own and
 * deterministic, so loss and gradients are bitwise those of
 * nc_forward_backward.  ws_bytes >= nc_workspace_size_recompute(cfg).
 */
int nc_workspace_size_recompute(const nc_config* cfg, size_t* bytes);
int nc_forward_backward_recompute(const nc_config* cfg, const void* params,
                                  const int32_t* tokens, const int32_t* targets,
                                  float* loss, float* grads, void* ws,
                                  size_t ws_bytes, void* stream);

/* per-kernel account of one step (nc_forward_backward_timed) */
typedef struct nc_kernel_stat {
    char name[48];      /* kernel label, e.g. "gemm_nt_relu2" */
    int32_t launches;   /* launches of this kernel in the step */
    double total_ms;    /* summed durations, HIP events on `stream` around each launch */
    double flops;       /* algorithmic floating-point operations, summed over launches */
    double bytes;       /* algorithmic HBM bytes (each input read once, each output
                           written once), summed over launches */
} nc_kernel_stat;

/*
 * nc_forward_backward with a HIP event recorded on `stream` before and after
 * every kernel launch.  Same outputs and arguments as nc_forward_backward,
 * plus `stats` (host array of `cap` entries) that receives one entry per
 * distinct kernel label, in first-launch order; *n_out is the number of
 * labels (NC_ERR_CAPACITY if cap is smaller, stats then holds the first cap).
 * Unlike the other calls this one synchronises `stream` before returning.
 * The events serialise nothing that stream order does not already serialise.
 */
int nc_forward_backward_timed(const nc_config* cfg, const void* params,
                              const int32_t* tokens, const int32_t* targets,
                              float* loss, float* grads, void* ws,
                              size_t ws_bytes, void* stream,
                              nc_kernel_stat* stats, int32_t cap,
                              int32_t* n_out);

/*
 * Count ids outside [0, vocab) in tokens and targets (B*T each) into *n_bad
 * (one device int32, overwritten).  The step functions assume valid ids.
 */
int nc_validate_tokens(const nc_config* cfg, const int32_t* tokens,
                       const int32_t* targets, int32_t* n_bad, void* stream);

/* static description of a status code */
const char* nc_status_string(int status);

/* HIP error code (hipError_t) behind the calling thread's last NC_ERR_HIP */
int nc_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NC_H */
