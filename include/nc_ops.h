/*
 * nc_ops.h -- unit-level entry points of the step library, one per kernel
 * family, so that each piece of the step can be checked on its own against a
 * CPU reference.  They run exactly the kernels nc_forward_backward runs.
 *
 * Conventions are those of nc.h: device pointers, caller-owned buffers,
 * asynchronous on `stream` (a hipStream_t), host-side validation before any
 * device work, NC_* status codes.  `dtype` is NC_F32 or NC_BF16 and gives the
 * element type of every tensor documented as "T"; fp32 tensors are float.
 * Every device pointer must be 16-byte aligned.
 */
#ifndef NC_OPS_H
#define NC_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * C[m][n] = sum_k A(m,k) B(n,k), fp32 accumulation, C fp32 [M, N] row stride
 * ldc.  A(m,k) = a_kmajor ? A[m*lda + k] : A[k*lda + m] (T), likewise B with
 * b_kmajor.  This is the contraction of every bias-free linear layer (forward
 * X W^T, data gradient dY W, weight gradient dY^T X).  bf16 supports the
 * (k-major, k-major), (k-major, mn-major) and (mn-major, mn-major) pairs with
 * K a multiple of 64;
 * both leading dimensions must be multiples of 8 (for mn-major operands at
 * least M resp. N rounded up to 8) and ldc a multiple of 4.  ws (may be NULL, ws_bytes 0) is scratch
 * for a k-split; with too little scratch the k loop is not split.
 */
int nc_op_matmul(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                 int32_t a_kmajor, const void* B, int64_t ldb, int32_t b_kmajor, float* C,
                 int64_t ldc, void* ws, size_t ws_bytes, void* stream);

/*
 * The bias-free linear layers' products with their fused epilogues, stored
 * as T in C [M, ldc] (same operand conventions as nc_op_matmul):
 *   NC_EPI_ROWSCALE        C = rowscale[m] * acc          (a normed input, n(x) W^T)
 *   NC_EPI_ROWSCALE_RELU2  C = relu(rowscale[m] * acc)^2  (the MLP's first layer)
 *   NC_EPI_RESID           C = aux[m][n] + acc            (a residual add)
 *   NC_EPI_RELU2_BWD       C = rowscale[m] * acc * 2 sqrt(aux[m][n])
 *                          (aux = relu(u)^2; the relu^2 derivative)
 *   NC_EPI_STORE           C = acc
 * rowscale fp32 [M]; aux T [M, ldc].  bf16 runs the (k-major, k-major) pair
 * with every mode and (k-major, mn-major) with NC_EPI_RELU2_BWD and
 * NC_EPI_STORE, K a multiple of 64; fp32 runs every pair.
 */
enum { NC_EPI_ROWSCALE = 1, NC_EPI_ROWSCALE_RELU2 = 2, NC_EPI_RESID = 3, NC_EPI_RELU2_BWD = 4,
       NC_EPI_STORE = 5 };
int nc_op_matmul_epilogue(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A,
                          int64_t lda, int32_t a_kmajor, const void* B, int64_t ldb,
                          int32_t b_kmajor, void* C, int64_t ldc, int32_t mode,
                          const float* rowscale, const void* aux, void* stream);

/*
 * Causal multi-query attention (one shared K/V head; architecture list of the
 * nanochat article).  q: T [B*T, H, hd] with token stride ldq (elements);
 * k, v: T [B*T, hd] with token stride ldkv; o: T [B*T, H*hd];
 * lse: fp32 [B*T*H], the log-sum-exp of each row's scaled scores.
 * o[t, j] = sum_{tau <= t} softmax(q[t,j].k[tau] / sqrt(hd)) v[tau].
 * hd is 64 or 128, T a multiple of 64.  qk_normed nonzero promises that
 * every q and k head has RMS 1 (QK-norm, as in the step), which bounds each
 * scaled score by sqrt(hd) (up to bf16 rounding): the bf16 kernel then
 * subtracts a fixed offset instead of a running maximum (same softmax).  The
 * result is undefined when the promise does not hold; fp32 ignores the flag.
 */
int nc_op_attention_fwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd,
                        const void* q, const void* k, const void* v, int64_t ldq, int64_t ldkv,
                        void* o, float* lse, int32_t qk_normed, void* stream);

/*
 * Backward of nc_op_attention_fwd for output gradient dout (T [B*T, H*hd]).
 * dq fp32 [B*T, H, hd]; dk, dv fp32 [B*T, hd]; scratch: device scratch of at
 * least nc_op_attention_bwd_scratch_bytes(...) bytes (else NC_ERR_WORKSPACE).
 */
int nc_op_attention_bwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd,
                        const void* q, const void* k, const void* v, int64_t ldq, int64_t ldkv,
                        const void* o, const void* dout, const float* lse, void* scratch,
                        size_t scratch_bytes, float* dq, float* dk, float* dv, void* stream);
int nc_op_attention_bwd_scratch_bytes(int32_t B, int32_t T, int32_t H, int32_t hd,
                                      size_t* bytes);

/*
 * Softcap + cross-entropy over the rows of z (T [N, ldz], V valid columns,
 * ldz a multiple of 8 and >= V, at most 131072 for bf16 and 65536 for fp32,
 * else NC_ERR_UNSUPPORTED): c = s tanh(z/s), tok_loss[t] =
 * logsumexp(c_t) - c_t[y_t].  If want_grad, z is overwritten with
 * rowscale[t] * inv_n * (softmax(c_t) - onehot(y_t)) * (1 - (c_t/s)^2) and the
 * columns V..ldz-1 with zeros.  0 < s <= 60.
 */
int nc_op_softcap_ce(int32_t dtype, int32_t N, int32_t V, int64_t ldz, void* z,
                     const int32_t* targets, float softcap, const float* rowscale, float inv_n,
                     float* tok_loss, int32_t want_grad, void* stream);

/*
 * Rotary embedding then QK-norm, in place on qkv (T [B*T, (H+2)*hd]): the H
 * query heads and the key head of each token are rotated (pair (i, i+hd/2) of
 * position t by angle t*base^(-2i/hd)) and RMS-normalised; the value head is
 * untouched.  rqk fp32 [B*T, H+1] receives 1/sqrt(mean(u^2)+eps) of each
 * rotated head.  tables: fp32 scratch of T*hd floats.
 */
int nc_op_rope_qknorm_fwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd, void* qkv,
                          float base, float eps, float* rqk, float* tables, void* stream);

/*
 * Embedding gradient (the backward of the token-embedding lookup, nanochat
 * article, architecture list): dwte[v] = sum of de[t] over the positions t
 * with tokens[t] == v.  de fp32 [N, D], tokens int32 [N] with every id in
 * [0, V), dwte fp32 [V, D], overwritten (rows of ids that do not occur are
 * 0).  The positions are sorted by id (stable radix sort) and each id's rows
 * are summed in position order (in pieces of at most 64 rows, whose sums are
 * then added in order), so the result is bitwise reproducible.  D must be a
 * multiple of 4.  ws: scratch of at least nc_op_embedding_grad_ws_bytes(N, D,
 * V) bytes (else NC_ERR_WORKSPACE), 256-byte aligned (else NC_ERR_ALIGN).  An
 * id outside [0, V) is a precondition violation that is not checked here
 * (nc_validate_tokens counts them).
 */
int nc_op_embedding_grad(int32_t N, int32_t D, int32_t V, const float* de, const int32_t* tokens,
                         float* dwte, void* ws, size_t ws_bytes, void* stream);
int nc_op_embedding_grad_ws_bytes(int32_t N, int32_t D, int32_t V, size_t* bytes);

#ifdef __cplusplus
}
#endif
#endif /* NC_OPS_H */
