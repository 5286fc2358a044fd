// Host-side launchers of the library's HIP kernels (internal interface between
// the step runtime and the kernel files; not part of the C ABI).
//
// Every launcher enqueues on `s` and returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace nc {

// ----------------------------------------------------------------- GEMM
// C[m][n] = sum_k A(m,k) * B(n,k), fp32 accumulation, followed by an epilogue.
//   A(m,k) = a_kmajor ? A[m*lda + k] : A[k*lda + m]
//   B(n,k) = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
enum EpiMode : int {
    EPI_STORE_F32 = 0,   // Cf[m][n] = acc (+ Cf[m][n] if accumulate)
    EPI_ROWSCALE = 1,    // C[m][n] = rowscale[m] * acc
    EPI_ROWSCALE_RELU2 = 2,  // C[m][n] = relu(rowscale[m] * acc)^2
    EPI_RESID = 3,       // C[m][n] = resid[m][n] + acc   (resid: T, ld = ldc)
    EPI_RELU2_BWD = 4,   // C[m][n] = rowscale[m] * acc * 2*sqrt(aux[m][n]) (aux: T, ld = ldc)
    EPI_STORE_T = 5,     // C[m][n] = acc, stored as T
    // QKV projection: u = rowscale[m] * acc; the query heads and the key head
    // of row m (position m % seq_len) are rotated and RMS-normalised, rqk
    // receives each head's 1/rms; the value head is stored as u.  bf16 only;
    // head_dim must divide 128.
    EPI_QKV_ROPE = 6,
    EPI_AXPBY = 7,       // C[m][n] = alpha * aux[m][n] + beta * acc (aux: T, ld = ldc)
};
struct Epilogue {
    int mode = EPI_STORE_F32;
    const float* rowscale = nullptr;
    const void* aux = nullptr;   // resid or g, element type T, same ld as C
    bool accumulate = false;     // EPI_STORE_F32 only
    // EPI_QKV_ROPE
    const float* cos_t = nullptr;   // [seq_len, head_dim / 2]
    const float* sin_t = nullptr;
    float* rqk = nullptr;           // [M, n_head + 1]
    int seq_len = 0, n_head = 0, head_dim = 0;
    float eps = 0.f;
    // EPI_AXPBY
    float alpha = 1.f, beta = 1.f;
};
// A batch of independent products of one shape: product i reads A + i*sa,
// B + i*sb and writes C + i*sc (the epilogue's aux at the same offset as C);
// elements of the operand and output types.  No k split, no row scale.
struct GemmBatch {
    int count = 1;
    int64_t sa = 0, sb = 0, sc = 0;
};

template <typename T>
hipError_t gemm(int M, int N, int K, const T* A, int64_t lda, bool a_kmajor,
                const T* B, int64_t ldb, bool b_kmajor, void* C, int64_t ldc,
                const Epilogue& epi, float* splitk_ws, size_t splitk_ws_bytes,
                hipStream_t s, const GemmBatch* batch = nullptr);
// bytes of split-K scratch gemm() may use for an fp32 output of M x N
size_t gemm_splitk_bytes(int M, int N, int K);

// ----------------------------------------------------------------- attention
// attn_fwd / attn_bwd below run the per-row kernels of attn_simt.hip for
// float and the matrix-core kernels for bf16.
// Matrix-core kernels (bf16, T a multiple of 64, hd 64 or 128).
// Decode attention of one token per sequence over a bf16 cache on the matrix
// cores (q fp32 [B, H, hd] with RMS-normalised heads; kc, vc [B][max_seq][hd]
// with RMS-normalised keys; hd 64 or 128, H <= 16): per chunk of
// attn_decode_chunks(npos) <= decode_chunks(npos) writes part_o [B][chunk][H][hd]
// and part_ml [B][chunk][H][2] = {0, sum p} for the combine kernel.
int attn_decode_chunks(int npos);
hipError_t attn_decode_mfma(const float* q, const bf16_t* kc, const bf16_t* vc, int max_seq,
                            int npos, int B, int H, int hd, float* part_o, float* part_ml,
                            hipStream_t s);
// qk_normed: q and k heads are RMS-normalised (QK-norm), which bounds every
// score and lets the bf16 forward drop its running maximum
hipError_t attn_fwd_mfma(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                         int64_t ldkv, bf16_t* o, float* lse, int B, int T, int H, int hd,
                         hipStream_t s, bool qk_normed = false);
// Tail of the step's attention backward fused into the bf16 kernels: instead
// of fp32 dq, dk, dv they write dqkv (bf16, same layout and stride as qkv) =
// r1[token] times, for the query heads and the key head, the backward of
// QK-norm then rotary (y: the saved normalised, rotated qkv; rqk: each head's
// 1/rms; cos_t, sin_t: [T, hd/2] tables), and r1[token] * dv for the value
// head.
struct AttnBwdFuse {
    const bf16_t* y = nullptr;
    const float* rqk = nullptr;
    const float* r1 = nullptr;
    const float* cos_t = nullptr;
    const float* sin_t = nullptr;
    bf16_t* dqkv = nullptr;
};
// fuse == nullptr: plain fp32 dq, dk, dv outputs
hipError_t attn_bwd_mfma(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                         int64_t ldkv, const bf16_t* o, const bf16_t* dout, const float* lse,
                         float* scratch, float* dq, float* dk, float* dv, int B, int T, int H,
                         int hd, hipStream_t s, const AttnBwdFuse* fuse = nullptr);
// bytes of the scratch attn_bwd needs (two values per query row: the row sum
// of dO*O and the scaled log-sum-exp; then the dK/dV partials)
size_t attn_bwd_scratch_bytes(int B, int T, int H, int hd);
// Causal multi-query attention of B sequences of length T with H query heads
// of width hd and one K/V head.  q: [B*T, H, hd] with token stride ldq;
// k, v: [B*T, hd] with token stride ldkv; o: [B*T, H*hd]; lse: [B*T*H] fp32.
template <typename T>
hipError_t attn_fwd(const T* q, const T* k, const T* v, int64_t ldq,
                    int64_t ldkv, T* o, float* lse, int B, int Tn, int H,
                    int hd, hipStream_t s, bool qk_normed = false);
// Backward: dq [B*T, H, hd], dk, dv [B*T, hd], all fp32; scratch holds
// attn_bwd_scratch_bytes(B, T, H, hd) bytes.
template <typename T>
hipError_t attn_bwd(const T* q, const T* k, const T* v, int64_t ldq,
                    int64_t ldkv, const T* o, const T* dout, const float* lse,
                    float* scratch, float* dq, float* dk, float* dv, int B,
                    int Tn, int H, int hd, hipStream_t s);

// ----------------------------------------------------------------- row kernels
template <typename T>
hipError_t embed_fwd(const T* wte, const int32_t* tok, int N, int D, float eps,
                     T* out, float* r, hipStream_t s);
template <typename T>
hipError_t rms_stats(const T* x, int N, int D, float eps, float* r, hipStream_t s);
hipError_t rope_tables(int Tn, int hd, float base, float* cos_t, float* sin_t,
                       hipStream_t s);
// in place on qkv [N, (H+2)*hd]: heads 0..H-1 (q) and H (k) are rotated and
// normalised; rqk [N, H+1] receives the norm scales.
template <typename T>
hipError_t rope_qknorm_fwd(T* qkv, int N, int Tn, int H, int hd,
                           const float* cos_t, const float* sin_t, float eps,
                           float* rqk, hipStream_t s);
// dqkv[N, (H+2)*hd] = r1[t] * d(pre-rotary q, k, v) from the attention-input
// gradients dq [N,H,hd], dk, dv [N,hd] (fp32) and the saved normalised q, k.
template <typename T>
hipError_t rope_qknorm_bwd(const T* qkv, const float* dq, const float* dk,
                           const float* dv, const float* rqk, const float* r1,
                           int N, int Tn, int H, int hd, const float* cos_t,
                           const float* sin_t, T* dqkv, hipStream_t s);
// dres = (has_res ? dres : 0) + dn - r^2 * x * mean(dn * x) over each row,
// in place, rounded to T (dn holds the row scale's product r * dL/dn)
template <typename T>
hipError_t norm_bwd_resid(const T* dn, const T* x, const float* r, int N, int D, T* dres,
                          bool has_res, hipStream_t s);
// de[t] = r0[t]*dh[t] - r0[t]^3 * e[t] * mean(dh[t]*e[t]), e[t] = wte[tok[t]]
template <typename T>
hipError_t embed_bwd_rows(const T* dh, const T* wte, const int32_t* tok,
                          const float* r0, int N, int D, float* de, hipStream_t s);
// Softcap + cross-entropy over rows of z [N, ldz] (V valid columns).
// tok_loss[t] = logsumexp(c) - c[y]; if want_grad, z is overwritten by
// rowscale[t] * inv_n * (softmax(c) - onehot(y)) * (1 - (c/s)^2), and the
// padding columns V..ldz-1 by zeros.
template <typename T>
hipError_t softcap_ce(T* z, int64_t ldz, int V, int N, const int32_t* tgt,
                      float cap, const float* rowscale, float inv_n,
                      float* tok_loss, bool want_grad, hipStream_t s);
// widest logits row (ldz) softcap_ce takes for elements of elem_bytes bytes:
// the kernel keeps a row in registers, 32 16-byte chunks per thread
int64_t softcap_ce_max_ld(int elem_bytes);
// loss = mean(tok_loss[0..N-1]) (fixed summation order)
hipError_t mean_reduce(const float* x, int N, float* out, hipStream_t s);
// out[c][r] = in[r][c] for a rows x cols matrix; out row stride ld_out;
// columns of out beyond `rows` up to ld_out are zero-filled.
template <typename T>
hipError_t transpose(const T* in, int rows, int cols, int64_t ld_in, T* out,
                     int64_t ld_out, hipStream_t s);

// ----------------------------------------------------------------- generation
// y[b][n] = epi(sum_k x[b][k] W[n][k]) for B <= 32 rows (W [N][K], K a
// multiple of 64): mode EPI_ROWSCALE, EPI_ROWSCALE_RELU2, EPI_RESID (aux
// [B][N] with ld ldy) into bf16 y, or EPI_STORE_F32 for fp32 y = rs[b] * acc.
// part: fp32 scratch of part_elems for a k-split (gemv_splits(N, K) * B * N
// elements; with less, the product runs unsplit)
hipError_t gemv(int mode, const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int N, int K,
                const float* rs, const bf16_t* aux, void* y, int64_t ldy, float* part,
                size_t part_elems, hipStream_t s);
int gemv_splits(int N, int K);
// Decode products whose split-K reduce carries the step's row work: both run
// gemv_splits(N, K) > 1 slices into part (gemv_fused_ok checks the shape and
// the scratch).  gemv_qkv_rope: qkv = rs[b] x W^T (N = (H+2) hd), then rotary
// at position pos (angle pos * base^(-2i/hd) in fp64) and QK-norm; query
// heads to q_out fp32 [B][H][hd], the key and value heads to cache row pos of
// kc, vc ([B][max_seq][hd]).  gemv_resid_rms: y = bf16(aux + x W^T) ([B][N],
// aux and y with row stride N), and r_out[b] = 1/sqrt(mean(y_b^2) + eps).
bool gemv_fused_ok(int N, int K, int B, size_t part_elems);
hipError_t gemv_qkv_rope(const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int H, int hd,
                         int K, const float* rs, int pos, double base, float eps, float* q_out,
                         bf16_t* kc, bf16_t* vc, int max_seq, float* part, hipStream_t s);
hipError_t gemv_resid_rms(const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int N, int K,
                          const bf16_t* aux, bf16_t* y, float eps, float* r_out, float* part,
                          hipStream_t s);
// rotary at position pos + QK-norm of B tokens' qkv rows ([B][(H+2) hd], row
// stride ldq): query heads into q_out fp32 [B][H][hd], the key head and the
// value head into cache row pos of kc, vc ([B][max_seq][hd])
template <typename T>
hipError_t decode_rope(const T* qkv, int64_t ldq, int B, int H, int hd, int pos,
                       const float* cos_t, const float* sin_t, float eps, float* q_out, T* kc,
                       T* vc, int max_seq, hipStream_t s);
// number of key chunks decode_attn splits npos keys into
int decode_chunks(int npos);
// o [B][H*hd] = attention of q over cache rows 0..npos-1 (H <= 16, hd <= 128);
// part_o [B][chunks][H][hd], part_ml [B][chunks][H][2] scratch
template <typename T>
hipError_t decode_attn(const float* q, const T* kc, const T* vc, int max_seq, int npos, int B,
                       int H, int hd, float* part_o, float* part_ml, T* o, hipStream_t s);
// key and value rows of B*t0 prefill tokens (qkv rows, stride ldq) into the cache
template <typename T>
hipError_t cache_fill(const T* qkv, int64_t ldq, int B, int t0, int H, int hd, T* kc, T* vc,
                      int max_seq, hipStream_t s);
// out [B][D] = rows b*t0 + t0-1 of x [B*t0][D]
template <typename T>
hipError_t gather_last(const T* x, int D, int t0, int B, T* out, hipStream_t s);
// z = cap * tanh(z / cap) over n fp32 values
hipError_t softcap_rows(float* z, int64_t n, float cap, hipStream_t s);

// ----------------------------------------------------------------- embedding grad
// Deterministic scatter-add of de rows into dwte (fully overwritten):
// dwte[v] = sum over t with tok[t] == v of de[t], summed in position order.
size_t embed_grad_ws_bytes(int N, int D, int V);
hipError_t embed_grad(const float* de, const int32_t* tok, int N, int D, int V,
                      float* dwte, void* ws, size_t ws_bytes, hipStream_t s);

// ----------------------------------------------------------------- misc
template <typename T>
hipError_t init_normal(T* p, int64_t n, float std, uint64_t seed,
                       uint64_t stream_id, hipStream_t s);
template <typename T>
hipError_t zero_elems(T* p, int64_t n, hipStream_t s);
// The stream of an entry point whose host-side checks have passed.  HIP keeps
// one "last error" per host thread, and a failed HIP call made earlier on the
// thread by the caller (or by a framework it uses) leaves it set; it is
// dropped here, before the entry point's first launch, so that the
// hipGetLastError checks after its launches report only its own errors.
inline hipStream_t enqueue_stream(void* stream) {
    (void)hipGetLastError();
    return static_cast<hipStream_t>(stream);
}
// records the HIP error behind an NC_ERR_HIP return (read by nc_last_hip_error)
void note_hip_error(int err);

// Per-kernel timing of the timed step variant.  A launcher that issues more
// than one kernel names each one: prof_label() renames the segment that is
// open (call it before the first kernel), prof_cut() closes the open segment
// at this point of the stream and opens one for the next kernel.  Both are
// no-ops outside the timed variant.  flops / bytes: the kernel's algorithmic
// work and HBM bytes.
hipError_t prof_label(const char* label, double flops, double bytes);
hipError_t prof_cut(const char* label, double flops, double bytes);
hipError_t count_bad_ids(const int32_t* a, const int32_t* b, int64_t n, int V,
                         int32_t* n_bad, hipStream_t s);

}  // namespace nc
