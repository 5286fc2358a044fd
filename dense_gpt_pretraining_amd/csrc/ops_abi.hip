// Unit-level entry points of include/nc_ops.h: thin validated wrappers that
// launch exactly the kernels the step uses.
#include "../../include/nc.h"
#include "../../include/nc_ops.h"
#include "kernels.h"

static_assert(NC_EPI_ROWSCALE == nc::EPI_ROWSCALE && NC_EPI_ROWSCALE_RELU2 == nc::EPI_ROWSCALE_RELU2 &&
                  NC_EPI_RESID == nc::EPI_RESID && NC_EPI_RELU2_BWD == nc::EPI_RELU2_BWD &&
                  NC_EPI_STORE == nc::EPI_STORE_T,
              "the unit ABI's epilogue codes are the library's modes");

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int ret(hipError_t e) {
    if (e == hipSuccess) return NC_OK;
    nc::note_hip_error((int)e);
    return NC_ERR_HIP;
}

}  // namespace

extern "C" {

int nc_op_matmul(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                 int32_t a_kmajor, const void* B, int64_t ldb, int32_t b_kmajor, float* C,
                 int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
    if (dtype != NC_F32 && dtype != NC_BF16) return NC_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 1) return NC_ERR_CONFIG;
    if (!A || !B || !C) return NC_ERR_NULL;
    if (!al16(A) || !al16(B) || !al16(C) || (ws && !al16(ws))) return NC_ERR_ALIGN;
    if (ldc < N) return NC_ERR_CONFIG;
    if (a_kmajor ? lda < K : lda < M) return NC_ERR_CONFIG;
    if (b_kmajor ? ldb < K : ldb < N) return NC_ERR_CONFIG;
    hipStream_t s = nc::enqueue_stream(stream);
    nc::Epilogue e;
    e.mode = nc::EPI_STORE_F32;
    if (dtype == NC_F32)
        return ret(nc::gemm<float>(M, N, K, static_cast<const float*>(A), lda, a_kmajor != 0,
                                   static_cast<const float*>(B), ldb, b_kmajor != 0, C, ldc, e,
                                   static_cast<float*>(ws), ws_bytes, s));
    if (!a_kmajor && b_kmajor) return NC_ERR_UNSUPPORTED;   // (mn-major, k-major) is not built
    if (K % 8 || lda % 8 || ldb % 8 || ldc % 4) return NC_ERR_UNSUPPORTED;
    if (K % 64) return NC_ERR_UNSUPPORTED;   // whole 64-deep k tiles are copied into LDS
    if (!a_kmajor && lda < ((M + 7) / 8) * 8) return NC_ERR_UNSUPPORTED;
    if (!b_kmajor && ldb < ((N + 7) / 8) * 8) return NC_ERR_UNSUPPORTED;
    return ret(nc::gemm<nc::bf16_t>(M, N, K, static_cast<const nc::bf16_t*>(A), lda,
                                    a_kmajor != 0, static_cast<const nc::bf16_t*>(B), ldb,
                                    b_kmajor != 0, C, ldc, e, static_cast<float*>(ws), ws_bytes,
                                    s));
}

int nc_op_matmul_epilogue(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A,
                          int64_t lda, int32_t a_kmajor, const void* B, int64_t ldb,
                          int32_t b_kmajor, void* C, int64_t ldc, int32_t mode,
                          const float* rowscale, const void* aux, void* stream) {
    if (dtype != NC_F32 && dtype != NC_BF16) return NC_ERR_DTYPE;
    if (M < 1 || N < 1 || K < 1) return NC_ERR_CONFIG;
    if (mode < NC_EPI_ROWSCALE || mode > NC_EPI_STORE) return NC_ERR_CONFIG;
    const bool need_rs = mode == NC_EPI_ROWSCALE || mode == NC_EPI_ROWSCALE_RELU2 ||
                         mode == NC_EPI_RELU2_BWD;
    const bool need_aux = mode == NC_EPI_RESID || mode == NC_EPI_RELU2_BWD;
    if (!A || !B || !C || (need_rs && !rowscale) || (need_aux && !aux)) return NC_ERR_NULL;
    if (!al16(A) || !al16(B) || !al16(C) || (aux && !al16(aux))) return NC_ERR_ALIGN;
    if (ldc < N) return NC_ERR_CONFIG;
    if (a_kmajor ? lda < K : lda < M) return NC_ERR_CONFIG;
    if (b_kmajor ? ldb < K : ldb < N) return NC_ERR_CONFIG;
    nc::Epilogue e;
    e.mode = mode;   // the NC_EPI_* values are the library's epilogue modes
    e.rowscale = need_rs ? rowscale : nullptr;
    e.aux = need_aux ? aux : nullptr;
    if (dtype == NC_F32) {
        hipStream_t s = nc::enqueue_stream(stream);
        return ret(nc::gemm<float>(M, N, K, static_cast<const float*>(A), lda, a_kmajor != 0,
                                   static_cast<const float*>(B), ldb, b_kmajor != 0, C, ldc, e,
                                   nullptr, 0, s));
    }
    // the bf16 products the step runs: (k, k) with every mode, (k, mn) with
    // the data-gradient modes
    if (!a_kmajor) return NC_ERR_UNSUPPORTED;
    if (!b_kmajor && mode != NC_EPI_STORE && mode != NC_EPI_RELU2_BWD) return NC_ERR_UNSUPPORTED;
    if (K % 64 || lda % 8 || ldb % 8 || ldc % 4) return NC_ERR_UNSUPPORTED;
    if (!b_kmajor && ldb < ((N + 7) / 8) * 8) return NC_ERR_UNSUPPORTED;
    hipStream_t s = nc::enqueue_stream(stream);
    return ret(nc::gemm<nc::bf16_t>(M, N, K, static_cast<const nc::bf16_t*>(A), lda, true,
                                    static_cast<const nc::bf16_t*>(B), ldb, b_kmajor != 0, C, ldc,
                                    e, nullptr, 0, s));
}

static int attn_check(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd, int64_t ldq,
                      int64_t ldkv) {
    if (dtype != NC_F32 && dtype != NC_BF16) return NC_ERR_DTYPE;
    if (B < 1 || T < 1 || H < 1) return NC_ERR_CONFIG;
    if (hd != 64 && hd != 128) return NC_ERR_UNSUPPORTED;
    if (T % 64) return NC_ERR_UNSUPPORTED;
    if (ldq < (int64_t)H * hd || ldkv < hd || ldq % 8 || ldkv % 8) return NC_ERR_CONFIG;
    return NC_OK;
}

int nc_op_attention_fwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd,
                        const void* q, const void* k, const void* v, int64_t ldq, int64_t ldkv,
                        void* o, float* lse, int32_t qk_normed, void* stream) {
    int rc = attn_check(dtype, B, T, H, hd, ldq, ldkv);
    if (rc != NC_OK) return rc;
    if (!q || !k || !v || !o || !lse) return NC_ERR_NULL;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(o) || !al16(lse)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    if (dtype == NC_F32)
        return ret(nc::attn_fwd<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                                       static_cast<const float*>(v), ldq, ldkv,
                                       static_cast<float*>(o), lse, B, T, H, hd, s));
    return ret(nc::attn_fwd<nc::bf16_t>(
        static_cast<const nc::bf16_t*>(q), static_cast<const nc::bf16_t*>(k),
        static_cast<const nc::bf16_t*>(v), ldq, ldkv, static_cast<nc::bf16_t*>(o), lse, B, T, H,
        hd, s, qk_normed != 0));
}

int nc_op_attention_bwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd,
                        const void* q, const void* k, const void* v, int64_t ldq, int64_t ldkv,
                        const void* o, const void* dout, const float* lse, void* scratch,
                        size_t scratch_bytes, float* dq, float* dk, float* dv, void* stream) {
    int rc = attn_check(dtype, B, T, H, hd, ldq, ldkv);
    if (rc != NC_OK) return rc;
    if (!q || !k || !v || !o || !dout || !lse || !scratch || !dq || !dk || !dv) return NC_ERR_NULL;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(o) || !al16(dout) || !al16(lse) ||
        !al16(scratch) || !al16(dq) || !al16(dk) || !al16(dv))
        return NC_ERR_ALIGN;
    if (scratch_bytes < nc::attn_bwd_scratch_bytes(B, T, H, hd)) return NC_ERR_WORKSPACE;
    hipStream_t s = nc::enqueue_stream(stream);
    float* sc = static_cast<float*>(scratch);
    if (dtype == NC_F32)
        return ret(nc::attn_bwd<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                                       static_cast<const float*>(v), ldq, ldkv,
                                       static_cast<const float*>(o),
                                       static_cast<const float*>(dout), lse, sc, dq, dk, dv, B, T,
                                       H, hd, s));
    return ret(nc::attn_bwd<nc::bf16_t>(
        static_cast<const nc::bf16_t*>(q), static_cast<const nc::bf16_t*>(k),
        static_cast<const nc::bf16_t*>(v), ldq, ldkv, static_cast<const nc::bf16_t*>(o),
        static_cast<const nc::bf16_t*>(dout), lse, sc, dq, dk, dv, B, T, H, hd, s));
}

int nc_op_attention_bwd_scratch_bytes(int32_t B, int32_t T, int32_t H, int32_t hd,
                                      size_t* bytes) {
    if (!bytes) return NC_ERR_NULL;
    if (B < 1 || T < 1 || H < 1) return NC_ERR_CONFIG;
    if (hd != 64 && hd != 128) return NC_ERR_UNSUPPORTED;
    *bytes = nc::attn_bwd_scratch_bytes(B, T, H, hd);
    return NC_OK;
}

int nc_op_softcap_ce(int32_t dtype, int32_t N, int32_t V, int64_t ldz, void* z,
                     const int32_t* targets, float softcap, const float* rowscale, float inv_n,
                     float* tok_loss, int32_t want_grad, void* stream) {
    if (dtype != NC_F32 && dtype != NC_BF16) return NC_ERR_DTYPE;
    if (N < 1 || V < 2 || ldz < V || ldz % 8) return NC_ERR_CONFIG;
    if (!(softcap > 0.f) || softcap > 60.f) return NC_ERR_UNSUPPORTED;
    if (ldz > nc::softcap_ce_max_ld(dtype == NC_BF16 ? 2 : 4)) return NC_ERR_UNSUPPORTED;
    if (!z || !targets || !tok_loss || (want_grad && !rowscale)) return NC_ERR_NULL;
    if (!al16(z) || !al16(targets) || !al16(tok_loss) || (rowscale && !al16(rowscale)))
        return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    if (dtype == NC_F32)
        return ret(nc::softcap_ce<float>(static_cast<float*>(z), ldz, V, N, targets, softcap,
                                         rowscale, inv_n, tok_loss, want_grad != 0, s));
    return ret(nc::softcap_ce<nc::bf16_t>(static_cast<nc::bf16_t*>(z), ldz, V, N, targets,
                                          softcap, rowscale, inv_n, tok_loss, want_grad != 0, s));
}

int nc_op_rope_qknorm_fwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t hd, void* qkv,
                          float base, float eps, float* rqk, float* tables, void* stream) {
    if (dtype != NC_F32 && dtype != NC_BF16) return NC_ERR_DTYPE;
    if (B < 1 || T < 1 || H < 1 || !(base > 1.f) || !(eps >= 0.f)) return NC_ERR_CONFIG;
    if (hd != 64 && hd != 128) return NC_ERR_UNSUPPORTED;
    if (!qkv || !rqk || !tables) return NC_ERR_NULL;
    if (!al16(qkv) || !al16(rqk) || !al16(tables)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    float* cos_t = tables;
    float* sin_t = tables + (int64_t)T * (hd / 2);
    hipError_t e = nc::rope_tables(T, hd, base, cos_t, sin_t, s);
    if (e != hipSuccess) return ret(e);
    const int N = B * T;
    if (dtype == NC_F32)
        return ret(nc::rope_qknorm_fwd<float>(static_cast<float*>(qkv), N, T, H, hd, cos_t, sin_t,
                                              eps, rqk, s));
    return ret(nc::rope_qknorm_fwd<nc::bf16_t>(static_cast<nc::bf16_t*>(qkv), N, T, H, hd, cos_t,
                                               sin_t, eps, rqk, s));
}

int nc_op_embedding_grad_ws_bytes(int32_t N, int32_t D, int32_t V, size_t* bytes) {
    if (N < 1 || D < 4 || V < 1 || V > (1 << 24)) return NC_ERR_CONFIG;
    if (D % 4) return NC_ERR_UNSUPPORTED;
    if (!bytes) return NC_ERR_NULL;
    *bytes = nc::embed_grad_ws_bytes(N, D, V);
    return NC_OK;
}

int nc_op_embedding_grad(int32_t N, int32_t D, int32_t V, const float* de, const int32_t* tokens,
                         float* dwte, void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    const int rc = nc_op_embedding_grad_ws_bytes(N, D, V, &need);
    if (rc != NC_OK) return rc;
    if (!de || !tokens || !dwte || !ws) return NC_ERR_NULL;
    if (!al16(de) || !al16(tokens) || !al16(dwte) || (reinterpret_cast<uintptr_t>(ws) & 255))
        return NC_ERR_ALIGN;
    if (ws_bytes < need) return NC_ERR_WORKSPACE;
    hipStream_t s = nc::enqueue_stream(stream);
    return ret(nc::embed_grad(de, tokens, N, D, V, dwte, ws, ws_bytes, s));
}

}  // extern "C"
