// Attention dispatch: the matrix-core kernels for bf16, the per-row kernels
// otherwise.
#include "kernels.h"

namespace nc {

template <>
hipError_t attn_fwd<float>(const float* q, const float* k, const float* v, int64_t ldq,
                           int64_t ldkv, float* o, float* lse, int B, int Tn, int H, int hd,
                           hipStream_t s) {
    return attn_fwd_simt<float>(q, k, v, ldq, ldkv, o, lse, B, Tn, H, hd, s);
}
template <>
hipError_t attn_bwd<float>(const float* q, const float* k, const float* v, int64_t ldq,
                           int64_t ldkv, const float* o, const float* dout, const float* lse,
                           float* scratch, float* dq, float* dk, float* dv, int B, int Tn, int H,
                           int hd, hipStream_t s) {
    // the per-row kernels need only the row sums (first B*T*H floats)
    return attn_bwd_simt<float>(q, k, v, ldq, ldkv, o, dout, lse, scratch, dq, dk, dv, B, Tn, H,
                                hd, s);
}
template <>
hipError_t attn_fwd<bf16_t>(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                            int64_t ldkv, bf16_t* o, float* lse, int B, int Tn, int H, int hd,
                            hipStream_t s) {
    return attn_fwd_mfma(q, k, v, ldq, ldkv, o, lse, B, Tn, H, hd, s);
}
template <>
hipError_t attn_bwd<bf16_t>(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                            int64_t ldkv, const bf16_t* o, const bf16_t* dout, const float* lse,
                            float* scratch, float* dq, float* dk, float* dv, int B, int Tn, int H,
                            int hd, hipStream_t s) {
    return attn_bwd_mfma(q, k, v, ldq, ldkv, o, dout, lse, scratch, dq, dk, dv, B, Tn, H, hd, s);
}

}  // namespace nc
