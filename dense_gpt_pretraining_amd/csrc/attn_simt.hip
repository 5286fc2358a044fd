// Causal multi-query attention, plain per-row kernels: the attention of the
// fp32 configuration (the bf16 configurations run the matrix-core kernels of
// attn_mfma.hip).
//
// Multi-query attention (architecture list of the nanochat article): the H
// query heads of a token share one key head and one value head.  Row (t, j)
// of a sequence attends to keys tau <= t with weights softmax(q.k/sqrt(hd)).
// Each thread owns one query row (forward, dq) or one key (dk, dv) and walks
// the other side in order, so every sum has a fixed order.
#include "kernels.h"

namespace nc {

namespace {

constexpr int kThreads = 64;

template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_fwd_simt(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ldq,
    int64_t ldkv, T* __restrict__ o, float* __restrict__ lse, int B, int Tn, int H) {
    const int64_t row = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // (b, t, j)
    if (row >= (int64_t)B * Tn * H) return;
    const int64_t tok = row / H;                 // b*T + t
    const int j = (int)(row % H);
    const int t = (int)(tok % Tn);
    const int64_t seq0 = tok - t;
    const float scale = 1.f / sqrtf((float)HD);
    const T* qr = q + tok * ldq + (int64_t)j * HD;
    float qf[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) qf[d] = Elt<T>::ld(qr + d) * scale;
    float acc[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) acc[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    for (int tau = 0; tau <= t; ++tau) {
        const T* kr = k + (seq0 + tau) * ldkv;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) s += qf[d] * Elt<T>::ld(kr + d);
        const float mn = fmaxf(m, s);
        const float corr = __expf(m - mn);
        const float p = __expf(s - mn);
        l = l * corr + p;
        const T* vr = v + (seq0 + tau) * ldkv;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = acc[d] * corr + p * Elt<T>::ld(vr + d);
        m = mn;
    }
    const float inv = 1.f / l;
    T* orow = o + tok * (int64_t)H * HD + (int64_t)j * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) Elt<T>::st(orow + d, acc[d] * inv);
    lse[row] = m + __logf(l);
}

// delta[(b,t,j)] = sum_d dout * o  (row sum used by the softmax backward)
template <typename T>
__global__ __launch_bounds__(256) void k_attn_delta(const T* __restrict__ o,
                                                    const T* __restrict__ dout, int64_t rows,
                                                    int hd, float* __restrict__ delta) {
    // one wave per row
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const T* a = o + row * hd;
    const T* b = dout + row * hd;
    float s = 0.f;
    for (int d = lane; d < hd; d += 64) s += Elt<T>::ld(a + d) * Elt<T>::ld(b + d);
    s = wave_sum(s);
    if (lane == 0) delta[row] = s;
}

template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_bwd_dq_simt(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ldq,
    int64_t ldkv, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, int B, int Tn, int H) {
    const int64_t row = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (row >= (int64_t)B * Tn * H) return;
    const int64_t tok = row / H;
    const int j = (int)(row % H);
    const int t = (int)(tok % Tn);
    const int64_t seq0 = tok - t;
    const float scale = 1.f / sqrtf((float)HD);
    const T* qr = q + tok * ldq + (int64_t)j * HD;
    const T* dr = dout + tok * (int64_t)H * HD + (int64_t)j * HD;
    float qf[HD], df[HD], acc[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        qf[d] = Elt<T>::ld(qr + d) * scale;
        df[d] = Elt<T>::ld(dr + d);
        acc[d] = 0.f;
    }
    const float L = lse[row], dl = delta[row];
    for (int tau = 0; tau <= t; ++tau) {
        const T* kr = k + (seq0 + tau) * ldkv;
        const T* vr = v + (seq0 + tau) * ldkv;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
            s += qf[d] * Elt<T>::ld(kr + d);
            dp += df[d] * Elt<T>::ld(vr + d);
        }
        const float p = __expf(s - L);
        const float ds = p * (dp - dl) * scale;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] += ds * Elt<T>::ld(kr + d);
    }
    float* out = dq + row * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) out[d] = acc[d];
}

template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_bwd_dkv_simt(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ldq,
    int64_t ldkv, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv, int B,
    int Tn, int H) {
    const int64_t key = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // (b, tau)
    if (key >= (int64_t)B * Tn) return;
    const int tau = (int)(key % Tn);
    const int64_t seq0 = key - tau;
    const float scale = 1.f / sqrtf((float)HD);
    float kf[HD], vf[HD], ak[HD], av[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        kf[d] = Elt<T>::ld(k + key * ldkv + d);
        vf[d] = Elt<T>::ld(v + key * ldkv + d);
        ak[d] = 0.f;
        av[d] = 0.f;
    }
    for (int t = tau; t < Tn; ++t) {
        for (int j = 0; j < H; ++j) {
            const int64_t row = (seq0 + t) * H + j;
            const T* qr = q + (seq0 + t) * ldq + (int64_t)j * HD;
            const T* dr = dout + (seq0 + t) * (int64_t)H * HD + (int64_t)j * HD;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int d = 0; d < HD; ++d) {
                s += Elt<T>::ld(qr + d) * kf[d];
                dp += Elt<T>::ld(dr + d) * vf[d];
            }
            const float p = __expf(s * scale - lse[row]);
            const float ds = p * (dp - delta[row]) * scale;
#pragma unroll
            for (int d = 0; d < HD; ++d) {
                av[d] += p * Elt<T>::ld(dr + d);
                ak[d] += ds * Elt<T>::ld(qr + d);
            }
        }
    }
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        dk[key * HD + d] = ak[d];
        dv[key * HD + d] = av[d];
    }
}

}  // namespace

template <typename T>
hipError_t attn_fwd_simt(const T* q, const T* k, const T* v, int64_t ldq, int64_t ldkv, T* o,
                         float* lse, int B, int Tn, int H, int hd, hipStream_t s) {
    const int64_t rows = (int64_t)B * Tn * H;
    const dim3 grid((unsigned)ceil_div(rows, kThreads));
    if (hd == 64)
        hipLaunchKernelGGL((k_attn_fwd_simt<T, 64>), grid, dim3(kThreads), 0, s, q, k, v, ldq, ldkv,
                           o, lse, B, Tn, H);
    else if (hd == 128)
        hipLaunchKernelGGL((k_attn_fwd_simt<T, 128>), grid, dim3(kThreads), 0, s, q, k, v, ldq,
                           ldkv, o, lse, B, Tn, H);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename T>
hipError_t attn_delta(const T* o, const T* dout, int64_t rows, int hd, float* delta,
                      hipStream_t s) {
    hipLaunchKernelGGL(k_attn_delta<T>, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, o,
                       dout, rows, hd, delta);
    return hipGetLastError();
}

template <typename T>
hipError_t attn_bwd_simt(const T* q, const T* k, const T* v, int64_t ldq, int64_t ldkv,
                         const T* o, const T* dout, const float* lse, float* delta, float* dq,
                         float* dk, float* dv, int B, int Tn, int H, int hd, hipStream_t s) {
    const int64_t rows = (int64_t)B * Tn * H;
    hipError_t e = attn_delta<T>(o, dout, rows, hd, delta, s);
    if (e != hipSuccess) return e;
    const dim3 gq((unsigned)ceil_div(rows, kThreads));
    const dim3 gk((unsigned)ceil_div((int64_t)B * Tn, kThreads));
    if (hd == 64) {
        hipLaunchKernelGGL((k_attn_bwd_dq_simt<T, 64>), gq, dim3(kThreads), 0, s, q, k, v, ldq,
                           ldkv, dout, lse, delta, dq, B, Tn, H);
        hipLaunchKernelGGL((k_attn_bwd_dkv_simt<T, 64>), gk, dim3(kThreads), 0, s, q, k, v, ldq,
                           ldkv, dout, lse, delta, dk, dv, B, Tn, H);
    } else if (hd == 128) {
        hipLaunchKernelGGL((k_attn_bwd_dq_simt<T, 128>), gq, dim3(kThreads), 0, s, q, k, v, ldq,
                           ldkv, dout, lse, delta, dq, B, Tn, H);
        hipLaunchKernelGGL((k_attn_bwd_dkv_simt<T, 128>), gk, dim3(kThreads), 0, s, q, k, v, ldq,
                           ldkv, dout, lse, delta, dk, dv, B, Tn, H);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t attn_fwd<float>(const float* q, const float* k, const float* v, int64_t ldq,
                           int64_t ldkv, float* o, float* lse, int B, int Tn, int H, int hd,
                           hipStream_t s, bool) {
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

}  // namespace nc
