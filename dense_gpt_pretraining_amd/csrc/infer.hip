// Generation with a key/value cache (include/nc_infer.h): the decode step and
// the kernels that prefill shares with it.
//
// The nanochat pages list a KV-cache inference engine with prefill and decode
// (tianqi.csdn.net feature list; vpshk.cn, section on the $100 run).  Under
// multi-query attention a position leaves one key row and one value row per
// layer for the positions after it; the cache holds exactly those rows (the
// key rotated and normalised, as attention reads it), [B][max_seq][hd] for
// keys and for values of each layer.
//
// A decode step is bound by HBM: it reads every weight matrix once (1 GB at
// depth 20) and the cache rows of every layer, for B <= 32 new tokens.
//   * Products y = x W^T of B rows run on the matrix cores as weight
//     streaming: a workgroup owns 32 rows of W, its four waves split the k
//     range, each issuing v_mfma_f32_32x32x16_bf16 with W's rows as the A
//     side and the B token rows as the B side straight from global memory
//     (W is read once; x is small and stays in L2); the four partial tiles
//     are summed in LDS in a fixed order and the epilogue (row scale,
//     relu^2, residual) applied there.  The fp32 configuration uses the
//     SIMT product of the GEMM family.
//     When N / 32 workgroups cannot keep the compute units streaming, the k
//     range is also cut into slices (raw sums to scratch, then a kernel that
//     adds them in slice order and applies the epilogue).
//   * Attention of the H query heads of a token over its cache is split
//     over chunks of keys (flash-decoding), and a second kernel merges the
//     chunks.  bf16 runs the chunks on the matrix cores (attn_mfma.hip, 256
//     keys per workgroup, the fixed softmax offset of QK-normalised heads);
//     fp32 uses chunks of 128 keys here: each workgroup scores one chunk for
//     every head (two threads per key, the key row read once for all H
//     heads), stages the chunk's value rows in LDS, keeps the chunk's max and
//     sum per head and its weighted value sum.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "../../include/nc.h"
#include "../../include/nc_infer.h"
#include "kernels.h"

namespace nc {

namespace {

constexpr int kGvThreads = 256;       // 4 waves, each a quarter of the k range
constexpr int kGvRows = 32;           // rows of W per workgroup
constexpr int kDecChunk = 128;        // keys per attention workgroup (two threads per key)
constexpr int kDecThreads = 2 * kDecChunk;
constexpr int kMaxHeads = 16;

// y[b][n] = epi(sum_k x[b][k] W[n][k]) for b < B <= 32, n < N; x row stride
// ldx, W [N][K] (K a multiple of 64), y row stride ldy.
// With gridDim.y = S > 1 the k range is cut into S slices: slice s writes its
// raw sums to part[s][b][n] and k_gemv_reduce applies the epilogue.
template <int MODE>
__global__ __launch_bounds__(kGvThreads) void k_gemv_mfma(const bf16_t* __restrict__ x,
                                                          int64_t ldx, int B,
                                                          const bf16_t* __restrict__ W, int N,
                                                          int K, const float* __restrict__ rs,
                                                          const bf16_t* __restrict__ aux,
                                                          void* __restrict__ y, int64_t ldy,
                                                          float* __restrict__ split_part) {
    __shared__ float part[4][kGvRows][kGvRows + 1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n0 = blockIdx.x * kGvRows;
    const int li = lane & 31, g = lane >> 5;
    const int nrow = min(n0 + li, N - 1);               // rows past N repeat the last one
    const bool brow = li < B;
    const int ks = K / (int)gridDim.y;                  // this slice's k range
    const int kq = ks / 4;
    const int kb = (int)blockIdx.y * ks + w * kq, ke = kb + kq;
    const bf16_t* wp = W + (int64_t)nrow * K + 8 * g;
    const bf16_t* xp = x + (int64_t)(brow ? li : 0) * ldx + 8 * g;
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    int k = kb;
    // four k steps per round: their loads are in flight together
    for (; k + 64 <= ke; k += 64) {
        uint4 a[4], bx[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = *reinterpret_cast<const uint4*>(wp + k + 16 * u);
            bx[u] = brow ? *reinterpret_cast<const uint4*>(xp + k + 16 * u) : z4;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma32(as_bf16x8(a[u]), as_bf16x8(bx[u]), acc);
    }
    for (; k < ke; k += 16) {
        const uint4 a = *reinterpret_cast<const uint4*>(wp + k);
        const uint4 bx = brow ? *reinterpret_cast<const uint4*>(xp + k) : z4;
        acc = mfma32(as_bf16x8(a), as_bf16x8(bx), acc);
    }
    // lane holds column b = li of D = W x^T, rows n = 8 (r/4) + 4 g + (r%4)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[w][8 * (r >> 2) + 4 * g + (r & 3)][li] = acc[r];
    __syncthreads();
    // thread t: four (b, n) outputs, consecutive n for consecutive threads
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = e * kGvThreads + threadIdx.x;
        const int b = idx / kGvRows, nn = idx % kGvRows;
        const int n = n0 + nn;
        if (b >= B || n >= N) continue;
        const float v = ((part[0][nn][b] + part[1][nn][b]) + part[2][nn][b]) + part[3][nn][b];
        if (gridDim.y > 1) {
            split_part[((int64_t)blockIdx.y * B + b) * N + n] = v;
            continue;
        }
        const int64_t o = (int64_t)b * ldy + n;
        if (MODE == EPI_STORE_F32) {
            static_cast<float*>(y)[o] = rs[b] * v;            // logits z = r f W^T, fp32
        } else {
            float u = v;
            if (MODE == EPI_ROWSCALE) u = rs[b] * v;
            if (MODE == EPI_ROWSCALE_RELU2) {
                const float t = fmaxf(rs[b] * v, 0.f);
                u = t * t;
            }
            if (MODE == EPI_RESID) u = bf2f(aux[o]) + v;
            static_cast<bf16_t*>(y)[o] = f2bf(u);
        }
    }
}

// the k slices' sums of k_gemv_mfma added in slice order, then its epilogue
template <int MODE>
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ part, int S, int B,
                                                     int N, const float* __restrict__ rs,
                                                     const bf16_t* __restrict__ aux,
                                                     void* __restrict__ y, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)B * N) return;
    const int b = (int)(i / N), n = (int)(i % N);
    float v = 0.f;
    for (int sl = 0; sl < S; ++sl) v += part[(int64_t)sl * B * N + i];
    const int64_t o = (int64_t)b * ldy + n;
    if (MODE == EPI_STORE_F32) {
        static_cast<float*>(y)[o] = rs[b] * v;
    } else {
        float u = v;
        if (MODE == EPI_ROWSCALE) u = rs[b] * v;
        if (MODE == EPI_ROWSCALE_RELU2) {
            const float t = fmaxf(rs[b] * v, 0.f);
            u = t * t;
        }
        if (MODE == EPI_RESID) u = bf2f(aux[o]) + v;
        static_cast<bf16_t*>(y)[o] = f2bf(u);
    }
}

// sum over k slices s = 0 .. S-1 of part[(s * B + b) * N + n], added in slice
// order; the loads of eight slices are issued before their adds
__device__ __forceinline__ float slice_sum(const float* __restrict__ part, int S, int B, int N,
                                           int b, int n) {
    const float* p = part + (int64_t)b * N + n;
    const int64_t st = (int64_t)B * N;
    float v = 0.f;
    int sl = 0;
    for (; sl + 8 <= S; sl += 8) {
        float a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = p[(sl + u) * st];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += a[u];
    }
    for (; sl < S; ++sl) v += p[sl * st];
    return v;
}

// The QKV product's k slices summed in slice order for token row b = blockIdx.x,
// then its epilogue: u = r[b] * sum; the query heads and the key head are
// rotated at position pos (pair (i, i + hd/2) by pos * base^(-2i/hd), the
// angle in fp64 as the step's tables) and RMS-normalised (queries to q_out in
// fp32, the key into its cache row); the value head goes to its cache row.
// Thread t takes rotary pairs t, t + 1024, ... of the row's (H + 2) hd/2
// pairs, head by head, so a head's pairs are hd/2 consecutive lanes.
__global__ __launch_bounds__(1024) void k_qkv_rope_reduce(
    const float* __restrict__ part, int S, int B, int H, int hd, const float* __restrict__ rs,
    int pos, double base, float eps, float* __restrict__ q_out, bf16_t* __restrict__ kc,
    bf16_t* __restrict__ vc, int max_seq) {
    // the hd/2 angles of position pos, once per workgroup
    __shared__ float cs_l[64], sn_l[64];
    const int b = blockIdx.x, t = threadIdx.x, half = hd >> 1;
    if (t < half) {
        const double ang = (double)pos * pow(base, -2.0 * (double)t / (double)hd);
        cs_l[t] = (float)cos(ang);
        sn_l[t] = (float)sin(ang);
    }
    __syncthreads();
    const int N = (H + 2) * hd;
    const float r = rs[b];
    const int64_t crow = ((int64_t)b * max_seq + pos) * hd;
    const int npairs = (H + 2) * half;
    // every pass covers whole heads (1024 is a multiple of hd/2)
    for (int p0 = 0; p0 < npairs; p0 += 1024) {
        const int p = p0 + t;
        const bool ok = p < npairs;
        const int h = ok ? p / half : H + 1, i = p % half;
        float u0 = 0.f, u1 = 0.f;
        if (ok) {
            const int n0 = h * hd + i;
            u0 = r * slice_sum(part, S, B, N, b, n0);
            u1 = r * slice_sum(part, S, B, N, b, n0 + half);
        }
        if (h == H + 1) {   // the value head (uniform over its lanes)
            if (ok) {
                vc[crow + i] = f2bf(u0);
                vc[crow + i + half] = f2bf(u1);
            }
            continue;
        }
        const float c = cs_l[i], sn = sn_l[i];
        const float y0 = u0 * c - u1 * sn, y1 = u0 * sn + u1 * c;
        // the head's sum of squares over its hd/2 lanes
        float ss = y0 * y0 + y1 * y1;
        for (int o = half >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        const float rr = 1.f / sqrtf(ss / (float)hd + eps);
        if (h < H) {
            float* qo = q_out + ((int64_t)b * H + h) * hd;
            qo[i] = y0 * rr;
            qo[i + half] = y1 * rr;
        } else {
            kc[crow + i] = f2bf(y0 * rr);
            kc[crow + i + half] = f2bf(y1 * rr);
        }
    }
}

// A residual product's k slices summed in slice order for token row
// b = blockIdx.x, plus the residual aux: y = bf16(aux + sum); and the RMS
// scale of the stored row, r[b] = 1 / sqrt(mean(y^2) + eps), for the next
// product's row scale.
__global__ __launch_bounds__(1024) void k_resid_rms_reduce(
    const float* __restrict__ part, int S, int B, int N, const bf16_t* __restrict__ aux,
    bf16_t* __restrict__ y, float eps, float* __restrict__ r_out) {
    __shared__ float red[16];
    const int b = blockIdx.x, t = threadIdx.x;
    float ss = 0.f;
    for (int n = t; n < N; n += 1024) {
        const float v = slice_sum(part, S, B, N, b, n);
        const int64_t o = (int64_t)b * N + n;
        const bf16_t w = f2bf(bf2f(aux[o]) + v);
        y[o] = w;
        const float f = bf2f(w);
        ss += f * f;
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    if (t == 0) {
        float tot = 0.f;
        for (int w = 0; w < 16; ++w) tot += red[w];
        r_out[b] = 1.f / sqrtf(tot / (float)N + eps);
    }
}

// Rotary at position pos then QK-norm for the H query heads (fp32 out) and
// the key head (T, into the cache row); the value head is copied to its cache
// row.  One wave per (token b, head h); lane i holds the pair (i, i + hd/2).
template <typename T>
__global__ __launch_bounds__(64) void k_decode_rope(const T* __restrict__ qkv, int64_t ldq,
                                                    int H, int hd, int pos,
                                                    const float* __restrict__ cos_t,
                                                    const float* __restrict__ sin_t, float eps,
                                                    float* __restrict__ q_out,
                                                    T* __restrict__ kc, T* __restrict__ vc,
                                                    int max_seq) {
    const int b = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
    const T* src = qkv + (int64_t)b * ldq + (int64_t)h * hd;
    const int64_t crow = ((int64_t)b * max_seq + pos) * hd;
    if (h == H + 1) {
        for (int d = i; d < hd; d += 64) vc[crow + d] = src[d];
        return;
    }
    const int half = hd >> 1;
    float y0 = 0.f, y1 = 0.f;
    if (i < half) {
        const float x0 = Elt<T>::ld(src + i), x1 = Elt<T>::ld(src + i + half);
        const float c = cos_t[(int64_t)pos * half + i], s = sin_t[(int64_t)pos * half + i];
        y0 = x0 * c - x1 * s;
        y1 = x0 * s + x1 * c;
    }
    const float ss = wave_sum(y0 * y0 + y1 * y1);
    const float rr = 1.f / sqrtf(ss / (float)hd + eps);
    if (i < half) {
        if (h < H) {
            float* qo = q_out + ((int64_t)b * H + h) * hd;
            qo[i] = y0 * rr;
            qo[i + half] = y1 * rr;
        } else {
            Elt<T>::st(kc + crow + i, y0 * rr);
            Elt<T>::st(kc + crow + i + half, y1 * rr);
        }
    }
}

// Chunk c of token b's keys 0 .. npos-1 (kDecChunk keys): per head j the
// chunk's max m, sum l of exp(s - m) and sum of exp(s - m) v, with
// s = q_j . k / sqrt(hd).  Two threads score one key (half of hd each); the
// chunk's value rows are staged in LDS with 16-byte copies, then thread t
// forms outputs (j, d) = (t + 256 r) / hd, % hd, reading consecutive d.
template <typename T>
__global__ __launch_bounds__(kDecThreads) void k_decode_attn(
    const float* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc, int max_seq,
    int npos, int H, int hd, float scale, int nch, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
    __shared__ float qs[kMaxHeads * 128];
    __shared__ float ps[kMaxHeads * kDecChunk];
    __shared__ __align__(16) T vs[kDecChunk * 128];
    __shared__ float red[kMaxHeads][kDecThreads / 64];
    const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int cnt = min(kDecChunk, npos - c * kDecChunk);
    for (int e = t; e < H * hd; e += kDecThreads) qs[e] = q[(int64_t)b * H * hd + e];
    {
        // value rows c*kDecChunk .. +cnt-1 are contiguous in the cache
        const uint4* src = reinterpret_cast<const uint4*>(
            vc + ((int64_t)b * max_seq + (int64_t)c * kDecChunk) * hd);
        uint4* dst = reinterpret_cast<uint4*>(vs);
        const int n16 = cnt * hd * (int)sizeof(T) / 16;
        for (int e = t; e < n16; e += kDecThreads) dst[e] = src[e];
    }
    __syncthreads();
    const int kl = t >> 1, hh = t & 1;
    const bool valid = kl < cnt;
    const int half = hd >> 1;
    const T* krow = kc + ((int64_t)b * max_seq + (int64_t)c * kDecChunk + (valid ? kl : 0)) * hd +
                    hh * half;
    float s[kMaxHeads];
#pragma unroll
    for (int j = 0; j < kMaxHeads; ++j) s[j] = 0.f;
    constexpr int kV = Elt<T>::kVec;
    for (int d0 = 0; d0 < half; d0 += kV) {
        float kv[kV];
        ld_vec<T>(krow + d0, kv);
#pragma unroll
        for (int j = 0; j < kMaxHeads; ++j) {
            if (j < H) {
                const float* qj = qs + j * hd + hh * half + d0;
#pragma unroll
                for (int e = 0; e < kV; ++e) s[j] = fmaf(qj[e], kv[e], s[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxHeads; ++j) {
        if (j < H) {
            s[j] += __shfl_xor(s[j], 1, 64);
            s[j] = valid ? s[j] * scale : -INFINITY;
            const float m = wave_max(s[j]);
            if (lane == 0) red[j][wv] = m;
        }
    }
    __syncthreads();
    float mj[kMaxHeads];
#pragma unroll
    for (int j = 0; j < kMaxHeads; ++j)
        mj[j] = j < H ? fmaxf(fmaxf(red[j][0], red[j][1]), fmaxf(red[j][2], red[j][3])) : 0.f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxHeads; ++j) {
        if (j < H) {
            const float p = valid ? expf(s[j] - mj[j]) : 0.f;
            if (hh == 0) ps[j * kDecChunk + kl] = p;
            const float l = wave_sum(hh == 0 ? p : 0.f);
            if (lane == 0) red[j][wv] = l;
        }
    }
    __syncthreads();
    const int64_t slot = (int64_t)b * nch + c;
    // thread j writes head j's max and sum (every thread holds every max)
#pragma unroll
    for (int j = 0; j < kMaxHeads; ++j) {
        if (j < H && t == j) {
            part_ml[(slot * H + j) * 2] = mj[j];
            part_ml[(slot * H + j) * 2 + 1] = (red[j][0] + red[j][1]) + (red[j][2] + red[j][3]);
        }
    }
    for (int idx = t; idx < H * hd; idx += kDecThreads) {
        const int j = idx / hd, d = idx - j * hd;
        const float* pj = ps + j * kDecChunk;
        const T* vd = vs + d;
        float acc = 0.f;
        for (int u = 0; u < cnt; ++u) acc = fmaf(pj[u], Elt<T>::ld(vd + u * hd), acc);
        part_o[(slot * H + j) * hd + d] = acc;
    }
}

// o[b][j*hd + d] = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c; one
// workgroup per (token b, head j), one thread per d
template <typename T>
__global__ __launch_bounds__(128) void k_decode_combine(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        int nch, int H, int hd,
                                                        T* __restrict__ o) {
    const int b = blockIdx.x, j = blockIdx.y, d = threadIdx.x;
    if (d >= hd) return;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, part_ml[(((int64_t)b * nch + c) * H + j) * 2]);
    float L = 0.f, acc = 0.f;
    for (int c = 0; c < nch; ++c) {
        const int64_t sl = ((int64_t)b * nch + c) * H + j;
        const float wgt = expf(part_ml[sl * 2] - M);
        L = fmaf(wgt, part_ml[sl * 2 + 1], L);
        acc = fmaf(wgt, part_o[sl * hd + d], acc);
    }
    Elt<T>::st(o + ((int64_t)b * H + j) * hd + d, acc / L);
}

// keys and values of prefill positions into the cache: token n = b*t0 + t
template <typename T>
__global__ __launch_bounds__(256) void k_cache_fill(const T* __restrict__ qkv, int64_t ldq,
                                                    int t0, int H, int hd, int64_t n_tok,
                                                    T* __restrict__ kc, T* __restrict__ vc,
                                                    int max_seq) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one element of 2*hd per token
    if (i >= n_tok * 2 * hd) return;
    const int64_t n = i / (2 * hd);
    const int e = (int)(i % (2 * hd));
    const int64_t b = n / t0, t = n % t0;
    const T val = qkv[n * ldq + (int64_t)H * hd + e];
    const int64_t row = (b * max_seq + t) * hd;
    if (e < hd) kc[row + e] = val;
    else vc[row + e - hd] = val;
}

// out[b] = x[b * t0 + t0 - 1] (the prompt's last position of each sequence)
template <typename T>
__global__ __launch_bounds__(256) void k_gather_last(const T* __restrict__ x, int D, int t0,
                                                     int B, T* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)B * D) return;
    const int64_t b = i / D, d = i % D;
    out[i] = x[(b * t0 + t0 - 1) * D + d];
}

// c = s tanh(z / s) in place over B rows of V logits (row stride V)
__global__ __launch_bounds__(256) void k_softcap_rows(float* __restrict__ z, int64_t n, float cap) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) z[i] = cap * tanhf(z[i] / cap);
}

}  // namespace

// k slices of a B-row product: enough workgroups to keep every compute unit
// streaming (about 512), each slice at least 256 of k (K / S a multiple of 64)
int gemv_splits(int N, int K) {
    const int wgs = (int)ceil_div(N, kGvRows);
    int best = 1;
    for (int sl = 2; sl <= 32; ++sl) {
        if (K % (64 * sl) || K / sl < 256) continue;
        if ((int64_t)wgs * sl > 1024) break;
        best = sl;
        if (wgs * sl >= 512) break;
    }
    return best;
}

template <int MODE>
hipError_t launch_gemv(const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int N, int K,
                       const float* rs, const bf16_t* aux, void* y, int64_t ldy, float* part,
                       int S, hipStream_t s) {
    hipLaunchKernelGGL(k_gemv_mfma<MODE>, dim3((unsigned)ceil_div(N, kGvRows), S),
                       dim3(kGvThreads), 0, s, x, ldx, B, W, N, K, rs, aux, y, ldy, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    hipLaunchKernelGGL(k_gemv_reduce<MODE>, dim3((unsigned)ceil_div((int64_t)B * N, 256)),
                       dim3(256), 0, s, part, S, B, N, rs, aux, y, ldy);
    return hipGetLastError();
}

hipError_t gemv(int mode, const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int N, int K,
                const float* rs, const bf16_t* aux, void* y, int64_t ldy, float* part,
                size_t part_elems, hipStream_t s) {
    if (B < 1 || B > 32 || K % 64 || N < 1) return hipErrorInvalidValue;
    int S = gemv_splits(N, K);
    if ((size_t)S * B * N > part_elems || !part) S = 1;
    switch (mode) {
        case EPI_STORE_F32:
            return launch_gemv<EPI_STORE_F32>(x, ldx, B, W, N, K, rs, aux, y, ldy, part, S, s);
        case EPI_ROWSCALE:
            return launch_gemv<EPI_ROWSCALE>(x, ldx, B, W, N, K, rs, aux, y, ldy, part, S, s);
        case EPI_ROWSCALE_RELU2:
            return launch_gemv<EPI_ROWSCALE_RELU2>(x, ldx, B, W, N, K, rs, aux, y, ldy, part, S,
                                                   s);
        case EPI_RESID:
            return launch_gemv<EPI_RESID>(x, ldx, B, W, N, K, rs, aux, y, ldy, part, S, s);
        default: return hipErrorInvalidValue;
    }
}

// The fused decode products: S k slices (gemv_splits of the shape) whose raw
// sums go to `part`, then the row-wise reduce with its epilogue.  Both need
// S > 1 (the caller checks gemv_fused_ok).
bool gemv_fused_ok(int N, int K, int B, size_t part_elems) {
    const int S = gemv_splits(N, K);
    return B >= 1 && B <= 32 && K % 64 == 0 && S > 1 && (size_t)S * B * N <= part_elems;
}

hipError_t gemv_qkv_rope(const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int H, int hd,
                         int K, const float* rs, int pos, double base, float eps, float* q_out,
                         bf16_t* kc, bf16_t* vc, int max_seq, float* part, hipStream_t s) {
    const int N = (H + 2) * hd;
    const int S = gemv_splits(N, K);
    if (S < 2 || 1024 % (hd / 2)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gemv_mfma<EPI_STORE_F32>, dim3((unsigned)ceil_div(N, kGvRows), S),
                       dim3(kGvThreads), 0, s, x, ldx, B, W, N, K, rs, nullptr, nullptr, 0, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_rope_reduce, dim3(B), dim3(1024), 0, s, part, S, B, H, hd, rs, pos,
                       base, eps, q_out, kc, vc, max_seq);
    return hipGetLastError();
}

hipError_t gemv_resid_rms(const bf16_t* x, int64_t ldx, int B, const bf16_t* W, int N, int K,
                          const bf16_t* aux, bf16_t* y, float eps, float* r_out, float* part,
                          hipStream_t s) {
    const int S = gemv_splits(N, K);
    if (S < 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gemv_mfma<EPI_STORE_F32>, dim3((unsigned)ceil_div(N, kGvRows), S),
                       dim3(kGvThreads), 0, s, x, ldx, B, W, N, K, nullptr, nullptr, nullptr, 0,
                       part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_resid_rms_reduce, dim3(B), dim3(1024), 0, s, part, S, B, N, aux, y, eps,
                       r_out);
    return hipGetLastError();
}

template <typename T>
hipError_t decode_rope(const T* qkv, int64_t ldq, int B, int H, int hd, int pos,
                       const float* cos_t, const float* sin_t, float eps, float* q_out, T* kc,
                       T* vc, int max_seq, hipStream_t s) {
    hipLaunchKernelGGL(k_decode_rope<T>, dim3(B, H + 2), dim3(64), 0, s, qkv, ldq, H, hd, pos,
                       cos_t, sin_t, eps, q_out, kc, vc, max_seq);
    return hipGetLastError();
}

int decode_chunks(int npos) { return (int)ceil_div(npos, kDecChunk); }

template <typename T>
hipError_t decode_attn(const float* q, const T* kc, const T* vc, int max_seq, int npos, int B,
                       int H, int hd, float* part_o, float* part_ml, T* o, hipStream_t s) {
    if (H > kMaxHeads || hd > 128 || hd % 16) return hipErrorInvalidValue;
    int nch;
    if (std::is_same<T, bf16_t>::value && (hd == 64 || hd == 128)) {
        // matrix-core chunks of 256 keys with the fixed softmax offset (the
        // step's queries and cached keys are QK-normalised)
        nch = attn_decode_chunks(npos);
        const hipError_t e = attn_decode_mfma(reinterpret_cast<const float*>(q),
                                              reinterpret_cast<const bf16_t*>(kc),
                                              reinterpret_cast<const bf16_t*>(vc), max_seq, npos,
                                              B, H, hd, part_o, part_ml, s);
        if (e != hipSuccess) return e;
    } else {
        nch = decode_chunks(npos);
        hipLaunchKernelGGL(k_decode_attn<T>, dim3(nch, B), dim3(kDecThreads), 0, s, q, kc, vc,
                           max_seq, npos, H, hd, 1.f / sqrtf((float)hd), nch, part_o, part_ml);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_decode_combine<T>, dim3(B, H), dim3(128), 0, s, part_o, part_ml, nch, H,
                       hd, o);
    return hipGetLastError();
}

template <typename T>
hipError_t cache_fill(const T* qkv, int64_t ldq, int B, int t0, int H, int hd, T* kc, T* vc,
                      int max_seq, hipStream_t s) {
    const int64_t n = (int64_t)B * t0 * 2 * hd;
    hipLaunchKernelGGL(k_cache_fill<T>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, qkv,
                       ldq, t0, H, hd, (int64_t)B * t0, kc, vc, max_seq);
    return hipGetLastError();
}

template <typename T>
hipError_t gather_last(const T* x, int D, int t0, int B, T* out, hipStream_t s) {
    const int64_t n = (int64_t)B * D;
    hipLaunchKernelGGL(k_gather_last<T>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, x, D,
                       t0, B, out);
    return hipGetLastError();
}

hipError_t softcap_rows(float* z, int64_t n, float cap, hipStream_t s) {
    hipLaunchKernelGGL(k_softcap_rows, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, z, n,
                       cap);
    return hipGetLastError();
}

#define NC_INST(T)                                                                              \
    template hipError_t decode_rope<T>(const T*, int64_t, int, int, int, int, const float*,    \
                                       const float*, float, float*, T*, T*, int, hipStream_t); \
    template hipError_t decode_attn<T>(const float*, const T*, const T*, int, int, int, int,   \
                                       int, float*, float*, T*, hipStream_t);                  \
    template hipError_t cache_fill<T>(const T*, int64_t, int, int, int, int, T*, T*, int,      \
                                      hipStream_t);                                            \
    template hipError_t gather_last<T>(const T*, int, int, int, T*, hipStream_t);
NC_INST(float)
NC_INST(bf16_t)
#undef NC_INST

}  // namespace nc
