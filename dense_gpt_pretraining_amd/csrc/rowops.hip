// Memory-bound kernels of the step: embedding + RMSNorm, RMSNorm statistics,
// rotary + QK-norm (forward and backward), the residual norm backward, the
// fused softcap + cross-entropy, reductions, transposes and initialisation.
//
// Row kernels give one wave (64 lanes) to a row and move 16 bytes per lane
// per access, so a wave reads 1 KiB contiguous per instruction.  Every
// statistic is accumulated in fp32.
#include <math.h>

#include "kernels.h"

namespace nc {

namespace {

constexpr int kRowsPerBlock = 4;   // 4 waves of 64 lanes
constexpr int kRowThreads = 256;

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_embed_fwd(
    const T* __restrict__ wte, const int32_t* __restrict__ tok, int N, int D,
    float eps, T* __restrict__ out, float* __restrict__ r) {
    constexpr int V = Elt<T>::kVec;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= N) return;
    const T* src = wte + (int64_t)tok[row] * D;
    float ss = 0.f;
    for (int c = lane * V; c < D; c += kWave * V) {
        float v[V];
        ld_vec<T>(src + c, v);
#pragma unroll
        for (int i = 0; i < V; ++i) ss += v[i] * v[i];
    }
    ss = wave_sum(ss);
    const float rr = 1.f / sqrtf(ss / (float)D + eps);
    T* dst = out + row * D;
    for (int c = lane * V; c < D; c += kWave * V) {
        float v[V];
        ld_vec<T>(src + c, v);
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] *= rr;
        st_vec<T>(dst + c, v);
    }
    if (lane == 0) r[row] = rr;
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_rms_stats(
    const T* __restrict__ x, int N, int D, float eps, float* __restrict__ r) {
    constexpr int V = Elt<T>::kVec;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= N) return;
    const T* src = x + row * D;
    float ss = 0.f;
    for (int c = lane * V; c < D; c += kWave * V) {
        float v[V];
        ld_vec<T>(src + c, v);
#pragma unroll
        for (int i = 0; i < V; ++i) ss += v[i] * v[i];
    }
    ss = wave_sum(ss);
    if (lane == 0) r[row] = 1.f / sqrtf(ss / (float)D + eps);
}

// rotary angle of pair i at position t is t * base^(-2i/hd), evaluated in fp64
__global__ void k_rope_tables(int Tn, int hd, double base, float* cos_t, float* sin_t) {
    const int half = hd / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)Tn * half) return;
    const int t = (int)(idx / half), i = (int)(idx % half);
    const double ang = (double)t * pow(base, -2.0 * (double)i / (double)hd);
    cos_t[idx] = (float)cos(ang);
    sin_t[idx] = (float)sin(ang);
}

// One unit = one head vector of one token; hd/2 lanes per unit, lane i owns
// the rotary pair (i, i + hd/2).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_rope_qknorm_fwd(
    T* __restrict__ qkv, int N, int Tn, int H, int hd,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, float eps,
    float* __restrict__ rqk) {
    const int half = hd >> 1;
    const int upw = kWave / half;
    const int lane = threadIdx.x & 63;
    const int64_t unit = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * upw + lane / half;
    const int i = lane % half;
    const int64_t n_units = (int64_t)N * (H + 1);
    const bool valid = unit < n_units;
    const int64_t token = valid ? unit / (H + 1) : 0;
    const int j = valid ? (int)(unit % (H + 1)) : 0;
    const int t = (int)(token % Tn);
    const int64_t ld = (int64_t)(H + 2) * hd;
    T* p = qkv + token * ld + (int64_t)j * hd;
    float x0 = 0.f, x1 = 0.f;
    if (valid) { x0 = Elt<T>::ld(p + i); x1 = Elt<T>::ld(p + i + half); }
    const float c = cos_t[(int64_t)t * half + i], s = sin_t[(int64_t)t * half + i];
    const float y0 = x0 * c - x1 * s;
    const float y1 = x0 * s + x1 * c;
    const float ss = group_sum(y0 * y0 + y1 * y1, half);
    const float rr = 1.f / sqrtf(ss / (float)hd + eps);
    if (valid) {
        Elt<T>::st(p + i, y0 * rr);
        Elt<T>::st(p + i + half, y1 * rr);
        if (i == 0) rqk[token * (H + 1) + j] = rr;
    }
}

// Units cover heads 0..H+1 of every token: q heads, the k head, the v head.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_rope_qknorm_bwd(
    const T* __restrict__ qkv, const float* __restrict__ dq,
    const float* __restrict__ dk, const float* __restrict__ dv,
    const float* __restrict__ rqk, const float* __restrict__ r1, int N, int Tn,
    int H, int hd, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, T* __restrict__ dqkv) {
    const int half = hd >> 1;
    const int upw = kWave / half;
    const int lane = threadIdx.x & 63;
    const int64_t unit = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * upw + lane / half;
    const int i = lane % half;
    const int64_t n_units = (int64_t)N * (H + 2);
    const bool valid = unit < n_units;
    const int64_t token = valid ? unit / (H + 2) : 0;
    const int j = valid ? (int)(unit % (H + 2)) : 0;
    const int t = (int)(token % Tn);
    const int64_t ld = (int64_t)(H + 2) * hd;
    const float scale = valid ? r1[token] : 0.f;
    T* out = dqkv + token * ld + (int64_t)j * hd;
    if (j == H + 1) {  // v head: no rotary, no norm (whole unit is uniform)
        if (valid) {
            const float* g = dv + token * hd;
            Elt<T>::st(out + i, scale * g[i]);
            Elt<T>::st(out + i + half, scale * g[i + half]);
        }
        return;
    }
    const float* g = (j < H) ? dq + (token * H + j) * hd : dk + token * hd;
    const T* y = qkv + token * ld + (int64_t)j * hd;
    float g0 = 0.f, g1 = 0.f, y0 = 0.f, y1 = 0.f, rr = 0.f;
    if (valid) {
        g0 = g[i]; g1 = g[i + half];
        y0 = Elt<T>::ld(y + i); y1 = Elt<T>::ld(y + i + half);
        rr = rqk[token * (H + 1) + j];
    }
    const float dot = group_sum(g0 * y0 + g1 * y1, half) / (float)hd;
    const float a0 = rr * (g0 - y0 * dot);
    const float a1 = rr * (g1 - y1 * dot);
    const float c = cos_t[(int64_t)t * half + i], s = sin_t[(int64_t)t * half + i];
    if (valid) {
        Elt<T>::st(out + i, scale * (a0 * c + a1 * s));
        Elt<T>::st(out + i + half, scale * (-a0 * s + a1 * c));
    }
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_embed_bwd_rows(
    const T* __restrict__ dh, const T* __restrict__ wte,
    const int32_t* __restrict__ tok, const float* __restrict__ r0, int N, int D,
    float* __restrict__ de) {
    constexpr int V = Elt<T>::kVec;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= N) return;
    const T* g = dh + row * D;
    const T* e = wte + (int64_t)tok[row] * D;
    float dot = 0.f;
    for (int c = lane * V; c < D; c += kWave * V) {
        float ev[V], gv[V];
        ld_vec<T>(e + c, ev);
        ld_vec<T>(g + c, gv);
#pragma unroll
        for (int k = 0; k < V; ++k) dot += gv[k] * ev[k];
    }
    dot = wave_sum(dot);
    const float rr = r0[row];
    const float coef = rr * rr * rr * dot / (float)D;
    float* o = de + row * D;
    for (int c = lane * V; c < D; c += kWave * V) {
        float ev[V], gv[V];
        ld_vec<T>(e + c, ev);
        ld_vec<T>(g + c, gv);
#pragma unroll
        for (int k = 0; k < V; ++k) o[c + k] = rr * gv[k] - coef * ev[k];
    }
}

// Softcap + cross-entropy, one 1024-thread block per row: at a 65536
// vocabulary each thread holds 8 chunks (60 registers), which leaves room for
// eight waves per SIMD, two rows per CU (9.5% faster than 512 threads with 16
// chunks and four waves per SIMD).  The raw row is held
// in registers (MAXC 16-byte chunks per thread), so logits are read from HBM
// once and gradients written once.  The softcap bounds every logit to
// |c| <= s, and the host admits only s <= 60, so sum(exp(c)) cannot overflow
// fp32 and the log-sum-exp needs no running maximum.
constexpr int kCeThreads = 1024;

template <typename T>
__device__ __forceinline__ void unpack_chunk(const uint4& raw, float* out);
template <>
__device__ __forceinline__ void unpack_chunk<float>(const uint4& raw, float* out) {
    out[0] = __uint_as_float(raw.x); out[1] = __uint_as_float(raw.y);
    out[2] = __uint_as_float(raw.z); out[3] = __uint_as_float(raw.w);
}
template <>
__device__ __forceinline__ void unpack_chunk<bf16_t>(const uint4& raw, float* out) {
    out[0] = bf_lo(raw.x); out[1] = bf_hi(raw.x); out[2] = bf_lo(raw.y); out[3] = bf_hi(raw.y);
    out[4] = bf_lo(raw.z); out[5] = bf_hi(raw.z); out[6] = bf_lo(raw.w); out[7] = bf_hi(raw.w);
}
template <typename T>
__device__ __forceinline__ uint4 pack_chunk(const float* in);
template <>
__device__ __forceinline__ uint4 pack_chunk<float>(const float* in) {
    return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                      __float_as_uint(in[3]));
}
template <>
__device__ __forceinline__ uint4 pack_chunk<bf16_t>(const float* in) {
    return make_uint4(pack_bf2(in[0], in[1]), pack_bf2(in[2], in[3]), pack_bf2(in[4], in[5]),
                      pack_bf2(in[6], in[7]));
}

// tanh(y) = 1 - 2 / (exp(2y) + 1) on the hardware exp2 and reciprocal units;
// saturates to +-1 (exp2 overflow gives 1/inf = 0).  Takes y2 = 2 y log2 e
// and returns r = 1/(exp(2y)+1), so that tanh = 1 - 2r and the softcapped
// logit is s (1 - 2r).
constexpr float kTwoLog2e = 2.8853900817779268f;
__device__ __forceinline__ float tanh_r(float y2) {
    return __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(y2) + 1.f);
}

// One wave per row.  The row's x, dn and residual gradient (all in the
// storage type T) are read once into registers (MAXC 16-byte chunks of each
// per lane), all requested before the row's dot product, so a row costs one
// round trip to HBM and HBM sees each input byte once.  The residual
// gradient is updated in place: dres <- dres + g - coef x, rounded to T once
// per norm.  With has_res = 0 (the final norm, where the residual gradient
// starts) dres is written without being read.
template <typename T, int MAXC>
__global__ __launch_bounds__(kRowThreads) void k_norm_bwd_resid(
    const T* __restrict__ dn, const T* __restrict__ x,
    const float* __restrict__ r, int N, int D, T* __restrict__ dres, int has_res) {
    constexpr int V = Elt<T>::kVec;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= N) return;
    const T* g = dn + row * D;
    const T* xr = x + row * D;
    T* d = dres + row * D;
    uint4 xraw[MAXC], graw[MAXC], draw[MAXC];
#pragma unroll
    for (int ci = 0; ci < MAXC; ++ci) {
        const int c = (ci * kWave + lane) * V;
        if (c < D) {
            xraw[ci] = *reinterpret_cast<const uint4*>(xr + c);
            graw[ci] = *reinterpret_cast<const uint4*>(g + c);
            draw[ci] = has_res ? *reinterpret_cast<const uint4*>(d + c) : make_uint4(0, 0, 0, 0);
        }
    }
    float dot = 0.f;
#pragma unroll
    for (int ci = 0; ci < MAXC; ++ci) {
        const int c = (ci * kWave + lane) * V;
        if (c < D) {
            float xv[V], gv[V];
            unpack_chunk<T>(xraw[ci], xv);
            unpack_chunk<T>(graw[ci], gv);
#pragma unroll
            for (int k = 0; k < V; ++k) dot += gv[k] * xv[k];
        }
    }
    dot = wave_sum(dot);
    const float rr = r[row];
    const float coef = rr * rr * dot / (float)D;
#pragma unroll
    for (int ci = 0; ci < MAXC; ++ci) {
        const int c = (ci * kWave + lane) * V;
        if (c < D) {
            float xv[V], gv[V], dv[V], o[V];
            unpack_chunk<T>(xraw[ci], xv);
            unpack_chunk<T>(graw[ci], gv);
            unpack_chunk<T>(draw[ci], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = dv[k] + gv[k] - coef * xv[k];
            st_vec<T>(d + c, o);
        }
    }
}

template <typename T, int MAXC>
__global__ __launch_bounds__(kCeThreads) void k_softcap_ce(
    T* __restrict__ z, int64_t ldz, int V, int N, const int32_t* __restrict__ tgt,
    float cap, const float* __restrict__ rowscale, float inv_n,
    float* __restrict__ tok_loss, int want_grad) {
    constexpr int VEC = Elt<T>::kVec;
    constexpr float kL2e = 1.4426950408889634f;
    __shared__ float red[kCeThreads / 64];
    const int64_t row = blockIdx.x;
    T* zr = z + row * ldz;
    // the argument of tanh_r: z / s times 2 log2 e
    const float zk = kTwoLog2e / cap;
    // exp(c) = 2^(s log2e (1 - 2r)) = 2^(a + b r)
    const float a = cap * kL2e, bb = -2.f * cap * kL2e;
    // With t = c/s = 1 - 2r, dL/dz = (softmax(c) - onehot) (1 - t^2) and
    // 1 - t^2 = 4 r (1 - r), so the softmax part of a column's gradient is
    // sc (4 / sum_j e_j) * e r (1 - r): every factor but the row's constant is
    // known in the first pass.  That pass overwrites each raw logit in
    // registers with g = e r (1 - r) in the storage type (zero for padding
    // columns), and the gradient pass is one product per column.
    uint4 raw[MAXC];
    float ssum = 0.f;
#pragma unroll
    for (int ci = 0; ci < MAXC; ++ci) {
        const int64_t c = ((int64_t)ci * kCeThreads + threadIdx.x) * VEC;
        if (c < ldz) {
            raw[ci] = *reinterpret_cast<const uint4*>(zr + c);
            float v[VEC], g[VEC];
            unpack_chunk<T>(raw[ci], v);
            if (c + VEC <= V) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const float r = tanh_r(v[k] * zk);
                    const float e = __builtin_amdgcn_exp2f(fmaf(bb, r, a));
                    ssum += e;
                    g[k] = e * fmaf(-r, r, r);
                }
            } else {
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    g[k] = 0.f;
                    if (c + k < V) {
                        const float r = tanh_r(v[k] * zk);
                        const float e = __builtin_amdgcn_exp2f(fmaf(bb, r, a));
                        ssum += e;
                        g[k] = e * fmaf(-r, r, r);
                    }
                }
            }
            raw[ci] = pack_chunk<T>(g);
        }
    }
    ssum = block_sum(ssum, red);
    const float lse = __logf(ssum);
    const int y = tgt[row];
    float zy = 0.f;   // the target's raw logit (thread 0)
    if (threadIdx.x == 0) {
        zy = Elt<T>::ld(zr + y);
        const float cy = cap * (1.f - 2.f * tanh_r(zy * zk));
        tok_loss[row] = lse - cy;
    }
    if (!want_grad) return;
    // every thread has finished reading z[y] before any thread overwrites it
    __syncthreads();
    const float sc = rowscale[row] * inv_n;
    const float kr = 4.f * sc / ssum;
    // column indices fit in 32 bits: rows are at most 16 chunks per thread
#pragma unroll
    for (int ci = 0; ci < MAXC; ++ci) {
        const int c = (ci * kCeThreads + (int)threadIdx.x) * VEC;
        if (c < ldz) {
            float g[VEC];
            unpack_chunk<T>(raw[ci], g);
#pragma unroll
            for (int k = 0; k < VEC; ++k) g[k] *= kr;
            st_vec<T>(zr + c, g);
        }
    }
    // the target column also carries the onehot term: thread 0 rewrites it,
    // from its raw logit in fp32, once every chunk store of the row has
    // completed
    __syncthreads();
    if (threadIdx.x == 0 && y >= 0 && y < V) {   // ids out of range write nothing
        const float ry = tanh_r(zy * zk);
        const float ey = __builtin_amdgcn_exp2f(fmaf(bb, ry, a));
        Elt<T>::st(zr + y, 4.f * sc * fmaf(-ry, ry, ry) * (ey / ssum - 1.f));
    }
}

__global__ __launch_bounds__(1024) void k_mean_reduce(const float* __restrict__ x, int N,
                                                     float* __restrict__ out) {
    __shared__ double red[1024];
    double s = 0.0;
    for (int i = threadIdx.x; i < N; i += 1024) s += (double)x[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = (float)(red[0] / (double)N);
}

template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ in, int rows,
                                                  int cols, int64_t ld_in,
                                                  T* __restrict__ out, int64_t ld_out) {
    __shared__ T tile[64][65];
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int k = ty; k < 64; k += 4) {
        const int r = r0 + k, c = c0 + tx;
        tile[k][tx] = (r < rows && c < cols) ? in[(int64_t)r * ld_in + c] : T(0);
    }
    __syncthreads();
    for (int k = ty; k < 64; k += 4) {
        const int c = c0 + k, r = r0 + tx;
        if (c < cols && r < ld_out) out[(int64_t)c * ld_out + r] = tile[tx][k];
    }
}

template <typename T>
__global__ void k_zero(T* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < n; k += stride) p[k] = T(0);
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) + Box-Muller
__device__ __forceinline__ void mulhilo(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
    const uint64_t p = (uint64_t)a * (uint64_t)b;
    hi = (uint32_t)(p >> 32);
    lo = (uint32_t)p;
}
__device__ __forceinline__ uint4 philox4x32_10(uint4 ctr, uint2 key) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(M0, ctr.x, hi0, lo0);
        mulhilo(M1, ctr.z, hi1, lo1);
        ctr = make_uint4(hi1 ^ ctr.y ^ key.x, lo1, hi0 ^ ctr.w ^ key.y, lo0);
        key.x += W0;
        key.y += W1;
    }
    return ctr;
}

template <typename T>
__global__ void k_init_normal(T* __restrict__ p, int64_t n, float stdv, uint64_t seed,
                              uint64_t stream_id) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 4 outputs each
    if (g * 4 >= n) return;
    const uint4 ctr = make_uint4((uint32_t)g, (uint32_t)((uint64_t)g >> 32),
                                 (uint32_t)stream_id, (uint32_t)(stream_id >> 32));
    const uint4 b = philox4x32_10(ctr, make_uint2((uint32_t)seed, (uint32_t)(seed >> 32)));
    const float k = 2.3283064365386963e-10f;  // 2^-32
    const float u1 = ((float)b.x + 1.f) * k, u2 = (float)b.y * k;
    const float u3 = ((float)b.z + 1.f) * k, u4 = (float)b.w * k;
    const float twopi = 6.283185307179586f;
    const float ra = sqrtf(-2.f * logf(fminf(u1, 1.f))), rb = sqrtf(-2.f * logf(fminf(u3, 1.f)));
    float o[4] = {ra * cosf(twopi * u2), ra * sinf(twopi * u2), rb * cosf(twopi * u4),
                  rb * sinf(twopi * u4)};
    for (int k2 = 0; k2 < 4; ++k2) {
        const int64_t idx = g * 4 + k2;
        if (idx < n) Elt<T>::st(p + idx, stdv * o[k2]);
    }
}

__global__ void k_count_bad(const int32_t* __restrict__ a, const int32_t* __restrict__ b,
                            int64_t n, int V, int32_t* __restrict__ n_bad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (i < n) bad = (a[i] < 0 || a[i] >= V) + (b[i] < 0 || b[i] >= V);
    // wave-level sum, one atomic per wave
    for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o, 64);
    if ((threadIdx.x & 63) == 0 && bad) atomicAdd(n_bad, bad);
}

inline int row_blocks(int64_t rows) { return (int)ceil_div(rows, kRowsPerBlock); }

}  // namespace

// ------------------------------------------------------------------ launchers
template <typename T>
hipError_t embed_fwd(const T* wte, const int32_t* tok, int N, int D, float eps, T* out,
                     float* r, hipStream_t s) {
    hipLaunchKernelGGL(k_embed_fwd<T>, dim3(row_blocks(N)), dim3(kRowThreads), 0, s, wte, tok,
                       N, D, eps, out, r);
    return hipGetLastError();
}

template <typename T>
hipError_t rms_stats(const T* x, int N, int D, float eps, float* r, hipStream_t s) {
    hipLaunchKernelGGL(k_rms_stats<T>, dim3(row_blocks(N)), dim3(kRowThreads), 0, s, x, N, D,
                       eps, r);
    return hipGetLastError();
}

hipError_t rope_tables(int Tn, int hd, float base, float* cos_t, float* sin_t, hipStream_t s) {
    const int64_t n = (int64_t)Tn * (hd / 2);
    hipLaunchKernelGGL(k_rope_tables, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, Tn, hd,
                       (double)base, cos_t, sin_t);
    return hipGetLastError();
}

template <typename T>
hipError_t rope_qknorm_fwd(T* qkv, int N, int Tn, int H, int hd, const float* cos_t,
                           const float* sin_t, float eps, float* rqk, hipStream_t s) {
    const int upw = kWave / (hd / 2);
    const int64_t waves = ceil_div((int64_t)N * (H + 1), upw);
    hipLaunchKernelGGL(k_rope_qknorm_fwd<T>, dim3(row_blocks(waves)), dim3(kRowThreads), 0, s,
                       qkv, N, Tn, H, hd, cos_t, sin_t, eps, rqk);
    return hipGetLastError();
}

template <typename T>
hipError_t rope_qknorm_bwd(const T* qkv, const float* dq, const float* dk, const float* dv,
                           const float* rqk, const float* r1, int N, int Tn, int H, int hd,
                           const float* cos_t, const float* sin_t, T* dqkv, hipStream_t s) {
    const int upw = kWave / (hd / 2);
    const int64_t waves = ceil_div((int64_t)N * (H + 2), upw);
    hipLaunchKernelGGL(k_rope_qknorm_bwd<T>, dim3(row_blocks(waves)), dim3(kRowThreads), 0, s,
                       qkv, dq, dk, dv, rqk, r1, N, Tn, H, hd, cos_t, sin_t, dqkv);
    return hipGetLastError();
}

template <typename T>
hipError_t norm_bwd_resid(const T* dn, const T* x, const float* r, int N, int D, T* dres,
                          bool has_res, hipStream_t s) {
    constexpr int VEC = Elt<T>::kVec;
    const int chunks = (int)ceil_div(D, kWave * VEC);
    const int hr = has_res ? 1 : 0;
#define NC_NB_CASE(C)                                                                         \
    if (chunks <= C) {                                                                        \
        hipLaunchKernelGGL((k_norm_bwd_resid<T, C>), dim3(row_blocks(N)), dim3(kRowThreads), 0, \
                           s, dn, x, r, N, D, dres, hr);                                      \
        return hipGetLastError();                                                             \
    }
    NC_NB_CASE(1)
    NC_NB_CASE(2)
    NC_NB_CASE(3)
    NC_NB_CASE(4)
    NC_NB_CASE(8)
    NC_NB_CASE(16)
#undef NC_NB_CASE
    return hipErrorInvalidValue;   // rows longer than 16 chunks per lane
}

template <typename T>
hipError_t embed_bwd_rows(const T* dh, const T* wte, const int32_t* tok, const float* r0,
                          int N, int D, float* de, hipStream_t s) {
    hipLaunchKernelGGL(k_embed_bwd_rows<T>, dim3(row_blocks(N)), dim3(kRowThreads), 0, s, dh,
                       wte, tok, r0, N, D, de);
    return hipGetLastError();
}

template <typename T>
hipError_t softcap_ce(T* z, int64_t ldz, int V, int N, const int32_t* tgt, float cap,
                      const float* rowscale, float inv_n, float* tok_loss, bool want_grad,
                      hipStream_t s) {
    constexpr int VEC = Elt<T>::kVec;
    const int64_t chunks = ceil_div(ldz, (int64_t)kCeThreads * VEC);
    const int wg = want_grad ? 1 : 0;
#define NC_CE_CASE(C)                                                                      \
    if (chunks <= C) {                                                                     \
        hipLaunchKernelGGL((k_softcap_ce<T, C>), dim3(N), dim3(kCeThreads), 0, s, z, ldz, V, N, \
                           tgt, cap, rowscale, inv_n, tok_loss, wg);                      \
        return hipGetLastError();                                                          \
    }
    NC_CE_CASE(1)
    NC_CE_CASE(4)
    NC_CE_CASE(8)
    NC_CE_CASE(16)
#undef NC_CE_CASE
    return hipErrorInvalidValue;  // rows wider than 16 chunks per thread are rejected on the host
}

hipError_t mean_reduce(const float* x, int N, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_mean_reduce, dim3(1), dim3(1024), 0, s, x, N, out);
    return hipGetLastError();
}

template <typename T>
hipError_t transpose(const T* in, int rows, int cols, int64_t ld_in, T* out, int64_t ld_out,
                     hipStream_t s) {
    dim3 grid((unsigned)ceil_div(ld_out, 64), (unsigned)ceil_div(cols, 64));
    hipLaunchKernelGGL(k_transpose<T>, grid, dim3(256), 0, s, in, rows, cols, ld_in, out, ld_out);
    return hipGetLastError();
}

template <typename T>
hipError_t zero_elems(T* p, int64_t n, hipStream_t s) {
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(n, 256), 65536);
    hipLaunchKernelGGL(k_zero<T>, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

template <typename T>
hipError_t init_normal(T* p, int64_t n, float stdv, uint64_t seed, uint64_t stream_id,
                       hipStream_t s) {
    const int64_t groups = ceil_div(n, 4);
    hipLaunchKernelGGL(k_init_normal<T>, dim3((unsigned)ceil_div(groups, 256)), dim3(256), 0, s,
                       p, n, stdv, seed, stream_id);
    return hipGetLastError();
}

int64_t softcap_ce_max_ld(int elem_bytes) { return (int64_t)16 * kCeThreads * (16 / elem_bytes); }

hipError_t count_bad_ids(const int32_t* a, const int32_t* b, int64_t n, int V, int32_t* n_bad,
                         hipStream_t s) {
    hipLaunchKernelGGL(k_count_bad, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, a, b, n,
                       V, n_bad);
    return hipGetLastError();
}

#define NC_INST(T)                                                                              \
    template hipError_t embed_fwd<T>(const T*, const int32_t*, int, int, float, T*, float*,   \
                                     hipStream_t);                                             \
    template hipError_t rms_stats<T>(const T*, int, int, float, float*, hipStream_t);          \
    template hipError_t rope_qknorm_fwd<T>(T*, int, int, int, int, const float*, const float*, \
                                           float, float*, hipStream_t);                        \
    template hipError_t rope_qknorm_bwd<T>(const T*, const float*, const float*, const float*, \
                                           const float*, const float*, int, int, int, int,     \
                                           const float*, const float*, T*, hipStream_t);       \
    template hipError_t norm_bwd_resid<T>(const T*, const T*, const float*, int, int, T*,  \
                                          bool, hipStream_t);                                  \
    template hipError_t embed_bwd_rows<T>(const T*, const T*, const int32_t*, const float*,   \
                                          int, int, float*, hipStream_t);                      \
    template hipError_t softcap_ce<T>(T*, int64_t, int, int, const int32_t*, float,           \
                                      const float*, float, float*, bool, hipStream_t);         \
    template hipError_t transpose<T>(const T*, int, int, int64_t, T*, int64_t, hipStream_t);  \
    template hipError_t zero_elems<T>(T*, int64_t, hipStream_t);                               \
    template hipError_t init_normal<T>(T*, int64_t, float, uint64_t, uint64_t, hipStream_t);
NC_INST(float)
NC_INST(bf16_t)
#undef NC_INST
template hipError_t zero_elems<int32_t>(int32_t*, int64_t, hipStream_t);

}  // namespace nc
