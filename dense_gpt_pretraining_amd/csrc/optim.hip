// Optimizer step after the forward+backward pass (include/nc_optim.h): AdamW
// for the embedding and the unembedding, Muon for the block matrices, global
// gradient-norm clipping, gradient accumulation and the schedule's multiplier.
//
// The nanochat article (vpshk.cn, optimizer paragraph of the section on the
// ~8000-line code base) names Muon with AdamW; the llm.c article (qian.cx,
// training-command paragraph) names accumulation, the schedule, weight decay
// and the gradient norm.  Their definitions are the published ones stated in
// nc_optim.h.
//
// Layout on the GPU.  The state holds three fp32 arrays with the parameters'
// offsets: the master weights, then AdamW's moments (or Muon's momentum and
// an unused array).  Every pass is elementwise and HBM-bound except the
// Newton-Schulz iteration, whose three products per step run on the GEMM
// family as one batched launch over the L layers' copies of a matrix (a
// 1280 x 1280 product alone fills 25 of the 256 compute units; the batch of
// 20 fills them).  The iteration keeps the matrix in the orientation it is
// stored in: for a tall matrix (rows > cols) the Gram matrix is X^T X, read
// as two mn-major operands, and the update is a X + X B (B is symmetric);
// for a wide one it is X X^T and a X + B X.  Reductions (norms) use a fixed
// partition and fixed summation order, so a step is bitwise reproducible.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/nc.h"
#include "../../include/nc_optim.h"
#include "kernels.h"

namespace nc {

namespace {

constexpr int kOptThreads = 256;
constexpr float kNsEps = 1e-7f;
constexpr float kClipEps = 1e-6f;
// quintic Newton-Schulz coefficients of the published Muon iteration
constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;

// block of `count` equally strided tensors of `len` elements each
struct Seg {
    int64_t off = 0, len = 0, stride = 0;
    int count = 1;
    int rows = 0, cols = 0;
    int nb = 1;          // reduction blocks per tensor
    int64_t part = 0;    // first partial of this block of tensors
};

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int s = blockDim.x >> 1; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    return red[0];
}

// chunk of a tensor taken by block b of nb: whole float4 groups
__device__ __forceinline__ void block_range(int64_t len, int nb, int b, int64_t& i0, int64_t& i1) {
    const int64_t chunk = ceil_div(ceil_div(len, nb), 4) * 4;
    i0 = min((int64_t)b * chunk, len);
    i1 = min(i0 + chunk, len);
}

// partials[part + y*nb + b] = sum of g^2 over block b's chunk of tensor y
__global__ __launch_bounds__(kOptThreads) void k_sumsq(const float* __restrict__ g, int64_t len,
                                                       int64_t stride, int nb,
                                                       float* __restrict__ partials) {
    __shared__ float red[kOptThreads / 64];
    const int y = blockIdx.y, b = blockIdx.x;
    const float* t = g + (int64_t)y * stride;
    int64_t i0, i1;
    block_range(len, nb, b, i0, i1);
    float s = 0.f;
    for (int64_t i = i0 + 4 * threadIdx.x; i < i1; i += 4 * kOptThreads) {
        const float4 v = *reinterpret_cast<const float4*>(t + i);
        s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    s = block_sum(s, red);
    if (threadIdx.x == 0) partials[(int64_t)y * nb + b] = s;
}

// out[y] = sqrt(sum of partials[y*n .. y*n + n-1]) in a fixed order; with
// clip_out, also the clipping factor of a single norm
__global__ __launch_bounds__(kOptThreads) void k_norms(const float* __restrict__ partials, int64_t n,
                                                       float* __restrict__ out, float max_norm,
                                                       float* __restrict__ clip_out) {
    __shared__ double red[kOptThreads];
    const int y = blockIdx.x;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kOptThreads) s += (double)partials[(int64_t)y * n + i];
    s = block_sum_f64(s, red);
    if (threadIdx.x == 0) {
        const float nrm = (float)sqrt(s);
        out[y] = nrm;
        if (clip_out) clip_out[0] = max_norm > 0.f ? fminf(1.f, max_norm / (nrm + kClipEps)) : 1.f;
    }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
    } else {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(a, b), pack_bf2(c, d));
    }
}
template <typename T>
__device__ __forceinline__ float4 load4(const T* p) {
    if constexpr (std::is_same<T, float>::value) {
        return *reinterpret_cast<const float4*>(p);
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
    }
}

// AdamW on one tensor of len elements (a multiple of 4)
template <typename T>
__global__ __launch_bounds__(kOptThreads) void k_adamw(
    T* __restrict__ params, float* __restrict__ master, float* __restrict__ m1,
    float* __restrict__ m2, const float* __restrict__ g, int64_t len,
    const float* __restrict__ clip, float lr, float b1, float b2, float eps, float decay,
    float inv_bc1, float inv_bc2) {
    const float cs = clip[0];
    const int64_t stride = (int64_t)gridDim.x * kOptThreads * 4;
    for (int64_t i = ((int64_t)blockIdx.x * kOptThreads + threadIdx.x) * 4; i < len; i += stride) {
        const float4 gv = *reinterpret_cast<const float4*>(g + i);
        float4 th = *reinterpret_cast<const float4*>(master + i);
        float4 a = *reinterpret_cast<const float4*>(m1 + i);
        float4 b = *reinterpret_cast<const float4*>(m2 + i);
        float* thp = &th.x;
        float* ap = &a.x;
        float* bp = &b.x;
        const float* gp = &gv.x;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float gq = gp[q] * cs;
            ap[q] = b1 * ap[q] + (1.f - b1) * gq;
            bp[q] = b2 * bp[q] + (1.f - b2) * gq * gq;
            const float mh = ap[q] * inv_bc1, vh = bp[q] * inv_bc2;
            thp[q] = thp[q] * decay - lr * (mh / (sqrtf(vh) + eps));
        }
        *reinterpret_cast<float4*>(master + i) = th;
        *reinterpret_cast<float4*>(m1 + i) = a;
        *reinterpret_cast<float4*>(m2 + i) = b;
        store4<T>(params + i, th.x, th.y, th.z, th.w);
    }
}

// Muon momentum on tensor y of a strided block: buf = mu buf + clip*g, and
// block b's partial sum of U^2 with U = clip*g + mu buf (Nesterov) or buf
__global__ __launch_bounds__(kOptThreads) void k_muon_momentum(
    const float* __restrict__ g, float* __restrict__ buf, int64_t len, int64_t stride, int nb,
    const float* __restrict__ clip, float mu, int nesterov, float* __restrict__ partials) {
    __shared__ float red[kOptThreads / 64];
    const int y = blockIdx.y, b = blockIdx.x;
    const float* gt = g + (int64_t)y * stride;
    float* bt = buf + (int64_t)y * stride;
    const float cs = clip[0];
    int64_t i0, i1;
    block_range(len, nb, b, i0, i1);
    float s = 0.f;
    for (int64_t i = i0 + 4 * threadIdx.x; i < i1; i += 4 * kOptThreads) {
        const float4 gv = *reinterpret_cast<const float4*>(gt + i);
        float4 bv = *reinterpret_cast<const float4*>(bt + i);
        const float* gp = &gv.x;
        float* bp = &bv.x;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float gq = gp[q] * cs;
            bp[q] = mu * bp[q] + gq;
            const float u = nesterov ? gq + mu * bp[q] : bp[q];
            s += u * u;
        }
        *reinterpret_cast<float4*>(bt + i) = bv;
    }
    s = block_sum(s, red);
    if (threadIdx.x == 0) partials[(int64_t)y * nb + b] = s;
}

// X[y] = U / (|U|_F + eps), U recomputed from g and the updated buf
template <typename T>
__global__ __launch_bounds__(kOptThreads) void k_muon_x0(
    const float* __restrict__ g, const float* __restrict__ buf, int64_t len, int64_t stride,
    const float* __restrict__ clip, float mu, int nesterov, const float* __restrict__ norms,
    T* __restrict__ X) {
    const int y = blockIdx.y;
    const float* gt = g + (int64_t)y * stride;
    const float* bt = buf + (int64_t)y * stride;
    T* xt = X + (int64_t)y * len;
    const float cs = clip[0];
    const float inv = 1.f / (norms[y] + kNsEps);
    const int64_t step = (int64_t)gridDim.x * kOptThreads * 4;
    for (int64_t i = ((int64_t)blockIdx.x * kOptThreads + threadIdx.x) * 4; i < len; i += step) {
        const float4 gv = *reinterpret_cast<const float4*>(gt + i);
        const float4 bv = *reinterpret_cast<const float4*>(bt + i);
        const float* gp = &gv.x;
        const float* bp = &bv.x;
        float u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] = (nesterov ? gp[q] * cs + mu * bp[q] : bp[q]) * inv;
        store4<T>(xt + i, u[0], u[1], u[2], u[3]);
    }
}

// theta = theta * decay - lr_eff * X[y]; params = (T) theta
template <typename T>
__global__ __launch_bounds__(kOptThreads) void k_muon_apply(
    T* __restrict__ params, float* __restrict__ master, const T* __restrict__ X, int64_t len,
    int64_t stride, float lr_eff, float decay) {
    const int y = blockIdx.y;
    T* pt = params + (int64_t)y * stride;
    float* mt = master + (int64_t)y * stride;
    const T* xt = X + (int64_t)y * len;
    const int64_t step = (int64_t)gridDim.x * kOptThreads * 4;
    for (int64_t i = ((int64_t)blockIdx.x * kOptThreads + threadIdx.x) * 4; i < len; i += step) {
        const float4 x = load4<T>(xt + i);
        float4 th = *reinterpret_cast<const float4*>(mt + i);
        th.x = th.x * decay - lr_eff * x.x;
        th.y = th.y * decay - lr_eff * x.y;
        th.z = th.z * decay - lr_eff * x.z;
        th.w = th.w * decay - lr_eff * x.w;
        *reinterpret_cast<float4*>(mt + i) = th;
        store4<T>(pt + i, th.x, th.y, th.z, th.w);
    }
}

// master = (float) params; s1 = s2 = 0
template <typename T>
__global__ __launch_bounds__(kOptThreads) void k_optim_init(const T* __restrict__ params,
                                                            float* __restrict__ master,
                                                            float* __restrict__ s1,
                                                            float* __restrict__ s2, int64_t n) {
    const int64_t step = (int64_t)gridDim.x * kOptThreads;
    for (int64_t i = (int64_t)blockIdx.x * kOptThreads + threadIdx.x; i < n; i += step) {
        master[i] = Elt<T>::ld(params + i);
        s1[i] = 0.f;
        s2[i] = 0.f;
    }
}

// acc = (overwrite ? 0 : acc) + scale * g; n4 float4 groups, then a tail
__global__ __launch_bounds__(kOptThreads) void k_grad_accumulate(float* __restrict__ acc,
                                                                 const float* __restrict__ g,
                                                                 int64_t n, float scale,
                                                                 int overwrite) {
    const int64_t n4 = n / 4;
    const int64_t step = (int64_t)gridDim.x * kOptThreads;
    for (int64_t i = (int64_t)blockIdx.x * kOptThreads + threadIdx.x; i < n4; i += step) {
        const float4 gv = reinterpret_cast<const float4*>(g)[i];
        float4 a = overwrite ? make_float4(0.f, 0.f, 0.f, 0.f) : reinterpret_cast<float4*>(acc)[i];
        a.x += scale * gv.x;
        a.y += scale * gv.y;
        a.z += scale * gv.z;
        a.w += scale * gv.w;
        reinterpret_cast<float4*>(acc)[i] = a;
    }
    const int64_t t = 4 * n4 + (int64_t)blockIdx.x * kOptThreads + threadIdx.x;
    if (t < n) acc[t] = (overwrite ? 0.f : acc[t]) + scale * g[t];
}

unsigned grid_for(int64_t len) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(len, 4 * kOptThreads), 4096));
}

int nb_for(int64_t len) { return (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(len, 65536), 512)); }

struct OptPlan {
    std::vector<Seg> adam;    // wte, wlm
    std::vector<Seg> muon;    // wq, wk, wv, wo, wfc, wproj (each over L layers)
    int64_t n_params = 0;
    int64_t gparts = 0;       // partials of the global norm
    int mparts = 0;           // partials of one Muon block of tensors
    int64_t max_x = 0, max_a = 0;
    size_t off_gpart = 0, off_gnorm = 0, off_mpart = 0, off_mnorm = 0, off_x0 = 0, off_x1 = 0,
           off_a = 0, off_b = 0, bytes = 0;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_opt_plan(const nc_config* cfg, OptPlan& p) {
    int rc = nc_param_count(cfg, &p.n_params);
    if (rc != NC_OK) return rc;
    int32_t n = 0;
    rc = nc_param_layout(cfg, nullptr, 0, &n);
    if (rc != NC_OK && rc != NC_ERR_CAPACITY) return rc;
    std::vector<nc_tensor_info> info(n);
    rc = nc_param_layout(cfg, info.data(), n, &n);
    if (rc != NC_OK) return rc;
    const int L = cfg->n_layer;
    auto one = [](const nc_tensor_info& t) {
        Seg s;
        s.off = t.offset;
        s.rows = t.rows;
        s.cols = t.cols;
        s.len = (int64_t)t.rows * t.cols;
        s.count = 1;
        return s;
    };
    p.adam = {one(info[0]), one(info[n - 1])};
    for (int k = 0; k < 6; ++k) {
        Seg s = one(info[1 + k]);
        s.count = L;
        s.stride = L > 1 ? info[1 + 6 + k].offset - info[1 + k].offset : 0;
        for (int l = 1; l < L; ++l)   // the layout repeats layer by layer
            if (info[1 + 6 * l + k].offset != s.off + l * s.stride) return NC_ERR_UNSUPPORTED;
        p.muon.push_back(s);
    }
    // every tensor is a whole number of float4 groups at 16-byte aligned offsets
    for (const std::vector<Seg>* v : {&p.adam, &p.muon})
        for (const Seg& s : *v)
            if (s.len % 4 || s.off % 4 || s.stride % 4) return NC_ERR_UNSUPPORTED;
    int64_t part = 0;
    int mparts = 0;
    for (Seg& s : p.adam) {
        s.nb = nb_for(s.len);
        s.part = part;
        part += s.nb;
    }
    for (Seg& s : p.muon) {
        s.nb = nb_for(s.len);
        s.part = part;
        part += (int64_t)s.nb * s.count;
        mparts = std::max(mparts, s.nb * s.count);
        p.max_x = std::max<int64_t>(p.max_x, s.len * s.count);
        const int64_t m = std::min(s.rows, s.cols);
        p.max_a = std::max<int64_t>(p.max_a, m * m * s.count);
    }
    p.gparts = part;
    p.mparts = mparts;
    const size_t es = cfg->dtype == NC_BF16 ? 2 : 4;
    size_t off = 0;
    auto take = [&](size_t b) { size_t r = off; off += al256(b); return r; };
    p.off_gpart = take((size_t)p.gparts * 4);
    p.off_gnorm = take(16);
    p.off_mpart = take((size_t)mparts * 4);
    p.off_mnorm = take((size_t)L * 4);
    p.off_x0 = take((size_t)p.max_x * es);
    p.off_x1 = take((size_t)p.max_x * es);
    p.off_a = take((size_t)p.max_a * es);
    p.off_b = take((size_t)p.max_a * es);
    p.bytes = off;
    return NC_OK;
}

int check_ocfg(const nc_optim_config* o) {
    auto fin = [](float x) { return std::isfinite(x); };
    if (!fin(o->adam_lr) || o->adam_lr < 0.f || !fin(o->muon_lr) || o->muon_lr < 0.f)
        return NC_ERR_CONFIG;
    if (!(o->adam_beta1 >= 0.f && o->adam_beta1 < 1.f) ||
        !(o->adam_beta2 >= 0.f && o->adam_beta2 < 1.f))
        return NC_ERR_CONFIG;
    if (!(o->adam_eps > 0.f) || !fin(o->adam_eps)) return NC_ERR_CONFIG;
    if (!(o->adam_weight_decay >= 0.f) || !fin(o->adam_weight_decay) ||
        !(o->muon_weight_decay >= 0.f) || !fin(o->muon_weight_decay))
        return NC_ERR_CONFIG;
    if (!(o->muon_momentum >= 0.f && o->muon_momentum < 1.f)) return NC_ERR_CONFIG;
    if (o->muon_ns_steps < 0 || o->muon_ns_steps > 16) return NC_ERR_CONFIG;
    if (o->muon_nesterov != 0 && o->muon_nesterov != 1) return NC_ERR_CONFIG;
    if (!(o->grad_clip >= 0.f) || !fin(o->grad_clip)) return NC_ERR_CONFIG;
    return NC_OK;
}

#define OPT_TRY(expr)                          \
    do {                                       \
        hipError_t e_ = (expr);                \
        if (e_ != hipSuccess) {                \
            note_hip_error((int)e_);           \
            return NC_ERR_HIP;                 \
        }                                      \
    } while (0)

hipError_t last() { return hipGetLastError(); }

// One Muon block of tensors (one kind over all layers): momentum, norms,
// X0, the Newton-Schulz iteration, the update.
template <typename T>
int muon_block(const nc_config* cfg, const nc_optim_config* o, float lr_mult, const Seg& s,
               const OptPlan& p, const float* grads, T* params, float* master, float* buf,
               char* ws, const float* clip, hipStream_t st) {
    float* mpart = reinterpret_cast<float*>(ws + p.off_mpart);
    float* mnorm = reinterpret_cast<float*>(ws + p.off_mnorm);
    T* X = reinterpret_cast<T*>(ws + p.off_x0);
    T* Xn = reinterpret_cast<T*>(ws + p.off_x1);
    T* A = reinterpret_cast<T*>(ws + p.off_a);
    T* Bm = reinterpret_cast<T*>(ws + p.off_b);
    const int L = s.count;
    hipLaunchKernelGGL(k_muon_momentum, dim3(s.nb, L), dim3(kOptThreads), 0, st, grads + s.off,
                       buf + s.off, s.len, s.stride, s.nb, clip, o->muon_momentum,
                       o->muon_nesterov, mpart);
    OPT_TRY(last());
    hipLaunchKernelGGL(k_norms, dim3(L), dim3(kOptThreads), 0, st, mpart, (int64_t)s.nb, mnorm,
                       0.f, nullptr);
    OPT_TRY(last());
    hipLaunchKernelGGL(k_muon_x0<T>, dim3(grid_for(s.len), L), dim3(kOptThreads), 0, st,
                       grads + s.off, buf + s.off, s.len, s.stride, clip, o->muon_momentum,
                       o->muon_nesterov, mnorm, X);
    OPT_TRY(last());
    const int r = s.rows, c = s.cols;
    const bool tall = r > c;
    const int m = tall ? c : r;
    const int64_t xs = (int64_t)r * c, as = (int64_t)m * m;
    for (int it = 0; it < o->muon_ns_steps; ++it) {
        Epilogue e;
        e.mode = EPI_STORE_T;
        GemmBatch bg{L, xs, xs, as};
        // Gram matrix: X X^T (wide) or X^T X (tall)
        if (tall)
            OPT_TRY(gemm<T>(m, m, r, X, c, false, X, c, false, A, m, e, nullptr, 0, st, &bg));
        else
            OPT_TRY(gemm<T>(m, m, c, X, c, true, X, c, true, A, m, e, nullptr, 0, st, &bg));
        // Bm = b A + c A A (A symmetric, so A A = A A^T)
        Epilogue ep;
        ep.mode = EPI_AXPBY;
        ep.aux = A;
        ep.alpha = kNsB;
        ep.beta = kNsC;
        GemmBatch bp{L, as, as, as};
        OPT_TRY(gemm<T>(m, m, m, A, m, true, A, m, true, Bm, m, ep, nullptr, 0, st, &bp));
        // X' = a X + Bm X (wide) or a X + X Bm (tall)
        Epilogue eu;
        eu.mode = EPI_AXPBY;
        eu.aux = X;
        eu.alpha = kNsA;
        eu.beta = 1.f;
        if (tall) {
            GemmBatch bu{L, xs, as, xs};
            OPT_TRY(gemm<T>(r, c, m, X, c, true, Bm, m, false, Xn, c, eu, nullptr, 0, st, &bu));
        } else {
            GemmBatch bu{L, as, xs, xs};
            OPT_TRY(gemm<T>(r, c, m, Bm, m, true, X, c, false, Xn, c, eu, nullptr, 0, st, &bu));
        }
        std::swap(X, Xn);
    }
    const float lr = o->muon_lr * lr_mult;
    const float scale = std::sqrt(std::max(1.f, (float)r / (float)c));
    hipLaunchKernelGGL(k_muon_apply<T>, dim3(grid_for(s.len), L), dim3(kOptThreads), 0, st,
                       params + s.off, master + s.off, X, s.len, s.stride, lr * scale,
                       1.f - lr * o->muon_weight_decay);
    OPT_TRY(last());
    return NC_OK;
}

template <typename T>
int optim_step(const nc_config* cfg, const nc_optim_config* o, int64_t step, float lr_mult,
               const float* grads, void* params_v, void* state, float* grad_norm, char* ws,
               const OptPlan& p, hipStream_t st) {
    T* params = static_cast<T*>(params_v);
    float* master = static_cast<float*>(state);
    const size_t arr = al256((size_t)p.n_params * 4);
    float* s1 = reinterpret_cast<float*>(static_cast<char*>(state) + arr);
    float* s2 = reinterpret_cast<float*>(static_cast<char*>(state) + 2 * arr);
    float* gpart = reinterpret_cast<float*>(ws + p.off_gpart);
    float* gnorm = reinterpret_cast<float*>(ws + p.off_gnorm);   // [norm, clip]
    // global gradient norm over every tensor, then the clipping factor
    for (const Seg& s : p.adam) {
        hipLaunchKernelGGL(k_sumsq, dim3(s.nb, 1), dim3(kOptThreads), 0, st, grads + s.off, s.len,
                           (int64_t)0, s.nb, gpart + s.part);
        OPT_TRY(last());
    }
    for (const Seg& s : p.muon) {
        hipLaunchKernelGGL(k_sumsq, dim3(s.nb, s.count), dim3(kOptThreads), 0, st, grads + s.off,
                           s.len, s.stride, s.nb, gpart + s.part);
        OPT_TRY(last());
    }
    hipLaunchKernelGGL(k_norms, dim3(1), dim3(kOptThreads), 0, st, gpart, p.gparts, gnorm,
                       o->grad_clip, gnorm + 1);
    OPT_TRY(last());
    if (grad_norm) OPT_TRY(hipMemcpyAsync(grad_norm, gnorm, 4, hipMemcpyDeviceToDevice, st));
    const float* clip = gnorm + 1;
    // AdamW: wte, wlm
    const double t = (double)step;
    const float inv_bc1 = (float)(1.0 / (1.0 - std::pow((double)o->adam_beta1, t)));
    const float inv_bc2 = (float)(1.0 / (1.0 - std::pow((double)o->adam_beta2, t)));
    const float lr_a = o->adam_lr * lr_mult;
    for (const Seg& s : p.adam) {
        hipLaunchKernelGGL(k_adamw<T>, dim3(grid_for(s.len)), dim3(kOptThreads), 0, st,
                           params + s.off, master + s.off, s1 + s.off, s2 + s.off, grads + s.off,
                           s.len, clip, lr_a, o->adam_beta1, o->adam_beta2, o->adam_eps,
                           1.f - lr_a * o->adam_weight_decay, inv_bc1, inv_bc2);
        OPT_TRY(last());
    }
    // Muon: each kind of block matrix over all layers
    for (const Seg& s : p.muon) {
        int rc = muon_block<T>(cfg, o, lr_mult, s, p, grads, params, master, s1, ws, clip, st);
        if (rc != NC_OK) return rc;
    }
    return NC_OK;
}

bool al(const void* q, size_t a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; }

}  // namespace
}  // namespace nc

extern "C" {

int nc_optim_state_size(const nc_config* cfg, size_t* bytes) {
    if (!bytes) return NC_ERR_NULL;
    int64_t n = 0;
    int rc = nc_param_count(cfg, &n);
    if (rc != NC_OK) return rc;
    *bytes = 3 * nc::al256((size_t)n * 4);
    return NC_OK;
}

int nc_optim_workspace_size(const nc_config* cfg, size_t* bytes) {
    if (!bytes) return NC_ERR_NULL;
    nc::OptPlan p;
    int rc = nc::make_opt_plan(cfg, p);
    if (rc != NC_OK) return rc;
    *bytes = p.bytes;
    return NC_OK;
}

int nc_optim_init(const nc_config* cfg, const void* params, void* state, void* stream) {
    int64_t n = 0;
    int rc = nc_param_count(cfg, &n);
    if (rc != NC_OK) return rc;
    if (!params || !state) return NC_ERR_NULL;
    if (!nc::al(params, 256) || !nc::al(state, 256)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    const size_t arr = nc::al256((size_t)n * 4);
    float* master = static_cast<float*>(state);
    float* s1 = reinterpret_cast<float*>(static_cast<char*>(state) + arr);
    float* s2 = reinterpret_cast<float*>(static_cast<char*>(state) + 2 * arr);
    const unsigned grid = (unsigned)std::min<int64_t>(nc::ceil_div(n, nc::kOptThreads), 65536);
    if (cfg->dtype == NC_BF16)
        hipLaunchKernelGGL(nc::k_optim_init<nc::bf16_t>, dim3(grid), dim3(nc::kOptThreads), 0, s,
                           static_cast<const nc::bf16_t*>(params), master, s1, s2, n);
    else
        hipLaunchKernelGGL(nc::k_optim_init<float>, dim3(grid), dim3(nc::kOptThreads), 0, s,
                           static_cast<const float*>(params), master, s1, s2, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        nc::note_hip_error((int)e);
        return NC_ERR_HIP;
    }
    return NC_OK;
}

int nc_optim_step(const nc_config* cfg, const nc_optim_config* ocfg, int64_t step,
                  float lr_mult, const float* grads, void* params, void* state,
                  float* grad_norm, void* ws, size_t ws_bytes, void* stream) {
    if (!ocfg) return NC_ERR_NULL;
    nc::OptPlan p;
    int rc = nc::make_opt_plan(cfg, p);
    if (rc != NC_OK) return rc;
    rc = nc::check_ocfg(ocfg);
    if (rc != NC_OK) return rc;
    if (step < 1 || !(lr_mult >= 0.f) || !std::isfinite(lr_mult)) return NC_ERR_CONFIG;
    if (!grads || !params || !state || !ws) return NC_ERR_NULL;
    if (!nc::al(grads, 256) || !nc::al(params, 256) || !nc::al(state, 256) ||
        !nc::al(ws, 256) || (grad_norm && !nc::al(grad_norm, 4)))
        return NC_ERR_ALIGN;
    if (ws_bytes < p.bytes) return NC_ERR_WORKSPACE;
    hipStream_t s = nc::enqueue_stream(stream);
    if (cfg->dtype == NC_BF16)
        return nc::optim_step<nc::bf16_t>(cfg, ocfg, step, lr_mult, grads, params, state,
                                          grad_norm, static_cast<char*>(ws), p, s);
    return nc::optim_step<float>(cfg, ocfg, step, lr_mult, grads, params, state, grad_norm,
                                 static_cast<char*>(ws), p, s);
}

int nc_grad_accumulate(float* acc, const float* grads, int64_t n, float scale, int32_t overwrite,
                       void* stream) {
    if (!acc || !grads) return NC_ERR_NULL;
    if (n < 0 || !std::isfinite(scale)) return NC_ERR_CONFIG;
    if (!nc::al(acc, 16) || !nc::al(grads, 16)) return NC_ERR_ALIGN;
    if (n == 0) return NC_OK;
    hipStream_t s = nc::enqueue_stream(stream);
    const unsigned grid = (unsigned)std::max<int64_t>(
        1, std::min<int64_t>(nc::ceil_div(n / 4, nc::kOptThreads), 65536));
    hipLaunchKernelGGL(nc::k_grad_accumulate, dim3(grid), dim3(nc::kOptThreads), 0, s, acc, grads,
                       n, scale, overwrite ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        nc::note_hip_error((int)e);
        return NC_ERR_HIP;
    }
    return NC_OK;
}

double nc_lr_multiplier(int64_t step, int64_t total, int64_t warmup, double final_frac) {
    if (total < 1 || warmup < 0 || !(final_frac >= 0.0 && final_frac <= 1.0) || step < 0)
        return -1.0;
    if (step < warmup) return (double)(step + 1) / (double)warmup;
    if (step >= total) return final_frac;
    const double span = (double)std::max<int64_t>(1, total - warmup);
    const double prog = (double)(step - warmup) / span;
    return final_frac + (1.0 - final_frac) * 0.5 * (1.0 + std::cos(M_PI * prog));
}

}  // extern "C"
