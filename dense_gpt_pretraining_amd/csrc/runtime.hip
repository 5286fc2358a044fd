// Host runtime behind the C ABI of include/nc.h: configuration checks, the
// parameter layout, the workspace plan and the launch sequence of one
// forward(+backward) step on one stream.
//
// Step (nanochat article on vpshk.cn, architecture list; pre-norm placement is
// the Llama-like reading): h0 = n(W_te[x]); per block
//   a = n(h); [q;k;v] = a W_qkv^T; q,k rotated then normalised per head;
//   h' = h + attn(q,k,v) W_o^T; m = n(h'); h'' = h' + relu(m W_fc^T)^2 W_proj^T;
// then f = n(h_L), z = f W_lm^T, c = s tanh(z/s), loss = mean(lse(c) - c[y]).
//
// Parameter-free RMSNorm makes n(x) W^T = diag(r) (x W^T) with
// r = 1/sqrt(mean(x^2) + eps), so no normalised copy of the residual stream
// is ever stored: the norm enters the producing GEMM's epilogue as a row scale
// r, and in the backward pass the same row scale is folded into the gradient
// dy' = r dy.  Then dW = dy'^T x and, with dn' = dy' W, the input gradient is
// dx = dn' - r^2 x mean(dn' * x).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/nc.h"
#include "../../include/nc_infer.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kAlignElems = 128;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int vocab_pad(const nc_config& c) { return (int)round_up(c.vocab, 256); }

int validate(const nc_config* c) {
    if (!c) return NC_ERR_NULL;
    if (c->dtype != NC_F32 && c->dtype != NC_BF16) return NC_ERR_DTYPE;
    if (c->n_layer < 1 || c->d_model < 8 || c->n_head < 1 || c->d_mlp < 8 || c->vocab < 2 ||
        c->seq_len < 1 || c->batch < 1 || c->n_kv_head < 1)
        return NC_ERR_CONFIG;
    if (!(c->softcap > 0.f) || !std::isfinite(c->softcap) || !(c->rms_eps >= 0.f) ||
        !std::isfinite(c->rms_eps) || !(c->rope_base > 1.f) || !std::isfinite(c->rope_base))
        return NC_ERR_CONFIG;
    if (c->head_dim != 64 && c->head_dim != 128) return NC_ERR_UNSUPPORTED;
    if (c->n_kv_head != 1) return NC_ERR_UNSUPPORTED;
    // k-major GEMM operands are staged 64 columns at a time straight into LDS
    if (c->d_model % 64 || c->d_mlp % 64) return NC_ERR_UNSUPPORTED;
    if (c->seq_len % 64) return NC_ERR_UNSUPPORTED;
    if (c->softcap > 60.f) return NC_ERR_UNSUPPORTED;
    if (c->vocab > (1 << 24)) return NC_ERR_UNSUPPORTED;
    // the fused cross-entropy keeps a padded vocabulary row in registers, and
    // the norm backward a residual row (16 chunks per lane of 64)
    const int64_t vec = c->dtype == NC_BF16 ? 8 : 4;
    if (vocab_pad(*c) > nc::softcap_ce_max_ld(c->dtype == NC_BF16 ? 2 : 4))
        return NC_ERR_UNSUPPORTED;
    if (c->d_model > 16 * 64 * vec) return NC_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)c->batch * c->seq_len;
    if (N > (1 << 24)) return NC_ERR_UNSUPPORTED;
    const int64_t widest = std::max<int64_t>(
        {(int64_t)vocab_pad(*c), c->d_mlp, (int64_t)(c->n_head + 2) * c->head_dim, c->d_model});
    if (N * widest >= ((int64_t)1 << 40)) return NC_ERR_UNSUPPORTED;
    return NC_OK;
}

struct TensorDesc {
    std::string name;
    int64_t offset;
    int32_t rows, cols;
};

// wq, wk, wv of a layer are adjacent with no padding between them so that
// together they form one [(H+2) hd, D] matrix
std::vector<TensorDesc> layout(const nc_config& c, int64_t* total) {
    std::vector<TensorDesc> out;
    const int D = c.d_model, H = c.n_head, hd = c.head_dim, F = c.d_mlp, V = c.vocab;
    int64_t off = 0;
    auto add = [&](const std::string& n, int r, int k, bool pad_after) {
        out.push_back({n, off, r, k});
        off += (int64_t)r * k;
        if (pad_after) off = round_up(off, kAlignElems);
    };
    add("wte", V, D, true);
    for (int l = 0; l < c.n_layer; ++l) {
        const std::string p = "h" + std::to_string(l) + ".";
        add(p + "wq", H * hd, D, false);
        add(p + "wk", hd, D, false);
        add(p + "wv", hd, D, true);
        add(p + "wo", D, H * hd, true);
        add(p + "wfc", F, D, true);
        add(p + "wproj", D, F, true);
    }
    add("wlm", V, D, true);
    if (total) *total = off;
    return out;
}

// ------------------------------------------------------------------ workspace plan
struct Plan {
    // per-layer saved tensors: element offsets relative to buffer bases
    size_t bytes = 0;
    // offsets (bytes) of each region inside the workspace
    size_t cos_t, sin_t, r0, x, r1, qkv, rqk, o, lse, xm, r2, g, rf, z, tok_loss, loss_tmp;
    size_t dres_t, dn, dgu, dout, delta, dq, dk, dv, dqkv, wt, splitk, embed;
    size_t splitk_bytes = 0, embed_bytes = 0;
    int slots = 1;     // saved-activation slots per layer tensor (L with backward, 1 without
                       // or with recompute)
    int x_slots = 2;   // block inputs: L+1 with backward, 2 (ping-pong) without
    bool recompute = false;   // the backward forms each block's tensors again
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// data-gradient product C = A W (M x N, contraction K) with the [K][N] weight
// read where it is stored, as an mn-major operand: no transposed copy
template <typename T>
hipError_t gemm_w(int M, int N, int K, const T* A, int64_t lda, const T* W, int64_t ldw, T* C,
                  int64_t ldc, const nc::Epilogue& e, hipStream_t s) {
    return nc::gemm<T>(M, N, K, A, lda, true, W, ldw, false, C, ldc, e, nullptr, 0, s);
}

Plan make_plan(const nc_config& c, bool bwd, bool recompute = false, bool infer = false) {
    Plan p;
    p.recompute = bwd && recompute;
    const int64_t N = (int64_t)c.batch * c.seq_len;
    const int64_t D = c.d_model, H = c.n_head, hd = c.head_dim, F = c.d_mlp, V = c.vocab;
    const int64_t Vp = vocab_pad(c);
    const int64_t Wq = (H + 2) * hd;
    const size_t es = c.dtype == NC_BF16 ? 2 : 4;
    const int L = c.n_layer;
    p.slots = bwd && !p.recompute ? L : 1;
    p.x_slots = bwd ? L + 1 : 2;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t r = off; off += align256(bytes); return r; };
    p.cos_t = take((size_t)c.seq_len * (hd / 2) * 4);
    p.sin_t = take((size_t)c.seq_len * (hd / 2) * 4);
    p.r0 = take((size_t)N * 4);
    p.x = take((size_t)p.x_slots * align256(N * D * es));
    p.r1 = take((size_t)p.slots * align256(N * 4));
    p.qkv = take((size_t)p.slots * align256(N * Wq * es));
    p.rqk = take((size_t)p.slots * align256(N * (H + 1) * 4));
    p.o = take((size_t)p.slots * align256(N * H * hd * es));
    p.lse = take((size_t)p.slots * align256(N * H * 4));
    p.xm = take((size_t)p.slots * align256(N * D * es));
    p.r2 = take((size_t)p.slots * align256(N * 4));
    p.g = take((size_t)p.slots * align256(N * F * es));
    p.rf = take((size_t)N * 4);
    // prefill reads the logits of one position per sequence only
    p.z = take(infer ? 0 : (size_t)N * Vp * es);
    p.tok_loss = take(infer ? 0 : (size_t)N * 4);
    p.loss_tmp = take(16);
    if (bwd) {
        p.dres_t = take((size_t)N * D * es);
        p.dn = take((size_t)N * D * 4);
        p.dgu = take((size_t)N * F * es);
        p.dout = take((size_t)N * H * hd * es);
        p.delta = take(nc::attn_bwd_scratch_bytes(c.batch, c.seq_len, (int)H, (int)hd));
        p.dq = take((size_t)N * H * hd * 4);
        p.dk = take((size_t)N * hd * 4);
        p.dv = take((size_t)N * hd * 4);
        p.dqkv = take((size_t)N * Wq * es);
        // the unembedding weight transposed to [D][Vp] with zero padding, for
        // a padded vocabulary only (otherwise the head's data gradient reads
        // W_lm where it is stored, as the per-layer data gradients do)
        p.wt = take(V == Vp ? 0 : (size_t)(D * Vp) * es);
        size_t sk = 0;
        sk = std::max(sk, nc::gemm_splitk_bytes((int)V, (int)D, (int)N));
        sk = std::max(sk, nc::gemm_splitk_bytes((int)D, (int)F, (int)N));
        sk = std::max(sk, nc::gemm_splitk_bytes((int)F, (int)D, (int)N));
        sk = std::max(sk, nc::gemm_splitk_bytes((int)D, (int)(H * hd), (int)N));
        sk = std::max(sk, nc::gemm_splitk_bytes((int)Wq, (int)D, (int)N));
        p.splitk_bytes = sk;
        p.splitk = take(sk);
        p.embed_bytes = nc::embed_grad_ws_bytes((int)N, (int)D, (int)V);
        p.embed = take(p.embed_bytes);
    }
    p.bytes = off;
    return p;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define NC_TRY(expr)                                   \
    do {                                               \
        hipError_t e_ = (expr);                        \
        if (e_ != hipSuccess) {                        \
            g_last_hip_error = (int)e_;                \
            return NC_ERR_HIP;                         \
        }                                              \
    } while (0)

// Per-kernel HIP events for the timed step variant.  A segment runs from one
// event to the next on the step's stream and covers one kernel.
struct Prof {
    struct Rec {
        const char* label;
        double flops, bytes;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    hipStream_t s = nullptr;
    Rec open{nullptr, 0, 0, nullptr, nullptr};
    hipError_t mark(hipEvent_t* ev) {
        hipError_t e = hipEventCreate(ev);
        if (e != hipSuccess) return e;
        return hipEventRecord(*ev, s);
    }
    hipError_t begin(const char* label, double flops, double bytes) {
        open = {label, flops, bytes, nullptr, nullptr};
        return mark(&open.a);
    }
    hipError_t close() {
        hipError_t e = mark(&open.b);
        recs.push_back(open);
        open = {nullptr, 0, 0, nullptr, nullptr};
        return e;
    }
    hipError_t cut(const char* label, double flops, double bytes) {
        hipEvent_t e = nullptr;
        hipError_t err = mark(&e);
        open.b = e;
        recs.push_back(open);
        open = {label, flops, bytes, e, nullptr};
        // the event now ends one segment and starts the next; keep ownership
        // with the earlier record only
        return err;
    }
    ~Prof() {
        for (size_t i = 0; i < recs.size(); ++i) {
            if (recs[i].a && (i == 0 || recs[i].a != recs[i - 1].b)) (void)hipEventDestroy(recs[i].a);
            if (recs[i].b) (void)hipEventDestroy(recs[i].b);
        }
        if (open.a && (recs.empty() || open.a != recs.back().b)) (void)hipEventDestroy(open.a);
    }
};

thread_local Prof* g_prof = nullptr;

// run one launcher; with a profiler, bracket it with events and record its
// algorithmic flops and HBM bytes under `label` (launchers that issue several
// kernels split the bracket with prof_cut)
#define NC_RUN(label, flops, bytes, expr)                                          \
    do {                                                                           \
        if (prof) NC_TRY(prof->begin(label, (double)(flops), (double)(bytes)));    \
        NC_TRY(expr);                                                              \
        if (prof) NC_TRY(prof->close());                                           \
    } while (0)

template <typename T>
struct Step {
    const nc_config& c;
    const Plan& p;
    char* ws;
    hipStream_t s;
    const T* params;
    Prof* prof;
    std::vector<TensorDesc> lay;
    int64_t N, D, H, hd, F, V, Vp, Wq;

    Step(const nc_config& cfg, const Plan& plan, void* w, hipStream_t st, const void* prm,
         Prof* pr)
        : c(cfg), p(plan), ws(static_cast<char*>(w)), s(st), params(static_cast<const T*>(prm)),
          prof(pr) {
        lay = layout(c, nullptr);
        N = (int64_t)c.batch * c.seq_len;
        D = c.d_model; H = c.n_head; hd = c.head_dim; F = c.d_mlp; V = c.vocab;
        Vp = vocab_pad(c);
        Wq = (H + 2) * hd;
    }
    template <typename U> U* at(size_t off) { return reinterpret_cast<U*>(ws + off); }
    template <typename U> U* slot(size_t base, int i, size_t per_bytes) {
        return reinterpret_cast<U*>(ws + base + (size_t)i * align256(per_bytes));
    }
    const T* W(int idx) const { return params + lay[idx].offset; }
    int i_wte() const { return 0; }
    int i_layer(int l, int k) const { return 1 + 6 * l + k; }  // k: 0 wq,1 wk,2 wv,3 wo,4 wfc,5 wproj
    int i_wlm() const { return 1 + 6 * c.n_layer; }

    double es() const { return (double)sizeof(T); }
    size_t ess() const { return sizeof(T); }
    T* X(int i) { return slot<T>(p.x, i, N * D * ess()); }
    float* R1(int l) { return slot<float>(p.r1, l, N * 4); }
    T* QKV(int l) { return slot<T>(p.qkv, l, N * Wq * ess()); }
    float* RQK(int l) { return slot<float>(p.rqk, l, N * (H + 1) * 4); }
    T* O(int l) { return slot<T>(p.o, l, N * H * hd * ess()); }
    float* LSE(int l) { return slot<float>(p.lse, l, N * H * 4); }
    T* XM(int l) { return slot<T>(p.xm, l, N * D * ess()); }
    float* R2(int l) { return slot<float>(p.r2, l, N * 4); }
    T* G(int l) { return slot<T>(p.g, l, N * F * ess()); }

    nc::Epilogue epi(int mode, const float* rs = nullptr, const void* aux = nullptr) {
        nc::Epilogue e;
        e.mode = mode;
        e.rowscale = rs;
        e.aux = aux;
        return e;
    }
    // algorithmic work of a GEMM C[M,N] = A[M,K] B[N,K]^T: both operands read
    // once, the output written once (out_es bytes per element), plus extra
    // bytes the epilogue reads
    double gf(int64_t m, int64_t n, int64_t k) const { return 2.0 * m * n * k; }
    double gb(int64_t m, int64_t n, int64_t k, double out_es, double extra = 0) const {
        return (double)(m * k + n * k) * es() + (double)m * n * out_es + extra;
    }
    // causal score pairs of one head over the batch: B * T(T+1)/2
    double pairs() const { return (double)c.batch * c.seq_len * (c.seq_len + 1) / 2.0; }

    // One block's forward from its input x: saves (into slot sl) everything
    // its backward reads; with_proj also forms the block output xn (the
    // recompute pass before a block's backward needs everything but xn).
    int layer_fwd(int l, int sl, T* x, T* xn, bool with_proj) {
        const float eps = c.rms_eps;
        float* cos_t = at<float>(p.cos_t);
        float* sin_t = at<float>(p.sin_t);
        const double rowb = (double)N * D * es();
        float* r1 = R1(sl);
        T* qkv = QKV(sl);
        NC_RUN("rms_stats", 0, rowb + N * 4.0, nc::rms_stats<T>(x, (int)N, (int)D, eps, r1, s));
        if constexpr (std::is_same<T, nc::bf16_t>::value) {
            // rotary + QK-norm in the projection's epilogue
            nc::Epilogue e = epi(nc::EPI_QKV_ROPE, r1);
            e.cos_t = cos_t;
            e.sin_t = sin_t;
            e.rqk = RQK(sl);
            e.seq_len = c.seq_len;
            e.n_head = (int)H;
            e.head_dim = (int)hd;
            e.eps = eps;
            NC_RUN("gemm_nt_qkv_rope", gf(N, Wq, D), gb(N, Wq, D, es(), N * (H + 5.0) * 4.0),
                   nc::gemm<T>((int)N, (int)Wq, (int)D, x, D, true, W(i_layer(l, 0)), D, true, qkv,
                               Wq, e, nullptr, 0, s));
        } else {
            NC_RUN("gemm_nt_rowscale", gf(N, Wq, D), gb(N, Wq, D, es(), N * 4.0),
                   nc::gemm<T>((int)N, (int)Wq, (int)D, x, D, true, W(i_layer(l, 0)), D, true, qkv,
                               Wq, epi(nc::EPI_ROWSCALE, r1), nullptr, 0, s));
            NC_RUN("rope_qknorm_fwd", 0, 2.0 * N * (H + 1) * hd * es() + N * (H + 1) * 4.0,
                   nc::rope_qknorm_fwd<T>(qkv, (int)N, c.seq_len, (int)H, (int)hd, cos_t, sin_t,
                                          eps, RQK(sl), s));
        }
        NC_RUN("attn_fwd", 4.0 * hd * H * pairs(),
               2.0 * N * H * hd * es() + 2.0 * N * hd * es() + N * H * 4.0,
               // q and k leave QK-norm with RMS 1 per head
               nc::attn_fwd<T>(qkv, qkv + H * hd, qkv + (H + 1) * hd, Wq, Wq, O(sl), LSE(sl),
                               c.batch, c.seq_len, (int)H, (int)hd, s, true));
        T* xm = XM(sl);
        NC_RUN("gemm_nt_resid", gf(N, D, H * hd), gb(N, D, H * hd, es(), rowb),
               nc::gemm<T>((int)N, (int)D, (int)(H * hd), O(sl), H * hd, true, W(i_layer(l, 3)),
                           H * hd, true, xm, D, epi(nc::EPI_RESID, nullptr, x), nullptr, 0, s));
        float* r2 = R2(sl);
        NC_RUN("rms_stats", 0, rowb + N * 4.0, nc::rms_stats<T>(xm, (int)N, (int)D, eps, r2, s));
        NC_RUN("gemm_nt_relu2", gf(N, F, D), gb(N, F, D, es(), N * 4.0),
               nc::gemm<T>((int)N, (int)F, (int)D, xm, D, true, W(i_layer(l, 4)), D, true, G(sl),
                           F, epi(nc::EPI_ROWSCALE_RELU2, r2), nullptr, 0, s));
        if (with_proj)
            NC_RUN("gemm_nt_resid", gf(N, D, F), gb(N, D, F, es(), rowb),
                   nc::gemm<T>((int)N, (int)D, (int)F, G(sl), F, true, W(i_layer(l, 5)), F, true,
                               xn, D, epi(nc::EPI_RESID, nullptr, xm), nullptr, 0, s));
        return NC_OK;
    }

    // slot of layer l's saved tensors: one per layer when the backward keeps
    // them all, a single one without backward or with recompute
    int slot_of(int l) const { return p.slots > 1 ? l : 0; }

    // Prefill: the forward of the blocks over B sequences of seq_len
    // positions, writing every layer's key and value rows into the cache;
    // returns the last block's output (nullptr on a failed launch).
    T* prefill_blocks(const int32_t* tok, T* cache, int max_seq) {
        const float eps = c.rms_eps;
        const double rowb = (double)N * D * es();
        auto fail = [](hipError_t e) { g_last_hip_error = (int)e; };
        hipError_t e = nc::rope_tables(c.seq_len, (int)hd, c.rope_base, at<float>(p.cos_t),
                                       at<float>(p.sin_t), s);
        if (e == hipSuccess)
            e = nc::embed_fwd<T>(W(i_wte()), tok, (int)N, (int)D, eps, X(0), at<float>(p.r0), s);
        if (e != hipSuccess) { fail(e); return nullptr; }
        (void)rowb;
        const int64_t per = (int64_t)c.batch * max_seq * hd;
        for (int l = 0; l < c.n_layer; ++l) {
            if (layer_fwd(l, 0, X(l & 1), X((l + 1) & 1), true) != NC_OK) return nullptr;
            e = nc::cache_fill<T>(QKV(0), Wq, c.batch, c.seq_len, (int)H, (int)hd,
                                  cache + 2 * l * per, cache + (2 * l + 1) * per, max_seq, s);
            if (e != hipSuccess) { fail(e); return nullptr; }
        }
        return X(c.n_layer & 1);
    }

    int forward(const int32_t* tok, const int32_t* tgt, float* loss, float* tok_loss, bool bwd) {
        const float eps = c.rms_eps;
        float* cos_t = at<float>(p.cos_t);
        float* sin_t = at<float>(p.sin_t);
        const double rowb = (double)N * D * es();
        NC_RUN("rope_tables", 0, c.seq_len * hd * 4.0,
               nc::rope_tables(c.seq_len, (int)hd, c.rope_base, cos_t, sin_t, s));
        NC_RUN("embed_fwd", 0, 2 * rowb + N * 8.0,
               nc::embed_fwd<T>(W(i_wte()), tok, (int)N, (int)D, eps, X(0), at<float>(p.r0), s));
        const int L = c.n_layer;
        for (int l = 0; l < L; ++l) {
            // with backward every block input is kept (L+1 slots); without,
            // two slots alternate
            T* x = X(bwd ? l : (l & 1));
            T* xn = X(bwd ? l + 1 : ((l + 1) & 1));
            int rc = layer_fwd(l, slot_of(l), x, xn, true);
            if (rc != NC_OK) return rc;
        }
        T* hL = X(bwd ? L : (L & 1));
        float* rf = at<float>(p.rf);
        NC_RUN("rms_stats", 0, rowb + N * 4.0, nc::rms_stats<T>(hL, (int)N, (int)D, eps, rf, s));
        T* z = at<T>(p.z);
        NC_RUN("gemm_nt_rowscale", gf(N, V, D), gb(N, V, D, es(), N * 4.0),
               nc::gemm<T>((int)N, (int)V, (int)D, hL, D, true, W(i_wlm()), D, true, z, Vp,
                           epi(nc::EPI_ROWSCALE, rf), nullptr, 0, s));
        float* tl = tok_loss ? tok_loss : at<float>(p.tok_loss);
        NC_RUN("softcap_ce", 0, (bwd ? 2.0 : 1.0) * N * Vp * es() + N * 12.0,
               nc::softcap_ce<T>(z, Vp, (int)V, (int)N, tgt, c.softcap, rf, 1.f / (float)N, tl,
                                 bwd, s));
        NC_RUN("mean_reduce", 0, N * 4.0 + 4, nc::mean_reduce(tl, (int)N, loss, s));
        return NC_OK;
    }

    int backward(const int32_t* tok, float* grads) {
        const int L = c.n_layer;
        T* wt = at<T>(p.wt);
        float* sk = at<float>(p.splitk);
        const size_t skb = p.splitk_bytes;
        // the residual-stream gradient, in the storage type (updated in place
        // by each norm backward, read by the products as their dY operand)
        T* dres_t = at<T>(p.dres_t);
        // data gradient entering a norm backward, stored as T (the buffer
        // keeps fp32 size: the embedding backward reuses it as fp32 de)
        T* dn = at<T>(p.dn);
        T* z = at<T>(p.z);  // now holds r_f/N * dloss/dz
        auto G_of = [&](int idx) { return grads + lay[idx].offset; };
        // norm backward with residual: reads dn, x, dres; writes dres
        const double nbb = (double)N * D * 4 * es() + N * 4.0;
        auto tb = [&](int64_t r, int64_t k) { return 2.0 * r * k * es(); };

        // head: df' = dz' W_lm, dW_lm = dz'^T h_L
        T* hL = X(L);
        if (V == Vp) {
            // no padded columns: the product reads W_lm where it is stored
            NC_RUN("gemm_nt_dn", gf(N, D, V), gb(N, D, V, es()),
                   gemm_w<T>((int)N, (int)D, (int)V, z, Vp, W(i_wlm()), D, dn, D,
                             epi(nc::EPI_STORE_T), s));
        } else {
            NC_RUN("transpose_w", 0, tb(V, D),
                   nc::transpose<T>(W(i_wlm()), (int)V, (int)D, D, wt, Vp, s));
            NC_RUN("gemm_nt_dn", gf(N, D, V), gb(N, D, V, es()),
                   nc::gemm<T>((int)N, (int)D, (int)Vp, z, Vp, true, wt, Vp, true, dn, D,
                               epi(nc::EPI_STORE_T), nullptr, 0, s));
        }
        NC_RUN("gemm_tn_f32", gf(V, D, N), gb(V, D, N, 4.0),
               nc::gemm<T>((int)V, (int)D, (int)N, z, Vp, false, hL, D, false, G_of(i_wlm()), D,
                           epi(nc::EPI_STORE_F32), sk, skb, s));
        // the residual gradient starts here: written, not read
        NC_RUN("norm_bwd_resid", 0, nbb - (double)N * D * es(),
               nc::norm_bwd_resid<T>(dn, hL, at<float>(p.rf), (int)N, (int)D, dres_t, false, s));

        T* dgu = at<T>(p.dgu);
        T* dout = at<T>(p.dout);
        T* dqkv = at<T>(p.dqkv);
        float* dq = at<float>(p.dq);
        float* dk = at<float>(p.dk);
        float* dv = at<float>(p.dv);
        const float* cos_t = at<float>(p.cos_t);
        const float* sin_t = at<float>(p.sin_t);
        for (int l = L - 1; l >= 0; --l) {
            T* x = X(l);
            if (p.recompute && l < L - 1) {
                // the block's saved tensors were overwritten by later blocks:
                // form them again from its input (same kernels, same bits)
                int rc = layer_fwd(l, slot_of(l), x, nullptr, false);
                if (rc != NC_OK) return rc;
            }
            const int sl = slot_of(l);
            T* xm = XM(sl);
            // MLP: x_{l+1} = xm + relu(r2 xm W_fc^T)^2 W_proj^T
            NC_RUN("gemm_nt_relu2_bwd", gf(N, F, D), gb(N, F, D, es(), N * F * es() + N * 4.0),
                   gemm_w<T>((int)N, (int)F, (int)D, dres_t, D, W(i_layer(l, 5)), F, dgu, F,
                             epi(nc::EPI_RELU2_BWD, R2(sl), G(sl)), s));
            NC_RUN("gemm_tn_f32", gf(D, F, N), gb(D, F, N, 4.0),
                   nc::gemm<T>((int)D, (int)F, (int)N, dres_t, D, false, G(sl), F, false,
                               G_of(i_layer(l, 5)), F, epi(nc::EPI_STORE_F32), sk, skb, s));
            NC_RUN("gemm_nt_dn", gf(N, D, F), gb(N, D, F, es()),
                   gemm_w<T>((int)N, (int)D, (int)F, dgu, F, W(i_layer(l, 4)), D, dn, D,
                             epi(nc::EPI_STORE_T), s));
            NC_RUN("gemm_tn_f32", gf(F, D, N), gb(F, D, N, 4.0),
                   nc::gemm<T>((int)F, (int)D, (int)N, dgu, F, false, xm, D, false,
                               G_of(i_layer(l, 4)), D, epi(nc::EPI_STORE_F32), sk, skb, s));
            NC_RUN("norm_bwd_resid", 0, nbb,
                   nc::norm_bwd_resid<T>(dn, xm, R2(sl), (int)N, (int)D, dres_t, true, s));
            // attention: xm = x + o W_o^T
            NC_RUN("gemm_nt_store", gf(N, H * hd, D), gb(N, H * hd, D, es()),
                   gemm_w<T>((int)N, (int)(H * hd), (int)D, dres_t, D, W(i_layer(l, 3)), H * hd,
                             dout, H * hd, epi(nc::EPI_STORE_T), s));
            NC_RUN("gemm_tn_f32", gf(D, H * hd, N), gb(D, H * hd, N, 4.0),
                   nc::gemm<T>((int)D, (int)(H * hd), (int)N, dres_t, D, false, O(sl), H * hd,
                               false, G_of(i_layer(l, 3)), H * hd, epi(nc::EPI_STORE_F32), sk, skb,
                               s));
            T* qkv = QKV(sl);
            if constexpr (std::is_same<T, nc::bf16_t>::value) {
                // QK-norm and rotary backward fused into the attention kernels,
                // which write the bf16 dqkv directly
                nc::AttnBwdFuse fz;
                fz.y = reinterpret_cast<const nc::bf16_t*>(qkv);
                fz.rqk = RQK(sl);
                fz.r1 = R1(sl);
                fz.cos_t = cos_t;
                fz.sin_t = sin_t;
                fz.dqkv = reinterpret_cast<nc::bf16_t*>(dqkv);
                const nc::bf16_t* qb = reinterpret_cast<const nc::bf16_t*>(qkv);
                NC_RUN("attn_bwd", 8.0 * hd * H * pairs(),
                       4.0 * N * H * hd * es() + 2.0 * N * hd * es() + N * H * 8.0 +
                           N * (H + 2) * hd * es(),
                       nc::attn_bwd_mfma(qb, qb + H * hd, qb + (H + 1) * hd, Wq, Wq,
                                         reinterpret_cast<const nc::bf16_t*>(O(sl)),
                                         reinterpret_cast<const nc::bf16_t*>(dout), LSE(sl),
                                         at<float>(p.delta), dq, dk, dv, c.batch, c.seq_len,
                                         (int)H, (int)hd, s, &fz));
            } else {
                NC_RUN("attn_bwd", 8.0 * hd * H * pairs(),
                       4.0 * N * H * hd * es() + 2.0 * N * hd * es() + N * H * 8.0 +
                           4.0 * N * (H + 2) * hd,
                       nc::attn_bwd<T>(qkv, qkv + H * hd, qkv + (H + 1) * hd, Wq, Wq, O(sl), dout,
                                       LSE(sl), at<float>(p.delta), dq, dk, dv, c.batch, c.seq_len,
                                       (int)H, (int)hd, s));
                NC_RUN("rope_qknorm_bwd", 0,
                       N * (H + 1) * hd * es() + 4.0 * N * (H + 2) * hd + N * (H + 2) * hd * es() +
                           N * (H + 2) * 4.0,
                       nc::rope_qknorm_bwd<T>(qkv, dq, dk, dv, RQK(sl), R1(sl), (int)N, c.seq_len,
                                              (int)H, (int)hd, cos_t, sin_t, dqkv, s));
            }
            NC_RUN("gemm_nt_dn", gf(N, D, Wq), gb(N, D, Wq, es()),
                   gemm_w<T>((int)N, (int)D, (int)Wq, dqkv, Wq, W(i_layer(l, 0)), D, dn, D,
                             epi(nc::EPI_STORE_T), s));
            NC_RUN("gemm_tn_f32", gf(Wq, D, N), gb(Wq, D, N, 4.0),
                   nc::gemm<T>((int)Wq, (int)D, (int)N, dqkv, Wq, false, x, D, false,
                               G_of(i_layer(l, 0)), D, epi(nc::EPI_STORE_F32), sk, skb, s));
            NC_RUN("norm_bwd_resid", 0, nbb,
                   nc::norm_bwd_resid<T>(dn, x, R1(sl), (int)N, (int)D, dres_t, true, s));
        }
        // embedding: h0 = r0 e, e = W_te[tok]
        float* de = at<float>(p.dn);
        NC_RUN("embed_bwd_rows", 0, N * D * (es() + es() + 4.0),
               nc::embed_bwd_rows<T>(dres_t, W(i_wte()), tok, at<float>(p.r0), (int)N, (int)D, de,
                                     s));
        NC_RUN("embed_grad", 0, N * D * 4.0 + (double)V * D * 4.0,
               nc::embed_grad(de, tok, (int)N, (int)D, (int)V, G_of(i_wte()), ws + p.embed,
                              p.embed_bytes, s));
        return NC_OK;
    }
};

template <typename T>
int run_step(const nc_config& c, const void* params, const int32_t* tok, const int32_t* tgt,
             float* loss, float* tok_loss, float* grads, void* ws, size_t ws_bytes,
             hipStream_t s, Prof* prof = nullptr, bool recompute = false) {
    const bool bwd = grads != nullptr;
    Plan p = make_plan(c, bwd, recompute);
    if (ws_bytes < p.bytes) return NC_ERR_WORKSPACE;
    Step<T> st(c, p, ws, s, params, prof);
    int rc = st.forward(tok, tgt, loss, tok_loss, bwd);
    if (rc != NC_OK || !bwd) return rc;
    return st.backward(tok, grads);
}

int check_common(const nc_config* cfg, const void* params, const int32_t* tok,
                 const int32_t* tgt, const float* loss, const float* tok_loss, const void* ws) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!params || !tok || !tgt || !loss || !ws) return NC_ERR_NULL;
    if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(tok, 16) || !aligned(tgt, 16) ||
        !aligned(loss, 4) || (tok_loss && !aligned(tok_loss, 16)))
        return NC_ERR_ALIGN;
    return NC_OK;
}

// ------------------------------------------------------------------ generation
// Decode workspace of nc_decode_step_noalloc, for callers that cannot
// allocate device memory: one array per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): each device's address is looked up once,
// with that device current, and kept.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kDecodeScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return NC_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return NC_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_hip_error = (int)e;
            return NC_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NC_OK;
}

// Decode workspace for B tokens and a cache of max_seq positions.
struct DecPlan {
    size_t x0, x1, xm, r, qkv, q, o, g, part_o, part_ml, cos_t, sin_t, gpart, bytes = 0;
    size_t gpart_elems = 0;
};

DecPlan make_dec_plan(const nc_config& c, int max_seq) {
    DecPlan d;
    const int64_t B = c.batch, D = c.d_model, H = c.n_head, hd = c.head_dim, F = c.d_mlp;
    const size_t es = c.dtype == NC_BF16 ? 2 : 4;
    const int64_t nch = nc::decode_chunks(max_seq);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t r = off; off += align256(bytes); return r; };
    d.x0 = take(B * D * es);
    d.x1 = take(B * D * es);
    d.xm = take(B * D * es);
    d.r = take(B * 4);
    d.qkv = take(B * (H + 2) * hd * es);
    d.q = take(B * H * hd * 4);
    d.o = take(B * H * hd * es);
    d.g = take(B * F * es);
    d.part_o = take(B * nch * H * hd * 4);
    d.part_ml = take(B * nch * H * 2 * 4);
    d.cos_t = take((size_t)max_seq * (hd / 2) * 4);
    d.sin_t = take((size_t)max_seq * (hd / 2) * 4);
    // k-slice sums of the B-row products (bf16 path)
    if (c.dtype == NC_BF16) {
        const int64_t Wq = (H + 2) * hd;
        const int64_t shapes[4][2] = {{Wq, D}, {D, H * hd}, {F, D}, {D, F}};
        for (const auto& nk : shapes)
            d.gpart_elems = std::max<size_t>(
                d.gpart_elems, (size_t)nc::gemv_splits((int)nk[0], (int)nk[1]) * B * nk[0]);
    }
    d.gpart = take(d.gpart_elems * 4);
    d.bytes = off;
    return d;
}

// config the training kernels see for a prefill of t0 positions
nc_config prefill_cfg(const nc_config& c, int t0) {
    nc_config p = c;
    p.seq_len = t0;
    return p;
}

size_t prefill_bytes(const nc_config& c, int t0) {
    const nc_config pc = prefill_cfg(c, t0);
    const size_t es = c.dtype == NC_BF16 ? 2 : 4;
    return make_plan(pc, false, false, true).bytes + align256((size_t)c.batch * c.d_model * es) +
           align256((size_t)c.batch * 4);
}

int check_infer(const nc_config* cfg, int max_seq) {
    if (!cfg) return NC_ERR_NULL;
    nc_config probe = *cfg;
    probe.seq_len = 64;   // the step's own length check does not apply here
    int rc = validate(&probe);
    if (rc != NC_OK) return rc;
    if (max_seq < 1) return NC_ERR_CONFIG;
    if (cfg->n_head > 16) return NC_ERR_UNSUPPORTED;   // decode attention keeps 16 heads
    return NC_OK;
}

// decode-step product y = epi(x W^T) of B rows: the weight-streaming matrix-
// core kernel for bf16, the SIMT product for fp32 (logits: EPI_STORE_F32)
template <typename T>
hipError_t dec_gemm(int mode, const T* x, int64_t ldx, int B, const T* W, int N, int K,
                    const float* rs, const T* aux, void* y, int64_t ldy, hipStream_t s,
                    float* part = nullptr, size_t part_elems = 0) {
    if constexpr (std::is_same<T, nc::bf16_t>::value) {
        return nc::gemv(mode, x, ldx, B, W, N, K, rs, aux, y, ldy, part, part_elems, s);
    } else {
        nc::Epilogue e;
        e.mode = mode == nc::EPI_STORE_F32 ? nc::EPI_ROWSCALE : mode;
        e.rowscale = rs;
        e.aux = aux;
        return nc::gemm<float>(B, N, K, x, ldx, true, W, K, true, y, ldy, e, nullptr, 0, s);
    }
}

template <typename T>
int decode_step(const nc_config& c, const T* params, const int32_t* tok, int pos, int max_seq,
                T* cache, float* logits, char* ws, hipStream_t s) {
    const DecPlan d = make_dec_plan(c, max_seq);
    std::vector<TensorDesc> lay = layout(c, nullptr);
    const int B = c.batch, D = c.d_model, H = c.n_head, hd = c.head_dim, F = c.d_mlp,
              V = c.vocab, L = c.n_layer;
    const int Wq = (H + 2) * hd;
    const float eps = c.rms_eps;
    auto P = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
    float* r = reinterpret_cast<float*>(ws + d.r);
    float* q = reinterpret_cast<float*>(ws + d.q);
    float* cos_t = reinterpret_cast<float*>(ws + d.cos_t);
    float* sin_t = reinterpret_cast<float*>(ws + d.sin_t);
    const T* Wt = params;
    auto Wl = [&](int l, int k) { return Wt + lay[1 + 6 * l + k].offset; };
    const int64_t per = (int64_t)B * max_seq * hd;
    float* gp = reinterpret_cast<float*>(ws + d.gpart);
    const size_t gpe = d.gpart_elems;
    T* x = P(d.x0);
    T* xn = P(d.x1);
    T* xm = P(d.xm);
    // bf16: the QKV product's reduce also applies rotary at pos and QK-norm and
    // fills the cache row, and the two residual products' reduces also emit
    // the next row scale, so a layer is 10 launches
    bool fused = false;
    if constexpr (std::is_same<T, nc::bf16_t>::value)
        fused = nc::gemv_fused_ok(Wq, D, B, gpe) && nc::gemv_fused_ok(D, H * hd, B, gpe) &&
                nc::gemv_fused_ok(D, F, B, gpe) && 1024 % (hd / 2) == 0;
    if (fused) {
        if constexpr (std::is_same<T, nc::bf16_t>::value) {
            NC_TRY(nc::embed_fwd<T>(Wt + lay[0].offset, tok, B, D, eps, x, r, s));
            NC_TRY(nc::rms_stats<T>(x, B, D, eps, r, s));
            for (int l = 0; l < L; ++l) {
                T* kc = cache + 2 * l * per;
                T* vc = cache + (2 * l + 1) * per;
                NC_TRY(nc::gemv_qkv_rope(x, D, B, Wl(l, 0), H, hd, D, r, pos,
                                         (double)c.rope_base, eps, q, kc, vc, max_seq, gp, s));
                NC_TRY(nc::decode_attn<T>(q, kc, vc, max_seq, pos + 1, B, H, hd,
                                          reinterpret_cast<float*>(ws + d.part_o),
                                          reinterpret_cast<float*>(ws + d.part_ml), P(d.o), s));
                NC_TRY(nc::gemv_resid_rms(P(d.o), H * hd, B, Wl(l, 3), D, H * hd, x, xm, eps, r,
                                          gp, s));
                NC_TRY(dec_gemm<T>(nc::EPI_ROWSCALE_RELU2, xm, D, B, Wl(l, 4), F, D, r, nullptr,
                                   P(d.g), F, s, gp, gpe));
                NC_TRY(nc::gemv_resid_rms(P(d.g), F, B, Wl(l, 5), D, F, xm, xn, eps, r, gp, s));
                std::swap(x, xn);
            }
            // r is the final norm's scale of x
            NC_TRY(dec_gemm<T>(nc::EPI_STORE_F32, x, D, B, Wt + lay[1 + 6 * L].offset, V, D, r,
                               nullptr, logits, V, s));
            NC_TRY(nc::softcap_rows(logits, (int64_t)B * V, c.softcap, s));
            return NC_OK;
        }
    }
    NC_TRY(nc::rope_tables(pos + 1, hd, c.rope_base, cos_t, sin_t, s));
    NC_TRY(nc::embed_fwd<T>(Wt + lay[0].offset, tok, B, D, eps, x, r, s));
    for (int l = 0; l < L; ++l) {
        T* kc = cache + 2 * l * per;
        T* vc = cache + (2 * l + 1) * per;
        NC_TRY(nc::rms_stats<T>(x, B, D, eps, r, s));
        NC_TRY(dec_gemm<T>(nc::EPI_ROWSCALE, x, D, B, Wl(l, 0), Wq, D, r, nullptr, P(d.qkv), Wq,
                           s, gp, gpe));
        NC_TRY(nc::decode_rope<T>(P(d.qkv), Wq, B, H, hd, pos, cos_t, sin_t, eps, q, kc, vc,
                                  max_seq, s));
        NC_TRY(nc::decode_attn<T>(q, kc, vc, max_seq, pos + 1, B, H, hd,
                                  reinterpret_cast<float*>(ws + d.part_o),
                                  reinterpret_cast<float*>(ws + d.part_ml), P(d.o), s));
        NC_TRY(dec_gemm<T>(nc::EPI_RESID, P(d.o), H * hd, B, Wl(l, 3), D, H * hd, nullptr, x, xm,
                           D, s, gp, gpe));
        NC_TRY(nc::rms_stats<T>(xm, B, D, eps, r, s));
        NC_TRY(dec_gemm<T>(nc::EPI_ROWSCALE_RELU2, xm, D, B, Wl(l, 4), F, D, r, nullptr, P(d.g),
                           F, s, gp, gpe));
        NC_TRY(dec_gemm<T>(nc::EPI_RESID, P(d.g), F, B, Wl(l, 5), D, F, nullptr, xm, xn, D, s, gp,
                           gpe));
        std::swap(x, xn);
    }
    NC_TRY(nc::rms_stats<T>(x, B, D, eps, r, s));
    NC_TRY(dec_gemm<T>(nc::EPI_STORE_F32, x, D, B, Wt + lay[1 + 6 * L].offset, V, D, r, nullptr,
                       logits, V, s));
    NC_TRY(nc::softcap_rows(logits, (int64_t)B * V, c.softcap, s));
    return NC_OK;
}

template <typename T>
int prefill(const nc_config& c, const T* params, const int32_t* tok, int t0, int max_seq,
            T* cache, float* logits, char* ws, hipStream_t s) {
    const nc_config pc = prefill_cfg(c, t0);
    const Plan p = make_plan(pc, false, false, true);
    Step<T> st(pc, p, ws, s, params, nullptr);
    T* hL = st.prefill_blocks(tok, cache, max_seq);
    if (!hL) return NC_ERR_HIP;
    const size_t es = sizeof(T);
    T* last = reinterpret_cast<T*>(ws + p.bytes);
    float* rf = reinterpret_cast<float*>(ws + p.bytes + align256((size_t)c.batch * c.d_model * es));
    const int B = c.batch, D = c.d_model;
    NC_TRY(nc::gather_last<T>(hL, D, t0, B, last, s));
    NC_TRY(nc::rms_stats<T>(last, B, D, c.rms_eps, rf, s));
    std::vector<TensorDesc> lay = layout(c, nullptr);
    if (B > 32 && std::is_same<T, nc::bf16_t>::value) {
        // the weight-streaming product takes 32 rows at a time
        for (int b0 = 0; b0 < B; b0 += 32) {
            const int nb = std::min(32, B - b0);
            NC_TRY(dec_gemm<T>(nc::EPI_STORE_F32, last + (int64_t)b0 * D, D, nb,
                               params + lay.back().offset, c.vocab, D, rf + b0, nullptr,
                               logits + (int64_t)b0 * c.vocab, c.vocab, s));
        }
    } else {
        NC_TRY(dec_gemm<T>(nc::EPI_STORE_F32, last, D, B, params + lay.back().offset, c.vocab, D,
                           rf, nullptr, logits, c.vocab, s));
    }
    NC_TRY(nc::softcap_rows(logits, (int64_t)B * c.vocab, c.softcap, s));
    return NC_OK;
}

}  // namespace

namespace nc {
void note_hip_error(int err) { g_last_hip_error = err; }

hipError_t prof_label(const char* label, double flops, double bytes) {
    if (g_prof && g_prof->open.a) {
        g_prof->open.label = label;
        g_prof->open.flops = flops;
        g_prof->open.bytes = bytes;
    }
    return hipSuccess;
}

hipError_t prof_cut(const char* label, double flops, double bytes) {
    if (g_prof && g_prof->open.a) return g_prof->cut(label, flops, bytes);
    return hipSuccess;
}
}  // namespace nc

extern "C" {

int nc_param_count(const nc_config* cfg, int64_t* n_elems) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!n_elems) return NC_ERR_NULL;
    layout(*cfg, n_elems);
    return NC_OK;
}

int nc_param_layout(const nc_config* cfg, nc_tensor_info* out, int32_t cap, int32_t* n_out) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!n_out) return NC_ERR_NULL;
    std::vector<TensorDesc> lay = layout(*cfg, nullptr);
    *n_out = (int32_t)lay.size();
    if (cap < (int32_t)lay.size()) return NC_ERR_CAPACITY;
    if (!out) return NC_ERR_NULL;
    for (size_t i = 0; i < lay.size(); ++i) {
        std::memset(out[i].name, 0, sizeof(out[i].name));
        std::strncpy(out[i].name, lay[i].name.c_str(), sizeof(out[i].name) - 1);
        out[i].offset = lay[i].offset;
        out[i].rows = lay[i].rows;
        out[i].cols = lay[i].cols;
    }
    return NC_OK;
}

int nc_workspace_size(const nc_config* cfg, int32_t with_backward, size_t* bytes) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!bytes) return NC_ERR_NULL;
    *bytes = make_plan(*cfg, with_backward != 0).bytes;
    return NC_OK;
}

int nc_init_params(const nc_config* cfg, uint64_t seed, void* params, void* stream) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!params) return NC_ERR_NULL;
    if (!aligned(params, 256)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    int64_t total = 0;
    std::vector<TensorDesc> lay = layout(*cfg, &total);
    const bool bf = cfg->dtype == NC_BF16;
    if (bf)
        NC_TRY(nc::zero_elems<nc::bf16_t>(static_cast<nc::bf16_t*>(params), total, s));
    else
        NC_TRY(nc::zero_elems<float>(static_cast<float*>(params), total, s));
    for (size_t i = 0; i < lay.size(); ++i) {
        const float stdv = (lay[i].name == "wlm") ? 0.001f : 0.02f;
        const int64_t n = (int64_t)lay[i].rows * lay[i].cols;
        if (bf)
            NC_TRY(nc::init_normal<nc::bf16_t>(static_cast<nc::bf16_t*>(params) + lay[i].offset, n,
                                               stdv, seed, (uint64_t)i, s));
        else
            NC_TRY(nc::init_normal<float>(static_cast<float*>(params) + lay[i].offset, n, stdv,
                                          seed, (uint64_t)i, s));
    }
    return NC_OK;
}

int nc_forward_loss(const nc_config* cfg, const void* params, const int32_t* tokens,
                    const int32_t* targets, float* loss, void* ws, size_t ws_bytes,
                    void* stream) {
    return nc_forward_token_loss(cfg, params, tokens, targets, loss, nullptr, ws, ws_bytes,
                                 stream);
}

int nc_forward_token_loss(const nc_config* cfg, const void* params, const int32_t* tokens,
                          const int32_t* targets, float* loss, float* token_loss, void* ws,
                          size_t ws_bytes, void* stream) {
    int rc = check_common(cfg, params, tokens, targets, loss, token_loss, ws);
    if (rc != NC_OK) return rc;
    hipStream_t s = nc::enqueue_stream(stream);
    if (cfg->dtype == NC_BF16)
        return run_step<nc::bf16_t>(*cfg, params, tokens, targets, loss, token_loss, nullptr, ws,
                                    ws_bytes, s);
    return run_step<float>(*cfg, params, tokens, targets, loss, token_loss, nullptr, ws, ws_bytes,
                           s);
}

int nc_forward_backward(const nc_config* cfg, const void* params, const int32_t* tokens,
                        const int32_t* targets, float* loss, float* grads, void* ws,
                        size_t ws_bytes, void* stream) {
    int rc = check_common(cfg, params, tokens, targets, loss, nullptr, ws);
    if (rc != NC_OK) return rc;
    if (!grads) return NC_ERR_NULL;
    if (!aligned(grads, 256)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    if (cfg->dtype == NC_BF16)
        return run_step<nc::bf16_t>(*cfg, params, tokens, targets, loss, nullptr, grads, ws,
                                    ws_bytes, s);
    return run_step<float>(*cfg, params, tokens, targets, loss, nullptr, grads, ws, ws_bytes, s);
}

int nc_workspace_size_recompute(const nc_config* cfg, size_t* bytes) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!bytes) return NC_ERR_NULL;
    *bytes = make_plan(*cfg, true, true).bytes;
    return NC_OK;
}

int nc_forward_backward_recompute(const nc_config* cfg, const void* params,
                                  const int32_t* tokens, const int32_t* targets, float* loss,
                                  float* grads, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_common(cfg, params, tokens, targets, loss, nullptr, ws);
    if (rc != NC_OK) return rc;
    if (!grads) return NC_ERR_NULL;
    if (!aligned(grads, 256)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    if (cfg->dtype == NC_BF16)
        return run_step<nc::bf16_t>(*cfg, params, tokens, targets, loss, nullptr, grads, ws,
                                    ws_bytes, s, nullptr, true);
    return run_step<float>(*cfg, params, tokens, targets, loss, nullptr, grads, ws, ws_bytes, s,
                           nullptr, true);
}

int nc_forward_backward_timed(const nc_config* cfg, const void* params, const int32_t* tokens,
                              const int32_t* targets, float* loss, float* grads, void* ws,
                              size_t ws_bytes, void* stream, nc_kernel_stat* stats, int32_t cap,
                              int32_t* n_out) {
    int rc = check_common(cfg, params, tokens, targets, loss, nullptr, ws);
    if (rc != NC_OK) return rc;
    if (!grads || !n_out || (cap > 0 && !stats)) return NC_ERR_NULL;
    if (!aligned(grads, 256)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    Prof prof;
    prof.s = s;
    g_prof = &prof;
    if (cfg->dtype == NC_BF16)
        rc = run_step<nc::bf16_t>(*cfg, params, tokens, targets, loss, nullptr, grads, ws,
                                  ws_bytes, s, &prof);
    else
        rc = run_step<float>(*cfg, params, tokens, targets, loss, nullptr, grads, ws, ws_bytes, s,
                             &prof);
    g_prof = nullptr;
    if (rc != NC_OK) return rc;
    NC_TRY(hipStreamSynchronize(s));
    std::vector<nc_kernel_stat> agg;
    for (auto& r : prof.recs) {
        float ms = 0.f;
        NC_TRY(hipEventElapsedTime(&ms, r.a, r.b));
        size_t k = 0;
        while (k < agg.size() && std::strcmp(agg[k].name, r.label) != 0) ++k;
        if (k == agg.size()) {
            nc_kernel_stat z;
            std::memset(&z, 0, sizeof(z));
            std::strncpy(z.name, r.label, sizeof(z.name) - 1);
            agg.push_back(z);
        }
        agg[k].launches += 1;
        agg[k].total_ms += ms;
        agg[k].flops += r.flops;
        agg[k].bytes += r.bytes;
    }
    *n_out = (int32_t)agg.size();
    for (size_t k = 0; k < agg.size() && (int32_t)k < cap; ++k) stats[k] = agg[k];
    return cap < (int32_t)agg.size() ? NC_ERR_CAPACITY : NC_OK;
}

int nc_validate_tokens(const nc_config* cfg, const int32_t* tokens, const int32_t* targets,
                       int32_t* n_bad, void* stream) {
    int rc = validate(cfg);
    if (rc != NC_OK) return rc;
    if (!tokens || !targets || !n_bad) return NC_ERR_NULL;
    if (!aligned(tokens, 4) || !aligned(targets, 4) || !aligned(n_bad, 4)) return NC_ERR_ALIGN;
    hipStream_t s = nc::enqueue_stream(stream);
    NC_TRY(nc::zero_elems<int32_t>(n_bad, 1, s));
    NC_TRY(nc::count_bad_ids(tokens, targets, (int64_t)cfg->batch * cfg->seq_len, cfg->vocab,
                             n_bad, s));
    return NC_OK;
}

int nc_kv_cache_size(const nc_config* cfg, int32_t max_seq, size_t* bytes) {
    int rc = check_infer(cfg, max_seq);
    if (rc != NC_OK) return rc;
    if (!bytes) return NC_ERR_NULL;
    const size_t es = cfg->dtype == NC_BF16 ? 2 : 4;
    *bytes = align256((size_t)2 * cfg->n_layer * cfg->batch * max_seq * cfg->head_dim * es);
    return NC_OK;
}

int nc_infer_workspace_size(const nc_config* cfg, int32_t max_seq, int32_t t0, size_t* bytes) {
    int rc = check_infer(cfg, max_seq);
    if (rc != NC_OK) return rc;
    if (!bytes) return NC_ERR_NULL;
    if (t0 < 0 || t0 > max_seq || t0 % 64) return NC_ERR_CONFIG;
    size_t b = make_dec_plan(*cfg, max_seq).bytes;
    if (t0 > 0) b = std::max(b, prefill_bytes(*cfg, t0));
    *bytes = b;
    return NC_OK;
}

int nc_prefill(const nc_config* cfg, const void* params, const int32_t* tokens, int32_t t0,
               int32_t max_seq, void* cache, float* logits, void* ws, size_t ws_bytes,
               void* stream) {
    int rc = check_infer(cfg, max_seq);
    if (rc != NC_OK) return rc;
    if (t0 < 64 || t0 > max_seq || t0 % 64) return NC_ERR_CONFIG;
    const nc_config pc = prefill_cfg(*cfg, t0);
    rc = validate(&pc);
    if (rc != NC_OK) return rc;
    if (!params || !tokens || !cache || !logits || !ws) return NC_ERR_NULL;
    if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(cache, 256) ||
        !aligned(tokens, 16) || !aligned(logits, 16))
        return NC_ERR_ALIGN;
    if (ws_bytes < prefill_bytes(*cfg, t0)) return NC_ERR_WORKSPACE;
    hipStream_t s = nc::enqueue_stream(stream);
    char* w = static_cast<char*>(ws);
    if (cfg->dtype == NC_BF16)
        return prefill<nc::bf16_t>(*cfg, static_cast<const nc::bf16_t*>(params), tokens, t0,
                                   max_seq, static_cast<nc::bf16_t*>(cache), logits, w, s);
    return prefill<float>(*cfg, static_cast<const float*>(params), tokens, t0, max_seq,
                          static_cast<float*>(cache), logits, w, s);
}

int nc_decode_step(const nc_config* cfg, const void* params, const int32_t* tokens, int32_t pos,
                   int32_t max_seq, void* cache, float* logits, void* ws, size_t ws_bytes,
                   void* stream) {
    int rc = check_infer(cfg, max_seq);
    if (rc != NC_OK) return rc;
    if (pos < 0 || pos >= max_seq) return NC_ERR_CONFIG;
    if (cfg->batch > 32) return NC_ERR_UNSUPPORTED;
    if (!params || !tokens || !cache || !logits || !ws) return NC_ERR_NULL;
    if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(cache, 256) ||
        !aligned(tokens, 4) || !aligned(logits, 16))
        return NC_ERR_ALIGN;
    if (ws_bytes < make_dec_plan(*cfg, max_seq).bytes) return NC_ERR_WORKSPACE;
    hipStream_t s = nc::enqueue_stream(stream);
    char* w = static_cast<char*>(ws);
    if (cfg->dtype == NC_BF16)
        return decode_step<nc::bf16_t>(*cfg, static_cast<const nc::bf16_t*>(params), tokens, pos,
                                       max_seq, static_cast<nc::bf16_t*>(cache), logits, w, s);
    return decode_step<float>(*cfg, static_cast<const float*>(params), tokens, pos, max_seq,
                              static_cast<float*>(cache), logits, w, s);
}

int nc_decode_step_noalloc(const nc_config* cfg, const void* params, const int32_t* tokens,
                           int32_t pos, int32_t max_seq, void* cache, float* logits,
                           void* stream) {
    int rc = check_infer(cfg, max_seq);
    if (rc != NC_OK) return rc;
    if (pos < 0 || pos >= max_seq) return NC_ERR_CONFIG;
    if (cfg->batch > 32) return NC_ERR_UNSUPPORTED;
    if (!params || !tokens || !cache || !logits) return NC_ERR_NULL;
    if (!aligned(params, 256) || !aligned(cache, 256) || !aligned(tokens, 4) ||
        !aligned(logits, 16))
        return NC_ERR_ALIGN;
    if (make_dec_plan(*cfg, max_seq).bytes > kDecodeScratchBytes) return NC_ERR_WORKSPACE;
    void* ws = nullptr;
    rc = scratch_for_current_device(&ws);
    if (rc != NC_OK) return rc;
    hipStream_t s = nc::enqueue_stream(stream);
    char* w = static_cast<char*>(ws);
    if (cfg->dtype == NC_BF16)
        return decode_step<nc::bf16_t>(*cfg, static_cast<const nc::bf16_t*>(params), tokens, pos,
                                       max_seq, static_cast<nc::bf16_t*>(cache), logits, w, s);
    return decode_step<float>(*cfg, static_cast<const float*>(params), tokens, pos, max_seq,
                              static_cast<float*>(cache), logits, w, s);
}

const char* nc_status_string(int status) {
    switch (status) {
        case NC_OK: return "ok";
        case NC_ERR_NULL: return "a required pointer is NULL";
        case NC_ERR_CONFIG: return "a config field is out of range";
        case NC_ERR_DTYPE: return "unknown dtype";
        case NC_ERR_WORKSPACE: return "workspace smaller than nc_workspace_size";
        case NC_ERR_ALIGN: return "a device pointer is not aligned";
        case NC_ERR_HIP: return "a HIP call or kernel launch failed";
        case NC_ERR_UNSUPPORTED: return "valid model, but a shape the library does not run";
        case NC_ERR_CAPACITY: return "output array too small";
        default: return "unknown status";
    }
}

int nc_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
