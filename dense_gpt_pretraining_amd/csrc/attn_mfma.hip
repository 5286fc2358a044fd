// Causal multi-query flash attention on CDNA4 matrix cores (bf16 in, fp32
// accumulate), forward and backward.
//
// Multi-query attention (architecture list of the nanochat article): all H
// query heads of a token share one key head and one value head.  The H query
// vectors of a sequence are read as one [T*H, hd] matrix whose row r is
// (position t = r / H, head j = r % H); row r may attend to keys tau <= t.
// A workgroup therefore takes 128 consecutive rows -- every head of ~128/H
// positions -- and streams the single K/V head through LDS once for all of
// them, instead of once per head.  The causal bound of a workgroup is set by
// its last position, so the diagonal waste is one key tile, not a triangle.
//
// Layout trick: scores are computed transposed, S^T = K Q^T, so that the
// 32x32 accumulator of a wave holds one query row per lane (lane & 31) and 16
// keys per lane in registers.  The online softmax is then lane-local (plus one
// exchange with lane ^ 32), and the probabilities are already where the next
// product O^T = V^T P^T wants its B operand: the 16 keys of one k-step of that
// product are exactly 8 registers of each of the lanes l and l ^ 32.  Only
// the A operand (V^T) is read transposed, and that tile is transposed once in
// registers on its way into LDS.  The backward pass uses the same two layouts.
//
// Forward: one pass over key tiles with the running max/sum (online softmax),
// output O and the log-sum-exp per row.
// Backward: dQ by a row-block kernel that recomputes P from the saved
// log-sum-exp; dK, dV by a key-block kernel that streams all query rows that
// can see its keys.  Both keep every sum in a fixed order (no atomics).
#include "kernels.h"

namespace nc {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKT = 64;     // keys per tile (forward and dq)
constexpr int kRB = 128;    // query rows per workgroup (forward and dq)

// element offset in a tile of rows made of NCH 16-byte chunks; chunk index
// XOR (row & 7) so 8 consecutive rows reading the same chunk hit distinct banks
template <int NCH>
__device__ __forceinline__ int rt_off(int row, int ch) {
    return row * NCH * 8 + ((ch ^ (row & 7 & (NCH - 1))) << 3);
}
// element offset of element `col` of row `row` in a transposed tile with
// NCH chunks per row; chunk index XOR ((row >> 1) & (NCH - 1))
template <int NCH>
__device__ __forceinline__ int tt_off(int row, int col) {
    return row * NCH * 8 + ((((col >> 3) ^ ((row >> 1) & (NCH - 1)))) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x8_t pack8(const float* x) {
    return as_bf16x8(make_uint4(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]),
                                pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])));
}

// A operand for a k-step over 16 keys (or rows) of a transposed tile: lane
// supplies row `row`, elements c0 .. c0+3 and c0+8 .. c0+11
template <int NCH>
__device__ __forceinline__ bf16x8_t tt_frag(const bf16_t* tile, int row, int c0) {
    const uint2 lo = *reinterpret_cast<const uint2*>(tile + tt_off<NCH>(row, c0));
    const uint2 hi = *reinterpret_cast<const uint2*>(tile + tt_off<NCH>(row, c0 + 8));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// ------------------------------------------------------------------ forward
template <int HD>
__global__ __launch_bounds__(256, 2) void k_attn_fwd_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    int64_t ldq, int64_t ldkv, bf16_t* __restrict__ o, float* __restrict__ lse, int B, int T,
    int H, float scale_log2) {
    constexpr int KCH = HD / 8;               // 16-byte chunks per K row
    constexpr int TILE = kKT * HD;            // elements of one K (or V^T) tile
    constexpr int K_PER = kKT * KCH / 256;    // K chunks staged per thread
    constexpr int V_BLK = (kKT / 8) * (HD / 8);
    __shared__ __align__(16) bf16_t sm[2 * 2 * TILE];

    const int rows_total = T * H;
    const int n_rb = (rows_total + kRB - 1) / kRB;
    const int rb = n_rb - 1 - (int)(blockIdx.x / B);     // heaviest row blocks first
    const int b = (int)(blockIdx.x % B);
    const int64_t seq0 = (int64_t)b * T;
    const int r0 = rb * kRB;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
    const int r = r0 + 32 * w + li;
    const bool valid = r < rows_total;
    const int t = valid ? r / H : 0;
    const int j = valid ? r % H : 0;

    bf16x8_t qf[HD / 16];
    {
        const bf16_t* qrow = q + (seq0 + t) * ldq + (int64_t)j * HD;
#pragma unroll
        for (int kk = 0; kk < HD / 16; ++kk)
            qf[kk] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * g))
                           : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
    const int last_row = min(r0 + kRB - 1, rows_total - 1);
    const int n_tiles = (last_row / H) / kKT + 1;
    const int w_first = r0 + 32 * w;
    const int tw_max = (w_first < rows_total) ? min(w_first + 31, rows_total - 1) / H : -1;

    f32x16_t oacc[HD / 32];
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) oacc[db] = zero16();
    float m_run = -INFINITY, l_run = 0.f;

    uint4 kreg[K_PER], vreg[8];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int item = tid + 256 * i, key = item / KCH, ch = item % KCH;
            kreg[i] = *reinterpret_cast<const uint4*>(k + (seq0 + kb + key) * ldkv + ch * 8);
        }
        if (tid < V_BLK) {
            const int kb8 = tid & 7, db8 = tid >> 3;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                vreg[i] = *reinterpret_cast<const uint4*>(v + (seq0 + kb + kb8 * 8 + i) * ldkv +
                                                          db8 * 8);
        }
    };
    auto store_tile = [&](int buf) {
        bf16_t* sK = sm + buf * 2 * TILE;
        bf16_t* sV = sK + TILE;
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int item = tid + 256 * i, key = item / KCH, ch = item % KCH;
            *reinterpret_cast<uint4*>(sK + rt_off<KCH>(key, ch)) = kreg[i];
        }
        if (tid < V_BLK) {
            const int kb8 = tid & 7, db8 = tid >> 3;
            uint4 tr[8];
            transpose8x8(vreg, tr);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                *reinterpret_cast<uint4*>(sV + tt_off<8>(db8 * 8 + c, kb8 * 8)) = tr[c];
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < n_tiles; ++it) {
        const int kb = it * kKT;
        const bool more = it + 1 < n_tiles;
        if (more) load_tile(kb + kKT);
        const bf16_t* sK = sm + (it & 1) * 2 * TILE;
        const bf16_t* sV = sK + TILE;
        if (kb <= tw_max) {
            f32x16_t s[2] = {zero16(), zero16()};
#pragma unroll
            for (int kk = 0; kk < HD / 16; ++kk)
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) {
                    const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(
                        sK + rt_off<KCH>(32 * bi + li, 2 * kk + g)));
                    s[bi] = mfma32(a, qf[kk], s[bi]);
                }
            float mx = -INFINITY;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int key = kb + 32 * bi + 8 * (rr >> 2) + 4 * g + (rr & 3);
                    float x = s[bi][rr] * scale_log2;
                    if (!valid || key > t) x = -INFINITY;
                    s[bi][rr] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            float m_new = fmaxf(m_run, mx);
            if (m_new == -INFINITY) m_new = 0.f;     // padding rows see no key
            const float alpha = exp2f(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const float p = exp2f(s[bi][rr] - m_new);
                    s[bi][rr] = p;
                    ps += p;
                }
            l_run = l_run * alpha + ps;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < HD / 32; ++db) oacc[db] *= alpha;
#pragma unroll
            for (int ks = 0; ks < kKT / 16; ++ks) {
                const int bi = ks >> 1, h = ks & 1;
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = s[bi][8 * h + e];
                const bf16x8_t bfrag = pack8(pv);
#pragma unroll
                for (int db = 0; db < HD / 32; ++db) {
                    const bf16x8_t a = tt_frag<8>(sV, 32 * db + li, 32 * bi + 16 * h + 4 * g);
                    oacc[db] = mfma32(a, bfrag, oacc[db]);
                }
            }
        }
        if (more) store_tile((it + 1) & 1);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (valid) {
        const float inv = 1.f / l_tot;
        bf16_t* orow = o + (seq0 * H + r) * HD;
#pragma unroll
        for (int db = 0; db < HD / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d = 32 * db + 8 * gq + 4 * g;
                *reinterpret_cast<uint2*>(orow + d) =
                    make_uint2(pack_bf2(oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv),
                               pack_bf2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv));
            }
        if (g == 0) lse[seq0 * H + r] = (m_run + log2f(l_tot)) * kLn2;
    }
}

// ------------------------------------------------------------------ backward: dq
template <int HD>
__global__ __launch_bounds__(256, 1) void k_attn_bwd_dq_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    int64_t ldq, int64_t ldkv, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, int B, int T, int H,
    float scale_log2, float scale) {
    constexpr int KCH = HD / 8;
    constexpr int TILE = kKT * HD;
    constexpr int K_BLK = (kKT / 8) * (HD / 8);      // 8x8 blocks of K (natural + transposed)
    constexpr int V_PER = kKT * KCH / 256;
    extern __shared__ __align__(16) unsigned char dq_lds[];
    bf16_t* sm = reinterpret_cast<bf16_t*>(dq_lds);  // [buf][K | V | K^T]

    const int rows_total = T * H;
    const int n_rb = (rows_total + kRB - 1) / kRB;
    const int rb = n_rb - 1 - (int)(blockIdx.x / B);
    const int b = (int)(blockIdx.x % B);
    const int64_t seq0 = (int64_t)b * T;
    const int r0 = rb * kRB;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
    const int r = r0 + 32 * w + li;
    const bool valid = r < rows_total;
    const int t = valid ? r / H : 0;
    const int j = valid ? r % H : 0;

    bf16x8_t qf[HD / 16], df[HD / 16];
    {
        const bf16_t* qrow = q + (seq0 + t) * ldq + (int64_t)j * HD;
        const bf16_t* drow = dout + (seq0 * H + (valid ? r : 0)) * HD;
#pragma unroll
        for (int kk = 0; kk < HD / 16; ++kk) {
            qf[kk] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * g))
                           : as_bf16x8(make_uint4(0, 0, 0, 0));
            df[kk] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(drow + 16 * kk + 8 * g))
                           : as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }
    const float lse2 = valid ? lse[seq0 * H + r] * kLog2e : 0.f;
    const float dl = valid ? delta[seq0 * H + r] : 0.f;
    const int last_row = min(r0 + kRB - 1, rows_total - 1);
    const int n_tiles = (last_row / H) / kKT + 1;
    const int w_first = r0 + 32 * w;
    const int tw_max = (w_first < rows_total) ? min(w_first + 31, rows_total - 1) / H : -1;

    f32x16_t acc[HD / 32];
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) acc[db] = zero16();

    uint4 kreg[8], vreg[V_PER];
    auto load_tile = [&](int kb) {
        if (tid < K_BLK) {
            const int kb8 = tid & 7, db8 = tid >> 3;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kreg[i] = *reinterpret_cast<const uint4*>(k + (seq0 + kb + kb8 * 8 + i) * ldkv +
                                                          db8 * 8);
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int item = tid + 256 * i, key = item / KCH, ch = item % KCH;
            vreg[i] = *reinterpret_cast<const uint4*>(v + (seq0 + kb + key) * ldkv + ch * 8);
        }
    };
    auto store_tile = [&](int buf) {
        bf16_t* sK = sm + buf * 3 * TILE;
        bf16_t* sV = sK + TILE;
        bf16_t* sKt = sV + TILE;
        if (tid < K_BLK) {
            const int kb8 = tid & 7, db8 = tid >> 3;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint4*>(sK + rt_off<KCH>(kb8 * 8 + i, db8)) = kreg[i];
            uint4 tr[8];
            transpose8x8(kreg, tr);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                *reinterpret_cast<uint4*>(sKt + tt_off<8>(db8 * 8 + c, kb8 * 8)) = tr[c];
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int item = tid + 256 * i, key = item / KCH, ch = item % KCH;
            *reinterpret_cast<uint4*>(sV + rt_off<KCH>(key, ch)) = vreg[i];
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < n_tiles; ++it) {
        const int kb = it * kKT;
        const bool more = it + 1 < n_tiles;
        if (more) load_tile(kb + kKT);
        const bf16_t* sK = sm + (it & 1) * 3 * TILE;
        const bf16_t* sV = sK + TILE;
        const bf16_t* sKt = sV + TILE;
        if (kb <= tw_max) {
            f32x16_t s[2] = {zero16(), zero16()}, dp[2] = {zero16(), zero16()};
#pragma unroll
            for (int kk = 0; kk < HD / 16; ++kk)
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) {
                    const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(
                        sK + rt_off<KCH>(32 * bi + li, 2 * kk + g)));
                    s[bi] = mfma32(a, qf[kk], s[bi]);
                    const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(
                        sV + rt_off<KCH>(32 * bi + li, 2 * kk + g)));
                    dp[bi] = mfma32(av, df[kk], dp[bi]);
                }
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int key = kb + 32 * bi + 8 * (rr >> 2) + 4 * g + (rr & 3);
                    const float p = (valid && key <= t) ? exp2f(s[bi][rr] * scale_log2 - lse2) : 0.f;
                    s[bi][rr] = p * (dp[bi][rr] - dl);
                }
#pragma unroll
            for (int ks = 0; ks < kKT / 16; ++ks) {
                const int bi = ks >> 1, h = ks & 1;
                float dv8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) dv8[e] = s[bi][8 * h + e];
                const bf16x8_t bfrag = pack8(dv8);
#pragma unroll
                for (int db = 0; db < HD / 32; ++db) {
                    const bf16x8_t a = tt_frag<8>(sKt, 32 * db + li, 32 * bi + 16 * h + 4 * g);
                    acc[db] = mfma32(a, bfrag, acc[db]);
                }
            }
        }
        if (more) store_tile((it + 1) & 1);
        __syncthreads();
    }
    if (valid) {
        float* out = dq + (seq0 * H + r) * HD;
#pragma unroll
        for (int db = 0; db < HD / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d = 32 * db + 8 * gq + 4 * g;
                *reinterpret_cast<float4*>(out + d) =
                    make_float4(acc[db][4 * gq] * scale, acc[db][4 * gq + 1] * scale,
                                acc[db][4 * gq + 2] * scale, acc[db][4 * gq + 3] * scale);
            }
    }
}

// ------------------------------------------------------------------ backward: dk, dv
constexpr int kKB = 128;   // keys per workgroup (4 waves x 32)
constexpr int kQT = 32;    // query rows per tile

// The query rows a key block can see are cut into chunks of `chunk_rows`
// (a multiple of kQT); chunk c of key block kb of sequence b is one workgroup,
// which writes its dK, dV sums to partial slot (b, first_slot(kb) + c).  The
// number of chunks of key block kb is chunks_of(kb).
__host__ __device__ __forceinline__ int kv_rows_begin(int kb, int H) {
    return (kb * kKB * H) / kQT * kQT;
}
__host__ __device__ __forceinline__ int kv_chunks(int kb, int H, int rows_total, int chunk_rows) {
    return (rows_total - kv_rows_begin(kb, H) + chunk_rows - 1) / chunk_rows;
}

template <int HD>
__global__ __launch_bounds__(256, 1) void k_attn_bwd_dkv_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    int64_t ldq, int64_t ldkv, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dk_part, float* __restrict__ dv_part,
    int B, int T, int H, float scale_log2, float scale, int chunk_rows, int slots_per_seq) {
    constexpr int KCH = HD / 8;
    constexpr int QTILE = kQT * HD;                  // elements of one row tile
    constexpr int BLK = (kQT / 8) * (HD / 8);        // 8x8 blocks of one row tile
    // per buffer: Q, dO (row tiles), Q^T, dO^T (transposed, kQT columns), lse, delta
    constexpr int BUF = 4 * QTILE + 2 * kQT * 2;     // in bf16 elements (floats take 2)
    __shared__ __align__(16) bf16_t sm[2 * BUF];

    const int rows_total = T * H;
    const int n_kb = (T + kKB - 1) / kKB;
    const int b = (int)(blockIdx.x % B);
    int rest = (int)(blockIdx.x / B), kbi = 0, slot = 0;
    for (; kbi < n_kb; ++kbi) {
        const int nc = kv_chunks(kbi, H, rows_total, chunk_rows);
        if (rest < nc) break;
        rest -= nc;
        slot += nc;
    }
    slot += rest;
    const int r_begin = kv_rows_begin(kbi, H) + rest * chunk_rows;
    const int r_end = min(r_begin + chunk_rows, rows_total);
    const int64_t seq0 = (int64_t)b * T;
    const int key0 = kbi * kKB;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
    const int wkey0 = key0 + 32 * w;
    const bool wvalid = wkey0 < T;
    const int key = wkey0 + li;

    bf16x8_t kf[HD / 16], vf[HD / 16];
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
        kf[kk] = wvalid ? as_bf16x8(*reinterpret_cast<const uint4*>(
                              k + (seq0 + key) * ldkv + 16 * kk + 8 * g))
                        : as_bf16x8(make_uint4(0, 0, 0, 0));
        vf[kk] = wvalid ? as_bf16x8(*reinterpret_cast<const uint4*>(
                              v + (seq0 + key) * ldkv + 16 * kk + 8 * g))
                        : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
    f32x16_t dka[HD / 32], dva[HD / 32];
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) { dka[db] = zero16(); dva[db] = zero16(); }

    const int n_qt = (r_end - r_begin + kQT - 1) / kQT;

    uint4 reg[8];
    float lreg = 0.f;
    // threads [0, BLK) stage Q blocks, [BLK, 2 BLK) dO blocks, then 2*kQT
    // threads the lse / delta values
    auto load_tile = [&](int R0) {
        if (tid < 2 * BLK) {
            const int blk = tid % BLK;
            const bool is_do = tid >= BLK;
            const int rb8 = blk % (kQT / 8), db8 = blk / (kQT / 8);
            // position and head of the block's first row; later rows step j
            const int row0 = R0 + rb8 * 8;
            int t = row0 / H, j = row0 - t * H;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = row0 + i;
                if (row < rows_total) {
                    const bf16_t* src = is_do ? dout + (seq0 * H + row) * HD
                                              : q + (seq0 + t) * ldq + (int64_t)j * HD;
                    reg[i] = *reinterpret_cast<const uint4*>(src + db8 * 8);
                } else {
                    reg[i] = make_uint4(0, 0, 0, 0);
                }
                if (++j == H) { j = 0; ++t; }
            }
        } else if (tid < 2 * BLK + 2 * kQT) {
            const int x = tid - 2 * BLK;
            const int row = R0 + (x % kQT);
            const float* src = (x < kQT) ? lse : delta;
            lreg = (row < rows_total) ? src[seq0 * H + row] : 0.f;
        }
    };
    auto store_tile = [&](int buf) {
        bf16_t* base = sm + buf * BUF;
        if (tid < 2 * BLK) {
            const int blk = tid % BLK;
            const bool is_do = tid >= BLK;
            const int rb8 = blk % (kQT / 8), db8 = blk / (kQT / 8);
            bf16_t* nat = base + (is_do ? QTILE : 0);
            bf16_t* tr_t = base + 2 * QTILE + (is_do ? QTILE : 0);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint4*>(nat + rt_off<KCH>(rb8 * 8 + i, db8)) = reg[i];
            uint4 tr[8];
            transpose8x8(reg, tr);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                *reinterpret_cast<uint4*>(tr_t + tt_off<kQT / 8>(db8 * 8 + c, rb8 * 8)) = tr[c];
        } else if (tid < 2 * BLK + 2 * kQT) {
            const int x = tid - 2 * BLK;
            float* lf = reinterpret_cast<float*>(base + 4 * QTILE);
            lf[x] = (x < kQT) ? lreg * kLog2e : lreg;   // [lse*log2e | delta]
        }
    };

    if (n_qt > 0) {
        load_tile(r_begin);
        store_tile(0);
    }
    __syncthreads();
    for (int it = 0; it < n_qt; ++it) {
        const int R0 = r_begin + it * kQT;
        const bool more = it + 1 < n_qt;
        if (more) load_tile(R0 + kQT);
        const bf16_t* base = sm + (it & 1) * BUF;
        const bf16_t* sQ = base;
        const bf16_t* sD = base + QTILE;
        const bf16_t* sQt = base + 2 * QTILE;
        const bf16_t* sDt = base + 3 * QTILE;
        const float* sL = reinterpret_cast<const float*>(base + 4 * QTILE);
        // rows of this tile reach keys up to their position; skip the tile if
        // even its last row precedes this wave's first key
        // some row of the tile sees this wave's first key iff its last row
        // r satisfies r >= wkey0 * H
        if (wvalid && min(R0 + kQT - 1, rows_total - 1) >= wkey0 * H) {
            f32x16_t s = zero16(), dp = zero16();
#pragma unroll
            for (int kk = 0; kk < HD / 16; ++kk) {
                const bf16x8_t aq = as_bf16x8(*reinterpret_cast<const uint4*>(
                    sQ + rt_off<KCH>(li, 2 * kk + g)));
                s = mfma32(aq, kf[kk], s);
                const bf16x8_t ad = as_bf16x8(*reinterpret_cast<const uint4*>(
                    sD + rt_off<KCH>(li, 2 * kk + g)));
                dp = mfma32(ad, vf[kk], dp);
            }
            // lane holds key `key`; register rr holds row R0 + 8(rr/4) + 4g + rr%4.
            // Row r sits at position r / H, and key <= r / H exactly when r >= key * H.
            float p[16], ds[16];
            const int first_vis = key * H;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int ro = 8 * (rr >> 2) + 4 * g + (rr & 3);
                const int row = R0 + ro;
                const bool vis = row < rows_total && row >= first_vis;
                const float pv = vis ? exp2f(s[rr] * scale_log2 - sL[ro]) : 0.f;
                p[rr] = pv;
                ds[rr] = pv * (dp[rr] - sL[kQT + ro]);
            }
#pragma unroll
            for (int ks = 0; ks < kQT / 16; ++ks) {
                const bf16x8_t bp = pack8(p + 8 * ks);
                const bf16x8_t bd = pack8(ds + 8 * ks);
#pragma unroll
                for (int db = 0; db < HD / 32; ++db) {
                    const bf16x8_t ado = tt_frag<kQT / 8>(sDt, 32 * db + li, 16 * ks + 4 * g);
                    dva[db] = mfma32(ado, bp, dva[db]);
                    const bf16x8_t aqt = tt_frag<kQT / 8>(sQt, 32 * db + li, 16 * ks + 4 * g);
                    dka[db] = mfma32(aqt, bd, dka[db]);
                }
            }
        }
        if (more) store_tile((it + 1) & 1);
        __syncthreads();
    }
    if (wvalid) {
        const int64_t pslot = ((int64_t)b * slots_per_seq + slot) * kKB + 32 * w + li;
        float* okr = dk_part + pslot * HD;
        float* ovr = dv_part + pslot * HD;
#pragma unroll
        for (int db = 0; db < HD / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d = 32 * db + 8 * gq + 4 * g;
                *reinterpret_cast<float4*>(okr + d) =
                    make_float4(dka[db][4 * gq] * scale, dka[db][4 * gq + 1] * scale,
                                dka[db][4 * gq + 2] * scale, dka[db][4 * gq + 3] * scale);
                *reinterpret_cast<float4*>(ovr + d) =
                    make_float4(dva[db][4 * gq], dva[db][4 * gq + 1], dva[db][4 * gq + 2],
                                dva[db][4 * gq + 3]);
            }
    }
}

// dk[b*T + key] = sum over the chunks of the key's block of the partials, in
// chunk order (same for dv); one thread per 4 consecutive elements
template <int HD>
__global__ __launch_bounds__(256) void k_attn_dkv_reduce(const float* __restrict__ dk_part,
                                                         const float* __restrict__ dv_part,
                                                         float* __restrict__ dk,
                                                         float* __restrict__ dv, int B, int T,
                                                         int H, int chunk_rows,
                                                         int slots_per_seq) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)B * T * (HD / 4)) return;
    const int d4 = (int)(idx % (HD / 4));
    const int64_t tok = idx / (HD / 4);
    const int b = (int)(tok / T), kk = (int)(tok % T);
    const int rows_total = T * H;
    const int kb = kk / kKB, kl = kk % kKB;
    int slot0 = 0;
    for (int i = 0; i < kb; ++i) slot0 += kv_chunks(i, H, rows_total, chunk_rows);
    const int nc = kv_chunks(kb, H, rows_total, chunk_rows);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
    for (int ci = 0; ci < nc; ++ci) {
        const int64_t off = (((int64_t)b * slots_per_seq + slot0 + ci) * kKB + kl) * HD + d4 * 4;
        const float4 x = *reinterpret_cast<const float4*>(dk_part + off);
        const float4 y = *reinterpret_cast<const float4*>(dv_part + off);
        a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
        c.x += y.x; c.y += y.y; c.z += y.z; c.w += y.w;
    }
    *reinterpret_cast<float4*>(dk + tok * HD + d4 * 4) = a;
    *reinterpret_cast<float4*>(dv + tok * HD + d4 * 4) = c;
}

int kv_slots_per_seq(int T, int H, int chunk_rows) {
    const int rows_total = T * H;
    const int n_kb = (T + kKB - 1) / kKB;
    int s = 0;
    for (int kb = 0; kb < n_kb; ++kb) s += kv_chunks(kb, H, rows_total, chunk_rows);
    return s;
}

constexpr int kChunkRows = 2048;

template <int HD>
hipError_t launch_fwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                      int64_t ldkv, bf16_t* o, float* lse, int B, int T, int H, hipStream_t s) {
    const int n_rb = (T * H + kRB - 1) / kRB;
    const float scale_log2 = kLog2e / sqrtf((float)HD);
    hipLaunchKernelGGL(k_attn_fwd_mfma<HD>, dim3(n_rb * B), dim3(256), 0, s, q, k, v, ldq, ldkv,
                       o, lse, B, T, H, scale_log2);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_bwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                      int64_t ldkv, const bf16_t* o, const bf16_t* dout, const float* lse,
                      float* scratch, float* dq, float* dk, float* dv, int B, int T, int H,
                      hipStream_t s) {
    // scratch: delta [B*T*H], then the dK and dV partials
    float* delta = scratch;
    const int64_t part = (int64_t)B * kv_slots_per_seq(T, H, kChunkRows) * kKB * HD;
    float* dk_part = scratch + ceil_div((int64_t)B * T * H, 64) * 64;
    float* dv_part = dk_part + part;
    // algorithmic work of each kernel: causal (row, key) pairs times the
    // products the kernel forms per pair (2 HD flops each), and the bytes of
    // its inputs read once and outputs written once
    const double rows = (double)B * T * H, toks = (double)B * T;
    const double pairs = (double)B * H * T * (T + 1) / 2.0;
    const double qo_b = rows * HD * 2.0, kv_b = toks * HD * 2.0;
    const int slots = kv_slots_per_seq(T, H, kChunkRows);
    hipError_t e = prof_label("attn_delta", 0, 2 * qo_b + rows * 4.0);
    if (e != hipSuccess) return e;
    e = attn_delta<bf16_t>(o, dout, (int64_t)B * T * H, HD, delta, s);
    if (e != hipSuccess) return e;
    const float scale = 1.f / sqrtf((float)HD);
    const float scale_log2 = kLog2e * scale;
    const int n_rb = (T * H + kRB - 1) / kRB;
    constexpr int dq_lds = 2 * 3 * kKT * HD * 2;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(k_attn_bwd_dq_mfma<HD>),
        hipFuncAttributeMaxDynamicSharedMemorySize, dq_lds);
    if (attr != hipSuccess) return attr;
    // dq: S, dP and dQ
    e = prof_cut("attn_bwd_dq", 3 * 2.0 * HD * pairs, 2 * qo_b + 2 * kv_b + 8.0 * rows +
                                                          rows * HD * 4.0);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_bwd_dq_mfma<HD>, dim3(n_rb * B), dim3(256), dq_lds, s, q, k, v, ldq,
                       ldkv, dout, lse, delta, dq, B, T, H, scale_log2, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dkv: S, dP, dV and dK; writes one partial per chunk
    const double part_b = 2.0 * B * slots * kKB * HD * 4.0;
    e = prof_cut("attn_bwd_dkv", 4 * 2.0 * HD * pairs, 2 * qo_b + 2 * kv_b + 8.0 * rows + part_b);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_bwd_dkv_mfma<HD>, dim3(slots * B), dim3(256), 0, s, q, k, v, ldq,
                       ldkv, dout, lse, delta, dk_part, dv_part, B, T, H, scale_log2, scale,
                       kChunkRows, slots);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = prof_cut("attn_dkv_reduce", 0, part_b + 2.0 * toks * HD * 4.0);
    if (e != hipSuccess) return e;
    const int64_t n4 = (int64_t)B * T * (HD / 4);
    hipLaunchKernelGGL(k_attn_dkv_reduce<HD>, dim3((unsigned)ceil_div(n4, 256)), dim3(256), 0, s,
                       dk_part, dv_part, dk, dv, B, T, H, kChunkRows, slots);
    return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd_mfma(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                         int64_t ldkv, bf16_t* o, float* lse, int B, int T, int H, int hd,
                         hipStream_t s) {
    if (hd == 128) return launch_fwd<128>(q, k, v, ldq, ldkv, o, lse, B, T, H, s);
    if (hd == 64) return launch_fwd<64>(q, k, v, ldq, ldkv, o, lse, B, T, H, s);
    return hipErrorInvalidValue;
}

hipError_t attn_bwd_mfma(const bf16_t* q, const bf16_t* k, const bf16_t* v, int64_t ldq,
                         int64_t ldkv, const bf16_t* o, const bf16_t* dout, const float* lse,
                         float* scratch, float* dq, float* dk, float* dv, int B, int T, int H,
                         int hd, hipStream_t s) {
    if (hd == 128)
        return launch_bwd<128>(q, k, v, ldq, ldkv, o, dout, lse, scratch, dq, dk, dv, B, T, H, s);
    if (hd == 64)
        return launch_bwd<64>(q, k, v, ldq, ldkv, o, dout, lse, scratch, dq, dk, dv, B, T, H, s);
    return hipErrorInvalidValue;
}

size_t attn_bwd_scratch_bytes(int B, int T, int H, int hd) {
    const int64_t delta = ceil_div((int64_t)B * T * H, 64) * 64;
    const int64_t part = (int64_t)B * kv_slots_per_seq(T, H, kChunkRows) * kKB * hd;
    return (size_t)(delta + 2 * part) * sizeof(float);
}

}  // namespace nc
