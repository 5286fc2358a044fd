// GEMM family of the step: C[m][n] = sum_k A(m,k) B(n,k) with fp32
// accumulation and a fused epilogue.  Every linear layer of the model is
// bias-free (architecture list of the nanochat article), so each forward
// projection is Y = X W^T, each data gradient dX = dY W and each weight
// gradient dW = dY^T X; all three are this one contraction with the operands
// read either along k ("k-major") or along m/n ("mn-major").
//
// bf16: CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).  A 512-thread
// workgroup (8 waves, two per SIMD) owns a 256 (m) x 256 (n) output tile;
// wave w owns 64 m rows x 128 n rows, held as 2 x 4 accumulator blocks of
// 32 x 32 fp32.  The k loop stages 256 x 64 tiles of both operands in two
// LDS buffers with an XOR swizzle of the 16-byte chunks of each row, so
// fragment reads of 8 or 16 consecutive rows at one logical chunk hit
// distinct banks (the bank-conflict counter reads zero).
//   Both operands go straight from global memory into LDS
//   (buffer loads with the LDS bit, no staging registers); the loads of tile k+1
//   are in flight while tile k is multiplied.
//   k-major tiles are stored 256 rows x 64 k and a fragment is one 16-byte
//   read.  mn-major tiles (the weight-gradient layout) are stored as they lie
//   in memory, 64 k x 256 rows, and a fragment (8 consecutive k of one row)
//   is two LDS transpose reads (ds_read_b64_tr_b16), so no layout is ever
//   transposed in registers.  In both, the fragments of k step s+1 are read
//   while the matrix instructions of step s issue.  The buffers are four
//   distinct LDS arrays, the k loop is unrolled by two so that each access
//   names its array at compile time, and every access is one byte offset from
//   its array: only then can the compiler tell that LDS reads of one buffer do
//   not alias copies in flight into the other (otherwise it waits for those
//   copies before the reads).
// The MFMA "A" side takes the n rows and the "B" side the m rows, which puts
// 4 consecutive n of one row m in each lane's accumulator registers: the
// epilogue stores 8 (bf16) or 16 (fp32) contiguous bytes per lane.
// Tiles are visited XCD by XCD (each of the 8 dies gets a contiguous range)
// and in groups of 4 m-tiles, so the operand rows they share stay in L2.
//
// fp32: a plain LDS-tiled SIMT kernel (64 x 64 tiles, 4 x 4 per thread).
#include "kernels.h"

namespace nc {

namespace {

struct EpiDev {
    int mode;
    const float* rowscale;
    const void* aux;
    int accumulate;
    const float* cos_t;
    const float* sin_t;
    float* rqk;
    int seq_len, n_head, head_dim;
    float eps;
    float alpha, beta;
};

EpiDev make_epi(const Epilogue& p) {
    return EpiDev{p.mode,   p.rowscale, p.aux,     p.accumulate ? 1 : 0, p.cos_t, p.sin_t,
                  p.rqk,    p.seq_len,  p.n_head,  p.head_dim,           p.eps,   p.alpha,
                  p.beta};
}

template <typename T>
__device__ __forceinline__ float epi_value(const EpiDev& e, int64_t m, int64_t idx, float acc) {
    switch (e.mode) {
        case EPI_ROWSCALE: return e.rowscale[m] * acc;
        case EPI_ROWSCALE_RELU2: {
            const float u = fmaxf(e.rowscale[m] * acc, 0.f);
            return u * u;
        }
        case EPI_RESID: return Elt<T>::ld(static_cast<const T*>(e.aux) + idx) + acc;
        case EPI_RELU2_BWD:
            return e.rowscale[m] * acc * 2.f * sqrtf(Elt<T>::ld(static_cast<const T*>(e.aux) + idx));
        case EPI_AXPBY:
            return e.alpha * Elt<T>::ld(static_cast<const T*>(e.aux) + idx) + e.beta * acc;
        default: return acc;  // EPI_STORE_T
    }
}

template <typename T>
__device__ __forceinline__ void epi_store1(const EpiDev& e, void* C, int64_t ldc, int64_t m,
                                           int64_t n, float acc) {
    const int64_t idx = m * ldc + n;
    if (e.mode == EPI_STORE_F32) {
        float* c = static_cast<float*>(C) + idx;
        *c = e.accumulate ? *c + acc : acc;
    } else {
        Elt<T>::st(static_cast<T*>(C) + idx, epi_value<T>(e, m, idx, acc));
    }
}

// ------------------------------------------------------------------ SIMT
constexpr int kSB = 64, kSK = 16;

template <typename T>
__global__ __launch_bounds__(256) void k_gemm_simt(int M, int N, int K, const T* __restrict__ A,
                                                   int64_t lda, int ak, const T* __restrict__ B,
                                                   int64_t ldb, int bk, void* C, int64_t ldc,
                                                   EpiDev e, int64_t bsa, int64_t bsb,
                                                   int64_t bsc) {
    // product blockIdx.z of a batch
    const int64_t bz = blockIdx.z;
    A += bz * bsa;
    B += bz * bsb;
    if (e.mode == EPI_STORE_F32) C = static_cast<float*>(C) + bz * bsc;
    else C = static_cast<T*>(C) + bz * bsc;
    if (e.aux) e.aux = static_cast<const T*>(e.aux) + bz * bsc;
    __shared__ float As[kSK][kSB + 4];
    __shared__ float Bs[kSK][kSB + 4];
    const int m0 = blockIdx.y * kSB, n0 = blockIdx.x * kSB;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kSK) {
        for (int i = threadIdx.x; i < kSB * kSK; i += 256) {
            int r, kk;
            if (ak) { r = i / kSK; kk = i % kSK; } else { kk = i / kSB; r = i % kSB; }
            const int64_t m = m0 + r, k = k0 + kk;
            float v = 0.f;
            if (m < M && k < K) v = Elt<T>::ld(A + (ak ? m * lda + k : k * lda + m));
            As[kk][r] = v;
        }
        for (int i = threadIdx.x; i < kSB * kSK; i += 256) {
            int r, kk;
            if (bk) { r = i / kSK; kk = i % kSK; } else { kk = i / kSB; r = i % kSB; }
            const int64_t n = n0 + r, k = k0 + kk;
            float v = 0.f;
            if (n < N && k < K) v = Elt<T>::ld(B + (bk ? n * ldb + k : k * ldb + n));
            Bs[kk][r] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kSK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < N) epi_store1<T>(e, C, ldc, m, n, acc[i][j]);
        }
    }
}

// ------------------------------------------------------------------ MFMA (bf16)
constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kThreads = 512;                         // 8 waves, 2 per SIMD
constexpr int kTileElems = kTM * kTK;                 // one operand tile (256 rows x 64 k)

// Stage one 256-row x 64-k operand tile into LDS.
//   k-major: straight from global memory into LDS (buffer load, LDS bit).
//     Wave w's instruction i fills the 64 consecutive 16-byte LDS slots of
//     rows 64 i + 8 w .. +7, so lane l holds row 64 i + 8 w + (l >> 3) at
//     physical chunk l & 7, i.e. logical chunk (l & 7) ^ (l >> 3) ^ w under
//     the swizzle -- the same for every i.  Each lane therefore keeps one
//     32-bit offset per instruction from a uniform tile base that advances
//     by 64 columns per k step.  Rows past `rows` are clamped to the last row
//     (those outputs are never stored).  Requires k0 + 64 <= K.
//   mn-major: 256 threads (half of the workgroup) each load an 8 (k) x 8 (row)
//     block into registers; tile_store_mn transposes and writes it.
struct KmajLoads {
    uint32_t off[4];   // byte offsets of this lane's four chunks from the tile base
};

__device__ __forceinline__ KmajLoads kmaj_offsets(int64_t ld, int rows, int r0, int w, int lane) {
    KmajLoads L;
    const int lc = (lane & 7) ^ (lane >> 3) ^ w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = min(r0 + 64 * i + 8 * w + (lane >> 3), rows - 1) - r0;
        L.off[i] = (uint32_t)(((int64_t)row * ld + lc * 8) * 2);
    }
    return L;
}

// tile_base points at element (r0, k0) of the operand; T is the LDS tile
__device__ __forceinline__ void kmaj_issue(const bf16_t* tile_base, const KmajLoads& L, bf16_t* T,
                                           int w) {
    const buf_rsrc_t r = make_rsrc(tile_base);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy<16>(r, (int)L.off[i], T + (i * 8 + w) * 512);
}

// mn-major operand P(r, k) = P[k * ld + r]: the tile is stored as it lies in
// memory, 64 k rows of 256 r (512 bytes, 32 chunks), chunk c of k row kr at
// chunk position c ^ ((kr & 3) << 2).  Copy instruction i of wave w fills k
// rows 2 (8 i + w) and 2 (8 i + w) + 1; lane l takes row + (l >> 5), chunk
// position l & 31.  Chunks past `rows` get an offset beyond the buffer
// resource's range, which the copy turns into zeros (their products land in
// outputs that are never stored).  Requires k0 + 64 <= K.
constexpr int kOutOfRange = (int)0x80000000u;
struct MnLoads {
    int off[4];   // byte offsets of this lane's four chunks from element (k0, r0)
};

__device__ __forceinline__ MnLoads mn_offsets(int64_t ld, int rows, int r0, int w, int lane) {
    MnLoads L;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = 2 * (8 * i + w) + (lane >> 5);
        const int c = (lane & 31) ^ ((kr & 3) << 2);
        L.off[i] = r0 + 8 * c < rows ? (int)(((int64_t)kr * ld + 8 * c) * 2) : kOutOfRange;
    }
    return L;
}

__device__ __forceinline__ void mn_issue(const bf16_t* tile_base, const MnLoads& L, bf16_t* T,
                                         int w) {
    const buf_rsrc_t r = make_rsrc(tile_base);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy<16>(r, L.off[i], T + (i * 8 + w) * 512);
}

// byte offset, in an mn-major tile, of this lane's first transpose read for
// the 32-row block starting at r (k step 0): rows k = 8 g + (s >> 2), columns
// r + 16 half + 4 (s & 3), s = lane & 15.  The second read of a fragment is
// 4 k rows further; k step ks adds 16 ks rows.  The chunk swizzle depends
// on k & 3 = s >> 2 only, so these offsets hold for every k step.
__device__ __forceinline__ int mn_frag_off(int r, int lane) {
    const int s = lane & 15, half = (lane >> 4) & 1, g = lane >> 5;
    const int kr = 8 * g + (s >> 2);
    const int col = r + 16 * half + 4 * (s & 3);
    return kr * 512 + ((((col >> 3) ^ ((kr & 3) << 2))) << 4) + ((col & 7) << 1);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
// 8 consecutive k of one row from an mn-major tile: two transpose reads
__device__ __forceinline__ bf16x8_t mn_frag(const char* p) {
    typedef __attribute__((address_space(3))) v4i16_t lds4;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4*)(p));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4*)(p + 4 * 512));
    const uint2 x = __builtin_bit_cast(uint2, lo), y = __builtin_bit_cast(uint2, hi);
    return as_bf16x8(make_uint4(x.x, x.y, y.x, y.y));
}

// wait until this thread's direct global->LDS loads have landed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until this thread's LDS reads and writes have completed
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// workgroup barrier without the memory fence __syncthreads() implies: the
// fence would wait for every outstanding load, including the direct loads of
// tiles still in flight.  LDS data the barrier publishes has landed through an
// explicit vmcnt wait; the empty asm keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}


__device__ __forceinline__ int xcd_remap(int pid, int total) {
    // consecutive workgroup ids land on different XCDs (round robin over 8);
    // give each XCD a contiguous range of work items so neighbours share its
    // L2: XCD x takes q + (x < r) items starting at x q + min(x, r), with
    // total = 8 q + r (a bijection of [0, total))
    const int q = total >> 3, r = total & 7;
    const int x = pid & 7, local = pid >> 3;
    return x * q + min(x, r) + local;
}

// output stores are marked non-temporal: the product never reads its output
// back, and streaming it past L2 keeps the operand panels that neighbouring
// tiles share resident (measured faster over the whole step)
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// cache-policy operand of the buffer stores: non-temporal
constexpr int kNonTemporal = 2;
__device__ __forceinline__ void st_nt(void* p, uint2 v) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), (u32x2*)p);
}
__device__ __forceinline__ void st_nt(void* p, float4 v) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4v, v), (f32x4v*)p);
}

template <int MODE>
__device__ __forceinline__ void epi_vec4(const EpiDev& e, void* C, int64_t idx, int64_t m,
                                         float v0, float v1, float v2, float v3) {
    if (MODE == EPI_STORE_F32) {
        float4* c = reinterpret_cast<float4*>(static_cast<float*>(C) + idx);
        float4 o = make_float4(v0, v1, v2, v3);
        if (e.accumulate) {
            const float4 p = *c;
            o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
        }
        st_nt(c, o);
    } else {
        float o[4] = {v0, v1, v2, v3};
        if (MODE == EPI_RESID || MODE == EPI_RELU2_BWD || MODE == EPI_AXPBY) {
            const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(e.aux) + idx);
            const float x[4] = {bf_lo(a.x), bf_hi(a.x), bf_lo(a.y), bf_hi(a.y)};
            if (MODE == EPI_RESID) {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] += x[q];
            } else if (MODE == EPI_AXPBY) {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = e.alpha * x[q] + e.beta * o[q];
            } else {
                const float rs = 2.f * e.rowscale[m];
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] *= rs * sqrtf(x[q]);
            }
        } else if (MODE == EPI_ROWSCALE) {
            const float rs = e.rowscale[m];
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] *= rs;
        } else if (MODE == EPI_ROWSCALE_RELU2) {
            const float rs = e.rowscale[m];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float u = fmaxf(rs * o[q], 0.f);
                o[q] = u * u;
            }
        }
        st_nt(static_cast<bf16_t*>(C) + idx, make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])));
    }
}

// epi_vec4 with the row scale and the 4 aux values already in registers
template <int MODE>
__device__ __forceinline__ void epi_vec4_pre(const EpiDev& e, void* C, int64_t idx, float4 v,
                                             uint2 a, float rs) {
    if (MODE == EPI_STORE_F32) {
        epi_vec4<MODE>(e, C, idx, 0, v.x, v.y, v.z, v.w);
        return;
    }
    float o[4] = {v.x, v.y, v.z, v.w};
    const float x[4] = {bf_lo(a.x), bf_hi(a.x), bf_lo(a.y), bf_hi(a.y)};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (MODE == EPI_RESID) o[q] += x[q];
        if (MODE == EPI_AXPBY) o[q] = e.alpha * x[q] + e.beta * o[q];
        if (MODE == EPI_RELU2_BWD) o[q] *= 2.f * rs * __builtin_amdgcn_sqrtf(x[q]);
        if (MODE == EPI_ROWSCALE) o[q] *= rs;
        if (MODE == EPI_ROWSCALE_RELU2) {
            const float u = fmaxf(rs * o[q], 0.f);
            o[q] = u * u;
        }
    }
    st_nt(static_cast<bf16_t*>(C) + idx, make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])));
}

// QKV epilogue for 4 consecutive columns n .. n+3 of row m held by lane li of
// a half-wave whose 32 lanes hold one 128-column stretch of the row (so every
// head of head_dim <= 128 lies in an aligned group of head_dim/4 lanes).
// u = rowscale * acc; a query or key head is rotated -- element i < hd/2 pairs
// with i + hd/2, which sits hd/8 lanes away -- and RMS-normalised over its
// group; the value head is stored as u.
__device__ __forceinline__ void qkv_rope_store(const EpiDev& e, bf16_t* C, int64_t ldc, int M,
                                               int N, int64_t m, int64_t n, float4 v,
                                               float rs_m) {
    // 32-bit index arithmetic (rows < 2^24, columns < 2^16); head_dim is a
    // power of two
    const int hd = e.head_dim, half = hd >> 1, H = e.n_head;
    const int hd_shift = __builtin_ctz((unsigned)hd);
    const int mi = (int)m, ni = (int)n;
    const bool valid = mi < M && ni < N;
    const float rs = valid ? rs_m : 0.f;
    float x[4] = {v.x * rs, v.y * rs, v.z * rs, v.w * rs};
    const int head = ni >> hd_shift;             // uniform over the lane group
    const int d = ni & (hd - 1);                 // first of this lane's 4 elements
    if (head <= H) {
        const int lanes = hd >> 2;               // lanes per head
        float px[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) px[q] = __shfl_xor(x[q], lanes >> 1, 64);
        const int i = d < half ? d : d - half;
        const int pos = valid ? mi % e.seq_len : 0;
        const float4 c4 = *reinterpret_cast<const float4*>(e.cos_t + pos * half + i);
        const float4 s4 = *reinterpret_cast<const float4*>(e.sin_t + pos * half + i);
        const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // first half: x0 = own, x1 = partner; second half: x0 = partner, x1 = own
            const float y = d < half ? x[q] * cs[q] - px[q] * sn[q] : px[q] * sn[q] + x[q] * cs[q];
            x[q] = y;
            ss += y * y;
        }
        ss = group_sum(ss, lanes);
        const float rr = __builtin_amdgcn_rsqf(ss / (float)hd + e.eps);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] *= rr;
        if (valid && d == 0) e.rqk[(int64_t)mi * (H + 1) + head] = rr;
    }
    if (valid)
        *reinterpret_cast<uint2*>(C + m * ldc + n) =
            make_uint2(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]));
}

// sum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1): every lane
// of the row ends with the same value
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, true));
    return v;
}

// The same for head_dim 128, where a wave's 128 columns are one head: 16
// lanes take one row, lane l the columns 4 l .. +3 and their rotation
// partners 64 + 4 l .. +3, so the rotation needs no exchange and the head's
// sum of squares is one 16-lane DPP reduction.  `stage` holds the wave's 32
// rows x 128 columns (16-byte chunk c of row r at chunk position c ^ r).
__device__ __forceinline__ void qkv_rope_pass128(const EpiDev& e, bf16_t* C, int64_t ldc, int M,
                                                 int N, const float* stage, int mrow0,
                                                 int ncol0, int lane, const float* rsl) {
    if (ncol0 >= N) return;
    const int H = e.n_head;
    const int head = ncol0 >> 7;
    const bool rot = head <= H;
    const int l16 = lane & 15, rsub = lane >> 4;
    // Whole 32-row passes inside one sequence (every pass of the step's
    // shapes: rows are tokens, sequences are multiples of 32 long) take a
    // branch-free path: the position is the pass's first position plus the
    // row, and the stores are buffer stores at scalar row offsets.
    if (mrow0 + 32 <= M && (e.seq_len & 31) == 0 && ldc <= (1 << 24)) {
        const int pos0 = mrow0 % e.seq_len;
        const buf_rsrc_t rc = make_rsrc(C + (int64_t)mrow0 * ldc + ncol0);
        const int voff = (rsub * (int)ldc + 4 * l16) * 2;
        float4 c4[8], s4[8];
        if (rot) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int pos = pos0 + 4 * t + rsub;
                c4[t] = *reinterpret_cast<const float4*>(e.cos_t + pos * 64 + 4 * l16);
                s4[t] = *reinterpret_cast<const float4*>(e.sin_t + pos * 64 + 4 * l16);
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = 4 * t + rsub;
            const float4 a = *reinterpret_cast<const float4*>(stage + row * 128 + ((l16 ^ row) << 2));
            const float4 b =
                *reinterpret_cast<const float4*>(stage + row * 128 + (((16 + l16) ^ row) << 2));
            const float rs = rsl[row];
            float x1[4] = {a.x * rs, a.y * rs, a.z * rs, a.w * rs};
            float x2[4] = {b.x * rs, b.y * rs, b.z * rs, b.w * rs};
            if (rot) {
                const float cs[4] = {c4[t].x, c4[t].y, c4[t].z, c4[t].w};
                const float sn[4] = {s4[t].x, s4[t].y, s4[t].z, s4[t].w};
                float ss = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float y1 = x1[q] * cs[q] - x2[q] * sn[q];
                    const float y2 = x1[q] * sn[q] + x2[q] * cs[q];
                    x1[q] = y1;
                    x2[q] = y2;
                    ss += y1 * y1 + y2 * y2;
                }
                ss = row16_sum(ss);
                const float rr = __builtin_amdgcn_rsqf(ss * (1.f / 128.f) + e.eps);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x1[q] *= rr;
                    x2[q] *= rr;
                }
                if (l16 == 0) e.rqk[(int64_t)(mrow0 + row) * (H + 1) + head] = rr;
            }
            const int so = 4 * t * (int)ldc * 2;
            const u32x2_t w1 = {pack_bf2(x1[0], x1[1]), pack_bf2(x1[2], x1[3])};
            const u32x2_t w2 = {pack_bf2(x2[0], x2[1]), pack_bf2(x2[2], x2[3])};
            __builtin_amdgcn_raw_buffer_store_b64(w1, rc, voff, so, kNonTemporal);
            __builtin_amdgcn_raw_buffer_store_b64(w2, rc, voff + 128, so, kNonTemporal);
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int row = 4 * t + rsub;
        const int mi = mrow0 + row;
        const float4 a = *reinterpret_cast<const float4*>(stage + row * 128 + ((l16 ^ row) << 2));
        const float4 b =
            *reinterpret_cast<const float4*>(stage + row * 128 + (((16 + l16) ^ row) << 2));
        const bool valid = mi < M;
        const float rs = valid ? rsl[row] : 0.f;
        float x1[4] = {a.x * rs, a.y * rs, a.z * rs, a.w * rs};
        float x2[4] = {b.x * rs, b.y * rs, b.z * rs, b.w * rs};
        if (rot) {
            const int pos = valid ? mi % e.seq_len : 0;
            const float4 c4 = *reinterpret_cast<const float4*>(e.cos_t + pos * 64 + 4 * l16);
            const float4 s4 = *reinterpret_cast<const float4*>(e.sin_t + pos * 64 + 4 * l16);
            const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
            float ss = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float y1 = x1[q] * cs[q] - x2[q] * sn[q];
                const float y2 = x1[q] * sn[q] + x2[q] * cs[q];
                x1[q] = y1;
                x2[q] = y2;
                ss += y1 * y1 + y2 * y2;
            }
            ss = row16_sum(ss);
            const float rr = __builtin_amdgcn_rsqf(ss * (1.f / 128.f) + e.eps);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x1[q] *= rr;
                x2[q] *= rr;
            }
            if (valid && l16 == 0) e.rqk[(int64_t)mi * (H + 1) + head] = rr;
        }
        if (valid) {
            bf16_t* o = C + (int64_t)mi * ldc + ncol0 + 4 * l16;
            st_nt(o, make_uint2(pack_bf2(x1[0], x1[1]), pack_bf2(x1[2], x1[3])));
            st_nt(o + 64, make_uint2(pack_bf2(x2[0], x2[1]), pack_bf2(x2[2], x2[3])));
        }
    }
}

// 512 threads: wave w owns m rows wm*64 .. +63 (wm = w & 3) and n rows
// wn*128 .. +127 (wn = w >> 2) of the 256 x 256 tile: 2 x 4 accumulator blocks.
// In a k-major tile, fragment row 32 i + (lane & 31) of a 32-aligned block
// has swizzle f0 ^ 4 (i & 1) with f0 that of (lane & 31), so the chunk
// offsets of the 4 k steps for the two parities are precomputed per lane
// (foff) and every fragment read is base + constant.
template <bool AK, bool BK, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mfma(int M, int N, int K, int k_per_split,
                                                           int nsplit,
                                                           const bf16_t* __restrict__ A,
                                                           int64_t lda,
                                                           const bf16_t* __restrict__ B,
                                                           int64_t ldb, void* C, int64_t ldc,
                                                           EpiDev e, int64_t split_stride,
                                                           int64_t bsa, int64_t bsb,
                                                           int64_t bsc) {
    // two buffers of an A tile and a B tile, as four distinct arrays: with the
    // buffer known at compile time (the k loop is unrolled by two) and one
    // byte offset from the array's start per access, the compiler can see
    // that copies into one buffer never alias reads of the other
    __shared__ __align__(16) bf16_t ldsA0[kTileElems];
    __shared__ __align__(16) bf16_t ldsA1[kTileElems];
    __shared__ __align__(16) bf16_t ldsB0[kTileElems];
    __shared__ __align__(16) bf16_t ldsB1[kTileElems];
    // the tile's row scales, copied into LDS with the first k tile: the
    // epilogue reads them there instead of waiting on global loads
    __shared__ __align__(16) float lds_rs[kTM];

    const int tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
    const int total = tiles_m * tiles_n;
    // one work item per (k split, tile), split-major, spread over the XCDs
    // in contiguous ranges
    const int item = xcd_remap(blockIdx.x, total * nsplit);
    const int split = item / total;
    const int pid = item - split * total;
    // grouped order: 4 m-tiles share a column sweep over n (of 2, 3, 4, 6, 8,
    // 16 and 32 the fastest over the whole training step)
    constexpr int kGroup = 4;
    const int group = pid / (kGroup * tiles_n);
    const int first_m = group * kGroup;
    const int gsize = min(tiles_m - first_m, kGroup);
    const int tm = first_m + (pid % (kGroup * tiles_n)) % gsize;
    const int tn = (pid % (kGroup * tiles_n)) / gsize;
    const int m0 = tm * kTM, n0 = tn * kTN;

    const int kb = split * k_per_split;
    const int ke = min(K, kb + k_per_split);
    if (MODE == EPI_STORE_F32 && split_stride)
        C = static_cast<float*>(C) + split * split_stride;
    // product blockIdx.y of a batch (the batched products run unsplit)
    {
        const int64_t bz = blockIdx.y;
        A += bz * bsa;
        B += bz * bsb;
        if (MODE == EPI_STORE_F32) C = static_cast<float*>(C) + bz * bsc;
        else C = static_cast<bf16_t*>(C) + bz * bsc;
        if (MODE == EPI_RESID || MODE == EPI_RELU2_BWD || MODE == EPI_AXPBY)
            e.aux = static_cast<const bf16_t*>(e.aux) + bz * bsc;
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 3, wn = wave >> 2;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    int foff[2][4];
    {
        const int fr = lane & 31, fch = lane >> 5;
        const int f0 = (fr ^ (fr >> 3)) & 7;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) foff[p][ks] = ((2 * ks + fch) ^ f0 ^ (4 * p)) << 3;
    }

    // both operands stream straight into LDS; the two layouts differ only in
    // the copy offsets and in how a fragment is read (one 16-byte row read
    // for k-major, two transpose reads for mn-major)
    KmajLoads la, lb;
    MnLoads ma, mb;
    if (AK) la = kmaj_offsets(lda, M, m0, wave, lane);
    else ma = mn_offsets(lda, M, m0, wave, lane);
    if (BK) lb = kmaj_offsets(ldb, N, n0, wave, lane);
    else mb = mn_offsets(ldb, N, n0, wave, lane);
    int tra[2], trb[4];
    if (!AK)
#pragma unroll
        for (int j = 0; j < 2; ++j) tra[j] = mn_frag_off(wm * 64 + j * 32, lane);
    if (!BK)
#pragma unroll
        for (int i = 0; i < 4; ++i) trb[i] = mn_frag_off(wn * 128 + i * 32, lane);
    const int nk = (ke - kb + kTK - 1) / kTK;
    auto issue = [&](int kt, bf16_t* ta, bf16_t* tb) {
        const int k0 = kb + kt * kTK;
        if (AK) kmaj_issue(A + (int64_t)m0 * lda + k0, la, ta, wave);
        else mn_issue(A + (int64_t)k0 * lda + m0, ma, ta, wave);
        if (BK) kmaj_issue(B + (int64_t)n0 * ldb + k0, lb, tb, wave);
        else mn_issue(B + (int64_t)k0 * ldb + n0, mb, tb, wave);
    };
    // the epilogue's aux rows (x of the residual, g of the relu^2 backward)
    constexpr bool kAux = MODE == EPI_RESID || MODE == EPI_RELU2_BWD || MODE == EPI_AXPBY;
    const int li = lane & 31, hi = lane >> 5;
    const bool full_n = n0 + kTN <= N;
    auto load_aux = [&](int j, uint2 (&dst)[16]) {
        const int64_t n = n0 + wn * 128 + 4 * li;
        const bool nok = full_n || n + 3 < N;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int64_t m = m0 + wm * 64 + 32 * j + 2 * t + hi;
            dst[t] = make_uint2(0, 0);
            if (m < M && nok)
                dst[t] = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(e.aux) +
                                                         m * ldc + n);
        }
    };
    constexpr bool kRsMode = MODE == EPI_ROWSCALE || MODE == EPI_ROWSCALE_RELU2 ||
                             MODE == EPI_RELU2_BWD || MODE == EPI_QKV_ROPE;
    if (kRsMode && wave == 0) {
        const buf_rsrc_t r = make_rsrc(e.rowscale + m0);
#pragma unroll
        for (int i = 0; i < kTM / 64; ++i)
            lds_copy<4>(r, m0 + 64 * i + lane < M ? (64 * i + lane) * 4 : kOutOfRange,
                        lds_rs + 64 * i);
    }
    if (nk > 0) issue(0, ldsA0, ldsB0);
    wait_vmem();
    __syncthreads();
    {
        // fragments of k step ks+1 are read while the 8 matrix instructions
        // of step ks issue
        const int rowoff = (lane & 31) * kTK;
        bf16x8_t fa[2][4], fb[2][2];
        auto ld16 = [](const bf16_t* t, int byte_off) {
            return as_bf16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(t) +
                                                             byte_off));
        };
        auto rd_a = [&](const bf16_t* tb, int ks, int set, int i) {
            fa[set][i] = BK ? ld16(tb, 2 * ((wn * 128 + i * 32) * kTK + rowoff + foff[i & 1][ks]))
                            : mn_frag(reinterpret_cast<const char*>(tb) + (trb[i] + ks * 16 * 512));
        };
        auto rd_b = [&](const bf16_t* ta, int ks, int set, int j) {
            fb[set][j] = AK ? ld16(ta, 2 * ((wm * 64 + j * 32) * kTK + rowoff + foff[j & 1][ks]))
                            : mn_frag(reinterpret_cast<const char*>(ta) + (tra[j] + ks * 16 * 512));
        };
        // a step's fragments are read in the order its products first use
        // them (block i outer, j inner), so its first products wait for the
        // first two reads only
        auto rd = [&](const bf16_t* ta, const bf16_t* tb, int ks, int set) {
            rd_a(tb, ks, set, 0);
            rd_b(ta, ks, set, 0);
            rd_b(ta, ks, set, 1);
            rd_a(tb, ks, set, 1);
            rd_a(tb, ks, set, 2);
            rd_a(tb, ks, set, 3);
        };
        // one k tile from (ca, cb); the next one is copied into (na, nb)
        auto step = [&](int kt, const bf16_t* ca, const bf16_t* cb, bf16_t* na, bf16_t* nb) {
            if (kt > 0) {
                // tile kt has landed (this wave's loads) and every wave is
                // done reading tile kt-1, whose buffer is refilled next
                wait_vmem();
                barrier_nofence();
            }
            if (kt == 0) {
                // first tile: its first fragments are read before the next
                // tile's copy is issued
                rd(ca, cb, 0, 0);
                if (kt + 1 < nk) issue(kt + 1, na, nb);
            } else {
                if (kt + 1 < nk) issue(kt + 1, na, nb);
                rd(ca, cb, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < kTK / 16; ++ks) {
                const int cs = ks & 1;
                if (ks + 1 < kTK / 16) rd(ca, cb, ks + 1, cs ^ 1);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = mfma32(fa[cs][i], fb[cs][j], acc[i][j]);
                // interleave the next step's fragment reads with this step's
                // products: k-major 2 MFMAs / 2 reads, with an mn-major operand
                // (two transpose reads per fragment) 1 MFMA / 3 reads
                if (ks + 1 < kTK / 16) {
                    constexpr bool kKm = AK && BK;
                    constexpr int kGroups = kKm ? 3 : 4;
                    constexpr int kMfmaPerGroup = kKm ? 2 : 1;
                    constexpr int kReadsPerGroup = kKm ? 2 : 3;
#pragma unroll
                    for (int x = 0; x < kGroups; ++x) {
                        __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerGroup, 0);   // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerGroup, 0);  // reads
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 8 - kGroups * kMfmaPerGroup,
                                                         0);                             // the rest
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int kt = 0; kt < nk; kt += 2) {
            step(kt, ldsA0, ldsB0, ldsA1, ldsB1);
            if (kt + 1 < nk) step(kt + 1, ldsA1, ldsB1, ldsA0, ldsB0);
        }
    }

    // epilogue, staged through LDS so that global reads and writes are whole
    // rows: lane holds m = m0 + wm*64 + 32 j + (lane & 31) and, for register
    // group q of block i, n = n0 + wn*128 + 32 i + 8 q + 4 (lane >> 5) + 0..3.
    // For each j the wave parks its 32 x 128 fp32 block in its own 16 KB of
    // LDS (16-byte chunk c of row r at chunk position c ^ r), then reads it
    // back two rows per instruction: lane l takes row 2 t + (l >> 5), columns
    // 4 (l & 31) .. +3, so 32 lanes cover one row's 128 columns contiguously.
    // Every wave is done reading the last k tile.  From here on each wave
    // works in its own slot of LDS, so the passes need no workgroup barrier
    // (a wave's LDS accesses are performed in order) and no fence, which would
    // wait for the previous pass's output stores.
    wait_lds();
    barrier_nofence();
    // (two waves' 16 KB per 32 KB array)
    bf16_t* const stage_arr = wave < 2 ? ldsA0 : wave < 4 ? ldsA1 : wave < 6 ? ldsB0 : ldsB1;
    float* stage = reinterpret_cast<float*>(stage_arr) + (wave & 1) * 4096;
    constexpr bool kRs = MODE == EPI_ROWSCALE || MODE == EPI_ROWSCALE_RELU2 || MODE == EPI_RELU2_BWD;
    // Whole tiles (every tile of the step's shapes but the ragged edges) take
    // a branch-free path: buffer loads and stores whose row offsets are scalar
    // multiples of the row stride, so a row costs no address arithmetic and
    // the 16 LDS reads of a pass are not serialised behind bounds tests.  Byte
    // offsets inside a tile must fit in 31 bits.
    constexpr int kEs = MODE == EPI_STORE_F32 ? 4 : 2;
    const bool fast = MODE != EPI_QKV_ROPE && full_n && m0 + kTM <= M && ldc <= (1 << 20) &&
                      !(MODE == EPI_STORE_F32 && e.accumulate);
    if (fast) {
        const int64_t tile0 = (int64_t)m0 * ldc + n0;
        const buf_rsrc_t rc = make_rsrc(static_cast<char*>(C) + tile0 * kEs);
        const int srow = 2 * (int)ldc * kEs;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row0 = wm * 64 + 32 * j + hi;
            const int voff = (row0 * (int)ldc + wn * 128 + 4 * li) * kEs;
            // the pass's epilogue inputs are requested before the LDS round trip
            u32x2_t auxv[16];
            float rsv[16];
            if (kAux) {
                const buf_rsrc_t ra = make_rsrc(static_cast<const bf16_t*>(e.aux) + tile0);
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    auxv[t] = __builtin_amdgcn_raw_buffer_load_b64(ra, voff, t * srow, 0);
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) rsv[t] = kRs ? lds_rs[row0 + 2 * t] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 8 * i + 2 * q + hi;
                    *reinterpret_cast<float4*>(stage + li * 128 + ((c ^ li) << 2)) =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]);
                }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int row = 2 * t + hi;
                const float4 v = *reinterpret_cast<const float4*>(stage + row * 128 + ((li ^ row) << 2));
                if (MODE == EPI_STORE_F32) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rc, voff,
                                                           t * srow, kNonTemporal);
                    continue;
                }
                float o[4] = {v.x, v.y, v.z, v.w};
                const float x[4] = {bf_lo(auxv[t].x), bf_hi(auxv[t].x), bf_lo(auxv[t].y),
                                    bf_hi(auxv[t].y)};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (MODE == EPI_RESID) o[q] += x[q];
                    if (MODE == EPI_AXPBY) o[q] = e.alpha * x[q] + e.beta * o[q];
                    if (MODE == EPI_RELU2_BWD) o[q] *= 2.f * rsv[t] * __builtin_amdgcn_sqrtf(x[q]);
                    if (MODE == EPI_ROWSCALE) o[q] *= rsv[t];
                    if (MODE == EPI_ROWSCALE_RELU2) {
                        const float u = fmaxf(rsv[t] * o[q], 0.f);
                        o[q] = u * u;
                    }
                }
                const u32x2_t w = {pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])};
                __builtin_amdgcn_raw_buffer_store_b64(w, rc, voff, t * srow, kNonTemporal);
            }
            __builtin_amdgcn_wave_barrier();
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        // the pass's epilogue inputs are requested before the LDS round trip
        uint2 auxv[16];
        float rsv[16];
        if (kAux) load_aux(j, auxv);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int64_t m = m0 + wm * 64 + 32 * j + 2 * t + hi;
            rsv[t] = (kRs && m < M) ? lds_rs[m - m0] : 0.f;
            if (!kAux) auxv[t] = make_uint2(0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = 8 * i + 2 * q + hi;
                *reinterpret_cast<float4*>(stage + li * 128 + ((c ^ li) << 2)) =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]);
            }
        __builtin_amdgcn_wave_barrier();
        const int64_t n = n0 + wn * 128 + 4 * li;
        if (MODE == EPI_QKV_ROPE && e.head_dim == 128) {
            qkv_rope_pass128(e, static_cast<bf16_t*>(C), ldc, M, N, stage, m0 + wm * 64 + 32 * j,
                             n0 + wn * 128, lane, lds_rs + wm * 64 + 32 * j);
        } else
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int row = 2 * t + hi;
            const float4 v = *reinterpret_cast<const float4*>(stage + row * 128 + ((li ^ row) << 2));
            const int64_t m = m0 + wm * 64 + 32 * j + row;
            if (MODE == EPI_QKV_ROPE) {
                // every lane of the half-wave joins the head's shuffles
                qkv_rope_store(e, static_cast<bf16_t*>(C), ldc, M, N, m, n, v,
                               m < M ? lds_rs[m - m0] : 0.f);
                continue;
            }
            if (m >= M) continue;
            if (full_n || n + 3 < N) {
                epi_vec4_pre<MODE>(e, C, m * ldc + n, v, auxv[t], rsv[t]);
            } else {
                const float a[4] = {v.x, v.y, v.z, v.w};
                for (int q = 0; q < 4; ++q)
                    if (n + q < N) epi_store1<bf16_t>(e, C, ldc, m, n + q, a[q]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// out[m][n] = (accumulate ? out[m][n] : 0) + sum_s part[s][m][n], s in order;
// partials have row stride ldp
__global__ void k_splitk_reduce(const float* __restrict__ part, int splits, int M, int N,
                                int64_t ldp, float* __restrict__ out, int64_t ldc, int accumulate) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int64_t m = i / N, n = i % N;
    float s = accumulate ? out[m * ldc + n] : 0.f;
    for (int p = 0; p < splits; ++p) s += part[((int64_t)p * M + m) * ldp + n];
    out[m * ldc + n] = s;
}

// the same, four consecutive n per thread (N, ldc, ldp multiples of 4 and
// 16-byte aligned rows); each element is summed in the same order
__global__ void k_splitk_reduce4(const float* __restrict__ part, int splits, int M, int N4,
                                 int64_t ldp, float* __restrict__ out, int64_t ldc,
                                 int accumulate) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * N4) return;
    const int64_t m = i / N4, n = (i - m * N4) * 4;
    float4 acc = accumulate ? *reinterpret_cast<const float4*>(out + m * ldc + n)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int p = 0; p < splits; ++p) {
        const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)p * M + m) * ldp + n);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + m * ldc + n) = acc;
}

// k-split of a GEMM with few output tiles: the split count s that minimises
// the modelled time rounds(s) * (k per split + c), rounds(s) = workgroup
// waves of tiles * s over the 256 compute units and c ~ the fixed cost of a
// workgroup (prologue, epilogue) in k units.  Each split keeps >= 512 of k.
int choose_splits(int M, int N, int K) {
    const int64_t tiles = ceil_div(M, kTM) * ceil_div(N, kTN);
    constexpr int64_t kCUs = 256, kFixed = 384;
    int best = 1;
    int64_t best_cost = ceil_div(tiles, kCUs) * ((int64_t)K + kFixed);
    for (int s = 2; s <= 32; ++s) {
        const int64_t kper = ceil_div(ceil_div(K, s), kTK) * kTK;
        if (kper < 512 || ceil_div(K, kper) < s) break;
        const int64_t cost = ceil_div(tiles * s, kCUs) * (kper + kFixed);
        if (cost < best_cost) { best = s; best_cost = cost; }
    }
    return best;
}

template <bool AK, bool BK, int MODE>
hipError_t launch_mfma(int M, int N, int K, const bf16_t* A, int64_t lda, const bf16_t* B,
                       int64_t ldb, void* C, int64_t ldc, const EpiDev& e, int splits,
                       int64_t split_stride, hipStream_t s, const GemmBatch& bt) {
    int k_per = (int)ceil_div(K, splits);
    k_per = (int)ceil_div(k_per, kTK) * kTK;
    const int tiles = (int)(ceil_div(M, kTM) * ceil_div(N, kTN));
    auto kern = k_gemm_mfma<AK, BK, MODE>;
    // one workgroup per (split, tile) item and product of the batch
    hipLaunchKernelGGL(kern, dim3(tiles * splits, bt.count, 1), dim3(kThreads), 0, s, M, N, K,
                       k_per, splits, A, lda, B, ldb, C, ldc, e, split_stride, bt.sa, bt.sb,
                       bt.sc);
    return hipGetLastError();
}

}  // namespace

// partial sums of a k-split keep rows 16-byte aligned
int64_t splitk_ld(int N) { return (int64_t)ceil_div(N, 4) * 4; }

size_t gemm_splitk_bytes(int M, int N, int K) {
    const int splits = choose_splits(M, N, K);
    return splits > 1 ? (size_t)splits * M * splitk_ld(N) * sizeof(float) : 0;
}

template <>
hipError_t gemm<float>(int M, int N, int K, const float* A, int64_t lda, bool a_kmajor,
                       const float* B, int64_t ldb, bool b_kmajor, void* C, int64_t ldc,
                       const Epilogue& epi, float*, size_t, hipStream_t s,
                       const GemmBatch* batch) {
    const GemmBatch bt = batch ? *batch : GemmBatch{};
    if (M <= 0 || N <= 0 || bt.count <= 0) return hipSuccess;
    if (epi.mode == EPI_QKV_ROPE) return hipErrorInvalidValue;   // bf16 only
    if (bt.count > 1 && epi.rowscale) return hipErrorInvalidValue;
    const EpiDev e = make_epi(epi);
    dim3 grid((unsigned)ceil_div(N, kSB), (unsigned)ceil_div(M, kSB), (unsigned)bt.count);
    hipLaunchKernelGGL(k_gemm_simt<float>, grid, dim3(256), 0, s, M, N, K, A, lda,
                       a_kmajor ? 1 : 0, B, ldb, b_kmajor ? 1 : 0, C, ldc, e, bt.sa, bt.sb,
                       bt.sc);
    return hipGetLastError();
}

template <>
hipError_t gemm<bf16_t>(int M, int N, int K, const bf16_t* A, int64_t lda, bool a_kmajor,
                        const bf16_t* B, int64_t ldb, bool b_kmajor, void* C, int64_t ldc,
                        const Epilogue& epi, float* splitk_ws, size_t splitk_ws_bytes,
                        hipStream_t s, const GemmBatch* batch) {
    const GemmBatch bt = batch ? *batch : GemmBatch{};
    if (M <= 0 || N <= 0 || bt.count <= 0) return hipSuccess;
    if (bt.count > 1 && (epi.rowscale || epi.mode == EPI_QKV_ROPE)) return hipErrorInvalidValue;
    const EpiDev e = make_epi(epi);
    if (epi.mode == EPI_QKV_ROPE &&
        (epi.head_dim <= 0 || 128 % epi.head_dim || epi.head_dim % 8 || !epi.cos_t ||
         !epi.sin_t || !epi.rqk || epi.seq_len <= 0 || N != (epi.n_head + 2) * epi.head_dim))
        return hipErrorInvalidValue;
    int splits = 1;
    if (epi.mode == EPI_STORE_F32 && bt.count == 1) {
        splits = choose_splits(M, N, K);
        if (gemm_splitk_bytes(M, N, K) > splitk_ws_bytes || splitk_ws == nullptr) splits = 1;
    }
    // the epilogue's vector stores need 16-byte aligned rows
    if (ldc % 4) return hipErrorInvalidValue;
    void* out = C;
    int64_t ld_out = ldc, stride = 0;
    EpiDev ek = e;
    if (splits > 1) {
        out = splitk_ws;
        ld_out = splitk_ld(N);
        stride = (int64_t)M * ld_out;
        ek.accumulate = 0;
    }
    hipError_t err;
    if (a_kmajor && b_kmajor) {
        switch (epi.mode) {
            case EPI_STORE_F32:
                err = launch_mfma<true, true, EPI_STORE_F32>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_ROWSCALE:
                err = launch_mfma<true, true, EPI_ROWSCALE>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_ROWSCALE_RELU2:
                err = launch_mfma<true, true, EPI_ROWSCALE_RELU2>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_RESID:
                err = launch_mfma<true, true, EPI_RESID>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_RELU2_BWD:
                err = launch_mfma<true, true, EPI_RELU2_BWD>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_STORE_T:
                err = launch_mfma<true, true, EPI_STORE_T>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_QKV_ROPE:
                err = launch_mfma<true, true, EPI_QKV_ROPE>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            case EPI_AXPBY:
                err = launch_mfma<true, true, EPI_AXPBY>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
                break;
            default: return hipErrorInvalidValue;
        }
    } else if (!a_kmajor && !b_kmajor && epi.mode == EPI_STORE_F32) {
        err = launch_mfma<false, false, EPI_STORE_F32>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
    } else if (!a_kmajor && !b_kmajor && epi.mode == EPI_STORE_T) {
        // Gram matrix X^T X of a tall matrix (orthogonalisation)
        err = launch_mfma<false, false, EPI_STORE_T>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
    } else if (a_kmajor && !b_kmajor && epi.mode == EPI_AXPBY) {
        err = launch_mfma<true, false, EPI_AXPBY>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
    } else if (a_kmajor && !b_kmajor && epi.mode == EPI_STORE_F32) {
        err = launch_mfma<true, false, EPI_STORE_F32>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
    } else if (a_kmajor && !b_kmajor && epi.mode == EPI_STORE_T) {
        // data gradients dX = dY W straight from the [out][in] weight
        err = launch_mfma<true, false, EPI_STORE_T>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
    } else if (a_kmajor && !b_kmajor && epi.mode == EPI_RELU2_BWD) {
        err = launch_mfma<true, false, EPI_RELU2_BWD>(M, N, K, A, lda, B, ldb, out, ld_out, ek, splits, stride, s, bt);
    } else {
        return hipErrorInvalidValue;  // layout/epilogue pair the step never uses
    }
    if (err != hipSuccess || splits == 1) return err;
    const int64_t n = (int64_t)M * N;
    err = prof_cut("splitk_reduce", 0, 4.0 * n * (splits + 1 + e.accumulate));
    if (err != hipSuccess) return err;
    if (N % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0) {
        const int64_t n4 = n / 4;
        hipLaunchKernelGGL(k_splitk_reduce4, dim3((unsigned)ceil_div(n4, 256)), dim3(256), 0, s,
                           splitk_ws, splits, M, N / 4, splitk_ld(N), static_cast<float*>(C),
                           ldc, e.accumulate);
    } else {
        hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s,
                           splitk_ws, splits, M, N, splitk_ld(N), static_cast<float*>(C), ldc,
                           e.accumulate);
    }
    return hipGetLastError();
}

}  // namespace nc
