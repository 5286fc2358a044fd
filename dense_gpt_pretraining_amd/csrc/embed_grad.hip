// Embedding gradient: dwte[v] = sum of de[t] over positions t with tok[t] == v.
//
// Token ids follow a heavy-headed law (the most frequent id holds ~14% of a
// batch), so float atomics on a row would serialise and make the sum order
// depend on timing.  Instead the positions are sorted by id with a stable LSD
// radix sort (8-bit digits), the sorted sequence is cut into pieces of at most
// 64 positions that never straddle two ids, each piece is summed by one
// workgroup, and ids spanning several pieces combine their piece sums in
// order.  Every sum is taken in position order, so the result is bitwise
// reproducible.
#include "kernels.h"

namespace nc {

namespace {

constexpr int kChunk = 256;     // elements per radix chunk (= threads per block)
constexpr int kPiece = 64;      // max rows per piece
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kChunk) void k_iota_keys(const int32_t* __restrict__ tok, int N,
                                                      int32_t* __restrict__ keys,
                                                      int32_t* __restrict__ vals) {
    const int i = blockIdx.x * kChunk + threadIdx.x;
    if (i < N) { keys[i] = tok[i]; vals[i] = i; }
}

// hist[d * G + chunk] = number of elements of the chunk with digit d
__global__ __launch_bounds__(kChunk) void k_radix_hist(const int32_t* __restrict__ keys, int N,
                                                       int shift, int G,
                                                       int32_t* __restrict__ hist) {
    __shared__ int32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int i = blockIdx.x * kChunk + threadIdx.x;
    if (i < N) atomicAdd(&h[(keys[i] >> shift) & 255], 1);
    __syncthreads();
    hist[(int64_t)threadIdx.x * G + blockIdx.x] = h[threadIdx.x];
}

// in-place exclusive scan of n int32 by one block; writes the total to *total.
// The array is taken in tiles of kScanThreads x kScanPer elements: each thread
// requests its kScanPer consecutive elements at once (four 16-byte loads when
// they lie inside the array and the array is 16-byte aligned), scans them in
// registers, and the per-thread sums are scanned across the wave (shuffles)
// and across the block's waves (one LDS slot per wave).  Integer sums: the
// result does not depend on the order of the additions.
constexpr int kScanPer = 16;
__global__ __launch_bounds__(kScanThreads) void k_exclusive_scan(int32_t* __restrict__ a, int64_t n,
                                                                 int32_t* __restrict__ total) {
    constexpr int kWaves = kScanThreads / 64;
    __shared__ int32_t wsum[kWaves];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(a) & 15) == 0;
    int32_t carry = 0;   // sum of every earlier tile
    for (int64_t base = 0; base < n; base += (int64_t)kScanThreads * kScanPer) {
        const int64_t i0 = base + (int64_t)t * kScanPer;
        const bool whole = vec_ok && i0 + kScanPer <= n;
        int32_t v[kScanPer];
        if (whole) {
#pragma unroll
            for (int q = 0; q < kScanPer / 4; ++q) {
                const int4 x = reinterpret_cast<const int4*>(a + i0)[q];
                v[4 * q] = x.x;
                v[4 * q + 1] = x.y;
                v[4 * q + 2] = x.z;
                v[4 * q + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kScanPer; ++k) v[k] = i0 + k < n ? a[i0 + k] : 0;
        }
        // exclusive prefix inside the thread; run = the thread's sum
        int32_t run = 0;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            const int32_t x = v[k];
            v[k] = run;
            run += x;
        }
        // inclusive scan of the thread sums across the wave
        int32_t inc = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(inc, off, 64);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wsum[w] = inc;
        __syncthreads();
        int32_t before = 0, tile_sum = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            const int32_t x = wsum[k];
            before += k < w ? x : 0;
            tile_sum += x;
        }
        const int32_t off = carry + before + inc - run;
        if (whole) {
#pragma unroll
            for (int q = 0; q < kScanPer / 4; ++q)
                reinterpret_cast<int4*>(a + i0)[q] =
                    make_int4(v[4 * q] + off, v[4 * q + 1] + off, v[4 * q + 2] + off,
                              v[4 * q + 3] + off);
        } else {
#pragma unroll
            for (int k = 0; k < kScanPer; ++k)
                if (i0 + k < n) a[i0 + k] = v[k] + off;
        }
        carry += tile_sum;
        __syncthreads();   // every wave has read wsum before the next tile writes it
    }
    if (t == 0 && total) *total = carry;
}

// stable scatter: rank of an element among the earlier elements of its chunk
// with the same digit, plus the scanned offset of (digit, chunk)
__global__ __launch_bounds__(kChunk) void k_radix_scatter(
    const int32_t* __restrict__ keys, const int32_t* __restrict__ vals, int N, int shift, int G,
    const int32_t* __restrict__ offs, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ vals_out) {
    __shared__ int32_t dig[kChunk];
    const int i = blockIdx.x * kChunk + threadIdx.x;
    const bool valid = i < N;
    const int32_t key = valid ? keys[i] : 0;
    const int d = valid ? ((key >> shift) & 255) : -1;
    dig[threadIdx.x] = d;
    __syncthreads();
    if (!valid) return;
    int rank = 0;
    for (int j = 0; j < (int)threadIdx.x; ++j) rank += (dig[j] == d);
    const int32_t dst = offs[(int64_t)d * G + blockIdx.x] + rank;
    keys_out[dst] = key;
    vals_out[dst] = vals[i];
}

// flag[i] = 1 where a piece starts: a new id or a multiple of kPiece
__global__ void k_piece_flags(const int32_t* __restrict__ keys, int N, int32_t* __restrict__ flag) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) flag[i] = (i % kPiece == 0 || keys[i] != keys[i - 1]) ? 1 : 0;
}

// after the exclusive scan, flag[i] holds the number of piece starts before i;
// record the start index of every piece
__global__ void k_piece_starts(const int32_t* __restrict__ keys, int N,
                               const int32_t* __restrict__ scanned, int32_t* __restrict__ start) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N && (i % kPiece == 0 || keys[i] != keys[i - 1])) start[scanned[i]] = i;
}

// one block per piece: sum its rows in order; a piece that is a whole id
// segment writes dwte directly, otherwise its sum goes to part[piece]
__global__ __launch_bounds__(256) void k_piece_sum(
    const float* __restrict__ de, const int32_t* __restrict__ keys,
    const int32_t* __restrict__ vals, int N, int D, const int32_t* __restrict__ start,
    const int32_t* __restrict__ n_pieces, float* __restrict__ part, float* __restrict__ dwte) {
    const int p = blockIdx.x;
    if (p >= *n_pieces) return;
    const int b = start[p];
    const int e = (p + 1 < *n_pieces) ? start[p + 1] : N;
    const int key = keys[b];
    const bool whole = (b == 0 || keys[b - 1] != key) && (e == N || keys[e] != key);
    float* dst = whole ? dwte + (int64_t)key * D : part + (int64_t)p * D;
    for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i = b; i < e; ++i) {
            const float4 v = *reinterpret_cast<const float4*>(de + (int64_t)vals[i] * D + c);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *reinterpret_cast<float4*>(dst + c) = acc;
    }
}

// one block per piece: the first piece of an id that spans several pieces
// adds up the piece sums of that id in order
__global__ __launch_bounds__(256) void k_piece_combine(
    const int32_t* __restrict__ keys, int N, int D, const int32_t* __restrict__ start,
    const int32_t* __restrict__ n_pieces, const float* __restrict__ part,
    float* __restrict__ dwte) {
    const int p = blockIdx.x;
    const int np = *n_pieces;
    if (p >= np) return;
    const int b = start[p];
    const int e = (p + 1 < np) ? start[p + 1] : N;
    const int key = keys[b];
    const bool first = (b == 0 || keys[b - 1] != key);
    const bool spans = (e < N && keys[e] == key);
    if (!first || !spans) return;
    int q_end = p + 1;
    while (q_end < np && keys[start[q_end]] == key) ++q_end;
    for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q = p; q < q_end; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)q * D + c);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *reinterpret_cast<float4*>(dwte + (int64_t)key * D + c) = acc;
    }
}

int radix_passes(int V) {
    int bits = 0;
    while ((1LL << bits) < (int64_t)V) ++bits;
    const int p = (bits + 7) / 8;
    return p > 0 ? p : 1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t embed_grad_ws_bytes(int N, int D, int V) {
    (void)V;
    const int G = (int)ceil_div(N, kChunk);
    const int64_t max_pieces = (int64_t)N + ceil_div(N, kPiece) + 1;
    size_t b = 0;
    b += 4 * align256((size_t)N * 4);               // keys a/b, vals a/b
    b += align256((size_t)256 * G * 4);             // histogram
    b += 2 * align256((size_t)N * 4);               // flags, starts
    b += align256(16);                              // piece count
    b += align256((size_t)max_pieces * D * 4);      // piece sums
    return b;
}

hipError_t embed_grad(const float* de, const int32_t* tok, int N, int D, int V, float* dwte,
                      void* ws, size_t ws_bytes, hipStream_t s) {
    if (ws_bytes < embed_grad_ws_bytes(N, D, V)) return hipErrorInvalidValue;
    const int G = (int)ceil_div(N, kChunk);
    char* p = static_cast<char*>(ws);
    auto take = [&](size_t bytes) { char* r = p; p += align256(bytes); return r; };
    int32_t* ka = reinterpret_cast<int32_t*>(take((size_t)N * 4));
    int32_t* kb = reinterpret_cast<int32_t*>(take((size_t)N * 4));
    int32_t* va = reinterpret_cast<int32_t*>(take((size_t)N * 4));
    int32_t* vb = reinterpret_cast<int32_t*>(take((size_t)N * 4));
    int32_t* hist = reinterpret_cast<int32_t*>(take((size_t)256 * G * 4));
    int32_t* flags = reinterpret_cast<int32_t*>(take((size_t)N * 4));
    int32_t* starts = reinterpret_cast<int32_t*>(take((size_t)N * 4));
    int32_t* npieces = reinterpret_cast<int32_t*>(take(16));
    float* part = reinterpret_cast<float*>(take(0));

    hipError_t e = zero_elems<float>(dwte, (int64_t)V * D, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_iota_keys, dim3(G), dim3(kChunk), 0, s, tok, N, ka, va);
    const int passes = radix_passes(V);
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = 8 * pass;
        hipLaunchKernelGGL(k_radix_hist, dim3(G), dim3(kChunk), 0, s, ka, N, shift, G, hist);
        hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(kScanThreads), 0, s, hist,
                           (int64_t)256 * G, (int32_t*)nullptr);
        hipLaunchKernelGGL(k_radix_scatter, dim3(G), dim3(kChunk), 0, s, ka, va, N, shift, G, hist,
                           kb, vb);
        std::swap(ka, kb);
        std::swap(va, vb);
    }
    const unsigned nb = (unsigned)ceil_div(N, 256);
    hipLaunchKernelGGL(k_piece_flags, dim3(nb), dim3(256), 0, s, ka, N, flags);
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(kScanThreads), 0, s, flags, (int64_t)N,
                       npieces);
    hipLaunchKernelGGL(k_piece_starts, dim3(nb), dim3(256), 0, s, ka, N, flags, starts);
    const unsigned max_pieces = (unsigned)(N + ceil_div(N, kPiece));
    hipLaunchKernelGGL(k_piece_sum, dim3(max_pieces), dim3(256), 0, s, de, ka, va, N, D, starts,
                       npieces, part, dwte);
    hipLaunchKernelGGL(k_piece_combine, dim3(max_pieces), dim3(256), 0, s, ka, N, D, starts,
                       npieces, part, dwte);
    return hipGetLastError();
}

}  // namespace nc
