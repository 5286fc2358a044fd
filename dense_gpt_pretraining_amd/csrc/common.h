// Device-side helpers shared by every kernel of the library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nc {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

constexpr int kWave = 64;

// ------------------------------------------------------------ bf16 <-> fp32
__device__ __forceinline__ float bf2f(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// fp32 -> bf16, round to nearest, ties to even.  gfx950 converts a pair in
// one instruction (v_cvt_pk_bf16_f32), which is what these lower to.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// element traits: storage type T <-> fp32 arithmetic
template <typename T> struct Elt;
template <> struct Elt<float> {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
    static constexpr int kVec = 4;  // elements per 16-byte access
};
template <> struct Elt<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
    static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
    static constexpr int kVec = 8;
};

// 16-byte vector load/store of kVec elements converted to/from fp32
template <typename T>
__device__ __forceinline__ void ld_vec(const T* p, float* out);
template <>
__device__ __forceinline__ void ld_vec<float>(const float* p, float* out) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <>
__device__ __forceinline__ void ld_vec<bf16_t>(const bf16_t* p, float* out) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    out[0] = bf_lo(v.x); out[1] = bf_hi(v.x); out[2] = bf_lo(v.y); out[3] = bf_hi(v.y);
    out[4] = bf_lo(v.z); out[5] = bf_hi(v.z); out[6] = bf_lo(v.w); out[7] = bf_hi(v.w);
}
template <typename T>
__device__ __forceinline__ void st_vec(T* p, const float* in);
template <>
__device__ __forceinline__ void st_vec<float>(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
}
template <>
__device__ __forceinline__ void st_vec<bf16_t>(bf16_t* p, const float* in) {
    uint4 v;
    v.x = pack_bf2(in[0], in[1]); v.y = pack_bf2(in[2], in[3]);
    v.z = pack_bf2(in[4], in[5]); v.w = pack_bf2(in[6], in[7]);
    *reinterpret_cast<uint4*>(p) = v;
}

// ------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
// sum over groups of `width` consecutive lanes (width a power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// block-wide sum for blockDim.x a multiple of 64 (<= 1024); `red` holds
// blockDim.x/64 floats of shared memory.  Every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < nw; ++i) s += red[i];
    return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = -INFINITY;
    for (int i = 0; i < nw; ++i) s = fmaxf(s, red[i]);
    return s;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ HBM -> LDS copies
// A buffer resource over [base, base + 2 GiB) with no format conversion; the
// copies below go through it as MUBUF loads with the LDS bit, which the
// compiler tracks as plain vector-memory loads (its flat-instruction path
// would also flush the LDS counter at every later LDS dependency).
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
__device__ __forceinline__ buf_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF,
                                             0x00020000);
}
// the same over [base, base + bytes): copies from beyond it read zeros
__device__ __forceinline__ buf_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                             0x00020000);
}
// lane l copies `bytes` (4 or 16) from base + voff to LDS at lds + l * bytes;
// `lds` must be the same for every lane of the wave
template <int BYTES>
__device__ __forceinline__ void lds_copy(buf_rsrc_t r, int voff, void* lds) {
    auto* l = (__attribute__((address_space(3))) void*)lds;
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 4, voff, 0, 0, 0);
}

// ------------------------------------------------------------ matrix cores
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D = A B + C for 32x32 fp32 blocks with K = 16 bf16 per instruction.  Lane l
// supplies row (l & 31) of A and column (l & 31) of B, 8 consecutive k each
// (k = 8 (l >> 5) .. +7); lane l receives column (l & 31) of D, rows
// 8 (r / 4) + 4 (l >> 5) + (r % 4) for registers r = 0..15.
__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b,
                                           const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// transpose an 8 x 8 block of 16-bit values: in[r] holds row r (8 elements,
// 2 per dword); out[c] receives column c
__device__ __forceinline__ void transpose8x8(const uint4* in, uint4* out) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int d = c >> 1;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t x = reinterpret_cast<const uint32_t*>(&in[2 * p])[d];
            const uint32_t y = reinterpret_cast<const uint32_t*>(&in[2 * p + 1])[d];
            w[p] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
        }
        out[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

}  // namespace nc
