// Device-side helpers shared by the Talker MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmoe {

constexpr int kWave = 64;

// bf16 is stored as its 16-bit pattern; arithmetic happens in fp32.
typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    // round to nearest even (inputs are finite)
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
    __device__ static __forceinline__ double load64(const float* p, int64_t i) { return (double)p[i]; }
};
template <> struct Elem<bf16_t> {
    __device__ static __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ static __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
    __device__ static __forceinline__ double load64(const bf16_t* p, int64_t i) { return (double)bf16_to_f32(p[i]); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// "a ranks before b": larger value first, equal values by lower index.
template <typename V>
__device__ __forceinline__ bool ranks_before(V va, int ia, V vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Wave-wide best (value, index) under ranks_before; index -1 marks "none".
template <typename V>
__device__ __forceinline__ void wave_best(V& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        V ov = __shfl_xor(v, o, kWave);
        int oi = __shfl_xor(i, o, kWave);
        bool take = (oi >= 0) && (i < 0 || ranks_before(ov, oi, v, i));
        if (take) { v = ov; i = oi; }
    }
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Rounding-error bound of a dot product of length n evaluated in fp32 in any
// order (exact products for bf16 and fp32*fp32 -> fp32 FMA alike), relative to
// sum |a_i b_i|: (n + 8) * 2^-23 covers round-to-nearest with a factor-2 margin,
// so it also holds if the matrix cores truncate instead of rounding.
__device__ __forceinline__ float dot_error_scale(int n) { return (float)(n + 8) * 1.1920928955078125e-07f; }

}  // namespace tmoe
