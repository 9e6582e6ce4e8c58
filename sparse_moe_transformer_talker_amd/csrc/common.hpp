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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (the packed hardware conversion)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)pack_bf16x2(f, 0.0f); }

// SiLU(g) = g / (1 + e^-g), with the hardware reciprocal (1 ulp)
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

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

// --- DPP wave primitives (row_shr within 16-lane rows, then row_bcast15 /
// row_bcast31 across rows).  Disabled or out-of-row source lanes contribute the
// `old` operand, which is the identity of the operation.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xc, 0xf, false);
    return x;
}

// Maximum of a 64-bit key over the wave, returned to every lane (0 is the identity).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
#define TMOE_MAX_STEP(CTRL, ROWS)                                                                    \
    {                                                                                                \
        uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)key, CTRL, ROWS, 0xf, false);        \
        uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(key >> 32), CTRL, ROWS, 0xf, false); \
        uint64_t o = ((uint64_t)hi << 32) | lo;                                                      \
        key = o > key ? o : key;                                                                     \
    }
    TMOE_MAX_STEP(kDppRowShr1, 0xf)
    TMOE_MAX_STEP(kDppRowShr2, 0xf)
    TMOE_MAX_STEP(kDppRowShr4, 0xf)
    TMOE_MAX_STEP(kDppRowShr8, 0xf)
    TMOE_MAX_STEP(kDppRowBcast15, 0xa)
    TMOE_MAX_STEP(kDppRowBcast31, 0xc)
#undef TMOE_MAX_STEP
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)key, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(key >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Sum / maximum over the wave, returned to every lane (fixed order: deterministic).
__device__ __forceinline__ float wave_sum_dpp(float x) {
#define TMOE_SUM_STEP(CTRL, ROWS) \
    x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, ROWS, 0xf, false));
    TMOE_SUM_STEP(kDppRowShr1, 0xf)
    TMOE_SUM_STEP(kDppRowShr2, 0xf)
    TMOE_SUM_STEP(kDppRowShr4, 0xf)
    TMOE_SUM_STEP(kDppRowShr8, 0xf)
    TMOE_SUM_STEP(kDppRowBcast15, 0xa)
    TMOE_SUM_STEP(kDppRowBcast31, 0xc)
#undef TMOE_SUM_STEP
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 63));
}
// fp64 sum over the wave (DPP on the two halves), returned to every lane.
__device__ __forceinline__ double wave_sum_dpp_f64(double x) {
#define TMOE_SUM64_STEP(CTRL, ROWS)                                                         \
    {                                                                                       \
        const uint64_t u = (uint64_t)__double_as_longlong(x);                               \
        const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, ROWS, 0xf, false);         \
        const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, ROWS, 0xf, false); \
        x += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));                   \
    }
    TMOE_SUM64_STEP(kDppRowShr1, 0xf)
    TMOE_SUM64_STEP(kDppRowShr2, 0xf)
    TMOE_SUM64_STEP(kDppRowShr4, 0xf)
    TMOE_SUM64_STEP(kDppRowShr8, 0xf)
    TMOE_SUM64_STEP(kDppRowBcast15, 0xa)
    TMOE_SUM64_STEP(kDppRowBcast31, 0xc)
#undef TMOE_SUM64_STEP
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
    const uint32_t ninf = 0xFF800000u;
#define TMOE_FMAX_STEP(CTRL, ROWS) \
    x = fmaxf(x, __uint_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_uint(x), CTRL, ROWS, 0xf, false)));
    TMOE_FMAX_STEP(kDppRowShr1, 0xf)
    TMOE_FMAX_STEP(kDppRowShr2, 0xf)
    TMOE_FMAX_STEP(kDppRowShr4, 0xf)
    TMOE_FMAX_STEP(kDppRowShr8, 0xf)
    TMOE_FMAX_STEP(kDppRowBcast15, 0xa)
    TMOE_FMAX_STEP(kDppRowBcast31, 0xc)
#undef TMOE_FMAX_STEP
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 63));
}

// --- all-reduce inside each 16-lane row (DPP row_ror by 8, 4, 2, 1): every
// lane of a row gets the row's result.  Sums associate differently per lane
// (each lane's value is deterministic).
#define TMOE_ROR(V, N) __builtin_amdgcn_update_dpp(0u, (V), 0x120 + (N), 0xf, 0xf, false)
__device__ __forceinline__ uint64_t row_max_key(uint64_t key) {
#define TMOE_RMAX(N)                                                          \
    {                                                                         \
        const uint32_t lo = TMOE_ROR((uint32_t)key, N);                       \
        const uint32_t hi = TMOE_ROR((uint32_t)(key >> 32), N);               \
        const uint64_t o = ((uint64_t)hi << 32) | lo;                         \
        key = o > key ? o : key;                                              \
    }
    TMOE_RMAX(8)
    TMOE_RMAX(4)
    TMOE_RMAX(2)
    TMOE_RMAX(1)
#undef TMOE_RMAX
    return key;
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
    x = umax32(x, (uint32_t)TMOE_ROR(x, 8));
    x = umax32(x, (uint32_t)TMOE_ROR(x, 4));
    x = umax32(x, (uint32_t)TMOE_ROR(x, 2));
    x = umax32(x, (uint32_t)TMOE_ROR(x, 1));
    return x;
}
__device__ __forceinline__ float row_sum(float x) {
    x += __uint_as_float(TMOE_ROR(__float_as_uint(x), 8));
    x += __uint_as_float(TMOE_ROR(__float_as_uint(x), 4));
    x += __uint_as_float(TMOE_ROR(__float_as_uint(x), 2));
    x += __uint_as_float(TMOE_ROR(__float_as_uint(x), 1));
    return x;
}
__device__ __forceinline__ float row_max(float x) {
    x = fmaxf(x, __uint_as_float(TMOE_ROR(__float_as_uint(x), 8)));
    x = fmaxf(x, __uint_as_float(TMOE_ROR(__float_as_uint(x), 4)));
    x = fmaxf(x, __uint_as_float(TMOE_ROR(__float_as_uint(x), 2)));
    x = fmaxf(x, __uint_as_float(TMOE_ROR(__float_as_uint(x), 1)));
    return x;
}
// Order-preserving map of a double to uint64, and the row minimum built on it.
__device__ __forceinline__ uint64_t double_order_key(double d) {
    const uint64_t u = __double_as_longlong(d + 0.0);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double double_from_order_key(uint64_t k) {
    return __longlong_as_double((long long)((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}
__device__ __forceinline__ double row_min(double x) {
    return double_from_order_key(~row_max_key(~double_order_key(x)));
}

// Order-preserving map of a finite float to uint32 (larger float -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t float_order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Key ranking larger values first and, among equal values, lower indices first.
__device__ __forceinline__ uint64_t rank_key(float v, int idx) {
    return ((uint64_t)float_order_key(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int rank_key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

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
