// Combine of expert outputs, RMSNorm and row gather: HBM-bound, one block per
// token row, 16-byte accesses where the row length allows.
//
// combine ("3C · Talker MoE (20 lớp, 128 Experts Top-6)", openarchlab, §3):
//   y_t = SharedMLP(x_t) + sum_{i in S_t} w_{t,i} Expert_i(x_t)  (+ residual_t)
// summed in fp32 in a fixed order (shared, slots 0..k-1, residual), so results
// are bitwise reproducible.
// RMSNorm (lab helper on "Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz
// Architecture"; eps 1e-6 in the Qwen3-TTS module print on the horus-space page):
//   out = x / sqrt(mean(x^2) + eps) * gain
#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {

// Source row of term j of token t.  Slot mode (rows == nullptr): expert
// outputs are stored per token in `slots` consecutive rows, weighted here by
// w[t * k + j] (w null: weights already applied).  The shared-expert term of
// token t is shared + t * sstride (nullptr: no shared term).
template <typename T>
__global__ __launch_bounds__(128) void combine_kernel(const T* __restrict__ ysrc, const int32_t* __restrict__ rows,
                                                      const float* __restrict__ w, int k, int slots,
                                                      const T* __restrict__ shared, int64_t sstride,
                                                      const T* residual, T* y, int64_t Ttok, int H) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    const T* shared_row = shared ? shared + t * sstride : nullptr;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float acc = shared_row ? Elem<T>::load(shared_row, h) : 0.f;
        for (int j = 0; j < k; ++j) {
            if (rows) {
                const int64_t r = rows[t * k + j];
                acc += w[t * k + j] * Elem<T>::load(ysrc, r * H + h);
            } else {
                const float wj = w ? w[t * k + j] : 1.0f;
                acc += wj * Elem<T>::load(ysrc, (t * slots + j) * (int64_t)H + h);
            }
        }
        if (residual) acc += Elem<T>::load(residual, t * H + h);
        Elem<T>::store(y, t * H + h, acc);
    }
}

// bf16, H % 8 == 0: eight elements per thread with 16-byte loads.
__global__ __launch_bounds__(128) void combine_bf16x8_kernel(const bf16_t* __restrict__ ysrc,
                                                             const int32_t* __restrict__ rows,
                                                             const float* __restrict__ w, int k, int slots,
                                                             const bf16_t* __restrict__ shared, int64_t sstride,
                                                             const bf16_t* residual, bf16_t* y, int64_t Ttok, int H) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    const bf16_t* shared_row = shared ? shared + t * sstride : nullptr;
    for (int h = threadIdx.x * 8; h < H; h += blockDim.x * 8) {
        float acc[8];
        if (shared_row) {
            u32x4 v = *reinterpret_cast<const u32x4*>(shared_row + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __uint_as_float(v[q] << 16);
                acc[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        }
        for (int j = 0; j < k; ++j) {
            const bf16_t* src;
            float wj = 1.0f;
            if (rows) {
                src = ysrc + (int64_t)rows[t * k + j] * H;
                wj = w[t * k + j];
            } else {
                src = ysrc + (t * slots + j) * (int64_t)H;
                if (w) wj = w[t * k + j];
            }
            u32x4 v = *reinterpret_cast<const u32x4*>(src + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += wj * __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += wj * __uint_as_float(v[q] & 0xFFFF0000u);
            }
        }
        if (residual) {
            u32x4 v = *reinterpret_cast<const u32x4*>(residual + t * H + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
            }
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *reinterpret_cast<u32x4*>(y + t * H + h) = o;
    }
}

// RMSNorm of bf16 rows (H % 8 == 0, H <= 1024 NCH): 128 threads, thread i
// holds elements 8 (i + 128 c) .. + 7 of chunk c.  Each thread sums its squares
// in element order, the two waves reduce by DPP and the block adds wave 0's
// total and wave 1's: one fixed order, shared with the fused combine below, so
// the stack's fused layer end and a separate moe_rmsnorm call give the same
// bits.  gain may be null (1.0).
template <int NCH>
__device__ __forceinline__ float rms_inv_bf16x8(const u32x4 (&v)[NCH], bool (&ok)[NCH], int H, float eps) {
    __shared__ float part[2];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (ok[c])
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = __uint_as_float(v[c][q] << 16), hi = __uint_as_float(v[c][q] & 0xFFFF0000u);
                ss = fmaf(lo, lo, ss);
                ss = fmaf(hi, hi, ss);
            }
    ss = wave_sum_dpp(ss);
    if (lane_id() == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float ms = (part[0] + part[1]) / (float)H;
    return 1.0f / sqrtf(ms + eps);
}
// The gains of this thread's 8-element chunks (1.0 where gain is null or the
// chunk lies past H), requested at a kernel's start so that they arrive with
// its row data rather than after the sum-of-squares barrier.
template <int NCH>
__device__ __forceinline__ void load_gain_bf16x8(const float* __restrict__ gain, int H, float (&g)[NCH][8]) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (threadIdx.x + 128 * c) * 8;
        if (gain && h < H) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(gain + h);
            const f32x4 b = *reinterpret_cast<const f32x4*>(gain + h + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g[c][i] = a[i];
                g[c][4 + i] = b[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) g[c][i] = 1.0f;
        }
    }
}
template <int NCH>
__device__ __forceinline__ void rms_store_bf16x8(const u32x4 (&v)[NCH], bool (&ok)[NCH], float inv,
                                                 const float (&g)[NCH][8], bf16_t* out_row) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (!ok[c]) continue;
        const int h = (threadIdx.x + 128 * c) * 8;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(__uint_as_float(v[c][q] << 16) * inv * g[c][2 * q],
                               __uint_as_float(v[c][q] & 0xFFFF0000u) * inv * g[c][2 * q + 1]);
        *reinterpret_cast<u32x4*>(out_row + h) = o;
    }
}
template <int NCH>
__global__ __launch_bounds__(128) void rmsnorm_bf16x8_kernel(const bf16_t* x, const float* __restrict__ gain,
                                                             float eps, int64_t Ttok, int H, bf16_t* out) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    float gv[NCH][8];
    load_gain_bf16x8<NCH>(gain, H, gv);
    u32x4 v[NCH];
    bool ok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (threadIdx.x + 128 * c) * 8;
        ok[c] = h < H;
        v[c] = ok[c] ? *reinterpret_cast<const u32x4*>(x + t * H + h) : u32x4{0, 0, 0, 0};
    }
    const float inv = rms_inv_bf16x8<NCH>(v, ok, H, eps);
    rms_store_bf16x8<NCH>(v, ok, inv, gv, out + t * H);
}

// The end of a stacked layer: the combine above (shared, slots 0..k-1,
// residual, rounded to bf16 and stored as y), then the next layer's pre-norm of
// that stored row (the lab's [3C] step normalises the layer input; the final
// norm before codec_head likewise), written to norm_out.
template <int NCH>
__global__ __launch_bounds__(128) void combine_norm_bf16x8_kernel(const bf16_t* __restrict__ ysrc,
                                                                  const float* __restrict__ w, int k, int slots,
                                                                  const bf16_t* __restrict__ shared, int64_t sstride,
                                                                  const bf16_t* residual, bf16_t* y, int64_t Ttok,
                                                                  int H, const float* __restrict__ gain, float eps,
                                                                  bf16_t* norm_out) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    float gv[NCH][8];
    load_gain_bf16x8<NCH>(norm_out ? gain : nullptr, H, gv);
    const bf16_t* shared_row = shared ? shared + t * sstride : nullptr;
    u32x4 yv[NCH];
    bool ok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (threadIdx.x + 128 * c) * 8;
        ok[c] = h < H;
        yv[c] = u32x4{0, 0, 0, 0};
        if (!ok[c]) continue;
        float acc[8];
        if (shared_row) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(shared_row + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __uint_as_float(v[q] << 16);
                acc[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        }
        for (int j = 0; j < k; ++j) {
            const float wj = w ? w[t * k + j] : 1.0f;
            const u32x4 v = *reinterpret_cast<const u32x4*>(ysrc + (t * slots + j) * (int64_t)H + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += wj * __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += wj * __uint_as_float(v[q] & 0xFFFF0000u);
            }
        }
        if (residual) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(residual + t * H + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) yv[c][q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *reinterpret_cast<u32x4*>(y + t * H + h) = yv[c];
    }
    const float inv = rms_inv_bf16x8<NCH>(yv, ok, H, eps);
    rms_store_bf16x8<NCH>(yv, ok, inv, gv, norm_out + t * H);
}

// Partial-row combine of the decode layer.  Token t's partial rows are
// part[t][0 .. NP) ([T, NP, H] bf16): rows j S .. j S + S - 1 add up to the
// output of its j-th routed expert, rows k S .. NP - 1 to the shared expert's.
//   y_t = sum_s part[t][k S + s] + sum_j w[t, j] (sum_s part[t][j S + s]) (+ residual_t)
// summed in fp32 in exactly this order (bitwise reproducible), stored bf16;
// norm_out (nullable) then receives RMSNorm(y_t) * gain with the same
// reduction as rmsnorm_bf16x8_kernel, so the fused layer end and a separate
// moe_rmsnorm call give the same bits.
template <int NCH, int K, int S, int SSH>
__global__ __launch_bounds__(128) void combine_partials_kernel(const bf16_t* __restrict__ part, int S_rt, int SSH_rt,
                                                               int k_rt, const float* __restrict__ w,
                                                               const bf16_t* residual, bf16_t* y, int64_t Ttok, int H,
                                                               const float* __restrict__ gain, float eps,
                                                               bf16_t* norm_out) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    float gv[NCH][8];
    load_gain_bf16x8<NCH>(norm_out ? gain : nullptr, H, gv);
    // K > 0: the sizes are compile-time, and every row of the token is loaded
    // before the first add (one memory round trip)
    const int k = K > 0 ? K : k_rt, s_n = K > 0 ? S : S_rt, ssh_n = K > 0 ? SSH : SSH_rt;
    const int NP = k * s_n + ssh_n;
    const bf16_t* prow = part + t * NP * (int64_t)H;
    u32x4 yv[NCH];
    bool ok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (threadIdx.x + 128 * c) * 8;
        ok[c] = h < H;
        yv[c] = u32x4{0, 0, 0, 0};
        if (!ok[c]) continue;
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        auto add = [&](float (&dst)[8], const u32x4& v) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                dst[2 * q] += __uint_as_float(v[q] << 16);
                dst[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
            }
        };
        auto row = [&](int r) { return *reinterpret_cast<const u32x4*>(prow + (int64_t)r * H + h); };
        if (K > 0) {
            constexpr int NPc = K * S + SSH;
            u32x4 v[NPc > 0 ? NPc : 1];
#pragma unroll
            for (int r = 0; r < NPc; ++r) v[r] = row(r);
            float wj[K > 0 ? K : 1];
#pragma unroll
            for (int j = 0; j < K; ++j) wj[j] = w[t * K + j];
#pragma unroll
            for (int r = 0; r < SSH; ++r) add(acc, v[K * S + r]);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                float e8[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e8[q] = 0.f;
#pragma unroll
                for (int r = 0; r < S; ++r) add(e8, v[j * S + r]);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj[j], e8[q], acc[q]);
            }
        } else {
            for (int r = 0; r < ssh_n; ++r) add(acc, row(k * s_n + r));
            for (int j = 0; j < k; ++j) {
                float e8[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e8[q] = 0.f;
                for (int r = 0; r < s_n; ++r) add(e8, row(j * s_n + r));
                const float wj = w[t * k + j];
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, e8[q], acc[q]);
            }
        }
        if (residual) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(residual + t * H + h);
            add(acc, v);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) yv[c][q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *reinterpret_cast<u32x4*>(y + t * H + h) = yv[c];
    }
    if (!norm_out) return;
    const float inv = rms_inv_bf16x8<NCH>(yv, ok, H, eps);
    rms_store_bf16x8<NCH>(yv, ok, inv, gv, norm_out + t * H);
}

hipError_t launch_combine_partials(const void* part, int S, int SSH, int k, const float* w, const void* residual,
                                   void* y, int64_t Ttok, int H, const float* gain, float eps, void* norm_out,
                                   hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    if (H % 8 != 0 || H > 1024) return hipErrorInvalidValue;
#define TMOE_CP(K_, S_, SSH_)                                                                               \
    combine_partials_kernel<1, K_, S_, SSH_><<<(unsigned)Ttok, 128, 0, st>>>(                                  \
        (const bf16_t*)part, S, SSH, k, w, (const bf16_t*)residual, (bf16_t*)y, Ttok, H, gain, eps,           \
        (bf16_t*)norm_out)
    if (k == 6 && S == 6 && SSH == 1) TMOE_CP(6, 6, 1);  // the Talker layer
    else if (k == 6 && S == 6 && SSH == 0) TMOE_CP(6, 6, 0);
    else TMOE_CP(0, 0, 0);
#undef TMOE_CP
    return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, const float* __restrict__ gain, float eps,
                                                      int64_t Ttok, int H, T* out) {
    __shared__ float part[4];
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    const T* xr = x + t * H;
    float ss = 0.f;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float v = Elem<T>::load(xr, h);
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane_id() == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float ms = (part[0] + part[1] + part[2] + part[3]) / (float)H;
    const float inv = 1.0f / sqrtf(ms + eps);
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float v = Elem<T>::load(xr, h);
        Elem<T>::store(out, t * H + h, v * inv * (gain ? gain[h] : 1.0f));
    }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T* __restrict__ x, const int32_t* __restrict__ rows,
                                                          int64_t n, int H, T* __restrict__ out) {
    const int64_t r = blockIdx.x;
    if (r >= n) return;
    const T* src = x + (int64_t)rows[r] * H;
    for (int h = threadIdx.x; h < H; h += blockDim.x) out[r * H + h] = src[h];
}

hipError_t launch_combine(int dtype, const void* ysrc, const int32_t* rows, const float* w, int k, int slots,
                          const void* shared, int64_t sstride, const void* residual, void* y, int64_t Ttok, int H,
                          hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    if (dtype == kBF16 && H % 8 == 0)
        combine_bf16x8_kernel<<<(unsigned)Ttok, 128, 0, st>>>((const bf16_t*)ysrc, rows, w, k, slots,
                                                               (const bf16_t*)shared, sstride,
                                                               (const bf16_t*)residual, (bf16_t*)y, Ttok, H);
    else if (dtype == kBF16)
        combine_kernel<bf16_t><<<(unsigned)Ttok, 128, 0, st>>>((const bf16_t*)ysrc, rows, w, k, slots,
                                                                (const bf16_t*)shared, sstride,
                                                                (const bf16_t*)residual, (bf16_t*)y, Ttok, H);
    else
        combine_kernel<float><<<(unsigned)Ttok, 128, 0, st>>>((const float*)ysrc, rows, w, k, slots,
                                                               (const float*)shared, sstride,
                                                               (const float*)residual, (float*)y, Ttok, H);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int32_t v, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, v, n);
    return hipGetLastError();
}

// Chunks of 1024 elements per row for the bf16 row kernels (0: they do not apply).
static int bf16x8_chunks(int dtype, int H) {
    if (dtype != kBF16 || H % 8 != 0 || H > 4 * 1024) return 0;
    return (H + 1023) / 1024;
}

// A frame's Talker input x = bf16(a + b) ("Bài Lab tổng hợp", step [3B]: the
// previous frame's audio embedding plus the frame's text condition), stored,
// then its RMSNorm: the same arithmetic as rmsnorm_bf16x8_kernel on the stored
// row, so the result equals moe_rmsnorm of x bit for bit.
template <int NCH>
__global__ __launch_bounds__(128) void add_rmsnorm_bf16x8_kernel(const bf16_t* __restrict__ a,
                                                                 const bf16_t* __restrict__ b, bf16_t* x,
                                                                 const float* __restrict__ gain, float eps,
                                                                 int64_t Ttok, int H, bf16_t* out) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    float gv[NCH][8];
    load_gain_bf16x8<NCH>(gain, H, gv);
    u32x4 v[NCH];
    bool ok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (threadIdx.x + 128 * c) * 8;
        ok[c] = h < H;
        v[c] = u32x4{0, 0, 0, 0};
        if (!ok[c]) continue;
        const u32x4 va = *reinterpret_cast<const u32x4*>(a + t * H + h);
        const u32x4 vb = *reinterpret_cast<const u32x4*>(b + t * H + h);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[c][q] = pack_bf16x2(__uint_as_float(va[q] << 16) + __uint_as_float(vb[q] << 16),
                                  __uint_as_float(va[q] & 0xFFFF0000u) + __uint_as_float(vb[q] & 0xFFFF0000u));
        *reinterpret_cast<u32x4*>(x + t * H + h) = v[c];
    }
    const float inv = rms_inv_bf16x8<NCH>(v, ok, H, eps);
    rms_store_bf16x8<NCH>(v, ok, inv, gv, out + t * H);
}

hipError_t launch_add_rmsnorm(const void* a, const void* b, void* x, const float* gain, float eps, int64_t Ttok,
                              int H, void* out, hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    const int nch = bf16x8_chunks(kBF16, H);
#define TMOE_ARMS(N)                                                                                            \
    add_rmsnorm_bf16x8_kernel<N><<<(unsigned)Ttok, 128, 0, st>>>((const bf16_t*)a, (const bf16_t*)b, (bf16_t*)x, \
                                                                 gain, eps, Ttok, H, (bf16_t*)out)
    if (nch == 1) TMOE_ARMS(1);
    else if (nch == 2) TMOE_ARMS(2);
    else if (nch == 3) TMOE_ARMS(3);
    else if (nch == 4) TMOE_ARMS(4);
    else return hipErrorInvalidValue;
#undef TMOE_ARMS
    return hipGetLastError();
}

// Row t of a code embedding table, gathered (a code outside [0, rows) gives a
// zero row) and stored to x, then its RMSNorm times the gain stored to out:
// a table gather followed by rmsnorm_bf16x8_kernel, in one launch and with the same bits.
template <int NCH>
__global__ __launch_bounds__(128) void embed_norm_bf16x8_kernel(const bf16_t* __restrict__ table, int rows,
                                                                const int32_t* __restrict__ idx, bf16_t* x,
                                                                const float* __restrict__ gain, float eps,
                                                                int64_t Ttok, int H, bf16_t* out) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    float gv[NCH][8];
    load_gain_bf16x8<NCH>(gain, H, gv);
    const int r = idx[t];
    const bool in = r >= 0 && r < rows;
    u32x4 v[NCH];
    bool ok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int h = (threadIdx.x + 128 * c) * 8;
        ok[c] = h < H;
        v[c] = u32x4{0, 0, 0, 0};
        if (!ok[c]) continue;
        if (in) v[c] = *reinterpret_cast<const u32x4*>(table + (int64_t)r * H + h);
        *reinterpret_cast<u32x4*>(x + t * H + h) = v[c];
    }
    const float inv = rms_inv_bf16x8<NCH>(v, ok, H, eps);
    rms_store_bf16x8<NCH>(v, ok, inv, gv, out + t * H);
}

hipError_t launch_embed_norm(const void* table, int rows, const int32_t* idx, void* x, const float* gain, float eps,
                             int64_t Ttok, int H, void* out, hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    const int nch = bf16x8_chunks(kBF16, H);
#define TMOE_EN(N)                                                                                       \
    embed_norm_bf16x8_kernel<N><<<(unsigned)Ttok, 128, 0, st>>>((const bf16_t*)table, rows, idx,        \
                                                                (bf16_t*)x, gain, eps, Ttok, H, (bf16_t*)out)
    if (nch == 1) TMOE_EN(1);
    else if (nch == 2) TMOE_EN(2);
    else if (nch == 3) TMOE_EN(3);
    else if (nch == 4) TMOE_EN(4);
    else return hipErrorInvalidValue;
#undef TMOE_EN
    return hipGetLastError();
}

// The end of a frame for stream t ("Bài Lab tổng hợp", step [3B]): the mean of
// its Q code embeddings (c_0 from c0_table [V0, H], c_j from tables[j - 1]
// [K, H]; a code outside its table is a zero row), summed in fp32 in code
// order, divided by Q and rounded to bf16, becomes the next frame's audio
// embedding; the stream's three TM-RoPE indices and its cache length advance
// by one.
__global__ __launch_bounds__(128) void frame_advance_kernel(const int32_t* __restrict__ codes, int Q,
                                                            const bf16_t* __restrict__ c0_table, int V0,
                                                            const bf16_t* __restrict__ tables, int K, int64_t Ttok,
                                                            int H, bf16_t* __restrict__ prev, int32_t* pos,
                                                            int32_t* len) {
    const int64_t t = blockIdx.x;
    if (t >= Ttok) return;
    for (int h = threadIdx.x * 8; h < H; h += 128 * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j = 0; j < Q; ++j) {
            const int c = codes[(int64_t)j * Ttok + t];
            const int rows = j == 0 ? V0 : K;
            if (c < 0 || c >= rows) continue;
            const bf16_t* row = j == 0 ? c0_table + (int64_t)c * H : tables + ((int64_t)(j - 1) * K + c) * H;
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
            }
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q] / (float)Q, acc[2 * q + 1] / (float)Q);
        *reinterpret_cast<u32x4*>(prev + t * H + h) = o;
    }
    if (threadIdx.x < 3) pos[t * 3 + threadIdx.x] += 1;
    if (threadIdx.x == 3) len[t] += 1;
}

hipError_t launch_frame_advance(const int32_t* codes, int Q, const void* c0_table, int V0, const void* tables, int K,
                                int64_t Ttok, int H, void* prev, int32_t* pos, int32_t* len, hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    if (H % 8 != 0 || Q < 1) return hipErrorInvalidValue;
    frame_advance_kernel<<<(unsigned)Ttok, 128, 0, st>>>(codes, Q, (const bf16_t*)c0_table, V0,
                                                         (const bf16_t*)tables, K, Ttok, H, (bf16_t*)prev, pos, len);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void* x, const float* gain, float eps, int64_t Ttok, int H, void* out,
                          hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    const int nch = bf16x8_chunks(dtype, H);
#define TMOE_RMS(N) \
    rmsnorm_bf16x8_kernel<N><<<(unsigned)Ttok, 128, 0, st>>>((const bf16_t*)x, gain, eps, Ttok, H, (bf16_t*)out)
    if (nch == 1) TMOE_RMS(1);
    else if (nch == 2) TMOE_RMS(2);
    else if (nch == 3) TMOE_RMS(3);
    else if (nch == 4) TMOE_RMS(4);
#undef TMOE_RMS
    else if (dtype == kBF16)
        rmsnorm_kernel<bf16_t><<<(unsigned)Ttok, 256, 0, st>>>((const bf16_t*)x, gain, eps, Ttok, H, (bf16_t*)out);
    else
        rmsnorm_kernel<float><<<(unsigned)Ttok, 256, 0, st>>>((const float*)x, gain, eps, Ttok, H, (float*)out);
    return hipGetLastError();
}

hipError_t launch_combine_norm(int dtype, const void* ysrc, const float* w, int k, int slots, const void* shared,
                               int64_t sstride, const void* residual, void* y, int64_t Ttok, int H, const float* gain,
                               float eps, void* norm_out, hipStream_t st) {
    if (Ttok <= 0) return hipSuccess;
    const int nch = bf16x8_chunks(dtype, H);
    if (nch == 0) {  // the two steps apart, with the same kernels as the separate calls
        hipError_t e = launch_combine(dtype, ysrc, nullptr, w, k, slots, shared, sstride, residual, y, Ttok, H, st);
        if (e != hipSuccess) return e;
        return launch_rmsnorm(dtype, y, gain, eps, Ttok, H, norm_out, st);
    }
#define TMOE_CN(N)                                                                                              \
    combine_norm_bf16x8_kernel<N><<<(unsigned)Ttok, 128, 0, st>>>((const bf16_t*)ysrc, w, k, slots,            \
                                                                 (const bf16_t*)shared, sstride,               \
                                                                 (const bf16_t*)residual, (bf16_t*)y, Ttok, H, \
                                                                 gain, eps, (bf16_t*)norm_out)
    if (nch == 1) TMOE_CN(1);
    else if (nch == 2) TMOE_CN(2);
    else if (nch == 3) TMOE_CN(3);
    else TMOE_CN(4);
#undef TMOE_CN
    return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* rows, int64_t n, int H, void* out,
                              hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (dtype == kBF16)
        gather_rows_kernel<bf16_t><<<(unsigned)n, 256, 0, st>>>((const bf16_t*)x, rows, n, H, (bf16_t*)out);
    else
        gather_rows_kernel<float><<<(unsigned)n, 256, 0, st>>>((const float*)x, rows, n, H, (float*)out);
    return hipGetLastError();
}

}  // namespace tmoe
