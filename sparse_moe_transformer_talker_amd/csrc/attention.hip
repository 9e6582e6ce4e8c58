// Decode-time attention of the Talker: per-head q/k RMSNorm, interleaved
// TM-RoPE, KV-cache append and grouped-query attention over each stream's cache.
//   "3C · Talker MoE (20 lớp, 128 Experts Top-6) & Đầu ra mã ngữ nghĩa c_0" §1:
//     16 query heads share 2 key/value heads of 128 dimensions.
//   "1B · Interleaved TM-RoPE 3D (24, 20, 20) & Đồng bộ trục thời gian 12.5 Hz"
//     §3: adjacent pairs (x_2k, x_2k+1) turn by the angle of their axis; the 64
//     pairs interleave T, H, W (24 / 20 / 20, the last four temporal);
//     rope_theta 1e6.
//   "用 print(model) 认识 Qwen3-TTS", the attention module print: q_norm / k_norm,
//     an RMSNorm over each 128-wide head.
// The projections run on the grouped GEMM kernels (a plain product is the
// shared-expert tile list of the down pass); these kernels do the rest.
#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {
namespace {

constexpr int kHead = 128;                       // head width (64 pairs, one per lane)
constexpr int kChunk = 128;                      // cached positions per partial
constexpr int kAttnWaves = 4;
constexpr int kKeysPerWave = kChunk / kAttnWaves;
constexpr int kSteps = kKeysPerWave / 4;         // a wave reads 4 positions per load (16 lanes each)

__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(v[q] << 16);
        f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
    }
}

// One wave per (token, head of the fused q / k / v row); lane l owns pair l.
// Query and key heads: RMSNorm over the head (fp32), times the gain, then the
// rotation of pair l by pos[axis(l)] * theta^(-2 l / 128) (angle and its sine
// and cosine in fp64).  Queries go to q_out [T, nq, 128]; keys and values to
// position len[t] of the stream's cache [T, nkv, max_len, 128] (values
// unchanged).  A stream whose len is outside [0, max_len) writes no cache row.
__global__ __launch_bounds__(64) void qk_rope_append_kernel(const bf16_t* __restrict__ qkv, int nq, int nkv,
                                                            const float* __restrict__ q_gain,
                                                            const float* __restrict__ k_gain, float eps,
                                                            const int32_t* __restrict__ pos,
                                                            const int32_t* __restrict__ len, int max_len,
                                                            int sec_h, int sec_w, double log_theta,
                                                            bf16_t* __restrict__ q_out, bf16_t* __restrict__ kc,
                                                            bf16_t* __restrict__ vc) {
    const int64_t t = blockIdx.x;
    const int y = blockIdx.y;
    const int l = threadIdx.x;
    const int64_t ld = (int64_t)(nq + 2 * nkv) * kHead;
    const uint32_t raw = *reinterpret_cast<const uint32_t*>(qkv + t * ld + (int64_t)y * kHead + 2 * l);
    const int n = len[t];
    const bool ok = n >= 0 && n < max_len;
    if (y >= nq + nkv) {
        const int g = y - nq - nkv;
        if (ok) *reinterpret_cast<uint32_t*>(vc + (((t * nkv + g) * (int64_t)max_len + n) * kHead + 2 * l)) = raw;
        return;
    }
    float x0 = __uint_as_float(raw << 16), x1 = __uint_as_float(raw & 0xFFFF0000u);
    const float ss = wave_sum_dpp(fmaf(x0, x0, x1 * x1));
    const float inv = 1.0f / sqrtf(ss * (1.0f / kHead) + eps);
    const float* gain = y < nq ? q_gain : k_gain;
    x0 = x0 * inv * gain[2 * l];
    x1 = x1 * inv * gain[2 * l + 1];
    const int axis = (l % 3 == 1 && l < 3 * sec_h) ? 1 : ((l % 3 == 2 && l < 3 * sec_w) ? 2 : 0);
    const double ang = (double)pos[t * 3 + axis] * exp(-2.0 * l / kHead * log_theta);
    double sd, cd;
    sincos(ang, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    const uint32_t packed = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
    if (y < nq) {
        *reinterpret_cast<uint32_t*>(q_out + (t * nq + y) * kHead + 2 * l) = packed;
    } else if (ok) {
        const int g = y - nq;
        *reinterpret_cast<uint32_t*>(kc + (((t * nkv + g) * (int64_t)max_len + n) * kHead + 2 * l)) = packed;
    }
}

// Partial attention of the G query heads of KV head g over positions
// [c * 128, c * 128 + 128) of stream t (the stream attends to len[t] + 1
// positions, the new one included).  Wave w takes 32 positions, four per load
// (16 lanes x 16 bytes per 256-byte row), all its key and value rows in flight
// at once; an online softmax per head, then the lanes' and waves' partials
// merge.  Writes the chunk's max m, sum l and unnormalised output per head; an
// empty chunk writes m = -inf, l = 0 and no output.
template <int G>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_partial_kernel(const bf16_t* __restrict__ q,
                                                                       const bf16_t* __restrict__ kc,
                                                                       const bf16_t* __restrict__ vc,
                                                                       const int32_t* __restrict__ len, int nkv,
                                                                       int max_len, int nch, float* __restrict__ pm,
                                                                       float* __restrict__ pl,
                                                                       float* __restrict__ pacc) {
    __shared__ float red_m[kAttnWaves][G], red_l[kAttnWaves][G];
    __shared__ float red_acc[kAttnWaves][G][kHead];
    const int c = blockIdx.x, g = blockIdx.y;
    const int64_t t = blockIdx.z;
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int sub = lane >> 4, part = lane & 15;
    const int nraw = len[t];
    const int n = (nraw >= 0 && nraw < max_len) ? nraw + 1 : 0;
    const int64_t pidx = (t * nkv + g) * nch + c;
    const int k0 = c * kChunk;
    if (k0 >= n) {  // block-uniform
        if (threadIdx.x < G) {
            pm[pidx * G + threadIdx.x] = -INFINITY;
            pl[pidx * G + threadIdx.x] = 0.f;
        }
        return;
    }
    const int nq = nkv * G;
    u32x4 qv[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        qv[j] = *reinterpret_cast<const u32x4*>(q + ((t * nq + g * G + j) * kHead + part * 8));
    const int64_t base = (t * nkv + g) * (int64_t)max_len * kHead + part * 8;
    u32x4 kr[kSteps], vr[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {  // branch-free: positions past the end repeat the last one, unused
        const int p = min(k0 + wave * kKeysPerWave + 4 * s + sub, n - 1);
        kr[s] = *reinterpret_cast<const u32x4*>(kc + base + (int64_t)p * kHead);
        vr[s] = *reinterpret_cast<const u32x4*>(vc + base + (int64_t)p * kHead);
    }
    const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const bool valid = k0 + wave * kKeysPerWave + 4 * s + sub < n;
        float kf[8], vf[8];
        unpack8(kr[s], kf);
        unpack8(vr[s], vf);
        float dot[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float qf[8];
            unpack8(qv[j], qf);
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = fmaf(qf[i], kf[i], a);
            dot[j] = a;
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1)
#pragma unroll
            for (int j = 0; j < G; ++j) dot[j] += __shfl_xor(dot[j], off);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float sc = valid ? dot[j] * scale : -INFINITY;
            const float mn = fmaxf(m[j], sc);
            const float alpha = m[j] == -INFINITY ? 0.f : __expf(m[j] - mn);
            const float p = valid ? __expf(sc - mn) : 0.f;
            l[j] = fmaf(l[j], alpha, p);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(acc[j][i], alpha, p * vf[i]);
            m[j] = mn;
        }
    }
    // merge the four position groups of the wave (lanes 16 apart)
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float om = __shfl_xor(m[j], off), ol = __shfl_xor(l[j], off);
            const float mn = fmaxf(m[j], om);
            const float a = m[j] == -INFINITY ? 0.f : __expf(m[j] - mn);
            const float b = om == -INFINITY ? 0.f : __expf(om - mn);
            l[j] = l[j] * a + ol * b;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] * a + __shfl_xor(acc[j][i], off) * b;
            m[j] = mn;
        }
    }
    if (sub == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) red_acc[wave][j][part * 8 + i] = acc[j][i];
        if (part == 0)
#pragma unroll
            for (int j = 0; j < G; ++j) {
                red_m[wave][j] = m[j];
                red_l[wave][j] = l[j];
            }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kHead; idx += 64 * kAttnWaves) {
        const int j = idx / kHead, dd = idx % kHead;
        float mx = red_m[0][j];
#pragma unroll
        for (int w = 1; w < kAttnWaves; ++w) mx = fmaxf(mx, red_m[w][j]);
        float a = 0.f, ls = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float f = red_m[w][j] == -INFINITY ? 0.f : __expf(red_m[w][j] - mx);
            a = fmaf(red_acc[w][j][dd], f, a);
            ls = fmaf(red_l[w][j], f, ls);
        }
        pacc[(pidx * G + j) * kHead + dd] = a;
        if (dd == 0) {
            pm[pidx * G + j] = mx;
            pl[pidx * G + j] = ls;
        }
    }
}

// Output of query head h of stream t: the chunk partials merged in chunk order
// (max of the maxima, rescaled sums), divided by the total weight; one thread
// per dimension.  A stream with no valid position gets zeros.
__global__ __launch_bounds__(kHead) void attn_combine_kernel(const float* __restrict__ pm,
                                                             const float* __restrict__ pl,
                                                             const float* __restrict__ pacc,
                                                             const int32_t* __restrict__ len, int nq, int nkv,
                                                             int max_len, int nch, bf16_t* __restrict__ o) {
    const int h = blockIdx.x;
    const int64_t t = blockIdx.y;
    const int G = nq / nkv, g = h / G, j = h % G;
    const int dd = threadIdx.x;
    const int nraw = len[t];
    const int n = (nraw >= 0 && nraw < max_len) ? nraw + 1 : 0;
    const int nc = (n + kChunk - 1) / kChunk;
    const int64_t p0 = (t * nkv + g) * nch;
    float mx = -INFINITY;
    for (int c = 0; c < nc; ++c) mx = fmaxf(mx, pm[(p0 + c) * G + j]);
    float a = 0.f, ls = 0.f;
    for (int c = 0; c < nc; ++c) {
        const float f = __expf(pm[(p0 + c) * G + j] - mx);
        ls = fmaf(pl[(p0 + c) * G + j], f, ls);
        a = fmaf(pacc[((p0 + c) * G + j) * kHead + dd], f, a);
    }
    const float r = nc > 0 ? a / ls : 0.f;
    o[(t * nq + h) * kHead + dd] = f32_to_bf16(r);
}

}  // namespace

bool attn_decode_ok(int head_dim, int nq, int nkv) {
    if (head_dim != kHead || nkv < 1 || nq % nkv != 0) return false;
    const int G = nq / nkv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

int attn_chunks(int max_len) { return (max_len + kChunk - 1) / kChunk; }

hipError_t launch_qk_rope_append(const void* qkv, int64_t T, int nq, int nkv, const float* q_gain,
                                 const float* k_gain, float eps, const int32_t* pos, const int32_t* len,
                                 int max_len, int sec_h, int sec_w, double theta, void* q_out, void* kc, void* vc,
                                 hipStream_t st) {
    if (T <= 0) return hipSuccess;
    dim3 grid((unsigned)T, (unsigned)(nq + 2 * nkv));
    qk_rope_append_kernel<<<grid, 64, 0, st>>>((const bf16_t*)qkv, nq, nkv, q_gain, k_gain, eps, pos, len, max_len,
                                               sec_h, sec_w, log(theta), (bf16_t*)q_out, (bf16_t*)kc, (bf16_t*)vc);
    return hipGetLastError();
}

hipError_t launch_attn_decode(const void* q, const void* kc, const void* vc, const int32_t* len, int64_t T, int nq,
                              int nkv, int max_len, float* pm, float* pl, float* pacc, void* o, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int nch = attn_chunks(max_len);
    dim3 grid((unsigned)nch, (unsigned)nkv, (unsigned)T);
    const int G = nq / nkv;
    const bf16_t *qb = (const bf16_t*)q, *kb = (const bf16_t*)kc, *vb = (const bf16_t*)vc;
    if (G == 8) attn_partial_kernel<8><<<grid, 64 * kAttnWaves, 0, st>>>(qb, kb, vb, len, nkv, max_len, nch, pm, pl, pacc);
    else if (G == 4) attn_partial_kernel<4><<<grid, 64 * kAttnWaves, 0, st>>>(qb, kb, vb, len, nkv, max_len, nch, pm, pl, pacc);
    else if (G == 2) attn_partial_kernel<2><<<grid, 64 * kAttnWaves, 0, st>>>(qb, kb, vb, len, nkv, max_len, nch, pm, pl, pacc);
    else attn_partial_kernel<1><<<grid, 64 * kAttnWaves, 0, st>>>(qb, kb, vb, len, nkv, max_len, nch, pm, pl, pacc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_combine_kernel<<<dim3((unsigned)nq, (unsigned)T), kHead, 0, st>>>(pm, pl, pacc, len, nq, nkv, max_len, nch,
                                                                          (bf16_t*)o);
    return hipGetLastError();
}

}  // namespace tmoe
