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
// The projections run on the split-K skinny product kernel (or, above 64
// tokens, the grouped GEMM's shared tile list); these kernels do the rest.
#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {
namespace {

constexpr int kHead = 128;                       // head width (64 pairs, one per lane)
constexpr int kKeysPerWave = 32;  // cached positions per wave of the partial kernel
// Waves per partial workgroup (a chunk is 32 positions per wave): 16 for long
// caches, where fewer, longer chunks leave less to merge; 4 for short ones
// (the predictor's 16-position frames), where idle waves would only cost.
constexpr int kAttnWavesLong = 16, kAttnWavesShort = 4;
__host__ __device__ constexpr int attn_waves(int max_len) { return max_len > 256 ? kAttnWavesLong : kAttnWavesShort; }
__host__ __device__ constexpr int attn_chunk(int max_len) { return kKeysPerWave * attn_waves(max_len); }

// One wave per (token, head of the fused q / k / v row), four heads per
// workgroup; lane l owns pair l.  The row comes as KS fp32 partial products
// (summed in order) or, with KS == 0, as bf16.  Query and key heads: RMSNorm
// over the head (fp32), times the gain, then the rotation of pair l by
// pos[axis(l)] * theta^(-2 l / 128) (the angle in fp64, reduced to [-pi, pi]
// before its sine and cosine).  Queries go to q_out [T, nq, 128]; keys to
// position len[t] of the key cache [T, nkv, max_len, 128], values (unchanged,
// rounded to bf16) to column len[t] of the transposed value cache
// [T, nkv, 128, max_len].  A stream whose len is outside [0, max_len) writes no
// cache entry.
constexpr int kRopeWaves = 4;

// Pair l (lane l) of row y (a query, key or value head of the fused q / k / v
// row) of token t, as the bf16 pair the attention reads: the KS fp32 partials
// summed in order (or the bf16 row when KS == 0); query and key heads then take
// the RMSNorm over the head times the gain and the rotation (above).  Called by
// one full wave.
__device__ __forceinline__ uint32_t rope_pair(const void* __restrict__ qkv, int KS, int64_t T, int nq, int nkv,
                                              int64_t t, int y, const float* __restrict__ q_gain,
                                              const float* __restrict__ k_gain, float eps,
                                              const int32_t* __restrict__ pos, int sec_h, int sec_w,
                                              double log_theta) {
    const int l = lane_id();
    const int64_t ld = (int64_t)(nq + 2 * nkv) * kHead;
    const int64_t e = t * ld + (int64_t)y * kHead + 2 * l;
    float x0, x1;
    if (KS > 0) {
        const float* p = reinterpret_cast<const float*>(qkv);
        x0 = 0.f;
        x1 = 0.f;
        // four partials requested at a time (the index clamped, the surplus
        // dropped), then added in order
        for (int s0 = 0; s0 < KS; s0 += 4) {
            f32x2_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = *reinterpret_cast<const f32x2_t*>(p + min(s0 + i, KS - 1) * T * ld + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x0 = s0 + i < KS ? x0 + v[i][0] : x0;
                x1 = s0 + i < KS ? x1 + v[i][1] : x1;
            }
        }
    } else {
        const uint32_t raw = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const bf16_t*>(qkv) + e);
        x0 = __uint_as_float(raw << 16);
        x1 = __uint_as_float(raw & 0xFFFF0000u);
    }
    if (y >= nq + nkv) return pack_bf16x2(x0, x1);  // values: unchanged
    const float ss = wave_sum_dpp(fmaf(x0, x0, x1 * x1));
    const float inv = 1.0f / sqrtf(ss * (1.0f / kHead) + eps);
    const float* gain = y < nq ? q_gain : k_gain;
    x0 = x0 * inv * gain[2 * l];
    x1 = x1 * inv * gain[2 * l + 1];
    const int axis = (l % 3 == 1 && l < 3 * sec_h) ? 1 : ((l % 3 == 2 && l < 3 * sec_w) ? 2 : 0);
    const double ang = (double)pos[t * 3 + axis] * exp(-2.0 * l / kHead * log_theta);
    const double two_pi = 6.283185307179586;
    const float red = (float)(ang - two_pi * rint(ang / two_pi));
    float s, c;
    sincosf(red, &s, &c);
    return pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
}

// rope_pair in two halves, for a caller that issues the loads before anything
// else it waits for: rope_load requests the first four partials (or the bf16
// pair), the gain pair and the position; rope_finish adds any further partials,
// four at a time, and does rope_pair's arithmetic, in its order (same bits).
struct RopeIn {
    f32x2_t v[4];  // partials 0 .. 3 (index clamped to KS - 1), or the bf16 pair in v[0]
    float g0, g1;  // the gain pair of a query or key head
    int p;         // the position index of this lane's axis
};

__device__ __forceinline__ RopeIn rope_load(const void* __restrict__ qkv, int KS, int64_t T, int nq, int nkv,
                                            int64_t t, int y, const float* __restrict__ q_gain,
                                            const float* __restrict__ k_gain, const int32_t* __restrict__ pos,
                                            int sec_h, int sec_w) {
    const int l = lane_id();
    const int64_t ld = (int64_t)(nq + 2 * nkv) * kHead;
    const int64_t e = t * ld + (int64_t)y * kHead + 2 * l;
    RopeIn r;
    if (KS > 0) {
        const float* p = reinterpret_cast<const float*>(qkv);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i] = *reinterpret_cast<const f32x2_t*>(p + min(i, KS - 1) * T * ld + e);
    } else {
        const uint32_t raw = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const bf16_t*>(qkv) + e);
        r.v[0][0] = __uint_as_float(raw << 16);
        r.v[0][1] = __uint_as_float(raw & 0xFFFF0000u);
    }
    r.g0 = r.g1 = 0.f;
    r.p = 0;
    if (y < nq + nkv) {  // wave-uniform: query and key heads
        const float* gain = y < nq ? q_gain : k_gain;
        r.g0 = gain[2 * l];
        r.g1 = gain[2 * l + 1];
        const int axis = (l % 3 == 1 && l < 3 * sec_h) ? 1 : ((l % 3 == 2 && l < 3 * sec_w) ? 2 : 0);
        r.p = pos[t * 3 + axis];
    }
    return r;
}

__device__ __forceinline__ uint32_t rope_finish(const RopeIn& r, const void* __restrict__ qkv, int KS, int64_t T,
                                                int nq, int nkv, int64_t t, int y, float eps, double log_theta) {
    const int l = lane_id();
    float x0, x1;
    if (KS > 0) {
        const float* p = reinterpret_cast<const float*>(qkv);
        const int64_t ld = (int64_t)(nq + 2 * nkv) * kHead;
        const int64_t e = t * ld + (int64_t)y * kHead + 2 * l;
        x0 = 0.f;
        x1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x0 = i < KS ? x0 + r.v[i][0] : x0;
            x1 = i < KS ? x1 + r.v[i][1] : x1;
        }
        // partials past the fourth, requested four at a time (the index
        // clamped, the surplus dropped), then added in order
        for (int s0 = 4; s0 < KS; s0 += 4) {
            f32x2_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = *reinterpret_cast<const f32x2_t*>(p + min(s0 + i, KS - 1) * T * ld + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x0 = s0 + i < KS ? x0 + v[i][0] : x0;
                x1 = s0 + i < KS ? x1 + v[i][1] : x1;
            }
        }
    } else {
        x0 = r.v[0][0];
        x1 = r.v[0][1];
    }
    if (y >= nq + nkv) return pack_bf16x2(x0, x1);  // values: unchanged
    const float ss = wave_sum_dpp(fmaf(x0, x0, x1 * x1));
    const float inv = 1.0f / sqrtf(ss * (1.0f / kHead) + eps);
    x0 = x0 * inv * r.g0;
    x1 = x1 * inv * r.g1;
    const double ang = (double)r.p * exp(-2.0 * l / kHead * log_theta);
    const double two_pi = 6.283185307179586;
    const float red = (float)(ang - two_pi * rint(ang / two_pi));
    float s, c;
    sincosf(red, &s, &c);
    return pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
}

// Pair `packed` of the new position's key (into the key cache [T, nkv, max_len,
// 128]) or value (into the transposed value cache [T, nkv, 128, max_len]) of
// KV head g at position n.
__device__ __forceinline__ void append_pair(bool is_value, uint32_t packed, int64_t t, int g, int nkv, int n,
                                            int max_len, bf16_t* __restrict__ kc, bf16_t* __restrict__ vc) {
    const int l = lane_id();
    if (is_value) {
        bf16_t* col = vc + ((t * nkv + g) * (int64_t)kHead + 2 * l) * max_len + n;
        col[0] = (bf16_t)(packed & 0xFFFFu);
        col[max_len] = (bf16_t)(packed >> 16);
    } else {
        *reinterpret_cast<uint32_t*>(kc + (((t * nkv + g) * (int64_t)max_len + n) * kHead + 2 * l)) = packed;
    }
}

// One wave per (token, head of the fused q / k / v row), four heads per
// workgroup; lane l owns pair l.  Queries go to q_out [T, nq, 128]; keys and
// values to position len[t] of the caches.  A stream whose len is outside
// [0, max_len) writes no cache entry.
__global__ __launch_bounds__(64 * kRopeWaves) void qk_rope_append_kernel(
    const void* __restrict__ qkv, int KS, int64_t T, int nq, int nkv, const float* __restrict__ q_gain,
    const float* __restrict__ k_gain, float eps, const int32_t* __restrict__ pos, const int32_t* __restrict__ len,
    int max_len, int sec_h, int sec_w, double log_theta, bf16_t* __restrict__ q_out, bf16_t* __restrict__ kc,
    bf16_t* __restrict__ vc) {
    const int64_t t = blockIdx.x;
    const int y = blockIdx.y * kRopeWaves + (int)(threadIdx.x >> 6);
    const int l = lane_id();
    if (y >= nq + 2 * nkv) return;  // wave-uniform
    const uint32_t packed = rope_pair(qkv, KS, T, nq, nkv, t, y, q_gain, k_gain, eps, pos, sec_h, sec_w, log_theta);
    if (y < nq) {
        *reinterpret_cast<uint32_t*>(q_out + (t * nq + y) * kHead + 2 * l) = packed;
        return;
    }
    const int n = len[t];
    if (n >= 0 && n < max_len)
        append_pair(y >= nq + nkv, packed, t, y >= nq + nkv ? y - nq - nkv : y - nq, nkv, n, max_len, kc, vc);
}

// y = sum of KS fp32 partial rows (in order) + residual, stored bf16; with
// norm_out, also RMSNorm of the stored y times the gain.  One workgroup per
// row, 8 contiguous features per thread per pass.  KSC > 0: KS == KSC, and
// every partial row is requested before the first add (one memory round trip
// instead of KS); the sums are the same, in the same order.  The first kKeep
// passes (H <= 2048) keep their stored values in registers and request their
// gains at the start, so the norm after the barrier needs no memory round trip.
constexpr int kKeep = 2;
template <int KSC>
__global__ __launch_bounds__(128) void attn_out_kernel(const float* __restrict__ part, int KS, int64_t T, int H,
                                                       const bf16_t* residual, bf16_t* y,
                                                       const float* __restrict__ gain, float eps,
                                                       bf16_t* __restrict__ norm_out) {
    __shared__ float wsum[2];
    const int64_t t = blockIdx.x;
    float gk[kKeep][8];
#pragma unroll
    for (int c = 0; c < kKeep; ++c) {
        const int h = threadIdx.x * 8 + 128 * 8 * c;
        if (norm_out && gain && h < H) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(gain + h);
            const f32x4 b = *reinterpret_cast<const f32x4*>(gain + h + 4);
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                gk[c][i2] = a[i2];
                gk[c][4 + i2] = b[i2];
            }
        } else {
#pragma unroll
            for (int i2 = 0; i2 < 8; ++i2) gk[c][i2] = 1.f;
        }
    }
    u32x4 yk[kKeep];
    float ss = 0.f;
    for (int h = threadIdx.x * 8, c = 0; h < H; h += 128 * 8, ++c) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
        auto add = [&](const f32x4& a, const f32x4& b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] += a[i];
                v[4 + i] += b[i];
            }
        };
        if (KSC > 0) {
            f32x4 pa[KSC > 0 ? KSC : 1], pb[KSC > 0 ? KSC : 1];
#pragma unroll
            for (int s = 0; s < KSC; ++s) {
                const float* p = part + (s * T + t) * (int64_t)H + h;
                pa[s] = *reinterpret_cast<const f32x4*>(p);
                pb[s] = *reinterpret_cast<const f32x4*>(p + 4);
            }
#pragma unroll
            for (int s = 0; s < KSC; ++s) add(pa[s], pb[s]);
        } else {
            for (int s = 0; s < KS; ++s) {
                const float* p = part + (s * T + t) * (int64_t)H + h;
                add(*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4));
            }
        }
        if (residual) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(residual + t * H + h);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[2 * q] += __uint_as_float(r[q] << 16);
                v[2 * q + 1] += __uint_as_float(r[q] & 0xFFFF0000u);
            }
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
            const float a = __uint_as_float(o[q] << 16), b = __uint_as_float(o[q] & 0xFFFF0000u);
            ss = fmaf(a, a, ss);
            ss = fmaf(b, b, ss);
        }
        *reinterpret_cast<u32x4*>(y + t * H + h) = o;
#pragma unroll
        for (int c2 = 0; c2 < kKeep; ++c2)
            if (c == c2) yk[c2] = o;
    }
    if (!norm_out) return;  // block-uniform
    ss = wave_sum_dpp(ss);
    if (lane_id() == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((wsum[0] + wsum[1]) / (float)H + eps);
    for (int h = threadIdx.x * 8, c = 0; h < H; h += 128 * 8, ++c) {
        u32x4 yv;
        float g[8];
        if (c < kKeep) {
#pragma unroll
            for (int c2 = 0; c2 < kKeep; ++c2)
                if (c == c2) {
                    yv = yk[c2];
#pragma unroll
                    for (int i = 0; i < 8; ++i) g[i] = gk[c2][i];
                }
        } else {  // rows wider than kKeep passes: the stored values and the gains from memory
            yv = *reinterpret_cast<const u32x4*>(y + t * H + h);
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = gain ? gain[h + i] : 1.f;
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(__uint_as_float(yv[q] << 16) * inv * g[2 * q],
                               __uint_as_float(yv[q] & 0xFFFF0000u) * inv * g[2 * q + 1]);
        *reinterpret_cast<u32x4*>(norm_out + t * H + h) = o;
    }
}

// Partial attention of the G query heads of KV head g over positions
// [c * 128, c * 128 + 128) of stream t (the stream attends to len[t] + 1
// positions, the new one included), on the matrix cores.  Wave w takes 32
// positions with all its key and value fragments in flight at once:
//   S = Q K^T: the G query heads (zero rows up to 16) against two 16-position
//     tiles, four 32-wide K steps each (v_mfma_f32_16x16x32_bf16; the operand
//     fragment of a lane is 8 consecutive dimensions of one row);
//   per head the maximum and the sum of exp over the wave's positions (16-lane
//   reductions), positions past the stream's end masked to -inf;
//   P (bf16) turns from the product layout to the operand layout through 1 KB of
//   LDS, and O = P V over eight 16-dimension tiles reads the transposed value
//   cache (8 consecutive positions of one dimension per lane; positions past
//   the end are zeroed, so stale cache contents never reach the sum).
// The waves' (max, sum, output) merge in LDS.  Writes the chunk's max m, sum l
// and unnormalised output per head; an empty chunk writes m = -inf, l = 0.  When
// the cache is a single chunk (nch == 1) the workgroup writes the normalised
// output od [T, nq, 128] instead (zeros for a stream with no valid position).
//
// FUSED: the workgroup also forms what qk_rope_append_kernel would (it then
// needs no q): waves 0 .. G - 1 its G query heads, wave G the new key and wave
// G + 1 the new value of KV head g (rope_pair), into LDS; the workgroup whose
// chunk holds the new position appends them to the caches, and every
// workgroup reads the new position's key and value from LDS rather than from
// the caches (which the append may not have reached).
struct RopeArgs {
    const void* qkv;  // the fused q / k / v rows: KS fp32 partials, or bf16 when KS == 0
    int KS;
    const float *q_gain, *k_gain;
    float eps;
    const int32_t* pos;
    int sec_h, sec_w;
    double log_theta;
    bf16_t *kc, *vc;  // the caches, written at len[t]
};

template <int G, int kAttnWaves, bool FUSED>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_partial_kernel(const bf16_t* __restrict__ q,
                                                                       const bf16_t* __restrict__ kc,
                                                                       const bf16_t* __restrict__ vt,
                                                                       const int32_t* __restrict__ len, int nkv,
                                                                       int max_len, int nch, float* __restrict__ pm,
                                                                       float* __restrict__ pl,
                                                                       float* __restrict__ pacc,
                                                                       bf16_t* __restrict__ od, RopeArgs ra) {
    static_assert(!FUSED || G + 2 <= kAttnWaves, "a wave per query head, the new key and the new value");
    __shared__ float red_m[kAttnWaves][16], red_l[kAttnWaves][16];
    __shared__ __attribute__((aligned(16))) bf16_t qs[FUSED ? G : 1][kHead];  // FUSED: the query heads
    __shared__ __attribute__((aligned(16))) bf16_t kvn[FUSED ? 2 : 1][kHead];  // FUSED: new key, new value
    __shared__ float red_acc[kAttnWaves][G][kHead];
    __shared__ __attribute__((aligned(16))) bf16_t pbuf[kAttnWaves][16][40];  // rows padded to 80 bytes
    const int c = blockIdx.x, g = blockIdx.y;
    const int64_t t = blockIdx.z;
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int col = lane & 15, grp = lane >> 4;
    // FUSED, long form: the waves of the q / k step request their partials,
    // gains and positions before the stream's length, which they do not depend
    // on (measured 0.4 us less per step at 1024 positions).  The short form
    // requests the cached keys and values first instead (below; its q / k
    // loads issued first measured slower there).
    constexpr bool rope_early = FUSED && kAttnWaves != kAttnWavesShort;
    RopeIn rin;
    if constexpr (rope_early) {
        if (wave < G + 2) {  // wave-uniform; the other waves' queues stay free for their cache chunk
            const int nqe = nkv * G;
            const int ye = wave < G ? g * G + wave : (wave == G ? nqe + g : nqe + nkv + g);
            rin = rope_load(ra.qkv, ra.KS, (int64_t)gridDim.z, nqe, nkv, t, ye, ra.q_gain, ra.k_gain, ra.pos,
                            ra.sec_h, ra.sec_w);
        }
    }
    const int nraw = len[t];
    const int n = (nraw >= 0 && nraw < max_len) ? nraw + 1 : 0;
    const int64_t pidx = (t * nkv + g) * nch + c;
    const int k0 = c * kKeysPerWave * kAttnWaves;
    const int nq = nkv * G;
    if (k0 >= n) {  // block-uniform
        if (nch == 1) {
            for (int i = threadIdx.x; i < G * kHead; i += 64 * kAttnWaves) od[(t * nq + g * G) * kHead + i] = 0;
        } else if (threadIdx.x < G) {
            pm[pidx * G + threadIdx.x] = -INFINITY;
            pl[pidx * G + threadIdx.x] = 0.f;
        }
        return;
    }
    const int key0 = k0 + wave * kKeysPerWave;
    const f32x4 zero = {0, 0, 0, 0};
    float m_r[4], l_r[4];
    f32x4 o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_r[i] = -INFINITY;
        l_r[i] = 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = zero;
    const bool act = key0 < n;  // wave-uniform
    const u32x4 z4 = {0, 0, 0, 0};
    u32x4 kb[2][4], vb[8];
    auto load_kv = [&]() {
        const int64_t kvrow = (t * nkv + g) * (int64_t)max_len;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {  // positions past the end load the last one (masked below)
            const int key = min(key0 + nt * 16 + col, n - 1);
            const bf16_t* kp = kc + (kvrow + key) * kHead + grp * 8;
#pragma unroll
            for (int s = 0; s < 4; ++s) kb[nt][s] = *reinterpret_cast<const u32x4*>(kp + s * 32);
        }
        // key0 + 32 <= max_len (max_len % 32 == 0), so the value rows stay in bounds
        const bf16_t* vp = vt + ((t * nkv + g) * (int64_t)kHead + col) * max_len + key0 + grp * 8;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vb[dt] = *reinterpret_cast<const u32x4*>(vp + (int64_t)dt * 16 * max_len);
    };
    // With the fused q / k / v step, a short workgroup (few waves, the
    // predictor's frames) requests the cached keys and values before it, so
    // their latency overlaps it.  In a long one the waves that form the query
    // heads and the new key and value request theirs after it (all waves first
    // measured slower: the q / k loads queue behind the whole chunk), the other
    // waves at once (measured 1.1 us less per step at 1024 positions).
    constexpr bool kv_first = !FUSED || kAttnWaves == kAttnWavesShort;
    const bool early = kv_first || wave >= G + 2;  // wave-uniform
    if (early && act) load_kv();
    if constexpr (FUSED) {
        if (wave < G + 2) {  // wave-uniform
            const int nq_ = nkv * G;
            const int y = wave < G ? g * G + wave : (wave == G ? nq_ + g : nq_ + nkv + g);
            uint32_t packed;
            if constexpr (rope_early)
                packed = rope_finish(rin, ra.qkv, ra.KS, (int64_t)gridDim.z, nq_, nkv, t, y, ra.eps, ra.log_theta);
            else
                packed = rope_pair(ra.qkv, ra.KS, (int64_t)gridDim.z, nq_, nkv, t, y, ra.q_gain, ra.k_gain, ra.eps,
                                   ra.pos, ra.sec_h, ra.sec_w, ra.log_theta);
            if (wave < G) {
                *reinterpret_cast<uint32_t*>(&qs[wave][2 * lane]) = packed;
            } else {
                *reinterpret_cast<uint32_t*>(&kvn[wave - G][2 * lane]) = packed;
                if (n > 0 && nraw / (kKeysPerWave * kAttnWaves) == c)  // this chunk holds the new position
                    append_pair(wave == G + 1, packed, t, g, nkv, nraw, max_len, ra.kc, ra.vc);
            }
        }
        __syncthreads();
    }
    if (!early && act) load_kv();
    if (act) {
        u32x4 qa[4];
        if constexpr (FUSED) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                qa[s] = col < G ? *reinterpret_cast<const u32x4*>(&qs[min(col, G - 1)][grp * 8 + s * 32]) : z4;
            // the new position (n - 1) from LDS: its key for the lanes it falls
            // on (the positions past the end load it too, masked below)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                if (min(key0 + nt * 16 + col, n - 1) == nraw)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        kb[nt][s] = *reinterpret_cast<const u32x4*>(&kvn[0][grp * 8 + s * 32]);
        } else {
            const bf16_t* qp = q + ((t * nq + g * G + min(col, G - 1)) * kHead + grp * 8);
#pragma unroll
            for (int s = 0; s < 4; ++s) qa[s] = col < G ? *reinterpret_cast<const u32x4*>(qp + s * 32) : z4;
        }
        if constexpr (FUSED) {
            // the new position's value (dimension 16 dt + col) from LDS
            const int j = nraw - (key0 + grp * 8);
            if (j >= 0 && j < 8) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const uint32_t nv = (uint32_t)kvn[1][16 * dt + col];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (e == (j >> 1))
                            vb[dt][e] = (j & 1) ? ((vb[dt][e] & 0x0000FFFFu) | (nv << 16))
                                                : ((vb[dt][e] & 0xFFFF0000u) | nv);
                }
            }
        }
        f32x4 sacc[2] = {zero, zero};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[s]),
                                                                   __builtin_bit_cast(bf16x8, kb[nt][s]), sacc[nt],
                                                                   0, 0, 0);
        // sacc[nt][i] = S[head 4 grp + i][position key0 + 16 nt + col]
        const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
        float sv[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[nt][i] = key0 + nt * 16 + col < n ? sacc[nt][i] * scale : -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = fmaxf(sv[0][i], sv[1][i]);
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            m_r[i] = mx;
        }
        float pv[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) pv[nt][i] = __expf(sv[nt][i] - m_r[i]);
            float sm = pv[0][i] + pv[1][i];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) sm += __shfl_xor(sm, off);
            l_r[i] = sm;
        }
        // P to the operand layout: row = head, 8 consecutive positions per lane
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) pbuf[wave][4 * grp + i][nt * 16 + col] = f32_to_bf16(pv[nt][i]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const u32x4 pa = *reinterpret_cast<const u32x4*>(&pbuf[wave][col][grp * 8]);
        // zero the value entries of positions past the end
        const int valid = n - (key0 + grp * 8);  // positions of this lane's 8 that are in range
        if (valid < 8) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t w2 = vb[dt][e];
                    if (2 * e >= valid) w2 &= 0xFFFF0000u;
                    if (2 * e + 1 >= valid) w2 &= 0x0000FFFFu;
                    vb[dt][e] = w2;
                }
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                            __builtin_bit_cast(bf16x8, vb[dt]), o[dt], 0, 0, 0);
    }
    // o[dt][i] = O[head 4 grp + i][dim 16 dt + col]
    if (col == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red_m[wave][4 * grp + i] = m_r[i];
            red_l[wave][4 * grp + i] = l_r[i];
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * grp + i;
        if (h < G)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) red_acc[wave][h][dt * 16 + col] = o[dt][i];
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
        if (nch == 1) {  // the only chunk: the output itself
            od[(t * nq + g * G + j) * kHead + dd] = f32_to_bf16(a / ls);
            continue;
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
// per dimension.  A stream with no valid position gets zeros.  With at most
// kMergeAtOnce chunks every chunk's maximum, sum and partial output is
// requested at once, beside the stream's length (indices clamped to the
// launch's chunks; those past the stream's end are not used), so the merge
// is one memory round trip; the arithmetic is the same in either form.
constexpr int kMergeAtOnce = 4;
__global__ __launch_bounds__(kHead) void attn_combine_kernel(const float* __restrict__ pm,
                                                             const float* __restrict__ pl,
                                                             const float* __restrict__ pacc,
                                                             const int32_t* __restrict__ len, int nq, int nkv,
                                                             int max_len, int nch, bf16_t* __restrict__ o) {
    const int h = blockIdx.x;
    const int64_t t = blockIdx.y;
    const int G = nq / nkv, g = h / G, j = h % G;
    const int dd = threadIdx.x;
    const int64_t p0 = (t * nkv + g) * nch;
    float m4[kMergeAtOnce], l4[kMergeAtOnce], a4[kMergeAtOnce];
    if (nch <= kMergeAtOnce) {
#pragma unroll
        for (int c = 0; c < kMergeAtOnce; ++c) {
            const int64_t pc = p0 + min(c, nch - 1);
            m4[c] = pm[pc * G + j];
            l4[c] = pl[pc * G + j];
            a4[c] = pacc[(pc * G + j) * kHead + dd];
        }
    }
    const int nraw = len[t];
    const int n = (nraw >= 0 && nraw < max_len) ? nraw + 1 : 0;
    const int chunk = attn_chunk(max_len);
    const int nc = (n + chunk - 1) / chunk;
    float mx = -INFINITY, a = 0.f, ls = 0.f;
    if (nch <= kMergeAtOnce) {
#pragma unroll
        for (int c = 0; c < kMergeAtOnce; ++c)
            if (c < nc) mx = fmaxf(mx, m4[c]);
#pragma unroll
        for (int c = 0; c < kMergeAtOnce; ++c)
            if (c < nc) {
                const float f = __expf(m4[c] - mx);
                ls = fmaf(l4[c], f, ls);
                a = fmaf(a4[c], f, a);
            }
    } else {
        for (int c = 0; c < nc; ++c) mx = fmaxf(mx, pm[(p0 + c) * G + j]);
        for (int c = 0; c < nc; ++c) {
            const float f = __expf(pm[(p0 + c) * G + j] - mx);
            ls = fmaf(pl[(p0 + c) * G + j], f, ls);
            a = fmaf(pacc[((p0 + c) * G + j) * kHead + dd], f, a);
        }
    }
    const float r = nc > 0 ? a / ls : 0.f;
    o[(t * nq + h) * kHead + dd] = f32_to_bf16(r);
}

}  // namespace

__global__ __launch_bounds__(256) void frame_setup_kernel(int32_t* __restrict__ pos, int32_t* __restrict__ len,
                                                          int P, int64_t T, const int32_t* __restrict__ c0,
                                                          int32_t* __restrict__ codes) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)P * T) return;
    const int p = (int)(i / T);
    len[i] = p;
    pos[3 * i] = p;
    pos[3 * i + 1] = p;
    pos[3 * i + 2] = p;
    if (i < T) codes[i] = c0[i];
}

hipError_t launch_frame_setup(int32_t* pos, int32_t* len, int P, int64_t T, const int32_t* c0, int32_t* codes,
                              hipStream_t st) {
    const int64_t n = (int64_t)P * T;
    if (n <= 0) return hipSuccess;
    frame_setup_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(pos, len, P, T, c0, codes);
    return hipGetLastError();
}

bool attn_decode_ok(int head_dim, int nq, int nkv, int max_len) {
    if (head_dim != kHead || nkv < 1 || nq % nkv != 0 || max_len % kKeysPerWave != 0) return false;
    const int G = nq / nkv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

int attn_chunks(int max_len) { return (max_len + attn_chunk(max_len) - 1) / attn_chunk(max_len); }

hipError_t launch_qk_rope_append(const float* qkv, int KS, int64_t T, int nq, int nkv, const float* q_gain,
                                 const float* k_gain, float eps, const int32_t* pos, const int32_t* len,
                                 int max_len, int sec_h, int sec_w, double theta, void* q_out, void* kc, void* vc,
                                 hipStream_t st) {
    if (T <= 0) return hipSuccess;
    dim3 grid((unsigned)T, (unsigned)((nq + 2 * nkv + kRopeWaves - 1) / kRopeWaves));
    qk_rope_append_kernel<<<grid, 64 * kRopeWaves, 0, st>>>(qkv, KS, T, nq, nkv, q_gain, k_gain, eps, pos, len,
                                                             max_len, sec_h, sec_w, log(theta), (bf16_t*)q_out,
                                                             (bf16_t*)kc, (bf16_t*)vc);
    return hipGetLastError();
}

hipError_t launch_attn_out(const float* part, int KS, const void* residual, void* y, int64_t T, int H,
                           const float* gain, float eps, void* norm_out, hipStream_t st) {
    if (T <= 0) return hipSuccess;
#define TMOE_AO(KSC)                                                                                        \
    attn_out_kernel<KSC><<<(unsigned)T, 128, 0, st>>>(part, KS, T, H, (const bf16_t*)residual, (bf16_t*)y, gain, \
                                                     eps, (bf16_t*)norm_out)
    switch (KS) {
        case 1: TMOE_AO(1); break;
        case 2: TMOE_AO(2); break;
        case 4: TMOE_AO(4); break;
        case 8: TMOE_AO(8); break;
        case 12: TMOE_AO(12); break;
        case 16: TMOE_AO(16); break;
        default: TMOE_AO(0); break;
    }
#undef TMOE_AO
    return hipGetLastError();
}

hipError_t launch_attn_decode(const void* q, const void* kc, const void* vc, const int32_t* len, int64_t T, int nq,
                              int nkv, int max_len, float* pm, float* pl, float* pacc, void* o, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int nch = attn_chunks(max_len);
    dim3 grid((unsigned)nch, (unsigned)nkv, (unsigned)T);
    const int G = nq / nkv;
    const bf16_t *qb = (const bf16_t*)q, *kb = (const bf16_t*)kc, *vb = (const bf16_t*)vc;
    bf16_t* ob = (bf16_t*)o;
#define TMOE_AP(GG, NW)                                                                                        \
    attn_partial_kernel<GG, NW, false><<<grid, 64 * NW, 0, st>>>(qb, kb, vb, len, nkv, max_len, nch, pm, pl, pacc, \
                                                                 ob, RopeArgs{})
#define TMOE_AP_G(NW)                \
    if (G == 8) TMOE_AP(8, NW);      \
    else if (G == 4) TMOE_AP(4, NW); \
    else if (G == 2) TMOE_AP(2, NW); \
    else TMOE_AP(1, NW);
    if (attn_waves(max_len) == kAttnWavesLong) { TMOE_AP_G(kAttnWavesLong) }
    else { TMOE_AP_G(kAttnWavesShort) }
#undef TMOE_AP_G
#undef TMOE_AP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nch == 1) return e;  // a single chunk wrote the output itself
    attn_combine_kernel<<<dim3((unsigned)nq, (unsigned)T), kHead, 0, st>>>(pm, pl, pacc, len, nq, nkv, max_len, nch,
                                                                          (bf16_t*)o);
    return hipGetLastError();
}

bool attn_rope_fused_ok(int nq, int nkv, int max_len) { return nq / nkv + 2 <= attn_waves(max_len); }

hipError_t launch_attn_rope_decode(const float* qkv, int KS, int64_t T, int nq, int nkv, const float* q_gain,
                                   const float* k_gain, float eps, const int32_t* pos, const int32_t* len,
                                   int max_len, int sec_h, int sec_w, double theta, void* kc, void* vc, float* pm,
                                   float* pl, float* pacc, void* o, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (!attn_rope_fused_ok(nq, nkv, max_len)) return hipErrorInvalidValue;
    const int nch = attn_chunks(max_len);
    dim3 grid((unsigned)nch, (unsigned)nkv, (unsigned)T);
    const int G = nq / nkv;
    const RopeArgs ra{qkv, KS, q_gain, k_gain, eps, pos, sec_h, sec_w, log(theta), (bf16_t*)kc, (bf16_t*)vc};
    const bf16_t *kb = (const bf16_t*)kc, *vb = (const bf16_t*)vc;
    bf16_t* ob = (bf16_t*)o;
#define TMOE_AF(GG, NW)                                                                                        \
    attn_partial_kernel<GG, NW, true><<<grid, 64 * NW, 0, st>>>(nullptr, kb, vb, len, nkv, max_len, nch, pm, pl, \
                                                                pacc, ob, ra)
    if (attn_waves(max_len) == kAttnWavesLong) {
        if (G == 8) TMOE_AF(8, kAttnWavesLong);
        else if (G == 4) TMOE_AF(4, kAttnWavesLong);
        else if (G == 2) TMOE_AF(2, kAttnWavesLong);
        else TMOE_AF(1, kAttnWavesLong);
    } else {
        if (G == 2) TMOE_AF(2, kAttnWavesShort);
        else if (G == 1) TMOE_AF(1, kAttnWavesShort);
        else return hipErrorInvalidValue;
    }
#undef TMOE_AF
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nch == 1) return e;  // a single chunk wrote the output itself
    attn_combine_kernel<<<dim3((unsigned)nq, (unsigned)T), kHead, 0, st>>>(pm, pl, pacc, len, nq, nkv, max_len, nch,
                                                                          (bf16_t*)o);
    return hipGetLastError();
}

}  // namespace tmoe
