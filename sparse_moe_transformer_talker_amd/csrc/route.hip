// Router scores, softmax, exact Top-k with renormalisation, and the codec-head
// argmax ("3C · Talker MoE (20 lớp, 128 Experts Top-6)", openarchlab, §3:
// p = softmax(W_r x), S = Top-6 of p, w_i = p_i / sum_{j in S} p_j; §1:
// codec_head 1024 -> 3072 picks c_0).
//
// Exact selection.  Each score s_e is accumulated from fp32 partial sums of
// 32 exact products (one matrix-core step, or 32 fp32 FMAs) added in fp64, and
// comes with a rigorous bound d_e on its distance to the exact value:
//   |s_e - exact_e| <= d_e = 33 * 2^-23 * (1 + 2^-9) * sum_h |x_h W_eh|  (+ tiny fp64 terms)
// (32 roundings per partial, counted at twice the round-to-nearest unit so
// truncating hardware is covered too).  Selection first runs on the scores
// rounded to fp32 (bound widened by that rounding): a token's Top-k is certain
// when every selected interval [s - d, s + d] lies strictly above every other
// interval that could displace it and the selected intervals are strictly
// ordered.  Otherwise the candidates are rescored in fp64 (bf16 and fp32
// products are exact in fp64) and selected again.  The result is the Top-k of
// the exact scores with ties to the lower index.
//
// The router also writes, per block of 16 tokens, a 16-bit mask per expert of
// which tokens chose it; the grouping kernels derive the stable per-expert
// order from these masks.
#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {

constexpr float kTwoM23 = 1.1920928955078125e-07f;
// per-32-term partial error (33 * 2^-23) with margin for the abs-sum's own rounding
__device__ __forceinline__ double partial_error_scale() { return 33.0 * 1.1920928955078125e-07 * (1.0 + 1.0 / 512); }
__device__ __forceinline__ double fp64_error_scale(int H) { return (double)(H / 32 + 8) * 2.220446049250313e-16; }

// ---------------------------------------------------------------------------
// fp64 rescoring of up to 4 candidates at once: dot(x_row, W[e_i]) over H,
// wave-cooperative, 16-byte loads issued for all candidates before use.
template <typename T>
__device__ void wave_dot64_x4(const T* __restrict__ xr, const T* __restrict__ W, int H, const int* e, int n,
                              double* out) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
    if (H % V == 0) {
        for (int c = lane_id(); c < H / V; c += kWave) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + c * V);
            u32x4 wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < n) wv[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)e[i] * H + c * V);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= n) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (sizeof(T) == 2) {
                        acc[i] = fma((double)__uint_as_float(xv[q] << 16), (double)__uint_as_float(wv[i][q] << 16),
                                     acc[i]);
                        acc[i] = fma((double)__uint_as_float(xv[q] & 0xFFFF0000u),
                                     (double)__uint_as_float(wv[i][q] & 0xFFFF0000u), acc[i]);
                    } else {
                        acc[i] = fma((double)__uint_as_float(xv[q]), (double)__uint_as_float(wv[i][q]), acc[i]);
                    }
                }
            }
        }
    } else {
        for (int h = lane_id(); h < H; h += kWave) {
            const double xv = Elem<T>::load64(xr, h);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < n) acc[i] = fma(xv, Elem<T>::load64(W + (int64_t)e[i] * H, h), acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = wave_sum(acc[i]);
}

// Per-wave selection state in LDS.
struct SelScratch {
    int idx[kMaxTopK];
    double score[kMaxTopK];
};

// Exact Top-k of one row of scores s[0..n) (fp32 or fp64) with error bounds
// d[0..n); writes idx / weights / probs and, when mask != nullptr, ORs bit
// `bit` into mask[e] for every selected e (LDS).  Called by one full wave;
// lanes own entries e = lane + 64 j.
template <typename T, int MAXJ, typename S>
__device__ void exact_select_row(const S* s, const float* d, int n, int k, const T* xrow, const T* W, int H,
                                 const float* bias, SelScratch* sc, int norm, int32_t* out_idx, float* out_w,
                                 float* out_probs, uint32_t* mask, int bit) {
    const int lane = lane_id();
    float v[MAXJ];
    double dv[MAXJ];
    bool taken[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        const int e = lane + kWave * j;
        const bool ok = e < n;
        v[j] = ok ? (float)s[e] + 0.0f : 0.0f;
        // bound of the fp32 value: the score's bound plus its rounding to fp32
        dv[j] = ok ? (double)d[e] + 1.1920928955078125e-07 * fabs((double)v[j]) : 0.0;
        taken[j] = !ok;  // out-of-range entries never compete
    }
    double low = 1.0e300;   // min over selected of (s - d)
    double prev_lo = 0.0;   // previous selected (s - d)
    bool certain = true;
    for (int r = 0; r < k; ++r) {
        uint64_t key = 0;
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            if (taken[j]) continue;
            const uint64_t kk = rank_key(v[j], lane + kWave * j);
            key = kk > key ? kk : key;
        }
        key = wave_max_key(key);
        const int bi = rank_key_index(key);
        const double bv = (double)float_from_order_key((uint32_t)(key >> 32));
        double bd = 0.0;
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            if ((bi >> 6) == j && (bi & 63) == lane) { taken[j] = true; bd = dv[j]; }
        bd = __shfl(bd, bi & 63, kWave);
        if (r > 0 && !(prev_lo > bv + bd)) certain = false;
        prev_lo = bv - bd;
        low = fmin(low, bv - bd);
        if (lane == 0) { sc->idx[r] = bi; sc->score[r] = bv; }
    }
    bool threat = false;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
        if (!taken[j] && (double)v[j] + dv[j] >= low) threat = true;
    if (__ballot(threat) != 0ull) certain = false;

    if (!certain) {
        // Candidates: the selected ones and every other one that may reach them.
        bool cand[MAXJ];
        double v64[MAXJ];
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int e = lane + kWave * j;
            cand[j] = (e < n) && (taken[j] || (double)v[j] + dv[j] >= low);
            v64[j] = 0.0;
        }
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            uint64_t m = __ballot(cand[j]);
            while (m) {
                int ids[4], cnt = 0;
                while (m && cnt < 4) {
                    ids[cnt++] = (__ffsll((unsigned long long)m) - 1) + kWave * j;
                    m &= m - 1;
                }
                double r4[4];
                wave_dot64_x4(xrow, W, H, ids, cnt, r4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < cnt) {
                        const double sc64 = r4[i] + (bias ? (double)bias[ids[i]] : 0.0);
                        if (lane == ids[i] - kWave * j) v64[j] = sc64;
                    }
                }
            }
        }
        for (int r = 0; r < k; ++r) {
            double bv = 0.0;
            int bi = -1;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                const int e = lane + kWave * j;
                if (cand[j] && (bi < 0 || ranks_before(v64[j], e, bv, bi))) { bv = v64[j]; bi = e; }
            }
            wave_best(bv, bi);
#pragma unroll
            for (int j = 0; j < MAXJ; ++j)
                if (lane + kWave * j == bi) cand[j] = false;
            if (lane == 0) { sc->idx[r] = bi; sc->score[r] = bv; }
        }
    }
    __builtin_amdgcn_wave_barrier();

    // Outputs.  Softmax statistics over all n scores in fp32 (probs and the
    // plain, non-renormalised weights); renormalised weights from differences
    // of the selected scores.
    float mx = -3.0e38f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
        if (lane + kWave * j < n) mx = fmaxf(mx, v[j]);
    mx = wave_max_dpp(mx);
    float z = 0.f;
    if (out_probs || !norm) {
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            if (lane + kWave * j < n) z += __expf(v[j] - mx);
        z = wave_sum_dpp(z);
    }
    if (out_probs) {
        const float inv = 1.0f / z;
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int e = lane + kWave * j;
            if (e < n) out_probs[e] = __expf(v[j] - mx) * inv;
        }
    }
    const double s0 = sc->score[0];
    float ex = 0.f;
    int my_e = 0;
    if (lane < k) {
        my_e = sc->idx[lane];
        ex = norm ? __expf((float)(sc->score[lane] - s0)) : __expf((float)s[my_e] - mx);
    }
    const float den = norm ? wave_sum_dpp(ex) : z;
    if (lane < k) {
        out_idx[lane] = my_e;
        out_w[lane] = ex / den;
        if (mask) atomicOr(&mask[my_e], 1u << bit);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core scores for 16 tokens x (NS*16) weight rows.  The NW waves of the
// block take the 32-wide K steps round robin (any H % 32 == 0); each step is
// a fresh fp32 partial added into fp64.  Partials of the waves are reduced into
// LDS in fixed wave order (deterministic).  Rows/tokens beyond the limits are
// clamped on load and their outputs are never read.
template <int NS, int NW>
__device__ void mfma_scores_tile(const bf16_t* __restrict__ x, int64_t T, int H, int64_t tok0,
                                 const bf16_t* __restrict__ W, int nrows, int e0, double* lg, float* ab, int ld) {
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    double acc[NS][4];
    f32x4 aacc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        aacc[s] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][r] = 0.0;
    }
    int64_t tok = tok0 + i;
    if (tok >= T) tok = T - 1;
    const bf16_t* xp = x + tok * (int64_t)H + kq;
    const bf16_t* wp[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        int r = e0 + s * 16 + i;
        if (r >= nrows) r = nrows - 1;
        wp[s] = W + (int64_t)r * H + kq;
    }
    const int nsteps = H / 32;
    const u32x4 absmask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    const f32x4 zero = {0, 0, 0, 0};
    if (wave < nsteps) {
        // software pipeline: the next step's operands load while this step computes
        u32x4 a = *reinterpret_cast<const u32x4*>(xp + wave * 32);
        u32x4 b[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) b[s] = *reinterpret_cast<const u32x4*>(wp[s] + wave * 32);
        for (int st = wave; st < nsteps; st += NW) {
            const int kn = (st + NW < nsteps ? st + NW : st) * 32;
            const u32x4 an = *reinterpret_cast<const u32x4*>(xp + kn);
            u32x4 bn[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) bn[s] = *reinterpret_cast<const u32x4*>(wp[s] + kn);
            const u32x4 aa = a & absmask;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b[s]), zero, 0, 0, 0);
                aacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aa),
                                                                  __builtin_bit_cast(bf16x8, b[s] & absmask),
                                                                  aacc[s], 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[s][r] += (double)p[r];
            }
            a = an;
#pragma unroll
            for (int s = 0; s < NS; ++s) b[s] = bn[s];
        }
    }
    // D[row = 4*(lane/16) + r][col = lane%16] per 16x16 block
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int q = ((lane >> 4) * 4 + r) * ld + s * 16 + i;
                    if (w == 0) { lg[q] = acc[s][r]; ab[q] = aacc[s][r]; }
                    else { lg[q] += acc[s][r]; ab[q] += aacc[s][r]; }
                }
        }
        __syncthreads();
    }
}

constexpr int kRouteWaves = 8;

// Fused route for bf16, E <= NS*16 <= 128, H % 32 == 0: 16 tokens per block.
// masks (nullable): [E][mstride] uint16, word = blockIdx.x, bit = token % 16.
template <int NS>
__global__ __launch_bounds__(64 * kRouteWaves) void route_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ bias, int64_t T, int H,
    int E, int k, int norm, int32_t* __restrict__ out_idx, float* __restrict__ out_w, float* __restrict__ out_probs,
    uint16_t* __restrict__ masks, int mstride) {
    constexpr int LD = NS * 16;
    __shared__ double lg[16 * LD];
    __shared__ float ab[16 * LD];
    __shared__ SelScratch sc[kRouteWaves];
    __shared__ uint32_t msk[LD];
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    for (int q = threadIdx.x; q < LD; q += blockDim.x) msk[q] = 0;
    mfma_scores_tile<NS, kRouteWaves>(x, T, H, tok0, W, E, 0, lg, ab, LD);
    const double es = partial_error_scale(), fs = fp64_error_scale(H);
    for (int q = threadIdx.x; q < 16 * LD; q += blockDim.x) {
        const int e = q % LD;
        const float b = (bias && e < E) ? bias[e] : 0.f;
        const double sv = lg[q] + (double)b;
        lg[q] = sv;
        const double a = (double)ab[q];
        ab[q] = (float)(es * a + fs * (a + fabs((double)b))) * (1.0f + kTwoM23);
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    for (int tt = wave; tt < 16; tt += kRouteWaves) {
        const int64_t t = tok0 + tt;
        if (t >= T) break;
        exact_select_row<bf16_t, (LD + 63) / 64, double>(lg + tt * LD, ab + tt * LD, E, k, x + t * H, W, H, bias,
                                                         &sc[wave], norm, out_idx + t * k, out_w + t * k,
                                                         out_probs ? out_probs + t * E : nullptr, msk, tt);
    }
    if (masks) {
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += blockDim.x) masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
    }
}

// ---------------------------------------------------------------------------
// Portable scores: one lane per weight row, 32-term fp32 partials added in
// fp64; writes fp32 scores and bounds (including the final rounding to fp32)
// to global [T, n].  Any H, any element type.
template <typename T>
__global__ __launch_bounds__(256) void scores_generic_kernel(const T* __restrict__ x, const T* __restrict__ W,
                                                             const float* __restrict__ bias, int64_t Ttok,
                                                             int H, int n, float* __restrict__ sc,
                                                             float* __restrict__ bd) {
    const int64_t t = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= Ttok || e >= n) return;
    const T* xr = x + t * H;
    const T* wr = W + (int64_t)e * H;
    double acc = 0.0;
    float aacc = 0.f;
    for (int h0 = 0; h0 < H; h0 += 32) {
        float part = 0.f;
        const int h1 = min(h0 + 32, H);
        for (int h = h0; h < h1; ++h) {
            const float a = Elem<T>::load(xr, h), b = Elem<T>::load(wr, h);
            part = fmaf(a, b, part);
            aacc = fmaf(fabsf(a), fabsf(b), aacc);
        }
        acc += (double)part;
    }
    const float b = bias ? bias[e] : 0.f;
    const double sv = acc + (double)b;
    // fp32 FMA partials: 32 roundings each; the abs-sum's own fp32 rounding is
    // covered by a relative (H + 8) * 2^-23 margin; storing the score in fp32
    // adds half an ulp.
    const double a = (double)aacc * (1.0 + (double)(H + 8) * 1.1920928955078125e-07);
    const double bound = partial_error_scale() * a + fp64_error_scale(H) * (a + fabs((double)b)) +
                         0.5 * 1.1920928955078125e-07 * fabs(sv);
    sc[t * n + e] = (float)sv;
    bd[t * n + e] = (float)bound * (1.0f + kTwoM23);
}

// Matrix-core scores to global [T, n] (bf16, H % 32 == 0): 16 tokens x 128 rows per block.
__global__ __launch_bounds__(64 * kRouteWaves) void scores_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ bias, int64_t T, int H,
    int n, float* __restrict__ sc, float* __restrict__ bd) {
    constexpr int NS = 8, LD = NS * 16;
    __shared__ double lg[16 * LD];
    __shared__ float ab[16 * LD];
    const int64_t tok0 = (int64_t)blockIdx.y * 16;
    const int e0 = blockIdx.x * LD;
    mfma_scores_tile<NS, kRouteWaves>(x, T, H, tok0, W, n, e0, lg, ab, LD);
    const double es = partial_error_scale(), fs = fp64_error_scale(H);
    for (int q = threadIdx.x; q < 16 * LD; q += blockDim.x) {
        const int row = q / LD, col = q % LD;
        const int64_t t = tok0 + row;
        const int e = e0 + col;
        if (t >= T || e >= n) continue;
        const float b = bias ? bias[e] : 0.f;
        const double sv = lg[q] + (double)b;
        const double a = (double)ab[q];
        sc[t * n + e] = (float)sv;
        bd[t * n + e] = (float)(es * a + fs * (a + fabs((double)b)) + 0.5 * 1.1920928955078125e-07 * fabs(sv)) *
                        (1.0f + kTwoM23);
    }
}

// Exact Top-k from global fp32 scores: 16 tokens per block, 4 per wave (n <= 1024).
template <typename T, int MAXJ>
__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ sc, const float* __restrict__ bd,
                                                          const T* __restrict__ x, const T* __restrict__ W,
                                                          const float* __restrict__ bias, int64_t Ttok, int H,
                                                          int n, int k, int norm, int32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_w, float* __restrict__ out_probs,
                                                          uint16_t* __restrict__ masks, int mstride) {
    __shared__ SelScratch scr[4];
    __shared__ uint32_t msk[kMaxExperts];
    for (int q = threadIdx.x; q < n; q += blockDim.x) msk[q] = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    for (int tt = wave; tt < 16; tt += 4) {
        const int64_t t = tok0 + tt;
        if (t >= Ttok) break;
        exact_select_row<T, MAXJ, float>(sc + t * n, bd + t * n, n, k, x + t * H, W, H, bias, &scr[wave], norm,
                                         out_idx + t * k, out_w + t * k, out_probs ? out_probs + t * n : nullptr,
                                         msk, tt);
    }
    if (masks) {
        __syncthreads();
        for (int e = threadIdx.x; e < n; e += blockDim.x) masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
    }
}

// Exact argmax over n scores of any length: one wave per token.
template <typename T>
__global__ __launch_bounds__(256) void argmax_exact_kernel(const float* __restrict__ sc, const float* __restrict__ bd,
                                                           const T* __restrict__ x, const T* __restrict__ W,
                                                           int64_t Ttok, int H, int n, int32_t* __restrict__ out) {
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= Ttok) return;
    const float* s = sc + t * n;
    const float* d = bd + t * n;
    // fp32 argmax and a lower bound of the maximum (interval ends in fp64)
    uint64_t key = 0;
    double low = -1.0e300;
    for (int e = lane; e < n; e += kWave) {
        const uint64_t kk = rank_key(s[e], e);
        key = kk > key ? kk : key;
        low = fmax(low, (double)s[e] - (double)d[e]);
    }
    key = wave_max_key(key);
    int bi = rank_key_index(key);
    for (int o = 32; o > 0; o >>= 1) low = fmax(low, __shfl_xor(low, o, kWave));
    int ncand = 0;
    for (int e = lane; e < n; e += kWave) ncand += ((double)s[e] + (double)d[e] >= low) ? 1 : 0;
    ncand = __builtin_amdgcn_readlane(wave_incl_scan(ncand), 63);
    if (ncand > 1) {
        double best = 0.0;
        int besti = -1;
        const T* xr = x + t * H;
        for (int base = 0; base < n; base += kWave) {
            const int e = base + lane;
            const bool c = e < n && (double)s[e] + (double)d[e] >= low;
            uint64_t m = __ballot(c);
            while (m) {
                int ids[4], cnt = 0;
                while (m && cnt < 4) {
                    ids[cnt++] = base + __ffsll((unsigned long long)m) - 1;
                    m &= m - 1;
                }
                double r4[4];
                wave_dot64_x4(xr, W, H, ids, cnt, r4);
                for (int i = 0; i < cnt; ++i)
                    if (besti < 0 || ranks_before(r4[i], ids[i], best, besti)) { best = r4[i]; besti = ids[i]; }
            }
        }
        bi = besti;
    }
    if (lane == 0) out[t] = bi;
}

// ---------------------------------------------------------------------------
// Host-side launchers.
template <typename T>
static hipError_t launch_select(const float* sc, const float* bd, const T* x, const T* W, const float* bias,
                                int64_t Ttok, int H, int n, int k, int norm, int32_t* idx, float* w, float* probs,
                                uint16_t* masks, int mstride, hipStream_t st) {
    dim3 grid((unsigned)((Ttok + 15) / 16));
#define TMOE_SEL(J)                                                                                      \
    select_topk_kernel<T, J><<<grid, 256, 0, st>>>(sc, bd, x, W, bias, Ttok, H, n, k, norm, idx, w, probs, \
                                                   masks, mstride)
    if (n <= 64) TMOE_SEL(1);
    else if (n <= 128) TMOE_SEL(2);
    else if (n <= 256) TMOE_SEL(4);
    else if (n <= 512) TMOE_SEL(8);
    else TMOE_SEL(16);
#undef TMOE_SEL
    return hipGetLastError();
}

static bool mfma_scores_ok(int dtype, int H) { return dtype == kBF16 && H % 32 == 0; }

hipError_t launch_scores(int dtype, const void* x, const void* W, const float* bias, int64_t Ttok, int H, int n,
                         float* sc, float* bd, hipStream_t st) {
    if (mfma_scores_ok(dtype, H)) {
        dim3 grid((unsigned)((n + 127) / 128), (unsigned)((Ttok + 15) / 16));
        scores_mfma_kernel<<<grid, 64 * kRouteWaves, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, n,
                                                              sc, bd);
    } else {
        dim3 grid((unsigned)((n + 255) / 256), (unsigned)Ttok);
        if (dtype == kBF16)
            scores_generic_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, n,
                                                                 sc, bd);
        else
            scores_generic_kernel<float><<<grid, 256, 0, st>>>((const float*)x, (const float*)W, bias, Ttok, H, n,
                                                                sc, bd);
    }
    return hipGetLastError();
}

bool route_fused_ok(int dtype, int H, int E) { return mfma_scores_ok(dtype, H) && E % 16 == 0 && E <= 128; }

hipError_t launch_route(int dtype, const void* x, const void* W, const float* bias, int64_t Ttok, int H, int E,
                        int k, int norm, int32_t* idx, float* w, float* probs, float* scratch_sc,
                        float* scratch_bd, uint16_t* masks, hipStream_t st) {
    // one block per 16 tokens (one mask word); mask rows are mask_stride(T) words apart
    const int nwords = mask_words(Ttok), mstride = mask_stride(Ttok);
    if (route_fused_ok(dtype, H, E)) {
        dim3 grid((unsigned)nwords);
        const bf16_t* xb = (const bf16_t*)x;
        const bf16_t* wb = (const bf16_t*)W;
#define TMOE_ROUTE(NS)                                                                                       \
    route_mfma_kernel<NS><<<grid, 64 * kRouteWaves, 0, st>>>(xb, wb, bias, Ttok, H, E, k, norm, idx, w, probs, \
                                                             masks, mstride)
        if (E <= 16) TMOE_ROUTE(1);
        else if (E <= 32) TMOE_ROUTE(2);
        else if (E <= 64) TMOE_ROUTE(4);
        else TMOE_ROUTE(8);
#undef TMOE_ROUTE
        return hipGetLastError();
    }
    hipError_t err = launch_scores(dtype, x, W, bias, Ttok, H, E, scratch_sc, scratch_bd, st);
    if (err != hipSuccess) return err;
    if (dtype == kBF16)
        return launch_select<bf16_t>(scratch_sc, scratch_bd, (const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, E, k,
                                     norm, idx, w, probs, masks, mstride, st);
    return launch_select<float>(scratch_sc, scratch_bd, (const float*)x, (const float*)W, bias, Ttok, H, E, k, norm,
                                idx, w, probs, masks, mstride, st);
}

hipError_t launch_argmax(int dtype, const float* sc, const float* bd, const void* x, const void* W, int64_t Ttok,
                         int H, int n, int32_t* out, hipStream_t st) {
    dim3 grid((unsigned)((Ttok + 3) / 4));
    if (dtype == kBF16)
        argmax_exact_kernel<bf16_t><<<grid, 256, 0, st>>>(sc, bd, (const bf16_t*)x, (const bf16_t*)W, Ttok, H, n, out);
    else
        argmax_exact_kernel<float><<<grid, 256, 0, st>>>(sc, bd, (const float*)x, (const float*)W, Ttok, H, n, out);
    return hipGetLastError();
}

}  // namespace tmoe
