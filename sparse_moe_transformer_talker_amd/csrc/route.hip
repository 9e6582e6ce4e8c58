// Router scores, softmax, exact Top-k with renormalisation, and the codec-head
// argmax ("3C · Talker MoE (20 lớp, 128 Experts Top-6)", openarchlab, §3:
// p = softmax(W_r x), S = Top-6 of p, w_i = p_i / sum_{j in S} p_j; §1:
// codec_head 1024 -> 3072 picks c_0).
//
// Exact selection.  Scores are computed in fp32 (bf16 matrix cores or fp32
// FMA) together with sum_h |x_h W_eh|, which bounds each score's rounding error
// d_e.  A token's fp32 Top-k is certain when every selected score's interval
// [s - d, s + d] lies strictly above every other interval that could displace
// it, and the selected intervals are strictly ordered.  Otherwise the possible
// candidates are rescored in fp64 (bf16 and fp32 products are exact in fp64)
// and selected again.  The result equals the Top-k of the exact scores with
// ties to the lower index.
#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {

// ---------------------------------------------------------------------------
// fp64 rescoring of one candidate: dot(x_row, w_row) over H, wave-cooperative.
template <typename T>
__device__ double wave_dot64(const T* __restrict__ xr, const T* __restrict__ wr, int H) {
    double acc = 0.0;
    for (int h = lane_id(); h < H; h += kWave) acc = fma(Elem<T>::load64(xr, h), Elem<T>::load64(wr, h), acc);
    return wave_sum(acc);
}

// Per-wave selection state in LDS.
struct SelScratch {
    int idx[kMaxTopK];
    double score[kMaxTopK];
};

// Select the top-k (or argmax when k == 1 and weights are not wanted) of one
// row of fp32 scores s[0..n) with error bounds d[0..n), exactly, then write
// outputs.  Lanes own entries e = lane + 64 j.  Called by one full wave.
template <typename T, int MAXJ>
__device__ void exact_select_row(const float* s, const float* d, int n, int k,
                                 const T* xrow, const T* W, int H, const float* bias,
                                 SelScratch* sc, int norm, int32_t* out_idx, float* out_w,
                                 float* out_probs) {
    const int lane = lane_id();
    float v[MAXJ], dv[MAXJ];
    bool taken[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        int e = lane + kWave * j;
        bool ok = e < n;
        v[j] = ok ? s[e] : 0.f;
        dv[j] = ok ? d[e] : 0.f;
        taken[j] = !ok;  // out-of-range entries never compete
    }
    // fp32 pass
    float low = 3.0e38f;          // min over selected of (s - d)
    float prev_lo = 0.f;          // previous selected (s - d)
    bool certain = true;
    for (int r = 0; r < k; ++r) {
        float bv = 0.f;
        int bi = -1;
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            int e = lane + kWave * j;
            if (!taken[j] && (bi < 0 || ranks_before(v[j], e, bv, bi))) { bv = v[j]; bi = e; }
        }
        wave_best(bv, bi);
        // everyone knows (bv, bi); the owner marks it taken
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            if (lane + kWave * j == bi) taken[j] = true;
        float bd = d[bi];
        if (r > 0 && !(prev_lo > bv + bd)) certain = false;
        prev_lo = bv - bd;
        low = fminf(low, bv - bd);
        if (lane == 0) { sc->idx[r] = bi; sc->score[r] = (double)bv; }
    }
    // can any unselected score reach the selected ones?
    bool threat = false;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
        if (!taken[j] && v[j] + dv[j] >= low) threat = true;
    if (__ballot(threat) != 0ull) certain = false;

    if (!certain) {
        // Candidates: selected ones and every unselected one that may reach them.
        bool cand[MAXJ];
        double v64[MAXJ];
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            int e = lane + kWave * j;
            cand[j] = (e < n) && (taken[j] || v[j] + dv[j] >= low);
            v64[j] = 0.0;
        }
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            uint64_t m = __ballot(cand[j]);
            while (m) {
                int src = __ffsll((unsigned long long)m) - 1;
                m &= m - 1;
                int e = src + kWave * j;
                double sc64 = wave_dot64(xrow, W + (int64_t)e * H, H);
                if (bias) sc64 += (double)bias[e];
                if (lane == src) v64[j] = sc64;
            }
        }
        for (int r = 0; r < k; ++r) {
            double bv = 0.0;
            int bi = -1;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                int e = lane + kWave * j;
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
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // Outputs.  Full softmax statistics in fp32 (needed for probs and for the
    // plain, non-renormalised weights).
    float m = -3.0e38f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
        if (lane + kWave * j < n) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float z = 0.f;
    if (out_probs || !norm) {
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            if (lane + kWave * j < n) z += __expf(v[j] - m);
        z = wave_sum(z);
    }
    if (out_probs) {
        float inv = 1.0f / z;
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            int e = lane + kWave * j;
            if (e < n) out_probs[e] = __expf(v[j] - m) * inv;
        }
    }
    if (out_w) {
        // weights of the selected experts: renormalised over S, or plain p
        double s0 = sc->score[0];
        float ex = 0.f;
        if (lane < k) {
            if (norm) ex = __expf((float)(sc->score[lane] - s0));
            else ex = __expf(s[sc->idx[lane]] - m);
        }
        float den = norm ? wave_sum(ex) : z;
        if (lane < k) {
            out_idx[lane] = sc->idx[lane];
            out_w[lane] = ex / den;
        }
    } else if (lane < k) {
        out_idx[lane] = sc->idx[lane];
    }
}

// ---------------------------------------------------------------------------
// Matrix-core scores for a tile of 16 tokens x (NS*16) weight rows, K split
// over the 4 waves of the block.  Each wave's partial sums are reduced into
// LDS in fixed wave order (deterministic).  Rows/tokens beyond the limits are
// clamped on load and their outputs are never read.
template <int NS>
__device__ void mfma_scores_tile(const bf16_t* __restrict__ x, int64_t T, int H, int64_t tok0,
                                 const bf16_t* __restrict__ W, int nrows, int e0,
                                 float* lg, float* ab, int ld) {
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    f32x4 acc[NS], aacc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) { acc[s] = f32x4{0, 0, 0, 0}; aacc[s] = f32x4{0, 0, 0, 0}; }
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
    const int kspan = H / 4;
    const int kbeg = wave * kspan;
    const u32x4 absmask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    for (int k0 = kbeg; k0 < kbeg + kspan; k0 += 32) {
        u32x4 a = *reinterpret_cast<const u32x4*>(xp + k0);
        u32x4 b[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) b[s] = *reinterpret_cast<const u32x4*>(wp[s] + k0);
        u32x4 aa = a & absmask;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, b[s]), acc[s], 0, 0, 0);
            u32x4 bb = b[s] & absmask;
            aacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aa),
                                                              __builtin_bit_cast(bf16x8, bb), aacc[s], 0, 0, 0);
        }
    }
    // D[row = 4*(lane/16) + r][col = lane%16] per 16x16 block
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int row = (lane >> 4) * 4 + r;
                    int col = s * 16 + i;
                    if (w == 0) { lg[row * ld + col] = acc[s][r]; ab[row * ld + col] = aacc[s][r]; }
                    else { lg[row * ld + col] += acc[s][r]; ab[row * ld + col] += aacc[s][r]; }
                }
        }
        __syncthreads();
    }
}

// Fused route for bf16, E <= NS*16 <= 128, H % 128 == 0: 16 tokens per block.
template <int NS>
__global__ __launch_bounds__(256) void route_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                         const float* __restrict__ bias, int64_t T, int H, int E,
                                                         int k, int norm, int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_w, float* __restrict__ out_probs) {
    constexpr int LD = NS * 16;
    __shared__ float lg[16 * LD];
    __shared__ float ab[16 * LD];
    __shared__ SelScratch sc[4];
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    mfma_scores_tile<NS>(x, T, H, tok0, W, E, 0, lg, ab, LD);
    const float es = dot_error_scale(H);
    for (int q = threadIdx.x; q < 16 * LD; q += blockDim.x) {
        int e = q % LD;
        float b = (bias && e < E) ? bias[e] : 0.f;
        float sv = lg[q] + b;
        lg[q] = sv;
        ab[q] = es * (ab[q] + fabsf(b)) + 1.1920928955078125e-07f * fabsf(sv);
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    for (int tt = wave; tt < 16; tt += 4) {
        int64_t t = tok0 + tt;
        if (t >= T) break;
        exact_select_row<bf16_t, (LD + 63) / 64>(lg + tt * LD, ab + tt * LD, E, k, x + t * H, W, H, bias,
                                                 &sc[wave], norm, out_idx + t * k, out_w + t * k,
                                                 out_probs ? out_probs + t * E : nullptr);
    }
}

// ---------------------------------------------------------------------------
// Portable scores: one lane per weight row, fp32 FMA over H; writes scores and
// bounds to global [T, n].  Any H, any element type.
template <typename T>
__global__ __launch_bounds__(256) void scores_generic_kernel(const T* __restrict__ x, const T* __restrict__ W,
                                                             const float* __restrict__ bias, int64_t Ttok,
                                                             int H, int n, float* __restrict__ sc,
                                                             float* __restrict__ bd) {
    int64_t t = blockIdx.y;
    int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= Ttok || e >= n) return;
    const T* xr = x + t * H;
    const T* wr = W + (int64_t)e * H;
    float acc = 0.f, aacc = 0.f;
    for (int h = 0; h < H; ++h) {
        float a = Elem<T>::load(xr, h), b = Elem<T>::load(wr, h);
        acc = fmaf(a, b, acc);
        aacc = fmaf(fabsf(a), fabsf(b), aacc);
    }
    float b = bias ? bias[e] : 0.f;
    float sv = acc + b;
    sc[t * n + e] = sv;
    bd[t * n + e] = dot_error_scale(H) * (aacc + fabsf(b)) + 1.1920928955078125e-07f * fabsf(sv);
}

// Matrix-core scores to global [T, n] (bf16, H % 128 == 0): 16 tokens x 128 rows per block.
__global__ __launch_bounds__(256) void scores_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                          const float* __restrict__ bias, int64_t T, int H, int n,
                                                          float* __restrict__ sc, float* __restrict__ bd) {
    constexpr int NS = 8, LD = NS * 16;
    __shared__ float lg[16 * LD];
    __shared__ float ab[16 * LD];
    const int64_t tok0 = (int64_t)blockIdx.y * 16;
    const int e0 = blockIdx.x * LD;
    mfma_scores_tile<NS>(x, T, H, tok0, W, n, e0, lg, ab, LD);
    const float es = dot_error_scale(H);
    for (int q = threadIdx.x; q < 16 * LD; q += blockDim.x) {
        int row = q / LD, col = q % LD;
        int64_t t = tok0 + row;
        int e = e0 + col;
        if (t >= T || e >= n) continue;
        float b = bias ? bias[e] : 0.f;
        float sv = lg[q] + b;
        sc[t * n + e] = sv;
        bd[t * n + e] = es * (ab[q] + fabsf(b)) + 1.1920928955078125e-07f * fabsf(sv);
    }
}

// Exact Top-k from global scores: one wave per token (n <= 1024).
template <typename T, int MAXJ>
__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ sc, const float* __restrict__ bd,
                                                          const T* __restrict__ x, const T* __restrict__ W,
                                                          const float* __restrict__ bias, int64_t Ttok, int H,
                                                          int n, int k, int norm, int32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_w, float* __restrict__ out_probs) {
    __shared__ SelScratch scr[4];
    const int wave = threadIdx.x >> 6;
    int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= Ttok) return;
    exact_select_row<T, MAXJ>(sc + t * n, bd + t * n, n, k, x + t * H, W, H, bias, &scr[wave], norm,
                              out_idx + t * k, out_w + t * k, out_probs ? out_probs + t * n : nullptr);
}

// Exact argmax over n scores of any length: one wave per token.
template <typename T>
__global__ __launch_bounds__(256) void argmax_exact_kernel(const float* __restrict__ sc, const float* __restrict__ bd,
                                                           const T* __restrict__ x, const T* __restrict__ W,
                                                           int64_t Ttok, int H, int n, int32_t* __restrict__ out) {
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
    int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= Ttok) return;
    const float* s = sc + t * n;
    const float* d = bd + t * n;
    // fp32 argmax and the best lower bound of the maximum
    float bv = 0.f, low = -3.0e38f;
    int bi = -1;
    for (int e = lane; e < n; e += kWave) {
        float v = s[e];
        if (bi < 0 || ranks_before(v, e, bv, bi)) { bv = v; bi = e; }
        low = fmaxf(low, v - d[e]);
    }
    wave_best(bv, bi);
    low = wave_max(low);
    int ncand = 0;
    for (int e = lane; e < n; e += kWave) ncand += (s[e] + d[e] >= low) ? 1 : 0;
    for (int o = 32; o > 0; o >>= 1) ncand += __shfl_xor(ncand, o, kWave);
    if (ncand > 1) {
        double best = 0.0;
        int besti = -1;
        const T* xr = x + t * H;
        for (int base = 0; base < n; base += kWave) {
            int e = base + lane;
            bool c = e < n && s[e] + d[e] >= low;
            uint64_t m = __ballot(c);
            while (m) {
                int src = __ffsll((unsigned long long)m) - 1;
                m &= m - 1;
                int ee = base + src;
                double v64 = wave_dot64(xr, W + (int64_t)ee * H, H);
                if (besti < 0 || ranks_before(v64, ee, best, besti)) { best = v64; besti = ee; }
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
                                int64_t Ttok, int H, int n, int k, int norm, int32_t* idx, float* w,
                                float* probs, hipStream_t st) {
    dim3 grid((unsigned)((Ttok + 3) / 4));
#define TMOE_SEL(J) \
    select_topk_kernel<T, J><<<grid, 256, 0, st>>>(sc, bd, x, W, bias, Ttok, H, n, k, norm, idx, w, probs)
    if (n <= 64) TMOE_SEL(1);
    else if (n <= 128) TMOE_SEL(2);
    else if (n <= 256) TMOE_SEL(4);
    else if (n <= 512) TMOE_SEL(8);
    else TMOE_SEL(16);
#undef TMOE_SEL
    return hipGetLastError();
}

hipError_t launch_scores(int dtype, const void* x, const void* W, const float* bias, int64_t Ttok, int H, int n,
                         float* sc, float* bd, hipStream_t st) {
    if (dtype == kBF16 && H % 128 == 0) {
        dim3 grid((unsigned)((n + 127) / 128), (unsigned)((Ttok + 15) / 16));
        scores_mfma_kernel<<<grid, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, n, sc, bd);
    } else {
        dim3 grid((unsigned)((n + 255) / 256), (unsigned)Ttok);
        if (dtype == kBF16)
            scores_generic_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, n, sc, bd);
        else
            scores_generic_kernel<float><<<grid, 256, 0, st>>>((const float*)x, (const float*)W, bias, Ttok, H, n, sc, bd);
    }
    return hipGetLastError();
}

bool route_fused_ok(int dtype, int H, int E) { return dtype == kBF16 && H % 128 == 0 && E % 16 == 0 && E <= 128; }

hipError_t launch_route(int dtype, const void* x, const void* W, const float* bias, int64_t Ttok, int H, int E,
                        int k, int norm, int32_t* idx, float* w, float* probs, float* scratch_sc,
                        float* scratch_bd, hipStream_t st) {
    if (route_fused_ok(dtype, H, E)) {
        dim3 grid((unsigned)((Ttok + 15) / 16));
        const bf16_t* xb = (const bf16_t*)x;
        const bf16_t* wb = (const bf16_t*)W;
        if (E <= 16) route_mfma_kernel<1><<<grid, 256, 0, st>>>(xb, wb, bias, Ttok, H, E, k, norm, idx, w, probs);
        else if (E <= 32) route_mfma_kernel<2><<<grid, 256, 0, st>>>(xb, wb, bias, Ttok, H, E, k, norm, idx, w, probs);
        else if (E <= 64) route_mfma_kernel<4><<<grid, 256, 0, st>>>(xb, wb, bias, Ttok, H, E, k, norm, idx, w, probs);
        else route_mfma_kernel<8><<<grid, 256, 0, st>>>(xb, wb, bias, Ttok, H, E, k, norm, idx, w, probs);
        return hipGetLastError();
    }
    hipError_t err = launch_scores(dtype, x, W, bias, Ttok, H, E, scratch_sc, scratch_bd, st);
    if (err != hipSuccess) return err;
    if (dtype == kBF16)
        return launch_select<bf16_t>(scratch_sc, scratch_bd, (const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, E, k,
                                     norm, idx, w, probs, st);
    return launch_select<float>(scratch_sc, scratch_bd, (const float*)x, (const float*)W, bias, Ttok, H, E, k, norm,
                                idx, w, probs, st);
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
