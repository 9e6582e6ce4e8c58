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
// Selection also records, per expert and block of 16 tokens, a 16-bit mask of
// the tokens that chose the expert; grouping derives the stable per-expert
// row order from these masks.
#include "grouping.hpp"
#include "skinny.hpp"

namespace tmoe {

constexpr float kTwoM23 = 1.1920928955078125e-07f;
// per-32-term partial error (33 * 2^-23) with margin for the abs-sum's own rounding
__device__ __forceinline__ double partial_error_scale() { return 33.0 * 1.1920928955078125e-07 * (1.0 + 1.0 / 512); }
__device__ __forceinline__ double fp64_error_scale(int H) { return (double)(H / 32 + 8) * 2.220446049250313e-16; }

// ---------------------------------------------------------------------------
// The next (up to) eight set bits of a wave-uniform mask m (m != 0), as
// indices base + bit in ids[0..8); slots past the count repeat the last index.
// Returns the count.  Static indexing keeps ids in registers.
__device__ __forceinline__ int take8(uint64_t& m, int base, int* ids) {
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (m) {
            ids[q] = base + (__ffsll((unsigned long long)m) - 1);
            m &= m - 1;
            cnt = q + 1;
        } else {
            ids[q] = ids[q > 0 ? q - 1 : 0];
        }
    }
    return cnt;
}

// fp64 rescoring of up to N candidates at once: dot(x_row, W[e_i]) over H,
// wave-cooperative, all 16-byte loads of a chunk issued before use.  Every
// e[0..N) is a valid row (entries past n are loaded and ignored).
template <typename T, int N>
__device__ void wave_dot64(const T* __restrict__ xr, const T* __restrict__ W, int H, const int* e, int n,
                           double* out) {
    double acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0;
    constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
    if (H % V == 0) {
        for (int c = lane_id(); c < H / V; c += kWave) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + c * V);
            u32x4 wv[N];
#pragma unroll
            for (int i = 0; i < N; ++i) wv[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)e[i] * H + c * V);
#pragma unroll
            for (int i = 0; i < N; ++i) {
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
            for (int i = 0; i < N; ++i)
                if (i < n) acc[i] = fma(xv, Elem<T>::load64(W + (int64_t)e[i] * H, h), acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = wave_sum_dpp_f64(acc[i]);
}

// Per-wave selection state in LDS.
struct SelScratch {
    int idx[kMaxTopK];
    double score[kMaxTopK];
};

// Where a token's selection is recorded besides idx / weights: per-expert
// lists (list[e * lstride + slot] = pair index t * k + j, slot from cnt[e]),
// when cnt is not null.
struct ListSink {
    int* cnt;
    int* list;
    int lstride;
};

// Exact Top-k of one row of scores s[0..n) with error bounds d[0..n); writes
// idx / weights / probs, ORs bit `bit` into mask[e * mstride] (when mask is not
// null) and appends pair `pair0 + rank` to the list of every selected e.
// Called by one full wave; lanes own entries e = lane + 64 j.
template <typename T, int MAXJ, typename S>
__device__ __noinline__ void exact_select_row(const S* s, const float* d, int n, int k, const T* xrow, const T* W, int H,
                                 const float* bias, SelScratch* sc, int norm, int32_t* out_idx, float* out_w,
                                 float* out_probs, uint32_t* mask, int mstride, int bit, ListSink ls, int pair0) {
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
        // Candidates: the selected ones and every other one that may reach them,
        // rescored eight at a time.
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
                int ids[8];
                const int cnt = take8(m, kWave * j, ids);
                double r8[8];
                wave_dot64<T, 8>(xrow, W, H, ids, cnt, r8);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i < cnt && lane == ids[i] - kWave * j)
                        v64[j] = r8[i] + (bias ? (double)bias[ids[i]] : 0.0);
                }
            }
        }
        // fp64 selection among the candidates: largest value, then lowest index
        for (int r = 0; r < k; ++r) {
            uint64_t key = 0;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                if (!cand[j]) continue;
                const uint64_t kk = double_order_key(v64[j]);
                key = kk > key ? kk : key;
            }
            const uint64_t kmax = wave_max_key(key);
            uint64_t ik = 0;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                if (cand[j] && double_order_key(v64[j]) == kmax) {
                    const uint64_t c = 0xFFFFFFFFull - (uint64_t)(lane + kWave * j);
                    ik = c > ik ? c : ik;
                }
            }
            ik = wave_max_key(ik);
            const int bi = (int)(0xFFFFFFFFull - ik);
#pragma unroll
            for (int j = 0; j < MAXJ; ++j)
                if (lane + kWave * j == bi) cand[j] = false;
            if (lane == 0) { sc->idx[r] = bi; sc->score[r] = double_from_order_key(kmax); }
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
        if (mask) atomicOr(&mask[my_e * mstride], 1u << bit);
        if (ls.cnt) ls.list[my_e * ls.lstride + atomicAdd(&ls.cnt[my_e], 1)] = pair0 + lane;
    }
}

// ---------------------------------------------------------------------------
// Row-group selection for n <= 16 * J <= 128 and k <= 16: each 16-lane row of
// a wave selects for its own token (lane ri holds entries ri + 16 j), with DPP
// rotations as the row all-reductions, so the four tokens of a wave advance
// together.  Rows whose fp32 selection is not certain are redone afterwards by
// the whole wave (exact_select_row).  The mask of expert e for token t is
// mask[e * mstride + word], bit t % 16.  t < 0 marks an empty row.
struct RowPicks {
    float v[4][16];
    double d[4][16];
    int idx[4][16];
};

// Tokens of a block whose fp32 selection was not certain, left for a later
// exact pass: token within the block and the lowest bound of its fp32 picks.
struct Deferred {
    int n;
    int tok[16];
    double low[16];
};

// Scores of token t are sc[(t - tbase) * n + e] (fp32 in global memory or fp64 in LDS).
// DEFER: uncertain rows are appended to *dfr (nothing recorded for them) instead
// of being redone here.
template <typename T, int J, typename S, bool DEFER = false>
__device__ __forceinline__ void select_rows_wave(const S* __restrict__ sc, const float* __restrict__ bd, int64_t tbase, int64_t t, int n, int k,
                                 const T* __restrict__ x, const T* __restrict__ W, int H, const float* bias, int norm,
                                 int32_t* out_idx, float* out_w, float* out_probs, uint32_t* mask, int mstride,
                                 int word_of_row0, RowPicks& pk, SelScratch* scr, ListSink ls = ListSink{},
                                 Deferred* dfr = nullptr) {
    const int lane = lane_id();
    const int row = lane >> 4, ri = lane & 15;
    const bool valid = t >= 0;
    float v[J];
    double dv[J];
    // Ranking keys: the score's order key with its low byte replaced by 255 - e
    // (n <= 128), unique and never 0; 0 once picked or absent.  Scores that
    // differ only in that byte may come out misordered, which the certificate
    // below (on the exact fp32 values) always rejects.
    uint32_t key[J];
    int pick[J];  // round in which the entry was picked, -1 if not
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = ri + 16 * j;
        const bool ok = valid && e < n;
        v[j] = ok ? (float)sc[(t - tbase) * n + e] + 0.0f : 0.0f;
        dv[j] = ok ? (double)bd[(t - tbase) * n + e] + 1.1920928955078125e-07 * fabs((double)v[j]) : 0.0;
        key[j] = ok ? ((float_order_key(v[j]) & 0xFFFFFF00u) | (uint32_t)(255 - e)) : 0u;
        pick[j] = -1;
    }
    for (int r = 0; r < k; ++r) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) m = umax32(m, key[j]);
        m = row_max_u32(m);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const bool hit = key[j] == m && m != 0;
            pick[j] = hit ? r : pick[j];
            key[j] = hit ? 0u : key[j];
        }
    }
    bool taken[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        taken[j] = !(valid && ri + 16 * j < n) || pick[j] >= 0;
        if (pick[j] >= 0) {
            pk.v[row][pick[j]] = v[j];
            pk.d[row][pick[j]] = dv[j];
            pk.idx[row][pick[j]] = ri + 16 * j;
        }
    }
    __builtin_amdgcn_wave_barrier();
    // certain: consecutive picks strictly separated, and nothing else can reach the lowest pick
    bool bad = false;
    double lo = 1.0e300;
    if (valid && ri < k) {
        lo = (double)pk.v[row][ri] - pk.d[row][ri];
        if (ri > 0) {
            const double prev_lo = (double)pk.v[row][ri - 1] - pk.d[row][ri - 1];
            bad = !(prev_lo > (double)pk.v[row][ri] + pk.d[row][ri]);
        }
    }
    const double low = row_min(lo);
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (!taken[j] && (double)v[j] + dv[j] >= low) bad = true;
    const uint64_t badmask = __ballot(valid && bad);
    const bool certain = ((badmask >> (16 * row)) & 0xFFFFull) == 0;
    if (valid && certain) {
        float mx = -3.0e38f;
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (ri + 16 * j < n) mx = fmaxf(mx, v[j]);
        mx = row_max(mx);
        float z = 0.f;
        if (out_probs || !norm) {
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (ri + 16 * j < n) z += __expf(v[j] - mx);
            z = row_sum(z);
        }
        if (out_probs) {
            const float inv = 1.0f / z;
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (ri + 16 * j < n) out_probs[t * n + ri + 16 * j] = __expf(v[j] - mx) * inv;
        }
        float ex = 0.f;
        if (ri < k) ex = norm ? __expf(pk.v[row][ri] - pk.v[row][0]) : __expf(pk.v[row][ri] - mx);
        const float den = norm ? row_sum(ex) : z;
        if (ri < k) {
            const int e = pk.idx[row][ri];
            out_idx[t * k + ri] = e;
            out_w[t * k + ri] = ex / den;
            if (mask) atomicOr(&mask[e * mstride + word_of_row0], 1u << (t & 15));
            if (ls.cnt) ls.list[e * ls.lstride + atomicAdd(&ls.cnt[e], 1)] = (int)(t * k + ri);
        }
    }
    if (DEFER) {
        if (valid && !certain && ri == 0) {
            const int u = atomicAdd(&dfr->n, 1);
            dfr->tok[u] = (int)(t - tbase);
            dfr->low[u] = low;
        }
        return;
    }
    // rows left uncertain: the whole wave redoes them with fp64 rescoring
    uint64_t redo = __ballot(valid && !certain && ri == 0);
    while (redo) {
        const int g = (__ffsll((unsigned long long)redo) - 1) >> 4;
        redo &= redo - 1;
        const int64_t tg = __shfl(t, g * 16, kWave);
        exact_select_row<T, (16 * J + 63) / 64, S>(sc + (tg - tbase) * n, bd + (tg - tbase) * n, n, k, x + tg * H, W, H, bias, scr, norm,
                                                out_idx + tg * k, out_w + tg * k,
                                                out_probs ? out_probs + tg * n : nullptr,
                                                mask ? mask + word_of_row0 : nullptr, mstride, (int)(tg & 15), ls,
                                                (int)(tg * k));
    }
}

// ---------------------------------------------------------------------------
// Matrix-core scores to global [T, n] (bf16, H % 32 == 0): a block computes
// 16 tokens x 32 weight rows.  Its 8 waves take the 32-wide K steps round
// robin, with the loads of up to 4 steps issued together; every step is a
// fresh fp32 partial added into fp64.  Partials of the waves are reduced in
// LDS in fixed wave order (deterministic).  Splitting the rows over blocks
// spreads the router's bytes over many CUs even for a few tokens.
constexpr int kScoreWaves = 8;

template <int kScoreRows>  // 16 or 32 weight rows per block
__global__ __launch_bounds__(64 * kScoreWaves) void scores_kernel(const bf16_t* __restrict__ x,
                                                                  const bf16_t* __restrict__ W,
                                                                  const float* __restrict__ bias, int64_t T, int H,
                                                                  int n, float* __restrict__ sc,
                                                                  float* __restrict__ bd) {
    constexpr bool two = kScoreRows == 32;
    __shared__ double lg[16 * kScoreRows];
    __shared__ float ab[16 * kScoreRows];
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    const int e0 = blockIdx.y * kScoreRows;
    int64_t tok = tok0 + i;
    if (tok >= T) tok = T - 1;
    int r0 = e0 + i, r1 = two ? e0 + 16 + i : r0;
    if (r0 >= n) r0 = n - 1;
    if (r1 >= n) r1 = n - 1;
    const bf16_t* xp = x + tok * (int64_t)H + kq;
    const bf16_t* w0 = W + (int64_t)r0 * H + kq;
    const bf16_t* w1 = W + (int64_t)r1 * H + kq;
    const u32x4 absmask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    const f32x4 zero = {0, 0, 0, 0};
    double acc0[4] = {0, 0, 0, 0}, acc1[4] = {0, 0, 0, 0};
    f32x4 aa0 = zero, aa1 = zero;
    const int nsteps = H / 32;
    for (int c0 = wave; c0 < nsteps; c0 += 4 * kScoreWaves) {
        u32x4 a[4], b0[4], b1[4];
        // branch-free loads (steps past the end repeat the last one, unused)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int st = min(c0 + u * kScoreWaves, nsteps - 1);
            a[u] = *reinterpret_cast<const u32x4*>(xp + st * 32);
            b0[u] = *reinterpret_cast<const u32x4*>(w0 + st * 32);
            if (two) b1[u] = *reinterpret_cast<const u32x4*>(w1 + st * 32);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (c0 + u * kScoreWaves >= nsteps) continue;
            const bf16x8 av = __builtin_bit_cast(bf16x8, a[u]);
            const bf16x8 aav = __builtin_bit_cast(bf16x8, a[u] & absmask);
            const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b0[u]), zero, 0, 0, 0);
            aa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aav, __builtin_bit_cast(bf16x8, b0[u] & absmask), aa0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc0[r] += (double)p0[r];
            if (two) {
                const f32x4 p1 =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b1[u]), zero, 0, 0, 0);
                aa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aav, __builtin_bit_cast(bf16x8, b1[u] & absmask), aa1,
                                                              0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc1[r] += (double)p1[r];
            }
        }
    }
    // D[row = 4*(lane/16) + r][col = lane%16] per 16x16 block
    for (int w = 0; w < kScoreWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int q = ((lane >> 4) * 4 + r) * kScoreRows + i;
                if (w == 0) {
                    lg[q] = acc0[r]; ab[q] = aa0[r];
                    if (two) { lg[q + 16] = acc1[r]; ab[q + 16] = aa1[r]; }
                } else {
                    lg[q] += acc0[r]; ab[q] += aa0[r];
                    if (two) { lg[q + 16] += acc1[r]; ab[q + 16] += aa1[r]; }
                }
            }
        }
        __syncthreads();
    }
    const double es = partial_error_scale(), fs = fp64_error_scale(H);
    for (int q = threadIdx.x; q < 16 * kScoreRows; q += blockDim.x) {
        const int row = q / kScoreRows, col = q % kScoreRows;
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

// ---------------------------------------------------------------------------
// Few tokens (bf16, H % 256 == 0): scores from exact products.  A bf16 x bf16
// product is exact in fp64, so on the fp64 matrix cores (v_mfma_f64_16x16x4_f64)
// only the fp64 additions round: each instruction adds four products to the
// running sum, so |s - exact| <= (H / 8 + 16) 2^-53 sum_h |x_h W_eh|, far below
// any gap that can separate two fp32 scores; the selection after it almost
// never needs its fp64 rescoring.  The abs-sum bound comes from one bf16
// matrix-core step per eight products (relative error below 2^-17).
// A block computes 16 tokens x 16 weight rows; wave w takes the w-th eighth of
// K, and the four lane groups of a wave contiguous quarters of it (the K order
// inside a product is immaterial as long as both operands use it).  Wave
// partials are added in LDS in wave order.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kS64Waves = 8;

__global__ __launch_bounds__(64 * kS64Waves) void scores64_kernel(const bf16_t* __restrict__ x,
                                                                  const bf16_t* __restrict__ W,
                                                                  const float* __restrict__ bias, int64_t T, int H,
                                                                  int n, float* __restrict__ sc,
                                                                  float* __restrict__ bd) {
    __shared__ double part[kS64Waves][256];
    __shared__ float apart[kS64Waves][256];
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int i = lane & 15, grp = lane >> 4;
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    const int e0 = blockIdx.y * 16;
    const int64_t tok = tok0 + i < T ? tok0 + i : T - 1;
    const int row = min(e0 + i, n - 1);
    const int kw = H / kS64Waves, kq = kw / 4;
    const bf16_t* xp = x + tok * (int64_t)H + wave * kw + grp * kq;
    const bf16_t* wp = W + (int64_t)row * H + wave * kw + grp * kq;
    const u32x4 absmask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    f64x4 acc = {0, 0, 0, 0};
    f32x4 aacc = {0, 0, 0, 0};
    for (int c = 0; c < kq; c += 32) {  // kq % 8 == 0; up to four 8-element chunks in flight
        u32x4 xa[4], wa[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // branch-free: chunks past the end repeat the last one, unused
            const int cu = min(c + 8 * u, kq - 8);
            xa[u] = *reinterpret_cast<const u32x4*>(xp + cu);
            wa[u] = *reinterpret_cast<const u32x4*>(wp + cu);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (c + 8 * u >= kq) continue;
            aacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u] & absmask),
                                                           __builtin_bit_cast(bf16x8, wa[u] & absmask), aacc, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(xa[u][q] << 16),
                                                           (double)__uint_as_float(wa[u][q] << 16), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(xa[u][q] & 0xFFFF0000u),
                                                           (double)__uint_as_float(wa[u][q] & 0xFFFF0000u), acc, 0, 0,
                                                           0);
            }
        }
    }
    // token row x weight row: the fp64 product leaves D[lane / 16 + 4 r][lane % 16]
    // in register r, the bf16 one D[4 (lane / 16) + r][lane % 16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        part[wave][(grp + 4 * r) * 16 + i] = acc[r];
        apart[wave][(grp * 4 + r) * 16 + i] = aacc[r];
    }
    __syncthreads();
    const double es = (double)(H / 8 + 16) * 1.1102230246251565e-16;  // (H / 8 + 16) 2^-53
    for (int q = threadIdx.x; q < 256; q += blockDim.x) {
        const int64_t t = tok0 + q / 16;
        const int e = e0 + q % 16;
        if (t >= T || e >= n) continue;
        double s = 0.0;
        float a32 = 0.f;
        for (int w = 0; w < kS64Waves; ++w) {
            s += part[w][q];
            a32 += apart[w][q];
        }
        const float b = bias ? bias[e] : 0.f;
        const double sv = s + (double)b;
        const double a = (double)a32 * (1.0 + 1.0 / 65536);
        sc[t * n + e] = (float)sv;
        bd[t * n + e] = (float)(es * (a + fabs((double)b)) + 0.5 * 1.1920928955078125e-07 * fabs(sv)) *
                        (1.0f + kTwoM23);
    }
}

// ---------------------------------------------------------------------------
// Router for bf16 with E = 16 NS experts (NS in {1, 2, 4, 8}), H a multiple of
// 128 (8 / NS), H <= 1024, k <= 16: one block of 8 waves per 16 tokens; scores never
// leave LDS.
//   scores: the block stages its 16 token rows in LDS (their loads go out
//     first, ahead of the weight stream).  Wave w scores expert tile w % NS
//     over the stages s (128 K-elements each) with s % (8 / NS) == w / NS,
//     streaming its own 16 W_r rows through a private LDS slice: lanes load
//     whole 256-byte row slices (four rows per instruction; reading the
//     matrix-core fragment shape, 16 rows x 64 bytes per instruction, straight
//     from memory streams several times slower), DEPTH stages in flight in
//     registers, and no block barrier in the loop.  Staged rows are padded by
//     16 bytes, so fragment reads are free of bank conflicts.  Every bf16
//     matrix-core step (32 exact products summed in fp32) is a fresh partial
//     added into fp64, beside the abs-sum that bounds the error; the K groups
//     are added in LDS in a fixed order (deterministic).
//   selection: one token per 32-lane half-wave (route_select_half: certified
//     fp32 ranking; lane ri holds experts ri + 32 j).  Tokens left uncertain
//     are redone exactly by the whole block: candidate lists, then the fp64
//     rescoring of every (token, candidate) pair spread over the eight waves,
//     then a rank count per token (route_exact_picks).
//   outputs: idx / weights (/ probs); per (expert, 16-token block) a token mask
//     (masks != null), or per block and expert the count and list of its pairs
//     t * k + j (bcnt != null; list order within a block is arbitrary).
constexpr int kRouteWaves = 8;
constexpr int kRouteThreads = 64 * kRouteWaves;
constexpr int kRouteMaxH = 1024;
constexpr int kRouteStageK = 128;  // K-elements per W_r stage

// All-reductions over a 32-lane half-wave: the 16-lane row step, then row
// 2h + 1 takes in lane 15 of row 2h (DPP row broadcast), and every lane of
// half h reads lane 32 h + 31.  No LDS round trip; one value per half.
template <typename F>
__device__ __forceinline__ uint32_t half_bcast(uint32_t x, F op) {
    const uint32_t y = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, kDppRowBcast15, 0xa, 0xf, false));
    const uint32_t h0 = __builtin_amdgcn_readlane(y, 31), h1 = __builtin_amdgcn_readlane(y, 63);
    return lane_id() < 32 ? h0 : h1;
}
__device__ __forceinline__ uint32_t half_max_u32(uint32_t x) {
    return half_bcast(row_max_u32(x), [](uint32_t a, uint32_t b) { return umax32(a, b); });
}
__device__ __forceinline__ float half_max(float x) {
    return __uint_as_float(half_bcast(__float_as_uint(row_max(x)), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float half_sum(float x) {
    return __uint_as_float(half_bcast(__float_as_uint(row_sum(x)), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}
__device__ __forceinline__ double half_min(double x) {
    uint64_t kk = row_max_key(~double_order_key(x));
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)kk, kDppRowBcast15, 0xa, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(kk >> 32), kDppRowBcast15, 0xa, 0xf, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    kk = o > kk ? o : kk;
    const uint32_t l0 = __builtin_amdgcn_readlane((uint32_t)kk, 31), h0 = __builtin_amdgcn_readlane((uint32_t)(kk >> 32), 31);
    const uint32_t l1 = __builtin_amdgcn_readlane((uint32_t)kk, 63), h1 = __builtin_amdgcn_readlane((uint32_t)(kk >> 32), 63);
    kk = lane_id() < 32 ? (((uint64_t)h0 << 32) | l0) : (((uint64_t)h1 << 32) | l1);
    return double_from_order_key(~kk);
}

// The picks of the block's tokens, by rank: fp32 value, its bound, expert.
struct BlockPicks {
    float v[16][16];
    double d[16][16];
    int e[16][16];
};

// Certified fp32 Top-k of token tt of the block on one 32-lane half-wave
// (lane ri holds experts ri + 32 j).  s / a: the token's fp64 score sums and
// fp32 abs-sums; on return s holds the biased score and a its error bound
// (for the exact pass).  A certain token's outputs are written here; an
// uncertain one is appended to dfr with the lowest bound of its picks.
template <int J>
__device__ __forceinline__ void route_select_half(double* __restrict__ s, float* __restrict__ a,
                                                  const float* __restrict__ bsh, int E, int H, int k, int norm,
                                                  bool valid, int tt, int64_t t, int32_t* __restrict__ out_idx,
                                                  float* __restrict__ out_w, float* __restrict__ out_probs,
                                                  uint32_t* msk, int* lcnt, int* llist, BlockPicks& pk,
                                                  Deferred* dfr) {
    const int lane = lane_id(), ri = lane & 31;
    const double es = partial_error_scale(), fs = fp64_error_scale(H);
    float v[J];
    double dv[J];
    // ranking keys: the order key of the value with its low byte replaced by
    // 255 - e (E <= 128), unique and never 0; 0 once picked or absent.  Values
    // that differ only in that byte may come out misordered, which the
    // certificate below (on the exact fp32 values) always rejects.
    uint32_t key[J];
    int pick[J];
    // all reads first (the write-backs below go to the same rows)
    double s0[J];
    float a0[J], b0[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int ec = ri + 32 * j < E ? ri + 32 * j : 0;
        s0[j] = s[ec];
        a0[j] = a[ec];
        b0[j] = bsh ? bsh[ec] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = ri + 32 * j;
        const bool ok = valid && e < E;
        const float bb = b0[j];
        const double sv = s0[j] + (double)bb;
        const double ab = (double)a0[j];
        const float dd = (float)(es * ab + fs * (ab + fabs((double)bb))) * (1.0f + kTwoM23);
        if (ok) {
            s[e] = sv;
            a[e] = dd;
        }
        v[j] = ok ? (float)sv + 0.0f : 0.0f;
        dv[j] = ok ? (double)dd + 1.1920928955078125e-07 * fabs((double)v[j]) : 0.0;
        key[j] = ok ? ((float_order_key(v[j]) & 0xFFFFFF00u) | (uint32_t)(255 - e)) : 0u;
        pick[j] = -1;
    }
    for (int r = 0; r < k; ++r) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) m = umax32(m, key[j]);
        m = half_max_u32(m);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const bool hit = key[j] == m && m != 0;
            pick[j] = hit ? r : pick[j];
            key[j] = hit ? 0u : key[j];
        }
    }
    bool taken[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        taken[j] = !(valid && ri + 32 * j < E) || pick[j] >= 0;
        if (pick[j] >= 0) {
            pk.v[tt][pick[j]] = v[j];
            pk.d[tt][pick[j]] = dv[j];
            pk.e[tt][pick[j]] = ri + 32 * j;
        }
    }
    __builtin_amdgcn_wave_barrier();
    // certain: consecutive picks strictly separated, and nothing else can reach the lowest pick
    bool bad = false;
    double lo = 1.0e300;
    if (valid && ri < k) {
        lo = (double)pk.v[tt][ri] - pk.d[tt][ri];
        if (ri > 0) bad = !((double)pk.v[tt][ri - 1] - pk.d[tt][ri - 1] > (double)pk.v[tt][ri] + pk.d[tt][ri]);
    }
    const double low = half_min(lo);
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (!taken[j] && (double)v[j] + dv[j] >= low) bad = true;
    const uint64_t badmask = __ballot(valid && bad);
    const bool certain = ((badmask >> (lane & 32)) & 0xFFFFFFFFull) == 0;
    if (valid && certain) {
        float mx = 0.f, z = 1.f;
        if (out_probs || !norm) {
            mx = -3.0e38f;
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (ri + 32 * j < E) mx = fmaxf(mx, v[j]);
            mx = half_max(mx);
            z = 0.f;
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (ri + 32 * j < E) z += __expf(v[j] - mx);
            z = half_sum(z);
            if (out_probs) {
                const float inv = 1.0f / z;
#pragma unroll
                for (int j = 0; j < J; ++j)
                    if (ri + 32 * j < E) out_probs[t * E + ri + 32 * j] = __expf(v[j] - mx) * inv;
            }
        }
        float ex = 0.f;
        if (ri < k) ex = norm ? __expf(pk.v[tt][ri] - pk.v[tt][0]) : __expf(pk.v[tt][ri] - mx);
        const float den = norm ? half_sum(ex) : z;
        if (ri < k) {
            const int e = pk.e[tt][ri];
            out_idx[t * k + ri] = e;
            out_w[t * k + ri] = ex / den;
            atomicOr(&msk[e], 1u << tt);
            if (lcnt) llist[e * 16 + atomicAdd(&lcnt[e], 1)] = (int)(t * k + ri);
        }
    }
    if (valid && !certain && ri == 0) {
        const int u = atomicAdd(&dfr->n, 1);
        dfr->tok[u] = tt;
        dfr->low[u] = low;
    }
}

// Exact Top-k of an uncertain token from its rescored candidates (one full
// wave): every score that may reach the fp32 picks (value + bound >= low, the
// picks included) has been rescored in fp64 (bf16 products are exact there),
// and the k best are taken by value, ties to the lower index.  Every expert of
// the exact Top-k is among the candidates, because the k picks all have exact
// scores >= low.  cs / ce: the candidates' exact scores and experts, in
// expert order; s: the token's biased scores (fp32 softmax statistics).
template <int J>
__device__ void route_exact_picks(const double* s, const double* cs, const int* ce, int nc, int E, int k, int norm,
                                  int tt, int64_t t, int32_t* oidx, float* ow, float* oprob, uint32_t* msk,
                                  int* lcnt, int* llist, BlockPicks& pk) {
    const int lane = lane_id();
    // rank of candidate l: how many candidates come before it (lane l holds
    // candidates l + 64 h; the others are broadcast with readlane)
    double sl[J];
    int el[J], rank[J];
#pragma unroll
    for (int h = 0; h < J; ++h) {
        const int l = lane + 64 * h;
        sl[h] = l < nc ? cs[l] : 0.0;
        el[h] = l < nc ? ce[l] : 0;
        rank[h] = 0;
    }
#pragma unroll
    for (int hm = 0; hm < J; ++hm) {
        const int n = min(nc - 64 * hm, 64);
        const uint64_t u = (uint64_t)__double_as_longlong(sl[hm]);
        for (int m = 0; m < n; ++m) {
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, m);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), m);
            const double sm = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
            const int em = __builtin_amdgcn_readlane(el[hm], m);
#pragma unroll
            for (int h = 0; h < J; ++h) rank[h] += (sm > sl[h] || (sm == sl[h] && em < el[h])) ? 1 : 0;
        }
    }
#pragma unroll
    for (int h = 0; h < J; ++h)
        if (lane + 64 * h < nc && rank[h] < k) {
            pk.d[tt][rank[h]] = sl[h];  // here: the exact score
            pk.e[tt][rank[h]] = el[h];
        }
    __builtin_amdgcn_wave_barrier();
    // softmax statistics over all E in fp32 (probs, and the plain weights)
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? (float)s[e] + 0.0f : 0.0f;
    }
    float mx = 0.f, z = 1.f;
    if (oprob || !norm) {
        mx = -3.0e38f;
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (lane + kWave * j < E) mx = fmaxf(mx, v[j]);
        mx = wave_max_dpp(mx);
        z = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (lane + kWave * j < E) z += __expf(v[j] - mx);
        z = wave_sum_dpp(z);
        if (oprob) {
            const float inv = 1.0f / z;
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (lane + kWave * j < E) oprob[t * E + lane + kWave * j] = __expf(v[j] - mx) * inv;
        }
    }
    const int r = lane < k ? lane : 0;
    const double my_s = pk.d[tt][r], s0 = pk.d[tt][0];
    const int my_e = pk.e[tt][r];
    // renormalised weights from the exact score differences (<= 0)
    const float ex = lane < k ? (norm ? __expf((float)(my_s - s0)) : __expf((float)my_s - mx)) : 0.f;
    const float den = norm ? wave_sum_dpp(ex) : z;
    if (lane < k) {
        oidx[t * k + lane] = my_e;
        ow[t * k + lane] = ex / den;
        atomicOr(&msk[my_e], 1u << tt);
        if (lcnt) llist[my_e * 16 + atomicAdd(&lcnt[my_e], 1)] = (int)(t * k + lane);
    }
}

// The router of one block of 16 tokens (blockIdx.x): the body of route_block_kernel.
template <int NS, int DEPTH>
__device__ __forceinline__ void route_block_body(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ bias, int64_t T, int H,
    int k, int norm, int32_t* __restrict__ out_idx, float* __restrict__ out_w, float* __restrict__ out_probs,
    uint16_t* __restrict__ masks, uint64_t* __restrict__ jmask, int mstride, int32_t* __restrict__ bcnt,
    int32_t* __restrict__ blist) {
    constexpr int E = NS * 16;
    constexpr int KG = kRouteWaves / NS;                        // K groups per expert tile
    constexpr int XCH = 16 * (kRouteMaxH / 8) / kRouteThreads;  // staged x chunks per thread (max)
    constexpr int SLD = kRouteStageK + 8;                       // bf16 per staged W_r row (272 bytes)
    constexpr int WI = 16 * kRouteStageK / 8 / kWave;           // load instructions per stage and wave (4)
    constexpr int CPL = kRouteMaxH / 8 / kWave;                 // 16-byte chunks per lane of one row (exact pass)
    __shared__ __attribute__((aligned(16))) bf16_t xs[16 * (kRouteMaxH + 8)];
    __shared__ __attribute__((aligned(16))) bf16_t wsb[kRouteWaves][16 * SLD];
    __shared__ double lg[16 * E];
    __shared__ float ab[16 * E];
    __shared__ float bsh[E];
    __shared__ uint32_t msk[E];
    __shared__ uint64_t jm[E];
    __shared__ int lcnt[E];
    __shared__ __attribute__((aligned(16))) int llist[E * 16];
    __shared__ BlockPicks picks;
    __shared__ Deferred dfr;
    __shared__ int cnc[16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    const int XLD = H + 8;
    const int tile = wave % NS, g = wave / NS;
    const int nmine = H / (kRouteStageK * KG);  // this wave's stages g, g + KG, ...; a multiple of DEPTH

    // the block's token rows (rows past T repeat row T - 1; never used): their
    // loads go out first, the weight stream behind them
    const int cpr = H / 8, nxc = 16 * cpr;
    u32x4 xv[XCH];
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
        const int c = min(tid + j * kRouteThreads, nxc - 1);
        const int r = c / cpr, q = c % cpr;
        const int64_t t = tok0 + r < T ? tok0 + r : T - 1;
        xv[j] = *reinterpret_cast<const u32x4*>(x + t * H + q * 8);
    }
    float bias_v = 0.f;  // E <= 128 < block size: one entry per thread
    if (bias != nullptr && tid < E) bias_v = bias[tid];
    // every wave's token-row loads enter the CU's load pipeline before any
    // weight load (which it serves in order): a barrier on issue, not on data
    __builtin_amdgcn_s_barrier();
    // stage m of this wave: lane l loads row 4 j + l / 16, 16-byte chunk l % 16
    // of K-slice st = g + m KG of rows tile * 16 .. + 15
    const bf16_t* wsrc = W + (int64_t)(tile * 16 + (lane >> 4)) * H + (lane & 15) * 8;
    auto wload = [&](int m, u32x4* r) {
        const int st = g + m * KG;
#pragma unroll
        for (int j = 0; j < WI; ++j)
            r[j] = *reinterpret_cast<const u32x4*>(wsrc + (int64_t)(4 * j) * H + st * kRouteStageK);
    };
    u32x4 wr[DEPTH][WI];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) wload(d, wr[d]);

    if (tid == 0) dfr.n = 0;
    if (tid < E) {
        msk[tid] = 0;
        jm[tid] = 0;
        lcnt[tid] = 0;
    }
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
        const int c = tid + j * kRouteThreads;
        if (c < nxc) *reinterpret_cast<u32x4*>(&xs[(c / cpr) * XLD + (c % cpr) * 8]) = xv[j];
    }
    if (tid < E) bsh[tid] = bias_v;
    __syncthreads();

    const int i = lane & 15, kq = (lane >> 4) * 8;
    const bf16_t* xr = &xs[i * XLD + kq];
    bf16_t* wb = wsb[wave];
    const int wst = (lane >> 4) * SLD + (lane & 15) * 8;  // this lane's store slot (row 4 j + lane / 16)
    const bf16_t* wfr = &wb[i * SLD + kq];               // fragment: row i, k offset kq
    const u32x4 absmask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    const f32x4 zero = {0, 0, 0, 0};
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    f32x4 aacc = zero;
    // stage m: its registers go to the wave's own LDS slice (its earlier
    // fragment reads are ordered before these stores), the registers are
    // refilled with stage m + DEPTH (refill false: none left), then the
    // stage's matrix work
    auto stage = [&](const int m, u32x4* r, const bool refill) {
#pragma unroll
        for (int j = 0; j < WI; ++j) *reinterpret_cast<u32x4*>(&wb[wst + 4 * j * SLD]) = r[j];
        if (refill) wload(m + DEPTH, r);
        const int k0 = (g + m * KG) * kRouteStageK;
#pragma unroll
        for (int ks = 0; ks < kRouteStageK; ks += 32) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(xr + k0 + ks);
            const u32x4 b = *reinterpret_cast<const u32x4*>(wfr + ks);
            const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), zero, 0, 0, 0);
            aacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a & absmask),
                                                           __builtin_bit_cast(bf16x8, b & absmask), aacc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += (double)p[r];
        }
    };
    // the last DEPTH stages issue no loads (nothing left in flight to wait for later)
    for (int m0 = 0; m0 + DEPTH < nmine; m0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) stage(m0 + d, wr[d], true);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) stage(nmine - DEPTH + d, wr[d], false);
    // D[token 4 (lane / 16) + r][expert lane % 16] per tile; K groups added in order
#pragma unroll
    for (int gg = 0; gg < KG; ++gg) {
        if (g == gg) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int q = ((lane >> 4) * 4 + r) * E + tile * 16 + i;
                if (gg == 0) { lg[q] = acc[r]; ab[q] = aacc[r]; }
                else { lg[q] += acc[r]; ab[q] += aacc[r]; }
            }
        }
        __syncthreads();
    }

    // certified selection, one token per half-wave
    {
        const int tt = 2 * wave + (lane >> 5);
        const int64_t t = tok0 + tt;
        route_select_half<(E + 31) / 32>(&lg[tt * E], &ab[tt * E], bias ? bsh : nullptr, E, H, k, norm, t < T,
                                         tt, t, out_idx, out_w, out_probs, msk, bcnt ? lcnt : nullptr, llist, picks,
                                         &dfr);
    }
    __syncthreads();
    const int nd = dfr.n;
    if (nd > 0) {
        // exact pass over the uncertain tokens (LDS of the weight slices reused:
        // candidate scores [16][E] fp64, then candidate experts [16][E])
        double* cs = reinterpret_cast<double*>(&wsb[0][0]);
        int* ce = reinterpret_cast<int*>(cs + 16 * E);
        static_assert(sizeof(wsb) >= 16 * E * (sizeof(double) + sizeof(int)), "exact-pass scratch fits");
        // 1. candidate lists, in expert order, one wave per token
        for (int u = wave; u < nd; u += kRouteWaves) {
            const int tt = dfr.tok[u];
            const double low = dfr.low[u];
            int nc = 0;
#pragma unroll
            for (int j = 0; j < (E + 63) / 64; ++j) {
                const int e = lane + 64 * j;
                const bool ok = e < E;
                const float v = ok ? (float)lg[tt * E + e] + 0.0f : 0.0f;
                const double dv = ok ? (double)ab[tt * E + e] + 1.1920928955078125e-07 * fabs((double)v) : 0.0;
                const bool c = ok && (double)v + dv >= low;
                const uint64_t m = __ballot(c);
                if (c) ce[u * E + nc + __popcll(m & lanemask_lt())] = e;
                nc += __popcll(m);
            }
            if (lane == 0) cnc[u] = nc;
        }
        __syncthreads();
        // 2. fp64 rescoring of every (token, candidate) pair: pairs p and p + 8
        // of every round of 16 go to wave p % 8, all loads of both issued first
        int np = 0, cnt_u = 0, off_u = 0;  // lane u < nd: token u's count and first pair
        if (lane < nd) cnt_u = cnc[lane];
        {
            const int incl = wave_incl_scan(cnt_u);
            off_u = incl - cnt_u;
            np = __builtin_amdgcn_readlane(incl, 15);  // nd <= 16
        }
        for (int p0 = wave; p0 < np; p0 += 2 * kRouteWaves) {
            int pu[2], pi[2], pe[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int p = min(p0 + h * kRouteWaves, np - 1);
                // token of pair p: the last u with off_u <= p
                const uint64_t le = __ballot(lane < nd && off_u <= p);
                const int u = 63 - __builtin_clzll(le);
                pu[h] = u;
                pi[h] = p - __builtin_amdgcn_readlane(off_u, u);
                pe[h] = ce[u * E + pi[h]];
            }
            u32x4 wv[2][CPL], xw[2][CPL];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = c * kWave + lane < cpr ? c * kWave + lane : 0;
                    wv[h][c] = *reinterpret_cast<const u32x4*>(W + (int64_t)pe[h] * H + ch * 8);
                }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = c * kWave + lane < cpr ? c * kWave + lane : 0;
                    xw[h][c] = *reinterpret_cast<const u32x4*>(&xs[dfr.tok[pu[h]] * XLD + ch * 8]);
                }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                double d = 0.0;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    if (c * kWave + lane >= cpr) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        d = fma((double)__uint_as_float(xw[h][c][q] << 16), (double)__uint_as_float(wv[h][c][q] << 16), d);
                        d = fma((double)__uint_as_float(xw[h][c][q] & 0xFFFF0000u),
                                (double)__uint_as_float(wv[h][c][q] & 0xFFFF0000u), d);
                    }
                }
                d = wave_sum_dpp_f64(d);
                const int p = p0 + h * kRouteWaves;
                if (lane == 0 && p < np) cs[pu[h] * E + pi[h]] = d + (double)bsh[pe[h]];
            }
        }
        __syncthreads();
        // 3. exact picks and outputs, one wave per token
        for (int u = wave; u < nd; u += kRouteWaves) {
            const int tt = dfr.tok[u];
            const int64_t t = tok0 + tt;
            route_exact_picks<(E + kWave - 1) / kWave>(&lg[tt * E], &cs[u * E], &ce[u * E], cnc[u], E, k, norm, tt,
                                                       t, out_idx, out_w, out_probs, msk, bcnt ? lcnt : nullptr,
                                                       llist, picks);
        }
        __syncthreads();
    }
    if (jmask) {
        // slot of every choice, 4 bits per token, from the block's picks
        for (int q = tid; q < 16 * k; q += blockDim.x) {
            const int tt = q / k, j = q % k;
            if (tok0 + tt < T) atomicOr((unsigned long long*)&jm[picks.e[tt][j]], (unsigned long long)j << (4 * tt));
        }
        __syncthreads();
        for (int e = tid; e < E; e += blockDim.x) jmask[(int64_t)e * mstride + blockIdx.x] = jm[e];
    }
    if (masks)
        for (int e = tid; e < E; e += blockDim.x) masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
    if (bcnt) {
        // whole list rows: entries past an expert's count are copied too, and
        // readers drop them
        int32_t* cnt_b = bcnt + (int64_t)blockIdx.x * E;
        int4* list_b = reinterpret_cast<int4*>(blist + (int64_t)blockIdx.x * E * 16);
        for (int e = tid; e < E; e += blockDim.x) cnt_b[e] = lcnt[e];
        for (int q = tid; q < E * 4; q += blockDim.x) list_b[q] = reinterpret_cast<const int4*>(llist)[q];
    }
}

template <int NS, int DEPTH>
__global__ __launch_bounds__(kRouteThreads) void route_block_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ bias, int64_t T, int H,
    int k, int norm, int32_t* __restrict__ out_idx, float* __restrict__ out_w, float* __restrict__ out_probs,
    uint16_t* __restrict__ masks, uint64_t* __restrict__ jmask, int mstride, int32_t* __restrict__ bcnt,
    int32_t* __restrict__ blist) {
    route_block_body<NS, DEPTH>(x, W, bias, T, H, k, norm, out_idx, out_w, out_probs, masks, jmask, mstride, bcnt,
                                blist);
}

// Blocks 0 .. ceil(T / 16) - 1 route (as route_block_kernel); the rest each
// compute 8 features of the shared expert's gate/up product for all T <= 64
// tokens (the 16-column skinny form over the whole K, one wave per K eighth).
// The two kinds share no data; the router's blocks come first in dispatch.
template <int NS, int DEPTH>
__global__ __launch_bounds__(kRouteThreads) void route_shared_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, const float* __restrict__ bias, int64_t T, int H,
    int k, int norm, int32_t* __restrict__ out_idx, float* __restrict__ out_w, int mstride,
    int32_t* __restrict__ bcnt, int32_t* __restrict__ blist, const bf16_t* __restrict__ sg,
    const bf16_t* __restrict__ su, int Is, bf16_t* __restrict__ hs, int nroute) {
    if ((int)blockIdx.x < nroute) {
        route_block_body<NS, DEPTH>(x, W, bias, T, H, k, norm, out_idx, out_w, nullptr, nullptr, nullptr, mstride,
                                    bcnt, blist);
        return;
    }
    skinny_body<kRouteWaves, 4, true>(x, sg, su, nullptr, hs, (int)T, 2 * Is, H, 1, (int)blockIdx.x - nroute, 0);
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

// ---------------------------------------------------------------------------
// Selection from global scores, 16 tokens per block (one mask word), with
// masks [E][mstride] uint16 written when non-null.
template <typename T, int J>
__global__ __launch_bounds__(256) void select_rows_kernel(const float* __restrict__ sc, const float* __restrict__ bd,
                                                          const T* __restrict__ x, const T* __restrict__ W,
                                                          const float* __restrict__ bias, int64_t Ttok, int H,
                                                          int n, int k, int norm, int32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_w, float* __restrict__ out_probs,
                                                          uint16_t* __restrict__ masks, int mstride) {
    __shared__ RowPicks picks[4];
    __shared__ SelScratch scr[4];
    __shared__ uint32_t msk[16 * J];
    for (int q = threadIdx.x; q < 16 * J; q += blockDim.x) msk[q] = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 16 + wave * 4 + (lane_id() >> 4);
    select_rows_wave<T, J, float>(sc, bd, 0, t < Ttok ? t : -1, n, k, x, W, H, bias, norm, out_idx, out_w, out_probs, msk, 1, 0,
                           picks[wave], &scr[wave]);
    if (masks) {
        __syncthreads();
        for (int e = threadIdx.x; e < n; e += blockDim.x) masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
    }
}

// Whole-wave selection (any n <= 1024, k <= 32): 16 tokens per block, 4 per wave.
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
                                  out_idx + t * k, out_w + t * k, out_probs ? out_probs + t * n : nullptr, msk, 1, tt,
                                  ListSink{}, 0);
    }
    if (masks) {
        __syncthreads();
        for (int e = threadIdx.x; e < n; e += blockDim.x) masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
    }
}

// ---------------------------------------------------------------------------
// Small batches (T <= 256, E <= 128): one block groups the routing — per-expert
// counts / offsets / prefixes of the token masks, GEMM tile lists, and the
// scatter of (token, slot) pairs — with the masks and prefixes in LDS.
constexpr int kSmallMaxT = 256;
constexpr int kSmallWords = kSmallMaxT / 16;

__global__ __launch_bounds__(1024) void group_small_kernel(const int32_t* __restrict__ idx,
                                                           const uint16_t* __restrict__ masks, int mstride, int Ttok,
                                                           int E, int k, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ row_pair, TileSpecs specs) {
    __shared__ uint32_t msk[128 * kSmallWords];
    __shared__ int pre[128 * kSmallWords];
    __shared__ int offs[128];
    __shared__ int lds[17];
    const int nw = (Ttok + 15) / 16;
    for (int q = threadIdx.x; q < E * nw; q += blockDim.x) {
        const int e = q / nw, w = q % nw;
        msk[e * kSmallWords + w] = masks[(int64_t)e * mstride + w];
    }
    __syncthreads();
    const int e = threadIdx.x;
    int c = 0;
    if (e < E) {
        for (int w = 0; w < nw; ++w) {
            pre[e * kSmallWords + w] = c;
            c += __popc(msk[e * kSmallWords + w]);
        }
    }
    int total;
    const int excl = block_exclusive_scan(e < E ? c : 0, lds, &total);
    if (e < E) {
        offs[e] = excl;
        counts[e] = c;
        offsets[e] = excl;
    }
    if (e == 0) offsets[E] = total;
    for (int s = 0; s < specs.n; ++s) block_build_items(c, excl, E, Ttok, specs.t[s], lds);
    __syncthreads();
    const int N = Ttok * k;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const int ee = idx[i];
        if (ee < 0 || ee >= E) continue;
        const int t = i / k, j = i % k;
        const int m = ee * kSmallWords + (t >> 4);
        const int dst = offs[ee] + pre[m] + __popc(msk[m] & ((1u << (t & 15)) - 1u));
        if (dst < 0 || dst >= N) continue;
        row_token[dst] = t;
        row_of[i] = dst;
        if (row_pair) row_pair[dst] = i;
    }
}

// Small batches, routing finished in the grouping block: each of the 8
// waves selects four tokens at a time from the global scores (certified, with
// fp64 rescoring of uncertain tokens) and records the token masks in LDS; the
// block then derives counts, offsets, stable row order, row maps and GEMM tile
// lists from those masks, as group_small_kernel does from global ones.
constexpr int kSelectGroupThreads = 512;

template <int J>
__global__ __launch_bounds__(kSelectGroupThreads) void select_group_small_kernel(
    const float* __restrict__ sc, const float* __restrict__ bd, const bf16_t* __restrict__ x,
    const bf16_t* __restrict__ W, const float* __restrict__ bias, int Ttok, int H, int E, int k, int norm,
    int32_t* __restrict__ out_idx, float* __restrict__ out_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ row_of,
    int32_t* __restrict__ row_pair, TileSpecs specs) {
    __shared__ uint32_t msk[128 * kSmallWords];
    __shared__ int pre[128 * kSmallWords];
    __shared__ int offs[128];
    __shared__ int lds[17];
    constexpr int kWaves = kSelectGroupThreads / 64;
    __shared__ RowPicks picks[kWaves];
    __shared__ SelScratch scr[kWaves];
    for (int q = threadIdx.x; q < 128 * kSmallWords; q += blockDim.x) msk[q] = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    for (int t0 = wave * 4; t0 < Ttok; t0 += 4 * kWaves) {
        const int t = t0 + (lane_id() >> 4);
        select_rows_wave<bf16_t, J, float>(sc, bd, 0, t < Ttok ? t : -1, E, k, x, W, H, bias, norm, out_idx, out_w,
                                           nullptr, msk, kSmallWords, t0 >> 4, picks[wave], &scr[wave]);
    }
    __syncthreads();
    const int nw = (Ttok + 15) / 16;
    const int e = threadIdx.x;
    int c = 0;
    if (e < E) {
        for (int w = 0; w < nw; ++w) {
            pre[e * kSmallWords + w] = c;
            c += __popc(msk[e * kSmallWords + w]);
        }
    }
    int total;
    const int excl = block_exclusive_scan(e < E ? c : 0, lds, &total);
    if (e < E) {
        offs[e] = excl;
        counts[e] = c;
        offsets[e] = excl;
    }
    if (e == 0) offsets[E] = total;
    for (int s = 0; s < specs.n; ++s) block_build_items(c, excl, E, Ttok, specs.t[s], lds);
    __syncthreads();
    const int N = Ttok * k;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const int ee = out_idx[i];
        if (ee < 0 || ee >= E) continue;
        const int t = i / k, j = i % k;
        const int m = ee * kSmallWords + (t >> 4);
        const int dst = offs[ee] + pre[m] + __popc(msk[m] & ((1u << (t & 15)) - 1u));
        if (dst < 0 || dst >= N) continue;
        row_token[dst] = t;
        row_of[i] = dst;
        if (row_pair) row_pair[dst] = i;
    }
}

// Exact argmax over n scores of any length (ties to the lower index): one block
// of four waves per token, thread j taking entries j + 256 i.  From the fp32
// scores s and their bounds d: the fp32 argmax, and low = max (s - d), a lower
// bound of the exact maximum; entries with s + d >= low are the candidates.  With
// more than one, each wave rescores the candidates among its own entries in
// fp64 from x and W, and the four winners are ranked.
constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxWaves = kArgmaxThreads / kWave;

template <typename T>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_exact_kernel(const float* __restrict__ sc,
                                                                      const float* __restrict__ bd,
                                                                      const T* __restrict__ x,
                                                                      const T* __restrict__ W, int H, int n,
                                                                      int32_t* __restrict__ out) {
    __shared__ uint64_t kx[kArgmaxWaves];
    __shared__ double lx[kArgmaxWaves], bx[kArgmaxWaves];
    __shared__ int nx[kArgmaxWaves], ix[kArgmaxWaves];
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int64_t t = blockIdx.x;
    const float* s = sc + t * n;
    const float* d = bd + t * n;
    constexpr int U = 4;  // entries per thread with loads in flight together
    // rows of at most R entries (R / 256 per thread: the code heads' 2048 and
    // 3072): every entry requested at once and kept in registers for the
    // candidate count, one memory round trip; longer rows loop U at a time
    constexpr int RPT = 16, R = RPT * kArgmaxThreads;
    const bool in_regs = n <= R;  // block-uniform
    float sr[RPT], dr[RPT];
    uint64_t key = 0;
    double low = -1.0e300;
    if (in_regs) {
#pragma unroll
        for (int u = 0; u < RPT; ++u) {  // entries past the end repeat the last one, unused
            const int e = min((int)threadIdx.x + u * kArgmaxThreads, n - 1);
            sr[u] = s[e];
            dr[u] = d[e];
        }
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int e = (int)threadIdx.x + u * kArgmaxThreads;
            if (e >= n) continue;
            const uint64_t kk = rank_key(sr[u], e);
            key = kk > key ? kk : key;
            low = fmax(low, (double)sr[u] - (double)dr[u]);
        }
    }
    for (int e0 = in_regs ? n : (int)threadIdx.x; e0 < n; e0 += U * kArgmaxThreads) {
        float sv[U], dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // branch-free: entries past the end repeat the last one, unused
            const int e = min(e0 + u * kArgmaxThreads, n - 1);
            sv[u] = s[e];
            dv[u] = d[e];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * kArgmaxThreads;
            if (e >= n) continue;
            const uint64_t kk = rank_key(sv[u], e);
            key = kk > key ? kk : key;
            low = fmax(low, (double)sv[u] - (double)dv[u]);
        }
    }
    key = wave_max_key(key);
    low = double_from_order_key(wave_max_key(double_order_key(low)));
    if (lane == 0) {
        kx[wave] = key;
        lx[wave] = low;
    }
    __syncthreads();
    key = kx[0];
    low = lx[0];
    for (int w = 1; w < kArgmaxWaves; ++w) {
        key = kx[w] > key ? kx[w] : key;
        low = fmax(low, lx[w]);
    }
    int bi = rank_key_index(key);
    int nc = 0;
    if (in_regs) {
#pragma unroll
        for (int u = 0; u < RPT; ++u)
            if ((int)threadIdx.x + u * kArgmaxThreads < n) nc += ((double)sr[u] + (double)dr[u] >= low) ? 1 : 0;
    }
    for (int e0 = in_regs ? n : (int)threadIdx.x; e0 < n; e0 += U * kArgmaxThreads) {
        float sv[U], dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = min(e0 + u * kArgmaxThreads, n - 1);
            sv[u] = s[e];
            dv[u] = d[e];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (e0 + u * kArgmaxThreads < n) nc += ((double)sv[u] + (double)dv[u] >= low) ? 1 : 0;
    }
    nc = __builtin_amdgcn_readlane(wave_incl_scan(nc), 63);
    if (lane == 0) nx[wave] = nc;
    __syncthreads();
    nc = 0;
    for (int w = 0; w < kArgmaxWaves; ++w) nc += nx[w];
    if (nc > 1) {  // block-uniform
        double best = 0.0;
        int besti = -1;
        const T* xr = x + t * H;
        for (int base = wave * kWave; base < n; base += kArgmaxThreads) {
            const int e = base + lane;
            const bool c = e < n && (double)s[e] + (double)d[e] >= low;
            uint64_t m = __ballot(c);
            while (m) {
                int ids[8];
                const int cnt = take8(m, base, ids);
                double r8[8];
                wave_dot64<T, 8>(xr, W, H, ids, cnt, r8);
                for (int i = 0; i < cnt; ++i)
                    if (besti < 0 || ranks_before(r8[i], ids[i], best, besti)) {
                        best = r8[i];
                        besti = ids[i];
                    }
            }
        }
        if (lane == 0) {
            bx[wave] = best;
            ix[wave] = besti;
        }
        __syncthreads();
        bi = -1;
        double bv = 0.0;
        for (int w = 0; w < kArgmaxWaves; ++w)
            if (ix[w] >= 0 && (bi < 0 || ranks_before(bx[w], ix[w], bv, bi))) {
                bv = bx[w];
                bi = ix[w];
            }
    }
    if (threadIdx.x == 0) out[t] = bi;
}

// ---------------------------------------------------------------------------
// c_0 drawn from softmax(logits / tau) by inverse transform: the first code v
// with sum_{i<=v} e_i > u * sum_i e_i, e_i = exp(l_i / tau) up to a common
// factor (the Qwen3-TTS module walkthrough, "Codec Head": a softmax over the
// codec head's logits, then a draw).  u outside [0, 1) clamps to the first or
// the last code.  One block of 16 waves per token; thread j owns the
// contiguous codes [j s, j s + s), s = ceil(n / 1024).
//  * Certified pass.  A score s_i with |s_i - l_i| <= d_i gives
//    e_i = exp((l_i - M) / tau) within exp(+-w_i) of c_i = exp((s_i - M) / tau)
//    (w_i = d_i / tau plus the argument's and exp's own rounding; the shift
//    M = max (s + d) bounds every exact logit from above), so e_i lies in
//    [lo_i, hi_i] = c_i [1 - w_i, 1 + w_i + w_i^2] for w_i <= 1 (exps otherwise).
//    Prefix sums of both bounds, with a bound gam on their own rounding, decide
//    for each v whether the exact prefix C_v certainly exceeds u Z, written
//    C_v (1 - u) > u R_v with R_v = Z - C_v ("above"), or certainly does not
//    ("below").  The draw is settled when the first v not below is also the
//    first v above.
//  * Exact pass, otherwise (u within the scores' error of a boundary): the
//    token's n logits are recomputed in fp64 from x and W into LDS (products
//    of the inputs are exact; only the fp64 additions round) and the
//    definition is applied to them.
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;

struct ScanF64 {
    double excl, total;
};
// Exclusive prefix sum of one value per thread in thread order, and the total
// (fixed association: deterministic).  tmp: kSampleThreads + 1 doubles.
__device__ ScanF64 block_scan_f64(double v, double* tmp) {
    constexpr int PER = kSampleThreads / kWave;  // consecutive threads per lane of wave 0
    __syncthreads();
    tmp[threadIdx.x] = v;
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int l = (int)threadIdx.x;
        double r[PER];
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            r[i] = acc;  // exclusive within the lane's run
            acc += tmp[PER * l + i];
        }
        double sum = acc;
        for (int off = 1; off < kWave; off <<= 1) {
            const double o = __shfl_up(sum, off);
            if (l >= off) sum += o;
        }
        const double up = __shfl_up(sum, 1);
        const double ex = l == 0 ? 0.0 : up;
#pragma unroll
        for (int i = 0; i < PER; ++i) tmp[PER * l + i] = ex + r[i];
        if (l == kWave - 1) tmp[kSampleThreads] = sum;
    }
    __syncthreads();
    return {tmp[threadIdx.x], tmp[kSampleThreads]};
}
__device__ double block_max_f64(double v, double* tmp) {
    for (int off = 1; off < kWave; off <<= 1) v = fmax(v, __shfl_xor(v, off));
    __syncthreads();
    if (lane_id() == 0) tmp[threadIdx.x >> 6] = v;
    __syncthreads();
    double m = tmp[0];
    for (int w = 1; w < kSampleWaves; ++w) m = fmax(m, tmp[w]);
    return m;
}
__device__ int block_min_i32(int v, int* tmp) {
    for (int off = 1; off < kWave; off <<= 1) v = min(v, __shfl_xor(v, off));
    __syncthreads();
    if (lane_id() == 0) tmp[threadIdx.x >> 6] = v;
    __syncthreads();
    int m = tmp[0];
    for (int w = 1; w < kSampleWaves; ++w) m = min(m, tmp[w]);
    return m;
}

// Half-width w (in the exponent) of the interval of e_i around c = exp(a),
// a = (s - M) * itau: the score's bound d, the rounding of a (three operations
// and 1 / tau) and exp's own error.
__device__ __forceinline__ double exp_halfwidth(float s, float d, double M, double itau) {
    return ((double)d * (1.0 + 0x1p-50) + ((double)fabsf(s) + fabs(M)) * 0x1p-50) * itau + 0x1p-50;
}
__device__ __forceinline__ void exp_interval(double c, double a, double w, double& lo, double& hi) {
    if (w <= 1.0) {  // exp(w) <= 1 + w + w^2 and exp(-w) >= 1 - w for 0 <= w <= 1
        hi = c * (1.0 + w + w * w) * (1.0 + 0x1p-50);
        lo = c * (1.0 - w) * (1.0 - 0x1p-50);
    } else {  // the sum a +- w rounds by up to (|a| + w) 2^-53 in the exponent
        const double r = (fabs(a) + w + 2.0) * 0x1p-50;
        hi = exp(a + w) * (1.0 + r);
        lo = exp(a - w) * (1.0 - r);
    }
}

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void sample_exact_kernel(const float* __restrict__ sc,
                                                                      const float* __restrict__ bd,
                                                                      const T* __restrict__ x,
                                                                      const T* __restrict__ W, int H, int n,
                                                                      double tau, const double* __restrict__ uin,
                                                                      int32_t* __restrict__ out) {
    extern __shared__ double lex[];  // c_i of the certified pass, then the exact logits
    __shared__ double tmp[kSampleThreads + 1];
    __shared__ int itmp[kSampleWaves];
    const int64_t t = blockIdx.x;
    const double u = uin[t];
    if (!(u >= 0.0) || u >= 1.0) {  // clamp (NaN to the first code)
        if (threadIdx.x == 0) out[t] = u >= 1.0 ? n - 1 : 0;
        return;
    }
    const int seg = (n + kSampleThreads - 1) / kSampleThreads;
    const int v0 = min((int)threadIdx.x * seg, n), v1 = min(v0 + seg, n);
    const float* s = sc + t * n;
    const float* d = bd + t * n;
    const double itau = 1.0 / tau;

    double ml = -INFINITY;
    for (int v = v0; v < v1; ++v) ml = fmax(ml, (double)s[v] + (double)d[v]);
    const double M = block_max_f64(ml, tmp);
    double sl = 0.0, sh = 0.0;
    for (int v = v0; v < v1; ++v) {
        const double a = ((double)s[v] - M) * itau;
        const double c = exp(a);
        lex[v] = c;
        double lo, hi;
        exp_interval(c, a, exp_halfwidth(s[v], d[v], M, itau), lo, hi);
        sl += lo;
        sh += hi;
    }
    const ScanF64 pl = block_scan_f64(sl, tmp);
    const ScanF64 ph = block_scan_f64(sh, tmp);
    const double ZL = pl.total, ZH = ph.total;
    // every computed prefix or total lies within gam of the exact sum of its terms
    const double gam = (double)(n + 2 * kSampleThreads) * 0x1p-52 * ZH;
    int first_above = n, first_open = n;
    double L = pl.excl, Hs = ph.excl;
    for (int v = v0; v < v1; ++v) {
        const double a = ((double)s[v] - M) * itau;
        double lo, hi;
        exp_interval(lex[v], a, exp_halfwidth(s[v], d[v], M, itau), lo, hi);
        L += lo;
        Hs += hi;
        const bool above = (L - gam) * (1.0 - u) > u * (ZH - Hs + 2.0 * gam) * (1.0 + 0x1p-50);
        const bool below = (Hs + gam) * (1.0 - u) * (1.0 + 0x1p-50) <= u * (ZL - L - 2.0 * gam);
        if (above && first_above == n) first_above = v;
        if (!below && first_open == n) first_open = v;
    }
    int fo = block_min_i32(first_open, itmp);
    const int fa = block_min_i32(first_above, itmp);
    if (fo != fa) {  // block-uniform: the exact pass
        const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
        const T* xr = x + t * H;
        __syncthreads();  // every thread is done with the c_i in lex
        for (int base = wave * 8; base < n; base += kSampleWaves * 8) {
            int ids[8];
            const int cnt = min(8, n - base);
#pragma unroll
            for (int i = 0; i < 8; ++i) ids[i] = min(base + i, n - 1);
            double r8[8];
            wave_dot64<T, 8>(xr, W, H, ids, cnt, r8);
            if (lane == 0)
                for (int i = 0; i < cnt; ++i) lex[base + i] = r8[i];
        }
        __syncthreads();
        double mx = -INFINITY;
        for (int v = v0; v < v1; ++v) mx = fmax(mx, lex[v]);
        mx = block_max_f64(mx, tmp);
        double se = 0.0;
        for (int v = v0; v < v1; ++v) se += exp((lex[v] - mx) / tau);
        const ScanF64 pe = block_scan_f64(se, tmp);
        const double thr = u * pe.total;
        int first = n;
        double c = pe.excl;
        for (int v = v0; v < v1; ++v) {
            c += exp((lex[v] - mx) / tau);
            if (c > thr && first == n) first = v;
        }
        fo = block_min_i32(first, itmp);
    }
    if (threadIdx.x == 0) out[t] = min(fo, n - 1);
}

// ---------------------------------------------------------------------------
// Host-side launchers.
template <typename T>
static hipError_t launch_select(const float* sc, const float* bd, const T* x, const T* W, const float* bias,
                                int64_t Ttok, int H, int n, int k, int norm, int32_t* idx, float* w, float* probs,
                                uint16_t* masks, int mstride, hipStream_t st) {
    dim3 grid((unsigned)((Ttok + 15) / 16));
    if (n <= 128 && k <= 16) {
#define TMOE_ROWS(J)                                                                                     \
    select_rows_kernel<T, J><<<grid, 256, 0, st>>>(sc, bd, x, W, bias, Ttok, H, n, k, norm, idx, w, probs, \
                                                   masks, mstride)
        if (n <= 16) TMOE_ROWS(1);
        else if (n <= 32) TMOE_ROWS(2);
        else if (n <= 64) TMOE_ROWS(4);
        else TMOE_ROWS(8);
#undef TMOE_ROWS
        return hipGetLastError();
    }
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

hipError_t launch_scores(int dtype, const void* x, const void* W, const float* bias, int64_t Ttok, int H, int n,
                         float* sc, float* bd, hipStream_t st) {
    if (dtype == kBF16 && H % 32 == 0) {
        // few tokens: exact-product scores, 16 weight rows per block
        if (Ttok <= 256 && H % 256 == 0) {
            dim3 grid((unsigned)((Ttok + 15) / 16), (unsigned)((n + 15) / 16));
            scores64_kernel<<<grid, 64 * kS64Waves, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, n,
                                                             sc, bd);
        } else if (Ttok <= 256) {
            dim3 grid((unsigned)((Ttok + 15) / 16), (unsigned)((n + 15) / 16));
            scores_kernel<16><<<grid, 64 * kScoreWaves, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H,
                                                                 n, sc, bd);
        } else {
            dim3 grid((unsigned)((Ttok + 15) / 16), (unsigned)((n + 31) / 32));
            scores_kernel<32><<<grid, 64 * kScoreWaves, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H,
                                                                 n, sc, bd);
        }
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

bool route_block_ok(int dtype, int H, int E, int k) {
    if (dtype != kBF16 || H > kRouteMaxH || k > 16 || !(E == 16 || E == 32 || E == 64 || E == 128)) return false;
    const int kg = kRouteWaves / (E / 16);
    return H % (kRouteStageK * kg) == 0;  // every wave streams at least one whole stage
}
bool group_small_ok(int64_t T, int E) { return T <= kSmallMaxT && E <= 128; }

hipError_t launch_route_block(const void* x, const void* W, const float* bias, int64_t Ttok, int H, int E, int k,
                              int norm, int32_t* idx, float* w, float* probs, uint16_t* masks, uint64_t* jmask,
                              int32_t* bcnt, int32_t* blist, hipStream_t st) {
    const unsigned grid = (unsigned)mask_words(Ttok);
    const int mstride = mask_stride(Ttok);
    const bf16_t* xb = (const bf16_t*)x;
    const bf16_t* wb = (const bf16_t*)W;
    const int nmine = H / (kRouteStageK * (kRouteWaves / (E / 16)));  // stages per wave
#define TMOE_RB(NS, D)                                                                                   \
    route_block_kernel<NS, D><<<grid, kRouteThreads, 0, st>>>(xb, wb, bias, Ttok, H, k, norm, idx, w, probs, \
                                                              masks, jmask, mstride, bcnt, blist)
#define TMOE_RB_E(D)                 \
    if (E == 16) TMOE_RB(1, D);      \
    else if (E == 32) TMOE_RB(2, D); \
    else if (E == 64) TMOE_RB(4, D); \
    else TMOE_RB(8, D);
    if (nmine % 4 == 0) { TMOE_RB_E(4) }
    else if (nmine % 2 == 0) { TMOE_RB_E(2) }
    else { TMOE_RB_E(1) }
#undef TMOE_RB_E
#undef TMOE_RB
    return hipGetLastError();
}

bool route_shared_ok(int64_t T, int H, int Is) {
    return T >= 1 && T <= kSkinnyRows && Is >= 8 && Is % 8 == 0 && H % (32 * kRouteWaves) == 0 &&
           kRouteThreads == 64 * kRouteWaves;
}

hipError_t launch_route_block_shared(const void* x, const void* W, const float* bias, int64_t Ttok, int H, int E,
                                     int k, int norm, int32_t* idx, float* w, int32_t* bcnt, int32_t* blist,
                                     const void* sg, const void* su, int Is, void* hs, hipStream_t st) {
    const int nroute = mask_words(Ttok);
    const unsigned grid = (unsigned)(nroute + Is / 8);
    const int mstride = mask_stride(Ttok);
    const bf16_t* xb = (const bf16_t*)x;
    const bf16_t* wb = (const bf16_t*)W;
    const int nmine = H / (kRouteStageK * (kRouteWaves / (E / 16)));  // stages per wave
#define TMOE_RS(NS, D)                                                                                             \
    route_shared_kernel<NS, D><<<grid, kRouteThreads, 0, st>>>(xb, wb, bias, Ttok, H, k, norm, idx, w, mstride,     \
                                                               bcnt, blist, (const bf16_t*)sg, (const bf16_t*)su, \
                                                               Is, (bf16_t*)hs, nroute)
#define TMOE_RS_E(D)                 \
    if (E == 16) TMOE_RS(1, D);      \
    else if (E == 32) TMOE_RS(2, D); \
    else if (E == 64) TMOE_RS(4, D); \
    else TMOE_RS(8, D);
    if (nmine % 4 == 0) { TMOE_RS_E(4) }
    else if (nmine % 2 == 0) { TMOE_RS_E(2) }
    else { TMOE_RS_E(1) }
#undef TMOE_RS_E
#undef TMOE_RS
    return hipGetLastError();
}

hipError_t launch_route(int dtype, const void* x, const void* W, const float* bias, int64_t Ttok, int H, int E,
                        int k, int norm, int32_t* idx, float* w, float* probs, float* scratch_sc,
                        float* scratch_bd, uint16_t* masks, uint64_t* jmask, hipStream_t st) {
    // one block per 16 tokens (one mask word); mask rows are mask_stride(T) words apart
    const int nwords = mask_words(Ttok), mstride = mask_stride(Ttok);
    if (route_block_ok(dtype, H, E, k))
        return launch_route_block(x, W, bias, Ttok, H, E, k, norm, idx, w, probs, masks, masks ? jmask : nullptr,
                                  nullptr, nullptr, st);
    hipError_t err = launch_scores(dtype, x, W, bias, Ttok, H, E, scratch_sc, scratch_bd, st);
    if (err != hipSuccess) return err;
    if (dtype == kBF16)
        return launch_select<bf16_t>(scratch_sc, scratch_bd, (const bf16_t*)x, (const bf16_t*)W, bias, Ttok, H, E, k,
                                     norm, idx, w, probs, masks, mstride, st);
    return launch_select<float>(scratch_sc, scratch_bd, (const float*)x, (const float*)W, bias, Ttok, H, E, k, norm,
                                idx, w, probs, masks, mstride, st);
}

hipError_t launch_group_small(const int32_t* idx, const uint16_t* masks, int64_t Ttok, int E, int k, int32_t* counts,
                              int32_t* offsets, int32_t* row_token, int32_t* row_of, int32_t* row_pair,
                              const TileSpec* t1, const TileSpec* t2, hipStream_t st) {
    group_small_kernel<<<1, 1024, 0, st>>>(idx, masks, mask_stride(Ttok), (int)Ttok, E, k, counts, offsets,
                                           row_token, row_of, row_pair, make_specs(t1, t2));
    return hipGetLastError();
}

bool route_group_small_ok(int dtype, int64_t T, int H, int E, int k) {
    return dtype == kBF16 && H % 32 == 0 && group_small_ok(T, E) && k <= 16;
}

hipError_t launch_select_group_small(const float* scratch_sc, const float* scratch_bd, const void* x, const void* W,
                                     const float* bias, int64_t Ttok, int H, int E, int k, int norm, int32_t* idx,
                                     float* w, int32_t* counts, int32_t* offsets, int32_t* row_token,
                                     int32_t* row_of, int32_t* row_pair, const TileSpec* t1, const TileSpec* t2,
                                     hipStream_t st) {
    const bf16_t* xb = (const bf16_t*)x;
    const bf16_t* wb = (const bf16_t*)W;
    const TileSpecs specs = make_specs(t1, t2);
#define TMOE_SG(J)                                                                                          \
    select_group_small_kernel<J><<<1, kSelectGroupThreads, 0, st>>>(scratch_sc, scratch_bd, xb, wb, bias, (int)Ttok, H, E, k, \
                                                     norm, idx, w, counts, offsets, row_token, row_of, row_pair, \
                                                     specs)
    if (E <= 16) TMOE_SG(1);
    else if (E <= 32) TMOE_SG(2);
    else if (E <= 64) TMOE_SG(4);
    else TMOE_SG(8);
#undef TMOE_SG
    return hipGetLastError();
}

hipError_t launch_argmax(int dtype, const float* sc, const float* bd, const void* x, const void* W, int64_t Ttok,
                         int H, int n, int32_t* out, hipStream_t st) {
    if (Ttok < 1) return hipSuccess;
    if (dtype == kBF16)
        argmax_exact_kernel<bf16_t><<<(unsigned)Ttok, kArgmaxThreads, 0, st>>>(sc, bd, (const bf16_t*)x,
                                                                              (const bf16_t*)W, H, n, out);
    else
        argmax_exact_kernel<float><<<(unsigned)Ttok, kArgmaxThreads, 0, st>>>(sc, bd, (const float*)x,
                                                                             (const float*)W, H, n, out);
    return hipGetLastError();
}

bool sample_ok(int n) { return n >= 1 && n <= kSampleMaxN; }

hipError_t launch_scores_argmax(int dtype, const void* x, const void* W, int64_t Ttok, int H, int n, float* sc,
                                float* bd, hipStream_t st) {
    if (dtype == kBF16 && H % 32 == 0 && Ttok <= 256) {
        // fp32 matrix-core partials into fp64: bounds near 5e-5 relative, ample
        // for an argmax whose rare near-ties the argmax rescores exactly
        dim3 grid((unsigned)((Ttok + 15) / 16), (unsigned)((n + 15) / 16));
        scores_kernel<16><<<grid, 64 * kScoreWaves, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, nullptr, Ttok, H, n,
                                                             sc, bd);
        return hipGetLastError();
    }
    return launch_scores(dtype, x, W, nullptr, Ttok, H, n, sc, bd, st);
}

hipError_t launch_scores_exact(int dtype, const void* x, const void* W, int64_t Ttok, int H, int n, float* sc,
                               float* bd, hipStream_t st) {
    if (dtype == kBF16 && H % 256 == 0) {
        dim3 grid((unsigned)((Ttok + 15) / 16), (unsigned)((n + 15) / 16));
        scores64_kernel<<<grid, 64 * kS64Waves, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, nullptr, Ttok, H, n, sc,
                                                         bd);
        return hipGetLastError();
    }
    return launch_scores(dtype, x, W, nullptr, Ttok, H, n, sc, bd, st);
}

hipError_t launch_sample(int dtype, const float* sc, const float* bd, const void* x, const void* W, int64_t Ttok,
                         int H, int n, double tau, const double* u, int32_t* out, hipStream_t st) {
    if (!sample_ok(n)) return hipErrorInvalidValue;
    const size_t lds = (size_t)n * sizeof(double);
    if (dtype == kBF16)
        sample_exact_kernel<bf16_t><<<(unsigned)Ttok, kSampleThreads, lds, st>>>(sc, bd, (const bf16_t*)x,
                                                                                  (const bf16_t*)W, H, n, tau, u,
                                                                                  out);
    else
        sample_exact_kernel<float><<<(unsigned)Ttok, kSampleThreads, lds, st>>>(sc, bd, (const float*)x,
                                                                                 (const float*)W, H, n, tau, u, out);
    return hipGetLastError();
}

}  // namespace tmoe
