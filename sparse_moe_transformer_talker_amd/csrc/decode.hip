// The Talker MoE layer at decode sizes (at most 64 tokens, bf16, hidden 1024):
// "3C · Talker MoE (20 lớp, 128 Experts Top-6) & Đầu ra mã ngữ nghĩa c_0"
// (openarchlab), §1 for the sizes and norm_topk_prob, §3 for
//   y_t = SharedMLP(x_t) + sum_{i in S_t} w_{t,i} Expert_i(x_t),
// with every expert a SwiGLU down(SiLU(gate x) * up x) ("用 print(model) 认识
// Qwen3-TTS", horus-space, MLP section).
//
// Four launches:
//  1. route_scores_kernel: the E router scores of every token on the matrix
//     cores with a rigorous error bound, spread over T / 8 x E / 16 workgroups.
//  2. route_select_kernel: one workgroup per token: the top-k (ties to the lower
//     expert index) is certified from the bounds or settled by fp64 rescoring of
//     the candidates, so it is the top-k of the scores computed in fp64, up to
//     fp64 summation rounding; then the routing weights.  Further workgroups of
//     the launch compute the shared expert's gate/up, which needs no routing.
//  3. decode_experts_kernel: one work item per (expert, 64-wide slice of the
//     intermediate dimension) plus tiles of the shared expert's down product.
//     A routed item runs its slice of gate/up and SwiGLU for its tokens, then
//     the slice's share of the down product, and stores those partial output
//     rows in bf16.  The weight stream of the whole layer is one launch: no seam
//     between gate/up and down.
//  4. the partial-row combine (elementwise.hip) sums each token's partial rows
//     in a fixed order and applies the routing weights.
//
// At this size the layer is bound by the weight bytes (about 4 flop per byte),
// so the expert kernel is organised around keeping HBM reads in flight: three
// workgroups per CU, each wave streaming its own weight rows through a
// wave-private LDS stage with about three 4 KB blocks in flight and no barrier
// inside the K loop, and items of equal weight bytes handed out only to
// touched experts, so that every CU carries about the same bytes.
#include "common.hpp"
#include "kernels.hpp"
#include "skinny.hpp"

namespace tmoe {
namespace dec {
constexpr int kH = 1024;           // hidden size of the matrix-core decode path
constexpr int kMaxT = 64;          // tokens per call on this path
constexpr int kSlice = 64;         // intermediate columns per work item
constexpr int kWaves = 4;
constexpr int kStage = 8192;       // bytes of one wave's weight block
constexpr int kHRow = 72;          // bf16 elements per row of the h tile (144 B: conflict-free fragment reads)
constexpr int kERow = 144;         // bytes per row of a wave's output staging tile
// Tokens per shared gate/up workgroup of the selection launch: 32 makes 192
// workgroups at T = 64, which with the 64 selection workgroups is one per CU,
// and reads 18 MB of token and weight rows instead of 24 MB with 16 (measured
// 1.2 us less per decode layer; 64 tokens, 96 workgroups, gained nothing).
constexpr int kSharedRows = 32;
static_assert(kSharedRows % 16 == 0 && kSharedRows <= kMaxT, "shared gate/up token group");
}  // namespace dec

namespace dec {
// keeps the compiler from hoisting later LDS reads above this point
// (scheduling only: no instruction is emitted)
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Buffer loads: a wave-uniform resource (base and byte extent, in SGPRs), a
// per-lane byte offset in one VGPR and a uniform byte offset in an SGPR, so
// the address of a whole block costs one VGPR.  Reads past the extent return
// zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t lane_off, uint32_t uoff) {
    // uoff is wave-uniform by construction; readfirstlane lets the compiler see it
    return __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, __builtin_amdgcn_readfirstlane(uoff), 0);
}
__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
    return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, const u32x4& v) {
    *reinterpret_cast<u32x4*>(base + off) = v;
}
// Stage layout (the expert kernel's stages use it too): 256-byte rows;
// 16-byte chunk c of row r sits at r * 256 + 16 (c ^ (r % 16)).  A block of 16
// rows is written by store i with lane (row 4 i + lg, chunk li), at
// stage_store_lane(q = i % 4) + 1024 i, and read back as the matrix-core B
// fragment of K step ks (row li, chunk 4 ks + lg) at stage_frag_lane(ks); both
// are conflict-free.
__device__ __forceinline__ int stage_store_lane(int q) {
    const int lane = (int)(threadIdx.x & 63), li = lane & 15, lg = lane >> 4;
    return lg * 256 + (((li ^ lg) ^ (4 * q)) << 4);
}
__device__ __forceinline__ int stage_frag_lane(int ks) {
    const int lane = (int)(threadIdx.x & 63), li = lane & 15, lg = lane >> 4;
    return li * 256 + (((li ^ lg) ^ (4 * ks)) << 4);
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
}  // namespace dec

// ---------------------------------------------------------------------------
// Router, in two launches.
//
// route_scores_kernel: workgroup (g, c) scores tokens 8 g .. 8 g + 7 against
// experts 16 c .. 16 c + 15, its four waves each over a quarter of K.  The
// weights (256 KB) and the token rows together are a few hundred KB, and one CU
// streams only some tens of GB/s, so the read is spread over T / 8 x E / 16
// workgroups; the workgroups of one expert group share an XCD (and its L2).
// Scores on the matrix cores: rows 0 .. 7 of the A operand are the tokens (8 ..
// 15 repeat them and are dropped), the B operand 16 expert rows.  Each 32-wide
// K step is one MFMA from a zero accumulator; its fp32 result (a sum of 32 exact
// bf16 products) is added into an fp64 accumulator, and the quarters are added
// in a fixed order.  A second MFMA chain over |x| and |W| gives B_e = sum_h |x_h
// W_eh| (fp32, inflated for its own rounding), so the fp64 score s_e is within
//   d_e = 40 * 2^-23 * B_e + 2^-40 B_e
// of the exactly computed score (the 32-product partials, however the matrix
// cores round or truncate, and the fp64 additions; plus 2^-52 |s_e| for the
// bias add).  Scores and bounds go to two [T, E] fp64 arrays.
//
// route_select_kernel: one workgroup per token, whose wave 0 picks the top k
// of s by (value, lower index).  It is certified when the intervals
// [s - d, s + d] of consecutive picks, and of the k-th pick against every other
// expert, are strictly ordered.  Otherwise every expert whose upper bound
// reaches the lowest lower bound of the picks is rescored in fp64 from exact
// products (the four waves take eight candidates each at a time, each lane
// summing elements 8 l .. 8 l + 7 of each 512-wide chunk in order, then the
// wave), which gives the top-k of the fp64 scores up to fp64 summation
// rounding; experts not rescored lie strictly below every pick.  Weights:
// e^(s_i - s_max) over their sum (norm_topk_prob) or over the sum of all E
// terms (the plain softmax probabilities), in fp64.

// Order-preserving 32-bit key of a score (its fp32 rounding) with the expert
// index in the low 7 bits: a larger key is a larger score, then a lower index.
__device__ __forceinline__ uint32_t topk_key32(double v, int e) {
    uint32_t u = __float_as_uint((float)v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (u & ~127u) | (uint32_t)(127 - e);
}

// Wave-wide maximum of an unsigned value, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr2, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr4, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr8, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xa, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int H>
__global__ __launch_bounds__(256) void route_scores_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                           const float* __restrict__ bias, int T, int E,
                                                           double* __restrict__ sc, double* __restrict__ dv,
                                                           uint32_t* __restrict__ mask,
                                                           int32_t* __restrict__ counts) {
    using namespace dec;
    // the selection launch ORs the touched experts into mask and counts the
    // routed pairs per expert: both start from zero here
    if (blockIdx.x == 0) {
        if (threadIdx.x < 4) mask[threadIdx.x] = 0u;
        for (int e = threadIdx.x; e < E; e += 256) counts[e] = 0;
    }
    constexpr int KW = H / 4;      // K quarter of a wave
    constexpr int NBK = KW / 128;  // 128-wide K blocks of a quarter
    constexpr int NKS = KW / 32;   // 32-wide K steps of a quarter
    __shared__ __attribute__((aligned(1024))) char wstage[4 * 4096];
    __shared__ double red[4][8][16];
    __shared__ float redb[4][8][16];
    const int neg = (E + 15) / 16;
    const int g = (int)blockIdx.x / neg, c = (int)blockIdx.x - g * neg;
    const int t0 = 8 * g, e0 = 16 * c;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int kw0 = KW * wave;

    // the token fragments (row li % 8, K 32 ks + 8 lg of the quarter), then the
    // 16 expert rows of the quarter: load i of block b brings rows 4 i + lg, 256
    // bytes each.  The row is in the lane offset, so a row past E is outside the
    // resource's extent and reads as zero (its results are dropped).
    const rsrc_t xr = make_rsrc(x, (uint32_t)T * H * 2);
    const rsrc_t wr = make_rsrc(W, (uint32_t)E * H * 2);
    const uint32_t x_l = (uint32_t)(min(t0 + (li & 7), T - 1) * H + 8 * lg) * 2;
    u32x4 xv[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) xv[ks] = bload(xr, x_l, (kw0 + 32 * ks) * 2);
    u32x4 wv[NBK][4];
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wv[b][i] = bload(wr, (uint32_t)((e0 + 4 * i + lg) * H + 8 * li) * 2, (kw0 + 128 * b) * 2);

    // the lane holds D rows 4 lg + r (tokens) of column li (expert)
    const u32x4 kAbs = u32x4{0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    f32x4 babs = f32x4{0, 0, 0, 0};
    char* wst = wstage + 4096 * wave;
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
        // block b into the wave's stage (LDS operations of a wave run in order)
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_write16(wst, stage_store_lane(i) + 1024 * i, wv[b][i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 wf = lds_read16(wst, stage_frag_lane(q));
            const u32x4 av = xv[4 * b + q];
            const f32x4 p = mfma(av, wf, f32x4{0, 0, 0, 0});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += (double)p[r];
            babs = mfma(av & kAbs, wf & kAbs, babs);
        }
        sched_fence();
    }
    if (lg < 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            red[wave][4 * lg + r][li] = acc[r];
            redb[wave][4 * lg + r][li] = babs[r];
        }
    }
    __syncthreads();
    if (tid < 128) {
        const int t = tid >> 4, e = tid & 15;
        if (t0 + t < T && e0 + e < E) {
            const double sum = ((red[0][t][e] + red[1][t][e]) + red[2][t][e]) + red[3][t][e];
            const double bsum = (((double)redb[0][t][e] + (double)redb[1][t][e]) + (double)redb[2][t][e]) +
                                (double)redb[3][t][e];
            // B_e rounded up past the fp32 rounding of its own sums (at most (H + 8)
            // 2^-23 relative, rounding or truncating), then the bound
            const double B = bsum * (1.0 + (double)(H + 8) * 1.2e-7);
            const double score = sum + (bias ? (double)bias[e0 + e] : 0.0);
            const int64_t o = (int64_t)(t0 + t) * E + e0 + e;
            sc[o] = score;
            dv[o] = B * (40.0 * 1.1920928955078125e-07 + 9.094947017729282e-13) + fabs(score) * 2.3e-16;
        }
    }
}

template <int H>
__global__ __launch_bounds__(256) void route_select_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                           const float* __restrict__ bias,
                                                           const double* __restrict__ sc,
                                                           const double* __restrict__ dv, int T, int E, int k,
                                                           int norm, int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out, uint32_t* __restrict__ mask,
                                                           int32_t* __restrict__ counts,
                                                           const bf16_t* __restrict__ sg,
                                                           const bf16_t* __restrict__ su, int Is,
                                                           bf16_t* __restrict__ hs) {
    const int nsel = T;
    if ((int)blockIdx.x >= nsel) {
        // the shared expert's gate/up beside the selection (it needs no
        // routing): hs [T, Is] = SiLU(x sg^T) * (x su^T) in bf16, 8 features of
        // kSharedRows tokens per workgroup (the 16-column skinny form over all
        // of K).  Workgroup tq * Is / 8 + f: the token groups of feature group f
        // share an XCD (Is / 8 is a multiple of 8), so its weight rows come from
        // HBM once.
        constexpr int R = dec::kSharedRows;
        const int nf = Is / 8, b = (int)blockIdx.x - nsel, tq = b / nf, f = b - tq * nf;
        skinny_body<4, 4, true, R / 16>(x + (int64_t)R * tq * H, sg, su, nullptr, hs + (int64_t)R * tq * Is,
                                        min(R, T - R * tq), 2 * Is, H, 1, f, 0);
        return;
    }
    constexpr int NC8 = H / 512;  // 8-element chunks per lane of a rescored row
    static_assert(H % 512 == 0, "hidden size");
    // one token per workgroup: wave 0 selects; when the certificate fails the
    // four waves share the candidates' rescoring
    __shared__ double sct[128];
    __shared__ double dvt[128];
    __shared__ double rst[128];
    __shared__ int cnd[128];
    __shared__ int s_nc;
    __shared__ int s_topi[8];
    __shared__ double s_topv[8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int64_t t = blockIdx.x;
    const bool ok0 = lane < E, ok1 = lane + 64 < E;
    int sel[8];
    double val[8];
    if (wave == 0) {
        const double v0 = ok0 ? sc[t * E + lane] : 0.0, v1 = ok1 ? sc[t * E + lane + 64] : 0.0;
        sct[lane] = v0;
        sct[lane + 64] = v1;
        dvt[lane] = ok0 ? dv[t * E + lane] : 0.0;
        dvt[lane + 64] = ok1 ? dv[t * E + lane + 64] : 0.0;
        // the picks by a 32-bit key: the order-preserving image of the score's
        // fp32 rounding with its low 7 bits replaced by 127 - expert (larger
        // first, then the lower index).  The fp64 certificate below proves the
        // picks and their order, or sends the token to the rescoring, so the
        // key's coarser resolution only matters for pairs the bounds cannot
        // separate anyway.
        uint32_t q0 = ok0 ? topk_key32(v0, lane) : 0u, q1 = ok1 ? topk_key32(v1, lane + 64) : 0u;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r >= k) { sel[r] = 0; val[r] = 0.0; continue; }
            const uint32_t best = wave_max_u32(q0 > q1 ? q0 : q1);
            const int e = 127 - (int)(best & 127u);
            sel[r] = e;
            val[r] = sct[e];
            if (e == lane) q0 = 0u;
            if (e == lane + 64) q1 = 0u;
        }
        // certificate: consecutive picks strictly ordered, the k-th strictly
        // above every other expert
        bool cert = true;
        double lo_min = 1e300, kth_lo = 0.0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r >= k) break;
            const double lo = val[r] - dvt[sel[r]];
            lo_min = fmin(lo_min, lo);
            if (r == k - 1) kth_lo = lo;
            if (r + 1 < k && !(lo > val[r + 1] + dvt[sel[r + 1]])) cert = false;
        }
        const double hi0 = ok0 ? v0 + dvt[lane] : -1e300, hi1 = ok1 ? v1 + dvt[lane + 64] : -1e300;
        bool picked0 = false, picked1 = false;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r >= k) break;
            picked0 |= sel[r] == lane;
            picked1 |= sel[r] == lane + 64;
        }
        const bool above = (!picked0 && hi0 >= kth_lo) || (!picked1 && hi1 >= kth_lo);
        cert = cert && !__any(above);
        int nc = 0;
        if (!cert) {
            // every expert whose interval reaches the lowest pick's lower bound,
            // listed in increasing index, for rescoring in fp64 from exact products
            const bool c0 = ok0 && hi0 >= lo_min, c1 = ok1 && hi1 >= lo_min;
            const uint64_t b0 = __ballot(c0), b1 = __ballot(c1);
            const int n0 = __popcll(b0);
            nc = n0 + __popcll(b1);
            if (c0) cnd[__popcll(b0 & lanemask_lt())] = lane;
            if (c1) cnd[n0 + __popcll(b1 & lanemask_lt())] = lane + 64;
        }
        if (lane == 0) s_nc = nc;
    }
    __syncthreads();
    const int nc = __builtin_amdgcn_readfirstlane(s_nc);  // 0: certified (uniform)
    if (nc > 0) {
        // wave w rescores candidates 8 w .. 8 w + 7, 8 w + 32 .., lane l holding
        // elements 8 l .. 8 l + 7 of every 512-wide chunk of the token row and of
        // each candidate row (16-byte loads), eight candidates' loads in flight
        double xh[8 * NC8];
#pragma unroll
        for (int c = 0; c < NC8; ++c) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(x + t * H + 512 * c + 8 * lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xh[8 * c + 2 * q] = (double)__uint_as_float(v[q] << 16);
                xh[8 * c + 2 * q + 1] = (double)__uint_as_float(v[q] & 0xFFFF0000u);
            }
        }
        for (int c0i = 8 * wave; c0i < nc; c0i += 32) {
            u32x4 wv[8][NC8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bf16_t* wr = W + (int64_t)cnd[min(c0i + u, nc - 1)] * H + 8 * lane;
#pragma unroll
                for (int c = 0; c < NC8; ++c) wv[u][c] = *reinterpret_cast<const u32x4*>(wr + 512 * c);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                double acc = 0.0;
#pragma unroll
                for (int c = 0; c < NC8; ++c)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc = fma(xh[8 * c + 2 * q], (double)__uint_as_float(wv[u][c][q] << 16), acc);
                        acc = fma(xh[8 * c + 2 * q + 1], (double)__uint_as_float(wv[u][c][q] & 0xFFFF0000u), acc);
                    }
                const double sum = wave_sum_dpp_f64(acc);
                if (lane == 0 && c0i + u < nc) {
                    const int e = cnd[c0i + u];
                    rst[c0i + u] = sum + (bias ? (double)bias[e] : 0.0);
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            // the rescored values replace the matrix-core ones (the plain softmax
            // sums over every expert), then the top k among the candidates by
            // fp64 value (all others lie below them), ties to the lower index: a
            // candidate's rank is the number before it in that order (the list
            // is in increasing index), and ranks below k are the picks
            if (lane < nc) sct[cnd[lane]] = rst[lane];
            if (lane + 64 < nc) sct[cnd[lane + 64]] = rst[lane + 64];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = lane + 64 * h;
                if (i < nc) {
                    const double v = rst[i];
                    int rank = 0;
                    for (int j = 0; j < nc; ++j) {
                        const double u = rst[j];
                        rank += (u > v || (u == v && j < i)) ? 1 : 0;
                    }
                    if (rank < k) {
                        s_topi[rank] = cnd[i];
                        s_topv[rank] = v;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r >= k) break;
                sel[r] = s_topi[r];
                val[r] = s_topv[r];
            }
        }
    }
    if (wave != 0) return;

    // weights: lane r < k takes pick r; e^(s - s_max) over the picks' sum
    // (norm_topk_prob) or over all E terms
    const double m = val[0];
    int my_e = 0;
    double my_v = 0.0;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        if (lane == r) { my_e = sel[r]; my_v = val[r]; }
    const double my_x = lane < k ? exp(my_v - m) : 0.0;
    double den;
    if (norm) {
        den = wave_sum_dpp_f64(my_x);
    } else {
        const double part = (ok0 ? exp(sct[lane] - m) : 0.0) + (ok1 ? exp(sct[lane + 64] - m) : 0.0);
        den = wave_sum_dpp_f64(part);
    }
    if (lane < k) {
        idx_out[t * k + lane] = my_e;
        w_out[t * k + lane] = (float)(my_x / den);
        atomicOr(&mask[my_e >> 5], 1u << (my_e & 31));
        atomicAdd(&counts[my_e], 1);
    }
}

// ---------------------------------------------------------------------------
// Expert kernel.
//
// Items, one per workgroup:
//  - b < Nsd (= H / 64): tile b of the shared expert's down product,
//    y_shared[:, 64 b .. 64 b + 63] = h_shared W_sd^T for all T tokens (h_shared
//    [T, Is] from the selection launch), stored complete as partial slot
//    k S.
//  - b >= Nsd: routed item q = b - Nsd: slice s = q % S of the (q / S)-th
//    touched expert e, in increasing index, from the 128-bit mask of touched
//    experts the selection launch leaves (one 16-byte read), so the items of
//    untouched experts take no workgroup and sit at the end of the grid.  Its
//    slice is 64 rows of gate and of up ([64, H] each) and the matching 64
//    columns of down ([H, 64]), 384 KB for H = 1024.  The item's first weight
//    blocks are requested before the rest of the routing is read; then wave 0
//    reads the whole routing (T k indices) and lists the item's tokens: the
//    pairs (t, j) with idx[t, j] == e, in (t, j) order.  For each pair the item
//    stores the partial output row
//      P[t, j S + s] = (SiLU(x_t gate_s^T) * (x_t up_s^T)) down_s^T      (bf16, [H])
//    so that the expert's output is the sum of its S slots.
//
// Up to 16 rows (the usual case: 3 tokens per expert on average at T = 64) the
// four waves split K.  Wave w streams the 128 gate/up rows over K quarter w (16
// blocks of 16 rows x 256 B), with the quarter of each token row it needs in
// registers, and then down rows H/4 w .. + H/4 (8 blocks of 32 rows x 128 B);
// the gate/up quarters meet once, in LDS.  Each 4 KB block goes global ->
// registers (about three blocks in flight) -> the wave's own LDS stage, stored
// so that the matrix-core fragments read back conflict-free: row r, 16-byte
// chunk c at r * 256 + 16 (c ^ (r % 16)).  LDS operations of one wave run in
// order, so the stage needs no barrier.
//
// More rows (a crowded expert) and the shared down tiles take the M-split form:
// wave w owns token rows 16 w .. 16 w + 15, and the four waves load each block
// together (one barrier on each side).
struct DecodeArgs {
    const bf16_t* x;          // [T, H]
    const int32_t* idx;       // [T, k]
    const uint32_t* mask;     // [4] touched experts (bit e of word e / 32)
    const bf16_t* gate;       // [E, I, H]
    const bf16_t* up;         // [E, I, H]
    const bf16_t* down;       // [E, H, I]
    const bf16_t* hs;         // [T, Is] shared expert's SiLU(gate) * up (nullable when Is == 0)
    const bf16_t* sdown;      // [H, Is]
    bf16_t* part;             // [T, NP, H]
    int T, E, k, I, Is, S, Nsd, NP;
};

// Stage layout: 256-byte rows; 16-byte chunk c of row r sits at
// r * 256 + 16 (c ^ (r % 16)).  A block is written with lane (row 4 i + lg,
// chunk li) per store i and read back as matrix-core fragments (row li or a
// row pair, chunk 4 ks + lg), both without bank conflicts.  Every offset below
// is a per-lane part (one of four XOR patterns) plus a constant.
template <int H>
__global__ __launch_bounds__(256, 3) void decode_experts_kernel(DecodeArgs a) {
    using namespace dec;
    constexpr int KQ = H / 4;             // K quarter of a wave (K-split form)
    constexpr int NKQ = KQ / 128;         // 128-wide K blocks per quarter
    constexpr int NGU = 8 * NKQ;          // gate/up blocks per wave: 16 gate or 16 up rows x 128 K
    constexpr int NDN = KQ / 32;          // down blocks per wave: 32 output rows x 64 K
    constexpr int NB = NGU + NDN;
    constexpr int NXK = KQ / 32;          // 32-wide K steps of a quarter
    constexpr int MGU = H / 128, MDN = H / 256, MB = MGU + MDN;  // M-split blocks
    static_assert(H % 512 == 0, "hidden size");

    __shared__ __attribute__((aligned(1024))) char stage[kWaves * kStage];
    __shared__ __attribute__((aligned(16))) bf16_t hl[kMaxT * kHRow];
    __shared__ int list[kMaxT];
    __shared__ int dst[kMaxT];
    __shared__ int s_m;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;

    // lane parts of the stage offsets
    int st_l[4];   // store i: st_l[i % 4] + 1024 i
    int gr_l[4];   // gate/up fragment of K step ks: gr_l[ks] + 4096 (16-row group)
    int dr_l[4];   // down fragment: dr_l[2 ks + (nt & 1)] + 2048 nt
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        st_l[q] = lg * 256 + (((li ^ lg) ^ (4 * q)) << 4);
        gr_l[q] = li * 256 + (((li ^ lg) ^ (4 * q)) << 4);
    }
    {
        const int bc = ((8 * (li & 1)) | lg) ^ (li >> 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int p = 0; p < 2; ++p) dr_l[2 * ks + p] = (li >> 1) * 256 + ((bc ^ (4 * ks) ^ (8 * p)) << 4);
    }
    auto stash = [&](char* base, const u32x4 (&r)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_write16(base, st_l[i & 3] + 1024 * i, r[i]);
    };
    auto stash4 = [&](char* base, const u32x4 (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_write16(base, st_l[i] + 1024 * i, r[i]);
    };

    if ((int)blockIdx.x < a.Nsd) {
        // ===================== shared down tile ===============================
        // out [T, 64] = hs [T, Is] sdown[n0 .. n0 + 63, :]^T, K in blocks of 128:
        // wave w loads weight rows 16 w .. 16 w + 15 of the block (stage rows)
        // and computes token rows 16 w .. 16 w + 15 over all 64 columns.
        const int n0 = 64 * blockIdx.x, Is = a.Is, T = a.T;
        const rsrc_t sw = make_rsrc(a.sdown + (int64_t)n0 * Is, 64 * Is * 2);
        const rsrc_t hw = make_rsrc(a.hs, (uint32_t)T * Is * 2);
        const uint32_t w_l = (uint32_t)((16 * wave + lg) * Is + 8 * li) * 2;
        const bool active = 16 * wave < T;
        const uint32_t h_l = (uint32_t)(min(16 * wave + li, T - 1) * Is + 8 * lg) * 2;
        const int nkb = Is / 128;
        u32x4 rw[4], ha[4];
        auto issue_s = [&](int b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rw[i] = bload(sw, w_l, (4 * i * Is + 128 * b) * 2);
        };
        issue_s(0);
        f32x4 acc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll 1
        for (int b = 0; b < nkb; ++b) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ha[ks] = bload(hw, h_l, 256 * b + 64 * ks);
            __syncthreads();  // every wave is done reading the previous block
            stash4(stage + 4096 * wave, rw);
            __syncthreads();
            if (b + 1 < nkb) issue_s(b + 1);
            if (active)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[nt] = mfma(ha[ks], lds_read16(stage, gr_l[ks] + 4096 * nt), acc[nt]);
                    sched_fence();
                }
        }
        if (!active) return;
        char* out = reinterpret_cast<char*>(a.part) + (int64_t)(a.k * a.S) * H * 2 + (n0 + li) * 2;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = acc[nt][r];
                const float vn = __uint_as_float(
                    __builtin_amdgcn_mov_dpp(__float_as_uint(v), 0xb1, 0xf, 0xf, false));  // lane ^ 1
                const int t = 16 * wave + 4 * lg + r;
                if ((li & 1) == 0 && t < T)
                    *reinterpret_cast<uint32_t*>(out + ((int64_t)t * a.NP * H + 16 * nt) * 2) = pack_bf16x2(v, vn);
            }
        return;
    }

    // ===================== routed item: which one, and its rows ==============
    const int q = (int)blockIdx.x - a.Nsd;
    const int s = q % a.S;
    // wave 0 requests the whole routing (T k indices) at once, beside the mask
    const int n_pairs = a.T * a.k;
    int v[8];
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 64 * i + lane < n_pairs ? a.idx[64 * i + lane] : -1;
    }
    int e = -1;
    {
        // the (q / S)-th touched expert, in increasing index (wave-uniform)
        const u32x4 mk = *reinterpret_cast<const u32x4*>(a.mask);
        int r = q / a.S;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t bits = __builtin_amdgcn_readfirstlane(mk[w]);
            const int c = __popc(bits);
            if (e < 0 && r < c) {
                for (int j = 0; j < r; ++j) bits &= bits - 1;  // drop the r lowest set bits
                e = 32 * w + __ffs(bits) - 1;
            }
            if (e < 0) r -= c;
        }
    }
    if (e < 0) return;  // past the last touched expert's items (uniform)
    const int ldd = a.I;
    // the slice: 64 gate rows and 64 up rows [64, H], 64 columns of down [H, I]
    const rsrc_t gw = make_rsrc(a.gate + ((int64_t)e * a.I + s * kSlice) * H, kSlice * H * 2);
    const rsrc_t uw = make_rsrc(a.up + ((int64_t)e * a.I + s * kSlice) * H, kSlice * H * 2);
    const rsrc_t dw = make_rsrc(a.down + (int64_t)e * H * a.I + s * kSlice, (uint32_t)((H - 1) * ldd + kSlice) * 2);
    const rsrc_t xw = make_rsrc(a.x, (uint32_t)a.T * H * 2);
    const uint32_t gu_l = (uint32_t)(lg * H + 8 * li) * 2;
    const uint32_t dn_l = (uint32_t)((2 * lg + (li >> 3)) * ldd + 8 * (li & 7)) * 2;
    char* wst = stage + wave * kStage;  // this wave's stage (K-split form)

    // K-split block b of this wave (4 KB): gate/up block b < NGU: 16 rows (gate
    // rows 16 rg .. + 15 when b is even, the same up rows when odd; rg = b / (2
    // NKQ)) over K range KQ wave + 128 kh .. + 127 (kh = (b / 2) % NKQ); down
    // block d = b - NGU: output rows KQ wave + 32 d .. + 31, two per stage row.
    auto issue_a = [&](int b, u32x4 (&r)[4]) {
        if (b < NGU) {
            const int rg = b / (2 * NKQ), kh = (b / 2) % NKQ;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = bload((b & 1) ? uw : gw, gu_l, ((16 * rg + 4 * i) * H + KQ * wave + 128 * kh) * 2);
        } else {
            const int n0 = KQ * wave + 32 * (b - NGU);
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = bload(dw, dn_l, (uint32_t)(n0 + 8 * i) * ldd * 2);
        }
    };
    // the K-split form's first two blocks are requested before the item's
    // tokens are listed (an M-split item drops them)
    u32x4 r0[4], r1[4];
    issue_a(0, r0);
    issue_a(1, r1);
    if (wave == 0) {
        // the item's tokens
        int base = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool hit = v[i] == e;
            const uint64_t bal = __ballot(hit);
            if (hit) {
                const int p = 64 * i + lane, at = base + __popcll(bal & lanemask_lt());
                const int t = p / a.k, j = p - t * a.k;
                list[at] = t;
                dst[at] = t * a.NP + j * a.S + s;
            }
            base += __popcll(bal);
        }
        if (lane == 0) s_m = base;
    }
    __syncthreads();
    const int m = __builtin_amdgcn_readfirstlane(s_m);  // uniform, so the two forms are separate paths

    if (m > 16) {
        // ========================= M-split form ==================================
        // block b of the workgroup (32 KB): gate/up block b < MGU: stage rows 0..63
        // gate, 64..127 up, K range 128 b .. + 127 (wave w loads stage rows
        // 32 w .. 32 w + 31); down block d = b - MGU: output rows 256 d .. + 255, two
        // per stage row.
        auto issue_m = [&](int b, u32x4 (&r)[8]) {
            if (b < MGU) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    r[i] = bload(wave < 2 ? gw : uw, gu_l, ((32 * (wave & 1) + 4 * i) * H + 128 * b) * 2);
            } else {
                const int n0 = 256 * (b - MGU) + 64 * wave;
#pragma unroll
                for (int i = 0; i < 8; ++i) r[i] = bload(dw, dn_l, (uint32_t)(n0 + 8 * i) * ldd * 2);
            }
        };
        u32x4 rm[8];
        char* mst = stage + wave * 8192;  // this wave's 32 stage rows
        for (int m0 = 0; m0 < m; m0 += 64) {
            const int mr = min(64, m - m0);
            const bool active = 16 * wave < mr;    // this wave's token rows exist
            const int row = m0 + 16 * wave + (li < mr - 16 * wave ? li : 0);
            const uint32_t x_l = (uint32_t)(list[active ? row : m0] * H + 8 * lg) * 2;
            issue_m(0, rm);
            u32x4 xa[4], xn[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) xa[ks] = bload(xw, x_l, 64 * ks);
            f32x4 ag[4], au[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { ag[i] = f32x4{0, 0, 0, 0}; au[i] = f32x4{0, 0, 0, 0}; }
#pragma unroll 1
            for (int b = 0; b < MGU; ++b) {
                __syncthreads();  // every wave is done reading the previous block
                stash(mst, rm);
                __syncthreads();
                issue_m(b + 1, rm);  // b + 1 <= MGU < MB
                const int bn = b + 1 < MGU ? b + 1 : b;  // the last block reloads its own x (unused)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) xn[ks] = bload(xw, x_l, 256 * bn + 64 * ks);
                if (active)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                        for (int nt = 0; nt < 4; ++nt) {
                            ag[nt] = mfma(xa[ks], lds_read16(stage, gr_l[ks] + 4096 * nt), ag[nt]);
                            au[nt] = mfma(xa[ks], lds_read16(stage, gr_l[ks] + 16384 + 4096 * nt), au[nt]);
                        }
                        sched_fence();
                    }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) xa[ks] = xn[ks];
            }
            // h rows of this wave's tokens (the lane holds rows 4 lg + r, column 16 nt + li)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hl[(16 * wave + 4 * lg + r) * kHRow + 16 * nt + li] = f32_to_bf16(silu(ag[nt][r]) * au[nt][r]);
            __syncthreads();
            u32x4 hA[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                hA[ks] = *reinterpret_cast<const u32x4*>(hl + (16 * wave + li) * kHRow + 32 * ks + 8 * lg);
            // output rows of this lane: 4 lg + r of the wave's 16
            uint32_t orow[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = 16 * wave + 4 * lg + r;
                orow[r] = rr < mr ? (uint32_t)dst[m0 + rr] * H * 2 : 0xFFFFFFFFu;
            }
#pragma unroll 1
            for (int d = 0; d < MDN; ++d) {
                __syncthreads();
                stash(mst, rm);
                __syncthreads();
                if (MGU + d + 1 < MB) issue_m(MGU + d + 1, rm);
                if (!active) continue;
                // four groups of four 16-column tiles, each stored as it completes
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    f32x4 acc[4];
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int nt = 4 * g4 + qq;
                        acc[qq] = f32x4{0, 0, 0, 0};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
                            acc[qq] = mfma(hA[ks], lds_read16(stage, dr_l[2 * ks + (nt & 1)] + 2048 * nt), acc[qq]);
                    }
                    // pairs of neighbouring columns into one 4-byte store from the even lane
                    char* out = reinterpret_cast<char*>(a.part) + (256 * d + 64 * g4 + li) * 2;
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float vv = acc[qq][r];
                            const float vn = __uint_as_float(
                                __builtin_amdgcn_mov_dpp(__float_as_uint(vv), 0xb1, 0xf, 0xf, false));  // lane ^ 1
                            if ((li & 1) == 0 && orow[r] != 0xFFFFFFFFu)
                                *reinterpret_cast<uint32_t*>(out + orow[r] + 32 * qq) = pack_bf16x2(vv, vn);
                        }
                    sched_fence();
                }
            }
            __syncthreads();  // hl and the stage are reused by the next group of 64 rows
        }
        return;
    }

    // ===================== K-split form ==================================
    const uint32_t x_l = (uint32_t)(list[li < m ? li : 0] * H + 8 * lg) * 2;
    u32x4 xr[NXK];
#pragma unroll
    for (int j = 0; j < NXK; ++j) xr[j] = bload(xw, x_l, (KQ * wave + 32 * j) * 2);
    f32x4 ag[4], au[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { ag[i] = f32x4{0, 0, 0, 0}; au[i] = f32x4{0, 0, 0, 0}; }
    u32x4 hA[2];
    const int erow = lane >> 2, ec = lane & 3;
    const uint32_t out_l = erow < m ? (uint32_t)dst[erow] * H * 2 + 16 * ec : 0;

#pragma unroll
    for (int b = 0; b < NB; ++b) {
        u32x4(&rc)[4] = (b & 1) ? r1 : r0;
        // block order is fixed: wait for block b, store it, refill its
        // registers with block b + 2, then compute on it
        sched_fence();
        if (b == NGU) {
            // The gate/up quarters meet: each wave's fp32 tile [128 columns][16
            // rows] goes to its own stage, then every thread forms 4 h values.
            float* red = reinterpret_cast<float*>(wst);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<f32x4*>(red + (16 * i + li) * 16 + 4 * lg) = ag[i];
                *reinterpret_cast<f32x4*>(red + (64 + 16 * i + li) * 16 + 4 * lg) = au[i];
            }
            __syncthreads();
            {
                const int col = tid & 63, rq = tid >> 6;  // rows 4 rq .. 4 rq + 3
                const float* r4 = reinterpret_cast<const float*>(stage);
                f32x4 g = f32x4{0, 0, 0, 0}, u = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    g += *reinterpret_cast<const f32x4*>(r4 + w * (kStage / 4) + col * 16 + 4 * rq);
                    u += *reinterpret_cast<const f32x4*>(r4 + w * (kStage / 4) + (64 + col) * 16 + 4 * rq);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) hl[(4 * rq + r) * kHRow + col] = f32_to_bf16(silu(g[r]) * u[r]);
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                hA[ks] = *reinterpret_cast<const u32x4*>(hl + li * kHRow + 32 * ks + 8 * lg);
        }
        stash4(wst, rc);
        if (b + 2 < NB) issue_a(b + 2, rc);
        sched_fence();
        if (b < NGU) {
            const int rg = b / (2 * NKQ), kh = (b / 2) % NKQ;
            f32x4& acc = (b & 1) ? au[rg] : ag[rg];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma(xr[4 * kh + ks], lds_read16(wst, gr_l[ks]), acc);
        } else {
            f32x4 acc[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    acc[nt] = mfma(hA[ks], lds_read16(wst, dr_l[2 * ks + nt] + 2048 * nt), acc[nt]);
            }
            // tile [16 rows][32 columns] -> bf16 rows in the stage -> 16-byte stores
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<bf16_t*>(wst + (4 * lg + r) * kERow + (16 * nt + li) * 2) =
                        f32_to_bf16(acc[nt][r]);
            const u32x4 o = lds_read16(wst, erow * kERow + 16 * ec);
            if (erow < m)
                *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.part) + (KQ * wave + 32 * (b - NGU)) * 2 +
                                          out_l) = o;
        }
    }
}

// ---------------------------------------------------------------------------
bool decode_layer_ok(int dtype, int64_t T, int H, int E, int k, int I, int Is) {
    return dtype == kBF16 && T >= 1 && T <= dec::kMaxT && H == dec::kH && E >= 1 && E <= 128 && k >= 1 &&
           k <= 8 && k <= E && I % dec::kSlice == 0 && I >= dec::kSlice && Is >= 0 && Is % 128 == 0;
}

int decode_partial_rows(int k, int I, int Is) { return k * (I / dec::kSlice) + (Is > 0 ? 1 : 0); }

hipError_t launch_route_decode(const void* x, const void* W, const float* bias, int64_t T, int H, int E, int k,
                               int norm, double* sc, double* dv, int32_t* idx, float* w, const void* sg,
                               const void* su, int Is, void* hs, uint32_t* mask, int32_t* counts, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (H != dec::kH || E < 1 || E > 128 || k < 1 || k > 8 || k > E || Is < 0 || Is % 128 != 0 ||
        (Is > 0 && (!sg || !su || !hs)) || !mask || !counts)
        return hipErrorInvalidValue;
    const int nsc = (int)(((T + 7) / 8) * ((E + 15) / 16));
    const int nsel = (int)T;                          // one selection workgroup per token
    // shared gate/up: feature groups x token groups
    const int nsk = (Is / 8) * (int)((T + dec::kSharedRows - 1) / dec::kSharedRows);
    route_scores_kernel<dec::kH><<<(unsigned)nsc, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)W, bias, (int)T,
                                                                E, sc, dv, mask, counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    route_select_kernel<dec::kH><<<(unsigned)(nsel + nsk), 256, 0, st>>>(
        (const bf16_t*)x, (const bf16_t*)W, bias, sc, dv, (int)T, E, k, norm, idx, w, mask, counts,
        (const bf16_t*)sg, (const bf16_t*)su, Is, (bf16_t*)hs);
    return hipGetLastError();
}

hipError_t launch_decode_experts(const void* x, const int32_t* idx, const uint32_t* mask, const void* gate,
                                 const void* up, const void* down, const void* hs, const void* sdown, void* part,
                                 int64_t T, int H, int E, int k, int I, int Is, hipStream_t st, hipEvent_t ev_start,
                                 hipEvent_t ev_stop) {
    if (T <= 0) return hipSuccess;
    if (H != dec::kH || !mask || (Is > 0 && (!hs || !sdown))) return hipErrorInvalidValue;
    DecodeArgs a;
    a.x = (const bf16_t*)x;
    a.idx = idx;
    a.mask = mask;
    a.gate = (const bf16_t*)gate;
    a.up = (const bf16_t*)up;
    a.down = (const bf16_t*)down;
    a.hs = (const bf16_t*)hs;
    a.sdown = (const bf16_t*)sdown;
    a.part = (bf16_t*)part;
    a.T = (int)T;
    a.E = E;
    a.k = k;
    a.I = I;
    a.Is = Is;
    a.S = I / dec::kSlice;
    a.Nsd = Is > 0 ? H / 64 : 0;
    a.NP = decode_partial_rows(k, I, Is);
    // the shared down tiles, then a slot for every (expert, slice); the items of
    // the touched experts come first and the rest end at once
    const unsigned grid = (unsigned)(a.Nsd + E * a.S);
    if (!ev_start && !ev_stop) {
        decode_experts_kernel<dec::kH><<<grid, 256, 0, st>>>(a);
        return hipGetLastError();
    }
    void* argv[] = {&a};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(decode_experts_kernel<dec::kH>), dim3(grid), dim3(256),
                              argv, 0, st, ev_start, ev_stop, 0);
}

}  // namespace tmoe
