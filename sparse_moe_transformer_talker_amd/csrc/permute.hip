// Grouping of (token, slot) pairs by expert: a stable counting sort over the
// Top-k routing, so that each expert's rows can be processed as one matrix
// product ("3C · Talker MoE (20 lớp, 128 Experts Top-6)", openarchlab, §3:
// every token visits the experts in its S).  Also builds the tile lists of the
// grouped matrix products on the device, so the host never waits for counts.
//
// A token's k experts are distinct, so the rows of expert e are exactly the
// tokens whose routing contains e, in ascending token order.  The router
// records that as one 16-bit mask per (expert, block of 16 tokens):
//   mask  : masks from topk_idx (only when the router did not write them)
//   prefix: per expert, exclusive prefix of mask popcounts; counts, offsets,
//           tile lists                                          (one block)
//   scatter: rank of (t, j) = prefix + popcount of the lower bits of its word;
//           one thread per pair, no atomics
#include "grouping.hpp"

namespace tmoe {

// masks[e * mstride + b], bit t % 16 of word b = t / 16: token t routes to e.
__global__ __launch_bounds__(256) void perm_mask_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                        uint16_t* __restrict__ masks, int mstride) {
    __shared__ uint32_t msk[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) msk[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    for (int q = threadIdx.x; q < 16 * k; q += blockDim.x) {
        const int64_t t = t0 + q / k;
        if (t >= T) continue;
        const int e = idx[t * k + q % k];
        if (e >= 0 && e < E) atomicOr(&msk[e], 1u << (q / k));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
}

// One block of 1024 threads.  Wave w takes experts w, w + 16, ...; lanes take
// 4 consecutive mask words (one 8-byte load), words >= nwords read as empty.
__global__ __launch_bounds__(1024) void perm_prefix_kernel(const uint16_t* __restrict__ masks, int nwords,
                                                           int mstride, int E, int64_t T,
                                                           int32_t* __restrict__ prefix,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets, TileSpecs specs) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int lds[17];
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    for (int e0 = wave; e0 < E; e0 += 4 * nwaves) {
        // four experts per pass, their loads issued together
        uint64_t wv[4];
        int run[4] = {0, 0, 0, 0};
        for (int c0 = 0; c0 < mstride; c0 += 4 * kWave) {
            const int wd = c0 + 4 * lane;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * nwaves;
                wv[u] = (e < E && wd < mstride)
                            ? *reinterpret_cast<const uint64_t*>(masks + (int64_t)e * mstride + wd)
                            : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * nwaves;
                int pc[4], sum = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t word = (wd + q < nwords) ? (uint32_t)((wv[u] >> (16 * q)) & 0xFFFFu) : 0u;
                    pc[q] = __popc(word);
                    sum += pc[q];
                }
                const int incl = wave_incl_scan(sum);
                int p = run[u] + incl - sum;
                if (e < E) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (wd + q < nwords) prefix[(int64_t)e * mstride + wd + q] = p;
                        p += pc[q];
                    }
                }
                run[u] += __builtin_amdgcn_readlane(incl, kWave - 1);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * nwaves;
            if (e < E && lane == 0) cnt[e] = run[u];
        }
    }
    __syncthreads();
    const int e = threadIdx.x;
    const int c = e < E ? cnt[e] : 0;
    int total;
    const int excl = block_exclusive_scan(c, lds, &total);
    if (e < E) {
        counts[e] = c;
        offsets[e] = excl;
    }
    if (e == 0) offsets[E] = total;
    for (int s = 0; s < specs.n; ++s) block_build_items(c, excl, E, T, specs.t[s], lds);
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                           const uint16_t* __restrict__ masks, int mstride,
                                                           const int32_t* __restrict__ prefix,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ row_of,
                                                           const float* __restrict__ w,
                                                           int32_t* __restrict__ row_dst,
                                                           float* __restrict__ row_scale, int slots) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const int e = idx[i];
    if (e < 0 || e >= E) return;
    const int t = (int)(i / k), j = (int)(i % k);
    const int64_t m = (int64_t)e * mstride + (t >> 4);
    const uint32_t below = (uint32_t)masks[m] & ((1u << (t & 15)) - 1u);
    const int dst = offsets[e] + prefix[m] + __popc(below);
    if (dst < 0 || dst >= N) return;  // only a grouping inconsistent with idx gets here
    row_token[dst] = t;
    row_of[i] = dst;
    if (row_dst) {
        row_dst[dst] = t * slots + j;
        row_scale[dst] = w[i];
    }
}

__global__ __launch_bounds__(1024) void build_items_kernel(const int32_t* __restrict__ offsets, int E, int64_t T,
                                                           TileSpecs specs) {
    __shared__ int lds[17];
    const int e = threadIdx.x;
    int c = 0, off = 0;
    if (e < E) { off = offsets[e]; c = offsets[e + 1] - off; }
    for (int s = 0; s < specs.n; ++s) block_build_items(c, off, E, T, specs.t[s], lds);
}

int mask_words(int64_t T) { return (int)((T + 15) / 16); }
int mask_stride(int64_t T) { return (mask_words(T) + 3) & ~3; }

int64_t tile_max_items(int64_t pairs, int E, int64_t T, int mt, int nt, int n_routed, int n_shared) {
    const int64_t routed = (pairs / mt + E) * (int64_t)(n_routed / nt);
    const int64_t shared = n_shared > 0 ? ((T + mt - 1) / mt) * (int64_t)(n_shared / nt) : 0;
    return routed + shared;
}

hipError_t launch_masks(const int32_t* idx, int64_t T, int k, int E, uint16_t* masks, hipStream_t st) {
    perm_mask_kernel<<<(unsigned)mask_words(T), 256, 0, st>>>(idx, T, k, E, masks, mask_stride(T));
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, const uint16_t* masks, int32_t* prefix,
                          int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_of, const float* w,
                          int32_t* row_dst, float* row_scale, int slots, const TileSpec* t1, const TileSpec* t2,
                          hipStream_t st) {
    const int64_t N = T * k;
    perm_prefix_kernel<<<1, 1024, 0, st>>>(masks, mask_words(T), mask_stride(T), E, T, prefix, counts, offsets,
                                            make_specs(t1, t2));
    perm_scatter_kernel<<<(unsigned)((N + 255) / 256), 256, 0, st>>>(idx, N, k, E, masks, mask_stride(T), prefix,
                                                                     offsets, row_token, row_of, w, row_dst,
                                                                     row_scale, slots);
    return hipGetLastError();
}

hipError_t launch_build_items(const int32_t* offsets, int E, int64_t T, const TileSpec* t1, const TileSpec* t2,
                              hipStream_t st) {
    build_items_kernel<<<1, 1024, 0, st>>>(offsets, E, T, make_specs(t1, t2));
    return hipGetLastError();
}

}  // namespace tmoe
