// Grouping of (token, slot) pairs by expert: a stable counting sort over the
// Top-k routing, so that each expert's rows can be processed as one matrix
// product ("3C · Talker MoE (20 lớp, 128 Experts Top-6)", openarchlab, §3:
// every token visits the experts in its S).  Also builds the tile lists of the
// grouped matrix products on the device, so the host never waits for counts.
//
//   hist    : per-block expert histogram          (blocks of kPermChunk pairs)
//   scan    : counts, offsets, per-block bases, tile lists   (one block)
//   scatter : stable ranks via wave ballots, writes the grouping
#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {

__device__ int block_exclusive_scan(int v, int* lds /* >= 17 ints */, int* total) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int nwaves = (blockDim.x + 63) >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    if (lane == kWave - 1) lds[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nwaves; ++w) { int t = lds[w]; lds[w] = run; run += t; }
        lds[16] = run;
    }
    __syncthreads();
    int res = lds[wave] + incl - v;
    *total = lds[16];
    __syncthreads();
    return res;
}

// Tile list of one grouped product from per-expert counts/offsets.  Items of
// one (expert, column tile) are consecutive so that tiles sharing a weight
// block are adjacent in the launch order.
__device__ void block_build_items(int c, int off, int E, int64_t T, const TileSpec& ts, int* lds) {
    // Never writes past max_items (which bounds every valid routing); a
    // malformed grouping only loses tiles.
    const int e = threadIdx.x;
    const int nN = ts.n_routed / ts.nt;
    if (c < 0) c = 0;
    const int nmt = (e < E) ? (c + ts.mt - 1) / ts.mt : 0;
    int total_routed;
    const int base = block_exclusive_scan(nmt * nN, lds, &total_routed);
    for (int n = 0; n < nN; ++n)
        for (int m = 0; m < nmt; ++m) {
            int rows = c - m * ts.mt;
            if (rows > ts.mt) rows = ts.mt;
            const int at = base + n * nmt + m;
            if (at < ts.max_items) ts.items[at] = make_int4(e, n * ts.nt, off + m * ts.mt, rows);
        }
    int count_s = 0;
    if (ts.n_shared > 0) {
        const int nNs = ts.n_shared / ts.nt;
        const int nmts = (int)((T + ts.mt - 1) / ts.mt);
        count_s = nNs * nmts;
        for (int q = threadIdx.x; q < count_s; q += blockDim.x) {
            int n = q / nmts, m = q % nmts;
            int64_t rows = T - (int64_t)m * ts.mt;
            if (rows > ts.mt) rows = ts.mt;
            if (total_routed + q < ts.max_items)
                ts.items[total_routed + q] = make_int4(E, n * ts.nt, m * ts.mt, (int)rows);
        }
    }
    if (threadIdx.x == 0) *ts.count = min(total_routed + count_s, ts.max_items);
}

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ idx, int64_t N, int E,
                                                        int32_t* __restrict__ hist) {
    __shared__ int cnt[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int64_t start = (int64_t)blockIdx.x * kPermChunk;
    const int64_t end = min(start + (int64_t)kPermChunk, N);
    for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) {
        int e = idx[i];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

struct TileSpecs {
    TileSpec t[2];
    int n;
};

__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ hist, int nb, int E, int64_t T,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         TileSpecs specs) {
    __shared__ int lds[17];
    const int e = threadIdx.x;
    int c = 0;
    if (e < E)
        for (int b = 0; b < nb; ++b) c += hist[(int64_t)b * E + e];
    int total;
    const int excl = block_exclusive_scan(e < E ? c : 0, lds, &total);
    if (e < E) {
        counts[e] = c;
        offsets[e] = excl;
        int run = excl;
        for (int b = 0; b < nb; ++b) {
            int h = hist[(int64_t)b * E + e];
            hist[(int64_t)b * E + e] = run;
            run += h;
        }
    }
    if (e == 0) offsets[E] = total;
    for (int s = 0; s < specs.n; ++s) block_build_items(c, excl, E, T, specs.t[s], lds);
}

__global__ __launch_bounds__(1024) void build_items_kernel(const int32_t* __restrict__ offsets, int E, int64_t T,
                                                           TileSpecs specs) {
    __shared__ int lds[17];
    const int e = threadIdx.x;
    int c = 0, off = 0;
    if (e < E) { off = offsets[e]; c = offsets[e + 1] - off; }
    for (int s = 0; s < specs.n; ++s) block_build_items(c, off, E, T, specs.t[s], lds);
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                          int nbits, const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ row_token, int32_t* __restrict__ row_of,
                                                          const float* __restrict__ w, int32_t* __restrict__ row_dst,
                                                          float* __restrict__ row_scale, int slots) {
    __shared__ int run[kMaxExperts];
    const int lane = lane_id();
    for (int e = lane; e < E; e += kWave) run[e] = base[(int64_t)blockIdx.x * E + e];
    __syncthreads();  // one wave per block: orders the stores above before the loop's reads
    const int64_t start = (int64_t)blockIdx.x * kPermChunk;
    const int64_t end = min(start + (int64_t)kPermChunk, N);
    const uint64_t lt = lanemask_lt();
    for (int64_t i0 = start; i0 < end; i0 += kWave) {
        const int64_t i = i0 + lane;
        bool valid = i < end;
        int e = valid ? idx[i] : 0;
        valid = valid && e >= 0 && e < E;
        uint64_t match = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            bool bit = (e >> b) & 1;
            uint64_t m = __ballot(bit);
            match &= bit ? m : ~m;
        }
        if (!valid) match = 0;
        const int leader = valid ? (__ffsll((unsigned long long)match) - 1) : lane;
        const int rank = __popcll(match & lt);
        int pos = 0;
        if (valid && lane == leader) {
            pos = run[e];
            run[e] = pos + __popcll(match);
        }
        pos = __shfl(pos, leader, kWave);
        if (valid) {
            const int dst = pos + rank;
            const int t = (int)(i / k), j = (int)(i % k);
            row_token[dst] = t;
            row_of[i] = dst;
            if (row_dst) {
                row_dst[dst] = t * slots + j;
                row_scale[dst] = w[i];
            }
        }
    }
}

int64_t tile_max_items(int64_t pairs, int E, int64_t T, int mt, int nt, int n_routed, int n_shared) {
    int64_t routed = (pairs / mt + E) * (int64_t)(n_routed / nt);
    int64_t shared = n_shared > 0 ? ((T + mt - 1) / mt) * (int64_t)(n_shared / nt) : 0;
    return routed + shared;
}

static TileSpecs make_specs(const TileSpec* t1, const TileSpec* t2) {
    TileSpecs s{};
    if (t1) s.t[s.n++] = *t1;
    if (t2) s.t[s.n++] = *t2;
    return s;
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, int32_t* hist, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* row_of, const float* w,
                          int32_t* row_dst, float* row_scale, int slots, const TileSpec* t1, const TileSpec* t2,
                          hipStream_t st) {
    const int64_t N = T * k;
    const int nb = (int)((N + kPermChunk - 1) / kPermChunk);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    perm_hist_kernel<<<nb, 256, 0, st>>>(idx, N, E, hist);
    perm_scan_kernel<<<1, 1024, 0, st>>>(hist, nb, E, T, counts, offsets, make_specs(t1, t2));
    perm_scatter_kernel<<<nb, 64, 0, st>>>(idx, N, k, E, nbits, hist, row_token, row_of, w, row_dst, row_scale,
                                           slots);
    return hipGetLastError();
}

hipError_t launch_build_items(const int32_t* offsets, int E, int64_t T, const TileSpec* t1, const TileSpec* t2,
                              hipStream_t st) {
    build_items_kernel<<<1, 1024, 0, st>>>(offsets, E, T, make_specs(t1, t2));
    return hipGetLastError();
}

}  // namespace tmoe
