// Block-level helpers of the grouping step, shared by the router's small-batch
// finish kernel and the grouping kernels: an exclusive scan over a block and
// the device-side construction of the grouped GEMM tile lists.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace tmoe {

struct TileSpecs {
    TileSpec t[2];
    int n;
};

inline TileSpecs make_specs(const TileSpec* t1, const TileSpec* t2) {
    TileSpecs s{};
    if (t1) s.t[s.n++] = *t1;
    if (t2) s.t[s.n++] = *t2;
    return s;
}

__device__ inline int block_exclusive_scan(int v, int* lds /* >= 17 ints */, int* total) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int nwaves = (blockDim.x + 63) >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) lds[wave] = incl;
    __syncthreads();
    if (wave == 0) {  // scan of the (at most 16) wave totals
        const int wt = lane < nwaves ? lds[lane] : 0;
        const int s = wave_incl_scan(wt);
        if (lane < nwaves) lds[lane] = s - wt;
        if (lane == kWave - 1) lds[16] = s;
    }
    __syncthreads();
    const int res = lds[wave] + incl - v;
    *total = lds[16];
    __syncthreads();
    return res;
}

// Tile list of one grouped product from per-expert counts/offsets (thread e
// holds expert e).  Items of one (expert, column tile) are consecutive so that
// tiles sharing a weight block are adjacent in the launch order.  Never writes
// past max_items, which bounds every valid routing.
__device__ inline void block_build_items(int c, int off, int E, int64_t T, const TileSpec& ts, int* lds) {
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
            const int n = q / nmts, m = q % nmts;
            int64_t rows = T - (int64_t)m * ts.mt;
            if (rows > ts.mt) rows = ts.mt;
            if (total_routed + q < ts.max_items)
                ts.items[total_routed + q] = make_int4(E, n * ts.nt, m * ts.mt, (int)rows);
        }
    }
    if (threadIdx.x == 0) *ts.count = min(total_routed + count_s, ts.max_items);
}

}  // namespace tmoe
