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

// masks[e * mstride + b], bit t % 16 of word b = t / 16: token t routes to e;
// jmask (nullable, k <= 16) the slot j of that choice in bits 4 (t % 16) .. + 3.
__global__ __launch_bounds__(256) void perm_mask_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                        uint16_t* __restrict__ masks, uint64_t* __restrict__ jmask,
                                                        int mstride) {
    __shared__ uint32_t msk[kMaxExperts];
    __shared__ uint64_t jm[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        msk[e] = 0;
        jm[e] = 0;
    }
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    for (int q = threadIdx.x; q < 16 * k; q += blockDim.x) {
        const int64_t t = t0 + q / k;
        if (t >= T) continue;
        const int e = idx[t * k + q % k];
        if (e >= 0 && e < E) {
            atomicOr(&msk[e], 1u << (q / k));
            if (jmask) atomicOr((unsigned long long*)&jm[e], (unsigned long long)(q % k) << (4 * (q / k)));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        masks[(int64_t)e * mstride + blockIdx.x] = (uint16_t)msk[e];
        if (jmask) jmask[(int64_t)e * mstride + blockIdx.x] = jm[e];
    }
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
                                                           int32_t* __restrict__ row_pair) {
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
    if (row_pair) row_pair[dst] = (int32_t)i;
}

// E <= 128: one block per expert, no cross-block dependency.  Every block
// popcounts the whole mask matrix (E x nwords words) for all counts, so it
// knows every offset and tile base; its first wave then ranks the expert's own
// tokens (word prefix + popcount of the lower bits: ascending token order),
// scatters their rows and writes the expert's tiles.  Block 0 also writes
// counts / offsets, the shared expert's tiles and the tile counts.  The slot j
// of each choice comes from jmask when given (no loads of the routing per
// token), else from idx.
constexpr int kGroupThreads = 256;
constexpr int kGroupMaxE = 128;
constexpr int kGroupLoads = 16;  // 16-byte mask chunks in flight per thread

__global__ __launch_bounds__(kGroupThreads) void group_experts_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, const uint16_t* __restrict__ masks, int nwords,
    int mstride, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_of, const uint64_t* __restrict__ jmask, int32_t* __restrict__ row_pair,
    TileSpecs specs) {
    __shared__ int part[kGroupThreads];
    __shared__ int cnt[kGroupMaxE], off[kGroupMaxE], tbase[2][kGroupMaxE];
    __shared__ int total_rows, total_tiles[2];
    const int tid = threadIdx.x, e = blockIdx.x, lane = tid & 63;
    // 1. counts of every expert: the mask matrix read as one flat array of
    //    16-byte chunks (8 words; words past nwords masked off), chunk q by
    //    thread q % 256, up to kGroupLoads chunks per thread in flight; per-row
    //    sums in LDS (integer adds: the result does not depend on their order)
    const int nch = mstride / 8, nq = E * nch;
    if (tid < kGroupMaxE) part[tid] = 0;
    __syncthreads();
    for (int q0 = tid; q0 < nq; q0 += kGroupLoads * kGroupThreads) {
        u32x4 v[kGroupLoads];
#pragma unroll
        for (int u = 0; u < kGroupLoads; ++u)
            v[u] = *reinterpret_cast<const u32x4*>(masks + 8 * (int64_t)min(q0 + u * kGroupThreads, nq - 1));
#pragma unroll
        for (int u = 0; u < kGroupLoads; ++u) {
            const int q = q0 + u * kGroupThreads;
            if (q >= nq) break;
            const int ch = q % nch;
            int c = 0;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {  // word pairs 8 ch + 2 w2, + 1
                const int valid = nwords - (8 * ch + 2 * w2);
                uint32_t x = v[u][w2];
                if (valid < 2) x &= valid >= 1 ? 0xFFFFu : 0u;
                c += __popc(x);
            }
            if (c) atomicAdd(&part[q / nch], c);
        }
    }
    __syncthreads();
    // 2. one wave: counts, offsets and the tile bases of every spec (two experts per lane)
    if (tid < kWave) {
        int c2[2], t2[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ee = 2 * lane + h;
            const int c = ee < E ? part[ee] : 0;
            c2[h] = c;
#pragma unroll
            for (int si = 0; si < 2; ++si) {
                int nt = 0;
                if (si < specs.n && ee < E) {
                    const TileSpec& ts = specs.t[si];
                    nt = ((c + ts.mt - 1) / ts.mt) * (ts.n_routed / ts.nt);
                }
                t2[si][h] = nt;
            }
        }
        const int ci = wave_incl_scan(c2[0] + c2[1]);
        int ex = ci - (c2[0] + c2[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ee = 2 * lane + h;
            if (ee < E) { cnt[ee] = c2[h]; off[ee] = ex; }
            ex += c2[h];
        }
        if (lane == kWave - 1) total_rows = ci;
#pragma unroll
        for (int si = 0; si < 2; ++si) {
            const int ti = wave_incl_scan(t2[si][0] + t2[si][1]);
            int tx = ti - (t2[si][0] + t2[si][1]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ee = 2 * lane + h;
                if (ee < E) tbase[si][ee] = tx;
                tx += t2[si][h];
            }
            if (lane == kWave - 1) total_tiles[si] = ti;
        }
    }
    __syncthreads();
    // 3. block 0: counts / offsets, the shared expert's tiles, the tile counts
    if (e == 0) {
        for (int ee = tid; ee < E; ee += blockDim.x) {
            counts[ee] = cnt[ee];
            offsets[ee] = off[ee];
        }
        if (tid == 0) offsets[E] = total_rows;
        for (int si = 0; si < specs.n; ++si) {
            const TileSpec& ts = specs.t[si];
            int count_s = 0;
            if (ts.n_shared > 0) {
                const int nNs = ts.n_shared / ts.nt;
                const int nmts = (int)((T + ts.mt - 1) / ts.mt);
                count_s = nNs * nmts;
                for (int q = tid; q < count_s; q += blockDim.x) {
                    const int n = q / nmts, m = q % nmts;
                    int64_t rows = T - (int64_t)m * ts.mt;
                    if (rows > ts.mt) rows = ts.mt;
                    if (total_tiles[si] + q < ts.max_items)
                        ts.items[total_tiles[si] + q] = make_int4(E, n * ts.nt, m * ts.mt, (int)rows);
                }
            }
            if (tid == 0) *ts.count = min(total_tiles[si] + count_s, ts.max_items);
        }
    }
    if (tid >= kWave) return;
    // 4. this expert's tiles (lanes over tiles) and rows (lanes over words)
    const int ce = cnt[e], oe = off[e];
    for (int si = 0; si < specs.n; ++si) {
        const TileSpec& ts = specs.t[si];
        const int nmt = (ce + ts.mt - 1) / ts.mt;
        for (int q = lane; q < nmt * (ts.n_routed / ts.nt); q += kWave) {
            const int n = q / nmt, m = q % nmt;
            int rows = ce - m * ts.mt;
            if (rows > ts.mt) rows = ts.mt;
            const int at = tbase[si][e] + q;
            if (at < ts.max_items) ts.items[at] = make_int4(e, n * ts.nt, oe + m * ts.mt, rows);
        }
    }
    const uint16_t* mrow = masks + (int64_t)e * mstride;
    const uint64_t* jrow = jmask ? jmask + (int64_t)e * mstride : nullptr;
    int base = oe;  // grouped row of the next group of words
    for (int w0 = 0; w0 < nwords; w0 += 4 * kWave) {
        // lane takes words w0 + 4 lane .. + 3
        uint32_t bits[4];
        uint64_t js[4];
        int mine = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int wd = min(w0 + 4 * lane + q, nwords - 1);
            const bool ok = w0 + 4 * lane + q < nwords;
            const uint32_t mw = (uint32_t)mrow[wd];
            bits[q] = ok ? mw : 0u;
            js[q] = jrow ? jrow[wd] : 0ull;
            mine += __popc(bits[q]);
        }
        const int incl = wave_incl_scan(mine);
        int rank = base + incl - mine;
        base += __builtin_amdgcn_readlane(incl, kWave - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t bb = bits[q];
            while (bb) {
                const int b = __ffs(bb) - 1;
                bb &= bb - 1;
                const int64_t t = (int64_t)(w0 + 4 * lane + q) * 16 + b;
                int j = 0;
                if (jrow) {
                    j = (int)((js[q] >> (4 * b)) & 15u);
                } else {
                    for (int jj = 0; jj < k; ++jj)
                        if (idx[t * k + jj] == e) j = jj;
                }
                const int dst = rank++;
                row_token[dst] = (int32_t)t;
                row_of[t * k + j] = dst;
                if (row_pair) row_pair[dst] = (int32_t)(t * k + j);
            }
        }
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
int mask_stride(int64_t T) { return (mask_words(T) + 7) & ~7; }  // 16-byte rows

int64_t tile_max_items(int64_t pairs, int E, int64_t T, int mt, int nt, int n_routed, int n_shared) {
    const int64_t routed = (pairs / mt + E) * (int64_t)(n_routed / nt);
    const int64_t shared = n_shared > 0 ? ((T + mt - 1) / mt) * (int64_t)(n_shared / nt) : 0;
    return routed + shared;
}

hipError_t launch_masks(const int32_t* idx, int64_t T, int k, int E, uint16_t* masks, uint64_t* jmask,
                        hipStream_t st) {
    perm_mask_kernel<<<(unsigned)mask_words(T), 256, 0, st>>>(idx, T, k, E, masks, k <= 16 ? jmask : nullptr,
                                                              mask_stride(T));
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, const uint16_t* masks, const uint64_t* jmask,
                          int32_t* prefix, int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_of,
                          int32_t* row_pair, const TileSpec* t1, const TileSpec* t2, hipStream_t st) {
    const int64_t N = T * k;
    if (E <= kGroupMaxE) {
        group_experts_kernel<<<(unsigned)E, kGroupThreads, 0, st>>>(idx, T, k, E, masks, mask_words(T),
                                                                    mask_stride(T), counts, offsets, row_token,
                                                                    row_of, k <= 16 ? jmask : nullptr, row_pair,
                                                                    make_specs(t1, t2));
        return hipGetLastError();
    }
    perm_prefix_kernel<<<1, 1024, 0, st>>>(masks, mask_words(T), mask_stride(T), E, T, prefix, counts, offsets,
                                            make_specs(t1, t2));
    perm_scatter_kernel<<<(unsigned)((N + 255) / 256), 256, 0, st>>>(idx, N, k, E, masks, mask_stride(T), prefix,
                                                                     offsets, row_token, row_of, row_pair);
    return hipGetLastError();
}

hipError_t launch_build_items(const int32_t* offsets, int E, int64_t T, const TileSpec* t1, const TileSpec* t2,
                              hipStream_t st) {
    build_items_kernel<<<1, 1024, 0, st>>>(offsets, E, T, make_specs(t1, t2));
    return hipGetLastError();
}

}  // namespace tmoe
