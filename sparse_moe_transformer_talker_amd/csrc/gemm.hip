// Grouped SwiGLU matrix products of the routed experts and the shared expert
// ("3C · Talker MoE (20 lớp, 128 Experts Top-6)", openarchlab, §1: each expert
// is a SwiGLU 1024 -> 384 -> 1024, the shared one 1024 -> 768 -> 1024; the
// SwiGLU form down(SiLU(gate x) * up x) is from "用 print(model) 认识 Qwen3-TTS",
// horus-space, MLP section).
//
// pass 0 (gate/up):  h[r, n] = SiLU(x_r . gate[e, n]) * (x_r . up[e, n])
// pass 1 (down):     y[dst(r), n] = h_r . down[e, n]   (the combine applies the routing weights)
//
// Work arrives as a device-built list of tiles (expert, n0, m0, rows); the
// launch is sized for the worst case and surplus workgroups exit at once.
// Consecutive tiles share a weight block; workgroup p runs on XCD p % 8, so the
// logical order is dealt out in 8 contiguous runs, one per XCD, which keeps
// tiles that reuse a weight block in the same L2.
//
// bf16 x bf16 -> fp32 on the matrix cores (v_mfma_f32_16x16x32_bf16); A and B
// tiles are staged through LDS (rows padded by 16 bytes against bank
// conflicts) with a register prefetch of the next K block.
#include "common.hpp"
#include "kernels.hpp"
#include "skinny.hpp"

#include <hip/hip_ext.h>

namespace tmoe {

// direct tiling: at most this many tokens (16-token router blocks)
constexpr int kDirectMaxT = 256;
constexpr int kDirectMaxBlocks = kDirectMaxT / 16;

// Item of workgroup p in a device-built tile list, or -1.  Workgroup p runs on
// XCD p % 8; each XCD takes a contiguous run of the routed items (tiles that
// share a weight block or token rows are adjacent) and an equal share of the
// shared-expert items, before or after its routed run.  The grid has at least
// 8 (ceil(n / 8) + 1) workgroups for a list of n items.
__device__ __forceinline__ int list_item(const GemmArgs& args, int p) {
    const int n = *args.count;
    const int ns = min(args.n_shared_items, n), nr = n - ns;
    const int cr = (nr + 7) >> 3, cs = (ns + 7) >> 3;
    const int slot = p >> 3, x = p & 7;
    const int first = args.shared_first ? cs : cr;  // slots of the kind taken first
    if (slot < first) {
        const int i = x * first + slot;
        if (args.shared_first) return i < ns ? nr + i : -1;
        return i < nr ? i : -1;
    }
    const int second = args.shared_first ? cr : cs;
    const int i = x * second + (slot - first);
    if (slot - first >= second) return -1;
    if (args.shared_first) return i < nr ? i : -1;
    return i < ns ? nr + i : -1;
}

template <int PASS, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(256, PASS == 1 ? 6 : 1) void grouped_gemm_kernel(GemmArgs args) {
    constexpr int BROWS = (PASS == 0) ? 2 * BN : BN;
    constexpr int LDK = BK + 8;
    constexpr int KC = BK / 8;                 // 16-byte chunks per tile row
    constexpr int NA = BM * KC, NB = BROWS * KC;
    constexpr int CA = (NA + 255) / 256, CB = (NB + 255) / 256;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MS = TM / 16, NS = TN / 16;
    static_assert(WM * WN == 4, "four waves");
    static_assert(TM % 16 == 0 && TN % 16 == 0 && BK % 32 == 0, "tile shape");
    static_assert(NB % 256 == 0, "B tile loads cover the block");

    __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[BROWS * LDK];
    const int tid = threadIdx.x;

    // Global sources of this thread's A and B chunks (fixed over K), and the
    // register copy of the next K block.  A tile is run in phases so that its
    // weight loads can be issued before its token rows are known.  Weight
    // chunk i of a thread is tile row tid / KC + RPI i, so its address is a
    // block base (uniform: gate or up rows of the tile) plus one per-thread
    // 32-bit offset.
    constexpr int RPI = 256 / KC;  // tile rows per chunk index
    static_assert(256 % KC == 0 && BN % RPI == 0, "weight chunks map to rows");
    const bf16_t* pa[CA];
    const bf16_t* bbase[2];
    int bK = 0;
    uint32_t blane = 0;
    u32x4 ra[CA], rb[CB];
    // weight rows n0 .. n0 + BN - 1 of expert e (gate rows, then up rows)
    auto set_b = [&](const GemmGroup& g, const int e, const int n0) {
        bK = g.K;
        bbase[0] = (const bf16_t*)g.wa + (int64_t)e * g.w_estride + (int64_t)n0 * g.K;
        bbase[1] = PASS == 0 ? (const bf16_t*)g.wb + (int64_t)e * g.w_estride + (int64_t)n0 * g.K : bbase[0];
        blane = (uint32_t)((tid / KC) * g.K + (tid % KC) * 8) * (uint32_t)sizeof(bf16_t);  // bytes
    };
    // tile row r < mrows reads A row amap[r] / a_div (amap not null), else
    // a_rows[m0 + r] / a_div (a_rows not null), else m0 + r; rows past mrows
    // repeat row 0 and are never stored
    auto set_a = [&](const GemmGroup& g, const int m0, const int mrows, const int* amap) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + 256 * i < NA ? tid + 256 * i : 0;
            const int row = c / KC, kc = c % KC;
            const int m = row < mrows ? row : 0;
            const int64_t grow = amap ? (int64_t)(amap[m] / g.a_div)
                                      : (g.a_rows ? (int64_t)(g.a_rows[m0 + m] / g.a_div) : (int64_t)(m0 + m));
            pa[i] = (const bf16_t*)g.a + grow * g.a_ld + kc * 8;
        }
    };
    auto load_a = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + k0);
    };
    auto load_b = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int sel = (PASS == 0 && i * RPI >= BN) ? 1 : 0;
            const char* b = reinterpret_cast<const char*>(bbase[sel] + (int64_t)((i * RPI) % BN) * bK + k0);
            rb[i] = *reinterpret_cast<const u32x4*>(b + blane);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            int c = tid + 256 * i;
            if (c < NA) *reinterpret_cast<u32x4*>(&As[(c / KC) * LDK + (c % KC) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            int c = tid + 256 * i;
            *reinterpret_cast<u32x4*>(&Bs[(c / KC) * LDK + (c % KC) * 8]) = rb[i];
        }
    };

    // The K loop and epilogue of one tile whose first K block is in flight:
    // output rows m0 .. m0 + mrows - 1 of group g (omap, nullable, replaces the
    // group's output row map, indexed by the row within the tile).
    auto run = [&](const GemmGroup& g, const int n0, const int m0, const int mrows, const int* omap) {
        const int K = g.K;
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / WN, wn = wave % WN;
        const int li = lane & 15, lk = (lane >> 4) * 8;

        f32x4 acc[MS][NS], accu[MS][NS];
#pragma unroll
        for (int a = 0; a < MS; ++a)
#pragma unroll
            for (int b = 0; b < NS; ++b) { acc[a][b] = f32x4{0, 0, 0, 0}; accu[a][b] = f32x4{0, 0, 0, 0}; }

        for (int k0 = 0; k0 < K; k0 += BK) {
            __syncthreads();  // (also: the previous tile's last LDS reads are done)
            stash();
            __syncthreads();
            if (k0 + BK < K) {
                load_b(k0 + BK);
                load_a(k0 + BK);
            }
#pragma unroll
            for (int ks = 0; ks < BK; ks += 32) {
                bf16x8 af[MS], bg[NS], bu[NS];
#pragma unroll
                for (int a = 0; a < MS; ++a)
                    af[a] = *reinterpret_cast<const bf16x8*>(&As[(wm * TM + a * 16 + li) * LDK + ks + lk]);
#pragma unroll
                for (int b = 0; b < NS; ++b) {
                    bg[b] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * TN + b * 16 + li) * LDK + ks + lk]);
                    if (PASS == 0)
                        bu[b] = *reinterpret_cast<const bf16x8*>(&Bs[(BN + wn * TN + b * 16 + li) * LDK + ks + lk]);
                }
#pragma unroll
                for (int a = 0; a < MS; ++a)
#pragma unroll
                    for (int b = 0; b < NS; ++b) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bg[b], acc[a][b], 0, 0, 0);
                        if (PASS == 0)
                            accu[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bu[b], accu[a][b], 0, 0, 0);
                    }
            }
        }

        // Epilogue: lane holds D[4*(lane/16) + r][lane % 16] of every 16x16 block.
        bf16_t* out = (bf16_t*)g.out;
#pragma unroll
        for (int a = 0; a < MS; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * TM + a * 16 + (lane >> 4) * 4 + r;
                if (row >= mrows) continue;
                const int64_t src = (int64_t)m0 + row;
                const int64_t v = omap ? (int64_t)omap[row] : (g.out_rows ? (int64_t)g.out_rows[src] : src);
                const int64_t dst = v * g.out_mul + g.out_add + (g.out_div > 0 ? v / g.out_div : 0);
#pragma unroll
                for (int b = 0; b < NS; ++b) {
                    const int col = n0 + wn * TN + b * 16 + li;
                    const float val = PASS == 0 ? silu(acc[a][b][r]) * accu[a][b][r] : acc[a][b][r];
                    out[dst * g.out_ld + col] = f32_to_bf16(val);
                }
            }
    };

    const int p = blockIdx.x;
    if (args.direct_bcnt) {
        // Workgroup p runs on XCD p % 8.  Each XCD takes a contiguous run of the
        // routed tiles first and then an equal share of the shared-expert tiles,
        // whose weights are re-read from L2 by their M-tiles, so the tiles
        // dispatched last on every XCD are the cheap ones.
        const int nt0 = args.direct_nt[0];
        const int n_routed = args.E * nt0;
        const int n_shared = args.direct_nt[1] * args.direct_mt1;
        const int n_all = n_routed + n_shared;
        const int cr = (n_routed + 7) >> 3, cs = (n_shared + 7) >> 3;
        const int slot = p >> 3, x = p & 7;
        int q;
        if (slot < cr) q = x * cr + slot < n_routed ? x * cr + slot : n_all;
        else q = x * cs + (slot - cr) < n_shared ? n_routed + x * cs + (slot - cr) : n_all;
        if (q >= n_all) return;
        if (q < n_routed) {
            const GemmGroup& g = args.g[0];
            const int e = q / nt0, n0 = (q % nt0) * BN;
            const int T = args.direct_T, base = e * T;
            // In the down pass neither operand depends on the routing (the A
            // rows of expert e are rows base .. base + T - 1 in order; rows the
            // expert does not use are loaded and never stored), so the first K
            // block goes out before the pair lists.  In the gate/up pass the
            // lists come first: weight loads issued ahead of them by every
            // workgroup would queue the lists (and then the token rows) behind
            // a whole round of weight traffic.
            if (PASS == 1) {
                set_b(g, e, n0);
                load_b(0);
                set_a(g, base, min(BM, T), nullptr);
                load_a(0);
            }
            // This expert's pairs: the per-block lists concatenated in block
            // order.  Counts and list entries are fetched together (entries
            // past a block's count are read and dropped).
            __shared__ int rl[kDirectMaxT];
            __shared__ int boff[kDirectMaxBlocks + 1], bc[kDirectMaxBlocks];
            const int nb = args.direct_nb;
            const int lv = tid < nb * 16 ? args.direct_blist[((int64_t)(tid >> 4) * args.E + e) * 16 + (tid & 15)] : 0;
            if (tid < kWave) {
                const int c = tid < nb ? args.direct_bcnt[tid * args.E + e] : 0;
                const int incl = wave_incl_scan(c);
                if (tid < nb) { boff[tid] = incl - c; bc[tid] = c; }
                if (tid == kWave - 1) boff[kDirectMaxBlocks] = incl;
            }
            __syncthreads();
            if (tid < nb * 16 && (tid & 15) < bc[tid >> 4]) rl[boff[tid >> 4] + (tid & 15)] = lv;
            __syncthreads();
            const int m = boff[kDirectMaxBlocks];
            if (n0 == 0 && tid == 0 && args.direct_counts) args.direct_counts[e] = m;
            if (m == 0) {
                if (PASS == 1) __builtin_amdgcn_s_waitcnt(0);  // nothing to compute: drain the early loads
                return;
            }
            for (int m0 = 0; m0 < m; m0 += BM) {
                const int mr = min(BM, m - m0);
                if (PASS == 1 && m0 > 0) {
                    load_b(0);
                    set_a(g, base + m0, mr, nullptr);
                    load_a(0);
                }
                if (PASS == 0) {
                    if (m0 == 0) set_b(g, e, n0);
                    set_a(g, 0, mr, rl + m0);
                    load_b(0);
                    load_a(0);
                }
                run(g, n0, base + m0, mr, PASS == 1 ? rl + m0 : nullptr);
            }
        } else {
            q -= n_routed;
            const GemmGroup& g = args.g[1];
            const int n0 = (q / args.direct_mt1) * BN, m0 = (q % args.direct_mt1) * BM;
            const int mr = min(BM, args.direct_T - m0);
            set_b(g, 0, n0);
            set_a(g, m0, mr, nullptr);
            load_b(0);
            load_a(0);
            run(g, n0, m0, mr, nullptr);
        }
        return;
    }
    const int q = list_item(args, p);
    if (q < 0) return;
    const int4 it = args.items[q];
    const int gi = it.x < args.E ? 0 : 1;
    const GemmGroup& g = args.g[gi];
    set_b(g, gi == 0 ? it.x : 0, it.y);
    set_a(g, it.z, it.w, nullptr);
    load_b(0);
    load_a(0);
    run(g, it.y, it.z, it.w, nullptr);
}

// ---------------------------------------------------------------------------
// Many rows per expert: BM x 256 tiles, BM = 128 or 256 (gate/up: 128 gate +
// 128 up columns; down: 256 output columns) on v_mfma_f32_32x32x16_bf16, four
// waves of (BM / 2) x 128.
// K advances in stages of 32; every stage is copied global -> LDS by the
// direct-to-LDS loads (no VGPR staging) into a ring of 4 buffers with 3 stages
// in flight, waited for with vmcnt and a raw s_barrier.  In LDS a tile row is
// 64 bytes (four 16-byte chunks); chunk c of row r is stored at position
// (c + r / 4) % 4, which spreads the 32 rows one fragment read touches over
// all banks.  The rotation is realised by choosing which global chunk each
// lane fetches, since lane i of a direct-to-LDS load writes bytes
// [16 i, 16 i + 16) of its 1 KB destination.
namespace lds_gemm {
constexpr int BNR = 256, BK = 32;
constexpr int NSTAGE = 4, INFLIGHT = NSTAGE - 1;
// Eight waves, two per SIMD (so one wave's matrix work covers the other's LDS
// reads and waits), as 4 token rows x 2 feature halves of 128.
constexpr int NWAVE = 8;
constexpr int B_BYTES = BNR * BK * 2;
constexpr int B_CALLS = B_BYTES / 1024 / NWAVE;  // per wave, per stage
template <int BM> struct Tile {
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_CALLS = A_BYTES / 1024 / NWAVE;
    static constexpr int CALLS = A_CALLS + B_CALLS;
    static constexpr int WROWS = BM / (NWAVE / 2);  // token rows per wave
    static constexpr int MI = WROWS / 32;           // 32-row blocks per wave
};
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int lds_chunk(int row, int c) { return (c + (row >> 2)) & 3; }

template <int N>
__device__ __forceinline__ void wait_vm() {
    // vmcnt <= N (N < 64) and lgkmcnt == 0: this wave's loads of stage s have
    // landed and its own LDS reads of earlier stages are done, so after the
    // barrier that follows no wave still reads the buffer about to be refilled
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
}  // namespace lds_gemm

template <int PASS, int BM>
__global__ __launch_bounds__(64 * lds_gemm::NWAVE) void grouped_gemm_lds_kernel(GemmArgs args) {
    using namespace lds_gemm;
    constexpr int A_BYTES = Tile<BM>::A_BYTES, STAGE = Tile<BM>::STAGE, A_CALLS = Tile<BM>::A_CALLS;
    constexpr int CALLS = Tile<BM>::CALLS, MI = Tile<BM>::MI;
    // one array per ring stage, so the compiler can tell which direct-to-LDS
    // load writes which buffer and waits only for the right one
    __shared__ __attribute__((aligned(1024))) char buf0[STAGE];
    __shared__ __attribute__((aligned(1024))) char buf1[STAGE];
    __shared__ __attribute__((aligned(1024))) char buf2[STAGE];
    __shared__ __attribute__((aligned(1024))) char buf3[STAGE];

    const int q = list_item(args, blockIdx.x);
    if (q < 0) return;
    const int4 it = args.items[q];
    const int gi = it.x < args.E ? 0 : 1;
    const GemmGroup& g = args.g[gi];
    const int e = gi == 0 ? it.x : 0;
    const int n0 = it.y, m0 = it.z, mrows = it.w;
    const int K = g.K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // Global sources of this lane's direct-to-LDS chunks (fixed over K).
    const bf16_t* pa[A_CALLS];
    const bf16_t* pb[B_CALLS];
#pragma unroll
    for (int j = 0; j < A_CALLS; ++j) {
        const int r = (wave * A_CALLS + j) * 16 + (lane >> 2);
        const int c = ((lane & 3) - (r >> 2)) & 3;  // global chunk landing at position lane & 3
        const int m = r < mrows ? r : 0;
        const int64_t grow = g.a_rows ? (int64_t)(g.a_rows[m0 + m] / g.a_div) : (int64_t)(m0 + m);
        pa[j] = (const bf16_t*)g.a + grow * g.a_ld + c * 8;
    }
#pragma unroll
    for (int j = 0; j < B_CALLS; ++j) {
        const int r = (wave * B_CALLS + j) * 16 + (lane >> 2);
        const int c = ((lane & 3) - (r >> 2)) & 3;
        const bf16_t* w;
        int wrow;
        if (PASS == 0) {
            w = (const bf16_t*)(r < BNR / 2 ? g.wa : g.wb);
            wrow = n0 + (r & (BNR / 2 - 1));
        } else {
            w = (const bf16_t*)g.wa;
            wrow = n0 + r;
        }
        pb[j] = w + (int64_t)e * g.w_estride + (int64_t)wrow * K + c * 8;
    }
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue = [&](int stage, char* base) {
        const int k0 = stage * BK;
#pragma unroll
        for (int j = 0; j < A_CALLS; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(pa[j] + k0),
                                             (lds_void*)(base + (wave * A_CALLS + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < B_CALLS; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(pb[j] + k0),
                                             (lds_void*)(base + A_BYTES + (wave * B_CALLS + j) * 1024), 16, 0, 0);
    };

    const int wm = __builtin_amdgcn_readfirstlane(wave >> 1), wn = wave & 1;
    const int lr = lane & 31, lh = lane >> 5;
    // Token block a of wave row wm is 32-row block a * 4 + wm of the tile, so the
    // blocks past the expert's last row fall on different waves; the waves of
    // a SIMD (w and w + 4) then keep equal shares of the live blocks and skip
    // the rest (a wave-uniform test).
    bool live[MI];
#pragma unroll
    for (int a = 0; a < MI; ++a) live[a] = (a * (NWAVE / 2) + wm) * 32 < mrows;
    f32x16 acc[MI][4];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
    // B-tile row of fragment column block b (32 columns)
    auto brow0 = [&](int b) {
        if (PASS == 0) return (b < 2 ? 0 : BNR / 2) + wn * 64 + (b & 1) * 32;
        return wn * 128 + b * 32;
    };
    auto compute = [&](const char* base) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = 2 * ks + lh;
            bf16x8 af[MI], bfr[4];
#pragma unroll
            for (int a = 0; a < MI; ++a) {
                const int r = (a * (NWAVE / 2) + wm) * 32 + lr;
                if (live[a]) af[a] = *reinterpret_cast<const bf16x8*>(base + r * 64 + lds_chunk(r, c) * 16);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int r = brow0(b) + lr;
                bfr[b] = *reinterpret_cast<const bf16x8*>(base + A_BYTES + r * 64 + lds_chunk(r, c) * 16);
            }
#pragma unroll
            for (int a = 0; a < MI; ++a)
                if (live[a])
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b], af[a], acc[a][b], 0, 0, 0);
        }
    };
    // stage s: wait until its loads (all waves') have landed, refill the buffer
    // freed by stage s - 1 with stage s + 3, compute stage s
    // Every branch below is resolved at compile time, so the wait counts are
    // the only synchronisation on the ring and the compiler adds none of its own.
    const int nst = K / BK;  // a multiple of 4, at least 4
    auto sync = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // keep each refill ahead of the stage's matrix work
    auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };
    issue(0, buf0);
    issue(1, buf1);
    issue(2, buf2);
    // The output row map is read behind the first stages and used only after
    // the last wait, so no wait of the prologue waits on it (nothing else
    // writes the register the load fills).
    const bool mapped = g.out_rows != nullptr;
    int32_t map_v = 0;
    if (mapped && tid < BM) map_v = g.out_rows[m0 + (tid < mrows ? tid : 0)];
    // steady state: stage s waits for itself with two newer stages in flight,
    // then refills the buffer stage s - 1 used with stage s + 3
    for (int s = 0; s + 4 < nst; s += 4) {
        wait_vm<2 * CALLS>(); sync(); issue(s + 3, buf3); fence(); compute(buf0);
        wait_vm<2 * CALLS>(); sync(); issue(s + 4, buf0); fence(); compute(buf1);
        wait_vm<2 * CALLS>(); sync(); issue(s + 5, buf1); fence(); compute(buf2);
        wait_vm<2 * CALLS>(); sync(); issue(s + 6, buf2); fence(); compute(buf3);
    }
    // last four stages: nst - 4 .. nst - 1 in buf0 .. buf3
    wait_vm<2 * CALLS>(); sync(); issue(nst - 1, buf3); fence(); compute(buf0);
    wait_vm<2 * CALLS>(); sync(); compute(buf1);
    wait_vm<CALLS>(); sync(); compute(buf2);
    wait_vm<0>(); sync(); compute(buf3);

    // Epilogue.  The weight tile is the MFMA's first operand, so block (a, b)
    // holds output features x tokens: lane l, entry i has feature
    // 8 * (i / 4) + 4 * (l / 32) + i % 4 of the block's 32 and token l % 32,
    // i.e. four consecutive features of one token per group of four entries.
    // They are rounded to bf16 and placed in the idle ring as a row-major
    // tile (16-byte chunks swizzled by row against bank conflicts); then whole
    // output rows are written, 16 bytes per lane (stores straight from the
    // fragment layout would touch 32 rows per instruction).
    constexpr int NOUT = PASS == 0 ? BNR / 2 : BNR;  // output columns of the tile
    constexpr int ROWB = NOUT * 2;                    // bytes per output row
    constexpr int CPR = ROWB / 16;                    // 16-byte chunks per row
    constexpr int RPB = STAGE / ROWB;                 // rows per ring buffer
    static_assert(4 * RPB >= BM, "the output tile fits in the ring");
    auto row_at = [&](int r) -> char* {
        const int bsel = r / RPB;
        char* base = bsel == 0 ? buf0 : (bsel == 1 ? buf1 : (bsel == 2 ? buf2 : buf3));
        return base + (r % RPB) * ROWB;
    };
    // destination row of every tile row, for the row stores below
    __shared__ int32_t dst_rows[BM];
    if (tid < BM) {
        const int32_t v = mapped ? map_v : m0 + tid;
        dst_rows[tid] = tid < mrows ? v * g.out_mul + g.out_add + (g.out_div > 0 ? v / g.out_div : 0) : -1;
    }
    sync();  // every wave is done with the ring
#pragma unroll
    for (int a = 0; a < MI; ++a) {
        const int r = (a * (NWAVE / 2) + wm) * 32 + lr;
        char* rp = row_at(r);
#pragma unroll
        for (int b = 0; b < (PASS == 0 ? 2 : 4); ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[q] = PASS == 0 ? silu(acc[a][b][4 * j + q]) * acc[a][b + 2][4 * j + q] : acc[a][b][4 * j + q];
                }
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                const int c = ((PASS == 0 ? wn * 64 : wn * 128) + b * 32 + 8 * j) / 8;  // 16-byte chunk
                *reinterpret_cast<uint2*>(rp + ((c ^ (r % CPR)) * 16) + lh * 8) = pk;
            }
        __builtin_amdgcn_sched_barrier(0);  // one token block at a time: bounds the live accumulator copies
    }
    sync();
    bf16_t* out = (bf16_t*)g.out;
    for (int q = tid; q < BM * CPR; q += 64 * NWAVE) {
        const int r = q / CPR, c = q % CPR;
        if (r >= mrows) break;  // rows ascend with q
        const u32x4 v = *reinterpret_cast<const u32x4*>(row_at(r) + ((c ^ (r % CPR)) * 16));
        *reinterpret_cast<u32x4*>(out + (int64_t)dst_rows[r] * g.out_ld + n0 + c * 8) = v;
    }
}

// ---------------------------------------------------------------------------
// Portable path (fp32 and shapes the matrix-core tiles do not cover): one
// thread per output element, fp32 accumulation.
template <typename T, int PASS>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmGroup g, const int32_t* __restrict__ offsets, int E,
                                                           int64_t rows) {
    const int64_t r = blockIdx.x;
    const int n = blockIdx.y * blockDim.x + threadIdx.x;
    if (r >= rows || n >= g.N) return;
    int e = 0;
    if (offsets) {  // expert of grouped row r: last e with offsets[e] <= r
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
        }
        e = lo;
    }
    const int64_t arow = g.a_rows ? (int64_t)g.a_rows[r] : r;
    const T* a = (const T*)g.a + arow * g.a_ld;
    const T* wa = (const T*)g.wa + (int64_t)e * g.w_estride + (int64_t)n * g.K;
    float s0 = 0.f, s1 = 0.f;
    if (PASS == 0) {
        const T* wb = (const T*)g.wb + (int64_t)e * g.w_estride + (int64_t)n * g.K;
        for (int kk = 0; kk < g.K; ++kk) {
            float av = Elem<T>::load(a, kk);
            s0 = fmaf(av, Elem<T>::load(wa, kk), s0);
            s1 = fmaf(av, Elem<T>::load(wb, kk), s1);
        }
        s0 = silu(s0) * s1;
    } else {
        for (int kk = 0; kk < g.K; ++kk) s0 = fmaf(Elem<T>::load(a, kk), Elem<T>::load(wa, kk), s0);
    }
    const int64_t v = g.out_rows ? (int64_t)g.out_rows[r] : r;
    const int64_t dst = v * g.out_mul + g.out_add + (g.out_div > 0 ? v / g.out_div : 0);
    Elem<T>::store((T*)g.out, dst * g.out_ld + n, s0);
}

// ---------------------------------------------------------------------------
// Tilings: small-M (few rows per expert: weight streaming) and large-M.
//                         BM   BN   BK  WM WN
constexpr int kSmallBM = 16, kSmallBN0 = 64, kSmallBN1 = 64;
#define TMOE_SMALL_GU 0, kSmallBM, kSmallBN0, 128, 1, 4
#define TMOE_SMALL_DN 1, kSmallBM, kSmallBN1, 128, 1, 4
#define TMOE_SMALL_DN64 1, kSmallBM, kSmallBN1, 64, 1, 4  // reductions of 64 * odd length
#define TMOE_LARGE_GU 0,  128,  64,  64, 2, 2
#define TMOE_LARGE_DN 1,  128, 128,  64, 2, 2

void gemm_tiles(int variant, int pass, int* mt, int* nt) {
    if (variant == kGemmSmallM) { *mt = kSmallBM; *nt = pass == 0 ? kSmallBN0 : kSmallBN1; }
    else if (variant == kGemmLargeLds) { *mt = 128; *nt = pass == 0 ? lds_gemm::BNR / 2 : lds_gemm::BNR; }
    else if (variant == kGemmHugeLds) { *mt = 256; *nt = pass == 0 ? lds_gemm::BNR / 2 : lds_gemm::BNR; }
    else { *mt = 128; *nt = pass == 0 ? 64 : 128; }
}

bool gemm_lds_ok(int H, int I, int Is) {
    // K stages of 32 in groups of 4 (K % 128) and whole 128 x 256 tiles
    return H % 256 == 0 && I % 128 == 0 && Is % 128 == 0;
}

bool gemm_mfma_ok(int dtype, int H, int I, int Is) {
    return dtype == kBF16 && H % 128 == 0 && I % 64 == 0 && Is % 64 == 0;
}

namespace {
// reduction lengths of both groups are multiples of m (absent groups pass)
bool k_multiple(const GemmArgs& a, int m) {
    return a.g[0].K % m == 0 && (a.g[1].N == 0 || a.g[1].K % m == 0);
}

// With events, the launch itself timestamps the kernel's start and end.
template <typename Kernel>
hipError_t launch_gemm(Kernel kernel, unsigned grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                       const GemmArgs& args, unsigned block = 256) {
    if (!e0 && !e1) {
        kernel<<<grid, block, 0, st>>>(args);
        return hipGetLastError();
    }
    GemmArgs copy = args;
    void* argv[] = {&copy};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), argv, 0, st, e0, e1, 0);
}
}  // namespace

hipError_t launch_grouped_gemm(int dtype, int variant, int pass, const GemmArgs& args, int64_t max_items,
                               hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)dtype;
    if (max_items <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(((max_items + 7) / 8 + 1) * 8);  // one more slot per XCD: see list_item
    if (variant == kGemmSmallM) {
        if (pass == 0) return launch_gemm(grouped_gemm_kernel<TMOE_SMALL_GU>, grid, st, ev_start, ev_stop, args);
        if (!k_multiple(args, 128))
            return launch_gemm(grouped_gemm_kernel<TMOE_SMALL_DN64>, grid, st, ev_start, ev_stop, args);
        return launch_gemm(grouped_gemm_kernel<TMOE_SMALL_DN>, grid, st, ev_start, ev_stop, args);
    }
    if (variant == kGemmLargeLds) {
        if (pass == 0) return launch_gemm(grouped_gemm_lds_kernel<0, 128>, grid, st, ev_start, ev_stop, args, 64 * lds_gemm::NWAVE);
        return launch_gemm(grouped_gemm_lds_kernel<1, 128>, grid, st, ev_start, ev_stop, args, 64 * lds_gemm::NWAVE);
    }
    if (variant == kGemmHugeLds) {
        if (pass == 0) return launch_gemm(grouped_gemm_lds_kernel<0, 256>, grid, st, ev_start, ev_stop, args, 64 * lds_gemm::NWAVE);
        return launch_gemm(grouped_gemm_lds_kernel<1, 256>, grid, st, ev_start, ev_stop, args, 64 * lds_gemm::NWAVE);
    }
    if (pass == 0) return launch_gemm(grouped_gemm_kernel<TMOE_LARGE_GU>, grid, st, ev_start, ev_stop, args);
    return launch_gemm(grouped_gemm_kernel<TMOE_LARGE_DN>, grid, st, ev_start, ev_stop, args);
}

int gemm_direct_tile(int pass, int* bm) {
    *bm = kSmallBM;
    return pass == 0 ? kSmallBN0 : kSmallBN1;
}

hipError_t launch_grouped_gemm_direct(int pass, const GemmArgs& args, hipStream_t st, hipEvent_t ev_start,
                                      hipEvent_t ev_stop) {
    const int64_t cr = ((int64_t)args.E * args.direct_nt[0] + 7) / 8;
    const int64_t cs = ((int64_t)args.direct_nt[1] * args.direct_mt1 + 7) / 8;
    const unsigned grid = (unsigned)(8 * (cr + cs));
    if (grid == 0) return hipSuccess;
    if (pass == 0) return launch_gemm(grouped_gemm_kernel<TMOE_SMALL_GU>, grid, st, ev_start, ev_stop, args);
    if (!k_multiple(args, 128))
        return launch_gemm(grouped_gemm_kernel<TMOE_SMALL_DN64>, grid, st, ev_start, ev_stop, args);
    return launch_gemm(grouped_gemm_kernel<TMOE_SMALL_DN>, grid, st, ev_start, ev_stop, args);
}

// ---------------------------------------------------------------------------
// Skinny products for M <= 64 rows (a decode batch), split over K:
// P[s] [M, N] = A [M, K_s] W_s^T in fp32, where K_s is the s-th of KS equal runs
// of K; the consumer adds the KS runs in run order (deterministic).  Two forms:
// - 16 columns per workgroup (below): one workgroup per (16 output columns,
//   run) reads its 16 x K_s weight block once; its four waves split the run
//   again, each covering all 64 rows as four 16-row matrix-core tiles
//   (v_mfma_f32_16x16x32_bf16, four 32-wide K steps with their loads in flight
//   together), and their partials are added in LDS in wave order;
// - 64 columns per workgroup with the run's token rows in LDS
//   (skinny_lds_kernel), where the shape gives enough runs of 256.
// SWIGLU: a workgroup's 16 columns are gate rows f .. f + 7 (of W) and up rows
// f .. f + 7 (of W2) for the 8 features f = 8 blockIdx.x ..; with the whole K in
// one run it stores h [M, N / 2] = SiLU(gate) * up in bf16 instead of partials.
namespace {
template <int NW, int U, bool SWIGLU>
__global__ __launch_bounds__(64 * NW) void skinny_gemm_kernel(const bf16_t* __restrict__ A,
                                                              const bf16_t* __restrict__ W,
                                                              const bf16_t* __restrict__ W2,
                                                              float* __restrict__ P, bf16_t* __restrict__ h, int M,
                                                              int N, int K, int KS) {
    skinny_body<NW, U, SWIGLU>(A, W, W2, P, h, M, N, K, KS, (int)blockIdx.x, (int)blockIdx.y);
}
}  // namespace

// Skinny products with the token rows in LDS.  A workgroup covers 64 output
// columns (one 16-column tile per wave) over one K run of KR: it reads the
// run's slice of all 64 token rows once into LDS and its waves read their
// 16 x KR weight blocks straight into matrix-core operand registers, every
// load of the run in flight at once.  Per workgroup the token bytes equal the
// weight bytes (the 16-column form reads 64 rows per 16 columns).
template <int KR>
__global__ __launch_bounds__(256) void skinny_lds_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                         float* __restrict__ P, int M, int N, int K) {
    constexpr int LDA = KR + 8;                // bf16 per LDS row (16-byte pad against bank conflicts)
    constexpr int CPR = KR / 8;                // 16-byte chunks per row of the slice
    constexpr int AC = kSkinnyRows * CPR / 256;
    constexpr int STEPS = KR / 32;
    static_assert(AC * 256 == kSkinnyRows * CPR, "the slice divides over the block");
    __shared__ __attribute__((aligned(16))) bf16_t As[kSkinnyRows * LDA];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kg = (lane >> 4) * 8;
    const int n0 = blockIdx.x * 64 + wave * 16;
    const int64_t k0 = (int64_t)blockIdx.y * KR;
    u32x4 b[STEPS];
    const bf16_t* wp = W + (int64_t)(n0 + r) * K + k0 + kg;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) b[s] = *reinterpret_cast<const u32x4*>(wp + 32 * s);
    u32x4 a[AC];
#pragma unroll
    for (int i = 0; i < AC; ++i) {  // rows past M repeat row M - 1 (computed, never stored)
        const int c = tid + 256 * i, row = c / CPR;
        a[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)min(row, M - 1) * K + k0 + (c % CPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int c = tid + 256 * i;
        *reinterpret_cast<u32x4*>(&As[(c / CPR) * LDA + (c % CPR) * 8]) = a[i];
    }
    __syncthreads();
    const f32x4 zero = {0, 0, 0, 0};
    f32x4 acc[4] = {zero, zero, zero, zero};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *reinterpret_cast<const bf16x8*>(&As[(mt * 16 + r) * LDA + 32 * s + kg]),
                __builtin_bit_cast(bf16x8, b[s]), acc[mt], 0, 0, 0);
    // D[row = 16 mt + 4 (lane / 16) + i][column n0 + lane % 16]
    float* out = P + (int64_t)blockIdx.y * M * N;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mt * 16 + 4 * (lane >> 4) + i;
            if (row < M) out[(int64_t)row * N + n0 + r] = acc[mt][i];
        }
}

// h [M, I] = SiLU(A Wg^T) * (A Wu^T) with all of K in one workgroup per 16
// features: the 64 token rows (K <= 1024) sit in LDS; eight waves take the
// gate or up tile over one K quarter each, and the quarters are added through
// LDS in quarter order.
template <int KQ>
__global__ __launch_bounds__(512) void skinny_swiglu_lds_kernel(const bf16_t* __restrict__ A,
                                                                const bf16_t* __restrict__ Wg,
                                                                const bf16_t* __restrict__ Wu, bf16_t* __restrict__ h,
                                                                int M, int I) {
    constexpr int K = 4 * KQ, LDA = K + 8, CPR = K / 8;
    constexpr int AC = kSkinnyRows * CPR / 512;
    constexpr int STEPS = KQ / 32;
    static_assert(AC * 512 == kSkinnyRows * CPR, "the rows divide over the block");
    static_assert(2 * 4 * kSkinnyRows * 16 * 4 <= kSkinnyRows * LDA * 2, "the quarter sums fit in the row buffer");
    __shared__ __attribute__((aligned(16))) bf16_t As[kSkinnyRows * LDA];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kg = (lane >> 4) * 8;
    const int tile = wave & 1, q = wave >> 1;  // tile 0: gate rows, 1: up rows
    const int f0 = blockIdx.x * 16;
    u32x4 b[STEPS];
    const bf16_t* wp = (tile ? Wu : Wg) + (int64_t)(f0 + r) * K + q * KQ + kg;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) b[s] = *reinterpret_cast<const u32x4*>(wp + 32 * s);
    u32x4 a[AC];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int c = tid + 512 * i, row = c / CPR;
        a[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)min(row, M - 1) * K + (c % CPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int c = tid + 512 * i;
        *reinterpret_cast<u32x4*>(&As[(c / CPR) * LDA + (c % CPR) * 8]) = a[i];
    }
    __syncthreads();
    const f32x4 zero = {0, 0, 0, 0};
    f32x4 acc[4] = {zero, zero, zero, zero};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *reinterpret_cast<const bf16x8*>(&As[(mt * 16 + r) * LDA + q * KQ + 32 * s + kg]),
                __builtin_bit_cast(bf16x8, b[s]), acc[mt], 0, 0, 0);
    __syncthreads();  // every wave is done with the token rows
    float* red = reinterpret_cast<float*>(As);  // [tile][quarter][64 rows][16 features]
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[((tile * 4 + q) * kSkinnyRows + mt * 16 + 4 * (lane >> 4) + i) * 16 + r] = acc[mt][i];
    __syncthreads();
    for (int idx = tid; idx < kSkinnyRows * 16; idx += 512) {
        const int row = idx >> 4, c = idx & 15;
        if (row >= M) continue;
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            g += red[(qq * kSkinnyRows + row) * 16 + c];
            u += red[((4 + qq) * kSkinnyRows + row) * 16 + c];
        }
        h[(int64_t)row * I + f0 + c] = f32_to_bf16(silu(g) * u);
    }
}

// Run length of the LDS form for a product (0: the 16-column form applies):
// runs of 256, when they give at least 128 workgroups.  Shorter runs and fewer
// workgroups measured slower than the 16-column form (more fp32 partials for
// the consumer to add, or too few CUs reading weights).
constexpr int kSkinnyRun = 256;
int skinny_lds_run(int64_t M, int N, int K) {
    if (M < 1 || M > kSkinnyRows || N < 64 || N % 64 || K % kSkinnyRun) return 0;
    return (int64_t)(N / 64) * (K / kSkinnyRun) >= 128 ? kSkinnyRun : 0;
}

int skinny_gemm_runs(int64_t M, int N, int K) {
    if (const int kr = skinny_lds_run(M, N, K)) return K / kr;
    if (M < 1 || M > kSkinnyRows || N < 16 || N % 16 || K % (32 * kSkinnyWaves)) return 0;
    // enough workgroups to fill the chip, each run at least 512 long
    int ks = 1;
    while (ks * 2 * 512 <= K && K % (ks * 2 * 32 * kSkinnyWaves) == 0 && (N / 16) * ks < 256) ks *= 2;
    return ks;
}

hipError_t launch_skinny_gemm(const void* A, const void* W, float* P, int64_t M, int N, int K, int KS,
                              hipStream_t st) {
    const int kr = skinny_lds_run(M, N, K);
    if (kr && KS == K / kr) {
        skinny_lds_kernel<kSkinnyRun><<<dim3((unsigned)(N / 64), (unsigned)KS), 256, 0, st>>>(
            (const bf16_t*)A, (const bf16_t*)W, P, (int)M, N, K);
        return hipGetLastError();
    }
    dim3 grid((unsigned)(N / 16), (unsigned)KS);
    skinny_gemm_kernel<kSkinnyWaves, 4, false><<<grid, 64 * kSkinnyWaves, 0, st>>>(
        (const bf16_t*)A, (const bf16_t*)W, nullptr, P, nullptr, (int)M, N, K, KS);
    return hipGetLastError();
}

bool skinny_swiglu_ok(int64_t M, int I, int K) {
    return M >= 1 && M <= kSkinnyRows && I >= 8 && I % 8 == 0 && K % (32 * kSkinnyWaves) == 0;
}

hipError_t launch_skinny_swiglu(const void* A, const void* Wg, const void* Wu, void* h, int64_t M, int I, int K,
                                hipStream_t st) {
    if (K == 1024 && I % 16 == 0) {
        skinny_swiglu_lds_kernel<256><<<(unsigned)(I / 16), 512, 0, st>>>(
            (const bf16_t*)A, (const bf16_t*)Wg, (const bf16_t*)Wu, (bf16_t*)h, (int)M, I);
        return hipGetLastError();
    }
    skinny_gemm_kernel<kSkinnyWaves, 4, true><<<(unsigned)(I / 8), 64 * kSkinnyWaves, 0, st>>>(
        (const bf16_t*)A, (const bf16_t*)Wg, (const bf16_t*)Wu, nullptr, (bf16_t*)h, (int)M, 2 * I, K, 1);
    return hipGetLastError();
}

hipError_t launch_gemm_generic(int dtype, int pass, const GemmGroup& g, const int32_t* offsets, int n_groups_rows,
                               int E, int64_t rows, hipStream_t st) {
    (void)n_groups_rows;
    if (rows <= 0) return hipSuccess;
    dim3 grid((unsigned)rows, (unsigned)((g.N + 255) / 256));
    if (dtype == kBF16) {
        if (pass == 0) gemm_generic_kernel<bf16_t, 0><<<grid, 256, 0, st>>>(g, offsets, E, rows);
        else gemm_generic_kernel<bf16_t, 1><<<grid, 256, 0, st>>>(g, offsets, E, rows);
    } else {
        if (pass == 0) gemm_generic_kernel<float, 0><<<grid, 256, 0, st>>>(g, offsets, E, rows);
        else gemm_generic_kernel<float, 1><<<grid, 256, 0, st>>>(g, offsets, E, rows);
    }
    return hipGetLastError();
}

}  // namespace tmoe
