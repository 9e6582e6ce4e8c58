// The 16-column skinny product as a device function, so that other launches
// can run it on their idle workgroups (see skinny_gemm_kernel in gemm.hip for
// the product and its layout).
#pragma once

#include "common.hpp"

namespace tmoe {

constexpr int kSkinnyRows = 64;
constexpr int kSkinnyWaves = 4;

// Workgroup (bx, by) of the 16-column form with NW waves: P[by] [M, 16] columns
// 16 bx .. (fp32 partials of K run by), or, for SWIGLU, h [M, N / 2] features
// 8 bx .. 8 bx + 7 = SiLU(gate) * up from gate rows of W and up rows of W2 over
// all of K (KS == 1).  M <= 16 MT; K % (KS * NW * 32) == 0.
template <int NW, int U, bool SWIGLU, int MT = 4>
__device__ __forceinline__ void skinny_body(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                            const bf16_t* __restrict__ W2, float* __restrict__ P,
                                            bf16_t* __restrict__ h, int M, int N, int K, int KS, int bx, int by) {
    __shared__ float part[NW][16 * MT][17];
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int n0 = bx * 16, run = by;
    const int r = lane & 15, kg = (lane >> 4) * 8;
    const int kw = K / KS / NW, kb = run * (K / KS) + wave * kw;
    const bf16_t* wp = (SWIGLU ? (r < 8 ? W + (int64_t)(n0 / 2 + r) * K : W2 + (int64_t)(n0 / 2 + r - 8) * K)
                               : W + (int64_t)(n0 + r) * K) + kb + kg;
    const bf16_t* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ap[mt] = A + (int64_t)min(mt * 16 + r, M - 1) * K + kb + kg;
    const f32x4 zero = {0, 0, 0, 0};
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = zero;
    for (int kk = 0; kk < kw; kk += 32 * U) {
        u32x4 b[U], a[MT][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // branch-free: steps past the end repeat the last one, unused
            const int k = min(kk + 32 * u, kw - 32);
            b[u] = *reinterpret_cast<const u32x4*>(wp + k);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt][u] = *reinterpret_cast<const u32x4*>(ap[mt] + k);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kk + 32 * u >= kw) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt][u]),
                                                                  __builtin_bit_cast(bf16x8, b[u]), acc[mt], 0, 0, 0);
        }
    }
    // D[row = 4 (lane / 16) + i][col = lane % 16] of each 16-row tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][mt * 16 + 4 * (lane >> 4) + i][r] = acc[mt][i];
    __syncthreads();
    if (SWIGLU) {
        for (int idx = threadIdx.x; idx < 16 * MT * 8; idx += 64 * NW) {
            const int row = idx >> 3, c = idx & 7;
            if (row >= M) continue;
            float gv = part[0][row][c], uv = part[0][row][c + 8];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                gv += part[w][row][c];
                uv += part[w][row][c + 8];
            }
            h[(int64_t)row * (N / 2) + n0 / 2 + c] = f32_to_bf16(silu(gv) * uv);
        }
        return;
    }
    float* out = P + (int64_t)run * M * N;
    for (int idx = threadIdx.x; idx < 16 * MT * 16; idx += 64 * NW) {
        const int row = idx >> 4, col = idx & 15;
        if (row >= M) continue;
        float v = part[0][row][col];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += part[w][row][col];
        out[(int64_t)row * N + n0 + col] = v;
    }
}

}  // namespace tmoe
