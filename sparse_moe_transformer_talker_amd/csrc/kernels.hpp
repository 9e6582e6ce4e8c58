// Host-side launchers of the Talker MoE kernels (one HIP translation unit each).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmoe {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;

// --- routing (route.hip) ---
// Row maps of a grouping: row_token[r] = token of grouped row r; row_of[t * k + j]
// = grouped row of pair (t, j); row_pair[r] = t * k + j (nullable).
struct TileSpec;
// Small batches: one block groups the routing from the router's masks (counts,
// offsets, tile lists and row maps).
bool group_small_ok(int64_t T, int E);
hipError_t launch_group_small(const int32_t* idx, const uint16_t* masks, int64_t T, int E, int k, int32_t* counts,
                              int32_t* offsets, int32_t* row_token, int32_t* row_of, int32_t* row_pair,
                              const TileSpec* t1, const TileSpec* t2, hipStream_t st);
// masks (nullable): [E][mask_stride(T)] uint16, bit t % 16 of word t / 16 set when
// token t routes to e; jmask (nullable, k <= 16): [E][mask_stride(T)] uint64 with
// the slot j of that choice in bits 4 (t % 16) .. + 3, written only when
// route_block_ok (the other selection kernels write masks alone)
hipError_t launch_route(int dtype, const void* x, const void* W, const float* bias, int64_t T, int H, int E, int k,
                        int norm, int32_t* idx, float* w, float* probs, float* scratch_sc, float* scratch_bd,
                        uint16_t* masks, uint64_t* jmask, hipStream_t st);
// Small batches, bf16: after launch_scores, one block selects every token and
// groups the routing (same outputs as launch_route + launch_group_small).
bool route_group_small_ok(int dtype, int64_t T, int H, int E, int k);
hipError_t launch_select_group_small(const float* sc, const float* bd, const void* x, const void* W,
                                     const float* bias, int64_t T, int H, int E, int k, int norm, int32_t* idx,
                                     float* w, int32_t* counts, int32_t* offsets, int32_t* row_token,
                                     int32_t* row_of, int32_t* row_pair, const TileSpec* t1, const TileSpec* t2,
                                     hipStream_t st);
hipError_t launch_scores(int dtype, const void* x, const void* W, const float* bias, int64_t T, int H, int n,
                         float* sc, float* bd, hipStream_t st);
// bf16, E in {16, 32, 64, 128}, H <= 1024 a multiple of 128 (8 / (E / 16)), k <= 16: scores and
// selection in one launch (one block per 16 tokens).  Writes masks (nullable,
// as launch_route), or per block b of 16 tokens and expert e the count
// bcnt[b * E + e] and the pairs t * k + j in blist[(b * E + e) * 16 + i]
// (bcnt / blist nullable; order inside a block's list is arbitrary).
bool route_block_ok(int dtype, int H, int E, int k);
hipError_t launch_route_block(const void* x, const void* W, const float* bias, int64_t T, int H, int E, int k,
                              int norm, int32_t* idx, float* w, float* probs, uint16_t* masks, uint64_t* jmask,
                              int32_t* bcnt, int32_t* blist, hipStream_t st);
// The same launch with the shared expert's gate/up product on further
// workgroups (the CUs the router leaves idle): hs [T, Is] = SiLU(x sg^T) * (x su^T)
// in bf16 (sg, su [Is, H]).  Needs route_shared_ok.
bool route_shared_ok(int64_t T, int H, int Is);
hipError_t launch_route_block_shared(const void* x, const void* W, const float* bias, int64_t T, int H, int E, int k,
                                     int norm, int32_t* idx, float* w, int32_t* bcnt, int32_t* blist,
                                     const void* sg, const void* su, int Is, void* hs, hipStream_t st);
hipError_t launch_argmax(int dtype, const float* sc, const float* bd, const void* x, const void* W, int64_t T, int H,
                         int n, int32_t* out, hipStream_t st);
// Draw per token from softmax(scores / tau) by inverse transform with the given
// uniform u[t] (fp64), exact up to fp64 rounding: certified from sc / bd, else
// from fp64 logits recomputed from x and W.  n <= kSampleMaxN.
constexpr int kSampleMaxN = 8192;
bool sample_ok(int n);
// Scores for an exact argmax (no bias): fp32 matrix-core partials added in fp64
// for bf16 with H % 32 == 0 and T <= 256 (the argmax rescores the rare
// near-ties in fp64); else launch_scores.
hipError_t launch_scores_argmax(int dtype, const void* x, const void* W, int64_t T, int H, int n, float* sc,
                                float* bd, hipStream_t st);
// Scores with the tightest bounds available (fp64 sums of exact products for bf16
// with H % 256 == 0, at any T; else launch_scores).
hipError_t launch_scores_exact(int dtype, const void* x, const void* W, int64_t T, int H, int n, float* sc, float* bd,
                               hipStream_t st);
hipError_t launch_sample(int dtype, const float* sc, const float* bd, const void* x, const void* W, int64_t T, int H,
                         int n, double tau, const double* u, int32_t* out, hipStream_t st);

// --- grouping (permute.hip) ---
// Tiling of one grouped GEMM: items are (expert, n0, m0, rows) tiles of at most
// mt rows and nt columns of an output of width n_routed (routed experts) or
// n_shared (the shared expert, taken as expert index E, rows = tokens).
struct TileSpec {
    int mt, nt;
    int n_routed, n_shared;
    int4* items;
    int* count;
    int max_items;
};
int64_t tile_max_items(int64_t pairs, int E, int64_t T, int mt, int nt, int n_routed, int n_shared);
int mask_words(int64_t T);
int mask_stride(int64_t T);
hipError_t launch_masks(const int32_t* idx, int64_t T, int k, int E, uint16_t* masks, uint64_t* jmask,
                        hipStream_t st);
// prefix: [E][mask_stride(T)] int32 scratch (E > 128 only); jmask nullable
hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, const uint16_t* masks, const uint64_t* jmask,
                          int32_t* prefix, int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_of,
                          int32_t* row_pair, const TileSpec* t1, const TileSpec* t2, hipStream_t st);
hipError_t launch_build_items(const int32_t* offsets, int E, int64_t T, const TileSpec* t1, const TileSpec* t2,
                              hipStream_t st);

// --- grouped SwiGLU matrix products (gemm.hip) ---
struct GemmGroup {
    const void* wa;        // gate (gate/up pass) or down (down pass): [n_experts, N, K]
    const void* wb;        // up (gate/up pass); unused in the down pass
    int64_t w_estride;     // elements between experts
    int N, K;              // output width, reduction length
    const void* a;         // A rows
    int64_t a_ld;          // elements between A rows
    const int32_t* a_rows; // row r -> A row a_rows[r] / a_div, or nullptr (A row r)
    int a_div;
    void* out;
    int64_t out_ld;
    const int32_t* out_rows;  // row r -> v = out_rows[r], or nullptr (v = r)
    int out_mul, out_add;     // destination row = v * out_mul + out_add (+ v / out_div if out_div > 0)
    int out_div;
};
struct GemmArgs {
    GemmGroup g[2];  // [0] routed experts, [1] shared expert (expert index == E)
    const int4* items;
    const int* count;
    int E;
    // The list holds the routed tiles, then n_shared_items shared-expert tiles.
    // Each XCD takes an equal share of both kinds, the shared ones first when
    // shared_first (their reduction is longer), else last.
    int n_shared_items;
    int shared_first;
    // Direct tiling (when direct_bcnt is not null; small-M kernel only): the grid
    // is E * direct_nt[0] routed tiles, expert-major, then direct_nt[1] x
    // direct_mt1 shared tiles.  A routed tile of expert e concatenates the
    // router's per-block pair lists (direct_bcnt / direct_blist of
    // launch_route_block, direct_nb blocks) into its m rows, which are rows
    // e * direct_T .. e * direct_T + m - 1 of its h buffer; in the gate/up pass
    // the pair p gives A row p / a_div, in the down pass output row p.  Tiles
    // of column 0 write m to direct_counts[e] (nullable).
    const int* direct_bcnt;
    const int* direct_blist;
    int direct_nb;
    int* direct_counts;
    int direct_T;
    int direct_nt[2];
    int direct_mt1;
};
enum GemmVariant { kGemmSmallM = 0, kGemmLargeM = 1, kGemmLargeLds = 2, kGemmHugeLds = 3 };
void gemm_tiles(int variant, int pass, int* mt, int* nt);
bool gemm_mfma_ok(int dtype, int H, int I, int Is);
bool gemm_lds_ok(int H, int I, int Is);  // shapes of the 128 x 256 direct-to-LDS tiles
// ev_start / ev_stop (nullable): timestamped by the launch at the kernel's start and end
hipError_t launch_grouped_gemm(int dtype, int variant, int pass, const GemmArgs& args, int64_t max_items,
                               hipStream_t st, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// Direct tiling of the small-M kernel: tile width of a pass, and the launch.
int gemm_direct_tile(int pass, int* bm);
hipError_t launch_grouped_gemm_direct(int pass, const GemmArgs& args, hipStream_t st, hipEvent_t ev_start = nullptr,
                                      hipEvent_t ev_stop = nullptr);
// Split-K skinny product: P[s] [M, N] (fp32, s < KS) = A [M, K_s] W_s^T over the
// s-th of KS equal runs of K; bf16 inputs, M <= 64, N % 16 == 0.  KS from
// skinny_gemm_runs (0: the shape does not fit).
int skinny_gemm_runs(int64_t M, int N, int K);
hipError_t launch_skinny_gemm(const void* A, const void* W, float* P, int64_t M, int N, int K, int KS,
                              hipStream_t st);
// h [M, I] bf16 = SiLU(A Wg^T) * (A Wu^T) for M <= 64 (Wg, Wu [I, K]; I % 8 == 0,
// K % 128 == 0), in one launch without partials
bool skinny_swiglu_ok(int64_t M, int I, int K);
hipError_t launch_skinny_swiglu(const void* A, const void* Wg, const void* Wu, void* h, int64_t M, int I, int K,
                                hipStream_t st);
// Portable path: one thread per output; rows of group 0 find their expert in offsets.
hipError_t launch_gemm_generic(int dtype, int pass, const GemmGroup& g, const int32_t* offsets, int n_groups_rows,
                               int E, int64_t rows, hipStream_t st);

// --- element-wise (elementwise.hip) ---
// Term j < k of token t: row rows[t * k + j] of ysrc (rows not null) or slot j
// of the token's `slots` consecutive rows (rows null), times w[t * k + j] (w
// nullable in slot mode: the slots already carry their weights).
hipError_t launch_combine(int dtype, const void* ysrc, const int32_t* rows, const float* w, int k, int slots,
                          const void* shared, int64_t sstride, const void* residual, void* y, int64_t T, int H,
                          hipStream_t st);
// gain nullable (1.0)
hipError_t launch_rmsnorm(int dtype, const void* x, const float* gain, float eps, int64_t T, int H, void* out,
                          hipStream_t st);
// Slot-mode combine (as launch_combine with rows == nullptr) followed by the
// RMSNorm of the stored y into norm_out, fused for bf16 rows; same results as
// the two launches.
hipError_t launch_combine_norm(int dtype, const void* ysrc, const float* w, int k, int slots, const void* shared,
                               int64_t sstride, const void* residual, void* y, int64_t T, int H, const float* gain,
                               float eps, void* norm_out, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t st);
hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* rows, int64_t n, int H, void* out,
                              hipStream_t st);

// The frame loop (elementwise.hip): x = bf16(a + b) and out = RMSNorm(x) * gain
// (bf16, H % 8 == 0, H <= 4096); then, after the frame, prev [T, H] = the mean
// of the frame's code embeddings (codes [Q, T]: c_0 from c0_table [V0, H], c_j
// from tables [Q - 1, K, H]) and pos [T, 3], len [T] advanced by one.
hipError_t launch_add_rmsnorm(const void* a, const void* b, void* x, const float* gain, float eps, int64_t Ttok,
                              int H, void* out, hipStream_t st);
hipError_t launch_frame_advance(const int32_t* codes, int Q, const void* c0_table, int V0, const void* tables, int K,
                                int64_t Ttok, int H, void* prev, int32_t* pos, int32_t* len, hipStream_t st);

// Decode layer part of a partial-row combine (elementwise.hip): y [T, H] from the
// partial rows [T, k S + SSH, H] of launch_decode_experts and the routing
// weights w [T, k] (+ residual), then norm_out = RMSNorm(y) * gain when
// norm_out is not null.  bf16, H % 8 == 0, H <= 1024.
hipError_t launch_combine_partials(const void* part, int S, int SSH, int k, const float* w, const void* residual,
                                   void* y, int64_t T, int H, const float* gain, float eps, void* norm_out,
                                   hipStream_t st);

// --- the decode-size layer (decode.hip) ---
// bf16, 1 <= T <= 64, H == 1024, k <= E <= 128, k <= 8, I a multiple of 64, Is a multiple of 128 (or 0).
bool decode_layer_ok(int dtype, int64_t T, int H, int E, int k, int I, int Is);
// partial rows per token: k I / 64 routed slots, then one slot for the shared expert (Is > 0)
int decode_partial_rows(int k, int I, int Is);
// idx [T, k], w [T, k]: top-k of the scores (certified, else fp64-rescored), ties
// to the lower index; sc, dv [T, E] fp64 scratch (the scores and their bounds);
// mask [4] the touched experts, counts [E] the pairs per expert; with Is > 0
// also hs [T, Is] = SiLU(x sg^T) * (x su^T) in bf16
hipError_t launch_route_decode(const void* x, const void* W, const float* bias, int64_t T, int H, int E, int k,
                               int norm, double* sc, double* dv, int32_t* idx, float* w, const void* sg,
                               const void* su, int Is, void* hs, uint32_t* mask, int32_t* counts, hipStream_t st);
// part [T, decode_partial_rows, H] bf16 (see decode.hip) from the routing (idx and
// the mask of launch_route_decode)
hipError_t launch_decode_experts(const void* x, const int32_t* idx, const uint32_t* mask, const void* gate,
                                 const void* up, const void* down, const void* hs, const void* sdown, void* part,
                                 int64_t T, int H, int E, int k, int I, int Is, hipStream_t st,
                                 hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// --- decode-time attention (attention.hip) ---
// head_dim 128, nq / nkv in {1, 2, 4, 8}, max_len a multiple of 32
bool attn_decode_ok(int head_dim, int nq, int nkv, int max_len);
int attn_chunks(int max_len);  // partials per (stream, KV head): 512 positions each (128 up to 256)
// qkv: KS fp32 partials [KS][T][(nq + 2 nkv) 128] of the projection (summed in
// order) -> q_out [T, nq, 128] (normalised, rotated), the new
// key row at position len[t] of kc [T, nkv, max_len, 128] and the new value
// column at len[t] of the transposed vc [T, nkv, 128, max_len]
hipError_t launch_qk_rope_append(const float* qkv, int KS, int64_t T, int nq, int nkv, const float* q_gain,
                                 const float* k_gain, float eps, const int32_t* pos, const int32_t* len,
                                 int max_len, int sec_h, int sec_w, double theta, void* q_out, void* kc, void* vc,
                                 hipStream_t st);
// o [T, nq, 128] = attention of q over positions 0..len[t] of each stream's
// cache; pm / pl [T nkv chunks (nq / nkv)], pacc [.. x 128] fp32 scratch
hipError_t launch_attn_decode(const void* q, const void* kc, const void* vc, const int32_t* len, int64_t T, int nq,
                              int nkv, int max_len, float* pm, float* pl, float* pacc, void* o, hipStream_t st);
// launch_qk_rope_append and launch_attn_decode in one launch (no q buffer):
// each attention workgroup forms its query heads and the new key and value
// itself; when attn_rope_fused_ok (nq / nkv + 2 waves fit the workgroup)
bool attn_rope_fused_ok(int nq, int nkv, int max_len);
hipError_t launch_attn_rope_decode(const float* qkv, int KS, int64_t T, int nq, int nkv, const float* q_gain,
                                   const float* k_gain, float eps, const int32_t* pos, const int32_t* len,
                                   int max_len, int sec_h, int sec_w, double theta, void* kc, void* vc, float* pm,
                                   float* pl, float* pacc, void* o, hipStream_t st);
// y [T, H] = sum of the KS fp32 partials [KS][T][H] (in order) + residual
// (nullable), stored bf16; norm_out (nullable) = RMSNorm(y) * gain (nullable)
hipError_t launch_attn_out(const float* part, int KS, const void* residual, void* y, int64_t T, int H,
                           const float* gain, float eps, void* norm_out, hipStream_t st);
// x [T, H] = table[idx[t]] (bf16 rows, H % 8 == 0; indices outside [0, rows) give zero rows) and
// out = RMSNorm(x) * gain (H <= 4096)
hipError_t launch_embed_norm(const void* table, int rows, const int32_t* idx, void* x, const float* gain, float eps,
                             int64_t T, int H, void* out, hipStream_t st);
// Frame set-up of the code predictor: pos [P][T][3] = p, len [P][T] = p, codes
// row 0 = c0 (codes [num][T])
hipError_t launch_frame_setup(int32_t* pos, int32_t* len, int P, int64_t T, const int32_t* c0, int32_t* codes,
                              hipStream_t st);

}  // namespace tmoe
