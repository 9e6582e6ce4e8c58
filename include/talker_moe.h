/*
 * talker_moe.h — C ABI of libtalker_moe.so: the Talker mixture-of-experts
 * feed-forward layer on AMD Instinct MI355X (gfx950), hand-written HIP.
 *
 * What it computes ("3C · Talker MoE (20 lớp, 128 Experts Top-6) & Đầu ra mã
 * ngữ nghĩa c_0", openarchlab, §1 Định nghĩa and §3 Giải pháp):
 *   p   = softmax(W_r x)                       router over E experts
 *   S   = the k experts with the largest p    (Top-6 of 128 in the Talker)
 *   w_i = p_i / sum_{j in S} p_j               (norm_topk_prob = True)
 *   y   = SharedMLP(x) + sum_{i in S} w_i * Expert_i(x)
 * Each expert and the shared expert is a SwiGLU MLP, down(SiLU(gate x) * up x)
 * ("用 print(model) 认识 Qwen3-TTS", horus-space, MLP section); routed experts
 * are 1024 -> 384 -> 1024 and the shared one 1024 -> 768 -> 1024 in the Talker.
 *
 * Conventions for every entry point
 *   - Pointers marked [dev] are device memory owned by the caller; the library
 *     never allocates, frees, retains or synchronises.  Host-side structs
 *     (moe_config, moe_weights) are read during the call only.
 *   - Matrices are row-major with the last index contiguous.  Weights use the
 *     nn.Linear layout [out_features, in_features].
 *   - Element type of activations and weights is cfg->dtype: MOE_BF16 (bf16 bit
 *     patterns, 2 bytes) or MOE_F32.  Indices are int32, gate weights, router
 *     bias and probabilities fp32.  MOE_BF16 accumulates in fp32 and rounds
 *     stored results to bf16 (nearest even).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous; kernel faults surface at the caller's next synchronisation.
 *   - Scratch comes from the caller's workspace `ws` of `ws_bytes` bytes,
 *     256-byte aligned; moe_workspace_size() gives a size that suffices for every
 *     entry point at that T.  Calls that share one workspace must not overlap.
 *   - Every argument is checked on the host before anything is enqueued.  The
 *     return value is MOE_OK or a negative status (moe_status_string() names
 *     it); on a negative status nothing was enqueued, except MOE_ERR_HIP,
 *     which reports a failed launch.  T == 0 is a successful no-op.
 *   - Device pointers must be 16-byte aligned; inputs must be finite (no NaN,
 *     Inf or subnormal values).
 *   - Expert selection is fp64-rescored: the library's Top-k equals the Top-k
 *     of the scores W_r x (+ bias) computed in fp64 from the exact bf16
 *     products (so up to fp64 summation rounding), ties going to the lower
 *     expert index, listed by descending weight.  It scores on the matrix cores
 *     and rescores in fp64 every token whose order is not certain under a
 *     rigorous rounding-error bound.
 *
 * Supported shapes: 1 <= k <= 32, k <= E <= 1024, 1 <= H, I <= 16384,
 * 0 <= Is <= 16384, T * k <= 2^22.  The bf16 matrix-core paths are taken when
 * H % 128 == 0 and I % 64 == 0, Is % 64 == 0 (expert products) and
 * E % 16 == 0, E <= 128 (fused router); other shapes and MOE_F32 run portable
 * kernels of the same library.
 */
#ifndef TALKER_MOE_H
#define TALKER_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID (-1)     /* bad argument: NULL required pointer, T < 0, k > E, misaligned pointer, ... */
#define MOE_ERR_UNSUPPORTED (-2) /* valid but outside the supported shapes / dtypes */
#define MOE_ERR_WORKSPACE (-3)   /* ws_bytes below what the call needs */
#define MOE_ERR_HIP (-4)         /* a HIP launch failed */
#define MOE_ERR_SCRATCH (-5)     /* the call needs more than the static scratch (MOE_STATIC_SCRATCH_BYTES) */

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer configuration, named after the model's configuration fields
 * (openarchlab Talker MoE page, §1). */
typedef struct moe_config {
    int32_t hidden_size;                     /* H (1024) */
    int32_t num_experts;                     /* E (128) */
    int32_t num_experts_per_tok;             /* k (6) */
    int32_t moe_intermediate_size;           /* I (384) */
    int32_t shared_expert_intermediate_size; /* Is (768); 0 = no shared expert */
    int32_t norm_topk_prob;                  /* 1: w_i = p_i / sum_S p; 0: w_i = p_i */
    int32_t dtype;                           /* moe_dtype */
} moe_config;

/* Weights of one layer; every pointer [dev]. */
typedef struct moe_weights {
    const void* router;       /* [E, H] */
    const float* router_bias; /* [E] fp32 added to the router scores, or NULL */
    const void* gate;         /* [E, I, H] */
    const void* up;           /* [E, I, H] */
    const void* down;         /* [E, H, I] */
    const void* shared_gate;  /* [Is, H]  (NULL when Is == 0) */
    const void* shared_up;    /* [Is, H]  (NULL when Is == 0) */
    const void* shared_down;  /* [H, Is]  (NULL when Is == 0) */
} moe_weights;

/* Text for a status code (static storage). */
const char* moe_status_string(int status);

/* MOE_OK if cfg is a valid, supported configuration, else the status a call
 * with it would return.  Host only. */
int moe_check_config(const moe_config* cfg);

/* Workspace bytes that suffice for any entry point below at T tokens
 * (0 on an invalid configuration).  Host only. */
size_t moe_workspace_size(const moe_config* cfg, int64_t T);

/*
 * moe_route — router, softmax, Top-k and renormalisation (Talker MoE page §3).
 *   x        [dev] [T, H] token hidden states
 *   router   [dev] [E, H] router weight W_r
 *   bias     [dev] [E] fp32 score bias, or NULL
 *   topk_idx [dev] [T, k] int32 out: selected experts, largest weight first,
 *                  equal scores in ascending expert index
 *   topk_w   [dev] [T, k] fp32 out: w_i (renormalised when cfg->norm_topk_prob)
 *   probs    [dev] [T, E] fp32 out: the full softmax p, or NULL to skip
 */
int moe_route(const moe_config* cfg, const void* x, const void* router, const float* bias,
              int64_t T, int32_t* topk_idx, float* topk_w, float* probs,
              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute — group the T*k (token, slot) pairs by expert (a stable counting
 * sort; the data layout that lets each expert run as one matrix product).
 *   topk_idx  [dev] [T, k] int32, every entry in [0, E)
 *   counts    [dev] [E] int32 out: pairs per expert
 *   offsets   [dev] [E+1] int32 out: exclusive prefix sum of counts
 *   row_token [dev] [T*k] int32 out: token of grouped row r; rows of one expert
 *                   are consecutive and in ascending (token, slot) order
 *   row_of    [dev] [T, k] int32 out: grouped row of pair (t, j)
 *   x, x_perm [dev] optional gather: when both are non-NULL,
 *                   x_perm[r, :] = x[row_token[r], :]  ([T*k, H])
 */
int moe_permute(const moe_config* cfg, const int32_t* topk_idx, int64_t T,
                int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_of,
                const void* x, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_swiglu — every routed expert applied to its grouped rows
 * (Talker MoE page §1: each expert is a SwiGLU 1024 -> 384 -> 1024).
 *   x         [dev] [T, H] hidden states, or [T*k, H] already grouped when
 *                   row_token is NULL
 *   row_token [dev] [T*k] from moe_permute, or NULL (x already grouped)
 *   offsets   [dev] [E+1] from moe_permute
 *   gate, up  [dev] [E, I, H];  down [dev] [E, H, I]
 *   y_perm    [dev] [T*k, H] out: y_perm[r] = Expert_e(x_r) for grouped row r
 *                   of expert e (unweighted)
 */
int moe_grouped_swiglu(const moe_config* cfg, const void* x, const int32_t* row_token,
                       const int32_t* offsets, int64_t T, const void* gate, const void* up,
                       const void* down, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_shared_swiglu — the always-on shared expert (Talker MoE page §1, §3:
 * SharedMLP(x), intermediate 768).
 *   x [dev] [T, H];  sg, su [dev] [Is, H];  sd [dev] [H, Is]
 *   y_shared [dev] [T, H] out
 * Returns MOE_ERR_INVALID when cfg has Is == 0.
 */
int moe_shared_swiglu(const moe_config* cfg, const void* x, int64_t T, const void* sg,
                      const void* su, const void* sd, void* y_shared,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine — weighted sum of the expert outputs (Talker MoE page §3):
 *   y[t] = y_shared[t] + sum_{j<k} topk_w[t,j] * y_perm[row_of[t,j]] + residual[t]
 * accumulated in fp32 in that order (shared, slots 0..k-1, residual).
 *   y_perm [dev] [T*k, H];  row_of [dev] [T, k];  topk_w [dev] [T, k] fp32
 *   y_shared, residual [dev] [T, H] or NULL (term omitted)
 *   y [dev] [T, H] out (may alias residual)
 */
int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of,
                const float* topk_w, const void* y_shared, const void* residual,
                int64_t T, void* y, void* stream);

/*
 * moe_layer_forward — the whole layer: route, group, routed and shared SwiGLU
 * experts, combine (Talker MoE page §3 equation), plus an optional residual
 * add (the [3C] step of the lab on "Bài Lab tổng hợp — Qwen3-Omni &
 * Qwen3-TTS-12Hz Architecture" adds the layer input back).
 *   w        host struct of [dev] weight pointers
 *   x        [dev] [T, H];  residual [dev] [T, H] or NULL
 *   y        [dev] [T, H] out (must not alias x; may alias residual)
 *   topk_idx_out [dev] [T, k] int32, topk_w_out [dev] [T, k] fp32,
 *   counts_out   [dev] [E] int32: optional copies of the routing, or NULL
 */
int moe_layer_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                      const void* residual, int64_t T, void* y, int32_t* topk_idx_out,
                      float* topk_w_out, int32_t* counts_out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward_timed — moe_layer_forward that also records HIP events at
 * its stage boundaries, for per-stage timing on the caller's stream (the
 * Talker MoE page's §4 profiling advice: pin numbers on the real workload and
 * keep percentiles).  stage_events is NULL or an array of 8 hipEvent_t, each
 * NULL or created by the caller; events 0-5 are recorded on `stream`:
 *   0 before routing, 1 after routing, 2 after grouping, 3 after the gate/up
 *   pass of all experts, 4 after the down pass, 5 after the combine (at decode
 *   sizes, T <= 64 of the Talker shape, there is no grouping launch and one
 *   expert launch holds both passes: 1 = 2 and 3 = 4);
 * events 6 and 7 are timestamped by the dominant kernel's own launch at its
 * start and end (hipExtLaunchKernel): the expert launch at decode sizes, else
 * the gate/up pass; so 6 -> 7 excludes dispatch latency.
 * Other arguments, results and errors are those of moe_layer_forward.
 */
int moe_layer_forward_timed(const moe_config* cfg, const moe_weights* w, const void* x,
                            const void* residual, int64_t T, void* y, int32_t* topk_idx_out,
                            float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                            void* stream, void* const* stage_events);

/*
 * moe_layer_forward_static — moe_layer_forward without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Its scratch is one
 * file-scope device array of MOE_STATIC_SCRATCH_BYTES per GPU that the library
 * is loaded on (held until the process ends); the call itself allocates
 * nothing.  The decode-size layer (T <= 64 tokens of the Talker shape needs
 * about 5 MB) fits; a call whose workspace would exceed the array returns
 * MOE_ERR_SCRATCH before anything is enqueued.
 *   The array of the current device is used (stream must belong to it); its
 *   address is looked up on the first call on each device.  Every call on one
 *   GPU shares that array, so calls that overlap on one GPU (two streams, two
 *   host threads) race and must be serialised by the caller.  Arguments,
 *   results and other errors are those of moe_layer_forward.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
int moe_layer_forward_static(const moe_config* cfg, const moe_weights* w, const void* x,
                             const void* residual, int64_t T, void* y, int32_t* topk_idx_out,
                             float* topk_w_out, int32_t* counts_out, void* stream);

/*
 * moe_rmsnorm — out = x / sqrt(mean(x^2) + eps) * gain over each row of H
 * (the pre-norm of the lab's [3C] step; eps 1e-6 and the final norm before
 * codec_head from the Qwen3-TTS module print on the horus-space page).
 *   x [dev] [T, H] (cfg->dtype);  gain [dev] [H] fp32;  out [dev] [T, H] (may alias x)
 */
int moe_rmsnorm(const moe_config* cfg, const void* x, const float* gain, float eps,
                int64_t T, void* out, void* stream);

/*
 * moe_codec_head_argmax — c_0 = argmax_v (W_c x)_v, the first codec code
 * (Talker MoE page §1: codec_head Linear 1024 -> 3072 after the last layer;
 * the lab picks the argmax).  fp64-rescored like the routing: ties go to the lowest v.
 *   x [dev] [T, H];  w_head [dev] [V, H] (cfg->dtype, bias-free)
 *   logits [dev] [T, V] fp32 out, or NULL;  c0 [dev] [T] int32 out
 */
int moe_codec_head_argmax(const moe_config* cfg, const void* x, const void* w_head, int32_t V,
                          int64_t T, float* logits, int32_t* c0,
                          void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_codec_head_argmax at (V, T). Host only. */
size_t moe_codec_head_workspace_size(const moe_config* cfg, int32_t V, int64_t T);

/*
 * Decode-time attention of the Talker ("3C · Talker MoE (20 lớp, 128 Experts
 * Top-6) & Đầu ra mã ngữ nghĩa c_0" §1: grouped-query attention, 16 query heads
 * over 2 key/value heads of 128; "1B · Interleaved TM-RoPE 3D (24, 20, 20)" §3:
 * the rotation of adjacent pairs, T/H/W interleaved, rope_theta 1e6;
 * "用 print(model) 认识 Qwen3-TTS": bias-free q/k/v/o projections and an RMSNorm
 * over each query and key head).
 */
typedef struct {
    int32_t hidden_size;       /* 1024 */
    int32_t num_heads;         /* 16 query heads */
    int32_t num_kv_heads;      /* 2; num_heads / num_kv_heads in {1, 2, 4, 8} */
    int32_t head_dim;          /* 128 (the only width supported) */
    int32_t rope_sections[3];  /* pairs on the T, H, W axes, sum head_dim / 2: {24, 20, 20} */
    float rope_theta;          /* 1e6; pair k turns by index * rope_theta^(-2k / head_dim) */
    float eps;                 /* q_norm / k_norm epsilon, 1e-6 */
    int32_t max_len;           /* cache capacity per stream (positions), a multiple of 32 */
    int32_t dtype;             /* MOE_BF16 */
} moe_attn_config;

typedef struct {
    const void* w_qkv;   /* [(num_heads + 2 num_kv_heads) head_dim, hidden]: query, key, value rows */
    const float* q_norm; /* [head_dim] gain */
    const float* k_norm; /* [head_dim] gain */
    const void* w_o;     /* [hidden, num_heads head_dim] */
} moe_attn_weights;

/*
 * moe_attention_decode — one decode step for T streams, each with its own cache.
 *   x          [dev] [T, hidden] the normalised layer input of each stream's new token
 *   pos        [dev] [T, 3] int32: its (T, H, W) indices (speech: three equal values)
 *   cache_len  [dev] [T] int32: positions already cached for stream t; the new key
 *              and value go to position cache_len[t] and the query attends to
 *              positions 0 .. cache_len[t].  The library does not advance it.  A
 *              value outside [0, max_len) writes no cache row and gives that
 *              stream a zero attention output.
 *   k_cache    [dev] [T, num_kv_heads, max_len, head_dim] bf16, in/out: keys after
 *              q/k norm and rotation, one row per position
 *   v_cache    [dev] [T, num_kv_heads, head_dim, max_len] bf16, in/out: values,
 *              transposed (one row per dimension, positions contiguous)
 *   y          [dev] [T, hidden] out: o_proj(attention) (+ residual, nullable);
 *              may alias residual or x
 *   norm_out   [dev] [T, hidden] out or NULL: RMSNorm(y) with norm_gain (nullable,
 *              1.0) and norm_eps, the next sub-layer's input, from the same pass
 * Workspace: moe_attention_workspace_size(cfg, T).  T <= 65535.
 */
int moe_attention_decode(const moe_attn_config* cfg, const moe_attn_weights* w, const void* x, int64_t T,
                         const int32_t* pos, const int32_t* cache_len, void* k_cache, void* v_cache,
                         const void* residual, void* y, const float* norm_gain, float norm_eps,
                         void* norm_out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_attention_decode at T (0 for an invalid config). Host only. */
size_t moe_attention_workspace_size(const moe_attn_config* cfg, int64_t T);

/*
 * Depth code predictor ("Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz
 * Architecture", step [4A]: the predictor is prefilled with [h_talker, embed(c_0)]
 * and produces c_1 .. c_15 in 15 autoregressive steps, one head per code;
 * "用 print(model) 认识 Qwen3-TTS", the code_predictor print: 5 decoder layers
 * with the Talker's attention (q/k norms), a SwiGLU MLP, input / post-attention
 * RMSNorms, a final norm, 15 codec_embedding tables and 15 lm_heads).
 */
typedef struct {
    moe_attn_config attn;       /* the layers' attention; max_len is ignored (the frame's positions) */
    int32_t num_layers;         /* 5 */
    int32_t intermediate_size;  /* 3072 */
    int32_t num_codes;          /* 16: c_0 .. c_15 */
    int32_t codebook_size;      /* 2048 */
    int32_t c0_vocab;           /* 3072: rows of the c_0 embedding table */
    float eps;                  /* RMSNorm eps, 1e-6 */
} moe_predictor_config;

typedef struct {
    moe_attn_weights attn;
    const float* in_norm;    /* [hidden] input_layernorm gain */
    const float* post_norm;  /* [hidden] post_attention_layernorm gain */
    const void* gate;        /* [intermediate, hidden] */
    const void* up;          /* [intermediate, hidden] */
    const void* down;        /* [hidden, intermediate] */
} moe_predictor_layer;

typedef struct {
    const moe_predictor_layer* layers;  /* host array [num_layers] */
    const float* final_norm;            /* [hidden] */
    const void* c0_embedding;           /* [c0_vocab, hidden] (the Talker's codec embedding) */
    const void* codec_embedding;        /* [num_codes - 1, codebook_size, hidden]: table j - 1 embeds c_j */
    const void* lm_head;                /* [num_codes - 1, codebook_size, hidden]: head j - 1 gives c_j */
} moe_predictor_weights;

/*
 * moe_predictor_frame — one frame for T streams (1 <= T <= 64):
 *   position 0 is h_talker, position 1 the embedding of c_0, position j + 1 that
 *   of c_j from table j - 1; each position passes the layers (pre-norm attention
 *   over the frame's own positions, residual, pre-norm SwiGLU, residual); from
 *   position 1 on, code j = argmax (exact, ties to the lowest code) of head j - 1
 *   on the final norm of position j's output.
 *   h_talker [dev] [T, hidden] bf16;  c0 [dev] [T] int32 (outside [0, c0_vocab):
 *   a zero embedding);  codes [dev] [num_codes, T] int32 out (row 0 = c0)
 *   xn_out   [dev] [num_codes, T, hidden] bf16 out or NULL: the final-normed state
 *            at every position (the heads' input)
 * The frame's key / value caches live in the workspace:
 * moe_predictor_workspace_size(cfg, T).
 */
int moe_predictor_frame(const moe_predictor_config* cfg, const moe_predictor_weights* w, const void* h_talker,
                        const int32_t* c0, int64_t T, int32_t* codes, void* xn_out, void* ws, size_t ws_bytes,
                        void* stream);

/* Workspace bytes for moe_predictor_frame at T (0 for an invalid or unsupported case). Host only. */
size_t moe_predictor_workspace_size(const moe_predictor_config* cfg, int64_t T);

/*
 * The Talker's decode step through L whole decoder layers ("3C · Talker MoE (20
 * lớp, 128 Experts Top-6) & Đầu ra mã ngữ nghĩa c_0" §1-§2: each of the 20
 * layers runs GQA, then the Top-6-of-128 MoE with its shared expert; after the
 * last, codec_head gives c_0), pre-norm as in the Qwen3-TTS module print:
 *   a = h + Attn(RMSNorm_in(h));  h' = a + MoE(RMSNorm_post(a));
 * then xn = RMSNorm_final(h_L) and c_0 = argmax codec_head(xn).
 */
typedef struct {
    moe_weights moe;          /* the layer's MoE feed-forward */
    moe_attn_weights attn;    /* the layer's attention */
    const float* in_norm;     /* [hidden] input_layernorm gain, or NULL (1.0) */
    const float* post_norm;   /* [hidden] post_attention_layernorm gain, or NULL (1.0) */
    void* k_cache;            /* [T, num_kv_heads, max_len, head_dim], in/out (as moe_attention_decode) */
    void* v_cache;            /* [T, num_kv_heads, head_dim, max_len], in/out */
} moe_talker_layer;

/*
 * moe_talker_decode — one decode step of T streams through layers[0 .. L):
 * each layer's attention adds its residual and writes the post-attention norm in
 * its last launch, and its MoE combine adds its residual and writes the next
 * layer's input norm (or the final norm) in one launch; results equal those of
 * moe_rmsnorm, moe_attention_decode (with norm_out) and moe_layer_forward called
 * layer by layer.
 *   x          [dev] [T, hidden] the stack input;  h_out [dev] [T, hidden] out
 *   pos, cache_len  as moe_attention_decode (shared by all layers; not advanced)
 *   final_norm [dev] [hidden] or NULL (1.0);  eps: every RMSNorm's epsilon
 *   codec_head [dev] [V, hidden] or NULL;  c0 [dev] [T] int32 out or NULL
 *   xn_out     [dev] [T, hidden] out or NULL: the final-normed state
 * Workspace: moe_talker_decode_workspace_size(cfg, acfg, T, V) (V = 0 without
 * the head).  T <= 65535.
 */
int moe_talker_decode(const moe_config* cfg, const moe_attn_config* acfg, const moe_talker_layer* layers, int32_t L,
                      const void* x, int64_t T, const int32_t* pos, const int32_t* cache_len,
                      const float* final_norm, float eps, const void* codec_head, int32_t V, void* h_out,
                      void* xn_out, int32_t* c0, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_talker_decode (0 for an invalid or unsupported case). Host only. */
size_t moe_talker_decode_workspace_size(const moe_config* cfg, const moe_attn_config* acfg, int64_t T, int32_t V);

/*
 * moe_talker_frame — one 80 ms frame of T streams of the Dual-Track loop ("Bài
 * Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz Architecture", steps [3B] and
 * [4A]; "3C · Talker MoE" §2, the pair [h_talker, c_0] handed to the code
 * predictor):
 *   x = prev_emb + cond (rounded to bf16);
 *   the Talker step through layers[0 .. L) as moe_talker_decode (keys and values
 *   appended at cache_len, queries at pos), its final-normed state xn and c_0;
 *   codes = moe_predictor_frame(xn, c_0);
 *   prev_emb = the mean of the frame's num_codes code embeddings (c_0 from the
 *   predictor's c0_embedding, c_j from codec_embedding table j - 1; a code
 *   outside its table is a zero row), summed in fp32 and rounded to bf16;
 *   pos (all three indices) and cache_len advance by one.
 * Every step runs on the stream from device data, so one captured graph replays
 * frame after frame: between replays the caller only writes the next cond.
 * Results equal moe_talker_decode on x, then moe_predictor_frame, bit for bit.
 *   cond      [dev] [T, hidden] bf16: the frame's text condition (the trailing
 *             text hidden state, or the pad embedding once the text has run out)
 *   prev_emb  [dev] [T, hidden] bf16, in/out: the previous frame's audio embedding
 *             (the codec BOS embedding before the first frame); the frame's own on return
 *   pos       [dev] [T, 3] int32, in/out;  cache_len [dev] [T] int32, in/out
 *   codes     [dev] [num_codes, T] int32 out (row 0 = c_0)
 *   h_out, xn_out  [dev] [T, hidden] bf16 out or NULL: the Talker's last hidden
 *             state and its final-normed state
 *   codec_head [dev] [V, hidden] (V >= 1); final_norm as moe_talker_decode
 * 1 <= T <= 64; bf16; the predictor's hidden size equals the Talker's.
 * Workspace: moe_talker_frame_workspace_size(cfg, acfg, pcfg, T, V).
 */
int moe_talker_frame(const moe_config* cfg, const moe_attn_config* acfg, const moe_talker_layer* layers, int32_t L,
                     const float* final_norm, float eps, const void* codec_head, int32_t V,
                     const moe_predictor_config* pcfg, const moe_predictor_weights* pw, const void* cond, int64_t T,
                     void* prev_emb, int32_t* pos, int32_t* cache_len, int32_t* codes, void* h_out, void* xn_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_talker_frame (0 for an invalid or unsupported case). Host only. */
size_t moe_talker_frame_workspace_size(const moe_config* cfg, const moe_attn_config* acfg,
                                       const moe_predictor_config* pcfg, int64_t T, int32_t V);

/*
 * moe_codec_head_sample — c_0 drawn from the softmax of the codec head's logits
 * ("用 print(model) 认识 Qwen3-TTS", "Codec Head：语义码预测": the 3072 logits go
 * through a softmax and the next semantic code is sampled).  Inverse transform
 * with one caller-supplied uniform per token:
 *   e_v = exp(logit_v / temperature) (up to a common factor),
 *   c0[t] = the first v with  sum_{i<=v} e_i > u[t] * sum_i e_i.
 * The decision is exact up to fp64 rounding: it is certified from the fp32
 * logits and their error bounds, and tokens whose u falls within that error of
 * a boundary are decided on logits recomputed in fp64.  The random numbers are
 * inputs, so a draw is reproducible.
 *   x [dev] [T, H]; w_head [dev] [V, H]; 1 <= V <= 8192; temperature > 0 (finite)
 *   u      [dev] [T] fp64 uniforms; u < 0 or NaN gives code 0, u >= 1 code V - 1
 *   logits [dev] [T, V] fp32 out, or NULL;  c0 [dev] [T] int32 out
 * Workspace: moe_codec_head_workspace_size(cfg, V, T).
 */
int moe_codec_head_sample(const moe_config* cfg, const void* x, const void* w_head, int32_t V, int64_t T,
                          float temperature, const double* u, float* logits, int32_t* c0, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * moe_stack_forward — L stacked layers and the codec head, the lab's [3C]
 * step layer by layer ("Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz
 * Architecture"; 20 layers and codec_head 1024 -> 3072 on the Talker MoE page,
 * §1; the norm before codec_head from the Qwen3-TTS module print):
 *   h_0 = x;  h_{l+1} = h_l + MoE_l(RMSNorm_l(h_l));  xn = RMSNorm_L(h_L);
 *   c_0 = argmax_v (W_c xn)_v  (ties to the lowest v).
 * Each layer's combine, residual add and the next RMSNorm run as one launch;
 * results equal those of moe_rmsnorm and moe_layer_forward (residual = h_l)
 * called layer by layer.
 *   layers     host array of L weight structs (L >= 1)
 *   x          [dev] [T, H] stack input;  h_out [dev] [T, H] out: h_L (may alias x)
 *   gains      [dev] [L + 1, H] fp32 (norm l before layer l; norm L before
 *              the head), or NULL for gains of 1.0;  eps >= 0
 *   codec_head [dev] [V, H] or NULL;  c0 [dev] [T] int32 out or NULL (needs
 *              codec_head and V >= 1)
 *   xn_out     [dev] [T, H] out: the final normalised state, or NULL (must not
 *              alias x or h_out)
 * All layer pointers are checked before anything is enqueued.  Workspace:
 * moe_stack_workspace_size(cfg, T, V) (V = 0 without the head).
 */
int moe_stack_forward(const moe_config* cfg, const moe_weights* layers, int32_t L, const void* x,
                      int64_t T, const float* gains, float eps, const void* codec_head, int32_t V,
                      void* h_out, void* xn_out, int32_t* c0, void* ws, size_t ws_bytes,
                      void* stream);

/* Workspace bytes for moe_stack_forward at (T, V); V = 0 when no c0 is asked for. Host only. */
size_t moe_stack_workspace_size(const moe_config* cfg, int64_t T, int32_t V);

#ifdef __cplusplus
}
#endif

#endif /* TALKER_MOE_H */
