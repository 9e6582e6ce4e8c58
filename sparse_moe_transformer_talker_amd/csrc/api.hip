// C ABI of libtalker_moe.so (declared in include/talker_moe.h): argument
// checks, workspace carving and the launch sequence of each entry point.
// Every check runs on the host before anything is enqueued; the library never
// allocates or synchronises.
#include "talker_moe.h"

#include <stdint.h>

#include <mutex>

#include "kernels.hpp"

using namespace tmoe;

namespace {

constexpr int64_t kMaxPairs = int64_t(1) << 22;
constexpr int kMaxDim = 16384;
constexpr int kMaxStackLayers = 1024;

// Carves 256-byte aligned regions out of the caller's workspace; with a null
// base it only measures.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(int64_t n) {
        off = (off + 255) & ~size_t(255);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += size_t(n > 0 ? n : 0) * sizeof(T);
        return p;
    }
    size_t size() const { return (off + 255) & ~size_t(255); }
};

size_t esize(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
int64_t nb_of(int64_t T) { return mask_words(T); }  // 16-token router blocks

int check_cfg(const moe_config* c) {
    if (!c) return MOE_ERR_INVALID;
    if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID;
    if (c->hidden_size < 1 || c->num_experts < 1 || c->num_experts_per_tok < 1 || c->moe_intermediate_size < 1 ||
        c->shared_expert_intermediate_size < 0)
        return MOE_ERR_INVALID;
    if (c->num_experts_per_tok > c->num_experts) return MOE_ERR_INVALID;
    if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1) return MOE_ERR_INVALID;
    if (c->num_experts > kMaxExperts || c->num_experts_per_tok > kMaxTopK || c->hidden_size > kMaxDim ||
        c->moe_intermediate_size > kMaxDim || c->shared_expert_intermediate_size > kMaxDim)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_T(const moe_config* c, int64_t T) {
    if (T < 0) return MOE_ERR_INVALID;
    if (T * c->num_experts_per_tok > kMaxPairs) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// --- workspace plans ---------------------------------------------------------
struct RoutePlan {
    float* sc = nullptr;
    float* bd = nullptr;
};
void plan_route(const moe_config* c, int64_t T, Carver& cv, RoutePlan& p) {
    p.sc = cv.take<float>(T * c->num_experts);
    p.bd = cv.take<float>(T * c->num_experts);
}

struct GemmPlan {
    bool mfma = false;
    int variant = kGemmSmallM;
    TileSpec t[2]{};
    int64_t max_items[2]{0, 0};
};
// Tile lists for the two passes when the matrix-core path applies.
void plan_gemm(const moe_config* c, int64_t T, bool routed, bool shared, Carver& cv, GemmPlan& g,
               int64_t small_rows = 32) {
    const int H = c->hidden_size, E = c->num_experts, k = c->num_experts_per_tok;
    const int I = c->moe_intermediate_size, Is = shared ? c->shared_expert_intermediate_size : 0;
    g.mfma = gemm_mfma_ok(c->dtype, H, I, Is);
    if (!g.mfma) return;
    const int64_t pairs = routed ? T * k : 0;
    const int64_t rows_per_expert = routed ? pairs / E : T;
    if (rows_per_expert < small_rows) g.variant = kGemmSmallM;
    else if (!gemm_lds_ok(H, I, Is)) g.variant = kGemmLargeM;
    else g.variant = rows_per_expert >= 160 ? kGemmHugeLds : kGemmLargeLds;
    int* counters = cv.take<int>(4);
    for (int pass = 0; pass < 2; ++pass) {
        int mt, nt;
        gemm_tiles(g.variant, pass, &mt, &nt);
        const int n_routed = pass == 0 ? I : H;
        const int n_shared = Is > 0 ? (pass == 0 ? Is : H) : 0;
        g.max_items[pass] = tile_max_items(pairs, routed ? E : 0, T, mt, nt, n_routed, n_shared);
        TileSpec& ts = g.t[pass];
        ts.mt = mt;
        ts.nt = nt;
        ts.n_routed = n_routed;
        ts.n_shared = n_shared;
        ts.items = cv.take<int4>(g.max_items[pass]);
        ts.count = counters ? counters + pass : nullptr;
        ts.max_items = (int)g.max_items[pass];
    }
}

struct LayerPlan {
    int32_t* idx;
    float* w;
    RoutePlan route;
    uint16_t* masks;
    uint64_t* jmask;
    int32_t *prefix, *counts, *offsets, *row_token, *row_of, *row_pair;
    GemmPlan gemm;
    void *hr, *hs, *ybuf;
    // direct decode path: the router's per-block pair lists, h rows at e * T + i
    bool direct;
    int32_t *bcnt, *blist;
    void* hd;
    // decode-size path (decode.hip): spread router scores, per-token selection,
    // one expert launch, partial rows
    bool decode;
    void* part;
    double *sc, *dv;
    uint32_t* mask;
};
// Small batches on the matrix-core path: the router writes per-block pair
// lists and the expert products tile themselves from them (no grouping launch).
constexpr int64_t kDirectMaxT = 256;
bool direct_ok(const moe_config* c, int64_t T, const GemmPlan& g) {
    const int E = c->num_experts, I = c->moe_intermediate_size;
    return g.mfma && g.variant == kGemmSmallM && T <= kDirectMaxT &&
           route_block_ok(c->dtype, c->hidden_size, E, c->num_experts_per_tok) &&
           (int64_t)E * T * I * (int64_t)esize(c->dtype) <= (64ll << 20);
}
bool decode_ok(const moe_config* c, int64_t T) {
    return decode_layer_ok(c->dtype, T, c->hidden_size, c->num_experts, c->num_experts_per_tok,
                           c->moe_intermediate_size, c->shared_expert_intermediate_size);
}
void plan_layer(const moe_config* c, int64_t T, Carver& cv, LayerPlan& p) {
    const int E = c->num_experts, k = c->num_experts_per_tok, H = c->hidden_size;
    const int I = c->moe_intermediate_size, Is = c->shared_expert_intermediate_size;
    const int64_t N = T * k;
    const size_t es = esize(c->dtype);
    p.idx = cv.take<int32_t>(N);
    p.w = cv.take<float>(N);
    p.decode = decode_ok(c, T);
    if (p.decode) {
        // everything else of the plan stays null: the decode path uses only these
        p.route = RoutePlan{};
        p.counts = cv.take<int32_t>(E);
        p.part = cv.take<char>(T * decode_partial_rows(k, I, Is) * (int64_t)H * (int64_t)es);
        p.sc = cv.take<double>(T * E);
        p.dv = cv.take<double>(T * E);
        p.mask = cv.take<uint32_t>(4);
        p.hs = cv.take<char>(T * Is * (int64_t)es);
        p.masks = nullptr;
        p.jmask = nullptr;
        p.prefix = p.offsets = p.row_token = p.row_of = p.row_pair = nullptr;
        p.gemm = GemmPlan{};
        p.hr = p.ybuf = p.hd = nullptr;
        p.direct = false;
        p.bcnt = p.blist = nullptr;
        return;
    }
    p.part = nullptr;
    p.sc = p.dv = nullptr;
    p.mask = nullptr;
    plan_route(c, T, cv, p.route);
    p.counts = cv.take<int32_t>(E);
    p.offsets = cv.take<int32_t>(E + 1);
    p.masks = cv.take<uint16_t>((int64_t)E * mask_stride(T));
    p.jmask = cv.take<uint64_t>((int64_t)E * mask_stride(T));
    p.prefix = cv.take<int32_t>((int64_t)E * mask_stride(T));
    p.row_token = cv.take<int32_t>(N);
    p.row_of = cv.take<int32_t>(N);
    p.row_pair = cv.take<int32_t>(N);
    plan_gemm(c, T, true, Is > 0, cv, p.gemm);
    p.hr = cv.take<char>(N * I * (int64_t)es);
    p.hs = cv.take<char>(T * Is * (int64_t)es);
    p.ybuf = cv.take<char>(T * (k + 1) * (int64_t)H * (int64_t)es);
    p.direct = direct_ok(c, T, p.gemm);
    const int64_t nb = mask_words(T);
    p.bcnt = p.direct ? cv.take<int32_t>(nb * E) : nullptr;
    p.blist = p.direct ? cv.take<int32_t>(nb * E * 16) : nullptr;
    p.hd = p.direct ? cv.take<char>((int64_t)E * T * I * (int64_t)es) : nullptr;
}

size_t route_ws(const moe_config* c, int64_t T) {
    Carver cv(nullptr);
    RoutePlan p;
    plan_route(c, T, cv, p);
    return cv.size();
}
size_t permute_ws(const moe_config* c, int64_t T) {
    Carver cv(nullptr);
    cv.take<uint16_t>((int64_t)c->num_experts * mask_stride(T));
    cv.take<uint64_t>((int64_t)c->num_experts * mask_stride(T));
    cv.take<int32_t>((int64_t)c->num_experts * mask_stride(T));
    return cv.size();
}
size_t grouped_ws(const moe_config* c, int64_t T, void* base, GemmPlan* g, void** hr) {
    Carver cv(base);
    GemmPlan tmp;
    plan_gemm(c, T, true, false, cv, g ? *g : tmp);
    void* h = cv.take<char>(T * c->num_experts_per_tok * (int64_t)c->moe_intermediate_size * (int64_t)esize(c->dtype));
    if (hr) *hr = h;
    return cv.size();
}
size_t shared_ws(const moe_config* c, int64_t T, void* base, GemmPlan* g, void** hs) {
    Carver cv(base);
    GemmPlan tmp;
    plan_gemm(c, T, false, true, cv, g ? *g : tmp);
    void* h = cv.take<char>(T * (int64_t)c->shared_expert_intermediate_size * (int64_t)esize(c->dtype));
    if (hs) *hs = h;
    return cv.size();
}
size_t layer_ws(const moe_config* c, int64_t T) {
    Carver cv(nullptr);
    LayerPlan p;
    plan_layer(c, T, cv, p);
    return cv.size();
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
#define TMOE_TRY(expr)                                \
    do {                                              \
        hipError_t _e = (expr);                       \
        if (_e != hipSuccess) return MOE_ERR_HIP;     \
    } while (0)

// The two passes of the grouped SwiGLU experts over a plan's tile lists, or the
// portable kernels.  g0 / g1 describe routed / shared work (g1.N == 0: none).
int run_gemm_pass(const moe_config* c, const GemmPlan& plan, int pass, const GemmGroup& g0, const GemmGroup& g1,
                  const int32_t* offsets, int64_t routed_rows, int64_t T, hipStream_t st,
                  hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
    if (plan.mfma) {
        GemmArgs a{};
        a.g[0] = g0;
        a.g[1] = g1;
        const TileSpec& ts = plan.t[pass];
        a.items = ts.items;
        a.count = ts.count;
        a.E = routed_rows > 0 ? c->num_experts : 0;
        a.n_shared_items = (g1.N > 0 && T > 0) ? (int)(((T + ts.mt - 1) / ts.mt) * (g1.N / ts.nt)) : 0;
        a.shared_first = (g1.N > 0 && routed_rows > 0 && g1.K > g0.K) ? 1 : 0;
        TMOE_TRY(launch_grouped_gemm(c->dtype, plan.variant, pass, a, plan.max_items[pass], st, ev_start, ev_stop));
        return MOE_OK;
    }
    if (ev_start) TMOE_TRY(hipEventRecord(ev_start, st));
    if (routed_rows > 0) TMOE_TRY(launch_gemm_generic(c->dtype, pass, g0, offsets, 0, c->num_experts, routed_rows, st));
    if (g1.N > 0 && T > 0) TMOE_TRY(launch_gemm_generic(c->dtype, pass, g1, nullptr, 0, 1, T, st));
    if (ev_stop) TMOE_TRY(hipEventRecord(ev_stop, st));
    return MOE_OK;
}

GemmGroup group(const void* wa, const void* wb, int64_t estride, int N, int K, const void* a, int64_t a_ld,
                const int32_t* a_rows, void* out, int64_t out_ld, const int32_t* out_rows, int mul, int add) {
    GemmGroup g{};
    g.wa = wa;
    g.wb = wb;
    g.w_estride = estride;
    g.N = N;
    g.K = K;
    g.a = a;
    g.a_ld = a_ld;
    g.a_rows = a_rows;
    g.a_div = 1;
    g.out = out;
    g.out_ld = out_ld;
    g.out_rows = out_rows;
    g.out_mul = mul;
    g.out_add = add;
    return g;
}

GemmGroup no_group() {
    GemmGroup g{};
    g.N = 0;
    return g;
}

// A plain product C [T, N] = A [T, K] W^T (W [N, K]) is the shared-expert tile
// list of the down pass alone: a layer shape whose hidden size is N and whose
// shared expert is K wide.  Up to 256 rows take the 16-row tiles.
moe_config dense_cfg(int dtype, int N, int K) {
    moe_config c{};
    c.hidden_size = N;
    c.num_experts = 1;
    c.num_experts_per_tok = 1;
    c.moe_intermediate_size = 64;
    c.shared_expert_intermediate_size = K;
    c.norm_topk_prob = 1;
    c.dtype = dtype;
    return c;
}
void plan_dense(const moe_config* c, int64_t T, Carver& cv, GemmPlan& g) { plan_gemm(c, T, false, true, cv, g, 257); }
int run_dense(const moe_config* c, const GemmPlan& plan, const void* A, const void* W, void* C, int64_t T, hipStream_t s) {
    const int N = c->hidden_size, K = c->shared_expert_intermediate_size;
    if (plan.mfma) TMOE_TRY(launch_build_items(nullptr, 0, T, &plan.t[0], &plan.t[1], s));
    const GemmGroup dn = group(W, nullptr, 0, N, K, A, K, nullptr, C, N, nullptr, 1, 0);
    return run_gemm_pass(c, plan, 1, no_group(), dn, nullptr, 0, T, s);
}

// --- decode-time attention ---
struct AttnPlan {
    moe_config cq, co;  // the two projections as plain products
    GemmPlan gq, go;
    int ksq = 0, kso = 0;  // split-K runs of the skinny products (0: the grouped GEMM path)
    float *pq = nullptr, *po = nullptr;
    void *qkv = nullptr, *q, *o, *ao = nullptr;
    float *pm, *pl, *pacc;
};
void plan_attn(const moe_attn_config* a, int64_t T, Carver& cv, AttnPlan& p) {
    const int H = a->hidden_size, nq = a->num_heads, nkv = a->num_kv_heads, d = a->head_dim;
    const int nqkv = (nq + 2 * nkv) * d;
    const int64_t parts = T * nkv * (int64_t)attn_chunks(a->max_len) * (nq / nkv);
    p.cq = dense_cfg(a->dtype, nqkv, H);
    p.co = dense_cfg(a->dtype, H, nq * d);
    p.ksq = skinny_gemm_runs(T, nqkv, H);
    p.kso = skinny_gemm_runs(T, H, nq * d);
    if (p.ksq && p.kso) {
        p.pq = cv.take<float>(p.ksq * T * (int64_t)nqkv);
        p.po = cv.take<float>(p.kso * T * (int64_t)H);
    } else {
        p.ksq = p.kso = 0;
        plan_dense(&p.cq, T, cv, p.gq);
        plan_dense(&p.co, T, cv, p.go);
        p.qkv = cv.take<char>(T * (int64_t)nqkv * 2);
        p.ao = cv.take<char>(T * (int64_t)H * 2);
    }
    p.q = cv.take<char>(T * (int64_t)nq * d * 2);
    p.o = cv.take<char>(T * (int64_t)nq * d * 2);
    p.pm = cv.take<float>(parts);
    p.pl = cv.take<float>(parts);
    p.pacc = cv.take<float>(parts * d);
}
int check_attn_cfg(const moe_attn_config* a) {
    if (!a) return MOE_ERR_INVALID;
    if (a->hidden_size < 1 || a->num_heads < 1 || a->num_kv_heads < 1 || a->head_dim < 2 || a->head_dim % 2 ||
        a->max_len < 1 || !(a->eps >= 0.0f) || !(a->rope_theta > 1.0f) || !(a->rope_theta < INFINITY))
        return MOE_ERR_INVALID;
    const int* sec = a->rope_sections;
    if (sec[0] < 0 || sec[1] < 0 || sec[2] < 0 || sec[0] + sec[1] + sec[2] != a->head_dim / 2) return MOE_ERR_INVALID;
    if (a->num_heads % a->num_kv_heads) return MOE_ERR_INVALID;
    if (a->dtype != MOE_BF16 || !attn_decode_ok(a->head_dim, a->num_heads, a->num_kv_heads, a->max_len) ||
        a->hidden_size % 128 || a->hidden_size > 16384 || a->max_len > (1 << 24))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// --- depth code predictor ---
struct PredPlan {
    moe_attn_config acfg;  // the layers' attention over the frame's positions
    AttnPlan ap;
    int ksd = 0;
    float *pd, *sc, *bd;
    void *h, *X, *Hh, *XN, *HN;
    char *kc, *vc;
    size_t cache_bytes;  // per layer, each of K and V
    int32_t *pos, *len;
};
moe_attn_config pred_attn_cfg(const moe_predictor_config* c) {
    moe_attn_config a = c->attn;
    a.max_len = (c->num_codes + 31) / 32 * 32;
    return a;
}
// Every weight pointer of the predictor present and 16-byte aligned.
bool pred_weights_ok(const moe_predictor_config* c, const moe_predictor_weights* w) {
    if (!w || !w->layers || !ok_ptr(w->final_norm) || !ok_ptr(w->c0_embedding) || !ok_ptr(w->codec_embedding) ||
        !ok_ptr(w->lm_head))
        return false;
    for (int l = 0; l < c->num_layers; ++l) {
        const moe_predictor_layer& L = w->layers[l];
        if (!ok_ptr(L.attn.w_qkv) || !ok_ptr(L.attn.q_norm) || !ok_ptr(L.attn.k_norm) || !ok_ptr(L.attn.w_o) ||
            !ok_ptr(L.in_norm) || !ok_ptr(L.post_norm) || !ok_ptr(L.gate) || !ok_ptr(L.up) || !ok_ptr(L.down))
            return false;
    }
    return true;
}

int check_pred_cfg(const moe_predictor_config* c, int64_t T) {
    if (!c) return MOE_ERR_INVALID;
    const moe_attn_config a = pred_attn_cfg(c);
    if (c->num_layers < 1 || c->num_codes < 2 || c->codebook_size < 1 || c->c0_vocab < 1 || c->intermediate_size < 1 ||
        !(c->eps >= 0.0f))
        return MOE_ERR_INVALID;
    int st = check_attn_cfg(&a);
    if (st != MOE_OK) return st;
    const int H = a.hidden_size, I = c->intermediate_size;
    if (c->num_layers > 256 || c->num_codes > 256 || c->codebook_size > (1 << 20) || I % 16) return MOE_ERR_UNSUPPORTED;
    if (T < 1 || T > 64 || !skinny_swiglu_ok(T, I, H) || !skinny_gemm_runs(T, H, I) ||
        !skinny_gemm_runs(T, (a.num_heads + 2 * a.num_kv_heads) * a.head_dim, H) ||
        !skinny_gemm_runs(T, H, a.num_heads * a.head_dim))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}
void plan_pred(const moe_predictor_config* c, int64_t T, Carver& cv, PredPlan& p) {
    p.acfg = pred_attn_cfg(c);
    const int H = p.acfg.hidden_size, I = c->intermediate_size, K = c->codebook_size, P = c->num_codes;
    plan_attn(&p.acfg, T, cv, p.ap);
    p.ksd = skinny_gemm_runs(T, H, I);
    p.pd = cv.take<float>((int64_t)p.ksd * T * H);
    p.h = cv.take<char>(T * (int64_t)I * 2);
    p.X = cv.take<char>(T * (int64_t)H * 2);
    p.Hh = cv.take<char>(T * (int64_t)H * 2);
    p.XN = cv.take<char>(T * (int64_t)H * 2);
    p.HN = cv.take<char>(T * (int64_t)H * 2);
    p.cache_bytes = (size_t)T * p.acfg.num_kv_heads * p.acfg.max_len * p.acfg.head_dim * 2;
    p.kc = cv.take<char>((int64_t)p.cache_bytes * c->num_layers);
    p.vc = cv.take<char>((int64_t)p.cache_bytes * c->num_layers);
    p.pos = cv.take<int32_t>((int64_t)P * T * 3);
    p.len = cv.take<int32_t>((int64_t)P * T);
    p.sc = cv.take<float>(T * (int64_t)K);
    p.bd = cv.take<float>(T * (int64_t)K);
}

// One attention step with a prepared plan (arguments already checked).
int attn_run(const moe_attn_config* cfg, const moe_attn_weights* w, const AttnPlan& p, const void* x, int64_t T,
             const int32_t* pos, const int32_t* cache_len, void* k_cache, void* v_cache, const void* residual,
             void* y, const float* norm_gain, float norm_eps, void* norm_out, hipStream_t s) {
    const int H = cfg->hidden_size, nq = cfg->num_heads, nkv = cfg->num_kv_heads;
    const int d = cfg->head_dim, nqkv = (nq + 2 * nkv) * d;
    if (p.ksq) {
        TMOE_TRY(launch_skinny_gemm(x, w->w_qkv, p.pq, T, nqkv, H, p.ksq, s));
    } else {
        const int r = run_dense(&p.cq, p.gq, x, w->w_qkv, p.qkv, T, s);
        if (r != MOE_OK) return r;
    }
    const float* qkv_rows = p.ksq ? p.pq : reinterpret_cast<const float*>(p.qkv);
    if (attn_rope_fused_ok(nq, nkv, cfg->max_len)) {
        // q / k norms, rotation and the cache append inside the attention launch
        TMOE_TRY(launch_attn_rope_decode(qkv_rows, p.ksq, T, nq, nkv, w->q_norm, w->k_norm, cfg->eps, pos, cache_len,
                                         cfg->max_len, cfg->rope_sections[1], cfg->rope_sections[2],
                                         (double)cfg->rope_theta, k_cache, v_cache, p.pm, p.pl, p.pacc, p.o, s));
    } else {
        TMOE_TRY(launch_qk_rope_append(qkv_rows, p.ksq, T, nq, nkv, w->q_norm, w->k_norm, cfg->eps, pos, cache_len,
                                       cfg->max_len, cfg->rope_sections[1], cfg->rope_sections[2],
                                       (double)cfg->rope_theta, p.q, k_cache, v_cache, s));
        TMOE_TRY(launch_attn_decode(p.q, k_cache, v_cache, cache_len, T, nq, nkv, cfg->max_len, p.pm, p.pl, p.pacc,
                                    p.o, s));
    }
    if (p.kso) {
        TMOE_TRY(launch_skinny_gemm(p.o, w->w_o, p.po, T, H, nq * d, p.kso, s));
        return hip_status(launch_attn_out(p.po, p.kso, residual, y, T, H, norm_gain, norm_eps, norm_out, s));
    }
    if (!residual && !norm_out) return run_dense(&p.co, p.go, p.o, w->w_o, y, T, s);
    const int r = run_dense(&p.co, p.go, p.o, w->w_o, p.ao, T, s);
    if (r != MOE_OK) return r;
    if (norm_out)
        return hip_status(launch_combine_norm(cfg->dtype, nullptr, nullptr, 0, 0, p.ao, H, residual, y, T, H,
                                              norm_gain, norm_eps, norm_out, s));
    return hip_status(launch_combine(cfg->dtype, nullptr, nullptr, nullptr, 0, 0, p.ao, H, residual, y, T, H, s));
}


// Optional end of a stacked layer: the next pre-norm of y, fused into the combine.
struct LayerEnd {
    const float* gain = nullptr;  // nullable: 1.0
    float eps = 0.f;
    void* norm_out = nullptr;     // null: plain combine
};

// The layer's combine: slot j < k of token t (an unweighted expert output) times
// w[t * k + j], the shared slot, the residual; then the next pre-norm when
// end.norm_out is set.
hipError_t finish_layer(int dtype, const void* ybuf, const float* w, int k, int slots, const void* shared,
                        int64_t sstride, const void* residual, void* y, int64_t T, int H, const LayerEnd& end,
                        hipStream_t s) {
    if (end.norm_out)
        return launch_combine_norm(dtype, ybuf, w, k, slots, shared, sstride, residual, y, T, H, end.gain, end.eps,
                                   end.norm_out, s);
    return launch_combine(dtype, ybuf, nullptr, w, k, slots, shared, sstride, residual, y, T, H, s);
}

// ws: the caller's workspace, or nullptr for the static scratch (not checked here)
int check_layer_args(const moe_config* cfg, const moe_weights* w, const void* x, const void* residual,
                     const void* y, const void* ws, bool static_scratch = false) {
    if (!w) return MOE_ERR_INVALID;
    const int Is = cfg->shared_expert_intermediate_size;
    if (!ok_ptr(x) || !ok_ptr(y) || !ok_opt(residual) || !ok_ptr(w->router) || !ok_opt(w->router_bias) ||
        !ok_ptr(w->gate) || !ok_ptr(w->up) || !ok_ptr(w->down) || (!static_scratch && !ok_ptr(ws)))
        return MOE_ERR_INVALID;
    if (Is > 0 && (!ok_ptr(w->shared_gate) || !ok_ptr(w->shared_up) || !ok_ptr(w->shared_down)))
        return MOE_ERR_INVALID;
    if (x == y) return MOE_ERR_INVALID;
    return MOE_OK;
}

// One layer on stream s (arguments already checked).
int layer_run(const moe_config* cfg, const moe_weights* w, const void* x, const void* residual, int64_t T, void* y,
              int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* ws, hipStream_t s,
              void* const* stage_events, const LayerEnd& end) {
    const int H = cfg->hidden_size, E = cfg->num_experts, k = cfg->num_experts_per_tok;
    const int I = cfg->moe_intermediate_size, Is = cfg->shared_expert_intermediate_size;
    const int64_t N = T * k;
    Carver cv(ws);
    LayerPlan p;
    plan_layer(cfg, T, cv, p);
    int32_t* idx = topk_idx_out ? topk_idx_out : p.idx;
    float* wt = topk_w_out ? topk_w_out : p.w;
    int32_t* counts = counts_out ? counts_out : p.counts;
    auto mark = [&](int i) -> hipError_t {
        return (stage_events && stage_events[i]) ? hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s)
                                                 : hipSuccess;
    };

    const int slots = k + 1;  // per token: k unweighted expert rows (the combine applies w), then the shared row
    const TileSpec* t1 = p.gemm.mfma ? &p.gemm.t[0] : nullptr;
    const TileSpec* t2 = p.gemm.mfma ? &p.gemm.t[1] : nullptr;
    TMOE_TRY(mark(0));
    auto ev = [&](int i) { return stage_events ? static_cast<hipEvent_t>(stage_events[i]) : nullptr; };
    if (p.decode) {
        // scores -> selection (beside it, the shared gate/up) -> every expert
        // slice and the shared down tiles in one launch -> the partial rows
        // summed per token with the routing weights
        TMOE_TRY(launch_route_decode(x, w->router, w->router_bias, T, H, E, k, cfg->norm_topk_prob, p.sc, p.dv, idx,
                                     wt, Is > 0 ? w->shared_gate : nullptr, Is > 0 ? w->shared_up : nullptr, Is, p.hs,
                                     p.mask, counts, s));
        TMOE_TRY(mark(1));
        TMOE_TRY(mark(2));
        TMOE_TRY(launch_decode_experts(x, idx, p.mask, w->gate, w->up, w->down, p.hs,
                                       Is > 0 ? w->shared_down : nullptr, p.part, T, H, E, k, I, Is, s, ev(6), ev(7)));
        TMOE_TRY(mark(3));
        TMOE_TRY(mark(4));
        TMOE_TRY(launch_combine_partials(p.part, I / 64, Is > 0 ? 1 : 0, k, wt, residual, y, T, H, end.gain, end.eps,
                                         end.norm_out, s));
        TMOE_TRY(mark(5));
        return MOE_OK;
    }
    if (p.direct) {
        // With at most 64 tokens the shared expert's gate/up runs in the router's
        // launch, on the CUs the router leaves idle; the gate/up pass then holds
        // the routed tiles alone.
        const bool shared_early = Is > 0 && route_shared_ok(T, H, Is);
        if (shared_early)
            TMOE_TRY(launch_route_block_shared(x, w->router, w->router_bias, T, H, E, k, cfg->norm_topk_prob, idx, wt,
                                               p.bcnt, p.blist, w->shared_gate, w->shared_up, Is, p.hs, s));
        else
            TMOE_TRY(launch_route_block(x, w->router, w->router_bias, T, H, E, k, cfg->norm_topk_prob, idx, wt,
                                        nullptr, nullptr, nullptr, p.bcnt, p.blist, s));
        TMOE_TRY(mark(1));
        TMOE_TRY(mark(2));
        int bm;
        GemmArgs a{};
        a.E = E;
        a.direct_bcnt = p.bcnt;
        a.direct_blist = p.blist;
        a.direct_nb = (int)nb_of(T);
        a.direct_counts = counts;
        a.direct_T = (int)T;
        a.g[0] = group(w->gate, w->up, (int64_t)I * H, I, H, x, H, nullptr, p.hd, I, nullptr, 1, 0);
        a.g[0].a_div = k;
        a.g[1] = Is > 0 && !shared_early
                     ? group(w->shared_gate, w->shared_up, 0, Is, H, x, H, nullptr, p.hs, Is, nullptr, 1, 0)
                     : no_group();
        int bn = gemm_direct_tile(0, &bm);
        a.direct_nt[0] = I / bn;
        a.direct_nt[1] = shared_early ? 0 : Is / bn;
        a.direct_mt1 = (int)((T + bm - 1) / bm);
        TMOE_TRY(launch_grouped_gemm_direct(0, a, s, ev(6), ev(7)));
        TMOE_TRY(mark(3));
        a.direct_counts = nullptr;  // written by the gate/up pass
        a.g[0] = group(w->down, nullptr, (int64_t)H * I, H, I, p.hd, I, nullptr, p.ybuf, H, nullptr, 1, 0);
        a.g[0].out_div = k;
        a.g[1] = Is > 0 ? group(w->shared_down, nullptr, 0, H, Is, p.hs, Is, nullptr, p.ybuf, H, nullptr, slots, k)
                        : no_group();
        bn = gemm_direct_tile(1, &bm);
        a.direct_nt[0] = H / bn;
        a.direct_nt[1] = Is > 0 ? H / bn : 0;
        TMOE_TRY(launch_grouped_gemm_direct(1, a, s));
        TMOE_TRY(mark(4));
        const char* sb = Is > 0 ? static_cast<const char*>(p.ybuf) + (int64_t)k * H * esize(cfg->dtype) : nullptr;
        TMOE_TRY(finish_layer(cfg->dtype, p.ybuf, wt, k, slots, sb, (int64_t)slots * H, residual, y, T, H, end, s));
        TMOE_TRY(mark(5));
        return MOE_OK;
    }
    if (!route_block_ok(cfg->dtype, H, E, k) && route_group_small_ok(cfg->dtype, T, H, E, k)) {
        // scores over many CUs, then selection and grouping in one block
        TMOE_TRY(launch_scores(cfg->dtype, x, w->router, w->router_bias, T, H, E, p.route.sc, p.route.bd, s));
        TMOE_TRY(mark(1));
        TMOE_TRY(launch_select_group_small(p.route.sc, p.route.bd, x, w->router, w->router_bias, T, H, E, k,
                                           cfg->norm_topk_prob, idx, wt, counts, p.offsets, p.row_token, p.row_of,
                                           p.row_pair, t1, t2, s));
    } else {
        // choice slots come with the masks only from the one-launch router
        uint64_t* jm = route_block_ok(cfg->dtype, H, E, k) ? p.jmask : nullptr;
        TMOE_TRY(launch_route(cfg->dtype, x, w->router, w->router_bias, T, H, E, k, cfg->norm_topk_prob, idx, wt,
                              nullptr, p.route.sc, p.route.bd, p.masks, jm, s));
        TMOE_TRY(mark(1));
        if (group_small_ok(T, E))
            TMOE_TRY(launch_group_small(idx, p.masks, T, E, k, counts, p.offsets, p.row_token, p.row_of, p.row_pair,
                                        t1, t2, s));
        else
            TMOE_TRY(launch_permute(idx, T, k, E, p.masks, jm, p.prefix, counts, p.offsets, p.row_token,
                                    p.row_of, p.row_pair, t1, t2, s));
    }
    TMOE_TRY(mark(2));

    GemmGroup gu_r = group(w->gate, w->up, (int64_t)I * H, I, H, x, H, p.row_token, p.hr, I, nullptr, 1, 0);
    GemmGroup gu_s = Is > 0 ? group(w->shared_gate, w->shared_up, 0, Is, H, x, H, nullptr, p.hs, Is, nullptr, 1, 0)
                            : no_group();
    int r = run_gemm_pass(cfg, p.gemm, 0, gu_r, gu_s, p.offsets, N, T, s, ev(6), ev(7));
    if (r != MOE_OK) return r;
    TMOE_TRY(mark(3));
    // row_pair v = t * k + j goes to slot j of token t: row v + v / k of [T, k + 1, H]; the combine weights it
    GemmGroup dn_r = group(w->down, nullptr, (int64_t)H * I, H, I, p.hr, I, nullptr, p.ybuf, H, p.row_pair, 1, 0);
    dn_r.out_div = k;
    GemmGroup dn_s = Is > 0 ? group(w->shared_down, nullptr, 0, H, Is, p.hs, Is, nullptr, p.ybuf, H, nullptr, slots, k)
                            : no_group();
    r = run_gemm_pass(cfg, p.gemm, 1, dn_r, dn_s, p.offsets, N, T, s);
    if (r != MOE_OK) return r;
    TMOE_TRY(mark(4));
    const char* shared_base = Is > 0 ? static_cast<const char*>(p.ybuf) + (int64_t)k * H * esize(cfg->dtype) : nullptr;
    TMOE_TRY(finish_layer(cfg->dtype, p.ybuf, wt, k, slots, shared_base, (int64_t)slots * H, residual, y, T, H, end,
                          s));
    TMOE_TRY(mark(5));
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_SCRATCH: return "the call needs more than the static scratch";
        default: return "unknown status";
    }
}

int moe_check_config(const moe_config* cfg) { return check_cfg(cfg); }

size_t moe_workspace_size(const moe_config* cfg, int64_t T) {
    if (check_cfg(cfg) != MOE_OK || check_T(cfg, T) != MOE_OK) return 0;
    size_t s = layer_ws(cfg, T);
    s = s > route_ws(cfg, T) ? s : route_ws(cfg, T);
    s = s > permute_ws(cfg, T) ? s : permute_ws(cfg, T);
    size_t g = grouped_ws(cfg, T, nullptr, nullptr, nullptr);
    s = s > g ? s : g;
    if (cfg->shared_expert_intermediate_size > 0) {
        size_t h = shared_ws(cfg, T, nullptr, nullptr, nullptr);
        s = s > h ? s : h;
    }
    return s < 256 ? 256 : s;
}

int moe_route(const moe_config* cfg, const void* x, const void* router, const float* bias, int64_t T,
              int32_t* topk_idx, float* topk_w, float* probs, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(router) || !ok_ptr(topk_idx) || !ok_ptr(topk_w) || !ok_opt(bias) || !ok_opt(probs) ||
        !ok_opt(ws))
        return MOE_ERR_INVALID;
    if (ws_bytes < route_ws(cfg, T) || (route_ws(cfg, T) > 0 && !ws)) return MOE_ERR_WORKSPACE;
    Carver cv(ws);
    RoutePlan p;
    plan_route(cfg, T, cv, p);
    return hip_status(launch_route(cfg->dtype, x, router, bias, T, cfg->hidden_size, cfg->num_experts,
                                   cfg->num_experts_per_tok, cfg->norm_topk_prob, topk_idx, topk_w, probs, p.sc, p.bd,
                                   nullptr, nullptr, as_stream(stream)));
}

int moe_permute(const moe_config* cfg, const int32_t* topk_idx, int64_t T, int32_t* counts, int32_t* offsets,
                int32_t* row_token, int32_t* row_of, const void* x, void* x_perm, void* ws, size_t ws_bytes,
                void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    const int E = cfg->num_experts, k = cfg->num_experts_per_tok;
    hipStream_t s = as_stream(stream);
    if (!ok_ptr(counts) || !ok_ptr(offsets)) return MOE_ERR_INVALID;
    if (T == 0) {
        // an empty routing still has well-defined counts and offsets
        TMOE_TRY(launch_fill_i32(counts, 0, E, s));
        TMOE_TRY(launch_fill_i32(offsets, 0, E + 1, s));
        return MOE_OK;
    }
    if (!ok_ptr(topk_idx) || !ok_ptr(row_token) || !ok_ptr(row_of) || !ok_opt(x) || !ok_opt(x_perm) || !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID;
    if (ws_bytes < permute_ws(cfg, T)) return MOE_ERR_WORKSPACE;
    Carver cv(ws);
    uint16_t* masks = cv.take<uint16_t>((int64_t)E * mask_stride(T));
    uint64_t* jmask = cv.take<uint64_t>((int64_t)E * mask_stride(T));
    int32_t* prefix = cv.take<int32_t>((int64_t)E * mask_stride(T));
    TMOE_TRY(launch_masks(topk_idx, T, k, E, masks, jmask, s));
    TMOE_TRY(launch_permute(topk_idx, T, k, E, masks, jmask, prefix, counts, offsets, row_token, row_of, nullptr,
                            nullptr, nullptr, s));
    if (x) TMOE_TRY(launch_gather_rows(cfg->dtype, x, row_token, T * k, cfg->hidden_size, x_perm, s));
    return MOE_OK;
}

int moe_grouped_swiglu(const moe_config* cfg, const void* x, const int32_t* row_token, const int32_t* offsets,
                       int64_t T, const void* gate, const void* up, const void* down, void* y_perm, void* ws,
                       size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_opt(row_token) || !ok_ptr(offsets) || !ok_ptr(gate) || !ok_ptr(up) || !ok_ptr(down) ||
        !ok_ptr(y_perm) || !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (ws_bytes < grouped_ws(cfg, T, nullptr, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
    const int H = cfg->hidden_size, I = cfg->moe_intermediate_size, E = cfg->num_experts;
    const int64_t N = T * cfg->num_experts_per_tok;
    GemmPlan plan;
    void* hr = nullptr;
    grouped_ws(cfg, T, ws, &plan, &hr);
    hipStream_t s = as_stream(stream);
    if (plan.mfma) TMOE_TRY(launch_build_items(offsets, E, T, &plan.t[0], &plan.t[1], s));
    GemmGroup gu = group(gate, up, (int64_t)I * H, I, H, x, H, row_token, hr, I, nullptr, 1, 0);
    int r = run_gemm_pass(cfg, plan, 0, gu, no_group(), offsets, N, 0, s);
    if (r != MOE_OK) return r;
    GemmGroup dn = group(down, nullptr, (int64_t)H * I, H, I, hr, I, nullptr, y_perm, H, nullptr, 1, 0);
    return run_gemm_pass(cfg, plan, 1, dn, no_group(), offsets, N, 0, s);
}

int moe_shared_swiglu(const moe_config* cfg, const void* x, int64_t T, const void* sg, const void* su,
                      const void* sd, void* y_shared, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    const int Is = cfg->shared_expert_intermediate_size;
    if (Is == 0) return MOE_ERR_INVALID;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(sg) || !ok_ptr(su) || !ok_ptr(sd) || !ok_ptr(y_shared) || !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (ws_bytes < shared_ws(cfg, T, nullptr, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
    const int H = cfg->hidden_size;
    GemmPlan plan;
    void* hs = nullptr;
    shared_ws(cfg, T, ws, &plan, &hs);
    hipStream_t s = as_stream(stream);
    if (plan.mfma) TMOE_TRY(launch_build_items(nullptr, 0, T, &plan.t[0], &plan.t[1], s));
    GemmGroup gu = group(sg, su, 0, Is, H, x, H, nullptr, hs, Is, nullptr, 1, 0);
    int r = run_gemm_pass(cfg, plan, 0, no_group(), gu, nullptr, 0, T, s);
    if (r != MOE_OK) return r;
    GemmGroup dn = group(sd, nullptr, 0, H, Is, hs, Is, nullptr, y_shared, H, nullptr, 1, 0);
    return run_gemm_pass(cfg, plan, 1, no_group(), dn, nullptr, 0, T, s);
}

int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of, const float* topk_w,
                const void* y_shared, const void* residual, int64_t T, void* y, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(y_perm) || !ok_ptr(row_of) || !ok_ptr(topk_w) || !ok_opt(y_shared) || !ok_opt(residual) ||
        !ok_ptr(y))
        return MOE_ERR_INVALID;
    return hip_status(launch_combine(cfg->dtype, y_perm, row_of, topk_w, cfg->num_experts_per_tok, 0, y_shared,
                                     cfg->hidden_size, residual, y, T, cfg->hidden_size, as_stream(stream)));
}

int moe_layer_forward(const moe_config* cfg, const moe_weights* w, const void* x, const void* residual, int64_t T,
                      void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* ws,
                      size_t ws_bytes, void* stream) {
    return moe_layer_forward_timed(cfg, w, x, residual, T, y, topk_idx_out, topk_w_out, counts_out, ws, ws_bytes,
                                   stream, nullptr);
}

int moe_layer_forward_timed(const moe_config* cfg, const moe_weights* w, const void* x, const void* residual,
                            int64_t T, void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                            void* ws, size_t ws_bytes, void* stream, void* const* stage_events) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if ((st = check_layer_args(cfg, w, x, residual, y, ws)) != MOE_OK) return st;
    if (!ok_opt(topk_idx_out) || !ok_opt(topk_w_out) || !ok_opt(counts_out)) return MOE_ERR_INVALID;
    if (ws_bytes < layer_ws(cfg, T)) return MOE_ERR_WORKSPACE;
    return layer_run(cfg, w, x, residual, T, y, topk_idx_out, topk_w_out, counts_out, ws, as_stream(stream),
                     stage_events, LayerEnd{});
}

}  // extern "C"

namespace {
// Scratch of moe_layer_forward_static: one array per GPU, for callers that
// cannot allocate.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

extern "C" {

int moe_layer_forward_static(const moe_config* cfg, const moe_weights* w, const void* x, const void* residual,
                             int64_t T, void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                             void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if ((st = check_layer_args(cfg, w, x, residual, y, nullptr, true)) != MOE_OK) return st;
    if (!ok_opt(topk_idx_out) || !ok_opt(topk_w_out) || !ok_opt(counts_out)) return MOE_ERR_INVALID;
    if (layer_ws(cfg, T) > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    void* ws = nullptr;
    if ((st = static_scratch(&ws)) != MOE_OK) return st;
    return layer_run(cfg, w, x, residual, T, y, topk_idx_out, topk_w_out, counts_out, ws, as_stream(stream), nullptr,
                     LayerEnd{});
}

size_t moe_stack_workspace_size(const moe_config* cfg, int64_t T, int32_t V) {
    if (check_cfg(cfg) != MOE_OK || check_T(cfg, T) != MOE_OK || V < 0) return 0;
    Carver cv(nullptr);
    cv.take<char>(T * cfg->hidden_size * (int64_t)esize(cfg->dtype));  // the normalised layer input
    cv.take<char>(layer_ws(cfg, T));
    if (V > 0) cv.take<char>(moe_codec_head_workspace_size(cfg, V, T));
    return cv.size();
}

int moe_stack_forward(const moe_config* cfg, const moe_weights* layers, int32_t L, const void* x, int64_t T,
                      const float* gains, float eps, const void* codec_head, int32_t V, void* h_out, void* xn_out,
                      int32_t* c0, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if (L < 1 || L > kMaxStackLayers || !layers || !(eps >= 0.0f) || V < 0) return MOE_ERR_INVALID;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(h_out) || !ok_opt(xn_out) || !ok_opt(gains) || !ok_opt(codec_head) || !ok_opt(c0) ||
        !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (c0 && (!codec_head || V < 1)) return MOE_ERR_INVALID;
    if (V > (1 << 20)) return MOE_ERR_UNSUPPORTED;
    if (xn_out && (xn_out == x || xn_out == h_out)) return MOE_ERR_INVALID;
    if (ws_bytes < moe_stack_workspace_size(cfg, T, c0 ? V : 0)) return MOE_ERR_WORKSPACE;
    const int H = cfg->hidden_size;
    Carver cv(ws);
    void* xn_ws = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));
    void* lws = cv.take<char>(layer_ws(cfg, T));
    void* hws = c0 ? cv.take<char>(moe_codec_head_workspace_size(cfg, V, T)) : nullptr;
    void* xn = xn_out ? xn_out : xn_ws;
    for (int l = 0; l < L; ++l)
        if ((st = check_layer_args(cfg, &layers[l], xn, l == 0 ? x : h_out, h_out, lws)) != MOE_OK) return st;

    hipStream_t s = as_stream(stream);
    TMOE_TRY(launch_rmsnorm(cfg->dtype, x, gains, eps, T, H, xn, s));
    for (int l = 0; l < L; ++l) {
        LayerEnd end;
        end.gain = gains ? gains + (int64_t)(l + 1) * H : nullptr;
        end.eps = eps;
        end.norm_out = xn;
        const int r = layer_run(cfg, &layers[l], xn, l == 0 ? x : h_out, T, h_out, nullptr, nullptr, nullptr, lws,
                                s, nullptr, end);
        if (r != MOE_OK) return r;
    }
    if (!c0) return MOE_OK;
    return moe_codec_head_argmax(cfg, xn, codec_head, V, T, nullptr, c0, hws,
                                 moe_codec_head_workspace_size(cfg, V, T), stream);
}

size_t moe_talker_decode_workspace_size(const moe_config* cfg, const moe_attn_config* acfg, int64_t T, int32_t V) {
    if (check_cfg(cfg) != MOE_OK || check_T(cfg, T) != MOE_OK || check_attn_cfg(acfg) != MOE_OK || V < 0 ||
        T > 65535 || acfg->hidden_size != cfg->hidden_size || acfg->dtype != cfg->dtype)
        return 0;
    const int H = cfg->hidden_size;
    Carver cv(nullptr);
    for (int i = 0; i < 3; ++i) cv.take<char>(T * H * (int64_t)esize(cfg->dtype));
    AttnPlan ap;
    plan_attn(acfg, T, cv, ap);
    cv.take<char>(layer_ws(cfg, T));
    if (V > 0) cv.take<char>(moe_codec_head_workspace_size(cfg, V, T));
    return cv.size();
}

}  // extern "C"

namespace {
// The Talker decode step; with x_add the input is x + x_add (rounded to bf16,
// stored in xsum and used as layer 0's residual).
int talker_run(const moe_config* cfg, const moe_attn_config* acfg, const moe_talker_layer* layers, int32_t L,
               const void* x, const void* x_add, void* xsum, int64_t T, const int32_t* pos, const int32_t* cache_len,
               const float* final_norm, float eps, const void* codec_head, int32_t V, void* h_out, void* xn_out,
               int32_t* c0, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_T(cfg, T)) != MOE_OK) return st;
    if ((st = check_attn_cfg(acfg)) != MOE_OK) return st;
    if (acfg->hidden_size != cfg->hidden_size || acfg->dtype != cfg->dtype) return MOE_ERR_INVALID;
    if (L < 1 || L > kMaxStackLayers || !layers || !(eps >= 0.0f) || V < 0) return MOE_ERR_INVALID;
    if (T > 65535 || V > (1 << 20)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(pos) || !ok_ptr(cache_len) || !ok_ptr(h_out) || !ok_opt(xn_out) || !ok_opt(final_norm) ||
        !ok_opt(codec_head) || !ok_opt(c0) || !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (c0 && (!codec_head || V < 1)) return MOE_ERR_INVALID;
    if (xn_out && (xn_out == x || xn_out == h_out)) return MOE_ERR_INVALID;
    if (ws_bytes < moe_talker_decode_workspace_size(cfg, acfg, T, c0 ? V : 0)) return MOE_ERR_WORKSPACE;
    const int H = cfg->hidden_size;
    Carver cv(ws);
    void* xa = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));    // attention input (normalised)
    void* hmid = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));  // after the attention's residual add
    void* xm = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));    // MoE input (normalised)
    AttnPlan ap;
    plan_attn(acfg, T, cv, ap);
    void* lws = cv.take<char>(layer_ws(cfg, T));
    void* hws = c0 ? cv.take<char>(moe_codec_head_workspace_size(cfg, V, T)) : nullptr;
    void* xf = xn_out ? xn_out : xa;
    for (int l = 0; l < L; ++l) {
        const moe_talker_layer& ly = layers[l];
        if ((st = check_layer_args(cfg, &ly.moe, xm, hmid, h_out, lws)) != MOE_OK) return st;
        if (!ok_ptr(ly.attn.w_qkv) || !ok_ptr(ly.attn.q_norm) || !ok_ptr(ly.attn.k_norm) || !ok_ptr(ly.attn.w_o) ||
            !ok_opt(ly.in_norm) || !ok_opt(ly.post_norm) || !ok_ptr(ly.k_cache) || !ok_ptr(ly.v_cache))
            return MOE_ERR_INVALID;
    }
    hipStream_t s = as_stream(stream);
    if (x_add) {
        TMOE_TRY(launch_add_rmsnorm(x, x_add, xsum, layers[0].in_norm, eps, T, H, xa, s));
        x = xsum;
    } else {
        TMOE_TRY(launch_rmsnorm(cfg->dtype, x, layers[0].in_norm, eps, T, H, xa, s));
    }
    for (int l = 0; l < L; ++l) {
        const moe_talker_layer& ly = layers[l];
        int r = attn_run(acfg, &ly.attn, ap, xa, T, pos, cache_len, ly.k_cache, ly.v_cache, l == 0 ? x : h_out, hmid,
                         ly.post_norm, eps, xm, s);
        if (r != MOE_OK) return r;
        LayerEnd end;
        end.gain = l + 1 < L ? layers[l + 1].in_norm : final_norm;
        end.eps = eps;
        end.norm_out = l + 1 < L ? xa : xf;
        r = layer_run(cfg, &ly.moe, xm, hmid, T, h_out, nullptr, nullptr, nullptr, lws, s, nullptr, end);
        if (r != MOE_OK) return r;
    }
    if (!c0) return MOE_OK;
    return moe_codec_head_argmax(cfg, xf, codec_head, V, T, nullptr, c0, hws, moe_codec_head_workspace_size(cfg, V, T),
                                 stream);
}
}  // namespace

extern "C" {

int moe_talker_decode(const moe_config* cfg, const moe_attn_config* acfg, const moe_talker_layer* layers, int32_t L,
                      const void* x, int64_t T, const int32_t* pos, const int32_t* cache_len, const float* final_norm,
                      float eps, const void* codec_head, int32_t V, void* h_out, void* xn_out, int32_t* c0, void* ws,
                      size_t ws_bytes, void* stream) {
    return talker_run(cfg, acfg, layers, L, x, nullptr, nullptr, T, pos, cache_len, final_norm, eps, codec_head, V,
                      h_out, xn_out, c0, ws, ws_bytes, stream);
}

size_t moe_talker_frame_workspace_size(const moe_config* cfg, const moe_attn_config* acfg,
                                       const moe_predictor_config* pcfg, int64_t T, int32_t V) {
    if (!pcfg || check_pred_cfg(pcfg, T) != MOE_OK || V < 1 || T < 1) return 0;
    const size_t td = moe_talker_decode_workspace_size(cfg, acfg, T, V);
    const size_t pd = moe_predictor_workspace_size(pcfg, T);
    if (td == 0 || pd == 0) return 0;
    const int H = cfg->hidden_size;
    Carver cv(nullptr);
    for (int i = 0; i < 3; ++i) cv.take<char>(T * H * (int64_t)esize(cfg->dtype));  // x, h, xn
    cv.take<int32_t>(T);                                                            // c_0
    cv.take<char>((int64_t)td);
    cv.take<char>((int64_t)pd);
    return cv.size();
}

int moe_talker_frame(const moe_config* cfg, const moe_attn_config* acfg, const moe_talker_layer* layers, int32_t L,
                     const float* final_norm, float eps, const void* codec_head, int32_t V,
                     const moe_predictor_config* pcfg, const moe_predictor_weights* pw, const void* cond, int64_t T,
                     void* prev_emb, int32_t* pos, int32_t* cache_len, int32_t* codes, void* h_out, void* xn_out,
                     void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if (!pcfg || !pw) return MOE_ERR_INVALID;
    if (T == 0) return MOE_OK;
    if ((st = check_pred_cfg(pcfg, T)) != MOE_OK) return st;
    if (cfg->dtype != MOE_BF16 || pcfg->attn.hidden_size != cfg->hidden_size) return MOE_ERR_UNSUPPORTED;
    // everything the predictor and the frame's end read is checked here, before
    // the Talker step is enqueued (the Talker step checks its own layers first)
    if (!codec_head || V < 1 || !ok_ptr(cond) || !ok_ptr(prev_emb) || !ok_ptr(pos) || !ok_ptr(cache_len) ||
        !ok_ptr(codes) || !ok_opt(h_out) || !ok_opt(xn_out) || !ok_ptr(ws) || !pred_weights_ok(pcfg, pw))
        return MOE_ERR_INVALID;
    if (h_out && xn_out && h_out == xn_out) return MOE_ERR_INVALID;
    const size_t need = moe_talker_frame_workspace_size(cfg, acfg, pcfg, T, V);
    if (need == 0) return MOE_ERR_INVALID;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    const int H = cfg->hidden_size;
    const size_t td = moe_talker_decode_workspace_size(cfg, acfg, T, V);
    const size_t pd = moe_predictor_workspace_size(pcfg, T);
    Carver cv(ws);
    void* x = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));
    void* h = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));
    void* xn = cv.take<char>(T * H * (int64_t)esize(cfg->dtype));
    int32_t* c0 = cv.take<int32_t>(T);
    void* tws = cv.take<char>((int64_t)td);
    void* pws = cv.take<char>((int64_t)pd);
    if (h_out) h = h_out;
    if (xn_out) xn = xn_out;
    // the Talker step on prev_emb + cond, then the predictor's frame on its
    // final-normed state and c_0, then the next frame's input and positions
    if ((st = talker_run(cfg, acfg, layers, L, prev_emb, cond, x, T, pos, cache_len, final_norm, eps, codec_head, V, h,
                         xn, c0, tws, td, stream)) != MOE_OK)
        return st;
    if ((st = moe_predictor_frame(pcfg, pw, xn, c0, T, codes, nullptr, pws, pd, stream)) != MOE_OK) return st;
    return hip_status(launch_frame_advance(codes, pcfg->num_codes, pw->c0_embedding, pcfg->c0_vocab,
                                           pw->codec_embedding, pcfg->codebook_size, T, H, prev_emb, pos, cache_len,
                                           as_stream(stream)));
}

int moe_rmsnorm(const moe_config* cfg, const void* x, const float* gain, float eps, int64_t T, void* out,
                void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if (T < 0 || !(eps >= 0.0f)) return MOE_ERR_INVALID;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(gain) || !ok_ptr(out)) return MOE_ERR_INVALID;
    return hip_status(launch_rmsnorm(cfg->dtype, x, gain, eps, T, cfg->hidden_size, out, as_stream(stream)));
}

size_t moe_codec_head_workspace_size(const moe_config* cfg, int32_t V, int64_t T) {
    if (check_cfg(cfg) != MOE_OK || V < 1 || T < 0) return 0;
    Carver cv(nullptr);
    cv.take<float>(T * V);
    cv.take<float>(T * V);
    return cv.size();
}

int moe_codec_head_argmax(const moe_config* cfg, const void* x, const void* w_head, int32_t V, int64_t T,
                          float* logits, int32_t* c0, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if (T < 0 || V < 1) return MOE_ERR_INVALID;
    if (V > (1 << 20) || T > (int64_t(1) << 22)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(w_head) || !ok_opt(logits) || !ok_ptr(c0) || !ok_ptr(ws)) return MOE_ERR_INVALID;
    if (ws_bytes < moe_codec_head_workspace_size(cfg, V, T)) return MOE_ERR_WORKSPACE;
    Carver cv(ws);
    float* sc = cv.take<float>(T * V);
    float* bd = cv.take<float>(T * V);
    if (logits) sc = logits;
    hipStream_t s = as_stream(stream);
    TMOE_TRY(launch_scores_argmax(cfg->dtype, x, w_head, T, cfg->hidden_size, V, sc, bd, s));
    return hip_status(launch_argmax(cfg->dtype, sc, bd, x, w_head, T, cfg->hidden_size, V, c0, s));
}

size_t moe_attention_workspace_size(const moe_attn_config* cfg, int64_t T) {
    if (check_attn_cfg(cfg) != MOE_OK || T < 0 || T > 65535) return 0;
    Carver cv(nullptr);
    AttnPlan p;
    plan_attn(cfg, T, cv, p);
    return cv.size();
}

int moe_attention_decode(const moe_attn_config* cfg, const moe_attn_weights* w, const void* x, int64_t T,
                         const int32_t* pos, const int32_t* cache_len, void* k_cache, void* v_cache,
                         const void* residual, void* y, const float* norm_gain, float norm_eps, void* norm_out,
                         void* ws, size_t ws_bytes, void* stream) {
    int st = check_attn_cfg(cfg);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_ERR_INVALID;
    if (T > 65535) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!w || !ok_ptr(w->w_qkv) || !ok_ptr(w->q_norm) || !ok_ptr(w->k_norm) || !ok_ptr(w->w_o) || !ok_ptr(x) ||
        !ok_ptr(pos) || !ok_ptr(cache_len) || !ok_ptr(k_cache) || !ok_ptr(v_cache) || !ok_opt(residual) ||
        !ok_ptr(y) || !ok_opt(norm_gain) || !ok_opt(norm_out) || !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (norm_out && (!(norm_eps >= 0.0f) || norm_out == y)) return MOE_ERR_INVALID;
    if (ws_bytes < moe_attention_workspace_size(cfg, T)) return MOE_ERR_WORKSPACE;
    Carver cv(ws);
    AttnPlan p;
    plan_attn(cfg, T, cv, p);
    return attn_run(cfg, w, p, x, T, pos, cache_len, k_cache, v_cache, residual, y, norm_gain, norm_eps, norm_out,
                    as_stream(stream));
}

size_t moe_predictor_workspace_size(const moe_predictor_config* cfg, int64_t T) {
    if (check_pred_cfg(cfg, T) != MOE_OK) return 0;
    Carver cv(nullptr);
    PredPlan p;
    plan_pred(cfg, T, cv, p);
    return cv.size();
}

int moe_predictor_frame(const moe_predictor_config* cfg, const moe_predictor_weights* w, const void* h_talker,
                        const int32_t* c0, int64_t T, int32_t* codes, void* xn_out, void* ws, size_t ws_bytes,
                        void* stream) {
    if (T == 0 && cfg) return MOE_OK;
    int st = check_pred_cfg(cfg, T);
    if (st != MOE_OK) return st;
    if (!pred_weights_ok(cfg, w) || !ok_ptr(h_talker) || !ok_ptr(c0) || !ok_ptr(codes) || !ok_opt(xn_out) ||
        !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (ws_bytes < moe_predictor_workspace_size(cfg, T)) return MOE_ERR_WORKSPACE;
    Carver cv(ws);
    PredPlan p;
    plan_pred(cfg, T, cv, p);
    hipStream_t s = as_stream(stream);
    const int H = p.acfg.hidden_size, I = cfg->intermediate_size, K = cfg->codebook_size;
    const int P = cfg->num_codes, L = cfg->num_layers;
    const float eps = cfg->eps;
    const int64_t table = (int64_t)K * H * 2;  // bytes per embedding table / head
    TMOE_TRY(launch_frame_setup(p.pos, p.len, P, T, c0, codes, s));
    for (int q = 0; q < P; ++q) {
        // the position's input row (h_talker, or the embedding of the previous
        // code) and its first pre-norm
        const void* src = h_talker;
        if (q == 0) {
            TMOE_TRY(launch_rmsnorm(MOE_BF16, src, w->layers[0].in_norm, eps, T, H, p.XN, s));
        } else {
            const bool first = q == 1;
            TMOE_TRY(launch_embed_norm(first ? w->c0_embedding
                                             : static_cast<const char*>(w->codec_embedding) + (q - 2) * table,
                                       first ? cfg->c0_vocab : K, first ? c0 : codes + (int64_t)(q - 1) * T, p.X,
                                       w->layers[0].in_norm, eps, T, H, p.XN, s));
            src = p.X;
        }
        for (int l = 0; l < L; ++l) {
            const moe_predictor_layer& ly = w->layers[l];
            const int r = attn_run(&p.acfg, &ly.attn, p.ap, p.XN, T, p.pos + (int64_t)q * T * 3, p.len + (int64_t)q * T,
                                   p.kc + l * p.cache_bytes, p.vc + l * p.cache_bytes, l == 0 ? src : p.X, p.Hh,
                                   ly.post_norm, eps, p.HN, s);
            if (r != MOE_OK) return r;
            TMOE_TRY(launch_skinny_swiglu(p.HN, ly.gate, ly.up, p.h, T, I, H, s));
            TMOE_TRY(launch_skinny_gemm(p.h, ly.down, p.pd, T, H, I, p.ksd, s));
            const bool last = l + 1 == L;
            const float* next = last ? w->final_norm : w->layers[l + 1].in_norm;
            void* xn = last && xn_out ? static_cast<char*>(xn_out) + (int64_t)q * T * H * 2 : p.XN;
            TMOE_TRY(launch_attn_out(p.pd, p.ksd, p.Hh, p.X, T, H, next, eps, xn, s));
        }
        if (q >= 1) {
            const void* head = static_cast<const char*>(w->lm_head) + (q - 1) * table;
            const void* xf = xn_out ? static_cast<const char*>(xn_out) + (int64_t)q * T * H * 2 : p.XN;
            TMOE_TRY(launch_scores_argmax(MOE_BF16, xf, head, T, H, K, p.sc, p.bd, s));
            TMOE_TRY(launch_argmax(MOE_BF16, p.sc, p.bd, xf, head, T, H, K, codes + (int64_t)q * T, s));
        }
    }
    return MOE_OK;
}

int moe_codec_head_sample(const moe_config* cfg, const void* x, const void* w_head, int32_t V, int64_t T,
                          float temperature, const double* u, float* logits, int32_t* c0, void* ws, size_t ws_bytes,
                          void* stream) {
    int st = check_cfg(cfg);
    if (st != MOE_OK) return st;
    if (T < 0 || V < 1 || !(temperature > 0.0f) || !(temperature < INFINITY)) return MOE_ERR_INVALID;
    if (!sample_ok(V) || T > (int64_t(1) << 22)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!ok_ptr(x) || !ok_ptr(w_head) || !ok_ptr(u) || !ok_opt(logits) || !ok_ptr(c0) || !ok_ptr(ws))
        return MOE_ERR_INVALID;
    if (ws_bytes < moe_codec_head_workspace_size(cfg, V, T)) return MOE_ERR_WORKSPACE;
    Carver cv(ws);
    float* sc = cv.take<float>(T * V);
    float* bd = cv.take<float>(T * V);
    if (logits) sc = logits;
    hipStream_t s = as_stream(stream);
    TMOE_TRY(launch_scores_exact(cfg->dtype, x, w_head, T, cfg->hidden_size, V, sc, bd, s));
    return hip_status(launch_sample(cfg->dtype, sc, bd, x, w_head, T, cfg->hidden_size, V, (double)temperature, u,
                                    c0, s));
}

}  // extern "C"
