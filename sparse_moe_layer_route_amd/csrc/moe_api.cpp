// moe_api.cpp -- the C ABI declared in include/moe.h: argument checks,
// workspace layout and the order of launches.  No call allocates, frees or
// synchronises; everything is enqueued on the caller's stream.
#include "moe.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Dims {
    int64_t T, P;
    int H, E, k, I, Is;
    bool fp8;
};

moe_status_t check_config(const moe_config_t* c, int64_t T) {
    if (!c || T < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (c->hidden_size <= 0 || c->num_experts <= 0 || c->top_k <= 0 || c->moe_intermediate_size <= 0 ||
        c->share_expert_dim < 0)
        return MOE_ERR_INVALID_ARGUMENT;
    if (c->top_k > c->num_experts) return MOE_ERR_INVALID_ARGUMENT;
    if (!isfinite(c->router_scaling_factor)) return MOE_ERR_INVALID_ARGUMENT;
    if (!(c->swiglu_limit >= 0.0f) || !isfinite(c->swiglu_limit)) return MOE_ERR_INVALID_ARGUMENT;
    if (!(c->swiglu_limit_shared >= 0.0f) || !isfinite(c->swiglu_limit_shared))
        return MOE_ERR_INVALID_ARGUMENT;
    if (c->norm_expert_weight != 0 && c->norm_expert_weight != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (c->expert_dtype != MOE_BF16 && c->expert_dtype != MOE_FP8_E4M3_B128) return MOE_ERR_INVALID_ARGUMENT;
    if (c->out_dtype != MOE_FP32 && c->out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (c->hidden_size % 64 || c->moe_intermediate_size % 64 || c->share_expert_dim % 64)
        return MOE_ERR_UNSUPPORTED;
    if (c->top_k > 32 || c->num_experts > 1024) return MOE_ERR_UNSUPPORTED;
    if (T * (int64_t)c->top_k >= ((int64_t)1 << 31) || T >= ((int64_t)1 << 31) / 8)
        return MOE_ERR_UNSUPPORTED;
    // the 256-row expert GEMMs address the gathered rows of x, and one
    // expert's (or the shared expert's) first-projection weights, by 32-bit
    // byte offsets
    const int64_t H = c->hidden_size;
    if (T * H >= ((int64_t)1 << 31) || 2 * (int64_t)c->moe_intermediate_size * H >= ((int64_t)1 << 31) ||
        2 * (int64_t)c->share_expert_dim * H >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (c->expert_dtype == MOE_FP8_E4M3_B128 && (c->hidden_size % 128 || c->moe_intermediate_size % 128))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// bf16 experts take no scales; FP8 experts need both
moe_status_t check_scales(const moe_config_t* c, const float* s1, const float* s2) {
    if (c->expert_dtype == MOE_BF16) return (s1 || s2) ? MOE_ERR_INVALID_ARGUMENT : MOE_OK;
    return (s1 && s2) ? MOE_OK : MOE_ERR_INVALID_ARGUMENT;
}

Dims dims(const moe_config_t* c, int64_t T) {
    return Dims{T, T * c->top_k, c->hidden_size, c->num_experts, c->top_k, c->moe_intermediate_size,
                c->share_expert_dim, c->expert_dtype == MOE_FP8_E4M3_B128};
}

int tile_m(const Dims& d);

// scratch each step needs at the start of the workspace it is handed
size_t route_ws(const Dims& d) { return align_up((size_t)moe::router_splits(d.T, d.H) * d.T * d.E * 4); }
size_t permute_ws(const Dims& d) { return align_up(moe::permute_scratch_bytes(d.P, d.E)); }
// the tile plan, then (256-row tiles) the work-item table of the grouped
// launches, sized for the larger of the two projections' column-tile counts
// and for the shared expert as one more group
size_t plan_head(const Dims& d) { return align_up((size_t)(d.E + 2) * 4); }
int64_t max_tiles(const Dims& d, bool extra);
size_t item_ws(const Dims& d) {
    const int n_up = (2 * d.I + 255) / 256, n_down = (d.H + 255) / 256;
    return align_up(moe::grouped_item_bytes(max_tiles(d, true), std::max(n_up, n_down)));
}
size_t plan_ws(const Dims& d) { return plan_head(d) + item_ws(d); }
// FP8: x quantised per token, codes [T, H] then scales [H/128][T]
size_t xq_bytes(const Dims& d) { return align_up((size_t)d.T * d.H); }
size_t xq_ws(const Dims& d) { return d.fp8 ? xq_bytes(d) + align_up((size_t)(d.H / 128) * d.T * 4) : 0; }
size_t up_ws(const Dims& d) { return plan_ws(d) + xq_ws(d); }
// h: bf16 [P, I]; FP8: codes [P, I] then scales [I/128][P]
size_t hcode_bytes(const Dims& d) { return align_up((size_t)d.P * d.I); }
// The shared expert can run as one more group of the routed experts'
// launches when it has their width and dtype.
bool fuse_shared(const Dims& d) { return !d.fp8 && d.Is > 0 && d.Is == d.I; }
size_t hidden_bytes(const Dims& d) {
    if (d.fp8) return hcode_bytes(d) + (size_t)(d.I / 128) * d.P * 4;
    return (size_t)(d.P + (fuse_shared(d) ? d.T : 0)) * d.I * 2;
}
size_t grouped_ws(const Dims& d) { return up_ws(d) + align_up(hidden_bytes(d)); }
size_t shared_ws(const Dims& d) { return align_up((size_t)d.T * d.Is * 2); }

// the whole layer: its own buffers followed by each step's scratch
struct LayerWs {
    size_t ids, w, counts, offsets, r2p, p2r, plan, x, y_rows, y_sh, step, total;
};
// bytes of one expert output row (H fp16 values + one exponent per 128 columns)
size_t row_bytes(const Dims& d) { return (size_t)moe::expert_row_bytes(d.H); }

LayerWs layer_ws(const Dims& d) {
    const bool fuse = fuse_shared(d);
    const int64_t rows = d.P + (fuse ? d.T : 0);      // routed rows, then the shared expert's
    LayerWs L;
    size_t o = 0;
    L.ids = o;     o += align_up((size_t)d.P * 4);
    L.w = o;       o += align_up((size_t)d.P * 4);
    L.counts = o;  o += align_up((size_t)d.E * 4);
    L.offsets = o; o += align_up((size_t)(d.E + 1) * 4);
    L.r2p = o;     o += align_up((size_t)d.P * 4);
    L.p2r = o;     o += align_up((size_t)d.P * 4);
    L.plan = o;    o += plan_ws(d);
    L.x = o;       o += align_up((size_t)d.T * d.H * 2);    // the normalised input (moe_block_forward)
    L.y_rows = o;  o += align_up((size_t)rows * row_bytes(d));
    L.y_sh = o;    o += (d.Is > 0 && !fuse) ? align_up((size_t)d.T * d.H * 4) : 0;
    L.step = o;
    const size_t grouped = fuse ? align_up(hidden_bytes(d)) : grouped_ws(d);
    o += std::max(std::max(route_ws(d), permute_ws(d)), std::max(grouped, shared_ws(d)));
    L.total = o;
    return L;
}

inline moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                              \
    do {                                           \
        moe_status_t _st = (expr);                 \
        if (_st != MOE_OK) return _st;             \
    } while (0)
#define HIP_TRY(expr) MOE_TRY(hip_status(expr))

// ---- the steps, without argument checks ----------------------------------

moe_status_t do_route(const moe_config_t* c, const Dims& d, const void* x, const void* wr, const float* b,
                      int32_t* ids, float* w, char* ws, hipStream_t s) {
    float* logits = (float*)ws;
    HIP_TRY(moe::launch_router_logits(x, wr, logits, (int)d.T, d.E, d.H, s));
    HIP_TRY(moe::launch_topk(logits, moe::router_splits(d.T, d.H), b, (int)d.T, d.E, d.k,
                             c->router_scaling_factor, c->norm_expert_weight, ids, w, s));
    return MOE_OK;
}

// the RMSNorm, then the routing of its output; with `fused`, where the shape
// allows, the norm and the router logits in one pass (the same bits as the
// two steps)
moe_status_t do_norm_route(const moe_config_t* c, const Dims& d, const float* resid, const float* g, float eps,
                           const void* wr, const float* b, void* x, int32_t* ids, float* w, char* ws,
                           bool fused, hipStream_t s) {
    if (!fused || !moe::rmsnorm_router_fusable(d.T, d.H, d.E)) {
        HIP_TRY(moe::launch_rmsnorm(resid, g, eps, x, (int)d.T, d.H, s));
        return do_route(c, d, x, wr, b, ids, w, ws, s);
    }
    float* logits = (float*)ws;
    HIP_TRY(moe::launch_rmsnorm_router(resid, g, eps, wr, x, logits, (int)d.T, d.E, d.H, s));
    HIP_TRY(moe::launch_topk(logits, 1, b, (int)d.T, d.E, d.k, c->router_scaling_factor, c->norm_expert_weight,
                             ids, w, s));
    return MOE_OK;
}

// router logits, then the weights of caller-supplied ids
moe_status_t do_replay(const moe_config_t* c, const Dims& d, const void* x, const void* wr, const int32_t* ids,
                       float* w, char* ws, hipStream_t s) {
    float* logits = (float*)ws;
    HIP_TRY(moe::launch_router_logits(x, wr, logits, (int)d.T, d.E, d.H, s));
    HIP_TRY(moe::launch_replay_weights(logits, moe::router_splits(d.T, d.H), ids, (int)d.T, d.E, d.k,
                                       c->router_scaling_factor, c->norm_expert_weight, w, s));
    return MOE_OK;
}

int tile_m(const Dims& d) { return d.fp8 ? moe::fp8_tile_m() : moe::grouped_tile_m(d.P, d.E); }

// upper bound on the tiles of a grouped launch: every group may end in a
// partial tile (the extra group holds T rows)
int64_t max_tiles(const Dims& d, bool extra) {
    const int bm = tile_m(d);
    return (d.P + bm - 1) / bm + d.E + (extra ? (d.T + bm - 1) / bm + 1 : 0);
}
// the work-item table sits right after the tile plan
void* item_table(const Dims& d, const int32_t* tile_start) { return (char*)tile_start + plan_head(d); }

// the bf16 grouped launches of the routed experts (optionally with the
// shared expert as an extra group of T rows after the P routed rows)
moe::GroupedArgs up_args(const moe_config_t* c, const Dims& d, const void* x, const int32_t* offsets,
                         const int32_t* r2p, const void* w13, void* h, const int32_t* tile_start,
                         const void* ws13 = nullptr) {
    moe::GroupedArgs a;
    a.A = x;
    a.a_rows = r2p;
    a.a_div = d.k;
    a.a_nrows = (int)d.T;
    a.W = w13;
    a.w_group_stride = (int64_t)2 * d.I * d.H;
    a.C = h;
    a.M = (int)d.P;
    a.N = d.I;
    a.K = d.H;
    a.limit = c->swiglu_limit;
    a.offsets = offsets;
    a.tile_start = tile_start;
    a.groups = d.E;
    a.bm = tile_m(d);
    a.max_tiles = (int)max_tiles(d, ws13 != nullptr);
    a.items = item_table(d, tile_start);
    if (ws13) {
        a.extra_rows = (int)d.T;
        a.W_extra = ws13;
        a.limit_extra = c->swiglu_limit_shared;
    }
    return a;
}

moe::GroupedArgs down_args(const Dims& d, const void* h, const int32_t* offsets, const void* w2, void* y_rows,
                           const int32_t* tile_start, const void* ws2 = nullptr) {
    moe::GroupedArgs a;
    a.A = h;
    a.a_nrows = (int)(d.P + (ws2 ? d.T : 0));
    a.W = w2;
    a.w_group_stride = (int64_t)d.H * d.I;
    a.C = y_rows;
    a.M = (int)d.P;
    a.N = d.H;
    a.K = d.I;
    a.offsets = offsets;
    a.tile_start = tile_start;
    a.groups = d.E;
    a.bm = tile_m(d);
    a.max_tiles = (int)max_tiles(d, ws2 != nullptr);
    a.items = item_table(d, tile_start);
    if (ws2) {
        a.extra_rows = (int)d.T;
        a.W_extra = ws2;
    }
    return a;
}

// routed experts' first projection + clipped SwiGLU -> h
moe_status_t do_up(const moe_config_t* c, const Dims& d, const void* x, const int32_t* offsets,
                   const int32_t* r2p, const void* w13, const float* w13s, void* h, char* ws, hipStream_t s,
                   const void* ws13 = nullptr) {
    int32_t* tile_start = (int32_t*)ws;
    HIP_TRY(moe::launch_tile_plan(offsets, d.E, tile_m(d), ws13 ? (int)d.T : 0, tile_start, s));
    if (d.fp8) {
        char* xq = ws + plan_ws(d);
        float* xs = (float*)(xq + xq_bytes(d));
        float* hs = (float*)((char*)h + hcode_bytes(d));
        HIP_TRY(moe::launch_quant_rows(x, (int)d.T, d.H, xq, xs, (int)d.T, s));
        HIP_TRY(moe::launch_fp8_up(xq, xs, (int)d.T, r2p, d.k, (int)d.T, w13, w13s, h, hs, (int)d.P, d.I, d.H,
                                   c->swiglu_limit, offsets, tile_start, d.E, (int)max_tiles(d, false),
                                   item_table(d, tile_start), s));
        return MOE_OK;
    }
    HIP_TRY(moe::launch_grouped_up(up_args(c, d, x, offsets, r2p, w13, h, tile_start, ws13), s));
    return MOE_OK;
}

// routed experts' second projection -> y_rows
moe_status_t do_down(const moe_config_t* c, const Dims& d, const void* h, const int32_t* offsets,
                     const void* w2, const float* w2s, void* y_rows, char* ws, hipStream_t s,
                     const void* ws2 = nullptr) {
    (void)c;
    int32_t* tile_start = (int32_t*)ws;
    HIP_TRY(moe::launch_tile_plan(offsets, d.E, tile_m(d), ws2 ? (int)d.T : 0, tile_start, s));
    if (d.fp8) {
        const float* hs = (const float*)((const char*)h + hcode_bytes(d));
        HIP_TRY(moe::launch_fp8_down(h, hs, (int)d.P, (int)d.P, w2, w2s, y_rows, d.H, d.I, offsets, tile_start,
                                     d.E, (int)max_tiles(d, false), item_table(d, tile_start), s));
        return MOE_OK;
    }
    HIP_TRY(moe::launch_grouped_down(down_args(d, h, offsets, w2, y_rows, tile_start, ws2), false, s));
    return MOE_OK;
}

moe_status_t do_grouped(const moe_config_t* c, const Dims& d, const void* x, const int32_t* offsets,
                        const int32_t* r2p, const void* w13, const float* w13s, const void* w2, const float* w2s,
                        void* y_rows, char* ws, hipStream_t s) {
    void* h = ws + up_ws(d);
    MOE_TRY(do_up(c, d, x, offsets, r2p, w13, w13s, h, ws, s));
    MOE_TRY(do_down(c, d, h, offsets, w2, w2s, y_rows, ws, s));
    return MOE_OK;
}

// shared expert on its own: dense launches, fp32 output
moe_status_t do_shared(const moe_config_t* c, const Dims& d, const void* x, const void* ws13,
                       const void* ws2, float* y_sh, char* ws, hipStream_t s) {
    uint16_t* hs = (uint16_t*)ws;
    moe::GroupedArgs a;
    a.A = x;
    a.a_nrows = (int)d.T;
    a.W = ws13;
    a.C = hs;
    a.M = (int)d.T;
    a.N = d.Is;
    a.K = d.H;
    a.limit = c->swiglu_limit_shared;
    a.bm = d.T <= 64 ? 64 : 256;
    HIP_TRY(moe::launch_grouped_up(a, s));
    moe::GroupedArgs b;
    b.A = hs;
    b.a_nrows = (int)d.T;
    b.W = ws2;
    b.C = y_sh;
    b.M = (int)d.T;
    b.N = d.H;
    b.K = d.Is;
    b.bm = a.bm;
    HIP_TRY(moe::launch_grouped_down(b, true, s));
    return MOE_OK;
}

// argument checks shared by the whole-layer entry points
moe_status_t check_layer(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                         const void* w13, const float* w13_scale, const void* w2, const float* w2_scale,
                         const void* ws13, const void* ws2, const void* out, const void* ws, size_t ws_bytes) {
    MOE_TRY(check_config(cfg, T));
    MOE_TRY(check_scales(cfg, w13_scale, w2_scale));
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !w13 || !w2 || !out || !ws) return MOE_ERR_INVALID_ARGUMENT;
    if (cfg->share_expert_dim > 0 && (!ws13 || !ws2)) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < layer_ws(dims(cfg, T)).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// the layer after routing: permute, routed + shared experts, combine.  The
// shared expert runs as group E of the routed experts' launches when it has
// their width and dtype (bf16, Is == I: both models), else in dense launches
// of its own after them; everything is on the caller's stream.
moe_status_t layer_experts(const moe_config_t* cfg, const Dims& d, const LayerWs& L, char* base, const void* x,
                           const int32_t* ids, const float* w, const void* w13, const float* w13_scale,
                           const void* w2, const float* w2_scale, const void* ws13, const void* ws2, void* out,
                           int32_t* expert_counts_out, hipStream_t stream, const float* resid = nullptr) {
    const int T = (int)d.T;
    int32_t* counts = expert_counts_out ? expert_counts_out : (int32_t*)(base + L.counts);
    int32_t* offsets = (int32_t*)(base + L.offsets);
    int32_t* r2p = (int32_t*)(base + L.r2p);
    int32_t* p2r = (int32_t*)(base + L.p2r);
    char* y_rows = base + L.y_rows;
    char* step = base + L.step;
    const bool out_bf16 = cfg->out_dtype == MOE_BF16;
    if (fuse_shared(d)) {
        // one tile plan for both projections; the shared expert is group E.
        // The plan sits in the layer's own area: the permutation's scratch
        // (at `step`) is still in use while the plan is made.
        int32_t* tile_start = (int32_t*)(base + L.plan);
        void* h = step;
        HIP_TRY(moe::launch_permute_plan(ids, T, d.k, d.E, counts, offsets, r2p, p2r, step, tile_m(d), T,
                                         tile_start, stream));
        HIP_TRY(moe::launch_grouped_up(up_args(cfg, d, x, offsets, r2p, w13, h, tile_start, ws13), stream));
        HIP_TRY(moe::launch_grouped_down(down_args(d, h, offsets, w2, y_rows, tile_start, ws2), false, stream));
        HIP_TRY(moe::launch_combine(y_rows, p2r, w, nullptr, y_rows + (size_t)d.P * row_bytes(d), resid, out,
                                    out_bf16, T, d.H, d.k, stream));
        return MOE_OK;
    }
    HIP_TRY(moe::launch_permute(ids, T, d.k, d.E, counts, offsets, r2p, p2r, step, stream));
    float* y_sh = d.Is > 0 ? (float*)(base + L.y_sh) : nullptr;
    MOE_TRY(do_grouped(cfg, d, x, offsets, r2p, w13, w13_scale, w2, w2_scale, y_rows, step, stream));
    if (d.Is > 0) MOE_TRY(do_shared(cfg, d, x, ws13, ws2, y_sh, step, stream));
    HIP_TRY(moe::launch_combine(y_rows, p2r, w, y_sh, nullptr, resid, out, out_bf16, T, d.H, d.k, stream));
    return MOE_OK;
}

// ---- training: what the forward keeps, the backward's scratch -------------

// The backward runs the shared expert as one more group of the routed
// experts' launches, so it needs bf16 experts and Is == I (or no shared expert).
bool train_ok(const Dims& d) { return !d.fp8 && (d.Is == 0 || d.Is == d.I); }
int64_t train_rows(const Dims& d) { return d.P + (d.Is > 0 ? d.T : 0); }

struct SavedWs {
    size_t ids, w, s, counts, offsets, r2p, p2r, gu, h, y, total;
};
SavedWs saved_ws(const Dims& d) {
    const int64_t rows = train_rows(d);
    SavedWs S;
    size_t o = 0;
    S.ids = o;     o += align_up((size_t)d.P * 4);
    S.w = o;       o += align_up((size_t)d.P * 4);
    S.s = o;       o += align_up((size_t)d.P * 4);
    S.counts = o;  o += align_up((size_t)d.E * 4);
    S.offsets = o; o += align_up((size_t)(d.E + 1) * 4);
    S.r2p = o;     o += align_up((size_t)d.P * 4);
    S.p2r = o;     o += align_up((size_t)d.P * 4);
    S.gu = o;      o += align_up((size_t)rows * 2 * d.I * 2);
    S.h = o;       o += align_up((size_t)rows * d.I * 2);
    S.y = o;       o += align_up((size_t)rows * row_bytes(d));
    S.total = o;
    return S;
}

struct BwdWs {
    size_t plan, zero, dy, dgu, dxr, da, xp, total;
};
BwdWs bwd_ws(const Dims& d) {
    const int64_t rows = train_rows(d);
    BwdWs B;
    size_t o = 0;
    B.plan = o;  o += plan_ws(d);
    B.zero = o;  o += align_up((size_t)std::max(d.H, 2 * d.I) * 2);
    B.dy = o;    o += align_up((size_t)rows * d.H * 2);
    B.dgu = o;   o += align_up((size_t)rows * 2 * d.I * 2);
    B.dxr = o;   o += align_up((size_t)rows * d.H * 4);
    B.da = o;    o += align_up((size_t)d.P * 4);
    B.xp = o;    o += align_up((size_t)rows * d.H * 2);   // x rows in row order
    B.total = o;
    return B;
}
int bwd_max_tiles(const Dims& d) {
    return (int)((d.P + 255) / 256) + d.E + (d.Is > 0 ? (int)((d.T + 255) / 256) + 1 : 0);
}

// ---- the allocation-free entry point's scratch -----------------------------
// A file-scope device array that moe_layer_forward_noalloc uses as its
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel: the
// name is a host-side stand-in, not a device address.  The device address
// is looked up once per device (with that device current) and kept.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// the scratch array's address on the device `stream` belongs to
moe_status_t noalloc_scratch(hipStream_t stream, char** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return MOE_ERR_HIP;
        // the same address whichever thread stores it
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = (char*)p;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_config(cfg, T));
    *bytes = layer_ws(dims(cfg, T)).total;
    return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                       const float* router_bias, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !router_bias || !topk_ids || !topk_w || !ws) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < route_ws(d)) return MOE_ERR_WORKSPACE;
    return do_route(cfg, d, x, w_router, router_bias, topk_ids, topk_w, (char*)ws, stream);
}

moe_status_t moe_permute(const moe_config_t* cfg, int64_t T, const int32_t* topk_ids, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* row_to_pair, int32_t* pair_to_row, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (T > 0 && (!topk_ids || !row_to_pair || !pair_to_row || !ws)) return MOE_ERR_INVALID_ARGUMENT;
    if (T > 0 && ws_bytes < permute_ws(d)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_ids, (int)T, d.k, d.E, expert_counts, expert_offsets,
                                          row_to_pair, pair_to_row, ws, stream));
}

moe_status_t moe_grouped_swiglu(const moe_config_t* cfg, int64_t T, const void* x, const int32_t* expert_offsets,
                                const int32_t* row_to_pair, const void* w13, const float* w13_scale,
                                const void* w2, const float* w2_scale, void* y_rows, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    MOE_TRY(check_scales(cfg, w13_scale, w2_scale));
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !row_to_pair || !w13 || !w2 || !y_rows || !ws) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < grouped_ws(d)) return MOE_ERR_WORKSPACE;
    return do_grouped(cfg, d, x, expert_offsets, row_to_pair, w13, w13_scale, w2, w2_scale, y_rows, (char*)ws,
                      stream);
}

moe_status_t moe_expert_up(const moe_config_t* cfg, int64_t T, const void* x, const int32_t* expert_offsets,
                           const int32_t* row_to_pair, const void* w13, const float* w13_scale, const void* ws13,
                           void* h, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    MOE_TRY(check_scales(cfg, w13_scale, w13_scale));
    if (ws13 && !fuse_shared(dims(cfg, T))) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !row_to_pair || !w13 || !h || !ws) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < up_ws(d)) return MOE_ERR_WORKSPACE;
    return do_up(cfg, d, x, expert_offsets, row_to_pair, w13, w13_scale, h, (char*)ws, stream, ws13);
}

moe_status_t moe_expert_down(const moe_config_t* cfg, int64_t T, const void* h, const int32_t* expert_offsets,
                             const void* w2, const float* w2_scale, const void* ws2, void* y_rows, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    MOE_TRY(check_scales(cfg, w2_scale, w2_scale));
    if (ws2 && !fuse_shared(dims(cfg, T))) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!h || !expert_offsets || !w2 || !y_rows || !ws) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < plan_ws(d)) return MOE_ERR_WORKSPACE;
    return do_down(cfg, d, h, expert_offsets, w2, w2_scale, y_rows, (char*)ws, stream, ws2);
}

moe_status_t moe_expert_rows_bytes(const moe_config_t* cfg, int64_t rows, size_t* bytes) {
    if (!bytes || rows < 0) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_config(cfg, 0));
    *bytes = (size_t)rows * (size_t)moe::expert_row_bytes(cfg->hidden_size);
    return MOE_OK;
}

moe_status_t moe_hidden_bytes(const moe_config_t* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_config(cfg, T));
    *bytes = hidden_bytes(dims(cfg, T));
    return MOE_OK;
}

moe_status_t moe_shared_ffn(const moe_config_t* cfg, int64_t T, const void* x, const void* ws13, const void* ws2,
                            float* y_shared, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (cfg->share_expert_dim == 0) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!x || !ws13 || !ws2 || !y_shared || !ws) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < shared_ws(d)) return MOE_ERR_WORKSPACE;
    return do_shared(cfg, d, x, ws13, ws2, y_shared, (char*)ws, stream);
}

moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const void* y_rows, const int32_t* pair_to_row,
                         const float* topk_w, const float* y_shared, const void* shared_rows, const float* residual,
                         void* out, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (y_shared && shared_rows) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!y_rows || !pair_to_row || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
    if (residual && cfg->out_dtype != MOE_FP32 && (const void*)residual == out) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_combine(y_rows, pair_to_row, topk_w, y_shared, shared_rows, residual, out,
                                          cfg->out_dtype == MOE_BF16, (int)T, cfg->hidden_size, cfg->top_k, stream));
}

moe_status_t moe_rmsnorm(const moe_config_t* cfg, int64_t T, const float* resid, const float* norm_weight, float eps,
                         void* x, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!resid || !norm_weight || !x) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_rmsnorm(resid, norm_weight, eps, x, (int)T, cfg->hidden_size, stream));
}

moe_status_t moe_rmsnorm_route(const moe_config_t* cfg, int64_t T, const float* resid, const float* norm_weight,
                               float eps, const void* w_router, const float* router_bias, void* x,
                               int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!resid || !norm_weight || !w_router || !router_bias || !x || !topk_ids || !topk_w || !ws)
        return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < route_ws(d)) return MOE_ERR_WORKSPACE;
    return do_norm_route(cfg, d, resid, norm_weight, eps, w_router, router_bias, x, topk_ids, topk_w, (char*)ws,
                         true, stream);
}

moe_status_t moe_layer_forward(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                               const float* router_bias, const void* w13, const float* w13_scale, const void* w2,
                               const float* w2_scale, const void* ws13, const void* ws2, void* out,
                               int32_t* topk_ids_out, float* topk_w_out, int32_t* expert_counts_out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_layer(cfg, T, x, w_router, w13, w13_scale, w2, w2_scale, ws13, ws2, out, ws, ws_bytes));
    if (T == 0) return MOE_OK;
    if (!router_bias) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    LayerWs L = layer_ws(d);
    char* base = (char*)ws;
    int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
    float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
    MOE_TRY(do_route(cfg, d, x, w_router, router_bias, ids, w, base + L.step, stream));
    return layer_experts(cfg, d, L, base, x, ids, w, w13, w13_scale, w2, w2_scale, ws13, ws2, out,
                         expert_counts_out, stream);
}

size_t moe_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                                       const float* router_bias, const void* w13, const float* w13_scale,
                                       const void* w2, const float* w2_scale, const void* ws13, const void* ws2,
                                       void* out, int32_t* topk_ids_out, float* topk_w_out,
                                       int32_t* expert_counts_out, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (T == 0) return MOE_OK;
    if (layer_ws(dims(cfg, T)).total > kNoallocScratchBytes) return MOE_ERR_WORKSPACE;
    char* base = nullptr;
    MOE_TRY(noalloc_scratch(stream, &base));
    return moe_layer_forward(cfg, T, x, w_router, router_bias, w13, w13_scale, w2, w2_scale, ws13, ws2, out,
                             topk_ids_out, topk_w_out, expert_counts_out, base, kNoallocScratchBytes, stream);
}

moe_status_t moe_route_replay(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                              const int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w || !ws) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    if (ws_bytes < route_ws(d)) return MOE_ERR_WORKSPACE;
    return do_replay(cfg, d, x, w_router, topk_ids, topk_w, (char*)ws, stream);
}

moe_status_t moe_balanced_ids(const moe_config_t* cfg, int64_t T, int32_t* topk_ids, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    if (T == 0) return MOE_OK;
    if (!topk_ids) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_balanced_ids(topk_ids, T * cfg->top_k, cfg->num_experts, stream));
}

moe_status_t moe_layer_forward_routed(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                                      const int32_t* topk_ids, const void* w13, const float* w13_scale,
                                      const void* w2, const float* w2_scale, const void* ws13, const void* ws2,
                                      void* out, float* topk_w_out, int32_t* expert_counts_out, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_layer(cfg, T, x, w_router, w13, w13_scale, w2, w2_scale, ws13, ws2, out, ws, ws_bytes));
    if (T == 0) return MOE_OK;
    if (!topk_ids) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    LayerWs L = layer_ws(d);
    char* base = (char*)ws;
    float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
    MOE_TRY(do_replay(cfg, d, x, w_router, topk_ids, w, base + L.step, stream));
    return layer_experts(cfg, d, L, base, x, topk_ids, w, w13, w13_scale, w2, w2_scale, ws13, ws2, out,
                         expert_counts_out, stream);
}

moe_status_t moe_block_forward(const moe_config_t* cfg, int64_t T, const float* resid_in, const float* norm_weight,
                               float eps, const void* w_router, const float* router_bias, const void* w13,
                               const float* w13_scale, const void* w2, const float* w2_scale, const void* ws13,
                               const void* ws2, float* resid_out, int32_t* topk_ids_out, float* topk_w_out,
                               int32_t* expert_counts_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_layer(cfg, T, resid_in, w_router, w13, w13_scale, w2, w2_scale, ws13, ws2, resid_out, ws,
                        ws_bytes));
    if (cfg->out_dtype != MOE_FP32) return MOE_ERR_INVALID_ARGUMENT;
    if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!norm_weight || !router_bias) return MOE_ERR_INVALID_ARGUMENT;
    Dims d = dims(cfg, T);
    LayerWs L = layer_ws(d);
    char* base = (char*)ws;
    void* x = base + L.x;
    int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
    float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
    // the norm and the routing as two steps: faster here than the fused pass
    // of moe_rmsnorm_route at the Step-5 prefill shape, with the same bits
    MOE_TRY(do_norm_route(cfg, d, resid_in, norm_weight, eps, w_router, router_bias, x, ids, w, base + L.step,
                          false, stream));
    return layer_experts(cfg, d, L, base, x, ids, w, w13, w13_scale, w2, w2_scale, ws13, ws2, resid_out,
                         expert_counts_out, stream, resid_in);
}

moe_status_t moe_saved_bytes(const moe_config_t* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_config(cfg, T));
    Dims d = dims(cfg, T);
    if (!train_ok(d)) return MOE_ERR_UNSUPPORTED;
    *bytes = saved_ws(d).total;
    return MOE_OK;
}

moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_config(cfg, T));
    Dims d = dims(cfg, T);
    if (!train_ok(d)) return MOE_ERR_UNSUPPORTED;
    *bytes = bwd_ws(d).total;
    return MOE_OK;
}

moe_status_t moe_layer_forward_train(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                                     const float* router_bias, const int32_t* topk_ids_in, const void* w13,
                                     const void* w2, const void* ws13,
                                     const void* ws2, void* out, void* saved, size_t saved_bytes, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_layer(cfg, T, x, w_router, w13, nullptr, w2, nullptr, ws13, ws2, out, ws, ws_bytes));
    Dims d = dims(cfg, T);
    if (!train_ok(d)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if ((!router_bias && !topk_ids_in) || !saved) return MOE_ERR_INVALID_ARGUMENT;
    const SavedWs S = saved_ws(d);
    if (saved_bytes < S.total) return MOE_ERR_WORKSPACE;
    const LayerWs L = layer_ws(d);
    char* base = (char*)ws;
    char* sv = (char*)saved;
    char* step = base + L.step;
    int32_t* ids = (int32_t*)(sv + S.ids);
    float* w = (float*)(sv + S.w);
    int32_t* offsets = (int32_t*)(sv + S.offsets);
    int32_t* r2p = (int32_t*)(sv + S.r2p);
    int32_t* p2r = (int32_t*)(sv + S.p2r);
    const bool shared = d.Is > 0;
    HIP_TRY(moe::launch_router_logits(x, w_router, (float*)step, (int)T, d.E, d.H, stream));
    if (topk_ids_in)
        HIP_TRY(moe::launch_replay_weights((const float*)step, moe::router_splits(d.T, d.H), topk_ids_in, (int)T,
                                           d.E, d.k, cfg->router_scaling_factor, cfg->norm_expert_weight, w, stream,
                                           ids, (float*)(sv + S.s)));
    else
        HIP_TRY(moe::launch_topk((const float*)step, moe::router_splits(d.T, d.H), router_bias, (int)T, d.E, d.k,
                                 cfg->router_scaling_factor, cfg->norm_expert_weight, ids, w, stream,
                                 (float*)(sv + S.s)));
    int32_t* tile_start = (int32_t*)(base + L.plan);
    HIP_TRY(moe::launch_permute_plan(ids, (int)T, d.k, d.E, (int32_t*)(sv + S.counts), offsets, r2p, p2r, step,
                                     tile_m(d), shared ? (int)T : 0, tile_start, stream));
    moe::GroupedArgs up = up_args(cfg, d, x, offsets, r2p, w13, sv + S.h, tile_start, shared ? ws13 : nullptr);
    up.gu_out = sv + S.gu;
    HIP_TRY(moe::launch_grouped_up(up, stream));
    HIP_TRY(moe::launch_grouped_down(down_args(d, sv + S.h, offsets, w2, sv + S.y, tile_start,
                                               shared ? ws2 : nullptr), false, stream));
    HIP_TRY(moe::launch_combine(sv + S.y, p2r, w, nullptr, shared ? sv + S.y + (size_t)d.P * row_bytes(d) : nullptr,
                                nullptr, out, cfg->out_dtype == MOE_BF16, (int)T, d.H, d.k, stream));
    return MOE_OK;
}

moe_status_t moe_layer_backward(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                                const void* w13, const void* w2, const void* ws13, const void* ws2,
                                const void* saved, size_t saved_bytes, const float* dout, float* dx,
                                float* dw_router, float* dw13, float* dw2, float* dws13, float* dws2, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_config(cfg, T));
    Dims d = dims(cfg, T);
    if (!train_ok(d)) return MOE_ERR_UNSUPPORTED;
    const bool shared = d.Is > 0;
    if (!dw_router || !dw13 || !dw2 || (shared && (!dws13 || !dws2))) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) {
        // no rows: every weight gradient is zero
        HIP_TRY(moe::launch_zero_u32(dw2, (int64_t)d.E * d.H * d.I, stream));
        HIP_TRY(moe::launch_zero_u32(dw13, (int64_t)d.E * 2 * d.I * d.H, stream));
        HIP_TRY(moe::launch_zero_u32(dw_router, (int64_t)d.E * d.H, stream));
        if (shared) {
            HIP_TRY(moe::launch_zero_u32(dws2, (int64_t)d.H * d.I, stream));
            HIP_TRY(moe::launch_zero_u32(dws13, (int64_t)2 * d.I * d.H, stream));
        }
        return MOE_OK;
    }
    if (!x || !w_router || !w13 || !w2 || !saved || !dout || !dx || !ws) return MOE_ERR_INVALID_ARGUMENT;
    if (shared && (!ws13 || !ws2)) return MOE_ERR_INVALID_ARGUMENT;
    const SavedWs S = saved_ws(d);
    const BwdWs B = bwd_ws(d);
    if (saved_bytes < S.total || ws_bytes < B.total) return MOE_ERR_WORKSPACE;
    char* base = (char*)ws;
    const char* sv = (const char*)saved;
    const int32_t* ids = (const int32_t*)(sv + S.ids);
    const int32_t* offsets = (const int32_t*)(sv + S.offsets);
    const int32_t* r2p = (const int32_t*)(sv + S.r2p);
    const int32_t* p2r = (const int32_t*)(sv + S.p2r);
    int32_t* tile_start = (int32_t*)(base + B.plan);
    float* da = (float*)(base + B.da);
    const int extra = shared ? (int)T : 0;
    {
        HIP_TRY(moe::launch_zero_u32(base + B.zero, (int64_t)std::max(d.H, 2 * d.I) / 2, stream));
        HIP_TRY(moe::launch_tile_plan(offsets, d.E, 256, extra, tile_start, stream));
        HIP_TRY(moe::launch_bwd_prep(dout, sv + S.y, p2r, (const float*)(sv + S.w), (const float*)(sv + S.s),
                                     cfg->router_scaling_factor, cfg->norm_expert_weight, shared, base + B.dy, da,
                                     (int)T, d.H, d.k, stream));
        // dh -> dgu: dy [rows][H] against W2 [H][I] (contracted over H)
        moe::BwdArgs a2;
        a2.A = base + B.dy;
        a2.lda = d.H;
        a2.B = w2;
        a2.ldb = d.I;
        a2.b_group_stride = (int64_t)d.H * d.I;
        a2.B_extra = ws2;
        a2.C = base + B.dgu;
        a2.gu = sv + S.gu;
        a2.limit = cfg->swiglu_limit;
        a2.limit_extra = cfg->swiglu_limit_shared;
        a2.N = d.I;
        a2.K = d.H;
        a2.offsets = offsets;
        a2.tile_start = tile_start;
        a2.groups = d.E;
        a2.extra_rows = extra;
        a2.max_tiles = bwd_max_tiles(d);
        HIP_TRY(moe::launch_bwd_dgrad(a2, true, stream));
        // dx rows: dgu [rows][2I] against W13 [2I][H]
        moe::BwdArgs a1 = a2;
        a1.A = base + B.dgu;
        a1.lda = 2 * d.I;
        a1.B = w13;
        a1.ldb = d.H;
        a1.b_group_stride = (int64_t)2 * d.I * d.H;
        a1.B_extra = ws13;
        a1.C = base + B.dxr;
        a1.ldc = d.H;
        a1.gu = nullptr;
        a1.N = d.H;
        a1.K = 2 * d.I;
        HIP_TRY(moe::launch_bwd_dgrad(a1, false, stream));
        HIP_TRY(moe::launch_bwd_dx((const float*)(base + B.dxr), p2r, da, ids, w_router, shared, dx, (int)T, d.H,
                                   d.k, stream));
    }
    // weight gradients (every expert; those without rows get zeros)
    moe::BwdArgs g2;
    g2.A = base + B.dy;
    g2.lda = d.H;
    g2.B = sv + S.h;
    g2.ldb = d.I;
    g2.zero_row = base + B.zero;
    g2.C = dw2;
    g2.ldc = d.I;
    g2.c_group_stride = (int64_t)d.H * d.I;
    g2.C_extra = dws2;
    g2.M = d.H;
    g2.N = d.I;
    g2.offsets = offsets;
    g2.groups = d.E;
    g2.extra_rows = extra;
    moe::BwdArgs g1 = g2;
    g1.A = base + B.dgu;
    g1.lda = 2 * d.I;
    g1.B = base + B.xp;
    g1.ldb = d.H;
    g1.C = dw13;
    g1.ldc = d.H;
    g1.c_group_stride = (int64_t)2 * d.I * d.H;
    g1.C_extra = dws13;
    g1.M = 2 * d.I;
    g1.N = d.H;
    HIP_TRY(moe::launch_bwd_wgrad(g2, stream));
    HIP_TRY(moe::launch_gather_rows(x, r2p, shared, base + B.xp, (int)T, d.H, d.k, stream));
    HIP_TRY(moe::launch_bwd_wgrad(g1, stream));
    HIP_TRY(moe::launch_bwd_router_wgrad(da, offsets, r2p, x, dw_router, d.E, d.H, d.k, stream));
    return MOE_OK;
}

const char* moe_status_string(moe_status_t status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

}  // extern "C"
