// api.hip -- the C ABI of libmoe: validation, workspace layout, launches.
//
// Every entry point validates all of its arguments before enqueueing anything,
// never allocates and never synchronises; the workspace is carved into
// 256-byte aligned regions in a fixed order that moe_workspace_size() mirrors.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.hpp"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

moe_status dev_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Carves (or, with base == nullptr, only measures) the workspace.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base((char*)b) {}
    template <typename T>
    T* take(size_t n) {
        off = (off + 255) & ~(size_t)255;
        T* p = base ? (T*)(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
};

moe_status check_desc(const moe_desc* d) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
    if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", d->T);
    if (d->h <= 0 || d->H <= 0 || d->E <= 0 || d->K <= 0 || d->f <= 0)
        return fail(MOE_ERR_INVALID_ARG, "h, H, E, K and f must be positive");
    if (d->h % d->H != 0) return fail(MOE_ERR_INVALID_ARG, "h = %d is not a multiple of H = %d", d->h, d->H);
    if (d->K > d->E) return fail(MOE_ERR_INVALID_ARG, "K = %d > E = %d", d->K, d->E);
    if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
    if (d->score != MOE_SOFTMAX && d->score != MOE_SIGMOID) return fail(MOE_ERR_INVALID_ARG, "unknown score %d", d->score);
    if (d->act != MOE_SWIGLU && d->act != MOE_GELU) return fail(MOE_ERR_INVALID_ARG, "unknown act %d", d->act);
    if (d->n_shared != 0 && d->n_shared != 1) return fail(MOE_ERR_UNSUPPORTED, "n_shared must be 0 or 1");
    if (d->has_wo != 0 && d->has_wo != 1) return fail(MOE_ERR_INVALID_ARG, "has_wo must be 0 or 1");
    if (d->n_shared && d->H != 1) return fail(MOE_ERR_UNSUPPORTED, "a shared expert needs H = 1");
    if (d->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 256 experts per head", d->E);
    if (d->H > 256) return fail(MOE_ERR_UNSUPPORTED, "H = %d > 256 heads", d->H);
    if ((long)d->H * d->E > 4096) return fail(MOE_ERR_UNSUPPORTED, "H*E = %ld > 4096", (long)d->H * d->E);
    const int dd = d->h / d->H;
    if (dd % 8 != 0 || d->f % 8 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "d = h/H = %d and f = %d must be multiples of 8", dd, d->f);
    if ((long long)d->T * d->H * d->K > 0x3fffffffLL)
        return fail(MOE_ERR_UNSUPPORTED, "T*H*K = %lld assignments is too many", (long long)d->T * d->H * d->K);
    if (!(d->capacity_factor == d->capacity_factor)) return fail(MOE_ERR_INVALID_ARG, "capacity_factor is NaN");
    if (!(d->capacity_factor_eval == d->capacity_factor_eval))
        return fail(MOE_ERR_INVALID_ARG, "capacity_factor_eval is NaN");
    if (d->eval != 0 && d->eval != 1) return fail(MOE_ERR_INVALID_ARG, "eval must be 0 or 1");
    if (d->gate != MOE_GATE_TOPK && d->gate != MOE_GATE_HASH) return fail(MOE_ERR_INVALID_ARG, "unknown gate %d", d->gate);
    if (d->gate == MOE_GATE_HASH && d->K != 1) return fail(MOE_ERR_INVALID_ARG, "the hash gate needs K = 1");
    if (d->queue != MOE_QUEUE_TOKEN && d->queue != MOE_QUEUE_CHOICE)
        return fail(MOE_ERR_INVALID_ARG, "unknown queue order %d", d->queue);
    if (d->n_groups < 0) return fail(MOE_ERR_INVALID_ARG, "n_groups = %d < 0", d->n_groups);
    if (d->n_groups > 1) {
        if (d->gate != MOE_GATE_TOPK) return fail(MOE_ERR_INVALID_ARG, "a group limit needs the top-K gate");
        if (d->E % d->n_groups != 0)
            return fail(MOE_ERR_INVALID_ARG, "E = %d is not a multiple of n_groups = %d", d->E, d->n_groups);
        if (d->group_limit < 1 || d->group_limit > d->n_groups)
            return fail(MOE_ERR_INVALID_ARG, "group_limit = %d outside [1, n_groups = %d]", d->group_limit, d->n_groups);
        if ((long)d->group_limit * (d->E / d->n_groups) < d->K)
            return fail(MOE_ERR_INVALID_ARG, "K = %d > group_limit * E / n_groups", d->K);
    }
    return MOE_OK;
}

int esize(const moe_desc* d) { return d->dtype == MOE_BF16 ? 2 : 4; }

// C = CF * K * T / E rounded up; a value within 1e-6 (relative) of an integer
// is that integer.
int64_t capacity_of(const moe_desc* d) {
    const float cf = d->eval ? d->capacity_factor_eval : d->capacity_factor;
    if (cf <= 0.0f) return INT32_MAX;
    const double v = (double)cf * d->K * (double)d->T / d->E;
    const double nearest = floor(v + 0.5);
    const double slack = 1e-6 * (v > 1.0 ? v : 1.0);
    double c = (fabs(v - nearest) <= slack) ? nearest : ceil(v);
    if (c > (double)INT32_MAX) c = (double)INT32_MAX;
    return (int64_t)c;
}

struct Plan {
    int T, h, H, E, K, f, d, Et, A, esz;
    int64_t cap;
    int max_rows;
    int route_nbx;
    int nch;
};

Plan plan_of(const moe_desc* d) {
    Plan p;
    p.T = d->T; p.h = d->h; p.H = d->H; p.E = d->E; p.K = d->K; p.f = d->f;
    p.d = d->h / d->H;
    p.Et = d->H * d->E;
    p.A = d->T * d->H * d->K;
    p.esz = esize(d);
    p.cap = capacity_of(d);
    const int64_t byc = p.cap >= INT32_MAX ? (int64_t)p.A : (int64_t)p.Et * p.cap;
    p.max_rows = (int)(byc < p.A ? byc : p.A);
    p.route_nbx = route_blocks(d->T, d->E, d->dtype);
    p.nch = permute_chunks(p.A);
    return p;
}

struct RouteWs { float* prob_part; };
RouteWs carve_route(Carver& c, const Plan& p) {
    RouteWs w;
    w.prob_part = c.take<float>((size_t)p.H * p.route_nbx * p.E + 1);
    return w;
}
int32_t* carve_permute(Carver& c, const Plan& p) { return c.take<int32_t>((size_t)p.nch * p.Et + 1); }
GemmTile* carve_ffn(Carver& c, const Plan& p, int dtype) {
    return c.take<GemmTile>(ffn_workspace_bytes(p.Et, p.max_rows, dtype) / sizeof(GemmTile) + 1);
}

struct LayerWs {
    int32_t *topk_idx, *counts, *kept, *offsets, *dest_row, *src_token, *hist, *off_sh, *off_wo;
    float *topk_w, *prob_part, *prob_mean;
    GemmTile *tiles, *tiles_sh, *tiles_wo;
    void *h_tmp, *y_perm, *h_sh, *y_sh, *y_cat;
};

LayerWs carve_layer(Carver& c, const Plan& p, const moe_desc* d) {
    LayerWs w{};
    w.topk_idx = c.take<int32_t>((size_t)p.A + 1);
    w.topk_w = c.take<float>((size_t)p.A + 1);
    w.counts = c.take<int32_t>(p.Et);
    w.prob_part = c.take<float>((size_t)p.H * p.route_nbx * p.E + 1);
    w.prob_mean = c.take<float>(p.Et);
    w.kept = c.take<int32_t>(p.Et);
    w.offsets = c.take<int32_t>(p.Et + 1);
    w.hist = c.take<int32_t>((size_t)p.nch * p.Et + 1);
    w.dest_row = c.take<int32_t>((size_t)p.A + 1);
    w.src_token = c.take<int32_t>((size_t)p.A + 1);
    w.tiles = carve_ffn(c, p, d->dtype);
    w.h_tmp = c.take<char>((size_t)p.max_rows * p.f * p.esz + 16);
    w.y_perm = c.take<char>((size_t)p.max_rows * p.d * p.esz + 16);
    if (d->n_shared) {
        w.h_sh = c.take<char>((size_t)p.T * p.f * p.esz + 16);
        w.y_sh = c.take<char>((size_t)p.T * p.h * p.esz + 16);
        w.off_sh = c.take<int32_t>(2);
        w.tiles_sh = c.take<GemmTile>(ffn_workspace_bytes(1, p.T, d->dtype) / sizeof(GemmTile) + 1);
    }
    if (d->has_wo) {
        w.y_cat = c.take<char>((size_t)p.T * p.h * p.esz + 16);
        w.off_wo = c.take<int32_t>(2);
        w.tiles_wo = c.take<GemmTile>(ffn_workspace_bytes(1, p.T, d->dtype) / sizeof(GemmTile) + 1);
    }
    return w;
}

moe_status check_ws(void* ws, size_t have, size_t need) {
    if (need == 0) return MOE_OK;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (((uintptr_t)ws & 255) != 0) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    return MOE_OK;
}

size_t ws_bytes_of(const moe_desc* d, int kind) {
    const Plan p = plan_of(d);
    Carver c(nullptr);
    switch (kind) {
        case MOE_WS_ROUTE: carve_route(c, p); break;
        case MOE_WS_PERMUTE: carve_permute(c, p); break;
        case MOE_WS_FFN: carve_ffn(c, p, d->dtype); break;
        default: carve_layer(c, p, d); break;
    }
    return c.off + 256;
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "libmoe 0.1 (gfx950)"; }

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

int32_t moe_capacity(const moe_desc* d) {
    if (check_desc(d) != MOE_OK) return -1;
    return (int32_t)capacity_of(d);
}

moe_status moe_workspace_size(const moe_desc* d, int32_t kind, size_t* bytes) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    if (kind < MOE_WS_LAYER || kind > MOE_WS_FFN) return fail(MOE_ERR_INVALID_ARG, "unknown workspace kind %d", kind);
    *bytes = ws_bytes_of(d, kind);
    return MOE_OK;
}

moe_status moe_route(const moe_desc* d, const void* x, const void* w_router, const float* logit_bias,
                     const float* select_bias, float* logits, uint32_t flags, int32_t* topk_idx,
                     float* topk_w, int32_t* counts, float* prob_mean, void* ws, size_t ws_bytes,
                     void* stream) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (flags & ~(MOE_LOGITS_IN | MOE_LOGITS_OUT)) return fail(MOE_ERR_INVALID_ARG, "unknown route flags 0x%x", flags);
    if ((flags & MOE_LOGITS_IN) && (flags & MOE_LOGITS_OUT))
        return fail(MOE_ERR_INVALID_ARG, "MOE_LOGITS_IN and MOE_LOGITS_OUT are exclusive");
    if (d->gate == MOE_GATE_HASH) return fail(MOE_ERR_INVALID_ARG, "the hash gate routes with moe_route_hash");
    if (d->T == 0) return MOE_OK;
    if ((flags & (MOE_LOGITS_IN | MOE_LOGITS_OUT)) && !logits)
        return fail(MOE_ERR_INVALID_ARG, "logits is NULL but a logits flag is set");
    if (!(flags & MOE_LOGITS_IN) && (!x || !w_router)) return fail(MOE_ERR_INVALID_ARG, "x or w_router is NULL");
    if (!topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "topk_idx or topk_w is NULL");
    const Plan p = plan_of(d);
    const size_t need = ws_bytes_of(d, MOE_WS_ROUTE);
    if (prob_mean && (s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    Carver c(ws);
    RouteWs w = prob_mean ? carve_route(c, p) : RouteWs{nullptr};
    hipError_t e;
    if (counts && (e = launch_fill_i32(counts, p.Et, 0, st)) != hipSuccess) return dev_fail(e, "fill");
    RouteArgs a{};
    a.T = d->T; a.h = d->h; a.H = d->H; a.E = d->E; a.K = d->K; a.dtype = d->dtype; a.score = d->score;
    a.n_groups = d->n_groups > 1 ? d->n_groups : 1; a.group_limit = d->group_limit;
    a.flags = flags; a.x = x; a.w_router = w_router; a.logit_bias = logit_bias;
    a.select_bias = d->score == MOE_SIGMOID ? select_bias : nullptr;
    a.logits = logits; a.topk_idx = topk_idx; a.topk_w = topk_w; a.counts = counts; a.prob_part = w.prob_part;
    if ((e = launch_route(a, st)) != hipSuccess) return dev_fail(e, "route kernel");
    if (prob_mean && (e = launch_prob_mean(w.prob_part, p.route_nbx, p.H, p.E, p.T, prob_mean, st)) != hipSuccess)
        return dev_fail(e, "prob_mean kernel");
    return MOE_OK;
}

moe_status moe_route_hash(const moe_desc* d, const int32_t* hash_keys, int32_t* topk_idx, float* topk_w,
                          int32_t* counts, void* stream) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (d->gate != MOE_GATE_HASH) return fail(MOE_ERR_INVALID_ARG, "desc->gate is not MOE_GATE_HASH");
    if (d->T == 0) return MOE_OK;
    if (!topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "topk_idx or topk_w is NULL");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (counts && (e = launch_fill_i32(counts, d->H * d->E, 0, st)) != hipSuccess) return dev_fail(e, "fill");
    if ((e = launch_route_hash(hash_keys, d->T, d->H, d->E, topk_idx, topk_w, counts, st)) != hipSuccess)
        return dev_fail(e, "hash route kernel");
    return MOE_OK;
}

moe_status moe_permute(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t capacity,
                       int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* dest_row,
                       int32_t* src_token, void* x_perm, int32_t* n_kept, void* ws, size_t ws_bytes,
                       void* stream) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (capacity < 0) return fail(MOE_ERR_INVALID_ARG, "capacity = %d < 0", capacity);
    if (!counts || !kept || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts, kept or offsets is NULL");
    const Plan p = plan_of(d);
    if (p.A > 0 && (!topk_idx || !dest_row || !src_token))
        return fail(MOE_ERR_INVALID_ARG, "topk_idx, dest_row or src_token is NULL");
    if (x && !x_perm) return fail(MOE_ERR_INVALID_ARG, "x given but x_perm is NULL");
    const size_t need = ws_bytes_of(d, MOE_WS_PERMUTE);
    if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
    Carver c(ws);
    PermuteArgs a{};
    a.A = p.A; a.K = p.K; a.H = p.H; a.Et = p.Et; a.d = p.d; a.h = p.h; a.dtype = d->dtype;
    a.capacity = capacity; a.queue = d->queue; a.topk_idx = topk_idx; a.x = x; a.counts = counts; a.kept = kept;
    a.offsets = offsets; a.dest_row = dest_row; a.src_token = src_token; a.x_perm = x_perm;
    a.n_kept = n_kept; a.hist = carve_permute(c, p);
    const int64_t byc = capacity >= INT32_MAX ? (int64_t)p.A : (int64_t)p.Et * capacity;
    a.max_rows = (int)(byc < p.A ? byc : p.A);
    hipError_t e = launch_permute(a, (hipStream_t)stream);
    if (e != hipSuccess) return dev_fail(e, "permute kernels");
    return MOE_OK;
}

static moe_status grouped_ffn(const moe_desc* d, const void* x_perm, const int32_t* src_rows,
                              const int32_t* offsets, int32_t max_rows, const void* w_gate, const void* w_up,
                              const void* w_down, void* h_tmp, void* y_perm, uint32_t flags, void* ws,
                              size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    const Plan p = plan_of(d);
    if (flags & ~(MOE_FFN_GEMM1 | MOE_FFN_GEMM2)) return fail(MOE_ERR_INVALID_ARG, "unknown ffn flags 0x%x", flags);
    if (max_rows < 0 || max_rows > p.A)
        return fail(MOE_ERR_INVALID_ARG, "max_rows = %d outside [0, T*H*K = %d]", max_rows, p.A);
    if (max_rows == 0) return MOE_OK;
    const uint32_t fl = flags ? flags : (MOE_FFN_GEMM1 | MOE_FFN_GEMM2);
    if (!offsets || !h_tmp) return fail(MOE_ERR_INVALID_ARG, "offsets or h_tmp is NULL");
    if ((fl & MOE_FFN_GEMM1) && (!x_perm || !w_gate || (d->act == MOE_SWIGLU && !w_up)))
        return fail(MOE_ERR_INVALID_ARG, "x_perm, w_gate or w_up is NULL");
    if ((fl & MOE_FFN_GEMM2) && (!w_down || !y_perm)) return fail(MOE_ERR_INVALID_ARG, "w_down or y_perm is NULL");
    Plan q = p;
    q.max_rows = max_rows;
    Carver cm(nullptr);
    carve_ffn(cm, q, d->dtype);
    if ((s = check_ws(ws, ws_bytes, cm.off + 256)) != MOE_OK) return s;
    Carver c(ws);
    FfnArgs a{};
    a.G = p.Et; a.d = p.d; a.f = p.f; a.dtype = d->dtype; a.act = d->act; a.max_rows = max_rows;
    a.x_perm = x_perm; a.offsets = offsets; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down;
    a.h_tmp = h_tmp; a.y_perm = y_perm; a.flags = fl; a.tiles = carve_ffn(c, q, d->dtype);
    a.src_rows = src_rows; a.a_nrows = p.T * p.H;
    hipError_t e = launch_ffn(a, (hipStream_t)stream);
    if (e != hipSuccess) return dev_fail(e, "grouped ffn kernels");
    return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_desc* d, const void* x_perm, const int32_t* offsets, int32_t max_rows,
                           const void* w_gate, const void* w_up, const void* w_down, void* h_tmp,
                           void* y_perm, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
    return grouped_ffn(d, x_perm, nullptr, offsets, max_rows, w_gate, w_up, w_down, h_tmp, y_perm, flags, ws,
                       ws_bytes, stream);
}

moe_status moe_grouped_ffn_rows(const moe_desc* d, const void* x, const int32_t* src_token,
                                const int32_t* offsets, int32_t max_rows, const void* w_gate, const void* w_up,
                                const void* w_down, void* h_tmp, void* y_perm, uint32_t flags, void* ws,
                                size_t ws_bytes, void* stream) {
    if (!src_token && max_rows > 0 && (!flags || (flags & MOE_FFN_GEMM1))) {
        g_err[0] = 0;
        return fail(MOE_ERR_INVALID_ARG, "src_token is NULL");
    }
    return grouped_ffn(d, x, src_token, offsets, max_rows, w_gate, w_up, w_down, h_tmp, y_perm, flags, ws,
                       ws_bytes, stream);
}

moe_status moe_combine(const moe_desc* d, const int32_t* dest_row, const float* topk_w, const void* y_perm,
                       const void* y_shared, void* y, void* stream) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (d->T == 0) return MOE_OK;
    if (!dest_row || !topk_w || !y) return fail(MOE_ERR_INVALID_ARG, "dest_row, topk_w or y is NULL");
    if (y_shared && d->H != 1) return fail(MOE_ERR_UNSUPPORTED, "y_shared needs H = 1");
    CombineArgs a{};
    a.T = d->T; a.H = d->H; a.K = d->K; a.d = d->h / d->H; a.h = d->h; a.dtype = d->dtype;
    a.dest_row = dest_row; a.topk_w = topk_w; a.y_perm = y_perm; a.y_shared = y_shared; a.y = y;
    hipError_t e = launch_combine(a, (hipStream_t)stream);
    if (e != hipSuccess) return dev_fail(e, "combine kernel");
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_desc* d, const moe_weights* w, const void* x, void* y, moe_aux* aux,
                             void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    if (d->T == 0) return MOE_OK;
    if (!x || !y) return fail(MOE_ERR_INVALID_ARG, "x or y is NULL");
    if ((d->gate == MOE_GATE_TOPK && !w->w_router) || !w->w_gate || !w->w_down || (d->act == MOE_SWIGLU && !w->w_up))
        return fail(MOE_ERR_INVALID_ARG, "a routed-expert or router weight is NULL");
    if (d->n_shared && (!w->sh_gate || !w->sh_down || (d->act == MOE_SWIGLU && !w->sh_up)))
        return fail(MOE_ERR_INVALID_ARG, "a shared-expert weight is NULL");
    if (d->has_wo && !w->w_o) return fail(MOE_ERR_INVALID_ARG, "w_o is NULL");
    const size_t need = ws_bytes_of(d, MOE_WS_LAYER);
    if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;

    const Plan p = plan_of(d);
    hipStream_t st = (hipStream_t)stream;
    Carver c(ws);
    LayerWs L = carve_layer(c, p, d);
    int32_t* topk_idx = aux && aux->topk_idx ? aux->topk_idx : L.topk_idx;
    float* topk_w = aux && aux->topk_w ? aux->topk_w : L.topk_w;
    int32_t* dest_row = aux && aux->dest_row ? aux->dest_row : L.dest_row;
    int32_t* counts = aux && aux->counts ? aux->counts : L.counts;
    const bool want_stats = aux && (aux->f || aux->P || aux->l_aux || aux->kept || aux->n_kept || aux->n_dropped);
    hipError_t e;

    if (d->gate == MOE_GATE_HASH) {
        // no router and no scores: P (and so L_aux) is zero
        if ((e = launch_route_hash(w->hash_keys, p.T, p.H, p.E, topk_idx, topk_w, nullptr, st)) != hipSuccess)
            return dev_fail(e, "hash route kernel");
        if (want_stats && (e = launch_fill_i32((int32_t*)L.prob_mean, p.Et, 0, st)) != hipSuccess)
            return dev_fail(e, "fill");
    } else {
        RouteArgs ra{};
        ra.T = p.T; ra.h = p.h; ra.H = p.H; ra.E = p.E; ra.K = p.K; ra.dtype = d->dtype; ra.score = d->score;
        ra.n_groups = d->n_groups > 1 ? d->n_groups : 1; ra.group_limit = d->group_limit;
        ra.flags = 0; ra.x = x; ra.w_router = w->w_router; ra.logit_bias = w->logit_bias;
        ra.select_bias = d->score == MOE_SIGMOID ? w->select_bias : nullptr;
        ra.logits = nullptr; ra.topk_idx = topk_idx; ra.topk_w = topk_w; ra.counts = nullptr;
        ra.prob_part = want_stats ? L.prob_part : nullptr;
        if ((e = launch_route(ra, st)) != hipSuccess) return dev_fail(e, "route kernel");
        if (want_stats && (e = launch_prob_mean(L.prob_part, p.route_nbx, p.H, p.E, p.T, L.prob_mean, st)) != hipSuccess)
            return dev_fail(e, "prob_mean kernel");
    }

    PermuteArgs pa{};
    pa.A = p.A; pa.K = p.K; pa.H = p.H; pa.Et = p.Et; pa.d = p.d; pa.h = p.h; pa.dtype = d->dtype;
    pa.capacity = (int)p.cap; pa.queue = d->queue; pa.topk_idx = topk_idx; pa.x = x; pa.counts = counts; pa.kept = L.kept;
    // no row gather: the gate/up GEMM reads its rows of x through src_token
    pa.offsets = L.offsets; pa.dest_row = dest_row; pa.src_token = L.src_token; pa.x = nullptr;
    pa.x_perm = nullptr; pa.n_kept = nullptr; pa.hist = L.hist; pa.max_rows = p.max_rows;
    if ((e = launch_permute(pa, st)) != hipSuccess) return dev_fail(e, "permute kernels");

    FfnArgs fa{};
    fa.G = p.Et; fa.d = p.d; fa.f = p.f; fa.dtype = d->dtype; fa.act = d->act; fa.max_rows = p.max_rows;
    fa.x_perm = x; fa.src_rows = L.src_token; fa.a_nrows = p.T * p.H;
    fa.offsets = L.offsets; fa.w_gate = w->w_gate; fa.w_up = w->w_up;
    fa.w_down = w->w_down; fa.h_tmp = L.h_tmp; fa.y_perm = L.y_perm; fa.flags = 0; fa.tiles = L.tiles;
    if ((e = launch_ffn(fa, st)) != hipSuccess) return dev_fail(e, "grouped ffn kernels");

    if (d->n_shared) {
        if ((e = launch_set2(L.off_sh, 0, p.T, st)) != hipSuccess) return dev_fail(e, "offsets kernel");
        FfnArgs sa{};
        sa.G = 1; sa.d = p.h; sa.f = p.f; sa.dtype = d->dtype; sa.act = d->act; sa.max_rows = p.T;
        sa.x_perm = x; sa.offsets = L.off_sh; sa.w_gate = w->sh_gate; sa.w_up = w->sh_up;
        sa.w_down = w->sh_down; sa.h_tmp = L.h_sh; sa.y_perm = L.y_sh; sa.flags = 0; sa.tiles = L.tiles_sh;
        if ((e = launch_ffn(sa, st)) != hipSuccess) return dev_fail(e, "shared expert kernels");
    }

    CombineArgs ca{};
    ca.T = p.T; ca.H = p.H; ca.K = p.K; ca.d = p.d; ca.h = p.h; ca.dtype = d->dtype;
    ca.dest_row = dest_row; ca.topk_w = topk_w; ca.y_perm = L.y_perm;
    ca.y_shared = d->n_shared ? L.y_sh : nullptr;
    ca.y = d->has_wo ? L.y_cat : y;
    if ((e = launch_combine(ca, st)) != hipSuccess) return dev_fail(e, "combine kernel");

    if (d->has_wo && (e = launch_dense(p.T, p.h, p.h, d->dtype, L.y_cat, w->w_o, y, L.tiles_wo, L.off_wo, st)) != hipSuccess)
        return dev_fail(e, "output projection kernel");

    if (want_stats) {
        StatsArgs sa{};
        sa.T = p.T; sa.H = p.H; sa.E = p.E; sa.K = p.K; sa.A = p.A; sa.alpha = d->aux_alpha;
        sa.counts = counts; sa.kept_in = L.kept; sa.offsets = L.offsets; sa.prob_mean = L.prob_mean;
        sa.f = aux->f; sa.P = aux->P; sa.l_aux = aux->l_aux; sa.n_kept = aux->n_kept;
        sa.n_dropped = aux->n_dropped; sa.kept_out = aux->kept;
        if ((e = launch_stats(sa, st)) != hipSuccess) return dev_fail(e, "stats kernel");
    }
    return MOE_OK;
}

}  // extern "C"
