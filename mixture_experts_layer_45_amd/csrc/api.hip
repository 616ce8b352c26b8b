// api.hip -- the C ABI of libmoe: validation, workspace layout, launches.
//
// Every entry point validates all of its arguments before enqueueing anything,
// never allocates and never synchronises; the workspace is carved into
// 256-byte aligned regions in a fixed order that moe_workspace_size() mirrors.
#include <math.h>
#include <stdarg.h>

#include <algorithm>
#include <mutex>
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
    if (d->packed != 0 && d->packed != 1) return fail(MOE_ERR_INVALID_ARG, "packed must be 0 or 1");
    if (d->packed) {
        // fragment-ordered weights are read by the 4-wave and 64-wide kernels
        // alone: bf16, contraction lengths and output widths multiples of 64,
        // every operand under 2 GB (32-bit buffer offsets)
        if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "packed weights need MOE_BF16");
        if (dd % 64 || d->f % 64)
            return fail(MOE_ERR_UNSUPPORTED, "packed weights need d = %d and f = %d to be multiples of 64", dd, d->f);
        const long long lim = 1ll << 31;
        const long long f = d->f, h = d->h;
        if ((long long)d->T * h * 2 >= lim || (long long)d->T * d->H * d->K * f * 2 >= lim || f * dd * 2 >= lim ||
            (d->n_shared && (f * h * 2 >= lim || (long long)d->T * f * 2 >= lim)) || (d->has_wo && h * h * 2 >= lim))
            return fail(MOE_ERR_UNSUPPORTED, "packed weights need every GEMM operand under 2 GB");
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
    p.route_nbx = route_blocks(d->T, d->h, d->H, d->E, d->dtype);
    p.nch = permute_chunks(p.A);
    return p;
}

// route partials of P up to this size are summed by the stats kernel (one
// block) rather than by their own launch
constexpr size_t kFoldPartials = 65536;

struct RouteWs { float* prob_part; void* split; };
RouteWs carve_route(Carver& c, const Plan& p, int dtype) {
    RouteWs w;
    w.prob_part = c.take<float>((size_t)p.H * p.route_nbx * p.E + 1);
    const size_t sb = route_split_ws_bytes(p.T, p.h, p.H, p.E, dtype);
    w.split = sb ? c.take<char>(sb) : nullptr;
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
    void* route_split;
};

LayerWs carve_layer(Carver& c, const Plan& p, const moe_desc* d) {
    LayerWs w{};
    w.topk_idx = c.take<int32_t>((size_t)p.A + 1);
    w.topk_w = c.take<float>((size_t)p.A + 1);
    w.counts = c.take<int32_t>(p.Et);
    w.prob_part = c.take<float>((size_t)p.H * p.route_nbx * p.E + 1);
    {
        const size_t sb = route_split_ws_bytes(p.T, p.h, p.H, p.E, d->dtype);
        w.route_split = sb ? c.take<char>(sb) : nullptr;
    }
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

// ---- backward pass: sizes and workspace
struct BwdPlan {
    int NA, Ep, ms_h;
    long long Np_h;
    bool router, shared, wo;
};
BwdPlan bwd_plan_of(const moe_desc* d, const Plan& p) {
    BwdPlan b;
    b.NA = d->act == MOE_SWIGLU ? 2 : 1;
    b.Ep = (p.E + 63) / 64 * 64;
    const int tst = (p.T + 63) / 64;
    b.ms_h = p.H * (tst + 1);
    b.Np_h = 64ll * b.ms_h;
    b.router = d->gate == MOE_GATE_TOPK;
    b.shared = d->n_shared != 0;
    b.wo = d->has_wo != 0;
    return b;
}

struct BwdWs {
    int2* kspan_h;
    int32_t *stage_h, *off_T, *off_h, *off_w, *off_f, *off_E, *off_hr, *off_fr;
    void* wgT;
    void *dcat, *dYp, *dAU, *dXp, *dl, *dxr, *dAUs, *dxs;
    float* dw;
    void *xp, *dlT, *xhT;
    GemmTile* tiles;
};

size_t bwd_tiles_bytes(const Plan& p, const BwdPlan& b) {
    size_t m = 0;
    auto upd = [&](int G, long long rows) { m = std::max(m, grouped_gemm_ws_bytes(G, (int)std::min(rows, (long long)INT32_MAX))); };
    upd(p.Et, p.max_rows);
    upd(p.Et, (long long)p.Et * p.d);
    upd(p.Et, (long long)p.Et * p.f);
    if (b.router) {
        upd(p.H, (long long)p.H * p.T);
        upd(p.H, (long long)p.H * p.E);
    }
    if (b.shared || b.wo) {
        upd(1, p.T);
        upd(1, p.h);
        upd(1, p.f);
    }
    return m + 256;
}

BwdWs carve_bwd(Carver& c, const Plan& p, const BwdPlan& b) {
    BwdWs w{};
    const size_t e2 = 2;  // bf16
    const size_t N = p.max_rows, T = p.T, S = (size_t)p.T * p.H, nf = (size_t)b.NA * p.f;
    w.kspan_h = c.take<int2>(p.H);
    w.stage_h = c.take<int32_t>(b.ms_h);
    w.off_T = c.take<int32_t>(2);
    w.off_h = c.take<int32_t>(p.H + 1);
    w.off_w = c.take<int32_t>(p.Et + 1);
    w.off_f = c.take<int32_t>(p.Et + 1);
    w.off_E = c.take<int32_t>(p.H + 1);
    w.off_hr = c.take<int32_t>(2);
    w.off_fr = c.take<int32_t>(2);
    w.dYp = c.take<char>(N * p.d * e2 + 16);
    w.dw = c.take<float>((size_t)p.A + 1);
    w.dAU = c.take<char>(N * nf * e2 + 16);
    w.dXp = c.take<char>(N * p.d * e2 + 16);
    w.xp = c.take<char>(N * p.d * e2 + 16);
    if (b.router) {
        w.wgT = c.take<char>((size_t)p.H * p.d * b.Ep * e2);
        w.dl = c.take<char>(S * b.Ep * e2);
        w.dxr = c.take<char>(S * p.d * e2 + 16);
        w.dlT = c.take<char>((size_t)b.Ep * b.Np_h * e2);
        w.xhT = c.take<char>((size_t)p.d * b.Np_h * e2);
    }
    if (b.wo) {
        w.dcat = c.take<char>(T * p.h * e2 + 16);
    }
    if (b.shared) {
        w.dAUs = c.take<char>(T * nf * e2 + 16);
        w.dxs = c.take<char>(T * p.h * e2 + 16);
    }
    w.tiles = c.take<GemmTile>(bwd_tiles_bytes(p, b) / sizeof(GemmTile) + 1);
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
        case MOE_WS_ROUTE: carve_route(c, p, d->dtype); break;
        case MOE_WS_PERMUTE: carve_permute(c, p); break;
        case MOE_WS_FFN: carve_ffn(c, p, d->dtype); break;
        case MOE_WS_BACKWARD: carve_bwd(c, p, bwd_plan_of(d, p)); break;
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
    if (kind < MOE_WS_LAYER || kind > MOE_WS_BACKWARD) return fail(MOE_ERR_INVALID_ARG, "unknown workspace kind %d", kind);
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
    // a workspace is needed for P and for the split router GEMM of many experts
    const bool need_ws = prob_mean || route_split_ws_bytes(p.T, p.h, p.H, p.E, d->dtype) > 0;
    if (need_ws && (s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    Carver c(ws);
    RouteWs w = need_ws ? carve_route(c, p, d->dtype) : RouteWs{nullptr, nullptr};
    if (!prob_mean) w.prob_part = nullptr;
    hipError_t e;
    if (counts && (e = launch_fill_i32(counts, p.Et, 0, st)) != hipSuccess) return dev_fail(e, "fill");
    RouteArgs a{};
    a.T = d->T; a.h = d->h; a.H = d->H; a.E = d->E; a.K = d->K; a.dtype = d->dtype; a.score = d->score;
    a.n_groups = d->n_groups > 1 ? d->n_groups : 1; a.group_limit = d->group_limit;
    a.flags = flags; a.x = x; a.w_router = w_router; a.logit_bias = logit_bias;
    a.select_bias = d->score == MOE_SIGMOID ? select_bias : nullptr;
    a.logits = logits; a.topk_idx = topk_idx; a.topk_w = topk_w; a.counts = counts; a.prob_part = w.prob_part;
    a.split_ws = w.split;
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

}  // extern "C"

namespace {

// argument checks shared by moe_permute and moe_permute_noalloc
moe_status check_permute(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t capacity,
                         const int32_t* counts, const int32_t* kept, const int32_t* offsets, const int32_t* dest_row,
                         const int32_t* src_token, const void* x_perm) {
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (capacity < 0) return fail(MOE_ERR_INVALID_ARG, "capacity = %d < 0", capacity);
    if (!counts || !kept || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts, kept or offsets is NULL");
    const Plan p = plan_of(d);
    if (p.A > 0 && (!topk_idx || !dest_row || !src_token))
        return fail(MOE_ERR_INVALID_ARG, "topk_idx, dest_row or src_token is NULL");
    if (x && !x_perm) return fail(MOE_ERR_INVALID_ARG, "x given but x_perm is NULL");
    return MOE_OK;
}

moe_status run_permute(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t capacity, int32_t* counts,
                       int32_t* kept, int32_t* offsets, int32_t* dest_row, int32_t* src_token, void* x_perm,
                       int32_t* n_kept, int32_t* hist, hipStream_t stream) {
    const Plan p = plan_of(d);
    PermuteArgs a{};
    a.A = p.A; a.K = p.K; a.H = p.H; a.Et = p.Et; a.d = p.d; a.h = p.h; a.dtype = d->dtype;
    a.capacity = capacity; a.queue = d->queue; a.topk_idx = topk_idx; a.x = x; a.counts = counts; a.kept = kept;
    a.offsets = offsets; a.dest_row = dest_row; a.src_token = src_token; a.x_perm = x_perm;
    a.n_kept = n_kept; a.hist = hist;
    const int64_t byc = capacity >= INT32_MAX ? (int64_t)p.A : (int64_t)p.Et * capacity;
    a.max_rows = (int)(byc < p.A ? byc : p.A);
    hipError_t e = launch_permute(a, stream);
    if (e != hipSuccess) return dev_fail(e, "permute kernels");
    return MOE_OK;
}

// The scratch of moe_permute_noalloc: the per-chunk histogram [nch][H*E] int32
// (nch = ceil(T*H*K / 1024)), at most kScratchInts entries.  One copy per GPU,
// alive until the process ends, shared by every call on that GPU.  Nothing in
// it has to start at zero (the histogram kernel writes every entry the scan
// and rank kernels read).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchInts = (size_t)1 << 20;  // 4 MiB
__device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_of_current_device(int32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return dev_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = (int32_t*)g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_permute(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t capacity,
                       int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* dest_row,
                       int32_t* src_token, void* x_perm, int32_t* n_kept, void* ws, size_t ws_bytes,
                       void* stream) {
    g_err[0] = 0;
    moe_status s = check_permute(d, topk_idx, x, capacity, counts, kept, offsets, dest_row, src_token, x_perm);
    if (s != MOE_OK) return s;
    const size_t need = ws_bytes_of(d, MOE_WS_PERMUTE);
    if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
    Carver c(ws);
    const Plan p = plan_of(d);
    return run_permute(d, topk_idx, x, capacity, counts, kept, offsets, dest_row, src_token, x_perm, n_kept,
                       carve_permute(c, p), (hipStream_t)stream);
}

size_t moe_permute_noalloc_max_ints(void) { return kScratchInts; }

moe_status moe_permute_noalloc(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t capacity,
                               int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* dest_row,
                               int32_t* src_token, void* x_perm, int32_t* n_kept, void* stream) {
    g_err[0] = 0;
    moe_status s = check_permute(d, topk_idx, x, capacity, counts, kept, offsets, dest_row, src_token, x_perm);
    if (s != MOE_OK) return s;
    const Plan p = plan_of(d);
    const size_t need = (size_t)p.nch * p.Et + 1;
    if (need > kScratchInts)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_permute_noalloc: the histogram needs %zu int32 (ceil(T*H*K/1024) * H*E + 1), more than the "
                    "%zu of its static scratch; use moe_permute with a workspace",
                    need, kScratchInts);
    int32_t* hist = nullptr;
    if ((s = scratch_of_current_device(&hist)) != MOE_OK) return s;
    return run_permute(d, topk_idx, x, capacity, counts, kept, offsets, dest_row, src_token, x_perm, n_kept, hist,
                       (hipStream_t)stream);
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
    if (d->packed && ((((fl & MOE_FFN_GEMM1) ? (uintptr_t)h_tmp : 0) | ((fl & MOE_FFN_GEMM2) ? (uintptr_t)y_perm : 0)) & 15))
        return fail(MOE_ERR_INVALID_ARG, "packed weights need h_tmp and y_perm 16-byte aligned");
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
    a.src_rows = src_rows; a.a_nrows = p.T * p.H; a.packed = d->packed;
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
    // any kept row is read from y_perm, and whether one is kept is known only on
    // the device: a NULL y_perm is refused whenever there are assignments
    if (!dest_row || !topk_w || !y_perm || !y) return fail(MOE_ERR_INVALID_ARG, "dest_row, topk_w, y_perm or y is NULL");
    if (y_shared && d->H != 1) return fail(MOE_ERR_UNSUPPORTED, "y_shared needs H = 1");
    CombineArgs a{};
    a.T = d->T; a.H = d->H; a.K = d->K; a.d = d->h / d->H; a.h = d->h; a.dtype = d->dtype;
    a.dest_row = dest_row; a.topk_w = topk_w; a.y_perm = y_perm; a.y_shared = y_shared; a.y = y;
    hipError_t e = launch_combine(a, (hipStream_t)stream);
    if (e != hipSuccess) return dev_fail(e, "combine kernel");
    return MOE_OK;
}

static moe_status layer_forward(const moe_desc* d, const moe_weights* w, const void* x, void* y, moe_aux* aux,
                                const moe_saved* sv, void* ws, size_t ws_bytes, void* stream) {
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
    if (d->packed && d->has_wo && ((uintptr_t)y & 15))
        return fail(MOE_ERR_INVALID_ARG, "packed weights with W_o need y 16-byte aligned");
    const size_t need = ws_bytes_of(d, MOE_WS_LAYER);
    if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;

    const Plan p = plan_of(d);
    hipStream_t st = (hipStream_t)stream;
    Carver c(ws);
    LayerWs L = carve_layer(c, p, d);
    if (sv) {  // training: the state the backward pass reads lands in the caller's buffers
        L.topk_idx = sv->topk_idx;
        L.topk_w = sv->topk_w;
        L.dest_row = sv->dest_row;
        L.src_token = sv->src_token;
        L.offsets = sv->offsets;
        L.counts = sv->counts;
        L.h_tmp = sv->h;
        L.y_perm = sv->y_perm;
        if (d->n_shared) L.h_sh = sv->sh_h;
        if (d->has_wo) L.y_cat = sv->y_cat;
    }
    int32_t* topk_idx = aux && aux->topk_idx && !sv ? aux->topk_idx : L.topk_idx;
    float* topk_w = aux && aux->topk_w && !sv ? aux->topk_w : L.topk_w;
    int32_t* dest_row = aux && aux->dest_row && !sv ? aux->dest_row : L.dest_row;
    int32_t* counts = aux && aux->counts && !sv ? aux->counts : L.counts;
    const bool want_stats = aux && (aux->f || aux->P || aux->l_aux || aux->kept || aux->n_kept || aux->n_dropped);
    // few experts and small partial tables: the stats kernel sums P itself (one
    // launch fewer; measured on one MI355X: top-2 layer 10.5 -> 7.5 us, Zipf
    // top-1 12.9 -> 10.6 us; with 256 experts its one block is slower than the
    // P kernel's many)
    const bool fold_p = d->gate == MOE_GATE_TOPK && p.Et <= 64 && (size_t)p.route_nbx * p.Et <= kFoldPartials;
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
        ra.flags = sv ? MOE_LOGITS_OUT : 0; ra.x = x; ra.w_router = w->w_router; ra.logit_bias = w->logit_bias;
        ra.select_bias = d->score == MOE_SIGMOID ? w->select_bias : nullptr;
        ra.logits = sv ? sv->logits : nullptr; ra.topk_idx = topk_idx; ra.topk_w = topk_w; ra.counts = nullptr;
        ra.prob_part = want_stats ? L.prob_part : nullptr;
        ra.split_ws = L.route_split;
        if ((e = launch_route(ra, st)) != hipSuccess) return dev_fail(e, "route kernel");
        if (want_stats && !fold_p && (e = launch_prob_mean(L.prob_part, p.route_nbx, p.H, p.E, p.T, L.prob_mean, st)) != hipSuccess)
            return dev_fail(e, "prob_mean kernel");
    }

    PermuteArgs pa{};
    pa.A = p.A; pa.K = p.K; pa.H = p.H; pa.Et = p.Et; pa.d = p.d; pa.h = p.h; pa.dtype = d->dtype;
    pa.capacity = (int)p.cap; pa.queue = d->queue; pa.topk_idx = topk_idx; pa.x = x; pa.counts = counts; pa.kept = L.kept;
    // no row gather: the gate/up GEMM reads its rows of x through src_token
    pa.offsets = L.offsets; pa.dest_row = dest_row; pa.src_token = L.src_token; pa.x = nullptr;
    pa.x_perm = nullptr; pa.n_kept = nullptr; pa.hist = L.hist; pa.max_rows = p.max_rows;
    if ((e = launch_permute(pa, st)) != hipSuccess) return dev_fail(e, "permute kernels");

    // One slot per token (K = 1, one head, nothing added after the routed
    // sum): the gate weight is exactly 1 and a token has at most one row, so
    // the down GEMM's epilogue stores each expert row straight to its token's
    // row of y (lesson 10, item 3, the un-permute fused into the expert GEMM),
    // which is bitwise what the combine would write; tokens whose assignment
    // was dropped get 0.  The training forward keeps y_perm (the backward
    // reads it) and so the combine.
    const bool fused_combine = !sv && p.K == 1 && p.H == 1 && !d->n_shared && !d->has_wo && ((uintptr_t)y & 15) == 0;
    if (fused_combine && (e = launch_zero_dropped(dest_row, p.T, p.h * p.esz, y, st)) != hipSuccess)
        return dev_fail(e, "zero-dropped kernel");

    FfnArgs fa{};
    fa.G = p.Et; fa.d = p.d; fa.f = p.f; fa.dtype = d->dtype; fa.act = d->act; fa.max_rows = p.max_rows;
    fa.x_perm = x; fa.src_rows = L.src_token; fa.a_nrows = p.T * p.H;
    fa.offsets = L.offsets; fa.w_gate = w->w_gate; fa.w_up = w->w_up;
    fa.w_down = w->w_down; fa.h_tmp = L.h_tmp; fa.y_perm = fused_combine ? y : L.y_perm; fa.flags = 0;
    fa.tiles = L.tiles;
    fa.act_save = sv ? sv->act_grad : nullptr;
    fa.c_rows = fused_combine ? L.src_token : nullptr;
    fa.c_nrows = p.T;
    fa.packed = d->packed;
    if ((e = launch_ffn(fa, st)) != hipSuccess) return dev_fail(e, "grouped ffn kernels");

    if (d->n_shared) {
        if ((e = launch_set2(L.off_sh, 0, p.T, st)) != hipSuccess) return dev_fail(e, "offsets kernel");
        FfnArgs sa{};
        sa.G = 1; sa.d = p.h; sa.f = p.f; sa.dtype = d->dtype; sa.act = d->act; sa.max_rows = p.T;
        sa.x_perm = x; sa.offsets = L.off_sh; sa.w_gate = w->sh_gate; sa.w_up = w->sh_up;
        sa.w_down = w->sh_down; sa.h_tmp = L.h_sh; sa.y_perm = L.y_sh; sa.flags = 0; sa.tiles = L.tiles_sh;
        sa.act_save = sv ? sv->sh_act_grad : nullptr;
        sa.packed = d->packed;
        if ((e = launch_ffn(sa, st)) != hipSuccess) return dev_fail(e, "shared expert kernels");
    }

    if (!fused_combine) {
        CombineArgs ca{};
        ca.T = p.T; ca.H = p.H; ca.K = p.K; ca.d = p.d; ca.h = p.h; ca.dtype = d->dtype;
        ca.dest_row = dest_row; ca.topk_w = topk_w; ca.y_perm = L.y_perm;
        ca.y_shared = d->n_shared ? L.y_sh : nullptr;
        ca.y = d->has_wo ? L.y_cat : y;
        if ((e = launch_combine(ca, st)) != hipSuccess) return dev_fail(e, "combine kernel");
    }

    if (d->has_wo && (e = launch_dense(p.T, p.h, p.h, d->dtype, L.y_cat, w->w_o, y, L.tiles_wo, L.off_wo, st, d->packed)) != hipSuccess)
        return dev_fail(e, "output projection kernel");

    if (want_stats) {
        StatsArgs sa{};
        sa.T = p.T; sa.H = p.H; sa.E = p.E; sa.K = p.K; sa.A = p.A; sa.alpha = d->aux_alpha;
        sa.counts = counts; sa.kept_in = L.kept; sa.offsets = L.offsets;
        sa.prob_mean = fold_p ? nullptr : L.prob_mean;
        sa.prob_part = fold_p ? L.prob_part : nullptr;
        sa.nbx = p.route_nbx;
        sa.f = aux->f; sa.P = aux->P; sa.l_aux = aux->l_aux; sa.n_kept = aux->n_kept;
        sa.n_dropped = aux->n_dropped; sa.kept_out = aux->kept;
        if ((e = launch_stats(sa, st)) != hipSuccess) return dev_fail(e, "stats kernel");
    }
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_desc* d, const moe_weights* w, const void* x, void* y, moe_aux* aux,
                             void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    return layer_forward(d, w, x, y, aux, nullptr, ws, ws_bytes, stream);
}

moe_status moe_pack_weights(const void* w, void* w_packed, int64_t n_mat, int32_t n_out, int32_t k, void* stream) {
    g_err[0] = 0;
    if (n_mat < 0) return fail(MOE_ERR_INVALID_ARG, "n_mat = %lld < 0", (long long)n_mat);
    if (n_out <= 0 || n_out % 32 || k <= 0 || k % 16)
        return fail(MOE_ERR_INVALID_ARG, "n_out = %d must be a positive multiple of 32 and k = %d of 16", n_out, k);
    if (n_mat == 0) return MOE_OK;
    if (n_mat > (1ll << 60) / ((long long)n_out * k)) return fail(MOE_ERR_INVALID_ARG, "the matrices are too large");
    if (!w || !w_packed) return fail(MOE_ERR_INVALID_ARG, "w or w_packed is NULL");
    const uintptr_t bytes = (uintptr_t)n_mat * (uintptr_t)n_out * (uintptr_t)k * 2u;
    const uintptr_t a = (uintptr_t)w, b = (uintptr_t)w_packed;
    if ((a < b ? b - a : a - b) < bytes) return fail(MOE_ERR_INVALID_ARG, "w and w_packed overlap");
    if ((a | b) & 15) return fail(MOE_ERR_INVALID_ARG, "w and w_packed must be 16-byte aligned");
    hipError_t e = launch_pack_weights(w, w_packed, n_mat, n_out, k, (hipStream_t)stream);
    if (e != hipSuccess) return dev_fail(e, "pack kernel");
    return MOE_OK;
}

int32_t moe_max_rows(const moe_desc* d) {
    if (check_desc(d) != MOE_OK) return -1;
    return plan_of(d).max_rows;
}

// the training path runs its expert GEMMs on the 64-wide kernel: bf16 with
// every contraction length a multiple of 64
static moe_status check_training(const moe_desc* d) {
    moe_status s = check_desc(d);
    if (s != MOE_OK) return s;
    if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "training needs MOE_BF16");
    if (d->packed) return fail(MOE_ERR_UNSUPPORTED, "training reads row-major weights (packed = 0)");
    const int dd = d->h / d->H;
    if (dd % 64 || d->f % 64 || d->h % 64)
        return fail(MOE_ERR_UNSUPPORTED, "training needs d = %d, f = %d and h = %d to be multiples of 64", dd, d->f, d->h);
    return MOE_OK;
}

static moe_status check_saved(const moe_desc* d, const moe_saved* sv) {
    if (!sv) return fail(MOE_ERR_INVALID_ARG, "saved is NULL");
    if (!sv->topk_idx || !sv->topk_w || !sv->dest_row || !sv->src_token || !sv->offsets || !sv->counts ||
        !sv->act_grad || !sv->h || !sv->y_perm)
        return fail(MOE_ERR_INVALID_ARG, "a routing or expert buffer of saved is NULL");
    if (d->gate == MOE_GATE_TOPK && !sv->logits) return fail(MOE_ERR_INVALID_ARG, "saved->logits is NULL");
    if (d->n_shared && (!sv->sh_act_grad || !sv->sh_h)) return fail(MOE_ERR_INVALID_ARG, "saved shared-expert buffer is NULL");
    if (d->has_wo && !sv->y_cat) return fail(MOE_ERR_INVALID_ARG, "saved->y_cat is NULL");
    return MOE_OK;
}

moe_status moe_layer_forward_train(const moe_desc* d, const moe_weights* w, const void* x, void* y, moe_aux* aux,
                                   const moe_saved* saved, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    moe_status s = check_training(d);
    if (s != MOE_OK) return s;
    if (d->T == 0) return MOE_OK;
    if ((s = check_saved(d, saved)) != MOE_OK) return s;
    return layer_forward(d, w, x, y, aux, saved, ws, ws_bytes, stream);
}

moe_status moe_layer_backward(const moe_desc* d, const moe_weights* w, const void* x, const void* dy,
                              const moe_saved* sv, float aux_weight, moe_grads* gr, void* ws, size_t ws_bytes,
                              void* stream) {
    g_err[0] = 0;
    moe_status s = check_training(d);
    if (s != MOE_OK) return s;
    if (d->T == 0) return MOE_OK;
    if (!w || !x || !dy || !gr) return fail(MOE_ERR_INVALID_ARG, "weights, x, dy or grads is NULL");
    if ((s = check_saved(d, sv)) != MOE_OK) return s;
    if (!(aux_weight == aux_weight)) return fail(MOE_ERR_INVALID_ARG, "aux_weight is NaN");
    const bool router = d->gate == MOE_GATE_TOPK;
    if (!w->w_gate || !w->w_down || (d->act == MOE_SWIGLU && !w->w_up) || (router && !w->w_router))
        return fail(MOE_ERR_INVALID_ARG, "a routed-expert or router weight is NULL");
    if (d->n_shared && (!w->sh_gate || !w->sh_down || (d->act == MOE_SWIGLU && !w->sh_up)))
        return fail(MOE_ERR_INVALID_ARG, "a shared-expert weight is NULL");
    if (d->has_wo && !w->w_o) return fail(MOE_ERR_INVALID_ARG, "w_o is NULL");
    if (!gr->dx || !gr->w_gate || !gr->w_down || (d->act == MOE_SWIGLU && !gr->w_up) || (router && !gr->w_router) ||
        (d->n_shared && (!gr->sh_gate || !gr->sh_down || (d->act == MOE_SWIGLU && !gr->sh_up))) ||
        (d->has_wo && !gr->w_o))
        return fail(MOE_ERR_INVALID_ARG, "a gradient buffer of the layer is NULL");
    const Plan p = plan_of(d);
    const BwdPlan b = bwd_plan_of(d, p);
    // the 64-wide kernel addresses each operand through a 32-bit buffer range
    const long long lim = 1ll << 31;
    const long long nf = (long long)b.NA * p.f;
    if ((long long)p.max_rows * p.f * 2 >= lim || (long long)p.max_rows * nf * 2 >= lim ||
        (long long)p.max_rows * p.d * 2 >= lim || (long long)p.f * p.d * 2 >= lim || (long long)p.d * nf * 2 >= lim ||
        (long long)b.Ep * b.Np_h * 2 >= lim || (long long)p.d * b.Np_h * 2 >= lim || (long long)p.T * nf * 2 >= lim ||
        (long long)p.T * p.f * 2 >= lim || (long long)p.T * p.h * 2 >= lim || (b.wo && (long long)p.h * p.h * 2 >= lim))
        return fail(MOE_ERR_UNSUPPORTED, "an operand of the backward GEMMs exceeds 2 GB");
    const size_t need = ws_bytes_of(d, MOE_WS_BACKWARD);
    if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    Carver c(ws);
    BwdWs W = carve_bwd(c, p, b);
    hipError_t e;
#define MOE_TRY(call, what) \
    if ((e = (call)) != hipSuccess) return dev_fail(e, what)
    const int T = p.T, H = p.H, E = p.E, K = p.K, dd = p.d, f = p.f, h = p.h, Et = p.Et, N = p.max_rows;
    const int NA = b.NA;
    auto gemm = [&](int mode, const void* A, long long a_bytes, const void* B0, const void* B1, void* C, void* aux,
                    int Kc, int Nout, const int32_t* offs, int G, int rows, const int2* kspan, int a_mod,
                    int b_shared, const int32_t* a_rows) -> hipError_t {
        GemmSpec gs{};
        gs.A = A; gs.B0 = B0; gs.B1 = B1; gs.C = C; gs.aux = aux; gs.K = Kc; gs.Nout = Nout; gs.a_bytes = a_bytes;
        gs.a_rows = a_rows; gs.kspan = kspan; gs.a_mod = a_mod; gs.b_shared = b_shared;
        return launch_grouped_gemm(mode, gs, offs, G, rows, W.tiles, st);
    };
    // weight gradient: C rows [g*m, (g+1)*m) of group g = sum over its rows k in
    // [krows[g], krows[g+1]) of A[k][0:m]^T B[k][0:Nout] (A, B as stored)
    auto wgrad = [&](const void* A, long long a_bytes, int lda, int m, const void* B, long long b_bytes, int ldb, void* C,
                     int Nout, const int32_t* krows, const int32_t* c_offs, int G) -> hipError_t {
        GemmSpec gs{};
        gs.A = A; gs.B0 = B; gs.C = C; gs.K = 64; gs.Nout = Nout; gs.a_bytes = a_bytes; gs.a_mod = m;
        gs.kmajor = 2; gs.krows = krows; gs.lda = lda; gs.ldb = ldb; gs.b_bytes = b_bytes;
        return launch_grouped_gemm(GEMM_PLAIN, gs, c_offs, G, G * m, W.tiles, st);
    };
    // C = A B with B the forward weights as stored ([G][K][Nout]: the product by
    // their transpose); with B1, k rows >= kb1 are B1's
    auto gemm_t = [&](int mode, const void* A, long long a_bytes, const void* B0, const void* B1, int kb1, void* C,
                      void* aux, int Kc, int Nout, const int32_t* offs, int G, int rows) -> hipError_t {
        GemmSpec gs{};
        gs.A = A; gs.B0 = B0; gs.B1 = B1; gs.C = C; gs.aux = aux; gs.K = Kc; gs.Nout = Nout; gs.a_bytes = a_bytes;
        gs.kmajor = 1; gs.kb1 = kb1;
        return launch_grouped_gemm(mode, gs, offs, G, rows, W.tiles, st);
    };
    // ---- group tables
    MOE_TRY(launch_set2(W.off_T, 0, T, st), "offsets");
    MOE_TRY(launch_set2(W.off_hr, 0, h, st), "offsets");
    MOE_TRY(launch_set2(W.off_fr, 0, f, st), "offsets");
    MOE_TRY(launch_iota(W.off_h, H, T, st), "offsets");
    MOE_TRY(launch_iota(W.off_w, Et, dd, st), "offsets");
    MOE_TRY(launch_iota(W.off_f, Et, f, st), "offsets");
    MOE_TRY(launch_iota(W.off_E, H, E, st), "offsets");
    MOE_TRY(launch_kspan(W.off_h, H, b.ms_h, W.kspan_h, W.stage_h, st), "row-block table");
    const void* dc = dy;
    // ---- W_o: dcat = dy W_o, dW_o = dy^T y_cat
    if (b.wo) {
        MOE_TRY(gemm_t(GEMM_PLAIN, dy, (long long)T * h * 2, w->w_o, nullptr, 0, W.dcat, nullptr, h, h, W.off_T, 1, T),
                "W_o dgrad");
        MOE_TRY(wgrad(dy, (long long)T * h * 2, h, h, sv->y_cat, (long long)T * h * 2, h, gr->w_o, h, W.off_T, W.off_hr, 1),
                "W_o wgrad");
        dc = W.dcat;
    }
    // ---- combine: dYp = w dcat, dw = <dcat, y_perm>
    MOE_TRY(launch_combine_bwd(dc, H, dd, K, p.A, sv->dest_row, sv->topk_w, sv->y_perm, W.dYp, W.dw, st), "combine bwd");
    // ---- routed experts
    MOE_TRY(gemm_t(NA == 2 ? GEMM_DSWIGLU : GEMM_DGELU, W.dYp, (long long)N * dd * 2, w->w_down, nullptr, 0, W.dAU,
                   sv->act_grad, dd, f, sv->offsets, Et, N), "expert down dgrad");
    MOE_TRY(gemm_t(GEMM_PLAIN, W.dAU, (long long)N * nf * 2, w->w_gate, NA == 2 ? w->w_up : nullptr, NA == 2 ? f : 0,
                   W.dXp, nullptr, (int)nf, dd, sv->offsets, Et, N), "expert gate/up dgrad");
    MOE_TRY(launch_gather_rows(x, sv->src_token, T * H, sv->offsets + Et, N, dd, W.xp, st), "gather x");
    const long long nb = (long long)N * nf * 2;
    MOE_TRY(wgrad(W.dYp, (long long)N * dd * 2, dd, dd, sv->h, (long long)N * f * 2, f, gr->w_down, f, sv->offsets,
                  W.off_w, Et), "expert down wgrad");
    MOE_TRY(wgrad(W.dAU, nb, (int)nf, f, W.xp, (long long)N * dd * 2, dd, gr->w_gate, dd, sv->offsets, W.off_f, Et),
            "expert gate wgrad");
    if (NA == 2)
        MOE_TRY(wgrad((const char*)W.dAU + (size_t)f * 2, nb - (long long)f * 2, (int)nf, f, W.xp, (long long)N * dd * 2,
                      dd, gr->w_up, dd, sv->offsets, W.off_f, Et), "expert up wgrad");
    // ---- router: through the gate weights and the aux loss
    if (router) {
        const float caux = aux_weight * d->aux_alpha * (float)E / ((float)H * (float)T);
        MOE_TRY(launch_transpose_batched(w->w_router, H, E, dd, W.wgT, b.Ep, 0, st), "transpose");
        MOE_TRY(launch_router_bwd(T, H, E, K, b.Ep, d->score, caux, sv->logits, w->logit_bias, sv->topk_idx, sv->topk_w,
                                  W.dw, sv->counts, W.dl, st), "router bwd");
        MOE_TRY(gemm(GEMM_PLAIN, W.dl, (long long)H * T * b.Ep * 2, W.wgT, nullptr, W.dxr, nullptr, b.Ep, dd, W.off_h, H,
                     H * T, nullptr, 0, 0, nullptr), "router dgrad");
        MOE_TRY(launch_row_blocks(W.dl, b.Ep, 0, 0, nullptr, H * T, 0, W.off_h, W.kspan_h, W.stage_h, b.ms_h, b.Ep, W.dlT,
                                  b.Np_h, st), "row blocks");
        MOE_TRY(launch_row_blocks(x, h, 0, dd, nullptr, T, 1, W.off_h, W.kspan_h, W.stage_h, b.ms_h, dd, W.xhT, b.Np_h,
                                  st), "row blocks");
        MOE_TRY(gemm(GEMM_PLAIN, W.dlT, (long long)b.Ep * b.Np_h * 2, W.xhT, nullptr, gr->w_router, nullptr,
                     (int)b.Np_h, dd, W.off_E, H, H * E, W.kspan_h, E, 1, nullptr), "router wgrad");
    }
    // ---- shared expert (H = 1)
    if (b.shared) {
        MOE_TRY(gemm_t(NA == 2 ? GEMM_DSWIGLU : GEMM_DGELU, dc, (long long)T * h * 2, w->sh_down, nullptr, 0, W.dAUs,
                       sv->sh_act_grad, h, f, W.off_T, 1, T), "shared down dgrad");
        MOE_TRY(gemm_t(GEMM_PLAIN, W.dAUs, (long long)T * nf * 2, w->sh_gate, NA == 2 ? w->sh_up : nullptr,
                       NA == 2 ? f : 0, W.dxs, nullptr, (int)nf, h, W.off_T, 1, T), "shared gate/up dgrad");
        const long long sb = (long long)T * nf * 2;
        MOE_TRY(wgrad(dc, (long long)T * h * 2, h, h, sv->sh_h, (long long)T * f * 2, f, gr->sh_down, f, W.off_T, W.off_hr,
                      1), "shared down wgrad");
        MOE_TRY(wgrad(W.dAUs, sb, (int)nf, f, x, (long long)T * h * 2, h, gr->sh_gate, h, W.off_T, W.off_fr, 1),
                "shared gate wgrad");
        if (NA == 2)
            MOE_TRY(wgrad((const char*)W.dAUs + (size_t)f * 2, sb - (long long)f * 2, (int)nf, f, x, (long long)T * h * 2,
                          h, gr->sh_up, h, W.off_T, W.off_fr, 1), "shared up wgrad");
    }
    // ---- dx
    MOE_TRY(launch_dx(W.dXp, sv->dest_row, T, H, dd, K, router ? W.dxr : nullptr, b.shared ? W.dxs : nullptr, gr->dx, st),
            "dx");
#undef MOE_TRY
    return MOE_OK;
}

}  // extern "C"
