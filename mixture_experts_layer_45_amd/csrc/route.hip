// route.hip -- router GEMM, scoring, top-K selection and gate weights.
//
// Lesson 10 "专家并行 EP" (learn.payai.win), "核心概念" item 1: a token's
// affinities to the E experts are x . W_g; the K largest are kept and scored
// with a softmax over the kept logits (GShard/Switch gates of "HAI-LLM MoE",
// "HAI-LLM 上的使用"), or with sigmoids renormalised over the kept experts, the
// selection then using sigma + a per-expert bias ("Chương 10: Song song MoE",
// item 4, DeepSeek's bias balancing).  Multi-head routing ("Multi-Head
// LatentMoE 与 Head 并行", "核心方法与创新"): head g routes slice g of the token
// with its own router among its own experts.
//
// Routers with at most 64 bf16 experts per head use route_small_kernel (below);
// the others use route_kernel.  route_kernel: one block = 16 tokens of one
// head.  Phase 1: the four waves split the
// reduction over d, each running 16x16x32 bf16 MFMAs over its quarter; the
// partial logit tiles are summed in LDS in wave order (fixed order, so the
// logits are reproducible).  Phase 2: each wave takes four of the 16 tokens;
// the lanes hold the keys of experts lane, lane+64, ...; K rounds of a wave
// arg-max (key descending, index ascending) pick the experts.  Gate weights,
// the per-block score sums for P and the per-block expert histogram follow.
//
// Group-limited selection (lesson 10, item 5: a token's experts lie in at
// most M nodes): a head's experts form n_groups contiguous groups scored by
// their largest key, and only the group_limit best groups are eligible.  Both
// kernels find those groups with group_limit arg-max rounds over the experts of
// groups not yet kept: the best remaining key lies in the best remaining
// group, and on equal scores the lower expert, hence the lower group, wins.
//
// The hash gate ("HAI-LLM MoE" HashGate; "Multi-Head LatentMoE 与 Head 并行",
// "3. 理论基础") has no router: route_hash_kernel maps sub-token t*H + g to
// expert fmix32(key_t*H + g) mod E of head g, fmix32 being MurmurHash3's
// 32-bit finaliser.
#include <algorithm>

#include "common.hpp"

namespace moe {

constexpr int RT_ROWS = 16;
constexpr int kMaxParts = 8;  // partial-logit slices of the split-K router GEMM
constexpr int RT_THREADS = 256;

// tokens per route block: 16, except for bf16 routers with 17..64 experts (64)
static bool route_split_applies(int T, int h, int H, int E, int dtype);
constexpr int RT_ROWS_SPLIT = 4;  // tokens per selection block behind the split-K router GEMM
int route_rows(int T, int h, int H, int E, int dtype) {
    if (route_split_applies(T, h, H, E, dtype)) return RT_ROWS_SPLIT;
    if (dtype != MOE_BF16 || E <= 16 || E > 64) return RT_ROWS;
    return 4 * RT_ROWS;
}
int route_blocks(int T, int h, int H, int E, int dtype) {
    const int r = route_rows(T, h, H, E, dtype);
    return (T + r - 1) / r;
}

// Routing-key exp: a fixed sequence of fp32 operations (Cody and Waite's range
// reduction with ln 2 split into a 16-bit head and an fp32 tail, the Taylor
// series of e^r through r^7 in Horner form with fused multiply-adds, scaling by
// 2^n).  Constants are the mathematical values rounded to fp32.  Valid for
// |x| <= 80.
__device__ __attribute__((noinline)) float key_exp(float x) {
#pragma clang fp contract(off)
    const float inv_ln2 = 0x1.715476p+0f;   // 1 / ln 2
    const float ln2_hi = 0x1.62e4p-1f;      // 45426 / 2^16
    const float ln2_lo = 0x1.7f7d1cp-20f;   // ln 2 - ln2_hi
    const float n = __builtin_rintf(x * inv_ln2);
    float r = __builtin_fmaf(-n, ln2_hi, x);
    r = __builtin_fmaf(-n, ln2_lo, r);
    float p = 0x1.a01a02p-13f;                  // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

// sigma(l) = 1 / (1 + e^{-l}) with l clamped to [-80, 80]; IEEE division.
__device__ __attribute__((noinline)) float key_sigmoid(float l) {
#pragma clang fp contract(off)
    const float c = l < -80.0f ? -80.0f : (l > 80.0f ? 80.0f : l);
    const float e = key_exp(-c);
    const float den = 1.0f + e;
    return 1.0f / den;
}

// (key, index) order: larger key first, lower index on ties.
__device__ __forceinline__ bool better(float ka, int ea, float kb, int eb) {
    return ka > kb || (ka == kb && ea < eb);
}

__device__ __forceinline__ float wave_sum(float v) {
    // partners add the same two values, so every lane ends with the same,
    // order-fixed sum
    bfly_steps<64>([&](auto O) __attribute__((always_inline)) { v += bfly<decltype(O)::value>(v); });
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    bfly_steps<64>([&](auto O) __attribute__((always_inline)) { v = fmaxf(v, bfly<decltype(O)::value>(v)); });
    return v;
}
// arg-max of (key, index) over the wave
__device__ __forceinline__ void wave_best(float& bk, int& be) {
    bfly_steps<64>([&](auto O) __attribute__((always_inline)) {
        constexpr int off = decltype(O)::value;
        const float ok = bfly<off>(bk);
        const int oe = bfly<off>(be);
        if (better(ok, oe, bk, be)) { bk = ok; be = oe; }
    });
}

// NB = 16-expert column blocks of the logit tile (E <= 16*NB); EJ = E/64 slots
// per lane; ROWS tokens per block (16, or 4 -- one token per wave -- behind
// the split-K router GEMM, where the logits are given and only selection runs).
template <int NB, bool BF16, int ROWS = RT_ROWS>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
    constexpr int LDE = NB * 16 + 1;
    constexpr int EJ = (NB * 16 + 63) / 64;
    constexpr int RT_ROWS = ROWS;
    __shared__ float part[ROWS == 16 ? 4 : 1][RT_ROWS][LDE];  // per-wave partial logits; part[0] ends as the tile
    __shared__ int hist[NB * 16];
    __shared__ float pw[4][NB * 16];

    const int g = blockIdx.y;
    const int t0 = blockIdx.x * RT_ROWS;
    const int T = a.T, H = a.H, E = a.E, K = a.K;
    const int d = a.h / H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int Et = H * E;

    for (int i = threadIdx.x; i < NB * 16; i += RT_THREADS) hist[i] = 0;

    // ---------------------------------------------------------------- logits
    if (a.logit_parts || (a.flags & MOE_LOGITS_IN)) {
        // logits given: the split-K router GEMM's partial logits (at most
        // kMaxParts, summed in part order), or the caller's.  Four elements per
        // thread per pass, every load of a pass issued before the first add.
        const int n = RT_ROWS * E;
        const int np = a.logit_parts ? a.n_parts : 1;
        for (int i0 = threadIdx.x; i0 < n; i0 += 4 * RT_THREADS) {
            float v[4][kMaxParts];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * RT_THREADS;
                const int r = i / E, e = i - r * E, t = t0 + r;
                const bool ok = i < n && t < T;
#pragma unroll
                for (int q = 0; q < kMaxParts; ++q) {
                    float x = 0.0f;
                    if (ok && q < np)
                        x = a.logit_parts ? a.logit_parts[((size_t)q * T + t) * E + e]
                                          : a.logits[((size_t)t * H + g) * E + e];
                    v[u][q] = x;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * RT_THREADS;
                if (i >= n) continue;
                const int r = i / E, e = i - r * E;
                float sum = v[u][0];
#pragma unroll
                for (int q = 1; q < kMaxParts; ++q)
                    if (q < np) sum += v[u][q];
                part[0][r][e] = sum;
            }
        }
    } else if constexpr (BF16 && ROWS == 16) {
        floatx4 acc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int row = min(t0 + (lane & 15), T - 1);
        const uint16_t* xr = (const uint16_t*)a.x + (size_t)row * a.h + (size_t)g * d;
        const uint16_t* wg = (const uint16_t*)a.w_router + (size_t)g * E * d;
        const int nks = (d + 31) / 32;
        const int ks0 = wave * nks / 4, ks1 = (wave + 1) * nks / 4;
        const int kq = (lane >> 4) * 8;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        // U k steps of loads are issued before their MFMAs, so a wave keeps
        // U*(1+NB) 16-byte loads in flight instead of one step's worth
        constexpr int U = NB <= 2 ? 8 : (NB <= 4 ? 4 : 2);
        for (int kb = ks0; kb < ks1; kb += U) {
            u32x4 av[U], bv[U][NB];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = (kb + u) * 32 + kq;
                const bool kin = kb + u < ks1 && k < d;
                av[u] = kin ? *(const u32x4*)(xr + k) : zero;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int e = j * 16 + (lane & 15);
                    bv[u][j] = (kin && e < E) ? *(const u32x4*)(wg + (size_t)e * d + k) : zero;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(bv[u][j]), acc[j], 0, 0, 0);
        }
        // 16x16 result: lane holds rows 4*(lane/16)+i of column lane%16
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[wave][(lane >> 4) * 4 + i][j * 16 + (lane & 15)] = acc[j][i];
        __syncthreads();
        for (int i = threadIdx.x; i < RT_ROWS * NB * 16; i += RT_THREADS) {
            const int r = i / (NB * 16), e = i - r * (NB * 16);
            float s = part[0][r][e];
            s += part[1][r][e];
            s += part[2][r][e];
            s += part[3][r][e];
            part[0][r][e] = s;
        }
    } else if constexpr (ROWS == 16) {
        const float* x = (const float*)a.x;
        const float* wg = (const float*)a.w_router + (size_t)g * E * d;
        for (int i = threadIdx.x; i < RT_ROWS * E; i += RT_THREADS) {
            const int r = i / E, e = i - r * E;
            const int t = min(t0 + r, T - 1);
            const float* xr = x + (size_t)t * a.h + (size_t)g * d;
            const float* wr = wg + (size_t)e * d;
            float s = 0.0f;
            for (int k = 0; k < d; ++k) s = fmaf(xr[k], wr[k], s);
            part[0][r][e] = s;
        }
    }
    __syncthreads();
    if (a.flags & MOE_LOGITS_OUT) {
        for (int i = threadIdx.x; i < RT_ROWS * E; i += RT_THREADS) {
            const int r = i / E, e = i - r * E, t = t0 + r;
            if (t < T) a.logits[((size_t)t * H + g) * E + e] = part[0][r][e];
        }
    }

    // --------------------------------------------------- selection and weights
    float pacc[EJ];
#pragma unroll
    for (int j = 0; j < EJ; ++j) pacc[j] = 0.0f;
    const float NEG = -__builtin_inff();
    for (int rr = 0; rr < RT_ROWS / 4; ++rr) {
        const int r = wave * (RT_ROWS / 4) + rr;
        const int t = t0 + r;
        if (t >= T) break;
        const size_t s = (size_t)t * H + g;
        float lp[EJ], key[EJ], sg[EJ];
        bool used[EJ];
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            const int e = lane + 64 * j;
            const bool valid = e < E;
            float l = valid ? part[0][r][e] : NEG;
            if (valid && a.logit_bias) l = l + a.logit_bias[g * E + e];
            lp[j] = l;
            if (a.score == MOE_SIGMOID) {
                sg[j] = valid ? key_sigmoid(l) : 0.0f;
                key[j] = valid ? (a.select_bias ? sg[j] + a.select_bias[g * E + e] : sg[j]) : NEG;
            } else {
                sg[j] = 0.0f;
                key[j] = l;
            }
            used[j] = !valid;
        }
        if (a.n_groups > 1) {
            const int gsz = E / a.n_groups;
            bool gk[EJ];
#pragma unroll
            for (int j = 0; j < EJ; ++j) gk[j] = false;
            for (int m = 0; m < a.group_limit; ++m) {
                float bk = NEG;
                int be = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < EJ; ++j) {
                    const int e = lane + 64 * j;
                    if (!used[j] && !gk[j] && better(key[j], e, bk, be)) { bk = key[j]; be = e; }
                }
                wave_best(bk, be);
                const int gb = be / gsz;
#pragma unroll
                for (int j = 0; j < EJ; ++j) gk[j] = gk[j] || (lane + 64 * j) / gsz == gb;
            }
#pragma unroll
            for (int j = 0; j < EJ; ++j) used[j] = used[j] || !gk[j];
        }
        // K rounds of wave arg-max; slot k is kept by lane k % 64
        int my_e[4] = {0, 0, 0, 0};
        float my_v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < K; ++k) {
            float bk = NEG;
            int be = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                const int e = lane + 64 * j;
                if (!used[j] && better(key[j], e, bk, be)) { bk = key[j]; be = e; }
            }
            wave_best(bk, be);
            // the owner of `be` marks it used and broadcasts the value the weight needs
            float v = 0.0f;
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                if (lane + 64 * j == be) {
                    used[j] = true;
                    v = a.score == MOE_SIGMOID ? sg[j] : lp[j];
                }
            }
            v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), __builtin_amdgcn_readfirstlane(be) & 63));
            if ((k & 63) == lane) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if ((k >> 6) == q) { my_e[q] = be; my_v[q] = v; }
            }
        }
        // gate weights: softmax over the kept biased logits (the first kept is the
        // largest), or kept sigmoids over their sum
        const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v[0]), 0));
        float u[4], loc = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool mine = lane + 64 * q < K;
            u[q] = mine ? (a.score == MOE_SIGMOID ? my_v[q] : expf(my_v[q] - vmax)) : 0.0f;
            loc += u[q];
        }
        const float den = wave_sum(loc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = lane + 64 * q;
            if (k < K) {
                a.topk_idx[s * K + k] = g * E + my_e[q];
                a.topk_w[s * K + k] = u[q] / den;
                atomicAdd(&hist[my_e[q]], 1);
            }
        }
        // full score distribution for P
        if (a.prob_part) {
            if (a.score == MOE_SIGMOID) {
                float sl = 0.0f;
#pragma unroll
                for (int j = 0; j < EJ; ++j) sl += sg[j];
                const float tot = wave_sum(sl);
#pragma unroll
                for (int j = 0; j < EJ; ++j) pacc[j] += sg[j] / tot;
            } else {
                float ml = NEG;
#pragma unroll
                for (int j = 0; j < EJ; ++j) ml = fmaxf(ml, lp[j]);
                const float m = wave_max(ml);
                float ex[EJ], sl = 0.0f;
#pragma unroll
                for (int j = 0; j < EJ; ++j) {
                    ex[j] = lane + 64 * j < E ? expf(lp[j] - m) : 0.0f;
                    sl += ex[j];
                }
                const float tot = wave_sum(sl);
#pragma unroll
                for (int j = 0; j < EJ; ++j) pacc[j] += ex[j] / tot;
            }
        }
    }
    if (a.prob_part) {
#pragma unroll
        for (int j = 0; j < EJ; ++j)
            if (lane + 64 * j < NB * 16) pw[wave][lane + 64 * j] = pacc[j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += RT_THREADS) {
        if (a.counts && hist[e]) atomicAdd(&a.counts[g * E + e], hist[e]);
        if (a.prob_part) {
            float s = pw[0][e];
            s += pw[1][e];
            s += pw[2][e];
            s += pw[3][e];
            a.prob_part[((size_t)g * gridDim.x + blockIdx.x) * E + e] = s;
        }
    }
    (void)Et;
}

// Selection for the RS tokens t0, t0+1, ... of head g (phase 2 of
// route_small_kernel): LPT lanes per token (threads tid < RS*LPT; the
// others idle), each lane holding experts lq, lq + LPT, ... of the token's row
// of logits lg [RS][NB*16+1] (LDS); every arg-max round is a lane-local scan
// then a butterfly over the token's lanes on the (key desc, index asc) order.
// Writes topk_idx/topk_w, counts the kept experts in hist (LDS) and, when
// a.prob_part is set, the token's full score distribution to pr (LDS, same
// layout).
template <int NB, int RS, int LPT, bool SIG>
__device__ __forceinline__ void select_tile(const RouteArgs& a, int g, int t0, int tid, const float* lg, float* pr,
                                            int* hist) {
    constexpr int EP = NB * 16;
    constexpr int LDE = EP + 1;
    constexpr int EPL = EP / LPT;
    static_assert(EPL >= 1 && LPT <= 64, "a token's lanes lie in one wave and hold one expert or more each");
    const int T = a.T, H = a.H, E = a.E, K = a.K;
    const float NEG = -__builtin_inff();
    const int r = tid / LPT, lq = tid % LPT;
    const int t = t0 + r;
    // arg-max of (key, expert, value) over the token's lanes
    auto group_best = [&](float& bk, int& be, float& bv) __attribute__((always_inline)) {
        bfly_steps<LPT>([&](auto O) __attribute__((always_inline)) {
            constexpr int off = decltype(O)::value;
            const float ok = bfly<off>(bk);
            const int oe = bfly<off>(be);
            const float ov = bfly<off>(bv);
            if (better(ok, oe, bk, be)) { bk = ok; be = oe; bv = ov; }
        });
    };
    auto group_sum = [&](float v) __attribute__((always_inline)) {
        bfly_steps<LPT>([&](auto O) __attribute__((always_inline)) { v += bfly<decltype(O)::value>(v); });
        return v;
    };
    auto group_max = [&](float v) __attribute__((always_inline)) {
        bfly_steps<LPT>([&](auto O) __attribute__((always_inline)) { v = fmaxf(v, bfly<decltype(O)::value>(v)); });
        return v;
    };
    if (r < RS && t < T) {  // uniform over a token's lanes
        const size_t sidx = (size_t)t * H + g;
        // softmax router: key = biased logit; sigmoid router: key = sigma + bias,
        // weights from sigma
        float key[EPL], sg[SIG ? EPL : 1];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lq + LPT * j;
            const bool valid = e < E;
            float l = valid ? lg[r * LDE + e] : NEG;
            if (valid && a.logit_bias) l = l + a.logit_bias[g * E + e];
            if constexpr (SIG) {
                sg[j] = valid ? key_sigmoid(l) : 0.0f;
                key[j] = valid ? (a.select_bias ? sg[j] + a.select_bias[g * E + e] : sg[j]) : NEG;
            } else {
                key[j] = l;
            }
        }
        // group limit: experts outside the group_limit best groups are excluded
        // (the best remaining key lies in the best remaining group)
        uint32_t excl = 0;  // bit j: expert lq + LPT*j excluded
        if (a.n_groups > 1) {
            const int gsz = E / a.n_groups;
            uint32_t kept = 0;
            for (int m = 0; m < a.group_limit; ++m) {
                float bk = NEG, bv = 0.0f;
                int be = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < EPL; ++j) {
                    const int e = lq + LPT * j;
                    if (e < E && !((kept >> j) & 1u) && better(key[j], e, bk, be)) { bk = key[j]; be = e; }
                }
                group_best(bk, be, bv);
                const int gb = be / gsz;
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    if ((lq + LPT * j) / gsz == gb) kept |= 1u << j;
            }
            excl = ~kept;
        }
        // two passes of K arg-max rounds: the first sums the kept scores, the
        // second writes the normalised weights (lane k % LPT writes slot k)
        float den = 0.0f, vmax = 0.0f;
        for (int pass = 0; pass < 2; ++pass) {
            uint32_t used = excl;
            for (int k = 0; k < K; ++k) {
                float bk = NEG, bv = 0.0f;
                int be = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < EPL; ++j) {
                    const int e = lq + LPT * j;
                    if (e < E && !((used >> j) & 1u) && better(key[j], e, bk, be)) {
                        bk = key[j];
                        be = e;
                        if constexpr (SIG) bv = sg[j];
                        else bv = key[j];
                    }
                }
                group_best(bk, be, bv);
                if (be % LPT == lq) used |= 1u << (be / LPT);
                if (k == 0) vmax = bv;  // the first kept has the largest biased logit
                const float u = SIG ? bv : expf(bv - vmax);
                if (pass == 0) {
                    den += u;
                } else if (k % LPT == lq) {
                    a.topk_idx[sidx * K + k] = g * E + be;
                    a.topk_w[sidx * K + k] = u / den;
                    atomicAdd(&hist[be], 1);
                }
            }
        }
        // full score distribution of this token, for P
        if (a.prob_part) {
            if constexpr (SIG) {
                float tot = 0.0f;
#pragma unroll
                for (int j = 0; j < EPL; ++j) tot += sg[j];
                tot = group_sum(tot);
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    if (lq + LPT * j < E) pr[r * LDE + lq + LPT * j] = sg[j] / tot;
            } else {
                float m = NEG;
#pragma unroll
                for (int j = 0; j < EPL; ++j) m = fmaxf(m, key[j]);
                m = group_max(m);
                float ex[EPL], tot = 0.0f;
#pragma unroll
                for (int j = 0; j < EPL; ++j) {
                    ex[j] = lq + LPT * j < E ? expf(key[j] - m) : 0.0f;
                    tot += ex[j];
                }
                tot = group_sum(tot);
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    if (lq + LPT * j < E) pr[r * LDE + lq + LPT * j] = ex[j] / tot;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 routers with at most 64 experts per head: RS = 16*R tokens of one head
// per block (R = 1 for E <= 16, 4 for E <= 64, so that the router rows a block
// reads stay small next to its token rows; measured on one MI355X, 8 heads of
// 32 experts over 8192 tokens: R = 4 took the route from 35.3 to 29.2 us, while
// R = 2 or 4 for 8 experts was no faster than R = 1).  Phase 1 as above, the four waves
// splitting the reduction over d, with R x NB MFMA tiles per wave and U k steps
// of loads in flight.  Phase 2 gives each token 256/RS lanes (16, 8 or 4), each
// holding every LPT-th expert of the token's row of logits in registers: an
// arg-max round (key descending, index ascending) is a lane-local scan and a
// butterfly over the token's lanes.  The full score distribution goes to an
// LDS tile whose columns are summed in token order.
template <int NB, int R, bool SIG>
__global__ __launch_bounds__(RT_THREADS) void route_small_kernel(RouteArgs a) {
    constexpr int RS = 16 * R;
    constexpr int EP = NB * 16;
    constexpr int LDE = EP + 1;
    __shared__ float part[4][RS][LDE];  // per-wave partial logits; part[0] ends as the tile, part[1] holds P rows
    __shared__ int hist[EP];

    const int g = blockIdx.y;
    const int t0 = blockIdx.x * RS;
    const int T = a.T, H = a.H, E = a.E, K = a.K;
    const int d = a.h / H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < EP; i += RT_THREADS) hist[i] = 0;

    if (a.flags & MOE_LOGITS_IN) {
        for (int i = threadIdx.x; i < RS * E; i += RT_THREADS) {
            const int r = i / E, e = i - r * E, t = t0 + r;
            part[0][r][e] = t < T ? a.logits[((size_t)t * H + g) * E + e] : 0.0f;
        }
    } else {
        floatx4 acc[R][NB];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* xr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(t0 + 16 * r + (lane & 15), T - 1);
            xr[r] = (const uint16_t*)a.x + (size_t)row * a.h + (size_t)g * d;
        }
        const uint16_t* wg = (const uint16_t*)a.w_router + (size_t)g * E * d;
        const int nks = (d + 31) / 32;
        const int ks0 = wave * nks / 4, ks1 = (wave + 1) * nks / 4;
        const int kq = (lane >> 4) * 8;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        constexpr int U = 16 / (R + NB) > 0 ? 16 / (R + NB) : 1;
        for (int kb = ks0; kb < ks1; kb += U) {
            u32x4 av[U][R], bv[U][NB];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = (kb + u) * 32 + kq;
                const bool kin = kb + u < ks1 && k < d;
#pragma unroll
                for (int r = 0; r < R; ++r) av[u][r] = kin ? *(const u32x4*)(xr[r] + k) : zero;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int e = j * 16 + (lane & 15);
                    bv[u][j] = (kin && e < E) ? *(const u32x4*)(wg + (size_t)e * d + k) : zero;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u][r]), as_bf16x8(bv[u][j]), acc[r][j], 0, 0, 0);
        }
        // 16x16 result: lane holds rows 4*(lane/16)+i of column lane%16
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) part[wave][16 * r + (lane >> 4) * 4 + i][j * 16 + (lane & 15)] = acc[r][j][i];
        __syncthreads();
        for (int i = threadIdx.x; i < RS * EP; i += RT_THREADS) {
            const int r = i / EP, e = i - r * EP;
            float v = part[0][r][e];
            v += part[1][r][e];
            v += part[2][r][e];
            v += part[3][r][e];
            part[0][r][e] = v;
        }
    }
    __syncthreads();
    if (a.flags & MOE_LOGITS_OUT) {
        for (int i = threadIdx.x; i < RS * E; i += RT_THREADS) {
            const int r = i / E, e = i - r * E, t = t0 + r;
            if (t < T) a.logits[((size_t)t * H + g) * E + e] = part[0][r][e];
        }
    }

    select_tile<NB, RS, RT_THREADS / RS, SIG>(a, g, t0, threadIdx.x, &part[0][0][0], &part[1][0][0], hist);
    __syncthreads();
    const int rows = min(RS, T - t0);
    for (int e = threadIdx.x; e < E; e += RT_THREADS) {
        if (a.counts && hist[e]) atomicAdd(&a.counts[g * E + e], hist[e]);
        if (a.prob_part) {
            float v = 0.0f;
            for (int q = 0; q < rows; ++q) v += part[1][q][e];
            a.prob_part[((size_t)g * gridDim.x + blockIdx.x) * E + e] = v;
        }
    }
}

// P_e for 256/LANES experts per block of 256 threads (prob_mean_of's lane layout)
template <int LANES>
__global__ __launch_bounds__(256) void prob_mean_kernel(const float* part, int nbx, int H, int E, int T, float* out) {
    const int ge = blockIdx.x * (256 / LANES) + (int)(threadIdx.x / LANES), j = threadIdx.x % LANES;
    const bool valid = ge < H * E;
    const float v = prob_mean_of<LANES>(part, nbx, E, T, ge, valid, j);
    if (valid && j == 0) out[ge] = v;
}

__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// one thread per sub-token; integer atomics only, so counts are exact
__global__ __launch_bounds__(256) void route_hash_kernel(const int32_t* keys, int T, int H, int E,
                                                         int32_t* topk_idx, float* topk_w, int32_t* counts) {
    const int s = blockIdx.x * 256 + threadIdx.x;
    if (s >= T * H) return;
    const int t = s / H, g = s - t * H;
    const uint32_t key = keys ? (uint32_t)keys[t] : (uint32_t)t;
    const uint32_t u = key * (uint32_t)H + (uint32_t)g;
    const int e = (int)(fmix32(u) % (uint32_t)E);
    topk_idx[s] = g * E + e;
    topk_w[s] = 1.0f;
    if (counts) atomicAdd(&counts[g * E + e], 1);
}

hipError_t launch_route_hash(const int32_t* keys, int T, int H, int E, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, hipStream_t st) {
    const int S = T * H;
    if (S == 0) return hipSuccess;
    hipLaunchKernelGGL(route_hash_kernel, dim3((S + 255) / 256), dim3(256), 0, st, keys, T, H, E, topk_idx,
                       topk_w, counts);
    return hipGetLastError();
}

template <int NB>
static hipError_t launch_nb(const RouteArgs& a, hipStream_t st) {
    dim3 grid((a.T + RT_ROWS - 1) / RT_ROWS, a.H);
    if (a.dtype == MOE_BF16)
        hipLaunchKernelGGL((route_kernel<NB, true>), grid, dim3(RT_THREADS), 0, st, a);
    else
        hipLaunchKernelGGL((route_kernel<NB, false>), grid, dim3(RT_THREADS), 0, st, a);
    return hipGetLastError();
}

template <int NB, int R>
static hipError_t launch_small(const RouteArgs& a, hipStream_t st) {
    dim3 grid((a.T + 16 * R - 1) / (16 * R), a.H);
    if (a.score == MOE_SIGMOID)
        hipLaunchKernelGGL((route_small_kernel<NB, R, true>), grid, dim3(RT_THREADS), 0, st, a);
    else
        hipLaunchKernelGGL((route_small_kernel<NB, R, false>), grid, dim3(RT_THREADS), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K router GEMM for bf16 routers with more than 64 experts (one head):
// the 16-token blocks of route_kernel would each pull all E x d router weights
// through one CU; instead the 64-wide grouped GEMM computes fp32 partial logits
// over KS slices of d (group q = slice q: every group reads the same token
// rows and router rows, with its own k span), and route_kernel sums the KS
// partials in slice order before selecting.
struct RouteSplit {
    int KS, nst;
};
static RouteSplit route_split_of(int T, int h, int H, int E, int dtype);
static bool route_split_applies(int T, int h, int H, int E, int dtype) {
    return route_split_of(T, h, H, E, dtype).KS > 0;
}
static RouteSplit route_split_of(int T, int h, int H, int E, int dtype) {
    RouteSplit r{0, 0};
    if (dtype != MOE_BF16 || H != 1 || E <= 64 || E % 8 != 0 || h % 64 != 0 || T < 256) return r;
    r.nst = h / 64;
    const int m_tiles = (T + 127) / 128;
    int ks = 256 / m_tiles;
    ks = std::max(1, std::min(ks, std::min(kMaxParts, r.nst / 4)));
    r.KS = ks;
    return r;
}
static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t route_split_ws_bytes(int T, int h, int H, int E, int dtype) {
    const RouteSplit r = route_split_of(T, h, H, E, dtype);
    if (r.KS == 0) return 0;
    return al256((size_t)r.KS * T * E * 4) + al256((size_t)(r.KS + 1) * 4) + al256((size_t)r.KS * 8) +
           grouped_gemm_ws_bytes(r.KS, r.KS * T) + 256;
}

__global__ void route_split_tables_kernel(int KS, int T, int nst, int32_t* offsets, int2* kspan) {
    const int q = threadIdx.x;
    if (q <= KS) offsets[q] = q * T;
    if (q < KS) {
        const int k0 = q * nst / KS, k1 = (q + 1) * nst / KS;
        kspan[q] = make_int2(k0, k1 - k0);
    }
}

hipError_t launch_route(const RouteArgs& a0, hipStream_t st) {
    RouteArgs a = a0;
    const RouteSplit rs = route_split_of(a.T, a.h, a.H, a.E, a.dtype);
    if (rs.KS > 0 && !(a.flags & MOE_LOGITS_IN)) {
        if (!a.split_ws) return hipErrorInvalidValue;
        char* w = (char*)a.split_ws;
        float* parts = (float*)w;
        w += al256((size_t)rs.KS * a.T * a.E * 4);
        int32_t* offs = (int32_t*)w;
        w += al256((size_t)(rs.KS + 1) * 4);
        int2* kspan = (int2*)w;
        w += al256((size_t)rs.KS * 8);
        GemmTile* tiles = (GemmTile*)w;
        hipLaunchKernelGGL(route_split_tables_kernel, dim3(1), dim3(64), 0, st, rs.KS, a.T, rs.nst, offs, kspan);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        GemmSpec gs{};
        gs.A = a.x;
        gs.B0 = a.w_router;
        gs.C = parts;
        gs.K = a.h;
        gs.Nout = a.E;
        gs.a_bytes = (long long)a.T * a.h * 2;
        gs.kspan = kspan;
        gs.a_mod = a.T;
        gs.b_shared = 1;
        if ((err = launch_grouped_gemm(GEMM_F32OUT, gs, offs, rs.KS, rs.KS * a.T, tiles, st, 128)) != hipSuccess)
            return err;
        a.logit_parts = parts;
        a.n_parts = rs.KS;
    }
    if (rs.KS > 0) {  // selection only, one token per wave (the logits are given)
        dim3 grid((a.T + RT_ROWS_SPLIT - 1) / RT_ROWS_SPLIT, a.H);
        if (a.E <= 128)
            hipLaunchKernelGGL((route_kernel<8, true, RT_ROWS_SPLIT>), grid, dim3(RT_THREADS), 0, st, a);
        else
            hipLaunchKernelGGL((route_kernel<16, true, RT_ROWS_SPLIT>), grid, dim3(RT_THREADS), 0, st, a);
        return hipGetLastError();
    }
    if (a.dtype == MOE_BF16 && a.E <= 64) {
        if (a.E <= 16) return launch_small<1, 1>(a, st);
        if (a.E <= 32) return launch_small<2, 4>(a, st);
        return launch_small<4, 4>(a, st);
    }
    if (a.E <= 16) return launch_nb<1>(a, st);
    if (a.E <= 32) return launch_nb<2>(a, st);
    if (a.E <= 64) return launch_nb<4>(a, st);
    if (a.E <= 128) return launch_nb<8>(a, st);
    return launch_nb<16>(a, st);
}

hipError_t launch_prob_mean(const float* part, int nbx, int H, int E, int T, float* out, hipStream_t st) {
    const int n = H * E;
    if (p_lanes(n) == 16)
        hipLaunchKernelGGL(prob_mean_kernel<16>, dim3((n + 15) / 16), dim3(256), 0, st, part, nbx, H, E, T, out);
    else
        hipLaunchKernelGGL(prob_mean_kernel<64>, dim3((n + 3) / 4), dim3(256), 0, st, part, nbx, H, E, T, out);
    return hipGetLastError();
}

}  // namespace moe
