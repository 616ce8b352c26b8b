/*
 * moe_oracle.c -- plain, slow CPU oracle for the forward pass of one sparse
 * mixture-of-experts (MoE) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU-baseline
 * leg use it.  It shares no code, header, table or constant with the HIP
 * library; it defines its own descriptor, its own bf16 decoding and its own
 * exp.  Every floating-point quantity is carried in double precision except
 * where the method fixes fp32 (the routing key of the sigmoid router, see
 * orc_sigmoid_key).
 *
 * Sources (the pages this follows; cited by title and section):
 *  [L10]  "第 10 课：专家并行 EP" (learn.payai.win, train/lesson10), section
 *         "核心概念" item 1 (router score s(x) = Softmax(TopK(x W_g, K)) or a
 *         sigmoid normalisation; output y = sum over the top-K of s_i FFN_i(x)),
 *         item 3 (pack rows per destination, group rows by local expert, run the
 *         experts, return rows and take the gate-weighted sum), item 4 (aux loss
 *         L_aux = alpha E sum_i f_i P_i, capacity C = CF K T / E with overflow
 *         tokens dropped), and the worked example under "具体演示与数值推演".
 *  [HAI]  "HAI-LLM MoE：一键实现大模型的混合专家并行训练" (maimai.cn), section
 *         "HAI-LLM 上的使用": gate kinds (GShard top-2, Switch top-1), n_expert,
 *         capacity_factor, alpha, top_k.
 *  [VI10] "Chương 10: Song song MoE" (infra-guide), item 1 (E experts replace one
 *         FFN, top-K per token, capacity factor and token dropping) and item 4
 *         (aux loss, DeepSeek's bias-based balancing, capacity and drop/pad).
 *  [MH]   "Multi-Head LatentMoE 与 Head 并行" (ai-stack.site), "核心方法与创新":
 *         the token vector is split into heads and each head routes on its own;
 *         "3. 理论基础": an expert may be chosen by a hash or a fixed map of the
 *         input's index instead of a learned gate.
 *  [HAI] also lists a HashGate (top-1 only) and a (train, val) pair of
 *         capacity factors; [L10] item 5 (node-limited routing): the K experts
 *         of a token may lie in at most M nodes.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): ties in the routing key go to the lower expert index; C is
 * ceil(CF K T / E), except that a value within 1e-6 (relative) of an integer
 * counts as that integer, so fp32 noise in CF cannot add a slot;
 * the capacity queue of an expert is first-come by (sub-)token index; a dropped
 * assignment contributes zero and the remaining weights are not renormalised;
 * f_i = counts_i / (T K) counted before drops; P_i averages the full score
 * distribution over all T tokens; group-limited routing splits a head's E
 * experts into n_groups contiguous groups (the expert-to-node map of [L10]'s
 * worked exercise), scores a group by the largest key in it, keeps the
 * group_limit best groups (ties to the lower group index) and takes the top-K
 * among their experts; the hash gate sends sub-token s = t H + g to expert
 * fmix32(key_t H + g) mod E of its head with weight 1 (fmix32 is the 32-bit
 * finaliser of Appleby's MurmurHash3; key_t is a caller-given integer per
 * token, by default t) and has no scores, so P and L_aux are 0; the
 * choice-major queue ranks all first choices of an expert (by sub-token)
 * before any second choice; SwiGLU = (silu(x Wg^T) * (x Wu^T)) Wd^T and
 * GELU uses the exact erf form; no biases; the multi-head layer routes the
 * contiguous d = h/H slice of each token with its own router and its own E
 * experts, concatenates the head outputs and applies W_o.
 *
 * Parity unpinned: P_i of the sigmoid router (the mean of sigma_i / sum sigma)
 * and L_aux of the multi-head layer (the mean over heads of alpha E sum f P,
 * f and P per head).  No page fixes either; the tests check them only through
 * invariants (P sums to 1 per head, L_aux recomputed from the returned f and P).
 *
 * Layouts (the same bytes the HIP library receives):
 *   x            [T][h]                  row-major, fp32 or bf16
 *   w_router     [H][E][d]               one row of d inputs per expert (out-major)
 *   w_gate,w_up  [H*E][f][d]             per expert: f rows of d inputs
 *   w_down       [H*E][d][f]             per expert: d rows of f inputs
 *   shared_*     same as one expert with d = h
 *   w_o          [h][h]                  out-major
 * so every linear map computes out[o] = sum_i in[i] * W[o][i].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- descriptor */
typedef struct {
    int32_t T, h, H, E, K, f;
    int32_t n_shared, has_wo;
    int32_t dtype; /* 0 = fp32, 1 = bf16 (activations and weights) */
    int32_t score; /* 0 = softmax, 1 = sigmoid */
    int32_t act;   /* 0 = SwiGLU, 1 = GELU */
    float capacity_factor; /* <= 0 : no capacity limit */
    float alpha;
    int32_t gate;        /* 0 = top-K of router scores, 1 = hash gate (K = 1) */
    int32_t n_groups;    /* > 1: group-limited top-K over this many groups per head */
    int32_t group_limit; /* groups a sub-token may choose from */
    int32_t queue;       /* 0 = capacity queue by sub-token, 1 = by choice, then sub-token */
    float capacity_factor_eval; /* capacity factor in evaluation mode */
    int32_t eval;        /* 1: use capacity_factor_eval */
} orc_desc;

typedef struct {
    const void *w_router;    /* [H][E][d] */
    const float *logit_bias; /* [H*E] or NULL: added to the logits (fp32 add) */
    const float *select_bias;/* [H*E] or NULL: added to the sigmoid key only */
    const void *w_gate, *w_up, *w_down;
    const void *sh_gate, *sh_up, *sh_down; /* shared expert or NULL */
    const void *w_o;                       /* [h][h] or NULL */
    const int32_t *hash_keys;              /* [T] keys of the hash gate or NULL (key = t) */
} orc_weights;

/* Optional outputs of orc_layer_forward; any pointer may be NULL. */
typedef struct {
    int32_t *topk_idx;  /* [T*H*K] */
    double *topk_w;     /* [T*H*K] */
    double *margin;     /* [T*H] */
    int32_t *counts;    /* [H*E] */
    int32_t *kept;      /* [H*E] */
    int32_t *offsets;   /* [H*E+1] */
    int32_t *dest_row;  /* [T*H*K] */
    int32_t *src_sub;   /* [T*H*K] (first n_kept entries used) */
    int32_t *n_kept;    /* [1] */
    double *f;          /* [H*E] */
    double *P;          /* [H*E] */
    double *l_aux;      /* [1] */
    float *logits;      /* [T*H*E] */
} orc_aux;

/* ------------------------------------------------------------ element access */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return (double)v;
}

/* element i of an activation or weight array of the descriptor's dtype */
static double ld(const void *p, int32_t dtype, int64_t i)
{
    if (dtype == 1) return bf16_bits_to_double(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/* ----------------------------------------------- fp32 exp for the routing key
 * The sigmoid router selects on sigma(l) + b in fp32.  For that selection to be
 * reproducible bit for bit on another device, sigma must be a fixed sequence of
 * fp32 operations.  This follows Cody and Waite's method (Software Manual for
 * the Elementary Functions, 1980): n = nearest integer to x / ln 2,
 * r = x - n ln 2 with ln 2 split into a 16-significant-bit head (so n * head is
 * exact) and an fp32 tail, e^r by its Taylor series through r^7 in Horner form
 * with fused multiply-adds, then scaling by 2^n.  The constants are the
 * mathematical values rounded to fp32:
 *   1/ln 2 -> 0x1.715476p+0, ln 2 head = 45426 / 2^16 = 0x1.62e4p-1,
 *   ln 2 - head -> 0x1.7f7d1cp-20, 1/k! for k = 2..7.
 * Defined for |x| <= 80, where 2^n stays a normal number.                   */
float orc_exp_spec(float x)
{
    const float inv_ln2 = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;
    const float ln2_lo = 0x1.7f7d1cp-20f;
    float n = rintf(x * inv_ln2);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = 0x1.a01a02p-13f;        /* 1/5040 */
    p = fmaf(p, r, 0x1.6c16c2p-10f);  /* 1/720  */
    p = fmaf(p, r, 0x1.111112p-7f);   /* 1/120  */
    p = fmaf(p, r, 0x1.555556p-5f);   /* 1/24   */
    p = fmaf(p, r, 0x1.555556p-3f);   /* 1/6    */
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* sigma(l) = 1 / (1 + e^{-l}) in fp32 with the logit clamped to [-80, 80]. */
float orc_sigmoid_spec(float l)
{
    float c = l < -80.0f ? -80.0f : (l > 80.0f ? 80.0f : l);
    float e = orc_exp_spec(-c);
    float den = 1.0f + e;
    return 1.0f / den;
}

/* Routing key of the sigmoid router: fp32 sigma(l) plus the per-expert
 * selection bias, one fp32 add (DeepSeek-style bias balancing, [VI10] item 4). */
float orc_sigmoid_key(float l, float b)
{
    float s = orc_sigmoid_spec(l);
    return s + b;
}

/* --------------------------------------------------------------- capacity
 * [L10] item 4: C = CF * K * T / E per expert.  E is the number of experts a
 * token chooses among (per head for the multi-head layer, where each head sees
 * T sub-tokens).  Returns -1 for "no limit" (CF <= 0).                       */
int64_t orc_capacity(const orc_desc *d)
{
    /* [HAI]: the capacity factor is a (train, val) pair; eval selects the second */
    float cf = d->eval ? d->capacity_factor_eval : d->capacity_factor;
    if (cf <= 0.0f) return -1;
    double v = (double)cf * (double)d->K * (double)d->T / (double)d->E;
    double r = nearbyint(v);
    double tol = 1e-6 * (v > 1.0 ? v : 1.0);
    if (fabs(v - r) <= tol) return (int64_t)r;
    return (int64_t)ceil(v);
}

/* --------------------------------------------------------------- router GEMM
 * [L10] item 1: the affinities of a token are x . W_g, one per expert.  For the
 * multi-head layer ([MH]) sub-token s = t*H + g uses the g-th slice of x and
 * router g.  Output logits[s][e] rounded once from fp64 to fp32.           */
void orc_logits(const orc_desc *d, const void *x, const void *w_router, float *logits)
{
    const int32_t T = d->T, H = d->H, E = d->E, dd = d->h / d->H;
    int64_t s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < (int64_t)T * H; ++s) {
        int64_t t = s / H, g = s % H;
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t j = 0; j < dd; ++j)
                acc += ld(x, d->dtype, t * d->h + g * dd + j) *
                       ld(w_router, d->dtype, ((int64_t)g * E + e) * dd + j);
            logits[s * E + e] = (float)acc;
        }
    }
}

/* ------------------------------------------------------ selection and weights
 * For every sub-token: the biased logit l' = l + logit_bias (one fp32 add),
 * the routing key (l' for softmax, sigma(l') + select_bias for sigmoid), the K
 * experts with the largest keys (ties to the lower index), listed by key
 * descending (with n_groups > 1, only experts of the group_limit groups with
 * the largest group scores are candidates, and the margin is the smaller of
 * the expert margin and the gap between the last kept and the best dropped
 * group score); the gate weights over the selected set ([L10] item 1):
 *   softmax: w_k = exp(l'_k) / sum_{j in S} exp(l'_j)
 *   sigmoid: w_k = sigma(l'_k) / sum_{j in S} sigma(l'_j)   (unbiased sigma)
 * with sigma in exact double here; the margin key_(K) - key_(K+1) (+inf when
 * K = E); counts per expert; and psum_e = sum over sub-tokens of the full
 * score distribution (softmax over all E, or sigma_e / sum_all sigma).      */
static int key_before(float ka, int ea, float kb, int eb)
{
    if (ka > kb) return 1;
    if (ka < kb) return 0;
    return ea < eb;
}

void orc_select(const orc_desc *d, const float *logits, const float *logit_bias,
                const float *select_bias, int32_t *topk_idx, double *topk_w,
                double *margin, int32_t *counts, double *psum)
{
    const int32_t T = d->T, H = d->H, E = d->E, K = d->K;
    const int64_t S = (int64_t)T * H;
    float *keys = (float *)malloc(sizeof(float) * (size_t)S * E);
    float *lb = (float *)malloc(sizeof(float) * (size_t)S * E);
    int64_t s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < S; ++s) {
        int64_t g = s % H;
        for (int32_t e = 0; e < E; ++e) {
            float l = logits[s * E + e];
            float lbias = logit_bias ? logit_bias[g * E + e] : 0.0f;
            float lp = logit_bias ? l + lbias : l;
            lb[s * E + e] = lp;
            if (d->score == 1) {
                float b = select_bias ? select_bias[g * E + e] : 0.0f;
                keys[s * E + e] = select_bias ? orc_sigmoid_key(lp, b) : orc_sigmoid_spec(lp);
            } else {
                keys[s * E + e] = lp;
            }
        }
    }
    for (s = 0; s < S; ++s) {
        int64_t g = s % H;
        const float *ks = keys + s * E;
        const float *ls = lb + s * E;
        /* selection by repeated arg-max under the (key desc, index asc) order */
        int32_t chosen[4096];
        unsigned char *used = (unsigned char *)calloc((size_t)E, 1);
        /* group limit ([L10] item 5): score each group by its largest key,
         * keep the group_limit best groups (larger score first, lower group
         * index on ties) and take no expert outside them */
        double gmargin = INFINITY;
        if (d->n_groups > 1) {
            const int32_t G = d->n_groups, gs = E / G;
            float gscore[4096];
            unsigned char gkeep[4096];
            for (int32_t q = 0; q < G; ++q) {
                gscore[q] = ks[q * gs];
                for (int32_t j = 1; j < gs; ++j)
                    if (ks[q * gs + j] > gscore[q]) gscore[q] = ks[q * gs + j];
                gkeep[q] = 0;
            }
            int32_t last = -1;
            for (int32_t m = 0; m < d->group_limit; ++m) {
                int32_t bq = -1;
                for (int32_t q = 0; q < G; ++q)
                    if (!gkeep[q] && (bq < 0 || gscore[q] > gscore[bq])) bq = q;
                gkeep[bq] = 1;
                last = bq;
            }
            int32_t nq = -1;
            for (int32_t q = 0; q < G; ++q)
                if (!gkeep[q] && (nq < 0 || gscore[q] > gscore[nq])) nq = q;
            if (nq >= 0) gmargin = (double)gscore[last] - (double)gscore[nq];
            for (int32_t e = 0; e < E; ++e) used[e] = !gkeep[e / gs];
        }
        for (int32_t k = 0; k < K; ++k) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (used[e]) continue;
                if (best < 0 || key_before(ks[e], e, ks[best], best)) best = e;
            }
            used[best] = 1;
            chosen[k] = best;
        }
        int32_t next = -1;
        for (int32_t e = 0; e < E; ++e) {
            if (used[e]) continue;
            if (next < 0 || key_before(ks[e], e, ks[next], next)) next = e;
        }
        free(used);
        if (margin) {
            double em = next < 0 ? INFINITY : (double)ks[chosen[K - 1]] - (double)ks[next];
            margin[s] = em < gmargin ? em : gmargin;
        }
        /* gate weights over the selected set */
        double wsum = 0.0, wv[4096];
        if (d->score == 1) {
            for (int32_t k = 0; k < K; ++k) {
                wv[k] = 1.0 / (1.0 + exp(-(double)ls[chosen[k]]));
                wsum += wv[k];
            }
        } else {
            double m = -INFINITY;
            for (int32_t k = 0; k < K; ++k) m = fmax(m, (double)ls[chosen[k]]);
            for (int32_t k = 0; k < K; ++k) {
                wv[k] = exp((double)ls[chosen[k]] - m);
                wsum += wv[k];
            }
        }
        for (int32_t k = 0; k < K; ++k) {
            topk_idx[s * K + k] = (int32_t)(g * E + chosen[k]);
            topk_w[s * K + k] = wv[k] / wsum;
            if (counts) counts[g * E + chosen[k]] += 1;
        }
        /* full score distribution for the aux statistics */
        if (psum) {
            double tot = 0.0;
            if (d->score == 1) {
                for (int32_t e = 0; e < E; ++e) tot += 1.0 / (1.0 + exp(-(double)ls[e]));
                for (int32_t e = 0; e < E; ++e)
                    psum[g * E + e] += (1.0 / (1.0 + exp(-(double)ls[e]))) / tot;
            } else {
                double m = -INFINITY;
                for (int32_t e = 0; e < E; ++e) m = fmax(m, (double)ls[e]);
                for (int32_t e = 0; e < E; ++e) tot += exp((double)ls[e] - m);
                for (int32_t e = 0; e < E; ++e) psum[g * E + e] += exp((double)ls[e] - m) / tot;
            }
        }
    }
    free(keys);
    free(lb);
}

/* ------------------------------------------------------------- hash gate
 * [HAI] HashGate (top-1) and [MH] "3. 理论基础" (the expert follows from a hash
 * of the input's index, not from its values).  fmix32 is the finalisation
 * step of MurmurHash3 (Austin Appleby, SMHasher, public domain): xor-shift by
 * 16, multiply by 0x85ebca6b, xor-shift by 13, multiply by 0xc2b2ae35,
 * xor-shift by 16, all mod 2^32.  Sub-token s = t H + g of token t goes to
 * expert g E + fmix32(key_t H + g) mod E with weight 1, key_t = hash_keys[t]
 * (or t when hash_keys is NULL), the product and sum taken mod 2^32.        */
uint32_t orc_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

void orc_hash_select(const orc_desc *d, const int32_t *hash_keys, int32_t *topk_idx, double *topk_w,
                     int32_t *counts)
{
    const int32_t T = d->T, H = d->H, E = d->E;
    for (int64_t t = 0; t < T; ++t) {
        uint32_t key = hash_keys ? (uint32_t)hash_keys[t] : (uint32_t)t;
        for (int32_t g = 0; g < H; ++g) {
            uint32_t u = key * (uint32_t)H + (uint32_t)g;
            int32_t e = (int32_t)(orc_fmix32(u) % (uint32_t)E);
            int64_t s = t * H + g;
            topk_idx[s] = g * E + e;
            topk_w[s] = 1.0;
            if (counts) counts[g * E + e] += 1;
        }
    }
}

/* ------------------------------------------------------ capacity and permute
 * [L10] items 3-4: rows are grouped by expert; an expert keeps at most C of the
 * assignments sent to it and drops the rest.  The queue of expert e is ordered
 * by sub-token index (an expert appears at most once in a sub-token's top-K),
 * so pos(s, k) is the number of earlier sub-tokens that chose the same expert.
 * With the choice-major queue (GShard-style priority to first choices), it is
 * ordered by slot k first, then sub-token: pos(s, k) counts the assignments
 * (s', k') to the same expert with k' < k, or k' = k and s' < s.
 *   counts[e]  assignments to e before drops
 *   kept[e]    min(counts[e], C)
 *   offsets    exclusive prefix sum of kept (length H*E+1)
 *   dest_row   offsets[e] + pos if pos < C else -1
 *   src_sub    the sub-token that fills each kept row                        */
void orc_permute(const orc_desc *d, const int32_t *topk_idx, int64_t capacity,
                 int32_t *counts, int32_t *kept, int32_t *offsets, int32_t *dest_row,
                 int32_t *src_sub, int32_t *n_kept)
{
    const int32_t Et = d->H * d->E, K = d->K;
    const int64_t S = (int64_t)d->T * d->H;
    int64_t *seen = (int64_t *)calloc((size_t)Et, sizeof(int64_t));
    for (int32_t e = 0; e < Et; ++e) counts[e] = 0;
    for (int64_t a = 0; a < S * K; ++a) counts[topk_idx[a]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < Et; ++e) {
        int64_t c = counts[e];
        kept[e] = (int32_t)((capacity >= 0 && c > capacity) ? capacity : c);
        offsets[e + 1] = offsets[e] + kept[e];
    }
    /* walk the assignments in queue order */
    for (int64_t i = 0; i < S * K; ++i) {
        int64_t s = d->queue == 1 ? i % S : i / K;
        int32_t k = (int32_t)(d->queue == 1 ? i / S : i % K);
        int32_t e = topk_idx[s * K + k];
        int64_t pos = seen[e]++;
        if (capacity >= 0 && pos >= capacity) {
            dest_row[s * K + k] = -1;
        } else {
            int32_t row = offsets[e] + (int32_t)pos;
            dest_row[s * K + k] = row;
            src_sub[row] = (int32_t)s;
        }
    }
    *n_kept = offsets[Et];
    free(seen);
}

/* ------------------------------------------------------------- expert FFN
 * One row through one expert ([VI10] item 1: each expert is an ordinary FFN):
 *   SwiGLU: a = x W1^T, u = x W3^T, hdn = silu(a) * u, out = hdn W2^T,
 *           silu(z) = z / (1 + e^{-z})
 *   GELU:   a = x W1^T, hdn = a * (1 + erf(a / sqrt 2)) / 2, out = hdn W2^T
 * W1, W3: [f][din]; W2: [din][f]; all in double.
 * Two optional by-products size the parity bound of an evaluation in bf16
 * (they play no part in out):
 *   out_abs[o] = sum_j |hdn_j| |W2[o][j]|, the magnitude of the terms of the
 *                last contraction (any rounding of hdn and out to a format
 *                with unit roundoff u errs by at most about 2u times it);
 *   out_var[o] = sum_j W2[o][j]^2 ulp(hdn_j)^2 / 12, the variance that
 *                rounding every hdn_j to bf16 (to nearest: an error uniform
 *                on half an ulp either side) adds to out[o]; 0 for fp32.   */
static double ulp_bf16(double v)
{
    int ex;
    if (v == 0.0) return 0.0;
    frexp(v, &ex); /* |v| = m 2^ex, 1/2 <= m < 1: 8 significant bits give ulp 2^(ex-8) */
    return ldexp(1.0, ex - 8 < -133 ? -133 : ex - 8);
}

void orc_expert_ffn(int32_t dtype, int32_t act, int32_t din, int32_t f,
                    const void *w1, const void *w3, const void *w2,
                    const double *xin, double *out, double *out_abs, double *out_var)
{
    double *hdn = (double *)malloc(sizeof(double) * (size_t)f);
    double *hu2 = (double *)malloc(sizeof(double) * (size_t)f);
    for (int32_t j = 0; j < f; ++j) {
        double a = 0.0;
        for (int32_t i = 0; i < din; ++i) a += xin[i] * ld(w1, dtype, (int64_t)j * din + i);
        if (act == 0) {
            double u = 0.0;
            for (int32_t i = 0; i < din; ++i) u += xin[i] * ld(w3, dtype, (int64_t)j * din + i);
            hdn[j] = a / (1.0 + exp(-a)) * u;
        } else {
            hdn[j] = 0.5 * a * (1.0 + erf(a / sqrt(2.0)));
        }
        hu2[j] = dtype == 1 ? ulp_bf16(hdn[j]) * ulp_bf16(hdn[j]) / 12.0 : 0.0;
    }
    for (int32_t o = 0; o < din; ++o) {
        double acc = 0.0, mag = 0.0, var = 0.0;
        for (int32_t j = 0; j < f; ++j) {
            double w = ld(w2, dtype, (int64_t)o * f + j);
            acc += hdn[j] * w;
            mag += fabs(hdn[j]) * fabs(w);
            var += w * w * hu2[j];
        }
        out[o] = acc;
        if (out_abs) out_abs[o] = mag;
        if (out_var) out_var[o] = var;
    }
    free(hdn);
    free(hu2);
}

/* n rows of xin [n][din] through the same expert: orc_expert_ffn row by row
 * (rows in parallel; each row's arithmetic is the same as above).          */
void orc_expert_ffn_rows(int32_t dtype, int32_t act, int32_t din, int32_t f,
                         const void *w1, const void *w3, const void *w2, int64_t n,
                         const double *xin, double *out, double *out_abs, double *out_var)
{
    int64_t r;
#pragma omp parallel for schedule(dynamic, 4)
    for (r = 0; r < n; ++r)
        orc_expert_ffn(dtype, act, din, f, w1, w3, w2, xin + r * din, out + r * din,
                       out_abs ? out_abs + r * din : NULL, out_var ? out_var + r * din : NULL);
}

/* ------------------------------------------------------------- combine
 * [L10] item 1 (output formula) and item 3 (returned rows times the saved gate
 * weights, summed): y[t][g*d + j] = sum over kept slots k of w[s][k] *
 * y_perm[dest_row[s][k]][j], plus y_shared[t][j] (weight 1) when given, in
 * double.  y_perm and y_shared are arrays of the descriptor's dtype.         */
void orc_combine(const orc_desc *d, const int32_t *dest_row, const double *topk_w,
                 const void *y_perm, const void *y_shared, double *y)
{
    const int32_t T = d->T, H = d->H, K = d->K, h = d->h, dd = d->h / d->H;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        for (int32_t j = 0; j < h; ++j) y[t * h + j] = 0.0;
        for (int32_t g = 0; g < H; ++g) {
            int64_t s = t * H + g;
            for (int32_t k = 0; k < K; ++k) {
                int32_t row = dest_row[s * K + k];
                if (row < 0) continue;
                for (int32_t j = 0; j < dd; ++j)
                    y[t * h + g * dd + j] += topk_w[s * K + k] * ld(y_perm, d->dtype, (int64_t)row * dd + j);
            }
        }
        if (y_shared)
            for (int32_t j = 0; j < h; ++j) y[t * h + j] += ld(y_shared, d->dtype, t * h + j);
    }
}

/* ------------------------------------------------------------- whole layer
 * [L10] item 1 and item 3: route every token, apply the capacity, then for each
 * requested token t: y[t] = sum over kept (k) of w_k FFN_{e_k}(x[t]) (per head
 * on the head's slice), plus the always-on shared expert (weight 1, no
 * capacity), then the output projection W_o over the concatenated heads.
 * tokens == NULL computes every token.  y is written unrounded, in double.
 * ymag (may be NULL) gets the magnitude that scales the rounding error of an
 * evaluation in a narrower format: sum over kept k of w_k * sum_j |hdn_j||W2_j|
 * (plus the shared expert's), and through W_o sum_i (|cat_i| + mag_i)|W_o[r][i]|.
 * yvar (may be NULL; bf16 layers only, else 0) gets the variance that the
 * intermediate roundings of a bf16 evaluation add to y when each rounds to
 * nearest (an error uniform on half an ulp either side, variance ulp^2/12,
 * the roundings independent): every hdn_j (orc_expert_ffn's out_var), every
 * expert output row and the shared expert's output (stored in bf16 before the
 * weighted sum), and, before W_o, the concatenated head outputs:
 *   var(cat_j) = sum_k w_k^2 (out_var_k[j] + ulp(out_k[j])^2 / 12)
 *                + shared (out_var[j] + ulp(out[j])^2 / 12)
 *   var(y_r)   = sum_i W_o[r][i]^2 (var(cat_i) + ulp(cat_i)^2 / 12)  with W_o,
 *                var(cat_r) without.
 * The last rounding of y itself is not included.
 * Aux statistics ([L10] item 4): f = counts / (T K), P = psum / T,
 * L_aux = alpha * E * sum_e f_e P_e, averaged over heads.                     */
int orc_layer_forward(const orc_desc *d, const orc_weights *w, const void *x,
                      const int32_t *tokens, int32_t n_tokens, double *y, double *ymag,
                      double *yvar, orc_aux *aux)
{
    const int32_t T = d->T, h = d->h, H = d->H, E = d->E, K = d->K, f = d->f;
    const int32_t dd = h / H, Et = H * E;
    const int64_t S = (int64_t)T * H, A = S * K;
    if (H <= 0 || h % H != 0 || K <= 0 || K > E || E > 4096) return 1;
    if (d->gate == 1 && K != 1) return 1;
    if (d->n_groups > 1 && (E % d->n_groups != 0 || d->group_limit < 1 || d->group_limit > d->n_groups ||
                            (int64_t)d->group_limit * (E / d->n_groups) < K))
        return 1;

    float *logits = (float *)malloc(sizeof(float) * (size_t)(S * E + 1));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A + 1));
    double *wts = (double *)malloc(sizeof(double) * (size_t)(A + 1));
    double *mrg = (double *)malloc(sizeof(double) * (size_t)(S + 1));
    int32_t *cnt = (int32_t *)calloc((size_t)Et, sizeof(int32_t));
    int32_t *kep = (int32_t *)calloc((size_t)Et, sizeof(int32_t));
    int32_t *off = (int32_t *)calloc((size_t)Et + 1, sizeof(int32_t));
    int32_t *dst = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A + 1));
    int32_t *src = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A + 1));
    double *psum = (double *)calloc((size_t)Et, sizeof(double));
    int32_t nk = 0;

    if (d->gate == 1) {
        /* the hash gate has no router: no logits, no scores (P = 0), no margin */
        memset(logits, 0, sizeof(float) * (size_t)(S * E + 1));
        orc_hash_select(d, w->hash_keys, idx, wts, NULL);
        for (int64_t s = 0; s < S; ++s) mrg[s] = INFINITY;
    } else {
        orc_logits(d, x, w->w_router, logits);
        orc_select(d, logits, w->logit_bias, w->select_bias, idx, wts, mrg, NULL, psum);
    }
    orc_permute(d, idx, orc_capacity(d), cnt, kep, off, dst, src, &nk);

    int32_t nt = tokens ? n_tokens : T;
    int32_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nt; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        double *xin = (double *)malloc(sizeof(double) * (size_t)h);
        double *cat = (double *)calloc((size_t)h, sizeof(double));
        double *o = (double *)malloc(sizeof(double) * (size_t)h);
        double *om = (double *)malloc(sizeof(double) * (size_t)h);
        double *cm = (double *)calloc((size_t)h, sizeof(double));
        double *ov = (double *)malloc(sizeof(double) * (size_t)h);
        double *cv = (double *)calloc((size_t)h, sizeof(double));
        const int bf = d->dtype == 1;
        for (int32_t j = 0; j < h; ++j) xin[j] = ld(x, d->dtype, t * h + j);
        for (int32_t g = 0; g < H; ++g) {
            int64_t s = t * H + g;
            for (int32_t k = 0; k < K; ++k) {
                if (dst[s * K + k] < 0) continue; /* dropped: contributes 0 */
                int64_t e = idx[s * K + k];
                size_t wsz = d->dtype == 1 ? 2 : 4;
                const char *w1 = (const char *)w->w_gate + (size_t)e * f * dd * wsz;
                const char *w3 = d->act == 0 ? (const char *)w->w_up + (size_t)e * f * dd * wsz : NULL;
                const char *w2 = (const char *)w->w_down + (size_t)e * dd * f * wsz;
                orc_expert_ffn(d->dtype, d->act, dd, f, w1, w3, w2, xin + g * dd, o, om, ov);
                const double wk = wts[s * K + k];
                for (int32_t j = 0; j < dd; ++j) {
                    cat[g * dd + j] += wk * o[j];
                    cm[g * dd + j] += wk * om[j];
                    if (bf) cv[g * dd + j] += wk * wk * (ov[j] + ulp_bf16(o[j]) * ulp_bf16(o[j]) / 12.0);
                }
            }
        }
        if (d->n_shared > 0) {
            orc_expert_ffn(d->dtype, d->act, h, f, w->sh_gate, w->sh_up, w->sh_down, xin, o, om, ov);
            for (int32_t j = 0; j < h; ++j) {
                cat[j] += o[j];
                cm[j] += om[j];
                if (bf) cv[j] += ov[j] + ulp_bf16(o[j]) * ulp_bf16(o[j]) / 12.0;
            }
        }
        if (d->has_wo) {
            for (int32_t r = 0; r < h; ++r) {
                double acc = 0.0, mag = 0.0, var = 0.0;
                for (int32_t j = 0; j < h; ++j) {
                    double wo = ld(w->w_o, d->dtype, (int64_t)r * h + j);
                    acc += cat[j] * wo;
                    mag += (fabs(cat[j]) + cm[j]) * fabs(wo);
                    if (bf) var += wo * wo * (cv[j] + ulp_bf16(cat[j]) * ulp_bf16(cat[j]) / 12.0);
                }
                y[(int64_t)i * h + r] = acc;
                if (ymag) ymag[(int64_t)i * h + r] = mag;
                if (yvar) yvar[(int64_t)i * h + r] = var;
            }
        } else {
            for (int32_t j = 0; j < h; ++j) {
                y[(int64_t)i * h + j] = cat[j];
                if (ymag) ymag[(int64_t)i * h + j] = cm[j];
                if (yvar) yvar[(int64_t)i * h + j] = cv[j];
            }
        }
        free(ov);
        free(cv);
        free(xin);
        free(cat);
        free(o);
        free(om);
        free(cm);
    }

    if (aux) {
        if (aux->topk_idx) memcpy(aux->topk_idx, idx, sizeof(int32_t) * (size_t)A);
        if (aux->topk_w) memcpy(aux->topk_w, wts, sizeof(double) * (size_t)A);
        if (aux->margin) memcpy(aux->margin, mrg, sizeof(double) * (size_t)S);
        if (aux->counts) memcpy(aux->counts, cnt, sizeof(int32_t) * (size_t)Et);
        if (aux->kept) memcpy(aux->kept, kep, sizeof(int32_t) * (size_t)Et);
        if (aux->offsets) memcpy(aux->offsets, off, sizeof(int32_t) * (size_t)(Et + 1));
        if (aux->dest_row) memcpy(aux->dest_row, dst, sizeof(int32_t) * (size_t)A);
        if (aux->src_sub) memcpy(aux->src_sub, src, sizeof(int32_t) * (size_t)nk);
        if (aux->n_kept) *aux->n_kept = nk;
        if (aux->logits) memcpy(aux->logits, logits, sizeof(float) * (size_t)(S * E));
        double laux = 0.0;
        for (int32_t g = 0; g < H; ++g) {
            double sfp = 0.0;
            for (int32_t e = 0; e < E; ++e) {
                double fe = (double)cnt[g * E + e] / ((double)T * K);
                double pe = T > 0 ? psum[g * E + e] / (double)T : 0.0;
                if (aux->f) aux->f[g * E + e] = fe;
                if (aux->P) aux->P[g * E + e] = pe;
                sfp += fe * pe;
            }
            laux += (double)d->alpha * E * sfp;
        }
        if (aux->l_aux) *aux->l_aux = laux / H;
    }
    free(logits); free(idx); free(wts); free(mrg); free(cnt); free(kep);
    free(off); free(dst); free(src); free(psum);
    return 0;
}

/* sets the number of threads the oracle's parallel loops use (n >= 1) */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* number of threads the oracle's parallel loops use */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ============================================================ backward pass
 * Gradients of the loss L = sum_{t,j} dy[t][j] * y[t][j] + c_aux * L_aux with
 * respect to x and every weight, by the chain rule through the forward pass
 * above ([L10] item 1: y = sum over the kept top-K of w_k FFN_k(x), plus the
 * shared expert, then W_o; item 4: L_aux = alpha E sum_i f_i P_i).  Every
 * quantity is recomputed here in double from the inputs.
 *   - Selection (top-K, group limit, capacity) is piecewise constant, so only
 *     the gate weights carry a gradient to the logits: for the softmax gate
 *     w_k = exp(l_k) / sum_{j in S} exp(l_j), dl_j = w_j (dw_j - sum_k w_k dw_k)
 *     for j in the selected set S (dropped slots included: their dw is 0 but
 *     their logit still normalises the kept weights); for the sigmoid gate
 *     w_k = s_k / sum_S s, ds_j = (dw_j - sum_k w_k dw_k) / sum_S s and
 *     dl_j = ds_j s_j (1 - s_j).  Experts outside S get 0.  K = 1 gives 0.
 *   - f_i is a count (no gradient); P_i = mean_t p_t,i, so with c = alpha E / (H T)
 *     softmax:  dL_aux/dl_j = c p_j (f_j - sum_i f_i p_i)
 *     sigmoid:  dL_aux/dl_j = c s_j (1 - s_j) / sum_all s * (f_j - sum_i f_i p_i).
 *   - The hash gate has no router and no scores: no router gradient.
 *   - silu'(a) = sigma(a) (1 + a (1 - sigma(a))); gelu'(a) = Phi(a) + a phi(a).
 * With absm = 1 every factor is replaced by its absolute value (and every
 * difference by a sum), which yields, per gradient element, the magnitude
 * sum |terms| that scales the rounding error of a narrower evaluation.       */
typedef struct {
    double *dx;        /* [T][h] */
    double *dw_router; /* [H][E][d] */
    double *dw_gate;   /* [H*E][f][d] */
    double *dw_up;     /* [H*E][f][d] (SwiGLU) */
    double *dw_down;   /* [H*E][d][f] */
    double *dsh_gate;  /* [f][h] */
    double *dsh_up;    /* [f][h] */
    double *dsh_down;  /* [h][f] */
    double *dw_o;      /* [h][h] */
    double *dlogits;   /* [T*H][E] */
    double *dtopk_w;   /* [T*H*K] */
} orc_grads;

static double mabs(double v, int absm) { return absm ? fabs(v) : v; }

static double sig_d(double a) { return 1.0 / (1.0 + exp(-a)); }

/* activation value and derivative for one pre-activation pair */
static void act_fwd_bwd(int act, double a, double u, double *hval, double *dh_da, double *dh_du)
{
    if (act == 0) {
        double sg = sig_d(a), silu = a * sg;
        *hval = silu * u;
        *dh_da = u * sg * (1.0 + a * (1.0 - sg));
        *dh_du = silu;
    } else {
        double phi = exp(-0.5 * a * a) / sqrt(8.0 * atan(1.0));
        double Phi = 0.5 * (1.0 + erf(a / sqrt(2.0)));
        *hval = a * Phi;
        *dh_da = Phi + a * phi;
        *dh_du = 0.0;
    }
}

int orc_layer_backward(const orc_desc *d, const orc_weights *w, const void *x, const double *dy,
                       double c_aux, int absm, orc_grads *gr)
{
    const int32_t T = d->T, h = d->h, H = d->H, E = d->E, K = d->K, f = d->f;
    const int32_t dd = h / H, Et = H * E, dt = d->dtype;
    const int64_t S = (int64_t)T * H, A = S * K;
    if (H <= 0 || h % H != 0 || K <= 0 || K > E || E > 4096) return 1;
    if (d->gate == 1 && K != 1) return 1;
    const size_t wsz = dt == 1 ? 2 : 4;

    /* ---- routing, as in the forward pass */
    float *logits = (float *)calloc((size_t)(S * E + 1), sizeof(float));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A + 1));
    double *wts = (double *)malloc(sizeof(double) * (size_t)(A + 1));
    int32_t *cnt = (int32_t *)calloc((size_t)Et, sizeof(int32_t));
    int32_t *kep = (int32_t *)calloc((size_t)Et, sizeof(int32_t));
    int32_t *off = (int32_t *)calloc((size_t)Et + 1, sizeof(int32_t));
    int32_t *dst = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A + 1));
    int32_t *src = (int32_t *)malloc(sizeof(int32_t) * (size_t)(A + 1));
    double *psum = (double *)calloc((size_t)Et, sizeof(double));
    int32_t nk = 0;
    if (d->gate == 1) {
        orc_hash_select(d, w->hash_keys, idx, wts, NULL);
    } else {
        orc_logits(d, x, w->w_router, logits);
        orc_select(d, logits, w->logit_bias, w->select_bias, idx, wts, NULL, NULL, psum);
    }
    orc_permute(d, idx, orc_capacity(d), cnt, kep, off, dst, src, &nk);
    int64_t *row_asg = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nk + 1));
    for (int64_t a = 0; a < A; ++a)
        if (dst[a] >= 0) row_asg[dst[a]] = a;

    /* ---- per-row forward quantities of the routed experts */
    const int nact = d->act == 0 ? 2 : 1;
    double *ra = (double *)malloc(sizeof(double) * ((size_t)nk * f + 1));
    double *ru = (double *)malloc(sizeof(double) * ((size_t)nk * f + 1));
    double *rh = (double *)malloc(sizeof(double) * ((size_t)nk * f + 1));
    double *ro = (double *)malloc(sizeof(double) * ((size_t)nk * dd + 1));
    int64_t r;
#pragma omp parallel for schedule(dynamic, 4)
    for (r = 0; r < nk; ++r) {
        int64_t a = row_asg[r], s = a / K, t = s / H, g = s % H;
        int64_t e = idx[a];
        const char *w1 = (const char *)w->w_gate + (size_t)e * f * dd * wsz;
        const char *w3 = nact == 2 ? (const char *)w->w_up + (size_t)e * f * dd * wsz : NULL;
        const char *w2 = (const char *)w->w_down + (size_t)e * dd * f * wsz;
        for (int32_t j = 0; j < f; ++j) {
            double av = 0.0, uv = 0.0;
            for (int32_t i = 0; i < dd; ++i) {
                double xv = ld(x, dt, t * h + g * dd + i);
                av += xv * ld(w1, dt, (int64_t)j * dd + i);
                if (w3) uv += xv * ld(w3, dt, (int64_t)j * dd + i);
            }
            double hv, t1, t2;
            act_fwd_bwd(d->act, av, uv, &hv, &t1, &t2);
            ra[r * f + j] = av;
            ru[r * f + j] = uv;
            rh[r * f + j] = hv;
        }
        for (int32_t o = 0; o < dd; ++o) {
            double acc = 0.0;
            for (int32_t j = 0; j < f; ++j) acc += rh[r * f + j] * ld(w2, dt, (int64_t)o * f + j);
            ro[r * dd + o] = acc;
        }
    }

    /* ---- shared expert forward (per token) */
    double *sa = NULL, *su = NULL, *sh = NULL, *so = NULL;
    if (d->n_shared > 0) {
        sa = (double *)malloc(sizeof(double) * (size_t)T * f);
        su = (double *)malloc(sizeof(double) * (size_t)T * f);
        sh = (double *)malloc(sizeof(double) * (size_t)T * f);
        so = (double *)malloc(sizeof(double) * (size_t)T * h);
        int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
        for (t = 0; t < T; ++t) {
            for (int32_t j = 0; j < f; ++j) {
                double av = 0.0, uv = 0.0;
                for (int32_t i = 0; i < h; ++i) {
                    double xv = ld(x, dt, t * h + i);
                    av += xv * ld(w->sh_gate, dt, (int64_t)j * h + i);
                    if (nact == 2) uv += xv * ld(w->sh_up, dt, (int64_t)j * h + i);
                }
                double hv, t1, t2;
                act_fwd_bwd(d->act, av, uv, &hv, &t1, &t2);
                sa[t * f + j] = av;
                su[t * f + j] = uv;
                sh[t * f + j] = hv;
            }
            for (int32_t o = 0; o < h; ++o) {
                double acc = 0.0;
                for (int32_t j = 0; j < f; ++j) acc += sh[t * f + j] * ld(w->sh_down, dt, (int64_t)o * f + j);
                so[t * h + o] = acc;
            }
        }
    }

    /* ---- W_o: dcat = dy W_o, dW_o = dy^T cat (cat = the concatenated head outputs) */
    double *dcat = (double *)malloc(sizeof(double) * (size_t)T * h);
    if (d->has_wo) {
        double *cat = (double *)calloc((size_t)T * h, sizeof(double));
        for (int64_t a = 0; a < A; ++a) {
            if (dst[a] < 0) continue;
            int64_t s = a / K, t = s / H, g = s % H;
            for (int32_t j = 0; j < dd; ++j) cat[t * h + g * dd + j] += wts[a] * ro[(int64_t)dst[a] * dd + j];
        }
        if (so)
            for (int64_t i = 0; i < (int64_t)T * h; ++i) cat[i] += so[i];
        int64_t t;
#pragma omp parallel for schedule(static)
        for (t = 0; t < T; ++t)
            for (int32_t i = 0; i < h; ++i) {
                double acc = 0.0;
                for (int32_t q = 0; q < h; ++q)
                    acc += mabs(dy[t * h + q], absm) * mabs(ld(w->w_o, dt, (int64_t)q * h + i), absm);
                dcat[t * h + i] = acc;
            }
        if (gr->dw_o) {
            int64_t q;
#pragma omp parallel for schedule(static)
            for (q = 0; q < h; ++q)
                for (int32_t i = 0; i < h; ++i) {
                    double acc = 0.0;
                    for (int64_t t2 = 0; t2 < T; ++t2)
                        acc += mabs(dy[t2 * h + q], absm) * mabs(cat[t2 * h + i], absm);
                    gr->dw_o[q * h + i] = acc;
                }
        }
        free(cat);
    } else {
        for (int64_t i = 0; i < (int64_t)T * h; ++i) dcat[i] = mabs(dy[i], absm);
    }

    /* ---- gate-weight gradients dw[a] = <dcat slice, o[row]> */
    double *dw = (double *)calloc((size_t)(A + 1), sizeof(double));
    for (int64_t a = 0; a < A; ++a) {
        if (dst[a] < 0) continue;
        int64_t s = a / K, t = s / H, g = s % H;
        double acc = 0.0;
        for (int32_t j = 0; j < dd; ++j)
            acc += dcat[t * h + g * dd + j] * mabs(ro[(int64_t)dst[a] * dd + j], absm);
        dw[a] = acc;
    }
    if (gr->dtopk_w) memcpy(gr->dtopk_w, dw, sizeof(double) * (size_t)A);

    /* ---- routed experts backward, per row: dO = w dcat, dH = W2^T dO, da, du */
    double *rda = (double *)malloc(sizeof(double) * ((size_t)nk * f + 1));
    double *rdu = (double *)malloc(sizeof(double) * ((size_t)nk * f + 1));
    double *rdo = (double *)malloc(sizeof(double) * ((size_t)nk * dd + 1));
#pragma omp parallel for schedule(dynamic, 4)
    for (r = 0; r < nk; ++r) {
        int64_t a = row_asg[r], s = a / K, t = s / H, g = s % H;
        int64_t e = idx[a];
        const char *w2 = (const char *)w->w_down + (size_t)e * dd * f * wsz;
        for (int32_t o = 0; o < dd; ++o) rdo[r * dd + o] = mabs(wts[a], absm) * dcat[t * h + g * dd + o];
        for (int32_t j = 0; j < f; ++j) {
            double dh = 0.0;
            for (int32_t o = 0; o < dd; ++o) dh += rdo[r * dd + o] * mabs(ld(w2, dt, (int64_t)o * f + j), absm);
            double hv, t1, t2;
            act_fwd_bwd(d->act, ra[r * f + j], ru[r * f + j], &hv, &t1, &t2);
            rda[r * f + j] = dh * mabs(t1, absm);
            rdu[r * f + j] = dh * mabs(t2, absm);
        }
    }
    /* weight gradients, one expert per iteration (rows of an expert are contiguous) */
    int64_t e;
#pragma omp parallel for schedule(dynamic, 1)
    for (e = 0; e < Et; ++e) {
        int64_t g = e / E;
        for (int32_t o = 0; o < dd; ++o)
            for (int32_t j = 0; j < f; ++j) {
                double acc = 0.0;
                for (int64_t rr = off[e]; rr < off[e + 1]; ++rr)
                    acc += rdo[rr * dd + o] * mabs(rh[rr * f + j], absm);
                if (gr->dw_down) gr->dw_down[(e * dd + o) * (int64_t)f + j] = acc;
            }
        for (int32_t j = 0; j < f; ++j)
            for (int32_t i = 0; i < dd; ++i) {
                double ag = 0.0, au = 0.0;
                for (int64_t rr = off[e]; rr < off[e + 1]; ++rr) {
                    int64_t t = (row_asg[rr] / K) / H;
                    double xv = mabs(ld(x, dt, t * h + g * dd + i), absm);
                    ag += rda[rr * f + j] * xv;
                    au += rdu[rr * f + j] * xv;
                }
                if (gr->dw_gate) gr->dw_gate[(e * f + j) * (int64_t)dd + i] = ag;
                if (gr->dw_up && nact == 2) gr->dw_up[(e * f + j) * (int64_t)dd + i] = au;
            }
    }

    /* ---- router: dlogits from dw (+ the aux-loss term), per sub-token */
    double *dl = (double *)calloc((size_t)(S * E + 1), sizeof(double));
    if (d->gate == 0) {
        double *fq = (double *)calloc((size_t)Et, sizeof(double));
        double *pm = (double *)calloc((size_t)Et, sizeof(double));
        for (int32_t q = 0; q < Et; ++q) {
            fq[q] = (double)cnt[q] / ((double)T * K);
            pm[q] = T > 0 ? psum[q] / (double)T : 0.0;
        }
        const double caux = c_aux * (double)d->alpha * (double)E / ((double)H * (double)T);
        int64_t s;
#pragma omp parallel for schedule(static)
        for (s = 0; s < S; ++s) {
            int64_t g = s % H;
            double lp[4096], p[4096], sgv[4096];
            for (int32_t q = 0; q < E; ++q)
                lp[q] = (double)logits[s * E + q] + (w->logit_bias ? (double)w->logit_bias[g * E + q] : 0.0);
            /* gate-weight part over the selected set */
            double wdw = 0.0;
            for (int32_t k = 0; k < K; ++k) wdw += mabs(wts[s * K + k], absm) * dw[s * K + k];
            double ssel = 0.0;
            if (d->score == 1)
                for (int32_t k = 0; k < K; ++k) ssel += sig_d(lp[idx[s * K + k] - g * E]);
            for (int32_t k = 0; k < K; ++k) {
                int32_t q = idx[s * K + k] - (int32_t)(g * E);
                double diff = absm ? dw[s * K + k] + wdw : dw[s * K + k] - wdw;
                if (d->score == 1) {
                    double sq = sig_d(lp[q]);
                    dl[s * E + q] += diff / ssel * sq * (1.0 - sq);
                } else {
                    dl[s * E + q] += mabs(wts[s * K + k], absm) * diff;
                }
            }
            /* aux part: every expert of the head */
            if (c_aux != 0.0) {
                double tot = 0.0;
                if (d->score == 1) {
                    for (int32_t q = 0; q < E; ++q) { sgv[q] = sig_d(lp[q]); tot += sgv[q]; }
                    for (int32_t q = 0; q < E; ++q) p[q] = sgv[q] / tot;
                } else {
                    double m = -INFINITY;
                    for (int32_t q = 0; q < E; ++q) m = fmax(m, lp[q]);
                    for (int32_t q = 0; q < E; ++q) { p[q] = exp(lp[q] - m); tot += p[q]; }
                    for (int32_t q = 0; q < E; ++q) p[q] /= tot;
                }
                double fp = 0.0;
                for (int32_t q = 0; q < E; ++q) fp += fq[g * E + q] * p[q];
                for (int32_t q = 0; q < E; ++q) {
                    double diff = absm ? fq[g * E + q] + fp : fq[g * E + q] - fp;
                    double jac = d->score == 1 ? sgv[q] * (1.0 - sgv[q]) / tot : p[q];
                    dl[s * E + q] += caux * jac * diff;
                }
            }
        }
        free(fq);
        free(pm);
        if (gr->dw_router) {
            int64_t q;
#pragma omp parallel for schedule(static)
            for (q = 0; q < Et; ++q) {
                int64_t g = q / E, ee = q % E;
                for (int32_t i = 0; i < dd; ++i) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < T; ++t)
                        acc += dl[(t * H + g) * E + ee] * mabs(ld(x, dt, t * h + g * dd + i), absm);
                    gr->dw_router[q * dd + i] = acc;
                }
            }
        }
    }
    if (gr->dlogits) memcpy(gr->dlogits, dl, sizeof(double) * (size_t)(S * E));

    /* ---- shared expert backward */
    if (d->n_shared > 0) {
        double *sda = (double *)malloc(sizeof(double) * (size_t)T * f);
        double *sdu = (double *)malloc(sizeof(double) * (size_t)T * f);
        int64_t t;
#pragma omp parallel for schedule(static)
        for (t = 0; t < T; ++t)
            for (int32_t j = 0; j < f; ++j) {
                double dh = 0.0;
                for (int32_t o = 0; o < h; ++o) dh += dcat[t * h + o] * mabs(ld(w->sh_down, dt, (int64_t)o * f + j), absm);
                double hv, t1, t2;
                act_fwd_bwd(d->act, sa[t * f + j], su[t * f + j], &hv, &t1, &t2);
                sda[t * f + j] = dh * mabs(t1, absm);
                sdu[t * f + j] = dh * mabs(t2, absm);
            }
        int64_t q;
#pragma omp parallel for schedule(static)
        for (q = 0; q < h; ++q)
            for (int32_t j = 0; j < f; ++j) {
                double acc = 0.0;
                for (int64_t t2 = 0; t2 < T; ++t2) acc += dcat[t2 * h + q] * mabs(sh[t2 * f + j], absm);
                if (gr->dsh_down) gr->dsh_down[q * f + j] = acc;
            }
#pragma omp parallel for schedule(static)
        for (q = 0; q < f; ++q)
            for (int32_t i = 0; i < h; ++i) {
                double ag = 0.0, au = 0.0;
                for (int64_t t2 = 0; t2 < T; ++t2) {
                    double xv = mabs(ld(x, dt, t2 * h + i), absm);
                    ag += sda[t2 * f + q] * xv;
                    au += sdu[t2 * f + q] * xv;
                }
                if (gr->dsh_gate) gr->dsh_gate[q * h + i] = ag;
                if (gr->dsh_up && nact == 2) gr->dsh_up[q * h + i] = au;
            }
        /* shared part of dx */
        if (gr->dx) {
#pragma omp parallel for schedule(static)
            for (t = 0; t < T; ++t)
                for (int32_t i = 0; i < h; ++i) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < f; ++j) {
                        acc += sda[t * f + j] * mabs(ld(w->sh_gate, dt, (int64_t)j * h + i), absm);
                        if (nact == 2) acc += sdu[t * f + j] * mabs(ld(w->sh_up, dt, (int64_t)j * h + i), absm);
                    }
                    gr->dx[t * h + i] = acc;
                }
        }
        free(sda);
        free(sdu);
    } else if (gr->dx) {
        for (int64_t i = 0; i < (int64_t)T * h; ++i) gr->dx[i] = 0.0;
    }

    /* ---- dx: routed experts (dX rows summed per sub-token) + router */
    if (gr->dx) {
        int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
        for (t = 0; t < T; ++t) {
            for (int32_t g = 0; g < H; ++g) {
                int64_t s = t * H + g;
                for (int32_t k = 0; k < K; ++k) {
                    int64_t a = s * K + k;
                    if (dst[a] < 0) continue;
                    int64_t rr = dst[a], ee = idx[a];
                    const char *w1 = (const char *)w->w_gate + (size_t)ee * f * dd * wsz;
                    const char *w3 = nact == 2 ? (const char *)w->w_up + (size_t)ee * f * dd * wsz : NULL;
                    for (int32_t i = 0; i < dd; ++i) {
                        double acc = 0.0;
                        for (int32_t j = 0; j < f; ++j) {
                            acc += rda[rr * f + j] * mabs(ld(w1, dt, (int64_t)j * dd + i), absm);
                            if (w3) acc += rdu[rr * f + j] * mabs(ld(w3, dt, (int64_t)j * dd + i), absm);
                        }
                        gr->dx[t * h + g * dd + i] += acc;
                    }
                }
                if (d->gate == 0)
                    for (int32_t i = 0; i < dd; ++i) {
                        double acc = 0.0;
                        for (int32_t q = 0; q < E; ++q)
                            acc += dl[s * E + q] * mabs(ld(w->w_router, dt, ((int64_t)g * E + q) * dd + i), absm);
                        gr->dx[t * h + g * dd + i] += acc;
                    }
            }
        }
    }

    free(logits); free(idx); free(wts); free(cnt); free(kep); free(off); free(dst); free(src);
    free(psum); free(row_asg); free(ra); free(ru); free(rh); free(ro); free(dcat); free(dw);
    free(rda); free(rdu); free(rdo); free(dl);
    free(sa); free(su); free(sh); free(so);
    return 0;
}
