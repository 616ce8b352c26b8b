/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) forward pass of one sparse
 * mixture-of-experts (MoE) layer.
 *
 * The layer (lesson 10 "专家并行 EP" of the learn.payai.win distributed-training
 * course, section "核心概念" items 1, 3 and 4; "HAI-LLM MoE" (maimai.cn), section
 * "HAI-LLM 上的使用"; "Chương 10: Song song MoE", items 1 and 4):
 *   a router scores every token against E experts (logits = x . W_g), keeps the
 *   K best (softmax over the kept logits, or sigmoid scores renormalised over
 *   the kept experts, with an optional selection-only bias), groups the token
 *   rows by expert under a per-expert capacity C = CF * K * T / E (assignments
 *   past C are dropped), runs each expert's FFN (SwiGLU or GELU) over its rows
 *   as one grouped GEMM, and returns y = sum over kept experts of w_k FFN_k(x),
 *   plus the load statistics f_i (routing frequency) and P_i (mean score) of the
 *   auxiliary loss L_aux = alpha * E * sum_i f_i P_i.
 *   The multi-head variant ("Multi-Head LatentMoE 与 Head 并行", ai-stack.site,
 *   "核心方法与创新") splits each token into H contiguous slices of d = h/H; each
 *   slice is routed by its own router among its own E experts, and the head
 *   outputs are concatenated and multiplied by W_o.
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers unless stated, and every call is
 *     asynchronous on `stream` (a hipStream_t; NULL = the null stream).  The
 *     library keeps no pointer after returning and holds no state between calls;
 *     buffers must stay valid until the stream has passed the call.
 *   - The library never allocates memory and never synchronises.  Scratch
 *     memory is a caller-owned workspace of moe_workspace_size() bytes.
 *   - Activations are row-major [rows][features].  Every weight matrix is stored
 *     out-major, one row per output feature: out[o] = sum_i in[i] * W[o][i].
 *       w_router    [H][E][d]         router of head g is rows [g*E, g*E+E)
 *       w_gate/w_up [H*E][f][d]       (w_up unused for GELU; GELU uses w_gate as W1)
 *       w_down      [H*E][d][f]
 *       sh_gate/sh_up [f][h], sh_down [h][f]   (always-on shared expert, H = 1 only)
 *       w_o         [h][h]
 *     Experts are numbered globally: expert e of head g is g*E + e.
 *   - Sub-token s = t*H + g is head g of token t (s = t when H = 1).  Routing
 *     arrays are [T*H][K]; slot k of a sub-token holds its k-th best expert.
 *   - dtype MOE_BF16: activations and weights bf16, accumulation fp32, logits,
 *     keys and gate weights fp32, the FFN hidden activation rounded once to bf16,
 *     expert outputs bf16, y rounded once (round-to-nearest-even) from fp32.
 *     dtype MOE_F32: everything fp32.
 *   - Validation (null pointers, sizes, workspace size) happens before any
 *     launch: a call that returns an error has enqueued nothing.  A launch
 *     failure returns MOE_ERR_DEVICE.  moe_last_error() gives the detail of the
 *     last error on the calling thread.  T = 0 is a valid no-op.
 *   - Results are deterministic: no floating-point atomics; every reduction has
 *     a fixed order, so repeated calls give bitwise-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, K > E, h % H != 0 ... */
    MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle     */
    MOE_ERR_WORKSPACE = 3,   /* workspace pointer NULL or smaller than needed  */
    MOE_ERR_DEVICE = 4       /* a HIP call or kernel launch failed            */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;
typedef enum { MOE_SWIGLU = 0, MOE_GELU = 1 } moe_act;
/* Gate kinds ("HAI-LLM MoE", "HAI-LLM 上的使用": GShard/Switch gates score the
 * tokens, the HashGate sends each token to one expert by a hash). */
typedef enum { MOE_GATE_TOPK = 0, MOE_GATE_HASH = 1 } moe_gate;
/* Order of an expert's capacity queue: by sub-token, or all first choices
 * (by sub-token) before any second choice (GShard-style priority). */
typedef enum { MOE_QUEUE_TOKEN = 0, MOE_QUEUE_CHOICE = 1 } moe_queue;

/* Layer description.  T tokens of width h; H router heads (1 = ordinary MoE);
 * E experts per head; top-K; expert hidden width f; n_shared 0 or 1 shared
 * experts (weight 1, never dropped, H = 1 only); has_wo applies W_o after the
 * head concat.  capacity_factor <= 0 means no capacity limit.  aux_alpha is
 * the alpha of L_aux.
 * Routing variants (all zero = plain top-K, token-order queue, training CF):
 *   gate         MOE_GATE_HASH: top-1 by hash, no router (K must be 1)
 *   n_groups     > 1: group-limited top-K (lesson 10, item 5: a token's experts
 *                lie in at most group_limit nodes).  A head's E experts form
 *                n_groups contiguous groups of E/n_groups; a group's score is
 *                its largest routing key; the group_limit best groups (ties to
 *                the lower group) are eligible and the top-K is taken among
 *                their experts.  Needs E % n_groups == 0, 1 <= group_limit <=
 *                n_groups and K <= group_limit * E / n_groups.
 *   queue        moe_queue order of each expert's capacity queue
 *   capacity_factor_eval, eval   "HAI-LLM MoE" (train, val) capacity factors:
 *                with eval = 1 the capacity uses capacity_factor_eval.
 *   packed       1: the expert weights (w_gate, w_up, w_down, the shared
 *                expert's and w_o) are in the fragment order that
 *                moe_pack_weights writes; forward entry points only (training
 *                and the backward pass read row-major weights).  Needs
 *                MOE_BF16, d and f multiples of 64 and every GEMM operand
 *                under 2 GB, else MOE_ERR_UNSUPPORTED.
 * Limits: 1 <= K <= E <= 256; h % H == 0; for MOE_BF16, d = h/H and f are
 * multiples of 8 (16-byte rows). */
typedef struct moe_desc {
    int32_t T, h, H, E, K, f;
    int32_t n_shared, has_wo;
    int32_t dtype; /* moe_dtype */
    int32_t score; /* moe_score */
    int32_t act;   /* moe_act   */
    float capacity_factor;
    float aux_alpha;
    int32_t gate;        /* moe_gate  */
    int32_t n_groups;    /* 0 or 1: no group limit */
    int32_t group_limit;
    int32_t queue;       /* moe_queue */
    float capacity_factor_eval;
    int32_t eval;        /* 0: capacity_factor, 1: capacity_factor_eval */
    int32_t packed;      /* 0: row-major expert weights, 1: fragment order */
} moe_desc;

/* Flags of moe_route. */
#define MOE_LOGITS_IN 1u  /* skip x . W_g; read logits[T*H][E] (pre-bias) instead */
#define MOE_LOGITS_OUT 2u /* also write the computed pre-bias logits[T*H][E]     */

/* Flags of moe_grouped_ffn (0 = both GEMMs). */
#define MOE_FFN_GEMM1 1u /* x_perm -> h_tmp (gate/up GEMM + activation) */
#define MOE_FFN_GEMM2 2u /* h_tmp -> y_perm (down GEMM)                  */

/* Which call a workspace is sized for. */
typedef enum {
    MOE_WS_LAYER = 0, /* moe_layer_forward (also enough for every stage call) */
    MOE_WS_ROUTE = 1,
    MOE_WS_PERMUTE = 2,
    MOE_WS_FFN = 3,
    MOE_WS_BACKWARD = 4 /* moe_layer_backward */
} moe_ws_kind;

/* Expert capacity C = CF * K * T / E rounded up (CF = capacity_factor, or
 * capacity_factor_eval when eval = 1), where a value within 1e-6
 * (relative) of an integer counts as that integer (lesson 10, item 4: each
 * expert keeps at most C of the assignments sent to it).  Returns INT32_MAX
 * when capacity_factor <= 0 (no limit) and -1 for an invalid descriptor. */
int32_t moe_capacity(const moe_desc *desc);

/* Bytes of workspace `kind` needs for this descriptor (host pointer `bytes`).
 * The workspace must be 256-byte aligned device memory. */
moe_status moe_workspace_size(const moe_desc *desc, int32_t kind, size_t *bytes);

/* Router, scoring and top-K (lesson 10, item 1; "HAI-LLM MoE", gate kinds).
 *   x          [T][h]          activations (unused with MOE_LOGITS_IN)
 *   w_router   [H][E][d]       router weights (unused with MOE_LOGITS_IN)
 *   logit_bias [H*E] fp32|NULL added to every logit (one fp32 add) before
 *                              scoring; it changes selection, weights and P
 *   select_bias[H*E] fp32|NULL sigmoid router only: key = sigma(l) + bias; the
 *                              gate weights use the unbiased sigma
 *   logits     [T*H][E] fp32|NULL  input with MOE_LOGITS_IN, output with
 *                              MOE_LOGITS_OUT (pre-bias in both cases)
 *   topk_idx   [T*H][K] int32  global expert ids, key descending, ties to the
 *                              lower index.  Softmax router: key = biased
 *                              logit.  Sigmoid router: key = fp32
 *                              1/(1+exp(-l)) + select_bias, with exp computed by
 *                              Cody-Waite reduction and a degree-7 Taylor
 *                              polynomial (so the key is reproducible bit for bit)
 *   topk_w     [T*H][K] fp32   gate weights, summing to 1 over the K slots
 *   counts     [H*E] int32|NULL  assignments per expert (before any capacity)
 *   prob_mean  [H*E] fp32|NULL   P_e = mean over the T tokens of the full score
 *                              distribution of the expert's head (softmax over
 *                              all E, or sigma_e / sum of all sigma)
 * With n_groups > 1 the selection is group-limited (see moe_desc).  The hash
 * gate does not use this call (MOE_ERR_INVALID_ARG): see moe_route_hash.
 * Needs moe_workspace_size(MOE_WS_ROUTE) bytes of workspace. */
moe_status moe_route(const moe_desc *desc, const void *x, const void *w_router,
                     const float *logit_bias, const float *select_bias, float *logits,
                     uint32_t flags, int32_t *topk_idx, float *topk_w, int32_t *counts,
                     float *prob_mean, void *ws, size_t ws_bytes, void *stream);

/* Hash gate ("HAI-LLM MoE", HashGate, top-1; "Multi-Head LatentMoE 与 Head
 * 并行", "3. 理论基础": the expert follows from a hash of the input's index).
 * Sub-token s = t*H + g goes to expert g*E + fmix32(key_t*H + g) mod E with
 * weight 1, where key_t = hash_keys[t] (e.g. the token's vocabulary id) or t
 * when hash_keys is NULL, the arithmetic mod 2^32, and fmix32 the 32-bit
 * finaliser of MurmurHash3 (xor-shift 16, * 0x85ebca6b, xor-shift 13,
 * * 0xc2b2ae35, xor-shift 16).  Needs desc->gate == MOE_GATE_HASH, K = 1.
 *   hash_keys [T] int32|NULL;  topk_idx [T*H][1] int32;  topk_w [T*H][1] fp32
 *   counts    [H*E] int32|NULL  assignments per expert
 * No workspace. */
moe_status moe_route_hash(const moe_desc *desc, const int32_t *hash_keys, int32_t *topk_idx,
                          float *topk_w, int32_t *counts, void *stream);

/* Histogram, prefix scan, capacity and permutation (lesson 10, items 3-4).
 *   topk_idx   [T*H][K] int32  from moe_route
 *   x          [T][h]|NULL     activations; NULL skips the row gather
 *   capacity   C >= 0 (INT32_MAX = no limit); normally moe_capacity(desc)
 *   counts     [H*E] int32     assignments per expert before drops
 *   kept       [H*E] int32     min(counts, C)
 *   offsets    [H*E+1] int32   exclusive prefix sum of kept; rows of expert e
 *                              are [offsets[e], offsets[e+1])
 *   dest_row   [T*H*K] int32   row of each assignment in x_perm, -1 if dropped.
 *                              The queue of an expert is ordered by sub-token
 *                              index (MOE_QUEUE_TOKEN) or by slot, then
 *                              sub-token (MOE_QUEUE_CHOICE); the first C
 *                              assignments are kept, in queue order.
 *   src_token  [T*H*K] int32   sub-token that fills each row (first n_kept used)
 *   x_perm     [T*H*K][d]      x_perm[row] = slice g of x[t] for s = t*H + g
 *   n_kept     [1] int32       total kept rows = offsets[H*E]
 * Needs moe_workspace_size(MOE_WS_PERMUTE) bytes of workspace. */
moe_status moe_permute(const moe_desc *desc, const int32_t *topk_idx, const void *x,
                       int32_t capacity, int32_t *counts, int32_t *kept, int32_t *offsets,
                       int32_t *dest_row, int32_t *src_token, void *x_perm, int32_t *n_kept,
                       void *ws, size_t ws_bytes, void *stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and validation as moe_permute
 * (bit-identical outputs), minus ws / ws_bytes: its one scratch buffer, the
 * per-chunk expert histogram of ceil(T*H*K / 1024) * H*E + 1 int32, lives in
 * a static device array of moe_permute_noalloc_max_ints() int32 (4 MiB) that
 * the library holds on each GPU it runs on until the process ends.  A larger
 * problem is MOE_ERR_UNSUPPORTED (nothing launched).  The first call on a
 * device looks up the array's device address (hipGetSymbolAddress); no call
 * allocates or frees memory.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must be serialised by the caller. */
moe_status moe_permute_noalloc(const moe_desc *desc, const int32_t *topk_idx, const void *x,
                               int32_t capacity, int32_t *counts, int32_t *kept, int32_t *offsets,
                               int32_t *dest_row, int32_t *src_token, void *x_perm, int32_t *n_kept,
                               void *stream);
size_t moe_permute_noalloc_max_ints(void);

/* Expert FFNs as a ragged grouped GEMM (lesson 10, item 3: rows grouped by
 * expert run as one grouped GEMM).  H*E groups; group e owns rows
 * [offsets[e], offsets[e+1]) of x_perm / h_tmp / y_perm.
 *   SwiGLU: h_tmp = silu(x_perm W_gate_e^T) * (x_perm W_up_e^T), silu(z) = z/(1+e^-z)
 *   GELU:   h_tmp = gelu(x_perm W_gate_e^T), gelu(z) = z (1 + erf(z/sqrt 2)) / 2
 *   then    y_perm = h_tmp W_down_e^T
 *   x_perm [max_rows][d], h_tmp [max_rows][f], y_perm [max_rows][d];
 *   max_rows: host-side upper bound on offsets[H*E] (<= T*H*K); it sizes the
 *   launch, the kernels read the actual row ranges from offsets.
 *   flags: MOE_FFN_GEMM1, MOE_FFN_GEMM2 or 0 for both.
 * Needs moe_workspace_size(MOE_WS_FFN) bytes of workspace. */
moe_status moe_grouped_ffn(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                           int32_t max_rows, const void *w_gate, const void *w_up,
                           const void *w_down, void *h_tmp, void *y_perm, uint32_t flags,
                           void *ws, size_t ws_bytes, void *stream);

/* The same grouped FFN with the row gather fused into the gate/up GEMM's
 * loads (lesson 10, item 3: the packed rows are only read by the expert
 * GEMM, so they are fetched from x where they lie).  Row i of the first GEMM
 * is row src_token[i] of x viewed as [T*H][d] (sub-token s = t*H + g is
 * x[t][g*d : g*d+d]), i.e. exactly the row moe_permute would have copied to
 * x_perm[i]; no x_perm is read or written.  src_token as produced by
 * moe_permute; values outside [0, T*H) are clamped to that range (never read
 * out of bounds).  Everything else as in moe_grouped_ffn; same workspace. */
moe_status moe_grouped_ffn_rows(const moe_desc *desc, const void *x, const int32_t *src_token,
                                const int32_t *offsets, int32_t max_rows, const void *w_gate,
                                const void *w_up, const void *w_down, void *h_tmp, void *y_perm,
                                uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Expert weights in fragment order, for the forward kernels (lesson 10, item
 * 3: the local experts run as one grouped GEMM; this is the weight layout that
 * GEMM reads fastest on gfx950).  w holds n_mat bf16 matrices [n_out][k]
 * (row-major, one after the other, as the expert weights are given);
 * w_packed receives the same n_mat * n_out * k values, matrix by matrix in
 * the same order and size, each reordered so that the 8 values one lane
 * passes to a 32x32x16 MFMA are contiguous: 16-byte piece
 *   ((nb * k/16 + s) * 64 + l)  of a matrix  =  W[32 nb + l % 32][16 s + 8 (l / 32) + 0..7]
 * for row block nb < n_out/32, 16-k step s < k/16 and lane l < 64.  Pack
 * w_gate, w_up and w_down (and sh_*, w_o) once, then pass the packed buffers
 * with desc->packed = 1.  Both buffers are device memory owned by the caller;
 * they must be 16-byte aligned and must not overlap.  n_out must be a
 * positive multiple of 32 and k of 16, else MOE_ERR_INVALID_ARG and nothing
 * is launched; n_mat = 0 is a no-op.  Asynchronous on `stream`. */
moe_status moe_pack_weights(const void *w, void *w_packed, int64_t n_mat, int32_t n_out, int32_t k,
                            void *stream);

/* Gate-weighted unpermute and combine (lesson 10, item 1 output formula and
 * item 3 weighted sum): y[t][g*d + j] = sum over k with dest_row >= 0, in slot
 * order, of topk_w[s][k] * y_perm[dest_row[s][k]][j] (fp32), plus
 * y_shared[t][j] when given (weight 1), rounded once.  A token whose
 * assignments are all dropped gets 0.
 *   y_shared [T][h] | NULL (H = 1 only);  y [T][h].
 * dest_row, topk_w, y_perm and y must be non-NULL when T > 0 (a NULL one is
 * MOE_ERR_INVALID_ARG, nothing launched). */
moe_status moe_combine(const moe_desc *desc, const int32_t *dest_row, const float *topk_w,
                       const void *y_perm, const void *y_shared, void *y, void *stream);

/* Weights of the whole layer; device pointers, unused ones NULL. */
typedef struct moe_weights {
    const void *w_router;
    const float *logit_bias;
    const float *select_bias;
    const void *w_gate, *w_up, *w_down;
    const void *sh_gate, *sh_up, *sh_down;
    const void *w_o;
    const int32_t *hash_keys; /* [T] keys of the hash gate, or NULL (key = token index) */
} moe_weights;

/* Optional outputs of moe_layer_forward; device pointers, any may be NULL.
 *   f_e = counts_e / (T K) (before drops), P_e as in moe_route,
 *   l_aux = alpha * E * sum_e f_e P_e, averaged over heads (lesson 10, item 4),
 *   n_dropped = T*H*K - n_kept. */
typedef struct moe_aux {
    int32_t *topk_idx; /* [T*H][K] */
    float *topk_w;     /* [T*H][K] */
    int32_t *dest_row; /* [T*H*K]  */
    int32_t *counts;   /* [H*E]    */
    int32_t *kept;     /* [H*E]    */
    int32_t *n_kept;   /* [1]      */
    int32_t *n_dropped;/* [1]      */
    float *f;          /* [H*E]    */
    float *P;          /* [H*E]    */
    float *l_aux;      /* [1]      */
} moe_aux;

/* The whole layer: route -> permute -> grouped FFN (+ shared expert) ->
 * combine (-> W_o) -> aux statistics, all on `stream` with no host sync.
 * With the hash gate, w_router is unused and P and l_aux are 0 (no scores).
 *   x [T][h], y [T][h]; capacity = moe_capacity(desc).
 * Needs moe_workspace_size(MOE_WS_LAYER) bytes of workspace. */
moe_status moe_layer_forward(const moe_desc *desc, const moe_weights *w, const void *x, void *y,
                             moe_aux *aux, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------ training
 * Every page is about training these layers (lesson 10; "HAI-LLM MoE"): the
 * backward pass of L = sum(dy * y) + aux_weight * L_aux, by the chain rule
 * through the forward pass above.  Selection (top-K, group limit, capacity)
 * is piecewise constant, so the router receives gradient only through the
 * gate weights (softmax or sigmoid over the selected experts, dropped slots
 * included) and through P_i of the aux loss (f_i is a count):
 *   softmax: dl_j = w_j (dw_j - sum_k w_k dw_k) + c p_j (f_j - sum_i f_i p_i)
 *   sigmoid: dl_j = (dw_j - sum_k w_k dw_k) / sum_S s * s_j (1 - s_j)
 *                   + c s_j (1 - s_j) / sum_all s * (f_j - sum_i f_i p_i)
 * with dw_k = <dy_t, expert output of slot k> (0 if dropped) and
 * c = aux_weight * alpha * E / (H * T).  The hash gate has no router.
 * Supported for MOE_BF16 with d = h/H, f and h multiples of 64.  Gradients
 * are bf16 (fp32 accumulation, one rounding); the intermediate row gradients
 * are bf16 as in the forward pass. */

/* State a training forward leaves for the backward pass: device buffers the
 * caller owns.  R = moe_max_rows(desc), n_act = 2 (SwiGLU) or 1 (GELU). */
typedef struct moe_saved {
    int32_t *topk_idx; /* [T*H][K] */
    float *topk_w;     /* [T*H][K] */
    int32_t *dest_row; /* [T*H*K] */
    int32_t *src_token;/* [T*H*K] (first n_kept used) */
    int32_t *offsets;  /* [H*E+1] */
    int32_t *counts;   /* [H*E] assignments before drops */
    float *logits;     /* [T*H][E] pre-bias router logits (unused by the hash gate) */
    void *act_grad;    /* [R][n_act*f] local derivatives of the expert activation h at the
                        * pre-activations a = x W_gate^T, u = x W_up^T: dh/da | dh/du
                        * (SwiGLU: u silu'(a) | silu(a); GELU: gelu'(a)), from fp32 */
    void *h;           /* [R][f] expert hidden activations */
    void *y_perm;      /* [R][d] expert outputs */
    void *sh_act_grad; /* [T][n_act*f] the same for the shared expert (n_shared) */
    void *sh_h;        /* [T][f] shared expert hidden activations (n_shared) */
    void *y_cat;       /* [T][h] combined output before W_o (has_wo) */
} moe_saved;

/* Gradients (device buffers, same shapes and dtype as the weights); every
 * one the layer has must be given. */
typedef struct moe_grads {
    void *dx;          /* [T][h] */
    void *w_router;    /* [H][E][d] (top-K gate) */
    void *w_gate, *w_up, *w_down;
    void *sh_gate, *sh_up, *sh_down;
    void *w_o;
} moe_grads;

/* R: rows of the packed expert buffers, min(T*H*K, H*E*C); -1 if invalid. */
int32_t moe_max_rows(const moe_desc *desc);

/* moe_layer_forward that also fills `saved` (every field the layer uses must
 * be non-NULL); the expert GEMMs then run on the 64-wide kernel.  Same
 * workspace as moe_layer_forward. */
moe_status moe_layer_forward_train(const moe_desc *desc, const moe_weights *w, const void *x, void *y,
                                   moe_aux *aux, const moe_saved *saved, void *ws, size_t ws_bytes,
                                   void *stream);

/* Gradients of L = sum(dy * y) + aux_weight * L_aux for the batch that the
 * training forward saved.  x [T][h] and the weights as in that call, dy
 * [T][h].  Needs moe_workspace_size(MOE_WS_BACKWARD) bytes (it holds the
 * row gradients, the routed copy of x's rows and the router's transposed
 * operands; the expert weights are read in place).  Deterministic. */
moe_status moe_layer_backward(const moe_desc *desc, const moe_weights *w, const void *x, const void *dy,
                              const moe_saved *saved, float aux_weight, moe_grads *grads, void *ws,
                              size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *moe_status_string(moe_status s);
/* Detail of the last error returned on the calling thread ("" if none). */
const char *moe_last_error(void);
/* Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
