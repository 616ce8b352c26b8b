// common.hpp -- device helpers and internal launcher declarations of libmoe.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16, round to nearest even, on gfx950's conversion instruction
// (v_cvt_pk_bf16_f32; for every non-NaN fp32 value it gives the bits of the
// integer formula u += 0x7fff + ((u >> 16) & 1), u >> 16, checked over all 2^32
// inputs; NaN stays NaN).  Two at a time where possible (pack_bf16x2).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2v v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte register vector
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------ wave helpers
__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// Partner value of one step of a butterfly all-reduce over groups of lanes,
// steps taken in the order OFF = 1, 2, 4, ..., with DPP and lane-swap
// instructions instead of an LDS permute.  OFF = 1, 2: quad permutes (lane ^
// OFF); 4: the mirror lane within each group of 8 (lane ^ 7), which holds the
// value of lane ^ 4 because each quad is uniform after the first two steps;
// 8: a rotation of each 16-lane row by 8 (lane ^ 8); 16, 32: the row and
// half-wave swaps (lane ^ 16, lane ^ 32).  Both partners of a step combine
// the same two values, so every lane of a group ends with the same bits, the
// ones the plain xor butterfly gives.
template <int V>
struct Off {
    static constexpr int value = V;
};
template <int LPT, typename F>
__device__ __forceinline__ void bfly_steps(F&& f) {
    if constexpr (LPT > 1) f(Off<1>{});
    if constexpr (LPT > 2) f(Off<2>{});
    if constexpr (LPT > 4) f(Off<4>{});
    if constexpr (LPT > 8) f(Off<8>{});
    if constexpr (LPT > 16) f(Off<16>{});
    if constexpr (LPT > 32) f(Off<32>{});
}
template <int OFF>
__device__ __forceinline__ uint32_t bfly_u32(uint32_t v) {
    if constexpr (OFF == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    if constexpr (OFF == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    if constexpr (OFF == 4) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
    if constexpr (OFF == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false); // row_ror:8
    if constexpr (OFF == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & 16) ? p[0] : p[1];
    }
    if constexpr (OFF == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? p[0] : p[1];
    }
}
template <int OFF>
__device__ __forceinline__ float bfly(float v) { return __uint_as_float(bfly_u32<OFF>(__float_as_uint(v))); }
template <int OFF>
__device__ __forceinline__ int bfly(int v) { return (int)bfly_u32<OFF>((uint32_t)v); }

// P from the route kernels' partials part[(g*nbx + b)*E + e] (block b's sum of
// head g's score distributions over its tokens): P_e = (sum over b) / T in one
// fixed order, LANES consecutive lanes per expert ge = g*E + e (16 for at most
// 64 experts in all, else 64: p_lanes), lane j adding b = j, j+LANES, ... in
// turn, then the butterfly over the LANES lanes.  All LANES lanes of the group
// must call it (valid false: no loads, any value); each returns the same bits.
constexpr int p_lanes(int Et) { return Et <= 64 ? 16 : 64; }
template <int LANES>
__device__ __forceinline__ float prob_mean_of(const float* part, int nbx, int E, int T, int ge, bool valid, int j) {
    float s = 0.0f;
    if (valid) {
        const int g = ge / E, e = ge - g * E;
        const float* p = part + (size_t)g * nbx * E + e;
#pragma unroll 8
        for (int b = j; b < nbx; b += LANES) s += p[(size_t)b * E];
    }
    bfly_steps<LANES>([&](auto O) __attribute__((always_inline)) { s += bfly<decltype(O)::value>(s); });
    return T > 0 ? s / (float)T : 0.0f;
}

// ------------------------------------------------------- internal launchers
// Every launcher enqueues on `st` and returns hipGetLastError() of the launch.
struct RouteArgs {
    int T, h, H, E, K, dtype, score;
    int n_groups, group_limit;  // group-limited top-K when n_groups > 1
    uint32_t flags;
    const void* x;
    const void* w_router;
    const float* logit_bias;
    const float* select_bias;
    float* logits;
    int32_t* topk_idx;
    float* topk_w;
    int32_t* counts;      // may be null
    float* prob_part;     // [n_blocks][H*E] partial sums of the score distribution, may be null
    void* split_ws;       // route_split_ws_bytes() of workspace for the split-K router GEMM, or null
    const float* logit_parts;  // internal: [n_parts][T][E] partial logits to sum (fixed order)
    int n_parts;
};
// workspace of the split-K router GEMM (0 where that path does not apply)
size_t route_split_ws_bytes(int T, int h, int H, int E, int dtype);
int route_blocks(int T, int h, int H, int E, int dtype);  // route blocks per head (= rows of prob_part per head)
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
// hash gate: topk_idx/topk_w [T*H] (K = 1); counts (may be null) accumulated
hipError_t launch_route_hash(const int32_t* keys, int T, int H, int E, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, hipStream_t st);
hipError_t launch_prob_mean(const float* prob_part, int n_blocks_per_head, int H, int E, int T,
                            float* prob_mean, hipStream_t st);

struct PermuteArgs {
    int A;        // assignments = T*H*K
    int K, H, Et, d, h, dtype;
    int capacity;
    int queue;            // MOE_QUEUE_TOKEN or MOE_QUEUE_CHOICE
    const int32_t* topk_idx;
    const void* x;        // may be null (no gather)
    int32_t* counts;
    int32_t* kept;
    int32_t* offsets;
    int32_t* dest_row;
    int32_t* src_token;
    void* x_perm;
    int32_t* n_kept;      // may be null
    int32_t* hist;        // ws: [n_chunks][Et]
    int max_rows;         // rows the gather grid covers
};
int permute_chunks(int A);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);

// one row tile of a grouped GEMM: rows [row0, row_end) of group `group`
// (group -1: an unused slot of the table)
struct GemmTile {
    int32_t group, row0, row_end, pad;
};
struct FfnArgs {
    int G;          // groups
    int d, f;       // in/out width of the layer and hidden width
    int dtype, act;
    int max_rows;
    const void* x_perm;         // GEMM1 activations: rows [max_rows][d], or x [a_nrows][d] with src_rows
    const int32_t* src_rows;    // null, or row i of GEMM1 reads row src_rows[i] of x_perm
    int a_nrows;                // rows behind x_perm when src_rows is given
    const int32_t* offsets;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    void* h_tmp;
    void* y_perm;
    uint32_t flags;
    GemmTile* tiles;  // ws: tile table
    void* act_save;   // training: GEMM1 also stores its pre-activations here [max_rows][n_act*f], or null
    const int32_t* c_rows;  // null, or row i of GEMM2 is stored to row c_rows[i] of y_perm (clamped to [0, c_nrows))
    int c_nrows;
    int packed;             // 1: w_gate, w_up, w_down in the fragment order of moe_pack_weights
};
size_t ffn_workspace_bytes(int G, int max_rows, int dtype);
hipError_t launch_ffn(const FfnArgs& a, hipStream_t st);

// One grouped bf16 GEMM on the 64-wide kernel: C[rows][Nout] = A[rows][K] B_g^T
// with group g owning rows [offsets[g], offsets[g+1]).  K % 64 == 0.
enum GemmMode { GEMM_SWIGLU = 0, GEMM_GELU = 1, GEMM_PLAIN = 2, GEMM_SWIGLU_SAVE = 3, GEMM_GELU_SAVE = 4,
                GEMM_DSWIGLU = 5, GEMM_DGELU = 6, GEMM_F32OUT = 7 };
struct GemmSpec {
    const void* A;          // [rows][K], or [a_mod][K] shared by the groups
    const void* B0;         // [G][Nout][K], or [Nout][K] with b_shared ([G][K][Nout] with b_kmajor)
    const void* B1;         // gated modes: the up weights, like B0
    void* C;                // [rows][Nout] ([rows][2*Nout] for GEMM_DSWIGLU)
    void* aux;              // SAVE / D modes: pre-activations [rows][n_act*Nout]
    int K, Nout;
    long long a_bytes;      // bytes of A the loads may address
    const int32_t* a_rows;  // optional row map of A
    const int2* kspan;      // optional per-group {first k stage, k stages}
    int a_mod;              // > 0: tile row r reads A row r % a_mod
    int b_shared;           // 1: one B for all groups
    int kmajor;             // 1: B0/B1 are [G][K][Nout] (the forward weights, for products by their
                            // transpose); ungated modes only.  2: A [rows][lda] and B0 [rows][ldb] are
                            // both k-major and group g sums their rows [krows[g], krows[g+1]) into its
                            // C rows (C row r of the group: column r % a_mod of A); plain mode only
    int kb1;                // kmajor 1: k rows >= kb1 are B1's rows k - kb1 (B0 and B1 then hold kb1
                            // rows each per group); 0: every k row is B0's
    const int32_t* krows;   // kmajor 2: the groups' k row ranges (G + 1 entries)
    int lda, ldb;           // kmajor 2: row strides of A and B0 in elements
    long long b_bytes;      // kmajor 2: bytes of B0 the loads may address
};
size_t grouped_gemm_ws_bytes(int G, int max_rows);  // its tile table
// bm: 128 or 256 forces the row-tile height, anything else picks it
hipError_t launch_grouped_gemm(int mode, const GemmSpec& s, const int32_t* offsets, int G, int max_rows,
                               GemmTile* tiles, hipStream_t st, int bm = 0);
// Dense GEMM y[rows][n] = x[rows][k] W^T with W [n][k] (one group; used for W_o).
hipError_t launch_dense(int rows, int k, int n, int dtype, const void* x, const void* w, void* y,
                        GemmTile* tiles, int32_t* offsets2, hipStream_t st, int packed = 0);
// n_mat bf16 matrices [n_out][k] (n_out % 32 == 0, k % 16 == 0) into fragment order
hipError_t launch_pack_weights(const void* w, void* out, long long n_mat, int n_out, int k, hipStream_t st);

struct CombineArgs {
    int T, H, K, d, h, dtype;
    const int32_t* dest_row;
    const float* topk_w;
    const void* y_perm;
    const void* y_shared;
    void* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
// K = 1, one head: y[t] = 0 for every token whose assignment was dropped (the
// kept ones are stored by the down GEMM's epilogue)
hipError_t launch_zero_dropped(const int32_t* dest_row, int T, int row_bytes, void* y, hipStream_t st);

struct StatsArgs {
    int T, H, E, K, A;
    float alpha;
    const int32_t* counts;
    const int32_t* kept_in;
    const int32_t* offsets;
    const float* prob_mean;   // P as computed, or null with prob_part
    const float* prob_part;   // the route kernels' partials (prob_mean_of), nbx blocks per head
    int nbx;
    float* f;
    float* P;
    float* l_aux;
    int32_t* n_kept;
    int32_t* n_dropped;
    int32_t* kept_out;
};
hipError_t launch_stats(const StatsArgs& a, hipStream_t st);

// backward pass (backward.hip)
hipError_t launch_kspan(const int32_t* offsets, int G, int max_stages, int2* kspan, int32_t* stage_grp,
                        hipStream_t st);
hipError_t launch_row_blocks(const void* in, int ld_in, int col0, int gcol, const int32_t* rowmap, int nrows_in,
                             int local_rows, const int32_t* offsets, const int2* kspan, const int32_t* stage_grp,
                             int max_stages, int ncols, void* out, long long ld_out, hipStream_t st);
hipError_t launch_gather_rows(const void* in, const int32_t* rowmap, int nrows_in, const int32_t* n_rows, int max_rows,
                              int ncols, void* out, hipStream_t st);
hipError_t launch_transpose_batched(const void* in, int B, int R, int Cc, void* out, int ld_out, int out_col0,
                                    hipStream_t st);
hipError_t launch_iota(int32_t* out, int n, int step, hipStream_t st);
hipError_t launch_combine_bwd(const void* dcat, int H, int d, int K, int A, const int32_t* dest_row,
                              const float* topk_w, const void* y_perm, void* dYp, float* dw, hipStream_t st);
hipError_t launch_router_bwd(int T, int H, int E, int K, int Ep, int score, float caux, const float* logits,
                             const float* logit_bias, const int32_t* topk_idx, const float* topk_w, const float* dw,
                             const int32_t* counts, void* dl, hipStream_t st);
hipError_t launch_dx(const void* dXp, const int32_t* dest_row, int T, int H, int d, int K, const void* dxr,
                     const void* dxs, void* dx, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);
hipError_t launch_set2(int32_t* p, int32_t a, int32_t b, hipStream_t st);

}  // namespace moe
