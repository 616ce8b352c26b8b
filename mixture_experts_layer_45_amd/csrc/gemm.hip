// gemm.hip -- the experts' FFNs as a ragged grouped GEMM.
//
// Lesson 10 "专家并行 EP" (learn.payai.win), "核心概念" item 3: once the rows are
// grouped by expert, the local experts run back to back as one grouped GEMM.
// "Chương 10: Song song MoE", item 1: each expert is an ordinary FFN.
//
// Group g owns rows [offsets[g], offsets[g+1]) of the activation matrix and
// its own weights W_g [Nout][K] (out-major).  The row ranges live on the
// device, so the launch is sized from host-side bounds and a one-block kernel
// first writes a table of the real M-tiles (group, first row, end row); the
// GEMM blocks read their tile from it and surplus blocks exit.
//
// Four bf16 kernels for gfx950 share the tile table, the XCD-aware schedule
// and the fused epilogue (activation in fp32, one rounding to bf16):
//   * gemm_bf16_w4_kernel -- 256-row tiles with K a multiple of 64 and at least
//     2048 (the top-2 layer's GEMMs, the shared expert, W_o): persistent, one
//     wave per SIMD holding a 128 x 128 quarter of the 256 x 256 tile, with a
//     hand-laid instruction schedule and the activations loaded two stages
//     ahead;
//   * gemm_bf16_k64_kernel  -- other shapes with K a multiple of 64: persistent,
//     8 waves, BM x 256 tiles, 64-wide k stages of whole 128-byte rows, 16-byte
//     row stores;
//   * gemm_bf16_ring8_kernel -- K % 64 == 32, and the training forward's gated
//     product on 256-row tiles with K >= 4096: persistent, 8 waves, a deeper
//     ring of 32-wide k stages;
//   * gemm_bf16_kernel -- any K (zero-filled tail), 4 waves, one tile per block.
// Measured on one MI355X: the 64-wide kernel is 10-25 % faster on 128-row tiles
// (256 experts x ~128 rows, d = 7168) and on short K (d = 512, f = 1024).
// The backward pass runs the 64-wide kernel on k-major operands, read where
// they lie through the LDS transposing load: the forward weights for the input
// gradients (KM = 1) and the activations for the weight gradients (KM = 2).
#include <algorithm>
#include <utility>

#include "common.hpp"

namespace moe {

// Epilogue modes.  The forward FFN uses SWIGLU/GELU (GEMM1) and PLAIN (GEMM2).
// Training and the backward pass add, on the 64-wide kernel only:
//   SWIGLU_SAVE / GELU_SAVE  GEMM1 that also stores the activation's local
//                            derivatives to `aux` [rows][n_act*Nout]: for
//                            h = silu(a) u, dh/da = u silu'(a) at column j and
//                            dh/du = silu(a) at Nout + j; for h = gelu(a),
//                            gelu'(a).  They are computed in fp32 from the fp32
//                            accumulators and rounded once, so the backward
//                            never differentiates a rounded pre-activation
//                            (silu' changes sign near a = -1.28, where that
//                            would lose every digit);
//   DSWIGLU / DGELU          a plain product dH whose epilogue multiplies it by
//                            those derivatives: da = dH dh/da, du = dH dh/du,
//                            stored to C [rows][n_act*Nout].
//   F32OUT                   a plain product stored in fp32 (C [rows][Nout] float):
//                            the router's partial logits.
enum { MODE_SWIGLU = 0, MODE_GELU = 1, MODE_PLAIN = 2, MODE_SWIGLU_SAVE = 3, MODE_GELU_SAVE = 4, MODE_DSWIGLU = 5,
       MODE_DGELU = 6, MODE_F32OUT = 7 };
__host__ __device__ constexpr bool gated_mode(int m) { return m == MODE_SWIGLU || m == MODE_SWIGLU_SAVE; }

// tile-claim counters after the tile table's header: 4 GemmTile entries = 16
// counters, 8 (one per XCD) for each of the two GEMM launches sharing a table
constexpr int kClaimSets = 4;

// ------------------------------------------------------------- tile table
// Row ranges are clamped to [0, max_rows) so inconsistent offsets can never send
// a tile past the buffers the launch was sized for.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* offsets, int G, int BM, int max_rows,
                                                          int max_tiles, GemmTile* tiles) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int per = (G + 1023) / 1024;
    int32_t nt[4];
    int32_t run = 0;
    for (int q = 0; q < per; ++q) {
        const int g = tid * per + q;
        int32_t r0 = 0, r1 = 0;
        if (g < G) {
            r0 = min(max(offsets[g], 0), max_rows);
            r1 = min(max(offsets[g + 1], r0), max_rows);
        }
        nt[q] = (r1 - r0 + BM - 1) / BM;
        run += nt[q];
    }
    part[tid] = run;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t pos = part[tid] - run;
    const int32_t total = part[1023];
    for (int q = 0; q < per; ++q) {
        const int g = tid * per + q;
        if (g >= G) break;
        const int32_t r0 = min(max(offsets[g], 0), max_rows);
        const int32_t r1 = min(max(offsets[g + 1], r0), max_rows);
        for (int i = 0; i < nt[q] && pos + i < max_tiles; ++i) {
            GemmTile t;
            t.group = g;
            t.row0 = r0 + i * BM;
            t.row_end = r1;
            t.pad = i;  // index within the group (the schedule finds the group's first tile from it)
            tiles[pos + i] = t;
        }
        pos += nt[q];
    }
    for (int i = total + tid; i < max_tiles; i += 1024) {
        GemmTile t;
        t.group = -1;
        t.row0 = t.row_end = t.pad = 0;
        tiles[i] = t;
    }
    if (tid == 0) {  // header after the table: the number of real tiles
        GemmTile h;
        h.group = min(total, max_tiles);
        h.row0 = h.row_end = h.pad = 0;
        tiles[max_tiles] = h;
    }
    // then the tile-claim counters of the GEMM launches that use this table
    // (8 per launch, one per XCD), cleared here because the table is rebuilt
    // in stream order before every such launch
    if (tid < 4 * kClaimSets) ((int32_t*)(tiles + max_tiles + 1))[tid] = 0;
}

constexpr int NGROUP = 4;  // consecutive N-tiles that walk the M-tiles together (default width)

struct GArgs {
    const void* A;   // [rows][K]
    const void* B0;  // [G][Nout][K]
    const void* B1;  // [G][Nout][K] (SwiGLU up) or null
    void* C;         // [rows][Nout]
    const GemmTile* tiles;
    int m_tiles, n_tiles, K, Nout, total, per_xcd;
    long long a_bytes;  // bytes of A the tiles may address (buffer bound of the 8-wave kernel)
    int32_t* claim;     // 8 zeroed tile-claim counters for this launch (persistent kernels)
    float* partial;     // fp32 partial tiles of the split last round (64-wide kernel), or null
    const int32_t* a_rows;  // row map: tile row i reads row a_rows[i] of A (null: row i)
    const int32_t* c_rows;  // row map of the plain, gated and GELU epilogues: tile row i is stored to row
                            // c_rows[i] of C, clamped to [0, c_nrows) (null: row i)
    int c_nrows;
    // 64-wide kernel only:
    void* aux;              // pre-activations: written by the SAVE modes, read by the D modes
    const int2* kspan;      // per group {first 64-wide k stage, k stages}, or null (0, K/64)
    int a_mod;              // > 0: tile row r reads A row r % a_mod (every group reads the same rows)
    int b_shared;           // 1: every group reads B0 itself (no per-group weight offset)
    int kb1;                // k-major B only: k rows >= kb1 come from B1 (row k - kb1); 0: all from B0
    // both operands k-major (A [rows][lda], B [rows][ldb], C row r = group g's
    // row r % a_mod): group g sums k rows [krows[g], krows[g+1]) of both
    const int32_t* krows;
    int lda, ldb;           // row strides in elements (k-major B alone: ldb 0 = Nout)
    long long b_bytes;      // bytes of B the loads may address
    int ngroup;             // column tiles per schedule group of the persistent kernels (0: NGROUP)
    int b_packed;           // 1: B0/B1 in the fragment-ordered layout of moe_pack_weights (forward kernels)
};

// the A row behind tile row r, clamped to the nrows rows of A
__device__ __forceinline__ int a_row(const GArgs& a, int r, int nrows) {
    if (a.a_mod > 0) return r % a.a_mod;
    if (!a.a_rows) return r;
    return min(max(a.a_rows[r], 0), nrows - 1);
}

// the C row that tile row r is stored to
__device__ __forceinline__ int c_row(const int32_t* c_rows, int c_nrows, int r) {
    return c_rows ? min(max(c_rows[r], 0), c_nrows - 1) : r;
}

// The last round of an XCD's slice is usually short (r < B tiles for B blocks):
// the 64-wide kernel then splits each of those r tiles into S pieces along K,
// one block each, that store fp32 partial tiles; a follow-up kernel adds each
// tile's pieces in piece order and runs the epilogue.  S <= B / r, at most
// kTailSlots pieces per XCD and at least kMinPieceStages k stages per piece.
constexpr int kTailSlots = 32;
constexpr int kMinPieceStages = 4;
__device__ __forceinline__ void tail_split(int Tx, int B, int nk, bool enabled, int& r, int& S) {
    r = B > 0 ? Tx % B : 0;
    S = 1;
    if (enabled && r > 0) {
        S = min(min(B / r, kTailSlots / r), nk / kMinPieceStages);
        if (S < 2) S = 1;
    }
}
// schedule index -> (row tile, column tile) and the row tile's table entry:
// groups of ng column tiles, each sweeping every real row tile.  Within a
// column group the items of one group's (expert's) ne row tiles are
// consecutive.  Groups of at most kPairedRows rows run column tile by column
// tile, so the row tiles that read one weight tile run back to back (measured:
// the 256-expert layer's gate/up GEMM, 128-row tiles, 3.30 -> 3.23 ms and 9 %
// fewer L2 misses); larger groups run row tile by row tile (four 256-row tiles
// of the multi-head layer's ~1000-row groups in the other order: 0.73 -> 0.74 ms).
// tiles[m].pad is the row tile's index within its group, so the group's first
// tile and tile count follow from any one of its tiles.
// The group width ng is NGROUP (4) for 256-row tiles.  128-row tiles take all
// column tiles in one group: each row tile's activations are then fetched by
// one XCD instead of one per group of 4 column tiles, and the weight tile
// still reaches its row tiles back to back (the 256-expert layer's down GEMM,
// 28 column tiles: 1.86 -> 1.75 ms; for 256-row tiles a wider group measured
// slower: top-2 gate/up 3.18 -> 3.46 ms at 16).
constexpr int kPairedRows = 512;
__device__ __forceinline__ GemmTile sched_decode(int si, int n_m, int n_tiles, const GemmTile* tiles, int BM, int& mt,
                                                 int& nt, int ng) {
    const int gsz = n_m * ng;
    const int nb = si / gsz;
    const int rem = si - nb * gsz;
    const int width = min(ng, n_tiles - nb * ng);
    const int m0 = rem / width;
    const GemmTile t0 = tiles[m0];
    const int f = m0 - t0.pad;  // the group's first row tile
    const int ne = min((t0.row_end - (t0.row0 - t0.pad * BM) + BM - 1) / BM, n_m - f);
    if (ne > 1 && ne * BM <= kPairedRows) {
        const int local = rem - width * f;
        mt = f + local % ne;
        nt = nb * ng + local / ne;
        return mt == m0 ? t0 : tiles[mt];
    }
    mt = m0;
    nt = nb * ng + (rem - m0 * width);
    return t0;
}
__device__ __forceinline__ int sched_width(const GArgs& a) { return a.ngroup > 0 ? a.ngroup : NGROUP; }


// block -> (m tile, n tile): blocks are dealt to the 8 XCDs round-robin, so block
// b runs on XCD b % 8; give each XCD a contiguous range of the schedule, and order
// the schedule as groups of NGROUP N-tiles sweeping all M-tiles.
__device__ __forceinline__ bool decode_tile(const GArgs& a, int& mt, int& nt) {
    const int b = blockIdx.x;
    const int s = (b & 7) * a.per_xcd + (b >> 3);
    if (s >= a.total) return false;
    const int gsz = a.m_tiles * NGROUP;
    const int nb = s / gsz;
    const int rem = s - nb * gsz;
    const int width = min(NGROUP, a.n_tiles - nb * NGROUP);
    mt = rem / width;
    nt = nb * NGROUP + (rem - mt * width);
    return true;
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (about 1 ulp in fp32):
// the result is rounded to bf16 (relative 2^-9) right after, so an IEEE
// division sequence per element would buy nothing but epilogue time
__device__ __forceinline__ float act_silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
// erf by Abramowitz and Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (|error| <= 1.5e-7 for x >= 0, odd extension below 0): inline, so the
// epilogue keeps its accumulators in registers.  The bf16 rounding of the
// result (relative 2^-9) dwarfs the approximation error.
__device__ __forceinline__ float erf_as(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    float p = 1.061405429f;
    p = p * t - 1.453152027f;
    p = p * t + 1.421413741f;
    p = p * t - 0.284496736f;
    p = p * t + 0.254829592f;
    p = p * t;
    const float r = 1.0f - p * __expf(-ax * ax);
    return x < 0.0f ? -r : r;
}
__device__ __forceinline__ float act_gelu(float a) { return 0.5f * a * (1.0f + erf_as(a * 0.70710678118654752f)); }

// ------------------------------------------------------------- bf16 MFMA
template <int BM, int MODE>
struct TileCfg {
    static constexpr int NMAT = MODE == MODE_SWIGLU ? 2 : 1;
    static constexpr int BNM = MODE == MODE_SWIGLU ? 128 : 256;  // output columns per matrix
    static constexpr int WM = BM / 2;
    static constexpr int WNM = BNM / 2;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WNM / 32;
    static constexpr int NACC = NMAT * TM * TN;
    static constexpr int A_BYTES = BM * 128;     // BM rows x 64 bf16
    static constexpr int B_BYTES = 256 * 128;    // 256 weight rows x 64 bf16
    static constexpr int STAGE = A_BYTES + B_BYTES;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int BM, int MODE>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GArgs a) {
    using C = TileCfg<BM, MODE>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    int mt, nt;
    if (!decode_tile(a, mt, nt)) return;
    const GemmTile tl = a.tiles[mt];
    if (tl.group < 0) return;
    const int grp = tl.group, row0 = tl.row0, row_end = tl.row_end;
    const int K = a.K, Nout = a.Nout;
    const int n0 = nt * C::BNM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = tid >> 3, lch = tid & 7;

    const uint16_t* Ab = (const uint16_t*)a.A;
    const uint16_t* B0 = (const uint16_t*)a.B0 + (size_t)grp * Nout * K;
    const uint16_t* B1 = MODE == MODE_SWIGLU ? (const uint16_t*)a.B1 + (size_t)grp * Nout * K : B0;

    const uint16_t* pa[BM / 32];
#pragma unroll
    for (int p = 0; p < BM / 32; ++p) {
        const int r = a_row(a, min(row0 + lrow + 32 * p, row_end - 1), (int)(a.a_bytes / ((long long)K * 2)));
        pa[p] = Ab + (size_t)r * K + lch * 8;
    }
    const uint16_t* pb[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int br = lrow + 32 * p;
        const int mat = br / C::BNM;
        const int col = min(n0 + br - mat * C::BNM, Nout - 1);
        pb[p] = (mat ? B1 : B0) + (size_t)col * K + lch * 8;
    }
    const int sw = (lch ^ (lrow & 7)) << 4;

    u32x4 ra[BM / 32], rb[8];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    floatx16 acc[C::NACC];
#pragma unroll
    for (int i = 0; i < C::NACC; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;

    const int nk = (K + 63) / 64;
    {
        const bool kin = lch * 8 < K;
#pragma unroll
        for (int p = 0; p < BM / 32; ++p) ra[p] = kin ? *(const u32x4*)(pa[p]) : zero;
#pragma unroll
        for (int p = 0; p < 8; ++p) rb[p] = kin ? *(const u32x4*)(pb[p]) : zero;
#pragma unroll
        for (int p = 0; p < BM / 32; ++p) *(u32x4*)(smem + (lrow + 32 * p) * 128 + sw) = ra[p];
#pragma unroll
        for (int p = 0; p < 8; ++p) *(u32x4*)(smem + C::A_BYTES + (lrow + 32 * p) * 128 + sw) = rb[p];
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * 64;
            const bool kin = k0 + lch * 8 < K;
#pragma unroll
            for (int p = 0; p < BM / 32; ++p) ra[p] = kin ? *(const u32x4*)(pa[p] + k0) : zero;
#pragma unroll
            for (int p = 0; p < 8; ++p) rb[p] = kin ? *(const u32x4*)(pb[p] + k0) : zero;
        }
        const uint8_t* As = smem + (kt & 1) * C::STAGE;
        const uint8_t* Bs = As + C::A_BYTES;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int ch = kk * 2 + (lane >> 5);
            bf16x8 af[C::TM], bfr[C::NMAT * C::TN];
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm) {
                const int r = wm * C::WM + tm * 32 + (lane & 31);
                af[tm] = *(const bf16x8*)(As + swz(r, ch));
            }
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) {
                    const int r = m * C::BNM + wn * C::WNM + tn * 32 + (lane & 31);
                    bfr[m * C::TN + tn] = *(const bf16x8*)(Bs + swz(r, ch));
                }
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < C::TN; ++tn) {
                        const int ai = (m * C::TM + tm) * C::TN + tn;
                        acc[ai] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm], bfr[m * C::TN + tn], acc[ai], 0, 0, 0);
                    }
        }
        if (more) {
            uint8_t* Ad = smem + ((kt + 1) & 1) * C::STAGE;
            uint8_t* Bd = Ad + C::A_BYTES;
#pragma unroll
            for (int p = 0; p < BM / 32; ++p) *(u32x4*)(Ad + (lrow + 32 * p) * 128 + sw) = ra[p];
#pragma unroll
            for (int p = 0; p < 8; ++p) *(u32x4*)(Bd + (lrow + 32 * p) * 128 + sw) = rb[p];
        }
        __syncthreads();
    }

    // epilogue: 32x32 accumulator element i of a lane is row 8*(i/4) + 4*(lane/32) + i%4,
    // column lane%32.  The activation is applied in place first (every index a
    // compile-time constant, so the accumulators stay in registers).
    if constexpr (MODE == MODE_SWIGLU) {
#pragma clang loop unroll(full)
        for (int t = 0; t < C::TM * C::TN; ++t)
#pragma clang loop unroll(full)
            for (int i = 0; i < 16; ++i) acc[t][i] = act_silu(acc[t][i]) * acc[C::TM * C::TN + t][i];
    } else if constexpr (MODE == MODE_GELU) {
#pragma clang loop unroll(full)
        for (int t = 0; t < C::TM * C::TN; ++t)
#pragma clang loop unroll(full)
            for (int i = 0; i < 16; ++i) acc[t][i] = act_gelu(acc[t][i]);
    }
    uint16_t* Cp = (uint16_t*)a.C;
#pragma clang loop unroll(full)
    for (int tm = 0; tm < C::TM; ++tm)
#pragma clang loop unroll(full)
        for (int tn = 0; tn < C::TN; ++tn) {
            const int col = n0 + wn * C::WNM + tn * 32 + (lane & 31);
#pragma clang loop unroll(full)
            for (int i = 0; i < 16; ++i) {
                const int row = row0 + wm * C::WM + tm * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                if (row < row_end && col < Nout)
                    Cp[(size_t)c_row(a.c_rows, a.c_nrows, row) * Nout + col] = f32_to_bf16(acc[tm * C::TN + tn][i]);
            }
        }
}

// ------------------------------------------------- bf16 MFMA, 8 waves, LDS ring
// 512 threads = 8 waves as 2 (M) x 4 (N), two waves per SIMD, each owning a
// (BM/2) x 64 sub-tile of the BM x 256 block tile (SwiGLU: 32 gate + 32 up
// columns), accumulators in registers.  A ring of NS = 4 LDS stages of BK = 32
// is filled by buffer loads that write straight into LDS.  Only waves 0-3 issue
// loads (a whole stage: BM/4 A rows and 64 weight rows each), so the MFMAs of
// waves 4-7 keep the matrix cores busy while a loading wave waits to issue; the
// four loads of a 4 KB run share one M0 value and differ by the instruction
// offset, which advances the global and the LDS address alike.  The 16-byte
// chunks of each 64-byte row are XOR-permuted by (row/2)%4 so that the 32x32x16
// fragment reads (8 lanes = 8 consecutive rows, one chunk) hit 8 distinct
// 16-byte bank groups; a load lane fetches the logical chunk its LDS slot holds.
// Iteration kt multiplies stage kt; the first fragments of stage kt+1 are read
// while the second half of stage kt is multiplied; stage kt+3 is loaded into the
// slot the barrier ending iteration kt-1 freed.  Needs K % 32 == 0 and every
// byte offset below 2^31 (checked by the launcher).
template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int BM, int MODE>
struct Ring8Cfg {
    static constexpr int NMAT = gated_mode(MODE) ? 2 : 1;
    static constexpr int BNM = gated_mode(MODE) ? 128 : 256;  // output columns per matrix
    static constexpr int WM = BM / 2;
    static constexpr int WNM = BNM / 4;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WNM / 32;
    static constexpr int NACC = NMAT * TM * TN;
    static constexpr int A_BYTES = BM * 64;
    static constexpr int B_BYTES = 256 * 64;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // ring depth: as many 32-wide k steps as fit in 160 KB of LDS (4 x 32 KB for
    // BM = 256, 6 x 24 KB for BM = 128), so NS-2 steps of loads are in flight
    static constexpr int NS = BM == 256 ? 4 : 6;
    static constexpr int A_LOADS = BM / 64;  // per loading wave: BM/4 rows in 16-row loads
    static constexpr int B_LOADS = 4;        // 64 weight rows per loading wave
    static constexpr int LOADS = A_LOADS + B_LOADS;
};

// 64-byte rows (32-wide stages): a 16-lane fragment read covers 16 rows at one
// logical chunk, i.e. 4 rows per 256-byte bank period; XOR-ing the chunk with
// (row/4)%4 gives those 16 lanes 16 distinct 16-byte bank groups
__device__ __forceinline__ int swz32(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) const uint8_t* lds_u8_ptr;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v* lds_s4_ptr;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt/lgkmcnt at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// gfx9 buffer descriptor word 3 for raw 32-bit-format buffer access
constexpr int kBufWord3 = 0x00020000;

// N buffer loads into consecutive 1 KB LDS runs sharing one M0 value: load i
// carries immediate offset 1024*i (a compile-time constant, as the instruction
// requires), which moves both its global and its LDS address.
// N loads on one LDS base, load i with immediate offset 1024 i (the offset
// field holds 12 bits, so at most four); AUX: the loads' cache-policy bits
// (kCpolNT: non-temporal)
constexpr int kCpolNT = 2;
template <int N, int AUX = 0>
struct LdsRun {
    static_assert(N <= 4, "immediate offsets above 4095 do not encode");
    static __device__ __forceinline__ void go(__amdgpu_buffer_rsrc_t r, lds_void_ptr lds, const uint32_t* v, int soff) {
        LdsRun<N - 1, AUX>::go(r, lds, v, soff);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, v[N - 1], soff, (N - 1) * 1024, AUX);
    }
};
template <int AUX>
struct LdsRun<0, AUX> {
    static __device__ __forceinline__ void go(__amdgpu_buffer_rsrc_t, lds_void_ptr, const uint32_t*, int) {}
};

// Epilogue of the persistent kernels (weight fragment as the MFMA's first
// operand): activation in fp32, one rounding to bf16, then (lane l holding row
// l%32 and, per group q of four, columns 8q + 4*(l/32) + 0..3) one
// v_permlane32_swap per register pair so that every lane stores 8 consecutive
// outputs (16 bytes).  C gives the wave tile (TM x TN 32x32 tiles, WM rows,
// WNM columns per matrix).
// Lane's 8 consecutive fp32 results of half pp of a 32x32 tile (columns
// 16pp + 8*(lane/32) + 0..7 of the tile), gathered with the same lane swap.
__device__ __forceinline__ void row8(const floatx16& v, int pp, float* e) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[8 * pp + j]), __float_as_uint(v[8 * pp + 4 + j]),
                                                        false, false);
        e[j] = __uint_as_float(s[0]);
        e[4 + j] = __uint_as_float(s[1]);
    }
}

__device__ __forceinline__ void bf16x8_to_f32(u32x4 v, float* e) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        e[2 * j] = __uint_as_float(v[j] << 16);
        e[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4 f32_to_bf16x8(const float* e) {
    return u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
}

// silu'(a) = sigma(a) (1 + a (1 - sigma(a))); gelu'(a) = Phi(a) + a phi(a)
__device__ __forceinline__ float sigma_f(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float dgelu_f(float a) {
    return 0.5f * (1.0f + erf_as(a * 0.70710678118654752f)) + a * 0.39894228040143268f * __expf(-0.5f * a * a);
}

template <typename C, int MODE>
__device__ __forceinline__ void rowstore_epilogue(floatx16* acc, int row0, int row_end, int n0, int Nout, uint8_t* Cp,
                                                  int wm, int wn, int lane, uint8_t* aux = nullptr,
                                                  const int32_t* c_rows = nullptr, int c_nrows = 0) {
    if constexpr (MODE == MODE_DSWIGLU || MODE == MODE_DGELU) {
        // acc holds dH; aux the saved pre-activations; C gets da (and du)
        constexpr int NA = MODE == MODE_DSWIGLU ? 2 : 1;
        const int ld = NA * Nout;
        const bool hi = lane >= 32;
#pragma clang loop unroll(full)
        for (int tm = 0; tm < C::TM; ++tm) {
            const int row = row0 + wm * C::WM + tm * 32 + (lane & 31);
            // the row block's saved derivatives are loaded first, all in flight
            // together (loads placed after a store to C would wait for it: the
            // compiler cannot tell that C and aux do not overlap)
            u32x4 sv[C::TN][2][NA];
#pragma clang loop unroll(full)
            for (int tn = 0; tn < C::TN; ++tn)
#pragma clang loop unroll(full)
                for (int pp = 0; pp < 2; ++pp) {
                    const int col = n0 + wn * C::WNM + tn * 32 + 16 * pp + (hi ? 8 : 0);
                    const bool ok = row < row_end && col < Nout;
                    const size_t at = ((size_t)row * ld + col) * 2;
#pragma unroll
                    for (int m = 0; m < NA; ++m)
                        sv[tn][pp][m] = ok ? *(const u32x4*)(aux + at + (size_t)m * Nout * 2) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma clang loop unroll(full)
            for (int tn = 0; tn < C::TN; ++tn) {
#pragma clang loop unroll(full)
                for (int pp = 0; pp < 2; ++pp) {
                    float g[8];
                    row8(acc[tm * C::TN + tn], pp, g);
                    const int col = n0 + wn * C::WNM + tn * 32 + 16 * pp + (hi ? 8 : 0);
                    if (row < row_end && col < Nout) {
                        const size_t at = ((size_t)row * ld + col) * 2;
#pragma unroll
                        for (int m = 0; m < NA; ++m) {
                            float dv[8];
                            bf16x8_to_f32(sv[tn][pp][m], dv);
#pragma unroll
                            for (int j = 0; j < 8; ++j) dv[j] *= g[j];
                            *(u32x4*)(Cp + at + (size_t)m * Nout * 2) = f32_to_bf16x8(dv);
                        }
                    }
                }
            }
        }
        return;
    }
    if constexpr (MODE == MODE_F32OUT) {
        const bool hi = lane >= 32;
#pragma clang loop unroll(full)
        for (int tm = 0; tm < C::TM; ++tm) {
            const int row = row0 + wm * C::WM + tm * 32 + (lane & 31);
#pragma clang loop unroll(full)
            for (int tn = 0; tn < C::TN; ++tn) {
#pragma clang loop unroll(full)
                for (int pp = 0; pp < 2; ++pp) {
                    float g[8];
                    row8(acc[tm * C::TN + tn], pp, g);
                    const int col = n0 + wn * C::WNM + tn * 32 + 16 * pp + (hi ? 8 : 0);
                    if (row < row_end && col < Nout) {
                        float* o = (float*)Cp + (size_t)row * Nout + col;
                        *(floatx4*)o = floatx4{g[0], g[1], g[2], g[3]};
                        *(floatx4*)(o + 4) = floatx4{g[4], g[5], g[6], g[7]};
                    }
                }
            }
        }
        return;
    }
    if constexpr (MODE == MODE_SWIGLU_SAVE) {
        // dh/da and dh/du of h = silu(a) u, eight outputs at a time (few live
        // registers next to the accumulators)
        const bool hi = lane >= 32;
#pragma clang loop unroll(full)
        for (int t = 0; t < C::TM * C::TN; ++t) {
            const int row = row0 + wm * C::WM + (t / C::TN) * 32 + (lane & 31);
#pragma clang loop unroll(full)
            for (int pp = 0; pp < 2; ++pp) {
                float av[8], uv[8], ga[8], gu[8];
                row8(acc[t], pp, av);
                row8(acc[C::TM * C::TN + t], pp, uv);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float sg = sigma_f(av[j]);
                    ga[j] = uv[j] * (sg * (1.0f + av[j] * (1.0f - sg)));
                    gu[j] = av[j] * sg;
                }
                const int col = n0 + wn * C::WNM + (t % C::TN) * 32 + 16 * pp + (hi ? 8 : 0);
                if (row < row_end && col < Nout) {
                    uint8_t* p = aux + ((size_t)row * 2 * Nout + col) * 2;
                    *(u32x4*)p = f32_to_bf16x8(ga);
                    *(u32x4*)(p + (size_t)Nout * 2) = f32_to_bf16x8(gu);
                }
            }
        }
    } else if constexpr (MODE == MODE_GELU_SAVE) {
        const bool hi = lane >= 32;
#pragma clang loop unroll(full)
        for (int t = 0; t < C::TM * C::TN; ++t) {
            const int row = row0 + wm * C::WM + (t / C::TN) * 32 + (lane & 31);
#pragma clang loop unroll(full)
            for (int pp = 0; pp < 2; ++pp) {
                float av[8], ga[8];
                row8(acc[t], pp, av);
#pragma unroll
                for (int j = 0; j < 8; ++j) ga[j] = dgelu_f(av[j]);
                const int col = n0 + wn * C::WNM + (t % C::TN) * 32 + 16 * pp + (hi ? 8 : 0);
                if (row < row_end && col < Nout) *(u32x4*)(aux + ((size_t)row * Nout + col) * 2) = f32_to_bf16x8(ga);
            }
        }
    }
    if constexpr (gated_mode(MODE)) {
#pragma clang loop unroll(full)
        for (int t = 0; t < C::TM * C::TN; ++t)
#pragma clang loop unroll(full)
            for (int i = 0; i < 16; ++i) acc[t][i] = act_silu(acc[t][i]) * acc[C::TM * C::TN + t][i];
    } else if constexpr (MODE == MODE_GELU || MODE == MODE_GELU_SAVE) {
#pragma clang loop unroll(full)
        for (int t = 0; t < C::TM * C::TN; ++t)
#pragma clang loop unroll(full)
            for (int i = 0; i < 16; ++i) acc[t][i] = act_gelu(acc[t][i]);
    }
    const bool hi = lane >= 32;
#pragma clang loop unroll(full)
    for (int tm = 0; tm < C::TM; ++tm) {
        const int row = row0 + wm * C::WM + tm * 32 + (lane & 31);
        const int crow = row < row_end ? c_row(c_rows, c_nrows, row) : row;
#pragma clang loop unroll(full)
        for (int tn = 0; tn < C::TN; ++tn) {
            const floatx16& v = acc[tm * C::TN + tn];
#pragma clang loop unroll(full)
            for (int pp = 0; pp < 2; ++pp) {
                // groups 2pp (columns 16pp + 0..7) and 2pp+1 (16pp + 8..15)
                uint32_t x0 = pack_bf16x2(v[8 * pp + 0], v[8 * pp + 1]), x1 = pack_bf16x2(v[8 * pp + 2], v[8 * pp + 3]);
                uint32_t y0 = pack_bf16x2(v[8 * pp + 4], v[8 * pp + 5]), y1 = pack_bf16x2(v[8 * pp + 6], v[8 * pp + 7]);
                const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                const u32x4 o = {s0[0], s1[0], s0[1], s1[1]};
                const int col = n0 + wn * C::WNM + tn * 32 + 16 * pp + (hi ? 8 : 0);
                if (row < row_end && col < Nout) *(u32x4*)(Cp + ((size_t)crow * Nout + col) * 2) = o;
            }
        }
    }
}

// Persistent form: one block per CU.  XCD x (blocks b with b % 8 == x) takes a
// contiguous slice of the tile schedule: its blocks start on the slice's first
// tiles and then claim the next unclaimed one from the XCD's counter (claimed at
// the start of a tile, so the atomic's latency hides under the k loop).  Tiles
// running at once on an XCD stay neighbours in the schedule (groups of NGROUP
// weight-column tiles sweeping one expert's row tiles) and share their rows in
// that XCD's L2, and a block that drew short tiles (the ragged last row tile
// of an expert) simply takes more of them.  When a tile's k loop ends, every
// LDS slot is free: the first stages of the block's next tile are loaded before
// the current tile's epilogue, which hides their latency.
template <int BM, int MODE>
__global__ __launch_bounds__(512, 1) void gemm_bf16_ring8_kernel(GArgs a) {
    // device pass only: the LDS address-space casts and the buffer-to-LDS loads
    // have no host meaning; the host pass needs nothing but the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Ring8Cfg<BM, MODE>;
    // the stages, then one word for the tile this block claimed for after the
    // current one (inside the same LDS array, so the compiler sees a single
    // LDS object and does not order fragment reads behind in-flight loads)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::NS * C::STAGE + 16];
    int32_t& next_tile = *(int32_t*)(smem + C::NS * C::STAGE);

    const int n_m = a.tiles[a.m_tiles].group;  // real row tiles (header of the table)
    const int total = n_m * a.n_tiles;
    const int xcd = blockIdx.x & 7, per = gridDim.x >> 3;
    const int q = (total + 7) / 8;
    const int s_end = min((xcd + 1) * q, total);
    int s = xcd * q + (blockIdx.x >> 3);
    if (s >= s_end) return;

    const int K = a.K, Nout = a.Nout;
    const uint32_t rowbytes = (uint32_t)K * 2u;
    const int nk = K / 32;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const bool loader = wu < 4;
    const int w4 = wu & 3;
    const bool upper = (w4 * 64) / C::BNM != 0;  // this loader's weight rows come from B1 (SwiGLU up)
    const int a_dst = w4 * (BM / 4) * 64;
    const int b_dst = C::A_BYTES + w4 * 64 * 64;
    const uint8_t* Ab = (const uint8_t*)a.A;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)Ab, (short)0, (int)a.a_bytes, kBufWord3);
    const int a_nrows = (int)(a.a_bytes / rowbytes);

    struct Tile {
        int row0, row_end, n0;
        __amdgpu_buffer_rsrc_t rB;
        uint32_t va[C::A_LOADS], vb[C::B_LOADS];
    };
    // per-lane byte offsets of this loader's rows; load i is issued with
    // immediate offset 1024*i, so the offset here is reduced by that amount
    auto setup = [&](int si, Tile& t) __attribute__((always_inline)) {
        int mt, nt;
        const GemmTile tl = sched_decode(si, n_m, a.n_tiles, a.tiles, BM, mt, nt, sched_width(a));
        t.row0 = tl.row0;
        t.row_end = tl.row_end;
        t.n0 = nt * C::BNM;
        const uint8_t* B0 = (const uint8_t*)a.B0 + (size_t)tl.group * Nout * rowbytes;
        const uint8_t* B1 = gated_mode(MODE) ? (const uint8_t*)a.B1 + (size_t)tl.group * Nout * rowbytes : B0;
        t.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(upper ? B1 : B0), (short)0, (int)((size_t)Nout * rowbytes), kBufWord3);
        const int lr = lane >> 2, pc = lane & 3;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            const int r = w4 * (BM / 4) + 16 * i + lr;
            const int c = pc ^ ((r >> 2) & 3);
            const int gr = a_row(a, min(t.row0 + r, t.row_end - 1), a_nrows);
            t.va[i] = (uint32_t)gr * rowbytes + (uint32_t)(c * 16) - 1024u * i;
        }
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
            const int r = w4 * 64 + 16 * i + lr;
            const int c = pc ^ ((r >> 2) & 3);
            const int mat = r / C::BNM;
            const int col = min(t.n0 + r - mat * C::BNM, Nout - 1);
            t.vb[i] = (uint32_t)col * rowbytes + (uint32_t)(c * 16) - 1024u * i;
        }
    };
    auto issue = [&](const Tile& t, int ks, int st) __attribute__((always_inline)) {
        if (!loader) return;
        const int koff = ks * 64;
        uint8_t* base = smem + st * C::STAGE;
        LdsRun<C::A_LOADS>::go(rA, (lds_void_ptr)(base + a_dst), t.va, koff);
        LdsRun<C::B_LOADS>::go(t.rB, (lds_void_ptr)(base + b_dst), t.vb, koff);
    };
    auto prologue = [&](const Tile& t) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < C::NS - 1; ++st)
            if (st < nk) issue(t, st, st);
    };
    // wait until at most `n` k steps of this wave's loads are still in flight
    auto wait_steps = [&](int n) __attribute__((always_inline)) {
        if (n >= 3) wait_vmcnt<3 * C::LOADS>();
        else if (n == 2) wait_vmcnt<2 * C::LOADS>();
        else if (n == 1) wait_vmcnt<C::LOADS>();
        else wait_vmcnt<0>();
    };
    // nv: this wave's 32-row blocks that hold rows of the tile (the others are
    // neither read nor multiplied; their accumulators stay zero, stores skip them)
    auto load_frags = [&](int st, int kk, bf16x8* af, bf16x8* bfr, int nv) __attribute__((always_inline)) {
        const uint8_t* As = smem + st * C::STAGE;
        const uint8_t* Bs = As + C::A_BYTES;
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
            if (tm < nv) af[tm] = *(const bf16x8*)(As + swz32(wm * C::WM + tm * 32 + (lane & 31), ch));
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn)
                bfr[m * C::TN + tn] = *(const bf16x8*)(Bs + swz32(m * C::BNM + wn * C::WNM + tn * 32 + (lane & 31), ch));
    };
    floatx16 acc[C::NACC];
    auto mfmas = [&](const bf16x8* af, const bf16x8* bfr, int nv) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) {
                    if (tm >= nv) continue;
                    const int ai = (m * C::TM + tm) * C::TN + tn;
                    acc[ai] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[m * C::TN + tn], af[tm], acc[ai], 0, 0, 0);
                }
    };

    Tile cur;
    setup(s, cur);
    prologue(cur);
    bf16x8 a0[C::TM], b0[C::NMAT * C::TN], a1[C::TM], b1[C::NMAT * C::TN];
    int32_t claim = 0;  // lane 0 of wave 0: the claim counter's answer for the current tile
    while (true) {
#pragma unroll
        for (int i = 0; i < C::NACC; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
        // claim the block's next tile now; the answer is needed only after the k loop
        if (tid == 0) claim = __hip_atomic_fetch_add(a.claim + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_steps(min(C::NS - 3, nk - 2));  // steps 0 and 1 landed
        __builtin_amdgcn_s_barrier();
        auto kloop = [&](auto NV) __attribute__((always_inline)) {
            constexpr int nv = decltype(NV)::value;
            load_frags(0, 0, a0, b0, nv);
            for (int kt = 0; kt < nk; ++kt) {
                if (kt + C::NS - 1 < nk) issue(cur, kt + C::NS - 1, (kt + C::NS - 1) % C::NS);
                load_frags(kt % C::NS, 1, a1, b1, nv);
                mfmas(a0, b0, nv);
                load_frags((kt + 1) % C::NS, 0, a0, b0, nv);  // last step: a valid slot, values unused
                mfmas(a1, b1, nv);
                wait_steps(min(C::NS - 3, nk - 3 - kt));  // step kt+2 landed
                if (kt == nk - 1) {  // this wave's loads (and the claim) have landed
                    if (tid == 0) next_tile = xcd * q + per + claim;
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the write is visible at the barrier
                }
                __builtin_amdgcn_s_barrier();
            }
        };
        // a ragged last row tile of a group leaves some waves' row blocks empty
        const int nvb = __builtin_amdgcn_readfirstlane(min(max((cur.row_end - cur.row0 - wm * C::WM + 31) / 32, 0), C::TM));
        if (nvb == C::TM) kloop(IntC<C::TM>{});
        else if (nvb == 0) kloop(IntC<0>{});
        else if (nvb == 1) kloop(IntC<1>{});
        else if constexpr (C::TM > 2) {
            if (nvb == 2) kloop(IntC<2>{});
            else kloop(IntC<3>{});
        }
        // every slot is free: start the next tile's loads, then store this one
        const int s_next = __builtin_amdgcn_readfirstlane(next_tile);
        const bool more = s_next < s_end;
        Tile nxt;
        if (more) {
            setup(s_next, nxt);
            prologue(nxt);
        }
        rowstore_epilogue<C, MODE>(acc, cur.row0, cur.row_end, cur.n0, Nout, (uint8_t*)a.C, wm, wn, lane, (uint8_t*)a.aux,
                                   a.c_rows, a.c_nrows);
        if (!more) break;
        cur = nxt;
        s = s_next;
    }
    wait_vmcnt<0>();
#endif
}

// ------------------------------------- bf16 MFMA, 8 waves, 64-wide k stages
// The block tile and wave grid of the ring kernel, but each LDS stage holds 64
// k values: every row of a stage is one whole 128-byte line of global memory,
// so a load instruction (64 lanes x 16 bytes = 8 rows) asks the L2 for full
// lines and no later k step re-requests the other half of a line.  The 16-byte
// chunks of a 128-byte row are XOR-permuted by (row/2)%8: the 16 lanes that the
// LDS serves together in a fragment read (16 consecutive rows, one chunk) then
// cover all 16 distinct 16-byte bank groups.  Two stages (BM = 256, 128 KB) or
// three (BM = 128, 144 KB); all eight waves load.
//
// The MFMA takes the weight fragment as its first operand, so a lane's
// accumulators run along an output row: lane l holds row l%32 and, in group q
// of four, columns 8q + 4*(l/32) + 0..3.  One v_permlane32_swap per register
// pair hands lane l the partner lane's half, after which every lane stores 8
// consecutive bf16 (16 bytes) -- two stores per 32x32 tile instead of sixteen.
template <int BM, int MODE>
struct K64Cfg {
    static constexpr int NMAT = gated_mode(MODE) ? 2 : 1;
    static constexpr int BNM = gated_mode(MODE) ? 128 : 256;  // output columns per matrix
    static constexpr int WM = BM / 2;
    static constexpr int WNM = BNM / 4;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WNM / 32;
    static constexpr int NACC = NMAT * TM * TN;
    static constexpr int NFR = TM + NMAT * TN;  // fragments per 16-wide k step
    static constexpr int A_BYTES = BM * 128;
    static constexpr int B_BYTES = 256 * 128;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int NS = BM == 256 ? 2 : 3;
    static constexpr int A_PW = BM / 64;  // activation loads per wave per stage (8 rows each)
    static constexpr int B_PW = 4;        // weight loads per wave per stage (32 rows)
    static constexpr int LPW = A_PW + B_PW;
};

__device__ __forceinline__ int swz64(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// k-major weights (B stored [K][Nout], as the forward weights are when the
// backward multiplies by their transpose): a stage holds 64 k rows of 512
// bytes (256 columns).  Row k's 16-byte chunk c sits at chunk c ^ kmaj_swz(k),
// so that the transposing fragment reads (4 rows x 32 bytes per 16 lanes, 4
// rows x 64 bytes per 32 lanes) touch distinct LDS banks.
__device__ __forceinline__ int kmaj_swz(int k) { return ((k & 3) << 1) ^ ((k & 1) << 3); }

// One transposing LDS read.  Through a restrict parameter the inlined read
// carries alias-scope information, without which the compiler waits for every
// LDS-DMA load in flight (the next stage's prefetch) before it.
__device__ __forceinline__ short4v lds_read_tr16(const uint8_t* __restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(lds_u8_ptr)p);
}


// fp32 partial tile of one piece: register (ai, 4q..4q+3) of thread tid at
// float4 index (ai*4 + q)*512 + tid of the slot (coalesced 16-byte stores)
template <int BM, int MODE>
__device__ __forceinline__ void k64_store_partial(const floatx16* acc, float* partial, int slot, int tid) {
    using C = K64Cfg<BM, MODE>;
    floatx4* P = (floatx4*)partial + (size_t)slot * (C::NACC * 4 * 512);
#pragma clang loop unroll(full)
    for (int ai = 0; ai < C::NACC; ++ai)
#pragma clang loop unroll(full)
        for (int q = 0; q < 4; ++q)
            P[(ai * 4 + q) * 512 + tid] = floatx4{acc[ai][4 * q], acc[ai][4 * q + 1], acc[ai][4 * q + 2], acc[ai][4 * q + 3]};
}

// KM = 1: B is k-major ([G][K][Nout]); its fragments are read with the LDS
// transposing load (each 16-lane group turns 4 k rows of 16 columns into 16
// lanes of 4 consecutive k), two reads per 8-k fragment.  KM = 2: A and B are
// both k-major, as the activations of a weight gradient are stored ([rows][.]
// with the rows of every group contiguous); group g's k range is its rows
// [krows[g], krows[g+1]), and the rows of a last stage past it load as zeros
// (their offsets are put past the buffer's range, which the load turns into
// zeros).
// PK: fragment-ordered weights (forward only).  Wave wu's four weight loads of
// a stage are then the 1 KB pieces of its 32-row block for the stage's four
// 16-k steps, each 1 KB of consecutive bytes, and the weight half of the stage
// keeps that order in LDS ([row block][16-k step][lane][16 bytes]): a wave's
// weight fragment is one conflict-free 1 KB read.
template <int BM, int MODE, int KM, bool PK = false>
__global__ __launch_bounds__(512, 1) void gemm_bf16_k64_kernel(GArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = K64Cfg<BM, MODE>;
    constexpr bool BT = KM >= 1, AT = KM == 2;
    static_assert(!BT || !gated_mode(MODE), "k-major weights are read by the ungated modes only");
    static_assert(!PK || KM == 0, "fragment-ordered weights are read by the forward products only");
    static_assert(!AT || BM == 256, "k-major activations fill 64 rows of 512 bytes per stage");
    constexpr int NS = C::NS;
    // the stages, then one word for the tile this block claimed for after the
    // current one (inside the same LDS array, so the compiler sees a single
    // LDS object and does not order fragment reads behind in-flight loads)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE + 16];
    int32_t& next_tile = *(int32_t*)(smem + NS * C::STAGE);

    const int K = a.K, Nout = a.Nout;
    const uint32_t rowbytes = (uint32_t)K * 2u;
    const int nk = K / 64;
    const int n_m = a.tiles[a.m_tiles].group;  // real row tiles (header of the table)
    const int total = n_m * a.n_tiles;
    const int xcd = blockIdx.x & 7, per = gridDim.x >> 3;
    const int q = (total + 7) / 8;
    const int tx0 = xcd * q;                     // this XCD's slice of the schedule
    const int Tx = max(0, min(q, total - tx0));
    int r_tail, S;
    tail_split(Tx, per, nk, a.partial != nullptr, r_tail, S);
    const int n_whole = S > 1 ? Tx - r_tail : Tx;  // items: whole tiles, then S pieces of each tail tile
    const int s_end = n_whole + (S > 1 ? r_tail * S : 0);
    int s = blockIdx.x >> 3;  // first item static, later ones claimed
    if (s >= s_end) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const bool upper = (wu * 32) / C::BNM != 0;  // this wave's weight rows come from B1 (SwiGLU up)
    const int a_dst = wu * (BM / 8) * 128;
    const int b_dst = C::A_BYTES + wu * 32 * 128;
    const uint8_t* Ab = (const uint8_t*)a.A;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)Ab, (short)0, (int)a.a_bytes, kBufWord3);
    const int a_nrows = (int)(a.a_bytes / rowbytes);

    // k-major operands: bytes per k row, and the k rows each weight matrix holds
    const uint32_t ldb = (uint32_t)(AT || a.ldb > 0 ? a.ldb : Nout) * 2u;
    const uint32_t lda = (uint32_t)a.lda * 2u;
    const int kmat = BT && a.kb1 > 0 ? a.kb1 : K;
    constexpr int bstage = PK ? 4096 : 128;  // weight bytes per 64-wide k stage along a row (row block)

    struct Tile {
        int row0, row_end, n0;
        int kb, nkl, slot;  // first k stage (KM = 2: first k row), k stages, partial slot (-1: a whole tile)
        int kend;           // KM = 2: the group's end row
        bool once;          // PK: the tile's group has one row tile, so its weights are read once
        __amdgpu_buffer_rsrc_t rB, rB1;
        uint32_t va[C::A_PW], vb[C::B_PW];
    };
    // per-lane byte offsets: lane l fills LDS chunk l%8 of row l/8 of its 8-row
    // run, so it fetches the logical chunk stored there; load i carries
    // immediate offset 1024*i, which is taken off here
    auto setup = [&](int item, Tile& t) __attribute__((always_inline)) {
        int si = tx0 + item;
        t.kb = 0;
        t.nkl = nk;
        t.slot = -1;
        if (item >= n_whole) {  // piece p of tail tile jt
            const int j = item - n_whole, jt = j / S, p = j - jt * S;
            si = tx0 + n_whole + jt;
            t.kb = p * nk / S;
            t.nkl = (p + 1) * nk / S - t.kb;
            t.slot = xcd * kTailSlots + j;
        }
        int mt, nt;
        const GemmTile tl = sched_decode(si, n_m, a.n_tiles, a.tiles, BM, mt, nt, sched_width(a));
        t.row0 = tl.row0;
        t.row_end = tl.row_end;
        t.n0 = nt * C::BNM;
        t.once = tl.row_end - (tl.row0 - tl.pad * BM) <= BM;
        if (a.kspan) {  // the group's own k range (no split pieces are made then)
            const int2 ks = a.kspan[tl.group];
            t.kb = ks.x;
            t.nkl = ks.y;
        }
        if constexpr (AT) {  // at least one stage, so that an empty group stores zeros
            t.kb = a.krows[tl.group];
            t.kend = a.krows[tl.group + 1];
            t.nkl = max(1, (t.kend - t.kb + 63) / 64);
        }
        const int lr = lane >> 3, pc = lane & 7;
        if constexpr (AT) {
            t.rB = __builtin_amdgcn_make_buffer_rsrc((void*)a.B0, (short)0, (int)a.b_bytes, kBufWord3);
            t.rB1 = t.rB;
        } else if constexpr (BT) {
            const size_t mbytes = (size_t)kmat * ldb;
            const size_t bgo = a.b_shared ? 0 : (size_t)tl.group * mbytes;
            t.rB = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.B0 + bgo), (short)0, (int)mbytes, kBufWord3);
            t.rB1 = a.kb1 > 0 ? __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.B1 + bgo), (short)0, (int)mbytes,
                                                                  kBufWord3)
                              : t.rB;
        } else {
            const size_t bgo = a.b_shared ? 0 : (size_t)tl.group * Nout * rowbytes;
            const uint8_t* B0 = (const uint8_t*)a.B0 + bgo;
            const uint8_t* B1 = gated_mode(MODE) ? (const uint8_t*)a.B1 + bgo : B0;
            t.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(upper ? B1 : B0), (short)0, (int)((size_t)Nout * rowbytes),
                                                     kBufWord3);
            t.rB1 = t.rB;
        }
        if constexpr (AT) {
            // as the k-major B below, columns = this tile's rows of the group
            const int m0 = t.row0 % a.a_mod;
#pragma unroll
            for (int i = 0; i < C::A_PW; ++i) {
                const int kr = wu * 8 + 2 * i + (lane >> 5);
                const int c = (lane & 31) ^ kmaj_swz(kr);
                const int col = min(m0 + c * 8, a.a_mod - 8);
                t.va[i] = (uint32_t)kr * lda + (uint32_t)col * 2u - 1024u * i;
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::A_PW; ++i) {
                const int r = wu * (BM / 8) + 8 * i + lr;
                const int c = pc ^ ((r >> 1) & 7);
                const int gr = a_row(a, min(t.row0 + r, t.row_end - 1), a_nrows);
                t.va[i] = (uint32_t)gr * rowbytes + (uint32_t)(c * 16) - 1024u * i;
            }
        }
        if constexpr (BT) {
            // load i of wave wu fills k rows 8wu+2i and 8wu+2i+1: lane l the
            // chunk at position l%32 of row l/32; chunks past Nout (whose
            // columns are never stored) reread the last real one.  With rows
            // under 512 bytes the offset less 1024*i can go below zero: the
            // unit adds offset and immediate in 32 bits, so the sum is exact
#pragma unroll
            for (int i = 0; i < C::B_PW; ++i) {
                const int kr = wu * 8 + 2 * i + (lane >> 5);
                const int c = (lane & 31) ^ kmaj_swz(kr);
                const int col = min(t.n0 + c * 8, Nout - 8);
                t.vb[i] = (uint32_t)kr * ldb + (uint32_t)col * 2u - 1024u * i;
            }
        } else if constexpr (PK) {
            // load i: piece `lane` of 16-k step 4 ks + i of the wave's 32-row
            // block (the load's immediate 1024 i selects the step); a block past
            // Nout (its columns are never stored) rereads the last one
            const int r0 = wu * 32;
            const int mat = r0 / C::BNM;
            const int nb32 = min((t.n0 + r0 - mat * C::BNM) >> 5, (Nout >> 5) - 1);
#pragma unroll
            for (int i = 0; i < C::B_PW; ++i) t.vb[i] = ((uint32_t)nb32 * (uint32_t)(K >> 4) * 64u + (uint32_t)lane) * 16u;
        } else {
#pragma unroll
            for (int i = 0; i < C::B_PW; ++i) {
                const int r = wu * 32 + 8 * i + lr;
                const int c = pc ^ ((r >> 1) & 7);
                const int mat = r / C::BNM;
                const int col = min(t.n0 + r - mat * C::BNM, Nout - 1);
                t.vb[i] = (uint32_t)col * rowbytes + (uint32_t)(c * 16) - 1024u * i;
            }
        }
    };
    // KM = 2: the offsets of stage ks, with the rows at or past the group's end
    // moved out of the buffer's range (they load as zeros); load i covers k
    // rows 8wu+2i (lanes 0-31) and 8wu+2i+1 (lanes 32-63) of the stage
    auto masked = [&](const Tile& t, int ks, const uint32_t* v, uint32_t* m) __attribute__((always_inline)) {
        const int rem = t.kend - (t.kb + 64 * ks);
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = wu * 8 + 2 * i + (lane >> 5) < rem ? v[i] : 0x80000000u;
    };
    // stage ks of the tile's k range
    auto issue_a = [&](const Tile& t, int ks) __attribute__((always_inline)) {
        lds_void_ptr dst = (lds_void_ptr)(smem + (ks % NS) * C::STAGE + a_dst);
        if constexpr (AT) {
            uint32_t m[C::A_PW];
            masked(t, ks, t.va, m);
            LdsRun<C::A_PW>::go(rA, dst, m, (int)((uint32_t)(t.kb + 64 * ks) * lda));
        } else {
            LdsRun<C::A_PW>::go(rA, dst, t.va, (t.kb + ks) * 128);
        }
    };
    auto issue_b = [&](const Tile& t, int ks) __attribute__((always_inline)) {
        lds_void_ptr dst = (lds_void_ptr)(smem + (ks % NS) * C::STAGE + b_dst);
        if constexpr (AT) {
            uint32_t m[C::B_PW];
            masked(t, ks, t.vb, m);
            LdsRun<C::B_PW>::go(t.rB, dst, m, (int)((uint32_t)(t.kb + 64 * ks) * ldb));
        } else if constexpr (BT) {
            const int k0 = (t.kb + ks) * 64;
            if (k0 >= kmat) LdsRun<C::B_PW>::go(t.rB1, dst, t.vb, (int)((uint32_t)(k0 - kmat) * ldb));
            else LdsRun<C::B_PW>::go(t.rB, dst, t.vb, (int)((uint32_t)k0 * ldb));
        } else if constexpr (PK) {
            // weights that no other tile reads stream past L2 (non-temporal), so
            // the activation rows that the group's column tiles share stay in it
            // (the 256-expert layer 5.32 -> 5.25 ms, the Zipf top-1 layer's expert
            // GEMMs 0.100 -> 0.085 and 0.103 -> 0.092 ms; non-temporal weights for
            // groups of two row tiles, which read each weight tile twice: 256-expert
            // layer 5.72 ms)
            if (t.once) LdsRun<C::B_PW, kCpolNT>::go(t.rB, dst, t.vb, (t.kb + ks) * bstage);
            else LdsRun<C::B_PW>::go(t.rB, dst, t.vb, (t.kb + ks) * bstage);
        } else {
            LdsRun<C::B_PW>::go(t.rB, dst, t.vb, (t.kb + ks) * bstage);
        }
    };
    auto prologue = [&](const Tile& t) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NS - 1; ++st)
            if (st < t.nkl) {
                issue_a(t, st);
                issue_b(t, st);
            }
    };
    // wait until at most n stages of this wave's loads are in flight (n <= 1)
    auto wait_stages = [&](int n) __attribute__((always_inline)) {
        if (n >= 1) wait_vmcnt<C::LPW>();
        else wait_vmcnt<0>();
    };
    // nv: this wave's 32-row blocks that hold rows of the tile (the others are
    // neither read nor multiplied; their accumulators stay zero, stores skip them)
    // k-major B: lane l's byte offset for column block tn of k step 0 (the
    // others add 8 KB per k step and 2 KB for the second 4-k read).  Lane
    // i = l%16 of group g = l/16 reads 4 columns (8 bytes) of k row
    // 8(g/2) + i/4 starting at column 16(g%2) + 4(i%4) of the block; the read
    // hands lane i the 4 rows of column 16(g%2) + i.
    // (k-major A alike, with column block wm*WM + 32 tm)
    int bt_off[C::TN], at_off[C::TM];
    if constexpr (BT) {
        const int kr = 8 * (lane >> 5) + ((lane >> 2) & 3);
        auto off = [&](int col0) {
            const int chunk = col0 / 8 + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
            return kr * 512 + ((chunk ^ kmaj_swz(kr)) << 4) + 8 * (lane & 1);
        };
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) bt_off[tn] = off(wn * C::WNM + tn * 32);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) at_off[tm] = off(wm * C::WM + tm * 32);
    }
    auto read_frags = [&](int st, int kk, bf16x8* fr, int nv) __attribute__((always_inline)) {
        const uint8_t* As = smem + st * C::STAGE;
        const uint8_t* Bs = As + C::A_BYTES;
        const int ch = kk * 2 + (lane >> 5);
        if constexpr (AT) {
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
                if (tm < nv) {
                    const uint8_t* p = As + at_off[tm] + kk * 8192;
                    const short4v lo = lds_read_tr16(p);
                    const short4v hi = lds_read_tr16(p + 2048);
                    fr[tm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
        } else {
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
                if (tm < nv) fr[tm] = *(const bf16x8*)(As + swz64(wm * C::WM + tm * 32 + (lane & 31), ch));
        }
        if constexpr (BT) {
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) {
                const uint8_t* p = Bs + bt_off[tn] + kk * 8192;
                const short4v lo = lds_read_tr16(p);
                const short4v hi = lds_read_tr16(p + 2048);
                fr[C::TM + tn] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        } else if constexpr (PK) {
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) {
                    const int rb = (m * C::BNM + wn * C::WNM + tn * 32) >> 5;
                    fr[C::TM + m * C::TN + tn] = *(const bf16x8*)(Bs + (rb * 4 + kk) * 1024 + lane * 16);
                }
        } else {
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn)
                    fr[C::TM + m * C::TN + tn] =
                        *(const bf16x8*)(Bs + swz64(m * C::BNM + wn * C::WNM + tn * 32 + (lane & 31), ch));
        }
    };
    floatx16 acc[C::NACC];
    auto mfmas = [&](const bf16x8* fr, int nv) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) {
                    if (tm >= nv) continue;
                    const int ai = (m * C::TM + tm) * C::TN + tn;
                    acc[ai] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[C::TM + m * C::TN + tn], fr[tm], acc[ai], 0, 0, 0);
                }
    };

    Tile cur;
    setup(s, cur);
    prologue(cur);
    bf16x8 fa[C::NFR], fb[C::NFR];
    int32_t claim = 0;  // lane 0 of wave 0: the claim counter's answer for the current tile
    // 256-row tiles set up the next tile (its table entry and row offsets, two
    // dependent global loads) during stage 1 of the current one, so that its
    // first loads go out as soon as the k loop ends (the multi-head layer's
    // K = 512 gate/up GEMM: 0.68 -> 0.66 ms); 128-row tiles do it after the k
    // loop (early: the 256-expert gate/up GEMM 3.17 -> 3.19 ms), and so do the
    // training and backward modes, whose 256-row variants would then spill
    constexpr bool kEarly = BM == 256 && KM == 0 && MODE <= MODE_PLAIN;
    Tile nxt;
    int s_next = s_end;
    bool more = false;
    while (true) {
#pragma unroll
        for (int i = 0; i < C::NACC; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
        // claim the block's next tile now; the answer is needed at the end of stage 0
        // (256-row tiles) or of the k loop
        if (tid == 0) claim = __hip_atomic_fetch_add(a.claim + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int nkl = cur.nkl;
        wait_stages(min(NS - 2, nkl - 1));  // stage 0 landed
        __builtin_amdgcn_s_barrier();
        auto kloop = [&](auto NV) __attribute__((always_inline)) {
            constexpr int nv = decltype(NV)::value;
            read_frags(0, 0, fa, nv);
            for (int kt = 0; kt < nkl; ++kt) {
                const int slot = kt % NS;
                const int ls = kt + NS - 1;  // stage loaded during this one, into the slot freed by the last barrier
                if (ls < nkl) issue_a(cur, ls);
                read_frags(slot, 1, fb, nv);
                mfmas(fa, nv);
                if (ls < nkl) issue_b(cur, ls);
                read_frags(slot, 2, fa, nv);
                mfmas(fb, nv);
                read_frags(slot, 3, fb, nv);
                mfmas(fa, nv);
                mfmas(fb, nv);
                wait_stages(min(NS - 2, nkl - 2 - kt));  // stage kt+1 landed
                // the claim, issued before stage NS-1's loads, has landed
                if (kt == (kEarly ? 0 : nkl - 1)) {
                    if (tid == 0) next_tile = per + claim;
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the write is visible at the barrier
                }
                __builtin_amdgcn_s_barrier();
                if (kEarly && kt == 0) {
                    // the next tile's table entry and row offsets load during stage 1
                    s_next = __builtin_amdgcn_readfirstlane(next_tile);
                    more = s_next < s_end;
                    if (more) setup(s_next, nxt);
                }
                if (kt + 1 < nkl) read_frags((kt + 1) % NS, 0, fa, nv);
            }
        };
        // a ragged last row tile of a group leaves some waves' row blocks empty
        const int nvb = __builtin_amdgcn_readfirstlane(min(max((cur.row_end - cur.row0 - wm * C::WM + 31) / 32, 0), C::TM));
        if (nvb == C::TM) kloop(IntC<C::TM>{});
        else if (nvb == 0) kloop(IntC<0>{});
        else if (nvb == 1) kloop(IntC<1>{});
        else if constexpr (C::TM > 2) {
            if (nvb == 2) kloop(IntC<2>{});
            else kloop(IntC<3>{});
        }
        // every slot is free: start the next tile's loads, then store this one
        if constexpr (!kEarly) {
            s_next = __builtin_amdgcn_readfirstlane(next_tile);
            more = s_next < s_end;
            if (more) setup(s_next, nxt);
        }
        if (more) prologue(nxt);
        if (cur.slot >= 0)
            k64_store_partial<BM, MODE>(acc, a.partial, cur.slot, tid);
        else
            rowstore_epilogue<K64Cfg<BM, MODE>, MODE>(acc, cur.row0, cur.row_end, cur.n0, Nout, (uint8_t*)a.C, wm, wn, lane,
                                                      (uint8_t*)a.aux, a.c_rows, a.c_nrows);
        if (!more) break;
        cur = nxt;
        s = s_next;
    }
    wait_vmcnt<0>();
#endif
}

// Sums the pieces of each split tail tile (in piece order) and runs the
// epilogue.  One block per (XCD, tail tile); `per` = blocks per XCD of the GEMM
// launch, so the split is recomputed exactly as that launch made it.
template <int BM, int MODE>
__global__ __launch_bounds__(512) void gemm_k64_tail_kernel(GArgs a, int per) {
    using C = K64Cfg<BM, MODE>;
    const int xcd = blockIdx.x / kTailSlots, jt = blockIdx.x % kTailSlots;
    const int nk = a.K / 64;
    const int n_m = a.tiles[a.m_tiles].group;
    const int total = n_m * a.n_tiles;
    const int q = (total + 7) / 8;
    const int tx0 = xcd * q;
    const int Tx = max(0, min(q, total - tx0));
    int r_tail, S;
    tail_split(Tx, per, nk, a.partial != nullptr, r_tail, S);
    if (S < 2 || jt >= r_tail) return;
    int mt, nt;
    const GemmTile tl = sched_decode(tx0 + Tx - r_tail + jt, n_m, a.n_tiles, a.tiles, BM, mt, nt, sched_width(a));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    floatx16 acc[C::NACC];
#pragma unroll
    for (int i = 0; i < C::NACC; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
    for (int p = 0; p < S; ++p) {
        const floatx4* P = (const floatx4*)a.partial + (size_t)(xcd * kTailSlots + jt * S + p) * (C::NACC * 4 * 512);
#pragma unroll
        for (int ai = 0; ai < C::NACC; ++ai)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4 v = P[(ai * 4 + q4) * 512 + tid];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[ai][4 * q4 + i] += v[i];
            }
    }
    rowstore_epilogue<K64Cfg<BM, MODE>, MODE>(acc, tl.row0, tl.row_end, nt * C::BNM, a.Nout, (uint8_t*)a.C, wave >> 2, wave & 3, lane,
                                              (uint8_t*)a.aux, a.c_rows, a.c_nrows);
}


// ------------------------------------ bf16 MFMA, 4 waves of 128 x 128, 256-row tiles
// One wave per SIMD (256 threads) on a 256 x 256 block tile (the 64-wide
// kernel's stage layout, swizzle, loads, schedule order and split tail), each
// wave owning a 128 x 128 quarter: 16 accumulator tiles (256 registers, all in
// AGPRs) and, per 16-wide k sub-step, 4 activation and 4 weight fragments for
// 16 MFMAs -- a third fewer LDS reads per MFMA than the 8-wave kernel's
// 128 x 64 waves.  With no second wave on the SIMD to cover for it, the wave's
// instruction stream is laid out by hand (scheduling barriers fix the order):
// every sub-step reads the next one's 8 fragments behind its first 8 MFMAs;
// the loads ride on the stage's first 32 MFMAs, one per two; the stage's wait
// and block barrier sit before the last 8 MFMAs, which then cover the reads of
// the next stage's first fragments.  All of LDS holds three stages of
// activation rows and two of weight rows, so the activations load two stages
// ahead; with no room left for a claim word, each block takes every 32nd item
// of its XCD's slice.  Measured on the top-2 layer (gate/up, down): 3.45, 1.72
// ms on the ring and 64-wide kernels; 3.26-3.32, 1.70-1.76 ms here with two
// stages of each operand; 3.18-3.24, 1.59-1.61 ms with the activation ring.
// The clock under the gate/up GEMM rose from 1.58 to 1.70 GHz with the
// 4-wave layout (fewer LDS operations) at the same MFMA count.
template <int MODE>
struct W4Cfg {
    static constexpr int NMAT = gated_mode(MODE) ? 2 : 1;
    static constexpr int BNM = gated_mode(MODE) ? 128 : 256;  // output columns per matrix
    static constexpr int WM = 128;
    static constexpr int WNM = BNM / 2;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WNM / 32;
    static constexpr int NB = NMAT * TN;    // weight fragments per sub-step
    static constexpr int NACC = TM * NB;    // 32 x 32 accumulator tiles per wave
    static constexpr int NRD = TM + NB;     // fragment reads per sub-step
    static constexpr int A_BYTES = 256 * 128;  // one stage of activation rows (64 k values each)
    static constexpr int B_BYTES = 256 * 128;  // one stage of weight rows
    static constexpr int LPW = 16;          // loads per wave per stage (8 activation, 8 weight rows x 8)
    static constexpr int WN = 2;           // waves along the weight rows (2 x 2)
    static_assert(NACC == 16 && NRD == 8, "the hand-laid schedule assumes 16 MFMAs and 8 reads per sub-step");
};

// The fragment-order kernel's waves: 1 x 4, each wave all 256 rows of the
// tile and a quarter of its weight rows (gated: 32 gate and the same 32 up
// columns), so no two waves load the same weight fragment.  Per sub-step a
// wave reads 8 activation fragments from LDS and takes 2 weight fragments
// from registers for its 16 MFMAs.
template <int MODE>
struct W4PCfg {
    static constexpr int NMAT = gated_mode(MODE) ? 2 : 1;
    static constexpr int BNM = gated_mode(MODE) ? 128 : 256;  // output columns per matrix
    static constexpr int WM = 256;
    static constexpr int WNM = BNM / 4;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WNM / 32;
    static constexpr int NB = NMAT * TN;  // weight fragments per sub-step
    static constexpr int NACC = TM * NB;
    static constexpr int NRD = TM + NB;
    static constexpr int A_BYTES = 256 * 128;
    static constexpr int WN = 4;          // waves along the weight rows
    static_assert(NACC == 16 && NB == 2, "16 MFMAs and 2 weight fragments per sub-step");
};

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(IntC<Is>{}), ...);
}
// f(IntC<0>{}), ..., f(IntC<N-1>{}) in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One 32 x 32 output tile of the 4-wave kernel: activation in fp32, one
// rounding, one lane swap per register pair, 16-byte row stores (the layout
// of rowstore_epilogue).  g (and u, the up product of SwiGLU) are in VGPRs.
template <int MODE>
__device__ __forceinline__ void w4_store_tile(floatx16 g, const floatx16& u, int row, int row_end, int crow, int col0,
                                              int Nout, uint8_t* Cp, bool hi) {
    if constexpr (gated_mode(MODE)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) g[i] = act_silu(g[i]) * u[i];
    } else if constexpr (MODE == MODE_GELU) {
#pragma unroll
        for (int i = 0; i < 16; ++i) g[i] = act_gelu(g[i]);
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        // groups 2pp (columns 16pp + 0..7) and 2pp+1 (16pp + 8..15)
        const uint32_t x0 = pack_bf16x2(g[8 * pp + 0], g[8 * pp + 1]), x1 = pack_bf16x2(g[8 * pp + 2], g[8 * pp + 3]);
        const uint32_t y0 = pack_bf16x2(g[8 * pp + 4], g[8 * pp + 5]), y1 = pack_bf16x2(g[8 * pp + 6], g[8 * pp + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const u32x4 o = {s0[0], s1[0], s0[1], s1[1]};
        const int col = col0 + 16 * pp + (hi ? 8 : 0);
        if (row < row_end && col < Nout) *(u32x4*)(Cp + ((size_t)crow * Nout + col) * 2) = o;
    }
}

// The wave's tiles one at a time.  Each accumulator tile is pinned to AGPRs
// (an empty asm with an "a" operand) right before it is copied out: otherwise
// the compiler copies all 256 accumulators to VGPRs at the end of the k loop
// and spills.
template <typename C, int MODE>
__device__ __forceinline__ void w4_epilogue_cfg(const floatx16* acc, int row0, int row_end, int n0, int Nout,
                                                uint8_t* Cp, int wm, int wn, int lane, const int32_t* c_rows,
                                                int c_nrows) {
    const bool hi = lane >= 32;
#pragma clang loop unroll(full)
    for (int tm = 0; tm < C::TM; ++tm) {
        const int row = row0 + wm * C::WM + tm * 32 + (lane & 31);
        const int crow = row < row_end ? c_row(c_rows, c_nrows, row) : row;
#pragma clang loop unroll(full)
        for (int tn = 0; tn < C::TN; ++tn) {
            floatx16 g = acc[tm * C::TN + tn];
            asm volatile("" : "+a"(g));
            if constexpr (gated_mode(MODE)) {
                floatx16 u = acc[C::TM * C::TN + tm * C::TN + tn];
                asm volatile("" : "+a"(u));
                w4_store_tile<MODE>(g, u, row, row_end, crow, n0 + wn * C::WNM + tn * 32, Nout, Cp, hi);
            } else {
                w4_store_tile<MODE>(g, g, row, row_end, crow, n0 + wn * C::WNM + tn * 32, Nout, Cp, hi);
            }
        }
    }
}

template <int MODE>
__device__ __forceinline__ void w4_epilogue(const floatx16* acc, int row0, int row_end, int n0, int Nout, uint8_t* Cp,
                                            int wm, int wn, int lane, const int32_t* c_rows, int c_nrows) {
    w4_epilogue_cfg<W4Cfg<MODE>, MODE>(acc, row0, row_end, n0, Nout, Cp, wm, wn, lane, c_rows, c_nrows);
}

// fp32 partial tile of one piece: accumulator (ai, 4q..4q+3) of thread tid at
// float4 index (ai*4 + q)*256 + tid of the slot
template <int MODE>
__device__ __forceinline__ void w4_store_partial(const floatx16* acc, float* partial, int slot, int tid) {
    using C = W4Cfg<MODE>;
    floatx4* P = (floatx4*)partial + (size_t)slot * (C::NACC * 4 * 256);
#pragma clang loop unroll(full)
    for (int ai = 0; ai < C::NACC; ++ai) {
        floatx16 v = acc[ai];
        asm volatile("" : "+a"(v));
#pragma unroll
        for (int q = 0; q < 4; ++q) P[(ai * 4 + q) * 256 + tid] = floatx4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    }
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void gemm_bf16_w4_kernel(GArgs a) {
    // device pass only (LDS address-space casts, buffer-to-LDS loads)
#if defined(__HIP_DEVICE_COMPILE__)
    using C = W4Cfg<MODE>;
    constexpr int TM = C::TM, NB = C::NB, NRD = C::NRD;
    // all of LDS: the activation rows of three stages, then the weight rows of two
    __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * C::A_BYTES + 2 * C::B_BYTES];
    constexpr int B_OFF = 3 * C::A_BYTES;

    const int K = a.K, Nout = a.Nout;
    const uint32_t rowbytes = (uint32_t)K * 2u;
    const int nk = K / 64;
    const int n_m = a.tiles[a.m_tiles].group;  // real row tiles (header of the table)
    const int total = n_m * a.n_tiles;
    const int xcd = blockIdx.x & 7, per = gridDim.x >> 3;
    const int q = (total + 7) / 8;
    const int tx0 = xcd * q;  // this XCD's slice of the schedule
    const int Tx = max(0, min(q, total - tx0));
    int r_tail, S;
    tail_split(Tx, per, nk, a.partial != nullptr, r_tail, S);
    const int n_whole = S > 1 ? Tx - r_tail : Tx;  // items: whole tiles, then S pieces of each tail tile
    const int s_end = n_whole + (S > 1 ? r_tail * S : 0);
    int s = blockIdx.x >> 3;  // items s, s + per, s + 2 per, ... of the XCD's slice
    if (s >= s_end) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const bool upper = (wu * 64) / C::BNM != 0;  // this wave's weight rows come from B1 (SwiGLU up)
    const int a_dst = wu * 64 * 128;  // this wave's 64 rows of a slot
    const int b_dst = B_OFF + wu * 64 * 128;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, (short)0, (int)a.a_bytes, kBufWord3);
    const int a_nrows = (int)(a.a_bytes / rowbytes);

    struct Tile {
        int row0, row_end, n0;
        int kb, nkl, slot;  // first k stage, k stages, partial slot (-1: a whole tile)
        __amdgpu_buffer_rsrc_t rB;
        uint32_t va[8], vb[8];
    };
    // lane l of load i fills LDS chunk l%8 of row 8i + l/8 of the wave's 64-row
    // run, so it fetches the logical chunk stored there; loads come in groups
    // of four on one LDS base with immediate offsets 1024*(i%4), taken off here
    auto setup = [&](int item, Tile& t) __attribute__((always_inline)) {
        int si = tx0 + item;
        t.kb = 0;
        t.nkl = nk;
        t.slot = -1;
        if (item >= n_whole) {  // piece p of tail tile jt
            const int j = item - n_whole, jt = j / S, p = j - jt * S;
            si = tx0 + n_whole + jt;
            t.kb = p * nk / S;
            t.nkl = (p + 1) * nk / S - t.kb;
            t.slot = xcd * kTailSlots + j;
        }
        int mt, nt;
        const GemmTile tl = sched_decode(si, n_m, a.n_tiles, a.tiles, 256, mt, nt, sched_width(a));
        t.row0 = tl.row0;
        t.row_end = tl.row_end;
        t.n0 = nt * C::BNM;
        const size_t bgo = a.b_shared ? 0 : (size_t)tl.group * Nout * rowbytes;
        const uint8_t* B0 = (const uint8_t*)a.B0 + bgo;
        const uint8_t* B1 = gated_mode(MODE) ? (const uint8_t*)a.B1 + bgo : B0;
        t.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(upper ? B1 : B0), (short)0, (int)((size_t)Nout * rowbytes), kBufWord3);
        const int lr = lane >> 3, pc = lane & 7;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wu * 64 + 8 * i + lr;
            const int c = pc ^ ((r >> 1) & 7);
            const int gr = a_row(a, min(t.row0 + r, t.row_end - 1), a_nrows);
            t.va[i] = (uint32_t)gr * rowbytes + (uint32_t)(c * 16) - 1024u * (i % 4);
            const int mat = r / C::BNM;
            const int col = min(t.n0 + r - mat * C::BNM, Nout - 1);
            t.vb[i] = (uint32_t)col * rowbytes + (uint32_t)(c * 16) - 1024u * (i % 4);
        }
    };
    // load j of stage ks of the tile: activation rows for j < 8 (into slot
    // ks % 3), weight rows for j >= 8 (slot ks % 2)
    auto ld1 = [&](const Tile& t, int ks, auto J) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        constexpr int i = j % 8;
        uint8_t* dst = smem + (j < 8 ? (ks % 3) * C::A_BYTES + a_dst : (ks % 2) * C::B_BYTES + b_dst) + 4096 * (i / 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 8 ? rA : t.rB, (lds_void_ptr)dst, 16, j < 8 ? t.va[i] : t.vb[i],
                                                 (t.kb + ks) * 128, 1024 * (i % 4), 0);
    };
    // fragment addresses: every row a lane reads is (lane % 32) plus a multiple
    // of 32, so its swizzle term ((row / 2) % 8) is lane-constant
    const int xsw = ((lane & 31) >> 1) & 7;
    const uint32_t a_lane = (uint32_t)((wm * C::WM + (lane & 31)) * 128);
    const uint32_t b_lane = (uint32_t)(B_OFF + (wn * C::WNM + (lane & 31)) * 128);
    uint32_t chofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) chofs[kk] = (uint32_t)(((kk * 2 + (lane >> 5)) ^ xsw) << 4);
    // read j of sub-step kk, in the order the MFMAs below use them: activation
    // block 0, the NB weight fragments, activation blocks 1..TM-1 (blocks past
    // the tile's rows, tm >= nv, are skipped)
    // (ks: the k stage, whose activations sit in slot ks % 3 and weights in ks % 2)
    auto rd1 = [&](int ks, int kk, bf16x8* fr, auto J, auto NV) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value, nv = decltype(NV)::value;
        const uint32_t abase = (uint32_t)((ks % 3) * C::A_BYTES) + chofs[kk];
        const uint32_t bbase = (uint32_t)((ks % 2) * C::B_BYTES) + chofs[kk];
        if constexpr (j == 0) {
            if constexpr (nv > 0) fr[0] = *(const bf16x8*)(smem + (abase + a_lane));
        } else if constexpr (j <= NB) {
            constexpr int bi = j - 1, m = bi / C::TN, tn = bi % C::TN;
            fr[TM + bi] = *(const bf16x8*)(smem + (bbase + b_lane + (m * C::BNM + tn * 32) * 128));
        } else {
            constexpr int tm = j - NB;
            if constexpr (tm < nv) fr[tm] = *(const bf16x8*)(smem + (abase + a_lane + tm * 32 * 128));
        }
    };
    floatx16 acc[C::NACC];
    // MFMA i of a sub-step: activation block tm = i / NB, weight fragment i % NB
    auto mf1 = [&](const bf16x8* fr, auto I, auto NV) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value, nv = decltype(NV)::value;
        constexpr int tm = i / NB, bi = i % NB, m = bi / C::TN, tn = bi % C::TN;
        constexpr int ai = (m * TM + tm) * C::TN + tn;
        if constexpr (tm < nv) acc[ai] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[TM + bi], fr[tm], acc[ai], 0, 0, 0);
    };

    // an item's first loads: stage 0's activations and weights, then stage 1's activations
    auto prologue = [&](const Tile& t) __attribute__((always_inline)) {
        static_for<C::LPW>([&](auto J) { ld1(t, 0, J); });
        if (t.nkl > 1) static_for<8>([&](auto J) { ld1(t, 1, J); });
    };
    Tile cur;
    setup(s, cur);
    prologue(cur);
    bf16x8 fa[NRD], fb[NRD];
    while (true) {
#pragma unroll
        for (int i = 0; i < C::NACC; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
        // stage 0 landed (and the last item's stores); stage 1's activations may be in flight
        if (cur.nkl > 1) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        auto kloop = [&](auto NV) __attribute__((always_inline)) {
            static_for<NRD>([&](auto J) { rd1(0, 0, fa, J, NV); });
            // stage kt in MFMA slots p = 16 kk + i: sub-steps on fa, fb, fa, fb.
            // It loads stage kt+1's weights (the slot of stage kt-1, freed by the
            // last barrier) and then stage kt+2's activations, so that waiting
            // for stage kt+1 leaves those last 8 loads in flight.
            auto stage = [&](int kt, auto HN, auto HA) __attribute__((always_inline)) {
                constexpr bool hn = decltype(HN)::value;  // stage kt+1 exists
                constexpr bool ha = decltype(HA)::value;  // stage kt+2 exists
                static_for<64>([&](auto P) {
                    constexpr int p = decltype(P)::value, kk = p / 16, i = p % 16;
                    if constexpr (p == 56) {
                        // this wave's reads of the stage have returned and its loads of
                        // stage kt+1 have landed
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                        if constexpr (ha) wait_vmcnt<8>();
                        else wait_vmcnt<0>();
                        __builtin_amdgcn_s_barrier();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    mf1(kk % 2 == 0 ? fa : fb, IntC<i>{}, NV);
                    if constexpr (kk < 3) {
                        if constexpr (i < NRD) rd1(kt, kk + 1, kk % 2 == 0 ? fb : fa, IntC<i>{}, NV);
                    } else if constexpr (hn && p >= 56) {
                        rd1(kt + 1, 0, fa, IntC<p - 56>{}, NV);
                    }
                    if constexpr (hn && p < 16 && p % 2 == 0) ld1(cur, kt + 1, IntC<8 + p / 2>{});
                    if constexpr (ha && p >= 16 && p < 32 && p % 2 == 0) ld1(cur, kt + 2, IntC<(p - 16) / 2>{});
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            const int nkl = cur.nkl;
            for (int kt = 0; kt < nkl - 2; ++kt) stage(kt, IntC<1>{}, IntC<1>{});
            if (nkl >= 2) stage(nkl - 2, IntC<1>{}, IntC<0>{});
            stage(nkl - 1, IntC<0>{}, IntC<0>{});
        };
        // a ragged last row tile of a group leaves some waves' row blocks empty
        const int nvb = __builtin_amdgcn_readfirstlane(min(max((cur.row_end - cur.row0 - wm * C::WM + 31) / 32, 0), TM));
        if (nvb == TM) kloop(IntC<TM>{});
        else if (nvb == 0) kloop(IntC<0>{});
        else if (nvb == 1) kloop(IntC<1>{});
        else if (nvb == 2) kloop(IntC<2>{});
        else kloop(IntC<3>{});
        // every slot is free: start the next item's first stages, then store this one
        const int s_next = s + per;
        const bool more = s_next < s_end;
        Tile nxt;
        if (more) {
            setup(s_next, nxt);
            prologue(nxt);
        }
        if (cur.slot >= 0)
            w4_store_partial<MODE>(acc, a.partial, cur.slot, tid);
        else
            w4_epilogue<MODE>(acc, cur.row0, cur.row_end, cur.n0, Nout, (uint8_t*)a.C, wm, wn, lane, a.c_rows, a.c_nrows);
        if (!more) break;
        cur = nxt;
        s = s_next;
    }
    wait_vmcnt<0>();
#endif
}

// The 4-wave kernel on fragment-ordered weights (moe_pack_weights): every
// weight fragment a wave multiplies is 1 KB of consecutive bytes, so the waves
// load their weight fragments straight into registers, three sub-steps (48
// MFMAs) ahead in a ring of four, and LDS holds the activation rows alone
// (four stages, loaded three stages ahead).  The waves are laid 1 x 4 (each
// all 256 rows and a quarter of the weight rows, W4PCfg), so every weight
// fragment is loaded by one wave.  Every output still sums the same products
// in the same k order as on row-major weights, so both kernels give the same
// bits.  Measured on the top-2 layer: gate/up 3.17 -> 3.07 ms and down 1.62 ->
// 1.56 ms with 2 x 2 waves (each weight fragment loaded by two), then 3.10 ->
// 3.02 ms and 1.56 -> 1.52 ms with 1 x 4.
template <int MODE>
__global__ __launch_bounds__(256, 1) void gemm_bf16_w4p_kernel(GArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = W4PCfg<MODE>;
    constexpr int TM = C::TM, NB = C::NB;
    // activation stages in LDS, loaded NAS - 1 stages ahead (top-2 layer, one
    // box: 3 stages 4.78 ms, 4 stages 4.72 ms, 5 stages 4.84 ms)
    constexpr int NAS = 4;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NAS * C::A_BYTES];

    const int K = a.K, Nout = a.Nout;
    const uint32_t rowbytes = (uint32_t)K * 2u;
    const int nk = K / 64;
    const int nk16 = K / 16;
    const int n_m = a.tiles[a.m_tiles].group;
    const int total = n_m * a.n_tiles;
    const int xcd = blockIdx.x & 7, per = gridDim.x >> 3;
    const int q = (total + 7) / 8;
    const int tx0 = xcd * q;
    const int Tx = max(0, min(q, total - tx0));
    int r_tail, S;
    tail_split(Tx, per, nk, a.partial != nullptr, r_tail, S);
    const int n_whole = S > 1 ? Tx - r_tail : Tx;
    const int s_end = n_whole + (S > 1 ? r_tail * S : 0);
    int s = blockIdx.x >> 3;
    if (s >= s_end) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = 0, wn = wave;  // 1 x 4 waves
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int a_dst = wu * 64 * 128;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, (short)0, (int)a.a_bytes, kBufWord3);
    const int a_nrows = (int)(a.a_bytes / rowbytes);

    struct Tile {
        int row0, row_end, n0;
        int kb, nkl, slot;
        __amdgpu_buffer_rsrc_t rB0, rB1;
        uint32_t va[8], vb[NB];
    };
    auto setup = [&](int item, Tile& t) __attribute__((always_inline)) {
        int si = tx0 + item;
        t.kb = 0;
        t.nkl = nk;
        t.slot = -1;
        if (item >= n_whole) {
            const int j = item - n_whole, jt = j / S, p = j - jt * S;
            si = tx0 + n_whole + jt;
            t.kb = p * nk / S;
            t.nkl = (p + 1) * nk / S - t.kb;
            t.slot = xcd * kTailSlots + j;
        }
        int mt, nt;
        const GemmTile tl = sched_decode(si, n_m, a.n_tiles, a.tiles, 256, mt, nt, sched_width(a));
        t.row0 = tl.row0;
        t.row_end = tl.row_end;
        t.n0 = nt * C::BNM;
        const size_t bgo = a.b_shared ? 0 : (size_t)tl.group * Nout * rowbytes;
        const uint8_t* B0 = (const uint8_t*)a.B0 + bgo;
        const uint8_t* B1 = gated_mode(MODE) ? (const uint8_t*)a.B1 + bgo : B0;
        t.rB0 = __builtin_amdgcn_make_buffer_rsrc((void*)B0, (short)0, (int)((size_t)Nout * rowbytes), kBufWord3);
        t.rB1 = __builtin_amdgcn_make_buffer_rsrc((void*)B1, (short)0, (int)((size_t)Nout * rowbytes), kBufWord3);
        const int lr = lane >> 3, pc = lane & 7;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wu * 64 + 8 * i + lr;
            const int c = pc ^ ((r >> 1) & 7);
            const int gr = a_row(a, min(t.row0 + r, t.row_end - 1), a_nrows);
            t.va[i] = (uint32_t)gr * rowbytes + (uint32_t)(c * 16) - 1024u * (i % 4);
        }
        // the wave's weight fragment bi (matrix bi / TN, 32-column block bi % TN):
        // lane l reads 16 bytes at piece l of each 16-k step of its 32-row block
        // (blocks past Nout, whose columns are never stored, reread the last one)
        const int nb_last = (Nout + 31) / 32 - 1;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int tn = bi % C::TN;
            const int nb32 = min((t.n0 + wn * C::WNM + tn * 32) / 32, nb_last);
            t.vb[bi] = (uint32_t)nb32 * (uint32_t)nk16 * 1024u + (uint32_t)lane * 16u;
        }
    };
    // activation load i of stage ks (8 rows of the wave's 64, into LDS slot ks % 3)
    auto lda1 = [&](const Tile& t, int ks, auto J) __attribute__((always_inline)) {
        constexpr int i = decltype(J)::value;
        uint8_t* dst = smem + (ks % NAS) * C::A_BYTES + a_dst + 4096 * (i / 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_ptr)dst, 16, t.va[i], (t.kb + ks) * 128, 1024 * (i % 4), 0);
    };
    // weight fragments of k16 step g (= 4 * stage + sub-step) into ring slot d[0..NB)
    auto ldb1 = [&](const Tile& t, int g, u32x4* d, auto B) __attribute__((always_inline)) {
        constexpr int bi = decltype(B)::value, m = bi / C::TN;
        d[bi] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(m ? t.rB1 : t.rB0, (int)t.vb[bi],
                                                                                 (t.kb * 4 + g) * 1024, 0));
    };
    const int xsw = ((lane & 31) >> 1) & 7;
    const uint32_t a_lane = (uint32_t)((wm * C::WM + (lane & 31)) * 128);
    uint32_t chofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) chofs[kk] = (uint32_t)(((kk * 2 + (lane >> 5)) ^ xsw) << 4);
    // activation block tm of sub-step kk of stage ks, from LDS
    auto rda = [&](int ks, int kk, bf16x8* fr, auto J, auto NV) __attribute__((always_inline)) {
        constexpr int tm = decltype(J)::value, nv = decltype(NV)::value;
        const uint32_t abase = (uint32_t)((ks % NAS) * C::A_BYTES) + chofs[kk];
        if constexpr (tm < nv) fr[tm] = *(const bf16x8*)(smem + (abase + a_lane + tm * 32 * 128));
    };
    floatx16 acc[C::NACC];
    u32x4 bR[4][NB];  // weight fragments of the next sub-steps, slot = sub-step % 4
    auto mf1 = [&](const bf16x8* fr, const u32x4* bcur, auto I, auto NV) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value, nv = decltype(NV)::value;
        constexpr int tm = i / NB, bi = i % NB, m = bi / C::TN, tn = bi % C::TN;
        constexpr int ai = (m * TM + tm) * C::TN + tn;
        if constexpr (tm < nv)
            acc[ai] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bcur[bi]), fr[tm], acc[ai], 0, 0, 0);
    };
    // an item's first loads: stage 0's activations, the weights of its first
    // three sub-steps, the activations of stages 1 .. NAS - 2
    auto prologue = [&](const Tile& t) __attribute__((always_inline)) {
        static_for<8>([&](auto J) { lda1(t, 0, J); });
        static_for<3>([&](auto G) { static_for<NB>([&](auto B) { ldb1(t, decltype(G)::value, bR[decltype(G)::value], B); }); });
        static_for<NAS - 2>([&](auto S) {
            constexpr int st = decltype(S)::value + 1;
            if (st < t.nkl) static_for<8>([&](auto J) { lda1(t, st, J); });
        });
    };
    Tile cur;
    setup(s, cur);
    prologue(cur);
    bf16x8 fa[TM], fb[TM];
    while (true) {
#pragma unroll
        for (int i = 0; i < C::NACC; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
        // stage 0's activations landed (the weights of its first three sub-steps
        // and the later stages' activations may still be in flight; the compiler
        // waits for each weight register before its first MFMA)
        static_assert(NAS == 4, "the waits below count 3 NB weight and 8 activation loads per stage");
        {
            const int ahead = min(NAS - 2, cur.nkl - 1);  // activation stages loaded after stage 0's weights
            if (ahead >= 2) wait_vmcnt<3 * NB + 16>();
            else if (ahead == 1) wait_vmcnt<3 * NB + 8>();
            else wait_vmcnt<3 * NB>();
        }
        __builtin_amdgcn_s_barrier();
        auto kloop = [&](auto NV) __attribute__((always_inline)) {
            static_for<TM>([&](auto J) { rda(0, 0, fa, J, NV); });
            auto stage = [&](int kt, auto HN, auto HA) __attribute__((always_inline)) {
                constexpr bool hn = decltype(HN)::value;
                constexpr bool ha = decltype(HA)::value;
                static_for<64>([&](auto P) {
                    constexpr int p = decltype(P)::value, kk = p / 16, i = p % 16;
                    if constexpr (p == 56) {
                        // own LDS reads done; stage kt+1's activations landed (they were
                        // issued before this stage's last weight loads, which this
                        // stage has already waited for); ha: stage kt + NAS - 1 exists
                        __builtin_amdgcn_s_waitcnt(0xC07F);
                        wait_vmcnt<(ha ? 8 : 0) + (hn ? 2 * NB : 0)>();
                        __builtin_amdgcn_s_barrier();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    mf1(kk % 2 == 0 ? fa : fb, bR[kk], IntC<i>{}, NV);
                    if constexpr (kk < 3) {
                        if constexpr (i < TM) rda(kt, kk + 1, kk % 2 == 0 ? fb : fa, IntC<i>{}, NV);
                    } else if constexpr (hn && p >= 56 && p < 56 + TM) {
                        rda(kt + 1, 0, fa, IntC<p - 56>{}, NV);
                    }
                    if constexpr (ha && p >= 16 && p < 32 && p % 2 == 0) lda1(cur, kt + NAS - 1, IntC<(p - 16) / 2>{});
                    // sub-step kk loads the weights of sub-step kk + 3
                    if constexpr (i >= 8 && i % 2 == 0 && (i - 8) / 2 < NB && (kk == 0 || hn))
                        ldb1(cur, 4 * kt + kk + 3, bR[(kk + 3) % 4], IntC<(i - 8) / 2>{});
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            const int nkl = cur.nkl;
            int kt = 0;
            for (; kt < nkl - (NAS - 1); ++kt) stage(kt, IntC<1>{}, IntC<1>{});
            for (; kt < nkl - 1; ++kt) stage(kt, IntC<1>{}, IntC<0>{});
            stage(nkl - 1, IntC<0>{}, IntC<0>{});
        };
        const int nvb = __builtin_amdgcn_readfirstlane(min(max((cur.row_end - cur.row0 - wm * C::WM + 31) / 32, 0), TM));
        static_assert(TM == 8, "row-block counts 0..8");
        if (nvb == TM) kloop(IntC<TM>{});
        else if (nvb == 0) kloop(IntC<0>{});
        else if (nvb == 1) kloop(IntC<1>{});
        else if (nvb == 2) kloop(IntC<2>{});
        else if (nvb == 3) kloop(IntC<3>{});
        else if (nvb == 4) kloop(IntC<4>{});
        else if (nvb == 5) kloop(IntC<5>{});
        else if (nvb == 6) kloop(IntC<6>{});
        else kloop(IntC<7>{});
        const int s_next = s + per;
        const bool more = s_next < s_end;
        Tile nxt;
        if (more) {
            setup(s_next, nxt);
            prologue(nxt);
        }
        if (cur.slot >= 0)
            w4_store_partial<MODE>(acc, a.partial, cur.slot, tid);  // the same slot layout (NACC = 16)
        else
            w4_epilogue_cfg<C, MODE>(acc, cur.row0, cur.row_end, cur.n0, Nout, (uint8_t*)a.C, wm, wn, lane, a.c_rows,
                                     a.c_nrows);
        if (!more) break;
        cur = nxt;
        s = s_next;
    }
    wait_vmcnt<0>();
#endif
}

// The split tail tiles of the 4-wave kernels (ungated products: the gated one
// is never split): each (XCD, tail tile) block sums the tile's pieces in piece
// order and runs the epilogue.  1024 threads: thread t takes the accumulators
// of the 4-wave kernel's thread t % 256 in its activation row blocks
// RB (t / 256) .. RB (t / 256) + RB - 1, RB = TM / 4 (C: that kernel's waves).
template <int MODE, typename C = W4Cfg<MODE>>
__global__ __launch_bounds__(1024) void gemm_w4_tail_kernel(GArgs a, int per) {
    static_assert(!gated_mode(MODE), "the gated product keeps whole tiles");
    constexpr int RB = C::TM / 4;
    static_assert(RB * 4 == C::TM, "the row blocks split evenly over four thread groups");
    const int xcd = blockIdx.x / kTailSlots, jt = blockIdx.x % kTailSlots;
    const int nk = a.K / 64;
    const int n_m = a.tiles[a.m_tiles].group;
    const int total = n_m * a.n_tiles;
    const int q = (total + 7) / 8;
    const int tx0 = xcd * q;
    const int Tx = max(0, min(q, total - tx0));
    int r_tail, S;
    tail_split(Tx, per, nk, a.partial != nullptr, r_tail, S);
    if (S < 2 || jt >= r_tail) return;
    int mt, nt;
    const GemmTile tl = sched_decode(tx0 + Tx - r_tail + jt, n_m, a.n_tiles, a.tiles, 256, mt, nt, sched_width(a));
    const int tid = threadIdx.x & 255, grp = threadIdx.x >> 8, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const bool hi = lane >= 32;
    const floatx4* P0 = (const floatx4*)a.partial + (size_t)(xcd * kTailSlots + jt * S) * (C::NACC * 4 * 256);
    auto sum_tile = [&](int ai) {
        floatx16 v;
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = 0.0f;
#pragma unroll 2
        for (int p = 0; p < S; ++p) {
            const floatx4* P = P0 + (size_t)p * (C::NACC * 4 * 256);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4 x = P[(ai * 4 + q4) * 256 + tid];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[4 * q4 + i] += x[i];
            }
        }
        return v;
    };
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int tm = grp * RB + r;
        const int row = tl.row0 + wm * C::WM + tm * 32 + (lane & 31);
        const int crow = row < tl.row_end ? c_row(a.c_rows, a.c_nrows, row) : row;
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
            const floatx16 g = sum_tile(tm * C::TN + tn);
            w4_store_tile<MODE>(g, g, row, tl.row_end, crow, nt * C::BNM + wn * C::WNM + tn * 32, a.Nout, (uint8_t*)a.C,
                                hi);
        }
    }
}

// ------------------------------------------------------------- fp32 VALU
// 64 x 64 output tile per matrix, BK = 16, 256 threads each computing 4x4.
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GArgs a) {
    constexpr int NMAT = MODE == MODE_SWIGLU ? 2 : 1;
    __shared__ float As[FBK][FBM + 4];
    __shared__ float Bs[NMAT][FBK][FBN + 4];
    const int mt = blockIdx.x, nt = blockIdx.y;
    if (mt >= a.m_tiles) return;
    const GemmTile tl = a.tiles[mt];
    if (tl.group < 0) return;
    const int K = a.K, Nout = a.Nout;
    const int n0 = nt * FBN;
    const float* A = (const float*)a.A;
    const float* Bm[2] = {(const float*)a.B0 + (size_t)tl.group * Nout * K,
                          MODE == MODE_SWIGLU ? (const float*)a.B1 + (size_t)tl.group * Nout * K : nullptr};
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    float acc[NMAT][4][4] = {};
    for (int k0 = 0; k0 < K; k0 += FBK) {
        for (int i = tid; i < FBM * FBK; i += 256) {
            const int r = i / FBK, k = i % FBK;
            const int gr = a_row(a, min(tl.row0 + r, tl.row_end - 1), (int)(a.a_bytes / ((long long)K * 4)));
            As[k][r] = k0 + k < K ? A[(size_t)gr * K + k0 + k] : 0.0f;
        }
        for (int m = 0; m < NMAT; ++m)
            for (int i = tid; i < FBN * FBK; i += 256) {
                const int c = i / FBK, k = i % FBK;
                const int gc = min(n0 + c, Nout - 1);
                Bs[m][k][c] = k0 + k < K ? Bm[m][(size_t)gc * K + k0 + k] : 0.0f;
            }
        __syncthreads();
        for (int k = 0; k < FBK; ++k)
            for (int m = 0; m < NMAT; ++m)
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j)
                        acc[m][i][j] = fmaf(As[k][ty * 4 + i], Bs[m][k][tx * 4 + j], acc[m][i][j]);
        __syncthreads();
    }
    float* Cp = (float*)a.C;
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
            const int row = tl.row0 + ty * 4 + i, col = n0 + tx * 4 + j;
            if (row >= tl.row_end || col >= Nout) continue;
            float v;
            if constexpr (MODE == MODE_SWIGLU) {
                v = acc[0][i][j] / (1.0f + expf(-acc[0][i][j])) * acc[1][i][j];
            } else if constexpr (MODE == MODE_GELU) {
                v = act_gelu(acc[0][i][j]);
            } else {
                v = acc[0][i][j];
            }
            Cp[(size_t)c_row(a.c_rows, a.c_nrows, row) * Nout + col] = v;
        }
}

// ------------------------------------------------------------- launchers
// 256-row tiles when groups average 512 rows or more; otherwise 128-row tiles,
// which waste less of a ragged group and keep a deeper load ring
static int pick_bm(int dtype, int G, int max_rows) {
    if (dtype != MOE_BF16) return FBM;
    return (G > 0 && max_rows / G >= 512) ? 256 : 128;
}
static int max_m_tiles(int BM, int G, int max_rows) { return (max_rows + BM - 1) / BM + G; }

// FFN workspace: the tile table, its header and the claim counters, then (bf16)
// the fp32 partial tiles of split tail tiles: 8 XCDs x kTailSlots slots of one
// BM x 256 fp32 tile (256 KB for BM = 256)
static size_t table_bytes(int BM, int G, int max_rows) {
    const size_t b = (size_t)(max_m_tiles(BM, G, max_rows) + 1 + kClaimSets) * sizeof(GemmTile);
    return (b + 255) & ~(size_t)255;
}
static size_t partial_bytes(int BM, int dtype) {
    return dtype == MOE_BF16 ? (size_t)8 * kTailSlots * BM * 256 * sizeof(float) : 0;
}
static float* partial_of(GemmTile* tiles, int BM, int G, int max_rows, int dtype) {
    return dtype == MOE_BF16 ? (float*)((char*)tiles + table_bytes(BM, G, max_rows)) : nullptr;
}
size_t ffn_workspace_bytes(int G, int max_rows, int dtype) {
    const int BM = pick_bm(dtype, G, max_rows);
    return table_bytes(BM, G, max_rows) + partial_bytes(BM, dtype);
}

// one block per compute unit of the current device (a multiple of the 8 XCDs)
static int persistent_blocks() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached[dev] = cus < 8 ? 8 : cus - cus % 8;
    }
    return cached[dev];
}

// the 4-wave kernel (and its split-tail sums): 256-row tiles, K a multiple of
// 64.  The gated product keeps whole tiles: the training forward runs it on the
// ring kernel with a saving epilogue, and both then sum every output in the
// same k order, so the two forwards agree bit for bit.
template <int MODE>
static hipError_t run_w4(GArgs g, hipStream_t st) {
    using R = W4Cfg<MODE>;
    g.n_tiles = (g.Nout + R::BNM - 1) / R::BNM;
    if constexpr (gated_mode(MODE)) g.partial = nullptr;
    const int pb = persistent_blocks();
    if (g.b_packed)
        hipLaunchKernelGGL((gemm_bf16_w4p_kernel<MODE>), dim3(pb), dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL((gemm_bf16_w4_kernel<MODE>), dim3(pb), dim3(256), 0, st, g);
    hipError_t err = hipGetLastError();
    if constexpr (!gated_mode(MODE)) {
        if (err == hipSuccess && g.partial) {
            if (g.b_packed)
                hipLaunchKernelGGL((gemm_w4_tail_kernel<MODE, W4PCfg<MODE>>), dim3(8 * kTailSlots), dim3(1024), 0, st,
                                   g, pb / 8);
            else
                hipLaunchKernelGGL((gemm_w4_tail_kernel<MODE>), dim3(8 * kTailSlots), dim3(1024), 0, st, g, pb / 8);
            err = hipGetLastError();
        }
    }
    return err;
}
// shortest K for the 4-wave kernel: with one wave per SIMD nothing covers a
// tile's first stage and epilogue, which short-K tiles repeat often (the
// multi-head layer's K = 512 gate/up GEMM: 0.75 -> 0.80 ms on it)
constexpr int kW4MinK = 2048;
// the fragment-order kernel (weights in registers, four activation stages)
// from K = 1024 for the ungated products: the multi-head layer's down GEMM
// 0.34 -> 0.325 ms (at K = 512 its gate/up GEMM went 0.66 -> 0.71 ms).  Gated
// products keep the 64-wide kernel below 2048, whose split tail tiles the
// 4-wave kernel would not split (both layouts then sum in one order).
constexpr int kW4PMinK = 1024;

template <int BM, int MODE>
static hipError_t run_bf16(GArgs g, hipStream_t st) {
    using C = TileCfg<BM, MODE>;
    g.n_tiles = (g.Nout + C::BNM - 1) / C::BNM;
    g.total = g.m_tiles * g.n_tiles;
    g.per_xcd = (g.total + 7) / 8;
    const int blocks = g.per_xcd * 8;
    if (blocks == 0) return hipSuccess;
    const long long b_bytes = (long long)g.Nout * g.K * 2;
    const bool offsets_fit = g.a_bytes < (1ll << 31) && b_bytes < (1ll << 31);
    // 256-row tiles with a long K (a multiple of 64): the 4-wave kernel
    if constexpr (BM == 256) {
        if (offsets_fit && g.K % 64 == 0 && g.K >= (g.b_packed && !gated_mode(MODE) ? kW4PMinK : kW4MinK) && g.Nout % 8 == 0 &&
            ((uintptr_t)g.C & 15) == 0 && !g.kspan)
            return run_w4<MODE>(g, st);
    }
    // otherwise the 64-wide-stage kernel whenever K allows it (K a multiple of
    // 64, output rows 16-byte aligned), except for a gated product on 256-row
    // tiles with K >= 4096 that the 4-wave kernel does not take, where the ring
    // kernel measured ahead of it; for the plain long-K products it measured
    // behind (top-2 down 1.72 -> 1.90 ms, W_o 0.23 -> 0.25 ms)
    // Fragment-ordered weights are read by the 4-wave kernel above and by the
    // 64-wide kernel only; the entry points check the conditions beforehand.
    const bool ring_first = MODE != MODE_PLAIN && BM == 256 && g.K >= 4096 && !g.b_packed;
    if (g.b_packed && !(offsets_fit && g.K % 64 == 0 && g.Nout % 32 == 0 && ((uintptr_t)g.C & 15) == 0))
        return hipErrorInvalidValue;
    if (!ring_first && offsets_fit && g.K % 64 == 0 && g.Nout % 8 == 0 && ((uintptr_t)g.C & 15) == 0) {
        using R = K64Cfg<BM, MODE>;
        g.n_tiles = (g.Nout + R::BNM - 1) / R::BNM;
        if (BM == 128) g.ngroup = g.n_tiles;  // one schedule group per row tile sweep
        const int pb = persistent_blocks();
        if (g.b_packed)
            hipLaunchKernelGGL((gemm_bf16_k64_kernel<BM, MODE, 0, true>), dim3(pb), dim3(512), 0, st, g);
        else
            hipLaunchKernelGGL((gemm_bf16_k64_kernel<BM, MODE, 0>), dim3(pb), dim3(512), 0, st, g);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || !g.partial) return err;
        hipLaunchKernelGGL((gemm_k64_tail_kernel<BM, MODE>), dim3(8 * kTailSlots), dim3(512), 0, st, g, pb / 8);
        return hipGetLastError();
    }
    if (g.K % 32 == 0 && offsets_fit && g.Nout % 8 == 0 && ((uintptr_t)g.C & 15) == 0) {
        using R = Ring8Cfg<BM, MODE>;
        g.n_tiles = (g.Nout + R::BNM - 1) / R::BNM;
        if (BM == 128) g.ngroup = g.n_tiles;
        hipLaunchKernelGGL((gemm_bf16_ring8_kernel<BM, MODE>), dim3(persistent_blocks()), dim3(512), 0, st, g);
    } else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, MODE>), dim3(blocks), dim3(256), 0, st, g);
    return hipGetLastError();
}

template <int MODE>
static hipError_t run_f32(GArgs g, hipStream_t st) {
    g.n_tiles = (g.Nout + FBN - 1) / FBN;
    if (g.m_tiles == 0 || g.n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_f32_kernel<MODE>), dim3(g.m_tiles, g.n_tiles), dim3(256), 0, st, g);
    return hipGetLastError();
}

static hipError_t run_gemm(int dtype, int BM, int mode, const GArgs& g, hipStream_t st) {
    if (dtype == MOE_BF16) {
        if (BM == 256) {
            if (mode == MODE_SWIGLU) return run_bf16<256, MODE_SWIGLU>(g, st);
            if (mode == MODE_GELU) return run_bf16<256, MODE_GELU>(g, st);
            return run_bf16<256, MODE_PLAIN>(g, st);
        }
        if (mode == MODE_SWIGLU) return run_bf16<128, MODE_SWIGLU>(g, st);
        if (mode == MODE_GELU) return run_bf16<128, MODE_GELU>(g, st);
        return run_bf16<128, MODE_PLAIN>(g, st);
    }
    if (mode == MODE_SWIGLU) return run_f32<MODE_SWIGLU>(g, st);
    if (mode == MODE_GELU) return run_f32<MODE_GELU>(g, st);
    return run_f32<MODE_PLAIN>(g, st);
}

// the 64-wide kernel alone, without split tail tiles (the training and
// backward modes, per-group k ranges)
template <int BM, int MODE, int KM = 0>
static hipError_t run_k64_only(GArgs g, hipStream_t st) {
    constexpr bool BT = KM >= 1;
    using R = K64Cfg<BM, MODE>;
    g.n_tiles = (g.Nout + R::BNM - 1) / R::BNM;
    g.total = g.m_tiles * g.n_tiles;
    g.per_xcd = (g.total + 7) / 8;
    g.partial = nullptr;
    if (g.total == 0) return hipSuccess;
    const long long b_bytes = (long long)g.Nout * (BT && g.kb1 > 0 ? g.kb1 : g.K) * 2;
    if (g.a_bytes >= (1ll << 31) || b_bytes >= (1ll << 31) || g.K % 64 != 0 || g.Nout % 8 != 0 ||
        ((uintptr_t)g.C & 15) != 0)
        return hipErrorInvalidValue;
    if (KM == 1 && g.kb1 != 0 && (g.kb1 < 0 || g.kb1 % 64 != 0 || g.kb1 >= g.K || !g.B1)) return hipErrorInvalidValue;
    if (KM == 2 && (!g.krows || g.a_mod < 8 || g.a_mod % 8 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0 || g.lda < g.a_mod ||
                    g.ldb < g.Nout || g.b_bytes >= (1ll << 31) || g.b_bytes < 0))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_k64_kernel<BM, MODE, KM>), dim3(persistent_blocks()), dim3(512), 0, st, g);
    return hipGetLastError();
}

// the ring kernel with a training epilogue (the shapes where it leads: gated,
// 256-row tiles, K >= 4096, K % 32 == 0)
template <int MODE>
static hipError_t run_ring8_save(GArgs g, hipStream_t st) {
    using R = Ring8Cfg<256, MODE>;
    g.n_tiles = (g.Nout + R::BNM - 1) / R::BNM;
    g.total = g.m_tiles * g.n_tiles;
    g.per_xcd = (g.total + 7) / 8;
    g.partial = nullptr;
    if (g.total == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_bf16_ring8_kernel<256, MODE>), dim3(persistent_blocks()), dim3(512), 0, st, g);
    return hipGetLastError();
}

static hipError_t run_k64_mode(int BM, int mode, const GArgs& g, hipStream_t st, int kmajor = 0) {
    if (kmajor == 2) {
        if (mode != MODE_PLAIN || BM != 256) return hipErrorInvalidValue;
        return run_k64_only<256, MODE_PLAIN, 2>(g, st);
    }
    if (kmajor == 1) {
        switch (mode) {
            case MODE_PLAIN:
                return BM == 256 ? run_k64_only<256, MODE_PLAIN, 1>(g, st) : run_k64_only<128, MODE_PLAIN, 1>(g, st);
            case MODE_DSWIGLU:
                return BM == 256 ? run_k64_only<256, MODE_DSWIGLU, 1>(g, st) : run_k64_only<128, MODE_DSWIGLU, 1>(g, st);
            case MODE_DGELU:
                return BM == 256 ? run_k64_only<256, MODE_DGELU, 1>(g, st) : run_k64_only<128, MODE_DGELU, 1>(g, st);
        }
        return hipErrorInvalidValue;
    }
    if (mode == MODE_SWIGLU_SAVE && BM == 256 && g.K >= 4096 && g.K % 32 == 0 && g.Nout % 8 == 0 &&
        ((uintptr_t)g.C & 15) == 0 && g.a_bytes < (1ll << 31) && (long long)g.Nout * g.K * 2 < (1ll << 31) &&
        !g.kspan && !g.a_mod && !g.b_shared)
        return run_ring8_save<MODE_SWIGLU_SAVE>(g, st);
#define MOE_K64_CASE(M)                                                         \
    case M:                                                                     \
        return BM == 256 ? run_k64_only<256, M>(g, st) : run_k64_only<128, M>(g, st);
    switch (mode) {
        MOE_K64_CASE(MODE_SWIGLU)
        MOE_K64_CASE(MODE_GELU)
        MOE_K64_CASE(MODE_PLAIN)
        MOE_K64_CASE(MODE_SWIGLU_SAVE)
        MOE_K64_CASE(MODE_GELU_SAVE)
        MOE_K64_CASE(MODE_DSWIGLU)
        MOE_K64_CASE(MODE_DGELU)
        MOE_K64_CASE(MODE_F32OUT)
    }
#undef MOE_K64_CASE
    return hipErrorInvalidValue;
}

static hipError_t build_tiles(const int32_t* offsets, int G, int BM, int max_rows, int max_tiles,
                              GemmTile* tiles, hipStream_t st) {
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, st, offsets, G, BM, max_rows, max_tiles, tiles);
    return hipGetLastError();
}

hipError_t launch_ffn(const FfnArgs& f, hipStream_t st) {
    if (f.max_rows <= 0 || f.G <= 0) return hipSuccess;
    const int BM = pick_bm(f.dtype, f.G, f.max_rows);
    const int mtiles = max_m_tiles(BM, f.G, f.max_rows);
    hipError_t err = build_tiles(f.offsets, f.G, BM, f.max_rows, mtiles, f.tiles, st);
    if (err != hipSuccess) return err;
    const uint32_t fl = f.flags ? f.flags : (MOE_FFN_GEMM1 | MOE_FFN_GEMM2);
    if (fl & MOE_FFN_GEMM1) {
        GArgs g{};
        g.A = f.x_perm;
        g.B0 = f.w_gate;
        g.B1 = f.act == MOE_SWIGLU ? f.w_up : nullptr;
        g.C = f.h_tmp;
        g.tiles = f.tiles;
        g.claim = (int32_t*)(f.tiles + mtiles + 1);
        g.partial = partial_of(f.tiles, BM, f.G, f.max_rows, f.dtype);
        g.m_tiles = mtiles;
        g.K = f.d;
        g.Nout = f.f;
        const int esz = f.dtype == MOE_BF16 ? 2 : 4;
        g.a_bytes = f.src_rows ? (long long)f.a_nrows * f.d * esz : (long long)f.max_rows * f.d * esz;
        g.a_rows = f.src_rows;
        g.b_packed = f.packed;
        if (f.act_save) {  // training: also keep the pre-activations for the backward pass
            g.aux = f.act_save;
            err = run_k64_mode(BM, f.act == MOE_SWIGLU ? MODE_SWIGLU_SAVE : MODE_GELU_SAVE, g, st);
        } else {
            err = run_gemm(f.dtype, BM, f.act == MOE_SWIGLU ? MODE_SWIGLU : MODE_GELU, g, st);
        }
        if (err != hipSuccess) return err;
    }
    if (fl & MOE_FFN_GEMM2) {
        GArgs g{};
        g.A = f.h_tmp;
        g.B0 = f.w_down;
        g.B1 = nullptr;
        g.C = f.y_perm;
        g.tiles = f.tiles;
        g.claim = (int32_t*)(f.tiles + mtiles + 1) + 8;
        g.partial = partial_of(f.tiles, BM, f.G, f.max_rows, f.dtype);
        g.m_tiles = mtiles;
        g.K = f.f;
        g.Nout = f.d;
        g.a_bytes = (long long)f.max_rows * f.f * (f.dtype == MOE_BF16 ? 2 : 4);
        g.c_rows = f.c_rows;
        g.c_nrows = f.c_nrows;
        g.b_packed = f.packed;
        err = run_gemm(f.dtype, BM, MODE_PLAIN, g, st);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

__global__ void set2_kernel(int32_t* p, int32_t a, int32_t b) {
    p[0] = a;
    p[1] = b;
}

hipError_t launch_dense(int rows, int k, int n, int dtype, const void* x, const void* w, void* y,
                        GemmTile* tiles, int32_t* offsets2, hipStream_t st, int packed) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(set2_kernel, dim3(1), dim3(1), 0, st, offsets2, 0, rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int BM = pick_bm(dtype, 1, rows);
    const int mtiles = max_m_tiles(BM, 1, rows);
    if ((err = build_tiles(offsets2, 1, BM, rows, mtiles, tiles, st)) != hipSuccess) return err;
    GArgs g{};
    g.A = x;
    g.B0 = w;
    g.C = y;
    g.tiles = tiles;
    g.claim = (int32_t*)(tiles + mtiles + 1);
    g.partial = partial_of(tiles, BM, 1, rows, dtype);
    g.m_tiles = mtiles;
    g.K = k;
    g.Nout = n;
    g.a_bytes = (long long)rows * k * (dtype == MOE_BF16 ? 2 : 4);
    g.b_packed = packed;
    return run_gemm(dtype, BM, MODE_PLAIN, g, st);
}

size_t grouped_gemm_ws_bytes(int G, int max_rows) {
    return std::max(table_bytes(128, G, max_rows), table_bytes(256, G, max_rows));
}

hipError_t launch_grouped_gemm(int mode, const GemmSpec& s, const int32_t* offsets, int G, int max_rows,
                               GemmTile* tiles, hipStream_t st, int bm) {
    if (max_rows <= 0 || G <= 0) return hipSuccess;
    const int BM = s.kmajor == 2 ? 256 : bm == 128 || bm == 256 ? bm : pick_bm(MOE_BF16, G, max_rows);
    const int mtiles = max_m_tiles(BM, G, max_rows);
    hipError_t err = build_tiles(offsets, G, BM, max_rows, mtiles, tiles, st);
    if (err != hipSuccess) return err;
    GArgs g{};
    g.A = s.A;
    g.B0 = s.B0;
    g.B1 = s.B1;
    g.C = s.C;
    g.aux = s.aux;
    g.tiles = tiles;
    g.claim = (int32_t*)(tiles + mtiles + 1);
    g.m_tiles = mtiles;
    g.K = s.K;
    g.Nout = s.Nout;
    g.a_bytes = s.a_bytes;
    g.a_rows = s.a_rows;
    g.kspan = s.kspan;
    g.a_mod = s.a_mod;
    g.b_shared = s.b_shared;
    g.kb1 = s.kb1;
    g.krows = s.krows;
    g.lda = s.lda;
    g.ldb = s.ldb;
    g.b_bytes = s.b_bytes;
    return run_k64_mode(BM, mode, g, st, s.kmajor);
}

// ------------------------------------------------------------- weight packing
// Fragment order of a bf16 matrix W [n_out][k] (n_out % 32 == 0, k % 16 == 0):
// 16-byte piece ((nb * k/16 + s) * 64 + l) holds W[32 nb + l % 32][16 s + 8 (l / 32)
// + 0..7], the 8 values lane l gives a 32x32x16 MFMA as the 32-row operand of
// 16-k step s of row block nb.  The matrices of a stack keep their order and
// size, so piece p of the stack is found from the global row block alone.
__global__ __launch_bounds__(256) void pack_weights_kernel(const u32x4* __restrict__ w, u32x4* __restrict__ out,
                                                           long long n_pieces, int k) {
    const int k16 = k >> 4;
    for (long long p = (long long)blockIdx.x * 256 + threadIdx.x; p < n_pieces; p += (long long)gridDim.x * 256) {
        const int l = (int)(p & 63);
        const long long q = p >> 6;  // row block * k16 + s
        const int s = (int)(q % k16);
        const long long row = (q / k16) * 32 + (l & 31);
        out[p] = w[row * (k >> 3) + 2 * s + (l >> 5)];
    }
}

hipError_t launch_pack_weights(const void* w, void* out, long long n_mat, int n_out, int k, hipStream_t st) {
    const long long n_pieces = n_mat * n_out * (long long)k / 8;
    if (n_pieces <= 0) return hipSuccess;
    const long long blocks = std::min<long long>((n_pieces + 255) / 256, 16384);
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)w, (u32x4*)out,
                       n_pieces, k);
    return hipGetLastError();
}

hipError_t launch_set2(int32_t* p, int32_t a, int32_t b, hipStream_t st) {
    hipLaunchKernelGGL(set2_kernel, dim3(1), dim3(1), 0, st, p, a, b);
    return hipGetLastError();
}

}  // namespace moe
