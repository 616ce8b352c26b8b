// combine.hip -- gate-weighted unpermute/combine and the aux-loss statistics.
//
// Lesson 10 "专家并行 EP" (learn.payai.win), "核心概念" item 1: the output is the
// gate-weighted sum of the kept experts' outputs; item 3: expert outputs return
// to their token and are summed with the saved gate weights; item 4: the aux
// loss L_aux = alpha E sum_i f_i P_i from routing frequency f_i and mean score
// P_i.  "Multi-Head LatentMoE 与 Head 并行" ("核心方法与创新", determinism): the
// sums here are gathers in a fixed slot order with no atomics, so the output is
// bitwise reproducible.
#include "common.hpp"

namespace moe {

// One sub-token row per `tpr` threads; each thread owns 8 consecutive features
// (bf16: one 16-byte load per kept slot).  fp32 accumulation in slot order,
// then + y_shared, then one rounding.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int tpr) {
    const int rpb = 256 / tpr;
    const long s = (long)blockIdx.x * rpb + threadIdx.x / tpr;
    const int c = threadIdx.x % tpr;
    const long S = (long)a.T * a.H;
    if (s >= S) return;
    const int K = a.K, d = a.d;
    const long t = s / a.H;
    const int g = (int)(s - t * a.H);
    const int32_t* dr = a.dest_row + s * K;
    const float* wr = a.topk_w + s * K;
    for (int j0 = c * 8; j0 < d; j0 += tpr * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
            // up to KB slots' rows are loaded before the first is added, so their
            // latencies overlap; the sums still run in slot order
            constexpr int KB = 8;
            for (int k0 = 0; k0 < K; k0 += KB) {
                uint4 v[KB];
                float w[KB];
                bool kept[KB];
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    const int k = k0 + u;
                    const int row = k < K ? dr[k] : -1;
                    kept[u] = row >= 0;
                    w[u] = kept[u] ? wr[k] : 0.0f;
                    v[u] = kept[u] ? *(const uint4*)((const uint16_t*)a.y_perm + (size_t)row * d + j0)
                                   : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    if (!kept[u]) continue;
                    const uint32_t uu[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = fmaf(w[u], __uint_as_float(uu[q] << 16), acc[2 * q]);
                        acc[2 * q + 1] = fmaf(w[u], __uint_as_float(uu[q] & 0xffff0000u), acc[2 * q + 1]);
                    }
                }
            }
        } else {
            for (int k = 0; k < K; ++k) {
                const int row = dr[k];
                if (row < 0) continue;
                const float w = wr[k];
                const float* yp = (const float*)a.y_perm + (size_t)row * d + j0;
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = fmaf(w, yp[q], acc[q]);
            }
        }
        const size_t o = (size_t)t * a.h + (size_t)g * d + j0;
        if constexpr (BF16) {
            if (a.y_shared) {
                const uint4 v = *(const uint4*)((const uint16_t*)a.y_shared + o);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] += __uint_as_float(u[q] << 16);
                    acc[2 * q + 1] += __uint_as_float(u[q] & 0xffff0000u);
                }
            }
            uint4 out;
            out.x = pack_bf16x2(acc[0], acc[1]);
            out.y = pack_bf16x2(acc[2], acc[3]);
            out.z = pack_bf16x2(acc[4], acc[5]);
            out.w = pack_bf16x2(acc[6], acc[7]);
            *(uint4*)((uint16_t*)a.y + o) = out;
        } else {
            float* yo = (float*)a.y + o;
            const float* ys = a.y_shared ? (const float*)a.y_shared + o : nullptr;
#pragma unroll
            for (int q = 0; q < 8; ++q) yo[q] = ys ? acc[q] + ys[q] : acc[q];
        }
    }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    const long S = (long)a.T * a.H;
    if (S == 0) return hipSuccess;
    int tpr = a.d / 8;
    if (tpr > 256) tpr = 256;
    int p2 = 1;
    while (p2 * 2 <= tpr) p2 *= 2;
    tpr = p2;
    const int rpb = 256 / tpr;
    const long blocks = (S + rpb - 1) / rpb;
    if (a.dtype == MOE_BF16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, a, tpr);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, a, tpr);
    return hipGetLastError();
}

// K = 1, one head: the row of a token whose one assignment was dropped is 0;
// a kept token's row is left alone (the down GEMM stores it there).  One row
// per `tpr` threads, 16-byte stores.
__global__ __launch_bounds__(256) void zero_dropped_kernel(const int32_t* dest_row, int T, int row16, int tpr,
                                                           uint4* y) {
    const int rpb = 256 / tpr;
    const long t = (long)blockIdx.x * rpb + threadIdx.x / tpr;
    if (t >= T || dest_row[t] >= 0) return;
    uint4* row = y + t * row16;
    for (int j = threadIdx.x % tpr; j < row16; j += tpr) row[j] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero_dropped(const int32_t* dest_row, int T, int row_bytes, void* y, hipStream_t st) {
    if (T == 0) return hipSuccess;
    if (row_bytes % 16 != 0 || ((uintptr_t)y & 15) != 0) return hipErrorInvalidValue;
    const int row16 = row_bytes / 16;
    int tpr = 1;
    while (tpr * 2 <= row16 && tpr < 256) tpr *= 2;
    const int rpb = 256 / tpr;
    hipLaunchKernelGGL(zero_dropped_kernel, dim3((T + rpb - 1) / rpb), dim3(256), 0, st, dest_row, T, row16, tpr,
                       (uint4*)y);
    return hipGetLastError();
}

// f_e = counts_e / (T K); P as given, or (at most 64 experts in all) summed
// here from the route kernels' partials (the same order as prob_mean_kernel, so
// the same bits); L_aux =
// mean over heads of alpha E sum_e f_e P_e (fixed-order serial sums; E is at
// most 256).  One block.
constexpr int kStatsMaxEt = 4096;
__global__ __launch_bounds__(1024) void stats_kernel(StatsArgs a) {
    const int Et = a.H * a.E;
    const int tid = threadIdx.x;
    __shared__ float Pl[kStatsMaxEt];
    __shared__ float fl[kStatsMaxEt];
    __shared__ float headsum[256];
    if (a.prob_part) {  // the layer folds P here for at most 64 experts in all (one pass)
        for (int e0 = 0; e0 < Et; e0 += 1024 / 16) {
            const int ge = e0 + tid / 16, j = tid % 16;
            const bool valid = ge < Et;
            const float v = prob_mean_of<16>(a.prob_part, a.nbx, a.E, a.T, ge, valid, j);
            if (valid && j == 0) Pl[ge] = v;
        }
    } else {
        for (int i = tid; i < Et; i += 1024) Pl[i] = a.prob_mean[i];
    }
    for (int i = tid; i < Et; i += 1024) {
        const float fe = (float)a.counts[i] / ((float)a.T * (float)a.K);
        fl[i] = fe;
        if (a.f) a.f[i] = fe;
        if (a.kept_out) a.kept_out[i] = a.kept_in[i];
    }
    __syncthreads();
    for (int i = tid; i < Et; i += 1024)
        if (a.P) a.P[i] = Pl[i];
    for (int g = tid; g < a.H; g += 1024) {
        float s = 0.0f;
        for (int e = 0; e < a.E; ++e) s += fl[g * a.E + e] * Pl[g * a.E + e];
        headsum[g] = a.alpha * (float)a.E * s;
    }
    __syncthreads();
    if (tid == 0) {
        if (a.l_aux) {
            float s = 0.0f;
            for (int g = 0; g < a.H; ++g) s += headsum[g];
            *a.l_aux = s / (float)a.H;
        }
        const int32_t nk = a.offsets[Et];
        if (a.n_kept) *a.n_kept = nk;
        if (a.n_dropped) *a.n_dropped = a.A - nk;
    }
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(1024), 0, st, a);
    return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

}  // namespace moe
