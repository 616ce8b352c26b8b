// backward.hip -- kernels of the layer's backward pass.
//
// The gradient of L = sum(dy * y) + c_aux L_aux follows the forward pass of
// lesson 10 "专家并行 EP" (learn.payai.win), "核心概念" items 1, 3 and 4, in
// reverse: W_o, then the gate-weighted combine (each kept row receives
// w_k dy, each gate weight the dot product of dy with its expert's output),
// the experts (down projection, activation, gate/up projections), the router
// through the gate weights (softmax or sigmoid over the kept experts) plus the
// aux loss through P_i, and finally dx as the sum of the rows' input
// gradients and the router's.  Selection itself is piecewise constant.
//
// The heavy products run on the grouped 64-wide GEMM kernel (gemm.hip), which
// reads k-major operands where they lie through the LDS transposing load:
//   * input gradients (dgrad) multiply by each weight's transpose, reading the
//     forward weights as stored;
//   * weight gradients (wgrad) sum over an expert's rows: both operands are
//     the activations as stored (rows of a group contiguous); the x rows of
//     the gate/up gradients are first gathered into routed order.
// The router's weight gradient (per-head column slices of x, a small product)
// still uses "row blocks": for group g with n_g rows, a column segment of
// max(1, ceil(n_g / 64)) 64-wide stages starting at stage kb_g (the prefix of
// the earlier groups' stage counts), zero-filled past n_g; the GEMM then reads,
// for group g, only the stages [kb_g, kb_g + nk_g) of every row of both
// operands.
#include "common.hpp"

namespace moe {

// ------------------------------------------------------- row-block layout
// kspan[g] = {kb_g, nk_g}; stage_grp[s] = the group owning stage s, -1 past the
// last one.  One block; each thread owns a run of groups.
__global__ __launch_bounds__(1024) void kspan_kernel(const int32_t* offsets, int G, int max_stages, int2* kspan,
                                                     int32_t* stage_grp) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int per = (G + 1023) / 1024;
    int32_t run = 0;
    for (int q = 0; q < per; ++q) {
        const int g = tid * per + q;
        if (g < G) {
            const int32_t n = max(offsets[g + 1] - offsets[g], 0);
            run += max(1, (n + 63) / 64);
        }
    }
    part[tid] = run;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t kb = part[tid] - run;
    const int32_t total = part[1023];
    for (int q = 0; q < per; ++q) {
        const int g = tid * per + q;
        if (g >= G) break;
        const int32_t n = max(offsets[g + 1] - offsets[g], 0);
        const int32_t nk = max(1, (n + 63) / 64);
        kspan[g] = make_int2(kb, nk);
        for (int i = 0; i < nk && kb + i < max_stages; ++i) stage_grp[kb + i] = g;
        kb += nk;
    }
    for (int i = total + tid; i < max_stages; i += 1024) stage_grp[i] = -1;
}

// out[c][64*s + i] = in[src(r)][col0 + g*gcol + c] for stage s of group g,
// r = offsets[g] + 64*(s - kb_g) + i, zero where r >= offsets[g+1].  src(r) =
// rowmap[r] (clamped to [0, nrows_in)) if given, else r - offsets[g] with
// local_rows, else r.  64 x 64 tiles through LDS; ncols % 64 == 0.
__global__ __launch_bounds__(256) void row_blocks_kernel(const uint16_t* in, int ld_in, int col0, int gcol,
                                                         const int32_t* rowmap, int nrows_in, int local_rows,
                                                         const int32_t* offsets, const int2* kspan,
                                                         const int32_t* stage_grp, uint16_t* out, long long ld_out) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const int s = blockIdx.y;
    const int g = stage_grp[s];
    if (g < 0) return;
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * 64;
    const int r0 = offsets[g] + (s - kspan[g].x) * 64;
    const int rend = offsets[g + 1];
    const int cb = col0 + g * gcol + c0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int rr = tid / 8 + 32 * i, ch = tid % 8;
        const int r = r0 + rr;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < rend) {
            int src = r;
            if (rowmap) src = min(max(rowmap[r], 0), nrows_in - 1);
            else if (local_rows) src = r - offsets[g];
            v = *(const u32x4*)(in + (size_t)src * ld_in + cb + ch * 8);
        }
        *(u32x4*)&tile[rr][ch * 8] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid % 64, q = tid / 64 + 4 * i;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)tile[q * 8 + 2 * j][c] | ((uint32_t)tile[q * 8 + 2 * j + 1][c] << 16);
        *(u32x4*)(out + (size_t)(c0 + c) * ld_out + (size_t)s * 64 + q * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// Batched transpose: out[b][c][out_col0 + r] = in[b][r][c] for r < R, and 0 for
// R <= r < min(roundup(R, 64), ld_out - out_col0) (zero padding of the last
// tile); c < Cc with Cc % 8 == 0, out_col0 % 8 == 0, ld_out % 8 == 0.
__global__ __launch_bounds__(256) void transpose_batched_kernel(const uint16_t* in, int R, int Cc, long long bs_in,
                                                                uint16_t* out, int ld_out, int out_col0,
                                                                long long bs_out) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const int b = blockIdx.z;
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const uint16_t* ib = in + (size_t)b * bs_in;
    uint16_t* ob = out + (size_t)b * bs_out;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int rr = tid / 8 + 32 * i, ch = tid % 8;
        const int r = r0 + rr, c = c0 + ch * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < R && c < Cc) v = *(const u32x4*)(ib + (size_t)r * Cc + c);
        *(u32x4*)&tile[rr][ch * 8] = v;
    }
    __syncthreads();
    const int rlim = ld_out - out_col0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid % 64, q = tid / 64 + 4 * i;
        const int r = r0 + q * 8;
        if (c0 + c >= Cc || r >= rlim) continue;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)tile[q * 8 + 2 * j][c] | ((uint32_t)tile[q * 8 + 2 * j + 1][c] << 16);
        *(u32x4*)(ob + (size_t)(c0 + c) * ld_out + out_col0 + r) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// out[i] = i * step for i <= n
__global__ void iota_kernel(int32_t* out, int n, int step) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i <= n) out[i] = i * step;
}

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Combine backward, one wave per assignment a = s*K + k (s = t*H + g):
//   dw[a]      = sum_j dcat[t][g*d + j] * y_perm[row][j]   (fp32, 0 if dropped)
//   dYp[row][j] = bf16(w[a] * dcat[t][g*d + j])
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* dcat, int H, int d, int K, int A,
                                                          const int32_t* dest_row, const float* topk_w,
                                                          const uint16_t* y_perm, uint16_t* dYp, float* dw) {
    const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (a >= A) return;
    const int s = a / K, t = s / H, g = s - t * H;
    const int row = dest_row[a];
    if (row < 0) {
        if (lane == 0) dw[a] = 0.0f;
        return;
    }
    const float w = topk_w[a];
    const uint16_t* dr = dcat + (size_t)t * H * d + (size_t)g * d;
    const uint16_t* yr = y_perm + (size_t)row * d;
    uint16_t* orow = dYp + (size_t)row * d;
    float acc = 0.0f;
    for (int j = lane * 8; j < d; j += 512) {
        const u32x4 dv = *(const u32x4*)(dr + j), yv = *(const u32x4*)(yr + j);
        float de[8], ye[8], oe[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            de[2 * q] = __uint_as_float(dv[q] << 16);
            de[2 * q + 1] = __uint_as_float(dv[q] & 0xffff0000u);
            ye[2 * q] = __uint_as_float(yv[q] << 16);
            ye[2 * q + 1] = __uint_as_float(yv[q] & 0xffff0000u);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            acc = fmaf(de[q], ye[q], acc);
            oe[q] = w * de[q];
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(oe[2 * q], oe[2 * q + 1]);
        *(u32x4*)(orow + j) = o;
    }
    acc = wsum(acc);
    if (lane == 0) dw[a] = acc;
}

// Router backward, one wave per sub-token s = t*H + g; lane l holds experts
// l, l+64, ... of the head.  With l' = logit + logit_bias:
//   softmax: dl_j = w_j (dw_j - sum_k w_k dw_k) for the K selected experts;
//            aux: + c p_j (f_j - sum_i f_i p_i), p = softmax(l')
//   sigmoid: dl_j = (dw_j - sum_k w_k dw_k) / sum_S sigma * sigma_j (1 - sigma_j);
//            aux: + c sigma_j (1 - sigma_j) / sum_all sigma * (f_j - sum_i f_i p_i)
// with f_i = counts_i / (T K) and c = c_aux alpha E / (H T).  Written as bf16
// to dl [H][T][Ep] (head-major, zero in the columns E..Ep-1).
struct RouterBwdArgs {
    int T, H, E, K, Ep, score;
    float caux;  // c_aux * alpha * E / (H * T)
    const float* logits;
    const float* logit_bias;
    const int32_t* topk_idx;
    const float* topk_w;
    const float* dw;
    const int32_t* counts;
    uint16_t* dl;
};

__global__ __launch_bounds__(256) void router_bwd_kernel(RouterBwdArgs a) {
    const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int S = a.T * a.H;
    if (s >= S) return;
    const int t = s / a.H, g = s - t * a.H;
    const int E = a.E, K = a.K;
    constexpr int EJ = 4;  // E <= 256
    float lp[EJ], dl[EJ];
    const float NEG = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = lane + 64 * j;
        float l = NEG;
        if (e < E) {
            l = a.logits[(size_t)s * E + e];
            if (a.logit_bias) l += a.logit_bias[g * E + e];
        }
        lp[j] = l;
        dl[j] = 0.0f;
    }
    // gate-weight part
    float wdw = 0.0f, ssel = 0.0f;
    for (int k = 0; k < K; ++k) {
        wdw += a.topk_w[(size_t)s * K + k] * a.dw[(size_t)s * K + k];
        if (a.score == MOE_SIGMOID) {
            const int e = a.topk_idx[(size_t)s * K + k] - g * E;
            const float l = a.logits[(size_t)s * E + e] + (a.logit_bias ? a.logit_bias[g * E + e] : 0.0f);
            ssel += 1.0f / (1.0f + expf(-l));
        }
    }
    for (int k = 0; k < K; ++k) {
        const int e = a.topk_idx[(size_t)s * K + k] - g * E;
        const float diff = a.dw[(size_t)s * K + k] - wdw;
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            if (lane + 64 * j != e) continue;
            if (a.score == MOE_SIGMOID) {
                const float sg = 1.0f / (1.0f + expf(-lp[j]));
                dl[j] += diff / ssel * sg * (1.0f - sg);
            } else {
                dl[j] += a.topk_w[(size_t)s * K + k] * diff;
            }
        }
    }
    // aux part
    if (a.caux != 0.0f) {
        const float inv = 1.0f / ((float)a.T * (float)K);
        float p[EJ], jac[EJ], loc = 0.0f;
        if (a.score == MOE_SIGMOID) {
            float sg[EJ];
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                sg[j] = lane + 64 * j < E ? 1.0f / (1.0f + expf(-lp[j])) : 0.0f;
                loc += sg[j];
            }
            const float tot = wsum(loc);
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                p[j] = sg[j] / tot;
                jac[j] = sg[j] * (1.0f - sg[j]) / tot;
            }
        } else {
            float m = NEG;
#pragma unroll
            for (int j = 0; j < EJ; ++j) m = fmaxf(m, lp[j]);
            m = wmax(m);
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                p[j] = lane + 64 * j < E ? expf(lp[j] - m) : 0.0f;
                loc += p[j];
            }
            const float tot = wsum(loc);
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                p[j] /= tot;
                jac[j] = p[j];
            }
        }
        float fl[EJ], fp = 0.0f;
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            const int e = lane + 64 * j;
            fl[j] = e < E ? (float)a.counts[g * E + e] * inv : 0.0f;
            fp += fl[j] * p[j];
        }
        fp = wsum(fp);
#pragma unroll
        for (int j = 0; j < EJ; ++j)
            if (lane + 64 * j < E) dl[j] += a.caux * jac[j] * (fl[j] - fp);
    }
    uint16_t* out = a.dl + ((size_t)g * a.T + t) * a.Ep;
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = lane + 64 * j;
        if (e < a.Ep) out[e] = e < E ? f32_to_bf16(dl[j]) : (uint16_t)0;
    }
}

// dx[t][g*d + i] = sum over kept k of dXp[dest_row[s*K + k]][i] + dxr[g][t][i]
// (router, may be null) + dxs[t][g*d + i] (shared expert, may be null), summed
// in fp32 in that order and rounded once.  One thread per 8 outputs.
__global__ __launch_bounds__(256) void dx_kernel(const uint16_t* dXp, const int32_t* dest_row, int T, int H, int d,
                                                 int K, const uint16_t* dxr, const uint16_t* dxs, uint16_t* dx) {
    const int h = H * d;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * (h / 8)) return;
    const int t = (int)(idx / (h / 8));
    const int col = (int)(idx - (long long)t * (h / 8)) * 8;
    const int g = col / d, i = col - g * d;
    const int s = t * H + g;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](const u32x4 v) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += __uint_as_float(v[q] << 16);
            acc[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
        }
    };
    // up to 8 slots' rows are loaded before the first is added (in slot order)
    for (int k0 = 0; k0 < K; k0 += 8) {
        u32x4 v[8];
        bool kept[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = k0 + u;
            const int row = k < K ? dest_row[(size_t)s * K + k] : -1;
            kept[u] = row >= 0;
            v[u] = kept[u] ? *(const u32x4*)(dXp + (size_t)row * d + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (kept[u]) add(v[u]);
    }
    if (dxr) add(*(const u32x4*)(dxr + ((size_t)g * T + t) * d + i));
    if (dxs) add(*(const u32x4*)(dxs + (size_t)t * h + col));
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *(u32x4*)(dx + (size_t)t * h + col) = o;
}

// ------------------------------------------------------------- launchers
hipError_t launch_kspan(const int32_t* offsets, int G, int max_stages, int2* kspan, int32_t* stage_grp,
                        hipStream_t st) {
    hipLaunchKernelGGL(kspan_kernel, dim3(1), dim3(1024), 0, st, offsets, G, max_stages, kspan, stage_grp);
    return hipGetLastError();
}

hipError_t launch_row_blocks(const void* in, int ld_in, int col0, int gcol, const int32_t* rowmap, int nrows_in,
                             int local_rows, const int32_t* offsets, const int2* kspan, const int32_t* stage_grp,
                             int max_stages, int ncols, void* out, long long ld_out, hipStream_t st) {
    if (max_stages <= 0 || ncols <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_blocks_kernel, dim3(ncols / 64, max_stages), dim3(256), 0, st, (const uint16_t*)in, ld_in,
                       col0, gcol, rowmap, nrows_in, local_rows, offsets, kspan, stage_grp, (uint16_t*)out, ld_out);
    return hipGetLastError();
}

// out[r] = in[rowmap[r]] (rows of ncols elements) for r < *n_rows; one block per row
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* in, const int32_t* rowmap, int nrows_in,
                                                          const int32_t* n_rows, int ncols, uint16_t* out) {
    const int r = blockIdx.x;
    if (r >= *n_rows) return;
    const int src = min(max(rowmap[r], 0), nrows_in - 1);
    const u32x4* a = (const u32x4*)(in + (size_t)src * ncols);
    u32x4* b = (u32x4*)(out + (size_t)r * ncols);
    for (int c = threadIdx.x; c < ncols / 8; c += 256) b[c] = a[c];
}

hipError_t launch_gather_rows(const void* in, const int32_t* rowmap, int nrows_in, const int32_t* n_rows, int max_rows,
                              int ncols, void* out, hipStream_t st) {
    if (max_rows <= 0 || ncols <= 0) return hipSuccess;
    if (ncols % 8 != 0 || ((uintptr_t)in & 15) != 0 || ((uintptr_t)out & 15) != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_rows_kernel, dim3(max_rows), dim3(256), 0, st, (const uint16_t*)in, rowmap, nrows_in,
                       n_rows, ncols, (uint16_t*)out);
    return hipGetLastError();
}

hipError_t launch_transpose_batched(const void* in, int B, int R, int Cc, void* out, int ld_out, int out_col0,
                                    hipStream_t st) {
    if (B <= 0 || R <= 0 || Cc <= 0) return hipSuccess;
    const int rpad = min((R + 63) / 64 * 64, ld_out - out_col0);
    hipLaunchKernelGGL(transpose_batched_kernel, dim3((Cc + 63) / 64, (rpad + 63) / 64, B), dim3(256), 0, st,
                       (const uint16_t*)in, R, Cc, (long long)R * Cc, (uint16_t*)out, ld_out, out_col0,
                       (long long)Cc * ld_out);
    return hipGetLastError();
}

hipError_t launch_iota(int32_t* out, int n, int step, hipStream_t st) {
    hipLaunchKernelGGL(iota_kernel, dim3((n + 256) / 256), dim3(256), 0, st, out, n, step);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dcat, int H, int d, int K, int A, const int32_t* dest_row,
                              const float* topk_w, const void* y_perm, void* dYp, float* dw, hipStream_t st) {
    if (A <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_bwd_kernel, dim3((A + 3) / 4), dim3(256), 0, st, (const uint16_t*)dcat, H, d, K, A,
                       dest_row, topk_w, (const uint16_t*)y_perm, (uint16_t*)dYp, dw);
    return hipGetLastError();
}

hipError_t launch_router_bwd(int T, int H, int E, int K, int Ep, int score, float caux, const float* logits,
                             const float* logit_bias, const int32_t* topk_idx, const float* topk_w, const float* dw,
                             const int32_t* counts, void* dl, hipStream_t st) {
    const int S = T * H;
    if (S <= 0) return hipSuccess;
    RouterBwdArgs a{T, H, E, K, Ep, score, caux, logits, logit_bias, topk_idx, topk_w, dw, counts, (uint16_t*)dl};
    hipLaunchKernelGGL(router_bwd_kernel, dim3((S + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_dx(const void* dXp, const int32_t* dest_row, int T, int H, int d, int K, const void* dxr,
                     const void* dxs, void* dx, hipStream_t st) {
    const long long n = (long long)T * H * d / 8;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(dx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const uint16_t*)dXp, dest_row,
                       T, H, d, K, (const uint16_t*)dxr, (const uint16_t*)dxs, (uint16_t*)dx);
    return hipGetLastError();
}

}  // namespace moe
