// permute.hip -- expert histogram, prefix scan under capacity, stable rank and
// row gather.
//
// Lesson 10 "专家并行 EP" (learn.payai.win), "核心概念" item 3: the rows bound
// for each expert are packed together before the experts run; item 4: an
// expert keeps at most C = CF K T / E of them and the rest are dropped
// ("Chương 10: Song song MoE", items 1 and 4: capacity factor, drop/pad).  On
// one GPU the pack is a permutation of the token rows into expert-major order.
//
// The assignment list (T*H*K expert ids) is walked in queue order -- the
// stored sub-token-major order, or, for the choice-major queue (all first
// choices, then all second choices, ...), position i = k*S + s holding
// assignment s*K + k -- and cut into chunks of CHUNK positions, one wave per
// chunk:
//   1. hist:    per-chunk expert counts (LDS integer atomics; exact):
//               hist[chunk][e].
//   2. scan:    per expert, the exclusive prefix over chunks (chunk order), the
//               totals (counts) and kept = min(counts, C); blocks of 16 or
//               more experts, each expert's column of chunk counts cut into
//               segments, one thread each (consecutive lanes take consecutive
//               experts, so every access is coalesced): segment sums, their
//               prefix, then each segment rewritten in place.  The offsets
//               (exclusive prefix of kept) are formed by every rank block.
//               Integer sums: exact.
//   When the histogram is small (chunks x experts <= 8192, at most 1024
//   experts), steps 2 and 3 share one launch: each chunk's rank block reads
//   the whole histogram and forms its own bases, the totals, kept and the
//   offsets (the same integer sums, so the same tables).
//   3. rank:    lanes holding the same expert find each other with ballots
//               over the bits of the id and a lane's rank among them is the
//               popcount of the lower lanes; with at most 1024 experts the 16
//               waves of a chunk's block take 64 positions each and add
//               per-wave bases scanned in LDS, otherwise one wave walks the
//               chunk 64 positions at a time with a per-expert running count.
//               pos < C keeps the row at offsets[e]+pos.
//   4. gather:  token-major: the slice of each sub-token is read once and
//               copied to each of its kept rows (16-byte copies).
// No step depends on the order in which blocks run, so the result is unique.
#include "common.hpp"

namespace moe {

constexpr int CHUNK = 1024;       // assignments per chunk (16 steps of 64)
constexpr int MAX_ET = 4096;      // experts the LDS tables hold

int permute_chunks(int A) { return (A + CHUNK - 1) / CHUNK; }

// assignment at queue position i (S sub-tokens, K slots)
__device__ __forceinline__ int queue_at(int i, int S, int K, bool choice) {
    if (!choice) return i;
    const int k = i / S;
    return (i - k * S) * K + k;
}

// the chunk's ids in queue order, position a0 + 64 j + lane in v[j] (-1 past A);
// all CHUNK/64 loads are issued before any is used
__device__ __forceinline__ void load_chunk(const int32_t* idx, int a0, int A, int K, bool choice, int32_t* v) {
    const int S = A / K;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < CHUNK / 64; ++j) {
        const int i = a0 + 64 * j + lane;
        v[j] = i < A ? idx[queue_at(i, S, K, choice)] : -1;
    }
}

// one thread per queue position of the chunk
static_assert(CHUNK == 1024, "hist_kernel and the 16-wave rank kernels take one thread per queue position");
__global__ __launch_bounds__(1024) void hist_kernel(const int32_t* idx, int A, int K, bool choice, int Et, int nch,
                                                    int32_t* hist) {
    __shared__ int cnt[MAX_ET];
    const int tid = threadIdx.x;
    const int i = blockIdx.x * CHUNK + tid;
    const int32_t e = i < A ? idx[queue_at(i, A / K, K, choice)] : -1;
    for (int x = tid; x < Et; x += 1024) cnt[x] = 0;
    __syncthreads();
    if ((unsigned)e < (unsigned)Et) atomicAdd(&cnt[e], 1);  // out-of-range ids are dropped
    __syncthreads();
    for (int x = tid; x < Et; x += 1024) hist[(size_t)blockIdx.x * Et + x] = cnt[x];
}

// Experts [blockIdx.x * epb, +epb) per block of 1024 threads.  hist [nch][Et]
// is rewritten in place as the per-chunk exclusive base of each expert.  S
// threads per expert (S a power of two, S * epb <= 1024), each owning a
// contiguous run of the chunks; counts and kept follow from the totals.  The
// offsets (a prefix over all experts) are left to the rank blocks.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* hist, int nch, int Et, int epb, int capacity,
                                                    int32_t* counts, int32_t* kept) {
    __shared__ int32_t seg[1024];
    const int tid = threadIdx.x;
    const int eb = blockIdx.x * epb, ee = min(eb + epb, Et);
    int S = 1;
    while (S * 2 * epb <= 1024 && S * 2 <= nch) S *= 2;
    const int epp = 1024 / S;              // experts per pass
    const int L = (nch + S - 1) / S;       // chunks per segment
    const int el = tid % epp, sg = tid / epp;  // expert within the pass, segment
    for (int e0 = eb; e0 < ee; e0 += epp) {
        const int e = e0 + el;
        const bool mine = el < epp && e < ee;
        const int c0 = min(sg * L, nch), c1 = min(c0 + L, nch);
        int32_t* col = hist + e;  // chunk c of expert e at col[c * Et]
        // segments are read 16 counts at a time, so 16 loads are in flight
        constexpr int B = 16;
        int32_t sum = 0;
        if (mine)
            for (int cb = c0; cb < c1; cb += B) {
                int32_t v[B];
#pragma unroll
                for (int j = 0; j < B; ++j) v[j] = cb + j < c1 ? col[(size_t)(cb + j) * Et] : 0;
#pragma unroll
                for (int j = 0; j < B; ++j) sum += v[j];
            }
        seg[tid] = sum;
        __syncthreads();
        int32_t base = 0;  // chunks of this expert before the segment
        for (int q = 0; q < sg; ++q) base += seg[q * epp + el];
        if (mine) {
            for (int cb = c0; cb < c1; cb += B) {
                int32_t v[B];
#pragma unroll
                for (int j = 0; j < B; ++j) v[j] = cb + j < c1 ? col[(size_t)(cb + j) * Et] : 0;
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    if (cb + j < c1) col[(size_t)(cb + j) * Et] = base;
                    base += v[j];
                }
            }
            if (sg == S - 1) {
                counts[e] = base;
                kept[e] = base > capacity ? capacity : base;
            }
        }
        __syncthreads();
    }
}

// One wave: off[0..Et) (LDS) holds each expert's kept count and becomes its
// first row, the exclusive prefix over the experts (lane l owns the run
// [l*per, (l+1)*per)); with `store`, also written to offsets[0..Et] and n_kept.
__device__ __forceinline__ void offsets_from_kept(int32_t* off, int Et, bool store, int32_t* offsets,
                                                  int32_t* n_kept) {
    const int lane = threadIdx.x & 63;
    const int per = (Et + 63) / 64;
    int32_t loc = 0;
    for (int q = 0; q < per; ++q) {
        const int e = lane * per + q;
        if (e < Et) loc += off[e];
    }
    int32_t incl = loc;  // inclusive prefix over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
    }
    int32_t b = incl - loc;
    for (int q = 0; q < per; ++q) {
        const int e = lane * per + q;
        if (e < Et) {
            const int32_t k = off[e];
            off[e] = b;
            if (store) offsets[e] = b;
            b += k;
        }
    }
    if (store && lane == 63) {
        offsets[Et] = incl;
        if (n_kept) *n_kept = incl;
    }
}

// Step 3 for one chunk whose ids v were preloaded: run[e] enters as the
// chunk's base for expert e (its earlier queue positions) and is advanced in
// place; off[e] is the expert's first row.
__device__ __forceinline__ void rank_chunk(const int32_t* v, int a0, int A, int K, bool choice, int Et, int nbits,
                                           int capacity, int32_t* run, const int32_t* off, int32_t* dest_row,
                                           int32_t* src_token) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt = lanemask_lt();
    const int S = A / K;
#pragma unroll
    for (int step = 0; step < CHUNK / 64; ++step) {
        const int i = a0 + step * 64 + lane;
        if (a0 + step * 64 >= A) break;  // uniform
        const int a = i < A ? queue_at(i, S, K, choice) : A;
        const int ev = v[step];
        const bool valid = (unsigned)ev < (unsigned)Et;
        const int e = valid ? ev : 0;
        // lanes with the same (valid, e)
        uint64_t peers = __ballot(valid);
        if (!valid) peers = ~peers;
        for (int bit = 0; bit < nbits; ++bit) {
            const bool b = (e >> bit) & 1;
            const uint64_t m = __ballot(b);
            peers &= b ? m : ~m;
        }
        int32_t pos = 0;
        if (valid) pos = run[e] + __popcll(peers & lt);
        __builtin_amdgcn_wave_barrier();
        // the highest lane of each group advances the expert's running count
        if (valid && (peers >> lane) == 1ull) run[e] = pos + 1;
        __builtin_amdgcn_wave_barrier();
        if (a < A && !valid) dest_row[a] = -1;
        if (valid) {
            if (pos < capacity) {
                const int32_t row = off[e] + pos;
                dest_row[a] = row;
                src_token[row] = a / K;
            } else {
                dest_row[a] = -1;
            }
        }
    }
}

// The offsets come from kept (the same prefix in every block; block 0 stores
// it).  base may be null (no chunks): every base is then 0.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* idx, int A, int K, bool choice, int Et, int nbits,
                                                  int capacity, const int32_t* base, const int32_t* kept,
                                                  int32_t* offsets, int32_t* n_kept, int32_t* dest_row,
                                                  int32_t* src_token) {
    __shared__ int32_t run[MAX_ET];
    __shared__ int32_t off[MAX_ET];
    const int a0 = blockIdx.x * CHUNK;
    int32_t v[CHUNK / 64];
    load_chunk(idx, a0, A, K, choice, v);
    for (int e = threadIdx.x; e < Et; e += 64) {
        run[e] = base ? base[(size_t)blockIdx.x * Et + e] : 0;
        off[e] = kept[e];
    }
    __syncthreads();
    offsets_from_kept(off, Et, blockIdx.x == 0, offsets, n_kept);
    __syncthreads();
    rank_chunk(v, a0, A, K, choice, Et, nbits, capacity, run, off, dest_row, src_token);
}

// Step 3 over one chunk with 16 waves (Et <= kWideEt): wave w owns queue
// positions a0 + 64 w + lane and finds, with the ballots of rank_chunk, the
// lanes holding the same expert.  The highest lane of each group stores the
// group's size to cnt[w][e] (LDS, zeroed beforehand); the block then turns
// cnt into each wave's base per expert (chunk base, then the waves in order)
// and every lane's position is its wave's base plus the popcount of its lower
// peers.  The same positions as rank_chunk's 16 sequential steps.
constexpr int kWideEt = 1024;
__device__ __forceinline__ void rank_chunk_wide(int32_t ev, int a0, int A, int K, bool choice, int Et, int nbits,
                                                int capacity, int32_t (*cnt)[kWideEt], const int32_t* chunk_base,
                                                const int32_t* off, int32_t* dest_row, int32_t* src_token) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int i = a0 + 64 * w + lane;
    const int S = A / K;
    const int a = i < A ? queue_at(i, S, K, choice) : A;
    const bool valid = (unsigned)ev < (unsigned)Et;
    const int e = valid ? ev : 0;
    uint64_t peers = __ballot(valid);
    if (!valid) peers = ~peers;
    for (int bit = 0; bit < nbits; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t m = __ballot(b);
        peers &= b ? m : ~m;
    }
    if (valid && (peers >> lane) == 1ull) cnt[w][e] = __popcll(peers);
    __syncthreads();
    for (int x = tid; x < Et; x += 1024) {
        int32_t run = chunk_base[x];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int32_t c = cnt[q][x];
            cnt[q][x] = run;
            run += c;
        }
    }
    __syncthreads();
    if (a < A && !valid) dest_row[a] = -1;
    if (valid) {
        const int32_t pos = cnt[w][e] + __popcll(peers & lanemask_lt());
        if (pos < capacity) {
            const int32_t row = off[e] + pos;
            dest_row[a] = row;
            src_token[row] = a / K;
        } else {
            dest_row[a] = -1;
        }
    }
}

// Step 3 after the scan kernel, 16 waves per chunk (Et <= kWideEt): the bases
// come from hist as the scan rewrote it, the offsets from kept (the same prefix
// in every block; block 0 stores it).  base may be null (no chunks).
__global__ __launch_bounds__(1024) void rank_wide_kernel(const int32_t* idx, int A, int K, bool choice, int Et,
                                                         int nbits, int capacity, const int32_t* base,
                                                         const int32_t* kept, int32_t* offsets, int32_t* n_kept,
                                                         int32_t* dest_row, int32_t* src_token) {
    __shared__ int32_t cnt[16][kWideEt];
    __shared__ int32_t cb[kWideEt];
    __shared__ int32_t off[kWideEt];
    const int tid = threadIdx.x;
    const int c = blockIdx.x, a0 = c * CHUNK;
    const int S = A / K;
    const int i = a0 + tid;
    const int32_t ev = i < A ? idx[queue_at(i, S, K, choice)] : -1;
    for (int x = tid; x < 16 * Et; x += 1024) cnt[x / Et][x % Et] = 0;
    for (int e = tid; e < Et; e += 1024) {
        cb[e] = base ? base[(size_t)c * Et + e] : 0;
        off[e] = kept[e];
    }
    __syncthreads();
    if (tid < 64) offsets_from_kept(off, Et, c == 0, offsets, n_kept);
    rank_chunk_wide(ev, a0, A, K, choice, Et, nbits, capacity, cnt, cb, off, dest_row, src_token);
}

// Steps 2 and 3 in one launch when the histogram is small (nch * Et <= kFusedHist,
// Et <= kWideEt): every chunk's block (16 waves) reads the whole histogram,
// forms its own bases (the counts of the earlier chunks, in chunk order), the
// totals, kept = min(total, C) and the offsets (a wave prefix over the experts,
// each lane owning a run of Et/64 of them), then ranks its ids
// (rank_chunk_wide).  Block 0 also stores the tables.  Integer sums, so every
// block derives the same tables as the scan kernel would.
constexpr int kFusedHist = 8192;
__global__ __launch_bounds__(1024) void rank_fused_kernel(const int32_t* idx, int A, int K, bool choice, int Et,
                                                          int nbits, int capacity, int nch, const int32_t* hist,
                                                          int32_t* counts, int32_t* kept, int32_t* offsets,
                                                          int32_t* n_kept, int32_t* dest_row, int32_t* src_token) {
    __shared__ int32_t cnt[16][kWideEt];
    __shared__ int32_t base[kWideEt];
    __shared__ int32_t off[kWideEt];
    const int tid = threadIdx.x;
    const int c = blockIdx.x, a0 = c * CHUNK;
    // this thread's id (queue position a0 + tid), loaded first
    const int S = A / K;
    const int i = a0 + tid;
    const int32_t ev = i < A ? idx[queue_at(i, S, K, choice)] : -1;
    for (int x = tid; x < 16 * Et; x += 1024) cnt[x / Et][x % Et] = 0;
    // per expert: base over chunks < c, total over all chunks (16 loads in flight)
    for (int e = tid; e < Et; e += 1024) {
        int32_t b = 0, tot = 0;
        for (int q0 = 0; q0 < nch; q0 += 16) {
            int32_t h[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) h[j] = q0 + j < nch ? hist[(size_t)(q0 + j) * Et + e] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                b += q0 + j < c ? h[j] : 0;
                tot += h[j];
            }
        }
        base[e] = b;
        off[e] = tot > capacity ? capacity : tot;  // kept, turned into offsets below
        if (c == 0) {
            counts[e] = tot;
            kept[e] = off[e];
        }
    }
    __syncthreads();
    if (tid < 64) offsets_from_kept(off, Et, c == 0, offsets, n_kept);
    // (rank_chunk_wide's first barrier orders the offsets before their use)
    rank_chunk_wide(ev, a0, A, K, choice, Et, nbits, capacity, cnt, base, off, dest_row, src_token);
}

// Steps 1-3 in one block of 1024 threads (16 waves) when the assignment list
// is short (at most kOneBlockA) and the experts few (at most kOneBlockEt):
// wave w owns queue positions [w L, (w+1) L) (L a multiple of 64), loads its
// ids once into registers, counts them per expert into its own LDS row, the
// block scans those rows over the waves (the wave bases) and the kept counts
// over the experts (the offsets), and the wave ranks its ids 64 at a time with
// the same ballots as rank_kernel.  One launch instead of three; the tables
// are the same (the stable rank is unique).  Measured on one MI355X: 16 -> 9 us
// at 512 assignments, but slower than the chunked kernels from 16 384 on
// (21.7 -> 30.7 us for 64 experts), hence the small limit.
constexpr int kOneBlockA = 4096, kOneBlockEt = 1024;
constexpr int kOneBlockSteps = kOneBlockA / (16 * 64);  // 64-position steps per wave, at most

__global__ __launch_bounds__(1024) void tables_one_block_kernel(const int32_t* idx, int A, int K, bool choice, int Et,
                                                                int nbits, int capacity, int32_t* counts,
                                                                int32_t* kept, int32_t* offsets, int32_t* n_kept,
                                                                int32_t* dest_row, int32_t* src_token) {
    __shared__ int32_t tab[16 * kOneBlockEt];  // per-wave counts, then per-wave bases / running counts
    __shared__ int32_t off[kOneBlockEt];
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int L = (A + 16 * 64 - 1) / (16 * 64) * 64;
    const int p0 = w * L, p1 = min(p0 + L, A);
    const int S = A / K;
    int32_t* row = tab + w * Et;
    for (int e = lane; e < Et; e += 64) row[e] = 0;
    // this wave's ids in queue order: position p0 + 64 j + lane in ids[j]
    int32_t ids[kOneBlockSteps];
#pragma unroll
    for (int j = 0; j < kOneBlockSteps; ++j) {
        const int i = p0 + 64 * j + lane;
        ids[j] = i < p1 ? idx[queue_at(i, S, K, choice)] : -1;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kOneBlockSteps; ++j)
        if ((unsigned)ids[j] < (unsigned)Et) atomicAdd(&row[ids[j]], 1);  // out-of-range ids are dropped
    __syncthreads();
    // per expert: exclusive prefix over the waves (queue order), totals, kept
    for (int e = tid; e < Et; e += 1024) {
        int32_t run = 0;
        for (int q = 0; q < 16; ++q) {
            const int32_t v = tab[q * Et + e];
            tab[q * Et + e] = run;
            run += v;
        }
        counts[e] = run;
        const int32_t k = run > capacity ? capacity : run;
        kept[e] = k;
        off[e] = k;
    }
    __syncthreads();
    // offsets: exclusive prefix of kept over experts (each thread owns a run)
    const int per = (Et + 1023) / 1024;
    int32_t run = 0;
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < Et) run += off[e];
    }
    part[tid] = run;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const int32_t v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t b = part[tid] - run;
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < Et) {
            const int32_t k = off[e];
            off[e] = b;
            offsets[e] = b;
            b += k;
        }
    }
    if (tid == 1023) {
        offsets[Et] = part[1023];
        if (n_kept) *n_kept = part[1023];
    }
    __syncthreads();
    // ranks: row holds this wave's base per expert and becomes its running count
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int j = 0; j < kOneBlockSteps; ++j) {
        if (p0 + 64 * j >= p1) break;  // uniform over the wave
        const int i = p0 + 64 * j + lane;
        const int a = i < p1 ? queue_at(i, S, K, choice) : A;
        const int ev = ids[j];
        const bool valid = (unsigned)ev < (unsigned)Et;
        const int e = valid ? ev : 0;
        uint64_t peers = __ballot(valid);
        if (!valid) peers = ~peers;
        for (int bit = 0; bit < nbits; ++bit) {
            const bool v = (e >> bit) & 1;
            const uint64_t m = __ballot(v);
            peers &= v ? m : ~m;
        }
        int32_t pos = 0;
        if (valid) pos = row[e] + __popcll(peers & lt);
        __builtin_amdgcn_wave_barrier();
        if (valid && (peers >> lane) == 1ull) row[e] = pos + 1;
        __builtin_amdgcn_wave_barrier();
        if (a < A && !valid) dest_row[a] = -1;
        if (valid) {
            if (pos < capacity) {
                const int32_t r = off[e] + pos;
                dest_row[a] = r;
                src_token[r] = a / K;
            } else {
                dest_row[a] = -1;
            }
        }
    }
}

// Token-major copy: sub-token s = t*H + g reads its slice x[t][g*d : g*d+d]
// once and stores it to x_perm[dest_row[s*K + k]] for each kept slot k.
// `tps` threads per sub-token (a power of two, at most 256) copy 16 bytes each
// per step; 256/tps sub-tokens per block.
__global__ __launch_bounds__(256) void gather_kernel(const void* x, int H, int rowbytes, int K, int S,
                                                     const int32_t* dest_row, int tps, int max_rows, void* x_perm) {
    const int spb = 256 / tps;
    const int s = blockIdx.x * spb + threadIdx.x / tps;
    const int c = threadIdx.x % tps;
    if (s >= S) return;
    const int t = s / H, g = s - t * H;
    const char* src = (const char*)x + (size_t)t * (size_t)(rowbytes * H) + (size_t)g * rowbytes;
    const int32_t* dr = dest_row + (size_t)s * K;
    bool any = false;  // a sub-token whose every slot was dropped is not read at all
    for (int k = 0; k < K; ++k) any |= dr[k] >= 0;
    if (!any) return;
    for (int o = c * 16; o < rowbytes; o += tps * 16) {
        const uint4 v = *(const uint4*)(src + o);
        for (int k = 0; k < K; ++k) {
            const int row = dr[k];
            if (row >= 0 && row < max_rows) *(uint4*)((char*)x_perm + (size_t)row * rowbytes + o) = v;
        }
    }
}

static hipError_t launch_tables_chunked(const PermuteArgs& p, int nch, int nbits, hipStream_t st) {
    hipError_t err;
    if (nch > 0) {
        hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(1024), 0, st, p.topk_idx, p.A, p.K, p.queue == MOE_QUEUE_CHOICE,
                           p.Et, nch, p.hist);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (nch > 0 && (size_t)nch * p.Et <= (size_t)kFusedHist && p.Et <= kWideEt) {
        hipLaunchKernelGGL(rank_fused_kernel, dim3(nch), dim3(1024), 0, st, p.topk_idx, p.A, p.K,
                           p.queue == MOE_QUEUE_CHOICE, p.Et, nbits, p.capacity, nch, p.hist, p.counts, p.kept,
                           p.offsets, p.n_kept, p.dest_row, p.src_token);
        return hipGetLastError();
    }
    // 16 experts per scan block (measured on one MI355X, 256 chunks x 256
    // experts: one block for all experts 20 us)
    const int epb = std::max(16, (p.Et + 63) / 64);
    hipLaunchKernelGGL(scan_kernel, dim3((p.Et + epb - 1) / epb), dim3(1024), 0, st, p.hist, nch, p.Et, epb,
                       p.capacity, p.counts, p.kept);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // no assignments: one block stores the (zero) offsets
    const int nb = nch > 0 ? nch : 1;
    const int32_t* base = nch > 0 ? p.hist : nullptr;
    if (p.Et <= kWideEt)
        hipLaunchKernelGGL(rank_wide_kernel, dim3(nb), dim3(1024), 0, st, p.topk_idx, p.A, p.K,
                           p.queue == MOE_QUEUE_CHOICE, p.Et, nbits, p.capacity, base, p.kept, p.offsets, p.n_kept,
                           p.dest_row, p.src_token);
    else
        hipLaunchKernelGGL(rank_kernel, dim3(nb), dim3(64), 0, st, p.topk_idx, p.A, p.K, p.queue == MOE_QUEUE_CHOICE,
                           p.Et, nbits, p.capacity, base, p.kept, p.offsets, p.n_kept, p.dest_row, p.src_token);
    return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& p, hipStream_t st) {
    const int nch = permute_chunks(p.A);
    hipError_t err;
    int nbits = 1;
    while ((1 << nbits) < p.Et) ++nbits;
    if (p.A > 0 && p.A <= kOneBlockA && p.Et <= kOneBlockEt) {
        hipLaunchKernelGGL(tables_one_block_kernel, dim3(1), dim3(1024), 0, st, p.topk_idx, p.A, p.K,
                           p.queue == MOE_QUEUE_CHOICE, p.Et, nbits, p.capacity, p.counts, p.kept, p.offsets, p.n_kept,
                           p.dest_row, p.src_token);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    } else {
        if ((err = launch_tables_chunked(p, nch, nbits, st)) != hipSuccess) return err;
    }
    if (nch == 0) return hipSuccess;
    if (p.x && p.x_perm && p.max_rows > 0) {
        const int esz = p.dtype == MOE_BF16 ? 2 : 4;
        const int rowbytes = p.d * esz;
        int tps = 1;
        while (tps < 256 && tps * 16 < rowbytes) tps *= 2;
        const int S = p.A / p.K;  // sub-tokens
        const int spb = 256 / tps;
        const int blocks = (S + spb - 1) / spb;
        hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, st, p.x, p.H, rowbytes, p.K, S, p.dest_row, tps,
                           p.max_rows, p.x_perm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace moe
