// Dispatch on one GPU: the expert histogram, the exclusive scan into segment
// offsets, the stable position of every (token, slot) and the coalesced gather
// of token rows into expert-contiguous rows (Weave, §2.1 stage 1 and Figure 3;
// each source row is read once and written to all its local slots, the
// single-GPU counterpart of the dispatch-side deduplication of Weave §4).
//
// Determinism: counts come from LDS atomics (order-free); positions come from
// per-expert token bitmaps, so a row's position is fixed by its token index:
// offsets[e] + (rows of e in earlier token blocks) + (tokens before it in its
// block that chose e).
#include "moe_internal.h"

namespace moe {
namespace {

// counts of local assignments per (token block, local expert)
__global__ __launch_bounds__(PERM_TB) void hist_kernel(int64_t T, int64_t k, int64_t e_lo,
                                                       int64_t EL, const int32_t *__restrict__ ids,
                                                       int32_t *__restrict__ blk_counts) {
    extern __shared__ int32_t s_cnt[];  // [EL]
    for (int64_t e = threadIdx.x; e < EL; e += PERM_TB) s_cnt[e] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * PERM_TB + threadIdx.x;
    if (t < T)
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = (int64_t)ids[t * k + j] - e_lo;
            if (e >= 0 && e < EL) atomicAdd(&s_cnt[e], 1);
        }
    __syncthreads();
    for (int64_t e = threadIdx.x; e < EL; e += PERM_TB) blk_counts[blockIdx.x * EL + e] = s_cnt[e];
}

// One workgroup: per-expert running sums over token blocks, counts, offsets,
// optionally the GEMM m-tile table and a cleared scheduler state.
constexpr int SCAN_THREADS = 1024;
__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(
    int64_t EL, int64_t nblk, const int32_t *__restrict__ blk_counts, int32_t *__restrict__ blk_base,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, MTile *__restrict__ mtiles,
    int32_t *__restrict__ n_mtiles, int32_t *__restrict__ mtile_base, int32_t *__restrict__ sched,
    int64_t sched_ints) {
    extern __shared__ int32_t s_tmp[];  // [2*EL + 2]
    int32_t *s_cnt = s_tmp;
    int32_t *s_mt = s_tmp + EL + 1;
    for (int64_t e = threadIdx.x; e < EL; e += SCAN_THREADS) {
        int32_t run = 0;
        for (int64_t b = 0; b < nblk; ++b) {
            int32_t c = blk_counts[b * EL + e];
            blk_base[b * EL + e] = run;
            run += c;
        }
        s_cnt[e] = run;
        counts[e] = run;
        s_mt[e] = (run + BM - 1) / BM;
    }
    for (int64_t i = threadIdx.x; i < sched_ints; i += SCAN_THREADS) sched[i] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        // exclusive scans over at most 1024 experts
        int32_t off = 0, mt = 0;
        for (int64_t e = 0; e < EL; ++e) {
            int32_t c = s_cnt[e], m = s_mt[e];
            s_cnt[e] = off;
            s_mt[e] = mt;
            off += c;
            mt += m;
        }
        s_cnt[EL] = off;
        s_mt[EL] = mt;
    }
    __syncthreads();
    for (int64_t e = threadIdx.x; e <= EL; e += SCAN_THREADS) offsets[e] = s_cnt[e];
    if (mtiles) {
        if (threadIdx.x == 0) *n_mtiles = s_mt[EL];
        for (int64_t e = threadIdx.x; e < EL; e += SCAN_THREADS) {
            int32_t base = s_mt[e], n = s_mt[e + 1] - base;
            int32_t row0 = s_cnt[e], cnt = s_cnt[e + 1] - row0;
            mtile_base[e] = base;
            for (int32_t m = 0; m < n; ++m) {
                MTile t;
                t.e = (int32_t)e;
                t.row0 = row0 + m * BM;
                t.rows = min(BM, cnt - m * BM);
                t.pad = 0;
                mtiles[base + m] = t;
            }
        }
    }
}

// Stable rank of each (token, slot) inside its token block via per-expert
// bitmaps; writes perm_src and inv_perm.
__global__ __launch_bounds__(PERM_TB) void rank_kernel(int64_t T, int64_t k, int64_t e_lo,
                                                       int64_t EL, const int32_t *__restrict__ ids,
                                                       const int32_t *__restrict__ offsets,
                                                       const int32_t *__restrict__ blk_base,
                                                       int32_t *__restrict__ perm_src,
                                                       int32_t *__restrict__ inv_perm) {
    constexpr int WORDS = PERM_TB / 32;
    extern __shared__ uint32_t s_bits[];  // [EL][WORDS]
    for (int64_t i = threadIdx.x; i < EL * WORDS; i += PERM_TB) s_bits[i] = 0;
    __syncthreads();
    const int tl = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.x * PERM_TB + tl;
    if (t < T)
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = (int64_t)ids[t * k + j] - e_lo;
            if (e >= 0 && e < EL) atomicOr(&s_bits[e * WORDS + (tl >> 5)], 1u << (tl & 31));
        }
    __syncthreads();
    if (t < T)
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = (int64_t)ids[t * k + j] - e_lo;
            if (e >= 0 && e < EL) {
                const uint32_t *b = s_bits + e * WORDS;
                int32_t r = __popc(b[tl >> 5] & ((1u << (tl & 31)) - 1u));
                for (int w = 0; w < (tl >> 5); ++w) r += __popc(b[w]);
                int32_t pos = offsets[e] + blk_base[blockIdx.x * EL + e] + r;
                perm_src[pos] = (int32_t)t;
                inv_perm[t * k + j] = pos;
            } else {
                inv_perm[t * k + j] = -1;
            }
        }
}

// Row gather: each workgroup copies GATHER_TOK token rows, each read once and
// written to every local slot of that token.  16-byte vectors.
constexpr int GATHER_TOK = 4;
constexpr int GATHER_THREADS = 256;
__global__ __launch_bounds__(GATHER_THREADS) void gather_kernel(int64_t T, int64_t d, int64_t k,
                                                                const bf16_t *__restrict__ x,
                                                                const int32_t *__restrict__ inv_perm,
                                                                bf16_t *__restrict__ x_perm) {
    const int64_t nv = d / 8;
    for (int u = 0; u < GATHER_TOK; ++u) {
        const int64_t t = (int64_t)blockIdx.x * GATHER_TOK + u;
        if (t >= T) return;
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + t * d);
        for (int64_t v = threadIdx.x; v < nv; v += GATHER_THREADS) {
            const u32x4_t val = src[v];
            for (int64_t j = 0; j < k; ++j) {
                int32_t p = inv_perm[t * k + j];
                if (p >= 0) reinterpret_cast<u32x4_t *>(x_perm + (int64_t)p * d)[v] = val;
            }
        }
    }
}

}  // namespace

hipError_t launch_permute(const Dims &D, const bf16_t *x, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *perm_src, int32_t *inv_perm, bf16_t *x_perm,
                          int32_t *blk_counts, int32_t *blk_base, MTile *mtiles,
                          int32_t *n_mtiles, int32_t *mtile_base, int32_t *sched_state,
                          int64_t sched_state_ints, hipStream_t s) {
    const int64_t EL = D.EL(), nblk = D.perm_blocks();
    hipError_t e;
    if (nblk > 0) {
        hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nblk), dim3(PERM_TB), EL * sizeof(int32_t),
                           s, D.T, D.k, D.e_lo, EL, ids, blk_counts);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(SCAN_THREADS), (2 * EL + 2) * sizeof(int32_t), s,
                       EL, nblk, blk_counts, blk_base, counts, offsets, mtiles, n_mtiles,
                       mtile_base, sched_state, sched_state ? sched_state_ints : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (nblk > 0) {
        hipLaunchKernelGGL(rank_kernel, dim3((unsigned)nblk), dim3(PERM_TB),
                           EL * (PERM_TB / 32) * sizeof(uint32_t), s, D.T, D.k, D.e_lo, EL, ids,
                           offsets, blk_base, perm_src, inv_perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const unsigned g = (unsigned)((D.T + GATHER_TOK - 1) / GATHER_TOK);
        hipLaunchKernelGGL(gather_kernel, dim3(g), dim3(GATHER_THREADS), 0, s, D.T, D.d, D.k, x,
                           inv_perm, x_perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_build_mtiles(const Dims &D, const int32_t *offsets, MTile *mtiles,
                               int32_t *n_mtiles, int32_t *mtile_base, hipStream_t s);

}  // namespace moe
