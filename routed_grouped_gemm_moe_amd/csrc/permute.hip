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
//
// For the fused layer the gathered rows go to the packed fragment layout of
// the expert GEMM (gemm_pa.h), each expert segment starting at the 32-aligned
// row pstart[e] (exclusive scan of the counts rounded up to 32); the row index
// inside the segment is the same as in the row-major x_perm.  The same packed
// gather repacks a caller's row-major x_perm for the staged FFN.
#include "gemm_pa.h"
#include "scan.h"

namespace moe {
namespace {

// counts of local assignments per (token block, local expert); with
// scan.arrive set, the last workgroup to finish also runs the scan.
__global__ __launch_bounds__(PERM_TB) void hist_kernel(int64_t T, int64_t k, int64_t e_lo,
                                                       int64_t EL, const int32_t *__restrict__ ids,
                                                       int32_t *__restrict__ blk_counts,
                                                       ScanArgs scan) {
    extern __shared__ int32_t s_cnt[];  // [EL], then the scan's LDS
    for (int64_t e = threadIdx.x; e < EL; e += PERM_TB) s_cnt[e] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * PERM_TB + threadIdx.x;
    if (t < T)
        for (int64_t j0 = 0; j0 < k; j0 += 8) {  // 8 ids in flight at a time
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = j0 + u < k ? ids[t * k + j0 + u] : -1;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t e = (int64_t)v[u] - e_lo;
                if (j0 + u < k && e >= 0 && e < EL) atomicAdd(&s_cnt[e], 1);
            }
        }
    __syncthreads();
    // device-scope stores: the last workgroup of the folded scan reads them
    for (int64_t e = threadIdx.x; e < EL; e += PERM_TB)
        __hip_atomic_store(blk_counts + blockIdx.x * EL + e, s_cnt[e], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (!scan.arrive) return;
    __shared__ int32_t s_last;
    if (scan_arrive_last(scan.arrive, gridDim.x, &s_last)) scan_block<PERM_TB>(scan, s_cnt);
}

// The scan as a kernel of its own (one workgroup).
constexpr int SCAN_THREADS = 1024;
__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(ScanArgs scan) {
    extern __shared__ int32_t s_scan[];
    scan_block<SCAN_THREADS>(scan, s_scan);
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
    extern __shared__ uint32_t s_bits[];  // [EL][WORDS], then the block's segment bases [EL]
    int32_t *s_base = reinterpret_cast<int32_t *>(s_bits + EL * WORDS);
    for (int64_t i = threadIdx.x; i < EL * WORDS; i += PERM_TB) s_bits[i] = 0;
    for (int64_t e = threadIdx.x; e < EL; e += PERM_TB)
        s_base[e] = offsets[e] + blk_base[blockIdx.x * EL + e];
    __syncthreads();
    const int tl = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.x * PERM_TB + tl;
    // ids 8 at a time, loaded before they are used
    auto load8 = [&](int32_t (&v)[8], int64_t j0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = j0 + u < k ? ids[t * k + j0 + u] : -1;
    };
    if (t < T)
        for (int64_t j0 = 0; j0 < k; j0 += 8) {
            int32_t v[8];
            load8(v, j0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t e = (int64_t)v[u] - e_lo;
                if (j0 + u < k && e >= 0 && e < EL)
                    atomicOr(&s_bits[e * WORDS + (tl >> 5)], 1u << (tl & 31));
            }
        }
    __syncthreads();
    if (t < T)
        for (int64_t j0 = 0; j0 < k; j0 += 8) {
            int32_t v[8];
            load8(v, j0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u >= k) break;
                const int64_t e = (int64_t)v[u] - e_lo;
                if (e >= 0 && e < EL) {
                    const uint32_t *b = s_bits + e * WORDS;
                    int32_t r = __popc(b[tl >> 5] & ((1u << (tl & 31)) - 1u));
                    for (int w = 0; w < (tl >> 5); ++w) r += __popc(b[w]);
                    const int32_t pos = s_base[e] + r;
                    perm_src[pos] = (int32_t)t;
                    inv_perm[t * k + j0 + u] = pos;
                } else {
                    inv_perm[t * k + j0 + u] = -1;
                }
            }
        }
}

// Row gather into row-major x_perm (moe_permute): each workgroup copies
// GATHER_TOK token rows, each read once and written to every local slot of
// that token.  16-byte vectors.
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

// Packed gather: one workgroup per (packed 32-row block, 256 columns).  The
// 32 source rows (x[perm_src[...]] for the fused layer, the caller's
// row-major x_perm for the staged FFN; zeros for the padding rows of a
// segment) are read as 512-byte row pieces, transposed through LDS and
// written as 16 contiguous 1 KiB fragments.  LDS slot of fragment kk, lane
// position p: kk*64 + (p ^ (kk & 15)), which spreads both the row-order
// writes and the fragment-order reads over the banks.
constexpr int PACK_THREADS = 256;
constexpr int PACK_COLS = 256;
__global__ __launch_bounds__(PACK_THREADS) void pack_kernel(int64_t d, int64_t EL,
                                                            const bf16_t *__restrict__ src,
                                                            const int32_t *__restrict__ perm_src,
                                                            const int32_t *__restrict__ offsets,
                                                            const int32_t *__restrict__ pstart,
                                                            bf16_t *__restrict__ dst) {
    __shared__ u32x4_t s_frag[32 * (PACK_COLS / 8)];  // 16 KiB
    __shared__ int32_t s_row[32];
    const int64_t rb = blockIdx.x;
    const int64_t prow0 = rb * 32;
    if (prow0 >= pstart[EL]) return;  // past the last segment (uniform)
    if (threadIdx.x < 32) {
        int64_t lo = 0, hi = EL - 1;  // segment holding prow0: last e with pstart[e] <= prow0
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (pstart[mid] <= prow0) lo = mid;
            else hi = mid - 1;
        }
        const int64_t local = prow0 + threadIdx.x - pstart[lo];
        const int64_t cnt = offsets[lo + 1] - offsets[lo];
        int32_t r = -1;
        if (local < cnt) r = perm_src ? perm_src[offsets[lo] + local] : (int32_t)(offsets[lo] + local);
        s_row[threadIdx.x] = r;
    }
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.y * PACK_COLS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = threadIdx.x + PACK_THREADS * i;
        const int r = q >> 5, c = q & 31;
        const int32_t srow = s_row[r];
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (srow >= 0) v = *reinterpret_cast<const u32x4_t *>(src + (int64_t)srow * d + c0 + c * 8);
        const int kk = c >> 1, pos = r + 32 * (c & 1);
        s_frag[kk * 64 + (pos ^ (kk & 15))] = v;
    }
    __syncthreads();
    u32x4_t *o = reinterpret_cast<u32x4_t *>(dst) + (rb * (d / 16) + blockIdx.y * (PACK_COLS / 16)) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = threadIdx.x + PACK_THREADS * i;
        const int kk = g >> 6, pos = g & 63;
        o[g] = s_frag[kk * 64 + (pos ^ (kk & 15))];
    }
}

hipError_t launch_pack(const Dims &D, const bf16_t *src, const int32_t *perm_src,
                       const int32_t *offsets, const int32_t *pstart, bf16_t *dst, hipStream_t s) {
    const int64_t nrb = D.pcap() / 32;
    if (nrb == 0 || D.EL() == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)nrb, (unsigned)(D.d / PACK_COLS)),
                       dim3(PACK_THREADS), 0, s, D.d, D.EL(), src, perm_src, offsets, pstart, dst);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_rows(const Dims &D, const bf16_t *x_perm, const int32_t *offsets,
                            const int32_t *pstart, bf16_t *xp, hipStream_t s) {
    return launch_pack(D, x_perm, nullptr, offsets, pstart, xp, s);
}

hipError_t launch_permute(const Dims &D, const bf16_t *x, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *perm_src, int32_t *inv_perm, bf16_t *x_perm,
                          int32_t *blk_counts, int32_t *blk_base, int32_t *pstart, MTile *mtiles,
                          int32_t *n_mtiles, int32_t *mtile_base, int32_t *sched_state,
                          int64_t sched_state_ints, hipStream_t s, int prep, int32_t *arrive) {
    const int64_t EL = D.EL(), nblk = D.perm_blocks();
    ScanArgs sa = make_scan_args(D, blk_counts, blk_base, counts, offsets, pstart, mtiles, n_mtiles,
                                 mtile_base, sched_state, sched_state_ints, nullptr);
    const size_t scan_lds = (size_t)scan_lds_ints(EL) * sizeof(int32_t);
    hipError_t e;
    if (prep != PREP_SCAN_DONE) {
        if (nblk > 0) {
            // with the arrival counter cleared by the router, the last
            // histogram workgroup runs the scan
            if (prep == PREP_ARRIVE_CLEARED) sa.arrive = arrive;
            const size_t lds = sa.arrive ? scan_lds : EL * sizeof(int32_t);
            hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nblk), dim3(PERM_TB), lds, s, D.T, D.k,
                               D.e_lo, EL, ids, blk_counts, sa);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (!sa.arrive) {
            hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(SCAN_THREADS), scan_lds, s, sa);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (nblk > 0) {
        hipLaunchKernelGGL(rank_kernel, dim3((unsigned)nblk), dim3(PERM_TB),
                           EL * (PERM_TB / 32 + 1) * sizeof(uint32_t), s, D.T, D.k, D.e_lo, EL, ids,
                           offsets, blk_base, perm_src, inv_perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (pstart) {
            if (x_perm) e = launch_pack(D, x, perm_src, offsets, pstart, x_perm, s);
        } else if (x_perm) {
            const unsigned g = (unsigned)((D.T + GATHER_TOK - 1) / GATHER_TOK);
            hipLaunchKernelGGL(gather_kernel, dim3(g), dim3(GATHER_THREADS), 0, s, D.T, D.d, D.k, x,
                               inv_perm, x_perm);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe
