// The dispatch scan (Weave, §2.1 stage 1: tokens are grouped by expert, so
// every expert's rows need a start offset): from the per-(token block,
// expert) counts, the running base of every block inside its expert's
// segment, the expert counts and exclusive offsets and, for the expert GEMM,
// the 32-aligned packed segment starts, the m-tile table and a cleared
// scheduler state.
//
// One workgroup runs it: either a kernel of its own, or the last workgroup to
// finish of the kernel that produced the counts (it takes a ticket from an
// arrival counter that an earlier kernel of the same call set to zero).
#pragma once

#include "moe_internal.h"

namespace moe {

struct ScanArgs {
    int64_t EL, nblk;
    int32_t *blk_counts;        // [nblk][EL]
    int32_t *blk_base;          // [nblk][EL]
    int32_t *counts, *offsets;  // [EL], [EL + 1]
    int32_t *pstart;            // [EL + 1]; null: no GEMM tables (and no scheduler state)
    MTile *mtiles;
    int32_t *n_mtiles, *mtile_base;
    int32_t *sched;  // cleared: sched_ints ints
    int64_t sched_ints;
    int32_t *arrive;  // arrival counter of the folded form; null when the scan has its own kernel
};

__host__ inline ScanArgs make_scan_args(const Dims &D, int32_t *blk_counts, int32_t *blk_base,
                                        int32_t *counts, int32_t *offsets, int32_t *pstart,
                                        MTile *mtiles, int32_t *n_mtiles, int32_t *mtile_base,
                                        int32_t *sched, int64_t sched_ints, int32_t *arrive) {
    ScanArgs a;
    a.EL = D.EL();
    a.nblk = D.perm_blocks();
    a.blk_counts = blk_counts;
    a.blk_base = blk_base;
    a.counts = counts;
    a.offsets = offsets;
    a.pstart = pstart;
    a.mtiles = mtiles;
    a.n_mtiles = n_mtiles;
    a.mtile_base = mtile_base;
    a.sched = sched;
    a.sched_ints = sched ? sched_ints : 0;
    a.arrive = arrive;
    return a;
}

// Counts staged in LDS per pass of the block running sums.
constexpr int SCAN_TILE = 4096;
__host__ __device__ constexpr int64_t scan_lds_ints(int64_t EL) { return 3 * (EL + 1) + SCAN_TILE + 64; }

// Inclusive sum over the workgroup's threads of (a, b, c), in thread order;
// returns the three totals.  s_w: 3 * (NT / 64) ints of LDS.
template <int NT>
__device__ __forceinline__ int3 block_inclusive3(int &a, int &b, int &c, int32_t *s_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int pa = __shfl_up(a, o), pb = __shfl_up(b, o), pc = __shfl_up(c, o);
        if (lane >= o) {
            a += pa;
            b += pb;
            c += pc;
        }
    }
    if (lane == 63) {
        s_w[3 * wave] = a;
        s_w[3 * wave + 1] = b;
        s_w[3 * wave + 2] = c;
    }
    __syncthreads();
    int3 tot = make_int3(0, 0, 0);
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int wa = s_w[3 * w], wb = s_w[3 * w + 1], wc = s_w[3 * w + 2];
        if (w < wave) {
            a += wa;
            b += wb;
            c += wc;
        }
        tot.x += wa;
        tot.y += wb;
        tot.z += wc;
    }
    __syncthreads();
    return tot;
}

// The scan, by one workgroup of NT threads (NT a multiple of 64, EL <= 1024).
// lds: scan_lds_ints(EL) ints.
template <int NT>
__device__ void scan_block(const ScanArgs &a, int32_t *lds) {
    const int64_t EL = a.EL;
    int32_t *s_cnt = lds;                 // running totals, then offsets
    int32_t *s_mt = lds + (EL + 1);       // m-tiles per expert, then their bases
    int32_t *s_ps = lds + 2 * (EL + 1);   // padded counts, then packed starts
    int32_t *s_tile = lds + 3 * (EL + 1); // block counts of one pass
    int32_t *s_w = s_tile + SCAN_TILE;    // wave totals
    const int tid = threadIdx.x;
    for (int64_t e = tid; e < EL; e += NT) s_cnt[e] = 0;
    // running sums over the blocks, SCAN_TILE counts at a time (coalesced
    // loads into LDS; one thread per expert then walks the blocks in order)
    const int64_t tb = EL > 0 ? (SCAN_TILE / EL > 0 ? SCAN_TILE / EL : 1) : 1;
    for (int64_t b0 = 0; b0 < a.nblk; b0 += tb) {
        const int64_t nb = a.nblk - b0 < tb ? a.nblk - b0 : tb;
        __syncthreads();  // previous pass done with s_tile
        // device-coherent loads: in the folded form the counts were written
        // by other workgroups with device-scope stores or atomics
        for (int64_t i = tid; i < nb * EL; i += NT)
            s_tile[i] = __hip_atomic_load(a.blk_counts + b0 * EL + i, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        for (int64_t e = tid; e < EL; e += NT) {
            int32_t run = s_cnt[e];
            for (int64_t b = 0; b < nb; ++b) {
                a.blk_base[(b0 + b) * EL + e] = run;
                run += s_tile[b * EL + e];
            }
            s_cnt[e] = run;
        }
    }
    for (int64_t i = tid; i < a.sched_ints; i += NT) a.sched[i] = 0;
    __syncthreads();
    // per-expert values; thread tid owns experts [tid*per, tid*per + per)
    const int per = (int)((EL + NT - 1) / NT);
    const int64_t e_beg = (int64_t)tid * per;
    int sc = 0, sm = 0, sp = 0;
    for (int i = 0; i < per; ++i) {
        const int64_t e = e_beg + i;
        if (e < EL) {
            const int32_t c = s_cnt[e];
            a.counts[e] = c;
            s_mt[e] = (c + BM - 1) / BM;
            s_ps[e] = (c + 31) & ~31;
            sc += c;
            sm += s_mt[e];
            sp += s_ps[e];
        }
    }
    const int3 tot = block_inclusive3<NT>(sc, sm, sp, s_w);
    // exclusive prefix of this thread's first expert, then its own run
    int oc = sc, om = sm, op = sp;
    for (int i = per - 1; i >= 0; --i) {
        const int64_t e = e_beg + i;
        if (e < EL) {
            oc -= s_cnt[e];
            om -= s_mt[e];
            op -= s_ps[e];
        }
    }
    for (int i = 0; i < per; ++i) {
        const int64_t e = e_beg + i;
        if (e < EL) {
            const int32_t c = s_cnt[e], m = s_mt[e], p = s_ps[e];
            s_cnt[e] = oc;
            s_mt[e] = om;
            s_ps[e] = op;
            oc += c;
            om += m;
            op += p;
        }
    }
    if (tid == 0) {
        s_cnt[EL] = tot.x;
        s_mt[EL] = tot.y;
        s_ps[EL] = tot.z;
    }
    __syncthreads();
    for (int64_t e = tid; e <= EL; e += NT) a.offsets[e] = s_cnt[e];
    if (a.pstart) {
        for (int64_t e = tid; e <= EL; e += NT) a.pstart[e] = s_ps[e];
        if (tid == 0) *a.n_mtiles = s_mt[EL];
        for (int64_t e = tid; e < EL; e += NT) {
            const int32_t base = s_mt[e], n = s_mt[e + 1] - base;
            const int32_t row0 = s_cnt[e], cnt = s_cnt[e + 1] - row0;
            a.mtile_base[e] = base;
            for (int32_t m = 0; m < n; ++m) {
                MTile t;
                t.e = (int32_t)e;
                t.row0 = row0 + m * BM;
                t.rows = min(BM, cnt - m * BM);
                t.prow0 = s_ps[e] + m * BM;
                a.mtiles[base + m] = t;
            }
        }
    }
}

// Arrival of a workgroup whose share of blk_counts is written with
// device-scope stores or atomics (performed at the device's coherence point,
// not held in an XCD's L2): every wave waits until its writes are performed,
// the workgroup meets, one ticket per workgroup; true (uniform) for the last
// of n workgroups, whose scan then reads the counts with device-coherent
// loads.  No L2 write-back or invalidate is needed on either side.  Every
// thread of the workgroup calls it, outside any loop; s_flag: one int of LDS.
__device__ __forceinline__ bool scan_arrive_last(int32_t *arrive, int64_t n, int32_t *s_flag) {
    __builtin_amdgcn_s_waitcnt(0x7 << 4 | 0xF << 8);  // vmcnt(0): this wave's writes performed
    __syncthreads();
    if (threadIdx.x == 0) {
        const int32_t old =
            __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = old == (int32_t)(n - 1);
    }
    __syncthreads();
    return *s_flag != 0;
}

}  // namespace moe
