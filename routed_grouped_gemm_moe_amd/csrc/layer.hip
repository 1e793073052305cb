// Persistent expert-FFN + combine kernel of moe_layer.
//
// One workgroup per CU stays resident and claims tiles until none are left
// (Weave, §4: a persistent kernel in which each SM claims its next tile with
// an atomicAdd on a global counter, in the order of the chunk pipeline's
// dependency graph).  Three tile kinds, claimed in dependency order:
//   1. gate/up tiles (m-tile, 128 h columns): GEMM0 + SiLU-mul epilogue;
//      each finished tile bumps gu_done[m-tile].
//   2. down tiles (m-tile, 256 y columns): wait until gu_done[m-tile] counts
//      every gate/up tile of that row block, then GEMM1; a finished tile sets
//      dn_flag[m-tile, column block].
//   3. combine tiles (32 tokens, up to 4 x 256 columns): wait for the dn_flag
//      of every (m-tile, column block) their rows live in, then the gated sum.
// A finished down tile thus hands its rows to the combine through a device-
// side flag as soon as it is written (the producer-consumer tile signaling of
// Cui et al., abstract), not at a kernel boundary.
//
// GEMM tiles are those of gemm_pa.h: x_perm and h are in its packed layout
// (h written by the gate/up epilogue, read as the down tiles' A operand).
//
// Interleaved order (moe_set_tile_order(1)): before each gate/up claim a
// workgroup takes the next down tile of its XCD's range if that tile's m-tile
// has all its gate/up tiles published (compare-and-swap, so only a ready
// tile is taken); such a tile never waits, so the argument below holds.
//
// Queues: gate/up and down tiles follow the blocked order of gemm_tile.h and
// each kind is split into 8 contiguous ranges, one per XCD.  A workgroup reads
// the XCD it runs on from the hardware (XCC_ID), drains that XCD's range
// first (so the tiles sharing weight and activation tiles meet in one L2),
// then steals from the others, and moves to the next kind only when every
// range of the current kind is claimed.  Deadlock freedom: a tile waits only
// on tiles of an earlier kind, all of which were claimed earlier by running
// workgroups whose own waits are, inductively, satisfiable.
//
// Memory ordering (MI355X: one L2 per XCD; an agent-scope release writes the
// issuing XCD's L2 back, an agent-scope acquire invalidates it):
//  - producers: each wave waits for its stores, the workgroup meets at a
//    barrier, then one wave publishes with a single agent-scope release RMW;
//  - gate/up producers also OR their XCD into gu_xcd[m-tile].  A down tile
//    whose producers all ran on its own XCD reads h through the shared L2 and
//    only invalidates the CU's L1; otherwise it takes the agent-scope acquire.
//    The blocked queues keep most chains inside one XCD, so most down tiles
//    leave the other workgroups' L2 contents alone;
//  - combine tiles read y with device-coherent (agent-scope atomic) loads, so
//    they never invalidate L2 either.
// Polling is bounded in time: a wait that exceeds the timeout records
// MOE_ERR_DEVICE_TIMEOUT in the status word and carries on (the result is
// then invalid, but the kernel drains).
#include "combine_tile.h"
#include "gemm_pa.h"

namespace moe {
namespace {

// Synchronisation helpers.  Every branch and loop exit next to a barrier is
// wave-uniform: work that one agent must do (claim a tile, bump a counter,
// poll a flag) is done by all 64 lanes of wave 0 with uniform values
// (readfirstlane, wave votes), never inside an `if (threadIdx.x == 0)`.  With
// a lane-divergent region at the edge of a loop that contains barriers, the
// compiler may rotate the loop so that lane 0 runs that region while the
// other lanes already re-enter the body and wait at a barrier with stale
// state -- the waves then never meet and the workgroup hangs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The XCD this wave runs on (hardware register XCC_ID).
__device__ __forceinline__ int hw_xcd() {
    int id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
    return id & (NUM_XCD - 1);
}

// Claim one tile of [0, n) for the calling wave.  Queue y covers
// [y*per, y*per + per); the own XCD's queue first, then the others.
__device__ __forceinline__ int claim_tile(int32_t *q, int n, int xcd) {
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    for (int r = 0; r < NUM_XCD; ++r) {
        const int y = (xcd + r) & (NUM_XCD - 1);
        const int lo = y * per;
        const int len = min(n, lo + per) - lo;
        if (len <= 0) continue;
        int32_t *c = q + y * QSTRIDE;
        if (uniform(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >= len)
            continue;
        // lane 0 adds 1, the others 0: lane 0's pre-op value is the claim
        const int old = uniform(__hip_atomic_fetch_add(c, lane_id() == 0 ? 1 : 0,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (old < len) return lo + old;
    }
    return -1;
}

// Interleaved order (X-Stage §4.3, in its ready-only form): the next down
// claim of this XCD's range, taken only if that tile's m-tile has every
// gate/up tile published -- so the down tile never waits on gate/up work that
// may not be claimed yet.  Compare-and-swap on the range's counter (lane 0
// swaps cur -> cur + 1, the other lanes cur -> cur, which never changes it);
// -1 if the range is drained, the tile is not ready, or another workgroup
// claimed first.
__device__ __forceinline__ int claim_ready_down(const LayerArgs &a, int32_t *q, int n, int n2,
                                                int nsp, int S, int MT, int NT1, int NT2,
                                                int xcd) {
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    const int lo = xcd * per;
    const int len = min(n, lo + per) - lo;
    if (len <= 0) return -1;
    int32_t *c = q + xcd * QSTRIDE;
    const int cur = uniform(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (cur >= len) return -1;
    int L, part, st, mt, nt;
    dn_claim(lo + cur, n2, nsp, S, &L, &part, &st);
    expert_tile(L, MT, NT2, (int)a.D.EL(), a.mtiles, a.mtile_base, &mt, &nt);
    if (uniform(__hip_atomic_load(a.gu_done + mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
        NT1)
        return -1;
    const int old = uniform(atomicCAS(c, cur, lane_id() == 0 ? cur + 1 : cur));
    return old == cur ? lo + cur : -1;
}

__device__ __forceinline__ int next_tile(int32_t *q, int n, int xcd, int *s_claim) {
    if (wave_id() == 0) *s_claim = claim_tile(q, n, xcd);  // all lanes store the same value
    __syncthreads();
    const int L = uniform(*s_claim);
    __syncthreads();
    return L;
}

// Wave-uniform wait until every lane's flag satisfies *p >= target (lanes with
// need == false do not wait).  Bounded in wall-clock time (wall_clock64
// ticks): past wait_ticks the status word records MOE_ERR_DEVICE_TIMEOUT, and
// once any wait has timed out every other wait of the launch returns at once,
// so a launch never outlives one timeout plus its own compute.
__device__ __forceinline__ void wave_wait_geq(const int32_t *p, int32_t target, bool need,
                                              int64_t wait_ticks, int32_t *status) {
    const int64_t t0 = (int64_t)wall_clock64();
    for (;;) {
        const bool ok = !need || __hip_atomic_load(p, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) >= target;
        if (__all(ok)) return;
        if (uniform(__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
            return;
        if ((int64_t)wall_clock64() - t0 > wait_ticks) {
            __hip_atomic_store(status, (int32_t)MOE_ERR_DEVICE_TIMEOUT, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// Publish a finished tile: every wave's stores have completed (reached L2)
// before the barrier; then wave 0 optionally records its XCD in *xmask and
// bumps (add) or sets (store 1) the counter with one agent-scope release,
// which writes this XCD's L2 back first.
__device__ __forceinline__ void publish(int32_t *p, bool add, int32_t *xmask, int xcd) {
    wait_vmcnt<0>();
    __syncthreads();
    if (wave_id() == 0) {
        const bool l0 = lane_id() == 0;
        if (xmask)
            __hip_atomic_fetch_or(xmask, l0 ? (1 << xcd) : 0, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        if (add)
            __hip_atomic_fetch_add(p, l0 ? 1 : 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(p, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void invalidate_l1() { asm volatile("buffer_inv sc0" ::: "memory"); }

// Optional per-tile trace (measurement aid): one 4 x int64 record per tile,
// {kind << 32 | tile, workgroup << 8 | xcd, start, end} (kind 1 gate/up, 2
// down, 4 half of a cut down tile, 3 combine), times in
// wall_clock64 ticks.  Written by lane 0 of wave 0; slots come from an atomic
// counter at trace[0]; records past the capacity are dropped.
__device__ __forceinline__ void trace_tile(const LayerArgs &a, int kind, int L, int xcd,
                                           int64_t t0) {
    if (!a.trace) return;
    const int64_t t1 = (int64_t)wall_clock64();
    if (wave_id() == 0 && lane_id() == 0) {
        const int64_t i = __hip_atomic_fetch_add(a.trace, (int64_t)1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        if (i < a.trace_cap) {
            int64_t *r = a.trace + 1 + 4 * i;
            r[0] = ((int64_t)kind << 32) | (int64_t)L;
            r[1] = ((int64_t)blockIdx.x << 8) | xcd;
            r[2] = t0;
            r[3] = t1;
        }
    }
}

// One down claim LS (a whole tile or a K part of a cut tile): wait until its
// m-tile's gate/up tiles are published, GEMM1 into y, publish dn_flag.
__device__ __forceinline__ void down_tile(const LayerArgs &a, int LS, int n2, int nsp, int S,
                                          int MT, int NT1, int NT2, int xcd, char *lds) {
    const Dims &D = a.D;
    const int64_t d = D.d, f = D.f;
    const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
    int L, part, st;
    dn_claim(LS, n2, nsp, S, &L, &part, &st);
    int mt, nt;
    expert_tile(L, MT, NT2, (int)a.D.EL(), a.mtiles, a.mtile_base, &mt, &nt);
    const MTile t = a.mtiles[mt];
    if (wave_id() == 0) wave_wait_geq(a.gu_done + mt, NT1, true, a.wait_ticks, a.status);
    __syncthreads();
    const int producers =
        uniform(__hip_atomic_load(a.gu_xcd + mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (producers & ~(1 << xcd))
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    else
        invalidate_l1();
    const int64_t prb = t.prow0 / 32;
    // a cut tile computes K part `part`, starting at k = part * f / S
    const int64_t Kp = part < 0 ? f : f / S, k0 = part < 0 ? 0 : part * Kp;
    const int64_t wo = ((int64_t)t.e * d + (int64_t)nt * BN_DN) * f + k0;
    const SplitCtl sc{a.dn_cnt + st, a.dn_part + (int64_t)st * (CUT_MAX * BM * BN_DN), part,
                      S};
    const bool wrote = gemm_tile_pa<PA_BF16>(
        a.h + (prb * (f / 16) + k0 / 16) * 512, f / 16, t.rows, (int)Kp, a.w_down + wo,
        nullptr, f, a.y + (int64_t)t.row0 * d + (int64_t)nt * BN_DN, d, lds,
        part < 0 ? nullptr : &sc);
    if (!wrote) {  // the last part to arrive writes the tile
        trace_tile(a, 4, LS, xcd, t0);
        return;
    }
    publish(a.dn_flag + (int64_t)mt * NT2 + nt, false, nullptr, xcd);
    // count published down tiles (after the release above, so a
    // reader that sees the full count also sees every y row)
    if (wave_id() == 0)
        __hip_atomic_fetch_add(a.dn_done, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    trace_tile(a, part < 0 ? 2 : 4, LS, xcd, t0);
}

template <bool OUT_F32>
__global__ __launch_bounds__(GEMM_THREADS, 1) void layer_kernel(LayerArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ int s_claim;
    const Dims &D = a.D;
    const int xcd = hw_xcd();
    const int MT = *a.n_mtiles;
    const int NT1 = (int)D.nt_gu();
    const int NT2 = (int)D.nt_dn();
    const int64_t d = D.d, f = D.f, k = D.k;

    // down claims: those of the last partial round (of gridDim.x workgroups)
    // are cut into S K parts, claimed after the whole tiles
    const int n2 = MT * NT2;
    const int S = (int)D.dn_parts();
    const int nsp = dn_split_tiles(S, n2, (int)gridDim.x);
    const int n2c = n2 + (S - 1) * nsp;

    // 1. gate/up tiles, then 2. down tiles, in one claim loop (so each tile
    // body is instantiated once).  Phase 1 claims gate/up tiles -- with the
    // interleaved order a ready down tile of this XCD's range first (kind bit
    // 1 << 30) -- and phase 2, once every gate/up range is drained, the
    // remaining down claims.
    const int n1 = MT * NT1;
    constexpr int DOWN = 1 << 30;
    int phase = n1 > 0 ? 1 : 2;
    if (n1 > 0 || n2 > 0)
        for (;;) {
            if (wave_id() == 0) {
                int v;
                if (phase == 1) {
                    const int r = a.interleave && n2 > 0
                                      ? claim_ready_down(a, a.queues + NUM_XCD * QSTRIDE, n2c, n2,
                                                         nsp, S, MT, NT1, NT2, xcd)
                                      : -1;
                    v = r >= 0 ? (r | DOWN) : claim_tile(a.queues, n1, xcd);
                    if (v < 0) v = -2;  // gate/up drained: move to phase 2
                } else {
                    const int r =
                        n2 > 0 ? claim_tile(a.queues + NUM_XCD * QSTRIDE, n2c, xcd) : -1;
                    v = r >= 0 ? (r | DOWN) : -1;
                }
                s_claim = v;  // every lane stores the same value
            }
            __syncthreads();
            const int v = uniform(s_claim);
            __syncthreads();
            if (v == -2) {
                phase = 2;
                continue;
            }
            if (v < 0) break;
            if (v & DOWN) {
                down_tile(a, v & ~DOWN, n2, nsp, S, MT, NT1, NT2, xcd, lds);
                continue;
            }
            const int L = v;
            const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
            int mt, nt;
            expert_tile(L, MT, NT1, (int)D.EL(), a.mtiles, a.mtile_base, &mt, &nt);
            const MTile t = a.mtiles[mt];
            const int64_t wo = ((int64_t)t.e * f + (int64_t)nt * BN_GU) * d;
            const int64_t prb = t.prow0 / 32;  // first packed row block
            bf16_t *ho = a.h + (prb * (f / 16) + nt * (BN_GU / 16)) * 512;
            if (a.gather)  // rows of x fetched through perm_src, both operands via LDS
                gemm_tile<EPI_SILU_PACKED>(a.x, d, 0, t.rows, a.w_gate + wo, a.w_up + wo, d, BN_GU,
                                           (int)d, ho, f / 16, 0, 0, lds, a.perm_src + t.row0,
                                           D.T);
            else
                gemm_tile_pa<PA_SILU_PACKED>(a.x_perm + prb * (d / 16) * 512, d / 16, t.rows,
                                             (int)d, a.w_gate + wo, a.w_up + wo, d, ho, f / 16,
                                             lds);
            publish(a.gu_done + mt, true, a.gu_xcd + mt, xcd);
            trace_tile(a, 1, L, xcd, t0);
        }

    // 3. combine tiles
    // tile = COMB_TOK tokens x up to COMB_CB column blocks of BN_DN
    const int NTB = (int)D.comb_blocks();
    const int NCG = (NT2 + COMB_CB - 1) / COMB_CB;
    const int n3 = NTB * NCG;
    bool all_done = false;
    if (n3 > 0)
        for (;;) {
            const int L = next_tile(a.queues + 2 * NUM_XCD * QSTRIDE, n3, xcd, &s_claim);
            if (L < 0) break;
            const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
            const int cg = L / NTB, tb = L % NTB;
            const int nt0 = cg * COMB_CB, ncb = min(COMB_CB, NT2 - nt0);
            // every (token, slot) of the tile waits for the down tile holding its
            // row -- unless every down tile has already been published
            if (!all_done)  // stays true once seen
                all_done = uniform(__hip_atomic_load(a.dn_done, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)) >= n2;
            for (int base = 0; !all_done && base < COMB_TOK * k; base += GEMM_THREADS) {  // uniform
                const int i = base + (int)threadIdx.x;
                const int64_t t = (int64_t)tb * COMB_TOK + i / k;
                const int64_t j = i % k;
                bool need = false;
                int32_t mt = 0;
                if (i < COMB_TOK * k && t < D.T) {
                    const int32_t p = a.inv_perm[t * k + j];
                    if (p >= 0) {
                        const int32_t e = a.ids[t * k + j] - (int32_t)D.e_lo;
                        mt = a.mtile_base[e] + (p - a.offsets[e]) / BM;
                        need = true;
                    }
                }
                for (int c = 0; c < ncb; ++c)
                    wave_wait_geq(a.dn_flag + (int64_t)mt * NT2 + nt0 + c, 1, need, a.wait_ticks,
                                  a.status);
            }
            __syncthreads();
            combine_tile_staged<OUT_F32, COMB_TOK, BN_DN / 8, GEMM_THREADS>(
                (int64_t)tb * COMB_TOK, D.T, (int64_t)nt0 * (BN_DN / 8), ncb, d, k, a.y,
                a.inv_perm, a.gates, a.out, lds);
            trace_tile(a, 3, L, xcd, t0);
        }
}

}  // namespace

int layer_grid_size() {
    static int cached = 0;
    if (cached) return cached;
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipFuncSetAttribute((const void *)layer_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS_BYTES) != hipSuccess ||
        hipFuncSetAttribute((const void *)layer_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS_BYTES) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)layer_kernel<false>,
                                                     GEMM_THREADS, GEMM_LDS_BYTES) != hipSuccess ||
        occ < 1)
        occ = 1;
    cached = cus * occ;
    return cached;
}

int64_t wall_clock_hz() {
    static int64_t cached = 0;
    if (cached) return cached;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        khz = 100000;  // 100 MHz, the documented constant rate
    cached = (int64_t)khz * 1000;
    return cached;
}

hipError_t launch_layer_persistent(const LayerArgs &a, int grid, hipStream_t s) {
    if (a.out_f32)
        hipLaunchKernelGGL(layer_kernel<true>, dim3(grid), dim3(GEMM_THREADS), GEMM_LDS_BYTES, s, a);
    else
        hipLaunchKernelGGL(layer_kernel<false>, dim3(grid), dim3(GEMM_THREADS), GEMM_LDS_BYTES, s,
                           a);
    return hipGetLastError();
}

}  // namespace moe
