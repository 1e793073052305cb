// Persistent expert-FFN + combine kernel of moe_layer.
//
// The grid is sized to the CUs that fit at once; each workgroup keeps taking
// work from device counters until every tile has been handed out, so the
// tiles of all stages share one launch and their order is a property of the
// queues rather than of kernel boundaries (the persistent scheduling of
// Weave, §4).  Three tile kinds, claimed in dependency order:
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
// GEMM tiles: the eight-wave tiles of gemm_w8.h (packed dispatch, 512
// threads) or the four-wave tiles of gemm_pa.h / gemm_tile.h (gather-on-load
// dispatch, 256 threads).  x_perm and h are in the packed layout of gemm_pa.h
// (h written by the gate/up epilogue, read as the down tiles' A operand).
//
// Interleaved order (MOE_ORDER_READY_DOWN): before each gate/up claim a
// workgroup takes the next down tile of its XCD's range if that tile's m-tile
// has all its gate/up tiles published (compare-and-swap, so only a ready
// tile is taken); such a tile never waits, so the argument below holds.
// The dependency-lead, combine-first and chunked orders replace the queues
// by a claim table that build_order_kernel writes before the launch; their
// rules sit beside that kernel.
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
//  - producers write their outputs with device-scope (write-through)
//    stores; each wave waits until its stores are performed, the workgroup
//    meets at a barrier, then one wave publishes with a relaxed agent-scope
//    RMW, so no XCD's L2 is written back.  (The gathered gate/up tile of the
//    gather-on-load dispatch writes h with ordinary stores and publishes with
//    an agent-scope release instead.)
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
#include "gemm_f8.h"
#include "gemm_f8w8.h"

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

// Schedule perturbation (a test aid for the flag protocol, off when the seed
// is 0): a pseudo-random delay, from the seed, the tile kind and the tile
// index, that a producer waits between writing its output and publishing it
// -- a quarter of the tiles wait 0 to 24 sleeps of 8128 clocks (about 100 us
// at most), far below the wait bound -- and claims taken from the far end of
// each range.  Consumers that did not wait correctly would then read
// unwritten rows.  Results are unchanged.
__device__ __forceinline__ uint32_t perturb_hash(uint32_t seed, uint32_t kind, uint32_t tile) {
    uint32_t h = seed ^ (kind * 0x9E3779B9u) ^ (tile * 0x85EBCA6Bu);
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    h *= 0x846CA68Bu;
    h ^= h >> 16;
    return h;
}
__device__ __forceinline__ int perturb_sleeps(uint32_t seed, uint32_t kind, uint32_t tile) {
    if (!seed) return 0;
    const uint32_t h = perturb_hash(seed, kind, tile);
    return (h & 3u) == 0 ? (int)((h >> 2) % 25u) : 0;
}
__device__ __forceinline__ void sleep_units(int n) {  // n wave-uniform
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
}

// Claim one tile of [0, n) for the calling wave.  Queue y covers
// [y*per, y*per + per); the own XCD's queue first, then the others.  With
// rev, each range is handed out from its far end.  The own queue is bumped
// at once (one round trip; a bump past its end is harmless, every claim
// compares the count with the range's length); the others are read first,
// so a drained range is passed over without a write.
__device__ __forceinline__ int claim_tile(int32_t *q, int n, int xcd, bool rev = false) {
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    for (int r = 0; r < NUM_XCD; ++r) {
        const int y = (xcd + r) & (NUM_XCD - 1);
        const int lo = y * per;
        const int len = min(n, lo + per) - lo;
        if (len <= 0) continue;
        int32_t *c = q + y * QSTRIDE;
        if (r > 0 &&
            uniform(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >= len)
            continue;
        // lane 0 adds 1, the others 0: lane 0's pre-op value is the claim
        const int old = uniform(__hip_atomic_fetch_add(c, lane_id() == 0 ? 1 : 0,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (old < len) return lo + (rev ? len - 1 - old : old);
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
    const int idx = lo + (a.perturb ? len - 1 - cur : cur);
    int L, part, st, mt, nt;
    dn_claim(idx, n2, nsp, S, &L, &part, &st);
    expert_tile(L, MT, NT2, (int)a.D.EL(), a.mtiles, a.mtile_base, &mt, &nt);
    if (uniform(__hip_atomic_load(a.gu_done + mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
        NT1)
        return -1;
    const int old = uniform(atomicCAS(c, cur, lane_id() == 0 ? cur + 1 : cur));
    return old == cur ? idx : -1;
}

// Claim the next entry of one global stream [0, n): a single counter, so
// the entries are handed out in stream order in time as well.
__device__ __forceinline__ int claim_in_order(int32_t *q, int n) {
    if (uniform(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >= n) return -1;
    const int old = uniform(__hip_atomic_fetch_add(q, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT));
    return old < n ? old : -1;
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
// before the barrier; then wave 0 (after the perturbation delay, if any)
// optionally records its XCD in *xmask and bumps (add) or sets (store 1) the
// counter with one agent-scope release, which writes this XCD's L2 back first.
__device__ __forceinline__ void publish(int32_t *p, bool add, int32_t *xmask, int xcd,
                                        int sleeps) {
    wait_vmcnt<0>();
    __syncthreads();
    if (wave_id() == 0) {
        sleep_units(sleeps);
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

// publish for a tile whose outputs were all written with device-scope stores
// or atomics: once every wave's writes are performed the counter is raised
// with a relaxed RMW -- no L2 write-back (which would flush every dirty line
// of the XCD's L2, other workgroups' included).
//
// With resv (a kind's queues), wave 0 also bumps this XCD's counter of that
// kind before the wait, so the next claim's round trip overlaps the drain of
// the tile's stores; returns lane 0's pre-op count in wave 0 (-1 otherwise),
// for own_slot.
__device__ __forceinline__ int publish_wt(int32_t *p, bool add, int32_t *xmask, int xcd,
                                          int sleeps, int32_t *resv = nullptr) {
    int old = -1;
    if (resv && wave_id() == 0)
        old = __hip_atomic_fetch_add(resv + xcd * QSTRIDE, lane_id() == 0 ? 1 : 0,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    __syncthreads();
    old = uniform(old);
    if (wave_id() == 0) {
        sleep_units(sleeps);
        const bool l0 = lane_id() == 0;
        if (xmask)
            __hip_atomic_fetch_or(xmask, l0 ? (1 << xcd) : 0, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        if (add)
            __hip_atomic_fetch_add(p, l0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return old;
}

// The tile of [0, n) in this XCD's range for a count taken by publish_wt's
// reservation, or -1 once that range is drained (a count past its end is
// harmless: every claim compares it with the range's length).
__device__ __forceinline__ int own_slot(int old, int n, int xcd, bool rev) {
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    const int lo = xcd * per;
    const int len = min(n, lo + per) - lo;
    if (old < 0 || len <= 0 || old >= len) return -1;
    return lo + (rev ? len - 1 - old : old);
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
template <int NT>
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
                      S, perturb_sleeps(a.perturb, 4, (uint32_t)LS)};
    const bf16_t *hA = a.h + (prb * (f / 16) + k0 / 16) * 512;
    bf16_t *yo = a.y + (int64_t)t.row0 * d + (int64_t)nt * BN_DN;
    bool wrote;
    if constexpr (NT == W8_THREADS)
        wrote = gemm_tile_w8<PA_BF16, true>(hA, f / 16, t.rows, (int)Kp, a.w_down + wo, nullptr, f,
                                            yo, d, lds, part < 0 ? nullptr : &sc);
    else
        wrote = gemm_tile_pa<PA_BF16, true>(hA, f / 16, t.rows, (int)Kp, a.w_down + wo, nullptr, f,
                                            yo, d, lds, part < 0 ? nullptr : &sc);
    if (!wrote) {  // the last part to arrive writes the tile
        trace_tile(a, 4, LS, xcd, t0);
        return;
    }
    publish_wt(a.dn_flag + (int64_t)mt * NT2 + nt, false, nullptr, xcd,
               perturb_sleeps(a.perturb, 2, (uint32_t)LS));
    // count published down tiles (y is performed before either atomic, so
    // a reader that sees the full count also sees every y row)
    if (wave_id() == 0) {
        __hip_atomic_fetch_add(a.dn_done, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(a.dn_cg + nt / COMB_CB, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    trace_tile(a, part < 0 ? 2 : 4, LS, xcd, t0);
}

// Combine-first order: the next combine tile of the first range that still
// has one, if that tile's column group has every down tile published (the
// group's count in dn_cg), claimed with a compare-and-swap as in
// claim_ready_down; -1 otherwise.  Such a tile's flag waits pass at once, so
// it never blocks.  Only the first open range is looked at: each look is a
// chain of L2 round trips paid before every down claim.
__device__ __forceinline__ int claim_ready_combine(const LayerArgs &a, int32_t *q, int n3,
                                                   int NTB, int NT2, int MT, bool rev) {
    const int per = (n3 + NUM_XCD - 1) / NUM_XCD;
    for (int y = 0; y < NUM_XCD; ++y) {
        const int lo = y * per;
        const int len = min(n3, lo + per) - lo;
        if (len <= 0) break;
        int32_t *c = q + y * QSTRIDE;
        const int cur = uniform(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (cur >= len) continue;
        const int idx = lo + (rev ? len - 1 - cur : cur);
        const int cg = idx / NTB;
        const int ncb = min(COMB_CB, NT2 - cg * COMB_CB);
        if (uniform(__hip_atomic_load(a.dn_cg + cg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
            MT * ncb)
            return -1;
        const int old = uniform(atomicCAS(c, cur, lane_id() == 0 ? cur + 1 : cur));
        return old == cur ? idx : -1;
    }
    return -1;
}

// One combine tile L (COMB_TOK tokens x up to COMB_CB column blocks of
// BN_DN): every (token, slot) waits for the down tile holding its row --
// unless every down tile has already been published -- then the gated sum.
template <bool OUT_F32, int NT>
__device__ __forceinline__ void combine_tile(const LayerArgs &a, int L, int NTB, int NT2, int n2,
                                             int xcd, bool &all_done, char *lds) {
    const Dims &D = a.D;
    const int64_t d = D.d, k = D.k;
    const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
    const int cg = L / NTB, tb = L % NTB;
    const int nt0 = cg * COMB_CB, ncb = min(COMB_CB, NT2 - nt0);
    if (!all_done)  // stays true once seen
        all_done = uniform(__hip_atomic_load(a.dn_done, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) >= n2;
    for (int base = 0; !all_done && base < COMB_TOK * k; base += NT) {  // uniform
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
    combine_tile_staged<OUT_F32, COMB_TOK, BN_DN / 8, NT>(
        (int64_t)tb * COMB_TOK, D.T, (int64_t)nt0 * (BN_DN / 8), ncb, d, k, a.y, a.inv_perm,
        a.gates, a.out, lds);
    trace_tile(a, 3, L, xcd, t0);
}

// NT = W8_THREADS: the eight-wave GEMM tiles of gemm_w8.h (packed dispatch);
// NT = GEMM_THREADS: the four-wave tiles (the gather-on-load dispatch, whose
// gate/up tile gathers x rows through LDS).
template <bool OUT_F32, int NT>
__global__ __launch_bounds__(NT, 1) void layer_kernel(LayerArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    // The claim broadcast slot.  The eight-wave tiles take all 160 KiB of LDS
    // dynamically, so there it is the last int of that: between tiles no
    // epilogue or combine tile reaches it, and a K loop starts with a barrier
    // that every wave passes only after reading the claim.
    int *s_claim_p;
    if constexpr (NT == W8_THREADS) {
        s_claim_p = reinterpret_cast<int *>(lds + W8_LDS_BYTES) - 1;
    } else {
        __shared__ int s_claim;
        s_claim_p = &s_claim;
    }
    int &s_claim = *s_claim_p;
    const Dims &D = a.D;
    const int xcd = hw_xcd();
    const int MT = *a.n_mtiles;
    const int NT1 = (int)D.nt_gu();
    const int NT2 = (int)D.nt_dn();
    const int64_t d = D.d, f = D.f;
    const bool rev = a.perturb != 0;  // claims from the far end of each range

    // down claims: those of the last partial round (of gridDim.x workgroups)
    // are cut into S K parts, claimed after the whole tiles
    const int n2 = MT * NT2;
    const int S = (int)D.dn_parts();
    const int nsp = dn_split_tiles(S, n2, (int)gridDim.x);
    const int n2c = n2 + (S - 1) * nsp;

    // combine tiles: COMB_TOK tokens x up to COMB_CB column blocks, column
    // group major (tile L covers column group L / NTB)
    const int NTB = (int)D.comb_blocks();
    const int NCG = (NT2 + COMB_CB - 1) / COMB_CB;
    const int n3 = NTB * NCG;
    int32_t *const q1 = a.queues, *const q2 = a.queues + NUM_XCD * QSTRIDE,
                   *const q3 = a.queues + 2 * NUM_XCD * QSTRIDE;
    bool all_done = false;

    // 1. gate/up tiles, 2. down tiles, 3. combine tiles, in one claim loop
    // (so each tile body is instantiated once).  Phase 1 claims gate/up tiles
    // -- with the ready-down order a ready down tile of this XCD's range first
    // (kind bit DOWN) -- phase 2, once every gate/up range is drained, the
    // down claims: with the combine-first order through the column-group-
    // sorted table, each preceded by a try for a combine tile whose column
    // group is complete (kind bit COMB) -- and phase 3 the remaining combine
    // tiles.  The dependency-lead order replaces phases 1 and 2 by phase 0:
    // the merged stream of its table, in the gate/up queues; the chunked order
    // replaces all three by phase 0 (its stream holds the combine tiles too).
    const int n1 = MT * NT1;
    constexpr int DOWN = 1 << 30, COMB = 1 << 29;
    const int nM = a.order == 2 ? n1 + n2c : a.order == 4 ? n1 + n2c + n3 : 0;
    int phase = a.order == 2 || a.order == 4 ? 0 : n1 > 0 ? 1 : 2;
    if (n1 > 0 || n2 > 0 || n3 > 0)
        for (;;) {
            if (wave_id() == 0) {
                int v;
                if (phase == 0) {
                    const int p = claim_in_order(q1, nM);  // never reversed: see build_order_kernel
                    v = p >= 0 ? uniform(a.order_tab[p]) : -1;
                } else if (phase == 1) {
                    const int r = a.order == 1 && n2 > 0
                                      ? claim_ready_down(a, q2, n2c, n2, nsp, S, MT, NT1, NT2, xcd)
                                      : -1;
                    v = r >= 0 ? (r | DOWN) : claim_tile(q1, n1, xcd, rev);
                    if (v < 0) v = -2;  // gate/up drained: move to phase 2
                } else if (phase == 2) {
                    const int c = a.order == 3 && n3 > 0
                                      ? claim_ready_combine(a, q3, n3, NTB, NT2, MT, rev)
                                      : -1;
                    if (c >= 0) {
                        v = c | COMB;
                    } else {
                        const int r = n2 > 0 ? claim_tile(q2, n2c, xcd, rev) : -1;
                        v = r < 0 ? -3 : (a.order == 3 ? uniform(a.order_tab[r]) : r) | DOWN;
                    }
                } else {
                    const int c = n3 > 0 ? claim_tile(q3, n3, xcd, rev) : -1;
                    v = c < 0 ? -1 : c | COMB;
                }
                s_claim = v;  // every lane stores the same value
            }
            __syncthreads();
            const int v = uniform(s_claim);
            __syncthreads();
            if (v == -2 || v == -3) {  // a kind drained: the next phase
                phase = v == -2 ? 2 : 3;
                continue;
            }
            if (v < 0) {
                if (phase == 0 && a.order == 2) {  // the merged stream is drained: combine tiles
                    phase = 3;
                    continue;
                }
                break;
            }
            if (v & COMB) {
                combine_tile<OUT_F32, NT>(a, v & ~COMB, NTB, NT2, n2, xcd, all_done, lds);
                continue;
            }
            if (v & DOWN) {
                down_tile<NT>(a, v & ~DOWN, n2, nsp, S, MT, NT1, NT2, xcd, lds);
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
            if constexpr (NT == W8_THREADS)
                gemm_tile_w8<PA_SILU_PACKED, true>(a.x_perm + prb * (d / 16) * 512, d / 16, t.rows,
                                                   (int)d, a.w_gate + wo, a.w_up + wo, d, ho, f / 16,
                                                   lds);
            else  // rows of x fetched through perm_src, both operands via LDS
                gemm_tile<EPI_SILU_PACKED>(a.x, d, 0, t.rows, a.w_gate + wo, a.w_up + wo, d, BN_GU,
                                           (int)d, ho, f / 16, 0, 0, lds, a.perm_src + t.row0,
                                           D.T);
            // the gathered tile writes h with ordinary stores: a release
            if (a.gather)
                publish(a.gu_done + mt, true, a.gu_xcd + mt, xcd,
                        perturb_sleeps(a.perturb, 1, (uint32_t)L));
            else
                publish_wt(a.gu_done + mt, true, a.gu_xcd + mt, xcd,
                           perturb_sleeps(a.perturb, 1, (uint32_t)L));
            trace_tile(a, 1, L, xcd, t0);
        }

}

// ---------------------------------------------------------------- W8A8
// The W8A8 layer in one persistent kernel (X-Stage, §4.3 runs the whole MoE
// block as one fused kernel and §5.3 evaluates it with W8A8): four tile
// kinds, claimed in dependency order from per-XCD queues as above --
//   1. gate/up tiles: E4M3 GEMM0 + SiLU-mul epilogue into bf16 h, with each
//      row's max |h| collected by atomic max; bump gu_done[m-tile];
//   2. quantisation tiles (m-tile, qrb row blocks of 32): once every gate/up
//      tile of the m-tile is published, the rows' power-of-two scales from
//      their maxima and their E4M3 codes in the packed layout; bump
//      q_done[m-tile];
//   3. down tiles: once all quantisation tiles of the m-tile are done, E4M3
//      GEMM1 into y; set dn_flag;
//   4. combine tiles, as in the bf16 kernel.
// Every tile computes exactly what the staged launches compute for it (the
// same tile functions and the same encoder), so the two give the same bits.
// Memory ordering: every output of a producer tile (h, its codes and
// scales, y) is written with device-scope stores, and h's row maxima with
// device-scope atomics, so a producer publishes with a relaxed RMW once its
// writes are performed, without writing its XCD's L2 back (measured: the
// write-backs cost 5-8% of the kernel); consumers acquire as in the bf16
// kernel and read the row maxima with device-coherent loads.

__device__ __forceinline__ void acquire_from(const int32_t *xmask, int xcd) {
    const int producers =
        uniform(__hip_atomic_load(xmask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (producers & ~(1 << xcd))
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    else
        invalidate_l1();
}

template <int NT>
__device__ __forceinline__ int quant_tile_f8(const LayerF8Args &a8, int Lq, int NT1, int xcd,
                                            int32_t *resv) {
    const LayerArgs &a = a8.b;
    const int64_t f = a.D.f;
    const int qpm = QB_PER_MT / a8.qrb;  // quantisation tiles per m-tile
    const int mt = Lq / qpm, rb0 = (Lq % qpm) * a8.qrb;
    const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
    if (wave_id() == 0) wave_wait_geq(a.gu_done + mt, NT1, true, a.wait_ticks, a.status);
    __syncthreads();
    acquire_from(a.gu_xcd + mt, xcd);
    const MTile t = a.mtiles[mt];
    // row blocks past the m-tile's rows belong to no segment (uniform bound)
    for (int rb = rb0; rb < rb0 + a8.qrb && rb * 32 < t.rows; ++rb) {
        const int r0 = rb * 32;
        const int lane = lane_id(), wave = wave_id();
        const int r = lane & 31;
        const bool valid = r0 + r < t.rows;  // padding rows: zero codes, scale 1
        const int64_t row = (int64_t)t.row0 + r0 + r;
        const float amax =
            valid ? __uint_as_float(__hip_atomic_load(a8.hmax + row, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT))
                  : 0.0f;
        const int e = row_scale_exp(amax);
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
        if (wave == 0 && lane < 32)
            __hip_atomic_store(a8.sh + t.prow0 + r0 + r, __uint_as_float((uint32_t)(127 + e) << 23),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u32x4_t *src =
            reinterpret_cast<const u32x4_t *>(a8.h + row * f + (lane >> 5) * 16);
        u32x4_t *o = reinterpret_cast<u32x4_t *>(a8.hq + ((int64_t)t.prow0 / 32 + rb) * (f / 32) * 1024);
        // fragments kk = wave + 4i; QB of them in flight per lane
        constexpr int QB = 4, NW = NT / 64;
        const int64_t nkk = f / 32;
        for (int64_t kk0 = wave; kk0 < nkk; kk0 += NW * QB) {
            u32x4_t raw[QB][2];
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int64_t kk = kk0 + NW * b;
                if (valid && kk < nkk) {
                    raw[b][0] = src[kk * 4];
                    raw[b][1] = src[kk * 4 + 1];
                } else {
                    raw[b][0] = raw[b][1] = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int64_t kk = kk0 + NW * b;
                if (kk < nkk) store16_wt(o + kk * 64 + lane, encode16(raw[b][0], raw[b][1], inv));
            }
        }
    }
    const int r = publish_wt(a8.q_done + mt, true, a8.q_xcd + mt, xcd,
                             perturb_sleeps(a.perturb, 5, (uint32_t)Lq), resv);
    trace_tile(a, 5, Lq, xcd, t0);
    return r;
}

__device__ __forceinline__ int down_tile_f8(const LayerF8Args &a8, int L, int MT, int NT2, int xcd,
                                            char *lds, int32_t *resv) {
    // (eight-wave tile: the W8A8 persistent kernel runs W8_THREADS threads)
    const LayerArgs &a = a8.b;
    const int64_t d = a.D.d, f = a.D.f;
    const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
    int mt, nt;
    expert_tile(L, MT, NT2, (int)a.D.EL(), a.mtiles, a.mtile_base, &mt, &nt);
    const MTile t = a.mtiles[mt];
    if (wave_id() == 0)
        wave_wait_geq(a8.q_done + mt, QB_PER_MT / a8.qrb, true, a.wait_ticks, a.status);
    __syncthreads();
    acquire_from(a8.q_xcd + mt, xcd);
    const int64_t wo = (int64_t)t.e * d + (int64_t)nt * BN_DN;
    gemm_tile_f8w8<F8_BF16, true>(a8.hq + (int64_t)(t.prow0 / 32) * (f / 32) * 1024, f / 32,
                                  t.rows, (int)f, a8.sh + t.prow0, a8.wd + wo * f, nullptr,
                                  a8.sd + wo, nullptr,
                                  a.y + (int64_t)t.row0 * d + (int64_t)nt * BN_DN, d, lds);
    const int r = publish_wt(a.dn_flag + (int64_t)mt * NT2 + nt, false, nullptr, xcd,
                             perturb_sleeps(a.perturb, 2, (uint32_t)L), resv);
    if (wave_id() == 0)  // after the flag, so a reader that sees the full count sees every y row
        __hip_atomic_fetch_add(a.dn_done, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    trace_tile(a, 2, L, xcd, t0);
    return r;
}

template <bool OUT_F32>
__global__ __launch_bounds__(W8_THREADS, 1) void layer_f8_kernel(LayerF8Args a8) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    // claim broadcast slot: the last int of the dynamic LDS, as in layer_kernel
    int &s_claim = *(reinterpret_cast<int *>(lds + W8_LDS_BYTES) - 1);
    const LayerArgs &a = a8.b;
    const Dims &D = a.D;
    const int xcd = hw_xcd();
    const int MT = *a.n_mtiles;
    const int NT1 = (int)D.nt_gu();
    const int NT2 = (int)D.nt_dn();
    const int64_t d = D.d, f = D.f;
    const bool rev = a.perturb != 0;
    const int n1 = MT * NT1, nq = MT * (QB_PER_MT / a8.qrb), n2 = MT * NT2;
    const int NTB = (int)D.comb_blocks();
    const int n3 = NTB * ((NT2 + COMB_CB - 1) / COMB_CB);
    int32_t *const q1 = a.queues, *const qq = a.queues + NUM_XCD * QSTRIDE,
                   *const q2 = a.queues + 2 * NUM_XCD * QSTRIDE,
                   *const q3 = a.queues + 3 * NUM_XCD * QSTRIDE;
    constexpr int KQ = 1 << 28, KD = 1 << 29, KC = 1 << 30;
    bool all_done = false;
    int phase = 1;  // 1 gate/up, 2 quantisation, 3 down, 4 combine
    int resv = -1;  // wave 0: count reserved on this XCD's queue of the phase by the last publish
    for (;;) {
        if (wave_id() == 0) {
            int v;
            if (phase == 1) {
                int c = own_slot(resv, n1, xcd, rev);
                if (c < 0) c = claim_tile(q1, n1, xcd, rev);
                v = c >= 0 ? c : -2;
            } else if (phase == 2) {
                int c = own_slot(resv, nq, xcd, rev);
                if (c < 0) c = claim_tile(qq, nq, xcd, rev);
                v = c >= 0 ? (c | KQ) : -2;
            } else if (phase == 3) {
                int c = own_slot(resv, n2, xcd, rev);
                if (c < 0) c = claim_tile(q2, n2, xcd, rev);
                v = c >= 0 ? (c | KD) : -2;
            } else {
                const int c = claim_tile(q3, n3, xcd, rev);
                v = c >= 0 ? (c | KC) : -1;
            }
            s_claim = v;  // every lane stores the same value
        }
        resv = -1;
        __syncthreads();
        const int v = uniform(s_claim);
        __syncthreads();
        if (v == -2) {  // this kind is drained: the next one
            ++phase;
            continue;
        }
        if (v < 0) break;
        if (v & KC) {
            combine_tile<OUT_F32, W8_THREADS>(a, v & ~KC, NTB, NT2, n2, xcd, all_done, lds);
        } else if (v & KD) {
            resv = down_tile_f8(a8, v & ~KD, MT, NT2, xcd, lds, q2);
        } else if (v & KQ) {
            resv = quant_tile_f8<W8_THREADS>(a8, v & ~KQ, NT1, xcd, qq);
        } else {
            const int64_t t0 = a.trace ? (int64_t)wall_clock64() : 0;
            int mt, nt;
            expert_tile(v, MT, NT1, (int)D.EL(), a.mtiles, a.mtile_base, &mt, &nt);
            const MTile t = a.mtiles[mt];
            const int64_t wo = (int64_t)t.e * f + (int64_t)nt * BN_GU;
            gemm_tile_f8w8<F8_SILU_ROWS, true>(a8.xq + (int64_t)(t.prow0 / 32) * (d / 32) * 1024,
                                               d / 32,
                                       t.rows, (int)d, a8.sx + t.prow0, a8.wg + wo * d,
                                       a8.wu + wo * d, a8.sg + wo, a8.su + wo,
                                       a8.h + (int64_t)t.row0 * f + (int64_t)nt * BN_GU, f, lds,
                                       a8.hmax + t.row0);
            resv = publish_wt(a.gu_done + mt, true, a.gu_xcd + mt, xcd,
                              perturb_sleeps(a.perturb, 1, (uint32_t)v), q1);
            trace_tile(a, 1, v, xcd, t0);
        }
    }
}

// Position, in the gate/up blocked order (expert_tile), of the last gate/up
// tile of m-tile mt: group [g0, g0 + s) is swept n-tile-major, so m-tile mt's
// tiles sit at g0 * NT1 + nt * s + (mt - g0).
__device__ __forceinline__ int gu_last_pos(int mt, int MT, int NT1, int EL, const MTile *mtiles,
                                           const int32_t *mtile_base) {
    const int e = mtiles[mt].e;
    const int base = mtile_base[e];
    const int end = e + 1 < EL ? mtile_base[e + 1] : MT;
    const int g0 = base + (mt - base) / GM_MAX * GM_MAX;
    const int s = min(GM_MAX, end - g0);
    return g0 * NT1 + (NT1 - 1) * s + (mt - g0);
}

// Claim tables of the tile orders that are not plain queues; one workgroup.
//
// Order 2 (dependency lead, X-Stage §4.3): gate/up tiles i (blocked order) and
// down claims LS (dn_claim order) merge into one stream, each kind keeping its
// own order, with a down claim placed as soon as at least `lead` gate/up tiles
// follow the last gate/up tile it reads: need(LS) = last(m-tile) + 1 + lead
// gate/up tiles before it (at most n1), P(LS) = the running maximum of need
// (down claims keep their order), so down claim LS lands at P(LS) + LS and
// gate/up tile i at i + #{LS : P(LS) <= i}.  Every claim's producers sit at
// earlier positions of the stream, which the persistent kernel hands out in
// order from one global counter (per-XCD ranges would let a later range run
// ahead of the producers its down tiles need, so a lead in stream positions
// would not be a lead in time); the earliest unfinished claim is therefore
// always runnable, so the stream cannot deadlock.  (That argument needs
// claims in stream order, which is why the schedule perturbation does not
// reverse this order.)
//
// Order 3 (combine first): the down claims of every per-XCD range, stably
// sorted by the combine column group of their tile (n-tile / COMB_CB), so
// each XCD finishes its share of column group 0 first; the K parts of cut
// tiles stay at the end of their range, where they fill its tail.  128
// threads per range count their run of claims per group (LDS), exclusive
// scans give every thread its slots, and a second pass places the claims.
//
// Order 4 (chunk pipeline, Weave §3.2.1): the tokens are cut into `chunks`
// equal ranges; an m-tile belongs to the chunk of its last row's token (rows
// are in token order inside an expert), a combine tile to the latest chunk of
// any m-tile its tokens' rows live in.  Every gate/up tile, down claim and
// combine tile gets the key (chunk, kind) and the stream is the stable sort by
// key: chunk by chunk, gate/up before down before combine.  A down claim's
// producers (its m-tile's gate/up tiles) and a combine tile's (the down tiles
// of its rows) have smaller keys, so they sit earlier in the stream, and the
// argument of order 2 applies.  Counting sort as in order 3, over all the
// stream's elements.
__global__ __launch_bounds__(1024) void build_order_kernel(LayerArgs a, int G) {
    // LDS of every order: order 2 a scan over the threads, order 3 per-thread
    // counts of each column group, order 4 per-thread counts of each key
    __shared__ int s_buf[1024 * 3 * ORDER4_MAX_CHUNKS];
    constexpr int K3 = ORDER3_MAX_CG + 1;  // order 3's keys: the column groups, then cut parts
    __shared__ int s_small[NUM_XCD * K3];
    const Dims &D = a.D;
    const int MT = *a.n_mtiles;
    const int NT1 = (int)D.nt_gu(), NT2 = (int)D.nt_dn(), EL = (int)D.EL();
    const int n1 = MT * NT1, n2 = MT * NT2;
    const int S = D.dn_parts();
    const int nsp = dn_split_tiles(S, n2, G);
    const int n2c = n2 + (S - 1) * nsp;
    const int tid = threadIdx.x;
    auto mt_of = [&](int LS, int *nt) {
        int L, part, st, mt;
        dn_claim(LS, n2, nsp, S, &L, &part, &st);
        expert_tile(L, MT, NT2, EL, a.mtiles, a.mtile_base, &mt, nt);
        return mt;
    };
    if (a.order == 2) {
        int *s_pre = s_buf;
        int32_t *P = a.order_tmp;
        const int q = (n2c + 1023) / 1024, lo = min(n2c, tid * q), hi = min(n2c, lo + q);
        int m = -1;
        for (int LS = lo; LS < hi; ++LS) {
            int nt;
            const int mt = mt_of(LS, &nt);
            const int need = min(n1, gu_last_pos(mt, MT, NT1, EL, a.mtiles, a.mtile_base) + 1 +
                                         a.lead);
            m = max(m, need);
            P[LS] = m;
        }
        s_pre[tid] = m;
        __syncthreads();
        for (int w = 1; w < 1024; w <<= 1) {  // inclusive max-scan over the threads
            const int o = tid >= w ? s_pre[tid - w] : -1;
            __syncthreads();
            s_pre[tid] = max(s_pre[tid], o);
            __syncthreads();
        }
        const int before = tid > 0 ? s_pre[tid - 1] : -1;
        for (int LS = lo; LS < hi; ++LS) {
            const int p = max(P[LS], before);
            P[LS] = p;
            a.order_tab[p + LS] = LS | (1 << 30);
        }
        __syncthreads();
        const int q1 = (n1 + 1023) / 1024, lo1 = min(n1, tid * q1), hi1 = min(n1, lo1 + q1);
        for (int i = lo1; i < hi1; ++i) {
            int l = 0, h = n2c;  // first LS with P(LS) > i
            while (l < h) {
                const int mid = (l + h) >> 1;
                if (P[mid] <= i) l = mid + 1;
                else h = mid;
            }
            a.order_tab[i + l] = i;
        }
    } else if (a.order == 3) {
        int(*s_cnt)[K3] = reinterpret_cast<int(*)[K3]>(s_buf);
        int(*s_start)[K3] = reinterpret_cast<int(*)[K3]>(s_small);
        const int NCG = (NT2 + COMB_CB - 1) / COMB_CB;
        const int per = (n2c + NUM_XCD - 1) / NUM_XCD;
        const int r = tid / 128, j = tid % 128;
        const int rlo = min(n2c, r * per), rhi = min(n2c, rlo + per);
        const int q = (rhi - rlo + 127) / 128, lo = min(rhi, rlo + j * q), hi = min(rhi, lo + q);
        // key: the column group of a whole tile; NCG (last) for a cut tile's part
        auto key3 = [&](int LS) {
            int L, part, st, nt;
            dn_claim(LS, n2, nsp, S, &L, &part, &st);
            if (part >= 0) return NCG;
            mt_of(LS, &nt);
            return nt / COMB_CB;
        };
        for (int c = 0; c < K3; ++c) s_cnt[tid][c] = 0;
        for (int LS = lo; LS < hi; ++LS) s_cnt[tid][key3(LS)] += 1;
        __syncthreads();
        if (j <= NCG) {  // thread (r, c = j): exclusive scan of key c over the range's threads
            int run = 0;
            for (int t = 0; t < 128; ++t) {
                const int v = s_cnt[r * 128 + t][j];
                s_cnt[r * 128 + t][j] = run;
                run += v;
            }
            s_start[r][j] = run;  // the group's total, turned into its start below
        }
        __syncthreads();
        if (j == 0) {
            int run = 0;
            for (int c = 0; c <= NCG; ++c) {
                const int v = s_start[r][c];
                s_start[r][c] = run;
                run += v;
            }
        }
        __syncthreads();
        for (int LS = lo; LS < hi; ++LS) {
            const int c = key3(LS);
            a.order_tab[rlo + s_start[r][c] + s_cnt[tid][c]++] = LS;
        }
    } else if (a.order == 4) {
        constexpr int NKMAX = 3 * ORDER4_MAX_CHUNKS;
        int(*s_cnt)[NKMAX] = reinterpret_cast<int(*)[NKMAX]>(s_buf);
        int *s_base = s_small;
        const int K = a.chunks, NK = 3 * K;
        const int64_t k = D.k;
        const int NTB = (int)D.comb_blocks(), NCG = (NT2 + COMB_CB - 1) / COMB_CB;
        const int n3 = NTB * NCG;
        auto chunk_of_mtile = [&](int m) {
            const MTile t = a.mtiles[m];
            const int64_t last = a.perm_src[t.row0 + t.rows - 1];
            return (int)min((int64_t)K - 1, (int64_t)K * last / D.T);
        };
        // the chunk of every combine token block, into order_tmp
        for (int tb = tid; tb < NTB; tb += 1024) {
            int c = 0;
            for (int64_t i = 0; i < COMB_TOK * k; ++i) {
                const int64_t t = (int64_t)tb * COMB_TOK + i / k, j = i % k;
                if (t >= D.T) break;
                const int32_t p = a.inv_perm[t * k + j];
                if (p < 0) continue;
                const int32_t e = a.ids[t * k + j] - (int32_t)D.e_lo;
                c = max(c, chunk_of_mtile(a.mtile_base[e] + (p - a.offsets[e]) / BM));
            }
            a.order_tmp[tb] = c;
        }
        __syncthreads();
        const int total = n1 + n2c + n3;
        auto key_of = [&](int x) {
            int nt;
            if (x < n1) {
                int m;
                expert_tile(x, MT, NT1, EL, a.mtiles, a.mtile_base, &m, &nt);
                return 3 * chunk_of_mtile(m);
            }
            if (x < n1 + n2c) return 3 * chunk_of_mtile(mt_of(x - n1, &nt)) + 1;
            return 3 * a.order_tmp[(x - n1 - n2c) % NTB] + 2;
        };
        const int q = (total + 1023) / 1024, lo = min(total, tid * q), hi = min(total, lo + q);
        for (int c = 0; c < NK; ++c) s_cnt[tid][c] = 0;
        for (int x = lo; x < hi; ++x) s_cnt[tid][key_of(x)] += 1;
        __syncthreads();
        if (tid < NK) {  // exclusive scan of key tid over the threads
            int run = 0;
            for (int t = 0; t < 1024; ++t) {
                const int v = s_cnt[t][tid];
                s_cnt[t][tid] = run;
                run += v;
            }
            s_base[tid] = run;
        }
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int c = 0; c < NK; ++c) {
                const int v = s_base[c];
                s_base[c] = run;
                run += v;
            }
        }
        __syncthreads();
        for (int x = lo; x < hi; ++x) {
            const int key = key_of(x);
            const int v = x < n1 ? x : x < n1 + n2c ? (x - n1) | (1 << 30) : (x - n1 - n2c) | (1 << 29);
            a.order_tab[s_base[key] + s_cnt[tid][key]++] = v;
        }
    }
}

}  // namespace

hipError_t launch_build_order(const LayerArgs &a, int grid, hipStream_t s) {
    if (a.order < 2 || a.order > 4) return hipSuccess;
    hipLaunchKernelGGL(build_order_kernel, dim3(1), dim3(1024), 0, s, a, grid);
    return hipGetLastError();
}

int layer_grid_size() {
    static int cached = 0;
    if (cached) return cached;
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    for (const void *k : {(const void *)layer_kernel<false, GEMM_THREADS>,
                          (const void *)layer_kernel<true, GEMM_THREADS>})
        if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS_BYTES) !=
            hipSuccess)
            return 0;
    for (const void *k : {(const void *)layer_kernel<false, W8_THREADS>,
                          (const void *)layer_kernel<true, W8_THREADS>,
                          (const void *)layer_f8_kernel<false>, (const void *)layer_f8_kernel<true>})
        if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, W8_LDS_BYTES) !=
            hipSuccess)
            return 0;
    // one workgroup per CU for either thread count (the LDS alone sees to it)
    int occ8 = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)layer_kernel<false, GEMM_THREADS>,
                                                     GEMM_THREADS, GEMM_LDS_BYTES) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ8, (const void *)layer_kernel<false, W8_THREADS>,
                                                     W8_THREADS, W8_LDS_BYTES) != hipSuccess ||
        occ < 1 || occ8 != occ)
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

hipError_t launch_layer_f8_persistent(const LayerF8Args &a, int grid, hipStream_t s) {
    if (a.b.out_f32)
        hipLaunchKernelGGL(layer_f8_kernel<true>, dim3(grid), dim3(W8_THREADS), W8_LDS_BYTES, s,
                           a);
    else
        hipLaunchKernelGGL(layer_f8_kernel<false>, dim3(grid), dim3(W8_THREADS), W8_LDS_BYTES, s,
                           a);
    return hipGetLastError();
}

hipError_t launch_layer_persistent(const LayerArgs &a, int grid, hipStream_t s) {
    if (a.gather) {
        if (a.out_f32)
            hipLaunchKernelGGL((layer_kernel<true, GEMM_THREADS>), dim3(grid), dim3(GEMM_THREADS),
                               GEMM_LDS_BYTES, s, a);
        else
            hipLaunchKernelGGL((layer_kernel<false, GEMM_THREADS>), dim3(grid), dim3(GEMM_THREADS),
                               GEMM_LDS_BYTES, s, a);
    } else {
        if (a.out_f32)
            hipLaunchKernelGGL((layer_kernel<true, W8_THREADS>), dim3(grid), dim3(W8_THREADS),
                               W8_LDS_BYTES, s, a);
        else
            hipLaunchKernelGGL((layer_kernel<false, W8_THREADS>), dim3(grid), dim3(W8_THREADS),
                               W8_LDS_BYTES, s, a);
    }
    return hipGetLastError();
}

}  // namespace moe
