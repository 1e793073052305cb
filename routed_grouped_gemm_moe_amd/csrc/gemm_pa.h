// Expert-FFN GEMM tile with a packed activation operand (gfx950 bf16 MFMA,
// float32 accumulation; Weave, §2.1: GEMM0 = gate and up projections, whose
// SiLU-gated product is h; GEMM1 = down projection of h).
//
// Tile and MFMA grid as in gemm_tile.h: 256 rows x 256 B rows, 4 waves in a
// 2x2 grid, each wave 128x128 = 4x4 v_mfma_f32_32x32x16_bf16 blocks.  What
// differs is how the operands reach the matrix cores:
//
//  * A (activations) is stored packed: the 32-row x 16-k MFMA fragment
//    (row block rb, k-step kk) is 1 KiB at ((rb * K/16 + kk) * 64 + lane) * 16,
//    lane l holding row 32 rb + l % 32, k = 16 kk + 8 (l / 32) .. + 7.  A wave
//    loads a fragment with one 16-byte buffer load per lane, 1 KiB contiguous,
//    straight into VGPRs: no LDS traffic for A.  The permute writes x_perm in
//    this layout and the gate/up epilogue writes h in it.
//  * B (weights, [out][K] as given) goes global -> LDS by buffer loads with
//    the LDS-DMA bit through a 4-stage ring, BK = 64 (32 KiB per stage).  The
//    16-byte chunk c of staged row r lands at chunk c ^ ((r >> 1) & 7), so
//    the fragment reads (32 consecutive rows, one chunk) are bank-conflict
//    free and every row's 128 bytes come from one cache line.
//
// Per stage and wave: 64 MFMAs, 16 A loads, 16 B-fragment LDS reads, 8 DMA
// instructions.  They are interleaved one memory instruction per MFMA by a
// fixed slot table (below), so their issue overlaps MFMA execution instead of
// draining the MFMA pipe between groups.  A is fetched two stages ahead into a
// two-deep register ring, B three stages ahead.
//
// The k-order is that of gemm_tile.h (k-steps of 16 ascending, lane half h
// holding k 8h..8h+7 of the step), so both tiles produce bit-identical
// accumulators for the same operands.
#pragma once

#include <type_traits>

#include "gemm_tile.h"

namespace moe {

constexpr int PA_BK = 64;
constexpr int PA_NST = 4;
constexpr int PA_ROWB = PA_BK * 2;                  // 128 bytes per staged B row
constexpr int PA_STAGE = BN_TILE * PA_ROWB;         // 32 KiB
constexpr int PA_LDS_BYTES = PA_NST * PA_STAGE;     // 128 KiB
static_assert(PA_LDS_BYTES == GEMM_LDS_BYTES, "persistent kernel sizes LDS for both tiles");
// Offset bias that puts a load past every descriptor's range: the pipeline's
// tail issues its loads for stages >= K/64 with it, and they read nothing.
constexpr uint32_t PA_OOB = 0x40000000u;

// 16-byte chunk index of (row, chunk c along k) in a packed matrix with kb =
// K/16 fragments per row block.
__host__ __device__ __forceinline__ int64_t packed_chunk(int64_t row, int64_t c, int64_t kb) {
    return (((row >> 5) * kb + (c >> 1)) << 6) + (row & 31) + ((c & 1) << 5);
}

// Cache-policy operand of a buffer load: sc1 (bit 4).
constexpr int PA_CPOL_SC1 = 16;

// A 16-byte store at device scope (sc1): written through to the device's
// point of coherence rather than held dirty in this XCD's L2, so a producer
// whose outputs all go out this way publishes them without an L2 write-back
// (it waits for the stores, then raises its flag).
//
// The compiler does not look inside the asm, so the hazard a store of more
// than 64 bits has on this chip -- a VALU write to its data registers in the
// next cycle can change the data still being read -- is covered by the
// asm's own wait states (without them, y stored straight from freshly
// converted registers came out wrong now and then).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void store16_wt(void *p, const u32x4_t &v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store8_wt(void *p, const u32x2_t &v) {
    asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
#pragma clang diagnostic pop

// Memory instruction issued after MFMA k (0..15) of sub-step q (0..3):
// kind 1: B-fragment LDS read idx (of sub-step q+1; of the next stage's
// sub-step 0 when q = 3), kind 2: A load for row block idx (after that block's
// 4 MFMAs, whose A registers it overwrites), kind 3: B DMA instruction idx
// (q = 0 only), kind 4: the stage's wait + barrier (q = 3).
struct PaSlot {
    int kind, idx;
};
__host__ __device__ constexpr PaSlot pa_slot(int q, int k) {
    if ((k & 3) == 3) return {2, k >> 2};
    if (q < 3) {
        if (k < 3) return {1, k};
        if (k == 4) return {1, 3};
        if (q == 0) return {3, k == 5 ? 0 : k == 6 ? 1 : k == 8 ? 2 : k == 9 ? 3 : k == 10 ? 4 : k == 12 ? 5 : k == 13 ? 6 : 7};
        return {0, 0};
    }
    if (k == 5) return {4, 0};
    if (k == 6) return {1, 0};
    if (k >= 8 && k <= 10) return {1, k - 7};
    return {0, 0};
}

// Epilogues: h = silu(g) * u as bf16 written in the packed layout (gate/up,
// dual B), or y as bf16 rows (down).
enum { PA_SILU_PACKED = 0, PA_BF16 = 1 };

// The DMA below names M0 (the LDS-DMA destination register) as clobbered; no
// other code of these kernels keeps a value in M0.  Every LDS-DMA asm of the
// library puts one wait state between its M0 write and the load that reads
// M0, the distance this chip generation asks for and which the compiler
// cannot add to asm it does not look into.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// The K loop.  FULL: all 256 rows valid (no per-block branches, so the slot
// table's interleaving holds); otherwise row blocks past a wave's last valid
// row skip their MFMAs.
template <bool GATE_UP, bool FULL>
__device__ __forceinline__ void pa_kloop(f32x16_t (&acc)[4][4], const i32x4_t &rsA,
                                         const int (&voffA)[4], const i32x4_t &rsB,
                                         const int (&voffB)[8], uint32_t lds_base, int KT, int nblk,
                                         int wave, int wn, int lane, const char *lds) {
    const int l32 = lane & 31, half = lane >> 5;
    int boff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) boff[q] = l32 * PA_ROWB + (((2 * q + half) ^ ((l32 >> 1) & 7)) << 4);
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        brow[j] = (GATE_UP ? (j < 2 ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32)
                           : wn * 128 + j * 32) * PA_ROWB;

    // One DMA instruction (n of 8) of stage s: LDS rows wave*64 + 8n + lane/8.
    // Issued as inline asm so that the compiler's wait-count tracking does not
    // tie the B-fragment reads to it; the stage waits and barriers order it.
    auto dma = [&](int s, int n) {
        const uint32_t so = s < KT ? (uint32_t)s * PA_ROWB : PA_OOB;
        const uint32_t m = __builtin_amdgcn_readfirstlane(lds_base + (s & (PA_NST - 1)) * PA_STAGE +
                                                          wave * 8192 + n * 1024);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m), "v"(voffB[n] + so), "s"(rsB) : "memory", "m0");
    };
    auto loadA = [&](bf16x8_t &dst, int s, int q, int i) {
        const uint32_t so = s < KT ? (uint32_t)(s * 4 + q) * 1024u : PA_OOB;
        dst = __builtin_bit_cast(bf16x8_t, raw_buffer_load_v4(rsA, voffA[i] + so, 0, 0));
    };
    auto readB = [&](bf16x8_t &dst, int s, int q, int j) {
        dst = *reinterpret_cast<const bf16x8_t *>(lds + (s & (PA_NST - 1)) * PA_STAGE + boff[q] + brow[j]);
    };

    bf16x8_t a[2][4][4];  // [stage parity][sub-step][row block]
    bf16x8_t b[2][4];     // B fragments, double-buffered by sub-step
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) loadA(a[0][q][i], 0, q, i);
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int n = 0; n < 8; ++n) dma(s, n);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) loadA(a[1][q][i], 1, q, i);
    wait_vmcnt<32>();  // A(0), B(0) landed; B(1), B(2) [16] and A(1) [16] may be in flight
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) readB(b[0][j], 0, 0, j);

    // Stage s (parity P): A(s) is in a[P], B(s) is visible in LDS and b[0]
    // holds (or is receiving) B(s, sub-step 0).
    auto stage = [&](int s, auto P_) {
        constexpr int P = decltype(P_)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = k >> 2, j = k & 3;
                if (FULL || i < nblk)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[P][q][i], b[q & 1][j],
                                                                        acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                const PaSlot sl = pa_slot(q, k);
                if (sl.kind == 1) {
                    if (q < 3) readB(b[(q + 1) & 1][sl.idx], s, q + 1, sl.idx);
                    else readB(b[0][sl.idx], s + 1, 0, sl.idx);
                } else if (sl.kind == 2) {
                    loadA(a[P][q][sl.idx], s + 2, q, sl.idx);
                } else if (sl.kind == 3) {
                    dma(s + 3, sl.idx);
                } else if (sl.kind == 4) {
                    // A(s+1) and B(s+1) must have landed.  Issued after A(s+1)'s last
                    // load: B(s+3) [8], A(s+2) sub-steps 0..2 [12], A(s+2, 3) block 0 [1].
                    wait_vmcnt<21>();
                    __syncthreads();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    for (int s = 0; s < KT; s += 2) {
        stage(s, std::integral_constant<int, 0>{});
        stage(s + 1, std::integral_constant<int, 1>{});
    }
    // Drain: the tail's loads read nothing but still complete; no wave may
    // reuse the ring before every wave's reads and DMAs are done.
    wait_vmcnt<0>();
    __syncthreads();
}

#pragma clang diagnostic pop

// A down tile whose K depth is cut into nparts parts, computed by as many
// workgroups (possibly on different XCDs) in any order.  Each stores its
// float32 accumulators as partial `self` of the tile and arrives at *cnt;
// the last one forms y = bf16(((P0 + P1) + P2) + ...) from all partials in
// part order, which does not depend on the order of arrival.  *cnt starts at
// zero.
struct SplitCtl {
    int32_t *cnt;
    float *part;  // nparts x (256 x 256) floats, each in accumulator-register order
    int self;     // which part this call computes (0 .. nparts-1)
    int nparts;   // 2 or 4
    int sleeps;   // schedule perturbation: s_sleep(127) count before arriving
};

// Wave grid of a tile of NT threads: 4 waves as 2 x 2 blocks of 128 x 128,
// 8 waves as 2 x 4 blocks of 128 x 64.  Wave w's accumulator block (i, j)
// starts at row tile_row0 + 32 i, column tile_col0 + 32 j.
template <int NT>
__device__ __forceinline__ int tile_row0(int w) { return (NT == 256 ? w >> 1 : w >> 2) * 128; }
template <int NT>
__device__ __forceinline__ int tile_col0(int w) { return NT == 256 ? (w & 1) * 128 : (w & 3) * 64; }

// Float offset of accumulator vector (wave, i, j, v/4 = g) of lane `lane` in
// an NI x NJ block grid per wave: every 16-byte store or load of a wave
// covers 1 KiB contiguously.
template <int NI, int NJ>
__device__ __forceinline__ int split_slot(int wave, int i, int j, int g, int lane) {
    return ((((wave * NI + i) * NJ + j) * 4 + g) * 64 + lane) * 4;
}

// y element (row r, column c) of a 256 x 256 bf16 tile staged in LDS: rows
// of 256, 16-byte chunk index xor-ed with r & RM (7 for tiles that write one
// element per lane along a row, 31 for tiles that write four columns of 32
// consecutive rows per instruction).
template <int RM = 7>
__device__ __forceinline__ int y_stage_index(int r, int c) {
    return r * 256 + (((c >> 3) ^ (r & RM)) << 3) + (c & 7);
}

// Returns false in all but the last-arriving workgroup.  In the last, the
// bf16 tile of the part-ordered sum is left in LDS (y_stage_index layout;
// SWAP: accumulators of transposed blocks, staged with y_stage_index<31>).
// LDS must be free (the K loop ends with a barrier); the caller copies the
// tile out.  WT: the partials go out with device-scope stores, so the
// arrival needs no L2 write-back.
template <bool WT, int NT = GEMM_THREADS, int NI = 4, int NJ = 4, bool SWAP = false>
__device__ __forceinline__ bool split_reduce(f32x16_t (&acc)[NI][NJ], const SplitCtl &sp, int tid,
                                             int wave, int lane, char *lds) {
    static_assert(NT / 64 * NI * NJ * 1024 == BM * BN_DN, "the waves' blocks cover the tile");
    float *mine = sp.part + sp.self * (BM * BN_DN);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4_t v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                   acc[i][j][4 * g + 3]};
                float *dst = mine + split_slot<NI, NJ>(wave, i, j, g, lane);
                if (WT) store16_wt(dst, __builtin_bit_cast(u32x4_t, v));
                else *reinterpret_cast<f32x4_t *>(dst) = v;
            }
    // every wave's stores are performed (WT) or reached L2; one agent-scope
    // RMW counts the arrival -- a release, which writes this XCD's L2 back,
    // unless the partials were written through
    wait_vmcnt<0>();
    __syncthreads();
    int *s_x = reinterpret_cast<int *>(lds);
    if (wave == 0) {
        for (int i = 0; i < sp.sleeps; ++i) __builtin_amdgcn_s_sleep(127);
        // lane 0 adds 1, the others 0: lane 0's pre-op value is the arrival
        const int old = __builtin_amdgcn_readfirstlane(
            WT ? __hip_atomic_fetch_add(sp.cnt, lane == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT)
               : __hip_atomic_fetch_add(sp.cnt, lane == 0 ? 1 : 0, __ATOMIC_RELEASE,
                                        __HIP_MEMORY_SCOPE_AGENT));
        *s_x = old;  // every lane stores the same value
    }
    __syncthreads();
    const bool last = __builtin_amdgcn_readfirstlane(*s_x) == sp.nparts - 1;
    __syncthreads();
    if (!last) return false;
    // All partials, read with device-coherent loads: the others may come from
    // other XCDs, and this XCD's L2 may hold stale lines of the buffer.
    // Buffer loads with the sc1 cache-policy bit (agent-scope coherence in
    // gfx950's memory model) miss in that L2.  Up to 16 loads in flight.
    i32x4_t rs = make_rsrc(sp.part, (uint32_t)(sp.nparts * BM * BN_DN * sizeof(float)));
#pragma unroll
    for (int w = 0; w < 4; ++w) rs[w] = __builtin_amdgcn_readfirstlane(rs[w]);
    constexpr int PSTRIDE = BM * BN_DN * sizeof(float);  // bytes between partials
    bf16_t *st = reinterpret_cast<bf16_t *>(lds);
    auto put = [&](int idx, const float (&v)[4]) {
        const int l = idx & 63, g = (idx >> 6) & 3, j = (idx >> 8) % NJ,
                  i = ((idx >> 8) / NJ) % NI, w = idx / (NI * NJ * 256);
        if (SWAP) {  // v: four consecutive columns of one row
            const int r = tile_row0<NT>(w) + i * 32 + (l & 31);
            const int c = tile_col0<NT>(w) + j * 32 + 8 * g + 4 * (l >> 5);
            *reinterpret_cast<u32x2_t *>(st + y_stage_index<31>(r, c)) =
u32x2_t{pk_bf16_sw(v[0], v[1]), pk_bf16_sw(v[2], v[3])};
        } else {  // v: four consecutive rows of one column
            const int r = tile_row0<NT>(w) + i * 32 + 8 * g + 4 * (l >> 5);
            const int c = tile_col0<NT>(w) + j * 32 + (l & 31);
#pragma unroll
            for (int e = 0; e < 4; ++e) st[y_stage_index(r + e, c)] = f2bf(v[e]);
        }
    };
    if (sp.nparts == 2) {
        for (int it = 0; it < (BM * BN_DN / 4) / NT; it += 8) {
            i32x4_t p[8][2];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    p[u][q] = raw_buffer_load_v4(rs, ((it + u) * NT + tid) * 16 + q * PSTRIDE,
                                                 0, PA_CPOL_SC1);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = __int_as_float(p[u][0][e]) + __int_as_float(p[u][1][e]);
                put((it + u) * NT + tid, v);
            }
        }
    } else {
        for (int it = 0; it < (BM * BN_DN / 4) / NT; it += 4) {
            i32x4_t p[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    p[u][q] = raw_buffer_load_v4(rs, ((it + u) * NT + tid) * 16 + q * PSTRIDE,
                                                 0, PA_CPOL_SC1);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = ((__int_as_float(p[u][0][e]) + __int_as_float(p[u][1][e])) +
                            __int_as_float(p[u][2][e])) +
                           __int_as_float(p[u][3][e]);
                put((it + u) * NT + tid, v);
            }
        }
    }
    (void)acc;
    (void)wave;
    return true;
}

// One tile.
//   Ap     packed A at the tile's first row block and first k-step
//   a_kb   fragments per packed row block (the full K of that matrix / 16)
//   a_rows valid rows (1..256); K depth multiplied (multiple of 128)
//   B0/B1  B rows (128 each for gate/up, 256 for down), stride ldb
//   out    PA_SILU_PACKED: packed h at (first row block, first of the 8
//          k-steps this tile writes), o_kb fragments per h row block;
//          PA_BF16: y at (row 0, column 0) of the tile, row stride o_ld
//   sp     PA_BF16 only: this call computes one of sp->nparts K parts of the
//          tile (Ap and B0 point at its first k, K is the part's depth); the
//          parts meet through sp (see SplitCtl) and the last one writes y.
// Returns whether this call wrote the tile's output (false only for a part
// of a cut tile that did not arrive last).
// LDS: PA_LDS_BYTES at lds, free again when the call returns.
// WT: every output (h, y, cut-tile partials) written with device-scope
// stores (store16_wt), for a producer that publishes without an L2
// write-back.
template <int EPI, bool WT = false>
__device__ __forceinline__ bool gemm_tile_pa(const bf16_t *__restrict__ Ap, int64_t a_kb,
                                             int a_rows, int K, const bf16_t *__restrict__ B0,
                                             const bf16_t *__restrict__ B1, int64_t ldb,
                                             bf16_t *__restrict__ out, int64_t o_ld, char *lds,
                                             const SplitCtl *sp = nullptr) {
    constexpr bool GATE_UP = EPI == PA_SILU_PACKED;
    // An opaque copy of the thread index keeps lane-dependent addresses from
    // being hoisted out of a persistent tile loop (and their registers live).
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, half = lane >> 5;
    const int KT = K / PA_BK;

    const int nb_all = (a_rows + 31) >> 5;
    const uint32_t a_bytes = (uint32_t)(((int64_t)(nb_all - 1) * a_kb + K / 16) * 1024);
    i32x4_t rsA = make_rsrc(Ap, a_bytes);
#pragma unroll
    for (int w = 0; w < 4; ++w) rsA[w] = __builtin_amdgcn_readfirstlane(rsA[w]);  // wave-uniform
    int voffA[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) voffA[i] = (int)((wm * 4 + i) * a_kb * 1024) + lane * 16;
    const int nblk = __builtin_amdgcn_readfirstlane(min(max((a_rows - wm * 128 + 31) >> 5, 0), 4));

    int voffB[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int r = wave * 64 + n * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        voffB[n] = (GATE_UP ? (r & 127) : r) * (int)ldb * 2 + c * 16;
    }
    const bf16_t *Bw = (GATE_UP && wave >= 2) ? B1 : B0;
    i32x4_t rsB = make_rsrc(Bw, (uint32_t)(((GATE_UP ? 127 : 255) * ldb + K) * 2));
#pragma unroll
    for (int w = 0; w < 4; ++w) rsB[w] = __builtin_amdgcn_readfirstlane(rsB[w]);  // wave-uniform
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    __syncthreads();  // the previous user of the LDS is done with it
    if (a_rows == BM)
        pa_kloop<GATE_UP, true>(acc, rsA, voffA, rsB, voffB, lds_base, KT, 4, wave, wn, lane, lds);
    else
        pa_kloop<GATE_UP, false>(acc, rsA, voffA, rsB, voffB, lds_base, KT, nblk, wave, wn, lane, lds);

    // Epilogue through LDS (the ring is free): accumulator v of lane l sits at
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32 of its 32x32 block.
    bf16_t *st = reinterpret_cast<bf16_t *>(lds);
    if (GATE_UP) {
        // h tile: 256 rows x 128 columns as 8 row blocks x 8 packed fragments.
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wn * 64 + j * 32 + l32;
                const int fo = ((col >> 4) * 64 + 32 * ((col >> 3) & 1)) * 8 + (col & 7);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r32 = 8 * (v >> 2) + 4 * half + (v & 3);
                    const float g = acc[i][j][v];
                    const float u = acc[i][j + 2][v];
                    st[(wm * 4 + i) * 4096 + fo + r32 * 8] = f2bf(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u);
                }
            }
        __syncthreads();
        // 8 row blocks x 8 KiB, each contiguous in h; blocks past the tile's
        // last valid row belong to the next segment and are not written.
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        for (int g = tid; g < nb_all * 512; g += GEMM_THREADS) {
            const int rb = g >> 9;
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(out + rb * o_ld * 512) + (g & 511);
            if (WT) store16_wt(dst, src[g]);
            else *dst = src[g];
        }
    } else {
        // y tile: 256 rows x 256 columns, row-major in LDS with the 16-byte
        // chunk index of row r xor-ed with r & 7 (even spread of the row
        // writes of the two lane halves over the banks).
        if (sp) {
            if (!split_reduce<WT>(acc, *sp, tid, wave, lane, lds)) return false;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        st[y_stage_index(r, wn * 128 + j * 32 + l32)] = f2bf(acc[i][j][v]);
                }
        }
        __syncthreads();
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        for (int g = tid; g < a_rows * 32; g += GEMM_THREADS) {
            const int r = g >> 5, c = g & 31;
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(out + (int64_t)r * o_ld) + c;
            if (WT) store16_wt(dst, src[r * 32 + (c ^ (r & 7))]);
            else *dst = src[r * 32 + (c ^ (r & 7))];
        }
    }
    return true;
}

}  // namespace moe
