// A GEMM tile with both operands staged through LDS, on gfx950 bf16 MFMA with
// float32 accumulation.  The router's logit GEMM uses it (EPI_F32); the expert
// FFN uses the packed-operand tile of gemm_pa.h, which keeps this tile's
// k-order.  Its epilogues also cover the expert GEMMs of Weave, §2.1 (GEMM0 =
// gate and up projections with the SiLU-gated product, GEMM1 = down).
//
// Tile: BM = 256 rows (one expert's rows, clamped at the segment end) by
// BN_TILE = 256 B rows.  256 threads = 4 waves in a 2x2 grid; each wave owns a
// 128x128 block made of 4x4 v_mfma_f32_32x32x16_bf16 tiles (256 float
// accumulators per lane, held in AGPRs).
//
// Staging: K advances by BK = 32 per stage through a ring of NSTAGE = 4 LDS
// stages (32 KiB each).  Operands go global -> LDS directly (buffer loads with
// the LDS-DMA bit, 16 bytes per lane), without passing through VGPRs, and the
// loads of stage s+3 are issued while stage s is multiplied, so three stages
// (~3000 MFMA cycles) of latency are covered.  Each lane of a DMA instruction
// writes 16 bytes at LDS base + 16*lane; the lane's global source is chosen so
// that the 16-byte chunk c of staged row r lands at chunk c ^ swz(r),
// swz(r) = ((r >> 1) ^ (r >> 3)) & 3, which keeps the MFMA fragment reads (32
// consecutive rows, one chunk) free of bank conflicts whether the LDS serves
// 8 or 16 lanes per cycle.  The buffer descriptors span exactly the tile's
// rows, so a stray offset reads zeros instead of faulting.
//
// Operands are K-contiguous in memory (activations [rows][K], weights
// [out][K]).  GATE_UP (GEMM0): B rows 0..127 are gate rows n0..n0+127 of
// expert e and rows 128..255 the matching up rows, so every wave holds gate
// and up accumulators for the same (row, column) and the epilogue writes
// h = silu(g) * u as bf16 without touching memory in between.  Otherwise
// (GEMM1) the 256 B rows are 256 down-projection columns and the epilogue
// writes y as bf16.
//
// The MFMA sequence (k-steps of 16 in ascending k, accumulator by
// accumulator) fixes the float32 result; the staging only changes when data
// arrive, so every schedule of tiles gives bit-identical outputs.
#pragma once

#include <type_traits>

#include "moe_internal.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// LLVM intrinsic: raw buffer load whose data go to LDS (M0 = LDS base).
__device__ void raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) void *lds,
                                    int size, int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
// LLVM intrinsic: raw buffer load of 16 bytes into VGPRs.
__device__ i32x4_t raw_buffer_load_v4(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

// Buffer descriptor over [p, p + bytes): raw (stride 0); lanes whose offset
// is out of range read zeros.
__device__ __forceinline__ i32x4_t make_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)p;
    i32x4_t r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)(uint32_t)(a >> 32);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 MFMAs of one k-step.  Row block i is skipped when it holds no valid row
// of the tile (nblk = valid 32-row blocks of this wave, wave-uniform), so a
// ragged m-tile with few rows costs a fraction of a full tile.
__device__ __forceinline__ void tile_mfma(f32x16_t (&acc)[4][4], const bf16x8_t (&a)[4],
                                          const bf16x8_t (&b)[4], int nblk) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < nblk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Blocked tile order shared by the grouped GEMM launches: m-tiles in groups of
// GM_GROUP, each group swept n-tile-major, so GM_GROUP m-tiles x a run of
// n-tiles are in flight together and share their weight and activation tiles
// in L2.  L in [0, MT*NT) -> (m-tile, n-tile).
constexpr int GM_GROUP = 4;
__host__ __device__ __forceinline__ void blocked_tile(int L, int MT, int NT, int *mt, int *nt) {
    const int g = L / (GM_GROUP * NT);
    const int r = L - g * (GM_GROUP * NT);
    const int s = min(GM_GROUP, MT - g * GM_GROUP);
    *nt = r / s;
    *mt = g * GM_GROUP + (r - *nt * s);
}

// Expert-aligned blocked order of the expert GEMMs: the m-tiles of one
// expert form groups of at most GM_MAX (16), each group swept n-tile-major, so
// the m-tiles that read the same weight tile are claimed one after another
// (and run side by side in one XCD's L2); groups never mix experts, whose
// weights differ.  L in [0, MT*NT) -> (m-tile, n-tile).  mtiles[m].e is the
// local expert of m-tile m, mtile_base[e] the first m-tile of expert e (EL
// local experts, MT m-tiles in all).  A group covers m-tiles [g0, g0 + s)
// and claims [g0*NT, (g0 + s)*NT), so L / NT names an m-tile of its group.
constexpr int GM_MAX = 16;
__host__ __device__ __forceinline__ void expert_tile(int L, int MT, int NT, int EL,
                                                     const MTile *mtiles,
                                                     const int32_t *mtile_base, int *mt,
                                                     int *nt) {
    const int m0 = L / NT;
    const int e = mtiles[m0].e;
    const int base = mtile_base[e];
    const int end = e + 1 < EL ? mtile_base[e + 1] : MT;
    const int g0 = base + (m0 - base) / GM_MAX * GM_MAX;
    const int s = min(GM_MAX, end - g0);
    const int r = L - g0 * NT;
    *nt = r / s;
    *mt = g0 + (r - *nt * s);
}

// Epilogues: h = silu(g) * u as bf16 (gate/up, dual B) in rows or in the
// packed fragment layout of gemm_pa.h, y as bf16 (down), or the raw float32
// accumulators (router logit partials; columns >= out_cols are not stored).
enum { EPI_SILU_BF16 = 0, EPI_BF16 = 1, EPI_F32 = 2, EPI_SILU_PACKED = 3 };

// A: a_rows rows from a_row0, stride lda -- or, with a_src != nullptr,
// gathered rows: row r of the tile is row a_src[r] of A, which then holds
// a_src_rows rows (the dispatch done on load, x_perm never written); B0 (and
// B1 for the dual-B tile): b_rows valid rows each, stride ldb; K columns of
// both are used.  The buffer descriptors cover exactly the bytes those rows
// and columns span.  EPI_SILU_PACKED: out is the packed h at the tile's first
// row block and first of its 8 k-steps, ldo its fragments per row block.
template <int EPI>
__device__ __forceinline__ void gemm_tile(const bf16_t *__restrict__ A, int64_t lda, int64_t a_row0,
                                          int a_rows, const bf16_t *__restrict__ B0,
                                          const bf16_t *__restrict__ B1, int64_t ldb, int b_rows,
                                          int K, void *__restrict__ out, int64_t ldo,
                                          int64_t out_col0, int out_cols, char *lds,
                                          const int32_t *__restrict__ a_src = nullptr,
                                          int64_t a_src_rows = 0) {
    constexpr bool GATE_UP = EPI == EPI_SILU_BF16 || EPI == EPI_SILU_PACKED;
    // An opaque copy of the thread index: inside a persistent tile loop this
    // keeps the compiler from hoisting every lane-dependent address out of the
    // loop (which would hold them live across the accumulators and spill).
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1;
    const int wn = wave & 1;

    // DMA sources: instruction i of this wave stages rows (wave*4 + i)*16 +
    // lane/4, physical chunk lane%4 of each.
    const int pc = lane & 3;
    int voffA[4], voffB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 16 + (lane >> 2);
        const int c = pc ^ swz(r);
        const int ar = min(r, a_rows - 1);
        voffA[i] = (a_src ? a_src[ar] : ar) * (int)lda * 2 + c * 16;
        const int br = GATE_UP ? (r & 127) : r;
        voffB[i] = min(br, b_rows - 1) * (int)ldb * 2 + c * 16;
    }
    const i32x4_t rsA =
        a_src ? make_rsrc(A, (uint32_t)(((a_src_rows - 1) * lda + K) * 2))
              : make_rsrc(A + a_row0 * lda, (uint32_t)(((int64_t)(a_rows - 1) * lda + K) * 2));
    const bf16_t *Bw = (GATE_UP && wave >= 2) ? B1 : B0;  // waves 2,3 stage the up rows
    const i32x4_t rsB = make_rsrc(Bw, (uint32_t)(((int64_t)(b_rows - 1) * ldb + K) * 2));
    const int ldsA_w = wave * 4 * 1024;
    const int ldsB_w = STAGE_A_BYTES + wave * 4 * 1024;

    auto issue = [&](int s) {
        const int kb = s * BK * 2;  // byte offset along K
        char *st = lds + (s & (NSTAGE - 1)) * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            raw_buffer_load_lds(
                rsA, (__attribute__((address_space(3))) void *)(uintptr_t)(st + ldsA_w + i * 1024),
                16, voffA[i], kb, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            raw_buffer_load_lds(
                rsB, (__attribute__((address_space(3))) void *)(uintptr_t)(st + ldsB_w + i * 1024),
                16, voffB[i], kb, 0, 0);
    };

    // Fragment of a 32x32x16 MFMA: lane l reads row l%32 of its 32-row block,
    // logical chunk 2*kstep + l/32.  swz(blk*32 + l%32) == swz(l%32).
    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    const int sw = swz(l32);
    const int fo0 = l32 * STAGE_ROW_BYTES + (((0 + khalf) ^ sw) << 4);
    const int fo1 = l32 * STAGE_ROW_BYTES + (((2 + khalf) ^ sw) << 4);
    int arow[4], brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = (wm * 128 + i * 32) * STAGE_ROW_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (GATE_UP)
            brow[j] = STAGE_A_BYTES +
                      (j < 2 ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32) * STAGE_ROW_BYTES;
        else
            brow[j] = STAGE_A_BYTES + (wn * 128 + j * 32) * STAGE_ROW_BYTES;
    }
    auto frags = [&](bf16x8_t (&a)[4], bf16x8_t (&b)[4], int s, int fo) {
        const char *st = lds + (s & (NSTAGE - 1)) * STAGE_BYTES + fo;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t *>(st + arow[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8_t *>(st + brow[j]);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // valid 32-row blocks of this wave (wave-uniform)
    const int nblk = __builtin_amdgcn_readfirstlane(max(0, min(4, (a_rows - wm * 128 + 31) >> 5)));

    // Pipeline.  Stage s lives in LDS slot s % 4.  Before stage s+1 is read,
    // each wave waits for its own DMA of that stage (the later stage may stay
    // in flight) and the barrier publishes every wave's part; the same barrier
    // certifies that all waves are done with slot (s-1) % 4, which the DMA of
    // stage s+3 then overwrites.  The last three steps are peeled so the loop
    // body has no branch: at a join of paths with different outstanding LDS
    // reads the compiler would wait for the prefetched fragments before the
    // second k-step's MFMAs instead of letting them overlap.
    const int KT = K / BK;  // >= 4 for every supported shape (K % 128 == 0)
    issue(0);
    issue(1);
    issue(2);
    wait_vmcnt<16>();
    __syncthreads();
    bf16x8_t a0[4], b0[4], a1[4], b1[4];
    frags(a0, b0, 0, fo0);
    auto step = [&](int s, auto wait_all, auto do_issue, auto has_next) {
        frags(a1, b1, s, fo1);
        __builtin_amdgcn_sched_barrier(0);
        tile_mfma(acc, a0, b0, nblk);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(has_next)::value) {
            if constexpr (decltype(wait_all)::value)
                wait_vmcnt<0>();
            else
                wait_vmcnt<8>();
            __syncthreads();
            if constexpr (decltype(do_issue)::value) issue(s + 3);
            frags(a0, b0, s + 1, fo0);
        }
        __builtin_amdgcn_sched_barrier(0);
        tile_mfma(acc, a1, b1, nblk);
        __builtin_amdgcn_sched_barrier(0);
    };
    using yes = std::true_type;
    using no = std::false_type;
    for (int s = 0; s < KT - 3; ++s) step(s, no{}, yes{}, yes{});
    step(KT - 3, no{}, no{}, yes{});
    step(KT - 2, yes{}, no{}, yes{});
    step(KT - 1, yes{}, no{}, no{});

    // Epilogue.  Accumulator v of lane l in a 32x32 tile sits at
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
    if (EPI == EPI_SILU_PACKED) {
        // h tile (256 rows x 128 columns) staged in LDS as 8 row blocks x 8
        // packed fragments, then copied out as 8 KiB contiguous runs; blocks
        // past the tile's last valid row belong to the next segment.
        __syncthreads();  // every wave is done reading the ring
        bf16_t *st = reinterpret_cast<bf16_t *>(lds);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wn * 64 + j * 32 + l32;
                const int fo = ((col >> 4) * 64 + 32 * ((col >> 3) & 1)) * 8 + (col & 7);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r32 = 8 * (v >> 2) + 4 * khalf + (v & 3);
                    const float g = acc[i][j][v];
                    const float u = acc[i][j + 2][v];
                    st[(wm * 4 + i) * 4096 + fo + r32 * 8] = f2bf(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u);
                }
            }
        __syncthreads();
        const int nb_all = (a_rows + 31) >> 5;
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        bf16_t *o = reinterpret_cast<bf16_t *>(out);
        for (int g = tid; g < nb_all * 512; g += GEMM_THREADS) {
            const int rb = g >> 9;
            reinterpret_cast<u32x4_t *>(o + rb * ldo * 512)[g & 511] = src[g];
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (r >= a_rows) continue;
            const int64_t orow = (a_row0 + r) * ldo + out_col0;
            if (EPI == EPI_SILU_BF16) {
                bf16_t *o = reinterpret_cast<bf16_t *>(out) + orow;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float g = acc[i][j][v];
                    const float u = acc[i][j + 2][v];
                    const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
                    o[wn * 64 + j * 32 + l32] = f2bf(h);
                }
            } else if (EPI == EPI_BF16) {
                bf16_t *o = reinterpret_cast<bf16_t *>(out) + orow;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[wn * 128 + j * 32 + l32] = f2bf(acc[i][j][v]);
            } else {
                float *o = reinterpret_cast<float *>(out) + orow;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = wn * 128 + j * 32 + l32;
                    if (col < out_cols) o[col] = acc[i][j][v];
                }
            }
        }
    }
}

}  // namespace moe
