// One output tile of the grouped expert GEMM on gfx950 bf16 MFMA with float32
// accumulation (Weave, §2.1: GEMM0 = up and gate projections, then "SiLU
// followed by element-wise multiplication", GEMM1 = down projection).
//
// Tile: BM = 256 rows (one expert's rows, clamped at the segment end) by
// BN_TILE = 256 B rows, stepping K by BK = 64 through double-buffered LDS.
// 256 threads = 4 waves in a 2x2 grid; each wave owns a 128x128 block made of
// 4x4 v_mfma_f32_32x32x16_bf16 tiles (256 float accumulators per lane).
//
// Operands are K-contiguous in memory (activations [rows][K], weights
// [out][K]), so A and B stage identically: every 16-byte chunk c of a 128-byte
// LDS row r is stored at chunk position c ^ (r & 7).  A lane's MFMA fragment is
// one 16-byte chunk (8 consecutive k) of one row; the xor spreads the 8 lanes
// that read the same chunk index of 8 consecutive rows over distinct banks.
//
// GATE_UP (GEMM0): B rows 0..127 are gate rows n0..n0+127 of expert e and rows
// 128..255 the matching up rows, so every wave holds gate and up accumulators
// for the same (row, column) and the epilogue writes h = silu(g) * u as bf16
// without touching memory in between.  Otherwise (GEMM1) the 256 B rows are
// 256 down-projection columns and the epilogue writes y as bf16.
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

// global -> registers: chunk (tid & 7) of rows (tid >> 3) + 32*i, i < 8
template <bool GATE_UP>
__device__ __forceinline__ void tile_gload(u32x4_t (&ra)[8], u32x4_t (&rb)[8], const bf16_t *gA,
                                           const bf16_t *B0, const bf16_t *B1,
                                           const int32_t (&offA)[8], const int32_t (&offB)[8],
                                           int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const u32x4_t *>(gA + offA[i] + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bf16_t *Bp = (GATE_UP && i >= 4) ? B1 : B0;
        rb[i] = *reinterpret_cast<const u32x4_t *>(Bp + offB[i] + k0);
    }
}

// registers -> one LDS stage (A tile then B tile)
__device__ __forceinline__ void tile_lstore(bf16_t *stage, int st_off, const u32x4_t (&ra)[8],
                                            const u32x4_t (&rb)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4_t *>(stage + st_off + i * 32 * BK) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4_t *>(stage + BM * BK + st_off + i * 32 * BK) = rb[i];
}

// fragments of k-step s (16 k values) for the 4 A and 4 B row blocks of a wave
__device__ __forceinline__ void tile_frags(bf16x8_t (&a)[4], bf16x8_t (&b)[4], const bf16_t *stage,
                                           const int (&arow)[4], const int (&brow)[4], int khalf,
                                           int s) {
    const bf16_t *sA = stage;
    const bf16_t *sB = stage + BM * BK;
    const int c = 2 * s + khalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t *>(sA + swz(arow[i], c));
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8_t *>(sB + swz(brow[j], c));
}

__device__ __forceinline__ void tile_mfma(f32x16_t (&acc)[4][4], const bf16x8_t (&a)[4],
                                          const bf16x8_t (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// 4 k-steps of 16 over one LDS stage; the fragments of step s+1 are read
// while the 16 MFMAs of step s run.
__device__ __forceinline__ void tile_compute(f32x16_t (&acc)[4][4], const bf16_t *stage,
                                             const int (&arow)[4], const int (&brow)[4],
                                             int khalf) {
    // sched_barrier(0) keeps the scheduler from sinking the next reads below
    // the current MFMAs (it would otherwise do so to save registers).
    bf16x8_t a0[4], b0[4], a1[4], b1[4];
    tile_frags(a0, b0, stage, arow, brow, khalf, 0);
    tile_frags(a1, b1, stage, arow, brow, khalf, 1);
    __builtin_amdgcn_sched_barrier(0);
    tile_mfma(acc, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    tile_frags(a0, b0, stage, arow, brow, khalf, 2);
    __builtin_amdgcn_sched_barrier(0);
    tile_mfma(acc, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    tile_frags(a1, b1, stage, arow, brow, khalf, 3);
    __builtin_amdgcn_sched_barrier(0);
    tile_mfma(acc, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    tile_mfma(acc, a1, b1);
}

template <bool GATE_UP>
__device__ __forceinline__ void gemm_tile(const bf16_t *__restrict__ A, int64_t lda, int64_t a_row0,
                                          int a_rows, const bf16_t *__restrict__ B0,
                                          const bf16_t *__restrict__ B1, int64_t ldb, int K,
                                          bf16_t *__restrict__ out, int64_t ldo, int64_t out_col0,
                                          bf16_t *lds) {
    // An opaque copy of the thread index: inside a persistent tile loop this
    // keeps the compiler from hoisting every lane-dependent address out of the
    // loop (which would hold them live across the accumulators and spill).
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    constexpr int STAGE = (BM + BN_TILE) * BK;  // elements per LDS stage

    const int lr0 = tid >> 3;
    const int lc = tid & 7;
    const bf16_t *gA = A + a_row0 * lda;
    int32_t offA[8], offB[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = lr0 + 32 * i;
        offA[i] = min(r, a_rows - 1) * (int32_t)lda + lc * 8;
        const int br = GATE_UP ? (r & 127) : r;
        offB[i] = br * (int32_t)ldb + lc * 8;
    }
    const int st_off = swz(lr0, lc);  // row lr0 + 32*i adds i*32*BK (same xor)

    const int l32 = lane & 31;
    const int khalf = lane >> 5;
    int arow[4], brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = wm * 128 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (GATE_UP)
            brow[j] = (j < 2 ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32) + l32;
        else
            brow[j] = wn * 128 + j * 32 + l32;
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    u32x4_t ra[8], rb[8];
    const int KT = K / BK;
    tile_gload<GATE_UP>(ra, rb, gA, B0, B1, offA, offB, 0);
    tile_lstore(lds, st_off, ra, rb);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        bf16_t *cur = lds + (kt & 1) * STAGE;
        bf16_t *nxt = lds + ((kt + 1) & 1) * STAGE;
        if (more) tile_gload<GATE_UP>(ra, rb, gA, B0, B1, offA, offB, (kt + 1) * BK);
        tile_compute(acc, cur, arow, brow, khalf);
        if (more) tile_lstore(nxt, st_off, ra, rb);
        __syncthreads();
    }

    // epilogue.  Accumulator v of lane l in a 32x32 tile sits at
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
    bf16_t *o = out + a_row0 * ldo + out_col0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (r >= a_rows) continue;
            if (GATE_UP) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float g = acc[i][j][v];
                    const float u = acc[i][j + 2][v];
                    const float h = g / (1.0f + __expf(-g)) * u;
                    o[(int64_t)r * ldo + wn * 64 + j * 32 + l32] = f2bf(h);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[(int64_t)r * ldo + wn * 128 + j * 32 + l32] = f2bf(acc[i][j][v]);
            }
        }
    }
}

}  // namespace moe
