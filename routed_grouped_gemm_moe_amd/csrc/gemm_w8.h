// Expert-FFN GEMM tile for eight waves, two per SIMD (gfx950 bf16 MFMA,
// float32 accumulation; Weave, §2.1: GEMM0 = gate and up projections, whose
// SiLU-gated product is h; GEMM1 = down projection of h).
//
// Same tile, operand layouts and k-order as gemm_pa.h (256 rows x 256 B
// rows, packed activations, weights as given), hence the same bits; what
// differs is how the operands reach the matrix cores.  On this chip a CU
// moves a 1 KiB wave load into VGPRs markedly slower than it moves the same
// kilobyte into LDS by LDS-DMA, and LDS fragment reads stream fastest when
// two waves per SIMD keep them in flight.  So here:
//
//  * both operands go global -> LDS by LDS-DMA, each byte once per
//    workgroup (the 2 x 2 grid of gemm_pa.h loads every A fragment twice,
//    into two waves' VGPRs);
//  * eight waves in a 2 x 4 grid, each 128 x 64 = 4 x 2 blocks of
//    v_mfma_f32_32x32x16_bf16 (128 accumulators), read their A and B
//    fragments from LDS; while one wave of a SIMD waits, the other issues.
//
// LDS (160 KiB): A in four slots of one half-stage (k 32: 8 row blocks x 2
// fragments of 1 KiB, 16 KiB), B in three slots of one stage (k 64: 256 rows
// x 128 bytes with the XOR chunk swizzle of gemm_pa.h, 32 KiB; each staged B
// row is one whole 128-byte line).  A slot is refilled as soon as the
// barrier that ends its last reads has passed: A(h + 4) right after the
// barrier of half-stage h, B(s + 3) right after the last barrier of stage s,
// so each DMA has about three (A) or four (B) half-stages to land.
//
// The MFMAs take the weight fragment as their first operand and the
// activation fragment as their second, so each accumulator block is the
// transpose of the output block: lane l holds output row l % 32 and, in
// accumulators 4g .. 4g + 3, the four consecutive output columns
// 8g + 4 (l / 32) .. + 3.  Every output element is still the same sum of
// the same products in the same k order (only the roles of the two
// operands in the instruction change), and the epilogues stage four
// columns per 8-byte LDS write instead of one per 2-byte write.
//
// Per half-stage (two k-steps of 16) and wave: 16 MFMAs, 12 fragment reads
// (4 A + 2 B per k-step, one k-step ahead, each issued as early as its
// buffer and, after the barrier, its slot allow), 2 A DMA instructions (plus 4 B
// in every second half-stage) and one wait + barrier, placed by a fixed
// slot table.  For a gate/up tile the
// wave's two column blocks are 32 gate columns and the 32 matching up
// columns, so g and u of one h element sit in the same lane.
#pragma once

#include "gemm_pa.h"

namespace moe {

constexpr int W8_THREADS = 512;
constexpr int W8_A_SLOT = 16384;
constexpr int W8_A_SLOTS = 4;
constexpr int W8_B_SLOT = BN_TILE * PA_ROWB;  // 32 KiB
constexpr int W8_B_SLOTS = 3;
constexpr int W8_B_BASE = W8_A_SLOTS * W8_A_SLOT;
constexpr int W8_LDS_BYTES = W8_B_BASE + W8_B_SLOTS * W8_B_SLOT;  // 160 KiB
static_assert(W8_LDS_BYTES <= 160 * 1024, "one workgroup per CU");
static_assert(W8_LDS_BYTES >= BM * BN_DN * 2, "the y tile is staged in the ring");

// s_waitcnt: vector-memory count <= N and every LDS access of the wave done.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// The K loop over KS stages of 64 (KH = 2 KS half-stages).  NB: this wave's
// row blocks holding valid rows (4 in every full tile; fewer in the last,
// partly filled m-tile of an expert).  The MFMAs and A fragment reads of the
// other blocks are left out at compile time (a wave with none also skips its
// B fragment reads), so no loop carries a branch between its MFMAs; every
// wave still issues all its DMAs and passes every barrier, so waves running
// different NB stay in step.
template <bool GATE_UP, int NB>
__device__ __forceinline__ void w8_kloop(f32x16_t (&acc)[4][2], const i32x4_t &rsA,
                                         const int (&voffA)[2], const i32x4_t &rsB,
                                         const int (&voffB)[4], uint32_t lds_base, int KS,
                                         int wave, int lane, const char *lds) {
    const int KH = 2 * KS;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, half = lane >> 5;
    // B fragment (sub-step q, column block j) of a slot: rows brow[j] + l32,
    // 16-byte chunk 2q + half after the swizzle
    int boff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) boff[q] = l32 * PA_ROWB + (((2 * q + half) ^ ((l32 >> 1) & 7)) << 4);
    int brow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        brow[j] = (GATE_UP ? (j == 0 ? wn * 32 : 128 + wn * 32) : wn * 64 + j * 32) * PA_ROWB;
    // A fragment (row block wm*4 + i, k-step kk) of a slot
    const int aoff = wm * 4 * 2048 + lane * 16;

    // A DMA n of half-stage h: fragment (row block = wave, k-step 2h + n)
    auto dmaA = [&](int h, int n) {
        const uint32_t so = h < KH ? (uint32_t)h * 2048u : PA_OOB;
        const uint32_t m = __builtin_amdgcn_readfirstlane(lds_base + (h & (W8_A_SLOTS - 1)) * W8_A_SLOT +
                                                          (wave * 2 + n) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m), "v"(voffA[n] + so), "s"(rsA) : "memory", "m0");
    };
    // B DMA n of stage s into slot bs: B rows (4 wave + n) * 8 .. + 7
    auto dmaB = [&](int s, uint32_t bs, int n) {
        const uint32_t so = s < KS ? (uint32_t)s * PA_ROWB : PA_OOB;
        const uint32_t m = __builtin_amdgcn_readfirstlane(lds_base + W8_B_BASE + bs * W8_B_SLOT +
                                                          (wave * 4 + n) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m), "v"(voffB[n] + so), "s"(rsB) : "memory", "m0");
    };
    auto readA = [&](bf16x8_t &dst, uint32_t as, int i, int kk) {
        if (i >= NB) return;
        dst = *reinterpret_cast<const bf16x8_t *>(lds + as * W8_A_SLOT + aoff + i * 2048 + kk * 1024);
    };
    auto readB = [&](bf16x8_t &dst, uint32_t bs, int q, int j) {
        if (NB == 0) return;
        dst = *reinterpret_cast<const bf16x8_t *>(lds + W8_B_BASE + bs * W8_B_SLOT + boff[q] + brow[j]);
    };

    bf16x8_t a[2][4];  // [k-step parity][row block]
    bf16x8_t b[2][2];  // [k-step parity][column block]
    // Prologue: B(0) A(0) B(1) A(1) A(2) B(2) A(3), in this order, so that
    // the first barriers find the same count of younger DMAs as the steady
    // state (8).
    auto dmaA2 = [&](int h) {
        dmaA(h, 0);
        dmaA(h, 1);
    };
    auto dmaB4 = [&](int s) {
#pragma unroll
        for (int n = 0; n < 4; ++n) dmaB(s, (uint32_t)s, n);
    };
    dmaB4(0);
    dmaA2(0);
    dmaB4(1);
    dmaA2(1);
    dmaA2(2);
    dmaB4(2);
    dmaA2(3);
    wait_vmcnt_lgkm0<14>();  // B(0), A(0) landed; B(1), A(1), A(2), B(2), A(3) [14] in flight
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) readB(b[0][j], 0, 0, j);
#pragma unroll
    for (int i = 0; i < 4; ++i) readA(a[0][i], 0, i, 0);

    // Half-stage h = 2 s + P (A slot h % 4, B slot s % 3).  On entry a[0] and
    // b[0] hold (or are receiving) the fragments of its first k-step 2h.
    auto half_stage = [&](int s, uint32_t bs, auto P_) {
        constexpr int P = decltype(P_)::value;
        const int h = 2 * s + P;
        const uint32_t as = (uint32_t)h & (W8_A_SLOTS - 1);
        const uint32_t as_n = (uint32_t)(h + 1) & (W8_A_SLOTS - 1);
        const uint32_t bs_n = P ? (bs == W8_B_SLOTS - 1 ? 0u : bs + 1) : bs;  // slot of k-step 2h + 2
        // k-step 2h: MFMAs on a[0], b[0]; fragments of k-step 2h + 1 (same
        // slots, A k-step 1, B sub-step 2P + 1)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = k >> 1, j = k & 1;
            if (i < NB)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[0][j], a[0][i], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (k < 2) readB(b[1][k], bs, 2 * P + 1, k);
            if (k < 4) readA(a[1][k], as, k, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // k-step 2h + 1: MFMAs on a[1], b[1].  After two of them, the wait +
        // barrier: A(h + 1) and (P = 1) B(s + 1) must have landed.  DMAs
        // issued after the last of them: those of half-stages h - 2 and
        // h - 1, one of which issued 2 and the other 6 [8] (a half-stage with
        // P = 1 issues its B DMAs before its A DMAs).  Every LDS read of the
        // wave is done too, so once all waves pass, A slot h % 4 (and for
        // P = 1 B slot s % 3) may be refilled: A(h + 4) and B(s + 3) go out
        // here, next to the fragment reads of k-step 2h + 2 into a[0], b[0].
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = k >> 1, j = k & 1;
            if (i < NB)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[1][j], a[1][i], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (k == 1) {
                wait_vmcnt_lgkm0<8>();
                __syncthreads();
            }
            if (k == 2 || k == 3) readB(b[0][k - 2], bs_n, (2 * P + 2) & 3, k - 2);
            if (k >= 2 && k < 6) readA(a[0][k - 2], as_n, k - 2, 0);
            if (P == 1 && k >= 2 && k < 6) dmaB(s + 3, bs, k - 2);
            if (k == 6) dmaA(h + 4, 0);
            if (k == 7) dmaA(h + 4, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    uint32_t bs = 0;
    for (int s = 0; s < KS; ++s) {
        half_stage(s, bs, std::integral_constant<int, 0>{});
        half_stage(s, bs, std::integral_constant<int, 1>{});
        bs = bs == W8_B_SLOTS - 1 ? 0 : bs + 1;
    }
    // Drain: the tail's DMAs read nothing but still complete, and no wave
    // may reuse the LDS before every wave's reads and DMAs are done.
    wait_vmcnt<0>();
    __syncthreads();
}

#pragma clang diagnostic pop

// One tile; arguments, return value and WT as gemm_tile_pa (gemm_pa.h); the
// caller runs W8_THREADS threads and provides W8_LDS_BYTES of LDS.
template <int EPI, bool WT = false>
__device__ __forceinline__ bool gemm_tile_w8(const bf16_t *__restrict__ Ap, int64_t a_kb, int a_rows,
                                             int K, const bf16_t *__restrict__ B0,
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
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, half = lane >> 5;
    const int KS = K / PA_BK;

    const int nb_all = (a_rows + 31) >> 5;
    const uint32_t a_bytes = (uint32_t)(((int64_t)(nb_all - 1) * a_kb + K / 16) * 1024);
    i32x4_t rsA = make_rsrc(Ap, a_bytes);
#pragma unroll
    for (int w = 0; w < 4; ++w) rsA[w] = __builtin_amdgcn_readfirstlane(rsA[w]);  // wave-uniform
    // this wave's A DMAs: row block `wave`, k-steps 2h and 2h + 1
    int voffA[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) voffA[n] = (int)((wave * a_kb + n) * 1024) + lane * 16;
    const int nblk = __builtin_amdgcn_readfirstlane(min(max((a_rows - wm * 128 + 31) >> 5, 0), 4));

    // this wave's B DMAs: staged rows wave * 32 + 8n + lane / 8 (waves 0-3
    // stage the gate rows, 4-7 the up rows of a gate/up tile)
    int voffB[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int r = wave * 32 + n * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        voffB[n] = (GATE_UP ? (r & 127) : r) * (int)ldb * 2 + c * 16;
    }
    const bf16_t *Bw = (GATE_UP && wave >= 4) ? B1 : B0;
    i32x4_t rsB = make_rsrc(Bw, (uint32_t)(((GATE_UP ? 127 : 255) * ldb + K) * 2));
#pragma unroll
    for (int w = 0; w < 4; ++w) rsB[w] = __builtin_amdgcn_readfirstlane(rsB[w]);  // wave-uniform
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    __syncthreads();  // the previous user of the LDS is done with it
    switch (nblk) {  // wave-uniform
    case 4: w8_kloop<GATE_UP, 4>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    case 3: w8_kloop<GATE_UP, 3>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    case 2: w8_kloop<GATE_UP, 2>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    case 1: w8_kloop<GATE_UP, 1>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    default: w8_kloop<GATE_UP, 0>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    }

    // Epilogues: accumulator 4g + e of lane l sits at row l % 32, column
    // 8g + 4 (l / 32) + e of its 32x32 block.  h goes out from the registers,
    // y through LDS (the rings are free).
    bf16_t *st = reinterpret_cast<bf16_t *>(lds);
    if (GATE_UP) {
        // h tile: 256 rows x 128 columns as 8 row blocks x 8 packed fragments;
        // this wave holds h columns 32 wn .. 32 wn + 31 of 4 row blocks, four
        // consecutive columns (8 bytes of one packed 16-byte slot) at a time.
        // For one (row block, g) the wave's 64 lanes fill 32 whole slots of
        // one fragment, 512 contiguous bytes, so h goes out straight from the
        // registers.  Row blocks past the tile's last valid row belong to the
        // next segment and are not written.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nblk) break;  // wave-uniform
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = wn * 32 + 8 * g + 4 * half;
                const int fo = ((col >> 4) * 64 + 32 * ((col >> 3) & 1) + l32) * 8 + (col & 7);
                uint32_t w[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float hv[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float gv = acc[i][0][4 * g + 2 * e + q];
                        const float uv = acc[i][1][4 * g + 2 * e + q];
                        hv[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                    }
                    w[e] = pk_bf16(hv[0], hv[1]);
                }
                bf16_t *dst = out + (int64_t)(wm * 4 + i) * o_ld * 512 + fo;
                if (WT) store8_wt(dst, u32x2_t{w[0], w[1]});
                else *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{w[0], w[1]};
            }
        }
    } else {
        if (sp) {
            if (!split_reduce<WT, W8_THREADS, 4, 2, true>(acc, *sp, tid, wave, lane, lds))
                return false;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int r = wm * 128 + i * 32 + l32;
                        const int c = wn * 64 + j * 32 + 8 * g + 4 * half;
                        const uint32_t w0 = pk_bf16(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
                        const uint32_t w1 = pk_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                        *reinterpret_cast<u32x2_t *>(st + y_stage_index<31>(r, c)) = u32x2_t{w0, w1};
                    }
        }
        __syncthreads();
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        for (int g = tid; g < a_rows * 32; g += W8_THREADS) {
            const int r = g >> 5, c = g & 31;
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(out + (int64_t)r * o_ld) + c;
            if (WT) store16_wt(dst, src[r * 32 + (c ^ (r & 31))]);
            else *dst = src[r * 32 + (c ^ (r & 31))];
        }
    }
    return true;
}

}  // namespace moe
