// W8A8 expert-FFN GEMM tile for eight waves (E4M3 operands,
// v_mfma_f32_32x32x64_f8f6f4, float32 accumulation, per-row and
// per-channel power-of-two scales in the epilogue; X-Stage, §5.3 evaluates
// MegaMoE in W8A8, the GEMMs are those of Weave, §2.1).
//
// The data movement of gemm_w8.h applied to the fp8 tile of gemm_f8.h: both
// operands staged once per workgroup by LDS-DMA into the same 160 KiB ring,
// eight waves in a 2 x 4 grid of 128 x 64 reading their fragments from LDS.
// An fp8 k-step (64 bytes of K per row) fills one A slot (8 row blocks x 2
// fragments of 1 KiB), so a half-stage of the ring is one fp8 k-step and a
// B stage (128 bytes per row) two; per half-stage and wave: 8 MFMAs of 64
// cycles (4 row blocks x 2 column blocks), 12 fragment reads for the next
// k-step, 2 A DMAs (plus 4 B every second half-stage), one wait + barrier.
// The ring slots are refilled as in gemm_w8.h, so the same wait counts hold.
// Same k-order and epilogue arithmetic as gemm_tile_f8, hence the same bits.
#pragma once

#include "gemm_f8.h"
#include "gemm_w8.h"

namespace moe {

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// KS stages of 128 bytes (KH = 2 KS fp8 k-steps).  NB: this wave's row
// blocks holding valid rows; the MFMAs and A fragment reads of the others
// are left out at compile time (no branch between MFMAs), every DMA and
// barrier stays, as in gemm_w8.h.
template <bool GATE_UP, int NB>
__device__ __forceinline__ void f8w8_kloop(f32x16_t (&acc)[4][2], const i32x4_t &rsA,
                                           const int (&voffA)[2], const i32x4_t &rsB,
                                           const int (&voffB)[4], uint32_t lds_base, int KS,
                                           int wave, int lane, const char *lds) {
    const int KH = 2 * KS;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, half = lane >> 5;
    // B chunk pair of k-step t within its stage: chunks 2q + half for
    // q = 2 (t & 1) and 2 (t & 1) + 1, after the swizzle
    int boff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) boff[q] = l32 * PA_ROWB + (((2 * q + half) ^ ((l32 >> 1) & 7)) << 4);
    int brow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        brow[j] = (GATE_UP ? (j == 0 ? wn * 32 : 128 + wn * 32) : wn * 64 + j * 32) * PA_ROWB;
    const int aoff = wm * 4 * 2048 + lane * 16;

    auto dmaA = [&](int h, int n) {
        const uint32_t so = h < KH ? (uint32_t)h * 2048u : PA_OOB;
        const uint32_t m = __builtin_amdgcn_readfirstlane(lds_base + (h & (W8_A_SLOTS - 1)) * W8_A_SLOT +
                                                          (wave * 2 + n) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m), "v"(voffA[n] + so), "s"(rsA) : "memory", "m0");
    };
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

    bf16x8_t a[2][4][2];  // [k-step parity][row block][fragment of the k-step]
    bf16x8_t b[2][2][2];  // [k-step parity][column block][chunk of the k-step]
    auto dmaA2 = [&](int h) {
        dmaA(h, 0);
        dmaA(h, 1);
    };
    auto dmaB4 = [&](int s) {
#pragma unroll
        for (int n = 0; n < 4; ++n) dmaB(s, (uint32_t)s, n);
    };
    // prologue in the order of gemm_w8.h
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
    for (int j = 0; j < 2; ++j) {
        readB(b[0][j][0], 0, 0, j);
        readB(b[0][j][1], 0, 1, j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        readA(a[0][i][0], 0, i, 0);
        readA(a[0][i][1], 0, i, 1);
    }

    // Half-stage = k-step h = 2 s + P (A slot h % 4, B slot s % 3); its
    // fragments are in a[P], b[P]; those of k-step h + 1 go to a[1 - P],
    // b[1 - P] after the barrier.
    auto half_stage = [&](int s, uint32_t bs, auto P_) {
        constexpr int P = decltype(P_)::value;
        const int h = 2 * s + P;
        const uint32_t as_n = (uint32_t)(h + 1) & (W8_A_SLOTS - 1);
        const uint32_t bs_n = P ? (bs == W8_B_SLOTS - 1 ? 0u : bs + 1) : bs;
        const int qn = P ? 0 : 2;  // first chunk pair index of k-step h + 1 in its stage
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = k >> 1, j = k & 1;
            if (i < NB)
                acc[i][j] = mfma_f8(f8_join(a[P][i][0], a[P][i][1]), f8_join(b[P][j][0], b[P][j][1]),
                                    acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (k == 1) {
                // A(h + 1) and (P = 1) B(s + 1) landed: issued at the barrier
                // of half-stage h - 3 (or before), followed by those of
                // half-stages h - 2 and h - 1 [8]; this wave's reads done
                wait_vmcnt_lgkm0<8>();
                __syncthreads();
            }
            if (k >= 2 && k < 4) {
                readB(b[1 - P][k - 2][0], bs_n, qn, k - 2);
                readB(b[1 - P][k - 2][1], bs_n, qn + 1, k - 2);
            }
            if (k >= 4) {
                readA(a[1 - P][k - 4][0], as_n, k - 4, 0);
                readA(a[1 - P][k - 4][1], as_n, k - 4, 1);
            }
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
    wait_vmcnt<0>();
    __syncthreads();
}

#pragma clang diagnostic pop

// One tile; arguments as gemm_tile_f8 (gemm_f8.h); the caller runs
// W8_THREADS threads and provides W8_LDS_BYTES of LDS.
template <int EPI, bool WT = false>
__device__ __forceinline__ void gemm_tile_f8w8(const uint8_t *__restrict__ Ap, int64_t a_kb,
                                               int a_rows, int K, const float *__restrict__ sa,
                                               const uint8_t *__restrict__ B0,
                                               const uint8_t *__restrict__ B1, const float *sb0,
                                               const float *sb1, bf16_t *__restrict__ out,
                                               int64_t o_ld, char *lds, uint32_t *rowmax = nullptr) {
    constexpr bool GATE_UP = EPI == F8_SILU_ROWS;
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, half = lane >> 5;
    const int KS = K / 128;

    const int nb_all = (a_rows + 31) >> 5;
    const uint32_t a_bytes = (uint32_t)(((int64_t)(nb_all - 1) * a_kb + K / 32) * 1024);
    i32x4_t rsA = make_rsrc(Ap, a_bytes);
#pragma unroll
    for (int w = 0; w < 4; ++w) rsA[w] = __builtin_amdgcn_readfirstlane(rsA[w]);
    int voffA[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) voffA[n] = (int)((wave * a_kb + n) * 1024) + lane * 16;
    const int nblk = __builtin_amdgcn_readfirstlane(min(max((a_rows - wm * 128 + 31) >> 5, 0), 4));

    int voffB[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int r = wave * 32 + n * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        voffB[n] = (GATE_UP ? (r & 127) : r) * K + c * 16;
    }
    const uint8_t *Bw = (GATE_UP && wave >= 4) ? B1 : B0;
    i32x4_t rsB = make_rsrc(Bw, (uint32_t)((GATE_UP ? 128 : 256) * K));
#pragma unroll
    for (int w = 0; w < 4; ++w) rsB[w] = __builtin_amdgcn_readfirstlane(rsB[w]);
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
    case 4: f8w8_kloop<GATE_UP, 4>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    case 3: f8w8_kloop<GATE_UP, 3>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    case 2: f8w8_kloop<GATE_UP, 2>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    case 1: f8w8_kloop<GATE_UP, 1>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    default: f8w8_kloop<GATE_UP, 0>(acc, rsA, voffA, rsB, voffB, lds_base, KS, wave, lane, lds); break;
    }

    // Epilogue through LDS, the arithmetic of gemm_tile_f8: accumulator v of
    // lane l sits at row 8*(v/4) + 4*(l/32) + v%4, column l%32 of its block.
    bf16_t *st = reinterpret_cast<bf16_t *>(lds);
    if (GATE_UP) {
        // h tile: 256 rows x 128 columns, rows of 128 with the 16-byte chunk
        // index of row r xor-ed with r & 15; this wave holds h columns
        // 32 wn .. 32 wn + 31
        const int c = wn * 32 + l32;
        const float sg = sb0[c], su = sb1[c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                const float s_r = r < a_rows ? sa[r] : 0.0f;
                const float g = acc[i][0][v] * s_r * sg;
                const float u = acc[i][1][v] * s_r * su;
                st[r * 128 + ((((c >> 3) ^ (r & 15))) << 3) + (c & 7)] = f2bf(g / (1.0f + expf(-g)) * u);
            }
        __syncthreads();
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        for (int g = tid; g < a_rows * 16; g += W8_THREADS) {
            const int r = g >> 4, cc = g & 15;
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(out + (int64_t)r * o_ld) + cc;
            if (WT) store16_wt(dst, src[r * 16 + (cc ^ (r & 15))]);
            else *dst = src[r * 16 + (cc ^ (r & 15))];
        }
        if (rowmax && tid < a_rows) {  // one thread per row: max |h| over the tile's columns
            float m = 0.0f;
#pragma unroll
            for (int cc = 0; cc < 16; ++cc)
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(bf16x8_elem(src[tid * 16 + cc], e)));
            atomicMax(rowmax + tid, __float_as_uint(m));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                const float s_r = r < a_rows ? sa[r] : 0.0f;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int c = wn * 64 + j * 32 + l32;
                    st[y_stage_index(r, c)] = f2bf(acc[i][j][v] * s_r * sb0[c]);
                }
            }
        __syncthreads();
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        for (int g = tid; g < a_rows * 32; g += W8_THREADS) {
            const int r = g >> 5, cc = g & 31;
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(out + (int64_t)r * o_ld) + cc;
            if (WT) store16_wt(dst, src[r * 32 + (cc ^ (r & 7))]);
            else *dst = src[r * 32 + (cc ^ (r & 7))];
        }
    }
    __syncthreads();  // LDS free for the next tile
}

}  // namespace moe
