// W8A8 expert-FFN GEMM tile: E4M3 operands on gfx950's fp8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, float32 accumulation), with one power-of-two
// scale per activation row and per weight row (output channel) applied in
// the epilogue.  X-Stage, §5.3, evaluates MegaMoE in W8A8; the GEMMs are
// those of Weave, §2.1 (GEMM0 = gate and up projections with the SiLU-gated
// product, GEMM1 = down projection).
//
// The tile moves bytes exactly as the bf16 packed tile of gemm_pa.h does: a
// 256 x 256 output tile, 4 waves of 128 x 128, A packed in 1 KiB fragments
// straight to VGPRs, B (weights, [out][K] bytes) through the 4-stage LDS-DMA
// ring with 128-byte staged rows.  A stage is 128 bytes of K per row, i.e.
// 128 fp8 values, two fp8 k-steps of 64.  The packed layout is that of
// gemm_pa.h over 16-bit units, so fragment q of a row block holds bytes
// 32q + 16h .. 32q + 16h + 15 of each row in lane half h; an fp8 k-step joins
// fragments 2kk and 2kk+1, so lane half h supplies bytes {16h..16h+15} and
// {32+16h..32+16h+15} of the 64-byte step for A, and the B fragment reads
// supply the same bytes of each weight row.  A and B use one and the same
// lane-to-k assignment, which is all a dot product needs.
//
// Issue order per k-step and wave (16 MFMAs of 64 cycles each): columns
// outer, row blocks inner, so the B registers of column block j are free
// after MFMA 4j+3 and are refilled at once for the next k-step (12 MFMAs of
// latency cover); the A registers of row block i are free after MFMA 12+i
// and are refilled for the stage two ahead; the 8 weight DMAs of the stage
// three ahead go out in the first k-step; the stage's wait and barrier sit
// after MFMA 2 of the second k-step, before its first read of the next
// stage's ring slot.
#pragma once

#include "gemm_pa.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8_t f8_join(const bf16x8_t &lo, const bf16x8_t &hi) {
    const i32x4_t a = __builtin_bit_cast(i32x4_t, lo), b = __builtin_bit_cast(i32x4_t, hi);
    return i32x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 32x32x64 E4M3 x E4M3 -> float32 (operand formats 0 = E4M3, no block scale).
__device__ __forceinline__ f32x16_t mfma_f8(const i32x8_t &a, const i32x8_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Per-row E4M3 quantisation (the rule of fp8.hip's header: scale 2^e, the
// smallest power of two with max|x| <= 448 * 2^e, codes rounded to nearest
// even), shared by the quantisation kernels and the persistent layer.
//
// E4M3 code of a finite float (bit arithmetic on the float32 encoding).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    if (a >= 0x43E00000u) return sign | 0x7Eu;  // |v| >= 448: saturate
    if (a < 0x3C800000u) {                       // |v| < 2^-6: multiples of 2^-9
        const float t = __uint_as_float(a) * 512.0f;  // exact
        return sign | (uint32_t)__builtin_rintf(t);   // 0..8 (8 is the smallest normal)
    }
    // normal: biased E4M3 exponent (a >> 23) - 120, top 3 mantissa bits, the
    // 20 bits below rounded to nearest even (a carry moves into the exponent)
    const uint32_t m = a & 0x7FFFFFu;
    uint32_t code = (((a >> 23) - 120u) << 3) | (m >> 20);
    const uint32_t rem = m & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
    return sign | code;
}

// Exponent of the row scale for a row whose largest magnitude is amax.
__device__ __forceinline__ int row_scale_exp(float amax) {
    if (amax == 0.0f) return 0;
    const uint32_t b = __float_as_uint(amax);
    const int E = (int)(b >> 23) - 127;  // amax = 1.m * 2^E (subnormal amax: clamped below)
    // 448 * 2^e = 1.75 * 2^(e+8) >= 1.m * 2^E  <=>  e >= E - 8, or E - 7 if 1.m > 1.75
    const int e = (b & 0x7FFFFFu) > 0x600000u ? E - 7 : E - 8;
    return e < -126 ? -126 : e;
}

__device__ __forceinline__ float amax8(const u32x4_t &v, float m) {
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(bf16x8_elem(v, q)));
    return m;
}

// 8 bf16 values times 2^-e -> 8 codes (two 32-bit words).
//
// The hardware conversion (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest
// even, two values per instruction) gives e4m3_code's bits on every input
// the quantisers produce -- |x * 2^-e| <= 448 by the choice of e, so its
// overflow case never arises; the GPU tests pin the quantiser against the
// oracle on every bf16 value up to 448 -- at a tenth of the instructions.
__device__ __forceinline__ uint2 encode8(const u32x4_t &v, float inv) {
    float x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = bf16x8_elem(v, q) * inv;
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// Codes of one 16-byte piece of a packed E4M3 fragment (the layout of
// gemm_pa.h over bytes): lane l of fragment kk holds row l % 32, k = 32 kk +
// 16 (l / 32) .. + 15, here taken from row (bf16, scaled by inv = 2^-e before
// encoding) or zero codes when row is null (padding rows).
__device__ __forceinline__ u32x4_t encode16(const u32x4_t &a, const u32x4_t &b, float inv) {
    const uint2 lo = encode8(a, inv), hi = encode8(b, inv);
    return u32x4_t{lo.x, lo.y, hi.x, hi.y};
}
__device__ __forceinline__ u32x4_t quant_frag(const bf16_t *row, float inv, int64_t kk, int lane) {
    if (!row) return u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(row + kk * 32 + (lane >> 5) * 16);
    return encode16(p[0], p[1], inv);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// The K loop (KT stages of 128 bytes, KT even).  FULL: all 256 rows valid;
// otherwise row blocks past a wave's last valid row skip their MFMAs.
template <bool GATE_UP, bool FULL>
__device__ __forceinline__ void f8_kloop(f32x16_t (&acc)[4][4], const i32x4_t &rsA,
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

    bf16x8_t a[2][4][4];  // [stage parity][16-byte fragment q][row block]
    bf16x8_t b[2][4];     // [fragment of the k-step][column block]
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
    for (int j = 0; j < 4; ++j) {
        readB(b[0][j], 0, 0, j);
        readB(b[1][j], 0, 1, j);
    }

    auto stage = [&](int s, auto P_) {
        constexpr int P = decltype(P_)::value;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int j = m >> 2, i = m & 3;
                if (FULL || i < nblk)
                    acc[i][j] = mfma_f8(f8_join(a[P][2 * kk][i], a[P][2 * kk + 1][i]),
                                        f8_join(b[0][j], b[1][j]), acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
                if (kk == 0 && m != 3 && m != 7 && m < 10)
                    dma(s + 3, m < 3 ? m : m < 7 ? m - 1 : m - 2);
                if (kk == 1 && m == 2) {
                    // A(s+1) and B(s+1) must have landed.  Issued since A(s+1)'s last
                    // load: B(s+3) [8] and A(s+2) fragments 0, 1 [8].
                    wait_vmcnt<16>();
                    __syncthreads();
                }
                if ((m & 3) == 3) {  // column block j is done with this k-step's B
                    if (kk == 0) {
                        readB(b[0][j], s, 2, j);
                        readB(b[1][j], s, 3, j);
                    } else {
                        readB(b[0][j], s + 1, 0, j);
                        readB(b[1][j], s + 1, 1, j);
                    }
                }
                if (m >= 12) {  // row block m - 12 is done with this k-step's A
                    loadA(a[P][2 * kk][m - 12], s + 2, 2 * kk, m - 12);
                    loadA(a[P][2 * kk + 1][m - 12], s + 2, 2 * kk + 1, m - 12);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    for (int s = 0; s < KT; s += 2) {
        stage(s, std::integral_constant<int, 0>{});
        stage(s + 1, std::integral_constant<int, 1>{});
    }
    wait_vmcnt<0>();
    __syncthreads();
}

#pragma clang diagnostic pop

enum { F8_SILU_ROWS = 0, F8_BF16 = 1 };

// One tile.
//   Ap     packed E4M3 A at the tile's first row block (a_kb fragments of
//          1 KiB per row block = K / 32); sa: scales of the tile's rows
//   a_rows valid rows (1..256); K depth in bytes (multiple of 256)
//   B0/B1  weight rows (128 gate + 128 up rows, or 256 down rows), K bytes
//          apart; sb0/sb1: their scales
//   out    F8_SILU_ROWS: h = bf16(silu(g) * u) for 128 columns, rows of o_ld
//          elements; F8_BF16: y = bf16(acc * sa * sb), 256 columns
//   rowmax F8_SILU_ROWS: per output row, the float bits of the largest |h|
//          written so far (atomic max; non-negative floats order as their
//          bits); zero before the first tile of a row
// LDS: PA_LDS_BYTES at lds, free again when the call returns.
// WT: outputs written with device-scope stores (store16_wt), for a producer
// that publishes without an L2 write-back.
template <int EPI, bool WT = false>
__device__ __forceinline__ void gemm_tile_f8(const uint8_t *__restrict__ Ap, int64_t a_kb,
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
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, half = lane >> 5;
    const int KT = K / 128;

    const int nb_all = (a_rows + 31) >> 5;
    const uint32_t a_bytes = (uint32_t)(((int64_t)(nb_all - 1) * a_kb + K / 32) * 1024);
    i32x4_t rsA = make_rsrc(Ap, a_bytes);
#pragma unroll
    for (int w = 0; w < 4; ++w) rsA[w] = __builtin_amdgcn_readfirstlane(rsA[w]);
    int voffA[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) voffA[i] = (int)((wm * 4 + i) * a_kb * 1024) + lane * 16;
    const int nblk = __builtin_amdgcn_readfirstlane(min(max((a_rows - wm * 128 + 31) >> 5, 0), 4));

    int voffB[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int r = wave * 64 + n * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        voffB[n] = (GATE_UP ? (r & 127) : r) * K + c * 16;
    }
    const uint8_t *Bw = (GATE_UP && wave >= 2) ? B1 : B0;
    i32x4_t rsB = make_rsrc(Bw, (uint32_t)((GATE_UP ? 128 : 256) * K));
#pragma unroll
    for (int w = 0; w < 4; ++w) rsB[w] = __builtin_amdgcn_readfirstlane(rsB[w]);
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
        f8_kloop<GATE_UP, true>(acc, rsA, voffA, rsB, voffB, lds_base, KT, 4, wave, wn, lane, lds);
    else
        f8_kloop<GATE_UP, false>(acc, rsA, voffA, rsB, voffB, lds_base, KT, nblk, wave, wn, lane, lds);

    // Epilogue through LDS: accumulator v of lane l sits at row
    // 8*(v/4) + 4*(l/32) + v%4, column l%32 of its 32x32 block.  Row scales
    // of padded rows (past a_rows) are never read.
    bf16_t *st = reinterpret_cast<bf16_t *>(lds);
    if (GATE_UP) {
        // h tile: 256 rows x 128 columns, rows of 128 with the 16-byte chunk
        // index of row r xor-ed with r & 15
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                const float s_r = r < a_rows ? sa[r] : 0.0f;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int c = wn * 64 + j * 32 + l32;
                    const float g = acc[i][j][v] * s_r * sb0[c];
                    const float u = acc[i][j + 2][v] * s_r * sb1[c];
                    st[r * 128 + ((((c >> 3) ^ (r & 15))) << 3) + (c & 7)] =
                        f2bf(g / (1.0f + expf(-g)) * u);
                }
            }
        __syncthreads();
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(lds);
        for (int g = tid; g < a_rows * 16; g += GEMM_THREADS) {
            const int r = g >> 4, c = g & 15;
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(out + (int64_t)r * o_ld) + c;
            if (WT) store16_wt(dst, src[r * 16 + (c ^ (r & 15))]);
            else *dst = src[r * 16 + (c ^ (r & 15))];
        }
        if (rowmax && tid < a_rows) {  // one thread per row: max |h| over the tile's columns
            float m = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(bf16x8_elem(src[tid * 16 + c], e)));
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
                for (int j = 0; j < 4; ++j) {
                    const int c = wn * 128 + j * 32 + l32;
                    st[y_stage_index(r, c)] = f2bf(acc[i][j][v] * s_r * sb0[c]);
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
    __syncthreads();  // LDS free for the next tile
}

}  // namespace moe
