// One 8-column vector of the combine for one token, shared by the standalone
// combine kernel and the combine tiles of the persistent layer kernel.
#pragma once

#include "moe_internal.h"

namespace moe {

// out[t, 8v .. 8v+8) = sum over slots j ascending (inv_perm >= 0) of
// gates[t,j] * y[inv_perm[t,j], 8v .. 8v+8), float32 accumulation.
// COHERENT: read y with device-coherent loads (two 8-byte agent-scope atomic
// loads), for y rows written moments ago by another XCD.
template <bool OUT_F32, bool COHERENT = false>
__device__ __forceinline__ void combine_vec(int64_t t, int64_t v, int64_t d, int64_t k,
                                            const bf16_t *__restrict__ y,
                                            const int32_t *__restrict__ inv_perm,
                                            const float *__restrict__ gates, void *__restrict__ out) {
    // Slots are taken in batches of 8: the indices, gates and rows of a batch
    // are all loaded before the first is used, so up to 8 row loads per lane
    // are in flight; the float32 sum still runs over j ascending.
    constexpr int SB = 8;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int64_t j0 = 0; j0 < k; j0 += SB) {
        int32_t p[SB];
        float w[SB];
        u32x4_t yv[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int64_t j = j0 + u;
            p[u] = j < k ? inv_perm[t * k + j] : -1;
            w[u] = p[u] >= 0 ? gates[t * k + j] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            yv[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (p[u] < 0) continue;
            if (COHERENT) {
                const uint64_t *q = reinterpret_cast<const uint64_t *>(y + (int64_t)p[u] * d) + 2 * v;
                const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t hi =
                    __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                yv[u] = u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
            } else {
                yv[u] = reinterpret_cast<const u32x4_t *>(y + (int64_t)p[u] * d)[v];
            }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            if (p[u] < 0) continue;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(w[u], bf16x8_elem(yv[u], q), acc[q]);
        }
    }
    if (OUT_F32) {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        f32x4v *o = reinterpret_cast<f32x4v *>(reinterpret_cast<float *>(out) + t * d) + 2 * v;
        o[0] = f32x4v{acc[0], acc[1], acc[2], acc[3]};
        o[1] = f32x4v{acc[4], acc[5], acc[6], acc[7]};
    } else {
        u32x4_t r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = pk_bf16(acc[2 * q], acc[2 * q + 1]);
        reinterpret_cast<u32x4_t *>(reinterpret_cast<bf16_t *>(out) + t * d)[v] = r;
    }
}

// One combine tile of the persistent kernel: NTOK tokens from t0, nblk
// blocks of NVEC 8-column vectors from vector v0, NTHR threads.  The tile's row indices and
// gates go to LDS in one coalesced pass, each token's local slots (inv_perm
// >= 0) are compacted there in slot order, and every thread then keeps the
// rows of its NTOK*NVEC/NTHR (token, vector) pairs in flight SB slots at a
// time with device-coherent loads (y rows may have been written moments ago
// on another XCD).  Sums run over the local slots in ascending j with the
// same operations as combine_vec, so both give the same bits.  LDS: 4 KiB +
// 16 * NTOK * k bytes at lds; barriers inside (uniform calls only).
template <bool OUT_F32, int NTOK, int NVEC, int NTHR>
__device__ __forceinline__ void combine_tile_staged(int64_t t0, int64_t T, int64_t v0, int nblk,
                                                    int64_t d, int64_t k,
                                                    const bf16_t *__restrict__ y,
                                                    const int32_t *__restrict__ inv_perm,
                                                    const float *__restrict__ gates,
                                                    void *__restrict__ out, char *lds) {
    constexpr int NV = NTOK * NVEC / NTHR;  // pairs per thread
    constexpr int TPASS = NTHR / NVEC;      // tokens per pass of the thread grid
    static_assert(NV * NTHR == NTOK * NVEC && NTHR % NVEC == 0, "combine tile shape");
    constexpr int SB = 4;
    int32_t *s_cnt = reinterpret_cast<int32_t *>(lds);          // [NTOK]
    int32_t *s_p = reinterpret_cast<int32_t *>(lds + 4096);     // [NTOK][k] raw
    float *s_w = reinterpret_cast<float *>(s_p + NTOK * k);     // [NTOK][k] raw
    int32_t *s_lp = reinterpret_cast<int32_t *>(s_w + NTOK * k);  // [NTOK][k] local, compacted
    float *s_lw = reinterpret_cast<float *>(s_lp + NTOK * k);
    const int tid = threadIdx.x;
    for (int64_t i = tid; i < NTOK * k; i += NTHR) {
        const int64_t t = t0 + i / k;
        const bool in = t < T;
        s_p[i] = in ? inv_perm[t0 * k + i] : -1;
        s_w[i] = in ? gates[t0 * k + i] : 0.0f;
    }
    __syncthreads();
    for (int tl = tid; tl < NTOK; tl += NTHR) {
        int c = 0;
        for (int64_t j = 0; j < k; ++j) {
            const int32_t p = s_p[tl * k + j];
            if (p >= 0) {
                s_lp[tl * k + c] = p;
                s_lw[tl * k + c] = s_w[tl * k + j];
                ++c;
            }
        }
        s_cnt[tl] = c;
    }
    __syncthreads();
    const int vl = tid % NVEC;
    int tl[NV], cnt[NV];
    int maxc = 0;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        tl[n] = tid / NVEC + n * TPASS;
        cnt[n] = s_cnt[tl[n]];
        maxc = max(maxc, cnt[n]);
    }
    for (int cb = 0; cb < nblk; ++cb) {
    const int64_t v = v0 + (int64_t)cb * NVEC + vl;
    float acc[NV][8];
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[n][q] = 0.0f;
    for (int c0 = 0; c0 < maxc; c0 += SB) {
        float w[NV][SB];
        u32x4_t yv[NV][SB];
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                yv[n][u] = u32x4_t{0u, 0u, 0u, 0u};
                w[n][u] = 0.0f;
                if (c0 + u >= cnt[n]) continue;
                const int32_t p = s_lp[tl[n] * k + c0 + u];
                w[n][u] = s_lw[tl[n] * k + c0 + u];
                const uint64_t *q = reinterpret_cast<const uint64_t *>(y + (int64_t)p * d) + 2 * v;
                const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                yv[n][u] = u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
            }
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                if (c0 + u >= cnt[n]) continue;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[n][q] = __builtin_fmaf(w[n][u], bf16x8_elem(yv[n][u], q), acc[n][q]);
            }
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int64_t t = t0 + tl[n];
        if (t >= T) continue;
        if (OUT_F32) {
            typedef float f32x4v __attribute__((ext_vector_type(4)));
            f32x4v *o = reinterpret_cast<f32x4v *>(reinterpret_cast<float *>(out) + t * d) + 2 * v;
            o[0] = f32x4v{acc[n][0], acc[n][1], acc[n][2], acc[n][3]};
            o[1] = f32x4v{acc[n][4], acc[n][5], acc[n][6], acc[n][7]};
        } else {
            u32x4_t r;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[q] = pk_bf16(acc[n][2 * q], acc[n][2 * q + 1]);
            reinterpret_cast<u32x4_t *>(reinterpret_cast<bf16_t *>(out) + t * d)[v] = r;
        }
    }
    }
}

}  // namespace moe
