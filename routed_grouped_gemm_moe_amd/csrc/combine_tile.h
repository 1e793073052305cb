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
            r[q] = (uint32_t)f2bf(acc[2 * q]) | ((uint32_t)f2bf(acc[2 * q + 1]) << 16);
        reinterpret_cast<u32x4_t *>(reinterpret_cast<bf16_t *>(out) + t * d)[v] = r;
    }
}

// The same sum for NV (token, vector) pairs of one thread at once: the
// indices, gates and rows of all NV pairs and SB slots are loaded before any
// is used, so NV*SB row loads are in flight; each pair's float32 sum still
// runs over j ascending with the same operations as combine_vec, so the two
// give the same bits.  Pairs with ok[n] false are skipped.
template <bool OUT_F32, bool COHERENT, int NV>
__device__ __forceinline__ void combine_vecs(const int64_t (&tt)[NV], const bool (&ok)[NV],
                                             int64_t v, int64_t d, int64_t k,
                                             const bf16_t *__restrict__ y,
                                             const int32_t *__restrict__ inv_perm,
                                             const float *__restrict__ gates,
                                             void *__restrict__ out) {
    constexpr int SB = 4;
    float acc[NV][8];
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[n][q] = 0.0f;
    for (int64_t j0 = 0; j0 < k; j0 += SB) {
        int32_t p[NV][SB];
        float w[NV][SB];
        u32x4_t yv[NV][SB];
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int64_t j = j0 + u;
                // the gate is loaded alongside the index, not after it
                const bool in = ok[n] && j < k;
                p[n][u] = in ? inv_perm[tt[n] * k + j] : -1;
                w[n][u] = in ? gates[tt[n] * k + j] : 0.0f;
            }
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                yv[n][u] = u32x4_t{0u, 0u, 0u, 0u};
                if (p[n][u] < 0) continue;
                if (COHERENT) {
                    const uint64_t *q =
                        reinterpret_cast<const uint64_t *>(y + (int64_t)p[n][u] * d) + 2 * v;
                    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const uint64_t hi =
                        __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    yv[n][u] = u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                                       (uint32_t)(hi >> 32)};
                } else {
                    yv[n][u] = reinterpret_cast<const u32x4_t *>(y + (int64_t)p[n][u] * d)[v];
                }
            }
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                if (p[n][u] < 0) continue;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[n][q] = __builtin_fmaf(w[n][u], bf16x8_elem(yv[n][u], q), acc[n][q]);
            }
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        if (!ok[n]) continue;
        const int64_t t = tt[n];
        if (OUT_F32) {
            typedef float f32x4v __attribute__((ext_vector_type(4)));
            f32x4v *o = reinterpret_cast<f32x4v *>(reinterpret_cast<float *>(out) + t * d) + 2 * v;
            o[0] = f32x4v{acc[n][0], acc[n][1], acc[n][2], acc[n][3]};
            o[1] = f32x4v{acc[n][4], acc[n][5], acc[n][6], acc[n][7]};
        } else {
            u32x4_t r;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[q] = (uint32_t)f2bf(acc[n][2 * q]) | ((uint32_t)f2bf(acc[n][2 * q + 1]) << 16);
            reinterpret_cast<u32x4_t *>(reinterpret_cast<bf16_t *>(out) + t * d)[v] = r;
        }
    }
}

}  // namespace moe
