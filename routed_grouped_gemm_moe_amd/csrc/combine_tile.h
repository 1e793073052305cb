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
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        const int32_t p = inv_perm[t * k + j];
        if (p < 0) continue;
        const float w = gates[t * k + j];
        u32x4_t yv;
        if (COHERENT) {
            const uint64_t *q = reinterpret_cast<const uint64_t *>(y + (int64_t)p * d) + 2 * v;
            const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            yv = u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
        } else {
            yv = reinterpret_cast<const u32x4_t *>(y + (int64_t)p * d)[v];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(w, bf16x8_elem(yv, q), acc[q]);
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

}  // namespace moe
