// Matrix-core probes (measurement aids).  The accumulation probe  Runs chains of MFMA
// instructions on caller-given operands and returns their float32 results, so
// that the rounding behaviour of gfx950's matrix cores can be measured
// against exact sums on the host.  Two correctness arguments of this library
// rest on that behaviour: the error bound of the fast router (its bf16 logit
// partials) and the tolerance of the W8A8 expert FFN (its E4M3 GEMMs).
//
// Operand layout per case i (one wave per case):
//   a [n][steps][32][K]  row r of A for step s: K contiguous elements
//   b [n][steps][32][K]  row c of B^T (output column c) for step s
//   c [n][32][32] float  accumulator before the first step (row-major)
//   d [n][32][32] float  c + sum over steps s (in order) of a_s . b_s^T
// K = 16 bf16 elements (v_mfma_f32_32x32x16_bf16) or 64 E4M3 bytes
// (v_mfma_f32_32x32x64_f8f6f4).  Lane l feeds row / column l % 32; lane half
// h = l / 32 supplies k = 8h .. 8h+7 (bf16), or k = 16h .. 16h+15 and
// 32+16h .. 32+16h+15 (fp8) -- the assignment the expert GEMM tiles use; a
// dot product does not depend on it.  Accumulator element v of lane l is
// (row 8*(v/4) + 4*h + v%4, column l % 32).
#include "gemm_f8.h"

namespace moe {
namespace {

__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

__global__ __launch_bounds__(64) void probe_bf16_kernel(int steps, const bf16_t *__restrict__ a,
                                                        const bf16_t *__restrict__ b,
                                                        const float *__restrict__ c,
                                                        float *__restrict__ d) {
    const int64_t i = blockIdx.x;
    const int lane = threadIdx.x, r = lane & 31, h = lane >> 5;
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = c[i * 1024 + acc_row(v, h) * 32 + r];
    for (int s = 0; s < steps; ++s) {
        const int64_t base = ((i * steps + s) * 32 + r) * 16 + 8 * h;
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(a + base);
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(b + base);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) d[i * 1024 + acc_row(v, h) * 32 + r] = acc[v];
}

__global__ __launch_bounds__(64) void probe_f8_kernel(int steps, const uint8_t *__restrict__ a,
                                                      const uint8_t *__restrict__ b,
                                                      const float *__restrict__ c,
                                                      float *__restrict__ d) {
    const int64_t i = blockIdx.x;
    const int lane = threadIdx.x, r = lane & 31, h = lane >> 5;
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = c[i * 1024 + acc_row(v, h) * 32 + r];
    for (int s = 0; s < steps; ++s) {
        const int64_t base = ((i * steps + s) * 32 + r) * 64;
        const bf16x8_t alo = *reinterpret_cast<const bf16x8_t *>(a + base + 16 * h);
        const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t *>(a + base + 32 + 16 * h);
        const bf16x8_t blo = *reinterpret_cast<const bf16x8_t *>(b + base + 16 * h);
        const bf16x8_t bhi = *reinterpret_cast<const bf16x8_t *>(b + base + 32 + 16 * h);
        acc = mfma_f8(f8_join(alo, ahi), f8_join(blo, bhi), acc);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) d[i * 1024 + acc_row(v, h) * 32 + r] = acc[v];
}

// Matrix-core rate probe: every wave issues iters x 16 independent
// v_mfma_f32_32x32x16_bf16 (16 accumulators), operands fixed per lane --
// zero (seed 0) or pseudo-random values in [-1, 1) from the seed -- so the
// sustained rate can be compared with the nominal peak: with real data the
// chip's power limit lowers the clock.  The sums go to sink so the work
// stays live.
__global__ __launch_bounds__(256) void probe_rate_kernel(int iters, uint32_t seed,
                                                         float *__restrict__ sink) {
    const int tid = threadIdx.x;
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t h = seed * 0x9E3779B9u ^ ((uint32_t)tid * 8u + (uint32_t)j) * 0x85EBCA6Bu;
        h ^= h >> 15;
        h *= 0x2C1B3C6Du;
        h ^= h >> 12;
        const float va = seed ? (float)(h & 0xFFFF) / 32768.0f - 1.0f : 0.0f;
        const float vb = seed ? (float)(h >> 16) / 32768.0f - 1.0f : 0.0f;
        a[j] = __builtin_bit_cast(__bf16, f2bf(va));
        b[j] = __builtin_bit_cast(__bf16, f2bf(vb));
    }
    f32x16_t acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += acc[i][v];
    sink[(int64_t)blockIdx.x * 256 + tid] = sum;
}

}  // namespace

hipError_t launch_probe_mfma_rate(int64_t workgroups, int iters, uint32_t seed, float *sink,
                                  hipStream_t s) {
    if (workgroups == 0) return hipSuccess;
    hipLaunchKernelGGL(probe_rate_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, iters, seed,
                       sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int kind, int64_t n, int steps, const void *a, const void *b,
                             const float *c, float *d, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (kind == 0)
        hipLaunchKernelGGL(probe_bf16_kernel, dim3((unsigned)n), dim3(64), 0, s, steps,
                           (const bf16_t *)a, (const bf16_t *)b, c, d);
    else
        hipLaunchKernelGGL(probe_f8_kernel, dim3((unsigned)n), dim3(64), 0, s, steps,
                           (const uint8_t *)a, (const uint8_t *)b, c, d);
    return hipGetLastError();
}

}  // namespace moe
