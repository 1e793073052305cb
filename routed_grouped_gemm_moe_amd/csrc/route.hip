// Router: top-k gating (Weave, §2.1: a learned gate sends each token to k
// experts; Figure 3 shows top-k routing).  One workgroup handles 16 tokens.
//
// Logit arithmetic (fixed by this library so ids are reproducible bit for
// bit): a 256-thread workgroup is 16 chunk lanes x 16 slots.  Lane c of a slot
// sums its chunk [c*d/16, (c+1)*d/16) of the hidden dimension sequentially in
// float32 (each bf16*bf16 product is exact, so the fma equals multiply-then-
// add), and the 16 chunk sums are folded with xor-shuffles 1, 2, 4, 8 -- the
// balanced pairwise tree ((s0+s1)+(s2+s3))+... -- before the bias is added.
// Selection is k rounds of a wave-wide argmax (ties to the lower expert id);
// gates are the float32 softmax over the selected logits.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT_TOK = 16;       // tokens per workgroup
constexpr int RT_THREADS = 256;  // 16 chunks x 16 slots

// TPT tokens x EPT experts of accumulators per thread.  TG = 16/TPT token
// groups, EG = 16/TG expert groups, EB = EG*EPT experts per pass.
template <int TPT, int EPT>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(
    int64_t T, int64_t d, int64_t E, int64_t k, const bf16_t *__restrict__ x,
    const bf16_t *__restrict__ w, const float *__restrict__ bias, int32_t *__restrict__ ids,
    float *__restrict__ gates, float *__restrict__ logits_out) {
    constexpr int TG = RT_TOK / TPT;
    constexpr int EG = 16 / TG;
    constexpr int EB = EG * EPT;
    extern __shared__ float s_logit[];  // [RT_TOK][E]

    const int tid = threadIdx.x;
    const int c = tid & 15;       // chunk lane
    const int slot = tid >> 4;    // 0..15
    const int tg = slot % TG;
    const int eg = slot / TG;
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;
    const int64_t dc = d / 16;

    const bf16_t *xrow[TPT];
    bool tok_ok[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        int64_t t = t0 + tg * TPT + u;
        tok_ok[u] = t < T;
        xrow[u] = x + (tok_ok[u] ? t : 0) * d + c * dc;
    }

    for (int64_t e0 = 0; e0 < E; e0 += EB) {
        float acc[TPT][EPT];
        const bf16_t *wrow[EPT];
        bool e_ok[EPT];
#pragma unroll
        for (int v = 0; v < EPT; ++v) {
            int64_t e = e0 + eg * EPT + v;
            e_ok[v] = e < E;
            wrow[v] = w + (e_ok[v] ? e : 0) * d + c * dc;
#pragma unroll
            for (int u = 0; u < TPT; ++u) acc[u][v] = 0.0f;
        }
        for (int64_t i = 0; i < dc; i += 8) {
            u32x4_t xv[TPT], wv[EPT];
#pragma unroll
            for (int u = 0; u < TPT; ++u) xv[u] = *reinterpret_cast<const u32x4_t *>(xrow[u] + i);
#pragma unroll
            for (int v = 0; v < EPT; ++v) wv[v] = *reinterpret_cast<const u32x4_t *>(wrow[v] + i);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float xf[TPT], wf[EPT];
#pragma unroll
                for (int u = 0; u < TPT; ++u) xf[u] = bf16x8_elem(xv[u], q);
#pragma unroll
                for (int v = 0; v < EPT; ++v) wf[v] = bf16x8_elem(wv[v], q);
#pragma unroll
                for (int u = 0; u < TPT; ++u)
#pragma unroll
                    for (int v = 0; v < EPT; ++v) acc[u][v] = __builtin_fmaf(xf[u], wf[v], acc[u][v]);
            }
        }
        // balanced pairwise tree over the 16 chunk lanes (low 4 lane bits)
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int u = 0; u < TPT; ++u)
#pragma unroll
                for (int v = 0; v < EPT; ++v) acc[u][v] = acc[u][v] + __shfl_xor(acc[u][v], m, 64);
        if (c == 0) {
#pragma unroll
            for (int u = 0; u < TPT; ++u)
#pragma unroll
                for (int v = 0; v < EPT; ++v)
                    if (e_ok[v]) {
                        int64_t e = e0 + eg * EPT + v;
                        float l = acc[u][v];
                        if (bias) l = l + bias[e];
                        s_logit[(tg * TPT + u) * E + e] = l;
                    }
        }
    }
    __syncthreads();

    // top-k per token: each wave takes 4 tokens
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int r = 0; r < RT_TOK / 4; ++r) {
        const int tl = wave * (RT_TOK / 4) + r;
        const int64_t t = t0 + tl;
        if (t >= T) break;
        const float *lt = s_logit + tl * E;
        if (logits_out)
            for (int64_t e = lane; e < E; e += 64) logits_out[t * E + e] = lt[e];
        // each lane owns experts lane, lane+64, ...; taken[] as a bitmask (E <= 1024)
        uint32_t taken = 0;
        float first = 0.0f, denom = 0.0f;
        // gates need all k selected logits; keep them in lane j of the wave
        float my_sel = 0.0f;
        int32_t my_id = 0;
        for (int64_t j = 0; j < k; ++j) {
            float bv = -__builtin_inff();
            int32_t bi = 0x7FFFFFFF;
            for (int r2 = 0; r2 * 64 + lane < E; ++r2) {
                if (taken & (1u << r2)) continue;
                int32_t e = r2 * 64 + lane;
                float v = lt[e];
                if (v > bv || (v == bv && e < bi)) { bv = v; bi = e; }
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                float ov = __shfl_xor(bv, m, 64);
                int32_t oi = __shfl_xor(bi, m, 64);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            if (lane == (int)j) { my_sel = bv; my_id = bi; }
            if (j == 0) first = bv;
        }
        // softmax over the k selected logits, float32, j ascending
        float ej = (lane < k) ? expf(my_sel - first) : 0.0f;
        // sequential sum over j = 0..k-1 (broadcast each term from lane j)
        for (int64_t j = 0; j < k; ++j) denom += __shfl(ej, (int)j, 64);
        if (lane < k) {
            ids[t * k + lane] = my_id;
            gates[t * k + lane] = ej / denom;
        }
    }
}

template <int TPT, int EPT>
hipError_t launch_route_t(const Dims &D, const bf16_t *x, const bf16_t *w, const float *bias,
                          int32_t *ids, float *gates, float *logits, hipStream_t s) {
    const size_t lds = (size_t)RT_TOK * D.E * sizeof(float);
    const unsigned grid = (unsigned)((D.T + RT_TOK - 1) / RT_TOK);
    if (grid == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)route_kernel<TPT, EPT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_kernel<TPT, EPT>), dim3(grid), dim3(RT_THREADS), lds, s, D.T, D.d,
                       D.E, D.k, x, w, bias, ids, gates, logits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Dims &D, const bf16_t *x, const bf16_t *w_router, const float *bias,
                        int32_t *ids, float *gates, float *logits, hipStream_t s) {
    // E <= 8: one token per thread slot, all experts in one pass.
    // E <= 16: same with 16 experts per thread.
    // Otherwise: 4 tokens x 8 experts per thread, 32 experts per pass.
    if (D.E <= 8) return launch_route_t<1, 8>(D, x, w_router, bias, ids, gates, logits, s);
    if (D.E <= 16) return launch_route_t<1, 16>(D, x, w_router, bias, ids, gates, logits, s);
    return launch_route_t<4, 8>(D, x, w_router, bias, ids, gates, logits, s);
}

}  // namespace moe
