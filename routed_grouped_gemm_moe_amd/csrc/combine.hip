// Combine: the gate-weighted sum of each token's expert outputs, back in
// token order (Weave, §2.1 stage 5: the gate-weighted sum).  A gather in slot
// order rather than a scatter, so every output element is written once and the
// result is deterministic: out[t] = sum_j gate[t,j] * y[inv_perm[t,j]] in
// float32, j ascending, slots with inv_perm < 0 skipped.
#include "combine_tile.h"

namespace moe {
namespace {

constexpr int CB_TOK = 4;  // tokens per workgroup
constexpr int CB_THREADS = 256;

template <bool OUT_F32>
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(int64_t T, int64_t d, int64_t k,
                                                             const bf16_t *__restrict__ y,
                                                             const int32_t *__restrict__ inv_perm,
                                                             const float *__restrict__ gates,
                                                             void *__restrict__ out) {
    const int64_t nv = d / 8;
    for (int u = 0; u < CB_TOK; ++u) {
        const int64_t t = (int64_t)blockIdx.x * CB_TOK + u;
        if (t >= T) return;
        for (int64_t v = threadIdx.x; v < nv; v += CB_THREADS)
            combine_vec<OUT_F32>(t, v, d, k, y, inv_perm, gates, out);
    }
}

}  // namespace

hipError_t launch_combine(const Dims &D, const bf16_t *y_perm, const int32_t *inv_perm,
                          const float *gates, void *out, bool out_f32, hipStream_t s) {
    const unsigned g = (unsigned)((D.T + CB_TOK - 1) / CB_TOK);
    if (g == 0) return hipSuccess;
    if (out_f32)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(g), dim3(CB_THREADS), 0, s, D.T, D.d, D.k,
                           y_perm, inv_perm, gates, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(g), dim3(CB_THREADS), 0, s, D.T, D.d, D.k,
                           y_perm, inv_perm, gates, out);
    return hipGetLastError();
}

}  // namespace moe
