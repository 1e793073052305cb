// Standalone grouped expert GEMMs (the moe_expert_ffn path) over the packed
// activation layout of gemm_pa.h, with the eight-wave tile of gemm_w8.h, and
// the m-tile table builder.  The tile table is built on the device from the
// segment offsets that the permute produced, so no count ever returns to
// the host (Weave §3: the workload is fixed once routing completes; §4: the
// routing result reaches the kernel as a parameter).
//
// Launch shape: one workgroup of W8_THREADS per (m-tile, n-tile), grid sized
// for the worst case and surplus workgroups exit at once.  Tiles follow the expert-aligned
// blocked order of gemm_tile.h (groups of up to 16 m-tiles of one expert swept
// n-tile-major, so the tiles in flight share weight and activation tiles --
// the same order as the persistent kernel, which fixes which down tiles are
// cut) and each of the 8 XCDs takes one
// contiguous eighth of that order: workgroup b runs on XCD b % 8 (round-robin
// dispatch), so the workgroups sharing a tile meet in one XCD's L2.
#include <algorithm>

#include "gemm_w8.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void build_mtiles_kernel(int64_t EL,
                                                            const int32_t *__restrict__ offsets,
                                                            MTile *__restrict__ mtiles,
                                                            int32_t *__restrict__ n_mtiles,
                                                            int32_t *__restrict__ mtile_base,
                                                            int32_t *__restrict__ pstart,
                                                            int32_t *__restrict__ clear,
                                                            int64_t clear_ints) {
    extern __shared__ int32_t s_mt[];  // [2 * (EL + 1)]: m-tile starts, packed segment starts
    int32_t *s_ps = s_mt + EL + 1;
    for (int64_t i = threadIdx.x; i < clear_ints; i += 1024) clear[i] = 0;
    for (int64_t e = threadIdx.x; e < EL; e += 1024) {
        const int32_t c = offsets[e + 1] - offsets[e];
        s_mt[e] = (c + BM - 1) / BM;
        s_ps[e] = (c + 31) & ~31;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0, ps = 0;
        for (int64_t e = 0; e < EL; ++e) {
            const int32_t m = s_mt[e], p = s_ps[e];
            s_mt[e] = run;
            s_ps[e] = ps;
            run += m;
            ps += p;
        }
        s_mt[EL] = run;
        s_ps[EL] = ps;
        *n_mtiles = run;
    }
    __syncthreads();
    for (int64_t e = threadIdx.x; e <= EL; e += 1024) pstart[e] = s_ps[e];
    for (int64_t e = threadIdx.x; e < EL; e += 1024) {
        const int32_t base = s_mt[e], n = s_mt[e + 1] - base;
        const int32_t row0 = offsets[e], cnt = offsets[e + 1] - row0;
        mtile_base[e] = base;
        for (int32_t m = 0; m < n; ++m) {
            MTile t;
            t.e = (int32_t)e;
            t.row0 = row0 + m * BM;
            t.rows = min(BM, cnt - m * BM);
            t.prow0 = s_ps[e] + m * BM;
            mtiles[base + m] = t;
        }
    }
}

// Map workgroup b to tile L in [0, n): XCD x = b % 8 takes [x*per, x*per+per).
__device__ __forceinline__ int xcd_tile(int n) {
    const int b = blockIdx.x;
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    const int j = b / NUM_XCD;
    if (j >= per) return -1;
    const int L = (b % NUM_XCD) * per + j;
    return L < n ? L : -1;
}

// State of the down tiles cut into K halves (unused by gate/up): the same
// tiles as in the persistent kernel with `grid` workgroups are cut, so both
// paths produce the same bits.
struct DownSplit {
    int32_t *cnt;
    float *part;
    int grid;
};

template <bool GATE_UP>
__global__ __launch_bounds__(W8_THREADS, 1) void grouped_gemm_kernel(
    int64_t d, int64_t f, int64_t EL, const bf16_t *__restrict__ A,
    const MTile *__restrict__ mtiles, const int32_t *__restrict__ n_mtiles,
    const int32_t *__restrict__ mtile_base, const bf16_t *__restrict__ W0,
    const bf16_t *__restrict__ W1, bf16_t *__restrict__ out, DownSplit ds) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int MT = *n_mtiles;
    const int NT = GATE_UP ? (int)(f / BN_GU) : (int)(d / BN_DN);
    const int S = GATE_UP ? 1 : Dims{0, d, f, 0, 0, 0, 0}.dn_parts();
    const int nsp = dn_split_tiles(S, MT * NT, ds.grid);
    const int LS = xcd_tile(MT * NT + (S - 1) * nsp);
    if (LS < 0) return;
    int L, part, st;
    dn_claim(LS, MT * NT, nsp, S, &L, &part, &st);
    int mt, nt;
    expert_tile(L, MT, NT, (int)EL, mtiles, mtile_base, &mt, &nt);
    const MTile t = mtiles[mt];
    const int64_t prb = t.prow0 / 32;  // first packed row block
    if (GATE_UP) {
        const bf16_t *wg = W0 + ((int64_t)t.e * f + (int64_t)nt * BN_GU) * d;
        const bf16_t *wu = W1 + ((int64_t)t.e * f + (int64_t)nt * BN_GU) * d;
        gemm_tile_w8<PA_SILU_PACKED>(A + prb * (d / 16) * 512, d / 16, t.rows, (int)d, wg, wu, d,
                                     out + (prb * (f / 16) + nt * (BN_GU / 16)) * 512, f / 16, lds);
    } else {
        // a cut tile computes K part `part`, starting at k = part * f / S
        const int64_t Kp = part < 0 ? f : f / S, k0 = part < 0 ? 0 : part * Kp;
        const bf16_t *wd = W0 + ((int64_t)t.e * d + (int64_t)nt * BN_DN) * f + k0;
        const SplitCtl sc{ds.cnt + st, ds.part + (int64_t)st * (CUT_MAX * BM * BN_DN), part, S, 0};
        gemm_tile_w8<PA_BF16>(A + (prb * (f / 16) + k0 / 16) * 512, f / 16, t.rows, (int)Kp, wd,
                              nullptr, f, out + (int64_t)t.row0 * d + (int64_t)nt * BN_DN, d, lds,
                              part < 0 ? nullptr : &sc);
    }
}

template <bool GATE_UP>
hipError_t launch_gemm(const Dims &D, const bf16_t *A, const MTile *mtiles, const int32_t *n_mtiles,
                       const int32_t *mtile_base, const bf16_t *W0, const bf16_t *W1, bf16_t *out,
                       const DownSplit &ds, hipStream_t s) {
    const int64_t NT = GATE_UP ? D.nt_gu() : D.nt_dn();
    int64_t grid = D.max_mtiles() * NT;
    if (!GATE_UP && D.dn_parts() > 1)  // extra claims of the cut tiles' parts
        grid += (D.dn_parts() - 1) * std::min<int64_t>(grid, SPLIT_MAX);
    grid = (grid + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    if (grid == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)grouped_gemm_kernel<GATE_UP>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, W8_LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_gemm_kernel<GATE_UP>), dim3((unsigned)grid), dim3(W8_THREADS),
                       W8_LDS_BYTES, s, D.d, D.f, D.EL(), A, mtiles, n_mtiles, mtile_base, W0, W1,
                       out, ds);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build_mtiles(const Dims &D, const int32_t *offsets, MTile *mtiles,
                               int32_t *n_mtiles, int32_t *mtile_base, int32_t *pstart,
                               int32_t *clear, int64_t clear_ints, hipStream_t s) {
    hipLaunchKernelGGL(build_mtiles_kernel, dim3(1), dim3(1024),
                       2 * (D.EL() + 1) * sizeof(int32_t), s, D.EL(), offsets, mtiles, n_mtiles,
                       mtile_base, pstart, clear, clear_ints);
    return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const Dims &D, const bf16_t *xp, const MTile *mtiles,
                               const int32_t *n_mtiles, const int32_t *mtile_base,
                               const bf16_t *w_gate, const bf16_t *w_up, bf16_t *h, hipStream_t s) {
    return launch_gemm<true>(D, xp, mtiles, n_mtiles, mtile_base, w_gate, w_up, h, DownSplit{}, s);
}

hipError_t launch_gemm_down(const Dims &D, const bf16_t *h, const MTile *mtiles,
                            const int32_t *n_mtiles, const int32_t *mtile_base,
                            const bf16_t *w_down, bf16_t *y, int32_t *dn_cnt, float *dn_part,
                            int grid, hipStream_t s) {
    return launch_gemm<false>(D, h, mtiles, n_mtiles, mtile_base, w_down, nullptr, y,
                              DownSplit{dn_cnt, dn_part, grid}, s);
}

}  // namespace moe
