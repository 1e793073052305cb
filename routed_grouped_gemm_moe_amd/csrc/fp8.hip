// W8A8 path (X-Stage, §5.3, evaluates MegaMoE in W8A8): per-row E4M3
// quantisation and the grouped E4M3 expert GEMMs of the staged fp8 FFN.
//
// Quantisation of a row: its scale is the smallest power of two 2^e with
// max|x| <= 448 * 2^e (e >= -126; 1 for an all-zero row), and each element's
// code is the E4M3 value nearest to x * 2^-e (exact: a power-of-two scaling),
// ties to the even code, saturating at 448.  E4M3 here is the OCP 8-bit float
// with 4 exponent bits (bias 7) and 3 mantissa bits, no infinities.
#include <algorithm>

#include "gemm_f8w8.h"

namespace moe {
namespace {

// Row-major quantisation: one wave per row, 4 rows per workgroup.
__global__ __launch_bounds__(256) void quant_rows_kernel(int64_t rows, int64_t cols,
                                                         const bf16_t *__restrict__ x,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ scale) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + r * cols);
    const int64_t nc = cols / 8;
    float m = 0.0f;
    for (int64_t c = lane; c < nc; c += 64) m = amax8(src[c], m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int e = row_scale_exp(m);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-126, 127]
    if (lane == 0) scale[r] = __uint_as_float((uint32_t)(127 + e) << 23);
    uint2 *dst = reinterpret_cast<uint2 *>(q + r * cols);
    for (int64_t c = lane; c < nc; c += 64) dst[c] = encode8(src[c], inv);
}

// Largest magnitude of each routed row (rows below offsets[EL]) of a
// row-major bf16 matrix: one wave per row, 4 rows per workgroup.
__global__ __launch_bounds__(256) void row_amax_kernel(int64_t K, int64_t EL,
                                                       const bf16_t *__restrict__ src,
                                                       const int32_t *__restrict__ offsets,
                                                       int64_t n_rows, float *__restrict__ amax) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= (offsets ? (int64_t)offsets[EL] : n_rows)) return;  // rows: routed, or n_rows
    const u32x4_t *row = reinterpret_cast<const u32x4_t *>(src + r * K);
    float m = 0.0f;
    for (int64_t c = lane; c < K / 8; c += 64) m = amax8(row[c], m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) amax[r] = m;
}

// Rows of a row-major bf16 matrix with K columns, grouped in expert segments
// (offsets[]), quantised into the packed E4M3 layout (segments start at
// pstart[], a multiple of 32; padding rows get zero codes and scale 1), with
// the row maxima of row_amax_kernel.  Workgroup (row block, y) writes
// fragments y*PACK_FR .. y*PACK_FR + PACK_FR - 1 of its 32 rows; each wave
// writes whole 1 KiB fragments, lane l holding row l % 32, bytes
// 32 kk + 16 (l / 32) .. + 15 of fragment kk.
constexpr int PACK_FR = 8;
__global__ __launch_bounds__(256) void quant_pack_kernel(int64_t K, int64_t EL,
                                                         const bf16_t *__restrict__ src,
                                                         const float *__restrict__ amax,
                                                         const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ pstart,
                                                         const int32_t *__restrict__ row_map,
                                                         uint8_t *__restrict__ dst,
                                                         float *__restrict__ scale) {
    __shared__ int32_t s_row[32];
    __shared__ float s_inv[32];
    const int64_t rb = blockIdx.x;
    const int64_t prow0 = rb * 32;
    if (prow0 >= pstart[EL]) return;  // past the last segment (uniform)
    const int tid = threadIdx.x;
    if (tid < 32) {
        int64_t lo = 0, hi = EL - 1;  // segment holding prow0: last e with pstart[e] <= prow0
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (pstart[mid] <= prow0) lo = mid;
            else hi = mid - 1;
        }
        const int64_t local = prow0 + tid - pstart[lo];
        const int64_t cnt = offsets[lo + 1] - offsets[lo];
        const int32_t rr = local < cnt ? (int32_t)(offsets[lo] + local) : -1;
        // with row_map, routed row rr is row row_map[rr] of src (and of amax)
        const int32_t sr = (rr >= 0 && row_map) ? row_map[rr] : rr;
        const int e = row_scale_exp(sr >= 0 ? amax[sr] : 0.0f);
        s_row[tid] = sr;
        s_inv[tid] = __uint_as_float((uint32_t)(127 - e) << 23);
        if (blockIdx.y == 0) scale[prow0 + tid] = __uint_as_float((uint32_t)(127 + e) << 23);
    }
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31;
    const int32_t sr = s_row[r];
    const float inv = s_inv[r];
    const int64_t kb = K / 32;  // fragments per row block
    const int64_t k_end = min<int64_t>(kb, (int64_t)(blockIdx.y + 1) * PACK_FR);
    u32x4_t *o = reinterpret_cast<u32x4_t *>(dst + rb * kb * 1024);
    const bf16_t *srow = sr >= 0 ? src + (int64_t)sr * K : nullptr;
    for (int64_t kk = (int64_t)blockIdx.y * PACK_FR + wave; kk < k_end; kk += 4)
        o[kk * 64 + lane] = quant_frag(srow, inv, kk, lane);
}

// Map workgroup b to tile L in [0, n): XCD x = b % 8 takes [x*per, x*per+per).
__device__ __forceinline__ int xcd_tile_f8(int n) {
    const int b = blockIdx.x;
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    const int j = b / NUM_XCD;
    if (j >= per) return -1;
    const int L = (b % NUM_XCD) * per + j;
    return L < n ? L : -1;
}

// One workgroup per (m-tile, n-tile) in the blocked order of gemm_tile.h,
// each XCD taking one contiguous eighth.  GATE_UP: A = packed x codes (K =
// d), W0/W1 = gate/up codes [E_loc][f][d], out = h rows [cap][f].  Down: A =
// packed h codes (K = f), W0 = down codes [E_loc][d][f], out = y rows
// [cap][d].
template <bool GATE_UP>
__global__ __launch_bounds__(W8_THREADS, 1) void grouped_gemm_f8_kernel(
    int64_t d, int64_t f, int64_t EL, const uint8_t *__restrict__ A, const float *__restrict__ sa,
    const MTile *__restrict__ mtiles, const int32_t *__restrict__ n_mtiles,
    const int32_t *__restrict__ mtile_base,
    const uint8_t *__restrict__ W0, const float *__restrict__ s0, const uint8_t *__restrict__ W1,
    const float *__restrict__ s1, bf16_t *__restrict__ out, uint32_t *__restrict__ rowmax) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int MT = *n_mtiles;
    const int NT = GATE_UP ? (int)(f / BN_GU) : (int)(d / BN_DN);
    const int L = xcd_tile_f8(MT * NT);
    if (L < 0) return;
    int mt, nt;
    expert_tile(L, MT, NT, (int)EL, mtiles, mtile_base, &mt, &nt);
    const MTile t = mtiles[mt];
    const int64_t prb = t.prow0 / 32;
    if (GATE_UP) {
        const int64_t wo = (int64_t)t.e * f + (int64_t)nt * BN_GU;
        gemm_tile_f8w8<F8_SILU_ROWS>(A + prb * (d / 32) * 1024, d / 32, t.rows, (int)d, sa + t.prow0,
                                   W0 + wo * d, W1 + wo * d, s0 + wo, s1 + wo,
                                   out + (int64_t)t.row0 * f + (int64_t)nt * BN_GU, f, lds,
                                   rowmax + t.row0);
    } else {
        const int64_t wo = (int64_t)t.e * d + (int64_t)nt * BN_DN;
        gemm_tile_f8w8<F8_BF16>(A + prb * (f / 32) * 1024, f / 32, t.rows, (int)f, sa + t.prow0,
                              W0 + wo * f, nullptr, s0 + wo, nullptr,
                              out + (int64_t)t.row0 * d + (int64_t)nt * BN_DN, d, lds);
    }
}

template <bool GATE_UP>
hipError_t launch_gemm_f8(const Dims &D, const uint8_t *A, const float *sa, const MTile *mtiles,
                          const int32_t *n_mtiles, const int32_t *mtile_base, const uint8_t *W0,
                          const float *s0,
                          const uint8_t *W1, const float *s1, bf16_t *out, uint32_t *rowmax,
                          hipStream_t s) {
    const int64_t NT = GATE_UP ? D.nt_gu() : D.nt_dn();
    int64_t grid = D.max_mtiles() * NT;
    grid = (grid + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    if (grid == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)grouped_gemm_f8_kernel<GATE_UP>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, W8_LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_gemm_f8_kernel<GATE_UP>), dim3((unsigned)grid), dim3(W8_THREADS),
                       W8_LDS_BYTES, s, D.d, D.f, D.EL(), A, sa, mtiles, n_mtiles, mtile_base, W0,
                       s0, W1, s1, out,
                       rowmax);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(int64_t rows, int64_t cols, const bf16_t *x, uint8_t *q,
                             float *scale, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows,
                       cols, x, q, scale);
    return hipGetLastError();
}

hipError_t launch_quant_pack(const Dims &D, int64_t K, const bf16_t *src, const int32_t *offsets,
                             const int32_t *pstart, float *amax, bool have_amax, uint8_t *dst,
                             float *scale, hipStream_t s, const int32_t *row_map,
                             int64_t map_rows) {
    const int64_t nrb = D.pcap() / 32, rows = row_map ? map_rows : D.cap();
    if (nrb == 0 || D.EL() == 0) return hipSuccess;
    hipError_t e;
    if (!have_amax && rows > 0) {
        // row maxima of src's rows: the routed rows (grid sized for every row a
        // segment may hold), or with row_map all map_rows rows, each once
        hipLaunchKernelGGL(row_amax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, K,
                           D.EL(), src, row_map ? nullptr : offsets, rows, amax);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const unsigned ny = (unsigned)((K / 32 + PACK_FR - 1) / PACK_FR);
    hipLaunchKernelGGL(quant_pack_kernel, dim3((unsigned)nrb, ny), dim3(256), 0, s, K, D.EL(), src,
                       amax, offsets, pstart, row_map, dst, scale);
    return hipGetLastError();
}

hipError_t launch_gemm_gate_up_f8(const Dims &D, const uint8_t *xq, const float *sx,
                                  const MTile *mtiles, const int32_t *n_mtiles,
                                  const int32_t *mtile_base, const uint8_t *wg, const float *sg,
                                  const uint8_t *wu, const float *su, bf16_t *h, uint32_t *hmax,
                                  hipStream_t s) {
    return launch_gemm_f8<true>(D, xq, sx, mtiles, n_mtiles, mtile_base, wg, sg, wu, su, h, hmax,
                                s);
}

hipError_t launch_gemm_down_f8(const Dims &D, const uint8_t *hq, const float *sh,
                               const MTile *mtiles, const int32_t *n_mtiles,
                               const int32_t *mtile_base, const uint8_t *wd, const float *sd,
                               bf16_t *y, hipStream_t s) {
    return launch_gemm_f8<false>(D, hq, sh, mtiles, n_mtiles, mtile_base, wd, sd, nullptr, nullptr,
                                 y, nullptr, s);
}

}  // namespace moe
