// Router: top-k gating (Weave, §2.1: a learned gate sends each token to k
// experts; Figure 3 shows top-k routing).
//
// Logit arithmetic (fixed by this library so ids are reproducible bit for
// bit): logit[t,e] is a float32 sum over 16 equal contiguous chunks of the
// hidden dimension, each chunk summed sequentially from +0 in ascending index
// (each bf16*bf16 product is exact, so the fma equals multiply-then-add), the
// 16 chunk sums folded by the balanced pairwise tree ((s0+s1)+(s2+s3))+...,
// which is what xor-shuffles 1, 2, 4, 8 over the 16 chunk lanes produce, then
// the bias added.  Selection is k rounds of a wave-wide argmax over
// (logit desc, id asc); gates are the float32 softmax over the selected
// logits.
//
// Implementations of that one definition:
//  - route_exact_kernel: every logit in the defined order (also the optional
//    logits output).  Used for the logits output and when no workspace is given.
//  - route_tok_* (E <= 16, with a workspace): lane = token, wave = chunk;
//    chunk sums go through the workspace to a kernel that folds and selects
//    (and, inside moe_layer, counts the dispatch histogram and runs the
//    dispatch scan in its last workgroup).  When d is a multiple of 1024 the
//    activations and weights are staged through LDS by DMA loads and each
//    weight reaches its multiply-adds by a DPP row broadcast
//    (route_tok_lds_kernel); otherwise the weights are wave-uniform scalar
//    loads (route_tok_chunks_kernel).
//  - route_small_kernel (E <= 16, no workspace): the same order with W_r
//    staged in LDS and the activations prefetched.
//  - fast path (E > 16, with a workspace): bf16 MFMA logits (split-K float32
//    partials) are an approximation l~ with |l~ - l| <= eps, eps bounded from
//    ||x_t||, ||w_e||, the float32 unit roundoff and the measured rounding of
//    one matrix-core step (see route_refine_kernel).  An expert
//    whose upper bound l~ + eps is below the k-th largest lower bound l~ - eps
//    has at least k experts strictly above it and cannot be selected; the
//    remaining candidates (typically k plus a few) get their logits evaluated
//    in the defined order, and the selection and gates are taken from those
//    exact values.  Ids and gates are therefore identical to the exact path.
#include <type_traits>

#include "gemm_tile.h"
#include "scan.h"

namespace moe {
namespace {

constexpr int RT_TOK = 16;       // tokens per workgroup of the exact kernels
constexpr int RT_THREADS = 256;  // 16 chunk lanes x 16 slots

// Top-k by (value desc, id asc) over n entries vals[0..n) with expert ids
// idmap[i] (identity when null), then the renormalised-softmax gates; one wave,
// results written by lanes 0..k-1.  n <= 1024, k <= 64.
__device__ __forceinline__ void wave_topk_gates(const float *vals, const int32_t *idmap, int n,
                                                int64_t k, int lane, int32_t *ids_row,
                                                float *gates_row) {
    uint32_t taken = 0;  // bit r2: entry r2*64 + lane already selected
    float first = 0.0f, denom = 0.0f;
    float my_sel = 0.0f;
    int32_t my_id = 0;
    for (int64_t j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int32_t bi = 0x7FFFFFFF;
        int32_t bs = -1;
        for (int r2 = 0; r2 * 64 + lane < n; ++r2) {
            if (taken & (1u << r2)) continue;
            const int i = r2 * 64 + lane;
            const float v = vals[i];
            const int32_t e = idmap ? idmap[i] : i;
            if (v > bv || (v == bv && e < bi)) {
                bv = v;
                bi = e;
                bs = i;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int32_t oi = __shfl_xor(bi, m, 64);
            const int32_t os = __shfl_xor(bs, m, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
                bs = os;
            }
        }
        if (bs >= 0 && (bs & 63) == lane) taken |= 1u << (bs >> 6);
        if (lane == (int)j) {
            my_sel = bv;
            my_id = bi;
        }
        if (j == 0) first = bv;
    }
    // softmax over the k selected logits, float32; the denominator is a
    // sequential sum over j = 0..k-1 (each term broadcast from lane j)
    const float ej = (lane < k) ? expf(my_sel - first) : 0.0f;
    for (int64_t j = 0; j < k; ++j) denom += __shfl(ej, (int)j, 64);
    if (lane < k) {
        ids_row[lane] = my_id;
        gates_row[lane] = ej / denom;
    }
}

// ------------------------------------------------------------ exact, any E
// TPT tokens x EPT experts of accumulators per thread.  TG = 16/TPT token
// groups, EG = 16/TG expert groups, EB = EG*EPT experts per pass.
template <int TPT, int EPT>
__global__ __launch_bounds__(RT_THREADS) void route_exact_kernel(
    int64_t T, int64_t d, int64_t E, int64_t k, const bf16_t *__restrict__ x,
    const bf16_t *__restrict__ w, const float *__restrict__ bias, int32_t *__restrict__ ids,
    float *__restrict__ gates, float *__restrict__ logits_out) {
    constexpr int TG = RT_TOK / TPT;
    constexpr int EG = 16 / TG;
    constexpr int EB = EG * EPT;
    extern __shared__ float s_logit[];  // [RT_TOK][E]

    const int tid = threadIdx.x;
    const int c = tid & 15;     // chunk lane
    const int slot = tid >> 4;  // 0..15
    const int tg = slot % TG;
    const int eg = slot / TG;
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;
    const int64_t dc = d / 16;

    const bf16_t *xrow[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int64_t t = t0 + tg * TPT + u;
        xrow[u] = x + (t < T ? t : 0) * d + c * dc;
    }

    for (int64_t e0 = 0; e0 < E; e0 += EB) {
        float acc[TPT][EPT];
        const bf16_t *wrow[EPT];
        bool e_ok[EPT];
#pragma unroll
        for (int v = 0; v < EPT; ++v) {
            const int64_t e = e0 + eg * EPT + v;
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
                        const int64_t e = e0 + eg * EPT + v;
                        float l = acc[u][v];
                        if (bias) l = l + bias[e];
                        s_logit[(tg * TPT + u) * E + e] = l;
                    }
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int r = 0; r < RT_TOK / 4; ++r) {
        const int tl = wave * (RT_TOK / 4) + r;
        const int64_t t = t0 + tl;
        if (t >= T) break;
        const float *lt = s_logit + tl * E;
        if (logits_out)
            for (int64_t e = lane; e < E; e += 64) logits_out[t * E + e] = lt[e];
        wave_topk_gates(lt, nullptr, (int)E, k, lane, ids + t * k, gates + t * k);
    }
}

// ------------------------------------------------------------ exact, E <= 16
// Chunk c of a staged row starts at c * (chunk bytes + 16): the 16-byte
// stagger puts the 16 chunk lanes' reads of one step in distinct banks.
__host__ __device__ __forceinline__ int64_t stag_pitch(int64_t d) { return 16 * (d / 16 * 2 + 16); }
// LDS of one refine wave: staged x_t, then candidate ids and exact logits
// (E of each), rounded up to 16 bytes so every wave's x_t stays 16-byte
// aligned whatever E is.
__host__ __device__ __forceinline__ int64_t refine_per_wave(int64_t d, int64_t E) {
    return stag_pitch(d) + ((E * 8 + 15) & ~(int64_t)15);
}
// A refine wave stages x_t in one window (all ppc = d/128 16-byte pieces of
// each chunk) when that leaves LDS for 16 waves per CU, else in two: pieces
// [0, h) of every chunk, then [h, ppc), h even.  Returns h.
__host__ __device__ __forceinline__ int64_t refine_split(int64_t d, int64_t E) {
    const int64_t ppc = d / 128;
    if (refine_per_wave(d, E) * 16 <= 160 * 1024 || ppc < 4) return ppc;
    return (ppc / 2) & ~(int64_t)1;
}
// Byte pitch of one chunk in the staging window (16-byte stagger as above).
__host__ __device__ __forceinline__ int64_t refine_chunk_pitch(int64_t d, int64_t E) {
    const int64_t ppc = d / 128, h = refine_split(d, E);
    return (h > ppc - h ? h : ppc - h) * 16 + 16;
}
// LDS of one refine wave as launched: the staging window, then candidate ids
// and exact logits.
__host__ __device__ __forceinline__ int64_t refine_lds_per_wave(int64_t d, int64_t E) {
    return 16 * refine_chunk_pitch(d, E) + ((E * 8 + 15) & ~(int64_t)15);
}

template <int EP>
__global__ __launch_bounds__(RT_THREADS) void route_small_kernel(
    int64_t T, int64_t d, int64_t E, int64_t k, const bf16_t *__restrict__ x,
    const bf16_t *__restrict__ w, const float *__restrict__ bias, int32_t *__restrict__ ids,
    float *__restrict__ gates) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int64_t dc = d / 16;
    const int64_t cbs = dc * 2 + 16;  // staged chunk stride, bytes
    const int64_t wp = 16 * cbs;      // staged row pitch
    float *s_logit = reinterpret_cast<float *>(smem + E * wp);  // [RT_TOK][E]

    // stage W_r: 16-byte piece p of row e (elements 8p..8p+7) -> chunk p / (dc/8)
    const int64_t ppr = d / 8, ppc = dc / 8;
    // eight independent loads in flight per thread before their stores
    for (int64_t p0 = threadIdx.x; p0 < E * ppr; p0 += 8 * RT_THREADS) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t p = p0 + u * RT_THREADS;
            if (p < E * ppr) v[u] = reinterpret_cast<const u32x4_t *>(w)[p];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t p = p0 + u * RT_THREADS;
            if (p >= E * ppr) break;
            const int64_t e = p / ppr, q = p % ppr;
            *reinterpret_cast<u32x4_t *>(smem + e * wp + (q / ppc) * cbs + (q % ppc) * 16) = v[u];
        }
    }
    __syncthreads();

    const int tid = threadIdx.x;
    const int c = tid & 15;
    const int slot = tid >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;
    const int64_t t = t0 + slot;
    const u32x4_t *xp = reinterpret_cast<const u32x4_t *>(x + (t < T ? t : 0) * d + c * dc);
    const char *wc = smem + c * cbs;
    const int nvec = (int)ppc;  // 16-byte vectors per chunk (even)

    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.0f;
    constexpr int PG = 16;  // vectors per prefetch group
    auto load = [&](u32x4_t (&r)[PG], int b) {
#pragma unroll
        for (int u = 0; u < PG; ++u) r[u] = (b + u < nvec) ? xp[b + u] : u32x4_t{0u, 0u, 0u, 0u};
    };
    auto compute = [&](const u32x4_t (&r)[PG], int b) {
#pragma unroll
        for (int u = 0; u < PG; ++u) {
            if (b + u >= nvec) break;
            u32x4_t wv[EP];
#pragma unroll
            for (int e = 0; e < EP; ++e)
                wv[e] = e < E ? *reinterpret_cast<const u32x4_t *>(wc + e * wp + (b + u) * 16)
                              : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float xf = bf16x8_elem(r[u], q);
#pragma unroll
                for (int e = 0; e < EP; ++e) acc[e] = __builtin_fmaf(xf, bf16x8_elem(wv[e], q), acc[e]);
            }
        }
    };
    // activations prefetched one group of PG vectors ahead
    u32x4_t xa[PG], xb[PG];
    load(xa, 0);
    for (int b = 0; b < nvec; b += 2 * PG) {
        if (b + PG < nvec) load(xb, b + PG);
        compute(xa, b);
        if (b + 2 * PG < nvec) load(xa, b + 2 * PG);
        if (b + PG < nvec) compute(xb, b + PG);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[e] = acc[e] + __shfl_xor(acc[e], m, 64);
    if (c == 0 && t < T) {
#pragma unroll
        for (int e = 0; e < EP; ++e)
            if (e < E) {
                float l = acc[e];
                if (bias) l = l + bias[e];
                s_logit[slot * E + e] = l;
            }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int r = 0; r < RT_TOK / 4; ++r) {
        const int tl = wave * (RT_TOK / 4) + r;
        const int64_t tt = t0 + tl;
        if (tt >= T) break;
        wave_topk_gates(s_logit + tl * E, nullptr, (int)E, k, lane, ids + tt * k, gates + tt * k);
    }
}

// ------------------------------------------------------------ E <= 16, token lanes
// Same defined order, laid out so that the router weights are wave-uniform:
// lane = token (64 per wave), wave = one chunk c, so each step's weights of
// every expert come from scalar loads and enter the FMAs as scalar operands;
// each lane keeps EP accumulators.  Only the activations use the vector
// memory path (each token row read once).
//  route_tok_chunks_kernel: workgroup = 64 tokens x 4 chunks x 4 experts;
//    writes the chunk sums part[blk][c][e][lane];
//  route_tok_finish_kernel: workgroup = 64 tokens; folds the 16 chunk sums by
//    the balanced tree, adds the bias, then one lane per token selects (logit
//    desc, id asc) and forms the gates with the same float32 operations, in
//    the same order, as wave_topk_gates.
constexpr int RTOK = 64;  // tokens per block (one per lane)

// Each wave takes EG of the EP experts (two or more waves per SIMD, so one
// wave's scalar-load waits overlap another's FMAs); grid = token blocks x 4
// chunk quads x EP/EG expert groups.  Workgroups are dealt to the 8 XCDs in
// turn, so the EP/EG expert groups of one (token block, chunk quad) unit are
// placed 8 workgroups apart: they run on one XCD at about the same time and
// all but the first read that unit's activations from the XCD's L2.  The
// grid is padded to whole sets of 8 units; padding workgroups exit at once.
constexpr int RT_EG = 4;

__host__ __device__ constexpr int64_t route_tok_units(int64_t T) {
    return 4 * ((T + RTOK - 1) / RTOK);
}
__host__ __device__ constexpr int64_t route_tok_grid(int64_t T, int ng) {
    return (route_tok_units(T) + 7) / 8 * 8 * ng;
}

template <int EP>
__global__ __launch_bounds__(256) void route_tok_chunks_kernel(int64_t T, int64_t d, int64_t E,
                                                               const bf16_t *__restrict__ x,
                                                               const bf16_t *__restrict__ w,
                                                               float *__restrict__ part,
                                                               int32_t *__restrict__ hist,
                                                               int64_t hist_n,
                                                               int32_t *__restrict__ arrive) {
    constexpr int NG = EP / RT_EG;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the permute's histogram, filled by the finish kernel, and the finish
    // kernel's arrival counter start at zero
    if (hist && blockIdx.x == 0) {
        for (int64_t i = threadIdx.x; i < hist_n; i += 256) hist[i] = 0;
        if (arrive && threadIdx.x == 0) *arrive = 0;
    }
    const int64_t rest = blockIdx.x / 8;
    const int64_t unit = (rest / NG) * 8 + blockIdx.x % 8;
    if (unit >= route_tok_units(T)) return;
    const int64_t blk = unit / 4;
    const int e0 = (int)(rest % NG) * RT_EG;    // first expert of this wave
    const int c = (int)(unit % 4) * 4 + wave;   // chunk, wave-uniform
    const int64_t t = blk * RTOK + lane;
    const int64_t dc = d / 16;
    const int nvec = (int)(dc / 8);  // 16-byte activation vectors per chunk
    const u32x4_t *xp = reinterpret_cast<const u32x4_t *>(x + (t < T ? t : T - 1) * d + c * dc);
    // W_r rows of this wave's experts (bf16, read by scalar loads and widened
    // exactly by a 16-bit shift); experts E..EP-1 repeat row E-1, and their
    // sums are never stored
    const u32x4_t *wp[RT_EG];
#pragma unroll
    for (int e = 0; e < RT_EG; ++e)
        wp[e] = reinterpret_cast<const u32x4_t *>(w + (e0 + e < E ? e0 + e : E - 1) * d + c * dc);

    float acc[RT_EG];
#pragma unroll
    for (int e = 0; e < RT_EG; ++e) acc[e] = 0.0f;
    constexpr int PG = 4;  // activation vectors per prefetch group (4 measured best of 2..16)
    u32x4_t xa[PG], xb[PG];
    auto load = [&](u32x4_t (&r)[PG], int b) {
#pragma unroll
        for (int u = 0; u < PG; ++u) r[u] = (b + u < nvec) ? xp[b + u] : u32x4_t{0u, 0u, 0u, 0u};
    };
    // the weights of vector v + 1 are loaded (scalar) while vector v computes
    u32x4_t wc[RT_EG], wn[RT_EG];
    auto loadw = [&](u32x4_t (&wv)[RT_EG], int v) {
        const int vv = v < nvec ? v : nvec - 1;
#pragma unroll
        for (int e = 0; e < RT_EG; ++e) wv[e] = wp[e][vv];
    };
    auto compute = [&](const u32x4_t (&r)[PG], int b) {
#pragma unroll
        for (int u = 0; u < PG; ++u) {
            if (b + u >= nvec) break;
            loadw(wn, b + u + 1);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float xf = bf16x8_elem(r[u], q);
#pragma unroll
                for (int e = 0; e < RT_EG; ++e)
                    acc[e] = __builtin_fmaf(xf, bf16x8_elem(wc[e], q), acc[e]);
            }
#pragma unroll
            for (int e = 0; e < RT_EG; ++e) wc[e] = wn[e];
        }
    };
    loadw(wc, 0);
    load(xa, 0);
    for (int b = 0; b < nvec; b += 2 * PG) {
        if (b + PG < nvec) load(xb, b + PG);
        compute(xa, b);
        if (b + 2 * PG < nvec) load(xa, b + 2 * PG);
        if (b + PG < nvec) compute(xb, b + PG);
    }
    float *pp = part + ((blk * 16 + c) * EP + e0) * RTOK + lane;
#pragma unroll
    for (int e = 0; e < RT_EG; ++e)
        if (e0 + e < E) pp[e * RTOK] = acc[e];
}

// Chunk sums with the activations and router weights staged through LDS
// (d a multiple of 1024).  The kernel above reads each lane's own row, so one
// load instruction touches 64 cache lines for 16 bytes of each, and widens
// every weight on the scalar unit between scalar loads whose latency it
// cannot hide.  Here:
//  - workgroup = 64 tokens x chunk quad q x NG groups of EG = 4 experts,
//    4*NG waves (two per SIMD for E <= 8); wave (j, g): chunk 4q + j,
//    experts EG*g .. EG*g + EG - 1;
//  - a step covers elements 64s .. 64s + 63 of every chunk.  Its activations
//    (one 128-byte line per token and chunk, 32 KiB) and weights (one line
//    per chunk and expert) come in by coalesced DMA loads (global -> LDS, no
//    registers) into one slot of a ring; all of d = 4096 is in flight at once;
//  - activation slot layout [chunk j][token t][16-byte piece], piece u of
//    token t at position u ^ ((t >> 1) & 7), so the 16 lanes of one LDS bank
//    sweep hit distinct banks; weights [chunk j][expert][128 bytes];
//  - lane = token; the weights are read 16 to a register (lane n of each
//    16-lane row holds element 2n or 2n + 1 of a 32-element half) and each
//    multiply-add takes its weight by a DPP row broadcast of lane n, so the
//    weight costs neither a scalar load nor a widening per use.
// Every sum is the same chain of float32 fmas, in the same order, as in the
// kernels above.
template <int EP, int EG>
struct RtlGeom {
    static constexpr int NG = EP / EG;                       // expert groups of EG
    static constexpr int WAVES = 4 * NG;
    static constexpr int X_BYTES = 4 * RTOK * 128;           // 32 KiB
    static constexpr int W_BYTES = WAVES * 1024;             // one weight DMA per wave
    static constexpr int SLOT = X_BYTES + W_BYTES;
    static constexpr int SLOTS = SLOT <= 36 * 1024 ? 4 : 3;  // ring depth (LDS <= 144 KiB)
    static constexpr int DPW = 32 / WAVES;                   // activation DMAs per wave and step
};

constexpr int RTL_EG = 4;  // experts per wave (measured: 4 beats 2 and 8)

__host__ __device__ constexpr bool route_tok_lds_ok(int64_t d) {
    return d % 1024 == 0 && d >= 1024;
}
template <int EP, int EG>
__host__ constexpr size_t route_tok_lds_bytes(int64_t d) {
    using G = RtlGeom<EP, EG>;
    return (size_t)(d / 1024 < G::SLOTS ? d / 1024 : G::SLOTS) * G::SLOT;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// acc = fma(w of lane n of this lane's 16-lane row, x, acc): one v_fmac_f32
// whose first operand is a DPP row broadcast (gfx950 row_newbcast).
#define RTL_FB(N)                                                                          \
    case N:                                                                                \
        asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #N " row_mask:0xf bank_mask:0xf"     \
            : "+v"(acc)                                                                    \
            : "v"(w), "v"(x));                                                             \
        break;
__device__ __forceinline__ void fma_row_bcast(float &acc, float w, float x, int n) {
    switch (n) {
        RTL_FB(0) RTL_FB(1) RTL_FB(2) RTL_FB(3) RTL_FB(4) RTL_FB(5) RTL_FB(6) RTL_FB(7)
        RTL_FB(8) RTL_FB(9) RTL_FB(10) RTL_FB(11) RTL_FB(12) RTL_FB(13) RTL_FB(14) RTL_FB(15)
    }
}
#undef RTL_FB
// The two bf16 of a 32-bit word widened to float32 (exact).  A DPP operand
// written by a VALU instruction needs two wait states before it is read; the
// s_nop inside the same statement provides them whatever the compiler places
// after it.
__device__ __forceinline__ void widen_pair(uint32_t raw, float &lo, float &hi) {
    asm("v_lshlrev_b32 %0, 16, %2\n\tv_and_b32 %1, 0xffff0000, %2\n\ts_nop 1"
        : "=&v"(lo), "=&v"(hi)
        : "v"(raw));
}

template <int EP, int EG>
__global__ __launch_bounds__(64 * (RtlGeom<EP, EG>::WAVES)) void route_tok_lds_kernel(
    int64_t T, int64_t d, int64_t E, const bf16_t *__restrict__ x, const bf16_t *__restrict__ w,
    float *__restrict__ part, int32_t *__restrict__ hist, int64_t hist_n,
    int32_t *__restrict__ arrive) {
    using G = RtlGeom<EP, EG>;
    constexpr int NTH = 64 * G::WAVES;
    constexpr int DPW = G::DPW;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (hist && blockIdx.x == 0) {  // the finish kernel's histogram and arrival counter
        for (int64_t i = threadIdx.x; i < hist_n; i += NTH) hist[i] = 0;
        if (arrive && threadIdx.x == 0) *arrive = 0;
    }
    const int64_t blk = blockIdx.x / 4;
    const int q = (int)(blockIdx.x % 4);
    const int j = wave & 3;           // chunk of this wave inside the quad
    const int e0 = (wave >> 2) * EG;  // first expert of this wave
    const int c = 4 * q + j;
    const int64_t dc = d / 16;
    const int NS = (int)(dc / 64);    // steps
    const int NSL = NS < G::SLOTS ? NS : G::SLOTS;

    // activation rows of this token block (rows past T read as zeros) and W_r
    const int64_t rows = T - blk * RTOK < RTOK ? T - blk * RTOK : RTOK;
    i32x4_t rx = make_rsrc(x + blk * RTOK * d, (uint32_t)(rows * d * 2));
    i32x4_t rw = make_rsrc(w, (uint32_t)(E * d * 2));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        rx[v] = __builtin_amdgcn_readfirstlane(rx[v]);
        rw[v] = __builtin_amdgcn_readfirstlane(rw[v]);
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    // activation DMA i = wave * DPW + r of a step: chunk i / 8, tokens
    // 8 (i % 8) .. + 7; lane L fetches piece (L & 7) ^ ((t >> 1) & 7) of token
    // t = 8 (i % 8) + L / 8 into LDS position L.  Weight DMA of wave m: (chunk,
    // expert) pairs 8m .. 8m + 7 (pair = chunk * EP + expert), lane L piece
    // L & 7 of pair 8m + L / 8; experts past E re-read row E - 1.
    uint32_t voff[DPW];
#pragma unroll
    for (int r = 0; r < DPW; ++r) {
        const int i = wave * DPW + r;
        const int t = 8 * (i % 8) + (lane >> 3);
        const int p = (lane & 7) ^ ((t >> 1) & 7);
        voff[r] = (uint32_t)(t * d * 2 + (4 * q + i / 8) * dc * 2 + p * 16);
    }
    // (pairs past 4 * EP, when there are more waves than weight lines, load a
    // second copy that nobody reads)
    const int wpair = (8 * wave + (lane >> 3)) % (4 * EP);
    const int we = wpair % EP < E ? wpair % EP : (int)E - 1;
    const uint32_t woff = (uint32_t)(we * d * 2 + (4 * q + wpair / EP) * dc * 2 + (lane & 7) * 16);
    auto issue = [&](int s) {
        const uint32_t sb = lds_base + (s % G::SLOTS) * G::SLOT;
#pragma unroll
        for (int r = 0; r < DPW; ++r) {
            const uint32_t m = __builtin_amdgcn_readfirstlane(sb + (wave * DPW + r) * 1024);
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(m), "v"(voff[r] + (uint32_t)s * 128u), "s"(rx) : "memory", "m0");
        }
        const uint32_t m = __builtin_amdgcn_readfirstlane(sb + G::X_BYTES + wave * 1024);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m), "v"(woff + (uint32_t)s * 128u), "s"(rw) : "memory", "m0");
    };
    for (int s = 0; s < NSL; ++s) issue(s);

    float acc[EG];
#pragma unroll
    for (int e = 0; e < EG; ++e) acc[e] = 0.0f;
    const int sw = (lane >> 1) & 7;
    const int n16 = lane & 15;
    for (int s = 0; s < NS; ++s) {
        // DMA steps issued after step s: min(NS - 1, s + NSL - 1) - s
        const int later = (s + NSL - 1 < NS - 1 ? s + NSL - 1 : NS - 1) - s;
        if (later >= 3) wait_vmcnt<3 * (DPW + 1)>();
        else if (later == 2) wait_vmcnt<2 * (DPW + 1)>();
        else if (later == 1) wait_vmcnt<DPW + 1>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wave's DMA of step s has landed
        const char *slot = lds + (s % G::SLOTS) * G::SLOT;
        const char *xrow = slot + (j * RTOK + lane) * 128;
        const uint32_t *wrow =
            reinterpret_cast<const uint32_t *>(slot + G::X_BYTES + (j * EP + e0) * 128) + n16;
        for (int h = 0; h < 2; ++h) {  // the two 32-element halves of the step
            float lo[EG], hi[EG];  // lane n: elements 32h + 2n, 32h + 2n + 1 of each expert
#pragma unroll
            for (int e = 0; e < EG; ++e) widen_pair(wrow[e * 32 + h * 16], lo[e], hi[e]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4_t xv =
                    *reinterpret_cast<const u32x4_t *>(xrow + (((4 * h + u) ^ sw) << 4));
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const float xf = bf16x8_elem(xv, qq);
#pragma unroll
                    for (int e = 0; e < EG; ++e)
                        fma_row_bcast(acc[e], (qq & 1) ? hi[e] : lo[e], xf, 4 * u + (qq >> 1));
                }
            }
        }
        if (s + NSL < NS) {
            __syncthreads();  // every wave is done with slot s % SLOTS
            issue(s + NSL);
        }
    }
    float *pp = part + ((blk * 16 + c) * EP + e0) * RTOK + lane;
#pragma unroll
    for (int e = 0; e < EG; ++e)
        if (e0 + e < E) pp[e * RTOK] = acc[e];
}
#pragma clang diagnostic pop

template <int EP>
__global__ __launch_bounds__(256) void route_tok_finish_kernel(int64_t T, int64_t E, int64_t k,
                                                               const float *__restrict__ part,
                                                               const float *__restrict__ bias,
                                                               int32_t *__restrict__ ids,
                                                               float *__restrict__ gates,
                                                               int64_t e_lo, int64_t EL,
                                                               int32_t *__restrict__ hist,
                                                               ScanArgs scan) {
    __shared__ float s_l[EP][RTOK];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t blk = blockIdx.x;
    const float *pb = part + blk * 16 * EP * RTOK + lane;
    for (int e = wave; e < E; e += 4) {
        float p[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) p[c] = pb[(c * EP + e) * RTOK];
        // ((s0+s1)+(s2+s3))+((s4+s5)+(s6+s7)), ... : the chunk-lane butterfly
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int c = 0; c < 16; c += 2 * m) p[c] = p[c] + p[c + m];
        float l = p[0];
        if (bias) l = l + bias[e];
        s_l[e][lane] = l;
    }
    __syncthreads();
    const int64_t t = blk * RTOK + lane;
    auto select = [&]() {  // wave 0: one lane per token
    const bool valid = t < T;  // lanes past T select on clamped rows, store nothing
    float l[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) l[e] = e < E ? s_l[e][lane] : -__builtin_inff();
    uint32_t taken = 0;
    float sel[EP];
    int32_t sid[EP];
    float first = 0.0f;
#pragma unroll
    for (int j = 0; j < EP; ++j) {
        sel[j] = 0.0f;
        sid[j] = 0;
        if (j >= k) continue;
        // ascending scan with a strict '>' keeps the lowest id among ties
        float bv = -__builtin_inff();
        int32_t be = -1;
#pragma unroll
        for (int e = 0; e < EP; ++e)
            if (e < E && !(taken & (1u << e)) && (be < 0 || l[e] > bv)) {
                bv = l[e];
                be = e;
            }
        taken |= 1u << be;
        sel[j] = bv;
        sid[j] = be;
        if (j == 0) first = bv;
    }
    float ej[EP];
    float denom = 0.0f;
#pragma unroll
    for (int j = 0; j < EP; ++j) {
        ej[j] = j < k ? expf(sel[j] - first) : 0.0f;
        if (j < k) denom += ej[j];
    }
#pragma unroll
    for (int j = 0; j < EP; ++j)
        if (valid && j < k) {
            ids[t * k + j] = sid[j];
            gates[t * k + j] = ej[j] / denom;
        }
    if (!hist) return;
    // The permute's count of (token block, local expert) assignments: this
    // wave's 64 tokens lie in one token block of PERM_TB, so they are counted
    // in LDS (s_l is free again) and added with one global atomic per expert.
    int32_t *s_h = reinterpret_cast<int32_t *>(&s_l[0][0]);
    if (lane < EL) s_h[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < EP; ++j) {
        const int64_t el = sid[j] - e_lo;
        if (valid && j < k && el >= 0 && el < EL) atomicAdd(&s_h[el], 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < EL && s_h[lane]) atomicAdd(&hist[(blk * RTOK / PERM_TB) * EL + lane], s_h[lane]);
    };
    if (wave == 0) select();
    // the permute's dispatch scan, by the last workgroup to finish counting
    if (hist && scan.arrive) {
        __shared__ int32_t s_last;
        __shared__ int32_t s_scan[scan_lds_ints(16)];  // EL <= E <= 16
        if (scan_arrive_last(scan.arrive, gridDim.x, &s_last)) scan_block<256>(scan, s_scan);
    }
}

// ------------------------------------------------------------ fast path
// Factor that rounds a float32 norm sqrt(sum of d squares) up past its exact
// value: the sum errs by at most d*2^-24 relative, the sqrt halves that and
// adds 2^-24.
__device__ __forceinline__ float norm_inflation(int64_t d) {
    return 1.0f + (float)d * 0x1p-24f + 0x1p-20f;
}

// W_r re-laid out so the 16 chunk pieces of one step are contiguous:
// piece (e, step i, chunk c) at ((e * (dc/8) + i) * 16 + c) * 16 bytes; and
// ||w_e|| (float32, rounded up by a relative 2^-10 to cover its own rounding).
__global__ __launch_bounds__(256) void route_wprep_kernel(int64_t d, const bf16_t *__restrict__ w,
                                                          bf16_t *__restrict__ wt,
                                                          float *__restrict__ wnorm,
                                                          int32_t *__restrict__ arrive) {
    __shared__ float s_red[256];
    const int64_t e = blockIdx.x;
    // the permute's histogram kernel counts its arrivals from zero
    if (arrive && e == 0 && threadIdx.x == 0) *arrive = 0;
    const int64_t ppr = d / 8, ppc = d / 16 / 8;
    float ss = 0.0f;
    for (int64_t p = threadIdx.x; p < ppr; p += 256) {
        const u32x4_t v = reinterpret_cast<const u32x4_t *>(w + e * d)[p];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float f = bf16x8_elem(v, q);
            ss = __builtin_fmaf(f, f, ss);
        }
        const int64_t c = p / ppc, i = p % ppc;
        reinterpret_cast<u32x4_t *>(wt + e * d)[i * 16 + c] = v;
    }
    s_red[threadIdx.x] = ss;
    __syncthreads();
    for (int m = 128; m >= 1; m >>= 1) {
        if ((int)threadIdx.x < m) s_red[threadIdx.x] += s_red[threadIdx.x + m];
        __syncthreads();
    }
    if (threadIdx.x == 0) wnorm[e] = sqrtf(s_red[0]) * norm_inflation(d);
}

// Approximate logits: float32 partial sums of x . w over K split S ways,
// part[s][t][e], one 256 x 256 MFMA tile (token block x expert block) per
// workgroup.
__global__ __launch_bounds__(GEMM_THREADS, 1) void route_gemm_kernel(
    int64_t T, int64_t d, int64_t E, int S, const bf16_t *__restrict__ x,
    const bf16_t *__restrict__ w, float *__restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int MT = (int)((T + BM - 1) / BM);
    const int NT = (int)((E + BN_TILE - 1) / BN_TILE);
    const int L = blockIdx.x;
    const int s = L / (MT * NT);
    const int mt = (L % (MT * NT)) % MT;
    const int nt = (L % (MT * NT)) / MT;
    const int64_t Ks = d / S, k0 = (int64_t)s * Ks;
    const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN_TILE;
    const int a_rows = (int)min((int64_t)BM, T - m0);
    const int b_rows = (int)min((int64_t)BN_TILE, E - n0);
    gemm_tile<EPI_F32>(x + k0, d, m0, a_rows, w + n0 * d + k0, nullptr, d, b_rows, (int)Ks,
                       part + (int64_t)s * T * E, E, n0, b_rows, lds);
}

// Cross-lane steps by DPP (register moves, no LDS round trip); the whole
// wave must be active.  Controls (gfx9): quad_perm [1,0,3,2] and [2,3,0,1]
// (partners xor 1, xor 2), row_half_mirror (lane i <-> 7 - i of each 8),
// row_mirror (i <-> 15 - i of each 16), row_bcast15 / row_bcast31 (lane 15 of
// a row to the next row, lane 31 to rows 2 and 3; rows outside ROWS keep
// their own value).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// Sum of each 16-lane row in the balanced pairwise order (partners xor 1, 2,
// 4, 8).  After the first two steps the four lanes of a quad hold the same
// bits (a + b == b + a exactly), so the half-mirror and mirror partners hold
// the values the xor-4 and xor-8 partners would: every lane of the row ends
// with ((s0 + s1) + (s2 + s3)) + ... bit for bit.
__device__ __forceinline__ float row16_tree_sum(float a) {
    a = a + dpp_f32<0xB1>(a);
    a = a + dpp_f32<0x4E>(a);
    a = a + dpp_f32<0x141>(a);
    a = a + dpp_f32<0x140>(a);
    return a;
}

// Maximum over the wave (every lane receives it).
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    v = fmaxf(v, dpp_f32<0x142, 0xA>(v));
    v = fmaxf(v, dpp_f32<0x143, 0xC>(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// wave_topk_gates for n <= 64 entries (entry i in lane i), without LDS round
// trips: each entry's rank under (value desc, id asc) is the count of
// entries ahead of it, from wave-uniform reads of every entry; the entries
// of rank 0 .. k-1 are the selection in order, and the gates take the same
// float32 operations in the same order (the denominator summed over ranks
// 0 .. k-1).  The whole wave must be active; k <= n.
__device__ __forceinline__ void wave_topk_gates_small(const float *vals, const int32_t *idmap,
                                                      int n, int64_t k, int lane,
                                                      int32_t *ids_row, float *gates_row) {
    const bool have = lane < n;
    const float v = have ? vals[lane] : -__builtin_inff();
    const int32_t e = have ? (idmap ? idmap[lane] : lane) : 0x7FFFFFFF;
    int rank = 0;
    for (int i = 0; i < n; ++i) {
        const float vi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
        const int32_t ei = __builtin_amdgcn_readlane(e, i);
        rank += (vi > v || (vi == v && ei < e)) ? 1 : 0;
    }
    const bool sel = have && rank < k;
    const int l0 = __builtin_ctzll(__ballot(have && rank == 0));
    const float first = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l0));
    const float ej = sel ? expf(v - first) : 0.0f;
    float denom = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        const int lj = __builtin_ctzll(__ballot(have && rank == (int)j));
        denom += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ej), lj));
    }
    if (sel) {
        ids_row[rank] = e;
        gates_row[rank] = ej / denom;
    }
}

// The chunk chains of NJ candidates over pieces lo .. lo + n - 1 of this
// lane's chunk (acc[j] += x_i * w_j,i, i ascending).  rw = buffer over the
// re-laid-out W_r; vo[j] = byte offset of candidate j's first 16-byte piece
// of the chunk, successive pieces 256 bytes apart; xc = the staged window of
// the chunk (piece lo first); n is even (d is a multiple of 256 and the
// windows split at an even piece).  NJ is a template parameter so every group
// of loads is unconditional: the pieces of RF_RING - 1 groups ahead are in
// flight while a group is summed, and each wait leaves exactly those
// outstanding.  A group's position is one wave-uniform scalar offset (the
// pieces within it are immediate offsets), so the loads cost no vector
// address arithmetic; positions past the window's end re-load its last group.
constexpr int RF_PG = 2;    // 16-byte pieces per candidate and group (divides n)
constexpr int RF_RING = 2;  // groups in the register ring
template <int NJ>
__device__ __forceinline__ void refine_chains(i32x4_t rw, const int (&vo)[4], const char *xc,
                                              int lo, int n, float (&acc)[4]) {
    u32x4_t r[RF_RING][NJ][RF_PG];
    auto load = [&](u32x4_t (&dst)[NJ][RF_PG], int i0) {
        const int so = __builtin_amdgcn_readfirstlane((lo + min(i0, n - RF_PG)) * 256);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < RF_PG; ++q)
                dst[j][q] = __builtin_bit_cast(u32x4_t, raw_buffer_load_v4(rw, vo[j] + q * 256, so, 0));
    };
    auto sum = [&](const u32x4_t (&src)[NJ][RF_PG], int i0) {
#pragma unroll
        for (int q = 0; q < RF_PG; ++q) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xc + (i0 + q) * 16);
            float xf[8];
#pragma unroll
            for (int h = 0; h < 8; ++h) xf[h] = bf16x8_elem(xv, h);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int h = 0; h < 8; ++h)
                    acc[j] = __builtin_fmaf(xf[h], bf16x8_elem(src[j][q], h), acc[j]);
        }
    };
#pragma unroll
    for (int u = 0; u < RF_RING - 1; ++u) {
        load(r[u], u * RF_PG);
        __builtin_amdgcn_sched_barrier(0);  // groups issued in ring order
    }
    for (int i0 = 0; i0 < n; i0 += RF_RING * RF_PG) {
#pragma unroll
        for (int u = 0; u < RF_RING; ++u) {
            load(r[(u + RF_RING - 1) % RF_RING], i0 + (u + RF_RING - 1) * RF_PG);
            if (i0 + u * RF_PG < n) sum(r[u], i0 + u * RF_PG);  // whole groups (uniform)
            // keep the next step's loads after this sum (hoisted, they would
            // all wait at the turn's last sum)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One wave per token: bounds, candidates, exact logits of the candidates in
// the defined order, selection and gates.
constexpr int RF_WAVES = 4;
// RMAX = expert slots per lane (E <= 64 * RMAX), a template parameter so the
// bound, selection and compaction loops run over only the slots E needs.
// BOUNDS: instead of selecting, write every (t, e)'s approximate logit and its
// bound eps to approx / eps_out [T, E] and return (the verification entry
// point moe_route_bounds; the arithmetic is the selection path's own).
template <int RMAX, bool BOUNDS = false>
__global__ __launch_bounds__(64 * RF_WAVES) void route_refine_kernel(
    int64_t T, int64_t d, int64_t E, int64_t k, int S, const bf16_t *__restrict__ x,
    const bf16_t *__restrict__ wt, const float *__restrict__ wnorm, const float *__restrict__ bias,
    const float *__restrict__ part, int32_t *__restrict__ ids, float *__restrict__ gates,
    float *__restrict__ approx = nullptr, float *__restrict__ eps_out = nullptr) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * RF_WAVES + wave;
    if (t >= T) return;  // wave-uniform; the kernel has no workgroup barrier

    const int64_t dc = d / 16, ppc = dc / 8;
    const int64_t h = refine_split(d, E);         // pieces of chunk in window 0
    const int64_t cbs = refine_chunk_pitch(d, E);  // chunk pitch in the window
    char *xs = smem + wave * refine_lds_per_wave(d, E);         // staged x_t window
    int32_t *cand = reinterpret_cast<int32_t *>(xs + 16 * cbs);  // [E]
    float *exact = reinterpret_cast<float *>(cand + E);          // [E]

    // ||x_t|| over the whole row (coalesced), staging window 0
    float ss = 0.0f;
    for (int64_t p0 = lane; p0 < d / 8; p0 += 8 * 64) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t p = p0 + u * 64;
            if (p < d / 8) v[u] = reinterpret_cast<const u32x4_t *>(x + t * d)[p];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t p = p0 + u * 64;
            if (p >= d / 8) break;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float f = bf16x8_elem(v[u], q);
                ss = __builtin_fmaf(f, f, ss);
            }
            if (p % ppc < h)
                *reinterpret_cast<u32x4_t *>(xs + (p / ppc) * cbs + (p % ppc) * 16) = v[u];
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float xn = sqrtf(ss) * norm_inflation(d);
    // |l~ - l| <= gam * sum|x_i w_i| + bias roundings, A = sum|x_i w_i| <=
    // ||x|| ||w|| (Cauchy-Schwarz).  Terms of gam, in units of 2^-24:
    //  - each split-K partial is a chain of n = d/(16 S) 32x32x16 bf16 matrix-
    //    core steps; one step errs by at most 2^-20 (sum over its products of
    //    |p| + |accumulator|) -- the premise, measured on gfx950 against exact
    //    sums on adversarial operands (at most 2^-21.3 seen); every running
    //    accumulator is at most the partial's A_s, so a chain errs by at most
    //    16 (n + 1) A_s, and the partials by 16 (n + 1) A together;
    //  - the S partials are added in float32: S roundings of at most 2^-24 A;
    //  - the defined-order logit l itself: d/16 sequential additions per chunk
    //    and 4 tree levels, at most d/16 + 4 roundings of 2^-24 A.
    // +4 and 2^-10 cover the float32 evaluation of the bound itself.
    const int64_t n_steps = d / (16 * (int64_t)S);
    const float gam =
        ((float)(16 * (n_steps + 1) + S + d / 16 + 8) * 0x1p-24f) * (1.0f + 0x1p-10f);

    // bounds of this lane's experts e = lane + 64*r2
    float lo[RMAX], hi[RMAX];
#pragma unroll
    for (int r2 = 0; r2 < RMAX; ++r2) {
        lo[r2] = -__builtin_inff();
        hi[r2] = -__builtin_inff();
    }
    // QN expert slots x up to 8 partials loaded before any is summed
    constexpr int QN = RMAX < 4 ? RMAX : 4;
#pragma unroll
    for (int r0 = 0; r0 < RMAX; r0 += QN) {
        if (r0 * 64 >= E) break;  // wave-uniform
        float pv[QN][8];
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int64_t e = (r0 + q) * 64 + lane;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2)
                pv[q][s2] = (s2 < S && e < E) ? part[((int64_t)s2 * T + t) * E + e] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int64_t e = (r0 + q) * 64 + lane;
            if (e >= E) continue;
            float la = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) la += pv[q][s2];
            if (bias) la += bias[e];
            const float g = gam * xn * wnorm[e];
            const float eps = g + 0x1p-21f * (fabsf(la) + g) + 1e-30f;
            lo[r0 + q] = la - eps;
            hi[r0 + q] = la + eps;
            if (BOUNDS) {
                approx[t * E + e] = la;
                eps_out[t * E + e] = eps;
            }
        }
    }
    if (BOUNDS) return;
    // Lk = k-th largest lower bound: k rounds of a wave max, each removing one
    // instance of the maximum (the value does not depend on which)
    uint32_t taken = 0;
    float Lk = -__builtin_inff();
    for (int64_t j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
#pragma unroll
        for (int r2 = 0; r2 < RMAX; ++r2)
            if (!(taken & (1u << r2)) && r2 * 64 + lane < E) bv = fmaxf(bv, lo[r2]);
        const float m = wave_max_f32(bv);
        const int owner = __builtin_ctzll(__ballot(bv == m));
        if (lane == owner) {
            bool done = false;
#pragma unroll
            for (int r2 = 0; r2 < RMAX; ++r2)
                if (!done && !(taken & (1u << r2)) && r2 * 64 + lane < E && lo[r2] == m) {
                    taken |= 1u << r2;
                    done = true;
                }
        }
        Lk = m;
    }
    // candidates: upper bound >= Lk, compacted in ascending expert order
    int ns = 0;
#pragma unroll
    for (int r2 = 0; r2 < RMAX; ++r2) {
        const bool keep = r2 * 64 + lane < E && hi[r2] >= Lk;
        const uint64_t bal = __ballot(keep);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (keep) cand[ns + before] = r2 * 64 + lane;
        ns += __popcll(bal);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // exact logits of the candidates, up to sixteen per pass: lane = (group
    // g, chunk c) runs the chunk-c chains of the pass's candidates g, g + 4,
    // g + 8, g + 12, so each staged x element is widened once for all of
    // them; every chain is the defined sequential order over its chunk, and
    // the 16 chunk sums of a candidate meet in the balanced tree
    const int c = lane & 15;
    const int g = lane >> 4;
    const char *xc = xs + c * cbs;
    const i32x4_t rw = make_rsrc(wt, (uint32_t)(E * d * 2));
    // window w holds pieces [lo, lo + n) of every chunk
    auto stage = [&](int64_t lo, int64_t n) {
        for (int64_t q0 = lane; q0 < 16 * n; q0 += 8 * 64) {
            u32x4_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t q = q0 + u * 64;
                if (q < 16 * n)
                    v[u] = reinterpret_cast<const u32x4_t *>(x + t * d)[(q / n) * ppc + lo + q % n];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t q = q0 + u * 64;
                if (q >= 16 * n) break;
                *reinterpret_cast<u32x4_t *>(xs + (q / n) * cbs + (q % n) * 16) = v[u];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    int staged = 0;  // window in LDS
    for (int b = 0; b < ns; b += 16) {
        const int nj = min(4, (ns - b + 3) >> 2);  // candidate slots per lane in use (uniform)
        int vo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ci = b + g + 4 * j;
            const int e = cand[ci < ns ? ci : b];
            vo[j] = (e * (int)d + c * 8) * 2;
        }
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int w = 0; w < (h < ppc ? 2 : 1); ++w) {  // the chains go on across windows
            const int64_t lo = w ? h : 0, n = w ? ppc - h : h;
            if (staged != w) {
                stage(lo, n);
                staged = w;
            }
            switch (nj) {  // wave-uniform
            case 4: refine_chains<4>(rw, vo, xc, (int)lo, (int)n, acc); break;
            case 3: refine_chains<3>(rw, vo, xc, (int)lo, (int)n, acc); break;
            case 2: refine_chains<2>(rw, vo, xc, (int)lo, (int)n, acc); break;
            default: refine_chains<1>(rw, vo, xc, (int)lo, (int)n, acc); break;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nj) acc[j] = row16_tree_sum(acc[j]);  // nj wave-uniform
            const int ci = b + g + 4 * j;
            if (c == 0 && j < nj && ci < ns) {
                float l = acc[j];
                if (bias) l = l + bias[cand[ci]];
                exact[ci] = l;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (ns <= 64)
        wave_topk_gates_small(exact, cand, ns, k, lane, ids + t * k, gates + t * k);
    else
        wave_topk_gates(exact, cand, ns, k, lane, ids + t * k, gates + t * k);
}

template <int TPT, int EPT>
hipError_t launch_exact_t(const Dims &D, const bf16_t *x, const bf16_t *w, const float *bias,
                          int32_t *ids, float *gates, float *logits, hipStream_t s) {
    const size_t lds = (size_t)RT_TOK * D.E * sizeof(float);
    const unsigned grid = (unsigned)((D.T + RT_TOK - 1) / RT_TOK);
    hipError_t e = hipFuncSetAttribute((const void *)route_exact_kernel<TPT, EPT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_exact_kernel<TPT, EPT>), dim3(grid), dim3(RT_THREADS), lds, s, D.T,
                       D.d, D.E, D.k, x, w, bias, ids, gates, logits);
    return hipGetLastError();
}

template <int EP>
hipError_t launch_small_t(const Dims &D, const bf16_t *x, const bf16_t *w, const float *bias,
                          int32_t *ids, float *gates, hipStream_t s) {
    const size_t lds = (size_t)(D.E * stag_pitch(D.d) + RT_TOK * D.E * sizeof(float));
    const unsigned grid = (unsigned)((D.T + RT_TOK - 1) / RT_TOK);
    hipError_t e = hipFuncSetAttribute((const void *)route_small_kernel<EP>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_small_kernel<EP>), dim3(grid), dim3(RT_THREADS), lds, s, D.T, D.d,
                       D.E, D.k, x, w, bias, ids, gates);
    return hipGetLastError();
}

constexpr size_t SMALL_LDS_MAX = 150 * 1024;

}  // namespace

int route_splits(const Dims &D) {
    const int64_t tiles = ((D.T + BM - 1) / BM) * ((D.E + BN_TILE - 1) / BN_TILE);
    int S = 1;
    while (S < 8 && tiles * S < 256 && D.d / (2 * S) >= 128 && (D.d / (2 * S)) % BK == 0) S *= 2;
    return S;
}

bool route_uses_fast_path(const Dims &D) {
    return D.E > 16 && (size_t)RF_WAVES * refine_per_wave(D.d, D.E) <= 150 * 1024;
}

static int tok_ep(const Dims &D) { return D.E <= 8 ? 8 : 16; }

size_t route_workspace_bytes(const Dims &D) {
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    if (D.E <= 16)  // token-lane chunk sums
        return al((size_t)((D.T + RTOK - 1) / RTOK) * 16 * tok_ep(D) * RTOK * sizeof(float));
    if (!route_uses_fast_path(D)) return 0;
    return al((size_t)route_splits(D) * D.T * D.E * 4) + al((size_t)D.E * D.d * 2) +
           al((size_t)D.E * 4);
}

template <int EP>
static hipError_t launch_tok_t(const Dims &D, const bf16_t *x, const bf16_t *w, const float *bias,
                               int32_t *ids, float *gates, void *ws, const ScanArgs *scan,
                               hipStream_t s) {
    const unsigned nblk = (unsigned)((D.T + RTOK - 1) / RTOK);
    int32_t *hist = scan ? scan->blk_counts : nullptr;
    int32_t *arrive = scan ? scan->arrive : nullptr;
    float *part = reinterpret_cast<float *>(ws);
    hipError_t e;
    if (route_tok_lds_ok(D.d)) {
        constexpr int EG = RTL_EG;
        const size_t lds = route_tok_lds_bytes<EP, EG>(D.d);
        e = hipFuncSetAttribute((const void *)route_tok_lds_kernel<EP, EG>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((route_tok_lds_kernel<EP, EG>), dim3(nblk * 4),
                           dim3(64 * RtlGeom<EP, EG>::WAVES),
                           lds, s, D.T, D.d, D.E, x, w, part, hist, D.perm_blocks() * D.EL(),
                           arrive);
    } else {
        hipLaunchKernelGGL((route_tok_chunks_kernel<EP>),
                           dim3((unsigned)route_tok_grid(D.T, EP / RT_EG)), dim3(256), 0, s, D.T,
                           D.d, D.E, x, w, part, hist, D.perm_blocks() * D.EL(), arrive);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScanArgs sa{};
    if (scan) sa = *scan;
    hipLaunchKernelGGL((route_tok_finish_kernel<EP>), dim3(nblk), dim3(256), 0, s, D.T, D.E, D.k,
                       part, bias, ids, gates, D.e_lo, D.EL(), hist, sa);
    return hipGetLastError();
}

// The E > 16 fast path: re-laid-out W_r and its norms, the MFMA split-K
// logit partials, then one wave per token for the bounds, the exact logits of
// the candidates and the selection -- or, with approx != NULL, only the
// bounds, written out (moe_route_bounds).
static hipError_t launch_route_fast(const Dims &D, const bf16_t *x, const bf16_t *w_router,
                                    const float *bias, int32_t *ids, float *gates, void *ws,
                                    hipStream_t s, float *approx, float *eps,
                                    int32_t *arrive = nullptr) {
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const int S = route_splits(D);
    float *part = reinterpret_cast<float *>(ws);
    bf16_t *wt = reinterpret_cast<bf16_t *>(reinterpret_cast<char *>(ws) +
                                            al((size_t)S * D.T * D.E * 4));
    float *wnorm = reinterpret_cast<float *>(reinterpret_cast<char *>(wt) + al((size_t)D.E * D.d * 2));
    hipLaunchKernelGGL(route_wprep_kernel, dim3((unsigned)D.E), dim3(256), 0, s, D.d, w_router, wt,
                       wnorm, arrive);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)route_gemm_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS_BYTES);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((D.T + BM - 1) / BM) * ((D.E + BN_TILE - 1) / BN_TILE) * S;
    hipLaunchKernelGGL(route_gemm_kernel, dim3((unsigned)tiles), dim3(GEMM_THREADS), GEMM_LDS_BYTES,
                       s, D.T, D.d, D.E, S, x, w_router, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t lds = (size_t)RF_WAVES * refine_lds_per_wave(D.d, D.E);
    const dim3 grid((unsigned)((D.T + RF_WAVES - 1) / RF_WAVES));
    auto refine = [&](auto rk) -> hipError_t {
        constexpr int R = decltype(rk)::value;
        hipError_t er;
        if (approx) {
            er = hipFuncSetAttribute((const void *)route_refine_kernel<R, true>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (er != hipSuccess) return er;
            hipLaunchKernelGGL((route_refine_kernel<R, true>), grid, dim3(64 * RF_WAVES), lds, s,
                               D.T, D.d, D.E, D.k, S, x, wt, wnorm, bias, part, ids, gates, approx,
                               eps);
        } else {
            er = hipFuncSetAttribute((const void *)route_refine_kernel<R>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (er != hipSuccess) return er;
            hipLaunchKernelGGL(route_refine_kernel<R>, grid, dim3(64 * RF_WAVES), lds, s, D.T, D.d,
                               D.E, D.k, S, x, wt, wnorm, bias, part, ids, gates, nullptr, nullptr);
        }
        return hipSuccess;
    };
    if (D.E <= 128) e = refine(std::integral_constant<int, 2>{});
    else if (D.E <= 256) e = refine(std::integral_constant<int, 4>{});
    else e = refine(std::integral_constant<int, 16>{});
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_route_bounds(const Dims &D, const bf16_t *x, const bf16_t *w_router,
                               const float *bias, float *approx, float *eps, void *ws,
                               hipStream_t s) {
    if (D.T == 0) return hipSuccess;
    return launch_route_fast(D, x, w_router, bias, nullptr, nullptr, ws, s, approx, eps);
}

hipError_t launch_route(const Dims &D, const bf16_t *x, const bf16_t *w_router, const float *bias,
                        int32_t *ids, float *gates, float *logits, void *ws, size_t ws_bytes,
                        hipStream_t s, const ScanArgs *scan, int *prep) {
    if (prep) *prep = PREP_NONE;
    if (!prep || (scan && !scan->arrive)) scan = nullptr;
    if (D.T == 0) return hipSuccess;
    if (logits || (route_uses_fast_path(D) && (!ws || ws_bytes < route_workspace_bytes(D)))) {
        // every logit in the defined order
        if (D.E <= 8) return launch_exact_t<1, 8>(D, x, w_router, bias, ids, gates, logits, s);
        if (D.E <= 16) return launch_exact_t<1, 16>(D, x, w_router, bias, ids, gates, logits, s);
        return launch_exact_t<4, 8>(D, x, w_router, bias, ids, gates, logits, s);
    }
    if (D.E <= 16 && ws && ws_bytes >= route_workspace_bytes(D)) {
        if (scan) *prep = PREP_SCAN_DONE;
        if (D.E <= 8) return launch_tok_t<8>(D, x, w_router, bias, ids, gates, ws, scan, s);
        return launch_tok_t<16>(D, x, w_router, bias, ids, gates, ws, scan, s);
    }
    if (!route_uses_fast_path(D)) {
        const size_t lds = (size_t)(D.E * stag_pitch(D.d) + RT_TOK * D.E * sizeof(float));
        if (lds > SMALL_LDS_MAX) {
            if (D.E <= 8) return launch_exact_t<1, 8>(D, x, w_router, bias, ids, gates, nullptr, s);
            return launch_exact_t<1, 16>(D, x, w_router, bias, ids, gates, nullptr, s);
        }
        if (D.E <= 8) return launch_small_t<8>(D, x, w_router, bias, ids, gates, s);
        return launch_small_t<16>(D, x, w_router, bias, ids, gates, s);
    }
    if (scan && scan->arrive) *prep = PREP_ARRIVE_CLEARED;
    return launch_route_fast(D, x, w_router, bias, ids, gates, ws, s, nullptr, nullptr,
                             scan ? scan->arrive : nullptr);
}

}  // namespace moe
