// Internal declarations of the gfx950 MoE library: tile constants, bf16
// helpers, the workspace layout and the kernel launchers.  Not part of the
// C ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- tiles
// Grouped GEMM tile: BM rows x BN_TILE output columns, K staged BK at a time
// through an NSTAGE-deep LDS ring; 256 threads = 4 waves in a 2x2 grid, each
// wave 128x128 with 32x32x16 MFMAs.
constexpr int BM = 256;
constexpr int BK = 32;
constexpr int NSTAGE = 4;
constexpr int BN_TILE = 256;          // B rows staged per tile
constexpr int BN_GU = 128;            // gate (and up) columns per gate/up tile
constexpr int BN_DN = 256;            // down columns per down tile
constexpr int GEMM_THREADS = 256;
constexpr int STAGE_ROW_BYTES = BK * 2;                 // 64
constexpr int STAGE_A_BYTES = BM * STAGE_ROW_BYTES;     // 16 KiB
constexpr int STAGE_BYTES = STAGE_A_BYTES + BN_TILE * STAGE_ROW_BYTES;  // 32 KiB
constexpr int GEMM_LDS_BYTES = NSTAGE * STAGE_BYTES;    // 128 KiB

// Permute: tokens per block of the histogram / rank kernels.
constexpr int PERM_TB = 256;
// Combine tile of the persistent kernel: COMB_TOK tokens x up to COMB_CB
// blocks of BN_DN columns.
constexpr int COMB_TOK = 32;
constexpr int COMB_CB = 4;

constexpr int NUM_XCD = 8;            // MI355X: 8 accelerator complex dies
constexpr int QSTRIDE = 32;           // ints between queue counters (128 B apart)

// Cut down tiles: at most this many per call (their partials are sized for
// it in the workspace), each cut into at most CUT_MAX K parts.
constexpr int SPLIT_MAX = 256;
constexpr int CUT_MAX = 4;
// Of n2 down tiles run by G workgroups, the last n2 % G (the partial last
// round) are cut into K parts when the tiles are deep (parts > 1); 0 otherwise.
__host__ __device__ inline int dn_split_tiles(int parts, int n2, int G) {
    if (parts <= 1 || G <= 0 || n2 <= G) return 0;
    const int r = n2 % G;
    return r < SPLIT_MAX ? r : SPLIT_MAX;
}
// Down claim index LS -> (tile L in blocked order, part: -1 whole, else the K
// part 0..S-1; st: index of a cut tile among the nsp cut tiles).  The
// n2 + (S-1)*nsp claims form NUM_XCD equal ranges (the per-XCD queues of the
// persistent kernel, and the per-XCD slices of the standalone launch); range
// r holds the next run of tiles in blocked order, whole tiles first and then
// the parts of its share (nsp / NUM_XCD, the first nsp % NUM_XCD ranges one
// more) of cut tiles, so the cut tiles run last on every XCD.  With n2 > G >
// nsp every range is long enough for its parts.
__host__ __device__ inline void dn_claim(int LS, int n2, int nsp, int S, int *L, int *part,
                                         int *st) {
    const int n = n2 + (S - 1) * nsp, per = (n + NUM_XCD - 1) / NUM_XCD;
    const int y = LS / per, i = LS - y * per;
    int base = 0, cbase = 0;
    for (int r = 0; r < y; ++r) {
        const int len = min(per, n - r * per);
        const int c = nsp / NUM_XCD + (r < nsp % NUM_XCD ? 1 : 0);
        base += len - (S - 1) * c;  // whole tiles + cut tiles of range r
        cbase += c;
    }
    const int len = min(per, n - y * per);
    const int c = nsp / NUM_XCD + (y < nsp % NUM_XCD ? 1 : 0);
    const int w = len - S * c;  // whole tiles of this range
    if (i < w) {
        *L = base + i;
        *part = -1;
        *st = -1;
    } else {
        *L = base + w + (i - w) / S;
        *part = (i - w) % S;
        *st = cbase + (i - w) / S;
    }
}

// ---------------------------------------------------------------- bf16
typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// Native 16-byte vector (HIP's uint4 is a union-based struct, which keeps
// arrays of it out of registers).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 element q (0..7) of a 16-byte vector, widened exactly to float.
__device__ __forceinline__ float bf16x8_elem(const u32x4_t &v, int q) {
    const uint32_t w = v[q >> 1];
    return __uint_as_float((q & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

__device__ __forceinline__ float bf2f(bf16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
// float -> bf16, round to nearest, ties to even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32), which rounds finite values exactly as
// IEEE round-to-nearest-even and keeps NaN a NaN.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// Two floats -> two bf16 in one 32-bit word (lo in the low half), one
// conversion instruction.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    typedef float f32x2v_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2v_t));
}
// The same pair by integer arithmetic (where the conversion instruction's
// scheduling would raise register pressure past the budget).
__device__ __forceinline__ uint32_t pk_bf16_sw(float lo, float hi) {
    uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    a += 0x7FFFu + ((a >> 16) & 1u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (a >> 16) | (b & 0xFFFF0000u);
}

// ---------------------------------------------------------------- sizes
struct Dims {
    int64_t T, d, f, E, k, e_lo, e_hi;
    __host__ __device__ int64_t EL() const { return e_hi - e_lo; }
    __host__ __device__ int64_t cap() const { return T * k; }                       // worst-case local rows
    __host__ __device__ int64_t max_mtiles() const { return (cap() + EL() * (BM - 1)) / BM; }
    // rows of the packed activation buffers: every expert segment starts on a
    // 32-row boundary
    __host__ __device__ int64_t pcap() const { return (cap() + EL() * 31 + 31) / 32 * 32; }
    __host__ __device__ int64_t nt_gu() const { return f / BN_GU; }
    __host__ __device__ int64_t nt_dn() const { return d / BN_DN; }
    // K parts of a cut down tile: deep down GEMMs (f >= 8192) are cut into 4
    // (2 when f is not a multiple of 512), each part an even number of
    // 64-deep stages; only the tiles of the schedule's last partial round are
    // cut (dn_split_tiles).  1 = never cut.
    __host__ __device__ int dn_parts() const {
        return f < 8192 ? 1 : f % 512 == 0 ? 4 : f % 256 == 0 ? 2 : 1;
    }
    __host__ __device__ int64_t perm_blocks() const { return (T + PERM_TB - 1) / PERM_TB; }
    __host__ __device__ int64_t comb_blocks() const { return (T + COMB_TOK - 1) / COMB_TOK; }
};

// An m-tile of the grouped GEMM: rows [row0, row0 + rows) of expert e.
struct MTile {
    int32_t e, row0, rows;
    int32_t prow0;  // first row in the packed buffers (x_perm, h): multiple of 32
};

// Byte offsets of every region in a workspace (each 256-byte aligned).
struct Layout {
    size_t status, queues, gu_done, gu_xcd, dn_cg, dn_flag, dn_cnt, dn_part, order_tab, order_tmp,
        route, ids, gates,
        blk_counts,
        blk_base, arrive, counts, offsets, pstart, perm_src, inv_perm, mtiles, n_mtiles, mtile_base,
        x_perm,
        h, y, total;
};

enum LayoutKind { LAYOUT_PERMUTE = 0, LAYOUT_FFN = 1, LAYOUT_LAYER = 2 };
Layout make_layout(const Dims &D, LayoutKind kind);

template <typename T>
__host__ __device__ inline T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

// ---------------------------------------------------------------- launches
// All return hipSuccess or the launch error.
struct ScanArgs;  // scan.h
enum { PREP_NONE = 0, PREP_SCAN_DONE = 1, PREP_ARRIVE_CLEARED = 2 };

// Router.  With logits != NULL, or without a large enough workspace when the
// fast path applies, every logit is evaluated in the defined order; otherwise
// E <= 16 uses the LDS-staged exact kernel and E > 16 the MFMA + exact-refine
// fast path (same ids and gates).  With scan != NULL the router also takes
// over part of the permute's dispatch scan and says how much in *prep:
//  - PREP_SCAN_DONE (E <= 16 token-lane path): it counted the histogram
//    (scan->blk_counts, per token block of PERM_TB tokens and local expert)
//    and its last workgroup ran the whole scan;
//  - PREP_ARRIVE_CLEARED (fast path): it set *scan->arrive to zero, so the
//    permute's histogram kernel can run the scan in its last workgroup;
//  - PREP_NONE: nothing (scan's buffers untouched).
size_t route_workspace_bytes(const Dims &D);
bool route_uses_fast_path(const Dims &D);
int route_splits(const Dims &D);
hipError_t launch_route(const Dims &D, const bf16_t *x, const bf16_t *w_router, const float *bias,
                        int32_t *ids, float *gates, float *logits, void *ws, size_t ws_bytes,
                        hipStream_t s, const ScanArgs *scan = nullptr, int *prep = nullptr);

// The fast router's approximate logits and their error bounds (E > 16 with a
// workspace of route_workspace_bytes): approx, eps [T, E].
hipError_t launch_route_bounds(const Dims &D, const bf16_t *x, const bf16_t *w_router,
                               const float *bias, float *approx, float *eps, void *ws,
                               hipStream_t s);

// Matrix-core probe (probe.hip): kind 0 bf16 32x32x16, kind 1 E4M3 32x32x64.
hipError_t launch_probe_mfma_rate(int64_t workgroups, int iters, uint32_t seed, float *sink,
                                  hipStream_t s);
hipError_t launch_probe_mfma(int kind, int64_t n, int steps, const void *a, const void *b,
                             const float *c, float *d, hipStream_t s);

// Permute.  With pstart != NULL (the fused layer) x_perm is written in the
// packed fragment layout of gemm_pa.h at the 32-aligned segment starts
// pstart[] (not at all when x_perm is NULL: gather-on-load dispatch), and the
// GEMM m-tile table is built and the scheduler state of the persistent kernel
// cleared; otherwise x_perm is row-major at offsets[] (not written when
// NULL: only the indices are produced).  prep: what the router already did
// (launch_route); arrive: the arrival counter it cleared.
hipError_t launch_permute(const Dims &D, const bf16_t *x, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *perm_src, int32_t *inv_perm, bf16_t *x_perm,
                          int32_t *blk_counts, int32_t *blk_base, int32_t *pstart,
                          MTile *mtiles, int32_t *n_mtiles, int32_t *mtile_base,
                          int32_t *sched_state, int64_t sched_state_ints, hipStream_t s,
                          int prep = PREP_NONE, int32_t *arrive = nullptr);

// Staged FFN: m-tile table and pstart[] from offsets[], then the row-major
// x_perm repacked into xp (packed, pcap rows).
// It also clears `clear_ints` ints at `clear` (the split down tiles' counters).
hipError_t launch_build_mtiles(const Dims &D, const int32_t *offsets, MTile *mtiles,
                               int32_t *n_mtiles, int32_t *mtile_base, int32_t *pstart,
                               int32_t *clear, int64_t clear_ints, hipStream_t s);
hipError_t launch_pack_rows(const Dims &D, const bf16_t *x_perm, const int32_t *offsets,
                            const int32_t *pstart, bf16_t *xp, hipStream_t s);

// Grouped GEMMs over packed activations: h (packed) from xp; y (row-major at
// the m-tiles' row0) from h.
hipError_t launch_gemm_gate_up(const Dims &D, const bf16_t *xp, const MTile *mtiles,
                               const int32_t *n_mtiles, const int32_t *mtile_base,
                               const bf16_t *w_gate, const bf16_t *w_up, bf16_t *h, hipStream_t s);
// Cut down tiles (dn_split_tiles with G = grid) meet through dn_cnt
// (cleared, one int per cut tile) and the float32 partials dn_part
// (CUT_MAX x 256 KiB per cut tile).
hipError_t launch_gemm_down(const Dims &D, const bf16_t *h, const MTile *mtiles,
                            const int32_t *n_mtiles, const int32_t *mtile_base,
                            const bf16_t *w_down, bf16_t *y, int32_t *dn_cnt, float *dn_part,
                            int grid, hipStream_t s);

hipError_t launch_combine(const Dims &D, const bf16_t *y_perm, const int32_t *inv_perm,
                          const float *gates, void *out, bool out_f32, hipStream_t s);

// W8A8 (fp8.hip): per-row E4M3 quantisation, row-major or into the packed
// layout at the segment starts pstart[] (rows of a row-major matrix with K
// columns grouped by offsets[]; row maxima computed first into amax, or
// given there when have_amax), and the grouped E4M3 GEMMs: h rows [cap][f]
// (and their row maxima, atomically into the zeroed hmax) from packed x
// codes, y rows [cap][d] from packed h codes.
hipError_t launch_quant_rows(int64_t rows, int64_t cols, const bf16_t *x, uint8_t *q,
                             float *scale, hipStream_t s);
// With row_map (the permute's perm_src), src holds map_rows unpermuted rows
// (the tokens' x) and routed row r is read from src row row_map[r]: each row
// is quantised once, however many slots use it, with the same codes.
hipError_t launch_quant_pack(const Dims &D, int64_t K, const bf16_t *src, const int32_t *offsets,
                             const int32_t *pstart, float *amax, bool have_amax, uint8_t *dst,
                             float *scale, hipStream_t s, const int32_t *row_map = nullptr,
                             int64_t map_rows = 0);
hipError_t launch_gemm_gate_up_f8(const Dims &D, const uint8_t *xq, const float *sx,
                                  const MTile *mtiles, const int32_t *n_mtiles,
                                  const int32_t *mtile_base,
                                  const uint8_t *wg, const float *sg, const uint8_t *wu,
                                  const float *su, bf16_t *h, uint32_t *hmax, hipStream_t s);
hipError_t launch_gemm_down_f8(const Dims &D, const uint8_t *hq, const float *sh,
                               const MTile *mtiles, const int32_t *n_mtiles,
                               const int32_t *mtile_base, const uint8_t *wd,
                               const float *sd, bf16_t *y, hipStream_t s);

struct LayerArgs {
    Dims D;
    const bf16_t *x_perm, *w_gate, *w_up, *w_down;
    // gather-on-load dispatch: gate/up tiles read their rows of x through
    // perm_src (x_perm is not written); 0 = packed x_perm from the permute
    int gather;
    // tile order (moe_tile_order): 0 by kind, 1 ready down tiles of the own
    // XCD's range taken between gate/up tiles, 2 one merged stream with a
    // dependency lead, 3 down tiles by combine column group, ready combine
    // tiles first
    int order;
    int lead;          // order 2: the lead in gate/up tiles
    int chunks;        // order 4: token chunks
    uint32_t perturb;  // schedule perturbation seed (0 = off)
    // orders 2 to 4: claim table built on the device (build_order_kernel):
    // order 2 the merged stream (gate/up index, or down claim | 1 << 30),
    // order 3 the down claims of every XCD range sorted by column group,
    // order 4 the chunked stream (as order 2, combine tiles | 1 << 29)
    int32_t *order_tab;
    int32_t *order_tmp;  // order 2: scratch of the table builder
    int32_t *dn_cg;      // published down tiles per combine column group (cleared per call)
    const bf16_t *x;
    const int32_t *perm_src;
    bf16_t *h, *y;
    const int32_t *ids, *inv_perm, *offsets, *mtile_base, *n_mtiles;
    const float *gates;
    const MTile *mtiles;
    int32_t *queues, *gu_done, *gu_xcd, *dn_flag, *dn_cnt, *status;
    float *dn_part;
    int32_t *dn_done;  // published down tiles (in the status block, cleared per call)
    void *out;
    int out_f32;
    int64_t wait_ticks;  // flag-wait timeout in wall_clock64 ticks
    int64_t *trace;      // optional per-tile trace: [0] = record count, then records
    int64_t trace_cap;   // records that fit after the count
};
hipError_t launch_layer_persistent(const LayerArgs &a, int grid, hipStream_t s);

// The W8A8 persistent kernel (layer.hip): b carries the shared state (the
// m-tile table, queues -- four kinds here --, gu_done/gu_xcd, dn_flag,
// dn_done, status, y, the combine inputs and output; b.order must be 0),
// plus the packed x codes and scales, the E4M3 weights and their row scales,
// h with its row maxima, h's packed codes and scales and the per-m-tile
// count of quantised row blocks.
struct LayerF8Args {
    LayerArgs b;
    const uint8_t *xq;
    const float *sx;
    const uint8_t *wg, *wu, *wd;
    const float *sg, *su, *sd;
    bf16_t *h;        // [cap][f] row-major
    uint32_t *hmax;   // [cap] float bits of max |h| per row (zero before the call)
    uint8_t *hq;      // packed codes of h
    float *sh;        // [pcap] row scales of hq
    int32_t *q_done;  // [MT] finished quantisation tiles per m-tile
    int32_t *q_xcd;   // [MT] XCDs that ran them
    int qrb;          // row blocks of 32 per quantisation tile: 1, 2, 4 or 8
};
// Row blocks of 32 per m-tile.
constexpr int QB_PER_MT = BM / 32;
// Row blocks per quantisation tile: enough rows for about 256 Ki elements
// of h (a tile's fixed costs -- the wait, the acquire, the publish -- then
// stay small against its memory traffic), at most one m-tile.
inline int quant_tile_row_blocks(int64_t f) {
    int q = 1;
    while (q < QB_PER_MT && (int64_t)q * 32 * f < (int64_t)1 << 18) q *= 2;
    return q;
}
hipError_t launch_layer_f8_persistent(const LayerF8Args &a, int grid, hipStream_t s);
// The claim table of tile orders 2 to 4 (a.order_tab), from the m-tile table
// on the device; nothing for the other orders.
hipError_t launch_build_order(const LayerArgs &a, int grid, hipStream_t s);
// Column groups of the combine tiles (COMB_CB column blocks each).
__host__ __device__ inline int64_t comb_groups(int64_t d) {
    return (d / BN_DN + COMB_CB - 1) / COMB_CB;
}
// Largest column-group count tile order 3 supports (its table builder keeps
// per-thread counts of every group in LDS).
constexpr int ORDER3_MAX_CG = 15;  // + 1 key for the cut tiles' parts
// Largest chunk count of tile order 4 (its table builder keeps per-thread
// counts of every (chunk, kind) key in LDS).
constexpr int ORDER4_MAX_CHUNKS = 8;
int layer_grid_size();  // resident workgroups of the persistent kernel (cached)
int64_t wall_clock_hz(); // frequency of wall_clock64 on the current device (cached)

}  // namespace moe
