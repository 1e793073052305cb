// Host runtime of the C ABI declared in include/moe.h: argument checks (run
// before any HIP call, so they also work on a machine without a GPU),
// workspace layout and the launch sequences of every entry point.  Nothing is
// kept between calls but a per-device property cache (grid size, clock rate):
// every option travels with its call.
#include <algorithm>
#include <mutex>

#include "moe_internal.h"
#include "scan.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout make_layout(const Dims &D, LayoutKind kind) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t Tk = (size_t)(D.T * D.k), EL = (size_t)D.EL(), cap = (size_t)D.cap();
    const size_t MT = (size_t)D.max_mtiles();
    const bool layer = kind == LAYOUT_LAYER;
    const bool ffn = kind == LAYOUT_FFN || layer;
    const bool perm = kind == LAYOUT_PERMUTE || layer;
    // scheduler state first and contiguous (cleared by one kernel)
    L.status = take(ffn ? 256 : 0);  // offset 0 of layer and FFN workspaces
    L.queues = take(layer ? 3 * NUM_XCD * QSTRIDE * sizeof(int32_t) : 0);
    L.gu_done = take(layer ? MT * sizeof(int32_t) : 0);
    L.gu_xcd = take(layer ? MT * sizeof(int32_t) : 0);
    L.dn_cg = take(layer ? (size_t)comb_groups(D.d) * sizeof(int32_t) : 0);
    L.dn_flag = take(layer ? MT * (size_t)D.nt_dn() * sizeof(int32_t) : 0);
    // cut down tiles (deep down GEMMs only): arrival counters, then partials
    const bool split = ffn && D.dn_parts() > 1;
    L.dn_cnt = take(split ? SPLIT_MAX * sizeof(int32_t) : 0);
    L.dn_part = take(split ? (size_t)SPLIT_MAX * CUT_MAX * BM * BN_DN * sizeof(float) : 0);
    // claim tables of tile orders 2 and 3 (written whole by their builder)
    const size_t n1max = MT * (size_t)D.nt_gu();
    const size_t n2max = MT * (size_t)D.nt_dn() + (CUT_MAX - 1) * (size_t)SPLIT_MAX;
    const size_t n3 = (size_t)(D.comb_blocks() * comb_groups(D.d));
    L.order_tab = take(layer ? (n1max + n2max + n3) * sizeof(int32_t) : 0);
    L.order_tmp = take(layer ? std::max(n2max, (size_t)D.comb_blocks()) * sizeof(int32_t) : 0);
    L.route = take(layer ? route_workspace_bytes(D) : 0);
    L.ids = take(layer ? Tk * sizeof(int32_t) : 0);
    L.gates = take(layer ? Tk * sizeof(float) : 0);
    L.blk_counts = take(perm ? (size_t)D.perm_blocks() * EL * sizeof(int32_t) : 0);
    L.blk_base = take(perm ? (size_t)D.perm_blocks() * EL * sizeof(int32_t) : 0);
    L.arrive = take(layer ? sizeof(int32_t) : 0);
    L.counts = take(layer ? EL * sizeof(int32_t) : 0);
    L.offsets = take(layer ? (EL + 1) * sizeof(int32_t) : 0);
    L.pstart = take(ffn ? (EL + 1) * sizeof(int32_t) : 0);
    L.perm_src = take(layer ? cap * sizeof(int32_t) : 0);
    L.inv_perm = take(layer ? Tk * sizeof(int32_t) : 0);
    L.mtiles = take(ffn ? MT * sizeof(MTile) : 0);
    L.n_mtiles = take(ffn ? sizeof(int32_t) : 0);
    L.mtile_base = take(ffn ? EL * sizeof(int32_t) : 0);
    // packed activations (gemm_pa.h): x_perm gathered (layer) or repacked
    // from the caller's rows (staged FFN), and h
    const size_t pcap = (size_t)D.pcap();
    L.x_perm = take(ffn ? pcap * (size_t)D.d * 2 : 0);
    L.h = take(ffn ? pcap * (size_t)D.f * 2 : 0);
    L.y = take(layer ? cap * (size_t)D.d * 2 : 0);
    L.total = off;
    return L;
}

}  // namespace moe

using namespace moe;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_dims(const moe_dims *dm, Dims *out) {
    if (!dm) return MOE_ERR_INVALID_ARG;
    Dims D{dm->T, dm->d, dm->f, dm->E, dm->k, dm->e_lo, dm->e_hi};
    if (D.T < 0 || D.d <= 0 || D.f <= 0 || D.E <= 0 || D.k <= 0 || D.k > D.E || D.e_lo < 0 ||
        D.e_hi > D.E || D.e_lo >= D.e_hi)
        return MOE_ERR_INVALID_ARG;
    if (D.E > 1024 || D.k > 64 || D.d % 256 != 0 || D.f % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (D.T * D.k >= (int64_t(1) << 31) || D.cap() * D.d >= (int64_t(1) << 40) ||
        D.d >= (1 << 20) || D.f >= (1 << 20))
        return MOE_ERR_UNSUPPORTED;
    *out = D;
    return MOE_OK;
}

moe_status check_ws(void *ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MOE_OK;
    if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < need) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Range checks of per-call options; the W8A8 layer takes events only.
moe_status check_opts(const moe_layer_opts *o, bool fp8) {
    if (!o) return MOE_OK;
    if (fp8) {
        if (o->dispatch || o->tile_order || o->lead || o->chunks) return MOE_ERR_INVALID_ARG;
        if (o->schedule == MOE_SCHEDULE_STAGED || o->schedule == MOE_SCHEDULE_AUTO)
            // separate launches: no tiles to perturb, bound or trace
            return o->perturb_seed || o->wait_timeout_us || o->trace || o->trace_records
                       ? MOE_ERR_INVALID_ARG
                       : MOE_OK;
        if (o->schedule != MOE_SCHEDULE_PERSISTENT || o->wait_timeout_us < 0 ||
            o->trace_records < 0 || (o->trace_records > 0 && !o->trace))
            return MOE_ERR_INVALID_ARG;
        return MOE_OK;
    }
    if (o->schedule != MOE_SCHEDULE_AUTO && o->schedule != MOE_SCHEDULE_PERSISTENT)
        return MOE_ERR_INVALID_ARG;
    if (o->dispatch != MOE_DISPATCH_PACKED && o->dispatch != MOE_DISPATCH_GATHER)
        return MOE_ERR_INVALID_ARG;
    if (o->tile_order < MOE_ORDER_BY_KIND || o->tile_order > MOE_ORDER_CHUNKED)
        return MOE_ERR_INVALID_ARG;
    if (o->lead < 0 || o->chunks < 0 || o->chunks > ORDER4_MAX_CHUNKS || o->wait_timeout_us < 0 ||
        o->trace_records < 0)
        return MOE_ERR_INVALID_ARG;
    if (o->trace_records > 0 && !o->trace) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// The scratch of moe_permute_noalloc: a file-scope device array, one copy per
// GPU, kept until the process ends.  Host code never passes its name to a
// kernel (on the host that name is only a stand-in): the device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and kept per device.
constexpr int64_t NOALLOC_SCRATCH_INTS = 1 << 18;  // 1 MiB
static __device__ __align__(256) int32_t scratch[NOALLOC_SCRATCH_INTS];
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

moe_status noalloc_scratch(int32_t **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Records opts->events[i] (if given) on the stream.
hipError_t mark_event(const moe_layer_opts *o, int i, hipStream_t s) {
    if (!o || !o->events[i]) return hipSuccess;
    return hipEventRecord((hipEvent_t)o->events[i], s);
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported dimensions";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_DEVICE_TIMEOUT: return "device-side flag wait timed out";
    }
    return "unknown status";
}

int moe_version(void) { return 100; }

size_t moe_route_workspace_bytes(const moe_dims *dims) {
    Dims D;
    if (check_dims(dims, &D) != MOE_OK) return 0;
    return route_workspace_bytes(D);
}

moe_status moe_route(const moe_dims *dims, const void *x, const void *w_router, const float *bias,
                     int32_t *topk_ids, float *topk_w, float *logits, void *ws, size_t ws_bytes,
                     void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (D.T == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
    if (ws && ((uintptr_t)ws & 255u) != 0) return MOE_ERR_WORKSPACE;
    return hip_status(launch_route(D, (const bf16_t *)x, (const bf16_t *)w_router, bias, topk_ids,
                                   topk_w, logits, ws, ws ? ws_bytes : 0, (hipStream_t)stream));
}

moe_status moe_route_bounds(const moe_dims *dims, const void *x, const void *w_router,
                            const float *bias, float *approx, float *eps, void *ws,
                            size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (!route_uses_fast_path(D)) return MOE_ERR_UNSUPPORTED;
    if (D.T == 0) return MOE_OK;
    if (!x || !w_router || !approx || !eps) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
    if ((st = check_ws(ws, ws_bytes, route_workspace_bytes(D))) != MOE_OK) return st;
    return hip_status(launch_route_bounds(D, (const bf16_t *)x, (const bf16_t *)w_router, bias,
                                          approx, eps, ws, (hipStream_t)stream));
}

moe_status moe_probe_mfma(int kind, int64_t n, int steps, const void *a, const void *b,
                          const float *c, float *d, void *stream) {
    if ((kind != 0 && kind != 1) || n < 0 || n >= ((int64_t)1 << 31) || steps < 1 ||
        steps > 4096)
        return MOE_ERR_INVALID_ARG;
    if (n == 0) return MOE_OK;
    if (!a || !b || !c || !d || !aligned16(a) || !aligned16(b) || !aligned16(c) || !aligned16(d))
        return MOE_ERR_INVALID_ARG;
    return hip_status(launch_probe_mfma(kind, n, steps, a, b, c, d, (hipStream_t)stream));
}

moe_status moe_probe_mfma_rate(int64_t workgroups, int iters, uint32_t seed, float *sink,
                               void *stream) {
    if (workgroups < 0 || workgroups > 65536 || iters < 1 || iters > (1 << 20))
        return MOE_ERR_INVALID_ARG;
    if (workgroups == 0) return MOE_OK;
    if (!sink || !aligned16(sink)) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_probe_mfma_rate(workgroups, iters, seed, sink, (hipStream_t)stream));
}

size_t moe_permute_workspace_bytes(const moe_dims *dims) {
    Dims D;
    if (check_dims(dims, &D) != MOE_OK) return 0;
    return make_layout(D, LAYOUT_PERMUTE).total;
}

moe_status moe_permute(const moe_dims *dims, const void *x, const int32_t *topk_ids,
                       int32_t *counts, int32_t *offsets, int32_t *perm_src, int32_t *inv_perm,
                       void *x_perm, void *ws, size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (D.T > 0 && (!x || !topk_ids || !perm_src || !inv_perm || !x_perm))
        return MOE_ERR_INVALID_ARG;
    if (D.T > 0 && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(D, LAYOUT_PERMUTE);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    return hip_status(launch_permute(D, (const bf16_t *)x, topk_ids, counts, offsets, perm_src,
                                     inv_perm, (bf16_t *)x_perm, at<int32_t>(ws, L.blk_counts),
                                     at<int32_t>(ws, L.blk_base), nullptr, nullptr, nullptr,
                                     nullptr, nullptr, 0, (hipStream_t)stream));
}

size_t moe_permute_noalloc_max_ints(void) { return NOALLOC_SCRATCH_INTS; }

moe_status moe_permute_noalloc(const moe_dims *dims, const void *x, const int32_t *topk_ids,
                               int32_t *counts, int32_t *offsets, int32_t *perm_src,
                               int32_t *inv_perm, void *x_perm, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (D.T > 0 && (!x || !topk_ids || !perm_src || !inv_perm || !x_perm))
        return MOE_ERR_INVALID_ARG;
    if (D.T > 0 && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
    // per-block counts and bases of the permute, both written whole by every call
    const int64_t blk = D.perm_blocks() * D.EL();
    if (2 * blk > NOALLOC_SCRATCH_INTS) return MOE_ERR_UNSUPPORTED;
    int32_t *scr = nullptr;
    if ((st = noalloc_scratch(&scr)) != MOE_OK) return st;
    return hip_status(launch_permute(D, (const bf16_t *)x, topk_ids, counts, offsets, perm_src,
                                     inv_perm, (bf16_t *)x_perm, scr, scr + blk, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, 0, (hipStream_t)stream));
}

size_t moe_expert_ffn_workspace_bytes(const moe_dims *dims) {
    Dims D;
    if (check_dims(dims, &D) != MOE_OK) return 0;
    return make_layout(D, LAYOUT_FFN).total;
}

moe_status moe_expert_ffn(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                          const void *w_gate, const void *w_up, const void *w_down, void *y_perm,
                          void *ws, size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (D.T == 0) return MOE_OK;
    if (!x_perm || !offsets || !w_gate || !w_up || !w_down || !y_perm) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
        !aligned16(y_perm))
        return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(D, LAYOUT_FFN);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    MTile *mt = at<MTile>(ws, L.mtiles);
    int32_t *nmt = at<int32_t>(ws, L.n_mtiles);
    bf16_t *h = at<bf16_t>(ws, L.h);
    int32_t *pstart = at<int32_t>(ws, L.pstart);
    bf16_t *xp = at<bf16_t>(ws, L.x_perm);
    // cleared per call: the status word and the cut down tiles' counters
    const int64_t clear_ints = (int64_t)((L.dn_cnt - L.status) / 4) + (D.dn_parts() > 1 ? SPLIT_MAX : 0);
    hipError_t e = launch_build_mtiles(D, offsets, mt, nmt, at<int32_t>(ws, L.mtile_base), pstart,
                                       at<int32_t>(ws, L.status), clear_ints, s);
    if (e == hipSuccess) e = launch_pack_rows(D, (const bf16_t *)x_perm, offsets, pstart, xp, s);
    if (e == hipSuccess)
        e = launch_gemm_gate_up(D, xp, mt, nmt, at<int32_t>(ws, L.mtile_base),
                                (const bf16_t *)w_gate, (const bf16_t *)w_up, h, s);
    if (e == hipSuccess)
        e = launch_gemm_down(D, h, mt, nmt, at<int32_t>(ws, L.mtile_base),
                             (const bf16_t *)w_down, (bf16_t *)y_perm,
                             at<int32_t>(ws, L.dn_cnt), at<float>(ws, L.dn_part), layer_grid_size(),
                             s);
    return hip_status(e);
}

moe_status moe_quantize_fp8(const void *x, int64_t rows, int64_t cols, void *q, float *scale,
                            void *stream) {
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows * cols >= ((int64_t)1 << 40))
        return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scale || !aligned16(x) || !aligned16(q)) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_rows(rows, cols, (const bf16_t *)x, (uint8_t *)q, scale,
                                        (hipStream_t)stream));
}

namespace {
// Workspace of moe_expert_ffn_fp8 (256-byte aligned regions).
struct Layout8 {
    size_t mtiles, n_mtiles, mtile_base, pstart, amax, hmax, xq, sx, h, hq, sh, total;
};
Layout8 make_layout8(const Dims &D) {
    Layout8 L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t MT = (size_t)D.max_mtiles(), EL = (size_t)D.EL(), pcap = (size_t)D.pcap();
    L.mtiles = take(MT * sizeof(MTile));
    L.n_mtiles = take(sizeof(int32_t));
    L.mtile_base = take(EL * sizeof(int32_t));
    L.pstart = take((EL + 1) * sizeof(int32_t));
    L.amax = take((size_t)D.cap() * sizeof(float));
    L.hmax = take((size_t)D.cap() * sizeof(float));
    L.xq = take(pcap * (size_t)D.d);
    L.sx = take(pcap * sizeof(float));
    L.h = take((size_t)D.cap() * (size_t)D.f * 2);
    L.hq = take(pcap * (size_t)D.f);
    L.sh = take(pcap * sizeof(float));
    L.total = off;
    return L;
}
moe_status check_dims_fp8(const moe_dims *dims, Dims *D) {
    moe_status st = check_dims(dims, D);
    if (st != MOE_OK) return st;
    if (D->f % 256 != 0) return MOE_ERR_UNSUPPORTED;  // K of both GEMMs: whole 256-byte stage pairs
    return MOE_OK;
}
}  // namespace

namespace {
// The launches of the W8A8 FFN over a Layout8 workspace at ws.
// x_perm: the routed rows, row-major; or, with perm_src, x_perm is the tokens'
// x and routed row r is token perm_src[r] (each token quantised once).
hipError_t run_ffn_fp8(const Dims &D, const bf16_t *x_perm, const int32_t *offsets,
                       const uint8_t *wq_gate, const float *s_gate, const uint8_t *wq_up,
                       const float *s_up, const uint8_t *wq_down, const float *s_down,
                       bf16_t *y_perm, void *ws, hipStream_t s,
                       const int32_t *perm_src = nullptr) {
    const Layout8 L = make_layout8(D);
    MTile *mt = at<MTile>(ws, L.mtiles);
    int32_t *nmt = at<int32_t>(ws, L.n_mtiles);
    int32_t *pstart = at<int32_t>(ws, L.pstart);
    uint8_t *xq = at<uint8_t>(ws, L.xq), *hq = at<uint8_t>(ws, L.hq);
    float *sx = at<float>(ws, L.sx), *sh = at<float>(ws, L.sh);
    bf16_t *h = at<bf16_t>(ws, L.h);
    // the tile-table kernel also zeroes h's row maxima (atomic max targets)
    hipError_t e = launch_build_mtiles(D, offsets, mt, nmt, at<int32_t>(ws, L.mtile_base), pstart,
                                       at<int32_t>(ws, L.hmax), D.cap(), s);
    if (e == hipSuccess)
        e = launch_quant_pack(D, D.d, x_perm, offsets, pstart, at<float>(ws, L.amax), false, xq, sx,
                              s, perm_src, perm_src ? D.T : 0);
    if (e == hipSuccess)
        e = launch_gemm_gate_up_f8(D, xq, sx, mt, nmt, at<int32_t>(ws, L.mtile_base), wq_gate,
                                   s_gate, wq_up, s_up, h,
                                   at<uint32_t>(ws, L.hmax), s);
    if (e == hipSuccess)
        e = launch_quant_pack(D, D.f, h, offsets, pstart, at<float>(ws, L.hmax), true, hq, sh, s);
    if (e == hipSuccess)
        e = launch_gemm_down_f8(D, hq, sh, mt, nmt, at<int32_t>(ws, L.mtile_base), wq_down, s_down,
                                y_perm, s);
    return e;
}

// Workspace of moe_layer_fp8: the persistent kernel's scheduler state first
// (status word at offset 0; cleared by the dispatch scan in one range, h's
// row maxima included), routing and permute indices, y rows, then the FFN's
// Layout8 region (m-tile table, packed codes and scales, h).
struct LayoutL8 {
    size_t status, queues, gu_done, gu_xcd, q_done, q_xcd, dn_flag, hmax, sched_end, route, ids,
        gates, blk_counts, blk_base, arrive, counts, offsets, perm_src, inv_perm, y, ffn, total;
};
LayoutL8 make_layout_l8(const Dims &D) {
    LayoutL8 L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t Tk = (size_t)(D.T * D.k), EL = (size_t)D.EL(), cap = (size_t)D.cap();
    const size_t MT = (size_t)D.max_mtiles();
    L.status = take(256);
    L.queues = take(4 * NUM_XCD * QSTRIDE * sizeof(int32_t));
    L.gu_done = take(MT * sizeof(int32_t));
    L.gu_xcd = take(MT * sizeof(int32_t));
    L.q_done = take(MT * sizeof(int32_t));
    L.q_xcd = take(MT * sizeof(int32_t));
    L.dn_flag = take(MT * (size_t)D.nt_dn() * sizeof(int32_t));
    L.hmax = take(cap * sizeof(uint32_t));
    L.sched_end = off;
    L.route = take(route_workspace_bytes(D));
    L.ids = take(Tk * sizeof(int32_t));
    L.gates = take(Tk * sizeof(float));
    L.blk_counts = take((size_t)D.perm_blocks() * EL * sizeof(int32_t));
    L.blk_base = take((size_t)D.perm_blocks() * EL * sizeof(int32_t));
    L.arrive = take(sizeof(int32_t));
    L.counts = take(EL * sizeof(int32_t));
    L.offsets = take((EL + 1) * sizeof(int32_t));
    L.perm_src = take(cap * sizeof(int32_t));
    L.inv_perm = take(Tk * sizeof(int32_t));
    L.y = take(cap * (size_t)D.d * 2);
    L.ffn = take(make_layout8(D).total);
    L.total = off;
    return L;
}
}  // namespace

size_t moe_layer_fp8_workspace_bytes(const moe_dims *dims) {
    Dims D;
    if (check_dims_fp8(dims, &D) != MOE_OK) return 0;
    return make_layout_l8(D).total;
}

moe_status moe_layer_fp8(const moe_dims *dims, const void *x, const void *w_router,
                         const float *bias, const void *wq_gate, const float *s_gate,
                         const void *wq_up, const float *s_up, const void *wq_down,
                         const float *s_down, void *out, moe_dtype out_dtype,
                         int32_t *topk_ids_out, float *topk_w_out, void *ws, size_t ws_bytes,
                         const moe_layer_opts *opts, void *stream) {
    Dims D;
    moe_status st = check_dims_fp8(dims, &D);
    if (st != MOE_OK) return st;
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
    if ((st = check_opts(opts, true)) != MOE_OK) return st;
    if (D.T == 0) return MOE_OK;
    if (!x || !w_router || !wq_gate || !s_gate || !wq_up || !s_up || !wq_down || !s_down || !out)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(wq_gate) || !aligned16(wq_up) ||
        !aligned16(wq_down) || !aligned16(out))
        return MOE_ERR_INVALID_ARG;
    const LayoutL8 L = make_layout_l8(D);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    moe_layer_opts o{};
    if (opts) o = *opts;
    const bool persistent = o.schedule == MOE_SCHEDULE_PERSISTENT;
    const int grid = persistent ? layer_grid_size() : 0;
    if (persistent && grid <= 0) return MOE_ERR_HIP;
    int32_t *ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
    float *gates = topk_w_out ? topk_w_out : at<float>(ws, L.gates);
    int32_t *offsets = at<int32_t>(ws, L.offsets), *inv_perm = at<int32_t>(ws, L.inv_perm);
    bf16_t *y = at<bf16_t>(ws, L.y);
    int32_t *perm_src = at<int32_t>(ws, L.perm_src);
    char *ffn = at<char>(ws, L.ffn);
    const Layout8 F = make_layout8(D);
    // The persistent schedule has the dispatch scan build the m-tile table
    // and clear its scheduler state; the staged FFN builds its own table.
    int32_t *pstart = persistent ? at<int32_t>(ffn, F.pstart) : nullptr;
    MTile *mt = persistent ? at<MTile>(ffn, F.mtiles) : nullptr;
    int32_t *nmt = persistent ? at<int32_t>(ffn, F.n_mtiles) : nullptr;
    int32_t *mtile_base = persistent ? at<int32_t>(ffn, F.mtile_base) : nullptr;
    int32_t *sched = persistent ? at<int32_t>(ws, L.status) : nullptr;
    const int64_t sched_ints = persistent ? (int64_t)((L.sched_end - L.status) / 4) : 0;
    // the router may also take over the permute's histogram and scan
    const ScanArgs sa = make_scan_args(D, at<int32_t>(ws, L.blk_counts), at<int32_t>(ws, L.blk_base),
                                       at<int32_t>(ws, L.counts), offsets, pstart, mt, nmt,
                                       mtile_base, sched, sched_ints, at<int32_t>(ws, L.arrive));
    int prep = PREP_NONE;
    hipError_t e = mark_event(opts, 0, s);
    if (e == hipSuccess)
        e = launch_route(D, (const bf16_t *)x, (const bf16_t *)w_router, bias, ids, gates, nullptr,
                         at<char>(ws, L.route), route_workspace_bytes(D), s, &sa, &prep);
    if (e == hipSuccess) e = mark_event(opts, 1, s);
    // No x_perm: each token's row of x is quantised once and its codes placed
    // at every routed row of that token through perm_src.
    if (e == hipSuccess)
        e = launch_permute(D, (const bf16_t *)x, ids, at<int32_t>(ws, L.counts), offsets, perm_src,
                           inv_perm, nullptr, at<int32_t>(ws, L.blk_counts),
                           at<int32_t>(ws, L.blk_base), pstart, mt, nmt, mtile_base, sched,
                           sched_ints, s, prep, sa.arrive);
    if (e == hipSuccess) e = mark_event(opts, 2, s);
    if (!persistent) {
        if (e == hipSuccess)
            e = run_ffn_fp8(D, (const bf16_t *)x, offsets, (const uint8_t *)wq_gate, s_gate,
                            (const uint8_t *)wq_up, s_up, (const uint8_t *)wq_down, s_down, y,
                            ffn, s, perm_src);
        if (e == hipSuccess)
            e = launch_combine(D, y, inv_perm, gates, out, out_dtype == MOE_F32, s);
    } else {
        uint8_t *xq = at<uint8_t>(ffn, F.xq);
        float *sx = at<float>(ffn, F.sx);
        if (e == hipSuccess)
            e = launch_quant_pack(D, D.d, (const bf16_t *)x, offsets, pstart, at<float>(ffn, F.amax),
                                  false, xq, sx, s, perm_src, D.T);
        if (e == hipSuccess) {
            const int64_t wait_us = o.wait_timeout_us > 0 ? o.wait_timeout_us : 2000000;
            LayerF8Args a8{};
            LayerArgs &a = a8.b;
            a.D = D;
            a.perturb = o.perturb_seed;
            a.ids = ids;
            a.inv_perm = inv_perm;
            a.offsets = offsets;
            a.mtile_base = mtile_base;
            a.n_mtiles = nmt;
            a.gates = gates;
            a.mtiles = mt;
            a.queues = at<int32_t>(ws, L.queues);
            a.gu_done = at<int32_t>(ws, L.gu_done);
            a.gu_xcd = at<int32_t>(ws, L.gu_xcd);
            a.dn_flag = at<int32_t>(ws, L.dn_flag);
            a.status = at<int32_t>(ws, L.status);
            a.dn_done = at<int32_t>(ws, L.status) + 32;  // 128 bytes past the status word
            a.y = y;
            a.out = out;
            a.out_f32 = out_dtype == MOE_F32;
            a.wait_ticks = wait_us * (wall_clock_hz() / 1000000);
            a.trace = o.trace_records > 0 ? o.trace : nullptr;
            a.trace_cap = o.trace_records > 0 ? o.trace_records : 0;
            a8.xq = xq;
            a8.sx = sx;
            a8.wg = (const uint8_t *)wq_gate;
            a8.wu = (const uint8_t *)wq_up;
            a8.wd = (const uint8_t *)wq_down;
            a8.sg = s_gate;
            a8.su = s_up;
            a8.sd = s_down;
            a8.h = at<bf16_t>(ffn, F.h);
            a8.hmax = at<uint32_t>(ws, L.hmax);
            a8.hq = at<uint8_t>(ffn, F.hq);
            a8.sh = at<float>(ffn, F.sh);
            a8.q_done = at<int32_t>(ws, L.q_done);
            a8.q_xcd = at<int32_t>(ws, L.q_xcd);
            a8.qrb = quant_tile_row_blocks(D.f);
            e = launch_layer_f8_persistent(a8, grid, s);
        }
    }
    if (e == hipSuccess) e = mark_event(opts, 3, s);
    return hip_status(e);
}

moe_status moe_gate_up_fp8(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                           const void *wq_gate, const float *s_gate, const void *wq_up,
                           const float *s_up, void *h, void *ws, size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims_fp8(dims, &D);
    if (st != MOE_OK) return st;
    if (D.T == 0) return MOE_OK;
    if (!x_perm || !offsets || !wq_gate || !s_gate || !wq_up || !s_up || !h)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm) || !aligned16(wq_gate) || !aligned16(wq_up) || !aligned16(h))
        return MOE_ERR_INVALID_ARG;
    const Layout8 L = make_layout8(D);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    MTile *mt = at<MTile>(ws, L.mtiles);
    int32_t *nmt = at<int32_t>(ws, L.n_mtiles);
    hipError_t e = launch_build_mtiles(D, offsets, mt, nmt, at<int32_t>(ws, L.mtile_base),
                                       at<int32_t>(ws, L.pstart), at<int32_t>(ws, L.hmax), D.cap(),
                                       s);
    if (e == hipSuccess)
        e = launch_quant_pack(D, D.d, (const bf16_t *)x_perm, offsets, at<int32_t>(ws, L.pstart),
                              at<float>(ws, L.amax), false, at<uint8_t>(ws, L.xq),
                              at<float>(ws, L.sx), s);
    if (e == hipSuccess)
        e = launch_gemm_gate_up_f8(D, at<uint8_t>(ws, L.xq), at<float>(ws, L.sx), mt, nmt,
                                   at<int32_t>(ws, L.mtile_base), (const uint8_t *)wq_gate, s_gate,
                                   (const uint8_t *)wq_up, s_up, (bf16_t *)h,
                                   at<uint32_t>(ws, L.hmax), s);
    return hip_status(e);
}

moe_status moe_down_fp8(const moe_dims *dims, const void *h, const int32_t *offsets,
                        const void *wq_down, const float *s_down, void *y_perm, void *ws,
                        size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims_fp8(dims, &D);
    if (st != MOE_OK) return st;
    if (D.T == 0) return MOE_OK;
    if (!h || !offsets || !wq_down || !s_down || !y_perm) return MOE_ERR_INVALID_ARG;
    if (!aligned16(h) || !aligned16(wq_down) || !aligned16(y_perm)) return MOE_ERR_INVALID_ARG;
    const Layout8 L = make_layout8(D);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    MTile *mt = at<MTile>(ws, L.mtiles);
    int32_t *nmt = at<int32_t>(ws, L.n_mtiles);
    hipError_t e = launch_build_mtiles(D, offsets, mt, nmt, at<int32_t>(ws, L.mtile_base),
                                       at<int32_t>(ws, L.pstart), nullptr, 0, s);
    // row maxima of h computed here (moe_expert_ffn_fp8 takes them from the
    // gate/up epilogue: the same values, so the same codes and scales)
    if (e == hipSuccess)
        e = launch_quant_pack(D, D.f, (const bf16_t *)h, offsets, at<int32_t>(ws, L.pstart),
                              at<float>(ws, L.hmax), false, at<uint8_t>(ws, L.hq),
                              at<float>(ws, L.sh), s);
    if (e == hipSuccess)
        e = launch_gemm_down_f8(D, at<uint8_t>(ws, L.hq), at<float>(ws, L.sh), mt, nmt,
                                at<int32_t>(ws, L.mtile_base), (const uint8_t *)wq_down, s_down,
                                (bf16_t *)y_perm, s);
    return hip_status(e);
}

size_t moe_expert_ffn_fp8_workspace_bytes(const moe_dims *dims) {
    Dims D;
    if (check_dims_fp8(dims, &D) != MOE_OK) return 0;
    return make_layout8(D).total;
}

moe_status moe_expert_ffn_fp8(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                              const void *wq_gate, const float *s_gate, const void *wq_up,
                              const float *s_up, const void *wq_down, const float *s_down,
                              void *y_perm, void *ws, size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims_fp8(dims, &D);
    if (st != MOE_OK) return st;
    if (D.T == 0) return MOE_OK;
    if (!x_perm || !offsets || !wq_gate || !s_gate || !wq_up || !s_up || !wq_down || !s_down ||
        !y_perm)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm) || !aligned16(wq_gate) || !aligned16(wq_up) || !aligned16(wq_down) ||
        !aligned16(y_perm))
        return MOE_ERR_INVALID_ARG;
    const Layout8 L = make_layout8(D);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    return hip_status(run_ffn_fp8(D, (const bf16_t *)x_perm, offsets, (const uint8_t *)wq_gate,
                                  s_gate, (const uint8_t *)wq_up, s_up, (const uint8_t *)wq_down,
                                  s_down, (bf16_t *)y_perm, ws, (hipStream_t)stream));
}

moe_status moe_combine(const moe_dims *dims, const void *y_perm, const int32_t *inv_perm,
                       const float *topk_w, void *out, moe_dtype out_dtype, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
    if (D.T == 0) return MOE_OK;
    if (!y_perm || !inv_perm || !topk_w || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(y_perm) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_combine(D, (const bf16_t *)y_perm, inv_perm, topk_w, out,
                                     out_dtype == MOE_F32, (hipStream_t)stream));
}

size_t moe_layer_workspace_bytes(const moe_dims *dims) {
    Dims D;
    if (check_dims(dims, &D) != MOE_OK) return 0;
    return make_layout(D, LAYOUT_LAYER).total;
}

moe_status moe_layer(const moe_dims *dims, const void *x, const void *w_router, const float *bias,
                     const void *w_gate, const void *w_up, const void *w_down, void *out,
                     moe_dtype out_dtype, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                     size_t ws_bytes, const moe_layer_opts *opts, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
    if ((st = check_opts(opts, false)) != MOE_OK) return st;
    if (opts && opts->tile_order == MOE_ORDER_COMBINE_FIRST && comb_groups(D.d) > ORDER3_MAX_CG)
        return MOE_ERR_UNSUPPORTED;
    if (D.T == 0) return MOE_OK;
    if (!x || !w_router || !w_gate || !w_up || !w_down || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
        !aligned16(w_down) || !aligned16(out))
        return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(D, LAYOUT_LAYER);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;

    const int grid = layer_grid_size();
    if (grid <= 0) return MOE_ERR_HIP;
    moe_layer_opts o{};
    if (opts) o = *opts;
    // 32-bit buffer offsets address x in gather mode
    const bool gather = o.dispatch == MOE_DISPATCH_GATHER && D.T * D.d * 2 < ((int64_t)1 << 31);
    const int64_t wait_us = o.wait_timeout_us > 0 ? o.wait_timeout_us : 2000000;

    int32_t *ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
    float *gates = topk_w_out ? topk_w_out : at<float>(ws, L.gates);
    int32_t *offsets = at<int32_t>(ws, L.offsets);
    MTile *mt = at<MTile>(ws, L.mtiles);
    int32_t *nmt = at<int32_t>(ws, L.n_mtiles);
    int32_t *mtile_base = at<int32_t>(ws, L.mtile_base);
    int32_t *inv_perm = at<int32_t>(ws, L.inv_perm);
    bf16_t *x_perm = at<bf16_t>(ws, L.x_perm);
    const int64_t sched_ints =
        D.dn_parts() > 1 ? (int64_t)((L.dn_cnt - L.status) / 4) + SPLIT_MAX
                    : (int64_t)((L.dn_flag - L.status) / 4) + D.max_mtiles() * D.nt_dn();

    // the router may also take over the permute's histogram and scan
    const ScanArgs sa = make_scan_args(D, at<int32_t>(ws, L.blk_counts), at<int32_t>(ws, L.blk_base),
                                       at<int32_t>(ws, L.counts), offsets, at<int32_t>(ws, L.pstart),
                                       mt, nmt, mtile_base, at<int32_t>(ws, L.status), sched_ints,
                                       at<int32_t>(ws, L.arrive));
    int prep = PREP_NONE;
    hipError_t e = mark_event(opts, 0, s);
    if (e == hipSuccess)
        e = launch_route(D, (const bf16_t *)x, (const bf16_t *)w_router, bias, ids, gates, nullptr,
                         at<char>(ws, L.route), route_workspace_bytes(D), s, &sa, &prep);
    if (e == hipSuccess) e = mark_event(opts, 1, s);
    if (e == hipSuccess)
        e = launch_permute(D, (const bf16_t *)x, ids, at<int32_t>(ws, L.counts), offsets,
                           at<int32_t>(ws, L.perm_src), inv_perm, gather ? nullptr : x_perm,
                           at<int32_t>(ws, L.blk_counts), at<int32_t>(ws, L.blk_base),
                           at<int32_t>(ws, L.pstart), mt, nmt, mtile_base,
                           at<int32_t>(ws, L.status), sched_ints, s, prep, sa.arrive);
    if (e == hipSuccess) e = mark_event(opts, 2, s);
    if (e == hipSuccess) {
        LayerArgs a;
        a.D = D;
        a.x_perm = x_perm;
        a.gather = gather ? 1 : 0;
        a.order = o.tile_order;
        a.lead = o.lead > 0 ? o.lead : grid;
        a.chunks = o.chunks > 0 ? o.chunks : 4;
        a.perturb = o.perturb_seed;
        a.x = (const bf16_t *)x;
        a.perm_src = at<int32_t>(ws, L.perm_src);
        a.w_gate = (const bf16_t *)w_gate;
        a.w_up = (const bf16_t *)w_up;
        a.w_down = (const bf16_t *)w_down;
        a.h = at<bf16_t>(ws, L.h);
        a.y = at<bf16_t>(ws, L.y);
        a.ids = ids;
        a.inv_perm = inv_perm;
        a.offsets = offsets;
        a.mtile_base = mtile_base;
        a.n_mtiles = nmt;
        a.gates = gates;
        a.mtiles = mt;
        a.queues = at<int32_t>(ws, L.queues);
        a.gu_done = at<int32_t>(ws, L.gu_done);
        a.gu_xcd = at<int32_t>(ws, L.gu_xcd);
        a.dn_flag = at<int32_t>(ws, L.dn_flag);
        a.dn_cnt = at<int32_t>(ws, L.dn_cnt);
        a.dn_part = at<float>(ws, L.dn_part);
        a.status = at<int32_t>(ws, L.status);
        a.dn_done = at<int32_t>(ws, L.status) + 32;  // 128 bytes past the status word
        a.dn_cg = at<int32_t>(ws, L.dn_cg);
        a.order_tab = at<int32_t>(ws, L.order_tab);
        a.order_tmp = at<int32_t>(ws, L.order_tmp);
        a.out = out;
        a.out_f32 = out_dtype == MOE_F32;
        a.wait_ticks = wait_us * (wall_clock_hz() / 1000000);
        a.trace = o.trace_records > 0 ? o.trace : nullptr;
        a.trace_cap = o.trace_records > 0 ? o.trace_records : 0;
        e = launch_build_order(a, grid, s);
        if (e == hipSuccess) e = launch_layer_persistent(a, grid, s);
    }
    if (e == hipSuccess) e = mark_event(opts, 3, s);
    return hip_status(e);
}

moe_status moe_device_status(const moe_dims *dims, const void *ws, size_t ws_bytes, void *stream) {
    Dims D;
    moe_status st = check_dims(dims, &D);
    if (st != MOE_OK) return st;
    // the status word sits at offset 0 of a layer or an FFN workspace
    if ((st = check_ws((void *)ws, ws_bytes, 256)) != MOE_OK) return st;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_ERR_HIP;
    int32_t v = 0;
    if (hipMemcpy(&v, (const int32_t *)ws, sizeof v, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return MOE_ERR_HIP;
    return v == 0 ? MOE_OK : (moe_status)v;
}

int64_t moe_wall_clock_hz(void) { return wall_clock_hz(); }

}  // extern "C"
