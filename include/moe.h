/*
 * moe.h -- C ABI of the MI355X (gfx950) routed grouped-GEMM MoE layer.
 *
 * One GPU's forward pass through an expert-parallel MoE layer, split into the
 * stages of Weave ("Fine-Grained Dynamic SM Scheduling in an MoE Megakernel",
 * §2.1 and Figure 3): top-k gating, dispatch into expert-contiguous buffers,
 * GEMM0 (gate and up projections) with the SiLU-multiply activation, GEMM1
 * (down projection), and the gate-weighted combine back to token order.
 * moe_layer runs all of them; its expert GEMMs and combine are one persistent
 * kernel that claims tiles with atomic counters in dependency order (Weave §4)
 * and lets combine tiles start as soon as device-side flags say the down
 * tiles they read are complete (tile-level signaling: Cui et al., "Fine-grained
 * Computation-Communication Overlap via Tile-level Signaling and Scheduling
 * for Mixture-of-Experts", abstract).
 *
 * Conventions for every call:
 *  - Data pointers are DEVICE pointers, owned by the caller, and must stay
 *    valid until the enqueued work completes.  `stream` is a hipStream_t
 *    (NULL = the default stream).  Calls only enqueue work; none synchronises
 *    with the host.  The library allocates no device memory per call: callers
 *    pass a workspace of at least *_workspace_bytes(dims) bytes, 256-byte
 *    aligned.
 *  - bf16 tensors are raw bf16 bit patterns (uint16), row-major.  Weights are
 *    stored [out][in] (each output unit's weights contiguous):
 *        w_router [E, d], w_gate [E_loc, f, d], w_up [E_loc, f, d],
 *        w_down [E_loc, d, f].
 *  - Local experts are [e_lo, e_hi); E_loc = e_hi - e_lo.  Weight tensors
 *    hold only the local experts.  Rows routed to other experts are skipped
 *    (their gates still come from the global top-k).
 *  - Host-side argument checks run before anything is enqueued; a call that
 *    returns an error has enqueued nothing.  Errors found on the device (a
 *    bounded flag wait that timed out) are recorded in the workspace and read
 *    with moe_device_status.
 *  - Calls on distinct workspaces are independent; calls sharing a workspace
 *    must be ordered on one stream.
 *
 * Routing arithmetic (the pages do not define the gate function; this library
 * fixes it so that ids are reproducible bit for bit): logit[t,e] is a float32
 * sum over 16 equal contiguous chunks of the hidden dimension, each chunk
 * summed sequentially from +0 in ascending index, the 16 chunk sums combined
 * by a balanced pairwise tree ((s0+s1)+(s2+s3))+..., then the optional bias
 * added.  The k largest logits are selected (ties to the lower expert id) and
 * listed by (logit descending, id ascending); the gates are the softmax over
 * the selected logits.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,    /* null pointer, inconsistent dims */
    MOE_ERR_UNSUPPORTED = -2,    /* dims outside what the kernels support */
    MOE_ERR_WORKSPACE = -3,      /* workspace null, misaligned or too small */
    MOE_ERR_HIP = -4,            /* a HIP runtime call or launch failed */
    MOE_ERR_DEVICE_TIMEOUT = -5  /* a device-side flag wait exceeded its bound */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

/* Problem size.  T tokens of hidden size d, expert FFN size f, E experts in
 * the router, top-k, local experts [e_lo, e_hi).
 * Supported: T >= 0, 1 <= k <= E <= 1024, 0 <= e_lo < e_hi <= E,
 * d % 256 == 0, f % 128 == 0, T*k < 2^31. */
typedef struct {
    int64_t T, d, f, E, k, e_lo, e_hi;
} moe_dims;

/* ---- Per-call options of moe_layer and moe_layer_fp8.  A NULL pointer, or
 * a zero-initialised struct, selects every default.  The options travel with
 * the call: nothing is kept between calls, so calls on distinct workspaces
 * (and streams) are independent whatever options each passes. */
typedef enum {
    MOE_DISPATCH_PACKED = 0,  /* the permute writes x_perm in the packed
                                 MFMA-fragment layout; gate/up tiles load it
                                 straight into registers (default) */
    MOE_DISPATCH_GATHER = 1   /* gather-on-load: x_perm is never written; each
                                 gate/up tile fetches its rows of x through
                                 perm_src into LDS (Weave §4 overlaps dispatch
                                 with the first GEMM; on one GPU the dispatch is
                                 this gather).  Inputs of 2 GiB or more
                                 (T*d*2 bytes) use the packed mode. */
} moe_dispatch;

/* Tile order of moe_layer's persistent kernel.  Every order runs the same
 * tiles with the same arithmetic, so the output bits do not depend on it. */
typedef enum {
    MOE_ORDER_BY_KIND = 0,    /* every workgroup claims gate/up tiles until none
                                 are left, then down tiles (each waiting on its
                                 m-tile's gate/up tiles), then combine tiles:
                                 Weave §4's claiming in dependency order */
    MOE_ORDER_READY_DOWN = 1, /* X-Stage §4.3, ready-only form: before each
                                 gate/up claim a workgroup takes the next down
                                 tile of its XCD's range if every gate/up tile
                                 of that tile's m-tile is already published */
    MOE_ORDER_LEAD = 2,       /* X-Stage §4.3 with a dependency lead: gate/up
                                 and down tiles form one stream in which a down
                                 tile follows the last gate/up tile it reads by
                                 at least `lead` gate/up tiles (down first
                                 whenever it is eligible) */
    MOE_ORDER_COMBINE_FIRST = 3, /* tile-level signaling, consumers first: down
                                 tiles are claimed column group by column group
                                 (the columns one combine tile covers), and
                                 before each down claim a workgroup takes a
                                 combine tile whose column group is complete */
    MOE_ORDER_CHUNKED = 4     /* Weave §3.2.1's chunk pipeline: the tokens are
                                 cut into `chunks` ranges; an m-tile belongs to
                                 the chunk of its last token, a combine tile to
                                 the latest chunk its rows live in; gate/up,
                                 down and combine tiles form one stream ordered
                                 by (chunk, kind), so chunk c's combine runs
                                 while chunk c+1's GEMMs do */
} moe_tile_order;

/* How a layer call runs its expert FFN and combine. */
typedef enum {
    MOE_SCHEDULE_AUTO = 0,       /* the library's choice (default): moe_layer runs
                                    its persistent kernel; moe_layer_fp8 its
                                    staged launches, which measured faster than
                                    its persistent kernel on every workload shape
                                    tried on MI355X */
    MOE_SCHEDULE_PERSISTENT = 1, /* one persistent kernel: gate/up, (W8A8: h
                                    quantisation,) down and combine tiles in
                                    dependency order with device-side flags */
    MOE_SCHEDULE_STAGED = 2      /* one launch per stage (moe_layer_fp8 only);
                                    the same tiles and arithmetic, so the same
                                    bits as the persistent kernel */
} moe_schedule;

typedef struct {
    int32_t dispatch;        /* moe_dispatch (moe_layer only) */
    int32_t tile_order;      /* moe_tile_order (moe_layer only) */
    int32_t lead;            /* MOE_ORDER_LEAD: the lead in gate/up tiles; 0 =
                                one round of the persistent grid */
    int32_t chunks;          /* MOE_ORDER_CHUNKED: token chunks, 1..8; 0 = 4 */
    uint32_t perturb_seed;   /* 0 = off.  A test aid for the
                                flag protocol: every producer tile waits a
                                seeded pseudo-random delay (0 to about 100 us)
                                between writing its output and publishing it,
                                and (orders 0, 1, 3) the tiles of each kind are
                                claimed in reverse order (orders 2 and 4 hand
                                out one dependency-ordered stream, which must be
                                claimed in order).  The result bits are
                                unchanged; only the timing is adversarial.
                                Also moe_layer_fp8's persistent schedule. */
    int32_t schedule;        /* moe_schedule; moe_layer: AUTO or PERSISTENT */
    int64_t wait_timeout_us; /* bound of each device-side flag
                                wait; 0 = 2 s.  A wait that times out records
                                MOE_ERR_DEVICE_TIMEOUT in the workspace and
                                makes every other wait of that launch return at
                                once, so the launch still drains. */
    int64_t *trace;          /* per-tile trace of the persistent kernel (measurement aid,
                                after X-Stage §5.1's per-tile clock traces), or
                                NULL.  Device memory, int64 [1 + 4*trace_records]:
                                [0] = records written (the caller zeroes it; it
                                may exceed trace_records, the excess is
                                dropped), then per tile of the persistent kernel
                                {kind << 32 | tile index, workgroup << 8 | XCD,
                                start tick, end tick}: kind 1 gate/up, 2 down,
                                4 a K part of a cut down tile, 3 combine, 5 an
                                h quantisation tile (moe_layer_fp8); ticks
                                of moe_wall_clock_hz(). */
    int64_t trace_records;
    void *events[4];         /* hipEvent_t handles or NULL: recorded on `stream`
                                before the route, after the route, after the
                                permute, and after the last launch (measurement
                                aid: stage times per call) */
} moe_layer_opts;

/* Human-readable name of a status code (static string). */
const char *moe_status_string(moe_status s);

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

/* ---- moe_route: top-k gating (Weave §2.1: each token selects its experts
 * through a learned gate; Figure 3 shows top-k routing).
 *   x        bf16 [T, d]       activations
 *   w_router bf16 [E, d]       router weight
 *   bias     f32  [E] or NULL  added to every logit (after the dot product)
 *   topk_ids i32  [T, k]  out  selected expert ids, by (logit desc, id asc)
 *   topk_w   f32  [T, k]  out  renormalised softmax gates of those experts
 *   logits   f32  [T, E]  out, optional (NULL to skip)
 *   ws, ws_bytes               workspace of moe_route_workspace_bytes(dims)
 *                              bytes (256-byte aligned), or NULL
 * A workspace enables the fast paths.  E <= 16: one lane per token and one
 * wave per chunk of the hidden dimension, with the router weights as
 * wave-uniform scalar operands (read as bf16 and widened exactly on the
 * scalar unit), chunk sums kept in the workspace and folded by a second
 * kernel.  E > 16: MFMA logits with a
 * rigorous rounding-error bound pick the candidate experts, whose logits are
 * then evaluated in the defined order.  Either way ids and gates are the same
 * as when every logit is evaluated in that order, which is what happens with
 * logits != NULL or without a workspace (slower).  moe_route_workspace_bytes
 * returns 0 when no workspace is used.
 */
size_t moe_route_workspace_bytes(const moe_dims *dims);
moe_status moe_route(const moe_dims *dims, const void *x, const void *w_router, const float *bias,
                     int32_t *topk_ids, float *topk_w, float *logits, void *ws, size_t ws_bytes,
                     void *stream);

/* moe_route_bounds: the quantities the E > 16 fast path of moe_route selects
 * with, written out so that a caller can check the premise its ids rest on
 * (verification aid).
 *   approx f32 [T, E] out  the sum of the split-K matrix-core partials of
 *                          x . w_e, plus the bias
 *   eps    f32 [T, E] out  the bound the router assumes: |approx - logit| <=
 *                          eps, logit being the defined-order value
 * Arguments otherwise as moe_route; ws (moe_route_workspace_bytes) is
 * required.  MOE_ERR_UNSUPPORTED when the fast path does not apply
 * (E <= 16, or d too large for its LDS staging). */
moe_status moe_route_bounds(const moe_dims *dims, const void *x, const void *w_router,
                            const float *bias, float *approx, float *eps, void *ws,
                            size_t ws_bytes, void *stream);

/* ---- moe_permute: dispatch into expert-contiguous rows (Weave §2.1 stage
 * 1, Figure 3; on one GPU the "send" is a gather; each source row is read
 * once, as with Weave's dispatch-side deduplication, §4).
 *   x         bf16 [T, d]          activations
 *   topk_ids  i32  [T, k]          from moe_route (global expert ids)
 *   counts    i32  [E_loc]    out  rows per local expert
 *   offsets   i32  [E_loc+1]  out  exclusive prefix of counts; offsets[E_loc] = N
 *   perm_src  i32  [T*k]      out  source token of each row (first N valid)
 *   inv_perm  i32  [T, k]     out  row of each (token, slot); -1 if not local
 *   x_perm    bf16 [T*k, d]   out  x_perm[r] = x[perm_src[r]] (first N valid)
 * Rows inside an expert segment are in ascending source-token order.
 */
size_t moe_permute_workspace_bytes(const moe_dims *dims);
moe_status moe_permute(const moe_dims *dims, const void *x, const int32_t *topk_ids,
                       int32_t *counts, int32_t *offsets, int32_t *perm_src, int32_t *inv_perm,
                       void *x_perm, void *ws, size_t ws_bytes, void *stream);

/* ---- moe_expert_ffn: grouped SwiGLU expert FFN over expert-contiguous rows
 * (Weave §2.1 stages 2-4: GEMM0 up+gate, SiLU followed by element-wise
 * multiplication, GEMM1 down; FLOP count 6*d*f per row, Weave §3.1).
 *   x_perm  bf16 [T*k, d]      rows, expert-contiguous (first offsets[E_loc])
 *   offsets i32  [E_loc+1]     device-resident segment offsets
 *   w_gate, w_up bf16 [E_loc, f, d];  w_down bf16 [E_loc, d, f]
 *   y_perm  bf16 [T*k, d] out  y = (silu(x Wg^T) * (x Wu^T)) Wd^T per row
 * The intermediate h is rounded to bf16; accumulation is float32.  When
 * f >= 8192 the down tiles of the schedule's last partial round (as the
 * persistent kernel of moe_layer runs it) are summed as two K halves added
 * once in float32, exactly as moe_layer does, so both give the same bits.
 * The workspace starts with the status word read by moe_device_status.
 */
/* ---- moe_permute_noalloc: moe_permute for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments and results as moe_permute, without the
 * workspace: the per-token-block counts and bases go to a scratch array that
 * the library holds in device memory, one per GPU, for the life of the
 * process (moe_permute_noalloc_max_ints() int32s; 2 * ceil(T / 256) * E_loc
 * of them are used, MOE_ERR_UNSUPPORTED beyond that).  The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.  Every
 * call writes the scratch it reads, so nothing needs clearing between calls;
 * but all calls on one GPU share it, so calls that may overlap on one GPU
 * (concurrent streams, or several host threads) race and must be ordered by
 * the caller.  The first call on a device looks up the array's device
 * address (MOE_ERR_HIP if that fails). */
size_t moe_permute_noalloc_max_ints(void);
moe_status moe_permute_noalloc(const moe_dims *dims, const void *x, const int32_t *topk_ids,
                               int32_t *counts, int32_t *offsets, int32_t *perm_src,
                               int32_t *inv_perm, void *x_perm, void *stream);

size_t moe_expert_ffn_workspace_bytes(const moe_dims *dims);
moe_status moe_expert_ffn(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                          const void *w_gate, const void *w_up, const void *w_down, void *y_perm,
                          void *ws, size_t ws_bytes, void *stream);

/* ---- W8A8 expert FFN (X-Stage, §5.3, evaluates MegaMoE in W8A8; the
 * pages give no recipe, so this one is a stated choice).  Element format:
 * OCP 8-bit float E4M3 (bias 7, 3 mantissa bits, no infinities, largest
 * finite 448).  Each row of an operand -- a token's activations, a weight
 * matrix's output channel -- has one scale, the smallest power of two 2^e
 * (e >= -126) with max|row| <= 448 * 2^e (1 for an all-zero row); an element's
 * code is the E4M3 value nearest to x / 2^e, ties to the even code,
 * saturating at 448.  Dequantisation multiplies by the scales, exactly.
 *
 * moe_quantize_fp8: x bf16 [rows, cols] (device, row-major, 16-byte aligned,
 *   cols a multiple of 16) -> q uint8 [rows, cols] codes (16-byte aligned)
 *   and scale f32 [rows].  Used for weights ([E_loc, out, K] as E_loc*out
 *   rows of K) and activations.  Caller-owned device buffers; no workspace.
 *   MOE_ERR_INVALID_ARG on bad sizes, null or misaligned pointers. */
moe_status moe_quantize_fp8(const void *x, int64_t rows, int64_t cols, void *q, float *scale,
                            void *stream);

/* moe_expert_ffn_fp8: the grouped SwiGLU FFN of moe_expert_ffn on E4M3
 * operands with float32 accumulation on the fp8 matrix cores.
 *   x_perm   bf16 [T*k, d] rows, expert-contiguous (quantised per row inside)
 *   offsets  i32 [E_loc+1]  device-resident segment offsets
 *   wq_gate, wq_up uint8 [E_loc, f, d], s_gate, s_up f32 [E_loc, f]
 *   wq_down  uint8 [E_loc, d, f], s_down f32 [E_loc, d]   (moe_quantize_fp8)
 *   y_perm   bf16 [T*k, d] out
 * g = sx * sg * (xq . wgq), u likewise, h = silu(g) * u rounded to bf16 and
 * re-quantised per row, y = sh * sd * (hq . wdq) rounded to bf16.  Requires
 * f % 256 == 0 (else MOE_ERR_UNSUPPORTED).  Kernels: per-row quantisation
 * into the packed fragment layout, the gate/up GEMM, quantisation of h, the
 * down GEMM; no device-side waits and no status word. */
size_t moe_expert_ffn_fp8_workspace_bytes(const moe_dims *dims);
moe_status moe_expert_ffn_fp8(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                              const void *wq_gate, const float *s_gate, const void *wq_up,
                              const float *s_up, const void *wq_down, const float *s_down,
                              void *y_perm, void *ws, size_t ws_bytes, void *stream);

/* The two halves of moe_expert_ffn_fp8 as separate calls (verification aid;
 * the same kernels, so down(gate_up(x)) equals moe_expert_ffn_fp8 bit for
 * bit).  ws: moe_expert_ffn_fp8_workspace_bytes(dims) bytes.
 * moe_gate_up_fp8: GEMM0 + SiLU-mul (Weave §2.1 stages 2-3) on E4M3 codes of
 *   the rows of x_perm, quantised per row inside:
 *   h bf16 [T*k, f] out (first offsets[E_loc] rows valid)
 * moe_down_fp8: GEMM1 (Weave §2.1 stage 4) of bf16 rows h [T*k, f],
 *   quantised per row inside:  y_perm bf16 [T*k, d] out. */
moe_status moe_gate_up_fp8(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                           const void *wq_gate, const float *s_gate, const void *wq_up,
                           const float *s_up, void *h, void *ws, size_t ws_bytes, void *stream);
moe_status moe_down_fp8(const moe_dims *dims, const void *h, const int32_t *offsets,
                        const void *wq_down, const float *s_down, void *y_perm, void *ws,
                        size_t ws_bytes, void *stream);

/* moe_layer_fp8: the whole forward pass with the W8A8 FFN (X-Stage §4.3
 * fuses the MoE block into one kernel, §5.3 evaluates it in W8A8): route (as
 * moe_route), permute, the per-row E4M3 quantisation of the routed rows of
 * x, then either moe_expert_ffn_fp8's launches and moe_combine
 * (MOE_SCHEDULE_STAGED, and the default MOE_SCHEDULE_AUTO) or, with
 * MOE_SCHEDULE_PERSISTENT, one persistent kernel whose workgroups claim
 * gate/up tiles (E4M3 GEMM0 with the SiLU-mul epilogue into bf16 h and each
 * row's max |h|), quantisation tiles (rows of h, once their m-tile's
 * gate/up tiles are published), down tiles (once their m-tile's rows are
 * quantised) and combine tiles (once the down tiles holding their rows are
 * published).  Both give the same bits.  One stream, one workspace, no host
 * synchronisation.
 * Arguments as moe_layer, with the E4M3 weights and scales of
 * moe_expert_ffn_fp8 in place of the bf16 weights.  Requires f % 256 == 0.
 * Of opts: events[], schedule, and for the persistent schedule
 * perturb_seed, wait_timeout_us and trace (trace kinds: 1 gate/up, 5
 * quantisation, 2 down, 3 combine); its status word sits at offset 0 of the
 * workspace, as moe_layer's: moe_device_status reads it.  dispatch,
 * tile_order, lead and chunks must be zero (MOE_ERR_INVALID_ARG otherwise). */
size_t moe_layer_fp8_workspace_bytes(const moe_dims *dims);
moe_status moe_layer_fp8(const moe_dims *dims, const void *x, const void *w_router,
                         const float *bias, const void *wq_gate, const float *s_gate,
                         const void *wq_up, const float *s_up, const void *wq_down,
                         const float *s_down, void *out, moe_dtype out_dtype,
                         int32_t *topk_ids_out, float *topk_w_out, void *ws, size_t ws_bytes,
                         const moe_layer_opts *opts, void *stream);

/* ---- moe_combine: gate-weighted sum back to token order (Weave §2.1 stage 5).
 *   y_perm   bf16 [T*k, d]  expert outputs by row
 *   inv_perm i32  [T, k]    row of each (token, slot), -1 = skip
 *   topk_w   f32  [T, k]    gates
 *   out      [T, d]   out   bf16 (round to nearest even) or f32 per out_dtype;
 *                           out[t] = sum over slots j ascending with
 *                           inv_perm >= 0 of topk_w[t,j] * y_perm[row], in f32;
 *                           tokens with no local slot get 0.
 */
moe_status moe_combine(const moe_dims *dims, const void *y_perm, const int32_t *inv_perm,
                       const float *topk_w, void *out, moe_dtype out_dtype, void *stream);

/* ---- moe_layer: the whole forward pass.  Route, permute, then one
 * persistent kernel whose workgroups claim gate/up tiles, then down tiles,
 * then combine tiles from per-XCD atomic queues (Weave §4: tiles claimed by
 * atomicAdd in the pipeline's dependency order).  A down tile waits on a
 * per-row-block counter of finished gate/up tiles; each finished down tile
 * releases a flag that the combine tiles reading it acquire.
 *   out          [T, d] bf16 or f32 (f32 for an expert-parallel partial)
 *   topk_ids_out i32 [T,k], topk_w_out f32 [T,k]: optional copies of routing
 *   opts         per-call options (moe_layer_opts) or NULL for the defaults;
 *                MOE_ERR_INVALID_ARG for a value outside its range
 */
size_t moe_layer_workspace_bytes(const moe_dims *dims);
moe_status moe_layer(const moe_dims *dims, const void *x, const void *w_router, const float *bias,
                     const void *w_gate, const void *w_up, const void *w_down, void *out,
                     moe_dtype out_dtype, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                     size_t ws_bytes, const moe_layer_opts *opts, void *stream);

/* ---- Matrix-core probe (measurement aid).  Runs, for each of n cases, a
 * chain of `steps` matrix-core instructions and returns the float32 results,
 * so that their rounding can be compared with exact sums: the fast router's
 * error bound and the W8A8 tolerance rest on it.
 *   kind 0: v_mfma_f32_32x32x16_bf16, K = 16, a and b bf16;
 *   kind 1: v_mfma_f32_32x32x64_f8f6f4 on E4M3 codes, K = 64, a and b bytes.
 *   a, b  [n][steps][32][K]  rows of A and of B^T for each step
 *   c     f32 [n][32][32]    accumulator before the first step
 *   d     f32 [n][32][32] out  c + sum over steps (in order) of a_s . b_s^T
 * Device pointers, 16-byte aligned; 1 <= steps <= 4096; n < 2^31.
 * MOE_ERR_INVALID_ARG otherwise. */
moe_status moe_probe_mfma(int kind, int64_t n, int steps, const void *a, const void *b,
                          const float *c, float *d, void *stream);

/* ---- Matrix-core rate probe (measurement aid).  `workgroups` workgroups of
 * 256 threads; each of their waves issues iters x 16 independent
 * v_mfma_f32_32x32x16_bf16 on operands fixed per lane: zero (seed 0) or
 * pseudo-random values in [-1, 1) drawn from the seed.  Work =
 * workgroups * 4 * iters * 16 * 32768 FLOP; the caller times it (the sustained
 * rate with real data is below the nominal peak where the power limit lowers
 * the clock).  sink: device f32 [workgroups * 256], 16-byte aligned, written
 * with each thread's sum.  0 <= workgroups <= 65536, 1 <= iters <= 2^20;
 * MOE_ERR_INVALID_ARG otherwise. */
moe_status moe_probe_mfma_rate(int64_t workgroups, int iters, uint32_t seed, float *sink,
                               void *stream);

/* Synchronises `stream`, then reads the device status word at offset 0 of a
 * workspace last used by moe_layer or moe_expert_ffn (MOE_OK, or
 * MOE_ERR_DEVICE_TIMEOUT if a flag wait gave up).  ws_bytes must be >= 256. */
moe_status moe_device_status(const moe_dims *dims, const void *ws, size_t ws_bytes, void *stream);

/* Frequency of the device's constant wall clock (ticks per second), the
 * time base of the per-tile trace. */
int64_t moe_wall_clock_hz(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
