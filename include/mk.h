/*
 * mk.h -- C ABI of the one-GPU MoE layer hot path for AMD MI355X (gfx950).
 *
 * The calls follow the functional API of Mixture-of-Kittens (MoK) as the
 * agentlenshq project card "Mixture-of-Kittens (MoK)" states it ("Use the
 * functional API", "Core concepts"): a config, a workspace created once per
 * model and reused, build_schedule from the routed expert ids, forward
 * returning the output plus a forward context, and backward consuming that
 * context.  The same card's "Core concepts" names the MXFP8 quantise op used
 * to pre-quantise weights.  Routing is added in front because the pages take
 * the top-k expert ids as an input.
 *
 * Conventions (every entry point):
 *  - Every pointer argument named *_dev is DEVICE memory on the current HIP
 *    device; the caller allocates and owns it.  The library owns only the
 *    workspace and what it allocates inside it.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it: they never synchronise with the host, never copy
 *    device data to the host and never size a launch from device-side counts.
 *  - bf16 tensors are raw 16-bit bf16 patterns (uint16), row-major.  Rows
 *    are read and written 16 bytes at a time: every tensor starts 16-byte
 *    aligned.
 *  - Return value: MK_OK (0) or a negative MK_ERR_* code, detected on the
 *    host before anything is enqueued.  Problems only the device can see
 *    set bits in the schedule's device error word (MK_DEVERR_*); read it
 *    with mk_device_error.  No call hangs on bad data and no exception
 *    crosses this boundary.
 *  - One workspace serves one stream at a time; calls on one workspace must
 *    be ordered (same stream, or externally synchronised).  A schedule
 *    (mk_schedule) belongs to the workspace it was created for; several
 *    schedules may be alive at once, so the forwards of several microbatches
 *    can run before their backwards, in any order.
 */
#ifndef MK_H_
#define MK_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MK_OK               0
#define MK_ERR_NULL        -1  /* a required pointer is NULL                 */
#define MK_ERR_SHAPE       -2  /* unsupported shape (see each call)           */
#define MK_ERR_RING        -3  /* ring smaller than one minibatch             */
#define MK_ERR_LIMIT       -4  /* above a workspace limit (rows, experts, k)  */
#define MK_ERR_HIP         -5  /* a HIP runtime call failed                   */
#define MK_ERR_STATE       -6  /* call out of order (e.g. forward before schedule) */
#define MK_ERR_UNSUPPORTED -7  /* combination not implemented                 */
#define MK_ERR_CONFIG      -8  /* invalid config field                        */

/* ---- device error word bits (one word per schedule, cleared by
 *      mk_build_schedule; read with mk_device_error) ---------------------- */
#define MK_DEVERR_EXPERT_RANGE   0x1u  /* a row_expert id outside [0, E): row dropped, its output is 0 */
#define MK_DEVERR_SCHED_OVERFLOW 0x2u  /* work table above capacity: trailing tiles dropped            */
#define MK_DEVERR_WAIT_TIMEOUT   0x4u  /* fused forward: a dependency wait passed its bound (results invalid) */

/* ---- enums --------------------------------------------------------------- */
#define MK_BF16   0
#define MK_MXFP8  1

#define MK_FULL_LAYER   0  /* rows r = t*k + j of T tokens; combine sums the k rows of a token */
#define MK_EXPERT_SHARE 1  /* rows already resident in arrival order; out_rows[r] = w[r]*y(r)   */

/*
 * Config (the card's MoKConfig knobs that apply to one GPU; "Core concepts",
 * "Limitations": minibatch granularity, macrobatch size via the ring, schedule
 * capacity multiplier).  The communication-SM knob has no one-GPU meaning.
 *   minibatch_rows      rows per minibatch (MB); 0 = all rows in one.  In
 *                       MK_FULL_LAYER mode a multiple of k.  At most 65535
 *                       minibatches of max_rows (else MK_ERR_LIMIT).
 *   ring_bytes          ring token buffer capacity; the ring holds
 *                       MB * floor(ring_bytes / (MB * row_bytes)) rows, a whole
 *                       number of minibatches (the macrobatch).  row_bytes is
 *                       2H (bf16) or H + H/32 (MXFP8).
 *   sched_capacity_mult work-table capacity as a multiple of the worst case
 *                       ceil(rows/256) + minibatches*E; >= 1 never overflows.
 *   precision           MK_BF16 or MK_MXFP8.
 *   renorm              router weights: 1 = softmax over the k chosen logits,
 *                       0 = full softmax over all E read at the chosen ones.
 *   enable_backward     1 = also allocate the backward's buffers.
 *   wgrad_mxfp8         1 = (precision MK_MXFP8 with enable_backward only)
 *                       the weight-gradient GEMMs take MXFP8 operands too,
 *                       each quantised along the contraction (the expert's
 *                       rows) in blocks of 32 rows of one minibatch, a
 *                       minibatch's last block completed with zero rows;
 *                       0 = bf16 weight gradients.  The pages give no MXFP8
 *                       recipe for these GEMMs; this blocking follows the
 *                       forward's (MX blocks along the contraction) with the
 *                       minibatch as the unit of arrival ([MTP] "Three design
 *                       decisions that matter": minibatch granularity).
 *                       Its row space holds max_rows + minibatches*E*31 +
 *                       E*127 rows (every minibatch segment rounded up to 32
 *                       rows, every expert to 128): MK_ERR_LIMIT above
 *                       65535 * 128 rows.
 *   fused_forward       1 = (precision MK_BF16) mk_forward runs the
 *                       permute, GEMM1 + SwiGLU and GEMM2 as one persistent
 *                       launch in which the permute of minibatch b+1, GEMM1
 *                       of b and GEMM2 of b-1 run at once on different
 *                       compute units ([MTP] opening paragraph: every step
 *                       in a single kernel; "Three design decisions that
 *                       matter": minibatch granularity), ordered by device
 *                       counters; the full layer's combine follows as a
 *                       second launch.  Same results bit for bit as the
 *                       phase-by-phase launches.  Applies when the ring
 *                       holds every minibatch of the call; a call whose
 *                       rows wrap the ring runs one launch per phase.
 *                       0 = one launch per phase.
 */
typedef struct mk_config {
  int32_t minibatch_rows;
  int32_t precision;
  int64_t ring_bytes;
  float   sched_capacity_mult;
  int32_t renorm;
  int32_t enable_backward;
  int32_t wgrad_mxfp8;
  int32_t fused_forward;
  int32_t reserved;
} mk_config;

typedef struct mk_workspace mk_workspace;   /* opaque */
typedef struct mk_schedule mk_schedule;     /* opaque */

/* Fill *cfg with defaults: MB = 0, bf16, 256 MiB ring, capacity 1.0,
 * renorm 1, no backward. */
void mk_config_default(mk_config* cfg);

/*
 * Workspace ("Core concepts": created once per model, reused).  Allocates the
 * ring, the schedule builder's scratch and the intermediate activations on
 * the current device (each schedule's tables come with mk_schedule_create).  Limits: max_rows >= 1 routed rows per call; H % 256 == 0,
 * I % 128 == 0 (I % 256 == 0 with enable_backward); 1 <= E <= 1024;
 * 1 <= k <= 32; ring_bytes below 2 GiB.  Returns MK_ERR_SHAPE / _LIMIT / _RING /
 * _CONFIG on a bad argument, MK_ERR_HIP if an allocation fails.
 */
int mk_workspace_create(const mk_config* cfg, int32_t max_rows, int32_t H, int32_t I,
                        int32_t E, int32_t k, mk_workspace** out);
int mk_workspace_destroy(mk_workspace* ws);

/* Host-known sizes of a workspace, for callers and tests. */
#define MK_Q_RING_ROWS      0   /* rows the ring holds                         */
#define MK_Q_MINIBATCH_ROWS 1   /* MB                                          */
#define MK_Q_NUM_MB         2   /* minibatches of a schedule (mk_schedule_query) */
#define MK_Q_ITEM_CAPACITY  3   /* work-table capacity (items)                 */
#define MK_Q_TILE_M         4   /* rows per work item (GEMM m-tile)            */
#define MK_Q_ROWS           5   /* R of a schedule (mk_schedule_query)         */
#define MK_Q_NUM_CU         6   /* compute units the persistent grids use      */
#define MK_Q_PACKED_BYTES   7   /* bytes of packed weights (forward only)      */
#define MK_Q_PACKED_BYTES_BWD 8 /* bytes of packed weights incl. backward copies */
#define MK_Q_FWD_CTX_BYTES  9   /* bytes of fwd_ctx for max_rows               */
int64_t mk_query(const mk_workspace* ws, int32_t what);
/* MK_Q_NUM_MB and MK_Q_ROWS of the schedule's last build (0 before one). */
int64_t mk_schedule_query(const mk_schedule* sched, int32_t what);

/*
 * Router: z[t,e] = sum_h x[t,h]*w_router[e,h] accumulated in fp32 in ascending
 * h from +0, plus bias[e] (fp32) if bias_dev is not NULL; top-k by descending
 * z with ties to the lower expert id (slot 0 = largest); weights from the
 * softmax selected by cfg.renorm.
 *   x_dev        [T, H] bf16          w_router_dev [E, H] bf16
 *   bias_dev     [E] fp32 or NULL
 *   topk_idx_dev [T, k] int32 (out)   topk_w_dev   [T, k] fp32 (out)
 * MK_ERR_LIMIT if T*k > max_rows.  With T = 0 nothing is launched and only
 * w_router_dev must be non-NULL.
 */
int mk_route(mk_workspace* ws, const void* x_dev, const void* w_router_dev,
             const float* bias_dev, int32_t T, int32_t* topk_idx_dev, float* topk_w_dev,
             void* stream);

/*
 * Dispatch schedule ([MTP] = MarkTechPost "Cursor Open-Sources
 * Mixture-of-Kittens (MoK)...", "Three design decisions that matter": one
 * schedule table serves dispatch, combine and both backward directions;
 * [CARD] "Use the functional API": build_schedule returns the schedule that
 * forward and backward take).
 *
 * mk_schedule_create allocates one schedule's device tables on the current
 * device, sized from the workspace's limits (MK_ERR_HIP if that fails, or if
 * the current device is not the workspace's); mk_schedule_destroy frees them.
 * A schedule is only valid with the workspace it was created for
 * (MK_ERR_STATE otherwise) and must not outlive it.
 *
 * mk_build_schedule: from row_expert_dev [R] int32 (full-layer mode: the
 * flattened topk_idx, row r = t*k + j) builds, on the device, per-expert and
 * per-minibatch counts and offsets, the stable expert-grouped position of
 * every row, its inverse, and the GEMM work items.  Rows with an expert id
 * outside [0, E) are dropped and flagged (MK_DEVERR_EXPERT_RANGE).  Clears the
 * schedule's device error word and forgets its last forward (a backward must
 * follow a forward on the rebuilt schedule).  MK_ERR_LIMIT if R > max_rows;
 * MK_ERR_SHAPE if R < 0 (in full-layer use, MB not a multiple of k is
 * checked at forward).
 */
int mk_schedule_create(mk_workspace* ws, mk_schedule** out);
int mk_schedule_destroy(mk_schedule* sched);
int mk_build_schedule(mk_workspace* ws, mk_schedule* sched, const int32_t* row_expert_dev, int32_t R,
                      void* stream);

/*
 * mk_build_schedule without a workspace or schedule object, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same tables as
 * mk_build_schedule, written to caller-owned device buffers, with the
 * build's scratch in a fixed 4 MiB device array of the library (one per
 * GPU, held until the process ends; no allocation happens in this call).
 *   row_expert_dev [R] int32, minibatch rows MB >= 1, E in [1, 1024],
 *   item_cap >= 1 (work items the items buffer holds; more set
 *   MK_DEVERR_SCHED_OVERFLOW in *err_dev and drop the trailing items).
 *   Outputs (nb = ceil(R / MB)): counts_dev [E], offsets_dev [E+1],
 *   mb_counts_dev [nb, E], mb_offsets_dev [nb, E+1], sorted_pos_dev [R],
 *   inv_dev [nb*MB], items_dev [item_cap, 4], mb_items_dev [nb+1], err_dev
 *   [1] (written whole); layouts as the MK_TAB_* tables.  With R = 0 only
 *   counts, offsets, items, mb_items and err are written (the others may be
 *   NULL).
 * MK_ERR_LIMIT if the build's scratch, nb * (c4 * E + c) * 4 bytes with
 * c = ceil(MB / 256) chunks and c4 = c rounded up to a multiple of 4,
 * exceeds the 4 MiB array, or nb > 65535; MK_ERR_SHAPE / _NULL on bad arguments; MK_ERR_HIP
 * if the scratch's device address cannot be found.  Calls on one GPU share
 * the scratch: calls that overlap on one GPU (different streams without
 * ordering) race.
 */
int mk_build_schedule_static(const int32_t* row_expert_dev, int32_t R, int32_t E, int32_t MB, int32_t item_cap,
                             int32_t* counts_dev, int32_t* offsets_dev, int32_t* mb_counts_dev,
                             int32_t* mb_offsets_dev, int32_t* sorted_pos_dev, int32_t* inv_dev, int32_t* items_dev,
                             int32_t* mb_items_dev, uint32_t* err_dev, void* stream);

/* Copy one table of a schedule (device) into dst_dev (device, >= bytes;
 * MK_ERR_LIMIT if bytes exceeds the table). */
#define MK_TAB_COUNTS     0   /* [E]        int32                                   */
#define MK_TAB_OFFSETS    1   /* [E+1]      int32                                   */
#define MK_TAB_MB_COUNTS  2   /* [nb, E]    int32                                   */
#define MK_TAB_MB_OFFSETS 3   /* [nb, E+1]  int32 (within each minibatch)           */
#define MK_TAB_SORTED_POS 4   /* [R]        int32, -1 for a dropped row             */
#define MK_TAB_INV        5   /* [nb*MB]    int32, -1 where no row                  */
#define MK_TAB_ITEMS      6   /* [capacity, 4] int32 (row_begin, rows, expert, mb)  */
#define MK_TAB_MB_ITEMS   7   /* [nb+1]     int32 first item of each minibatch      */
int mk_schedule_copy(const mk_schedule* sched, int32_t table, void* dst_dev, int64_t bytes, void* stream);

/*
 * Copy one of the workspace's device buffers into dst_dev (device, >= bytes):
 * what the last call on the workspace left there, for tests and inspection.
 * Rows at sorted positions p (expert order, [positions, ...] with positions =
 * minibatches * MB).  MK_ERR_CONFIG for a buffer this workspace does not
 * have (MXFP8 buffers in bf16 mode, backward buffers without
 * enable_backward), MK_ERR_LIMIT if bytes exceeds it.
 */
#define MK_BUF_RING        0   /* ring token buffer, ring_rows * row_bytes bytes (MXFP8: codes, then scales) */
#define MK_BUF_A           1   /* [positions, I] bf16: SwiGLU output a of the last forward                    */
#define MK_BUF_A_CODES     2   /* [positions, I] uint8: a quantised along I (MXFP8 forward)                   */
#define MK_BUF_A_SCALES    3   /* [positions, I/32] uint8: their E8M0 scales                                  */
#define MK_BUF_Y           4   /* [positions, H] fp32: GEMM2 output y of the last full-layer forward          */
#define MK_BUF_DGDU        5   /* [positions, 2I] bf16: dg (I values), then du (I values) of the last backward */
#define MK_BUF_DGDU_CODES  6   /* [positions, 2I] uint8: dg/du quantised along 2I (MXFP8 backward)            */
#define MK_BUF_DGDU_SCALES 7   /* [positions, 2I/32] uint8                                                    */
#define MK_BUF_WA          8   /* [positions, I] bf16: w*a of the last backward                               */
#define MK_BUF_DY_CODES    9   /* [positions, H] uint8: dY rows quantised along H (MXFP8 backward); the
                                 full layer with MXFP8 weight gradients keeps its T token rows here instead */
#define MK_BUF_DY_SCALES  10   /* [positions, H/32] uint8 (token rows as above)                               */
int mk_workspace_copy(const mk_workspace* ws, int32_t buffer, void* dst_dev, int64_t bytes, void* stream);

/*
 * MXFP8 quantise (the card's ops.mxfp8_quantize; OCP MX v1.0 with E4M3
 * elements): blocks of 32 along K; E8M0 scale s = clamp(floor(log2 amax) - 8,
 * -127, 127) + 127 (0 for an all-zero block); codes are E4M3-FN of v/2^(s-127)
 * rounded to nearest even and saturated at +-448, sign kept.
 *   in_dev [rows, K] bf16 -> codes_dev [rows, K] uint8, scales_dev [rows, K/32] uint8
 * MK_ERR_SHAPE unless K % 32 == 0.  Needs no workspace.
 */
int mk_mxfp8_quantize(const void* in_dev, int64_t rows, int32_t K, uint8_t* codes_dev,
                      uint8_t* scales_dev, void* stream);

/*
 * Weight packing (outside the timed path; the card's "Limitations": MXFP8
 * weights are pre-quantised).  Inputs, one row per output feature:
 *   w_gate_dev [E, I, H] bf16, w_up_dev [E, I, H] bf16, w_down_dev [E, H, I] bf16
 * packed_dev receives mk_query(MK_Q_PACKED_BYTES[_BWD]) bytes: gate and up
 * rows interleaved in blocks of 16 (GEMM1's B), the down rows (GEMM2's B),
 * with for_backward = 1 also the transposed copies the backward GEMMs read.
 * bf16 mode stores each of them as 32 KiB blocks of 256 rows x 64 K in the
 * order (expert, row block, K block), every block laid out as the GEMM keeps
 * it in LDS; MXFP8 mode quantises along each GEMM's K and stores, per
 * (expert, 256-row block, 128-K block), a 32 KiB block of E4M3 codes in the
 * same LDS-image form and a 1 KiB block of the rows' E8M0 scales.  The layout
 * is internal: only this library reads the buffer.
 */
int mk_prepare_weights(mk_workspace* ws, const void* w_gate_dev, const void* w_up_dev,
                       const void* w_down_dev, int32_t for_backward, void* packed_dev,
                       void* stream);

/*
 * Forward ([MTP] "Three design decisions that matter" and the paragraph after
 * them): permute rows into the ring minibatch by minibatch (MXFP8: quantised
 * on the way), expert-grouped GEMM1 (gate/up) with SwiGLU, GEMM2 (down), then
 * the router-weighted combine in a fixed order (bitwise repeatable).
 *   mode MK_FULL_LAYER:   x_src_dev [T, H] bf16, row r = t*k + j comes from
 *                         token t; row_w_dev = topk_w [T*k] fp32;
 *                         out_dev [T, H] bf16, out[t] = sum_j w[t,j] y(t,j), j ascending.
 *   mode MK_EXPERT_SHARE: x_src_dev [R, H] bf16 in arrival order; row_w_dev [R];
 *                         out_dev [R, H] bf16, out[r] = w[r] * y(r).
 *   fwd_ctx_dev: NULL, or mk_query(MK_Q_FWD_CTX_BYTES) bytes that receive what
 *                the backward needs (g and u in fp32; in MXFP8 mode the
 *                products of the dequantised operands).
 * sched: built by mk_build_schedule on this workspace (MK_ERR_STATE if not).
 * The forward overwrites the workspace's ring; the schedule records the mode,
 * fwd_ctx_dev and that its rows are now the ring's, for its backward.  In
 * MK_FULL_LAYER mode with mk_config.fused_forward (bf16), GEMM1 instead
 * gathers the token rows straight from x_src_dev through the schedule's
 * inverse map and the ring is left as it was; a backward of this schedule
 * then gathers the x rows again, as for minibatches evicted from the ring.
 * In MK_FULL_LAYER mode with precision MK_MXFP8, when the T token rows fit
 * the ring, the ring receives their MXFP8 codes (each quantised once) and
 * GEMM1 reads them through the inverse map (the MXFP8 backward gathers the
 * x rows again in any case).
 */
int mk_forward(mk_workspace* ws, mk_schedule* sched, int32_t mode, const void* x_src_dev,
               const float* row_w_dev, const void* packed_dev, void* out_dev, void* fwd_ctx_dev, void* stream);

/*
 * Backward ([MTP]: the ring is walked in reverse to minimise
 * forward-activation replay; the router-weight gradient is fused into the
 * SwiGLU backward), for the loss L = <dY, out> of mk_forward.  In MXFP8 mode
 * the two data-gradient GEMMs take MXFP8 operands quantised along their
 * contraction (dY and W_d^T along H; [dg | du] and [W_g; W_u]^T along the 2I
 * features, the I gate ones then the I up ones, blocks of 32), fp32
 * accumulation; the weight gradients
 * are bf16 GEMMs as in bf16 mode.  Evicted minibatches (an MXFP8 ring holds
 * codes, so all of them) have their x rows gathered again before the
 * gate/up weight gradient.  With cfg.wgrad_mxfp8 the weight gradients are
 * MXFP8 GEMMs too: dY rows, w*a, dg/du and x rows each quantised along the
 * rows of an expert (32 rows of one minibatch per block, a minibatch's last
 * block completed with zero rows), dY and x read straight from dY_dev and
 * x_src_dev through the schedule's inverse map; fp32 accumulation, each
 * output element by one workgroup over the expert's rows in a fixed order.
 *   mode MK_EXPERT_SHARE: x_src_dev [R, H], row_w_dev [R], dY_dev [R, H] and
 *       dX_dev [R, H] in arrival order; d_row_w_dev [R] fp32.
 *   mode MK_FULL_LAYER: x_src_dev [T, H], row_w_dev = topk_w [T*k],
 *       dY_dev [T, H], dX_dev [T, H] = sum over j ascending of the k routed
 *       rows' input gradients in fp32, rounded once; d_row_w_dev [T*k] =
 *       gradient w.r.t. topk_w.  The router is taken as external (its inputs
 *       topk_idx/topk_w are leaves); mk_backward_layer also differentiates it.
 *   dW_gate_dev [E, I, H] fp32, dW_up_dev [E, I, H] fp32, dW_down_dev [E, H, I] fp32
 * Weight gradients are reduced in a fixed order (minibatches in reverse walk
 * order, rows ascending inside each) with no float atomics: bitwise repeatable
 * at a fixed minibatch size.  sched must have had a forward in the same mode
 * since its last build, and fwd_ctx_dev must be the context that forward
 * wrote (MK_ERR_STATE otherwise; not checked when R = 0).  Other schedules'
 * forwards may have run in between: the ring then no longer holds this
 * schedule's rows and every minibatch's x rows are gathered again (the
 * result is the same).  packed_dev must have been prepared with
 * for_backward = 1.  MK_ERR_CONFIG if the workspace has no backward buffers;
 * MK_ERR_SHAPE in full-layer mode unless R and MB are multiples of k.  After
 * an empty schedule (R = 0) only the weight-gradient pointers are read (the
 * others may be NULL) and the weight gradients are written as zeros.
 */
int mk_backward(mk_workspace* ws, const mk_schedule* sched, int32_t mode, const void* fwd_ctx_dev,
                const void* x_src_dev, const float* row_w_dev, const void* packed_dev, const void* dY_dev,
                void* dX_dev, float* dW_gate_dev, float* dW_up_dev, float* dW_down_dev,
                float* d_row_w_dev, void* stream);

/*
 * Full-layer backward including the router (gradient through the softmax
 * top-k router that mk_route computes; the pages take routing as an input,
 * so this is the plain chain rule through that router).  The expert choice is
 * piecewise constant and carries no gradient; with d_topk_w the gradient
 * w.r.t. the top-k weights, the logit gradient dz [T, E] is the softmax
 * Jacobian applied to it: cfg.renorm = 1: dz[t, idx_j] = w_j (d_w_j - S),
 * other experts 0, S = sum_j w_j d_w_j; cfg.renorm = 0: dz[t, e] = p_e (g_e - S)
 * over all E, p the full softmax (recomputed from x, w_router and bias), g_e =
 * d_w_j where e = idx_j, else 0.  Then
 *   dW_router_dev [E, H] fp32 = dz^T x     d_bias_dev [E] fp32 = sum_t dz (NULL: skipped)
 *   dX_dev [T, H] bf16 = sum_j (routed rows' input gradients, j ascending)
 *                        + sum_e dz[t, e] w_router[e] (e ascending), fp32, one rounding
 *   d_topk_w_dev [T*k] fp32, dW_gate/up/down as mk_backward.
 * x_dev, w_router_dev, bias_dev (NULL if the router has none), topk_idx_dev and
 * topk_w_dev are the ones mk_route and mk_forward saw; sched must be the
 * schedule built from topk_idx.  Every sum runs in a fixed order: bitwise
 * repeatable.  Errors as mk_backward; with T = 0, w_router_dev and
 * dW_router_dev are still required and dW_router (and d_bias) become zeros.
 */
int mk_backward_layer(mk_workspace* ws, const mk_schedule* sched, const void* fwd_ctx_dev, const void* x_dev,
                      const void* w_router_dev, const float* bias_dev, const int32_t* topk_idx_dev,
                      const float* topk_w_dev, const void* packed_dev, const void* dY_dev,
                      void* dX_dev, float* dW_gate_dev, float* dW_up_dev, float* dW_down_dev,
                      float* dW_router_dev, float* d_bias_dev, float* d_topk_w_dev, void* stream);

/*
 * Per-phase timing (for benchmarks): with timing on, every launch sequence
 * records a HIP event pair on the caller's stream around each phase, and
 * mk_timing_read (HOST call: waits for the recorded events) adds up the
 * milliseconds per phase since the last read into ms_out[MK_PH_COUNT] and
 * launch counts into launches_out[MK_PH_COUNT] (either may be NULL), then
 * resets.  Costs one event record per phase boundary; off by default.
 */
#define MK_PH_ROUTE      0
#define MK_PH_SCHEDULE   1
#define MK_PH_PERMUTE    2   /* permute into the ring (MXFP8: fused quantise) */
#define MK_PH_GEMM1      3
#define MK_PH_QUANT_A    4   /* MXFP8: quantise a along I                    */
#define MK_PH_GEMM2      5   /* expert share: includes the fused weighted unpermute */
#define MK_PH_COMBINE    6   /* full layer combine / zeroing of dropped rows  */
#define MK_PH_BWD_GATHER 7
#define MK_PH_BWD_DACT   8
#define MK_PH_BWD_DW     9
#define MK_PH_BWD_DX     10
#define MK_PH_WGRAD_DOWN 11
#define MK_PH_WGRAD_GU   12
#define MK_PH_BWD_COMBINE 13  /* full layer: k-sum of dX rows (+ router term) */
#define MK_PH_ROUTER_BWD 14   /* router backward: logit gradient, dW_router, d_bias */
#define MK_PH_REPLAY     15   /* re-gather of the x rows of minibatches evicted from the ring */
#define MK_PH_WGRAD_QUANT 16  /* MXFP8 weight gradients: operands quantised along the rows */
#define MK_PH_FUSED_FWD  17   /* fused forward: the one persistent launch (permute, GEMM1, GEMM2) */
#define MK_PH_COUNT      18
int mk_timing_enable(mk_workspace* ws, int32_t on);
int mk_timing_read(mk_workspace* ws, float* ms_out, int32_t* launches_out);
/*
 * Limit the phases that record events while timing is on to those whose bit
 * (1u << MK_PH_x) is set in phase_mask (default: all).  Each recorded event
 * pair costs a few microseconds of stream time, so a benchmark that wants
 * one kernel's duration inside its timed region selects just that phase.
 */
int mk_timing_phases(mk_workspace* ws, uint32_t phase_mask);

/* Enqueue a copy of the schedule's device error word into dst_dev (device
 * uint32). */
int mk_device_error(const mk_schedule* sched, uint32_t* dst_dev, void* stream);

/*
 * For tests of the fused forward's failure path (not for production use):
 * every dependency wait of the fused launch (mk_config.fused_forward) is a
 * bounded poll of a device counter.  spin_limit > 0 sets the bound (in polls,
 * each a counter read and a short sleep; 0 restores the default, about a
 * quarter of a second); unreachable = 1 makes each wait's target one more
 * than its producers ever count, so every wait of the launch ends at its
 * bound.  Such a launch sets MK_DEVERR_WAIT_TIMEOUT in the schedule's error
 * word and runs to its end with every access in bounds; its results are
 * invalid.  Applies to the workspace's later forwards.  Returns MK_OK,
 * MK_ERR_NULL, or MK_ERR_CONFIG (spin_limit < 0 or unreachable not 0/1).
 */
int mk_debug_fused_waits(mk_workspace* ws, int32_t spin_limit, int32_t unreachable);

/* Minibatch floor of the two-wave rule ([MTP] "Three design decisions that
 * matter", overlap granularity): ceil(2 * n_cu * tile_m * tile_n / min(2I, H)). */
int64_t mk_two_wave_rows(int32_t H, int32_t I, int32_t n_cu, int32_t tile_m, int32_t tile_n);

const char* mk_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MK_H_ */
