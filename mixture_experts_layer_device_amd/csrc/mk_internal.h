// Host-side internals of the MoE layer library: the workspace and the
// launchers each kernel file exports to the C ABI in api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

#define MK_TILE_M 256        // rows per GEMM work item
#define MK_TILE_N 256
#define MK_SCHED_CHUNK 256   // rows per schedule workgroup
#define MK_MAX_EXPERTS 1024
#define MK_MAX_TOPK 32

#include <vector>

struct mk_phase_event {
  int phase;
  hipEvent_t start, stop;
};

// Device tables of one dispatch schedule (sizes from the workspace's limits).
struct SchedTables {
  uint32_t* err;              // device error word (MK_DEVERR_*), written whole by the build
  int32_t *mb_counts, *mb_offsets, *counts, *offsets;
  int32_t *sorted_pos, *inv, *items, *mb_items;
};
// Scratch of the schedule build and the sizes its launches use.
// Chunks per (minibatch, expert) column of the chunk histograms, padded to a
// multiple of 4 so each column starts 16-byte aligned.
__host__ __device__ inline int32_t sched_cps(int32_t cpm) { return (cpm + 3) & ~3; }
struct SchedScratch {
  int32_t* chunk_counts;      // [nb_max, E, sched_cps(cpm)] per-chunk expert histograms, by (b, e) column
  int32_t* chunk_bad;         // [nb_max, cpm]: a chunk holds an expert id out of range
};
struct SchedDims {
  int32_t MB, E, cpm, item_cap;
};

struct mk_schedule {
  uint64_t ws_id;             // id of the workspace it was created for
  void* base;
  size_t bytes;
  SchedTables t;
  int32_t E, MB, item_cap;    // the workspace's, for the table sizes
  int32_t R, nb, built;
  // the last forward that used this schedule: its mode, its fwd_ctx and the
  // workspace's ring epoch right after it (the ring still holds this
  // schedule's rows while the epoch is unchanged)
  int32_t fwd_valid, fwd_mode;
  const void* fwd_ctx;
  uint64_t fwd_ring_epoch;
};

struct mk_workspace {
  mk_config cfg;
  uint64_t id;                // process-unique, never reused
  uint64_t ring_epoch;        // bumped by every forward that writes the ring
  int32_t max_rows, H, I, E, k;
  int32_t MB, ring_rows, row_bytes, nb_max, cpm, item_cap, n_cu, device;
  int32_t dbg_wait_spins, dbg_wait_extra;   // mk_debug_fused_waits (0, 0: the default bound)
  int64_t npos;               // nb_max * MB sorted positions
  // device memory
  void* base;
  size_t bytes;
  SchedScratch sscr;
  uint8_t* ring;              // bf16 rows, or MXFP8 codes [ring_rows, H] then scales [ring_rows, H/32]
  uint16_t* a_buf;            // [npos, I] bf16 SwiGLU output, expert order
  uint8_t *a_codes, *a_scales;// MXFP8 copy of a
  float* y_buf;               // [npos, H] fp32 expert outputs, expert order (full-layer combine)
  uint16_t *dye, *dgdu, *wa;  // backward: [npos, H], [npos, 2I], [npos, I]
  float* dw_part;             // [npos, I/32]: router-weight gradient partials, 32 features each
  uint16_t* zero_row;         // 512 zero bytes (weight-gradient rows past a segment's end)
  uint32_t* fused_ctl;        // fused forward: ticket and dependency counters
  uint8_t *dye_c, *dye_s;     // MXFP8 backward: dY rows quantised along H  [npos, H], [npos, H/32]
  uint8_t *dgdu_c, *dgdu_s;   //                 dg/du quantised along 2I   [npos, 2I], [npos, 2I/32]
  float* dz;                  // [ceil(max_rows / k), E]: router logit gradient (and logits)
  float* rpart;               // [rsplits_max, E, H + 1]: router weight-gradient partials
  int32_t rsplits_max;
  // MXFP8 weight gradients: K table of the experts' padded row spaces and the
  // operands quantised along the rows, in the tiled MXFP8 layout
  int32_t *wq_kofs, *wq_order;  // [E+1] start of expert e's K range; [E] experts by descending K
  int32_t* wq_kmap;             // [kcap] position of each K row, -1 for pad rows
  int64_t wq_kcap;              // K capacity (multiple of 128)
  uint8_t *wq_ac, *wq_as;       // A operand: max(H, 2I) x kcap codes, / 32 scales
  uint8_t *wq_bc, *wq_bs;       // B operand: H x kcap codes (H >= I), / 32 scales
  // optional per-phase timing (phases whose bit is set in timing_mask)
  int timing;
  uint32_t timing_mask;
  std::vector<mk_phase_event>* events;
};

namespace mk {

// ---- schedule.hip --------------------------------------------------------
void launch_schedule(const SchedDims& d, const SchedScratch& scr, const SchedTables& t, const int32_t* row_expert,
                     int32_t R, hipStream_t s);

// ---- route.hip -----------------------------------------------------------
void launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H,
                  int E, int k, int renorm, int32_t* idx, float* w, hipStream_t s);
// the router logits alone, z [T, E] fp32, bit-identical to launch_route's
void launch_route_logits(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H,
                         int E, float* z, hipStream_t s);

// ---- router_bwd.hip ------------------------------------------------------
// dz [T, E] = gradient w.r.t. the logits from d_w = gradient w.r.t. the top-k
// weights (renorm 0: dz holds the logits on entry and is overwritten)
void launch_router_dz(const float* d_w, const float* w, const int32_t* idx, int T, int E, int k, int renorm,
                      float* dz, hipStream_t s);
// dX[t] = bf16(sum_j dx32[sorted_pos[t*k + j]] + sum_e dz[t, e] w_router[e]); dz may be null
void launch_dx_combine(const float* dx32, int64_t H, const int32_t* sorted_pos, int k, int64_t T,
                       const float* dz, const uint16_t* w_router, int E, uint16_t* dX, int n_cu,
                       hipStream_t s);
// dW_router [E, H] = dz^T x, d_bias [E] = sum_t dz (d_bias may be null), over NS
// token splits; part holds NS * E * (H + 1) floats
int router_wgrad_splits(int T, int E, int H, int max_splits);
void launch_router_wgrad(const float* dz, const uint16_t* x, int T, int H, int E, int NS, float* part,
                         float* dW_router, float* d_bias, hipStream_t s);

// ---- rows.hip ------------------------------------------------------------
// dst row (p mod ring_rows, or p if ring_rows == 0) <- src row src_of(inv[p]),
// for sorted positions p in [p_lo, p_hi); src_of(r) = r / src_div.
void launch_gather_rows(const uint16_t* src, int64_t H, const int32_t* inv, int src_div,
                        int64_t p_lo, int64_t p_hi, int32_t ring_rows, uint16_t* dst,
                        int n_cu, hipStream_t s);
// (copy: NULL, or also the bf16 rows at their positions p, [p, H])
void launch_gather_rows_mxfp8(const uint16_t* src, int64_t H, const int32_t* inv, int src_div,
                              int64_t p_lo, int64_t p_hi, int32_t ring_rows, uint8_t* codes,
                              uint8_t* scales, int n_cu, hipStream_t s, uint16_t* copy = nullptr);
void launch_combine(const float* y, int64_t H, const int32_t* sorted_pos, const float* row_w,
                    int k, int64_t n_out, uint16_t* out, int n_cu, hipStream_t s);
// zero the out rows whose sorted_pos is -1 (dropped rows; expert-share mode)
void launch_zero_dropped_rows(const int32_t* sorted_pos, int64_t R, uint16_t* out, int64_t H, hipStream_t s);
void launch_quantize(const uint16_t* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                     hipStream_t s);
// dX (arrival-order rows, may be null) gets zero rows where a row was dropped
void launch_dw_finalize(const float* dw_part, int slices, const int32_t* sorted_pos, int64_t R,
                        float* d_row_w, uint16_t* dX, int64_t H, hipStream_t s);
// tiled B operands (btile_* layout in mk_device.h); source rows: mode 0 rows of
// src_a, mode 1 the gate/up interleave of src_a (gate) and src_b (up)
//   tile_rows: B[e][n][k] = row(e, n)[k]    tile_cols: B[e][n][k] = row(e, k)[n]
void launch_tile_rows(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K, uint16_t* out,
                      hipStream_t s);
void launch_tile_cols(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K, uint16_t* out,
                      hipStream_t s);
// tiled MXFP8 B operand (mxt_* layout in mk_device.h), source rows as above,
// quantised along k:  quant_tile_rows: B[e][n][k] = row(e, n)[k]
//                     quant_tile_cols: B[e][n][k] = row(e, k)[n]
void launch_quant_tile_rows(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K,
                            uint8_t* codes, uint8_t* scales, hipStream_t s);
// MXFP8 weight gradients.  K space: expert e owns [kofs[e], kofs[e+1]), its
// minibatch segments in reverse order (nb-1 .. 0), each taking its row count
// rounded up to 32, the expert's total rounded up to 128; order = the experts
// by descending K (ties: lower id first).
void launch_wgrad_kofs(const int32_t* mb_counts, int nb, int E, int32_t* kofs, int32_t* order, hipStream_t s);
// kmap[k] for k < kofs[E]: the position p of K row k, -1 for a pad row
void launch_wgrad_kmap(const int32_t* kofs, const int32_t* mb_counts, const int32_t* mb_offsets, int E, int nb,
                       int MB, int32_t* kmap, hipStream_t s);
// Operand T[c][k] (C columns of the source rows, C % 256 == 0) quantised along
// k in 32-blocks, stored per expert in the tiled MXFP8 layout: expert e's
// blocks start at block (C/256) * kofs[e]/128 and run (row tile c/256, k step);
// row k is position kmap[k] (pad rows are zero); the source row of p is
// src + (inv ? inv[p] / src_div : p) * ld.  Grid covers kcap / 128 k steps;
// steps past kofs[E] exit.
void launch_quant_wgrad_operand(const uint16_t* src, int64_t ld, const int32_t* inv, int src_div, int C,
                                const int32_t* kofs, int E, const int32_t* kmap, int64_t kcap, uint8_t* codes,
                                uint8_t* scales, hipStream_t s);
void launch_quant_tile_cols(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K,
                            uint8_t* codes, uint8_t* scales, hipStream_t s);
void launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);

// ---- gemm_bf16.hip -------------------------------------------------------
struct ItemRange {
  const int32_t* items;     // [cap, 4]
  const int32_t* mb_items;  // [nb+1]
  int32_t mb_lo, mb_hi;     // minibatches covered by this launch
  int32_t item_cap;
};

void launch_gemm1_bf16(const ItemRange& ir, const uint16_t* ring, int32_t ring_rows,
                       const uint16_t* wgu, int H, int I, uint16_t* a_out, float* gu_save,
                       int n_cu, hipStream_t s);
// The bf16 forward's permute, GEMM1 + SwiGLU and GEMM2 in one persistent
// launch, minibatches overlapping (the ring must hold every minibatch: no
// slot reuse inside the launch), or with direct set, GEMM1 reading the x
// rows through the inverse map and no permute (the ring untouched); ctl is
// fused_ctl_words(item_cap) words of device memory (zeroed by the
// launcher), err the schedule's error word.  The full layer's combine (fp32
// y rows from every XCD) is the caller's next launch.
struct FusedFwd {
  ItemRange ir;               // all minibatches
  int nb, src_div, H, I, ring_rows, full;
  int item_local;             // contiguous runs of whole items per XCD (else units dealt evenly)
  int direct;                 // GEMM1 reads x rows through the inverse map (no permute, ring unused)
  int wait_spins;             // bound of each dependency wait in polls (0: the default)
  int wait_extra;             // added to every wait's target (tests of the timeout path)
  const uint16_t* x;
  const int32_t* inv;
  const float* row_w;
  uint16_t* ring;
  const uint16_t *wgu, *wd;
  uint16_t* a_buf;
  float* gu_save;
  float* y32;
  uint16_t* out;
  uint32_t* ctl;
  uint32_t* err;
};
inline int64_t fused_ctl_words(int64_t item_cap) { return 64 * 8 + 2 * item_cap; }
void launch_fused_forward_bf16(const FusedFwd& f, int n_cu, hipStream_t s);
// out != nullptr: expert share, out[inv[p]] = bf16(row_w[inv[p]] * y[p]); else y32[p] = y[p]
void launch_gemm2_bf16(const ItemRange& ir, const uint16_t* a, const uint16_t* wd, int H, int I,
                       float* y32, uint16_t* out, const int32_t* inv, const float* row_w, int n_cu,
                       hipStream_t s);
void launch_bwd_dact(const ItemRange& ir, const uint16_t* dye, const uint16_t* wdT, int H, int I,
                     const float* gu, const int32_t* inv, const float* row_w, uint16_t* dgdu,
                     uint16_t* wa, float* dw_part, int n_cu, hipStream_t s);
// dX != nullptr: dX[inv[p]] = bf16(dX_row[p]) (expert share); else dx32[p] = dX_row[p]
void launch_bwd_dx(const ItemRange& ir, const uint16_t* dgdu, const uint16_t* wguT, int H, int I,
                   const int32_t* inv, uint16_t* dX, float* dx32, int n_cu, hipStream_t s);

struct WgradArgs {
  int E, nb, MB;
  const int32_t* mb_counts;    // [nb, E]
  const int32_t* mb_offsets;   // [nb, E+1]
  const int32_t* inv;
  int src_div;
};
// dW_down[e] (H x I) = sum_p dye[p]^T (x) wa[p]
// (zero_row: 512 zero bytes in device memory, for rows past a segment's end;
// b3: the K loop with the B operand in three LDS buffers, for experts with few rows)
void launch_wgrad_down(const WgradArgs& wa_args, const uint16_t* dye, const uint16_t* wa, int H,
                       int I, float* dW_down, const uint16_t* zero_row, bool b3, int n_cu, hipStream_t s);
// dW_gate/dW_up[e] (I x H) from dgdu ([p, 2I]: I gate, then I up) and the x rows: minibatches
// b >= first_resident come from the ring, earlier (evicted) ones from replay,
// the x rows re-gathered at their positions p ([p, H]).
void launch_wgrad_gate_up(const WgradArgs& wa_args, const uint16_t* dgdu, const uint16_t* ring,
                          int32_t ring_rows, int first_resident, const uint16_t* replay, int H,
                          int I, float* dW_gate, float* dW_up, const uint16_t* zero_row, bool b3, int n_cu,
                          hipStream_t s);

// ---- gemm_mxfp8.hip -----------------------------------------------------
// gu_save: NULL, or the forward context (g and u in fp32, [p, 2I] packed like W_gu).
// inv: NULL (A rows are ring rows, position mod ring_rows), or the inverse map,
// with ring_codes / ring_scales holding token rows: position p reads token
// inv[p] / src_div.
void launch_gemm1_mxfp8(const ItemRange& ir, const uint8_t* ring_codes, const uint8_t* ring_scales,
                        int32_t ring_rows, const uint8_t* wgu_codes, const uint8_t* wgu_scales,
                        int H, int I, uint16_t* a_out, float* gu_save, const int32_t* inv, int src_div, int n_cu,
                        hipStream_t s);
// MXFP8 data-gradient GEMMs (operands quantised along their contraction);
// epilogues as launch_bwd_dact / launch_bwd_dx.  token_src_div > 0: dy_codes /
// dy_scales hold token rows, position p reads token inv[p] / token_src_div;
// 0: rows in expert order
void launch_bwd_dact_mxfp8(const ItemRange& ir, const uint8_t* dy_codes, const uint8_t* dy_scales,
                           const uint8_t* wdT_codes, const uint8_t* wdT_scales, int H, int I, const float* gu,
                           const int32_t* inv, const float* row_w, uint16_t* dgdu, uint16_t* wa, float* dw_part,
                           int token_src_div,
                           int n_cu, hipStream_t s);
// dW_down[e] (H x I) from the tiled operands dY^T (A, H rows) and (w a)^T
// (B, I rows); dW_gate/dW_up[e] (I x H) from [dg|du]^T (A, 2I rows: gate, then up)
// and X^T (B, H rows).  Every (e, m, n) tile by one workgroup over the
// expert's whole K in ascending k: deterministic, no atomics.
void launch_wgrad_down_mxfp8(int E, int H, int I, const int32_t* kofs, const int32_t* order, const uint8_t* ac,
                             const uint8_t* as, const uint8_t* bc, const uint8_t* bs, float* dW_down, int n_cu,
                             hipStream_t s);
void launch_wgrad_gate_up_mxfp8(int E, int H, int I, const int32_t* kofs, const int32_t* order, const uint8_t* ac,
                                const uint8_t* as, const uint8_t* bc, const uint8_t* bs, float* dW_gate,
                                float* dW_up, int n_cu, hipStream_t s);
void launch_bwd_dx_mxfp8(const ItemRange& ir, const uint8_t* dgdu_codes, const uint8_t* dgdu_scales,
                         const uint8_t* wguT_codes, const uint8_t* wguT_scales, int H, int I, const int32_t* inv,
                         uint16_t* dX, float* dx32, int n_cu, hipStream_t s);
void launch_gemm2_mxfp8(const ItemRange& ir, const uint8_t* a_codes, const uint8_t* a_scales,
                        const uint8_t* wd_codes, const uint8_t* wd_scales, int H, int I,
                        float* y32, uint16_t* out, const int32_t* inv, const float* row_w, int n_cu,
                        hipStream_t s);

}  // namespace mk
