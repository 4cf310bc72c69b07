// C ABI of the MoE layer library (declared in include/mk.h): argument
// checks, the workspace, and the launch sequences of forward and backward.
// Every call only enqueues work on the caller's stream.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "mk_device.h"
#include "mk_internal.h"

using namespace mk;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1));
    return o;
  }
};

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

int64_t packed_bytes(const mk_workspace* ws, bool bwd) {
  const int64_t E = ws->E, H = ws->H, I = ws->I;
  if (ws->cfg.precision == MK_MXFP8) {
    int64_t b = (int64_t)align_up(E * 2 * I * H) + (int64_t)align_up(E * 2 * I * H / 32) +
                (int64_t)align_up(E * H * I) + (int64_t)align_up(E * H * I / 32);
    if (bwd)
      b += (int64_t)align_up(E * I * H) + (int64_t)align_up(E * I * H / 32) + (int64_t)align_up(E * H * 2 * I) +
           (int64_t)align_up(E * H * 2 * I / 32);
    return b;
  }
  int64_t b = (int64_t)align_up(E * 2 * I * H * 2) + (int64_t)align_up(E * H * I * 2);
  if (bwd) b += (int64_t)align_up(E * I * H * 2) + (int64_t)align_up(E * H * 2 * I * 2);
  return b;
}

struct PackedBF16 {
  uint16_t *wgu, *wd, *wdT, *wguT;
};
PackedBF16 packed_bf16(const mk_workspace* ws, void* base) {
  const int64_t E = ws->E, H = ws->H, I = ws->I;
  char* p = (char*)base;
  PackedBF16 r;
  r.wgu = (uint16_t*)p;
  p += align_up(E * 2 * I * H * 2);
  r.wd = (uint16_t*)p;
  p += align_up(E * H * I * 2);
  r.wdT = (uint16_t*)p;
  p += align_up(E * I * H * 2);
  r.wguT = (uint16_t*)p;
  return r;
}

struct PackedMX {
  uint8_t *wgu_c, *wgu_s, *wd_c, *wd_s;
  uint8_t *wdT_c, *wdT_s, *wguT_c, *wguT_s;     // backward copies (W_d^T along H, W_gu^T along 2I)
};
PackedMX packed_mx(const mk_workspace* ws, void* base) {
  const int64_t E = ws->E, H = ws->H, I = ws->I;
  char* p = (char*)base;
  PackedMX r;
  r.wgu_c = (uint8_t*)p;
  p += align_up(E * 2 * I * H);
  r.wgu_s = (uint8_t*)p;
  p += align_up(E * 2 * I * H / 32);
  r.wd_c = (uint8_t*)p;
  p += align_up(E * H * I);
  r.wd_s = (uint8_t*)p;
  p += align_up(E * H * I / 32);
  r.wdT_c = (uint8_t*)p;
  p += align_up(E * I * H);
  r.wdT_s = (uint8_t*)p;
  p += align_up(E * I * H / 32);
  r.wguT_c = (uint8_t*)p;
  p += align_up(E * H * 2 * I);
  r.wguT_s = (uint8_t*)p;
  return r;
}

ItemRange item_range(const mk_workspace* ws, const mk_schedule* sc, int mb_lo, int mb_hi) {
  ItemRange ir;
  ir.items = sc->t.items;
  ir.mb_items = sc->t.mb_items;
  ir.mb_lo = mb_lo;
  ir.mb_hi = mb_hi;
  ir.item_cap = ws->item_cap;
  return ir;
}

// A schedule may only be used with the workspace it was created for.
bool sched_ok(const mk_workspace* ws, const mk_schedule* sc) { return ws && sc && sc->ws_id == ws->id; }

uint64_t next_workspace_id() {
  static uint64_t counter = 0;
  return __atomic_add_fetch(&counter, 1, __ATOMIC_RELAXED);
}

int check_launch() { return hipGetLastError() == hipSuccess ? MK_OK : MK_ERR_HIP; }

// Scope that brackets one phase with a pair of events when timing is on.
struct Phase {
  mk_workspace* ws;
  hipStream_t s;
  mk_phase_event ev;
  bool on;
  Phase(mk_workspace* w, int phase, hipStream_t st)
      : ws(w), s(st), on(w->timing != 0 && ((w->timing_mask >> phase) & 1u)) {
    if (!on) return;
    ev.phase = phase;
    if (hipEventCreate(&ev.start) != hipSuccess || hipEventCreate(&ev.stop) != hipSuccess) {
      on = false;
      return;
    }
    (void)hipEventRecord(ev.start, s);
  }
  ~Phase() {
    if (!on) return;
    (void)hipEventRecord(ev.stop, s);
    ws->events->push_back(ev);
  }
};

// Router inputs/outputs of the full-layer backward with the router backward.
struct RouterGrad {
  const uint16_t* w_router;   // [E, H] bf16
  const float* bias;          // [E] or null
  const int32_t* topk_idx;    // [T, k]
  float* dW_router;           // [E, H]
  float* d_bias;              // [E] or null
};

// The backward of both modes.  Expert share: rows in arrival order, dX rows
// straight from the dX GEMM.  Full layer: row r = t*k + j is token t's j-th
// routed row; the dX GEMM keeps its rows in fp32 (reusing the forward's y
// buffer, dead by now) and a combine sums each token's k rows in slot order,
// adds the router term when rg is given, and rounds once.
int backward_impl(mk_workspace* ws, const mk_schedule* sc, int32_t mode, const void* fwd_ctx, const void* x_src,
                  const float* row_w, const void* packed, const void* dY, void* dX, float* dW_gate, float* dW_up,
                  float* dW_down, float* d_row_w, const RouterGrad* rg, void* stream) {
  if (!ws || !sc) return MK_ERR_NULL;
  if (!sched_ok(ws, sc)) return MK_ERR_STATE;
  if (mode != MK_EXPERT_SHARE && mode != MK_FULL_LAYER) return MK_ERR_CONFIG;
  if (!ws->cfg.enable_backward) return MK_ERR_CONFIG;
  const bool mx = ws->cfg.precision == MK_MXFP8;
  const int H = ws->H, I = ws->I, MB = ws->MB, R = sc->R, nb = sc->nb, k = ws->k, E = ws->E;
  // an empty schedule reads no row buffer; the weight gradients become zeros
  if (!dW_gate || !dW_up || !dW_down) return MK_ERR_NULL;
  if (R > 0 && (!fwd_ctx || !x_src || !row_w || !packed || !dY || !dX || !d_row_w)) return MK_ERR_NULL;
  // the backward consumes the forward context of this schedule's last
  // forward, taken in the same mode; with R = 0 there is nothing to consume
  if (!sc->built) return MK_ERR_STATE;
  if (R > 0 && (!sc->fwd_valid || sc->fwd_ctx != fwd_ctx || sc->fwd_mode != mode)) return MK_ERR_STATE;
  const bool full = mode == MK_FULL_LAYER;
  if (full && (R % k || MB % k)) return MK_ERR_SHAPE;
  const int src_div = full ? k : 1;
  const int T = R / src_div;
  hipStream_t s = as_stream(stream);
  PackedBF16 p = packed_bf16(ws, (void*)packed);
  PackedMX pm = packed_mx(ws, (void*)packed);
  const ItemRange all = item_range(ws, sc, 0, nb);
  const SchedTables& st = sc->t;
  const int64_t npos_used = (int64_t)nb * MB;
  // pull the loss gradient into expert order (share of the reverse combine);
  // MXFP8: quantised along H for the dA' GEMM in the same pass, which also
  // keeps the bf16 rows for the down-projection weight gradient.  Full layer
  // with MXFP8 weight gradients (no bf16 copy needed: their dY operand is
  // quantised along the rows straight from the dY rows): a routed row's dY
  // is its token's, so the T token rows are quantised once and the dA' GEMM
  // reads their codes through the inverse map
  const bool dy_tokens = mx && full && ws->cfg.wgrad_mxfp8;
  {
    Phase ph(ws, MK_PH_BWD_GATHER, s);
    if (dy_tokens)
      launch_quantize((const uint16_t*)dY, T, H, ws->dye_c, ws->dye_s, s);
    else if (mx)
      launch_gather_rows_mxfp8((const uint16_t*)dY, H, st.inv, src_div, 0, npos_used, 0, ws->dye_c, ws->dye_s,
                               ws->n_cu, s, ws->cfg.wgrad_mxfp8 ? nullptr : ws->dye);
    else
      launch_gather_rows((const uint16_t*)dY, H, st.inv, src_div, 0, npos_used, 0, ws->dye, ws->n_cu, s);
  }
  // dA' GEMM with the SwiGLU backward and router-weight gradient fused
  {
    Phase ph(ws, MK_PH_BWD_DACT, s);
    if (mx)
      launch_bwd_dact_mxfp8(all, ws->dye_c, ws->dye_s, pm.wdT_c, pm.wdT_s, H, I, (const float*)fwd_ctx, st.inv,
                            row_w, ws->dgdu, ws->wa, ws->dw_part, dy_tokens ? src_div : 0, ws->n_cu, s);
    else
      launch_bwd_dact(all, ws->dye, p.wdT, H, I, (const float*)fwd_ctx, st.inv, row_w, ws->dgdu, ws->wa,
                      ws->dw_part, ws->n_cu, s);
  }
  {
    Phase ph(ws, MK_PH_BWD_DW, s);
    launch_dw_finalize(ws->dw_part, I / 32, st.sorted_pos, R, d_row_w, full ? nullptr : (uint16_t*)dX, H, s);
  }
  // dX GEMM: expert share stores rows back to arrival order (share of the
  // reverse dispatch); the full layer keeps fp32 rows for the k-sum
  if (mx) {
    Phase ph(ws, MK_PH_QUANT_A, s);
    launch_quantize(ws->dgdu, npos_used, 2 * I, ws->dgdu_c, ws->dgdu_s, s);
  }
  {
    Phase ph(ws, MK_PH_BWD_DX, s);
    if (mx)
      launch_bwd_dx_mxfp8(all, ws->dgdu_c, ws->dgdu_s, pm.wguT_c, pm.wguT_s, H, I, st.inv,
                          full ? nullptr : (uint16_t*)dX, ws->y_buf, ws->n_cu, s);
    else
      launch_bwd_dx(all, ws->dgdu, p.wguT, H, I, st.inv, full ? nullptr : (uint16_t*)dX, ws->y_buf, ws->n_cu, s);
  }
  if (full) {
    if (rg) {
      Phase ph(ws, MK_PH_ROUTER_BWD, s);
      if (!ws->cfg.renorm)
        launch_route_logits((const uint16_t*)x_src, rg->w_router, rg->bias, T, H, E, ws->dz, s);
      launch_router_dz(d_row_w, row_w, rg->topk_idx, T, E, k, ws->cfg.renorm, ws->dz, s);
    }
    {
      Phase ph(ws, MK_PH_BWD_COMBINE, s);
      launch_dx_combine(ws->y_buf, H, st.sorted_pos, k, T, rg ? ws->dz : nullptr, rg ? rg->w_router : nullptr, E,
                        (uint16_t*)dX, ws->n_cu, s);
    }
    if (rg) {
      Phase ph(ws, MK_PH_ROUTER_BWD, s);
      const int ns = router_wgrad_splits(T, E, H, ws->rsplits_max);
      launch_router_wgrad(ws->dz, (const uint16_t*)x_src, T, H, E, ns, ws->rpart, rg->dW_router, rg->d_bias, s);
    }
  }
  // weight gradients: row segments in reverse walk order; minibatches still in
  // the ring are read there, the evicted ones are replayed from x_src
  WgradArgs wa;
  wa.E = E;
  wa.nb = nb;
  wa.MB = MB;
  wa.mb_counts = st.mb_counts;
  wa.mb_offsets = st.mb_offsets;
  wa.inv = st.inv;
  wa.src_div = src_div;
  const int ring_mbs = ws->ring_rows / MB;
  // the ring holds this schedule's last minibatches only while no other
  // forward has run on the workspace since this schedule's; else every
  // minibatch is replayed
  const bool ring_ours = R > 0 && sc->fwd_ring_epoch == ws->ring_epoch;
  const int first_resident = ring_ours ? std::max(0, nb - ring_mbs) : nb;
  if (ws->cfg.wgrad_mxfp8) {
    // MXFP8 weight gradients: both operands of each GEMM quantised along the
    // rows (32 rows of one minibatch per block) into the tiled layout; the x
    // rows come straight from x_src through the inverse map (the ring holds
    // them quantised along H, the wrong axis), which is the replay of every
    // minibatch at once
    {
      Phase ph(ws, MK_PH_WGRAD_QUANT, s);
      launch_wgrad_kofs(st.mb_counts, nb, E, ws->wq_kofs, ws->wq_order, s);
      launch_wgrad_kmap(ws->wq_kofs, st.mb_counts, st.mb_offsets, E, nb, MB, ws->wq_kmap, s);
      if (R > 0)
        launch_quant_wgrad_operand((const uint16_t*)dY, H, st.inv, src_div, H, ws->wq_kofs, E, ws->wq_kmap,
                                   ws->wq_kcap, ws->wq_ac, ws->wq_as, s);
      launch_quant_wgrad_operand(ws->wa, I, nullptr, 1, I, ws->wq_kofs, E, ws->wq_kmap, ws->wq_kcap, ws->wq_bc,
                                 ws->wq_bs, s);
    }
    {
      Phase ph(ws, MK_PH_WGRAD_DOWN, s);
      launch_wgrad_down_mxfp8(E, H, I, ws->wq_kofs, ws->wq_order, ws->wq_ac, ws->wq_as, ws->wq_bc, ws->wq_bs, dW_down,
                              ws->n_cu, s);
    }
    {
      Phase ph(ws, MK_PH_WGRAD_QUANT, s);
      launch_quant_wgrad_operand(ws->dgdu, 2 * I, nullptr, 1, 2 * I, ws->wq_kofs, E, ws->wq_kmap, ws->wq_kcap,
                                 ws->wq_ac, ws->wq_as, s);
      if (R > 0)
        launch_quant_wgrad_operand((const uint16_t*)x_src, H, st.inv, src_div, H, ws->wq_kofs, E, ws->wq_kmap,
                                   ws->wq_kcap, ws->wq_bc, ws->wq_bs, s);
    }
    Phase ph(ws, MK_PH_WGRAD_GU, s);
    launch_wgrad_gate_up_mxfp8(E, H, I, ws->wq_kofs, ws->wq_order, ws->wq_ac, ws->wq_as, ws->wq_bc, ws->wq_bs,
                               dW_gate, dW_up, ws->n_cu, s);
    return check_launch();
  }
  // few rows per expert (a few K stages per tile): the weight-gradient K
  // loop with B in three buffers; thousands: both double-buffered
  const bool wgrad_b3 = (int64_t)R < (int64_t)1024 * E;
  {
    Phase ph(ws, MK_PH_WGRAD_DOWN, s);
    launch_wgrad_down(wa, ws->dye, ws->wa, H, I, dW_down, ws->zero_row, wgrad_b3, ws->n_cu, s);
  }
  // replay (the reverse walk's share of re-pulling evicted rows): the x rows
  // of the minibatches no longer in the ring (an MXFP8 ring holds codes: all
  // of them) are gathered again, into the dY rows' buffer, free once the
  // down-projection gradient has read it; the weight-gradient loader reads
  // them there by position
  const int replay_mbs = mx ? nb : first_resident;
  if (replay_mbs > 0) {
    Phase ph(ws, MK_PH_REPLAY, s);
    launch_gather_rows((const uint16_t*)x_src, H, st.inv, src_div, 0, (int64_t)replay_mbs * MB, 0, ws->dye,
                       ws->n_cu, s);
  }
  Phase ph(ws, MK_PH_WGRAD_GU, s);
  launch_wgrad_gate_up(wa, ws->dgdu, (const uint16_t*)ws->ring, ws->ring_rows, replay_mbs, ws->dye, H, I, dW_gate,
                       dW_up, ws->zero_row, wgrad_b3, ws->n_cu, s);
  return check_launch();
}

}  // namespace


extern "C" {

void mk_config_default(mk_config* cfg) {
  if (!cfg) return;
  memset(cfg, 0, sizeof(*cfg));
  cfg->minibatch_rows = 0;
  cfg->precision = MK_BF16;
  cfg->ring_bytes = (int64_t)256 << 20;
  cfg->sched_capacity_mult = 1.0f;
  cfg->renorm = 1;
  cfg->enable_backward = 0;
}

int mk_workspace_create(const mk_config* cfg, int32_t max_rows, int32_t H, int32_t I, int32_t E, int32_t k,
                        mk_workspace** out) {
  if (!cfg || !out) return MK_ERR_NULL;
  *out = nullptr;
  if (max_rows < 1 || H < 256 || I < 128 || H % 256 || I % 128) return MK_ERR_SHAPE;
  if (E < 1 || E > MK_MAX_EXPERTS || k < 1 || k > MK_MAX_TOPK) return MK_ERR_LIMIT;
  if (cfg->precision != MK_BF16 && cfg->precision != MK_MXFP8) return MK_ERR_CONFIG;
  if (cfg->minibatch_rows < 0 || !(cfg->sched_capacity_mult > 0.f) || cfg->ring_bytes <= 0) return MK_ERR_CONFIG;
  if (cfg->ring_bytes >= ((int64_t)1 << 31)) return MK_ERR_LIMIT;
  if (cfg->enable_backward && I % 256) return MK_ERR_SHAPE;
  if (cfg->wgrad_mxfp8 && (cfg->precision != MK_MXFP8 || !cfg->enable_backward)) return MK_ERR_CONFIG;
  if (cfg->fused_forward && cfg->precision != MK_BF16) return MK_ERR_CONFIG;

  mk_workspace* ws = (mk_workspace*)calloc(1, sizeof(mk_workspace));
  if (!ws) return MK_ERR_HIP;
  ws->id = next_workspace_id();
  ws->events = new std::vector<mk_phase_event>();
  ws->timing_mask = 0xFFFFFFFFu;
  ws->cfg = *cfg;
  ws->max_rows = max_rows;
  ws->H = H;
  ws->I = I;
  ws->E = E;
  ws->k = k;
  ws->MB = cfg->minibatch_rows > 0 ? cfg->minibatch_rows : max_rows;
  ws->row_bytes = cfg->precision == MK_MXFP8 ? H + H / 32 : 2 * H;
  const int64_t mbs_in_ring = cfg->ring_bytes / ((int64_t)ws->MB * ws->row_bytes);
  if (mbs_in_ring < 1) {
    delete ws->events;
    free(ws);
    return MK_ERR_RING;
  }
  if ((int64_t)ws->MB * mbs_in_ring > INT32_MAX / 2) {
    delete ws->events;
    free(ws);
    return MK_ERR_LIMIT;
  }
  ws->ring_rows = (int32_t)((int64_t)ws->MB * mbs_in_ring);
  ws->nb_max = (max_rows + ws->MB - 1) / ws->MB;
  // the schedule kernels launch one workgroup row per minibatch (grid y)
  if (ws->nb_max > 65535) {
    delete ws->events;
    free(ws);
    return MK_ERR_LIMIT;
  }
  ws->npos = (int64_t)ws->nb_max * ws->MB;
  ws->cpm = (ws->MB + MK_SCHED_CHUNK - 1) / MK_SCHED_CHUNK;
  const double worst = (double)((max_rows + MK_TILE_M - 1) / MK_TILE_M) + (double)ws->nb_max * E;
  ws->item_cap = (int32_t)std::max(1.0, std::ceil(cfg->sched_capacity_mult * worst));
  if (cfg->wgrad_mxfp8) {
    // the MXFP8 weight gradients' row space: every segment rounded up to 32
    // rows, every expert to 128; the quantisers launch one workgroup row per
    // 128-row K step (grid y)
    const int64_t kc = (int64_t)max_rows + (int64_t)ws->nb_max * E * 31 + (int64_t)E * 127;
    ws->wq_kcap = (kc + 127) / 128 * 128;
    if (ws->wq_kcap / 128 > 65535) {
      delete ws->events;
      free(ws);
      return MK_ERR_LIMIT;
    }
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    delete ws->events;
    free(ws);
    return MK_ERR_HIP;
  }
  ws->device = dev;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 8) {
    delete ws->events;
    free(ws);
    return MK_ERR_HIP;
  }
  ws->n_cu = ncu / 8 * 8;

  const int64_t npos = ws->npos;
  Carver c;
  const size_t o_zero = c.take(512);
  const size_t o_fctl = c.take((size_t)fused_ctl_words(ws->item_cap) * 4);
  const size_t o_cc = c.take((size_t)ws->nb_max * sched_cps(ws->cpm) * E * 4);
  const size_t o_cb = c.take((size_t)ws->nb_max * ws->cpm * 4);
  const size_t o_ring = c.take((size_t)ws->ring_rows * ws->row_bytes);
  const size_t o_a = c.take((size_t)npos * I * 2);
  size_t o_ac = 0, o_as = 0;
  if (cfg->precision == MK_MXFP8) {
    o_ac = c.take((size_t)npos * I);
    o_as = c.take((size_t)npos * I / 32);
  }
  const size_t o_y = c.take((size_t)npos * H * 4);
  size_t o_dye = 0, o_dgdu = 0, o_wa = 0, o_dwp = 0, o_dz = 0, o_rp = 0, o_dyc = 0, o_dys = 0, o_gc = 0, o_gs = 0;
  if (cfg->enable_backward) {
    o_dye = c.take((size_t)npos * H * 2);
    o_dgdu = c.take((size_t)npos * 2 * I * 2);
    o_wa = c.take((size_t)npos * I * 2);
    o_dwp = c.take((size_t)npos * (I / 32) * 4);
    o_dz = c.take((size_t)((max_rows + k - 1) / k) * E * 4);
    if (cfg->precision == MK_MXFP8) {
      o_dyc = c.take((size_t)npos * H);
      o_dys = c.take((size_t)npos * H / 32);
      o_gc = c.take((size_t)npos * 2 * I);
      o_gs = c.take((size_t)npos * 2 * I / 32);
    }
    // token splits of the router weight gradient: ~256 tokens each, partials
    // capped at 64 MiB
    const int64_t per_split = (int64_t)E * (H + 1) * 4;
    ws->rsplits_max = (int32_t)std::max<int64_t>(1, std::min<int64_t>(64, ((int64_t)64 << 20) / per_split));
    o_rp = c.take((size_t)ws->rsplits_max * per_split);
  }
  size_t o_wk = 0, o_wo = 0, o_wm = 0, o_wac = 0, o_was = 0, o_wbc = 0, o_wbs = 0;
  if (cfg->wgrad_mxfp8) {
    // every expert's K range: its minibatch segments rounded up to 32 rows,
    // the total to 128
    const int64_t ca = std::max(H, 2 * I), cb = std::max(H, I);
    o_wk = c.take((size_t)(E + 1) * 4);
    o_wo = c.take((size_t)E * 4);
    o_wm = c.take((size_t)ws->wq_kcap * 4);
    o_wac = c.take((size_t)(ca * ws->wq_kcap));
    o_was = c.take((size_t)(ca * ws->wq_kcap / 32));
    o_wbc = c.take((size_t)(cb * ws->wq_kcap));
    o_wbs = c.take((size_t)(cb * ws->wq_kcap / 32));
  }
  ws->bytes = c.off;
  if (hipMalloc(&ws->base, ws->bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete ws->events;
    free(ws);
    return MK_ERR_HIP;
  }
  char* b = (char*)ws->base;
  ws->zero_row = (uint16_t*)(b + o_zero);
  ws->fused_ctl = (uint32_t*)(b + o_fctl);
  ws->sscr.chunk_counts = (int32_t*)(b + o_cc);
  ws->sscr.chunk_bad = (int32_t*)(b + o_cb);
  ws->ring = (uint8_t*)(b + o_ring);
  ws->a_buf = (uint16_t*)(b + o_a);
  if (cfg->precision == MK_MXFP8) {
    ws->a_codes = (uint8_t*)(b + o_ac);
    ws->a_scales = (uint8_t*)(b + o_as);
  }
  ws->y_buf = (float*)(b + o_y);
  if (cfg->enable_backward) {
    ws->dye = (uint16_t*)(b + o_dye);
    ws->dgdu = (uint16_t*)(b + o_dgdu);
    ws->wa = (uint16_t*)(b + o_wa);
    ws->dw_part = (float*)(b + o_dwp);
    ws->dz = (float*)(b + o_dz);
    ws->rpart = (float*)(b + o_rp);
    if (cfg->precision == MK_MXFP8) {
      ws->dye_c = (uint8_t*)(b + o_dyc);
      ws->dye_s = (uint8_t*)(b + o_dys);
      ws->dgdu_c = (uint8_t*)(b + o_gc);
      ws->dgdu_s = (uint8_t*)(b + o_gs);
    }
  }
  if (cfg->wgrad_mxfp8) {
    ws->wq_kofs = (int32_t*)(b + o_wk);
    ws->wq_order = (int32_t*)(b + o_wo);
    ws->wq_kmap = (int32_t*)(b + o_wm);
    ws->wq_ac = (uint8_t*)(b + o_wac);
    ws->wq_as = (uint8_t*)(b + o_was);
    ws->wq_bc = (uint8_t*)(b + o_wbc);
    ws->wq_bs = (uint8_t*)(b + o_wbs);
  }
  // the zero row is zero
  launch_fill_u32((uint32_t*)ws->zero_row, 0u, 128, nullptr);
  if (hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(ws->base);
    delete ws->events;
    free(ws);
    return MK_ERR_HIP;
  }
  *out = ws;
  return MK_OK;
}

int mk_workspace_destroy(mk_workspace* ws) {
  if (!ws) return MK_ERR_NULL;
  int rc = MK_OK;
  for (auto& ev : *ws->events) {
    (void)hipEventDestroy(ev.start);
    (void)hipEventDestroy(ev.stop);
  }
  delete ws->events;
  if (ws->base && hipFree(ws->base) != hipSuccess) rc = MK_ERR_HIP;
  free(ws);
  return rc;
}

int64_t mk_query(const mk_workspace* ws, int32_t what) {
  if (!ws) return MK_ERR_NULL;
  switch (what) {
    case MK_Q_RING_ROWS: return ws->ring_rows;
    case MK_Q_MINIBATCH_ROWS: return ws->MB;
    case MK_Q_ITEM_CAPACITY: return ws->item_cap;
    case MK_Q_TILE_M: return MK_TILE_M;
    case MK_Q_NUM_CU: return ws->n_cu;
    case MK_Q_PACKED_BYTES: return packed_bytes(ws, false);
    case MK_Q_PACKED_BYTES_BWD: return packed_bytes(ws, true);
    case MK_Q_FWD_CTX_BYTES: return ws->npos * 2 * ws->I * 4;
    default: return MK_ERR_CONFIG;
  }
}

int mk_route(mk_workspace* ws, const void* x, const void* w_router, const float* bias, int32_t T, int32_t* topk_idx,
             float* topk_w, void* stream) {
  if (!ws || !w_router || (T > 0 && (!x || !topk_idx || !topk_w))) return MK_ERR_NULL;
  if (T < 0) return MK_ERR_SHAPE;
  if ((int64_t)T * ws->k > ws->max_rows) return MK_ERR_LIMIT;
  if (ws->k > ws->E) return MK_ERR_SHAPE;
  Phase ph(ws, MK_PH_ROUTE, as_stream(stream));
  launch_route((const uint16_t*)x, (const uint16_t*)w_router, bias, T, ws->H, ws->E, ws->k, ws->cfg.renorm, topk_idx,
               topk_w, as_stream(stream));
  return check_launch();
}

int mk_schedule_create(mk_workspace* ws, mk_schedule** out) {
  if (!ws || !out) return MK_ERR_NULL;
  *out = nullptr;
  const int E = ws->E;
  Carver c;
  const size_t o_err = c.take(256);
  const size_t o_mbc = c.take((size_t)ws->nb_max * E * 4);
  const size_t o_mbo = c.take((size_t)ws->nb_max * (E + 1) * 4);
  const size_t o_cnt = c.take((size_t)E * 4);
  const size_t o_off = c.take((size_t)(E + 1) * 4);
  const size_t o_sp = c.take((size_t)ws->max_rows * 4);
  const size_t o_inv = c.take((size_t)ws->npos * 4);
  const size_t o_items = c.take((size_t)ws->item_cap * 16);
  const size_t o_mbi = c.take((size_t)(ws->nb_max + 1) * 4);
  mk_schedule* sc = (mk_schedule*)calloc(1, sizeof(mk_schedule));
  if (!sc) return MK_ERR_HIP;
  sc->ws_id = ws->id;
  sc->E = ws->E;
  sc->MB = ws->MB;
  sc->item_cap = ws->item_cap;
  sc->bytes = c.off;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != ws->device || hipMalloc(&sc->base, sc->bytes) != hipSuccess) {
    (void)hipGetLastError();
    free(sc);
    return MK_ERR_HIP;
  }
  char* b = (char*)sc->base;
  sc->t.err = (uint32_t*)(b + o_err);
  sc->t.mb_counts = (int32_t*)(b + o_mbc);
  sc->t.mb_offsets = (int32_t*)(b + o_mbo);
  sc->t.counts = (int32_t*)(b + o_cnt);
  sc->t.offsets = (int32_t*)(b + o_off);
  sc->t.sorted_pos = (int32_t*)(b + o_sp);
  sc->t.inv = (int32_t*)(b + o_inv);
  sc->t.items = (int32_t*)(b + o_items);
  sc->t.mb_items = (int32_t*)(b + o_mbi);
  // the error word starts clear
  launch_fill_u32(sc->t.err, 0u, 1, nullptr);
  if (hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(sc->base);
    free(sc);
    return MK_ERR_HIP;
  }
  *out = sc;
  return MK_OK;
}

int mk_schedule_destroy(mk_schedule* sc) {
  if (!sc) return MK_ERR_NULL;
  int rc = MK_OK;
  if (sc->base && hipFree(sc->base) != hipSuccess) rc = MK_ERR_HIP;
  free(sc);
  return rc;
}

int64_t mk_schedule_query(const mk_schedule* sc, int32_t what) {
  if (!sc) return MK_ERR_NULL;
  switch (what) {
    case MK_Q_NUM_MB: return sc->built ? sc->nb : 0;
    case MK_Q_ROWS: return sc->built ? sc->R : 0;
    default: return MK_ERR_CONFIG;
  }
}

int mk_build_schedule(mk_workspace* ws, mk_schedule* sc, const int32_t* row_expert, int32_t R, void* stream) {
  if (!ws || !sc || (!row_expert && R > 0)) return MK_ERR_NULL;
  if (!sched_ok(ws, sc)) return MK_ERR_STATE;
  if (R < 0) return MK_ERR_SHAPE;
  if (R > ws->max_rows) return MK_ERR_LIMIT;
  {
    Phase ph(ws, MK_PH_SCHEDULE, as_stream(stream));
    const SchedDims d{ws->MB, ws->E, ws->cpm, ws->item_cap};
    launch_schedule(d, ws->sscr, sc->t, row_expert, R, as_stream(stream));
  }
  sc->R = R;
  sc->nb = R > 0 ? (R + ws->MB - 1) / ws->MB : 0;
  sc->built = 1;
  sc->fwd_valid = 0;          // a new schedule has had no forward yet
  sc->fwd_ctx = nullptr;
  return check_launch();
}

int mk_schedule_copy(const mk_schedule* sc, int32_t table, void* dst, int64_t bytes, void* stream) {
  if (!sc || !dst) return MK_ERR_NULL;
  const void* src = nullptr;
  int64_t have = 0;
  // sizes of the last build (E, MB and the capacity are fixed per workspace
  // and recorded with the tables)
  const int nb = sc->built ? sc->nb : 0;
  const int64_t E = sc->E, MB = sc->MB;
  switch (table) {
    case MK_TAB_COUNTS: src = sc->t.counts; have = E * 4; break;
    case MK_TAB_OFFSETS: src = sc->t.offsets; have = (E + 1) * 4; break;
    case MK_TAB_MB_COUNTS: src = sc->t.mb_counts; have = (int64_t)nb * E * 4; break;
    case MK_TAB_MB_OFFSETS: src = sc->t.mb_offsets; have = (int64_t)nb * (E + 1) * 4; break;
    case MK_TAB_SORTED_POS: src = sc->t.sorted_pos; have = (int64_t)(sc->built ? sc->R : 0) * 4; break;
    case MK_TAB_INV: src = sc->t.inv; have = (int64_t)nb * MB * 4; break;
    case MK_TAB_ITEMS: src = sc->t.items; have = (int64_t)sc->item_cap * 16; break;
    case MK_TAB_MB_ITEMS: src = sc->t.mb_items; have = (int64_t)(nb + 1) * 4; break;
    default: return MK_ERR_CONFIG;
  }
  if (bytes < 0 || bytes > have) return MK_ERR_LIMIT;
  if (bytes == 0) return MK_OK;
  return hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToDevice, as_stream(stream)) == hipSuccess
             ? MK_OK
             : MK_ERR_HIP;
}

int mk_workspace_copy(const mk_workspace* ws, int32_t buffer, void* dst, int64_t bytes, void* stream) {
  if (!ws || !dst) return MK_ERR_NULL;
  const void* src = nullptr;
  int64_t have = 0;
  const int64_t npos = ws->npos, H = ws->H, I = ws->I;
  const bool mx = ws->cfg.precision == MK_MXFP8, bwd = ws->cfg.enable_backward != 0;
  switch (buffer) {
    case MK_BUF_RING: src = ws->ring; have = (int64_t)ws->ring_rows * ws->row_bytes; break;
    case MK_BUF_A: src = ws->a_buf; have = npos * I * 2; break;
    case MK_BUF_A_CODES: src = mx ? ws->a_codes : nullptr; have = npos * I; break;
    case MK_BUF_A_SCALES: src = mx ? ws->a_scales : nullptr; have = npos * I / 32; break;
    case MK_BUF_Y: src = ws->y_buf; have = npos * H * 4; break;
    case MK_BUF_DGDU: src = bwd ? ws->dgdu : nullptr; have = npos * 2 * I * 2; break;
    case MK_BUF_DGDU_CODES: src = bwd && mx ? ws->dgdu_c : nullptr; have = npos * 2 * I; break;
    case MK_BUF_DGDU_SCALES: src = bwd && mx ? ws->dgdu_s : nullptr; have = npos * 2 * I / 32; break;
    case MK_BUF_WA: src = bwd ? ws->wa : nullptr; have = npos * I * 2; break;
    case MK_BUF_DY_CODES: src = bwd && mx ? ws->dye_c : nullptr; have = npos * H; break;
    case MK_BUF_DY_SCALES: src = bwd && mx ? ws->dye_s : nullptr; have = npos * H / 32; break;
    default: return MK_ERR_CONFIG;
  }
  if (!src) return MK_ERR_CONFIG;
  if (bytes < 0 || bytes > have) return MK_ERR_LIMIT;
  if (bytes == 0) return MK_OK;
  return hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToDevice, as_stream(stream)) == hipSuccess
             ? MK_OK
             : MK_ERR_HIP;
}

int mk_mxfp8_quantize(const void* in, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows > 0 && (!in || !codes || !scales)) return MK_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 32) return MK_ERR_SHAPE;
  launch_quantize((const uint16_t*)in, rows, K, codes, scales, as_stream(stream));
  return check_launch();
}

int mk_prepare_weights(mk_workspace* ws, const void* w_gate, const void* w_up, const void* w_down,
                       int32_t for_backward, void* packed, void* stream) {
  if (!ws || !w_gate || !w_up || !w_down || !packed) return MK_ERR_NULL;
  hipStream_t s = as_stream(stream);
  const int E = ws->E, H = ws->H, I = ws->I;
  if (ws->cfg.precision == MK_MXFP8) {
    PackedMX p = packed_mx(ws, packed);
    const uint16_t *wg = (const uint16_t*)w_gate, *wu = (const uint16_t*)w_up, *wd = (const uint16_t*)w_down;
    launch_quant_tile_rows(wg, wu, 1, E, 2 * I, H, p.wgu_c, p.wgu_s, s);      // GEMM1 B along H
    launch_quant_tile_rows(wd, nullptr, 0, E, H, I, p.wd_c, p.wd_s, s);       // GEMM2 B along I
    if (for_backward) {
      launch_quant_tile_cols(wd, nullptr, 0, E, I, H, p.wdT_c, p.wdT_s, s);   // dA' B: W_d^T along H
      launch_quant_tile_cols(wg, wu, 2, E, H, 2 * I, p.wguT_c, p.wguT_s, s);  // dX B: [W_g; W_u]^T along 2I
    }
    return check_launch();
  }
  PackedBF16 p = packed_bf16(ws, packed);
  const uint16_t *wg = (const uint16_t*)w_gate, *wu = (const uint16_t*)w_up, *wd = (const uint16_t*)w_down;
  launch_tile_rows(wg, wu, 1, E, 2 * I, H, p.wgu, s);      // GEMM1 B: [E][2I][H]
  launch_tile_rows(wd, nullptr, 0, E, H, I, p.wd, s);      // GEMM2 B: [E][H][I]
  if (for_backward) {
    launch_tile_cols(wd, nullptr, 0, E, I, H, p.wdT, s);   // dA' B: W_d^T [E][I][H]
    launch_tile_cols(wg, wu, 2, E, H, 2 * I, p.wguT, s);   // dX B: [W_g; W_u]^T [E][H][2I]
  }
  return check_launch();
}

int mk_forward(mk_workspace* ws, mk_schedule* sc, int32_t mode, const void* x_src, const float* row_w,
               const void* packed, void* out, void* fwd_ctx, void* stream) {
  if (!ws || !sc) return MK_ERR_NULL;
  if (!sched_ok(ws, sc) || !sc->built) return MK_ERR_STATE;
  const int R = sc->R;
  if (R > 0 && (!x_src || !row_w || !packed || !out)) return MK_ERR_NULL;
  if (mode != MK_FULL_LAYER && mode != MK_EXPERT_SHARE) return MK_ERR_CONFIG;
  const int H = ws->H, I = ws->I, MB = ws->MB, k = ws->k;
  int src_div = 1, kk = 1;
  if (mode == MK_FULL_LAYER) {
    if (R % k || MB % k) return MK_ERR_SHAPE;
    src_div = k;
    kk = k;
  }
  const bool mx = ws->cfg.precision == MK_MXFP8;
  // what the backward of this schedule will check: the mode, the context it
  // must be handed, and the ring epoch right after this forward's permute
  sc->fwd_valid = 1;
  sc->fwd_mode = mode;
  sc->fwd_ctx = fwd_ctx;
  if (R == 0) {
    sc->fwd_ring_epoch = 0;   // nothing was written to the ring
    return MK_OK;
  }
  sc->fwd_ring_epoch = ++ws->ring_epoch;
  hipStream_t s = as_stream(stream);
  const int nb = sc->nb;
  const SchedTables& st = sc->t;
  const int ring_mbs = ws->ring_rows / MB;
  const uint16_t* x = (const uint16_t*)x_src;
  const bool share = mode == MK_EXPERT_SHARE;
  // expert share: GEMM2 writes w*y straight to arrival order (one rounding);
  // full layer: GEMM2 keeps y in fp32 and the combine sums the k rows
  uint16_t* out_fused = share ? (uint16_t*)out : nullptr;
  // full layer: GEMM1 can gather its A rows straight from the token rows
  // (each token row serves k experts and stays in the last-level cache), so
  // the fused launch writes no ring and needs none
  const bool direct = !share && (int64_t)(R / kk) * H * 2 <= ((int64_t)1 << 32);
  if (ws->cfg.fused_forward && (direct || nb <= ring_mbs)) {
    // one persistent launch for GEMM1 and GEMM2 (and the permute into the
    // ring, which then holds every minibatch), minibatches overlapping; the
    // full layer's combine follows as its own launch
    FusedFwd f;
    f.ir = item_range(ws, sc, 0, nb);
    f.nb = nb;
    f.src_div = src_div;
    f.H = H;
    f.I = I;
    f.ring_rows = ws->ring_rows;
    f.full = !share;
    // placement of the units on the XCDs: with fewer than 2 tiles of rows
    // per expert in a minibatch on average, contiguous runs of whole items
    // per XCD (an item's ring and a rows stay in that L2, and an expert's
    // few items share its weight panels there); with more, spread every
    // segment's units evenly so that a panel stays on one XCD across the
    // expert's items
    f.item_local = (int64_t)std::min(MB, R) < (int64_t)2 * MK_TILE_M * ws->E;
    // without the ring a backward of this schedule replays the x rows
    f.direct = direct;
    if (f.direct) sc->fwd_ring_epoch = 0;
    f.wait_spins = ws->dbg_wait_spins;
    f.wait_extra = ws->dbg_wait_extra;
    f.x = x;
    f.inv = st.inv;
    f.row_w = row_w;
    f.ring = (uint16_t*)ws->ring;
    f.wgu = packed_bf16(ws, (void*)packed).wgu;
    f.wd = packed_bf16(ws, (void*)packed).wd;
    f.a_buf = ws->a_buf;
    f.gu_save = (float*)fwd_ctx;
    f.y32 = ws->y_buf;
    f.out = (uint16_t*)out;
    f.ctl = ws->fused_ctl;
    f.err = st.err;
    {
      Phase ph(ws, MK_PH_FUSED_FWD, s);
      launch_fused_forward_bf16(f, ws->n_cu, s);
    }
    Phase ph(ws, MK_PH_COMBINE, s);
    if (share)
      launch_zero_dropped_rows(st.sorted_pos, R, (uint16_t*)out, H, s);
    else
      launch_combine(ws->y_buf, H, st.sorted_pos, row_w, kk, (int64_t)R / kk, (uint16_t*)out, ws->n_cu, s);
    return check_launch();
  }
  if (!mx) {
    PackedBF16 p = packed_bf16(ws, (void*)packed);
    for (int b0 = 0; b0 < nb; b0 += ring_mbs) {
      const int b1 = std::min(nb, b0 + ring_mbs);
      {
        Phase ph(ws, MK_PH_PERMUTE, s);
        launch_gather_rows(x, H, st.inv, src_div, (int64_t)b0 * MB, (int64_t)b1 * MB, ws->ring_rows,
                           (uint16_t*)ws->ring, ws->n_cu, s);
      }
      Phase ph(ws, MK_PH_GEMM1, s);
      launch_gemm1_bf16(item_range(ws, sc, b0, b1), (const uint16_t*)ws->ring, ws->ring_rows, p.wgu, H, I,
                        ws->a_buf, (float*)fwd_ctx, ws->n_cu, s);
    }
    Phase ph(ws, MK_PH_GEMM2, s);
    launch_gemm2_bf16(item_range(ws, sc, 0, nb), ws->a_buf, p.wd, H, I, ws->y_buf, out_fused, st.inv, row_w,
                      ws->n_cu, s);
  } else {
    PackedMX p = packed_mx(ws, (void*)packed);
    uint8_t* rc = ws->ring;
    uint8_t* rsc = ws->ring + (size_t)ws->ring_rows * H;
    // full layer with its token rows fitting the ring: the T token rows are
    // quantised once into the ring (a routed row's codes are its token's) and
    // GEMM1 reads them through the inverse map, every minibatch in one
    // launch; the MXFP8 backward reads no ring rows (it gathers x again)
    const int64_t T = R / kk;
    if (!share && T <= ws->ring_rows) {
      sc->fwd_ring_epoch = 0;
      {
        Phase ph(ws, MK_PH_PERMUTE, s);
        launch_quantize(x, T, H, rc, rsc, s);
      }
      Phase ph(ws, MK_PH_GEMM1, s);
      launch_gemm1_mxfp8(item_range(ws, sc, 0, nb), rc, rsc, ws->ring_rows, p.wgu_c, p.wgu_s, H, I, ws->a_buf,
                         (float*)fwd_ctx, st.inv, src_div, ws->n_cu, s);
    }
    for (int b0 = 0; b0 < nb && (share || T > ws->ring_rows); b0 += ring_mbs) {
      const int b1 = std::min(nb, b0 + ring_mbs);
      {
        Phase ph(ws, MK_PH_PERMUTE, s);
        launch_gather_rows_mxfp8(x, H, st.inv, src_div, (int64_t)b0 * MB, (int64_t)b1 * MB, ws->ring_rows, rc,
                                 rsc, ws->n_cu, s);
      }
      Phase ph(ws, MK_PH_GEMM1, s);
      launch_gemm1_mxfp8(item_range(ws, sc, b0, b1), rc, rsc, ws->ring_rows, p.wgu_c, p.wgu_s, H, I, ws->a_buf,
                         (float*)fwd_ctx, nullptr, 1, ws->n_cu, s);
    }
    {
      Phase ph(ws, MK_PH_QUANT_A, s);
      launch_quantize(ws->a_buf, (int64_t)nb * MB, I, ws->a_codes, ws->a_scales, s);
    }
    Phase ph(ws, MK_PH_GEMM2, s);
    launch_gemm2_mxfp8(item_range(ws, sc, 0, nb), ws->a_codes, ws->a_scales, p.wd_c, p.wd_s, H, I, ws->y_buf,
                       out_fused, st.inv, row_w, ws->n_cu, s);
  }
  Phase ph(ws, MK_PH_COMBINE, s);
  if (share)
    launch_zero_dropped_rows(st.sorted_pos, R, (uint16_t*)out, H, s);
  else
    launch_combine(ws->y_buf, H, st.sorted_pos, row_w, kk, (int64_t)R / kk, (uint16_t*)out, ws->n_cu, s);
  return check_launch();
}

int mk_backward(mk_workspace* ws, const mk_schedule* sc, int32_t mode, const void* fwd_ctx, const void* x_src,
                const float* row_w, const void* packed, const void* dY, void* dX, float* dW_gate, float* dW_up,
                float* dW_down, float* d_row_w, void* stream) {
  return backward_impl(ws, sc, mode, fwd_ctx, x_src, row_w, packed, dY, dX, dW_gate, dW_up, dW_down, d_row_w,
                       nullptr, stream);
}

int mk_backward_layer(mk_workspace* ws, const mk_schedule* sc, const void* fwd_ctx, const void* x,
                      const void* w_router, const float* bias, const int32_t* topk_idx, const float* topk_w,
                      const void* packed, const void* dY, void* dX, float* dW_gate, float* dW_up, float* dW_down,
                      float* dW_router, float* d_bias, float* d_topk_w, void* stream) {
  if (!ws || !sc) return MK_ERR_NULL;
  if (!sched_ok(ws, sc) || !sc->built) return MK_ERR_STATE;
  if (!w_router || !dW_router || (sc->R > 0 && !topk_idx)) return MK_ERR_NULL;
  RouterGrad rg{(const uint16_t*)w_router, bias, topk_idx, dW_router, d_bias};
  return backward_impl(ws, sc, MK_FULL_LAYER, fwd_ctx, x, topk_w, packed, dY, dX, dW_gate, dW_up, dW_down, d_topk_w,
                       &rg, stream);
}

int mk_timing_enable(mk_workspace* ws, int32_t on) {
  if (!ws) return MK_ERR_NULL;
  ws->timing = on ? 1 : 0;
  return MK_OK;
}

int mk_debug_fused_waits(mk_workspace* ws, int32_t spin_limit, int32_t unreachable) {
  if (!ws) return MK_ERR_NULL;
  if (spin_limit < 0 || (unreachable != 0 && unreachable != 1)) return MK_ERR_CONFIG;
  ws->dbg_wait_spins = spin_limit;
  ws->dbg_wait_extra = unreachable;
  return MK_OK;
}

int mk_timing_phases(mk_workspace* ws, uint32_t phase_mask) {
  if (!ws) return MK_ERR_NULL;
  ws->timing_mask = phase_mask;
  return MK_OK;
}

int mk_timing_read(mk_workspace* ws, float* ms_out, int32_t* launches_out) {
  if (!ws) return MK_ERR_NULL;
  float ms[MK_PH_COUNT] = {0};
  int32_t n[MK_PH_COUNT] = {0};
  int rc = MK_OK;
  for (auto& ev : *ws->events) {
    float t = 0.f;
    if (hipEventSynchronize(ev.stop) != hipSuccess || hipEventElapsedTime(&t, ev.start, ev.stop) != hipSuccess)
      rc = MK_ERR_HIP;
    if (ev.phase >= 0 && ev.phase < MK_PH_COUNT) {
      ms[ev.phase] += t;
      n[ev.phase] += 1;
    }
    (void)hipEventDestroy(ev.start);
    (void)hipEventDestroy(ev.stop);
  }
  ws->events->clear();
  for (int i = 0; i < MK_PH_COUNT; ++i) {
    if (ms_out) ms_out[i] = ms[i];
    if (launches_out) launches_out[i] = n[i];
  }
  return rc;
}

int mk_device_error(const mk_schedule* sc, uint32_t* dst, void* stream) {
  if (!sc || !dst) return MK_ERR_NULL;
  return hipMemcpyAsync(dst, sc->t.err, 4, hipMemcpyDeviceToDevice, as_stream(stream)) == hipSuccess ? MK_OK
                                                                                                      : MK_ERR_HIP;
}

int64_t mk_two_wave_rows(int32_t H, int32_t I, int32_t n_cu, int32_t tile_m, int32_t tile_n) {
  if (H <= 0 || I <= 0 || n_cu <= 0 || tile_m <= 0 || tile_n <= 0) return MK_ERR_SHAPE;
  const int64_t num = 2LL * n_cu * tile_m * tile_n;
  const int64_t den = std::min<int64_t>(2LL * I, H);
  return (num + den - 1) / den;
}

const char* mk_status_string(int status) {
  switch (status) {
    case MK_OK: return "ok";
    case MK_ERR_NULL: return "a required pointer is NULL";
    case MK_ERR_SHAPE: return "unsupported shape";
    case MK_ERR_RING: return "ring smaller than one minibatch";
    case MK_ERR_LIMIT: return "above a workspace limit";
    case MK_ERR_HIP: return "HIP runtime call failed";
    case MK_ERR_STATE: return "call out of order";
    case MK_ERR_UNSUPPORTED: return "combination not implemented";
    case MK_ERR_CONFIG: return "invalid config field";
    default: return "unknown status";
  }
}

}  // extern "C"
