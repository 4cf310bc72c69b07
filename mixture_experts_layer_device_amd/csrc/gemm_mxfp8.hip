// Expert-grouped MXFP8 GEMMs on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3, one E8M0 scale per 32 K).
//
// Same persistent walk, tile shape (256 x 256, 8 waves of 128 x 64) and
// double-buffered LDS pipeline as the bf16 GEMMs; a K step is 128 codes (one
// MFMA deep), i.e. 4 MX blocks whose 4 scale bytes per row travel as one
// dword next to the tile.
//
// Operand layout of the block-scaled MFMA (measured on gfx950): lane group
// g = l/16 of a 16-row fragment supplies k in [16g, 16g+16) in its bytes
// 0..15 and k in [64+16g, 64+16g+16) in bytes 16..31, and its scale applies to
// k in [32g, 32g+32).  So lane group g takes 16-byte granules g and g+4 of the
// 128-byte K step (MX block g = granules 2g and 2g+1 land in hardware block g)
// and passes scale byte g.
#include <type_traits>

#include "gemm_common.h"

namespace mk {
namespace {

constexpr int BM = G_BM, BN = G_BN, BKB = 128, NT = G_NT;   // BKB: K bytes (= codes) per step
constexpr int FM = G_FM, FN = G_FN;
constexpr int TILE_BYTES = BM * BKB;                      // 32 KiB codes per operand
constexpr int SCALE_BYTES = BM * 4;                       // one dword per row
constexpr int STAGE_BYTES = 2 * TILE_BYTES + 2 * SCALE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES > STAGE_LDS_BYTES ? 2 * STAGE_BYTES : STAGE_LDS_BYTES;

typedef GAcc Acc;

// Fragment i of A (wave rows) or j of B (wave columns) with its scale byte.
__device__ __forceinline__ void read_frag_mx(const char* codes, const uint32_t* sc, int row, i32x8_t& f, int& s) {
  const int g = (threadIdx.x & 63) >> 4;
  const u32x4_t lo = *(const u32x4_t*)(codes + tswz(row, g));
  const u32x4_t hi = *(const u32x4_t*)(codes + tswz(row, g + 4));
  f = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  s = (int)((sc[row] >> (8 * g)) & 0xFFu);
}
__device__ __forceinline__ void read_a_mx(const char* st, int i, i32x8_t& f, int& s) {
  const int wm = threadIdx.x >> 8;
  read_frag_mx(st, (const uint32_t*)(st + 2 * TILE_BYTES), wm * 128 + i * 16 + (threadIdx.x & 15), f, s);
}
// (NB: rows of the B tile, 256 or 128 for a half tile: a wave's NB / 4 columns)
template <int NB = BN>
__device__ __forceinline__ void read_b_mx(const char* st, int j, i32x8_t& f, int& s) {
  const int wn = (threadIdx.x >> 6) & 3;
  read_frag_mx(st + TILE_BYTES, (const uint32_t*)(st + 2 * TILE_BYTES) + BM,
               wn * (NB / 4) + j * 16 + (threadIdx.x & 15), f, s);
}

// C = A . B^T over K codes.  arow / ascale give A's code row and scale row
// (abase / asbase: bases that every such row lies within 4 GiB after); B
// comes in the tiled MXFP8 layout: bcodes / bscales point at this tile's
// K / 128 code blocks (each the LDS image of a stage's B slice) and scale
// blocks.  Codes go to LDS by the buffer-resource DMA as in the bf16 K loop
// (A: each lane fetches the granule the swizzle puts in its slot; B: 1 KiB
// contiguous copies); waves 0-3 also fetch A's scale dwords (64 rows each)
// and waves 4-7 B's.  A stage's B fragments are read at its start and its A
// fragments one ahead of the 4 MFMAs that use them.
// ATILED: A comes in the tiled layout as well (abase / asbase: its tile's
// first code and scale blocks; arow, ascale unused) and is fetched like B.
// NB = 128 (a half tile): bcodes / bscales point at rows 128h .. 128h+127 of
// each block (h * 16 KiB of codes and h * 512 bytes of scales in), each wave
// copies its 2 KiB of B codes, waves 4-5 the B scales, and only fragments
// j < 2 of acc are computed.
template <bool ATILED, int NB = BN, typename ARow, typename ASc>
__device__ __forceinline__ void mainloop_t(const void* abase, ARow arow, const void* asbase, ASc ascale,
                                           const uint8_t* bcodes, const uint8_t* bscales, int K, char* lds,
                                           Acc& acc) {
  constexpr int NFB = NB / 64;                  // B fragments per wave (and B copies per wave and stage)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const buf_rsrc_t ra = make_rsrc(abase), rb = make_rsrc(bcodes);
  const buf_rsrc_t rs = make_rsrc(wave_uniform(wave < 4 ? asbase : (const void*)bscales));
  const int wbase = wave * 4096;
  const uint32_t bo = wbase + lane * 16;
  uint32_t ao[4];
  if constexpr (!ATILED) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 32 + j * 8 + (lane >> 3);
      ao[j] = (uint32_t)(arow(r) - (const uint8_t*)abase) + (((lane & 7) ^ tkey(r)) & 7) * 16;
    }
  }
  uint32_t so, sstep;                                   // sstep: bytes between K steps in the scale source
  if constexpr (ATILED) {
    so = (uint32_t)((wave & 3) * 256 + lane * 4);
    sstep = MXT_SCALES;
  } else {
    so = wave < 4 ? (uint32_t)(ascale(wave * 64 + lane) - (const uint8_t*)asbase)
                  : (uint32_t)((wave - 4) * 256 + lane * 4);
    sstep = wave < 4 ? 4 : MXT_SCALES;
  }
  const int sbase = 2 * TILE_BYTES + wave * 256;
  const int bwbase = wave * NB * 16;            // this wave's share of the B tile (NB rows x 128 B)
  const uint32_t bbo = NB == BN ? bo : bwbase + lane * 16;
  auto issue = [&](int kt, char* st) {
    const uint32_t kb = (uint32_t)kt * BKB;
    const uint32_t b = bo + (uint32_t)kt * MXT_CODES;
    const uint32_t bb = bbo + (uint32_t)kt * MXT_CODES;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (ATILED)
        b2lds16(ra, b + j * 1024, st + wbase + j * 1024);
      else
        b2lds16(ra, ao[j] + kb, st + wbase + j * 1024);
      if (j < NFB) b2lds16(rb, bb + j * 1024, st + TILE_BYTES + bwbase + j * 1024);
    }
    if (NB == BN || wave < 4 + NFB) b2lds4(rs, so + (uint32_t)kt * sstep, st + sbase);
  };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0, lds);
  wait_all_mem();
  __syncthreads();
  const int KT = K / BKB;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const char* st = lds + cur * STAGE_BYTES;
    if (kt + 1 < KT) issue(kt + 1, lds + (cur ^ 1) * STAGE_BYTES);
    i32x8_t bq[NFB], aq[2];
    int sbq[NFB], saq[2];
#pragma unroll
    for (int j = 0; j < NFB; ++j) read_b_mx<NB>(st, j, bq[j], sbq[j]);
    read_a_mx(st, 0, aq[0], saq[0]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i + 1 < FM) read_a_mx(st, i + 1, aq[(i + 1) & 1], saq[(i + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NFB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[i & 1], bq[j], acc[i][j], 0, 0, 0,
                                                                     saq[i & 1], 0, sbq[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_all_mem();
    __syncthreads();
  }
}

template <int NB = BN, typename ARow, typename ASc>
__device__ __forceinline__ void mainloop(const void* abase, ARow arow, const void* asbase, ASc ascale,
                                         const uint8_t* bcodes, const uint8_t* bscales, int K, char* lds,
                                         Acc& acc) {
  mainloop_t<false, NB>(abase, arow, asbase, ascale, bcodes, bscales, K, lds, acc);
}

// a[p, i] = silu(g) * u (bf16) from MXFP8 ring rows and packed MXFP8 W_gu.
// SAVE: also store g and u (fp32, packed like W_gu) as the backward's context.
// DIRECT: rc / rsc hold the token rows' codes and scales instead (the full
// layer), and sorted position p reads token inv[p] / src_div.
template <bool SAVE, bool DIRECT = false>
__global__ __launch_bounds__(NT) void gemm1_mxfp8_kernel(ItemRange ir, const uint8_t* __restrict__ rc,
                                                         const uint8_t* __restrict__ rsc, int ring_rows,
                                                         const uint8_t* __restrict__ wc,
                                                         const uint8_t* __restrict__ wsc, int H, int I,
                                                         uint16_t* __restrict__ a_out, float* __restrict__ gu_save,
                                                         const int32_t* __restrict__ inv, int src_div) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = 2 * I / BN;
  const int nbh = H / 32;
  // one tile of NB packed columns (NB / 2 features; a wave's NB / 4 columns
  // are NB / 128 gate/up groups of 32)
  auto tile = [&](const TileInfo& ti, auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    auto rrow = [&](int r) {
      const int p = ti.pos0 + min(r, ti.rows - 1);
      return DIRECT ? (int64_t)(inv[p] / src_div) : (int64_t)(p % ring_rows);
    };
    auto arow = [&](int r) { return rc + rrow(r) * H; };
    auto asc = [&](int r) { return rsc + rrow(r) * nbh; };
    const int64_t t0 = mxt_index(ti.e, ti.n0 / BN, 0, 2 * I, H);
    const int h = (ti.n0 % BN) / 128;          // the half of a 256-row block (half tiles)
    Acc acc;
    mainloop<NB>(rc, arow, rsc, asc, wc + t0 * MXT_CODES + h * 128 * MXT_K, wsc + t0 * MXT_SCALES + h * 128 * 4, H,
                 lds, acc);
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 3;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int q = 0; q < NB / 128; ++q) {
          const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
          const int r = frag_row(i, v);
          stage_put(lds, r, wn * (NB / 8) + q * 16 + (lane & 15), g * sigmoidf_(g) * u);
          if (SAVE && r < ti.rows) {
            float* dst = gu_save + (int64_t)(ti.pos0 + r) * 2 * I + ti.n0 + wn * (NB / 4) + q * 32 + (lane & 15);
            dst[0] = g;
            dst[16] = u;
          }
        }
    stage_flush<NB / 2>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? a_out + (int64_t)(ti.pos0 + r) * I + ti.n0 / 2 : nullptr;
    });
  };
  // a last round at most half full runs as 256 x 128 half tiles
  for_each_tile_split(ir, ntn, [&](const TileInfo& ti, int half) {
    if (half < 0)
      tile(ti, std::integral_constant<int, BN>{});
    else
      tile(ti, std::integral_constant<int, BN / 2>{});
  });
}

// y[p] = D(a_q[p]) . D(W_d[e])^T with W_d codes [E, H, I] + scales [E, H, I/32];
// SHARE: out[inv[p]] = bf16(w * y) (fused weighted unpermute); else fp32 y.
template <bool SHARE>
__global__ __launch_bounds__(NT) void gemm2_mxfp8_kernel(ItemRange ir, const uint8_t* __restrict__ ac,
                                                         const uint8_t* __restrict__ asc_,
                                                         const uint8_t* __restrict__ wc,
                                                         const uint8_t* __restrict__ wsc, int H, int I,
                                                         float* __restrict__ y32, uint16_t* __restrict__ out,
                                                         const int32_t* __restrict__ inv,
                                                         const float* __restrict__ row_w) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = H / BN;
  const int nbi = I / 32;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto prow = [&](int r) { return (int64_t)(ti.pos0 + min(r, ti.rows - 1)); };
    auto arow = [&](int r) { return ac + prow(r) * I; };
    auto asc = [&](int r) { return asc_ + prow(r) * nbi; };
    const int64_t t0 = mxt_index(ti.e, ti.n0 / BN, 0, H, I);
    Acc acc;
    mainloop(arow(0), arow, asc(0), asc, wc + t0 * MXT_CODES, wsc + t0 * MXT_SCALES, I, lds, acc);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = frag_row(i, v);
        if (SHARE) {
          const float w = r < ti.rows ? row_w[inv[ti.pos0 + r]] : 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j) stage_put(lds, r, frag_col(j), w * acc[i][j][v]);
        } else if (r < ti.rows) {
          float* dst = y32 + (int64_t)(ti.pos0 + r) * H + ti.n0;
#pragma unroll
          for (int j = 0; j < FN; ++j) dst[frag_col(j)] = acc[i][j][v];
        }
      }
    if (SHARE)
      stage_flush<256>(lds, [&](int r) -> uint16_t* {
        return r < ti.rows ? out + (int64_t)inv[ti.pos0 + r] * H + ti.n0 : nullptr;
      });
  });
}

// ------------------------------------------------- backward: dA' + SwiGLU ----
// dA'[p, i] = D(dY_q[p]) . D(W_d^T[e][i]) with dY quantised along H (rows at
// their positions p) and W_d^T in the tiled MXFP8 layout [E, I, H]; the
// SwiGLU backward epilogue is the bf16 kernel's (bf16 dg/du and w*a).
// DIRECT: dyc / dys hold the token rows' codes (the full layer), and sorted
// position p reads token inv[p] / src_div.
template <bool DIRECT = false>
__global__ __launch_bounds__(NT) void bwd_dact_mxfp8_kernel(ItemRange ir, const uint8_t* __restrict__ dyc,
                                                            const uint8_t* __restrict__ dys,
                                                            const uint8_t* __restrict__ wc,
                                                            const uint8_t* __restrict__ wsc, int H, int I,
                                                            const float* __restrict__ gu,
                                                            const int32_t* __restrict__ inv,
                                                            const float* __restrict__ row_w,
                                                            uint16_t* __restrict__ dgdu, uint16_t* __restrict__ wa,
                                                            float* __restrict__ dw_part, int src_div) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = I / BN;
  const int nbh = H / 32;
  auto tile = [&](const TileInfo& ti, auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    auto prow = [&](int r) {
      const int p = ti.pos0 + min(r, ti.rows - 1);
      return DIRECT ? (int64_t)(inv[p] / src_div) : (int64_t)p;
    };
    auto arow = [&](int r) { return dyc + prow(r) * H; };
    auto asc = [&](int r) { return dys + prow(r) * nbh; };
    const int64_t t0 = mxt_index(ti.e, ti.n0 / BN, 0, I, H);
    const int h = (ti.n0 % BN) / 128;          // the half of a 256-row block (half tiles)
    Acc acc;
    // (token rows: offsets from the buffers' starts, every row within 4 GiB of them)
    mainloop<NB>(DIRECT ? (const uint8_t*)dyc : arow(0), arow, DIRECT ? (const uint8_t*)dys : asc(0), asc,
                 wc + t0 * MXT_CODES + h * 128 * MXT_K, wsc + t0 * MXT_SCALES + h * 128 * 4, H, lds, acc);
    dact_epilogue<NB>(ti, acc, lds, I, gu, inv, row_w, dgdu, wa, dw_part);
  };
  // a last round at most half full runs as 256 x 128 half tiles
  for_each_tile_split(ir, ntn, [&](const TileInfo& ti, int half) {
    if (half < 0)
      tile(ti, std::integral_constant<int, BN>{});
    else
      tile(ti, std::integral_constant<int, BN / 2>{});
  });
}

// ------------------------------------------------------ backward: dX ----
// dX_row[p] = D(dgdu_q[p]) . D([W_g; W_u]^T[e]) over the 2I features (the I
// gate features, then the I up features), dgdu quantised along them (so each
// MX block is 32 consecutive gate or up features) and [W_g; W_u]^T in the
// tiled MXFP8 layout [E, H, 2I].
template <bool ROWS16>
__global__ __launch_bounds__(NT) void bwd_dx_mxfp8_kernel(ItemRange ir, const uint8_t* __restrict__ gc_,
                                                          const uint8_t* __restrict__ gs_,
                                                          const uint8_t* __restrict__ wc,
                                                          const uint8_t* __restrict__ wsc, int H, int I,
                                                          const int32_t* __restrict__ inv,
                                                          uint16_t* __restrict__ dX, float* __restrict__ dx32) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = H / BN;
  const int nbk = 2 * I / 32;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto prow = [&](int r) { return (int64_t)(ti.pos0 + min(r, ti.rows - 1)); };
    auto arow = [&](int r) { return gc_ + prow(r) * 2 * I; };
    auto asc = [&](int r) { return gs_ + prow(r) * nbk; };
    const int64_t t0 = mxt_index(ti.e, ti.n0 / BN, 0, H, 2 * I);
    Acc acc;
    mainloop(arow(0), arow, asc(0), asc, wc + t0 * MXT_CODES, wsc + t0 * MXT_SCALES, 2 * I, lds, acc);
    dx_epilogue<ROWS16>(ti, acc, lds, H, inv, dX, dx32);
  });
}

// ------------------------------------------------- weight gradients ----
// C[m, n] = sum over expert e's padded rows k of D(A[m, k]) D(B[n, k]): both
// operands quantised along k (the rows) and stored in the tiled layout per
// expert (its blocks from (M/256) * kofs[e]/128 on, row tile by row tile), so
// the K loop is the forward's with A fetched like B.  Tiles go expert by
// expert in order of descending K, each (m, n) tile by one workgroup over the
// whole K: fixed order, no atomics.  An expert without rows writes zeros.
// MODE 0: dW_down [E, H, I] (M = H, N = I); MODE 1: A rows are the I gate
// features, then the I up features -> dW_gate / dW_up [E, I, H].
template <int MODE>
__global__ __launch_bounds__(NT) void wgrad_mxfp8_kernel(int E, int M, int N, int I, const int32_t* __restrict__ kofs,
                                                         const int32_t* __restrict__ order,
                                                         const uint8_t* __restrict__ ac,
                                                         const uint8_t* __restrict__ as_,
                                                         const uint8_t* __restrict__ bc,
                                                         const uint8_t* __restrict__ bs, float* __restrict__ out0,
                                                         float* __restrict__ out1) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int tm = M / BM, tn = N / BN;
  const int per_e = tm * tn;
  const int total = E * per_e;
  for (int t = xcd_logical_block(); t < total; t += gridDim.x) {
    const int q = t / per_e;
    const int e = order[q];
    int mt, nt;
    tile_coords(t - q * per_e, tm, tn, mt, nt);
    const int k0 = kofs[e], K = kofs[e + 1] - k0;
    Acc acc;
    if (K > 0) {
      const int64_t ab = (int64_t)tm * (k0 / BKB) + (int64_t)mt * (K / BKB);
      const int64_t bb = (int64_t)tn * (k0 / BKB) + (int64_t)nt * (K / BKB);
      auto none = [](int) { return (const uint8_t*)nullptr; };
      mainloop_t<true>(ac + ab * MXT_CODES, none, as_ + ab * MXT_SCALES, none, bc + bb * MXT_CODES,
                       bs + bb * MXT_SCALES, K, lds, acc);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int m0 = mt * BM, n0 = nt * BN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + frag_row(i, v);
        float* dst;
        if (MODE == 0) {
          dst = out0 + ((int64_t)e * M + m) * N;
        } else {
          dst = (m < I ? out0 + ((int64_t)e * I + m) * N : out1 + ((int64_t)e * I + m - I) * N);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[n0 + frag_col(j)] = acc[i][j][v];
      }
  }
}

}  // namespace

void launch_wgrad_down_mxfp8(int E, int H, int I, const int32_t* kofs, const int32_t* order, const uint8_t* ac,
                             const uint8_t* as, const uint8_t* bc, const uint8_t* bs, float* dW_down, int n_cu,
                             hipStream_t s) {
  hipLaunchKernelGGL(wgrad_mxfp8_kernel<0>, dim3(n_cu), dim3(NT), 0, s, E, H, I, I, kofs, order, ac, as, bc, bs,
                     dW_down, (float*)nullptr);
}

void launch_wgrad_gate_up_mxfp8(int E, int H, int I, const int32_t* kofs, const int32_t* order, const uint8_t* ac,
                                const uint8_t* as, const uint8_t* bc, const uint8_t* bs, float* dW_gate,
                                float* dW_up, int n_cu, hipStream_t s) {
  hipLaunchKernelGGL(wgrad_mxfp8_kernel<1>, dim3(n_cu), dim3(NT), 0, s, E, 2 * I, H, I, kofs, order, ac, as, bc, bs,
                     dW_gate, dW_up);
}

void launch_bwd_dact_mxfp8(const ItemRange& ir, const uint8_t* dy_codes, const uint8_t* dy_scales,
                           const uint8_t* wdT_codes, const uint8_t* wdT_scales, int H, int I, const float* gu,
                           const int32_t* inv, const float* row_w, uint16_t* dgdu, uint16_t* wa, float* dw_part,
                           int token_src_div, int n_cu, hipStream_t s) {
  if (token_src_div > 0)
    hipLaunchKernelGGL(bwd_dact_mxfp8_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, dy_codes, dy_scales, wdT_codes,
                       wdT_scales, H, I, gu, inv, row_w, dgdu, wa, dw_part, token_src_div);
  else
    hipLaunchKernelGGL(bwd_dact_mxfp8_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, dy_codes, dy_scales, wdT_codes,
                       wdT_scales, H, I, gu, inv, row_w, dgdu, wa, dw_part, 1);
}

void launch_bwd_dx_mxfp8(const ItemRange& ir, const uint8_t* dgdu_codes, const uint8_t* dgdu_scales,
                         const uint8_t* wguT_codes, const uint8_t* wguT_scales, int H, int I, const int32_t* inv,
                         uint16_t* dX, float* dx32, int n_cu, hipStream_t s) {
  if (dX)
    hipLaunchKernelGGL(bwd_dx_mxfp8_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, dgdu_codes, dgdu_scales,
                       wguT_codes, wguT_scales, H, I, inv, dX, dx32);
  else
    hipLaunchKernelGGL(bwd_dx_mxfp8_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, dgdu_codes, dgdu_scales,
                       wguT_codes, wguT_scales, H, I, inv, dX, dx32);
}

void launch_gemm1_mxfp8(const ItemRange& ir, const uint8_t* ring_codes, const uint8_t* ring_scales,
                        int32_t ring_rows, const uint8_t* wgu_codes, const uint8_t* wgu_scales, int H, int I,
                        uint16_t* a_out, float* gu_save, const int32_t* inv, int src_div, int n_cu, hipStream_t s) {
  if (inv && gu_save)
    hipLaunchKernelGGL((gemm1_mxfp8_kernel<true, true>), dim3(n_cu), dim3(NT), 0, s, ir, ring_codes, ring_scales,
                       ring_rows, wgu_codes, wgu_scales, H, I, a_out, gu_save, inv, src_div);
  else if (inv)
    hipLaunchKernelGGL((gemm1_mxfp8_kernel<false, true>), dim3(n_cu), dim3(NT), 0, s, ir, ring_codes, ring_scales,
                       ring_rows, wgu_codes, wgu_scales, H, I, a_out, gu_save, inv, src_div);
  else if (gu_save)
    hipLaunchKernelGGL(gemm1_mxfp8_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, ring_codes, ring_scales, ring_rows,
                       wgu_codes, wgu_scales, H, I, a_out, gu_save, inv, src_div);
  else
    hipLaunchKernelGGL(gemm1_mxfp8_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, ring_codes, ring_scales, ring_rows,
                       wgu_codes, wgu_scales, H, I, a_out, gu_save, inv, src_div);
}

void launch_gemm2_mxfp8(const ItemRange& ir, const uint8_t* a_codes, const uint8_t* a_scales,
                        const uint8_t* wd_codes, const uint8_t* wd_scales, int H, int I, float* y32,
                        uint16_t* out, const int32_t* inv, const float* row_w, int n_cu, hipStream_t s) {
  if (out)
    hipLaunchKernelGGL(gemm2_mxfp8_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, a_codes, a_scales, wd_codes,
                       wd_scales, H, I, y32, out, inv, row_w);
  else
    hipLaunchKernelGGL(gemm2_mxfp8_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, a_codes, a_scales, wd_codes,
                       wd_scales, H, I, y32, out, inv, row_w);
}

}  // namespace mk
