// Pieces shared by the expert-grouped GEMM kernels: the persistent walk over
// the device work table, the XCD-aware block numbering, and the LDS-staged
// epilogue that turns the MFMA fragment layout into coalesced row stores.
#pragma once
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

constexpr int G_BM = 256, G_BN = 256, G_NT = 512;
constexpr int G_FM = 8, G_FN = 4;             // 16x16 fragments per wave (128 x 64)
constexpr int STAGE_ROW_BYTES = 528;          // 512 + 16 pad: conflict-light fragment writes
constexpr int STAGE_LDS_BYTES = G_BM * STAGE_ROW_BYTES;

typedef f32x4_t GAcc[G_FM][G_FN];

// Blocks are dealt to the 8 XCDs round-robin; renumber them so that
// consecutive logical ids share an XCD (and its L2).
__device__ __forceinline__ int xcd_logical_block() {
  const int b = blockIdx.x, G = gridDim.x;
  return (b & 7) * (G >> 3) + (b >> 3);
}

// Tile t -> (item, n-tile), in groups of 4 items so that tiles running at the
// same time on one XCD share A rows (same item) and B columns (same n).
__device__ __forceinline__ void tile_coords(int t, int n_items, int ntn, int& item, int& nt) {
  constexpr int GM = 4;
  const int group = GM * ntn;
  const int g = t / group;
  const int first = g * GM;
  const int gm = min(GM, n_items - first);
  const int local = t - g * group;
  item = first + local % gm;
  nt = local / gm;
}

struct TileInfo {
  int pos0, rows, e, n0;
};

// Persistent walk over the tiles of the items of minibatches [mb_lo, mb_hi).
template <typename Body>
__device__ __forceinline__ void for_each_tile(const ItemRange& ir, int ntn, Body body) {
  const int i_lo = min(ir.mb_items[ir.mb_lo], ir.item_cap);
  const int i_hi = min(ir.mb_items[ir.mb_hi], ir.item_cap);
  const int n_items = i_hi - i_lo;
  const int total = n_items * ntn;
  for (int t = xcd_logical_block(); t < total; t += gridDim.x) {
    int it, nt;
    tile_coords(t, n_items, ntn, it, nt);
    const int* item = ir.items + 4 * (i_lo + it);
    TileInfo ti{item[0], item[1], item[2], nt * G_BN};
    body(ti);
  }
}

// As for_each_tile, but a last round that would leave at least half of the
// workgroups idle is spread over twice as many workgroups: each of its tiles
// is cut into two 128-column halves (consecutive logical ids, so both halves
// run on one XCD and share the A rows in its L2).  body(ti, half): half = -1
// for a whole 256-column tile, else 0 / 1 with ti.n0 already at the half.
template <typename Body>
__device__ __forceinline__ void for_each_tile_split(const ItemRange& ir, int ntn, Body body) {
  const int i_lo = min(ir.mb_items[ir.mb_lo], ir.item_cap);
  const int i_hi = min(ir.mb_items[ir.mb_hi], ir.item_cap);
  const int n_items = i_hi - i_lo;
  const int total = n_items * ntn;
  const int G = gridDim.x;
  const int rem = total % G;
  const bool split = rem > 0 && 2 * rem <= G;
  const int t_end = split ? total - rem : total;
  const int b = xcd_logical_block();
  auto tile = [&](int t, int half) {
    int it, nt;
    tile_coords(t, n_items, ntn, it, nt);
    const int* item = ir.items + 4 * (i_lo + it);
    TileInfo ti{item[0], item[1], item[2], nt * G_BN + (half > 0 ? G_BN / 2 : 0)};
    body(ti, half);
  };
  for (int t = b; t < t_end; t += G) tile(t, -1);
  if (split && b < 2 * rem) tile(t_end + b / 2, b & 1);
}

__device__ __forceinline__ int frag_row(int i, int v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 2) * 128 + i * 16 + 4 * (lane >> 4) + v;
}
__device__ __forceinline__ int frag_col(int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 3) * 64 + j * 16 + (lane & 15);
}

// Stage a tile of bf16 values through LDS and store each row's COLS values
// (COLS * 2 bytes, contiguous) with 16-byte stores.
//   put(stage)            : the caller writes its fragments with stage_put()
//   row_dst(r) -> uint16* : destination of tile row r, or nullptr to skip it
// Must be called by the whole workgroup; LDS is free on entry and on exit.
__device__ __forceinline__ void stage_put(char* lds, int row, int col, float v) {
  *(uint16_t*)(lds + row * STAGE_ROW_BYTES + col * 2) = (uint16_t)f32_to_bf16(v);
}

template <int COLS, typename RowDst>
__device__ __forceinline__ void stage_flush(char* lds, RowDst row_dst) {
  constexpr int CPR = COLS / 8;                 // 16-byte chunks per row
  __syncthreads();
  for (int id = threadIdx.x; id < G_BM * CPR; id += G_NT) {
    const int r = id / CPR, c = id - r * CPR;
    uint16_t* dst = row_dst(r);
    if (dst) *(u32x4_t*)(dst + c * 8) = *(const u32x4_t*)(lds + r * STAGE_ROW_BYTES + c * 16);
  }
  __syncthreads();
}

// The same, with every 16-byte store written through to memory
// (device-coherent: a buffer store with the device-scope bit), for results
// that another XCD reads within the same launch.  row_off(r) gives the byte
// offset of tile row r from base (< 4 GiB), or -1 to skip the row.
template <int COLS, typename RowOff>
__device__ __forceinline__ void stage_flush_wt(char* lds, const void* base, RowOff row_off) {
  constexpr int CPR = COLS / 8;                 // 16-byte chunks per row
  const buf_rsrc_t rs = make_rsrc(base);
  __syncthreads();
  for (int id = threadIdx.x; id < G_BM * CPR; id += G_NT) {
    const int r = id / CPR, c = id - r * CPR;
    const int64_t off = row_off(r);
    if (off >= 0)
      __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4_t*)(lds + r * STAGE_ROW_BYTES + c * 16), rs,
                                             (uint32_t)off + c * 16, 0, MK_CPOL_DEVICE);
  }
  __syncthreads();
}

// s_waitcnt: vmcnt(n) (n < 64) and lgkmcnt(0); expcnt not waited for.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0_t() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// The workgroup barrier with no memory fence of its own, for callers that
// have already waited for exactly what must be complete (__syncthreads()
// would add a fence that waits for every copy in flight).  The clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_no_fence_t() { asm volatile("s_barrier" ::: "memory"); }

// ---- backward epilogues shared by the bf16 and MXFP8 kernels --------------

// dA' tile -> SwiGLU backward, from the forward's fp32 g, u (gu, packed like
// W_gu): a = silu(g) u; dw partial = sum of dA' a over 32 columns (slice
// n / 32 of I / 32, a wave's fragments 2s and 2s+1, added up later in slice
// order, so the partials do not depend on how tiles are cut); dA = w dA';
// dg = dA u s (1 + g (1 - s)), du = dA silu(g) (bf16, row p of dgdu holding
// the I gate features then the I up features, so the MX blocks of the dX
// GEMM's contraction are 32 consecutive dg or du values); and w*a (bf16, the
// down-projection weight gradient's operand).
// NB: the tile's columns (256, or 128 for a half tile: a wave's NB / 4
// columns are its fragments j < NB / 64).
// g and u of the tile (256 rows x 2 NB packed columns, 8 NB bytes per row)
// come through LDS in 8 chunks of 32 rows -- chunk c holds the rows of
// fragment c of both row halves -- with the LDS DMA, double-buffered: chunk
// c+1's copies are in flight while chunk c is used.  The row stride of 516
// floats puts the 4 row groups a fragment read touches on different banks.
// LDS must be free on entry (it is after the mainloop) and is free on exit.
template <int NB = G_BN>
__device__ __forceinline__ void dact_epilogue(const TileInfo& ti, GAcc& acc, char* lds, int I,
                                              const float* __restrict__ gu, const int32_t* __restrict__ inv,
                                              const float* __restrict__ row_w, uint16_t* __restrict__ dgdu,
                                              uint16_t* __restrict__ wa, float* __restrict__ dw_part) {
  constexpr int FM = G_FM, FN = NB / 64;        // fragments per wave (columns NB / 4)
  constexpr int HALVES = NB / 128;              // 1 KiB copies per g/u row
  constexpr int GS = 516;                       // LDS row stride (floats)
  constexpr int CROWS = 32;                     // rows per chunk
  constexpr int CBYTES = CROWS * GS * 4;        // one chunk buffer
  constexpr int PER = CROWS * HALVES / 8;       // copies per wave and chunk
  static_assert(2 * CBYTES + 1024 <= 135168, "two chunk buffers and the row weights in the LDS");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int slices = I / 32, slice0 = (ti.n0 + wn * (NB / 4)) / 32;
  // the tile's first row of packed g, u (2 NB columns from 2 n0); every row
  // the tile reads lies within 256 rows of it, far inside a buffer offset
  const buf_rsrc_t rg = make_rsrc(wave_uniform(gu + (int64_t)ti.pos0 * 2 * I + (int64_t)2 * ti.n0));
  // chunk c into buffer c mod 2: LDS row lr = 16 wm' + t is tile row
  // 128 wm' + 16 c + t.  Rows past the item's end copy its last row (never
  // read), so every wave issues the same PER copies for every chunk and the
  // waits below can count them.
  auto issue = [&](int c) {
    char* buf = lds + (c & 1) * CBYTES;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = wave * PER + k;
      const int lr = idx / HALVES, half = idx % HALVES;
      const int r = min((lr >> 4) * 128 + c * 16 + (lr & 15), ti.rows - 1);
      b2lds16(rg, (uint32_t)(((int64_t)r * 2 * I + half * 256 + lane * 4) * 4), buf + (lr * GS + half * 256) * 4);
    }
  };
  // the tile's row weights w = row_w[inv[p]] into LDS first: read from
  // there, the chunk loop waits on no global load (a wait for one would
  // also wait for the next chunk's copies, issued before it)
  float* const wl = (float*)(lds + 2 * CBYTES);
  if (threadIdx.x < 256) wl[threadIdx.x] = (int)threadIdx.x < ti.rows ? row_w[inv[ti.pos0 + threadIdx.x]] : 0.f;
  issue(0);
#pragma unroll
  for (int c = 0; c < FM; ++c) {
    if (c + 1 < FM) {
      issue(c + 1);
      wait_vm_lgkm0_t<PER>();                   // chunk c landed (c+1 still in flight)
    } else {
      wait_vm_lgkm0_t<0>();
    }
    barrier_no_fence_t();
    const float* sg = (const float*)(lds + (c & 1) * CBYTES);
    const int i = c;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = frag_row(i, v);
      const int lr = wm * 16 + 4 * (lane >> 4) + v;
      const bool valid = r < ti.rows;
      const int64_t p = ti.pos0 + (valid ? r : 0);
      const float w = wl[r];
#pragma unroll
      for (int sl = 0; sl < FN / 2; ++sl) {
        float dws = 0.f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * sl + jj;
          const int f = wn * (NB / 4) + j * 16 + (lane & 15);   // feature within the tile
          const int lc = 32 * (f >> 4) + (f & 15);                // its gate column; up at +16
          float g = 0.f, u = 0.f;
          if (valid) {
            g = sg[lr * GS + lc];
            u = sg[lr * GS + lc + 16];
          }
          const float s = sigmoidf_(g);
          const float sla = g * s;
          const float aa = sla * u;
          const float dap = acc[i][j][v];
          dws += dap * aa;
          const float da = w * dap;
          if (valid) {
            uint16_t* dst = dgdu + p * 2 * I + ti.n0 + f;
            dst[0] = (uint16_t)f32_to_bf16(da * u * s * (1.f + g * (1.f - s)));
            dst[I] = (uint16_t)f32_to_bf16(da * sla);
            wa[p * I + ti.n0 + f] = (uint16_t)f32_to_bf16(w * aa);
          }
        }
        // fixed butterfly over the 16 lanes that share this row
        dws += __shfl_xor(dws, 1);
        dws += __shfl_xor(dws, 2);
        dws += __shfl_xor(dws, 4);
        dws += __shfl_xor(dws, 8);
        if (valid && (lane & 15) == 0) dw_part[p * slices + slice0 + sl] = dws;
      }
    }
    // every wave has read this buffer before chunk c+2 is copied into it
    wait_vm_lgkm0_t<63>();                      // (LDS reads only: lgkmcnt(0))
    barrier_no_fence_t();
  }
}

// dX tile -> ROWS16: bf16 rows straight to arrival order, dX[inv[p]]; else
// fp32 rows at their position p ([p, H]) for the full layer's k-sum.
template <bool ROWS16>
__device__ __forceinline__ void dx_epilogue(const TileInfo& ti, GAcc& acc, char* lds, int H,
                                            const int32_t* __restrict__ inv, uint16_t* __restrict__ dX,
                                            float* __restrict__ dx32) {
  constexpr int FM = G_FM, FN = G_FN;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = frag_row(i, v);
      if (ROWS16) {
#pragma unroll
        for (int j = 0; j < FN; ++j) stage_put(lds, r, frag_col(j), acc[i][j][v]);
      } else if (r < ti.rows) {
        float* dst = dx32 + (int64_t)(ti.pos0 + r) * H + ti.n0;
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[frag_col(j)] = acc[i][j][v];
      }
    }
  if (ROWS16)
    stage_flush<256>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? dX + (int64_t)inv[ti.pos0 + r] * H + ti.n0 : nullptr;
    });
}

}  // namespace mk
