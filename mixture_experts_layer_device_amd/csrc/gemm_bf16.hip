// Expert-grouped bf16 GEMMs on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Every GEMM here is a persistent grid (one 256-thread workgroup per compute
// unit) that walks the device-side work table built by the schedule: an item
// is (first sorted row, rows, expert, minibatch) and each item is cut into
// 256-column tiles.  Tile counts are read on the device, so the host never
// learns per-expert counts.  Each 256x256 output tile is computed by one
// workgroup with a fixed K order, so results do not depend on which
// workgroup takes which tile (bitwise repeatable).
//
// Mainloop: K in steps of 64; A and B tiles (256 x 64 bf16 each) go global ->
// LDS with the asynchronous LDS-DMA loads (swizzled 16-byte granules),
// double-buffered so the next step's loads overlap this step's MFMAs.  4 waves
// as 2 (M) x 2 (N); a wave owns 128 x 128 outputs = 8 x 8 MFMA 16x16
// fragments, whose 256 fp32 accumulators per lane live in the accumulation
// registers (one wave per SIMD, 512 registers).  Epilogues stage their bf16
// results through LDS and store whole rows with 16-byte stores.
//
// Fragment layouts (measured on gfx950): A/B lane l holds row/col l%16 and
// k = 8*(l/16) .. +7; the 16x16 fp32 result in lane l is column l%16, rows
// 4*(l/16) .. +3.
#include "gemm_common.h"

namespace mk {
namespace {

constexpr int BM = G_BM, BN = G_BN, BK = 64, NT = G_NT;
constexpr int FM = G_FM, FN = G_FN;
constexpr int TILE_BYTES = BM * BK * 2;        // 32 KiB per operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES > STAGE_LDS_BYTES ? 2 * STAGE_BYTES : STAGE_LDS_BYTES;

typedef GAcc Acc;

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// One k half (32 of the stage's 64 k) of a wave's fragments: 8 A + 8 B
// 16x16x32 operands, read from a stage written with swizzle Key(row).
struct HalfFrags {
  bf16x8_t a[FM], b[FN];
};

template <int (*Key)(int)>
__device__ __forceinline__ void read_half(const char* st, int ks, HalfFrags& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = ks * 4 + (lane >> 4);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * 128 + i * 16 + (lane & 15);
    f.a[i] = *(const bf16x8_t*)(st + r * 128 + (((g ^ Key(r)) & 7) << 4));
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int r = wn * 128 + j * 16 + (lane & 15);
    f.b[j] = *(const bf16x8_t*)(st + TILE_BYTES + r * 128 + (((g ^ Key(r)) & 7) << 4));
  }
}

// 64 MFMAs on one k half, free to be scheduled around (the caller places
// them with scheduling group barriers).
__device__ __forceinline__ void mfma_half_free(const HalfFrags& f, Acc& acc) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// The same as one block: the scheduling barriers keep LDS reads, waits and
// workgroup barriers from being moved into the MFMA run.
__device__ __forceinline__ void mfma_half(const HalfFrags& f, Acc& acc) {
  __builtin_amdgcn_sched_barrier(0);
  mfma_half_free(f, acc);
  __builtin_amdgcn_sched_barrier(0);
  pin_acc(acc);
}

// ------------------------------------------------------- NT mainloop ----
// C[256 x 256] = A[256 x K] * B[256 x K]^T.  A is row-major (K-contiguous
// rows); B comes in the tiled layout, btile pointing at this tile's K / 64
// blocks, each the LDS image of one stage's B slice.
//
// K advances in steps of 64 through two LDS stages (A and B slices of 256 x
// 64, 128-byte rows, 32 KiB each), filled global -> LDS by the buffer DMA:
// wave w loads rows 64w .. 64w+63 of both operands, 8 rows (1 KiB) per
// instruction.  For A each lane fetches the granule that the swizzle puts
// in its slot (slot s of row r holds granule s ^ tkey(r)); B's block already
// has that order, so its copies are 1 KiB contiguous (whole DRAM bursts
// instead of 128-byte pieces of rows 4 KiB or more apart, which stream from
// HBM markedly slower).  A step is two halves of 64 MFMAs with one workgroup
// barrier between them:
//   half 1: MFMAs on k 0..31 of stage kt, while this wave reads k 32..63;
//   barrier (stage kt+1 landed, stage kt read by every wave);
//   half 2: MFMAs on k 32..63, while the DMA of stage kt+2 refills stage kt's
//           buffer and this wave reads k 0..31 of stage kt+1.
// The LDS reads and DMA issues are interleaved one by one between the MFMAs
// (scheduling group barriers), so the matrix core is fed while the LDS and
// the memory pipeline work; issuing them as a block in front of the MFMAs
// stalls all four waves on the LDS after every barrier.  Steps have no
// branches: past the last stage the DMA re-reads the last stage into the idle
// buffer and the reads go unused, which keeps the schedule in one block.
template <typename AOff>
__device__ __forceinline__ void mainloop_nt(const char* abase, AOff aoff, uint32_t a_bytes, const uint16_t* btile,
                                            int K, char* lds, Acc& acc) {
  constexpr int NR = FM + FN;           // LDS reads per k half
  constexpr int NM = FM * FN;           // MFMAs per k half
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KT = K / BK;
  uint32_t ao[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + (lane >> 3);
    ao[j] = aoff(r) + ((uint32_t)(((lane & 7) ^ tkey(r)) & 7) << 4);
  }
  const uint32_t bo = (uint32_t)(wave * 8192 + lane * 16);
  const buf_rsrc_t ra = make_rsrc(abase, a_bytes), rb = make_rsrc(btile, (uint32_t)KT * STAGE_BYTES / 2);
  auto issue = [&](int s, int buf) {
    char* st = lds + buf * STAGE_BYTES + wave * 8192;
    const uint32_t kb = (uint32_t)s * BK * 2;
    const uint32_t bb = (uint32_t)s * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      b2lds16(ra, ao[j], kb, st + j * 1024);
      b2lds16(rb, bo, bb + (uint32_t)j * 1024, st + TILE_BYTES + j * 1024);
    }
  };
  zero_acc(acc);
  pin_acc(acc);
  issue(0, 0);
  wait_all_mem();
  __syncthreads();
  issue(KT > 1 ? 1 : 0, 1);
  HalfFrags h0, h1;
  read_half<tkey>(lds, 0, h0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    read_half<tkey>(lds + buf * STAGE_BYTES, 1, h1);
    mfma_half_free(h0, acc);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);      // MFMAs
    }
    wait_all_mem();
    __syncthreads();
    issue(kt + 2 < KT ? kt + 2 : KT - 1, buf);
    read_half<tkey>(lds + (buf ^ 1) * STAGE_BYTES, 0, h0);
    mfma_half_free(h1, acc);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);            // 1 memory load (DMA)
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR - NM / NR / 2, 0);
    }
    pin_acc(acc);
  }
  // all DMA landed and every wave done with the LDS before an epilogue reuses it
  wait_all_mem();
  __syncthreads();
}

// ---------------------------------------------------------------- GEMM1 ----
// a[p, i] = silu(g) * u with [g | u] = ring[p] . W_gu[e]^T; W_gu is packed so
// that each 32-column group holds 16 gate columns then the 16 up columns of
// the same i.  a is a bf16 GEMM operand (stored [p, I]); optionally g and u
// are saved in fp32 (packed order, [p, 2I]) for the backward.
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm1_bf16_kernel(ItemRange ir, const uint16_t* __restrict__ ring,
                                                        int ring_rows, const uint16_t* __restrict__ wgu, int H,
                                                        int I, uint16_t* __restrict__ a_out,
                                                        float* __restrict__ gu_save) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = 2 * I / BN;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto aoff = [&](int r) {
      const int p = ti.pos0 + min(r, ti.rows - 1);
      return (uint32_t)(p % ring_rows) * (uint32_t)(H * 2);
    };
    Acc acc;
    mainloop_nt((const char*)ring, aoff, (uint32_t)ring_rows * (uint32_t)(H * 2),
                wgu + btile_block(ti.e, ti.n0 / BN, 0, 2 * I, H), H, lds, acc);
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = frag_row(i, v);
#pragma unroll
        for (int q = 0; q < FN / 2; ++q) {
          const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
          stage_put(lds, r, wn * 64 + q * 16 + (lane & 15), g * sigmoidf_(g) * u);
          if (gu_save && r < ti.rows) {
            float* dst = gu_save + (int64_t)(ti.pos0 + r) * 2 * I + ti.n0 + wn * 128 + q * 32 + (lane & 15);
            dst[0] = g;
            dst[16] = u;
          }
        }
      }
    });
    stage_flush<128>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? a_out + (int64_t)(ti.pos0 + r) * I + ti.n0 / 2 : nullptr;
    });
  });
}

// ---------------------------------------------------------------- GEMM2 ----
// y[p] = a[p] . W_d[e]^T  (W_d as the tiled B of [E, H, I]).
// SHARE: the router-weighted unpermute is fused: out[inv[p]] = bf16(w * y),
//        one rounding, rows stored straight to arrival order.
// else : y is kept in fp32 ([p, H]) for the full-layer combine.
template <bool SHARE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm2_bf16_kernel(ItemRange ir, const uint16_t* __restrict__ a,
                                                        const uint16_t* __restrict__ wd, int H, int I,
                                                        float* __restrict__ y32, uint16_t* __restrict__ out,
                                                        const int32_t* __restrict__ inv,
                                                        const float* __restrict__ row_w) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = H / BN;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto aoff = [&](int r) { return (uint32_t)min(r, ti.rows - 1) * (uint32_t)(I * 2); };
    Acc acc;
    mainloop_nt((const char*)(a + (int64_t)ti.pos0 * I), aoff, (uint32_t)ti.rows * (uint32_t)(I * 2),
                wd + btile_block(ti.e, ti.n0 / BN, 0, H, I), I, lds, acc);
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
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
    });
    if (SHARE)
      stage_flush<256>(lds, [&](int r) -> uint16_t* {
        return r < ti.rows ? out + (int64_t)inv[ti.pos0 + r] * H + ti.n0 : nullptr;
      });
  });
}

// ------------------------------------------------- backward: dA' + SwiGLU ----
// dA'[p, i] = dYe[p] . W_d[e][:, i]  (B = W_d^T, tiled [E, I, H]).  Epilogue,
// from the forward's fp32 g, u: a = silu(g) u; dw partial = sum_i dA' a over
// this wave's 128 columns; dA = w dA'; dg = dA u s (1 + g (1 - s)); du = dA
// silu(g) (bf16 GEMM operands, packed like W_gu); w*a (bf16 operand of the
// down-projection weight gradient).
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dact_kernel(ItemRange ir, const uint16_t* __restrict__ dye,
                                                      const uint16_t* __restrict__ wdT, int H, int I,
                                                      const float* __restrict__ gu,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ row_w,
                                                      uint16_t* __restrict__ dgdu, uint16_t* __restrict__ wa,
                                                      float* __restrict__ dw_part) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = I / BN;
  const int slices = I / 128;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto aoff = [&](int r) { return (uint32_t)min(r, ti.rows - 1) * (uint32_t)(H * 2); };
    Acc acc;
    mainloop_nt((const char*)(dye + (int64_t)ti.pos0 * H), aoff, (uint32_t)ti.rows * (uint32_t)(H * 2),
                wdT + btile_block(ti.e, ti.n0 / BN, 0, I, H), H, lds, acc);
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    const int slice = (ti.n0 + wn * 128) / 128;
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = frag_row(i, v);
        const bool valid = r < ti.rows;
        const int64_t p = ti.pos0 + (valid ? r : 0);
        const float w = valid ? row_w[inv[p]] : 0.f;
        float dws = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int ii = ti.n0 + frag_col(j);
          const int gc = 32 * (ii >> 4) + (ii & 15);
          // row p is a real row of this tile even when r is not (then w = 0)
          const float g = gu[p * 2 * I + gc];
          const float u = gu[p * 2 * I + gc + 16];
          const float s = sigmoidf_(g);
          const float sl = g * s;
          const float aa = sl * u;
          const float dap = acc[i][j][v];
          dws += dap * aa;
          const float da = w * dap;
          if (valid) {
            dgdu[p * 2 * I + gc] = (uint16_t)f32_to_bf16(da * u * s * (1.f + g * (1.f - s)));
            dgdu[p * 2 * I + gc + 16] = (uint16_t)f32_to_bf16(da * sl);
          }
          stage_put(lds, r, frag_col(j), w * aa);
        }
        // fixed butterfly over the 16 lanes that share this row
        dws += __shfl_xor(dws, 1);
        dws += __shfl_xor(dws, 2);
        dws += __shfl_xor(dws, 4);
        dws += __shfl_xor(dws, 8);
        if (valid && (lane & 15) == 0) dw_part[p * slices + slice] = dws;
      }
    });
    stage_flush<256>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? wa + (int64_t)(ti.pos0 + r) * I + ti.n0 : nullptr;
    });
  });
}

// ------------------------------------------------------ backward: dX ----
// dX[inv[p]] = dgdu[p] . W_gu[e]  (B = packed W_gu^T, tiled [E, H, 2I]); rows
// are stored straight back to arrival order.
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dx_kernel(ItemRange ir, const uint16_t* __restrict__ dgdu,
                                                    const uint16_t* __restrict__ wguT, int H, int I,
                                                    const int32_t* __restrict__ inv, uint16_t* __restrict__ dX) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = H / BN;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto aoff = [&](int r) { return (uint32_t)min(r, ti.rows - 1) * (uint32_t)(I * 4); };
    Acc acc;
    mainloop_nt((const char*)(dgdu + (int64_t)ti.pos0 * 2 * I), aoff, (uint32_t)ti.rows * (uint32_t)(I * 4),
                wguT + btile_block(ti.e, ti.n0 / BN, 0, H, 2 * I), 2 * I, lds, acc);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < FN; ++j) stage_put(lds, frag_row(i, v), frag_col(j), acc[i][j][v]);
    stage_flush<256>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? dX + (int64_t)inv[ti.pos0 + r] * H + ti.n0 : nullptr;
    });
  });
}

// ----------------------------------------------------------- weight grads ----
// C[m, n] = sum over the rows p of expert e of A[p, m] * B[p, n]: both operands
// are row-major over p, so each thread fetches an 8 (rows) x 8 (columns) bf16
// block of each, transposes it in registers and stores 8 K-contiguous
// granules.  The LDS swizzle here uses a key that also keeps these transposed
// stores (rows 8m + c over m) from piling onto a few banks.  The K loop walks
// expert e's row segments minibatch by minibatch in reverse (nb-1 .. 0), rows
// ascending inside each: a fixed order, no atomics.
__device__ __forceinline__ int wkey(int row) { return ((row >> 1) ^ (row >> 3) ^ (row >> 5)) & 7; }

struct SegIter {
  int b, k0, start, len;
};

__device__ __forceinline__ bool seg_next(SegIter& it, const WgradArgs& w, int e) {
  it.k0 += BK;
  while (it.k0 >= it.len) {
    if (--it.b < 0) return false;
    it.start = it.b * w.MB + w.mb_offsets[it.b * (w.E + 1) + e];
    it.len = w.mb_counts[it.b * w.E + e];
    it.k0 = 0;
  }
  return true;
}

template <int MODE>
struct WgradOperands {
  // MODE 0: A = dYe [p, H], B = w*a [p, I]          -> dW_down [E, H, I]
  // MODE 1: A = dgdu [p, 2I] (packed), B = x rows   -> dW_gate / dW_up [E, I, H]
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  const uint16_t* ring;
  int ring_rows, first_resident;
  const uint16_t* x_src;
  int64_t ldx;
};

// thread t loads rows k0 + 8*(t/32) .. +7, columns 8*(t%32) .. +7 of A and of B
template <int MODE>
__device__ __forceinline__ void wgrad_load(const WgradOperands<MODE>& op, const WgradArgs& w, const SegIter& it,
                                           int m0, int n0, u32x4_t (&va)[8], u32x4_t (&vb)[8]) {
  const int tid = threadIdx.x;
  const int mc = tid & 31, kc = tid >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int kk = it.k0 + kc * 8 + c;
    const bool in = kk < it.len;
    // rows past the segment read its last row and are zeroed (no branch)
    const int64_t p = it.start + (in ? kk : it.len - 1);
    const u32x4_t a = *(const u32x4_t*)(op.A + p * op.lda + m0 + mc * 8);
    const uint16_t* pb;
    if (MODE == 0)
      pb = op.B + p * op.ldb;
    else if (it.b >= op.first_resident)
      pb = op.ring + (int64_t)(p % op.ring_rows) * op.ldx;
    else
      pb = op.x_src + (int64_t)(w.inv[p] / w.src_div) * op.ldx;
    const u32x4_t b = *(const u32x4_t*)(pb + n0 + mc * 8);
    const u32x4_t z{0u, 0u, 0u, 0u};
    va[c] = in ? a : z;
    vb[c] = in ? b : z;
  }
}

__device__ __forceinline__ void wgrad_store_one(char* base, const u32x4_t (&v)[8]) {
  const int tid = threadIdx.x;
  const int mc = tid & 31, kc = tid >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4_t lo, hi;   // columns 2j and 2j+1, 8 k values each
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x0 = v[2 * d][j], x1 = v[2 * d + 1][j];
      lo[d] = (x0 & 0xFFFFu) | (x1 << 16);
      hi[d] = (x0 >> 16) | (x1 & 0xFFFF0000u);
    }
    const int r0 = mc * 8 + 2 * j, r1 = r0 + 1;
    *(u32x4_t*)(base + r0 * 128 + (((kc ^ wkey(r0)) & 7) << 4)) = lo;
    *(u32x4_t*)(base + r1 * 128 + (((kc ^ wkey(r1)) & 7) << 4)) = hi;
  }
}

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void wgrad_kernel(WgradArgs w, WgradOperands<MODE> op, int M, int N, int I,
                                                   float* __restrict__ out0, float* __restrict__ out1) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int tm = M / BM, tn = N / BN;
  const int per_e = tm * tn;
  const int total = w.E * per_e;
  for (int t = xcd_logical_block(); t < total; t += gridDim.x) {
    const int e = t / per_e;
    int mt, nt;
    tile_coords(t - e * per_e, tm, tn, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    Acc acc;
    zero_acc(acc);
    // Same two-half pipeline as the NT mainloop; the next stage's operands
    // travel through registers (loaded one step ahead) and are stored,
    // transposed, into the free LDS buffer halfway through a step.
    SegIter cur{w.nb, 0, 0, 0};
    if (seg_next(cur, w, e)) {
      u32x4_t va[8], vb[8];
      wgrad_load<MODE>(op, w, cur, m0, n0, va, vb);
      wgrad_store_one(lds, va);
      wgrad_store_one(lds + TILE_BYTES, vb);
      SegIter ld = cur;
      bool more = seg_next(ld, w, e);
      if (more) wgrad_load<MODE>(op, w, ld, m0, n0, va, vb);
      __syncthreads();
      HalfFrags f0, f1;
      read_half<wkey>(lds, 0, f0);
      read_half<wkey>(lds, 1, f1);
      int stage = 0;
      while (true) {
        char* nb = lds + (stage ^ 1) * STAGE_BYTES;
        mfma_half(f0, acc);
        bool more2 = false;
        if (more) {
          wgrad_store_one(nb, va);
          wgrad_store_one(nb + TILE_BYTES, vb);
          wait_all_mem();
          __syncthreads();
          read_half<wkey>(nb, 0, f0);
          more2 = seg_next(ld, w, e);
          if (more2) wgrad_load<MODE>(op, w, ld, m0, n0, va, vb);
        }
        mfma_half(f1, acc);
        if (!more) break;
        read_half<wkey>(nb, 1, f1);
        more = more2;
        stage ^= 1;
      }
      // the next tile's first stores must not overtake a slower wave's reads
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int m = m0 + frag_row(i, vv);
        float* dst;
        if (MODE == 0) {
          dst = out0 + ((int64_t)e * M + m) * N;
        } else {
          const int ii = (m >> 5) * 16 + (m & 15);
          dst = ((m & 31) < 16 ? out0 : out1) + ((int64_t)e * I + ii) * N;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[n0 + frag_col(j)] = acc[i][j][vv];
      }
  }
}

}  // namespace

void launch_gemm1_bf16(const ItemRange& ir, const uint16_t* ring, int32_t ring_rows, const uint16_t* wgu, int H,
                       int I, uint16_t* a_out, float* gu_save, int n_cu, hipStream_t s) {
  hipLaunchKernelGGL(gemm1_bf16_kernel, dim3(n_cu), dim3(NT), 0, s, ir, ring, ring_rows, wgu, H, I, a_out,
                     gu_save);
}

void launch_gemm2_bf16(const ItemRange& ir, const uint16_t* a, const uint16_t* wd, int H, int I, float* y32,
                       uint16_t* out, const int32_t* inv, const float* row_w, int n_cu, hipStream_t s) {
  if (out)
    hipLaunchKernelGGL(gemm2_bf16_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, a, wd, H, I, y32, out, inv, row_w);
  else
    hipLaunchKernelGGL(gemm2_bf16_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, a, wd, H, I, y32, out, inv,
                       row_w);
}

void launch_bwd_dact(const ItemRange& ir, const uint16_t* dye, const uint16_t* wdT, int H, int I, const float* gu,
                     const int32_t* inv, const float* row_w, uint16_t* dgdu, uint16_t* wa, float* dw_part, int n_cu,
                     hipStream_t s) {
  hipLaunchKernelGGL(bwd_dact_kernel, dim3(n_cu), dim3(NT), 0, s, ir, dye, wdT, H, I, gu, inv, row_w, dgdu, wa,
                     dw_part);
}

void launch_bwd_dx(const ItemRange& ir, const uint16_t* dgdu, const uint16_t* wguT, int H, int I,
                   const int32_t* inv, uint16_t* dX, int n_cu, hipStream_t s) {
  hipLaunchKernelGGL(bwd_dx_kernel, dim3(n_cu), dim3(NT), 0, s, ir, dgdu, wguT, H, I, inv, dX);
}

void launch_wgrad_down(const WgradArgs& w, const uint16_t* dye, const uint16_t* wa, int H, int I,
                       float* dW_down, int n_cu, hipStream_t s) {
  WgradOperands<0> op{dye, H, wa, I, nullptr, 1, 0, nullptr, 0};
  hipLaunchKernelGGL(wgrad_kernel<0>, dim3(n_cu), dim3(NT), 0, s, w, op, H, I, I, dW_down, (float*)nullptr);
}

void launch_wgrad_gate_up(const WgradArgs& w, const uint16_t* dgdu, const uint16_t* ring, int32_t ring_rows,
                          int first_resident, const uint16_t* x_src, int H, int I, float* dW_gate, float* dW_up,
                          int n_cu, hipStream_t s) {
  WgradOperands<1> op{dgdu, 2 * (int64_t)I, nullptr, 0, ring, ring_rows, first_resident, x_src, H};
  hipLaunchKernelGGL(wgrad_kernel<1>, dim3(n_cu), dim3(NT), 0, s, w, op, 2 * I, H, I, dW_gate, dW_up);
}

}  // namespace mk
