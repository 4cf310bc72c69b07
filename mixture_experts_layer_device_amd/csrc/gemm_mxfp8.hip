// Expert-grouped MXFP8 GEMMs on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3, one E8M0 scale per 32 K).
//
// Same persistent walk, tile shape (256 x 256, 4 waves of 128 x 128) and
// double-buffered LDS-DMA pipeline as the bf16 GEMMs; a K step is 128 codes
// (one MFMA deep), i.e. 4 MX blocks whose 4 scale bytes per row travel as one
// dword next to the tile.
//
// Operand layout of the block-scaled MFMA (measured on gfx950): lane group
// g = l/16 of a 16-row fragment supplies k in [16g, 16g+16) in its bytes
// 0..15 and k in [64+16g, 64+16g+16) in bytes 16..31, and its scale applies to
// k in [32g, 32g+32).  So lane group g takes 16-byte granules g and g+4 of the
// 128-byte K step (MX block g = granules 2g and 2g+1 land in hardware block g)
// and passes scale byte g.
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

// A quarter of a wave's operands for one K step: 4 fragments (of A rows or B
// columns) with their scale bytes.
struct Quarter {
  i32x8_t v[4];
  int sc;   // byte f: the lane's scale for fragment f (picked by the MFMA's op_sel)
};

// half h of the wave's A rows (OPB = 0) or B columns (OPB = 1) of a stage.
// Every row a lane reads has the same swizzle key ((l%16) >> 1), so the
// addresses are two lane bases (granules g and g+4) plus constants.
template <int OPB>
__device__ __forceinline__ void read_quarter(const char* st, int h, Quarter& q) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = OPB ? (wave & 1) : (wave >> 1);
  const int l16 = lane & 15, g = lane >> 4;
  const int key = (l16 >> 1) & 7;
  const char* base = st + OPB * TILE_BYTES + (w * 128 + h * 64) * 128 + l16 * 128;
  const char* plo = base + (((g ^ key) & 7) << 4);
  const char* phi = base + ((((g + 4) ^ key) & 7) << 4);
  const uint8_t* psc = (const uint8_t*)(st + 2 * TILE_BYTES + OPB * SCALE_BYTES) + (w * 128 + h * 64 + l16) * 4 + g;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const u32x4_t lo = *(const u32x4_t*)(plo + f * 2048);
    const u32x4_t hi = *(const u32x4_t*)(phi + f * 2048);
    q.v[f] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  q.sc = (int)((uint32_t)psc[0] | ((uint32_t)psc[64] << 8) | ((uint32_t)psc[128] << 16) | ((uint32_t)psc[192] << 24));
}

// 16 MFMAs: A rows of half IH x B columns of half JH.
template <int IH, int JH>
__device__ __forceinline__ void mfma_quarter(const Quarter& qa, const Quarter& qb, Acc& acc) {
  __builtin_amdgcn_sched_barrier(0);
  static_for<4>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    static_for<4>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      acc[4 * IH + i][4 * JH + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          qa.v[i], qb.v[j], acc[4 * IH + i][4 * JH + j], 0, 0, i, qa.sc, j, qb.sc);
    });
  });
  __builtin_amdgcn_sched_barrier(0);
  pin_acc(acc);
}

// C = A . B^T over K codes.  A row r's codes start at abase + aoff(r), its
// scale bytes at asbase + asoff(r) (likewise B); bases uniform, offsets 32-bit.
// Codes go global -> LDS directly as in the bf16 mainloop (wave w fills rows
// 64w .. 64w+63, 8 full 128-byte rows per instruction, swizzled); each wave
// also fetches the scale dwords of its 64 A rows and 64 B rows.
//
// Pipeline: the wave's operands of a stage are four quarters A0 A1 (row
// halves) and B0 B1 (column halves), consumed in four 16-MFMA phases
// (A0,B0) (A0,B1) (A1,B0) (A1,B1).  After the second phase A0 is free and,
// past the single workgroup barrier of the step (stage s+1 landed, stage s
// read by all), receives stage s+1 while the DMA of stage s+2 starts; B0 is
// refilled after the third phase, A1 and B1 after the fourth.  Each refilled
// quarter is first needed one or two phases later.
struct MxOperand {
  const char* codes;
  uint32_t code_bytes;
  const char* scales;
  uint32_t scale_bytes;
};

// B's rows are evenly spaced (K codes, K/32 scale bytes apart), so its 8 row
// groups share one offset register and differ in the scalar offset.
template <typename AOff, typename ASOff>
__device__ __forceinline__ void mainloop(const MxOperand& A, AOff aoff, ASOff asoff, const MxOperand& B, int K,
                                         char* lds, Acc& acc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t nb = (uint32_t)K / 32;
  uint32_t ao[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + (lane >> 3);
    const uint32_t g16 = (uint32_t)(((lane & 7) ^ tkey(r)) & 7) << 4;
    ao[j] = aoff(r) + g16;
  }
  // tkey(r) for these rows depends on (lane >> 3) and j only through bits
  // that j * 8 does not touch: (r >> 1) & 7 = ((lane >> 3) >> 1) | 4 * (j & 1)
  const int r0 = wave * 64 + (lane >> 3);
  const uint32_t bo_even = (uint32_t)r0 * (uint32_t)K + ((uint32_t)(((lane & 7) ^ tkey(r0)) & 7) << 4);
  const uint32_t bo_odd = (uint32_t)r0 * (uint32_t)K + ((uint32_t)(((lane & 7) ^ tkey(r0 + 8)) & 7) << 4);
  const uint32_t aso = asoff(wave * 64 + lane), bso = (uint32_t)(wave * 64 + lane) * nb;
  const int wbase = wave * 8192;
  const int sbase = 2 * TILE_BYTES + wave * 256;
  const buf_rsrc_t ra = make_rsrc(A.codes, A.code_bytes), rb = make_rsrc(B.codes, B.code_bytes);
  const buf_rsrc_t rsa = make_rsrc(A.scales, A.scale_bytes), rsb = make_rsrc(B.scales, B.scale_bytes);
  auto issue = [&](int kt, char* st) {
    const uint32_t kb = (uint32_t)kt * BKB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      b2lds16(ra, ao[j], kb, st + wbase + j * 1024);
      b2lds16(rb, (j & 1) ? bo_odd : bo_even, kb + (uint32_t)(j * 8 * K), st + TILE_BYTES + wbase + j * 1024);
    }
    b2lds4(rsa, aso, (uint32_t)kt * 4, st + sbase);
    b2lds4(rsb, bso, (uint32_t)kt * 4, st + sbase + SCALE_BYTES);
  };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  pin_acc(acc);
  const int KT = K / BKB;
  issue(0, lds);
  wait_all_mem();
  __syncthreads();
  if (KT > 1) issue(1, lds + STAGE_BYTES);
  Quarter a0, a1, b0, b1;
  read_quarter<0>(lds, 0, a0);
  read_quarter<1>(lds, 0, b0);
  read_quarter<1>(lds, 1, b1);
  read_quarter<0>(lds, 1, a1);
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    const char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
    mfma_quarter<0, 0>(a0, b0, acc);
    mfma_quarter<0, 1>(a0, b1, acc);
    if (more) {
      wait_all_mem();
      __syncthreads();
      if (kt + 2 < KT) issue(kt + 2, lds + (kt & 1) * STAGE_BYTES);
    }
    // refills are unconditional (after the last step they read an idle
    // buffer and go unused), so the quarters stay in place across steps
    read_quarter<0>(nxt, 0, a0);
    mfma_quarter<1, 0>(a1, b0, acc);
    read_quarter<1>(nxt, 0, b0);
    mfma_quarter<1, 1>(a1, b1, acc);
    read_quarter<1>(nxt, 1, b1);
    read_quarter<0>(nxt, 1, a1);
  }
  // every wave is done with both buffers before an epilogue reuses the LDS
  __syncthreads();
}

// a[p, i] = silu(g) * u (bf16) from MXFP8 ring rows and packed MXFP8 W_gu.
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm1_mxfp8_kernel(ItemRange ir, const uint8_t* __restrict__ rc,
                                                         const uint8_t* __restrict__ rsc, int ring_rows,
                                                         const uint8_t* __restrict__ wc,
                                                         const uint8_t* __restrict__ wsc, int H, int I,
                                                         uint16_t* __restrict__ a_out) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int ntn = 2 * I / BN;
  const int nbh = H / 32;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    // ring offsets stay below the ring's size (< 2 GiB)
    auto rrow = [&](int r) { return (uint32_t)((ti.pos0 + min(r, ti.rows - 1)) % ring_rows); };
    auto aoff = [&](int r) { return rrow(r) * (uint32_t)H; };
    auto asoff = [&](int r) { return rrow(r) * (uint32_t)nbh; };
    const int64_t wrow0 = (int64_t)ti.e * 2 * I + ti.n0;
    const MxOperand A{(const char*)rc, (uint32_t)ring_rows * (uint32_t)H, (const char*)rsc,
                      (uint32_t)ring_rows * (uint32_t)nbh};
    const MxOperand B{(const char*)(wc + wrow0 * H), (uint32_t)(BN * H), (const char*)(wsc + wrow0 * nbh),
                      (uint32_t)(BN * nbh)};
    Acc acc;
    mainloop(A, aoff, asoff, B, H, lds, acc);
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int q = 0; q < FN / 2; ++q) {
          const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
          stage_put(lds, frag_row(i, v), wn * 64 + q * 16 + (lane & 15), g * sigmoidf_(g) * u);
        }
    });
    stage_flush<128>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? a_out + (int64_t)(ti.pos0 + r) * I + ti.n0 / 2 : nullptr;
    });
  });
}

// y[p] = D(a_q[p]) . D(W_d[e])^T with W_d codes [E, H, I] + scales [E, H, I/32];
// SHARE: out[inv[p]] = bf16(w * y) (fused weighted unpermute); else fp32 y.
template <bool SHARE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm2_mxfp8_kernel(ItemRange ir, const uint8_t* __restrict__ ac,
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
    auto aoff = [&](int r) { return (uint32_t)min(r, ti.rows - 1) * (uint32_t)I; };
    auto asoff = [&](int r) { return (uint32_t)min(r, ti.rows - 1) * (uint32_t)nbi; };
    const int64_t wrow0 = (int64_t)ti.e * H + ti.n0;
    const MxOperand A{(const char*)(ac + (int64_t)ti.pos0 * I), (uint32_t)ti.rows * (uint32_t)I,
                      (const char*)(asc_ + (int64_t)ti.pos0 * nbi), (uint32_t)ti.rows * (uint32_t)nbi};
    const MxOperand B{(const char*)(wc + wrow0 * I), (uint32_t)(BN * I), (const char*)(wsc + wrow0 * nbi),
                      (uint32_t)(BN * nbi)};
    Acc acc;
    mainloop(A, aoff, asoff, B, I, lds, acc);
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

}  // namespace

void launch_gemm1_mxfp8(const ItemRange& ir, const uint8_t* ring_codes, const uint8_t* ring_scales,
                        int32_t ring_rows, const uint8_t* wgu_codes, const uint8_t* wgu_scales, int H, int I,
                        uint16_t* a_out, int n_cu, hipStream_t s) {
  hipLaunchKernelGGL(gemm1_mxfp8_kernel, dim3(n_cu), dim3(NT), 0, s, ir, ring_codes, ring_scales, ring_rows,
                     wgu_codes, wgu_scales, H, I, a_out);
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
