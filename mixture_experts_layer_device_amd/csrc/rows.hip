// Row-granular HBM kernels: the permute into the ring (bf16 copy or fused
// MXFP8 quantise), the backward's dY gather, the fixed-order combine, the
// standalone MXFP8 quantiser, the router-weight-gradient finalisation and the
// one-off weight packing.
//
// Every row here is a contiguous run of >= 512 bytes, so one wave per row
// with 16-byte lane accesses is fully coalesced as it stands; the loads of a
// row are all issued before its stores so each lane keeps several in flight.
#include "mk_device.h"
#include "mk_internal.h"
#include "rows_common.h"

#include <algorithm>

namespace mk {
namespace {

constexpr int RT = 256;   // threads per block in the row kernels

__device__ __forceinline__ int64_t wave_id() { return ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; }
__device__ __forceinline__ int64_t wave_count() { return ((int64_t)gridDim.x * blockDim.x) >> 6; }

// dst row (p mod ring_rows, or p) <- src row inv[p] / src_div
__global__ __launch_bounds__(RT) void gather_rows_kernel(const uint16_t* __restrict__ src, int64_t H,
                                                         const int32_t* __restrict__ inv, int src_div,
                                                         int64_t p_lo, int64_t p_hi, int32_t ring_rows,
                                                         uint16_t* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  for (int64_t p = p_lo + wave_id(); p < p_hi; p += wave_count()) {
    const int r = inv[p];
    if (r < 0) continue;
    copy_row_wave((const u32x4_t*)(src + (int64_t)(r / src_div) * H),
                  (u32x4_t*)(dst + (ring_rows ? p % ring_rows : p) * H), H / 8, lane);
  }
}

// Quantise one 32-element block (4 x 16 bytes of bf16) -> 32 codes + scale.
__device__ __forceinline__ uint32_t quant_block(const u32x4_t (&v)[4], u32x4_t (&c)[2]) {
  uint32_t amax = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      amax = max(amax, v[q][d] & 0x7FFFu);
      amax = max(amax, (v[q][d] >> 16) & 0x7FFFu);
    }
  const int s = mx_scale_code(amax);
  // 2^-se as an fp32 power of two (se in [-127, 119]: exponent field 8 .. 254)
  const float inv = __uint_as_float((uint32_t)(254 - s) << 23);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int d = 0; d < 4; d += 2) {
      float x[4] = {bf16_to_f32(v[q][d] & 0xFFFFu), bf16_to_f32(v[q][d] >> 16), bf16_to_f32(v[q][d + 1] & 0xFFFFu),
                    bf16_to_f32(v[q][d + 1] >> 16)};
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = e4m3_prescale(x[u], inv);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
      c[q >> 1][(q & 1) * 2 + (d >> 1)] = (uint32_t)w;
    }
  return (uint32_t)s;
}

// MXFP8 rows: codes[dst] / scales[dst] <- quantised src row (inv == nullptr: dst row = src row = p).
// MXFP8 quantise-gather: dst row (p mod ring_rows, or p) <- MX(src row
// inv[p] / src_div), or src row p with inv == nullptr.  Lane l takes values
// 8l .. 8l+7 of each 512-value chunk of the row (one 16-byte load, a whole
// wave reading 1 KiB contiguous), so an MX block of 32 is held by the 4 lanes
// 4q .. 4q+3: its amax is their maximum (two lane exchanges), every lane
// converts its own 8 values and stores 8 codes, and the first of the 4 stores
// the scale.  Eight chunks are in flight per lane.  H is a multiple of 32, so
// a block is never split across the row's end.
// (copy != nullptr: the bf16 row is also stored there, at row p)
__global__ __launch_bounds__(RT) void gather_rows_mxfp8_kernel(const uint16_t* __restrict__ src, int64_t H,
                                                               const int32_t* __restrict__ inv, int src_div,
                                                               int64_t p_lo, int64_t p_hi, int32_t ring_rows,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               uint16_t* __restrict__ copy) {
  const int lane = threadIdx.x & 63;
  for (int64_t p = p_lo + wave_id(); p < p_hi; p += wave_count()) {
    int64_t sr = p;
    if (inv) {
      const int r = inv[p];
      if (r < 0) continue;
      sr = r / src_div;
    }
    const int64_t dr = ring_rows ? p % ring_rows : p;
    const uint16_t* s = src + sr * H;
    uint8_t* dc = codes + dr * H;
    uint8_t* ds = scales + dr * (H / 32);
    for (int64_t c0 = 0; c0 < H; c0 += 8 * 512) {
      u32x4_t v[8];
      uint32_t am[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t e = c0 + u * 512 + lane * 8;
        v[u] = e < H ? __builtin_nontemporal_load((const u32x4_t*)(s + e)) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        uint32_t a = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) a = max(a, max(v[u][d] & 0x7FFFu, (v[u][d] >> 16) & 0x7FFFu));
        a = max(a, (uint32_t)__shfl_xor((int)a, 1));
        am[u] = max(a, (uint32_t)__shfl_xor((int)a, 2));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t e = c0 + u * 512 + lane * 8;
        if (e >= H) continue;
        const int sc = mx_scale_code(am[u]);
        // 2^-se as an fp32 power of two (se in [-127, 119]: exponent field 8 .. 254)
        const float invs = __uint_as_float((uint32_t)(254 - sc) << 23);
        uint32_t w2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t lo = v[u][2 * h], hi = v[u][2 * h + 1];
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale(bf16_to_f32(lo & 0xFFFFu), invs),
                                                  e4m3_prescale(bf16_to_f32(lo >> 16), invs), 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale(bf16_to_f32(hi & 0xFFFFu), invs),
                                              e4m3_prescale(bf16_to_f32(hi >> 16), invs), w, true);
          w2[h] = (uint32_t)w;
        }
        *(uint2*)(dc + e) = make_uint2(w2[0], w2[1]);
        if ((lane & 3) == 0) ds[e / 32] = (uint8_t)sc;
        if (copy) *(u32x4_t*)(copy + p * H + e) = v[u];
      }
    }
  }
}

// The full-layer combine (combine_row_wave): one wave per output row.
__global__ __launch_bounds__(RT) void combine_kernel(const float* __restrict__ y, int64_t H,
                                                     const int32_t* __restrict__ sorted_pos,
                                                     const float* __restrict__ row_w, int kk, int64_t n_out,
                                                     uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  for (int64_t o = wave_id(); o < n_out; o += wave_count()) combine_row_wave(y, H, sorted_pos, row_w, kk, o, out, lane);
}

__global__ void zero_dropped_rows_kernel(const int32_t* __restrict__ sorted_pos, int64_t R,
                                         uint16_t* __restrict__ out, int64_t H) {
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    if (sorted_pos[r] >= 0) continue;
    for (int64_t h = threadIdx.x; h < H; h += blockDim.x) out[r * H + h] = 0;
  }
}

// d_row_w[r] = sum over slices (ascending) of dw_part[sorted_pos[r]]; a dropped
// row gets 0 and (expert share, dX given) a zero dX row.  slices is a
// multiple of 8: the partials come in 16-byte loads, 8 in flight, and are
// added one by one in slice order.
__global__ void dw_finalize_kernel(const float* __restrict__ dw_part, int slices,
                                   const int32_t* __restrict__ sorted_pos, int64_t R, float* __restrict__ d_row_w,
                                   uint16_t* __restrict__ dX, int64_t H) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R; r += (int64_t)gridDim.x * blockDim.x) {
    const int pos = sorted_pos[r];
    if (pos >= 0) {
      const f32x4_t* q = (const f32x4_t*)(dw_part + (int64_t)pos * slices);
      float s = 0.f;
      for (int i0 = 0; i0 < slices / 4; i0 += 8) {
        f32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + u < slices / 4 ? q[i0 + u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u < slices / 4) s = (((s + v[u][0]) + v[u][1]) + v[u][2]) + v[u][3];
      }
      d_row_w[r] = s;
    } else {
      d_row_w[r] = 0.f;
      if (dX)
        for (int64_t h = 0; h < H; ++h) dX[r * H + h] = 0;
    }
  }
}

// Source row of the B operand rows: mode 0 -> src_a + (e * R + row) * len;
// mode 1 (gate/up, GEMM1's packing) -> packed row c of expert e: 32-row
// groups of 16 gate rows then the 16 up rows of the same i (R = 2I);
// mode 2 (gate then up) -> row c < I is gate row c, else up row c - I (R = 2I).
__device__ __forceinline__ const uint16_t* b_src_row(const uint16_t* src_a, const uint16_t* src_b, int mode, int e,
                                                     int row, int R, int64_t len) {
  if (mode == 0) return src_a + ((int64_t)e * R + row) * len;
  const int I = R / 2;
  if (mode == 2) return (row < I ? src_a + ((int64_t)e * I + row) * len : src_b + ((int64_t)e * I + row - I) * len);
  const int i = (row >> 5) * 16 + (row & 15);
  return ((row & 31) < 16 ? src_a : src_b) + ((int64_t)e * I + i) * len;
}

// Tiled B from source rows: B[e][n][k] = row(e, n)[k].  One thread per
// 16-byte granule, k fastest (reads of a row are contiguous).
__global__ void tile_rows_kernel(const uint16_t* __restrict__ src_a, const uint16_t* __restrict__ src_b, int mode,
                                 int E, int N, int K, uint16_t* __restrict__ out) {
  const int64_t kg = K / 8, total = (int64_t)E * N * kg;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(q % kg) * 8;
    const int64_t en = q / kg;
    const int e = (int)(en / N), n = (int)(en % N);
    const u32x4_t v = *(const u32x4_t*)(b_src_row(src_a, src_b, mode, e, n, N, K) + k);
    *(u32x4_t*)(out + btile_granule(e, n, k, N, K)) = v;
  }
}

// Tiled B from transposed source rows: B[e][n][k] = row(e, k)[n] (rows of
// length N, R = K rows per expert).  One workgroup per 256 x 64 block: the 64
// source row pieces (512 bytes each) go through LDS, then each thread
// assembles 8 output granules.
__global__ __launch_bounds__(256) void tile_cols_kernel(const uint16_t* __restrict__ src_a,
                                                        const uint16_t* __restrict__ src_b, int mode, int N, int K,
                                                        uint16_t* __restrict__ out) {
  constexpr int LD = BT_ROWS + 8;
  __shared__ uint16_t t[BT_K][LD];
  const int nt = blockIdx.x, kt = blockIdx.y, e = blockIdx.z, tid = threadIdx.x;
  const int n0 = nt * BT_ROWS, k0 = kt * BT_K;
  for (int q = tid; q < BT_K * (BT_ROWS / 8); q += 256) {
    const int kk = q / (BT_ROWS / 8), c = (q % (BT_ROWS / 8)) * 8;
    const u32x4_t v = *(const u32x4_t*)(b_src_row(src_a, src_b, mode, e, k0 + kk, K, N) + n0 + c);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      t[kk][c + 2 * d] = (uint16_t)(v[d] & 0xFFFFu);
      t[kk][c + 2 * d + 1] = (uint16_t)(v[d] >> 16);
    }
  }
  __syncthreads();
  uint16_t* blk = out + btile_block(e, nt, kt, N, K);
  for (int q = tid; q < BT_ROWS * (BT_K / 8); q += 256) {
    const int r = q / (BT_K / 8), g = q % (BT_K / 8);
    u32x4_t v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = (uint32_t)t[8 * g + 2 * d][r] | ((uint32_t)t[8 * g + 2 * d + 1][r] << 16);
    *(u32x4_t*)(blk + r * BT_K + ((g ^ tkey(r)) & 7) * 8) = v;
  }
}

// Tiled MXFP8 B from source rows (the b_src_row mapping): one wave per row
// (e, n), one 32-element MX block per lane step, codes and scale written to
// their places in the tiled layout.
__global__ __launch_bounds__(RT) void quant_tile_rows_kernel(const uint16_t* __restrict__ src_a,
                                                             const uint16_t* __restrict__ src_b, int mode,
                                                             int64_t n_rows, int N, int K,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int nblk = K / 32;
  for (int64_t row = wave_id(); row < n_rows; row += wave_count()) {
    const int e = (int)(row / N), n = (int)(row % N);
    const int r = n % MXT_ROWS;
    const u32x4_t* s = (const u32x4_t*)b_src_row(src_a, src_b, mode, e, n, N, K);
    for (int b = lane; b < nblk; b += 64) {
      u32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = s[b * 4 + q];
      u32x4_t cc[2];
      const uint32_t sc = quant_block(v, cc);
      const int64_t t = mxt_index(e, n / MXT_ROWS, b / 4, N, K);
      uint8_t* blk = codes + t * MXT_CODES + r * MXT_K;
      const int g0 = (b % 4) * 2;
      *(u32x4_t*)(blk + (((g0 ^ tkey(r)) & 7) << 4)) = cc[0];
      *(u32x4_t*)(blk + ((((g0 + 1) ^ tkey(r)) & 7) << 4)) = cc[1];
      scales[t * MXT_SCALES + r * 4 + (b % 4)] = (uint8_t)sc;
    }
  }
}

int row_grid(int64_t rows, int n_cu) {
  const int64_t want = (rows + (RT / 64) - 1) / (RT / 64);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)n_cu * 8));
}

}  // namespace

void launch_gather_rows(const uint16_t* src, int64_t H, const int32_t* inv, int src_div, int64_t p_lo,
                        int64_t p_hi, int32_t ring_rows, uint16_t* dst, int n_cu, hipStream_t s) {
  if (p_hi <= p_lo) return;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(row_grid(p_hi - p_lo, n_cu)), dim3(RT), 0, s, src, H, inv, src_div,
                     p_lo, p_hi, ring_rows, dst);
}

void launch_gather_rows_mxfp8(const uint16_t* src, int64_t H, const int32_t* inv, int src_div, int64_t p_lo,
                              int64_t p_hi, int32_t ring_rows, uint8_t* codes, uint8_t* scales, int n_cu,
                              hipStream_t s, uint16_t* copy) {
  if (p_hi <= p_lo) return;
  hipLaunchKernelGGL(gather_rows_mxfp8_kernel, dim3(row_grid(p_hi - p_lo, n_cu)), dim3(RT), 0, s, src, H, inv,
                     src_div, p_lo, p_hi, ring_rows, codes, scales, copy);
}

void launch_quantize(const uint16_t* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(gather_rows_mxfp8_kernel, dim3(row_grid(rows, 256)), dim3(RT), 0, s, in, (int64_t)K,
                     (const int32_t*)nullptr, 1, (int64_t)0, rows, 0, codes, scales, (uint16_t*)nullptr);
}

void launch_zero_dropped_rows(const int32_t* sorted_pos, int64_t R, uint16_t* out, int64_t H, hipStream_t s) {
  if (R <= 0) return;
  hipLaunchKernelGGL(zero_dropped_rows_kernel, dim3((unsigned)std::min<int64_t>(R, 4096)), dim3(256), 0, s,
                     sorted_pos, R, out, H);
}

void launch_combine(const float* y, int64_t H, const int32_t* sorted_pos, const float* row_w, int k,
                    int64_t n_out, uint16_t* out, int n_cu, hipStream_t s) {
  if (n_out <= 0) return;
  hipLaunchKernelGGL(combine_kernel, dim3(row_grid(n_out, n_cu)), dim3(RT), 0, s, y, H, sorted_pos, row_w, k,
                     n_out, out);
}

void launch_dw_finalize(const float* dw_part, int slices, const int32_t* sorted_pos, int64_t R, float* d_row_w,
                        uint16_t* dX, int64_t H, hipStream_t s) {
  if (R <= 0) return;
  const int blocks = (int)std::min<int64_t>((R + 255) / 256, 2048);
  hipLaunchKernelGGL(dw_finalize_kernel, dim3(blocks), dim3(256), 0, s, dw_part, slices, sorted_pos, R, d_row_w,
                     dX, H);
}

void launch_tile_rows(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K, uint16_t* out,
                      hipStream_t s) {
  const int64_t total = (int64_t)E * N * (K / 8);
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(tile_rows_kernel, dim3(blocks), dim3(256), 0, s, src_a, src_b, mode, E, N, K, out);
}

void launch_tile_cols(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K, uint16_t* out,
                      hipStream_t s) {
  hipLaunchKernelGGL(tile_cols_kernel, dim3(N / BT_ROWS, K / BT_K, E), dim3(256), 0, s, src_a, src_b, mode, N, K,
                     out);
}

// Tiled MXFP8 B from source columns: B[e][n][k] = row(e, k)[n], quantised
// along k.  Workgroup (n block of 256, k block of 128, e): the 128 source rows'
// 256-value slices go to LDS (16-byte granules), then each thread gathers a
// 32-value column segment, quantises it and stores its two code granules and
// its scale byte in the block.
__global__ __launch_bounds__(256) void quant_tile_cols_kernel(const uint16_t* __restrict__ src_a,
                                                              const uint16_t* __restrict__ src_b, int mode, int N,
                                                              int K, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  constexpr int LD = MXT_ROWS + 8;            // row stride 528 bytes: 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t t[MXT_K][LD];
  const int nt = blockIdx.x, kt = blockIdx.y, e = blockIdx.z, tid = threadIdx.x;
  const int n0 = nt * MXT_ROWS, k0 = kt * MXT_K;
  for (int q = tid; q < MXT_K * (MXT_ROWS / 8); q += 256) {
    const int kk = q / (MXT_ROWS / 8), c = (q % (MXT_ROWS / 8)) * 8;
    *(u32x4_t*)&t[kk][c] = *(const u32x4_t*)(b_src_row(src_a, src_b, mode, e, k0 + kk, K, N) + n0 + c);
  }
  __syncthreads();
  const int64_t ti = mxt_index(e, nt, kt, N, K);
  uint8_t* cblk = codes + ti * MXT_CODES;
  uint8_t* sblk = scales + ti * MXT_SCALES;
  for (int q = tid; q < MXT_ROWS * (MXT_K / 32); q += 256) {
    const int r = q % MXT_ROWS, kb = q / MXT_ROWS;
    u32x4_t v[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int k = kb * 32 + g * 8 + 2 * d;
        v[g][d] = (uint32_t)t[k][r] | ((uint32_t)t[k + 1][r] << 16);
      }
    u32x4_t cc[2];
    const uint32_t sc = quant_block(v, cc);
    const int g0 = kb * 2;
    *(u32x4_t*)(cblk + r * MXT_K + (((g0 ^ tkey(r)) & 7) << 4)) = cc[0];
    *(u32x4_t*)(cblk + r * MXT_K + ((((g0 + 1) ^ tkey(r)) & 7) << 4)) = cc[1];
    sblk[r * 4 + kb] = (uint8_t)sc;
  }
}

void launch_quant_tile_cols(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K,
                            uint8_t* codes, uint8_t* scales, hipStream_t s) {
  hipLaunchKernelGGL(quant_tile_cols_kernel, dim3(N / MXT_ROWS, K / MXT_K, E), dim3(256), 0, s, src_a, src_b, mode, N,
                     K, codes, scales);
}

void launch_quant_tile_rows(const uint16_t* src_a, const uint16_t* src_b, int mode, int E, int N, int K,
                            uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t n_rows = (int64_t)E * N;
  hipLaunchKernelGGL(quant_tile_rows_kernel, dim3(row_grid(n_rows, 256)), dim3(RT), 0, s, src_a, src_b, mode, n_rows,
                     N, K, codes, scales);
}


// ---- MXFP8 weight-gradient operands ----------------------------------------

namespace {

// One workgroup: expert e's K extent Kpad_e = roundup128(sum over minibatches
// of roundup32(rows)), an exclusive scan over the experts (Hillis-Steele in
// LDS), and the experts ranked by descending K for the GEMM's tile order.
__global__ __launch_bounds__(1024) void wgrad_kofs_kernel(const int32_t* __restrict__ mb_counts, int nb, int E,
                                                          int32_t* __restrict__ kofs, int32_t* __restrict__ order) {
  __shared__ int kp[1024], sc[1024];
  const int e = threadIdx.x;
  int v = 0;
  if (e < E) {
    for (int b = 0; b < nb; ++b) v += (mb_counts[b * E + e] + 31) & ~31;
    v = (v + 127) & ~127;
  }
  kp[e] = v;
  sc[e] = v;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int add = e >= d ? sc[e - d] : 0;
    __syncthreads();
    sc[e] += add;
    __syncthreads();
  }
  if (e < E) {
    kofs[e] = sc[e] - v;
    int rank = 0;
    for (int q = 0; q < E; ++q) rank += (kp[q] > v) || (kp[q] == v && q < e);
    order[rank] = e;
  }
  if (e == 0) kofs[E] = sc[E - 1];
}

// Row map of the K space: kmap[k] = position p of row k (or -1 for a pad
// row).  Workgroup (b, e) writes segment (b, e): its K start is kofs[e] plus
// the 32-rounded lengths of the later minibatches (the walk is nb-1 .. 0);
// the last segment of the walk (b = 0) also covers the expert's pad to 128.
__global__ __launch_bounds__(256) void wgrad_kmap_kernel(const int32_t* __restrict__ kofs,
                                                         const int32_t* __restrict__ mb_counts,
                                                         const int32_t* __restrict__ mb_offsets, int E, int nb, int MB,
                                                         int32_t* __restrict__ kmap) {
  __shared__ int sstart;
  const int b = blockIdx.x, e = blockIdx.y, tid = threadIdx.x;
  if (tid == 0) {
    int st = kofs[e];
    for (int q = nb - 1; q > b; --q) st += (mb_counts[q * E + e] + 31) & ~31;
    sstart = st;
  }
  __syncthreads();
  const int st = sstart;
  const int n = mb_counts[b * E + e];
  const int base = b * MB + mb_offsets[b * (E + 1) + e];
  const int end = b == 0 ? kofs[e + 1] : st + ((n + 31) & ~31);
  for (int j = tid; st + j < end; j += 256) kmap[st + j] = j < n ? base + j : -1;
}

// Workgroup (half ct of a 256-column block, global k step kc): the 128 rows
// of the step x 128 columns come to LDS (8 loads of 16 bytes per thread,
// all issued before the first LDS store); thread (r, h) then quantises MX
// blocks 2h and 2h+1 of column r (quant_block) into its half of row r of the
// tiled block's image, built in LDS over the staged rows, and the 16 KiB
// image goes out with 16-byte stores that are contiguous across the
// workgroup (a thread's own 64 bytes would be 16-byte pieces 128 bytes apart
// from its neighbours': a partial line each).  35 KiB of LDS and at most 128
// registers: four workgroups per compute unit, so one's loads overlap
// another's quantising.
__global__ __launch_bounds__(256, 4) void quant_wgrad_operand_kernel(
    const uint16_t* __restrict__ src, int64_t ld, const int32_t* __restrict__ inv, int src_div, int C,
    const int32_t* __restrict__ kofs, int E, const int32_t* __restrict__ kmap, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  constexpr int CW = MXT_ROWS / 2;                     // columns per workgroup
  constexpr int LD = CW + 8;
  constexpr int PER = MXT_K * (CW / 8) / 256;          // 16-byte loads per thread
  __shared__ __attribute__((aligned(16))) uint16_t t[MXT_K][LD];
  __shared__ int64_t srow[MXT_K];
  const int ct = blockIdx.x >> 1, half = blockIdx.x & 1, kc = blockIdx.y, tid = threadIdx.x;
  const int k0 = kc * MXT_K;
  if (k0 >= kofs[E]) return;                    // the whole workgroup leaves together
  // expert of this step: the last e with kofs[e] <= k0 (kofs is ascending)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kofs[mid] <= k0) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int ke = kofs[e], kpad = kofs[e + 1] - ke;
  if (tid < MXT_K) {
    const int p = kmap[k0 + tid];
    srow[tid] = p < 0 ? -1 : inv ? (int64_t)(inv[p] / src_div) : (int64_t)p;
  }
  __syncthreads();
  const int c0 = ct * MXT_ROWS + half * CW;
  u32x4_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = tid + i * 256;
    const int kk = q / (CW / 8), c = (q % (CW / 8)) * 8;
    const int64_t row = srow[kk];
    v[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (row >= 0) v[i] = *(const u32x4_t*)(src + row * ld + c0 + c);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = tid + i * 256;
    *(u32x4_t*)&t[q / (CW / 8)][(q % (CW / 8)) * 8] = v[i];
  }
  __syncthreads();
  const int64_t blk = (int64_t)(C / MXT_ROWS) * (ke / MXT_K) + (int64_t)ct * (kpad / MXT_K) + (k0 - ke) / MXT_K;
  const int r = tid & (CW - 1), kh = tid / CW;        // column within the half; MX blocks 2kh, 2kh+1
  const int br = half * CW + r;                        // its row in the tiled block
  uint32_t sc = 0;
  u32x4_t cc[4];                                       // granules 4kh .. 4kh+3 of the block row
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    const int kb = 2 * kh + b2;
    u32x4_t w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int k = kb * 32 + g * 8 + 2 * d;
        w[g][d] = (uint32_t)t[k][r] | ((uint32_t)t[k + 1][r] << 16);
      }
    u32x4_t c2[2];
    sc |= quant_block(w, c2) << (8 * b2);
    cc[2 * b2] = c2[0];
    cc[2 * b2 + 1] = c2[1];
  }
  // the row's scale bytes 2kh, 2kh+1 (MX blocks of this thread)
  *(uint16_t*)(scales + blk * MXT_SCALES + br * 4 + 2 * kh) = (uint16_t)sc;
  static_assert(CW * MXT_K <= MXT_K * LD * 2, "the half image fits over the staged rows");
  char* img = (char*)&t[0][0];
  __syncthreads();                              // every column read
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(u32x4_t*)(img + r * MXT_K + ((((4 * kh + g) ^ tkey(br)) & 7) << 4)) = cc[g];
  __syncthreads();
  uint8_t* cblk = codes + blk * MXT_CODES + half * CW * MXT_K;
#pragma unroll
  for (int i = 0; i < CW * MXT_K / (16 * 256); ++i) {
    const int off = (tid + 256 * i) * 16;
    *(u32x4_t*)(cblk + off) = *(const u32x4_t*)(img + off);
  }
}

}  // namespace

void launch_wgrad_kofs(const int32_t* mb_counts, int nb, int E, int32_t* kofs, int32_t* order, hipStream_t s) {
  hipLaunchKernelGGL(wgrad_kofs_kernel, dim3(1), dim3(1024), 0, s, mb_counts, nb, E, kofs, order);
}

void launch_wgrad_kmap(const int32_t* kofs, const int32_t* mb_counts, const int32_t* mb_offsets, int E, int nb,
                       int MB, int32_t* kmap, hipStream_t s) {
  if (nb > 0)
    hipLaunchKernelGGL(wgrad_kmap_kernel, dim3(nb, E), dim3(256), 0, s, kofs, mb_counts, mb_offsets, E, nb, MB, kmap);
}

void launch_quant_wgrad_operand(const uint16_t* src, int64_t ld, const int32_t* inv, int src_div, int C,
                                const int32_t* kofs, int E, const int32_t* kmap, int64_t kcap, uint8_t* codes,
                                uint8_t* scales, hipStream_t s) {
  hipLaunchKernelGGL(quant_wgrad_operand_kernel, dim3(2 * (C / MXT_ROWS), (unsigned)(kcap / MXT_K)), dim3(256), 0, s, src,
                     ld, inv, src_div, C, kofs, E, kmap, codes, scales);
}


}  // namespace mk
