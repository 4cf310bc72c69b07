// Wave-level row operations shared by the row kernels (rows.hip) and the
// fused forward (one persistent launch, gemm_bf16.hip): copying one token
// row into the ring, and the fixed-order router-weighted combine of one
// token's routed rows.
#pragma once
#include "mk_device.h"

namespace mk {

// Copy one row of n16 16-byte granules from s to d with the whole wave:
// lane l moves granules l, l + 64, ...; eight loads are issued before their
// stores so each lane keeps several in flight.
__device__ __forceinline__ void copy_row_wave(const u32x4_t* __restrict__ s, u32x4_t* __restrict__ d, int64_t n16,
                                              int lane) {
  for (int64_t g0 = lane; g0 < n16; g0 += 64 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (g0 + 64 * u < n16) v[u] = __builtin_nontemporal_load(s + g0 + 64 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (g0 + 64 * u < n16) d[g0 + 64 * u] = v[u];
  }
}

// copy_row_wave with the stores written through to memory (device-coherent)
// through the buffer resource rd, d_off the row's byte offset in it.
__device__ __forceinline__ void copy_row_wave_wt(const u32x4_t* __restrict__ s, buf_rsrc_t rd, uint32_t d_off,
                                                 int64_t n16, int lane) {
  for (int64_t g0 = lane; g0 < n16; g0 += 64 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (g0 + 64 * u < n16) v[u] = __builtin_nontemporal_load(s + g0 + 64 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (g0 + 64 * u < n16)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, d_off + (uint32_t)(g0 + 64 * u) * 16, 0, MK_CPOL_DEVICE);
  }
}

// out[o] = sum_{j < kk} w[o*kk + j] * y[sorted_pos[o*kk + j]], j ascending,
// fp32, one rounding to bf16, for one output row o, by one wave.  A dropped
// row (sorted_pos -1) adds nothing.  Lane j (< kk <= 64) fetches the j-th
// routed row's position and weight once; lane l takes columns 4l .. 4l+3 of
// each 256-column chunk (one 16-byte load per routed row, 1 KiB contiguous
// per wave), two chunks at a time, the routed rows' loads issued 8 at a
// time and summed in row order.
__device__ __forceinline__ void combine_row_wave(const float* __restrict__ y, int64_t H,
                                                 const int32_t* __restrict__ sorted_pos,
                                                 const float* __restrict__ row_w, int kk, int64_t o,
                                                 uint16_t* __restrict__ out, int lane) {
  const int pj = lane < kk ? sorted_pos[o * kk + lane] : -1;
  const float wj = lane < kk ? row_w[o * kk + lane] : 0.f;
  for (int64_t c0 = 0; c0 < H; c0 += 2 * 256) {
    float acc[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[h][q] = 0.f;
    const bool act1 = c0 + 256 < H;
    for (int j0 = 0; j0 < kk; j0 += 8) {
      f32x4_t v[8][2];
      float wv[8];
      bool live[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int pos = __shfl(pj, j < kk ? j : 0);
        wv[u] = __shfl(wj, j < kk ? j : 0);
        live[u] = j < kk && pos >= 0;
        if (live[u]) {
          const float* src = y + (int64_t)pos * H + c0 + lane * 4;
          v[u][0] = __builtin_nontemporal_load((const f32x4_t*)src);
          v[u][1] = act1 ? __builtin_nontemporal_load((const f32x4_t*)(src + 256)) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!live[u]) continue;   // a dropped row adds nothing
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[h][q] += wv[u] * v[u][h][q];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && !act1) break;
      u32x2_t ov;
      ov[0] = pack_bf16x2(acc[h][0], acc[h][1]);
      ov[1] = pack_bf16x2(acc[h][2], acc[h][3]);
      __builtin_nontemporal_store(ov, (u32x2_t*)(out + o * H + c0 + h * 256 + lane * 4));
    }
  }
}

}  // namespace mk
