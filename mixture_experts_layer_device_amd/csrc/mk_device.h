// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + __expf(-g)); }

// ---- MXFP8 (OCP MX v1.0, E4M3 elements, E8M0 shared scale per 32) ---------
//
// Shared exponent of a block from the bf16 bit pattern of its largest
// magnitude: floor(log2(amax)) - 8 (8 = E4M3's largest normal exponent),
// clamped below at -127.  Returns the biased E8M0 code; 0 for amax == 0.
__device__ __forceinline__ int mx_scale_code(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  int E = (int)(amax_bits >> 7);
  int fl = E ? E - 127 : (31 - __clz((int)(amax_bits & 0x7F))) - 133;
  int se = fl - 8;
  if (se < -127) se = -127;
  return se + 127;
}

// E4M3-FN code of (bf16 value) / 2^se, nearest-even, saturating at 448,
// sign kept.  Works on integer significands: exact for every bf16 input.
__device__ __forceinline__ uint32_t mx_encode(uint32_t bits, int se) {
  uint32_t sign = (bits >> 8) & 0x80u;
  int E = (int)((bits >> 7) & 0xFF);
  int m = (int)(bits & 0x7F);
  if (E == 0 && m == 0) return sign;
  int S, x;                                  // |v| = S * 2^x
  if (E) { S = 128 | m; x = E - 134; } else { S = m; x = -133; }
  int pb = 31 - __clz(S);                    // msb of S
  int eq = pb + x - se;                      // floor(log2 |v / 2^se|)
  bool normal = eq >= -6;
  int shift = normal ? pb - 3 : -(x - se + 9);
  uint32_t keep;
  if (shift <= 0) {
    keep = (uint32_t)S << (-shift);
  } else if (shift > 24) {
    keep = 0;
  } else {
    keep = (uint32_t)S >> shift;
    uint32_t rem = (uint32_t)S & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (keep & 1u))) ++keep;
  }
  uint32_t code;
  if (normal) {
    if (keep == 16) { keep = 8; ++eq; }
    if (eq > 8) return sign | 0x7Eu;
    code = ((uint32_t)(eq + 7) << 3) | (keep - 8);
    if (code > 0x7Eu) code = 0x7Eu;
  } else {
    code = keep;                              // 0..8 (8 = smallest normal, code 0x08)
  }
  return sign | code;
}

// XOR swizzle of 16-byte granules in a 128-byte-per-row LDS tile: conflict
// free for 8 or 16 consecutive rows reading the same logical granule.
__device__ __forceinline__ int lds_swz(int row, int g) {
  return row * 128 + ((((g ^ row ^ (row >> 3))) & 7) << 4);
}

// Inverse of lds_swz inside a row: the logical granule that lands in slot s.
__device__ __forceinline__ int lds_unswz(int row, int s) { return (s ^ row ^ (row >> 3)) & 7; }

// ---- tiled GEMM B operand ("LDS image" layout) ----------------------------
//
// A bf16 B operand B[e][n][k] (N a multiple of 256, K of 64) is stored as
// 32 KiB blocks, one per (e, n / 256, k / 64) in that order, each holding the
// 256 x 64 slice exactly as the GEMM stage keeps it in LDS: 128-byte rows,
// the row's 16-byte granule g (k = 8g .. 8g+7 of the slice) in slot
// g ^ tkey(row).  A stage's B slice then arrives with 1 KiB contiguous DMA
// copies.  tkey = (row >> 1) & 7 makes the MFMA fragment reads (16 rows, one
// granule) conflict-free and, using bits 1..3 of the row only, is the same for
// every 16-row fragment a lane reads.
__device__ __forceinline__ int tkey(int row) { return (row >> 1) & 7; }
constexpr int BT_ROWS = 256, BT_K = 64, BT_BLOCK = BT_ROWS * BT_K;   // elements per block
__device__ __forceinline__ int64_t btile_block(int e, int nt, int kt, int N, int K) {
  return (((int64_t)e * (N / BT_ROWS) + nt) * (K / BT_K) + kt) * BT_BLOCK;
}
// element offset of the 16-byte granule holding B[e][n][k .. k+7] (k % 8 == 0)
__device__ __forceinline__ int64_t btile_granule(int e, int n, int k, int N, int K) {
  const int r = n % BT_ROWS, g = (k % BT_K) / 8;
  return btile_block(e, n / BT_ROWS, k / BT_K, N, K) + r * BT_K + ((g ^ tkey(r)) & 7) * 8;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Asynchronous global -> LDS copy (global_load_lds_dwordx4 / _dword): lane i's
// bytes land at dst + size*i, where dst is the same for the whole wave.
__device__ __forceinline__ void g2lds16(const void* src, char* wave_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)wave_dst, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* src, char* wave_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)wave_dst, 4, 0, 0);
}
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace mk
