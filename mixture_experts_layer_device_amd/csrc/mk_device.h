// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
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

// The same code through the hardware conversion: the fp32 value times the
// power of two 2^-se (exact: the product is a normal fp32 number, or below
// 2^-126 and so far under E4M3's smallest subnormal that it encodes to a
// signed zero either way), clamped to +-448 (every value at or beyond 448
// encodes to 448 under saturating nearest-even rounding), then
// v_cvt_pk_fp8_f32 (OCP E4M3, nearest-even).
__device__ __forceinline__ float e4m3_prescale(float x, float inv_scale) {
  return fminf(fmaxf(x * inv_scale, -448.f), 448.f);
}


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
// byte offset of granule g of a 128-byte LDS row swizzled with tkey
__device__ __forceinline__ int tswz(int row, int g) { return row * 128 + (((g ^ tkey(row)) & 7) << 4); }
constexpr int BT_ROWS = 256, BT_K = 64, BT_BLOCK = BT_ROWS * BT_K;   // elements per block
__device__ __forceinline__ int64_t btile_block(int e, int nt, int kt, int N, int K) {
  return (((int64_t)e * (N / BT_ROWS) + nt) * (K / BT_K) + kt) * BT_BLOCK;
}
// element offset of the 16-byte granule holding B[e][n][k .. k+7] (k % 8 == 0)
__device__ __forceinline__ int64_t btile_granule(int e, int n, int k, int N, int K) {
  const int r = n % BT_ROWS, g = (k % BT_K) / 8;
  return btile_block(e, n / BT_ROWS, k / BT_K, N, K) + r * BT_K + ((g ^ tkey(r)) & 7) * 8;
}

// ---- tiled MXFP8 B operand -------------------------------------------------
//
// MXFP8 weights B[e][n][k] (E4M3 codes, one E8M0 scale per 32 k) are stored
// per (e, n / 256, k / 128), in that order, as a 32 KiB block of codes (256
// rows x 128 codes, the LDS image of one MXFP8 GEMM stage: 16-code granule g
// of row r in slot g ^ tkey(r)) and a 1 KiB block of scales (row r's four
// scale bytes of the K step at 4r).
constexpr int MXT_ROWS = 256, MXT_K = 128, MXT_CODES = MXT_ROWS * MXT_K, MXT_SCALES = MXT_ROWS * 4;
__device__ __forceinline__ int64_t mxt_index(int e, int nt, int kt, int N, int K) {
  return ((int64_t)e * (N / MXT_ROWS) + nt) * (K / MXT_K) + kt;
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

// The same copy through a buffer resource (buffer_load_dwordx4 ... lds):
// lane i's 16 bytes from base + voff land at dst + 16 i.  Unlike the global
// form, the compiler counts these on the vector-memory counter alone, so LDS
// reads issued after them can still be waited for one by one.  Offsets are
// 32-bit: every byte a kernel reads this way lies within 4 GiB of base.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
__device__ __forceinline__ buf_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
}
__device__ __forceinline__ void b2lds16(buf_rsrc_t r, uint32_t voff, char* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)wave_dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void b2lds4(buf_rsrc_t r, uint32_t voff, char* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)wave_dst, 4, voff, 0, 0, 0);
}
// Cache-policy operand of the buffer stores: the device-scope bit (sc1) --
// the store is made coherent for every XCD (written through its L2).
constexpr int MK_CPOL_DEVICE = 16;

// A pointer that is the same in every lane of the wave, made visibly uniform
// (so that a buffer resource built from it stays in scalar registers).
__device__ __forceinline__ const void* wave_uniform(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

}  // namespace mk
