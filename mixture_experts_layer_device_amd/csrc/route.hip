// Top-k softmax router.
//
// Logits are fp32 dot products accumulated in ascending h from +0 (one fused
// multiply-add per term; a bf16 x bf16 product is exact in fp32, so fma and
// multiply-then-add round the same), then + bias.  Fixing the order makes the
// logits, and with them the top-k decision, bit-identical to any other
// implementation that follows the same order.  An MFMA or tree reduction
// would not, so the parallelism comes from the (token, expert) pairs only.
//
// Workgroup = RT tokens x all experts, in chunks of RE experts.  x and the
// router rows are staged through LDS per RH-wide slice of h, converted to fp32
// once (x as [token][h], the router rows transposed to [h][expert]), double-
// buffered with the next slice's global loads in registers.  512 threads (two
// waves per SIMD, so one wave's LDS and barrier waits are covered by the
// other's FMAs); thread (tx, ty) keeps the chains of token ty x experts
// 4tx .. 4tx+3: per 8 h, two 16-byte x reads and eight 16-byte router reads
// (broadcast across the lanes that share them) feed 32 FMAs, read one group
// ahead.  Top-k
// then runs one wave per token over the logits kept in LDS: k rounds of a
// wave-wide (max logit, min id) reduction.  The LOGITS variant stops after
// the logits and stores them (the router backward needs the full softmax).
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {
namespace {

constexpr int RT = 16;     // tokens per workgroup
constexpr int RE = 128;    // experts per chunk
constexpr int RH = 64;     // h per LDS slice
constexpr int RNT = 512;   // threads
constexpr int TPT = RT * 32 / RNT;        // tokens per thread (32 threads span the RE experts)
constexpr int SQN = RH * 128 / RNT / 8;   // 8-h granules of a router row each thread stages

__device__ __forceinline__ bool better(float za, int ea, float zb, int eb) {
  return za > zb || (za == zb && ea < eb);
}

template <bool LOGITS>
__global__ __launch_bounds__(RNT) void route_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                    const float* __restrict__ bias, int T, int H, int E, int k,
                                                    int renorm, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out, float* __restrict__ z_out) {
  extern __shared__ float zbuf[];                                  // [RT][E]
  __shared__ __attribute__((aligned(16))) float xs[2][RT][RH];
  __shared__ __attribute__((aligned(16))) float ws[2][RH][RE];
  const int tid = threadIdx.x;
  const int tx = tid & 31, ty = tid >> 5;
  const int t0 = blockIdx.x * RT;
  // staging roles: router row e0 + (tid & 127), h part (tid >> 7) of the
  // slice (8 SQN h); threads 0..127 also stage token tid >> 3, h eighth (tid & 7)
  const int se = tid & 127, sh = (tid >> 7) * 8 * SQN;
  const int st_tok = tid >> 3, sq = (tid & 7) * 8;
  const bool x_stager = tid < 128 && t0 + st_tok < T;
  for (int e0 = 0; e0 < E; e0 += RE) {
    const bool w_valid = e0 + se < E;
    const uint16_t* wrow = w + (int64_t)(w_valid ? e0 + se : 0) * H + sh;
    const uint16_t* xrow = x + (int64_t)(x_stager ? t0 + st_tok : 0) * H + sq;
    u32x4_t wr[SQN], xr{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < SQN; ++q) wr[q] = u32x4_t{0u, 0u, 0u, 0u};
    auto load = [&](int h0) {
      if (w_valid) {
#pragma unroll
        for (int q = 0; q < SQN; ++q) wr[q] = *(const u32x4_t*)(wrow + h0 + 8 * q);
      }
      if (x_stager) xr = *(const u32x4_t*)(xrow + h0);
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int q = 0; q < SQN; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          ws[buf][sh + 8 * q + 2 * d][se] = bf16_to_f32(wr[q][d] & 0xFFFFu);
          ws[buf][sh + 8 * q + 2 * d + 1][se] = bf16_to_f32(wr[q][d] >> 16);
        }
      if (tid < 128) {
        f32x4_t lo, hi;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          lo[2 * d] = bf16_to_f32(xr[d] & 0xFFFFu);
          lo[2 * d + 1] = bf16_to_f32(xr[d] >> 16);
          hi[2 * d] = bf16_to_f32(xr[d + 2] & 0xFFFFu);
          hi[2 * d + 1] = bf16_to_f32(xr[d + 2] >> 16);
        }
        *(f32x4_t*)&xs[buf][st_tok][sq] = lo;
        *(f32x4_t*)&xs[buf][st_tok][sq + 4] = hi;
      }
    };
    float acc[TPT][4];
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    load(0);
    for (int h0 = 0, buf = 0; h0 < H; h0 += RH, buf ^= 1) {
      stage(buf);
      __syncthreads();
      if (h0 + RH < H) load(h0 + RH);
      // groups of 8 h, the next group's LDS reads issued before this group's
      // FMAs so their latency is covered; per group: 8 h of each of the
      // thread's 2 tokens (two 16-byte reads each) and 4 experts per h
      f32x4_t wa[8], wb[8];
      f32x4_t xa[TPT][2], xb[TPT][2];
      auto rdg = [&](int h, f32x4_t (&wv)[8], f32x4_t (&xv)[TPT][2]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) wv[u] = *(const f32x4_t*)&ws[buf][h + u][4 * tx];
#pragma unroll
        for (int i = 0; i < TPT; ++i)
#pragma unroll
          for (int q = 0; q < 2; ++q) xv[i][q] = *(const f32x4_t*)&xs[buf][TPT * ty + i][h + 4 * q];
      };
      auto fmg = [&](const f32x4_t (&wv)[8], const f32x4_t (&xv)[TPT][2]) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < TPT; ++i) acc[i][j] = __builtin_fmaf(xv[i][u / 4][u % 4], wv[u][j], acc[i][j]);
      };
      rdg(0, wa, xa);
#pragma unroll
      for (int h = 0; h < RH; h += 16) {
        rdg(h + 8, wb, xb);
        fmg(wa, xa);
        if (h + 16 < RH) rdg(h + 16, wa, xa);
        fmg(wb, xb);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 4 * tx + j;
      if (e < E) {
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const float z = bias ? acc[i][j] + b : acc[i][j];
          if (LOGITS) {
            if (t0 + TPT * ty + i < T) z_out[(int64_t)(t0 + TPT * ty + i) * E + e] = z;
          } else {
            zbuf[(TPT * ty + i) * E + e] = z;
          }
        }
      }
    }
    // the next chunk's first staging reuses the slice buffers
    __syncthreads();
  }
  if (LOGITS) return;
  // top-k: one wave per token
  const int lane = tid & 63, wave = tid >> 6, nwaves = RNT >> 6;
  for (int t = wave; t < RT; t += nwaves) {
    if (t0 + t >= T) break;
    const float* z = zbuf + t * E;
    uint32_t taken = 0;                       // bit i: expert lane + 64 i chosen
    float zsel0 = 0.f, zmax = -INFINITY;
    for (int i = 0; lane + 64 * i < E; ++i) zmax = fmaxf(zmax, z[lane + 64 * i]);
    for (int o = 32; o; o >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o));
    float wsum_sel = 0.f;
    float zs_j = 0.f;
    int es_j = 0;
    for (int j = 0; j < k; ++j) {
      float bz = -INFINITY;
      int be = 0x7FFFFFFF;
      for (int i = 0; lane + 64 * i < E; ++i) {
        const int ee = lane + 64 * i;
        if (!((taken >> i) & 1u) && better(z[ee], ee, bz, be)) {
          bz = z[ee];
          be = ee;
        }
      }
      for (int o = 32; o; o >>= 1) {
        const float oz = __shfl_xor(bz, o);
        const int oe = __shfl_xor(be, o);
        if (better(oz, oe, bz, be)) {
          bz = oz;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (j == 0) zsel0 = bz;
      if (lane == j) {
        zs_j = bz;
        es_j = be;
      }
      wsum_sel += expf(bz - zsel0);            // slot order, same on every lane
    }
    float denom;
    float ref;
    if (renorm) {
      denom = wsum_sel;
      ref = zsel0;
    } else {
      float s = 0.f;
      for (int i = 0; lane + 64 * i < E; ++i) s += expf(z[lane + 64 * i] - zmax);
      for (int o = 32; o; o >>= 1) s += __shfl_xor(s, o);
      denom = s;
      ref = zmax;
    }
    if (lane < k) {
      idx_out[(int64_t)(t0 + t) * k + lane] = es_j;
      w_out[(int64_t)(t0 + t) * k + lane] = expf(zs_j - ref) / denom;
    }
  }
}

}  // namespace

void launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H, int E, int k,
                  int renorm, int32_t* idx, float* w, hipStream_t s) {
  if (T <= 0) return;
  const int blocks = (T + RT - 1) / RT;
  hipLaunchKernelGGL(route_kernel<false>, dim3(blocks), dim3(RNT), RT * E * sizeof(float), s, x, w_router, bias, T,
                     H, E, k, renorm, idx, w, nullptr);
}

void launch_route_logits(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H, int E,
                         float* z, hipStream_t s) {
  if (T <= 0) return;
  const int blocks = (T + RT - 1) / RT;
  hipLaunchKernelGGL(route_kernel<true>, dim3(blocks), dim3(RNT), 0, s, x, w_router, bias, T, H, E, 0, 0, nullptr,
                     nullptr, z);
}

}  // namespace mk
