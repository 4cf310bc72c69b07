// Top-k softmax router.
//
// Logits are fp32 dot products accumulated in ascending h from +0 (one fused
// multiply-add per term; a bf16 x bf16 product is exact in fp32, so fma and
// multiply-then-add round the same), then + bias.  Fixing the order makes the
// logits, and with them the top-k decision, bit-identical to any other
// implementation that follows the same order.  An MFMA or tree reduction
// would not.
//
// Workgroup = one thread per expert (E rounded up to 64) x TT tokens; the x
// chunk is staged in LDS and broadcast, each thread streams its own router
// row.  Top-k then runs one wave per token: k rounds of a wave-wide
// (max logit, min id) reduction.
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {
namespace {

constexpr int TT = 8;      // tokens per workgroup
constexpr int HC = 64;     // h per LDS chunk

__device__ __forceinline__ bool better(float za, int ea, float zb, int eb) {
  return za > zb || (za == zb && ea < eb);
}

__global__ void route_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                             const float* __restrict__ bias, int T, int H, int E, int k, int renorm,
                             int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  extern __shared__ float zbuf[];                              // [TT][E]
  __shared__ __attribute__((aligned(16))) uint16_t xs[TT][HC];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int t0 = blockIdx.x * TT;
  const int e = tid;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  const uint16_t* wrow = w + (int64_t)min(e, E - 1) * H;
  for (int h0 = 0; h0 < H; h0 += HC) {
    __syncthreads();
    for (int g = tid; g < TT * HC / 8; g += nthr) {
      const int t = g / (HC / 8), c = g % (HC / 8);
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (t0 + t < T) v = *(const u32x4_t*)(x + (int64_t)(t0 + t) * H + h0 + c * 8);
      *(u32x4_t*)(&xs[t][c * 8]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < HC / 8; ++c) {
      const u32x4_t wv = *(const u32x4_t*)(wrow + h0 + c * 8);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const u32x4_t xv = *(const u32x4_t*)(&xs[t][c * 8]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[t] = __builtin_fmaf(bf16_to_f32(xv[d] & 0xFFFFu), bf16_to_f32(wv[d] & 0xFFFFu), acc[t]);
          acc[t] = __builtin_fmaf(bf16_to_f32(xv[d] >> 16), bf16_to_f32(wv[d] >> 16), acc[t]);
        }
      }
    }
  }
  if (e < E) {
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int t = 0; t < TT; ++t) zbuf[t * E + e] = bias ? acc[t] + b : acc[t];
  }
  __syncthreads();
  // top-k: one wave per token
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
  for (int t = wave; t < TT; t += nwaves) {
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
  const int threads = ((E + 63) / 64) * 64;
  const int blocks = (T + TT - 1) / TT;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(threads), TT * E * sizeof(float), s, x, w_router, bias, T,
                     H, E, k, renorm, idx, w);
}

}  // namespace mk
