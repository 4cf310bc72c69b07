// Top-k softmax router.
//
// Logits are fp32 dot products accumulated in ascending h from +0 (one fused
// multiply-add per term; a bf16 x bf16 product is exact in fp32, so fma and
// multiply-then-add round the same), then + bias.  Fixing the order makes the
// logits, and with them the top-k decision, bit-identical to any other
// implementation that follows the same order.  An MFMA or tree reduction
// would not, so the parallelism comes from the (token, expert) pairs only.
//
// Workgroup = RT = 16 tokens x all experts, in chunks of RE = 128 experts,
// sixteen waves (four per SIMD, so the waves' LDS, load and barrier waits
// are covered by the others' multiply-adds, and the DPP multiply-adds issue
// closer to their peak rate).  Lane l of a wave keeps the chains of token
// l mod 16 and the two experts of group 4 * wave + l / 16 (16-lane row r of
// wave w: experts 2 (4w + r), +1).  x and the router rows are staged through
// LDS per 128-wide slice of h (64-wide when E > 128, so the logits of all
// experts fit beside the slices) as fp32, double-buffered, with each slice's
// global loads issued two slices ahead into registers.  The router weights
// sit in LDS as [h / 8][expert][h mod 8], so one 4-byte read per lane brings
// a row its 16 values (2 experts x 8 h), and each multiply-add takes its
// weight from lane 8e + (h mod 8) of its row by a DPP row broadcast
// (row_newbcast) folded into v_fmac_f32: every LDS weight read feeds 16
// multiply-adds, which keeps the kernel off the LDS bandwidth bound.  Top-k
// then runs one wave per token over the logits kept in LDS: k rounds of a
// wave-wide (max logit, min id) reduction.  The LOGITS variant stops after
// the logits and stores them (the router backward needs the full softmax).
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {
namespace {

constexpr int RT = 16;     // tokens per workgroup
constexpr int RE = 128;    // experts per chunk (64 groups of 2, one per 16-lane row)
constexpr int RNT = 1024;  // threads (16 waves)
// h per LDS slice: 128 where the slice buffers and the [RT][E] logits fit
// the LDS together (E <= 128), else 64
constexpr int RH_WIDE = 128, RH_NARROW = 64;

// acc[e] += w(lane 8e + j of the row) * x_j for eight consecutive h (x0 ..
// x7 = xa, xb), in ascending h for every chain.  v_fmac_f32 rounds once (a
// fused multiply-add) like __builtin_fmaf.  The compiler's hazard checks do
// not see into the asm, so it opens with 5 wait states: a DPP source written
// by the VALU needs 2, an EXEC written by the VALU 5.
#define MK_FMAC(d, w, x, n) "v_fmac_f32_dpp %" #d ", %" #w ", %" #x " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"
__device__ __forceinline__ void fmac_group8(float (&acc)[2], float wv, f32x4_t xa, f32x4_t xb) {
  asm("s_nop 4\n"
      MK_FMAC(0, 2, 3, 0) MK_FMAC(1, 2, 3, 8) MK_FMAC(0, 2, 4, 1) MK_FMAC(1, 2, 4, 9)
      MK_FMAC(0, 2, 5, 2) MK_FMAC(1, 2, 5, 10) MK_FMAC(0, 2, 6, 3) MK_FMAC(1, 2, 6, 11)
      MK_FMAC(0, 2, 7, 4) MK_FMAC(1, 2, 7, 12) MK_FMAC(0, 2, 8, 5) MK_FMAC(1, 2, 8, 13)
      MK_FMAC(0, 2, 9, 6) MK_FMAC(1, 2, 9, 14) MK_FMAC(0, 2, 10, 7) MK_FMAC(1, 2, 10, 15)
      : "+v"(acc[0]), "+v"(acc[1])
      : "v"(wv), "v"(xa[0]), "v"(xa[1]), "v"(xa[2]), "v"(xa[3]), "v"(xb[0]), "v"(xb[1]), "v"(xb[2]), "v"(xb[3]));
}
#undef MK_FMAC

__device__ __forceinline__ bool better(float za, int ea, float zb, int eb) {
  return za > zb || (za == zb && ea < eb);
}

template <bool LOGITS, int RH>
__global__ __launch_bounds__(RNT) void route_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                    const float* __restrict__ bias, int T, int H, int E, int k,
                                                    int renorm, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out, float* __restrict__ z_out) {
  extern __shared__ float zbuf[];                                  // [RT][E]
  __shared__ __attribute__((aligned(16))) float ws[2][RH / 8][RE][8];
  constexpr int XS = RH + 4;   // floats per staged x row (the pad spreads a row's 16 tokens over the banks)
  constexpr int WQ = RH / 64;  // 8-h loads per thread and slice of a router row
  constexpr int XT = 2 * RH;   // threads staging x (8 h each)
  __shared__ __attribute__((aligned(16))) float xs[2][RT][XS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, tok = lane & 15, rl = lane & 15;
  const int grp = (tid >> 6) * 4 + (lane >> 4);                   // expert group of this lane's row
  const int t0 = blockIdx.x * RT;
  // staging roles: router row e0 + (tid & 127), h eighth (tid >> 7) of the
  // slice (WQ loads of 8 h); threads 0 .. XT-1 also stage token
  // tid / (RH / 8), h granule tid mod (RH / 8)
  const int se = tid & 127, sh = (tid >> 7) * (RH / 8);
  const int st_tok = tid / (RH / 8), sq = (tid % (RH / 8)) * 8;
  const bool x_stager = tid < XT && t0 + st_tok < T;
  for (int e0 = 0; e0 < E; e0 += RE) {
    const bool w_valid = e0 + se < E;
    const uint16_t* wrow = w + (int64_t)(w_valid ? e0 + se : 0) * H + sh;
    const uint16_t* xrow = x + (int64_t)(x_stager ? t0 + st_tok : 0) * H + sq;
    // two register sets: slice s's global loads are issued two slices ahead
    u32x4_t wr[2][WQ], xr[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      xr[r] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < WQ; ++q) wr[r][q] = u32x4_t{0u, 0u, 0u, 0u};
    }
    auto load = [&](int h0, int r) {
      if (w_valid) {
#pragma unroll
        for (int q = 0; q < WQ; ++q) wr[r][q] = *(const u32x4_t*)(wrow + h0 + 8 * q);
      }
      if (x_stager) xr[r] = *(const u32x4_t*)(xrow + h0);
    };
    // bf16 pair (h even, h odd) in one dword -> fp32 (d << 16, d & 0xFFFF0000);
    // register set r goes to LDS buffer r
    auto stage = [&](int r) {
#pragma unroll
      for (int q = 0; q < WQ; ++q)
#pragma unroll
        for (int d = 0; d < 4; d += 2) {
          f32x4_t v;
          v[0] = bf16_to_f32(wr[r][q][d] & 0xFFFFu);
          v[1] = bf16_to_f32(wr[r][q][d] >> 16);
          v[2] = bf16_to_f32(wr[r][q][d + 1] & 0xFFFFu);
          v[3] = bf16_to_f32(wr[r][q][d + 1] >> 16);
          *(f32x4_t*)&ws[r][sh / 8 + q][se][2 * d] = v;
        }
      if (tid < XT) {
        f32x4_t lo, hi;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          lo[2 * d] = bf16_to_f32(xr[r][d] & 0xFFFFu);
          lo[2 * d + 1] = bf16_to_f32(xr[r][d] >> 16);
          hi[2 * d] = bf16_to_f32(xr[r][d + 2] & 0xFFFFu);
          hi[2 * d + 1] = bf16_to_f32(xr[r][d + 2] >> 16);
        }
        *(f32x4_t*)&xs[r][st_tok][sq] = lo;
        *(f32x4_t*)&xs[r][st_tok][sq + 4] = hi;
      }
    };
    float acc[2] = {0.f, 0.f};
    // groups of 8 h, the next group's LDS reads issued before this group's
    // multiply-adds: per group one 4-byte weight read (2 experts x 8 h) and
    // two 16-byte x reads
    auto compute = [&](int buf) {
      const float* wl = &ws[buf][0][2 * grp][0] + rl;
      const float* xl = &xs[buf][tok][0];
      float wv = wl[0];
      f32x4_t xa = *(const f32x4_t*)xl, xb = *(const f32x4_t*)(xl + 4);
#pragma unroll
      for (int h = 0; h < RH; h += 8) {
        float nw = 0.f;
        f32x4_t nxa{0.f, 0.f, 0.f, 0.f}, nxb{0.f, 0.f, 0.f, 0.f};
        if (h + 8 < RH) {
          nw = wl[(h + 8) / 8 * RE * 8];
          nxa = *(const f32x4_t*)(xl + h + 8);
          nxb = *(const f32x4_t*)(xl + h + 12);
        }
        fmac_group8(acc, wv, xa, xb);
        wv = nw;
        xa = nxa;
        xb = nxb;
      }
    };
    // H is a multiple of 2 * RH: slices in pairs, even ones through register
    // set and LDS buffer 0, odd ones through 1
    load(0, 0);
    load(RH, 1);
    for (int h0 = 0; h0 < H; h0 += 2 * RH) {
      stage(0);
      __syncthreads();
      if (h0 + 2 * RH < H) load(h0 + 2 * RH, 0);
      compute(0);
      stage(1);
      __syncthreads();
      if (h0 + 3 * RH < H) load(h0 + 3 * RH, 1);
      compute(1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + 2 * grp + j;
      if (e < E) {
        const float z = bias ? acc[j] + bias[e] : acc[j];
        if (LOGITS) {
          if (t0 + tok < T) z_out[(int64_t)(t0 + tok) * E + e] = z;
        } else {
          zbuf[tok * E + e] = z;
        }
      }
    }
    // the next chunk's first staging reuses the slice buffers
    __syncthreads();
  }
  if (LOGITS) return;
  // top-k: one wave per token
  const int wave = tid >> 6, nwaves = RNT >> 6;
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
  if (E <= RE)
    hipLaunchKernelGGL((route_kernel<false, RH_WIDE>), dim3(blocks), dim3(RNT), RT * E * sizeof(float), s, x,
                       w_router, bias, T, H, E, k, renorm, idx, w, nullptr);
  else
    hipLaunchKernelGGL((route_kernel<false, RH_NARROW>), dim3(blocks), dim3(RNT), RT * E * sizeof(float), s, x,
                       w_router, bias, T, H, E, k, renorm, idx, w, nullptr);
}

void launch_route_logits(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H, int E,
                         float* z, hipStream_t s) {
  if (T <= 0) return;
  const int blocks = (T + RT - 1) / RT;
  hipLaunchKernelGGL((route_kernel<true, RH_WIDE>), dim3(blocks), dim3(RNT), 0, s, x, w_router, bias, T, H, E, 0, 0,
                     nullptr, nullptr, z);
}

}  // namespace mk
