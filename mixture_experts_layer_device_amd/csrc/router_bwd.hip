// Full-layer backward past the experts: the k-sum of each token's dX rows and
// the gradient through the softmax top-k router.
//
// The choice of experts is piecewise constant in the logits and carries no
// gradient; the weights are a softmax, so the gradient w.r.t. the logits is
// the softmax Jacobian applied to the gradient w.r.t. the weights:
//   renorm 1 (softmax over the k chosen): dz[idx_j] = w_j (dw_j - S), other
//            experts 0, S = sum_j w_j dw_j;
//   renorm 0 (softmax p over all E, read at the chosen experts):
//            dz[e] = p_e (g_e - S), g_e = dw_j if e = idx_j else 0.
// Through the linear logit map z = x W_r^T + b: dW_r = dz^T x, d_bias =
// sum_t dz, and dX gains dz W_r before its single rounding to bf16.
//
// All sums run in a fixed order (j ascending, e ascending, t ascending), so
// every output is bitwise repeatable.  Zero entries of dz add nothing and are
// skipped (renorm 1 has k nonzeros per token).
#include "mk_device.h"
#include "mk_internal.h"

#include <algorithm>

namespace mk {
namespace {

constexpr int RT = 256;

__device__ __forceinline__ int64_t wave_id() { return ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; }
__device__ __forceinline__ int64_t wave_count() { return ((int64_t)gridDim.x * blockDim.x) >> 6; }

// One wave per token.  Lane j < k holds slot j's weight, weight gradient and
// expert id; lanes then walk the E experts 64 at a time.
__global__ __launch_bounds__(RT) void router_dz_kernel(const float* __restrict__ d_w, const float* __restrict__ w,
                                                       const int32_t* __restrict__ idx, int T, int E, int k,
                                                       int renorm, float* __restrict__ dz) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = wave_id(); t < T; t += wave_count()) {
    const float dwj = lane < k ? d_w[t * k + lane] : 0.f;
    const float wj = lane < k ? w[t * k + lane] : 0.f;
    const int ej = lane < k ? idx[t * k + lane] : -1;
    float S = 0.f;
    for (int j = 0; j < k; ++j) S += __shfl(wj, j) * __shfl(dwj, j);
    float* row = dz + t * E;
    if (renorm) {
      for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        float v = 0.f;
        for (int j = 0; j < k; ++j) {
          const int ejj = __shfl(ej, j);
          const float wjj = __shfl(wj, j), dwjj = __shfl(dwj, j);
          if (ejj == e) v = wjj * (dwjj - S);
        }
        if (e < E) row[e] = v;
      }
    } else {
      // p from the logits in the row, as the forward router forms it
      float zmax = -INFINITY;
      for (int e = lane; e < E; e += 64) zmax = fmaxf(zmax, row[e]);
      for (int o = 32; o; o >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o));
      float sum = 0.f;
      for (int e = lane; e < E; e += 64) sum += expf(row[e] - zmax);
      for (int o = 32; o; o >>= 1) sum += __shfl_xor(sum, o);
      for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        float g = 0.f;
        for (int j = 0; j < k; ++j) {
          const int ejj = __shfl(ej, j);
          const float dwjj = __shfl(dwj, j);
          if (ejj == e) g = dwjj;
        }
        if (e < E) row[e] = expf(row[e] - zmax) / sum * (g - S);
      }
    }
  }
}

// One wave per token; lane l takes columns 4l .. 4l+3 of each 256-column
// chunk (one 16-byte load per routed row, a wave reading 1 KiB contiguous),
// two chunks at a time.  Row terms in batches of 8 loads in flight, then the
// router terms: the nonzero dz of each group of 64 experts (a ballot), again
// 8 rows of W_r in flight per batch.
__global__ __launch_bounds__(RT) void dx_combine_kernel(const float* __restrict__ dx32, int64_t H,
                                                        const int32_t* __restrict__ sorted_pos, int k, int64_t T,
                                                        const float* __restrict__ dz,
                                                        const uint16_t* __restrict__ wr, int E,
                                                        uint16_t* __restrict__ dX) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = wave_id(); t < T; t += wave_count()) {
    const int pj = lane < k ? sorted_pos[t * k + lane] : -1;
    for (int64_t c0 = 0; c0 < H; c0 += 2 * 256) {
      const bool act1 = c0 + 256 < H;
      float acc[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[h][q] = 0.f;
      for (int j0 = 0; j0 < k; j0 += 8) {
        f32x4_t v[8][2];
        bool live[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = j0 + u;
          const int pos = __shfl(pj, j < k ? j : 0);
          live[u] = j < k && pos >= 0;
          if (live[u]) {
            const float* src = dx32 + (int64_t)pos * H + c0 + lane * 4;
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
            for (int q = 0; q < 4; ++q) acc[h][q] += v[u][h][q];
        }
      }
      if (dz) {
        for (int e0 = 0; e0 < E; e0 += 64) {
          const float dzl = e0 + lane < E ? dz[t * E + e0 + lane] : 0.f;
          uint64_t m = __ballot(dzl != 0.f);
          while (m) {
            float c[8];
            int e[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              if (m) {
                const int b = __ffsll((unsigned long long)m) - 1;
                m &= m - 1;
                c[u] = __shfl(dzl, b);
                e[u] = e0 + b;
              } else {
                c[u] = 0.f;
                e[u] = -1;
              }
            }
            u32x2_t wv[8][2];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (e[u] >= 0) {
                const uint16_t* wrow = wr + (int64_t)e[u] * H + c0 + lane * 4;
                wv[u][0] = *(const u32x2_t*)wrow;
                wv[u][1] = act1 ? *(const u32x2_t*)(wrow + 256) : u32x2_t{0u, 0u};
              }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              if (e[u] < 0) continue;
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                  acc[h][2 * d] += c[u] * bf16_to_f32(wv[u][h][d] & 0xFFFFu);
                  acc[h][2 * d + 1] += c[u] * bf16_to_f32(wv[u][h][d] >> 16);
                }
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !act1) break;
        u32x2_t ov;
        ov[0] = pack_bf16x2(acc[h][0], acc[h][1]);
        ov[1] = pack_bf16x2(acc[h][2], acc[h][3]);
        __builtin_nontemporal_store(ov, (u32x2_t*)(dX + t * H + c0 + h * 256 + lane * 4));
      }
    }
  }
}

// dW_r = dz^T x as a reduction over tokens, split for parallelism: workgroup
// (e, 1024-column slice of h, token split s); its wave w takes token range
// 4s + w of 4*NS equal ranges, lane 16 consecutive columns.  A wave walks its
// tokens 64 at a time, takes the nonzero dz[t, e] by ballot and adds
// dz * x[t] in ascending t with 8 rows of x in flight.  The 4 wave partials
// are added in wave order through LDS and stored as split s's partial; a
// second kernel adds the NS partials in ascending s.  Fixed order throughout.
constexpr int WG_COLS = 1024;
__global__ __launch_bounds__(RT) void router_wgrad_part_kernel(const float* __restrict__ dz,
                                                               const uint16_t* __restrict__ x, int T, int H,
                                                               int E, int NS, float* __restrict__ part,
                                                               float* __restrict__ part_b) {
  __shared__ __attribute__((aligned(16))) float red[4][WG_COLS];
  __shared__ float redb[4];
  const int e = blockIdx.x, s = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y * WG_COLS + lane * 16;
  const bool act = h < H;
  const int nr = 4 * NS, ri = 4 * s + wave;
  const int tb = (int)((int64_t)T * ri / nr), te = (int)((int64_t)T * (ri + 1) / nr);
  float acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  float bsum = 0.f;
  for (int t0 = tb; t0 < te; t0 += 64) {
    const float dzl = t0 + lane < te ? dz[(int64_t)(t0 + lane) * E + e] : 0.f;
    uint64_t m = __ballot(dzl != 0.f);
    while (m) {
      float c[8];
      int tt[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (m) {
          const int b = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          c[u] = __shfl(dzl, b);
          tt[u] = t0 + b;
        } else {
          c[u] = 0.f;
          tt[u] = -1;
        }
      }
      u32x4_t xv[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (act && tt[u] >= 0) {
          const u32x4_t* src = (const u32x4_t*)(x + (int64_t)tt[u] * H + h);
          xv[u][0] = src[0];
          xv[u][1] = src[1];
        }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (tt[u] < 0) continue;
        bsum += c[u];
        if (!act) continue;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            acc[8 * q + 2 * d] += c[u] * bf16_to_f32(xv[u][q][d] & 0xFFFFu);
            acc[8 * q + 2 * d + 1] += c[u] * bf16_to_f32(xv[u][q][d] >> 16);
          }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 16; q += 4)
    *(f32x4_t*)&red[wave][lane * 16 + q] = f32x4_t{acc[q], acc[q + 1], acc[q + 2], acc[q + 3]};
  if (lane == 0) redb[wave] = bsum;
  __syncthreads();
  // thread i adds column i of the 4 wave partials (4 columns per thread)
  float* dst = part + ((int64_t)s * E + e) * H + blockIdx.y * WG_COLS;
  for (int c = threadIdx.x; c < WG_COLS; c += RT) {
    if (blockIdx.y * WG_COLS + c >= H) break;
    dst[c] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) part_b[(int64_t)s * E + e] = ((redb[0] + redb[1]) + redb[2]) + redb[3];
}

// dW[e, h] = sum over s ascending of part[s, e, h]; d_bias likewise.
__global__ __launch_bounds__(RT) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ part_b, int H, int E,
                                                              int NS, float* __restrict__ dW,
                                                              float* __restrict__ d_bias) {
  const int64_t n4 = (int64_t)E * H / 4;
  for (int64_t i = (int64_t)blockIdx.x * RT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * RT) {
    f32x4_t a = ((const f32x4_t*)part)[i];
    for (int s = 1; s < NS; ++s) {
      const f32x4_t b = ((const f32x4_t*)(part + (int64_t)s * E * H))[i];
      a += b;
    }
    ((f32x4_t*)dW)[i] = a;
  }
  if (d_bias && blockIdx.x == 0)
    for (int e = threadIdx.x; e < E; e += RT) {
      float b = part_b[e];
      for (int s = 1; s < NS; ++s) b += part_b[(int64_t)s * E + e];
      d_bias[e] = b;
    }
}

int row_blocks(int64_t waves, int cap) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((waves + RT / 64 - 1) / (RT / 64), cap));
}

}  // namespace

void launch_router_dz(const float* d_w, const float* w, const int32_t* idx, int T, int E, int k, int renorm,
                      float* dz, hipStream_t s) {
  if (T <= 0) return;
  hipLaunchKernelGGL(router_dz_kernel, dim3(row_blocks(T, 4096)), dim3(RT), 0, s, d_w, w, idx, T, E, k, renorm, dz);
}

void launch_dx_combine(const float* dx32, int64_t H, const int32_t* sorted_pos, int k, int64_t T, const float* dz,
                       const uint16_t* w_router, int E, uint16_t* dX, int n_cu, hipStream_t s) {
  if (T <= 0) return;
  hipLaunchKernelGGL(dx_combine_kernel, dim3(row_blocks(T, 8 * n_cu)), dim3(RT), 0, s, dx32, H, sorted_pos, k, T,
                     dz, w_router, E, dX);
}

int router_wgrad_splits(int T, int E, int H, int max_splits) {
  // ~256 tokens per split (64 per wave), at most max_splits
  return std::max(1, std::min(max_splits, (T + 255) / 256));
}

void launch_router_wgrad(const float* dz, const uint16_t* x, int T, int H, int E, int NS, float* part,
                         float* dW_router, float* d_bias, hipStream_t s) {
  hipLaunchKernelGGL(router_wgrad_part_kernel, dim3(E, (H + WG_COLS - 1) / WG_COLS, NS), dim3(RT), 0, s, dz, x, T,
                     H, E, NS, part, part + (int64_t)NS * E * H);
  const int64_t n4 = (int64_t)E * H / 4;
  hipLaunchKernelGGL(router_wgrad_sum_kernel, dim3((unsigned)std::min<int64_t>((n4 + RT - 1) / RT, 2048)), dim3(RT),
                     0, s, part, part + (int64_t)NS * E * H, H, E, NS, dW_router, d_bias);
}

}  // namespace mk
