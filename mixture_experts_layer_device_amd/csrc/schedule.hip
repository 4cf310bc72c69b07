// Device-built dispatch schedule: three small launches, all sized from R and
// the minibatch size (host-known), never from per-expert counts.
//
//  count   (minibatch b, chunk c of 256 rows): per-chunk expert histogram in
//          LDS, stored by (b, e) column ([b][e][c], columns padded to a
//          multiple of 4 chunks), and a flag for a chunk holding an expert id
//          out of range; also marks every sorted position of the chunk's
//          range empty.
//  scan    (one workgroup): per (b, e) prefix over chunks, per-minibatch
//          expert offsets, global counts/offsets, the GEMM work items (one
//          per 256-row m-tile of each (b, e) run) with their offsets, and the
//          device error word (written whole: building a schedule clears it).
//  scatter (b, c): stable rank of each row among the earlier rows of its
//          chunk with the same expert; sorted_pos and its inverse.
//
// Integer work only, no float and no order-dependent atomics (the LDS
// histogram uses integer atomics, whose result is order independent), so the
// tables are bit-exact and repeatable.
#include "mk_device.h"
#include "mk_internal.h"

#include <algorithm>
#include <mutex>

namespace mk {
namespace {

constexpr int CH = MK_SCHED_CHUNK;

__global__ __launch_bounds__(CH) void sched_count_kernel(const int32_t* __restrict__ row_expert, int R, int E,
                                                         int MB, int cpm, int32_t* __restrict__ chunk_counts,
                                                         int32_t* __restrict__ chunk_bad,
                                                         int32_t* __restrict__ inv) {
  __shared__ int hist[MK_MAX_EXPERTS];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  for (int e = tid; e < E; e += CH) hist[e] = 0;
  __syncthreads();
  const int off = c * CH + tid;
  const int64_t p = (int64_t)b * MB + off;
  int bad = 0;
  if (off < MB) {
    inv[p] = -1;
    if (p < R) {
      const int e = row_expert[p];
      if (e >= 0 && e < E)
        atomicAdd(&hist[e], 1);
      else
        bad = 1;
    }
  }
  bad = __syncthreads_or(bad);
  const int cps = sched_cps(cpm);
  int32_t* out = chunk_counts + (int64_t)b * E * cps + c;
  for (int e = tid; e < E; e += CH) out[(int64_t)e * cps] = hist[e];
  if (tid == 0) chunk_bad[b * cpm + c] = bad;
}

constexpr int SCAN_T = 1024;

// Exclusive scan of one value per thread over the workgroup; *total gets the
// sum.  Each wave scans its 64 values with lane shuffles, the 16 wave totals
// are scanned by wave 0 through LDS.
__device__ int block_exclusive_scan(int v, int* sbuf, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sbuf[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int wt = lane < SCAN_T / 64 ? sbuf[lane] : 0;
    int wi = wt;
#pragma unroll
    for (int o = 1; o < SCAN_T / 64; o <<= 1) {
      const int t = __shfl_up(wi, o);
      if (lane >= o) wi += t;
    }
    if (lane < SCAN_T / 64) sbuf[SCAN_T / 64 + lane] = wi - wt;   // exclusive wave offsets
    if (lane == SCAN_T / 64 - 1) sbuf[2 * (SCAN_T / 64)] = wi;    // total
  }
  __syncthreads();
  const int ex = sbuf[SCAN_T / 64 + wave] + incl - v;
  *total = sbuf[2 * (SCAN_T / 64)];
  __syncthreads();
  return ex;
}

// (b, e) counts and offsets kept in LDS when nb * (E + 1) fits, so the
// later passes read them there instead of from global memory
constexpr int SCAN_LDS = 8192;

__global__ __launch_bounds__(SCAN_T) void sched_scan_kernel(int E, int MB, int nb, int cpm, int tile_m,
                                                            int item_cap, int32_t* __restrict__ chunk_counts,
                                                            int32_t* __restrict__ mb_counts,
                                                            int32_t* __restrict__ mb_offsets,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ items,
                                                            int32_t* __restrict__ mb_items,
                                                            const int32_t* __restrict__ chunk_bad,
                                                            uint32_t* __restrict__ err) {
  __shared__ int sbuf[SCAN_T];
  __shared__ int s_cnt[SCAN_LDS], s_off[SCAN_LDS];
  const int tid = threadIdx.x;
  const int nbe = nb * E;
  const bool in_lds = nb * (E + 1) <= SCAN_LDS;
  // reads of the (b, e) tables after they are written: LDS copies when they fit
  const int32_t* mbc = in_lds ? (const int32_t*)s_cnt : mb_counts;
  const int32_t* mbo = in_lds ? (const int32_t*)s_off : mb_offsets;
  // an expert id out of range in any chunk (reduced at the end, so these
  // loads overlap the chunk pass)
  int bad = 0;
  for (int i = tid; i < nb * cpm; i += SCAN_T) bad |= chunk_bad[i];
  // per (b, e): exclusive prefix over the chunks of minibatch b (in place).
  // SG consecutive lanes share one (b, e) column, each taking a contiguous
  // run of chunks that starts 16-byte aligned: the run's counts loaded four
  // at a time (kept in registers when the run is at most 16 chunks, else
  // summed in a first pass and re-read), a shuffle scan across the SG lanes,
  // then the prefixes stored four at a time (a group that reaches past the
  // column's last chunk writes only into the column's padding).
  {
    constexpr int SG = 8, RUN = 16;
    const int cps = sched_cps(cpm);
    const int sub = tid & (SG - 1);
    const int per = sched_cps((cpm + SG - 1) / SG);
    const int c_lo = min(cpm, sub * per), c_hi = min(cpm, c_lo + per);
    for (int be0 = 0; be0 < nbe; be0 += SCAN_T / SG) {
      const int be = be0 + tid / SG;
      const bool on = be < nbe;
      int32_t* cc = chunk_counts + (on ? (int64_t)be * cps : 0);
      // counts of chunks c .. c+3 (those at or past c_hi read as 0)
      auto load4 = [&](int c, int* v) {
        u32x4_t q{0u, 0u, 0u, 0u};
        if (c < c_hi) q = *(const u32x4_t*)(cc + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = c + j < c_hi ? (int)q[j] : 0;
      };
      auto store_prefix4 = [&](int c, const int* v, int& run) {
        if (c >= c_hi) return;
        u32x4_t o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[j] = (uint32_t)run;
          run += v[j];
        }
        *(u32x4_t*)(cc + c) = o;
      };
      int sum = 0;
      int v[RUN];
      if (per <= RUN) {
#pragma unroll
        for (int q = 0; q < RUN / 4; ++q) {
          if (on) {
            load4(c_lo + 4 * q, v + 4 * q);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * q + j] = 0;
          }
        }
#pragma unroll
        for (int i = 0; i < RUN; ++i) sum += v[i];
      } else if (on) {
        for (int c = c_lo; c < c_hi; c += RUN) {
#pragma unroll
          for (int q = 0; q < RUN / 4; ++q) load4(c + 4 * q, v + 4 * q);
#pragma unroll
          for (int i = 0; i < RUN; ++i) sum += v[i];
        }
      }
      // inclusive scan over the SG lanes of the group (groups never straddle a wave)
      int incl = sum;
#pragma unroll
      for (int o = 1; o < SG; o <<= 1) {
        const int t = __shfl_up(incl, o, SG);
        if (sub >= o) incl += t;
      }
      const int total = __shfl(incl, SG - 1, SG);
      if (on) {
        int run = incl - sum;
        if (per <= RUN) {
#pragma unroll
          for (int q = 0; q < RUN / 4; ++q) store_prefix4(c_lo + 4 * q, v + 4 * q, run);
        } else {
          for (int c = c_lo; c < c_hi; c += RUN) {
#pragma unroll
            for (int q = 0; q < RUN / 4; ++q) load4(c + 4 * q, v + 4 * q);
#pragma unroll
            for (int q = 0; q < RUN / 4; ++q) store_prefix4(c + 4 * q, v + 4 * q, run);
          }
        }
        if (sub == 0) {
          mb_counts[be] = total;
          if (in_lds) s_cnt[be] = total;
        }
      }
    }
  }
  __syncthreads();
  // per minibatch: exclusive scan over experts
  for (int b = 0; b < nb; ++b) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += SCAN_T) {
      const int e = e0 + tid;
      const int v = e < E ? mbc[b * E + e] : 0;
      int tot;
      const int ex = block_exclusive_scan(v, sbuf, &tot);
      if (e < E) {
        mb_offsets[b * (E + 1) + e] = carry + ex;
        if (in_lds) s_off[b * (E + 1) + e] = carry + ex;
      }
      carry += tot;
    }
    if (tid == 0) {
      mb_offsets[b * (E + 1) + E] = carry;
      if (in_lds) s_off[b * (E + 1) + E] = carry;
    }
  }
  // global per-expert counts and offsets
  {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += SCAN_T) {
      const int e = e0 + tid;
      int v = 0;
      if (e < E)
        for (int b = 0; b < nb; ++b) v += mbc[b * E + e];
      int tot;
      const int ex = block_exclusive_scan(v, sbuf, &tot);
      if (e < E) {
        counts[e] = v;
        offsets[e] = carry + ex;
      }
      carry += tot;
    }
    if (tid == 0) offsets[E] = carry;
  }
  __syncthreads();
  // work items, ordered (b, e, m)
  int carry = 0;
  for (int be0 = 0; be0 < nbe; be0 += SCAN_T) {
    const int be = be0 + tid;
    int cnt = 0, nm = 0;
    if (be < nbe) {
      cnt = mbc[be];
      nm = (cnt + tile_m - 1) / tile_m;
    }
    int tot;
    const int start = carry + block_exclusive_scan(nm, sbuf, &tot);
    if (be < nbe) {
      const int b = be / E, e = be - b * E;
      const int base = b * MB + mbo[b * (E + 1) + e];
      for (int m = 0; m < nm; ++m) {
        const int idx = start + m;
        if (idx < item_cap) {
          int32_t* it = items + 4 * (int64_t)idx;
          it[0] = base + m * tile_m;
          it[1] = min(tile_m, cnt - m * tile_m);
          it[2] = e;
          it[3] = b;
        }
      }
      if (e == 0) mb_items[b] = start;
    }
    carry += tot;
  }
  bad = __syncthreads_or(bad);
  if (tid == 0) {
    mb_items[nb] = carry;
    *err = (bad ? MK_DEVERR_EXPERT_RANGE : 0u) | (carry > item_cap ? MK_DEVERR_SCHED_OVERFLOW : 0u);
  }
}

__global__ __launch_bounds__(CH) void sched_scatter_kernel(const int32_t* __restrict__ row_expert, int R, int E,
                                                           int MB, int cpm,
                                                           const int32_t* __restrict__ chunk_base,
                                                           const int32_t* __restrict__ mb_offsets,
                                                           int32_t* __restrict__ sorted_pos,
                                                           int32_t* __restrict__ inv) {
  __shared__ int ex[CH];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int off = c * CH + tid;
  const int64_t r = (int64_t)b * MB + off;
  const bool live = off < MB && r < R;
  int e = -1;
  if (live) {
    e = row_expert[r];
    if (e < 0 || e >= E) e = -1;
  }
  ex[tid] = e;
  __syncthreads();
  if (e >= 0) {
    int rank = 0;
    for (int j = 0; j < tid; ++j) rank += (ex[j] == e);
    const int pos =
        b * MB + mb_offsets[b * (E + 1) + e] + chunk_base[((int64_t)b * E + e) * sched_cps(cpm) + c] + rank;
    sorted_pos[r] = pos;
    inv[pos] = (int32_t)r;
  } else if (live) {
    sorted_pos[r] = -1;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

void launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
}

void launch_schedule(const SchedDims& d, const SchedScratch& scr, const SchedTables& t, const int32_t* row_expert,
                     int32_t R, hipStream_t s) {
  const int MB = d.MB, E = d.E, cpm = d.cpm;
  const int nb = R > 0 ? (R + MB - 1) / MB : 0;
  if (nb > 0)
    hipLaunchKernelGGL(sched_count_kernel, dim3(cpm, nb), dim3(CH), 0, s, row_expert, R, E, MB, cpm,
                       scr.chunk_counts, scr.chunk_bad, t.inv);
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(SCAN_T), 0, s, E, MB, nb, cpm, MK_TILE_M, d.item_cap,
                     scr.chunk_counts, t.mb_counts, t.mb_offsets, t.counts, t.offsets, t.items, t.mb_items,
                     scr.chunk_bad, t.err);
  if (nb > 0)
    hipLaunchKernelGGL(sched_scatter_kernel, dim3(cpm, nb), dim3(CH), 0, s, row_expert, R, E, MB, cpm,
                       scr.chunk_counts, t.mb_offsets, t.sorted_pos, t.inv);
}

// ---- schedule build without allocation -------------------------------------
//
// The scratch of the build (per-chunk histograms and flags) in a file-scope
// device array instead of a workspace: for callers that cannot allocate.
// Every GPU the library runs on holds its own copy until the process ends;
// calls on one GPU share it, so calls that overlap on one GPU race.  Every
// element the build reads is written by the same call first (the count
// kernel writes the whole [nb, cpm, E] histogram block and the flags), so
// nothing has to start at zero.
namespace {

constexpr int64_t kStaticScratchBytes = (int64_t)4 << 20;       // 4 MiB
static __device__ __align__(256) int32_t scratch[kStaticScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of this GPU's scratch (looked up once per device, with
// that device current); null on failure.
int32_t* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = (int32_t*)ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace mk

extern "C" int mk_build_schedule_static(const int32_t* row_expert, int32_t R, int32_t E, int32_t MB,
                                        int32_t item_cap, int32_t* counts, int32_t* offsets, int32_t* mb_counts,
                                        int32_t* mb_offsets, int32_t* sorted_pos, int32_t* inv, int32_t* items,
                                        int32_t* mb_items, uint32_t* err, void* stream) {
  using namespace mk;
  if (R < 0 || MB < 1 || item_cap < 1) return MK_ERR_SHAPE;
  if (E < 1 || E > MK_MAX_EXPERTS) return MK_ERR_LIMIT;
  if (!counts || !offsets || !mb_items || !err || !items) return MK_ERR_NULL;
  const int64_t nb = R > 0 ? ((int64_t)R + MB - 1) / MB : 0;
  if (R > 0 && (!row_expert || !mb_counts || !mb_offsets || !sorted_pos || !inv)) return MK_ERR_NULL;
  if (nb > 65535) return MK_ERR_LIMIT;
  const int64_t cpm = ((int64_t)MB + MK_SCHED_CHUNK - 1) / MK_SCHED_CHUNK;
  // scratch: [nb, E, cps] chunk histograms, then [nb, cpm] chunk flags
  const int64_t cps = sched_cps((int32_t)cpm);
  const int64_t need = (nb * cps * E + nb * cpm) * 4;
  if (need > kStaticScratchBytes) return MK_ERR_LIMIT;
  int32_t* base = device_scratch();
  if (!base) return MK_ERR_HIP;
  SchedScratch scr{base, base + nb * cps * E};
  SchedTables t{err, mb_counts, mb_offsets, counts, offsets, sorted_pos, inv, items, mb_items};
  const SchedDims d{MB, E, (int32_t)cpm, item_cap};
  launch_schedule(d, scr, t, row_expert, R, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_ERR_HIP;
}
