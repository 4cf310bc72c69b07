// Expert-grouped bf16 GEMMs on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Every GEMM here is a persistent grid (one 512-thread workgroup per compute
// unit, 132 KiB of LDS) that walks the device-side work table built by the
// schedule: an item is (first sorted row, rows, expert, minibatch) and each
// item is cut into 256-column tiles.  Tile counts are read on the device, so
// the host never learns per-expert counts.  Each 256x256 output tile is
// computed by one workgroup with a fixed K order, so results do not depend
// on which workgroup takes which tile (bitwise repeatable).
//
// Mainloop: K in steps of 64; A and B tiles (256 x 64 bf16 each) go global ->
// LDS with the asynchronous LDS-DMA loads (XOR-swizzled 16-byte granules),
// double-buffered so the next step's loads overlap this step's MFMAs.  8 waves
// as 2 (M) x 4 (N); a wave owns 128 x 64 outputs = 8 x 4 MFMA 16x16 fragments.
// Epilogues stage their bf16 results through LDS and store whole rows with
// 16-byte stores.
//
// Fragment layouts (measured on gfx950): A/B lane l holds row/col l%16 and
// k = 8*(l/16) .. +7; the 16x16 fp32 result in lane l is column l%16, rows
// 4*(l/16) .. +3.
#include <type_traits>

#include "gemm_common.h"
#include "rows_common.h"

namespace mk {
namespace {

constexpr int BM = G_BM, BN = G_BN, BK = 64, NT = G_NT;
constexpr int FM = G_FM, FN = G_FN;
constexpr int TILE_BYTES = BM * BK * 2;        // 32 KiB per operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES > STAGE_LDS_BYTES ? 2 * STAGE_BYTES : STAGE_LDS_BYTES;
// the K loop with B in three buffers: A in two, B in three (all 160 KiB of the LDS)
constexpr int NT_A_BUFS = 2, NT_B_BUFS = 3;
constexpr int NT3_LDS_BYTES = (NT_A_BUFS + NT_B_BUFS) * TILE_BYTES;
static_assert(NT3_LDS_BYTES >= STAGE_LDS_BYTES && NT3_LDS_BYTES <= 160 * 1024, "the LDS of one compute unit");
// GEMM1 over ring rows takes the three-buffer K loop for long contractions
// (measured slower at K = 2048); GEMM2, dA' and dX from K = 512 (measured
// faster or the same at K = 768 to 7168)
constexpr int NT3_MIN_K = 4096;
constexpr int NT3_MIN_K_L2A = 512;

typedef GAcc Acc;

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// LDS offset of granule g of tile row r in the NT GEMMs' stages: the tkey
// swizzle (the tiled B layout's).
struct SwzT {
  __device__ static int off(int r, int g) { return r * 128 + (((g ^ tkey(r)) & 7) << 4); }
};

// A stage is consumed in 8 groups of 8 MFMAs: group q takes A fragments
// 2(q & 3) and 2(q & 3) + 1 of k half q >> 2 against that half's 4 B
// fragments.
__device__ __forceinline__ void read_a_pair(const char* st, int q, bf16x8_t (&a)[2]) {
  const int lane = threadIdx.x & 63, wm = threadIdx.x >> 8;
  const int g = (q >> 2) * 4 + (lane >> 4);
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
    a[ii] = *(const bf16x8_t*)(st + SwzT::off(wm * 128 + (2 * (q & 3) + ii) * 16 + (lane & 15), g));
}
// NB: rows of the B tile (256, or 128 for a half tile): a wave's NB / 4
// columns are NB / 64 fragments.
// (bt: the B tile's buffer)
template <int NB = BN>
__device__ __forceinline__ void read_b_half(const char* bt, int ks, bf16x8_t (&b)[NB / 64]) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 3;
  const int g = ks * 4 + (lane >> 4);
#pragma unroll
  for (int j = 0; j < NB / 64; ++j)
    b[j] = *(const bf16x8_t*)(bt + SwzT::off(wn * (NB / 4) + j * 16 + (lane & 15), g));
}

// s_waitcnt: vmcnt(n) and lgkmcnt(0) (expcnt not waited for), n < 16.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4));
}
// The workgroup barrier with no memory fence of its own: the caller has
// already waited for exactly what must be complete (its share of one
// stage's LDS-DMA copies, and its LDS reads), where __syncthreads() would
// add a fence that waits for every LDS write in flight -- the later
// stage's copies included.  The clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }
template <int NB = BN>
__device__ __forceinline__ void mma_group(const bf16x8_t (&a)[2], const bf16x8_t (&b)[NB / 64], int pair, Acc& acc) {
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int j = 0; j < NB / 64; ++j)
      acc[2 * pair + ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ii], b[j], acc[2 * pair + ii][j], 0, 0, 0);
}

// C[256 x 256] = A[256 x K] * B[256 x K]^T.  arow(r) returns a pointer to
// element 0 of A tile row r (K-contiguous rows); B comes in the tiled layout,
// btile pointing at this tile's K / 64 blocks, each the LDS image of one
// stage's B slice.  Tiles go global -> LDS directly (no staging registers):
// wave w fills rows 32w .. 32w+31 of each operand, 8 rows (1 KiB) per
// instruction; for A each lane reads the granule that the swizzle puts in its
// slot, for B the copy is 1 KiB contiguous.  NB = 128 (a half tile): btile
// points at rows 128h .. 128h+127 of each block (h * 8192 elements in), each
// wave copies its 2 KiB, and only fragments j < 2 of acc are computed.
// mainloop_nt3 (B3 below) keeps A in two buffers (stage kt in A buffer
// kt mod 2) and B in three (kt mod 3),
// so while stage kt is multiplied, A of kt+1 and B of kt+1 and kt+2 are in
// flight: the B tiles (the weights, streamed from memory with little reuse)
// get two stages of latency to arrive instead of one.  The waits count this
// wave's copies (vmcnt: A of kt+1 was issued before B of kt+2), and the
// barriers carry no fence of their own (barrier_no_fence).
// rows: the tile's rows that hold data (1 .. 256).  With 128 or fewer, the
// four waves of rows 128 .. 255 hold only padding: they copy their share of
// B (which the other waves read) but no A rows, read no fragments, issue no
// MFMAs (their acc stays zero) and only keep step at the barriers.
template <int NB, typename ARow>
__device__ __forceinline__ void mainloop_nt3(const void* abase, ARow arow, const uint16_t* btile, int K, int rows,
                                            char* lds, Acc& acc) {
  constexpr int LB = NB / 64;                            // B copies per wave and stage
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // A rows and the B blocks through buffer resources: A offsets from abase
  // (every row arow returns lies within 4 GiB after it), B from btile
  const buf_rsrc_t ra = make_rsrc(wave_uniform(abase)), rb = make_rsrc(wave_uniform(btile));
  char* const abuf = lds;
  char* const bbuf = lds + NT_A_BUFS * TILE_BYTES;
  const int wbase = wave * 4096;
  const int bwbase = wave * NB * 16;                   // this wave's share of the B tile (NB rows x 128 B)
  const uint32_t bo = bwbase + lane * 16;
  auto a_of = [&](int kt) { return abuf + (kt & 1) * TILE_BYTES; };
  auto b_of = [&](int kt) { return bbuf + (kt % NT_B_BUFS) * TILE_BYTES; };
  auto issue_b = [&](int kt) {
    const uint32_t b = bo + (uint32_t)kt * TILE_BYTES;
    char* bt = b_of(kt);
#pragma unroll
    for (int j = 0; j < LB; ++j) b2lds16(rb, b + j * 1024, bt + bwbase + j * 1024);
  };
  zero_acc(acc);
  const int KT = K / BK;
  if (wave >= 4 && rows <= 128) {
    // a padding wave: its B copies and the barriers, one per stage as below
    issue_b(0);
    if (KT > 1) issue_b(1);
    if (KT > 1)
      wait_vm_lgkm0<LB>();
    else
      wait_vm_lgkm0<0>();
    barrier_no_fence();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 2 < KT) {
        issue_b(kt + 2);
        wait_vm_lgkm0<LB>();
      } else {
        wait_vm_lgkm0<0>();
      }
      barrier_no_fence();
    }
    return;
  }
  uint32_t ao[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + j * 8 + (lane >> 3);
    ao[j] = (uint32_t)((const char*)arow(r) - (const char*)abase) + (((lane & 7) ^ tkey(r)) & 7) * 16;
  }
  auto issue_a = [&](int kt) {
    const uint32_t ka = (uint32_t)kt * (BK * 2);
    char* at = a_of(kt);
#pragma unroll
    for (int j = 0; j < 4; ++j) b2lds16(ra, ao[j] + ka, at + wbase + j * 1024);
  };
  // stage 0's A and B, and B of stage 1; wait for stage 0
  issue_a(0);
  issue_b(0);
  if (KT > 1) issue_b(1);
  if (KT > 1)
    wait_vm_lgkm0<LB>();
  else
    wait_vm_lgkm0<0>();
  barrier_no_fence();
  // Fragments are read one group ahead of the MFMAs that use them (the
  // compiler, left alone, reuses one pair of registers and waits for every
  // read).  The stage's barrier sits before its last group, so the first
  // reads of the next stage are in flight while that group's MFMAs issue.
  // Scheduling barriers keep each group's reads ahead of the MFMAs before it.
  bf16x8_t bq[2][NB / 64], aq[2][2];
  read_b_half<NB>(b_of(0), 0, bq[0]);
  read_a_pair(a_of(0), 0, aq[0]);
  // Stage kt.  IB (the loop body: stage kt+2 exists): B of kt+2 is issued
  // now and the wait at the end leaves its LB copies in flight, a constant
  // wait that keeps the loop free of branches around it (so the compiler
  // adds no waits of its own).  The last two stages (no B left to issue)
  // wait for everything; whether stage kt+1 exists is then tested at run time.
  auto stage = [&](int kt, auto ib_c) {
    constexpr bool IB = decltype(ib_c)::value;
    const bool ia = IB || kt + 1 < KT;
    const char* at = a_of(kt);
    const char* bt = b_of(kt);
    if (ia) issue_a(kt + 1);
    if constexpr (IB) issue_b(kt + 2);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < 7) {
        if (q == 3) read_b_half<NB>(bt, 1, bq[1]);
        read_a_pair(at, q + 1, aq[(q + 1) & 1]);
      } else {
        if constexpr (IB)
          wait_vm_lgkm0<LB>();
        else
          wait_vm_lgkm0<0>();
        barrier_no_fence();
        if (ia) {
          read_b_half<NB>(b_of(kt + 1), 0, bq[0]);
          read_a_pair(a_of(kt + 1), 0, aq[0]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      mma_group<NB>(aq[q & 1], bq[q >> 2], q & 3, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int kt = 0;
  for (; kt + 2 < KT; ++kt) stage(kt, std::true_type{});
  for (; kt < KT; ++kt) stage(kt, std::false_type{});
}

// The K loop with both operands double-buffered (one 64 KiB stage in
// flight while the other is multiplied); the LDS it needs is LDS_BYTES.
template <int NB, typename ARow>
__device__ __forceinline__ void mainloop_nt2(const void* abase, ARow arow, const uint16_t* btile, int K, int rows,
                                            char* lds, Acc& acc) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // A rows and the B blocks through buffer resources: A offsets from abase
  // (every row arow returns lies within 4 GiB after it), B from btile
  const buf_rsrc_t ra = make_rsrc(abase), rb = make_rsrc(btile);
  uint32_t ao[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + j * 8 + (lane >> 3);
    ao[j] = (uint32_t)((const char*)arow(r) - (const char*)abase) + (((lane & 7) ^ tkey(r)) & 7) * 16;
  }
  const int wbase = wave * 4096;
  const int bwbase = wave * NB * 16;                   // this wave's share of the B tile (NB rows x 128 B)
  const uint32_t bo = bwbase + lane * 16;
  auto issue = [&](int64_t kb, char* st) {
    const uint32_t b = bo + (uint32_t)(kb / (BK * 2)) * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b2lds16(ra, ao[j] + (uint32_t)kb, st + wbase + j * 1024);
      if (j < NB / 64) b2lds16(rb, b + j * 1024, st + TILE_BYTES + bwbase + j * 1024);
    }
  };
  zero_acc(acc);
  const int KT = K / BK;
  if (wave >= 4 && rows <= 128) {
    // a padding wave: its B copies and the barriers, one per stage as below
    auto issue_b = [&](int64_t kb, char* st) {
      const uint32_t b = bo + (uint32_t)(kb / (BK * 2)) * TILE_BYTES;
#pragma unroll
      for (int j = 0; j < NB / 64; ++j) b2lds16(rb, b + j * 1024, st + TILE_BYTES + bwbase + j * 1024);
    };
    issue_b(0, lds);
    wait_all_mem();
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) issue_b((int64_t)(kt + 1) * BK * 2, lds + ((kt & 1) ^ 1) * STAGE_BYTES);
      wait_all_mem();
      __syncthreads();
    }
    return;
  }
  issue(0, lds);
  wait_all_mem();
  __syncthreads();
  // Fragments are read one group ahead of the MFMAs that use them (the
  // compiler, left alone, reuses one pair of registers and waits for every
  // read).  The stage's barrier sits before its last group, so the first
  // reads of the next stage are in flight while that group's MFMAs issue.
  // Scheduling barriers keep each group's reads ahead of the MFMAs before it.
  bf16x8_t bq[2][NB / 64], aq[2][2];
  read_b_half<NB>(lds + TILE_BYTES, 0, bq[0]);
  read_a_pair(lds, 0, aq[0]);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const char* st = lds + cur * STAGE_BYTES;
    const char* nst = lds + (cur ^ 1) * STAGE_BYTES;
    if (kt + 1 < KT) issue((int64_t)(kt + 1) * BK * 2, lds + (cur ^ 1) * STAGE_BYTES);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < 7) {
        if (q == 3) read_b_half<NB>(st + TILE_BYTES, 1, bq[1]);
        read_a_pair(st, q + 1, aq[(q + 1) & 1]);
      } else {
        wait_all_mem();
        __syncthreads();
        if (kt + 1 < KT) {
          read_b_half<NB>(nst + TILE_BYTES, 0, bq[0]);
          read_a_pair(nst, 0, aq[0]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      mma_group<NB>(aq[q & 1], bq[q >> 2], q & 3, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}


// B3: the K loop with B in three buffers (NT3_LDS_BYTES of LDS), for long K
// (the weights stream through it for many stages); else both operands
// double-buffered (LDS_BYTES), which measured faster for short K.
template <int NB = BN, bool B3 = false, typename ARow>
__device__ __forceinline__ void mainloop_nt(const void* abase, ARow arow, const uint16_t* btile, int K, int rows,
                                            char* lds, Acc& acc) {
  if constexpr (B3)
    mainloop_nt3<NB>(abase, arow, btile, K, rows, lds, acc);
  else
    mainloop_nt2<NB>(abase, arow, btile, K, rows, lds, acc);
}

// ---------------------------------------------------------------- GEMM1 ----
// a[p, i] = silu(g) * u with [g | u] = ring[p] . W_gu[e]^T; W_gu is packed so
// that each 32-column group holds 16 gate columns then the 16 up columns of
// the same i.  a is a bf16 GEMM operand (stored [p, I]); optionally g and u
// are saved in fp32 (packed order, [p, 2I]) for the backward.  NB packed
// columns of the tile: NB / 2 features, a wave's NB / 4 columns being
// NB / 128 gate/up groups of 32.  WT: the a rows are written through to
// memory (read by another XCD in the same launch).
// arow(r): the A row of tile row r (rows past the item repeat its last row),
// within 4 GiB after abase.
template <int NB, bool WT = false, bool B3 = false, typename ARow>
__device__ __forceinline__ void gemm1_tile_rows(const TileInfo& ti, const void* abase, ARow arow,
                                                const uint16_t* __restrict__ wgu, int H, int I,
                                                uint16_t* __restrict__ a_out, float* __restrict__ gu_save,
                                                char* lds) {
  Acc acc;
  mainloop_nt<NB, B3>(abase, arow, wgu + btile_block(ti.e, ti.n0 / BN, 0, 2 * I, H) + (ti.n0 % BN) * BK, H,
                      ti.rows, lds, acc);
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 3;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = frag_row(i, v);
#pragma unroll
      for (int q = 0; q < NB / 128; ++q) {
        const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
        stage_put(lds, r, wn * (NB / 8) + q * 16 + (lane & 15), g * sigmoidf_(g) * u);
        if (gu_save && r < ti.rows) {
          float* dst = gu_save + (int64_t)(ti.pos0 + r) * 2 * I + ti.n0 + wn * (NB / 4) + q * 32 + (lane & 15);
          dst[0] = g;
          dst[16] = u;
        }
      }
    }
  if constexpr (WT)
    stage_flush_wt<NB / 2>(lds, a_out, [&](int r) -> int64_t {
      return r < ti.rows ? ((int64_t)(ti.pos0 + r) * I + ti.n0 / 2) * 2 : -1;
    });
  else
    stage_flush<NB / 2>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? a_out + (int64_t)(ti.pos0 + r) * I + ti.n0 / 2 : nullptr;
    });
}

// GEMM1 tile whose A rows are the item's ring rows (positions mod ring_rows).
template <int NB, bool WT = false, bool B3 = false>
__device__ __forceinline__ void gemm1_tile(const TileInfo& ti, const uint16_t* __restrict__ ring, int ring_rows,
                                           const uint16_t* __restrict__ wgu, int H, int I,
                                           uint16_t* __restrict__ a_out, float* __restrict__ gu_save, char* lds) {
  auto arow = [&](int r) {
    const int p = ti.pos0 + min(r, ti.rows - 1);
    return ring + (int64_t)(p % ring_rows) * H;
  };
  gemm1_tile_rows<NB, WT, B3>(ti, ring, arow, wgu, H, I, a_out, gu_save, lds);
}

template <bool B3>
__global__ __launch_bounds__(NT) void gemm1_bf16_kernel(ItemRange ir, const uint16_t* __restrict__ ring,
                                                        int ring_rows, const uint16_t* __restrict__ wgu, int H,
                                                        int I, uint16_t* __restrict__ a_out,
                                                        float* __restrict__ gu_save) {
  __shared__ __attribute__((aligned(16))) char lds[B3 ? NT3_LDS_BYTES : LDS_BYTES];
  const int ntn = 2 * I / BN;
  for_each_tile_split(ir, ntn, [&](const TileInfo& ti, int half) {
    if (half < 0)
      gemm1_tile<BN, false, B3>(ti, ring, ring_rows, wgu, H, I, a_out, gu_save, lds);
    else
      gemm1_tile<BN / 2, false, B3>(ti, ring, ring_rows, wgu, H, I, a_out, gu_save, lds);
  });
}

// ---------------------------------------------------------------- GEMM2 ----
// y[p] = a[p] . W_d[e]^T  (W_d as the tiled B of [E, H, I]).
// SHARE: the router-weighted unpermute is fused: out[inv[p]] = bf16(w * y),
//        one rounding, rows stored straight to arrival order.
// else : y is kept in fp32 ([p, H]) for the full-layer combine.
template <bool SHARE, bool B3 = false>
__device__ __forceinline__ void gemm2_tile(const TileInfo& ti, const uint16_t* __restrict__ a,
                                           const uint16_t* __restrict__ wd, int H, int I, float* __restrict__ y32,
                                           uint16_t* __restrict__ out, const int32_t* __restrict__ inv,
                                           const float* __restrict__ row_w, char* lds) {
  auto arow = [&](int r) { return a + (int64_t)(ti.pos0 + min(r, ti.rows - 1)) * I; };
  Acc acc;
  mainloop_nt<BN, B3>(arow(0), arow, wd + btile_block(ti.e, ti.n0 / BN, 0, H, I), I, ti.rows, lds, acc);
#pragma unroll
  for (int i = 0; i < FM; ++i)
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
  if (SHARE)
    stage_flush<256>(lds, [&](int r) -> uint16_t* {
      return r < ti.rows ? out + (int64_t)inv[ti.pos0 + r] * H + ti.n0 : nullptr;
    });
}

template <bool SHARE, bool B3>
__global__ __launch_bounds__(NT) void gemm2_bf16_kernel(ItemRange ir, const uint16_t* __restrict__ a,
                                                        const uint16_t* __restrict__ wd, int H, int I,
                                                        float* __restrict__ y32, uint16_t* __restrict__ out,
                                                        const int32_t* __restrict__ inv,
                                                        const float* __restrict__ row_w) {
  __shared__ __attribute__((aligned(16))) char lds[B3 ? NT3_LDS_BYTES : LDS_BYTES];
  const int ntn = H / BN;
  for_each_tile(ir, ntn,
                [&](const TileInfo& ti) { gemm2_tile<SHARE, B3>(ti, a, wd, H, I, y32, out, inv, row_w, lds); });
}

// ------------------------------------------------- backward: dA' + SwiGLU ----
// dA'[p, i] = dYe[p] . W_d[e][:, i]  (B = W_d^T, tiled [E, I, H]).  Epilogue,
// from the forward's fp32 g, u: a = silu(g) u; dw partial = sum_i dA' a over
// this wave's 64 columns; dA = w dA'; dg = dA u s (1 + g (1 - s)); du = dA
// silu(g) (bf16 GEMM operands, row p = I gate then I up features); w*a (bf16 operand of the
// down-projection weight gradient).
template <bool B3>
__global__ __launch_bounds__(NT) void bwd_dact_kernel(ItemRange ir, const uint16_t* __restrict__ dye,
                                                      const uint16_t* __restrict__ wdT, int H, int I,
                                                      const float* __restrict__ gu,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ row_w,
                                                      uint16_t* __restrict__ dgdu, uint16_t* __restrict__ wa,
                                                      float* __restrict__ dw_part) {
  __shared__ __attribute__((aligned(16))) char lds[B3 ? NT3_LDS_BYTES : LDS_BYTES];
  const int ntn = I / BN;
  // a last round at most half full runs as 256 x 128 half tiles
  for_each_tile_split(ir, ntn, [&](const TileInfo& ti, int half) {
    auto arow = [&](int r) { return dye + (int64_t)(ti.pos0 + min(r, ti.rows - 1)) * H; };
    const uint16_t* bt = wdT + btile_block(ti.e, ti.n0 / BN, 0, I, H) + (ti.n0 % BN) * BK;
    Acc acc;
    if (half < 0) {
      mainloop_nt<BN, B3>(arow(0), arow, bt, H, ti.rows, lds, acc);
      dact_epilogue<BN>(ti, acc, lds, I, gu, inv, row_w, dgdu, wa, dw_part);
    } else {
      mainloop_nt<BN / 2, B3>(arow(0), arow, bt, H, ti.rows, lds, acc);
      dact_epilogue<BN / 2>(ti, acc, lds, I, gu, inv, row_w, dgdu, wa, dw_part);
    }
  });
}

// ------------------------------------------------------ backward: dX ----
// dX_row[p] = dgdu[p] . [W_g[e]; W_u[e]]  (B = [W_g; W_u]^T, tiled [E, H, 2I]:
// the I gate features, then the I up features, as in dgdu).
// ROWS16: rows stored as bf16 straight back to arrival order, dX[inv[p]];
// else : kept in fp32 at position p ([p, H]) for the full layer's k-sum.
template <bool ROWS16, bool B3>
__global__ __launch_bounds__(NT) void bwd_dx_kernel(ItemRange ir, const uint16_t* __restrict__ dgdu,
                                                    const uint16_t* __restrict__ wguT, int H, int I,
                                                    const int32_t* __restrict__ inv, uint16_t* __restrict__ dX,
                                                    float* __restrict__ dx32) {
  __shared__ __attribute__((aligned(16))) char lds[B3 ? NT3_LDS_BYTES : LDS_BYTES];
  const int ntn = H / BN;
  for_each_tile(ir, ntn, [&](const TileInfo& ti) {
    auto arow = [&](int r) { return dgdu + (int64_t)(ti.pos0 + min(r, ti.rows - 1)) * 2 * I; };
    Acc acc;
    mainloop_nt<BN, B3>(arow(0), arow, wguT + btile_block(ti.e, ti.n0 / BN, 0, H, 2 * I), 2 * I, ti.rows, lds, acc);
    dx_epilogue<ROWS16>(ti, acc, lds, H, inv, dX, dx32);
  });
}

// ----------------------------------------------------------- weight grads ----
// C[m, n] = sum over the rows p of expert e of A[p, m] * B[p, n]: both operands
// are row-major over p (the contraction), i.e. k-major for the MFMA.  A stage
// holds 64 rows x 256 columns of each operand in LDS exactly as they lie in
// memory, brought in by the LDS DMA like the other GEMMs' tiles; the MFMA
// fragments (8 consecutive k of one row m) are then built with the gfx950
// transpose read ds_read_b64_tr_b16: in each 16-lane group, lanes 4q..4q+3
// supply the 16 columns of tile row q and lane l receives column l of those
// 4 rows (measured on gfx950), so two reads give a lane its 8 k.  The 32-byte
// column chunks of tile row k sit at chunk slot c ^ trkey(k), which puts the
// 16 rows one read touches on different banks.  Rows past the end of a
// segment load a zero row.
// The K loop walks expert e's row segments minibatch by minibatch in reverse
// (nb-1 .. 0), rows ascending inside each: a fixed order, no atomics.
struct SegIter {
  int b, k0, start, len;
};

__device__ __forceinline__ bool seg_next(SegIter& it, const WgradArgs& w, int e) {
  it.k0 += BK;
  while (it.k0 >= it.len) {
    if (--it.b < 0) return false;
    it.start = it.b * w.MB + w.mb_offsets[it.b * (w.E + 1) + e];
    it.len = w.mb_counts[it.b * w.E + e];
    it.k0 = 0;
  }
  return true;
}

template <int MODE>
struct WgradOperands {
  // MODE 0: A = dYe [p, H], B = w*a [p, I]          -> dW_down [E, H, I]
  // MODE 1: A = dgdu [p, 2I] (gate | up), B = x rows -> dW_gate / dW_up [E, I, H]
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  const uint16_t* ring;
  int ring_rows, first_resident;
  const uint16_t* replay;      // x rows of minibatches < first_resident, at their positions p
  int64_t ldx;
  const uint16_t* zero;        // 512 zero bytes
};

__device__ __forceinline__ int trkey(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_t;
// The transposing read as inline assembly: issued through the builtin, the
// compiler cannot tell it apart from the LDS-DMA writes in flight to the
// other stage and waits for all of them (vmcnt(0)) before the first read of
// every stage, which serialises the prefetch.  Written here, it is not
// tracked: the caller waits for the LDS counter itself (mma_stage_kmajor),
// and the stage it reads was completed by the previous barrier.
__device__ __forceinline__ v4i16_t lds_read_tr(const char* p) {
  v4i16_t v;
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ void wait_lds_pinned() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_sched_barrier(0);
}

// One K step (64 rows) of the wave's 128 x 64 outputs from k-major tiles.
__device__ __forceinline__ void mma_stage_kmajor(const char* sA, const char* sB, Acc& acc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int g = lane >> 4, r = lane & 15;
  const int cb = (r & 3) * 8;                  // this lane's 8 bytes of a row's 32-byte chunk
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int k1 = ks * 32 + 8 * g + (r >> 2), k2 = k1 + 4;
    const int t1 = trkey(k1), t2 = trkey(k2);
    // the two halves of each fragment are joined into an MFMA operand only
    // after the wait: a copy made earlier would read registers the reads
    // have not written yet
    v4i16_t alo[FM], ahi[FM], blo[FN], bhi[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = wn * 4 + j;
      blo[j] = lds_read_tr(sB + k1 * 512 + ((c ^ t1) << 5) + cb);
      bhi[j] = lds_read_tr(sB + k2 * 512 + ((c ^ t2) << 5) + cb);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int c = wm * 8 + i;
      alo[i] = lds_read_tr(sA + k1 * 512 + ((c ^ t1) << 5) + cb);
      ahi[i] = lds_read_tr(sA + k2 * 512 + ((c ^ t2) << 5) + cb);
    }
    wait_lds_pinned();
    bf16x8_t bfr[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(blo[j], bhi[j], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(alo[i], ahi[i], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
    }
  }
}

// LDS-DMA of one stage's A (WHICH 0) or B (1) tile: wave w fills tile rows
// 8w .. 8w+7, two rows (1 KiB) per instruction; lane i takes row 8w + 2j +
// i/32 and the 16 bytes of logical chunk (slot ^ trkey(row)) that belong in
// its slot.
template <int MODE, int WHICH>
__device__ __forceinline__ void wgrad_issue(const WgradOperands<MODE>& op, const SegIter& it, int m0, int n0,
                                            char* tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = 8 * wave + 2 * j + (lane >> 5);
    const int off = ((((s >> 1) ^ trkey(k)) & 15) << 5) + ((s & 1) << 4);
    const bool live = it.k0 + k < it.len;
    const int64_t p = it.start + it.k0 + k;
    const char* src;
    if (!live) {
      src = (const char*)op.zero + off;
    } else if (WHICH == 0) {
      src = (const char*)(op.A + p * op.lda + m0) + off;
    } else if (MODE == 0) {
      src = (const char*)(op.B + p * op.ldb + n0) + off;
    } else if (it.b >= op.first_resident) {
      src = (const char*)(op.ring + (int64_t)(p % op.ring_rows) * op.ldx + n0) + off;
    } else {
      src = (const char*)(op.replay + p * op.ldx + n0) + off;
    }
    g2lds16(src, tile + (8 * wave + 2 * j) * 512);
  }
}

// B3: the K loop keeps A in two LDS buffers and B in three (all 160 KiB):
// while stage kt is multiplied, A of kt+1 and B of kt+1 and kt+2 are in
// flight.  Each wave waits for its own copies (vmcnt: B of kt+1 was issued
// before A of kt+1, which was issued before B of kt+2), and the barriers
// carry no fence of their own (the transposing reads are not tracked by the
// compiler and are waited for inside mma_stage_kmajor).  It pays when the
// experts have few rows (a few stages per tile) and measured slower with
// thousands of rows per expert, which keep both operands double-buffered.
// Both tiles of one stage (A at st, B at st + TILE_BYTES), each row's A and
// B copies issued together (the order the double-buffered loop measured
// fastest in).
template <int MODE>
__device__ __forceinline__ void wgrad_issue_ab(const WgradOperands<MODE>& op, const SegIter& it, int m0, int n0,
                                               char* st) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = 8 * wave + 2 * j + (lane >> 5);
    const int off = ((((s >> 1) ^ trkey(k)) & 15) << 5) + ((s & 1) << 4);
    const bool live = it.k0 + k < it.len;
    const int64_t p = it.start + it.k0 + k;
    const char* a = live ? (const char*)(op.A + p * op.lda + m0) + off : (const char*)op.zero + off;
    const char* b;
    if (!live) {
      b = (const char*)op.zero + off;
    } else if (MODE == 0) {
      b = (const char*)(op.B + p * op.ldb + n0) + off;
    } else if (it.b >= op.first_resident) {
      b = (const char*)(op.ring + (int64_t)(p % op.ring_rows) * op.ldx + n0) + off;
    } else {
      b = (const char*)(op.replay + p * op.ldx + n0) + off;
    }
    char* dst = st + (8 * wave + 2 * j) * 512;
    g2lds16(a, dst);
    g2lds16(b, dst + TILE_BYTES);
  }
}

template <int MODE, bool B3>
__global__ __launch_bounds__(NT) void wgrad_kernel(WgradArgs w, WgradOperands<MODE> op, int M, int N, int I,
                                                      float* __restrict__ out0, float* __restrict__ out1) {
  __shared__ __attribute__((aligned(16))) char lds[B3 ? NT3_LDS_BYTES : LDS_BYTES];
  char* const abuf = lds;
  char* const bbuf = lds + NT_A_BUFS * TILE_BYTES;
  const int tm = M / BM, tn = N / BN;
  const int per_e = tm * tn;
  const int total = w.E * per_e;
  for (int t = xcd_logical_block(); t < total; t += gridDim.x) {
    const int e = t / per_e;
    int mt, nt;
    tile_coords(t - e * per_e, tm, tn, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    Acc acc;
    zero_acc(acc);
    SegIter cur{w.nb, 0, 0, 0};
    bool have = seg_next(cur, w, e);
    if (have && !B3) {
      auto issue = [&](const SegIter& it, char* st) { wgrad_issue_ab<MODE>(op, it, m0, n0, st); };
      issue(cur, lds);
      wait_all_mem();
      __syncthreads();
      int stage = 0;
      while (true) {
        SegIter nxt = cur;
        const bool more = seg_next(nxt, w, e);
        if (more) issue(nxt, lds + (stage ^ 1) * STAGE_BYTES);
        mma_stage_kmajor(lds + stage * STAGE_BYTES, lds + stage * STAGE_BYTES + TILE_BYTES, acc);
        wait_all_mem();
        __syncthreads();
        if (!more) break;
        cur = nxt;
        stage ^= 1;
      }
    } else if (have) {
      // stage 0's A and B, and B of stage 1; wait for stage 0
      SegIter nxt = cur;
      bool have1 = seg_next(nxt, w, e);
      wgrad_issue<MODE, 0>(op, cur, m0, n0, abuf);
      wgrad_issue<MODE, 1>(op, cur, m0, n0, bbuf);
      if (have1) {
        wgrad_issue<MODE, 1>(op, nxt, m0, n0, bbuf + TILE_BYTES);
        wait_vm_lgkm0<4>();
      } else {
        wait_vm_lgkm0<0>();
      }
      barrier_no_fence();
      for (int kt = 0;; ++kt) {
        SegIter nxt2 = nxt;
        const bool have2 = have1 && seg_next(nxt2, w, e);
        if (have1) wgrad_issue<MODE, 0>(op, nxt, m0, n0, abuf + ((kt + 1) & 1) * TILE_BYTES);
        if (have2) wgrad_issue<MODE, 1>(op, nxt2, m0, n0, bbuf + ((kt + 2) % NT_B_BUFS) * TILE_BYTES);
        mma_stage_kmajor(abuf + (kt & 1) * TILE_BYTES, bbuf + (kt % NT_B_BUFS) * TILE_BYTES, acc);
        if (have2)
          wait_vm_lgkm0<4>();
        else
          wait_vm_lgkm0<0>();
        barrier_no_fence();
        if (!have1) break;
        nxt = nxt2;
        have1 = have2;
      }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int m = m0 + wm * 128 + i * 16 + 4 * (lane >> 4) + vv;
        float* dst;
        if (MODE == 0) {
          dst = out0 + ((int64_t)e * M + m) * N;
        } else {
          dst = (m < I ? out0 + ((int64_t)e * I + m) * N : out1 + ((int64_t)e * I + m - I) * N);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[n0 + wn * 64 + j * 16 + (lane & 15)] = acc[i][j][vv];
      }
  }
}

// ------------------------------------------------ fused forward, bf16 ----
// The forward's permute, GEMM1 + SwiGLU and GEMM2 in one persistent launch
// ([MTP] opening paragraph: every step in one kernel; "Three design
// decisions that matter": overlap at minibatch granularity): while some
// compute units permute minibatch b+1, others run GEMM1 of b and GEMM2 of
// b-1, and the tail of one phase fills with the next phase's units.  The
// full layer's combine, which needs every GEMM2 tile of the layer when it
// runs as one minibatch, follows as its own launch.
//
// Units: per item (256 rows of one expert in one minibatch) 4 permute
// chunks of 64 rows, 2I/256 GEMM1 tiles and H/256 GEMM2 tiles.  Placement,
// chosen by the host: unit u of a segment (item-major: u = item * tiles +
// tile) goes to queue u mod 8, so every queue gets an equal share (to one
// unit) and a weight column panel stays in one queue, or two, across the
// items of an expert; or (item_local, for experts with about one item per
// minibatch) queue x takes a contiguous run of items with all of their
// units: an item's ring rows and a rows are read from the L2 that wrote
// them, and the items of one expert (consecutive in the item list) share
// their weight panels in one L2.  Queue x is taken by
// the workgroups whose index is x mod 8 -- the workgroups the hardware
// places on XCD x, since a dispatch deals its workgroups to the 8 XCDs in
// turn -- so a panel is read into one XCD's L2.  (Only speed rests on that
// placement: each queue has workgroups whatever it is.)  A queue's
// workgroups take its units in a fixed order from its own ticket; per
// iteration j: GEMM1 of minibatch j-1, permute of j, GEMM2 of j-2.
// Dependencies (device counters): a GEMM1 tile waits for its item's 4
// permute chunks, a GEMM2 tile for its item's GEMM1 tiles.  With direct set
// (the full layer: its token rows are local), there are no permute units
// and GEMM1 tiles read the x rows through the inverse map.  Every wait
// points at a unit of an earlier iteration, so the unit with the smallest
// iteration never waits and every queue drains; waits are bounded anyway
// (about 0.25 s, then MK_DEVERR_WAIT_TIMEOUT and on).
//
// Coherence across the XCDs without cache maintenance: what one unit hands
// to another -- ring rows and a rows -- is stored with the device-scope
// bit, written through to memory; the producer waits for those stores to
// complete before bumping the counter; the consumer reads after seeing it.
// Every such location is written once, before any read of it in the launch
// (the ring holds every minibatch of the call: no slot is reused; a tile
// reads only its own item's rows), so no XCD can hold a stale copy in its
// L2 or L1.
constexpr int FUSE_CH = 64;                       // rows per permute unit
constexpr int FUSE_PCH = MK_TILE_M / FUSE_CH;     // permute units per item
constexpr int FUSE_XCD = 8;
enum { U_NONE = -1, U_G1 = 0, U_P = 1, U_G2 = 2 };

struct FusedArgs {
  const int32_t* items;       // [cap, 4] (row_begin, rows, expert, minibatch)
  const int32_t* mb_items;    // [nb + 1]
  int item_cap, nb, src_div, H, I, ring_rows;
  int item_local;             // placement: whole items per queue (else unit u to queue u mod 8)
  int direct;                 // GEMM1 reads its A rows from x through the inverse map: no permute units
  int wait_spins;             // bound of a dependency wait, in polls
  uint32_t wait_extra;        // added to every wait's target (0; 1 in tests of the timeout path)
  const uint16_t* x;          // token rows (full layer) or routed rows (expert share)
  const int32_t* inv;
  const float* row_w;
  uint16_t* ring;
  const uint16_t* wgu;
  const uint16_t* wd;
  uint16_t* a_buf;
  float* gu_save;
  float* y32;                 // full layer: GEMM2 rows in fp32
  uint16_t* out;
  uint32_t* ticket;           // [8 queues, 64 words apart]; zeroed before the launch, as are the counters
  uint32_t* p_done;           // [cap] permute units done per item
  uint32_t* g1_done;          // [cap] GEMM1 tiles done per item
  uint32_t* err;
};

struct FusedUnit {
  int kind, b, u;             // u: the unit's index in its segment
};

__device__ __forceinline__ int fused_items_lo(const FusedArgs& a, int b) { return min(a.mb_items[b], a.item_cap); }
__device__ __forceinline__ int fused_items(const FusedArgs& a, int b) {
  return min(a.mb_items[b + 1], a.item_cap) - min(a.mb_items[b], a.item_cap);
}
// units of segment (kind, b), all queues
__device__ __forceinline__ int fused_units(const FusedArgs& a, int kind, int b) {
  const int n = fused_items(a, b);
  return kind == U_P ? n * FUSE_PCH : kind == U_G1 ? n * (2 * a.I / BN) : n * (a.H / BN);
}

// Unit of ticket t of queue x (U_NONE past the last one).
__device__ FusedUnit fused_decode(const FusedArgs& a, int x, int t) {
  for (int j = 0; j < a.nb + 2; ++j) {
#pragma unroll 1
    for (int kind = 0; kind < 3; ++kind) {
      const int b = kind == U_G1 ? j - 1 : kind == U_P ? j : j - 2;
      if (b < 0 || b >= a.nb || (kind == U_P && a.direct)) continue;
      if (a.item_local) {
        // whole items: queue x takes the contiguous run of items
        // [x ni / 8, (x+1) ni / 8) of the minibatch, all of their units
        const int per = kind == U_P ? FUSE_PCH : kind == U_G1 ? 2 * a.I / BN : a.H / BN;
        const int ni = fused_items(a, b);
        const int lo = (int)((int64_t)x * ni / FUSE_XCD), hi = (int)((int64_t)(x + 1) * ni / FUSE_XCD);
        const int nx = (hi - lo) * per;
        if (t < nx) return FusedUnit{kind, b, lo * per + t};
        t -= nx;
      } else {
        const int n = fused_units(a, kind, b);
        const int nx = n > x ? (n - x + FUSE_XCD - 1) / FUSE_XCD : 0;
        if (t < nx) return FusedUnit{kind, b, x + FUSE_XCD * t};
        t -= nx;
      }
    }
  }
  return FusedUnit{U_NONE, 0, 0};
}

// Wave 0 (all of its lanes, so the loop is uniform): wait until *p >=
// target.  The wait is bounded (limit polls, by default about a quarter of
// a second); once any wait of the launch has timed out (the error bit is
// set) the others stop waiting too, so a launch whose counters went wrong
// still ends quickly.
constexpr int FUSE_WAIT_POLLS = 1 << 20;
__device__ __forceinline__ void fused_wait(const uint32_t* p, uint32_t target, uint32_t* err, int limit) {
  int spins = 0;
  while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
         target) {
    __builtin_amdgcn_s_sleep(8);
    ++spins;
    if ((spins & 1023) == 0 &&
        (__builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) &
         MK_DEVERR_WAIT_TIMEOUT))
      break;
    if (spins >= limit) {
      if ((threadIdx.x & 63) == 0) atomicOr(err, MK_DEVERR_WAIT_TIMEOUT);
      break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// GEMM tile u of minibatch b (item-major, ntn column tiles per item).
__device__ __forceinline__ TileInfo fused_tile(const FusedArgs& a, int b, int u, int ntn, int& item) {
  item = fused_items_lo(a, b) + u / ntn;
  const int* q = a.items + 4 * item;
  return TileInfo{q[0], q[1], q[2], (u % ntn) * BN};
}

// Control flow around the barriers is uniform: wave 0 as a whole takes the
// ticket (lane 0's atomic, broadcast), decodes it and waits, every wave
// reads the unit back from LDS as a scalar, and only the counter bumps are
// single-lane; no lane of a wave ever takes a different path to a barrier.
// B3: GEMM1 units (contraction H) take the three-buffer K loop, and with
// DIRECT the GEMM2 units too; the LDS is then all in use by the K loops, and
// the unit is passed in its first bytes (free between units: every unit
// ends at a barrier after its last LDS access, and a second barrier below
// comes before the next unit's copies).
// A workgroup takes its next ticket as soon as its current unit's inputs
// are ready, so the atomic's latency hides behind the unit; per queue a
// workgroup's tickets still increase, and a unit depends only on units of
// earlier segments, so the earliest unfinished unit is always running.
// GEMM2 units publish nothing, and no wave touches the LDS after a GEMM2
// unit's last barrier (the K loops read their last stage before it; the
// expert share's staged epilogue ends with one), so they end without
// waiting for their stores, which then drain under the next unit's ticket,
// wait and first loads; the next unit's hand-over in the LDS is safe.
template <bool SHARE, bool B3, bool DIRECT>
__global__ __launch_bounds__(NT) void fused_forward_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[B3 ? NT3_LDS_BYTES : LDS_BYTES + 16];
  int* const su = (int*)(lds + (B3 ? 0 : LDS_BYTES));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = blockIdx.x % FUSE_XCD;   // this workgroup's queue
  const int ntn1 = 2 * a.I / BN, ntn2 = a.H / BN;
  uint32_t t_next = 0;                   // wave 0, lane 0: the ticket of the next unit
  if (wave == 0 && lane == 0) t_next = atomicAdd(a.ticket + 64 * x, 1u);
  while (true) {
    if (wave == 0) {
      const FusedUnit un = fused_decode(a, x, (int)__builtin_amdgcn_readfirstlane(t_next));
      if (un.kind == U_G1 && !DIRECT) {
        fused_wait(a.p_done + fused_items_lo(a, un.b) + un.u / ntn1, (uint32_t)FUSE_PCH + a.wait_extra, a.err,
                   a.wait_spins);
      } else if (un.kind == U_G2) {
        fused_wait(a.g1_done + fused_items_lo(a, un.b) + un.u / ntn2, (uint32_t)ntn1 + a.wait_extra, a.err,
                   a.wait_spins);
      }
      if (un.kind != U_NONE && lane == 0) t_next = atomicAdd(a.ticket + 64 * x, 1u);
      if (lane == 0) {
        su[0] = un.kind;
        su[1] = un.b;
        su[2] = un.u;
      }
    }
    __syncthreads();
    const int kind = __builtin_amdgcn_readfirstlane(su[0]);
    const int b = __builtin_amdgcn_readfirstlane(su[1]);
    const int u = __builtin_amdgcn_readfirstlane(su[2]);
    if constexpr (B3) __syncthreads();   // every wave has the unit: the LDS is the unit's
    if (kind == U_NONE) break;
    int item = -1;
    if (kind == U_P) {
      // rows [64c, 64c + 64) of item u / 4, one wave per row, written through
      item = fused_items_lo(a, b) + u / FUSE_PCH;
      const int* q = a.items + 4 * item;
      const int r0 = (u % FUSE_PCH) * FUSE_CH, r1 = min(q[1], r0 + FUSE_CH);
      const buf_rsrc_t rr = make_rsrc(a.ring);
      for (int r = r0 + wave; r < r1; r += NT / 64) {
        const int64_t p = q[0] + r;
        const int src = a.inv[p];
        if (src >= 0)
          copy_row_wave_wt((const u32x4_t*)(a.x + (int64_t)(src / a.src_div) * a.H), rr,
                           (uint32_t)((p % a.ring_rows) * a.H * 2), a.H / 8, lane);
      }
    } else if (kind == U_G1) {
      const TileInfo ti = fused_tile(a, b, u, ntn1, item);
      if constexpr (DIRECT) {
        // the item's x rows through the inverse map (token = routed row / src_div)
        auto arow = [&](int r) {
          return a.x + (int64_t)(a.inv[ti.pos0 + min(r, ti.rows - 1)] / a.src_div) * a.H;
        };
        gemm1_tile_rows<BN, true, B3>(ti, a.x, arow, a.wgu, a.H, a.I, a.a_buf, a.gu_save, lds);
      } else {
        gemm1_tile<BN, true, B3>(ti, a.ring, a.ring_rows, a.wgu, a.H, a.I, a.a_buf, a.gu_save, lds);
      }
    } else {
      const TileInfo ti = fused_tile(a, b, u, ntn2, item);
      // with x read directly, GEMM2 units take the three-buffer loop too
      gemm2_tile<SHARE, B3 && DIRECT>(ti, a.a_buf, a.wd, a.H, a.I, a.y32, a.out, a.inv, a.row_w, lds);
    }
    if (kind == U_G2) continue;   // nothing to publish
    // publish: every wave's stores complete, then one counter bump
    wait_all_mem();
    __syncthreads();
    if (wave == 0 && lane == 0) {
      if (kind == U_P)
        __hip_atomic_fetch_add(a.p_done + item, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (kind == U_G1)
        __hip_atomic_fetch_add(a.g1_done + item, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

void launch_gemm1_bf16(const ItemRange& ir, const uint16_t* ring, int32_t ring_rows, const uint16_t* wgu,
                       int H, int I, uint16_t* a_out, float* gu_save, int n_cu, hipStream_t s) {
  if (H >= NT3_MIN_K)
    hipLaunchKernelGGL(gemm1_bf16_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, ring, ring_rows, wgu, H, I, a_out,
                       gu_save);
  else
    hipLaunchKernelGGL(gemm1_bf16_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, ring, ring_rows, wgu, H, I, a_out,
                       gu_save);
}

void launch_gemm2_bf16(const ItemRange& ir, const uint16_t* a, const uint16_t* wd, int H, int I, float* y32,
                       uint16_t* out, const int32_t* inv, const float* row_w, int n_cu, hipStream_t s) {
  const bool b3 = I >= NT3_MIN_K_L2A;
  if (out && b3)
    hipLaunchKernelGGL((gemm2_bf16_kernel<true, true>), dim3(n_cu), dim3(NT), 0, s, ir, a, wd, H, I, y32, out, inv,
                       row_w);
  else if (out)
    hipLaunchKernelGGL((gemm2_bf16_kernel<true, false>), dim3(n_cu), dim3(NT), 0, s, ir, a, wd, H, I, y32, out, inv,
                       row_w);
  else if (b3)
    hipLaunchKernelGGL((gemm2_bf16_kernel<false, true>), dim3(n_cu), dim3(NT), 0, s, ir, a, wd, H, I, y32, out, inv,
                       row_w);
  else
    hipLaunchKernelGGL((gemm2_bf16_kernel<false, false>), dim3(n_cu), dim3(NT), 0, s, ir, a, wd, H, I, y32, out,
                       inv, row_w);
}

void launch_fused_forward_bf16(const FusedFwd& f, int n_cu, hipStream_t s) {
  FusedArgs a;
  a.items = f.ir.items;
  a.mb_items = f.ir.mb_items;
  a.item_cap = f.ir.item_cap;
  a.nb = f.nb;
  a.src_div = f.src_div;
  a.H = f.H;
  a.I = f.I;
  a.ring_rows = f.ring_rows;
  a.item_local = f.item_local;
  a.direct = f.direct;
  a.wait_spins = f.wait_spins > 0 ? f.wait_spins : FUSE_WAIT_POLLS;
  a.wait_extra = (uint32_t)f.wait_extra;
  a.x = f.x;
  a.inv = f.inv;
  a.row_w = f.row_w;
  a.ring = f.ring;
  a.wgu = f.wgu;
  a.wd = f.wd;
  a.a_buf = f.a_buf;
  a.gu_save = f.gu_save;
  a.y32 = f.y32;
  a.out = f.out;
  uint32_t* c = f.ctl;
  a.ticket = c;
  a.p_done = c + 64 * FUSE_XCD;
  a.g1_done = a.p_done + f.ir.item_cap;
  a.err = f.err;
  // the tickets and the counters start at zero (a fill kernel, not a memset,
  // so the sequence can be captured in a graph)
  launch_fill_u32(c, 0u, fused_ctl_words(f.ir.item_cap), s);
  // one workgroup per compute unit, a multiple of the 8 queues
  const int grid = std::max(FUSE_XCD, n_cu / FUSE_XCD * FUSE_XCD);
  // GEMM1 units take the three-buffer loop for long contractions, and from
  // H = 2048 when their A rows come from x (lower latency than ring rows,
  // so the weights' latency is what the third buffer hides)
  const bool b3 = f.H >= NT3_MIN_K || (f.direct && f.H >= 2048);
  if (!f.full && b3)
    hipLaunchKernelGGL((fused_forward_kernel<true, true, false>), dim3(grid), dim3(NT), 0, s, a);
  else if (!f.full)
    hipLaunchKernelGGL((fused_forward_kernel<true, false, false>), dim3(grid), dim3(NT), 0, s, a);
  else if (b3 && f.direct)
    hipLaunchKernelGGL((fused_forward_kernel<false, true, true>), dim3(grid), dim3(NT), 0, s, a);
  else if (b3)
    hipLaunchKernelGGL((fused_forward_kernel<false, true, false>), dim3(grid), dim3(NT), 0, s, a);
  else if (f.direct)
    hipLaunchKernelGGL((fused_forward_kernel<false, false, true>), dim3(grid), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((fused_forward_kernel<false, false, false>), dim3(grid), dim3(NT), 0, s, a);
}

void launch_bwd_dact(const ItemRange& ir, const uint16_t* dye, const uint16_t* wdT, int H, int I, const float* gu,
                     const int32_t* inv, const float* row_w, uint16_t* dgdu, uint16_t* wa, float* dw_part, int n_cu,
                     hipStream_t s) {
  if (H >= NT3_MIN_K_L2A)
    hipLaunchKernelGGL(bwd_dact_kernel<true>, dim3(n_cu), dim3(NT), 0, s, ir, dye, wdT, H, I, gu, inv, row_w, dgdu,
                       wa, dw_part);
  else
    hipLaunchKernelGGL(bwd_dact_kernel<false>, dim3(n_cu), dim3(NT), 0, s, ir, dye, wdT, H, I, gu, inv, row_w, dgdu,
                       wa, dw_part);
}

void launch_bwd_dx(const ItemRange& ir, const uint16_t* dgdu, const uint16_t* wguT, int H, int I,
                   const int32_t* inv, uint16_t* dX, float* dx32, int n_cu, hipStream_t s) {
  const bool b3 = 2 * I >= NT3_MIN_K_L2A;
  if (dX && b3)
    hipLaunchKernelGGL((bwd_dx_kernel<true, true>), dim3(n_cu), dim3(NT), 0, s, ir, dgdu, wguT, H, I, inv, dX, dx32);
  else if (dX)
    hipLaunchKernelGGL((bwd_dx_kernel<true, false>), dim3(n_cu), dim3(NT), 0, s, ir, dgdu, wguT, H, I, inv, dX, dx32);
  else if (b3)
    hipLaunchKernelGGL((bwd_dx_kernel<false, true>), dim3(n_cu), dim3(NT), 0, s, ir, dgdu, wguT, H, I, inv, dX, dx32);
  else
    hipLaunchKernelGGL((bwd_dx_kernel<false, false>), dim3(n_cu), dim3(NT), 0, s, ir, dgdu, wguT, H, I, inv, dX,
                       dx32);
}

void launch_wgrad_down(const WgradArgs& w, const uint16_t* dye, const uint16_t* wa, int H, int I,
                       float* dW_down, const uint16_t* zero_row, bool b3, int n_cu, hipStream_t s) {
  WgradOperands<0> op{dye, H, wa, I, nullptr, 1, 0, nullptr, 0, zero_row};
  if (b3)
    hipLaunchKernelGGL((wgrad_kernel<0, true>), dim3(n_cu), dim3(NT), 0, s, w, op, H, I, I, dW_down, (float*)nullptr);
  else
    hipLaunchKernelGGL((wgrad_kernel<0, false>), dim3(n_cu), dim3(NT), 0, s, w, op, H, I, I, dW_down,
                       (float*)nullptr);
}

void launch_wgrad_gate_up(const WgradArgs& w, const uint16_t* dgdu, const uint16_t* ring, int32_t ring_rows,
                          int first_resident, const uint16_t* replay, int H, int I, float* dW_gate, float* dW_up,
                          const uint16_t* zero_row, bool b3, int n_cu, hipStream_t s) {
  WgradOperands<1> op{dgdu, 2 * (int64_t)I, nullptr, 0, ring, ring_rows, first_resident, replay, H, zero_row};
  if (b3)
    hipLaunchKernelGGL((wgrad_kernel<1, true>), dim3(n_cu), dim3(NT), 0, s, w, op, 2 * I, H, I, dW_gate, dW_up);
  else
    hipLaunchKernelGGL((wgrad_kernel<1, false>), dim3(n_cu), dim3(NT), 0, s, w, op, 2 * I, H, I, dW_gate, dW_up);
}

}  // namespace mk
