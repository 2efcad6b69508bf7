// Device tile schedule shared by the grouped GEMM kernels.
#pragma once
#include "moe_internal.h"

namespace moe {

// compute units of the device (queried once per process: the initializer of
// a function-local static runs exactly once even under concurrent first calls)
static inline int num_cus() {
  static const int n_cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      return n;
    return 256;
  }();
  return n_cus;
}

// ---------------------------------------------------------------------------
// Device tile schedule.  s_pre[e] = first tile of expert e, s_pre[L] = total.
// Row range of expert e: [min(offsets[e], cap), min(offsets[e+1], cap)).
// ---------------------------------------------------------------------------
// Row tiles of an expert with m rows: the fewest tiles of at most BM + tall
// rows, ceil(m / (BM + tall)) (tall = 0: ceil(m / BM)).
__device__ __forceinline__ int row_tiles(int m, int BM, int tall) { return (m + BM + tall - 1) / (BM + tall); }

// First row (within the expert) and row count of row tile i of an expert with
// m rows in nt = row_tiles(m, BM, tall) tiles.  When nt tiles of BM rows hold
// the m rows, they are BM rows each and the last takes the remainder;
// otherwise every tile has BM rows plus extra rows, `tall` each for the first
// ones, then what is left for one tile, then none (tall tiles; tall = 0
// never gets here).
__device__ __forceinline__ void tile_rows(int m, int nt, int BM, int tall, int i, int* r0, int* rows) {
  const int ex = m - nt * BM;  // rows beyond nt tiles of BM
  if (ex <= 0) {
    *r0 = i * BM;
    *rows = min(BM, m - i * BM);
    return;
  }
  const int q = ex / tall, rem = ex - q * tall;  // tiles [0, q) take `tall` extra rows, tile q takes rem
  *r0 = i * BM + min(i, q) * tall + (i > q ? rem : 0);
  *rows = BM + (i < q ? tall : (i == q ? rem : 0));
}

__device__ inline void build_schedule(int L, int64_t capacity, int BM, int NT, const int32_t* __restrict__ offsets,
                               int32_t* s_pre, int32_t* s_tmp, int tall = 0) {
  const int nth = blockDim.x, tid = threadIdx.x;
  const int per = (L + nth - 1) / nth;
  const int b0 = tid * per;
  int loc = 0;
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < L) {
      int64_t lo = offsets[e], hi = offsets[e + 1];
      lo = lo < capacity ? lo : capacity;
      hi = hi < capacity ? hi : capacity;
      const int m = hi > lo ? (int)(hi - lo) : 0;
      loc += row_tiles(m, BM, tall) * NT;
    }
  }
  const int incl = wave_incl_scan(loc);
  const int w = tid >> 6, l = tid & 63;
  if (l == 63) s_tmp[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += s_tmp[i];
  int run = base + incl - loc;
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < L) {
      s_pre[e] = run;
      int64_t lo = offsets[e], hi = offsets[e + 1];
      lo = lo < capacity ? lo : capacity;
      hi = hi < capacity ? hi : capacity;
      const int m = hi > lo ? (int)(hi - lo) : 0;
      run += row_tiles(m, BM, tall) * NT;
    }
  }
  if (tid == nth - 1) s_pre[L] = run;
  __syncthreads();
}

// rows of expert e: [min(offsets[e], cap), min(offsets[e+1], cap))
__device__ __forceinline__ int expert_rows(const int32_t* __restrict__ offsets, int e, int64_t capacity, int* r0) {
  int64_t lo = offsets[e], hi = offsets[e + 1];
  lo = lo < capacity ? lo : capacity;
  hi = hi < capacity ? hi : capacity;
  *r0 = (int)lo;
  return hi > lo ? (int)(hi - lo) : 0;
}

// largest e in [0, L) with pre[e] <= it (empty experts share their start
// with the next one)
__device__ __forceinline__ int find_expert(const int32_t* pre, int L, int it) {
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= it) lo = mid; else hi = mid - 1;
  }
  return lo;
}

#define TILE_MGROUP 4

struct TileInfo {
  int e, row0, rows, nt;
};

__device__ __forceinline__ TileInfo locate_tile(int it, int L, int64_t capacity, int BM, int NT,
                                                const int32_t* __restrict__ offsets, const int32_t* s_pre,
                                                int tall = 0) {
  // largest e with s_pre[e] <= it (empty experts share their start with the next)
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= it) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  int64_t r0 = offsets[e], r1 = offsets[e + 1];
  r0 = r0 < capacity ? r0 : capacity;
  r1 = r1 < capacity ? r1 : capacity;
  const int m = (int)(r1 - r0);
  const int mt_e = row_tiles(m, BM, tall);
  const int local = it - s_pre[e];
  // an expert's tiles go in groups of up to TILE_MGROUP row tiles: all column
  // tiles of a group, row tile fastest, then the next group.  The 32 CUs of an
  // XCD run 32 consecutive tiles; for an expert with many rows that is a block
  // of 4 row tiles x 8 column tiles, whose A rows and B panels both stay in
  // that XCD's L2, instead of one B panel with 32 row tiles of A.
  const int g = local / (TILE_MGROUP * NT);
  const int rem = local - g * (TILE_MGROUP * NT);
  const int mg = min(TILE_MGROUP, mt_e - g * TILE_MGROUP);
  TileInfo ti;
  ti.e = e;
  ti.nt = rem / mg;
  const int mt = g * TILE_MGROUP + rem % mg;
  int tr0, trows;
  tile_rows(m, mt_e, BM, tall, mt, &tr0, &trows);
  ti.row0 = (int)r0 + tr0;
  ti.rows = trows;
  return ti;
}

// ---------------------------------------------------------------------------
// Work units of a persistent grid of G workgroups over `total` tiles of 2*KT
// k steps (KT pairs): the first floor(total/G)*G tiles run whole; when the
// `left` tiles of the last, partial round number at most GEMM_SPLIT_UNITS/2,
// each is split into S >= 2 pieces along k (at most GEMM_SPLIT_UNITS pieces,
// at most 16 per tile, each piece at least 8 whole groups of 4 k steps).
// ---------------------------------------------------------------------------
#define GEMM_SPLIT_UNITS 256

struct SplitPlan {
  int dp;     // tiles run whole: units [0, dp)
  int S;      // pieces per split tile (1: no split)
  int units;  // dp + (total - dp) * S
};

// The most pieces a split tile of KT pairs of k steps may have: pieces of at
// least 8 groups of 4 k steps (shorter pieces cost more in partial-tile
// traffic and the reduce than they save), at most 16.  Below 2, no tile of
// that depth is ever split, and the host skips the reduce kernel.
__host__ __device__ inline int split_max_pieces(int KT) { return KT / 16 < 16 ? KT / 16 : 16; }

__device__ __forceinline__ SplitPlan split_plan(int total, int G, int KT) {
  SplitPlan p;
  const int left = total % G;
  p.dp = total - left;
  int S = left > 0 ? min(min(G, GEMM_SPLIT_UNITS) / left, split_max_pieces(KT)) : 1;
  if (S < 2) {
    p.dp = total;
    S = 1;
  }
  p.S = S;
  p.units = p.dp + (total - p.dp) * S;
  return p;
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row: rows 0..7 get
// distinct chunks, and rows r, r+8 (which share banks when 16 lanes are
// served per cycle from 64 banks) differ too.
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// chunk position swizzle of a 64-byte row in its 16-row block
__device__ __forceinline__ int swz4(int r) {
  return (((r >> 1) ^ (r >> 3)) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1);
}

// 16 bytes per lane from buffer `rsrc` at voff + soff into LDS at
// lds_addr + 16 * lane.  Issued as inline assembly so that the compiler does
// not wait for it at every LDS read and barrier; its completion is awaited
// explicitly (vmcnt, in issue order) before the barrier that publishes it.
__device__ __forceinline__ void lds_dma_b128(uint32_t lds_addr, int voff, __amdgpu_buffer_rsrc_t rsrc, int soff) {
  // s_nop 4: the wait states after an SALU write of M0 (1) and after a VALU
  // write of an SGPR that a VMEM instruction reads (5)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// 4 bytes per lane: lane i's dword lands at lds_addr + 4 * i
__device__ __forceinline__ void lds_dma_b32(uint32_t lds_addr, int voff, __amdgpu_buffer_rsrc_t rsrc, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// lds_dma_b32 when `sel` == `want` (both wave-uniform), as lds_dma_b128_if
__device__ __forceinline__ void lds_dma_b32_if(int sel, int want, uint32_t lds_addr, int voff,
                                               __amdgpu_buffer_rsrc_t rsrc, int soff) {
  asm volatile("s_cmp_eq_u32 %4, %5\n\ts_cbranch_scc0 1f\n\ts_mov_b32 m0, %0\n\ts_nop 4\n\t"
               "buffer_load_dword %1, %2, %3 offen lds\n1:"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff), "s"(sel), "s"(want)
               : "memory", "m0", "scc");
}

// lds_dma_b128 when `sel` == `want` (both wave-uniform).  The test and branch
// are inside the assembly so that the compiler sees straight-line code.
__device__ __forceinline__ void lds_dma_b128_if(int sel, int want, uint32_t lds_addr, int voff,
                                                __amdgpu_buffer_rsrc_t rsrc, int soff) {
  asm volatile("s_cmp_eq_u32 %4, %5\n\ts_cbranch_scc0 1f\n\ts_mov_b32 m0, %0\n\ts_nop 4\n\t"
               "buffer_load_dwordx4 %1, %2, %3 offen lds\n1:"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff), "s"(sel), "s"(want)
               : "memory", "m0", "scc");
}

// Split-K partial tiles: piece q of a split tile at part + q * piece_stride floats,
// wavefront w's 128 x 64 part at w * 8192, its 32 x 32 block (i, j) at
// (i * 2 + j) * 1024, lane l's 16 values of the MFMA D layout at l * 16.
// sum_partials adds the S pieces of row block i of one wavefront part in
// piece order (the result does not depend on timing); up to 4 pieces are
// loaded before they are added.
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void sum_partials(const float* __restrict__ src, int S, f32x16_p (&acc)[1][2],
                                             long piece_stride = 65536) {
  f32x4_p sum[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) sum[j][c] = *(const f32x4_p*)(src + j * 1024 + c * 4);
  for (int q = 1; q < S; q += 4) {
    f32x4_p t[4][2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u < S)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) t[u][j][c] = *(const f32x4_p*)(src + (q + u) * piece_stride + j * 1024 + c * 4);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u < S)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) sum[j][c] += t[u][j][c];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[0][j][4 * c + t] = sum[j][c][t];
}

__device__ __forceinline__ int virtual_block() {
  const int G = gridDim.x, b = blockIdx.x;
  return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace moe
