// Device count, scan and permute of the routed token rows into expert order.
//
// Sparser-MoE page (harryzhou2000), "Remove work that has no selected route":
// local pre-processing visits only the selected local slots of a token (a
// wavefront ballot over its K slots, iterating the set bits).  bpdata article,
// "Optimization 1: Grouped GEMM": expert token counts stay on the device.
//
// Three kernels, no host round trip:
//  k_count    per tile of TT tokens: per-local-expert histogram (LDS), and the
//             stable rank of every local slot among the tile's slots of the
//             same expert (wavefront ballots, flat slot order).
//  k_scan     one workgroup, one pass over the tile histograms: per-tile
//             expert bases, counts[L], offsets[L+1], overflow check.
//  k_permute  one wavefront per token: ballot over its K slots, read the row
//             once, write it to each selected local expert row.
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tokens per count tile: about T*K/256 slots per tile (at least 64, at most
// 512), so that small-K layers still spread the counting over many CUs.
int permute_tile_tokens(int T, int K) {
  if (K < 1) K = 1;
  long slots = (long)T * K / 256;
  slots = slots < 64 ? 64 : (slots > 512 ? 512 : slots);
  int tt = (int)(slots / K);
  if (tt < 1) tt = 1;
  return tt;
}

// ---------------------------------------------------------------------------
// k_count: grid = ntiles, 256 threads.  Dynamic LDS: cnt[4][L] int32 +
// rank[TT*K] int32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_count(int T, int K, int E_global, int e0, int L, int TT,
                                               const int16_t* __restrict__ ids,
                                               int32_t* __restrict__ hist, int32_t* __restrict__ rank,
                                               int32_t* err) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;              // [4][L]
  int32_t* srank = lds + 4 * L;    // [TT*K]
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int tile = blockIdx.x;
  const long f0 = (long)tile * TT * K;
  long fend = f0 + (long)TT * K;
  const long ftot = (long)T * K;
  if (fend > ftot) fend = ftot;
  const int nslot = (int)(fend - f0);
  for (int i = threadIdx.x; i < 4 * L; i += 256) cnt[i] = 0;
  __syncthreads();
  // wave w handles slots [w*part, (w+1)*part) of the tile, 64 at a time
  const int part = (((nslot + 3) / 4) + 63) / 64 * 64;
  const int s_begin = w * part, s_end = min(nslot, s_begin + part);
  int32_t* mycnt = cnt + w * L;
  bool bad = false;
  for (int c = s_begin; c < s_end; c += 64) {
    const int sl = c + l;
    int le = -1;
    if (sl < s_end) {
      const int id = ids[f0 + sl];
      if (id < -1 || id >= E_global) bad = true;
      else if (id >= e0 && id < e0 + L) le = id - e0;
    }
    uint64_t active = wave_ballot(le >= 0);
    int myrank = 0;
    while (active) {  // one iteration per distinct expert among the 64 slots
      const int leader = __builtin_ctzll(active);
      const int v = readlane_i(le, leader);
      const uint64_t m = wave_ballot(le == v);
      const int base = readlane_i(l == leader ? mycnt[v] : 0, leader);
      if (le == v) myrank = base + mask_rank(m);
      if (l == leader) mycnt[v] = base + __builtin_popcountll(m);
      active &= ~m;
    }
    if (sl < s_end) srank[sl] = myrank;
  }
  if (wave_ballot(bad) && l == 0) set_err(err, MOE_DEVERR_BAD_ID);
  __syncthreads();
  // tile histogram and per-wave bases
  for (int e = threadIdx.x; e < L; e += 256) {
    const int c0 = cnt[e], c1 = cnt[L + e], c2 = cnt[2 * L + e], c3 = cnt[3 * L + e];
    hist[(long)tile * L + e] = c0 + c1 + c2 + c3;
    cnt[e] = 0;
    cnt[L + e] = c0;
    cnt[2 * L + e] = c0 + c1;
    cnt[3 * L + e] = c0 + c1 + c2;
  }
  __syncthreads();
  for (int sl = threadIdx.x; sl < nslot; sl += 256) {
    const int id = ids[f0 + sl];
    int r = 0;
    if (id >= e0 && id < e0 + L && id < E_global) {
      const int ww = sl / part;
      r = srank[sl] + cnt[ww * L + (id - e0)];
    }
    rank[f0 + sl] = r;
  }
}

// ---------------------------------------------------------------------------
// k_scan: one workgroup of 1024 threads.  hist [ntiles][L] -> exclusive tile
// bases (in place), counts, offsets, overflow flag.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_scan(int ntiles, int L, int64_t capacity,
                                               int32_t* __restrict__ hist, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int32_t* err) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_tot[MOE_MAX_L];
  __shared__ int32_t s_wsum[16];
  const int tid = threadIdx.x;
  // experts handled in groups of up to 1024; each expert column split in nparts
  for (int eb = 0; eb < L; eb += 1024) {
    const int Lb = min(1024, L - eb);
    int nparts = 1024 / Lb;
    if (nparts > ntiles) nparts = ntiles > 0 ? ntiles : 1;
    const int per = (ntiles + nparts - 1) / nparts;
    const int e = tid % Lb, part = tid / Lb;
    const bool act = part < nparts;
    int sum = 0;
    if (act) {
      const int t0 = part * per, t1 = min(ntiles, t0 + per);
      for (int t = t0; t < t1; ++t) sum += hist[(long)t * L + eb + e];
    }
    __syncthreads();
    s_part[tid] = act ? sum : 0;
    __syncthreads();
    if (act) {
      int base = 0;
      for (int p = 0; p < part; ++p) base += s_part[p * Lb + e];
      const int t0 = part * per, t1 = min(ntiles, t0 + per);
      // 16 tiles at a time: all their loads are issued before the in-place
      // stores, which the compiler could not move the next loads across
      for (int tb = t0; tb < t1; tb += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = tb + u < t1 ? hist[(long)(tb + u) * L + eb + e] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (tb + u < t1) hist[(long)(tb + u) * L + eb + e] = base;
          base += c[u];
        }
      }
      if (part == nparts - 1) s_tot[eb + e] = base;
    }
    __syncthreads();
  }
  // offsets: exclusive scan of the totals (each thread owns up to 4 experts)
  const int per = (L + 1023) / 1024;
  const int b0 = tid * per;
  int loc = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < L) loc += s_tot[b0 + i];
  const int incl = wave_incl_scan(loc);
  const int wv = tid >> 6, l = tid & 63;
  if (l == 63) s_wsum[wv] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < wv; ++i) wbase += s_wsum[i];
  int run = wbase + incl - loc;
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < L) {
      counts[e] = s_tot[e];
      offsets[e] = run;
      run += s_tot[e];
    }
  }
  if (tid == 1023) {
    int total = 0;
    for (int i = 0; i < 16; ++i) total += s_wsum[i];
    offsets[L] = total;
    if ((int64_t)total > capacity) set_err(err, MOE_DEVERR_OVERFLOW);
  }
}

// ---------------------------------------------------------------------------
// k_permute: one wavefront per token, 4 per workgroup.
// ---------------------------------------------------------------------------
// Fused scan (SCAN = 1, for ntiles * L <= PERMUTE_SCAN_MAX and L <= 64, TT a
// multiple of 4): `tilebase` holds the raw tile histograms of k_count; every
// workgroup sums the ones it needs (the tiles before its own, and all of them
// for the offsets) instead of a separate k_scan, and workgroup 0 writes
// counts, offsets and the overflow flag.
#define PERMUTE_SCAN_MAX 4096
template <int OUT, int SCAN>  // OUT 0: copy rows (bf16 or fp32, row_bytes), 1: MXFP8-, 2: MXFP4-quantize bf16 rows
__global__ __launch_bounds__(256) void k_permute(int T, int K, int e0, int L, int TT, int64_t capacity,
                                                 int row_bytes, const uint8_t* __restrict__ x,
                                                 const int16_t* __restrict__ ids,
                                                 const int32_t* __restrict__ tilebase,
                                                 const int32_t* __restrict__ rank,
                                                 const int32_t* __restrict__ offsets,
                                                 uint8_t* __restrict__ x_perm, uint8_t* __restrict__ x_scales,
                                                 int32_t* __restrict__ row_to_slot,
                                                 int32_t* __restrict__ slot_to_row, int32_t* __restrict__ counts_out,
                                                 int32_t* __restrict__ offsets_out, int32_t* err) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  __shared__ int32_t s_sum[2][256];  // SCAN: partial sums (before the tile, total)
  __shared__ int32_t s_base[64], s_off[64];
  if (SCAN) {
    // the workgroup's 4 tokens share one tile (TT % 4 == 0); thread i sums
    // entries (tile' , e) with e = i % L, tile' = i / L, i / L + 256 / L, ...
    const int tile0 = (blockIdx.x * 4) / TT, ntiles = (T + TT - 1) / TT;
    const int e = threadIdx.x % L, step = 256 / L;
    int before = 0, all = 0;
    if (threadIdx.x < step * L) {
      for (int tt = threadIdx.x / L; tt < ntiles; tt += step) {
        const int c = tilebase[(long)tt * L + e];
        all += c;
        before += tt < tile0 ? c : 0;
      }
    }
    s_sum[0][threadIdx.x] = before;
    s_sum[1][threadIdx.x] = all;
    __syncthreads();
    if (w == 0) {
      int b = 0, a = 0;
      if (l < L)
        for (int q = 0; q < step; ++q) { b += s_sum[0][q * L + l]; a += s_sum[1][q * L + l]; }
      const int incl = wave_incl_scan(l < L ? a : 0);
      if (l < L) { s_base[l] = b; s_off[l] = incl - a; }
      if (blockIdx.x == 0) {
        if (l < L) { counts_out[l] = a; offsets_out[l] = incl - a; }
        if (l == 63) {
          offsets_out[L] = incl;
          if ((int64_t)incl > capacity) set_err(err, MOE_DEVERR_OVERFLOW);
        }
      }
    }
    __syncthreads();
  }
  if (t >= T) return;
  const int tile = t / TT;
  int dest = -1;
  if (l < K) {
    const long f = (long)t * K + l;
    const int id = ids[f];
    if (id >= e0 && id < e0 + L) {
      const int le = id - e0;
      const int64_t d = SCAN ? (int64_t)s_off[le] + s_base[le] + rank[f]
                             : (int64_t)offsets[le] + tilebase[(long)tile * L + le] + rank[f];
      dest = d < capacity ? (int)d : -1;
    }
    slot_to_row[f] = dest;
  }
  uint64_t bits = wave_ballot(dest >= 0);
  if (!bits) return;  // no selected local slot: the row is never read
  const uint8_t* src = x + (long)t * row_bytes;
  // rows move in 1 KiB pieces (16 bytes per lane), up to 8 pieces in flight
  const int npiece = (row_bytes + 1023) / 1024;
  for (int p0 = 0; p0 < npiece; p0 += 8) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int off = (p0 + j) * 1024 + l * 16;
      if (p0 + j < npiece && off < row_bytes) v[j] = *(const u32x4*)(src + off);
      else v[j] = u32x4{0, 0, 0, 0};
    }
    if (OUT == 0) {
      uint64_t b = bits;
      while (b) {
        const int k = __builtin_ctzll(b);
        b &= b - 1;
        const int d = readlane_i(dest, k);
        if (p0 == 0 && l == 0) row_to_slot[d] = t * K + k;
        uint8_t* dst = x_perm + (long)d * row_bytes;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int off = (p0 + j) * 1024 + l * 16;
          if (p0 + j < npiece && off < row_bytes) *(u32x4*)(dst + off) = v[j];
        }
      }
    } else {
      // quantize the pieces once: the 8 bf16 of a lane -> 8 codes; 4 lanes
      // share a 32-element block and its scale
      uint32_t lo[8], hi[8], sc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t am = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t a0 = v[j][q] & 0x7fffu, a1 = (v[j][q] >> 16) & 0x7fffu;
          am = am > a0 ? am : a0;
          am = am > a1 ? am : a1;
        }
        uint32_t o = (uint32_t)__shfl_xor((int)am, 1, 64);
        am = am > o ? am : o;
        o = (uint32_t)__shfl_xor((int)am, 2, 64);
        am = am > o ? am : o;
        if (OUT == 1) {
          const int E = mx_scale_exp(am);
          lo[j] = mx_e4m3x4(v[j][0], v[j][1], E);
          hi[j] = mx_e4m3x4(v[j][2], v[j][3], E);
          sc[j] = (uint32_t)(E + 127);
        } else {  // 8 E2M1 codes, element 2i in the low nibble of byte i
          const int E = mx4_scale_exp(am);
          uint32_t c = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            c |= (mx_e2m1(v[j][q] & 0xffffu, E) | (mx_e2m1(v[j][q] >> 16, E) << 4)) << (8 * q);
          lo[j] = c;
          hi[j] = 0;
          sc[j] = (uint32_t)(E + 127);
        }
      }
      // bf16 row of H = row_bytes/2 elements -> codes [H] (MXFP4: [H/2]
      // bytes) + scales [H/32]
      const int H = row_bytes >> 1;
      uint64_t b = bits;
      while (b) {
        const int k = __builtin_ctzll(b);
        b &= b - 1;
        const int d = readlane_i(dest, k);
        if (p0 == 0 && l == 0) row_to_slot[d] = t * K + k;
        uint8_t* dst = x_perm + (long)d * (OUT == 1 ? H : H >> 1);
        uint8_t* dsc = x_scales + (long)d * (H >> 5);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int off = (p0 + j) * 1024 + l * 16;  // byte offset in the bf16 row
          if (p0 + j < npiece && off < row_bytes) {
            const int e_off = off >> 1;  // element offset
            if (OUT == 1) *(uint2*)(dst + e_off) = make_uint2(lo[j], hi[j]);
            else *(uint32_t*)(dst + (e_off >> 1)) = lo[j];
            if ((l & 3) == 0) dsc[e_off >> 5] = (uint8_t)sc[j];
          }
        }
      }
    }
  }
}

template <int SCAN>
static void launch_permute_rows(int T, int K, int e0, int L, int TT, int64_t capacity, int row_bytes, int out_dtype,
                                const void* x, const int16_t* ids, const int32_t* hist, const int32_t* rank,
                                int32_t* offsets, void* x_perm, uint8_t* x_scales, int32_t* row_to_slot,
                                int32_t* slot_to_row, int32_t* counts, int32_t* err, hipStream_t s) {
  const dim3 g((T + 3) / 4), b(256);
  if (out_dtype == MOE_MXFP8)
    hipLaunchKernelGGL((k_permute<1, SCAN>), g, b, 0, s, T, K, e0, L, TT, capacity, row_bytes, (const uint8_t*)x,
                       ids, hist, rank, offsets, (uint8_t*)x_perm, x_scales, row_to_slot, slot_to_row, counts,
                       offsets, err);
  else if (out_dtype == MOE_MXFP4)
    hipLaunchKernelGGL((k_permute<2, SCAN>), g, b, 0, s, T, K, e0, L, TT, capacity, row_bytes, (const uint8_t*)x,
                       ids, hist, rank, offsets, (uint8_t*)x_perm, x_scales, row_to_slot, slot_to_row, counts,
                       offsets, err);
  else
    hipLaunchKernelGGL((k_permute<0, SCAN>), g, b, 0, s, T, K, e0, L, TT, capacity, row_bytes, (const uint8_t*)x,
                       ids, hist, rank, offsets, (uint8_t*)x_perm, x_scales, row_to_slot, slot_to_row, counts,
                       offsets, err);
}

hipError_t launch_permute(int T, int H, int K, int E_global, int e0, int L, int64_t capacity,
                          int x_dtype, int out_dtype, const void* x, const int16_t* ids,
                          int32_t* counts, int32_t* offsets, void* x_perm, uint8_t* x_scales,
                          int32_t* row_to_slot, int32_t* slot_to_row, int32_t* err, void* ws,
                          hipStream_t s) {
  int TT = permute_tile_tokens(T, K);
  int ntiles = (T + TT - 1) / TT;
  // few tiles and experts: the scan is done inside k_permute (tiles of a
  // multiple of 4 tokens, so that a permute workgroup's tokens share a tile)
  const int TT4 = (TT + 3) / 4 * 4;
  const bool fused = T > 0 && L <= 64 && (long)((T + TT4 - 1) / TT4) * L <= PERMUTE_SCAN_MAX;
  if (fused) {
    TT = TT4;
    ntiles = (T + TT - 1) / TT;
  }
  int32_t* hist = (int32_t*)ws;
  int32_t* rank = hist + (size_t)ntiles * L;  // within the workspace (sized for the unrounded tiling)
  if (ntiles > 0) {
    const size_t lds = (size_t)(4 * L + TT * K) * sizeof(int32_t);
    hipLaunchKernelGGL(k_count, dim3(ntiles), dim3(256), lds, s, T, K, E_global, e0, L, TT, ids, hist,
                       rank, err);
  }
  const int row_bytes = H * (x_dtype == MOE_F32 ? 4 : 2);
  if (fused) {
    launch_permute_rows<1>(T, K, e0, L, TT, capacity, row_bytes, out_dtype, x, ids, hist, rank, offsets, x_perm,
                           x_scales, row_to_slot, slot_to_row, counts, err, s);
  } else {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, ntiles, L, capacity, hist, counts, offsets, err);
    if (T > 0)
      launch_permute_rows<0>(T, K, e0, L, TT, capacity, row_bytes, out_dtype, x, ids, hist, rank, offsets, x_perm,
                             x_scales, row_to_slot, slot_to_row, counts, err, s);
  }
  return hipGetLastError();
}

}  // namespace moe
