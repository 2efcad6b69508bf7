// Device count, scan and permute of the routed token rows into expert order.
//
// Sparser-MoE page (harryzhou2000), "Remove work that has no selected route":
// local pre-processing visits only the selected local slots of a token (a
// wavefront ballot over its K slots, iterating the set bits).  bpdata article,
// "Optimization 1: Grouped GEMM": expert token counts stay on the device.
//
// k_count_scan: one workgroup per tile of TT consecutive tokens counts the
// tile's slots per local expert (ids staged in LDS), gives each local slot
// its row within the tile and expert, publishes the tile's counts and counts
// itself finished on a device counter.  The workgroup that finishes last
// scans every tile's counts (read at once, in parallel): each tile's base row
// per expert, the expert counts and offsets.  No workgroup waits for
// another (a single-pass scan without a look-back chain: the last arrival
// sees all counts).
// k_permute: one wavefront per token; each local slot's row is its expert's
// offset + its tile's base + its row within the tile; the token's row is
// copied (or MX-quantized) to each of them.
#include "moe_internal.h"

#include <mutex>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tiles: about PERM_TILE_SLOTS slots each, at most PERM_SCAN_MAX / L tiles
// (the scan reads ntiles * L counts); a tile is counted PERM_CHUNK slots at a
// time (its ids staged in LDS) by PERM_WAVES wavefronts.
#define PERM_TILE_SLOTS 2048
#define PERM_SCAN_MAX 16384
#define PERM_CHUNK 16384
#ifndef PERM_SINGLE_SLOTS
#define PERM_SINGLE_SLOTS PERM_TILE_SLOTS  // batches of at most this many slots are one tile
#endif
#define PERM_WAVES 8
#define PERM_THREADS (PERM_WAVES * 64)
int permute_tile_tokens(int T, int K, int L) {
  if (K < 1) K = 1;
  if (L < 1) L = 1;
  if ((long)T * K <= PERM_SINGLE_SLOTS) return T > 0 ? T : 1;  // one tile: no scan across tiles
  long tt = (PERM_TILE_SLOTS + K - 1) / K;
  long nt = ((long)T + tt - 1) / tt;
  const long ntmax = PERM_SCAN_MAX / L > 0 ? PERM_SCAN_MAX / L : 1;
  if (nt > ntmax) tt = ((long)T + ntmax - 1) / ntmax;
  return (int)(tt < 1 ? 1 : tt);
}

// ---------------------------------------------------------------------------
// Workspace of the permute (byte offsets; ntiles tiles of TT tokens):
//   0                       the count of finished tiles (uint32)
//   256                     tile counts [ntiles][L] uint32 (bit 30: published)
//   next 256-byte boundary  tile bases [ntiles][L] int32
//   next 256-byte boundary  each local slot's row within its tile and expert [T*K]
// The counter and the tile counts (the state) are zero between calls: the
// caller zero-fills the workspace once, and the scanning workgroup returns
// them to zero.  The bases and rows are written before they are read.
// ---------------------------------------------------------------------------
#define PERM_FLAGS_OFF 256

struct PermuteWs {
  uint32_t* done;
  uint32_t* flags;
  int32_t* tilebase;
  int32_t* rank;
};

static inline size_t ws_round(size_t v) { return (v + 255) / 256 * 256; }

static int permute_ntiles(int T, int K, int L) {
  const int TT = permute_tile_tokens(T, K, L);
  return T > 0 ? (T + TT - 1) / TT : 0;
}

static PermuteWs permute_ws(void* ws, int ntiles, int L) {
  uint8_t* b = (uint8_t*)ws;
  const size_t fl = ws_round((size_t)ntiles * L * 4);
  PermuteWs w;
  w.done = (uint32_t*)b;
  w.flags = (uint32_t*)(b + PERM_FLAGS_OFF);
  w.tilebase = (int32_t*)(b + PERM_FLAGS_OFF + fl);
  w.rank = (int32_t*)(b + PERM_FLAGS_OFF + 2 * fl);
  return w;
}

size_t permute_state_bytes(int T, int K, int L) {
  return PERM_FLAGS_OFF + ws_round((size_t)permute_ntiles(T, K, L) * L * 4);
}

size_t permute_workspace_bytes(int T, int K, int L) {
  const size_t fl = ws_round((size_t)permute_ntiles(T, K, L) * L * 4);
  return PERM_FLAGS_OFF + 2 * fl + ws_round((size_t)T * K * 4);
}

#define PERM_PUBLISHED (1u << 30)
#define PERM_VALUE ((1u << 30) - 1)
// bound on the polls of one tile's counts by the scanning workgroup: every
// tile has published its counts before it counts itself finished, so the
// polls only wait for those stores to become visible; the bound (about a
// second) is reached only when the counter was not zero at the start, and
// the call then reports MOE_DEVERR_WORKSPACE
#define PERM_MAX_POLLS (1 << 20)

__device__ __forceinline__ uint32_t flag_load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Poll a tile's count until published (relaxed loads at device scope),
// backing off from 64 to 2048 clocks between polls; still unpublished after
// the bound, it returns 0.  Out of line: the scan's unrolled loads each keep
// only a call.  The count is the data itself, so no acquire is needed.
__device__ __attribute__((noinline)) uint32_t flag_wait_slow(const uint32_t* p) {
  uint32_t f = flag_load_relaxed(p);
  for (int polls = 0; !(f & PERM_PUBLISHED); ++polls) {
    if (polls >= PERM_MAX_POLLS) return 0u;
    if (polls < 8) __builtin_amdgcn_s_sleep(1);
    else if (polls < 16) __builtin_amdgcn_s_sleep(4);
    else __builtin_amdgcn_s_sleep(32);
    f = flag_load_relaxed(p);
  }
  return f;
}

// The lanes of the wavefront holding the same local expert as this lane
// (among the lanes with one, mask `valid`), from one ballot per bit of the
// expert index: O(log L) wavefront instructions per 64 slots, however many
// distinct experts they hold.
__device__ __forceinline__ uint64_t same_expert_lanes(int le, uint64_t valid, int nbits) {
  uint64_t peers = valid;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (le >> b) & 1;
    const uint64_t m = wave_ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// One pass over a chunk of a tile's slots (staged in LDS, PERM_CHUNK
// entries), each wavefront over a contiguous part, 4 x 64 slots per step.
// PASS 0 adds each local slot to its wavefront's count of its expert (an
// LDS add per slot).  PASS 1 finds, for each 64 slots, the lanes of each
// local expert (bit ballots) and gives each local slot its row within the
// tile and expert (the wavefront's running row of that expert, read before
// the lowest of those lanes advances it, + the slot's rank among them).  The wavefront's LDS
// operations run in order, so the counts need no wait between the read and
// the add; the four id reads of a step are unconditional (clamped index,
// masked after), so one wait covers them.
template <int PASS>
__device__ __forceinline__ bool count_pass(int nslot, int e0, int L, int E_global, int nbits, const int16_t* s_ids,
                                           int32_t* mycnt, int32_t* __restrict__ rank, long f0) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int part = (((nslot + PERM_WAVES - 1) / PERM_WAVES) + 63) / 64 * 64;
  const int s_begin = w * part, s_end = min(nslot, s_begin + part);
  const uint64_t lt = (1ull << l) - 1;
  bool bad = false;
  for (int c = s_begin; c < s_end; c += 256) {
    int id[4], le[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) id[u] = s_ids[min(c + u * 64 + l, PERM_CHUNK - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = c + u * 64 + l < s_end;
      bad |= in && (id[u] < -1 || id[u] >= E_global);
      le[u] = (in && id[u] >= e0 && id[u] < e0 + L && id[u] < E_global) ? id[u] - e0 : -1;
    }
    if (PASS == 0) {  // counting only: one LDS add per local slot (the order does not matter)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (le[u] >= 0) __hip_atomic_fetch_add(mycnt + le[u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      continue;
    }
    uint64_t peers[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t valid = wave_ballot(le[u] >= 0);
      peers[u] = valid ? same_expert_lanes(le[u], valid, nbits) : 0ull;
    }
    int base[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      base[u] = 0;
      if (le[u] >= 0) {
        int32_t* cp = mycnt + le[u];
        if (PASS == 1) base[u] = __hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (!(peers[u] & lt))
          __hip_atomic_fetch_add(cp, __builtin_popcountll(peers[u]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    if (PASS == 1) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (le[u] >= 0) rank[f0 + c + u * 64 + l] = base[u] + __builtin_popcountll(peers[u] & lt);
    }
  }
  return bad;
}

// A workgroup barrier that waits only for this wavefront's LDS operations:
// __syncthreads also waits for every outstanding global load and store (the
// slot ranks, the published counts, the rows in flight), which nothing
// behind these barriers reads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Expert totals (LDS) -> counts, offsets (exclusive scan, offsets[L] = N),
// MOE_DEVERR_OVERFLOW when N > capacity; all threads of the workgroup.
__device__ __forceinline__ void expert_offsets(int L, int64_t capacity, const int32_t* tot, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int32_t* err, int* s_wsum) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int per = (L + PERM_THREADS - 1) / PERM_THREADS;
  const int b0 = threadIdx.x * per;
  int loc = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < L) loc += tot[b0 + i];
  const int incl = wave_incl_scan(loc);
  if (l == 63) s_wsum[w] = incl;
  lds_barrier();
  int r = incl - loc;
  for (int i = 0; i < w; ++i) r += s_wsum[i];
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < L) {
      counts[e] = tot[e];
      offsets[e] = r;
      r += tot[e];
    }
  }
  if (threadIdx.x == PERM_THREADS - 1) {
    offsets[L] = r;
    if ((int64_t)r > capacity) set_err(err, MOE_DEVERR_OVERFLOW);
  }
}

// ---------------------------------------------------------------------------
// k_count_scan: one workgroup of PERM_THREADS threads per tile.
// Dynamic LDS: cnt[PERM_WAVES][L] + run[L] int32, then the chunk's ids int16
// [PERM_CHUNK].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(PERM_THREADS) void k_count_scan(int T, int K, int E_global, int e0, int L, int TT, int ntiles,
                                                             bool fold,
                                                    int64_t capacity, const int16_t* __restrict__ ids,
                                                    uint32_t* __restrict__ done, uint32_t* __restrict__ flags,
                                                    int32_t* __restrict__ tilebase, int32_t* __restrict__ rank,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* err) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;                   // [PERM_WAVES][L]: per-wavefront counts of a chunk, then running rows
  int32_t* run = lds + PERM_WAVES * L;  // [L]: the tile's count so far (the scan: expert totals)
  int16_t* s_ids = (int16_t*)(lds + (PERM_WAVES + 1) * L);
  __shared__ int s_last;
  __shared__ int s_wsum[PERM_WAVES];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int tile = blockIdx.x;
  int nbits = 0;
  while ((1 << nbits) < L) ++nbits;
  const long f0 = (long)tile * TT * K;
  long fend = f0 + (long)TT * K;
  if (fend > (long)T * K) fend = (long)T * K;
  for (int e = threadIdx.x; e < L; e += PERM_THREADS) run[e] = 0;
  bool bad = false;
  for (long c0 = f0; c0 < fend; c0 += PERM_CHUNK) {
    const int n = (int)(fend - c0 < PERM_CHUNK ? fend - c0 : PERM_CHUNK);
    for (int i = threadIdx.x; i < PERM_WAVES * L; i += PERM_THREADS) cnt[i] = 0;
    for (int i0 = 0; i0 < n; i0 += PERM_THREADS * 4) {  // the chunk's ids, four loads in flight per thread
      int16_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * PERM_THREADS + threadIdx.x;
        v[u] = i < n ? ids[c0 + i] : (int16_t)-1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * PERM_THREADS + threadIdx.x;
        if (i < n) s_ids[i] = v[u];
      }
    }
    lds_barrier();
    bad |= count_pass<0>(n, e0, L, E_global, nbits, s_ids, cnt + w * L, rank, c0);
    lds_barrier();
    for (int e = threadIdx.x; e < L; e += PERM_THREADS) {  // each wavefront's running rows start after the earlier slots'
      int r = run[e];
#pragma unroll
      for (int v = 0; v < PERM_WAVES; ++v) {
        const int c = cnt[v * L + e];
        cnt[v * L + e] = r;
        r += c;
      }
      run[e] = r;
    }
    lds_barrier();
    count_pass<1>(n, e0, L, E_global, nbits, s_ids, cnt + w * L, rank, c0);
    lds_barrier();
  }
  if (wave_ballot(bad) && l == 0) set_err(err, MOE_DEVERR_BAD_ID);
  if (fold) {  // few tiles and experts: the permute kernel combines the tiles' counts itself
    lds_barrier();
    for (int e = threadIdx.x; e < L; e += PERM_THREADS) tilebase[(long)tile * L + e] = run[e];
    return;
  }
  if (ntiles == 1) {  // the whole batch in one tile: its counts are the totals
    lds_barrier();
    for (int e = threadIdx.x; e < L; e += PERM_THREADS) tilebase[e] = 0;
    expert_offsets(L, capacity, run, counts, offsets, err, s_wsum);
    return;
  }
  // publish the tile's counts, then count the tile finished.  Each count
  // carries the published bit, and the scanning workgroup polls every count
  // it reads until the bit is set, so neither store needs to be ordered
  // before the other (no fence: a release here would write back the L2 once
  // per wavefront of every tile).  The rows within the tile are read only
  // by the next kernel.
  for (int e = threadIdx.x; e < L; e += PERM_THREADS) flag_store_relaxed(flags + (long)tile * L + e, PERM_PUBLISHED | (uint32_t)run[e]);
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old >= (uint32_t)ntiles) set_err(err, MOE_DEVERR_WORKSPACE);  // the counter was not zero
    s_last = old == (uint32_t)ntiles - 1;
  }
  lds_barrier();
  if (!s_last) return;
  // ---- the last tile to finish: each tile's base row per expert (an
  // exclusive prefix of the counts over the tiles) and each expert's total.
  // Experts in chunks of NE columns (a power of two), tiles in batches whose
  // counts fit the LDS stage [tile][NE]; R threads per column (a power of
  // two, at most 64: a segment of a wavefront), each summing a contiguous run
  // of the batch's tiles, one segmented scan of those sums across the
  // column's threads, the batches chained by a running carry.  Rolled loops
  // throughout: this code runs in one workgroup only, so its instructions
  // are fetched cold, and its length is its latency.
  bool stuck = false;
  int lne = 0;
  while ((1 << lne) < L && (1 << lne) < PERM_THREADS) ++lne;
  const int NE = 1 << lne;
  int lr = 0;
  while ((1 << lr) * NE < PERM_THREADS && lr < 6) ++lr;
  const int R = 1 << lr;
  const int jc = threadIdx.x >> lr, rr = threadIdx.x & (R - 1);
  const int cap = TT * K;
  const int nbt = (PERM_CHUNK / 2) >> lne;  // tiles per batch (the stage holds PERM_CHUNK / 2 words)
  int32_t* s_stage = (int32_t*)s_ids;
  for (int ec = 0; ec < L; ec += NE) {
    const int e = ec + jc;
    const bool col = jc < NE && e < L;
    int carry = 0;
    for (int p0 = 0; p0 < ntiles; p0 += nbt) {
      const int nb = min(nbt, ntiles - p0), words = nb << lne;
      lds_barrier();
      // plain loads, sixteen in flight per thread (one round for up to 8K
      // counts): a count read stale reads unpublished and is polled again
      for (int i0 = 0; i0 < words; i0 += PERM_THREADS * 16) {
        uint32_t f[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int i = i0 + u * PERM_THREADS + threadIdx.x, ee = ec + (i & (NE - 1));
          f[u] = (i < words && ee < L) ? __hip_atomic_load(flags + (long)(p0 + (i >> lne)) * L + ee, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_WORKGROUP)
                                       : PERM_PUBLISHED;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int i = i0 + u * PERM_THREADS + threadIdx.x;
          if (i < words) s_stage[i] = (int32_t)f[u];
        }
      }
      lds_barrier();
      const int per = (nb + R - 1) >> lr, pa = min(nb, rr * per), pe = min(nb, pa + per);
      int mine = 0;
      if (col)
        for (int p = pa; p < pe; ++p) {
          uint32_t f = (uint32_t)s_stage[(p << lne) + jc];
          if (!(f & PERM_PUBLISHED)) {
            f = flag_wait_slow(flags + (long)(p0 + p) * L + e);
            stuck |= !(f & PERM_PUBLISHED);
            s_stage[(p << lne) + jc] = (int32_t)f;
          }
          mine += min((int)(f & PERM_VALUE), cap);
        }
      int incl = mine;
      for (int d = 1; d < R; d <<= 1) {
        const int y = __shfl_up(incl, d, R);
        if (rr >= d) incl += y;
      }
      if (col) {
        int base = carry + incl - mine;
        for (int p = pa; p < pe; ++p) {
          tilebase[(long)(p0 + p) * L + e] = base;
          base += min((int)((uint32_t)s_stage[(p << lne) + jc] & PERM_VALUE), cap);
        }
      }
      carry += __shfl(incl, R - 1, R);
    }
    if (col && rr == 0) run[e] = carry;
  }
  lds_barrier();
  expert_offsets(L, capacity, run, counts, offsets, err, s_wsum);
  if (stuck) set_err(err, MOE_DEVERR_WORKSPACE);
  // the state back to zero for the next call (every tile has published and
  // counted itself finished; the stream orders the next call after this one)
  const long nflags = (long)ntiles * L;
  for (long i = threadIdx.x; i < nflags; i += PERM_THREADS) flags[i] = 0u;
  if (threadIdx.x == 0) *done = 0u;
}

// Copy (OUT 0) or MX-quantize (OUT 1: MXFP8, 2: MXFP4) token t's row to the
// rows `dest` of its slots (lane k < K: slot k's row, or -1), k order; the
// first 8 KiB of the row are already in v.  One wavefront.
template <int OUT>
__device__ __forceinline__ void permute_rows(int t, int K, int l, int dest, int npiece, int row_bytes,
                                             const uint8_t* __restrict__ src, u32x4 (&v)[8],
                                             uint8_t* __restrict__ x_perm, uint8_t* __restrict__ x_scales,
                                             int32_t* __restrict__ row_to_slot) {
  const uint64_t bits = wave_ballot(dest >= 0);
  if (!bits) return;
  // rows move in 1 KiB pieces (16 bytes per lane), eight pieces in flight
  for (int p0 = 0; p0 < npiece; p0 += 8) {
    if (p0 > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (p0 + j) * 1024 + l * 16;
        v[j] = (p0 + j < npiece && off < row_bytes) ? *(const u32x4*)(src + off) : u32x4{0, 0, 0, 0};
      }
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

// ---------------------------------------------------------------------------
// k_permute: 4 tokens per workgroup, one wavefront each.
// ---------------------------------------------------------------------------
// PERM_FOLD_WORDS: with ntiles * L at most this (and L <= 64), the count
// kernel leaves each tile's counts in the tile-base array and every permute
// workgroup turns them into the bases and offsets itself (in LDS, while its
// rows load), so the count kernel needs no scan.
#define PERM_FOLD_WORDS 256
template <int OUT>  // OUT 0: copy rows (bf16 or fp32, row_bytes), 1: MXFP8-, 2: MXFP4-quantize bf16 rows
__global__ __launch_bounds__(256) void k_permute(int T, int K, int e0, int L, int TT, int ntiles, bool fold,
                                                 int64_t capacity, int row_bytes, const uint8_t* __restrict__ x,
                                                 const int16_t* __restrict__ ids,
                                                 const int32_t* __restrict__ tilebase,
                                                 const int32_t* __restrict__ rank, int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets, uint8_t* __restrict__ x_perm,
                                                 uint8_t* __restrict__ x_scales, int32_t* __restrict__ row_to_slot,
                                                 int32_t* __restrict__ slot_to_row, int32_t* err) {
  __shared__ int32_t s_tb[PERM_FOLD_WORDS];  // fold: tile counts, then their exclusive prefix over the tiles
  __shared__ int32_t s_off[64];              // fold: expert offsets
  const int l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool active = t < T;
  const int nw = ntiles * L;
  const long f = (long)t * K + l;
  int le = -1;
  if (active && l < K) {
    const int id = ids[f];
    if (id >= e0 && id < e0 + L) le = id - e0;
  }
  const int cw = (fold && (int)threadIdx.x < nw) ? tilebase[threadIdx.x] : 0;
  const long tl = (long)(t / TT) * L + le;
  // the slot's row within its tile and expert (and, without fold, its
  // expert's offset + its tile's base), issued before the row loads
  int64_t base = 0;
  if (le >= 0) base = (int64_t)rank[f] + (fold ? 0 : (int64_t)offsets[le] + tilebase[tl]);
  const uint64_t local = wave_ballot(le >= 0);
  // the row's first 8 KiB in flight while the bases are formed
  const uint8_t* src = x + (long)t * row_bytes;
  const int npiece = (row_bytes + 1023) / 1024;
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int off = j * 1024 + l * 16;
    v[j] = (local && j < npiece && off < row_bytes) ? *(const u32x4*)(src + off) : u32x4{0, 0, 0, 0};
  }
  if (fold) {
    if ((int)threadIdx.x < nw) s_tb[threadIdx.x] = cw;
    __syncthreads();
    if (threadIdx.x < 64) {  // wavefront 0, lane e: expert e's prefix over the tiles, then the offsets
      int tot = 0;
      if (l < L)
        for (int p = 0; p < ntiles; ++p) {
          const int c = s_tb[p * L + l];
          s_tb[p * L + l] = tot;
          tot += c;
        }
      const int incl = wave_incl_scan(tot);
      s_off[l] = incl - tot;
      if (blockIdx.x == 0) {
        if (l < L) {
          counts[l] = tot;
          offsets[l] = incl - tot;
        }
        if (l == 63) {
          offsets[L] = incl;
          if ((int64_t)incl > capacity) set_err(err, MOE_DEVERR_OVERFLOW);
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  int dest = -1;
  if (l < K) {
    if (le >= 0) {
      const int64_t d = fold ? base + s_off[le] + s_tb[tl] : base;
      dest = (d >= 0 && d < capacity) ? (int)d : -1;
    }
    slot_to_row[f] = dest;
  }
  permute_rows<OUT>(t, K, l, dest, npiece, row_bytes, src, v, x_perm, x_scales, row_to_slot);
}

// ---------------------------------------------------------------------------
// k_permute_small: batches of at most PERM_SMALL_SLOTS slots and at most 64
// local experts in one kernel, no workspace.  A workgroup of PSM_TOK
// wavefronts takes PSM_TOK consecutive tokens (one per wavefront) and, while
// its rows load, counts every slot of the batch itself (the ids are a few
// KiB, read from L2 by every workgroup): per local expert, the slots in the
// whole batch (the counts and offsets) and those before its first slot.  A
// slot's row is its expert's offset + the expert's slots before the
// workgroup + those of the workgroup's earlier tokens + its rank among the
// token's slots of that expert: the same rows as the two-kernel path (slot
// order within each expert), with no communication between workgroups.
// ---------------------------------------------------------------------------
#define PERM_SMALL_SLOTS 16384
#define PSM_TOK 16
template <int OUT>
__global__ __launch_bounds__(64 * PSM_TOK) void k_permute_small(int T, int K, int E_global, int e0, int L,
                                                                int64_t capacity, int row_bytes,
                                                                const uint8_t* __restrict__ x,
                                                                const int16_t* __restrict__ ids,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                uint8_t* __restrict__ x_perm,
                                                                uint8_t* __restrict__ x_scales,
                                                                int32_t* __restrict__ row_to_slot,
                                                                int32_t* __restrict__ slot_to_row, int32_t* err) {
  __shared__ int32_t s_tot[PSM_TOK][64];  // per wavefront: its share of the batch's slots, per expert
  __shared__ int32_t s_bef[PSM_TOK][64];  // ... of those before the workgroup's first slot
  __shared__ int32_t s_tok[PSM_TOK][64];  // per token of the workgroup
  __shared__ int32_t s_base[64];          // offset + the expert's slots before the workgroup
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * PSM_TOK + w;
  const bool active = t < T;
  const long nslot = (long)T * K, s0 = (long)blockIdx.x * PSM_TOK * K;
  s_tot[w][l] = 0;
  s_bef[w][l] = 0;
  s_tok[w][l] = 0;
  const long f = (long)t * K + l;
  int le = -1;
  if (active && l < K) {
    const int id = ids[f];
    if (id >= e0 && id < e0 + L && id < E_global) le = id - e0;
  }
  const uint64_t local = wave_ballot(le >= 0);
  // the batch's ids first (slot u * 64 * PSM_TOK + 64 w + l in id[u]), then
  // the row's first 8 KiB: the count waits only for the ids, which were
  // issued first, while the row is still loading
  // (buffer loads, unconditional: reads past a buffer's end return zeros
  // without touching memory, so the compiler sees no branches and waits for
  // the ids alone)
  int id[PERM_SMALL_SLOTS / (64 * PSM_TOK)];
  const __amdgpu_buffer_rsrc_t rid =
      __builtin_amdgcn_make_buffer_rsrc((void*)ids, (short)0, (int)(nslot * 2), 0x00020000);
#pragma unroll
  for (int u = 0; u < PERM_SMALL_SLOTS / (64 * PSM_TOK); ++u) {
    const int i = u * 64 * PSM_TOK + w * 64 + l;
    id[u] = (int)(int16_t)__builtin_amdgcn_raw_buffer_load_b16(rid, 2 * i, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the id loads ahead of the row loads
  const uint8_t* src = x + (long)(active ? t : 0) * row_bytes;
  const int npiece = (row_bytes + 1023) / 1024;
  // the row's bytes, or none for a token without a local slot
  const __amdgpu_buffer_rsrc_t rrow =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, local ? row_bytes : 0, 0x00020000);
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(rrow, j * 1024 + l * 16, 0, 0);
  lds_barrier();  // the counts are zero (the row loads stay in flight)
  bool bad = false;
#pragma unroll
  for (int u = 0; u < PERM_SMALL_SLOTS / (64 * PSM_TOK); ++u) {
    const long i = (long)u * 64 * PSM_TOK + w * 64 + l;
    if (i >= nslot) id[u] = -1;
    bad |= id[u] < -1 || id[u] >= E_global;
    if (id[u] >= e0 && id[u] < e0 + L && id[u] < E_global) {
      __hip_atomic_fetch_add(&s_tot[w][id[u] - e0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (i < s0) __hip_atomic_fetch_add(&s_bef[w][id[u] - e0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if (blockIdx.x == 0 && wave_ballot(bad) && l == 0) set_err(err, MOE_DEVERR_BAD_ID);
  if (le >= 0) __hip_atomic_fetch_add(&s_tok[w][le], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  lds_barrier();
  if (w == 0) {  // lane e: expert e's total, offset and base
    int tot = 0, bef = 0;
    if (l < L)
      for (int u = 0; u < PSM_TOK; ++u) {
        tot += s_tot[u][l];
        bef += s_bef[u][l];
      }
    const int incl = wave_incl_scan(tot);
    s_base[l] = incl - tot + bef;
    if (blockIdx.x == 0) {
      if (l < L) {
        counts[l] = tot;
        offsets[l] = incl - tot;
      }
      if (l == 63) {
        offsets[L] = incl;
        if ((int64_t)incl > capacity) set_err(err, MOE_DEVERR_OVERFLOW);
      }
    }
  }
  lds_barrier();
  if (!active) return;
  int dest = -1;
  if (l < K) {
    if (le >= 0) {
      int pre = 0;  // the expert's slots in the workgroup's earlier tokens
      for (int u = 0; u < w; ++u) pre += s_tok[u][le];
      int nbits = 0;
      while ((1 << nbits) < L) ++nbits;
      const uint64_t peers = same_expert_lanes(le, local, nbits);
      const int64_t d = (int64_t)s_base[le] + pre + __builtin_popcountll(peers & ((1ull << l) - 1));
      dest = (d >= 0 && d < capacity) ? (int)d : -1;
    }
    slot_to_row[f] = dest;
  }
  permute_rows<OUT>(t, K, l, dest, npiece, row_bytes, src, v, x_perm, x_scales, row_to_slot);
}

// counts and offsets of an empty batch
__global__ void k_zero_counts(int L, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= L; e += blockDim.x) {
    if (e < L) counts[e] = 0;
    offsets[e] = 0;
  }
}

hipError_t launch_permute(int T, int H, int K, int E_global, int e0, int L, int64_t capacity,
                          int x_dtype, int out_dtype, const void* x, const int16_t* ids,
                          int32_t* counts, int32_t* offsets, void* x_perm, uint8_t* x_scales,
                          int32_t* row_to_slot, int32_t* slot_to_row, int32_t* err, void* ws,
                          hipStream_t s) {
  if (T == 0) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(256), 0, s, L, counts, offsets);
    return hipGetLastError();
  }
  const int row_bytes = H * (x_dtype == MOE_F32 ? 4 : 2);
  if ((long)T * K <= PERM_SMALL_SLOTS && L <= 64) {  // one kernel, no workspace
    const dim3 g((T + PSM_TOK - 1) / PSM_TOK), b(64 * PSM_TOK);
#define PERMUTE_SMALL_ARGS                                                                                    \
  T, K, E_global, e0, L, capacity, row_bytes, (const uint8_t*)x, ids, counts, offsets, (uint8_t*)x_perm,      \
      x_scales, row_to_slot, slot_to_row, err
    if (out_dtype == MOE_MXFP8)
      hipLaunchKernelGGL(k_permute_small<1>, g, b, 0, s, PERMUTE_SMALL_ARGS);
    else if (out_dtype == MOE_MXFP4)
      hipLaunchKernelGGL(k_permute_small<2>, g, b, 0, s, PERMUTE_SMALL_ARGS);
    else
      hipLaunchKernelGGL(k_permute_small<0>, g, b, 0, s, PERMUTE_SMALL_ARGS);
#undef PERMUTE_SMALL_ARGS
    return hipGetLastError();
  }
  const int TT = permute_tile_tokens(T, K, L);
  const int ntiles = (T + TT - 1) / TT;
  const PermuteWs w = permute_ws(ws, ntiles, L);
  // at most (PERM_WAVES + 1) * MOE_MAX_L * 4 + 32 KiB = 104 KiB
  const size_t lds = (size_t)((PERM_WAVES + 1) * L) * sizeof(int32_t) + PERM_CHUNK * sizeof(int16_t);
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_count_scan, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)((PERM_WAVES + 1) * MOE_MAX_L * sizeof(int32_t) + PERM_CHUNK * sizeof(int16_t)));
    return true;
  }();
  (void)attr_done;
  const bool fold = (long)ntiles * L <= PERM_FOLD_WORDS && L <= 64;
  hipLaunchKernelGGL(k_count_scan, dim3(ntiles), dim3(PERM_THREADS), lds, s, T, K, E_global, e0, L, TT, ntiles, fold,
                     capacity, ids,
                     w.done, w.flags, w.tilebase, w.rank, counts, offsets, err);
  const dim3 g((T + 3) / 4), b(256);
#define PERMUTE_ARGS                                                                                          \
  T, K, e0, L, TT, ntiles, fold, capacity, row_bytes, (const uint8_t*)x, ids, (const int32_t*)w.tilebase,     \
      (const int32_t*)w.rank, counts, offsets, (uint8_t*)x_perm, x_scales, row_to_slot, slot_to_row, err
  if (out_dtype == MOE_MXFP8)
    hipLaunchKernelGGL(k_permute<1>, g, b, 0, s, PERMUTE_ARGS);
  else if (out_dtype == MOE_MXFP4)
    hipLaunchKernelGGL(k_permute<2>, g, b, 0, s, PERMUTE_ARGS);
  else
    hipLaunchKernelGGL(k_permute<0>, g, b, 0, s, PERMUTE_ARGS);
#undef PERMUTE_ARGS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// moe_permute_noalloc: the permute with its workspace in a fixed device array
// (for callers that cannot allocate).  Each GPU the library runs on holds its
// own copy of `scratch` until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns for the current device
// (the array's name on the host is a stand-in, not a device address).  Every
// call first clears the counter and tile counts with a fill kernel (no memset
// node, so the call can be captured in a graph), then runs the two kernels.
// Calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
#define PERMUTE_SCRATCH_BYTES ((size_t)16 << 20)
static __device__ __align__(256) uint8_t scratch[PERMUTE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

size_t permute_noalloc_max_bytes() { return PERMUTE_SCRATCH_BYTES; }

__global__ void k_fill_u32(uint32_t* __restrict__ p, long n, uint32_t v) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_permute_noalloc(int T, int H, int K, int E_global, int e0, int L, int64_t capacity, int x_dtype,
                                  int out_dtype, const void* x, const int16_t* ids, int32_t* counts,
                                  int32_t* offsets, void* x_perm, uint8_t* x_scales, int32_t* row_to_slot,
                                  int32_t* slot_to_row, int32_t* err, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current: the device address of its copy
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  void* ws = g_scratch_ptr[dev];
  const long state_words = (long)(permute_state_bytes(T, K, L) / 4);
  if (T > 0) {
    const long blocks = (state_words + 255) / 256;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, (uint32_t*)ws,
                       state_words, 0u);
  }
  return launch_permute(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, x, ids, counts, offsets, x_perm,
                        x_scales, row_to_slot, slot_to_row, err, ws, s);
}

}  // namespace moe
