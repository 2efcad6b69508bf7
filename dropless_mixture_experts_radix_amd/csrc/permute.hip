// Device count, scan and permute of the routed token rows into expert order.
//
// Sparser-MoE page (harryzhou2000), "Remove work that has no selected route":
// local pre-processing visits only the selected local slots of a token (a
// wavefront ballot over its K slots, iterating the set bits).  bpdata article,
// "Optimization 1: Grouped GEMM": expert token counts stay on the device.
//
// Two kernels, no host round trip:
//  k_count_scan  per tile of TT tokens: per-local-expert histogram (LDS), the
//                stable rank of every local slot among the tile's slots of
//                the same expert (wavefront ballots, flat slot order), and a
//                single-pass decoupled look-back scan across tiles: per-tile
//                expert bases; the last tile writes counts[L], offsets[L+1]
//                and the overflow flag.
//  k_permute     one wavefront per token: ballot over its K slots, read the
//                row once, write it to each selected local expert row.
#include "moe_internal.h"

#include <mutex>

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
// Workspace of the permute (byte offsets; ntiles tiles of TT tokens):
//   [0, 256)                    the tile ticket counter (uint32)
//   [256, ...)                  look-back flags [ntiles][L] uint32
//   next 256-byte boundary      each slot's row within its expert [T*K] int32
// All of it is zero between calls: the caller zero-fills the workspace once,
// and k_permute returns everything a call wrote to zero (the flags, the
// counter, and each slot's row once it has been read), so calls of different
// shapes can share one workspace.
// ---------------------------------------------------------------------------
struct PermuteWs {
  uint32_t* ticket;
  uint32_t* flags;
  int32_t* rank;
};

static inline size_t ws_round(size_t v) { return (v + 255) / 256 * 256; }

static PermuteWs permute_ws(void* ws, int ntiles, int L) {
  uint8_t* b = (uint8_t*)ws;
  PermuteWs w;
  w.ticket = (uint32_t*)b;
  w.flags = (uint32_t*)(b + 256);
  w.rank = (int32_t*)(b + 256 + ws_round((size_t)ntiles * L * 4));
  return w;
}

size_t permute_state_bytes(int T, int K, int L) {
  const int TT = permute_tile_tokens(T, K);
  const size_t ntiles = (size_t)(T > 0 ? (T + TT - 1) / TT : 0);
  return 256 + ws_round(ntiles * L * 4);
}

size_t permute_workspace_bytes(int T, int K, int L) {
  const int TT = permute_tile_tokens(T, K);
  const size_t ntiles = (size_t)(T > 0 ? (T + TT - 1) / TT : 0);
  return 256 + ws_round(ntiles * L * 4) + ws_round((size_t)T * K * 4);
}

// A look-back flag: the tile's count of one expert (AGG: its own slots; INCL:
// its slots and every earlier tile's) in the low 30 bits.  0: not yet known.
#define PERM_AGG (1u << 30)
#define PERM_INCL (2u << 30)
#define PERM_VALUE ((1u << 30) - 1)
// bound on the polls of one flag (each after s_sleep 2, about 0.1 us): a
// predecessor tile publishes its count within microseconds of starting, so
// the bound is only reached when the workspace was not zero-filled; the
// tile then reports MOE_DEVERR_WORKSPACE instead of waiting forever
#define PERM_MAX_POLLS (1 << 20)

__device__ __forceinline__ uint32_t flag_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// k_count_scan: grid = ntiles, 256 threads.  Dynamic LDS: cnt[4][L] + tot[L]
// + base[L] + rank[TT*K] int32.
//
// A workgroup takes the next tile from the ticket counter (so every earlier
// tile belongs to a workgroup that has started), counts its local slots per
// expert (LDS histograms; the stable rank of each slot among the tile's slots
// of its expert from wavefront ballots, flat slot order), and then finds each
// expert's count in all earlier tiles by a decoupled look-back (Merrill and
// Garland, "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016):
// it publishes its own count (AGG), adds the predecessors' published counts
// until one of them is inclusive (INCL), and publishes its inclusive count.
// The exclusive count is the tile's base for that expert; each local slot's
// row within its expert (base + its rank in the tile) goes to `rank`.  The
// last tile's inclusive counts are the expert totals: it writes counts,
// offsets (their exclusive scan) and the overflow flag.  One pass over the
// ids, no second kernel over the tile histograms.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_count_scan(int T, int K, int E_global, int e0, int L, int TT, int ntiles,
                                                    int64_t capacity, const int16_t* __restrict__ ids,
                                                    uint32_t* __restrict__ ticket, uint32_t* __restrict__ flags,
                                                    int32_t* __restrict__ rank,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* err) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;              // [4][L]
  int32_t* tot = lds + 4 * L;      // [L] inclusive counts (last tile)
  int32_t* base = lds + 5 * L;     // [L] exclusive counts: the tile's base per expert
  int32_t* srank = lds + 6 * L;    // [TT*K]
  __shared__ int s_tile;
  __shared__ int s_wsum[4];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (threadIdx.x == 0) s_tile = (int)atomicAdd(ticket, 1u);
  for (int i = threadIdx.x; i < 4 * L; i += 256) cnt[i] = 0;
  __syncthreads();
  const int tile = s_tile;
  if ((unsigned)tile >= (unsigned)ntiles) {  // the counter was not zero: a workspace that was not zero-filled
    if (threadIdx.x == 0) set_err(err, MOE_DEVERR_WORKSPACE);
    return;
  }
  const long f0 = (long)tile * TT * K;
  long fend = f0 + (long)TT * K;
  const long ftot = (long)T * K;
  if (fend > ftot) fend = ftot;
  const int nslot = (int)(fend - f0);
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
  // per-wave bases, the tile's count of each expert, the look-back
  bool stuck = false;
  for (int e = threadIdx.x; e < L; e += 256) {
    const int c0 = cnt[e], c1 = cnt[L + e], c2 = cnt[2 * L + e], c3 = cnt[3 * L + e];
    const int agg = c0 + c1 + c2 + c3;
    cnt[e] = 0;
    cnt[L + e] = c0;
    cnt[2 * L + e] = c0 + c1;
    cnt[3 * L + e] = c0 + c1 + c2;
    uint32_t* mine = flags + (long)tile * L + e;
    int excl = 0;
    if (tile == 0) {
      flag_store(mine, PERM_INCL | (uint32_t)agg);
    } else {
      flag_store(mine, PERM_AGG | (uint32_t)agg);
      for (int p = tile - 1; p >= 0; --p) {
        const uint32_t* fp = flags + (long)p * L + e;
        uint32_t f = flag_load(fp);
        for (int polls = 0; f == 0u; ++polls) {
          if (polls >= PERM_MAX_POLLS) { stuck = true; break; }
          __builtin_amdgcn_s_sleep(2);
          f = flag_load(fp);
        }
        if (stuck) break;
        excl += (int)(f & PERM_VALUE);
        if ((f & ~PERM_VALUE) == PERM_INCL) break;
      }
      flag_store(mine, PERM_INCL | (uint32_t)(excl + agg));
    }
    // a count outside [0, T*K] can only come from flags that were not zero
    // before the call: report it, and keep the offsets monotone and >= 0
    const int tk = T * K;
    if (excl < 0 || excl > tk - agg) {
      stuck = true;
      excl = excl < 0 ? 0 : tk - agg;
    }
    base[e] = excl;
    tot[e] = excl + agg;
  }
  if (stuck) set_err(err, MOE_DEVERR_WORKSPACE);
  __syncthreads();
  for (int sl = threadIdx.x; sl < nslot; sl += 256) {
    const int id = ids[f0 + sl];
    int r = 0;
    if (id >= e0 && id < e0 + L && id < E_global)
      r = base[id - e0] + srank[sl] + cnt[(sl / part) * L + (id - e0)];
    rank[f0 + sl] = r;
  }
  if (tile != ntiles - 1) return;
  // the last tile: expert totals -> counts, offsets (exclusive scan), overflow
  const int per = (L + 255) / 256;
  const int b0 = threadIdx.x * per;
  int loc = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < L) loc += tot[b0 + i];
  const int incl = wave_incl_scan(loc);
  if (l == 63) s_wsum[w] = incl;
  __syncthreads();
  int run = incl - loc;
  for (int i = 0; i < w; ++i) run += s_wsum[i];
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < L) {
      counts[e] = tot[e];
      offsets[e] = run;
      run += tot[e];
    }
  }
  if (threadIdx.x == 255) {
    offsets[L] = run;
    if ((int64_t)run > capacity) set_err(err, MOE_DEVERR_OVERFLOW);
  }
}

// counts and offsets of an empty batch
__global__ void k_zero_counts(int L, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= L; e += blockDim.x) {
    if (e < L) counts[e] = 0;
    offsets[e] = 0;
  }
}

// ---------------------------------------------------------------------------
// k_permute: one wavefront per token, 4 per workgroup.  It also returns the
// workspace to zero for the next call: the look-back state of k_count_scan
// (which has finished: same stream) and each slot's row once read.
// ---------------------------------------------------------------------------
template <int OUT>  // OUT 0: copy rows (bf16 or fp32, row_bytes), 1: MXFP8-, 2: MXFP4-quantize bf16 rows
__global__ __launch_bounds__(256) void k_permute(int T, int K, int e0, int L, int TT, int64_t capacity,
                                                 int row_bytes, const uint8_t* __restrict__ x,
                                                 const int16_t* __restrict__ ids,
                                                 int32_t* __restrict__ rank,
                                                 const int32_t* __restrict__ offsets,
                                                 uint8_t* __restrict__ x_perm, uint8_t* __restrict__ x_scales,
                                                 int32_t* __restrict__ row_to_slot,
                                                 int32_t* __restrict__ slot_to_row, uint32_t* __restrict__ ticket,
                                                 uint32_t* __restrict__ flags, long nflags) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < nflags; i += (long)gridDim.x * 256) flags[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0u;
  if (t >= T) return;
  int dest = -1;
  if (l < K) {
    const long f = (long)t * K + l;
    const int id = ids[f];
    if (id >= e0 && id < e0 + L) {
      const int le = id - e0;
      const int64_t d = (int64_t)offsets[le] + rank[f];
      dest = (d >= 0 && d < capacity) ? (int)d : -1;
    }
    rank[f] = 0;
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

hipError_t launch_permute(int T, int H, int K, int E_global, int e0, int L, int64_t capacity,
                          int x_dtype, int out_dtype, const void* x, const int16_t* ids,
                          int32_t* counts, int32_t* offsets, void* x_perm, uint8_t* x_scales,
                          int32_t* row_to_slot, int32_t* slot_to_row, int32_t* err, void* ws,
                          hipStream_t s) {
  if (T == 0) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(256), 0, s, L, counts, offsets);
    return hipGetLastError();
  }
  const int TT = permute_tile_tokens(T, K);
  const int ntiles = (T + TT - 1) / TT;
  const PermuteWs w = permute_ws(ws, ntiles, L);
  const size_t lds = (size_t)(6 * L + TT * K) * sizeof(int32_t);
  hipLaunchKernelGGL(k_count_scan, dim3(ntiles), dim3(256), lds, s, T, K, E_global, e0, L, TT, ntiles, capacity, ids,
                     w.ticket, w.flags, w.rank, counts, offsets, err);
  const int row_bytes = H * (x_dtype == MOE_F32 ? 4 : 2);
  const dim3 g((T + 3) / 4), b(256);
  const long nflags = (long)ntiles * L;
#define PERMUTE_ARGS                                                                                                 \
  T, K, e0, L, TT, capacity, row_bytes, (const uint8_t*)x, ids, w.rank,                                          \
      (const int32_t*)offsets, (uint8_t*)x_perm, x_scales, row_to_slot, slot_to_row, w.ticket, w.flags, nflags
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
// call first clears the look-back state with a fill kernel (no memset node,
// so the call can be captured in a graph), then runs the usual two kernels.
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
