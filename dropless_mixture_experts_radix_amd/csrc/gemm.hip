// Ragged grouped GEMMs of the expert SwiGLU MLP (fp32 and bf16).
//
// bpdata article, "Optimization 1: Grouped GEMM": all expert matmuls in one
// kernel, each with its expert's actual token count, computing only valid
// regions, with no device-to-host counts and no worst-case padding.
//
// Every workgroup builds the tile schedule from `offsets` on the device: expert
// e owns ceil(m_e/BM) x (N/BN) output tiles (none when m_e = 0), ordered in
// groups of 4 row tiles (all column tiles of a group, row tile fastest), and a
// persistent grid walks them.  Workgroups are assigned to the 8 XCDs in turn, so
// workgroup b works on the virtual slot (b % 8) * (G/8) + b/8: the 32 CUs of an
// XCD take consecutive tiles and share their A and B panels in that XCD's L2.
#include "gemm_common.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 grouped GEMM: out tile 256 x 256, k step 32, 512 threads = 8 wavefronts
// as 2 (rows) x 4 (columns), two per SIMD, each wavefront 128 x 64 = 4 x 2
// tiles of v_mfma_f32_32x32x16_bf16.
//
// What bounds this loop on gfx950 is how many operand bytes are in flight
// between global memory and LDS: a k step of a 256 x 256 tile needs 32 KiB,
// and under the load of all CUs the latency of a global read is of the order
// of a microsecond, several k steps.  So the tiles go straight from global
// memory into LDS (buffer loads with the LDS destination, no registers), into
// a ring of 4 LDS stages filled three k steps ahead.  Two wavefronts share
// each SIMD, so while one waits for its loads to be accepted or for a barrier
// the other keeps the matrix core busy.  A wavefront tile of 128 x 64 reads
// 12 KiB of MFMA fragments per k step from LDS for its 16 MFMAs.
//
// Pipeline: the wavefronts form two groups (0-3 and 4-7, one of each per
// SIMD) that alternate between a memory phase (read both sub-steps' fragments
// of step kt from stage kt % 4, load step kt+3 into stage (kt+3) % 4, wait for
// this wavefront's loads of step kt+1) and a compute phase (the 16 MFMAs of
// step kt), one phase apart, with a barrier of all 8 wavefronts between
// phases; the k loop below spells out which stage is free when.
//
// LDS layout: stage s at s * 32 KiB, A rows then B rows (256 each, 64 bytes:
// 32 k values); a 1 KiB block holds 16 rows and is written by one load
// instruction (lane i -> bytes 16i..16i+15), and the 16-byte chunk c of row r
// sits at chunk position c ^ swz4(r), so the 8 (or 16) lanes served together
// by a fragment read hit distinct banks.  A is [rows][Kd] (EPI 1: x_perm) or
// k-blocked [Kd/32][capacity][32] (EPI 0: the activations); B is the prepared
// weight panel of 256 output columns, k-blocked [Kd/32][256][32], so a k step
// of B is one contiguous 16 KiB block.  Buffer loads return zeros past the
// tile's rows.  Prefetch indices are clamped to the last k step of the range.
//
// Work units.  With G persistent workgroups and `total` tiles, the first
// floor(total/G)*G tiles run whole (data parallel).  The `left` tiles of a last,
// partial round would leave most CUs idle, so when left*2 <= GEMM_SPLIT_UNITS
// each of them is split into S pieces along k (split-K), S as large as fits
// the CUs and the partial buffer, each piece a whole number of 4-step groups.
// A piece writes its fp32 partial tile to `part`; k_splitk_reduce then sums the
// S partials of a tile in piece order (the result does not depend on timing)
// and applies the epilogue.
// EPI 0: out[row][col] = bf16(acc)                                   (N columns)
// EPI 1: gate/up chunks of 32 columns are interleaved in B; out = k-blocked
//        activations [N/64][capacity][32], a[row][j] = bf16(silu(gate) * up)
// EPI 3: (backward) h = x_perm . W1 recomputed: A as EPI 1, out = k-blocked
//        [N/32][capacity][32] in the prepared (gate/up interleaved) order
// EPI 4: (backward) A = d_y row-major, B = the prepared W2^T panels (N = F
//        columns): acc = d_a; with g, u read from `aux` (EPI 3's output) the
//        epilogue stores d_h = [d_a u silu'(g), d_a silu(g)] k-blocked
//        [2N/32][capacity][32] in natural column order (gates, then ups)
// EPI 5: (backward) weight gradient dW[e] = P_e^T Q_e over expert e's own
//        rows: A = P^T and B = Q^T in token-blocked form [blocks][I or J][32
//        tokens] (each expert's rows padded with zeros to a multiple of 128,
//        block prefix `offsets` = pb[L+1]), `capacity` = I output rows, N = J
//        columns; tiles (expert, I tile, J tile) of experts with rows, each over
//        its expert's blocks (no split); out = fp32 [L][I][J]
// EPI 2: the router projection, one dense GEMM of the `capacity` = T token
//        rows of x [T][Kd] with the prepared router weights [ceil(N/32)*32][Kd]
//        (row-major, loaded like A), N = E output columns.  Every tile is cut
//        into L pieces along k and piece q writes its fp32 partial logits to
//        part[q][T][N]; the selection kernel sums the L partials of a token in
//        piece order.  No expert schedule, no reduce kernel.
// ---------------------------------------------------------------------------
#define GB_BM 256
#define GB_BN 256
#define GB_BK 32
#define GB_THREADS 512
#define GB_X_OFF 32768              // the 64 extra A rows of a tall tile, after A and B
#define GB_STAGE_BYTES (GB_X_OFF + 4096)
#define GB_TALL 64                  // rows a tall tile has beyond GB_BM
// a split-K partial tile: the 8 wavefront parts of 128 x 64, then the 32 x 64
// extra-row blocks of the 8 wavefronts (tall tiles)
#define GB_PART_X (GB_BM * GB_BN)
#define GB_PART_FLOATS (GB_PART_X + 8 * 2048)

// split plan of the bf16 kernel: pieces are whole groups of 4 k steps
__device__ __forceinline__ SplitPlan gb_split_plan(int total, int G, int Kd) {
  return split_plan(total, G, Kd / 64);
}
// whether a bf16 GEMM over Kd may split a tile (else its reduce has no work)
static inline bool gb_may_split(int Kd) { return split_max_pieces(Kd / 64) >= 2; }

// Tile schedule and split plan of the bf16 kernel on a grid of G workgroups,
// with tall tiles: an expert takes the fewest tiles of at most GB_BM + GB_TALL
// rows (tall tiles of GB_BM + up to GB_TALL rows where GB_BM rows per tile do
// not cover its rows).
__device__ __forceinline__ SplitPlan gb_schedule(int L, int64_t capacity, int NT, int Kd, int G,
                                                 const int32_t* __restrict__ offsets, int32_t* s_pre,
                                                 int32_t* s_tmp) {
  build_schedule(L, capacity, GB_BM, NT, offsets, s_pre, s_tmp, GB_TALL);
  return gb_split_plan(s_pre[L], G, Kd);
}

// Epilogue of rows [i0, i0+NI) x 32 of one wavefront's 128 x 64 part of a
// tile (MFMA D layout: lane l holds column l%32, rows 8 (v/4) + 4 (l/32) + v%4
// of each 32 x 32 block).
template <int EPI, int NI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[NI][2], int i0, const TileInfo& ti, int N,
                                           int64_t capacity, int wm, int wn, int g, int r32,
                                           bf16_t* __restrict__ out, const bf16_t* __restrict__ aux) {
  const int col0 = ti.nt * GB_BN;
  // the lane's row and column offsets are made opaque here, so the compiler
  // cannot hoist the 16 row numbers per block out of the persistent loop into
  // registers held across the k loop (where they would be spilled)
  asm volatile("" : "+v"(g), "+v"(r32));
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int rb = wm * 128 + (i0 + ii) * 32;
    if (rb >= ti.rows) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = rb + 8 * (v >> 2) + 4 * g + (v & 3);
      if (row >= ti.rows) continue;
      const long grow = ti.row0 + row;
      if (EPI == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) out[grow * N + col] = (bf16_t)f32_to_bf16(acc[ii][j][v]);
        }
      } else if (EPI == 3) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) out[((long)(col >> 5) * capacity + grow) * GB_BK + (col & 31)] = (bf16_t)f32_to_bf16(acc[ii][j][v]);
        }
      } else if (EPI == 5) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) ((float*)out)[((long)ti.e * capacity + grow) * N + col] = acc[ii][j][v];
        }
      } else if (EPI == 4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = col0 + wn * 64 + j * 32 + r32;  // column of d_a
          if (f < N) {
            const int pg = (f >> 5) * 64 + (f & 31);    // gate's prepared column; up's is pg + 32
            const float gt = bf16_to_f32(aux[((long)(pg >> 5) * capacity + grow) * GB_BK + (f & 31)]);
            const float up = bf16_to_f32(aux[((long)((pg >> 5) + 1) * capacity + grow) * GB_BK + (f & 31)]);
            const float da = acc[ii][j][v];
            const float sg = 1.0f / (1.0f + expf(-gt));
            out[((long)(f >> 5) * capacity + grow) * GB_BK + (f & 31)] =
                (bf16_t)f32_to_bf16(da * up * sg * (1.0f + gt * (1.0f - sg)));
            out[((long)((N + f) >> 5) * capacity + grow) * GB_BK + (f & 31)] = (bf16_t)f32_to_bf16(da * gt * sg);
          }
        }
      } else {
        const int jcol = (col0 >> 1) + wn * 32 + r32;
        if (jcol < (N >> 1))
          out[((long)(jcol >> 5) * capacity + grow) * GB_BK + (jcol & 31)] =
              (bf16_t)f32_to_bf16(silu_mul(acc[ii][0][v], acc[ii][1][v]));
      }
    }
  }
}

// fp32 -> bf16 bits with the conversion instruction (round to nearest even)
__device__ __forceinline__ bf16_t bf16_rne(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// silu(g) * u with the reciprocal instruction (about 1 ulp), for the bf16
// activations (well inside their rounding)
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Epilogue of a whole tile's 256 rows (EPI 0 and 1) through LDS: each
// wavefront turns its 128 x 64 part, 32 rows at a time, from the MFMA layout
// (a lane holds one column) into rows in its own 4 KiB of LDS (ring stage 3,
// free between the k loops: the next unit's prologue fills stages 0-2), and
// stores whole 16-byte pieces of rows: EPI 0 writes 128 contiguous bytes of
// each output row, EPI 1 one contiguous 2 KiB block of the k-blocked
// activations per 32 rows (instead of one 2-byte store per value).  The 32
// rows of a lane group g = 1 sit 4 rows below those of g = 0, so their half
// of each LDS row is swapped to keep the two groups on distinct banks.
template <int EPI>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[4][2], const TileInfo& ti, int N,
                                               int64_t capacity, int wm, int wn, int g, int r32, int l,
                                               uint8_t* ep, bf16_t* __restrict__ out) {
  const int col0 = ti.nt * GB_BN;
  // lane-dependent offsets made opaque (as in store_tile): recomputed here
  // rather than hoisted out of the persistent loop and spilled
  asm volatile("" : "+v"(g), "+v"(r32), "+v"(l));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rb = wm * 128 + i * 32;  // the chunk's first row in the tile
    if (rb >= ti.rows) continue;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (EPI == 0) {  // [32 rows][64 columns] bf16, 128-byte rows
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 8 * (v >> 2) + 4 * g + (v & 3);
          *(bf16_t*)(ep + r * 128 + (((j * 32 + r32) * 2) ^ (g << 6))) = bf16_rne(acc[i][j][v]);
        }
    } else {  // [32 rows][32 activations] bf16, 64-byte rows
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * g + (v & 3);
        *(bf16_t*)(ep + r * 64 + ((r32 * 2) ^ (g << 5))) = bf16_rne(silu_mul_fast(acc[i][0][v], acc[i][1][v]));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (EPI == 0) {  // 256 pieces of 16 bytes: row q / 8, piece q % 8
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = k * 64 + l, r = q >> 3, c = q & 7;
        const u32x4 val = *(const u32x4*)(ep + r * 128 + ((c ^ (((r >> 2) & 1) << 2)) << 4));
        const int row = rb + r, col = col0 + wn * 64 + c * 8;
        if (row < ti.rows && col < N) *(u32x4*)(out + (ti.row0 + row) * (long)N + col) = val;
      }
    } else {  // 128 pieces of 16 bytes: row q / 4, piece q % 4
      const int jcol = (col0 >> 1) + wn * 32;  // the wavefront's 32 activations: one k block
      if (jcol < (N >> 1)) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int q = k * 64 + l, r = q >> 2, c = q & 3;
          const u32x4 val = *(const u32x4*)(ep + r * 64 + ((c ^ (((r >> 2) & 1) << 1)) << 4));
          const int row = rb + r;
          if (row < ti.rows) *(u32x4*)(out + ((long)(jcol >> 5) * capacity + ti.row0 + row) * GB_BK + c * 8) = val;
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(GB_THREADS, 1) void k_gemm_bf16(int L, int N, int Kd, int64_t capacity,
                                                             const bf16_t* __restrict__ A,
                                                             const int32_t* __restrict__ offsets,
                                                             const bf16_t* __restrict__ B, bf16_t* __restrict__ out,
                                                             float* __restrict__ part,
                                                             const bf16_t* __restrict__ aux) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* s_pre = (int32_t*)(smem + 4 * GB_STAGE_BYTES);  // [L+1]
  int32_t* s_tmp = s_pre + (L + 1);                         // [8]
  const int NT = (N + GB_BN - 1) / GB_BN;
  const int KT = Kd / GB_BK;
  SplitPlan plan;
  const int NTI = EPI == 5 ? (int)((capacity + GB_BM - 1) / GB_BM) : 1;  // EPI 5: I tiles
  if constexpr (EPI == 2) {  // every tile in L pieces, piece-major unit order
    plan.dp = 0;
    plan.S = L;
    plan.units = (int)((capacity + GB_BM - 1) / GB_BM) * NT * L;
  } else if constexpr (EPI == 5) {  // NTI x NT tiles per expert with rows (pb[e+1] > pb[e]), no split
    build_schedule(L, (int64_t)1 << 40, 1 << 30, NTI * NT, offsets, s_pre, s_tmp, 0);
    plan.dp = plan.units = s_pre[L];
    plan.S = 1;
  } else {
    plan = gb_schedule(L, capacity, NT, Kd, gridDim.x, offsets, s_pre, s_tmp);
  }
  const int tid = threadIdx.x, l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int gp = wm;  // group: wavefronts 0-3 and 4-7, one of each per SIMD
  const int g = l >> 5, r32 = l & 31;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // loads: wavefront wv fills rows [32 wv, 32 wv + 32) of the A and of the B
  // tile of a stage, 2 blocks of 16 rows each; lane l moves row 16q + l/4,
  // chunk (l%4) ^ swz4(l/4) of block q
  const int drow = l >> 2, dch = (l & 3) ^ swz4(drow);
  // fragment reads: A row wm*128 + i*32 + r32, B column wn*128 + j*32 + r32,
  // chunk 2s + g of the k step (sub-step s)
  const int fr0 = r32 * 64 + ((g ^ swz4(r32)) << 4);
  const int fr1 = r32 * 64 + (((2 + g) ^ swz4(r32)) << 4);

  // one work unit: a whole tile or a split-K piece of one
  struct Unit {
    TileInfo ti;
    int piece, k0, k1, akstep, bkstep;
    __amdgpu_buffer_rsrc_t rA, rB;
    int va[2], vb[2], vx[2];
  };
  auto setup = [&](int u) {
    Unit w;
    int tile = u;
    w.piece = -1;
    w.k0 = 0;
    w.k1 = KT;
    if constexpr (EPI == 5) {  // tile u: expert e, I tile fastest, then J tile
      const int e = find_expert(s_pre, L, u);
      const int local = u - s_pre[e];
      w.ti.e = e;
      w.ti.row0 = (local % NTI) * GB_BM;
      w.ti.rows = min(GB_BM, (int)capacity - w.ti.row0);
      w.ti.nt = local / NTI;
      w.k1 = offsets[e + 1] - offsets[e];  // the expert's 32-token blocks (a multiple of 4)
    } else if constexpr (EPI == 2) {  // unit u: piece u / tiles of tile u % tiles
      const int tiles = plan.units / plan.S;
      const int q = u / tiles, nq = KT / 4;
      tile = u - q * tiles;
      w.piece = q;
      w.k0 = 4 * (q * nq / plan.S);
      w.k1 = 4 * ((q + 1) * nq / plan.S);
      w.ti.e = 0;
      w.ti.nt = tile % NT;
      w.ti.row0 = (tile / NT) * GB_BM;
      w.ti.rows = min(GB_BM, (int)capacity - w.ti.row0);
    } else {
      if (u >= plan.dp) {  // split-K piece: k steps [k0, k1), whole groups of 4
        w.piece = u - plan.dp;
        tile = plan.dp + w.piece / plan.S;
        const int q = w.piece % plan.S, nq = KT / 4;
        w.k0 = 4 * (q * nq / plan.S);
        w.k1 = 4 * ((q + 1) * nq / plan.S);
      }
      w.ti = locate_tile(tile, L, capacity, GB_BM, NT, offsets, s_pre, GB_TALL);
    }
    // the unit is the same for every lane: keep it in scalar registers (the
    // buffer resources built from it are scalar operands of the loads)
    w.ti.e = __builtin_amdgcn_readfirstlane(w.ti.e);
    w.ti.row0 = __builtin_amdgcn_readfirstlane(w.ti.row0);
    w.ti.rows = __builtin_amdgcn_readfirstlane(w.ti.rows);
    w.ti.nt = __builtin_amdgcn_readfirstlane(w.ti.nt);
    int eb = 0;  // EPI 5: the expert's first 32-token block
    if constexpr (EPI == 5) eb = __builtin_amdgcn_readfirstlane(offsets[w.ti.e]);
    if constexpr (EPI == 2) {
      // the router weight rows of column tile nt, [rows][Kd]; rows past the
      // prepared ceil(N/32)*32 read as zeros
      const int c0 = w.ti.nt * GB_BN, crows = min(GB_BN, ((N + 31) & ~31) - c0);
      w.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (long)c0 * Kd), (short)0, crows * Kd * 2, 0x00020000);
    } else if constexpr (EPI == 5) {
      // Q^T blocks of the expert: step k at k * N * 32, the tile's columns
      // from nt * 256 within it
      const long b0 = ((long)eb * N + (long)w.ti.nt * GB_BN) * GB_BK;
      w.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(B + b0), (short)0,
                                               (int)(((long)w.k1 * N - (long)w.ti.nt * GB_BN) * GB_BK * 2), 0x00020000);
    } else {
      // the (expert, panel) B tile: KT blocks of [256 columns][32 k]
      w.rB = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(B + ((long)w.ti.e * NT + w.ti.nt) * (long)KT * GB_BN * GB_BK), (short)0,
          KT * GB_BN * GB_BK * 2, 0x00020000);
    }
    if constexpr (EPI == 5)  // P^T blocks of the expert: [k1][capacity = I][32]
      w.rA = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)eb * capacity * GB_BK), (short)0,
                                               (int)((long)w.k1 * capacity * GB_BK * 2), 0x00020000);
    else
      w.rA = EPI != 0 ? __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)w.ti.row0 * Kd), (short)0,
                                                          w.ti.rows * Kd * 2, 0x00020000)
                      : __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(KT * capacity * GB_BK * 2),
                                                          0x00020000);
    // per-lane byte offsets of the 2 A and the 2 B blocks of a wavefront; the
    // k step enters through the scalar offset
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = wv * 32 + q * 16 + drow;
      w.va[q] = (EPI != 0 && EPI != 5) ? (r * Kd + dch * 8) * 2 : ((w.ti.row0 + r) * GB_BK + dch * 8) * 2;
      w.vb[q] = EPI == 2 ? (r * Kd + dch * 8) * 2 : r * 64 + dch * 16;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // the two dwords of the extra rows (tall tile) that this lane moves: row
                                   // GB_BM + 4 (wv + 8h) + l/16, chunk position (l%16)/4, dword l%4
      const int xr = 4 * (wv + 8 * h) + (l >> 4), xc = (((l & 15) >> 2) ^ swz4(xr)) * 16 + (l & 3) * 4;
      w.vx[h] = EPI != 0 ? (GB_BM + xr) * Kd * 2 + xc : ((w.ti.row0 + GB_BM + xr) * GB_BK) * 2 + xc;
    }
    w.akstep = (EPI != 0 && EPI != 5) ? GB_BK * 2 : (int)(capacity * GB_BK * 2);
    w.bkstep = EPI == 2 ? GB_BK * 2 : EPI == 5 ? N * GB_BK * 2 : GB_BN * GB_BK * 2;
    return w;
  };

#define GB_DMA(W, ST, KT_, Q)                                                               \
  {                                                                                         \
    const int kq = (KT_);                                                                   \
    if ((Q) >= 4)                                                                           \
      lds_dma_b32(lds0 + (ST) * GB_STAGE_BYTES + GB_X_OFF + (wv + 8 * ((Q) - 4)) * 256, (W).vx[(Q) - 4], (W).rA, \
                  kq * (W).akstep);                                                         \
    else if ((Q) < 2)                                                                       \
      lds_dma_b128(lds0 + (ST) * GB_STAGE_BYTES + (wv * 2 + (Q)) * 1024, (W).va[Q], (W).rA, kq * (W).akstep); \
    else                                                                                    \
      lds_dma_b128(lds0 + (ST) * GB_STAGE_BYTES + 16384 + (wv * 2 + (Q) - 2) * 1024, (W).vb[(Q) - 2], (W).rB, \
                   kq * (W).bkstep);                                                        \
  }
// the ring prologue of a unit: its steps k0 .. k0+2 into stages 0..2 (a tall
// tile's steps also carry its extra rows: 6 loads per step instead of 4)
#define GB_PROLOGUE(W)                                                                      \
  {                                                                                         \
    if ((W).ti.rows > GB_BM) {                                                              \
      _Pragma("unroll") for (int st = 0; st < 3; ++st) {                                    \
        _Pragma("unroll") for (int q = 0; q < 6; ++q) GB_DMA(W, st, min((W).k0 + st, (W).k1 - 1), q); \
      }                                                                                     \
    } else {                                                                                \
      _Pragma("unroll") for (int st = 0; st < 3; ++st) {                                    \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) GB_DMA(W, st, min((W).k0 + st, (W).k1 - 1), q); \
      }                                                                                     \
    }                                                                                       \
  }
#define GB_READ(FA, FB, ST, FR, NB)                                                         \
  {                                                                                         \
    const uint8_t* pa = smem + (ST) * GB_STAGE_BYTES + wm * 8192 + (FR);                    \
    const uint8_t* pb = smem + (ST) * GB_STAGE_BYTES + 16384 + wn * 4096 + (FR);            \
    _Pragma("unroll") for (int i = 0; i < (NB); ++i) FA[i] = *(const bf16x8*)(pa + i * 2048); \
    if ((NB) > 0) {                                                                         \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) FB[j] = *(const bf16x8*)(pb + j * 2048); \
    }                                                                                       \
  }
#define GB_READX(FX, ST, FR) FX = *(const bf16x8*)(smem + (ST) * GB_STAGE_BYTES + GB_X_OFF + wm * 2048 + (FR));
#define GB_MMA1(FA, FB, T)                                                                  \
  acc[(T) >> 1][(T) & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[(T) >> 1], FB[(T) & 1], acc[(T) >> 1][(T) & 1], 0, 0, 0);
#define GB_FENCE __builtin_amdgcn_sched_barrier(0);

  int u = virtual_block();
  Unit cu;
  if (u < plan.units) {
    cu = setup(u);
    GB_PROLOGUE(cu);
  }
  while (u < plan.units) {
    const int k0 = cu.k0, k1 = cu.k1;
    bf16x8 fa[2][4], fb[2][2], fx[2];  // fragments of both sub-steps of one k step
    f32x16 acc[4][2], accx[1][2];      // accx: the extra rows of a tall tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    accx[0][0] = accx[0][1] = f32x16{};
    // wait for step k0 (the younger steps k0+1, k0+2 may still be loading;
    // loads complete in issue order, and the previous unit's epilogue stores
    // were issued after them)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    // the second group of wavefronts runs one phase behind the first
    if (gp) asm volatile("s_barrier" ::: "memory");
    // Phases, each ended by a barrier of all 8 wavefronts:
    //   memory phase of step kt: read both sub-steps' fragments from stage
    //     kt % 4, load step kt+3 into stage (kt+3) % 4 (read by both groups
    //     in step kt-1, free since the barrier before this phase), then wait
    //     for the reads and for this wavefront's loads of step kt+1;
    //   compute phase of step kt: its 16 MFMAs back to back.
    // Group 0 computes step kt while group 1 reads step kt; group 1 computes
    // step kt while group 0 reads step kt+1.  The stage of step kt+1 is complete
    // for all wavefronts at the barrier that starts group 0's memory phase of
    // step kt+1.
#define GB_KLOOP(NB, NL, XM)                                                                \
  for (int kt = k0; kt < k1; kt += 4) {                                                     \
    _Pragma("unroll") for (int h = 0; h < 4; ++h) {                                         \
      GB_READ(fa[0], fb[0], h, fr0, NB);                                                    \
      GB_READ(fa[1], fb[1], h, fr1, NB);                                                    \
      if (XM) {                                                                             \
        GB_READX(fx[0], h, fr0);                                                            \
        GB_READX(fx[1], h, fr1);                                                            \
      }                                                                                     \
      {                                                                                     \
        const int kn = min(kt + h + 3, k1 - 1);                                             \
        _Pragma("unroll") for (int q = 0; q < (NL); ++q) GB_DMA(cu, (h + 3) & 3, kn, q);   \
      }                                                                                     \
      if ((NL) == 6) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
      else asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");       \
      GB_FENCE;                                                                             \
      _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                       \
        if ((t >> 1) < (NB)) GB_MMA1(fa[0], fb[0], t);                                       \
      }                                                                                     \
      if (XM) {                                                                             \
        accx[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[0], fb[0][0], accx[0][0], 0, 0, 0); \
        accx[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[0], fb[0][1], accx[0][1], 0, 0, 0); \
      }                                                                                     \
      _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                       \
        if ((t >> 1) < (NB)) GB_MMA1(fa[1], fb[1], t);                                       \
      }                                                                                     \
      if (XM) {                                                                             \
        accx[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[1], fb[1][0], accx[0][0], 0, 0, 0); \
        accx[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[1], fb[1][1], accx[0][1], 0, 0, 0); \
      }                                                                                     \
      GB_FENCE;                                                                             \
      if ((NL) == 6) asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");       \
      else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");                  \
    }                                                                                       \
  }
    // a wavefront reads fragments for and multiplies only the 32-row blocks of
    // its 128 rows that hold rows of the tile (the short last tile of an
    // expert); all versions of the loop have the same loads and barriers.  A
    // tall tile (GB_BM + up to GB_TALL rows) moves its extra rows with a fifth
    // and sixth load per step in every wavefront, and wavefront (wm, wn)
    // multiplies extra rows 32 wm .. 32 wm + 31 (when the tile has them) by
    // the B fragments it holds (its 64 columns).
    if (cu.ti.rows > GB_BM) {
      if (cu.ti.rows > GB_BM + 32 * wm) {
        GB_KLOOP(4, 6, 1);
      } else {
        GB_KLOOP(4, 6, 0);
      }
    } else {
      switch (min(4, max(0, (cu.ti.rows - wm * 128 + 31) / 32))) {
        case 4: GB_KLOOP(4, 4, 0); break;
        case 3: GB_KLOOP(3, 4, 0); break;
        case 2: GB_KLOOP(2, 4, 0); break;
        case 1: GB_KLOOP(1, 4, 0); break;
        default: GB_KLOOP(0, 4, 0); break;
      }
    }
#undef GB_KLOOP
    if (!gp) asm volatile("s_barrier" ::: "memory");
    // every wavefront is past its last fragment read of this unit: start the
    // ring of the next unit, then store this one while those loads travel
    const Unit done = cu;
    u += gridDim.x;
    if (u < plan.units) {
      cu = setup(u);
      GB_PROLOGUE(cu);
    }
    if constexpr (EPI == 2) {
      // fp32 partial logits of piece q: part[q][T][N]
      float* dst = part + (long)done.piece * capacity * N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
          if (row >= done.ti.rows) continue;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = done.ti.nt * GB_BN + wn * 64 + j * 32 + r32;
            if (col < N) dst[(long)(done.ti.row0 + row) * N + col] = acc[i][j][v];
          }
        }
    } else if (done.piece < 0) {
      if constexpr (EPI == 0 || EPI == 1)
        store_tile_lds<EPI>(acc, done.ti, N, capacity, wm, wn, g, r32, l, smem + 3 * GB_STAGE_BYTES + wv * 4096, out);
      else
        store_tile<EPI, 4>(acc, 0, done.ti, N, capacity, wm, wn, g, r32, out, aux);
      if (done.ti.rows > GB_BM + 32 * wm)
        store_tile<EPI, 1>(accx, 8 + wm, done.ti, N, capacity, 0, wn, g, r32, out, aux);
    } else {
      // partial tile, per wavefront [i][j][lane][16 values of the MFMA D layout]
      float* dst = part + (long)done.piece * GB_PART_FLOATS + wv * 8192 + l * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *(f32x4*)(dst + (i * 2 + j) * 1024 + c * 4) =
                f32x4{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
      if (done.ti.rows > GB_BM + 32 * wm) {  // the extra rows: [wavefront][j][lane][16]
        float* dx = part + (long)done.piece * GB_PART_FLOATS + GB_PART_X + wv * 2048 + l * 16;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *(f32x4*)(dx + j * 1024 + c * 4) = f32x4{accx[0][j][4 * c], accx[0][j][4 * c + 1],
                                                     accx[0][j][4 * c + 2], accx[0][j][4 * c + 3]};
      }
    }
  }
#undef GB_DMA
#undef GB_PROLOGUE
#undef GB_READ
#undef GB_READX
#undef GB_MMA1
#undef GB_FENCE
  // the last prefetches of the ring (clamped repeats) land before the exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Sum the S split-K partials of each split tile (in piece order) and apply the
// epilogue.  Launched with the GEMM's grid size G on GEMM_SPLIT_UNITS / 2 x 8
// workgroups of five wavefronts: workgroup (b, w) handles the part of GEMM
// wavefront w of split tile b of the plan, its wavefront i < 4 row block i,
// and its wavefront 4 GEMM wavefront w's extra rows of a tall tile.
template <int EPI>
__global__ __launch_bounds__(320) void k_splitk_reduce(int L, int N, int Kd, int64_t capacity, int G,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ part, bf16_t* __restrict__ out,
                                                       const bf16_t* __restrict__ aux) {
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  const int NT = (N + GB_BN - 1) / GB_BN;
  const SplitPlan plan = gb_schedule(L, capacity, NT, Kd, G, offsets, s_pre, s_tmp);
  const int total = s_pre[L];
  const int b = blockIdx.x >> 3, wv = blockIdx.x & 7, i = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (plan.S < 2 || b >= total - plan.dp) return;
  const TileInfo ti = locate_tile(plan.dp + b, L, capacity, GB_BM, NT, offsets, s_pre, GB_TALL);
  const float* src = part + (long)b * plan.S * GB_PART_FLOATS + l * 16;
  f32x16 acc[1][2];
  if (i < 4) {
    if (ti.rows <= (wv >> 2) * 128 + i * 32) return;  // row block past the tile's rows
    sum_partials(src + wv * 8192 + i * 2048, plan.S, acc, GB_PART_FLOATS);
    store_tile<EPI, 1>(acc, i, ti, N, capacity, wv >> 2, wv & 3, l >> 5, l & 31, out, aux);
  } else {
    if (ti.rows <= GB_BM + 32 * (wv >> 2)) return;
    sum_partials(src + GB_PART_X + wv * 2048, plan.S, acc, GB_PART_FLOATS);
    store_tile<EPI, 1>(acc, 8 + (wv >> 2), ti, N, capacity, 0, wv & 3, l >> 5, l & 31, out, aux);
  }
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM (VALU): out tile 64 x 64, k step 16, 256 threads, each
// thread 4 rows x 4 columns: prepared columns 2tx, 2tx+1 and 32+2tx, 32+2tx+1
// of the tile, which are a matching (gate, up) pair for EPI 1.
// ---------------------------------------------------------------------------
#define GF_BM 64
#define GF_BN 64
#define GF_BK 16

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(int L, int N, int Kd, int64_t capacity,
                                                  const float* __restrict__ A,
                                                  const int32_t* __restrict__ offsets,
                                                  const float* __restrict__ B, float* __restrict__ out) {
  __shared__ float sA[GF_BM][GF_BK + 1];
  __shared__ float sB[GF_BN][GF_BK + 1];
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  const int NT = (N + GF_BN - 1) / GF_BN;
  build_schedule(L, capacity, GF_BM, NT, offsets, s_pre, s_tmp);
  const int total = s_pre[L];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const TileInfo ti = locate_tile(it, L, capacity, GF_BM, NT, offsets, s_pre);
    const int col0 = ti.nt * GF_BN;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const int ar = ti.row0 + min(lr, ti.rows - 1);
    const int bc = min(col0 + lr, N - 1);
    const float* pa = A + (long)ar * Kd + lk;
    const float* pb = B + ((long)ti.e * N + bc) * Kd + lk;
    for (int k0 = 0; k0 < Kd; k0 += GF_BK) {
      const float4 va = *(const float4*)(pa + k0);
      const float4 vb = *(const float4*)(pb + k0);
      __syncthreads();
      sA[lr][lk] = va.x; sA[lr][lk + 1] = va.y; sA[lr][lk + 2] = va.z; sA[lr][lk + 3] = va.w;
      sB[lr][lk] = vb.x; sB[lr][lk + 1] = vb.y; sB[lr][lk + 2] = vb.z; sB[lr][lk + 3] = vb.w;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < GF_BK; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = sA[ty * 4 + i][k];
        b[0] = sB[2 * tx][k];
        b[1] = sB[2 * tx + 1][k];
        b[2] = sB[32 + 2 * tx][k];
        b[3] = sB[32 + 2 * tx + 1][k];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ty * 4 + i;
      if (row >= ti.rows) continue;
      const long grow = ti.row0 + row;
      if (EPI == 0) {
        const int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = col0 + cols[j];
          if (col < N) out[grow * N + col] = acc[i][j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int jcol = (col0 >> 1) + 2 * tx + j;
          if (jcol < (N >> 1)) out[grow * (N >> 1) + jcol] = silu_mul(acc[i][j], acc[i][2 + j]);
        }
      }
    }
  }
}

static int grid_for(int64_t capacity, int L, int BM, int NT, int per_cu) {
  const int64_t upper = ((capacity + BM - 1) / BM + L) * (int64_t)NT;
  int64_t g = (int64_t)num_cus() * per_cu;
  if (upper < g) g = upper;
  return (int)(g > 0 ? g : 1);
}

hipError_t launch_grouped_mlp_f32(int L, int H, int F, int64_t capacity, const float* x,
                                  const int32_t* offsets, const float* w1p, const float* w2p,
                                  float* act, float* y, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  const int N1 = 2 * F, N2 = H;
  hipLaunchKernelGGL(k_gemm_f32<1>, dim3(grid_for(capacity, L, GF_BM, (N1 + GF_BN - 1) / GF_BN, 4)), dim3(256),
                     0, s, L, N1, H, capacity, x, offsets, w1p, act);
  hipLaunchKernelGGL(k_gemm_f32<0>, dim3(grid_for(capacity, L, GF_BM, (N2 + GF_BN - 1) / GF_BN, 4)), dim3(256),
                     0, s, L, N2, F, capacity, act, offsets, w2p, y);
  return hipGetLastError();
}

static size_t gemm_bf16_lds(int L) {
  return (size_t)4 * GB_STAGE_BYTES + (size_t)(L + 1 + 16) * sizeof(int32_t);
}

size_t grouped_mlp_bf16_part_bytes() { return (size_t)GEMM_SPLIT_UNITS * GB_PART_FLOATS * sizeof(float); }

// Pieces along k of the router projection GEMM for T tokens, E experts and H
// (a multiple of 128): enough units to give every CU one, at most 16 and at
// most one 4-step group per piece.
int router_gemm_pieces(int T, int E, int H) {
  const long tiles = (long)((T + GB_BM - 1) / GB_BM) * ((E + GB_BN - 1) / GB_BN);
  if (tiles <= 0 || H % 128 != 0) return 0;
  long S = (num_cus() + tiles - 1) / tiles;
  S = S < 16 ? S : 16;
  S = S < H / 128 ? S : H / 128;
  return (int)(S > 1 ? S : 1);
}

hipError_t launch_router_gemm_bf16(int T, int E, int H, int S, const bf16_t* x, const bf16_t* wp, float* partial,
                                   hipStream_t s) {
  if (T == 0) return hipSuccess;
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<2>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr_done;
  const long units = (long)((T + GB_BM - 1) / GB_BM) * ((E + GB_BN - 1) / GB_BN) * S;
  const int G = (int)(units < num_cus() ? units : num_cus());
  hipLaunchKernelGGL(k_gemm_bf16<2>, dim3(G), dim3(GB_THREADS), gemm_bf16_lds(S), s, S, E, H, (int64_t)T, x,
                     (const int32_t*)nullptr, wp, (bf16_t*)nullptr, partial, (const bf16_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_grouped_mlp_bf16(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* w1p, const bf16_t* w2p,
                                   bf16_t* act, float* part, bf16_t* y, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  const size_t lds = gemm_bf16_lds(L);
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr_done;
  const int N1 = 2 * F, N2 = H;
  const int G1 = grid_for(capacity, L, GB_BM, (N1 + GB_BN - 1) / GB_BN, 1);
  const int G2 = grid_for(capacity, L, GB_BM, (N2 + GB_BN - 1) / GB_BN, 1);
  const dim3 rgrid(GEMM_SPLIT_UNITS / 2 * 8), rblk(320), blk(GB_THREADS);
  hipLaunchKernelGGL(k_gemm_bf16<1>, dim3(G1), blk, lds, s, L, N1, H, capacity, x, offsets, w1p, act, part, (const bf16_t*)nullptr);
  if (gb_may_split(H))
    hipLaunchKernelGGL(k_splitk_reduce<1>, rgrid, rblk, 0, s, L, N1, H, capacity, G1, offsets, part, act, (const bf16_t*)nullptr);
  hipLaunchKernelGGL(k_gemm_bf16<0>, dim3(G2), blk, lds, s, L, N2, F, capacity, act, offsets, w2p, y, part, (const bf16_t*)nullptr);
  if (gb_may_split(F))
    hipLaunchKernelGGL(k_splitk_reduce<0>, rgrid, rblk, 0, s, L, N2, F, capacity, G2, offsets, part, y, (const bf16_t*)nullptr);
  return hipGetLastError();
}

// Data gradient of the grouped SwiGLU MLP (bf16): h = x . W1 recomputed into
// hbuf (EPI 3), d_h = swiglu'(h, d_y . W2^T) into dhbuf (EPI 4, W2^T panels
// w2t), d_x = d_h . W1^T (EPI 0 on the W1^T panels w1t), each GEMM followed
// by its split-K reduce.
hipError_t launch_grouped_mlp_bf16_backward(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                            const int32_t* offsets, const bf16_t* w1p, const bf16_t* w1t,
                                            const bf16_t* w2t, const bf16_t* dy, bf16_t* hbuf, bf16_t* dhbuf,
                                            float* part, bf16_t* dx, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  const size_t lds = gemm_bf16_lds(L);
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<3>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<4>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr_done;
  const bf16_t* nul = nullptr;
  const int G3 = grid_for(capacity, L, GB_BM, (2 * F + GB_BN - 1) / GB_BN, 1);
  const int G4 = grid_for(capacity, L, GB_BM, (F + GB_BN - 1) / GB_BN, 1);
  const int G0 = grid_for(capacity, L, GB_BM, (H + GB_BN - 1) / GB_BN, 1);
  const dim3 rgrid(GEMM_SPLIT_UNITS / 2 * 8), rblk(320), blk(GB_THREADS);
  hipLaunchKernelGGL(k_gemm_bf16<3>, dim3(G3), blk, lds, s, L, 2 * F, H, capacity, x, offsets, w1p, hbuf, part, nul);
  if (gb_may_split(H))
    hipLaunchKernelGGL(k_splitk_reduce<3>, rgrid, rblk, 0, s, L, 2 * F, H, capacity, G3, offsets, part, hbuf, nul);
  hipLaunchKernelGGL(k_gemm_bf16<4>, dim3(G4), blk, lds, s, L, F, H, capacity, dy, offsets, w2t, dhbuf, part,
                     (const bf16_t*)hbuf);
  if (gb_may_split(H))
    hipLaunchKernelGGL(k_splitk_reduce<4>, rgrid, rblk, 0, s, L, F, H, capacity, G4, offsets, part, dhbuf,
                       (const bf16_t*)hbuf);
  hipLaunchKernelGGL(k_gemm_bf16<0>, dim3(G0), blk, lds, s, L, H, 2 * F, capacity, dhbuf, offsets, w1t, dx, part,
                     nul);
  if (gb_may_split(2 * F))
    hipLaunchKernelGGL(k_splitk_reduce<0>, rgrid, rblk, 0, s, L, H, 2 * F, capacity, G0, offsets, part, dx, nul);
  return hipGetLastError();
}

// Weight gradient of the grouped SwiGLU MLP (bf16 operands, fp32 results):
// the token-blocked operand layouts (launch_wgrad_layouts), then dW1 = X^T d_h
// and dW2 = a^T d_y as EPI 5 GEMMs over each expert's own blocks.
hipError_t launch_grouped_mlp_bf16_wgrad(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                         const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf,
                                         const bf16_t* dhbuf, int32_t* pb, bf16_t* xt, bf16_t* dht, bf16_t* at,
                                         bf16_t* dyt, float* dW1, float* dW2, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  hipError_t e = launch_wgrad_layouts(L, H, F, capacity, nbmax, x, offsets, dy, hbuf, dhbuf, pb, xt, dht, at, dyt,
                                      dW1, dW2, s);
  if (e != hipSuccess) return e;
  const size_t lds = gemm_bf16_lds(L);
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<5>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr_done;
  auto grid = [&](int I, int J) {
    const long tiles = (long)((I + GB_BM - 1) / GB_BM) * ((J + GB_BN - 1) / GB_BN) * L;
    return (int)(tiles < num_cus() ? tiles : num_cus());
  };
  const dim3 blk(GB_THREADS);
  const bf16_t* nul = nullptr;
  hipLaunchKernelGGL(k_gemm_bf16<5>, dim3(grid(H, 2 * F)), blk, lds, s, L, 2 * F, 0, (int64_t)H, xt, pb, dht,
                     (bf16_t*)dW1, (float*)nullptr, nul);
  hipLaunchKernelGGL(k_gemm_bf16<5>, dim3(grid(F, H)), blk, lds, s, L, H, 0, (int64_t)F, at, pb, dyt,
                     (bf16_t*)dW2, (float*)nullptr, nul);
  return hipGetLastError();
}

}  // namespace moe
