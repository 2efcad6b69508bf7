// MX (MXFP8 and MXFP4) ragged grouped GEMMs of the expert SwiGLU MLP.
//
// bpdata article, "Transformer Engine building blocks for dropless MoE in JAX":
// group-aware MXFP8 quantization and an MXFP8 grouped GEMM for the expert
// matmuls ("Optimization 1: Grouped GEMM": MXFP8 block scaling).  Operands are
// OCP MX codes (E4M3 bytes, or E2M1 nibbles two per byte) with one E8M0 scale
// per 32 consecutive contraction elements; the CDNA4 instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 applies the scales inside the matrix core
// (fp32 accumulation).
//
// Lane layout of one 32x32x64 instruction (checked on the hardware): lane
// l = 32g + r holds row/column r and its scale operand is the scale of block g
// of row/column r.  E4M3: its bytes 0..15 are k = 16g..16g+15 (block 0) and
// bytes 16..31 are k = 32+16g..32+16g+15 (block 1).  E2M1 (format code 4):
// only its first 16 bytes are read, and all 32 nibbles belong to block g, so a
// lane takes the 16 code bytes of block g as they lie in memory.
//
// Structure as in the bf16 kernel: 256 x 256 output tiles, 8 wavefronts of
// 128 x 64, a ring of 4 LDS stages filled by LDS DMA, two groups of wavefronts
// one phase apart.  A stage holds 64 code bytes of each of the 256 A and 256 B
// rows: 64 E4M3 elements (2 blocks, one instruction per 32 x 32 block) or 128
// E2M1 elements (4 blocks, two instructions).  A is row-major codes with
// scales [rows][Kd/32]; B is the prepared weight panel, codes k-blocked by
// stage [Kd/stage][256][64 bytes] and scales [ceil(Kd/512)][256][16].  The 16
// scale bytes of a row and 512-wide k group (8 E4M3 or 4 E2M1 stages) travel
// in one 16-byte DMA granule into a double-buffered LDS scale ring.  The tiles
// of a last, partial round of the CUs are split along k and summed by
// k_mx_splitk_reduce in a fixed order (the split plan of the bf16 kernel).
// EPI 1 (GEMM1): a = silu(gate) * up is rounded to bf16 and MX-quantized along
// F in the epilogue (one 32-column gate chunk = one MX block of a row); with a
// non-null aux_o the bf16 values are also stored row-major [capacity][F] (a
// test hook that lets the quantization be checked bit for bit).
// EPI 0 (GEMM2): y stored as bf16.
// The data gradient (MXFP8):
// EPI 3: h = x_perm . W1 recomputed, stored bf16 k-blocked [N/32][capacity][32]
//        in the prepared (gate/up interleaved) column order.
// EPI 6: A = d_y (row-wise MX along H), B = the MX W2^T panels (N = F
//        columns): d_a stored fp32 row-major [capacity][N]; k_swiglu_bwd_mx
//        then forms d_h from it and h (a fused epilogue that read g and u of
//        every element from memory was latency bound: at the kernel's
//        register budget those loads went one at a time).
#include "gemm_common.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GM_BM 256
#define GM_BN 256
#define GM_BK 64                       // codes per row and ring stage
#define GM_THREADS 512
#define GM_TALL 32                     // rows a tall tile has beyond GM_BM
// LDS layout (TALL: the kernel instance with tall tiles, whose extra rows add
// 2 KiB of codes to every ring stage and 512 scale bytes to every scale group)
#define GM_STAGE_BYTES (TALL ? 34816 : 32768)  // A, B (and the extra rows) of one ring stage
#define GM_LDS_SCALES (4 * GM_STAGE_BYTES)  // scale buffers after the 4 stages
#define GM_SGROUP_HALF 4096            // 256 rows x 16 scale bytes (512 codes)
#define GM_SGROUP_BYTES (TALL ? 2 * GM_SGROUP_HALF + 512 : 2 * GM_SGROUP_HALF)  // A, B (, extra rows)
// a split-K partial tile: the 8 wavefront parts of 128 x 64, then the 32 x 64
// extra-row blocks [wn][wm] (tall tiles)
#define GM_PART_X (GM_BM * GM_BN)
#define GM_PART_FLOATS (GM_PART_X + 4 * 2048)

// split plan of the MX kernel over KT stages: pieces are whole groups of 4
__device__ __forceinline__ SplitPlan gm_split_plan(int total, int G, int KT) {
  return split_plan(total, G, KT / 2);
}
// whether an MX GEMM over Kd elements may split a tile (else its reduce has no work)
static inline bool gm_may_split(int Kd, bool fp4) { return split_max_pieces((fp4 ? Kd / 2 : Kd) / GM_BK / 2) >= 2; }

// Largest value over the 32 lanes of a half wavefront (lanes 32g .. 32g+31):
// DPP within each row of 16 lanes (quad swaps 1 and 2, then the half-row and
// row mirrors, each pairing a lane with one from the other half of its group),
// then a swizzle that swaps the two rows of the half.
__device__ __forceinline__ uint32_t max_half_wave(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));                 // lane ^ 16
}

// Epilogue of row blocks [i0, i0+NI) of one wavefront's 128 x 64 part of a
// tile (MFMA D layout: lane l holds column l%32, rows 8 (v/4) + 4 (l/32) + v%4
// of each 32 x 32 block).  Every lane of the wavefront must call it (EPI 1
// reduces across lanes).
template <int EPI, int NI, bool FP4>
__device__ __forceinline__ void mx_store_tile(const f32x16 (&acc)[NI][2], int i0, const TileInfo& ti, int N, int wm, int wn,
                                              int g, int r32, uint8_t* __restrict__ out,
                                              uint8_t* __restrict__ out_s, int64_t capacity,
                                              const bf16_t* __restrict__ aux, bf16_t* __restrict__ aux_o) {
  const int col0 = ti.nt * GM_BN;
  const int msub = max(0, (ti.rows - wm * 128 + 31) / 32);  // row blocks with rows (9: tall tile)
  // opaque lane offsets: the compiler cannot hoist the per-row numbers out of
  // the persistent loop into registers held (and spilled) across the k loop
  asm volatile("" : "+v"(g), "+v"(r32));
  if (EPI == 0) {
    bf16_t* y = (bf16_t*)out;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i0 + i >= msub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + (i0 + i) * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row >= ti.rows) continue;
        const long grow = ti.row0 + row;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) y[grow * N + col] = (bf16_t)f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  } else if (EPI == 3) {
    bf16_t* h = (bf16_t*)out;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i0 + i >= msub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + (i0 + i) * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row >= ti.rows) continue;
        const long grow = ti.row0 + row;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) h[((long)(col >> 5) * capacity + grow) * 32 + (col & 31)] = (bf16_t)f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  } else if (EPI == 6) {
    float* da = (float*)out;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i0 + i >= msub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + (i0 + i) * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row >= ti.rows) continue;
        const long grow = ti.row0 + row;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) da[grow * N + col] = acc[i][j][v];
        }
      }
    }
  } else {
    const int Fh = N >> 1;
    const int jcol = (col0 >> 1) + wn * 32 + r32;  // this lane's column of a
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i0 + i >= msub) continue;  // uniform over the wavefront
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + (i0 + i) * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        // bf16 value of a, then the amax of its MX block (the 32 lanes of this half)
        const uint32_t ab = f32_to_bf16(silu_mul(acc[i][0][v], acc[i][1][v]));
        const uint32_t am = max_half_wave(ab & 0x7fffu);
        // test hook: the bf16 value itself, row-major [capacity][F], when asked for
        if (aux_o && row < ti.rows && jcol < Fh) aux_o[(long)(ti.row0 + row) * Fh + jcol] = (bf16_t)ab;
        if (FP4) {
          // E2M1 codes of columns 2c and 2c+1 share byte c (low nibble first)
          const int E = mx4_scale_exp(am);
          const uint32_t code = mx_e2m1(ab, E);
          const uint32_t next = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)code, 0xB1, 0xF, 0xF, false);
          if (row < ti.rows && jcol < Fh) {
            const long grow = ti.row0 + row;
            if ((r32 & 1) == 0) out[grow * (Fh >> 1) + (jcol >> 1)] = (uint8_t)(code | (next << 4));
            if (r32 == 0) out_s[grow * (Fh >> 5) + (jcol >> 5)] = (uint8_t)(E + 127);
          }
        } else {
          const int E = mx_scale_exp(am);
          if (row < ti.rows && jcol < Fh) {
            const long grow = ti.row0 + row;
            out[grow * Fh + jcol] = (uint8_t)mx_e4m3(ab, E);
            if (r32 == 0) out_s[grow * (Fh >> 5) + (jcol >> 5)] = (uint8_t)(E + 127);
          }
        }
      }
    }
  }
}

template <int EPI, bool FP4, bool TALL>
__global__ __launch_bounds__(GM_THREADS, 1) void k_gemm_mx(int L, int N, int Kd, int64_t capacity,
                                                           const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ As,
                                                           const int32_t* __restrict__ offsets,
                                                           const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ Bs, uint8_t* __restrict__ out,
                                                           uint8_t* __restrict__ out_s, float* __restrict__ part,
                                                           const void* __restrict__ aux,
                                                           bf16_t* __restrict__ aux_o) {
  const int32_t* aux_i = (const int32_t*)aux;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* s_pre = (int32_t*)(smem + GM_LDS_SCALES + 2 * GM_SGROUP_BYTES);  // [L+1]
  int32_t* s_tmp = s_pre + (L + 1);                                          // [16]
  const int NT = (N + GM_BN - 1) / GM_BN;
  // EPI 5 (the MXFP8 weight gradient): offsets = pk (each expert's padded
  // rows, prefix), aux_i = png (its 512-row scale groups, prefix), capacity =
  // I rows of dW, N = J columns; NTI x NT tiles per expert with rows, no split
  const int NTI = EPI == 5 ? (int)((capacity + GM_BM - 1) / GM_BM) : 1;
  if (EPI == 5)
    build_schedule(L, (int64_t)1 << 40, 1 << 30, NTI * NT, offsets, s_pre, s_tmp, 0);
  else
    build_schedule(L, capacity, GM_BM, NT, offsets, s_pre, s_tmp, TALL ? GM_TALL : 0);
  // RB code bytes per row; KT stages of 64 bytes; SG stages per 16-block scale group
  constexpr int SG = FP4 ? 4 : 8, LG = FP4 ? 2 : 3;
  const int RB = FP4 ? Kd / 2 : Kd;
  const int KT = RB / GM_BK, KB = Kd / 32, NG = (Kd + 511) / 512;
  SplitPlan plan;
  if (EPI == 5) {
    plan.dp = plan.units = s_pre[L];
    plan.S = 1;
  } else {
    plan = gm_split_plan(s_pre[L], gridDim.x, KT);
  }
  const int tid = threadIdx.x, l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int gp = wm;  // group: wavefronts 0-3 and 4-7, one of each per SIMD
  const int g = l >> 5, r32 = l & 31;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // code loads: wavefront wv fills rows [32 wv, 32 wv + 32) of the A and of the
  // B tile of a stage, 2 blocks of 16 rows each; lane l moves row 16q + l/4,
  // chunk (l%4) ^ swz4(l/4) of block q
  const int drow = l >> 2, dch = (l & 3) ^ swz4(drow);
  // scale loads (once per 8 stages): wavefronts 0-3 the 16-byte groups of A
  // rows [64 w, 64 w + 64), wavefronts 4-7 those of B rows
  const int srow = (wv & 3) * 64 + l;
  // fragment reads: row wm*128 + i*32 + r32 of A, column wn*64 + j*32 + r32 of
  // B; bytes 0..15 of an operand are chunk g, bytes 16..31 chunk 2 + g
  const int fr0 = r32 * 64 + ((g ^ swz4(r32)) << 4);
  const int fr1 = r32 * 64 + (((2 + g) ^ swz4(r32)) << 4);

  struct Unit {
    TileInfo ti;
    int piece, k0, k1;
    __amdgpu_buffer_rsrc_t rA, rB, rS;
    int va[2], vb[2], vs, sgstep, vx, vxs, ng;
  };
  auto setup = [&](int u) {
    Unit w;
    int tile = u;
    w.piece = -1;
    w.k0 = 0;
    w.k1 = KT;
    w.ng = NG;
    if constexpr (EPI == 5) {
      const int e = find_expert(s_pre, L, u);
      const int local = u - s_pre[e];
      w.ti.e = e;
      w.ti.row0 = (local % NTI) * GM_BM;
      w.ti.rows = min(GM_BM, (int)capacity - w.ti.row0);
      w.ti.nt = local / NTI;
      const int Kp = offsets[e + 1] - offsets[e];  // the expert's padded rows
      w.k1 = Kp / GM_BK;
      w.ng = (Kp + 511) / 512;
      w.ti.e = __builtin_amdgcn_readfirstlane(w.ti.e);
      w.ti.row0 = __builtin_amdgcn_readfirstlane(w.ti.row0);
      w.ti.rows = __builtin_amdgcn_readfirstlane(w.ti.rows);
      w.ti.nt = __builtin_amdgcn_readfirstlane(w.ti.nt);
      w.k1 = __builtin_amdgcn_readfirstlane(w.k1);
      w.ng = __builtin_amdgcn_readfirstlane(w.ng);
      const long pke = __builtin_amdgcn_readfirstlane(offsets[e]), pge = __builtin_amdgcn_readfirstlane(aux_i[e]);
      const long CP = (long)NT * GM_BN;
      // A: codes [I][Kp] and scales [I][Kp/32] of the expert
      w.rA = __builtin_amdgcn_make_buffer_rsrc((void*)(A + pke * capacity + (long)w.ti.row0 * Kp), (short)0,
                                               w.ti.rows * Kp, 0x00020000);
      // B: the expert's panels [NT][Kp/64][256][64], scales [NT][ng][256][16]
      w.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(B + pke * CP + (long)w.ti.nt * w.k1 * (GM_BN * GM_BK)),
                                               (short)0, w.k1 * GM_BN * GM_BK, 0x00020000);
      if (wv < 4) {
        w.rS = __builtin_amdgcn_make_buffer_rsrc((void*)(As + (pke / 32) * capacity + (long)w.ti.row0 * (Kp / 32)),
                                                 (short)0, w.ti.rows * (Kp / 32), 0x00020000);
        w.vs = srow * (Kp / 32);
        w.sgstep = 16;
      } else {
        w.rS = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Bs + pge * CP * 16 + (long)w.ti.nt * w.ng * GM_SGROUP_HALF), (short)0, w.ng * GM_SGROUP_HALF,
            0x00020000);
        w.vs = srow * 16;
        w.sgstep = GM_SGROUP_HALF;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = wv * 32 + q * 16 + drow;
        w.va[q] = r * Kp + dch * 16;
        w.vb[q] = r * GM_BK + dch * 16;
      }
      w.vx = w.vxs = 0;
      return w;
    }
    if (u >= plan.dp) {  // split-K piece: stages [k0, k1), whole groups of 4
      w.piece = u - plan.dp;
      tile = plan.dp + w.piece / plan.S;
      const int q = w.piece % plan.S, nq = KT / 4;
      w.k0 = 4 * (q * nq / plan.S);
      w.k1 = 4 * ((q + 1) * nq / plan.S);
    }
    w.ti = locate_tile(tile, L, capacity, GM_BM, NT, offsets, s_pre, TALL ? GM_TALL : 0);
    // the unit is the same for every lane: keep it in scalar registers (the
    // buffer resources built from it are scalar operands of the loads)
    w.ti.e = __builtin_amdgcn_readfirstlane(w.ti.e);
    w.ti.row0 = __builtin_amdgcn_readfirstlane(w.ti.row0);
    w.ti.rows = __builtin_amdgcn_readfirstlane(w.ti.rows);
    w.ti.nt = __builtin_amdgcn_readfirstlane(w.ti.nt);
    const long panel = (long)w.ti.e * NT + w.ti.nt;
    w.rB = __builtin_amdgcn_make_buffer_rsrc((void*)(B + panel * KT * (GM_BN * GM_BK)), (short)0,
                                             KT * GM_BN * GM_BK, 0x00020000);
    w.rA = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)w.ti.row0 * RB), (short)0, w.ti.rows * RB,
                                             0x00020000);
    if (wv < 4) {  // A scale groups: row-major [rows][Kd/32] bytes
      w.rS = __builtin_amdgcn_make_buffer_rsrc((void*)(As + (long)w.ti.row0 * KB), (short)0, w.ti.rows * KB,
                                               0x00020000);
      w.vs = srow * KB;
      w.sgstep = 16;
    } else {  // B scale groups of the panel: [NG][256][16]
      w.rS = __builtin_amdgcn_make_buffer_rsrc((void*)(Bs + panel * NG * GM_SGROUP_HALF), (short)0,
                                               NG * GM_SGROUP_HALF, 0x00020000);
      w.vs = srow * 16;
      w.sgstep = GM_SGROUP_HALF;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = wv * 32 + q * 16 + drow;
      w.va[q] = r * RB + dch * 16;
      w.vb[q] = r * GM_BK + dch * 16;
    }
    // extra rows of a tall tile: code dword of row GM_BM + 4 wv + l/16, chunk
    // position (l%16)/4, dword l%4; scale dword l%4 of row GM_BM + 16 wv + l/4
    // (wavefronts 0 and 1, whose rS holds the A scales)
    const int xr = 4 * wv + (l >> 4);
    w.vx = (GM_BM + xr) * RB + ((((l & 15) >> 2) ^ swz4(xr)) << 4) + (l & 3) * 4;
    w.vxs = (GM_BM + 16 * wv + (l >> 2)) * KB + (l & 3) * 4;
    return w;
  };

#define GM_DMA(W, ST, KT_, Q)                                                               \
  {                                                                                         \
    const int kq = (KT_);                                                                   \
    if ((Q) == 4)                                                                           \
      lds_dma_b32(lds0 + (ST) * GM_STAGE_BYTES + 32768 + wv * 256, (W).vx, (W).rA, kq * GM_BK); \
    else if ((Q) < 2)                                                                       \
      lds_dma_b128(lds0 + (ST) * GM_STAGE_BYTES + (wv * 2 + (Q)) * 1024, (W).va[Q], (W).rA, kq * GM_BK); \
    else                                                                                    \
      lds_dma_b128(lds0 + (ST) * GM_STAGE_BYTES + 8192 * 2 + (wv * 2 + (Q) - 2) * 1024, (W).vb[(Q) - 2], (W).rB, \
                   kq * (GM_BN * GM_BK));                                                   \
  }
// the scale group G_ of the unit into scale buffer G_ % 2 (when SEL == WANT)
#define GM_SDMA_IF(W, G_, SEL, WANT)                                                        \
  {                                                                                         \
    const int gq = (G_);                                                                    \
    lds_dma_b128_if((SEL), (WANT),                                                          \
                    lds0 + GM_LDS_SCALES + (gq & 1) * GM_SGROUP_BYTES + (wv >= 4 ? GM_SGROUP_HALF : 0) + \
                        (wv & 3) * 1024,                                                    \
                    (W).vs, (W).rS, gq * (W).sgstep);                                       \
  }
// the extra rows' scale group G_ (tall tile; wavefronts 0 and 1)
// (the wavefront test joins the scalar test inside the assembly: straight-line
// code for the compiler)
#define GM_XSDMA_IF(W, G_, SEL, WANT)                                                       \
  {                                                                                         \
    const int gq = (G_);                                                                    \
    lds_dma_b32_if((SEL) + (wv < 2 ? 0 : 0x10000), (WANT),                                  \
                   lds0 + GM_LDS_SCALES + (gq & 1) * GM_SGROUP_BYTES + 2 * GM_SGROUP_HALF + (wv & 1) * 256, \
                   (W).vxs, (W).rS, gq * 16);                                               \
  }
// the ring prologue of a unit: the scale group of k0, then stages k0 .. k0+2
// (a tall tile: also its extra rows, 5 loads per stage)
#define GM_PROLOGUE(W)                                                                      \
  {                                                                                         \
    GM_SDMA_IF(W, (W).k0 >> LG, 0, 0);                                                      \
    if (TALL && (W).ti.rows > GM_BM) {                                                      \
      GM_XSDMA_IF(W, (W).k0 >> LG, 0, 0);                                                   \
      _Pragma("unroll") for (int st = 0; st < 3; ++st) {                                    \
        _Pragma("unroll") for (int q = 0; q < 5; ++q) GM_DMA(W, st, min((W).k0 + st, (W).k1 - 1), q); \
      }                                                                                     \
    } else {                                                                                \
      _Pragma("unroll") for (int st = 0; st < 3; ++st) {                                    \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) GM_DMA(W, st, min((W).k0 + st, (W).k1 - 1), q); \
      }                                                                                     \
    }                                                                                       \
  }
// fragments and scale bytes of stage KS_ (in ring stage ST)
#define GM_READ(ST, KS_, NB)                                                                \
  if ((NB) > 0) {                                                                           \
    const uint8_t* pa = smem + (ST) * GM_STAGE_BYTES + wm * 8192;                           \
    const uint8_t* pb = smem + (ST) * GM_STAGE_BYTES + 16384 + wn * 4096;                   \
    _Pragma("unroll") for (int i = 0; i < (NB); ++i) {                                      \
      const u32x4 lo = *(const u32x4*)(pa + i * 2048 + fr0);                                \
      const u32x4 hi = *(const u32x4*)(pa + i * 2048 + fr1);                                \
      fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]}; \
    }                                                                                       \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                         \
      const u32x4 lo = *(const u32x4*)(pb + j * 2048 + fr0);                                \
      const u32x4 hi = *(const u32x4*)(pb + j * 2048 + fr1);                                \
      fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]}; \
    }                                                                                       \
    const int ks = (KS_);                                                                   \
    /* scale words: E2M1, the 4 bytes of the stage; E4M3, stages ks and ks + 1 */          \
    /* (ks even: ring stage ST and ks have the same parity), bytes 0, 1 and    */            \
    /* 2, 3.  They are shifted by 8 g at the instructions, after the barrier,  */            \
    /* so that the memory phase does not wait for them on its own.             */            \
    if (FP4 || ((ST) & 1) == 0) {                                                           \
      const uint8_t* pw = smem + GM_LDS_SCALES + ((ks >> LG) & 1) * GM_SGROUP_BYTES + (ks & (SG - 1)) * (FP4 ? 4 : 2); \
      _Pragma("unroll") for (int i = 0; i < (NB); ++i) sa[i] = *(const uint32_t*)(pw + (wm * 128 + i * 32 + r32) * 16); \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                                         \
        sb[j] = *(const uint32_t*)(pw + GM_SGROUP_HALF + (wn * 64 + j * 32 + r32) * 16);    \
    }                                                                                       \
  }
// E4M3: one instruction per 32 x 32 block and stage.  E2M1: two, on the
// fragment's first 16 bytes (blocks 0, 1 of the stage) and its last 16 bytes
// (blocks 2, 3); the scale operand's byte select (checked on the hardware:
// op_sel k takes byte k) picks byte 0 or 2 of the shifted scale word.
// P: the E2M1 instruction of the block (0: first 16 bytes, 1: last); E4M3
// blocks have one, issued with P = 0
#define GM_MMA1(T, H_, P)                                                                   \
  if (FP4) {                                                                                \
    const i32x8 a_ = fa[(T) >> 1], b_ = fb[(T) & 1];                                        \
    if ((P) == 0)                                                                           \
      acc[(T) >> 1][(T) & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(             \
          __builtin_shufflevector(a_, a_, 0, 1, 2, 3, 0, 1, 2, 3), __builtin_shufflevector(b_, b_, 0, 1, 2, 3, 0, 1, 2, 3), \
          acc[(T) >> 1][(T) & 1], 4, 4, 0, (int)(sa[(T) >> 1] >> (8 * g)), 0, (int)(sb[(T) & 1] >> (8 * g))); \
    else                                                                                    \
      acc[(T) >> 1][(T) & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(             \
          __builtin_shufflevector(a_, a_, 4, 5, 6, 7, 4, 5, 6, 7), __builtin_shufflevector(b_, b_, 4, 5, 6, 7, 4, 5, 6, 7), \
          acc[(T) >> 1][(T) & 1], 4, 4, 2, (int)(sa[(T) >> 1] >> (8 * g)), 2, (int)(sb[(T) & 1] >> (8 * g))); \
  } else if ((P) == 1) {                                                                    \
  } else if ((H_ & 1) == 0) {                                                               \
    acc[(T) >> 1][(T) & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(               \
        fa[(T) >> 1], fb[(T) & 1], acc[(T) >> 1][(T) & 1], 0, 0, 0, (int)(sa[(T) >> 1] >> (8 * g)), 0, (int)(sb[(T) & 1] >> (8 * g))); \
  } else {                                                                                  \
    acc[(T) >> 1][(T) & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(               \
        fa[(T) >> 1], fb[(T) & 1], acc[(T) >> 1][(T) & 1], 0, 0, 2, (int)(sa[(T) >> 1] >> (8 * g)), 2, (int)(sb[(T) & 1] >> (8 * g))); \
  }
// the extra rows of a tall tile: fragment and scale word of stage KS_, and
// their instructions against B block J (wavefront (wm, wn) takes the 32 x 32
// block of columns wn * 64 + 32 wm, whose B fragment it holds as block J = wm)
#define GM_READX(ST, KS_)                                                                   \
  {                                                                                         \
    const uint8_t* px = smem + (ST) * GM_STAGE_BYTES + 32768;                               \
    const u32x4 lo = *(const u32x4*)(px + fr0);                                             \
    const u32x4 hi = *(const u32x4*)(px + fr1);                                             \
    fx = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]}; \
    const int ks = (KS_);                                                                   \
    if (FP4 || ((ST) & 1) == 0) {                                                           \
      const uint8_t* pw = smem + GM_LDS_SCALES + ((ks >> LG) & 1) * GM_SGROUP_BYTES + (ks & (SG - 1)) * (FP4 ? 4 : 2); \
      sx = *(const uint32_t*)(pw + 2 * GM_SGROUP_HALF + r32 * 16);                         \
    }                                                                                       \
  }
#define GM_MMAX(J, H_, P)                                                                   \
  if (FP4) {                                                                                \
    const i32x8 a_ = fx, b_ = fb[J];                                                        \
    if ((P) == 0)                                                                           \
      accx = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                               \
          __builtin_shufflevector(a_, a_, 0, 1, 2, 3, 0, 1, 2, 3), __builtin_shufflevector(b_, b_, 0, 1, 2, 3, 0, 1, 2, 3), \
          accx, 4, 4, 0, (int)(sx >> (8 * g)), 0, (int)(sb[J] >> (8 * g)));                 \
    else                                                                                    \
      accx = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                               \
          __builtin_shufflevector(a_, a_, 4, 5, 6, 7, 4, 5, 6, 7), __builtin_shufflevector(b_, b_, 4, 5, 6, 7, 4, 5, 6, 7), \
          accx, 4, 4, 2, (int)(sx >> (8 * g)), 2, (int)(sb[J] >> (8 * g)));                 \
  } else if ((P) == 1) {                                                                    \
  } else if ((H_ & 1) == 0) {                                                               \
    accx = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                                 \
        fx, fb[J], accx, 0, 0, 0, (int)(sx >> (8 * g)), 0, (int)(sb[J] >> (8 * g)));        \
  } else {                                                                                  \
    accx = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                                 \
        fx, fb[J], accx, 0, 0, 2, (int)(sx >> (8 * g)), 2, (int)(sb[J] >> (8 * g)));        \
  }
#define GM_FENCE __builtin_amdgcn_sched_barrier(0);

  int u = virtual_block();
  Unit cu;
  if (u < plan.units) {
    cu = setup(u);
    GM_PROLOGUE(cu);
  }
  while (u < plan.units) {
    const int k0 = cu.k0, k1 = cu.k1;
    i32x8 fa[4], fb[2], fx;
    uint32_t sa[4], sb[2], sx;
    f32x16 acc[4][2], accx;  // accx: this wavefront's block of the extra rows of a tall tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    accx = f32x16{};
    // wait for stage k0 and the scale group issued before it (the younger
    // stages k0+1, k0+2 may still be loading; loads complete in issue order)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    // the second group of wavefronts runs one phase behind the first
    if (gp) asm volatile("s_barrier" ::: "memory");
    // Phases as in the bf16 kernel: the memory phase of stage ks reads its
    // fragments and scale bytes, loads stage ks+3 (and, at ks % 8 == 5, the
    // scale group of stage ks+3 first) and waits; the compute phase is the
    // stage's 8 MFMAs.  A scale group is complete with the stage loaded after
    // it.  The vmcnt(8) waits allow the two younger stages' 8 loads in flight;
    // where a scale load is among them the wait is one load stronger than
    // needed.
#define GM_KLOOP(NB, NL, XM)                                                                \
  for (int kt = k0; kt < k1; kt += 4) {                                                     \
    _Pragma("unroll") for (int h = 0; h < 4; ++h) {                                         \
      GM_READ(h, kt + h, NB);                                                               \
      if (XM) GM_READX(h, kt + h);                                                          \
      {                                                                                     \
        const int kn = min(kt + h + 3, k1 - 1);                                             \
        GM_SDMA_IF(cu, min(((kt + h) >> LG) + 1, cu.ng - 1), (kt + h) & (SG - 1), SG - 3);  \
        if ((NL) == 5) GM_XSDMA_IF(cu, min(((kt + h) >> LG) + 1, cu.ng - 1), (kt + h) & (SG - 1), SG - 3); \
        _Pragma("unroll") for (int q = 0; q < (NL); ++q) GM_DMA(cu, (h + 3) & 3, kn, q);   \
      }                                                                                     \
      if ((NL) == 5) asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
      else asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");       \
      GM_FENCE;                                                                             \
      /* E2M1: all first instructions, then all second ones (8 apart on an    */            \
      /* accumulator, as in the bf16 kernel)                                   */            \
      _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                       \
        if ((t >> 1) < (NB)) GM_MMA1(t, h, 0);                                               \
      }                                                                                     \
      if (XM) GM_MMAX((XM) - 1, h, 0);                                                      \
      _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                       \
        if (FP4 && (t >> 1) < (NB)) GM_MMA1(t, h, 1);                                        \
      }                                                                                     \
      if (FP4 && XM) GM_MMAX((XM) - 1, h, 1);                                               \
      GM_FENCE;                                                                             \
      if ((NL) == 5) asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");       \
      else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");                  \
    }                                                                                       \
  }
    // a wavefront reads fragments for and multiplies only the 32-row blocks of
    // its 128 rows that hold rows of the tile; all versions of the loop have
    // the same loads and barriers.  A tall tile (GM_BM + up to GM_TALL rows)
    // moves its extra rows' codes with a fifth load per stage in every
    // wavefront (their scales with the scale groups, wavefronts 0 and 1), and
    // every wavefront multiplies them by one of the two B fragments it holds.
    if (TALL && cu.ti.rows > GM_BM) {
      if (wm == 0) {
        GM_KLOOP(4, 5, 1);
      } else {
        GM_KLOOP(4, 5, 2);
      }
    } else {
      switch (min(4, max(0, (cu.ti.rows - wm * 128 + 31) / 32))) {
        case 4: GM_KLOOP(4, 4, 0); break;
        case 3: GM_KLOOP(3, 4, 0); break;
        case 2: GM_KLOOP(2, 4, 0); break;
        case 1: GM_KLOOP(1, 4, 0); break;
        default: GM_KLOOP(0, 4, 0); break;
      }
    }
#undef GM_KLOOP
    if (!gp) asm volatile("s_barrier" ::: "memory");
    // every wavefront is past its last read of this unit: start the next
    // unit's loads, then store this one while they travel
    const Unit done = cu;
    u += gridDim.x;
    if (u < plan.units) {
      cu = setup(u);
      GM_PROLOGUE(cu);
    }
    if constexpr (EPI == 5) {  // fp32 dW[e][row][col]
      int gg = g, rr = r32;  // opaque, as in mx_store_tile: no row numbers held across the k loop
      asm volatile("" : "+v"(gg), "+v"(rr));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * gg + (v & 3);
          if (row >= done.ti.rows) continue;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = done.ti.nt * GM_BN + wn * 64 + j * 32 + rr;
            if (col < N) ((float*)out)[((long)done.ti.e * capacity + done.ti.row0 + row) * N + col] = acc[i][j][v];
          }
        }
    } else if (done.piece < 0) {
      mx_store_tile<EPI, 4, FP4>(acc, 0, done.ti, N, wm, wn, g, r32, out, out_s, capacity, (const bf16_t*)aux, aux_o);
      if (TALL && done.ti.rows > GM_BM) {
        // the extra rows: wavefront (1, wn) hands its block (columns wn * 64 +
        // 32) to wavefront (0, wn) through ring stage 3, which no load of this
        // unit's tail or of the next unit's prologue writes, and which every
        // wavefront has finished reading
        float* xch = (float*)(smem + 3 * GM_STAGE_BYTES) + (wn * 64 + l) * 16;
        if (wm == 1) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *(f32x4*)(xch + 4 * c) = f32x4{accx[4 * c], accx[4 * c + 1], accx[4 * c + 2], accx[4 * c + 3]};
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (wm == 0) {
          f32x16 pair[1][2];
          pair[0][0] = accx;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 v = *(const f32x4*)(xch + 4 * c);
            pair[0][1][4 * c] = v[0];
            pair[0][1][4 * c + 1] = v[1];
            pair[0][1][4 * c + 2] = v[2];
            pair[0][1][4 * c + 3] = v[3];
          }
          mx_store_tile<EPI, 1, FP4>(pair, 8, done.ti, N, 0, wn, g, r32, out, out_s, capacity, (const bf16_t*)aux,
                                     aux_o);
        }
      }
    } else {
      // partial tile, per wavefront [i][j][lane][16 values of the MFMA D layout]
      float* dst = part + (long)done.piece * GM_PART_FLOATS + wv * 8192 + l * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *(f32x4*)(dst + (i * 2 + j) * 1024 + c * 4) =
                f32x4{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
      if (TALL && done.ti.rows > GM_BM) {  // the extra rows: [wn][wm][lane][16]
        float* dx = part + (long)done.piece * GM_PART_FLOATS + GM_PART_X + wn * 2048 + wm * 1024 + l * 16;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *(f32x4*)(dx + c * 4) = f32x4{accx[4 * c], accx[4 * c + 1], accx[4 * c + 2], accx[4 * c + 3]};
      }
    }
  }
#undef GM_DMA
#undef GM_XSDMA_IF
#undef GM_READX
#undef GM_MMAX
#undef GM_SDMA_IF
#undef GM_PROLOGUE
#undef GM_READ
#undef GM_MMA1
#undef GM_FENCE
  // the last prefetches of the ring (clamped repeats) land before the exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Sum the S split-K partials of each split tile (in piece order) and apply the
// epilogue; workgroup (b, w) of five wavefronts handles GEMM wavefront w's
// part of split tile b of the plan of a GEMM launched with G workgroups, its
// wavefront i < 4 row block i and its wavefront 4 (w < 4) the extra rows of
// a tall tile in columns w * 64 .. w * 64 + 63.
template <int EPI, bool FP4, bool TALL>
__global__ __launch_bounds__(320) void k_mx_splitk_reduce(int L, int N, int Kd, int64_t capacity, int G,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ part, uint8_t* __restrict__ out,
                                                          uint8_t* __restrict__ out_s,
                                                          const bf16_t* __restrict__ aux, bf16_t* __restrict__ aux_o) {
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  const int NT = (N + GM_BN - 1) / GM_BN;
  build_schedule(L, capacity, GM_BM, NT, offsets, s_pre, s_tmp, TALL ? GM_TALL : 0);
  const int total = s_pre[L];
  const SplitPlan plan = gm_split_plan(total, G, (FP4 ? Kd / 2 : Kd) / GM_BK);
  const int b = blockIdx.x >> 3, wv = blockIdx.x & 7, i = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (plan.S < 2 || b >= total - plan.dp) return;
  const TileInfo ti = locate_tile(plan.dp + b, L, capacity, GM_BM, NT, offsets, s_pre, TALL ? GM_TALL : 0);
  const float* src = part + (long)b * plan.S * GM_PART_FLOATS + l * 16;
  f32x16 acc[1][2];
  if (i < 4) {
    if (ti.rows <= (wv >> 2) * 128 + i * 32) return;  // row block past the tile's rows
    sum_partials(src + wv * 8192 + i * 2048, plan.S, acc, GM_PART_FLOATS);
    mx_store_tile<EPI, 1, FP4>(acc, i, ti, N, wv >> 2, wv & 3, l >> 5, l & 31, out, out_s, capacity, aux, aux_o);
  } else {
    if (wv >= 4 || ti.rows <= GM_BM) return;
    sum_partials(src + GM_PART_X + wv * 2048, plan.S, acc, GM_PART_FLOATS);
    mx_store_tile<EPI, 1, FP4>(acc, 8, ti, N, 0, wv, l >> 5, l & 31, out, out_s, capacity, aux, aux_o);
  }
}

size_t grouped_mlp_mx_part_bytes() { return (size_t)GEMM_SPLIT_UNITS * GM_PART_FLOATS * sizeof(float); }

// dynamic LDS of the MX kernel: 4 ring stages, 2 scale groups, the schedule
static size_t mx_lds_bytes(int L, bool TALL) {
  return (size_t)GM_LDS_SCALES + 2 * GM_SGROUP_BYTES + (size_t)(L + 1 + 16) * sizeof(int32_t);
}

template <bool FP4, bool TALL>
static void launch_mx(int L, int H, int F, int64_t capacity, const uint8_t* x, const uint8_t* xs,
                      const int32_t* offsets, const uint8_t* w1p, const uint8_t* w1s, const uint8_t* w2p,
                      const uint8_t* w2s, uint8_t* act, uint8_t* act_s, float* part, bf16_t* y, bf16_t* act_bf16,
                      hipStream_t s) {
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<0, FP4, TALL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<1, FP4, TALL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    return true;
  }();
  (void)attr_done;
  const size_t lds = mx_lds_bytes(L, TALL);
  auto grid = [&](int N) {
    const int NT = (N + GM_BN - 1) / GM_BN;
    const int64_t upper = ((capacity + GM_BM - 1) / GM_BM + L) * (int64_t)NT;
    int64_t gsz = num_cus();
    if (upper < gsz) gsz = upper;
    return (int)(gsz > 0 ? gsz : 1);
  };
  const int G1 = grid(2 * F), G2 = grid(H);
  const dim3 rgrid(GEMM_SPLIT_UNITS / 2 * 8), rblk(320), blk(GM_THREADS);
  hipLaunchKernelGGL((k_gemm_mx<1, FP4, TALL>), dim3(G1), blk, lds, s, L, 2 * F, H, capacity, x, xs, offsets, w1p,
                     w1s, act, act_s, part, nullptr, act_bf16);
  if (gm_may_split(H, FP4))
    hipLaunchKernelGGL((k_mx_splitk_reduce<1, FP4, TALL>), rgrid, rblk, 0, s, L, 2 * F, H, capacity, G1, offsets,
                       part, act, act_s, (const bf16_t*)nullptr, act_bf16);
  hipLaunchKernelGGL((k_gemm_mx<0, FP4, TALL>), dim3(G2), blk, lds, s, L, H, F, capacity, act, act_s, offsets,
                     w2p, w2s, (uint8_t*)y, (uint8_t*)nullptr, part, nullptr, (bf16_t*)nullptr);
  if (gm_may_split(F, FP4))
    hipLaunchKernelGGL((k_mx_splitk_reduce<0, FP4, TALL>), rgrid, rblk, 0, s, L, H, F, capacity, G2, offsets, part,
                       (uint8_t*)y, (uint8_t*)nullptr, (const bf16_t*)nullptr, (bf16_t*)nullptr);
}

hipError_t launch_grouped_mlp_mx(int L, int H, int F, int64_t capacity, bool fp4, const uint8_t* x,
                                 const uint8_t* xs, const int32_t* offsets, const uint8_t* w1p,
                                 const uint8_t* w1s, const uint8_t* w2p, const uint8_t* w2s,
                                 uint8_t* act, uint8_t* act_s, float* part, bf16_t* y, bf16_t* act_bf16,
                                 hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  // E4M3: tall tiles when their larger LDS layout leaves room for the
  // schedule of L experts.  E2M1: plain tiles (measured on the Mixtral-like
  // shape: tall tiles 3% faster with E4M3 codes, 2.5% slower with E2M1).
  const bool tall = mx_lds_bytes(L, true) <= 160 * 1024;
  if (fp4)
    launch_mx<true, false>(L, H, F, capacity, x, xs, offsets, w1p, w1s, w2p, w2s, act, act_s, part, y, act_bf16, s);
  else if (tall)
    launch_mx<false, true>(L, H, F, capacity, x, xs, offsets, w1p, w1s, w2p, w2s, act, act_s, part, y, act_bf16, s);
  else
    launch_mx<false, false>(L, H, F, capacity, x, xs, offsets, w1p, w1s, w2p, w2s, act, act_s, part, y, act_bf16, s);
  return hipGetLastError();
}

// d_h from d_a (fp32 [capacity][F]) and h (bf16 k-blocked [2F/32][capacity][32],
// gate/up chunks of 32 interleaved): d_h = [d_a u silu'(g), d_a silu(g)]
// rounded to bf16, stored k-blocked [2F/32][capacity][32] in natural column
// order (gates, then ups) in dh, and MX-quantized along 2F (one 32-column
// chunk = one block) into codes [capacity][2F] and scales [capacity][2F/32].
// One wavefront per (row, 256 columns of F), 4 columns per lane: 8 lanes
// share a chunk (block amax by xor shuffles within the 8), d_a is read as
// 16-byte pieces and the codes written as 4-byte words.  F % 256 == 0; the
// rows are those below *n_rows.
__global__ __launch_bounds__(256) void k_swiglu_bwd_mx(int F, int64_t capacity, const int32_t* __restrict__ n_rows,
                                                       const float* __restrict__ da, const bf16_t* __restrict__ h,
                                                       bf16_t* __restrict__ dh, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t rows = min((int64_t)*n_rows, capacity);
  const int C = F >> 5;                       // chunks per row
  const int NG = F >> 8;                      // 256-column groups per row
  const int64_t items = rows * NG;
  const int l = threadIdx.x & 63, q = l & 7;
  const int64_t step = (int64_t)gridDim.x * 4;
  for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += step) {  // uniform per wave
    const int64_t row = it / NG;
    const int c = (int)(it - row * NG) * 8 + (l >> 3);   // this lane's chunk
    const int f0 = c * 32 + q * 4;                        // its first column
    const f32x4 a = *(const f32x4*)(da + row * F + f0);
    const uint2 gb = *(const uint2*)(h + ((int64_t)(2 * c) * capacity + row) * 32 + q * 4);
    const uint2 ub = *(const uint2*)(h + ((int64_t)(2 * c + 1) * capacity + row) * 32 + q * 4);
    uint32_t dg[4], du[4], mg = 0, mu = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t gw = k < 2 ? gb.x : gb.y, uw = k < 2 ? ub.x : ub.y;
      const float gt = __uint_as_float((k & 1) ? (gw & 0xffff0000u) : (gw << 16));
      const float up = __uint_as_float((k & 1) ? (uw & 0xffff0000u) : (uw << 16));
      const float sg = 1.0f / (1.0f + expf(-gt));
      dg[k] = f32_to_bf16(a[k] * up * sg * (1.0f + gt * (1.0f - sg)));
      du[k] = f32_to_bf16(a[k] * gt * sg);
      mg = max(mg, dg[k] & 0x7fffu);
      mu = max(mu, du[k] & 0x7fffu);
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {  // the 8 lanes of the chunk
      mg = max(mg, (uint32_t)__shfl_xor((int)mg, m));
      mu = max(mu, (uint32_t)__shfl_xor((int)mu, m));
    }
    const int Eg = mx_scale_exp(mg), Eu = mx_scale_exp(mu);
    const uint32_t pg0 = dg[0] | (dg[1] << 16), pg1 = dg[2] | (dg[3] << 16);
    const uint32_t pu0 = du[0] | (du[1] << 16), pu1 = du[2] | (du[3] << 16);
    *(uint2*)(dh + ((int64_t)c * capacity + row) * 32 + q * 4) = make_uint2(pg0, pg1);
    *(uint2*)(dh + ((int64_t)(C + c) * capacity + row) * 32 + q * 4) = make_uint2(pu0, pu1);
    *(uint32_t*)(codes + row * 2 * F + f0) = mx_e4m3x4(pg0, pg1, Eg);
    *(uint32_t*)(codes + row * 2 * F + F + f0) = mx_e4m3x4(pu0, pu1, Eu);
    if (q == 0) {
      scales[row * (F >> 4) + c] = (uint8_t)(Eg + 127);
      scales[row * (F >> 4) + C + c] = (uint8_t)(Eu + 127);
    }
  }
}

// MXFP8 data gradient: row-wise MX of x_perm and d_y (along H, unless the
// caller passes them), then
// h = x_perm . W1 (EPI 3), d_a = d_y . W2^T (EPI 6) and from it d_h (bf16,
// and MX along 2F: k_swiglu_bwd_mx), then d_x = d_h . W1^T (EPI 0); each GEMM
// followed by its split-K reduce.
template <bool TALL>
static void launch_mx_backward(int L, int H, int F, int64_t capacity, const uint8_t* xq, const uint8_t* xqs,
                               const int32_t* offsets, const uint8_t* w1p, const uint8_t* w1s, const uint8_t* w1t,
                               const uint8_t* w1ts, const uint8_t* w2t, const uint8_t* w2ts, const uint8_t* dyq,
                               const uint8_t* dyqs, bf16_t* hbuf, bf16_t* dhbuf, uint8_t* dhq, uint8_t* dhqs,
                               float* da, float* part, bf16_t* dx, hipStream_t s) {
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<0, false, TALL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<3, false, TALL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<6, false, TALL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    return true;
  }();
  (void)attr_done;
  const size_t lds = mx_lds_bytes(L, TALL);
  auto grid = [&](int N) {
    const int NT = (N + GM_BN - 1) / GM_BN;
    const int64_t upper = ((capacity + GM_BM - 1) / GM_BM + L) * (int64_t)NT;
    int64_t gsz = num_cus();
    if (upper < gsz) gsz = upper;
    return (int)(gsz > 0 ? gsz : 1);
  };
  const int G1 = grid(2 * F), G2 = grid(F), G3 = grid(H);
  const dim3 rgrid(GEMM_SPLIT_UNITS / 2 * 8), rblk(320), blk(GM_THREADS);
  hipLaunchKernelGGL((k_gemm_mx<3, false, TALL>), dim3(G1), blk, lds, s, L, 2 * F, H, capacity, xq, xqs, offsets,
                     w1p, w1s, (uint8_t*)hbuf, (uint8_t*)nullptr, part, nullptr, (bf16_t*)nullptr);
  if (gm_may_split(H, false))
    hipLaunchKernelGGL((k_mx_splitk_reduce<3, false, TALL>), rgrid, rblk, 0, s, L, 2 * F, H, capacity, G1, offsets,
                       part, (uint8_t*)hbuf, (uint8_t*)nullptr, (const bf16_t*)nullptr, (bf16_t*)nullptr);
  hipLaunchKernelGGL((k_gemm_mx<6, false, TALL>), dim3(G2), blk, lds, s, L, F, H, capacity, dyq, dyqs, offsets,
                     w2t, w2ts, (uint8_t*)da, (uint8_t*)nullptr, part, nullptr, (bf16_t*)nullptr);
  if (gm_may_split(H, false))
    hipLaunchKernelGGL((k_mx_splitk_reduce<6, false, TALL>), rgrid, rblk, 0, s, L, F, H, capacity, G2, offsets, part,
                       (uint8_t*)da, (uint8_t*)nullptr, (const bf16_t*)nullptr, (bf16_t*)nullptr);
  hipLaunchKernelGGL(k_swiglu_bwd_mx, dim3(num_cus() * 16), dim3(256), 0, s, F, capacity, offsets + L, da, hbuf,
                     dhbuf, dhq, dhqs);
  hipLaunchKernelGGL((k_gemm_mx<0, false, TALL>), dim3(G3), blk, lds, s, L, H, 2 * F, capacity, dhq, dhqs, offsets,
                     w1t, w1ts, (uint8_t*)dx, (uint8_t*)nullptr, part, nullptr, (bf16_t*)nullptr);
  if (gm_may_split(2 * F, false))
    hipLaunchKernelGGL((k_mx_splitk_reduce<0, false, TALL>), rgrid, rblk, 0, s, L, H, 2 * F, capacity, G3, offsets,
                       part, (uint8_t*)dx, (uint8_t*)nullptr, (const bf16_t*)nullptr, (bf16_t*)nullptr);
}

hipError_t launch_grouped_mlp_mx_backward(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                          const int32_t* offsets, const uint8_t* w1p, const uint8_t* w1s,
                                          const uint8_t* w1t, const uint8_t* w1ts, const uint8_t* w2t,
                                          const uint8_t* w2ts, const bf16_t* dy, uint8_t* xq, uint8_t* xqs,
                                          uint8_t* dyq, uint8_t* dyqs, bf16_t* hbuf, bf16_t* dhbuf, uint8_t* dhq,
                                          uint8_t* dhqs, float* da, float* part, bf16_t* dx, bool x_given,
                                          bool dy_given, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  // row-wise MX operands of x_perm and d_y: given by their producers (the
  // MXFP8 permute, the combine backward with MX output), else quantized here
  hipError_t e = hipSuccess;
  if (!x_given) e = launch_mx_quantize(capacity, H, x, offsets + L, xq, xqs, s);
  if (e == hipSuccess && !dy_given) e = launch_mx_quantize(capacity, H, dy, offsets + L, dyq, dyqs, s);
  if (e != hipSuccess) return e;
  if (mx_lds_bytes(L, true) <= 160 * 1024)
    launch_mx_backward<true>(L, H, F, capacity, xq, xqs, offsets, w1p, w1s, w1t, w1ts, w2t, w2ts, dyq, dyqs, hbuf,
                             dhbuf, dhq, dhqs, da, part, dx, s);
  else
    launch_mx_backward<false>(L, H, F, capacity, xq, xqs, offsets, w1p, w1s, w1t, w1ts, w2t, w2ts, dyq, dyqs, hbuf,
                              dhbuf, dhq, dhqs, da, part, dx, s);
  return hipGetLastError();
}

// MXFP8 weight gradient: the group-aware column-wise MX operands in the MX
// GEMM's own layouts (launch_wgrad_mx_layouts), then dW1 = X^T d_h and
// dW2 = a^T d_y as EPI 5 GEMMs over each expert's padded rows.
hipError_t launch_grouped_mlp_mx_wgrad(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                       const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf,
                                       const bf16_t* dhbuf, int32_t* pk, int32_t* png, uint8_t* xa, uint8_t* xas,
                                       uint8_t* dhb, uint8_t* dhbs, uint8_t* aa, uint8_t* aas, uint8_t* dyb,
                                       uint8_t* dybs, float* dW1, float* dW2, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  hipError_t e = launch_wgrad_mx_layouts(L, H, F, capacity, nbmax, x, offsets, dy, hbuf, dhbuf, pk, png, xa, xas, dhb,
                                         dhbs, aa, aas, dyb, dybs, dW1, dW2, s);
  if (e != hipSuccess) return e;
  // function attributes are set once per process; the initializer of a
  // function-local static runs exactly once even under concurrent first calls
  static const bool attr_done = [] {
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<5, false, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    return true;
  }();
  (void)attr_done;
  const size_t lds = mx_lds_bytes(L, false);
  auto grid = [&](int I, int J) {
    const long tiles = (long)((I + GM_BM - 1) / GM_BM) * ((J + GM_BN - 1) / GM_BN) * L;
    return (int)(tiles < num_cus() ? tiles : num_cus());
  };
  const dim3 blk(GM_THREADS);
  hipLaunchKernelGGL((k_gemm_mx<5, false, false>), dim3(grid(H, 2 * F)), blk, lds, s, L, 2 * F, 0, (int64_t)H, xa,
                     xas, pk, dhb, dhbs, (uint8_t*)dW1, (uint8_t*)nullptr, (float*)nullptr, (const void*)png, (bf16_t*)nullptr);
  hipLaunchKernelGGL((k_gemm_mx<5, false, false>), dim3(grid(F, H)), blk, lds, s, L, H, 0, (int64_t)F, aa, aas, pk,
                     dyb, dybs, (uint8_t*)dW2, (uint8_t*)nullptr, (float*)nullptr, (const void*)png, (bf16_t*)nullptr);
  return hipGetLastError();
}

}  // namespace moe
