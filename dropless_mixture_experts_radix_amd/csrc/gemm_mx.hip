// MXFP8 ragged grouped GEMMs of the expert SwiGLU MLP.
//
// bpdata article, "Transformer Engine building blocks for dropless MoE in JAX":
// group-aware MXFP8 quantization and an MXFP8 grouped GEMM for the expert
// matmuls ("Optimization 1: Grouped GEMM": MXFP8 block scaling).  Operands are
// OCP MX E4M3 codes with one E8M0 scale per 32 consecutive contraction
// elements; the CDNA4 instruction v_mfma_scale_f32_32x32x64_f8f6f4 applies the
// scales inside the matrix core (fp32 accumulation).
//
// Lane layout of one 32x32x64 instruction (checked on the hardware): lane
// l = 32g + r holds row/column r; its bytes 0..15 are k = 16g..16g+15 (scale
// block 0) and bytes 16..31 are k = 32+16g..32+16g+15 (scale block 1); its scale
// operand is the scale of block g of row/column r.
//
// Structure as in the bf16 kernel: 256 x 256 output tiles, 8 wavefronts of
// 128 x 64, a k step of 128 codes (two instructions) moves the same 64 KiB as a
// bf16 k step (a 256 x 128-byte A and B tile) through registers into padded
// LDS rows of 144 bytes, plus the 4 scale bytes of each of the 512 rows.  A is
// row-major codes [rows][Kd] with scales [rows][Kd/32]; B is the prepared
// weight panel, k-blocked codes [Kd/128][256][128] and scales [Kd/128][256][4].
// The tiles of a last, partial round of the CUs are split along k and summed by
// k_mx_splitk_reduce in a fixed order (the split plan of the bf16 kernel).
// EPI 1 (GEMM1): a = silu(gate) * up is rounded to bf16 and MX-quantized along
// F in the epilogue (one 32-column gate chunk = one MX block of a row).
// EPI 0 (GEMM2): y stored as bf16.
#include "gemm_common.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GM_BM 256
#define GM_BN 256
#define GM_BK 128                      // codes per row and k step
#define GM_LDB 144                     // padded LDS row (bytes)
#define GM_STAGE (GM_BM * GM_LDB)      // bytes of one operand stage
#define GM_THREADS 512
#define GM_PART_FLOATS (GM_BM * GM_BN)

// Epilogue of one wavefront's 128 x 64 part of a tile (MFMA D layout: lane l
// holds column l%32, rows 8 (v/4) + 4 (l/32) + v%4 of each 32 x 32 block).
// Every lane of the wavefront must call it (EPI 1 reduces across lanes).
template <int EPI>
__device__ __forceinline__ void mx_store_tile(const f32x16 (&acc)[4][2], const TileInfo& ti, int N, int wm, int wn,
                                              int g, int r32, uint8_t* __restrict__ out,
                                              uint8_t* __restrict__ out_s) {
  const int col0 = ti.nt * GM_BN;
  const int msub = min(4, max(0, (ti.rows - wm * 128 + 31) / 32));
  if (EPI == 0) {
    bf16_t* y = (bf16_t*)out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= msub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row >= ti.rows) continue;
        const long grow = ti.row0 + row;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) y[grow * N + col] = (bf16_t)f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  } else {
    const int Fh = N >> 1;
    const int jcol = (col0 >> 1) + wn * 32 + r32;  // this lane's column of a
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= msub) continue;  // uniform over the wavefront
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        // bf16 value of a, then the amax of its MX block (the 32 lanes of this half)
        const uint32_t ab = f32_to_bf16(silu_mul(acc[i][0][v], acc[i][1][v]));
        uint32_t am = ab & 0x7fffu;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
          const uint32_t x = (uint32_t)__shfl_xor((int)am, o, 64);
          am = am > x ? am : x;
        }
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

template <int EPI>
__global__ __launch_bounds__(GM_THREADS, 1) void k_gemm_mx(int L, int N, int Kd, int64_t capacity,
                                                           const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ As,
                                                           const int32_t* __restrict__ offsets,
                                                           const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ Bs, uint8_t* __restrict__ out,
                                                           uint8_t* __restrict__ out_s, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sA = smem;                                  // [2][256][144]
  uint8_t* sB = sA + 2 * GM_STAGE;                     // [2][256][144]
  uint32_t* sS = (uint32_t*)(sB + 2 * GM_STAGE);       // [2][512]: A rows, then B rows
  int32_t* s_pre = (int32_t*)(sS + 2 * 512);           // [L+1]
  int32_t* s_tmp = s_pre + (L + 1);                    // [16]
  const int NT = (N + GM_BN - 1) / GM_BN;
  build_schedule(L, capacity, GM_BM, NT, offsets, s_pre, s_tmp);
  const int KT = Kd / GM_BK, KB = Kd / 32;
  const SplitPlan plan = split_plan(s_pre[L], gridDim.x, KT);
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int wm = wv >> 2, wn = wv & 3;
  const int g = l >> 5, r32 = l & 31;
  // global -> LDS: thread moves 16-byte chunk lkc of rows lrow + 64 i (i < 4)
  // of the A and the B k-step tile, and the scale word of row tid (A rows for
  // tid < 256, B rows above)
  const int lrow = tid >> 3, lkc = tid & 7;
  const int st_off = lrow * GM_LDB + lkc * 16;
  const int fa_base = (wm * 128 + r32) * GM_LDB + g * 16;
  const int fb_base = (wn * 64 + r32) * GM_LDB + g * 16;
  const int vb = lrow * GM_BK + lkc * 16;
  const int va = lrow * Kd + lkc * 16;
  const bool a_scale = tid < 256;
  const int vs = a_scale ? tid * KB : (tid - 256) * 4;

  for (int u = virtual_block(); u < plan.units; u += gridDim.x) {
    int tile = u, k0 = 0, k1 = KT, piece = -1;
    if (u >= plan.dp) {  // split-K piece: k steps [k0, k1), an even count
      piece = u - plan.dp;
      tile = plan.dp + piece / plan.S;
      const int q = piece % plan.S, half = KT / 2;
      k0 = 2 * (q * half / plan.S);
      k1 = 2 * ((q + 1) * half / plan.S);
    }
    const TileInfo ti = locate_tile(tile, L, capacity, GM_BM, NT, offsets, s_pre);
    const long pblk = ((long)ti.e * NT + ti.nt) * KT;  // first k-step block of this panel
    const __amdgpu_buffer_rsrc_t rB =
        __builtin_amdgcn_make_buffer_rsrc((void*)(B + pblk * (GM_BN * GM_BK)), (short)0, KT * GM_BN * GM_BK, 0x00020000);
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)ti.row0 * Kd), (short)0,
                                                                        ti.rows * Kd, 0x00020000);
    // scale words: A rows of the tile (past them: zeros), or the panel's B block
    const __amdgpu_buffer_rsrc_t rS =
        a_scale ? __builtin_amdgcn_make_buffer_rsrc((void*)(As + (long)ti.row0 * KB), (short)0, ti.rows * KB, 0x00020000)
                : __builtin_amdgcn_make_buffer_rsrc((void*)(Bs + pblk * (GM_BN * 4)), (short)0, KT * GM_BN * 4,
                                                    0x00020000);
    const int sstep = a_scale ? 4 : GM_BN * 4;

    u32x4 ast[4], bst[4];  // register stage of the next k step
    uint32_t sst;
#define GM_LOAD(KT_)                                                                        \
  {                                                                                         \
    const int koa = va + (KT_) * GM_BK;                                                     \
    const int kob = (KT_) * (GM_BN * GM_BK);                                                \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
      ast[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, koa + i * 64 * Kd, 0, 0);          \
      bst[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, vb + i * (64 * GM_BK), kob, 0);    \
    }                                                                                       \
    sst = __builtin_amdgcn_raw_buffer_load_b32(rS, vs + (KT_) * sstep, 0, 0);               \
  }
#define GM_STORE(BUF)                                                                       \
  {                                                                                         \
    uint8_t* dA = sA + (BUF) * GM_STAGE + st_off;                                           \
    uint8_t* dB = sB + (BUF) * GM_STAGE + st_off;                                           \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
      *(u32x4*)(dA + i * 64 * GM_LDB) = ast[i];                                             \
      *(u32x4*)(dB + i * 64 * GM_LDB) = bst[i];                                             \
    }                                                                                       \
    sS[(BUF) * 512 + tid] = sst;                                                            \
  }
#define GM_COMPUTE(BUF)                                                                     \
  {                                                                                         \
    const uint8_t* cA = sA + (BUF) * GM_STAGE + fa_base;                                    \
    const uint8_t* cB = sB + (BUF) * GM_STAGE + fb_base;                                    \
    const uint32_t* cS = sS + (BUF) * 512;                                                  \
    uint32_t sa4[4], sb4[2];                                                                \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) sa4[i] = cS[wm * 128 + i * 32 + r32];     \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) sb4[j] = cS[256 + wn * 64 + j * 32 + r32]; \
    _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                         \
      const int sh = 8 * (2 * s + g);                                                       \
      i32x8 fa[4], fb[2];                                                                   \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                       \
        const u32x4 lo = *(const u32x4*)(cB + j * 32 * GM_LDB + s * 64);                   \
        const u32x4 hi = *(const u32x4*)(cB + j * 32 * GM_LDB + s * 64 + 32);               \
        fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],                       \
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};                      \
      }                                                                                     \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                       \
        const u32x4 lo = *(const u32x4*)(cA + i * 32 * GM_LDB + s * 64);                    \
        const u32x4 hi = *(const u32x4*)(cA + i * 32 * GM_LDB + s * 64 + 32);               \
        fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],                       \
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};                      \
      }                                                                                     \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                         \
        _Pragma("unroll") for (int j = 0; j < 2; ++j)                                       \
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                      \
              fa[i], fb[j], acc[i][j], 0, 0, 0, (int)((sa4[i] >> sh) & 255u), 0,            \
              (int)((sb4[j] >> sh) & 255u));                                                \
    }                                                                                       \
  }
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // prologue: k step k0 into LDS buffer 0, k step k0+1 in registers;
    // steady state: at step kt (kt - k0 even) LDS buffer 0 holds step kt and
    // the registers hold step kt+1
    GM_LOAD(k0);
    GM_STORE(0);
    GM_LOAD(k0 + 1);
    __syncthreads();
    for (int kt = k0; kt < k1; kt += 2) {
      GM_COMPUTE(0);
      GM_STORE(1);
      GM_LOAD(min(kt + 2, k1 - 1));
      __syncthreads();
      GM_COMPUTE(1);
      GM_STORE(0);
      GM_LOAD(min(kt + 3, k1 - 1));
      __syncthreads();
    }
#undef GM_LOAD
#undef GM_STORE
#undef GM_COMPUTE

    if (piece < 0) {
      mx_store_tile<EPI>(acc, ti, N, wm, wn, g, r32, out, out_s);
    } else {
      // partial tile, per wavefront [i][j][lane][16 values of the MFMA D layout]
      float* dst = part + (long)piece * GM_PART_FLOATS + wv * 8192 + l * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *(f32x4*)(dst + (i * 2 + j) * 1024 + c * 4) =
                f32x4{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
    }
  }
}

// Sum the S split-K partials of each split tile (in piece order) and apply the
// epilogue; workgroup (b, w) of one wavefront handles wavefront w's part of
// split tile b of the plan of a GEMM launched with G workgroups.
template <int EPI>
__global__ __launch_bounds__(64) void k_mx_splitk_reduce(int L, int N, int Kd, int64_t capacity, int G,
                                                         const int32_t* __restrict__ offsets,
                                                         const float* __restrict__ part, uint8_t* __restrict__ out,
                                                         uint8_t* __restrict__ out_s) {
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  const int NT = (N + GM_BN - 1) / GM_BN;
  build_schedule(L, capacity, GM_BM, NT, offsets, s_pre, s_tmp);
  const int total = s_pre[L];
  const SplitPlan plan = split_plan(total, G, Kd / GM_BK);
  const int b = blockIdx.x >> 3, wv = blockIdx.x & 7, l = threadIdx.x;
  if (plan.S < 2 || b >= total - plan.dp) return;
  const TileInfo ti = locate_tile(plan.dp + b, L, capacity, GM_BM, NT, offsets, s_pre);
  const float* src = part + (long)b * plan.S * GM_PART_FLOATS + wv * 8192 + l * 16;
  f32x4 sum[8][4];
#pragma unroll
  for (int ij = 0; ij < 8; ++ij)
#pragma unroll
    for (int c = 0; c < 4; ++c) sum[ij][c] = *(const f32x4*)(src + ij * 1024 + c * 4);
  for (int q = 1; q < plan.S; ++q) {
    const float* sq = src + (long)q * GM_PART_FLOATS;
#pragma unroll
    for (int ij = 0; ij < 8; ++ij)
#pragma unroll
      for (int c = 0; c < 4; ++c) sum[ij][c] += *(const f32x4*)(sq + ij * 1024 + c * 4);
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][j][4 * c + t] = sum[i * 2 + j][c][t];
  mx_store_tile<EPI>(acc, ti, N, wv >> 2, wv & 3, l >> 5, l & 31, out, out_s);
}

size_t grouped_mlp_mx_part_bytes() { return (size_t)GEMM_SPLIT_UNITS * GM_PART_FLOATS * sizeof(float); }

hipError_t launch_grouped_mlp_mx(int L, int H, int F, int64_t capacity, const uint8_t* x,
                                 const uint8_t* xs, const int32_t* offsets, const uint8_t* w1p,
                                 const uint8_t* w1s, const uint8_t* w2p, const uint8_t* w2s,
                                 uint8_t* act, uint8_t* act_s, float* part, bf16_t* y, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_done = true;
  }
  const size_t lds = (size_t)4 * GM_STAGE + (size_t)2 * 512 * 4 + (size_t)(L + 1 + 16) * sizeof(int32_t);
  auto grid = [&](int N) {
    const int NT = (N + GM_BN - 1) / GM_BN;
    const int64_t upper = ((capacity + GM_BM - 1) / GM_BM + L) * (int64_t)NT;
    int64_t gsz = num_cus();
    if (upper < gsz) gsz = upper;
    return (int)(gsz > 0 ? gsz : 1);
  };
  const int G1 = grid(2 * F), G2 = grid(H);
  const dim3 rgrid(GEMM_SPLIT_UNITS / 2 * 8), rblk(64), blk(GM_THREADS);
  hipLaunchKernelGGL(k_gemm_mx<1>, dim3(G1), blk, lds, s, L, 2 * F, H, capacity, x, xs, offsets, w1p, w1s, act,
                     act_s, part);
  hipLaunchKernelGGL(k_mx_splitk_reduce<1>, rgrid, rblk, 0, s, L, 2 * F, H, capacity, G1, offsets, part, act, act_s);
  hipLaunchKernelGGL(k_gemm_mx<0>, dim3(G2), blk, lds, s, L, H, F, capacity, act, act_s, offsets, w2p, w2s,
                     (uint8_t*)y, (uint8_t*)nullptr, part);
  hipLaunchKernelGGL(k_mx_splitk_reduce<0>, rgrid, rblk, 0, s, L, H, F, capacity, G2, offsets, part, (uint8_t*)y,
                     (uint8_t*)nullptr);
  return hipGetLastError();
}

}  // namespace moe
