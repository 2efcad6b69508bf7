// Ragged grouped GEMMs of the expert SwiGLU MLP (fp32 and bf16).
//
// bpdata article, "Optimization 1: Grouped GEMM": all expert matmuls in one
// kernel, each with its expert's actual token count, computing only valid
// regions, with no device-to-host counts and no worst-case padding.
//
// Every workgroup builds the tile schedule from `offsets` on the device: expert
// e owns ceil(m_e/BM) x (N/BN) output tiles (none when m_e = 0), tiles of one
// weight panel (same expert and column tile) are consecutive, and a
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
// bf16 grouped GEMM: out tile 256 x 256, k step 64, 512 threads = 8 wavefronts
// as 2 (rows) x 4 (columns), each wavefront 128 x 64 = 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16; two wavefronts per SIMD hide each other's waits.
//
// The L2 -> CU path (about 64 B/clk per CU) is the scarce resource of this
// loop, so every operand byte of a tile crosses it once per k step: each thread
// moves the same four 16-byte chunks of the A and of the B k-step tile
// (64 KiB per k step) into registers one k step ahead, then into padded LDS
// rows (144 bytes: 16 consecutive rows start in 16 different bank groups), and
// the wavefronts read their MFMA fragments from LDS.  A is [rows][Kd] (EPI 1:
// x_perm) or k-blocked [Kd/64][capacity][64] (EPI 0: the activations); B is the
// prepared weight panel of 256 output columns, k-blocked [Kd/64][256][64], so a
// k-step tile of B is one contiguous 32 KiB block.  Both are read with buffer
// loads, which return zeros past the tile's rows.  Prefetch indices are clamped
// to the last k step of the range instead of branching, and k ranges have even
// length so k steps come in pairs: the k loop has no branches.
//
// Work units.  With G persistent workgroups and `total` tiles, the first
// floor(total/G)*G tiles run whole (data parallel).  The `left` tiles of a last,
// partial round would leave most CUs idle, so when left*2 <= GEMM_SPLIT_UNITS
// each of them is split into S pieces along k (split-K), S as large as fits
// the CUs and the partial buffer.  A piece writes its fp32 partial tile to
// `part`; k_splitk_reduce then sums the S partials of a tile in piece order
// (the result does not depend on timing) and applies the epilogue.
// EPI 0: out[row][col] = bf16(acc)                                   (N columns)
// EPI 1: gate/up chunks of 32 columns are interleaved in B; out = k-blocked
//        activations [N/128][capacity][64], a[row][j] = bf16(silu(gate) * up)
// ---------------------------------------------------------------------------
#define GB_BM 256
#define GB_BN 256
#define GB_BK 64
#define GB_LDK 72                   // padded LDS row (elements)
#define GB_STAGE (GB_BM * GB_LDK)   // elements of one operand stage
#define GB_THREADS 512
#define GB_PART_FLOATS (GB_BM * GB_BN)

// Epilogue of one wavefront's 128 x 64 part of a tile (MFMA D layout: lane l
// holds column l%32, rows 8 (v/4) + 4 (l/32) + v%4 of each 32 x 32 block).
template <int EPI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][2], const TileInfo& ti, int N, int64_t capacity,
                                           int wm, int wn, int g, int r32, bf16_t* __restrict__ out) {
  const int col0 = ti.nt * GB_BN;
  const int msub = min(4, max(0, (ti.rows - wm * 128 + 31) / 32));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= msub) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (row >= ti.rows) continue;
      const long grow = ti.row0 + row;
      if (EPI == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + r32;
          if (col < N) out[grow * N + col] = (bf16_t)f32_to_bf16(acc[i][j][v]);
        }
      } else {
        const int jcol = (col0 >> 1) + wn * 32 + r32;
        if (jcol < (N >> 1))
          out[((long)(jcol >> 6) * capacity + grow) * GB_BK + (jcol & 63)] =
              (bf16_t)f32_to_bf16(silu_mul(acc[i][0][v], acc[i][1][v]));
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(GB_THREADS, 1) void k_gemm_bf16(int L, int N, int Kd, int64_t capacity,
                                                             const bf16_t* __restrict__ A,
                                                             const int32_t* __restrict__ offsets,
                                                             const bf16_t* __restrict__ B, bf16_t* __restrict__ out,
                                                             float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  bf16_t* sA = (bf16_t*)smem;                         // [2][256][72]
  bf16_t* sB = sA + 2 * GB_STAGE;                     // [2][256][72]
  int32_t* s_pre = (int32_t*)(sB + 2 * GB_STAGE);     // [L+1]
  int32_t* s_tmp = s_pre + (L + 1);                   // [16]
  const int NT = (N + GB_BN - 1) / GB_BN;
  build_schedule(L, capacity, GB_BM, NT, offsets, s_pre, s_tmp);
  const int KT = Kd / GB_BK;
  const SplitPlan plan = split_plan(s_pre[L], gridDim.x, KT);
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int wm = wv >> 2, wn = wv & 3;
  const int g = l >> 5, r32 = l & 31;
  // global -> LDS: thread moves 16-byte chunk lkc of rows lrow + 64 i (i < 4)
  // of both the A and the B k-step tile
  const int lrow = tid >> 3, lkc = tid & 7;
  const int st_off = lrow * GB_LDK + lkc * 8;
  // fragment reads: A row wm*128 + i*32 + r32, B column wn*64 + jj*32 + r32,
  // k chunk 2s + g of the k step
  const int fa_base = (wm * 128 + r32) * GB_LDK + g * 8;
  const int fb_base = (wn * 64 + r32) * GB_LDK + g * 8;
  const int vb = (lrow * GB_BK + lkc * 8) * 2;

  for (int u = virtual_block(); u < plan.units; u += gridDim.x) {
    int tile = u, k0 = 0, k1 = KT, piece = -1;
    if (u >= plan.dp) {  // split-K piece: k steps [k0, k1), an even count
      piece = u - plan.dp;
      tile = plan.dp + piece / plan.S;
      const int q = piece % plan.S, half = KT / 2;
      k0 = 2 * (q * half / plan.S);
      k1 = 2 * ((q + 1) * half / plan.S);
    }
    const TileInfo ti = locate_tile(tile, L, capacity, GB_BM, NT, offsets, s_pre);
    // the (expert, panel) B tile: KT blocks of [256 columns][64 k]
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + ((long)ti.e * NT + ti.nt) * (long)KT * GB_BN * GB_BK), (short)0,
        KT * GB_BN * GB_BK * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rA =
        EPI == 1 ? __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)ti.row0 * Kd), (short)0, ti.rows * Kd * 2,
                                                     0x00020000)
                 : __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(KT * capacity * GB_BK * 2), 0x00020000);
    const int va = EPI == 1 ? (lrow * Kd + lkc * 8) * 2 : ((ti.row0 + lrow) * GB_BK + lkc * 8) * 2;
    const int astride = EPI == 1 ? 64 * Kd * 2 : 64 * GB_BK * 2;
    const int akstep = EPI == 1 ? GB_BK * 2 : (int)(capacity * GB_BK * 2);

    u32x4 ast[4], bst[4];  // register stage of the next k step
#define GB_LOAD(KT_)                                                                        \
  {                                                                                         \
    const int koa = va + (KT_) * akstep;                                                    \
    const int kob = (KT_) * (GB_BN * GB_BK * 2);                                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
      ast[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, koa + i * astride, 0, 0);          \
      bst[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, vb + i * (64 * GB_BK * 2), kob, 0); \
    }                                                                                       \
  }
#define GB_STORE(BUF)                                                                       \
  {                                                                                         \
    bf16_t* dA = sA + (BUF) * GB_STAGE + st_off;                                            \
    bf16_t* dB = sB + (BUF) * GB_STAGE + st_off;                                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
      *(u32x4*)(dA + i * 64 * GB_LDK) = ast[i];                                             \
      *(u32x4*)(dB + i * 64 * GB_LDK) = bst[i];                                             \
    }                                                                                       \
  }
#define GB_COMPUTE(BUF)                                                                     \
  {                                                                                         \
    const bf16_t* cA = sA + (BUF) * GB_STAGE + fa_base;                                     \
    const bf16_t* cB = sB + (BUF) * GB_STAGE + fb_base;                                     \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                         \
      bf16x8 fa[4], fb[2];                                                                  \
      _Pragma("unroll") for (int jj = 0; jj < 2; ++jj)                                      \
        fb[jj] = *(const bf16x8*)(cB + jj * 32 * GB_LDK + s * 16);                          \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                         \
        fa[i] = *(const bf16x8*)(cA + i * 32 * GB_LDK + s * 16);                            \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                         \
        _Pragma("unroll") for (int jj = 0; jj < 2; ++jj)                                    \
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jj], acc[i][jj], 0, 0, 0); \
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
#define GB_KLOOP(C0, C1)                                                                    \
  GB_LOAD(k0);                                                                              \
  GB_STORE(0);                                                                              \
  GB_LOAD(k0 + 1);                                                                          \
  __syncthreads();                                                                          \
  for (int kt = k0; kt < k1; kt += 2) {                                                     \
    C0;                                                                                     \
    GB_STORE(1);                                                                            \
    GB_LOAD(min(kt + 2, k1 - 1));                                                           \
    __syncthreads();                                                                        \
    C1;                                                                                     \
    GB_STORE(0);                                                                            \
    GB_LOAD(min(kt + 3, k1 - 1));                                                           \
    __syncthreads();                                                                        \
  }
    // in a tile of at most 128 rows (the short last tile of an expert) the
    // second row of wavefronts has no rows: it only moves data.  The two loop
    // versions have the same barriers.
    if (ti.rows > 128 || wm == 0) {
      GB_KLOOP(GB_COMPUTE(0), GB_COMPUTE(1));
    } else {
      GB_KLOOP(, );
    }
#undef GB_KLOOP
#undef GB_LOAD
#undef GB_STORE
#undef GB_COMPUTE

    if (piece < 0) {
      store_tile<EPI>(acc, ti, N, capacity, wm, wn, g, r32, out);
    } else {
      // partial tile, per wavefront [i][j][lane][16 values of the MFMA D layout]
      float* dst = part + (long)piece * GB_PART_FLOATS + wv * 8192 + l * 16;
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
// epilogue.  Launched with the GEMM's grid size G on GEMM_SPLIT_UNITS / 2 x 8
// workgroups of one wavefront: workgroup (b, w) handles the part of wavefront w
// of split tile b of the plan.
template <int EPI>
__global__ __launch_bounds__(64) void k_splitk_reduce(int L, int N, int Kd, int64_t capacity, int G,
                                                      const int32_t* __restrict__ offsets,
                                                      const float* __restrict__ part, bf16_t* __restrict__ out) {
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  const int NT = (N + GB_BN - 1) / GB_BN;
  build_schedule(L, capacity, GB_BM, NT, offsets, s_pre, s_tmp);
  const int total = s_pre[L];
  const SplitPlan plan = split_plan(total, G, Kd / GB_BK);
  const int b = blockIdx.x >> 3, wv = blockIdx.x & 7, l = threadIdx.x;
  if (plan.S < 2 || b >= total - plan.dp) return;
  const TileInfo ti = locate_tile(plan.dp + b, L, capacity, GB_BM, NT, offsets, s_pre);
  const float* src = part + (long)b * plan.S * GB_PART_FLOATS + wv * 8192 + l * 16;
  f32x4 sum[8][4];
#pragma unroll
  for (int ij = 0; ij < 8; ++ij)
#pragma unroll
    for (int c = 0; c < 4; ++c) sum[ij][c] = *(const f32x4*)(src + ij * 1024 + c * 4);
  for (int q = 1; q < plan.S; ++q) {
    const float* sq = src + (long)q * GB_PART_FLOATS;
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
  store_tile<EPI>(acc, ti, N, capacity, wv >> 2, wv & 3, l >> 5, l & 31, out);
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
  return (size_t)4 * GB_STAGE * sizeof(bf16_t) + (size_t)(L + 1 + 16) * sizeof(int32_t);
}

size_t grouped_mlp_bf16_part_bytes() { return (size_t)GEMM_SPLIT_UNITS * GB_PART_FLOATS * sizeof(float); }

hipError_t launch_grouped_mlp_bf16(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* w1p, const bf16_t* w2p,
                                   bf16_t* act, float* part, bf16_t* y, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  const size_t lds = gemm_bf16_lds(L);
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_bf16<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_done = true;
  }
  const int N1 = 2 * F, N2 = H;
  const int G1 = grid_for(capacity, L, GB_BM, (N1 + GB_BN - 1) / GB_BN, 1);
  const int G2 = grid_for(capacity, L, GB_BM, (N2 + GB_BN - 1) / GB_BN, 1);
  const dim3 rgrid(GEMM_SPLIT_UNITS / 2 * 8), rblk(64), blk(GB_THREADS);
  hipLaunchKernelGGL(k_gemm_bf16<1>, dim3(G1), blk, lds, s, L, N1, H, capacity, x, offsets, w1p, act, part);
  hipLaunchKernelGGL(k_splitk_reduce<1>, rgrid, rblk, 0, s, L, N1, H, capacity, G1, offsets, part, act);
  hipLaunchKernelGGL(k_gemm_bf16<0>, dim3(G2), blk, lds, s, L, N2, F, capacity, act, offsets, w2p, y, part);
  hipLaunchKernelGGL(k_splitk_reduce<0>, rgrid, rblk, 0, s, L, N2, F, capacity, G2, offsets, part, y);
  return hipGetLastError();
}

}  // namespace moe
