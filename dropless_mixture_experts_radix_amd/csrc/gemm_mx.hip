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
// The schedule, tiling and XCD mapping match the bf16 kernel: 256 x 256 output
// tiles, k step 128 (two instructions), 8 wavefronts of 128 x 64.
// EPI 1 (GEMM1): a = silu(gate) * up is rounded to bf16 and MX-quantized along
// F in the epilogue (one 32-column gate chunk = one MX block of a row).
// EPI 0 (GEMM2): y stored as bf16.
#include "gemm_common.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GM_BM 256
#define GM_BN 256
#define GM_BK 128

struct MxTile {
  int e, row0, rows, nt;
};

__device__ __forceinline__ MxTile mx_locate(int it, int L, int64_t capacity, int NT,
                                            const int32_t* __restrict__ offsets, const int32_t* s_pre) {
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= it) lo = mid; else hi = mid - 1;
  }
  int64_t r0 = offsets[lo], r1 = offsets[lo + 1];
  r0 = r0 < capacity ? r0 : capacity;
  r1 = r1 < capacity ? r1 : capacity;
  const int m = (int)(r1 - r0);
  const int mt_e = (m + GM_BM - 1) / GM_BM;
  const int local = it - s_pre[lo];
  MxTile t;
  t.e = lo;
  t.nt = local / mt_e;
  const int mt = local % mt_e;
  t.row0 = (int)r0 + mt * GM_BM;
  t.rows = min(GM_BM, m - mt * GM_BM);
  return t;
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void k_gemm_mx(int L, int N, int Kd, int64_t capacity,
                                                    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                                                    const int32_t* __restrict__ offsets,
                                                    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
                                                    uint8_t* __restrict__ out, uint8_t* __restrict__ out_s) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sA = smem;                                 // [2][256][128]
  uint8_t* sB = sA + 2 * GM_BM * GM_BK;               // [2][256][128]
  uint8_t* sAs = sB + 2 * GM_BN * GM_BK;              // [2][256][4]
  uint8_t* sBs = sAs + 2 * GM_BM * 4;                 // [2][256][4]
  int32_t* s_pre = (int32_t*)(sBs + 2 * GM_BN * 4);   // [L+1]
  int32_t* s_tmp = s_pre + (L + 1);
  const int NT = (N + GM_BN - 1) / GM_BN;
  build_schedule(L, capacity, GM_BM, NT, offsets, s_pre, s_tmp);
  const int total = s_pre[L];
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int wm = wv >> 2, wn = wv & 3;
  const int g = l >> 5, r32 = l & 31;
  const int KT = Kd / GM_BK;
  const int KB = Kd / 32;  // scale bytes per row
  const int G = gridDim.x;
  const int vb = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  for (int it = vb; it < total; it += G) {
    const MxTile ti = mx_locate(it, L, capacity, NT, offsets, s_pre);
    const int col0 = ti.nt * GM_BN;
    const uint8_t* ga[4];
    const uint8_t* gb[4];
    int lds_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 512 * i, row = c >> 3, kc = c & 7;
      const int ar = ti.row0 + min(row, ti.rows - 1);
      ga[i] = A + (long)ar * Kd + kc * 16;
      const int bc = min(col0 + row, N - 1);
      gb[i] = B + ((long)ti.e * N + bc) * Kd + kc * 16;
      lds_off[i] = row * GM_BK + ((kc ^ lds_swz(row)) << 4);
    }
    // scales: thread tid < 256 loads the 4 A scale bytes of row tid, 256.. the B ones
    const int srow = tid & 255;
    const uint8_t* gs;
    if (tid < 256) gs = As + (long)(ti.row0 + min(srow, ti.rows - 1)) * KB;
    else gs = Bs + ((long)ti.e * N + min(col0 + srow, N - 1)) * KB;
    uint8_t* ss = (tid < 256 ? sAs : sBs) + srow * 4;

    u32x4 ra[4], rb[4];
    uint32_t rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *(const u32x4*)ga[i];
      rb[i] = *(const u32x4*)gb[i];
    }
    rs = *(const uint32_t*)gs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4*)(sA + lds_off[i]) = ra[i];
      *(u32x4*)(sB + lds_off[i]) = rb[i];
    }
    *(uint32_t*)ss = rs;
    __syncthreads();

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int msub = min(4, max(0, (ti.rows - wm * 128 + 31) / 32));

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) {
        const int ko = (kt + 1) * GM_BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ra[i] = *(const u32x4*)(ga[i] + ko);
          rb[i] = *(const u32x4*)(gb[i] + ko);
        }
        rs = *(const uint32_t*)(gs + (kt + 1) * 4);
      }
      const uint8_t* cA = sA + cur * GM_BM * GM_BK;
      const uint8_t* cB = sB + cur * GM_BN * GM_BK;
      const uint8_t* cAs = sAs + cur * GM_BM * 4;
      const uint8_t* cBs = sBs + cur * GM_BN * 4;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c0 = 4 * s + g, c1 = 4 * s + 2 + g;
        i32x8 fb[2];
        int sb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = wn * 64 + j * 32 + r32;
          const u32x4 lo = *(const u32x4*)(cB + n * GM_BK + ((c0 ^ lds_swz(n)) << 4));
          const u32x4 hi = *(const u32x4*)(cB + n * GM_BK + ((c1 ^ lds_swz(n)) << 4));
          fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          sb[j] = cBs[n * 4 + 2 * s + g];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < msub) {
            const int m = wm * 128 + i * 32 + r32;
            const u32x4 lo = *(const u32x4*)(cA + m * GM_BK + ((c0 ^ lds_swz(m)) << 4));
            const u32x4 hi = *(const u32x4*)(cA + m * GM_BK + ((c1 ^ lds_swz(m)) << 4));
            const i32x8 fa = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int sa = cAs[m * 4 + 2 * s + g];
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[j], acc[i][j], 0, 0, 0, sa, 0, sb[j]);
          }
        }
      }
      if (kt + 1 < KT) {
        uint8_t* nA = sA + (cur ^ 1) * GM_BM * GM_BK;
        uint8_t* nB = sB + (cur ^ 1) * GM_BN * GM_BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *(u32x4*)(nA + lds_off[i]) = ra[i];
          *(u32x4*)(nB + lds_off[i]) = rb[i];
        }
        *(uint32_t*)(ss + (cur ^ 1) * GM_BM * 4) = rs;
      }
      __syncthreads();
    }

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
        if (i >= msub) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
          // bf16 value of a, then the MX block (32 lanes of this half-wave)
          const uint32_t ab = f32_to_bf16(acc[i][0][v] / (1.0f + __expf(-acc[i][0][v])) * acc[i][1][v]);
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
}

hipError_t launch_grouped_mlp_mx(int L, int H, int F, int64_t capacity, const uint8_t* x,
                                 const uint8_t* xs, const int32_t* offsets, const uint8_t* w1p,
                                 const uint8_t* w1s, const uint8_t* w2p, const uint8_t* w2s,
                                 uint8_t* act, uint8_t* act_s, bf16_t* y, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_mx<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_done = true;
  }
  const size_t lds = (size_t)2 * (GM_BM + GM_BN) * GM_BK + (size_t)2 * (GM_BM + GM_BN) * 4 +
                     (size_t)(L + 1 + 16) * sizeof(int32_t);
  auto grid = [&](int N) {
    const int NT = (N + GM_BN - 1) / GM_BN;
    const int64_t upper = ((capacity + GM_BM - 1) / GM_BM + L) * (int64_t)NT;
    int64_t gsz = num_cus();
    if (upper < gsz) gsz = upper;
    return (int)(gsz > 0 ? gsz : 1);
  };
  hipLaunchKernelGGL(k_gemm_mx<1>, dim3(grid(2 * F)), dim3(512), lds, s, L, 2 * F, H, capacity, x, xs, offsets,
                     w1p, w1s, act, act_s);
  hipLaunchKernelGGL(k_gemm_mx<0>, dim3(grid(H)), dim3(512), lds, s, L, H, F, capacity, act, act_s, offsets,
                     w2p, w2s, (uint8_t*)y, (uint8_t*)nullptr);
  return hipGetLastError();
}

}  // namespace moe
