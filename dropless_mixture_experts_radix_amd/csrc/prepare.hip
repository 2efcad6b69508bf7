// One-time expert weight layout (+ MX quantization) and the standalone MX
// quantizer.
//
// bpdata article, reproduction settings: the expert weights are pre-fused once.
// Prepared rows (per expert): W1 row p = column c(p) of W1[e] with gate/up
// chunks of 32 interleaved, c(p) = (p/64)*32 + p%32 + ((p/32)%2 ? F : 0);
// W2 row n = column n of W2[e].  Rows run along the contraction dimension; the
// bf16 layout is additionally blocked so the grouped GEMM streams contiguous
// 16 KiB pieces.
#include "moe_internal.h"

namespace moe {

// One 32 x 32 tile of one expert: logical W [Kd][Ncols] -> prepared rows.
// MODE 0: fp32 -> fp32, row-major [Ncols][Kd].
// MODE 1: bf16 -> bf16 in k-blocked panels: per 256-row panel and 32-wide k
//         step one contiguous 16 KiB block [256 rows][32 k]; rows past Ncols in
//         the last panel are zero.
// MODE 2: bf16 -> MX E4M3 codes and E8M0 scales in k-blocked panels: per
//         256-row panel and 64-wide k step one contiguous 16 KiB block of codes
//         [256 rows][64 k], and per 512-wide k group one 4 KiB block of scales
//         [256 rows][16 blocks] (bytes past the last block of a short final
//         group are not written); rows past Ncols in the last panel are zero
//         (codes and scales).
// MODE 3: bf16 -> MXFP4: E2M1 codes two per byte (element 2i in the low
//         nibble) in k-blocked panels of [256 rows][128 k = 64 bytes] per
//         128-wide k step, scales as in MODE 2.
// TRANS: the input is stored transposed, [Ncols][Kd] (the backward's W2^T and
// W1^T panels are made from W2 [F][H] and W1 [H][2F] as they are).
template <int MODE, bool TRANS = false>
__global__ __launch_bounds__(256) void k_prepare(int Kd, int Ncols, int F_interleave,
                                                 const void* __restrict__ w, void* __restrict__ wp,
                                                 uint8_t* __restrict__ ws) {
  __shared__ uint32_t tile[32][33];
  const int e = blockIdx.z;
  const int pc = blockIdx.x;  // prepared 32-row chunk
  const int k0 = blockIdx.y * 32;
  const bool live = pc * 32 < Ncols;
  const int cbase = F_interleave ? (pc >> 1) * 32 + ((pc & 1) ? F_interleave : 0) : pc * 32;
  const long in_off = (long)e * Kd * Ncols;
  const int tid = threadIdx.x;
  for (int i = tid; i < 1024; i += 256) {
    const int kk = TRANS ? (i & 31) : (i >> 5), cc = TRANS ? (i >> 5) : (i & 31);
    uint32_t v = 0;
    if (live) {
      const long src = TRANS ? in_off + (long)(cbase + cc) * Kd + k0 + kk : in_off + (long)(k0 + kk) * Ncols + cbase + cc;
      v = MODE == 0 ? __float_as_uint(((const float*)w)[src]) : ((const bf16_t*)w)[src];
    }
    tile[cc][kk] = v;
  }
  __syncthreads();
  if (MODE == 0) {
    const long out_off = (long)e * Ncols * Kd;
    for (int i = tid; i < 1024; i += 256) {
      const int pp = i >> 5, kk = i & 31;
      ((float*)wp)[out_off + (long)(pc * 32 + pp) * Kd + k0 + kk] = __uint_as_float(tile[pp][kk]);
    }
  } else if (MODE == 1) {
    const int NP = (Ncols + 255) / 256, KT = Kd / 32;
    const long out_off = (long)e * NP * 256 * Kd;
    for (int i = tid; i < 1024; i += 256) {
      const int pp = i >> 5, kk = i & 31;
      const int p = pc * 32 + pp, k = k0 + kk;
      const long o = out_off + ((long)(p >> 8) * KT + (k >> 5)) * (256 * 32) + (p & 255) * 32 + (k & 31);
      ((bf16_t*)wp)[o] = (bf16_t)tile[pp][kk];
    }
  } else if (MODE == 3) {
    if (tid < 32) {
      const int pp = tid;
      uint32_t am = 0;
      for (int kk = 0; kk < 32; ++kk) {
        const uint32_t a = tile[pp][kk] & 0x7fffu;
        am = am > a ? am : a;
      }
      const int E = mx4_scale_exp(am);
      const int NP = (Ncols + 255) / 256, KT = Kd / 128, NG = (Kd + 511) / 512;
      const int p = pc * 32 + pp;
      const long panel = (long)e * NP + (p >> 8);
      uint8_t* dst = (uint8_t*)wp + (panel * KT + (k0 >> 7)) * (256 * 64) + (p & 255) * 64 + ((k0 & 127) >> 1);
      for (int kk = 0; kk < 32; kk += 2)
        dst[kk >> 1] = (uint8_t)(mx_e2m1(tile[pp][kk], E) | (mx_e2m1(tile[pp][kk + 1], E) << 4));
      ws[(panel * NG + (k0 >> 9)) * (256 * 16) + (p & 255) * 16 + ((k0 >> 5) & 15)] = (uint8_t)(E + 127);
    }
  } else if (tid < 32) {
    const int pp = tid;
    uint32_t am = 0;
    for (int kk = 0; kk < 32; ++kk) {
      const uint32_t a = tile[pp][kk] & 0x7fffu;
      am = am > a ? am : a;
    }
    const int E = mx_scale_exp(am);
    const int NP = (Ncols + 255) / 256, KT = Kd / 64, NG = (Kd + 511) / 512;
    const int p = pc * 32 + pp;
    const long panel = (long)e * NP + (p >> 8);
    uint8_t* dst = (uint8_t*)wp + (panel * KT + (k0 >> 6)) * (256 * 64) + (p & 255) * 64 + (k0 & 63);
    for (int kk = 0; kk < 32; ++kk) dst[kk] = (uint8_t)mx_e4m3(tile[pp][kk], E);
    ws[(panel * NG + (k0 >> 9)) * (256 * 16) + (p & 255) * 16 + ((k0 >> 5) & 15)] = (uint8_t)(E + 127);
  }
}

hipError_t launch_prepare_weights(int L, int H, int F, int dtype, const void* w1, const void* w2,
                                  void* w1p, void* w2p, uint8_t* w1s, uint8_t* w2s, hipStream_t s) {
  if (L == 0) return hipSuccess;
  const dim3 b(256);
  if (dtype == MOE_F32) {
    hipLaunchKernelGGL(k_prepare<0>, dim3(2 * F / 32, H / 32, L), b, 0, s, H, 2 * F, F, w1, w1p, (uint8_t*)nullptr);
    hipLaunchKernelGGL(k_prepare<0>, dim3(H / 32, F / 32, L), b, 0, s, F, H, 0, w2, w2p, (uint8_t*)nullptr);
  } else if (dtype == MOE_BF16) {
    // prepared rows padded to whole 256-row panels
    hipLaunchKernelGGL(k_prepare<1>, dim3((2 * F + 255) / 256 * 8, H / 32, L), b, 0, s, H, 2 * F, F, w1, w1p,
                       (uint8_t*)nullptr);
    hipLaunchKernelGGL(k_prepare<1>, dim3((H + 255) / 256 * 8, F / 32, L), b, 0, s, F, H, 0, w2, w2p,
                       (uint8_t*)nullptr);
  } else if (dtype == MOE_MXFP8) {
    hipLaunchKernelGGL(k_prepare<2>, dim3((2 * F + 255) / 256 * 8, H / 32, L), b, 0, s, H, 2 * F, F, w1, w1p, w1s);
    hipLaunchKernelGGL(k_prepare<2>, dim3((H + 255) / 256 * 8, F / 32, L), b, 0, s, F, H, 0, w2, w2p, w2s);
  } else {
    hipLaunchKernelGGL(k_prepare<3>, dim3((2 * F + 255) / 256 * 8, H / 32, L), b, 0, s, H, 2 * F, F, w1, w1p, w1s);
    hipLaunchKernelGGL(k_prepare<3>, dim3((H + 255) / 256 * 8, F / 32, L), b, 0, s, F, H, 0, w2, w2p, w2s);
  }
  return hipGetLastError();
}

// The backward's bf16 panels: W2^T (columns f of F, k = h of H) from W2
// [F][H], and W1^T (columns h of H, k = j of 2F in natural order) from W1
// [H][2F]; layout as MODE 1.
hipError_t launch_prepare_weights_backward(int L, int H, int F, int dtype, const void* w1, const void* w2,
                                           void* w1t, void* w2t, uint8_t* w1ts, uint8_t* w2ts, hipStream_t s) {
  if (L == 0) return hipSuccess;
  const dim3 b(256);
  if (dtype == MOE_MXFP8) {  // MODE 2 panels (E4M3 codes, E8M0 scales per 32 along k)
    hipLaunchKernelGGL((k_prepare<2, true>), dim3((F + 255) / 256 * 8, H / 32, L), b, 0, s, H, F, 0, w2, w2t, w2ts);
    hipLaunchKernelGGL((k_prepare<2, true>), dim3((H + 255) / 256 * 8, 2 * F / 32, L), b, 0, s, 2 * F, H, 0, w1,
                       w1t, w1ts);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_prepare<1, true>), dim3((F + 255) / 256 * 8, H / 32, L), b, 0, s, H, F, 0, w2, w2t,
                     (uint8_t*)nullptr);
  hipLaunchKernelGGL((k_prepare<1, true>), dim3((H + 255) / 256 * 8, 2 * F / 32, L), b, 0, s, 2 * F, H, 0, w1, w1t,
                     (uint8_t*)nullptr);
  return hipGetLastError();
}

// Standalone MX quantization: one thread per 32-element block of a row.
__global__ __launch_bounds__(256) void k_mx_quantize(int64_t rows, int cols, const bf16_t* __restrict__ in,
                                                     const int32_t* __restrict__ row_limit,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int nb = cols / 32;
  int64_t lim = rows;
  if (row_limit) {
    const int64_t rl = *row_limit;
    lim = rl < rows ? (rl > 0 ? rl : 0) : rows;
  }
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < lim * nb;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb;
    const int b = (int)(i % nb);
    const uint32_t* src = (const uint32_t*)(in + r * cols + b * 32);
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = ((const uint4*)src)[q];
      v[4 * q] = u.x; v[4 * q + 1] = u.y; v[4 * q + 2] = u.z; v[4 * q + 3] = u.w;
    }
    uint32_t am = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t a0 = v[q] & 0x7fffu, a1 = (v[q] >> 16) & 0x7fffu;
      am = am > a0 ? am : a0;
      am = am > a1 ? am : a1;
    }
    const int E = mx_scale_exp(am);
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      out[q] = mx_e4m3x4(v[2 * q], v[2 * q + 1], E);
    }
    uint4* dst = (uint4*)(codes + r * cols + b * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    scales[r * nb + b] = (uint8_t)(E + 127);
  }
}

hipError_t launch_mx_quantize(int64_t rows, int cols, const bf16_t* in, const int32_t* row_limit,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t work = rows * (cols / 32);
  const int blocks = (int)((work + 255) / 256 < 8192 ? (work + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_mx_quantize, dim3(blocks), dim3(256), 0, s, rows, cols, in, row_limit, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
