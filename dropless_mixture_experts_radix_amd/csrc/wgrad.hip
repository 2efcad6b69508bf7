// Operand layouts of the grouped MLP's weight gradient.
//
// dW1[e] = X_e^T d_h_e and dW2[e] = a_e^T d_y_e contract over expert e's own
// rows (a ragged contraction: the bpdata article's grouped GEMM on
// variable-length groups, seen from the weight side).  The matrix cores take
// both operands with the contraction index contiguous per lane, so the rows of
// each operand are regrouped here into token blocks: [block][C columns][32
// tokens], every expert's rows padded with zeros to a multiple of 128 (whole
// 4-step groups of the GEMM's k loop).  pb[e] = the first block of expert e.
#include "gemm_common.h"

namespace moe {

// pb[e] = sum over e' < e of ceil(m_e' / 128) * 4, pb[L] = all blocks
__global__ __launch_bounds__(1024) void k_wgrad_blocks(int L, int64_t capacity, const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ pb) {
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  build_schedule(L, capacity, 128, 4, offsets, s_pre, s_tmp);
  for (int e = threadIdx.x; e <= L; e += blockDim.x) pb[e] = s_pre[e];
}

// One block b (32 tokens) x 64 columns per workgroup of 256 threads.
// SRC 0: rows [capacity][C] bf16 (x_perm, d_y).
// SRC 1: k-blocked [C/32][capacity][32] bf16 (d_h, natural column order).
// SRC 2: a = bf16(silu(g) * u) from h, k-blocked [2C/32][capacity][32] with
//        gate/up chunks of 32 interleaved (g of column f in chunk 2 (f/32), u
//        in chunk 2 (f/32) + 1).
template <int SRC>
__global__ __launch_bounds__(256) void k_wgrad_pack(int L, int C, int64_t capacity, const bf16_t* __restrict__ src,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ pb, bf16_t* __restrict__ out) {
  __shared__ uint16_t tile[64][34];
  __shared__ int s_info[3];
  const int b = blockIdx.y, c0 = blockIdx.x * 64, tid = threadIdx.x;
  if (b >= pb[L]) return;  // uniform: blocks past the last expert's
  if (tid == 0) {
    const int e = find_expert(pb, L, b);
    int r0;
    const int m = expert_rows(offsets, e, capacity, &r0);
    s_info[0] = r0 + (b - pb[e]) * 32;             // first row of the block
    s_info[1] = min(32, max(0, m - (b - pb[e]) * 32));  // rows of the block that exist
  }
  __syncthreads();
  const int t0 = s_info[0], nt = s_info[1];
  const int tt = tid >> 3, cg = tid & 7, c = c0 + cg * 8;
  uint16_t v[8];
  if (tt < nt) {
    const long t = t0 + tt;
    uint4 q;
    if (SRC == 0) {
      q = *(const uint4*)(src + t * C + c);
    } else if (SRC == 1) {
      q = *(const uint4*)(src + ((long)(c >> 5) * capacity + t) * 32 + (c & 31));
    } else {
      const uint4 gq = *(const uint4*)(src + ((long)(2 * (c >> 5)) * capacity + t) * 32 + (c & 31));
      const uint4 uq = *(const uint4*)(src + ((long)(2 * (c >> 5) + 1) * capacity + t) * 32 + (c & 31));
      const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g0 = bf16_to_f32(gw[i] & 0xffffu), g1 = bf16_to_f32(gw[i] >> 16);
        const float u0 = bf16_to_f32(uw[i] & 0xffffu), u1 = bf16_to_f32(uw[i] >> 16);
        o[i] = f32_to_bf16(silu_mul(g0, u0)) | (f32_to_bf16(silu_mul(g1, u1)) << 16);
      }
      q = make_uint4(o[0], o[1], o[2], o[3]);
    }
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (uint16_t)(w4[i] & 0xffffu);
      v[2 * i + 1] = (uint16_t)(w4[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0;  // padding rows of the expert
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) tile[cg * 8 + i][tt] = v[i];
  __syncthreads();
  const int oc = tid >> 2, part = tid & 3;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (uint32_t)tile[oc][part * 8 + 2 * i] | ((uint32_t)tile[oc][part * 8 + 2 * i + 1] << 16);
  *(uint4*)(out + ((long)b * C + c0 + oc) * 32 + part * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Group-aware column-wise MX quantization of rows [capacity][C] bf16: the
// token blocks of k_wgrad_pack<0>, each column of a block one MX block (E4M3
// codes, E8M0 scale, OCP MX v1.0): codes [b][C][32], scales [b][C].  Four
// lanes hold one column's 32 values; their block maximum meets by two xor
// shuffles.
__global__ __launch_bounds__(256) void k_mx_columns_grouped(int L, int C, int64_t capacity,
                                                            const bf16_t* __restrict__ src,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ pb, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  __shared__ uint16_t tile[64][34];
  __shared__ int s_info[2];
  const int b = blockIdx.y, c0 = blockIdx.x * 64, tid = threadIdx.x;
  if (b >= pb[L]) return;  // uniform
  if (tid == 0) {
    const int e = find_expert(pb, L, b);
    int r0;
    const int m = expert_rows(offsets, e, capacity, &r0);
    s_info[0] = r0 + (b - pb[e]) * 32;
    s_info[1] = min(32, max(0, m - (b - pb[e]) * 32));
  }
  __syncthreads();
  const int t0 = s_info[0], nt = s_info[1];
  const int tt = tid >> 3, cg = tid & 7;
  uint4 q = make_uint4(0, 0, 0, 0);
  if (tt < nt) q = *(const uint4*)(src + (long)(t0 + tt) * C + c0 + cg * 8);
  const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tile[cg * 8 + 2 * i][tt] = (uint16_t)(w4[i] & 0xffffu);
    tile[cg * 8 + 2 * i + 1][tt] = (uint16_t)(w4[i] >> 16);
  }
  __syncthreads();
  const int oc = tid >> 2, part = tid & 3;
  uint32_t v[8], am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = tile[oc][part * 8 + i];
    am = max(am, v[i] & 0x7fffu);
  }
  am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
  const int E = mx_scale_exp(am);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= mx_e4m3(v[i], E) << (8 * i);
    hi |= mx_e4m3(v[4 + i], E) << (8 * i);
  }
  *(uint2*)(codes + ((long)b * C + c0 + oc) * 32 + part * 8) = make_uint2(lo, hi);
  if (part == 0) scales[(long)b * C + c0 + oc] = (uint8_t)(E + 127);
}

hipError_t launch_mx_columns_grouped(int L, int64_t capacity, int C, int nbmax, const bf16_t* in,
                                     const int32_t* offsets, int32_t* pb, uint8_t* codes, uint8_t* scales,
                                     hipStream_t s) {
  hipLaunchKernelGGL(k_wgrad_blocks, dim3(1), dim3(1024), 0, s, L, capacity, offsets, pb);
  if (nbmax > 0)
    hipLaunchKernelGGL(k_mx_columns_grouped, dim3(C / 64, nbmax), dim3(256), 0, s, L, C, capacity, in, offsets, pb,
                       codes, scales);
  return hipGetLastError();
}

// dW[e] = 0 for the experts without rows (the GEMM has no tiles for them)
__global__ __launch_bounds__(256) void k_wgrad_zero_empty(int L, int64_t capacity, long per_expert,
                                                          const int32_t* __restrict__ offsets, float* __restrict__ dw) {
  const int e = blockIdx.y;
  int r0;
  if (expert_rows(offsets, e, capacity, &r0) > 0) return;
  float4* p = (float4*)(dw + (long)e * per_expert);
  for (long i = blockIdx.x * 256L + threadIdx.x; i < per_expert / 4; i += (long)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// MXFP8 weight gradient operands: each expert's rows padded to Kp_e, a
// multiple of 256 (whole 4-stage groups of the MX GEMM); pk[e] = sum of Kp
// over the experts before e.  Each 32-row block of one expert and one column
// is an MX block (group-aware column-wise quantization).  Outputs in the MX
// GEMM's own layouts:
//   MODE 0 (A, rows = the C columns of the input): codes [C][Kp_e] per expert
//     at pk[e] * C, scales [C][Kp_e/32] at pk[e] * C / 32;
//   MODE 1 (B, columns = the C columns): per expert ceil(C/256) panels of
//     [Kp_e/64 stages][256][64] codes at pk[e] * CP (CP = ceil(C/256) * 256),
//     scales [panel][ceil(Kp_e/512)][256][16] at png[e] * CP * 16 (png = sum of
//     ceil(Kp/512)).
// SRC as k_wgrad_pack.
__global__ __launch_bounds__(1024) void k_wgrad_mx_prefix(int L, int64_t capacity, const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ pk, int32_t* __restrict__ png) {
  __shared__ int32_t s_pre[MOE_MAX_L + 1];
  __shared__ int32_t s_tmp[16];
  build_schedule(L, capacity, 256, 256, offsets, s_pre, s_tmp);   // Kp_e = ceil(m/256) * 256
  for (int e = threadIdx.x; e <= L; e += blockDim.x) pk[e] = s_pre[e];
  __syncthreads();
  build_schedule(L, capacity, 512, 1, offsets, s_pre, s_tmp);     // ceil(m/512) = ceil(Kp/512)
  for (int e = threadIdx.x; e <= L; e += blockDim.x) png[e] = s_pre[e];
}

template <int SRC, int MODE>
__global__ __launch_bounds__(256) void k_wgrad_mx_pack(int L, int C, int64_t capacity, const bf16_t* __restrict__ src,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ pk, const int32_t* __restrict__ png,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ uint16_t tile[64][34];
  __shared__ int s_info[5];
  const int b = blockIdx.y, c0 = blockIdx.x * 64, tid = threadIdx.x;
  if (b >= pk[L] / 32) return;  // uniform: blocks past the last expert's
  if (tid == 0) {
    const int e = find_expert(pk, L, b * 32);
    int r0;
    const int m = expert_rows(offsets, e, capacity, &r0);
    const int lb = b - pk[e] / 32;
    s_info[0] = r0 + lb * 32;
    s_info[1] = min(32, max(0, m - lb * 32));
    s_info[2] = e;
    s_info[3] = lb;
  }
  __syncthreads();
  const int t0 = s_info[0], nt = s_info[1], e = s_info[2], lb = s_info[3];
  const int tt = tid >> 3, cg = tid & 7, c = c0 + cg * 8;
  uint4 q = make_uint4(0, 0, 0, 0);
  if (tt < nt) {
    const long t = t0 + tt;
    if (SRC == 0) {
      q = *(const uint4*)(src + t * C + c);
    } else if (SRC == 1) {
      q = *(const uint4*)(src + ((long)(c >> 5) * capacity + t) * 32 + (c & 31));
    } else {
      const uint4 gq = *(const uint4*)(src + ((long)(2 * (c >> 5)) * capacity + t) * 32 + (c & 31));
      const uint4 uq = *(const uint4*)(src + ((long)(2 * (c >> 5) + 1) * capacity + t) * 32 + (c & 31));
      const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g0 = bf16_to_f32(gw[i] & 0xffffu), g1 = bf16_to_f32(gw[i] >> 16);
        const float u0 = bf16_to_f32(uw[i] & 0xffffu), u1 = bf16_to_f32(uw[i] >> 16);
        o[i] = f32_to_bf16(silu_mul(g0, u0)) | (f32_to_bf16(silu_mul(g1, u1)) << 16);
      }
      q = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tile[cg * 8 + 2 * i][tt] = (uint16_t)(w4[i] & 0xffffu);
    tile[cg * 8 + 2 * i + 1][tt] = (uint16_t)(w4[i] >> 16);
  }
  __syncthreads();
  const int oc = tid >> 2, part = tid & 3, col = c0 + oc;
  uint32_t v[8], am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = tile[oc][part * 8 + i];
    am = max(am, v[i] & 0x7fffu);
  }
  am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
  const int E = mx_scale_exp(am);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= mx_e4m3(v[i], E) << (8 * i);
    hi |= mx_e4m3(v[4 + i], E) << (8 * i);
  }
  const long Kp = pk[e + 1] - pk[e];
  long co, so;
  if (MODE == 0) {
    co = (long)pk[e] * C + (long)col * Kp + lb * 32 + part * 8;
    so = (long)(pk[e] / 32) * C + (long)col * (Kp / 32) + lb;
  } else {
    const long CP = (long)((C + 255) / 256) * 256, KT = Kp / 64, NG = (Kp + 511) / 512;
    const int p = col >> 8, rr = col & 255;
    co = (long)pk[e] * CP + (((long)p * KT + (lb >> 1)) * 256 + rr) * 64 + (lb & 1) * 32 + part * 8;
    so = (long)png[e] * CP * 16 + (((long)p * NG + (lb >> 4)) * 256 + rr) * 16 + (lb & 15);
  }
  *(uint2*)(codes + co) = make_uint2(lo, hi);
  if (part == 0) scales[so] = (uint8_t)(E + 127);
}

hipError_t launch_wgrad_mx_layouts(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf,
                                   const bf16_t* dhbuf, int32_t* pk, int32_t* png, uint8_t* xa, uint8_t* xas,
                                   uint8_t* dhb, uint8_t* dhbs, uint8_t* aa, uint8_t* aas, uint8_t* dyb,
                                   uint8_t* dybs, float* dW1, float* dW2, hipStream_t s) {
  hipLaunchKernelGGL(k_wgrad_mx_prefix, dim3(1), dim3(1024), 0, s, L, capacity, offsets, pk, png);
  const dim3 b(256);
  hipLaunchKernelGGL((k_wgrad_mx_pack<0, 0>), dim3(H / 64, nbmax), b, 0, s, L, H, capacity, x, offsets, pk, png, xa, xas);
  hipLaunchKernelGGL((k_wgrad_mx_pack<1, 1>), dim3(2 * F / 64, nbmax), b, 0, s, L, 2 * F, capacity, dhbuf, offsets, pk,
                     png, dhb, dhbs);
  hipLaunchKernelGGL((k_wgrad_mx_pack<2, 0>), dim3(F / 64, nbmax), b, 0, s, L, F, capacity, hbuf, offsets, pk, png, aa,
                     aas);
  hipLaunchKernelGGL((k_wgrad_mx_pack<0, 1>), dim3(H / 64, nbmax), b, 0, s, L, H, capacity, dy, offsets, pk, png, dyb,
                     dybs);
  hipLaunchKernelGGL(k_wgrad_zero_empty, dim3(256, L), b, 0, s, L, capacity, (long)H * 2 * F, offsets, dW1);
  hipLaunchKernelGGL(k_wgrad_zero_empty, dim3(256, L), b, 0, s, L, capacity, (long)F * H, offsets, dW2);
  return hipGetLastError();
}

hipError_t launch_wgrad_layouts(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf, const bf16_t* dhbuf,
                                int32_t* pb, bf16_t* xt, bf16_t* dht, bf16_t* at, bf16_t* dyt, float* dW1,
                                float* dW2, hipStream_t s) {
  hipLaunchKernelGGL(k_wgrad_blocks, dim3(1), dim3(1024), 0, s, L, capacity, offsets, pb);
  const dim3 b(256);
  hipLaunchKernelGGL(k_wgrad_pack<0>, dim3(H / 64, nbmax), b, 0, s, L, H, capacity, x, offsets, pb, xt);
  hipLaunchKernelGGL(k_wgrad_pack<1>, dim3(2 * F / 64, nbmax), b, 0, s, L, 2 * F, capacity, dhbuf, offsets, pb, dht);
  hipLaunchKernelGGL(k_wgrad_pack<2>, dim3(F / 64, nbmax), b, 0, s, L, F, capacity, hbuf, offsets, pb, at);
  hipLaunchKernelGGL(k_wgrad_pack<0>, dim3(H / 64, nbmax), b, 0, s, L, H, capacity, dy, offsets, pb, dyt);
  hipLaunchKernelGGL(k_wgrad_zero_empty, dim3(256, L), b, 0, s, L, capacity, (long)H * 2 * F, offsets, dW1);
  hipLaunchKernelGGL(k_wgrad_zero_empty, dim3(256, L), b, 0, s, L, capacity, (long)F * H, offsets, dW2);
  return hipGetLastError();
}

}  // namespace moe
