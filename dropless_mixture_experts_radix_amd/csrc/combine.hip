// Unpermute + probability-weighted combine back into token order.
//
// bpdata article, layer figure: the combine restores token order.  Sparser-MoE
// page, "Remove work that has no selected route": post-processing visits only
// the selected slots (a wavefront ballot over the token's K slots).
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One wavefront per token, 4 per workgroup.  Each lane owns 16 bytes of every
// 1 KiB piece of the row.  The token's rows are gathered RB = 8 / PCS at a
// time, PCS pieces of each (all RB x PCS loads in flight together), and added
// in k order; rows of more than 8 pieces go in chunks of 8 pieces, one row at
// a time.  Short rows (a 512-wide bf16 row is one piece) so wait for one
// memory round trip per 8 rows instead of one per row.  With probs NULL every
// weight is 1: the backward of the permute (a token's gradient is the sum of
// its routed rows' gradients, k order).
template <bool BF16, int PCS>
__global__ __launch_bounds__(256) void k_combine(int T, int K, int H, const uint8_t* __restrict__ y,
                                                 const int32_t* __restrict__ s2r,
                                                 const float* __restrict__ probs, uint8_t* __restrict__ out) {
  constexpr int EPL = BF16 ? 8 : 4;  // elements per lane per piece
  constexpr int RB = 8 / PCS;        // rows per batch
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  int r = -1;
  float p = 0.f;
  if (l < K) {
    r = s2r[(long)t * K + l];
    p = probs ? probs[(long)t * K + l] : 1.f;
  }
  const uint64_t bits = wave_ballot(r >= 0);
  const int row_bytes = H * (BF16 ? 2 : 4);
  const int npiece = (row_bytes + 1023) / 1024;
  uint8_t* dst = out + (long)t * row_bytes;
  for (int p0 = 0; p0 < npiece; p0 += PCS) {
    float acc[PCS][EPL];
#pragma unroll
    for (int j = 0; j < PCS; ++j)
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[j][i] = 0.f;
    uint64_t b = bits;
    while (b) {  // batches of RB rows, k order
      int d[RB];
      float pk[RB];
      bool ok[RB];  // wave-uniform
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        ok[i] = b != 0;
        const int k = ok[i] ? __builtin_ctzll(b) : 0;
        b &= b - 1;
        d[i] = readlane_i(r, k);
        pk[i] = readlane_f(p, k);
      }
      u32x4 v[RB][PCS];
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < PCS; ++j) {
          const int off = (p0 + j) * 1024 + l * 16;
          v[i][j] = (ok[i] && p0 + j < npiece && off < row_bytes) ? *(const u32x4*)(y + (long)d[i] * row_bytes + off)
                                                                  : u32x4{0, 0, 0, 0};
        }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (!ok[i]) continue;
#pragma unroll
        for (int j = 0; j < PCS; ++j) {
          if (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[j][2 * q] = fmaf(pk[i], bf16_to_f32(v[i][j][q] & 0xffffu), acc[j][2 * q]);
              acc[j][2 * q + 1] = fmaf(pk[i], bf16_to_f32(v[i][j][q] >> 16), acc[j][2 * q + 1]);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(pk[i], __uint_as_float(v[i][j][q]), acc[j][q]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PCS; ++j) {
      const int off = (p0 + j) * 1024 + l * 16;
      if (p0 + j < npiece && off < row_bytes) {
        u32x4 o;
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = f32_to_bf16(acc[j][2 * q]) | (f32_to_bf16(acc[j][2 * q + 1]) << 16);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[j][q]);
        }
        *(u32x4*)(dst + off) = o;
      }
    }
  }
}

// Backward of the combine, one wavefront per token: for each of its slots with
// a row r (k order) d_y[r] = p * dout[t] (rounded like y) and d_probs[t,k] =
// <dout[t], y[r]> (each lane's fixed-order fp32 partial, then the wavefront's
// fixed tree); slots without a row get d_probs 0.  The token's dout pieces are
// re-read per slot (cache hits after the first).  MX (bf16 rows): the bf16
// d_y row is also MX-quantized along H as it is written (E4M3 codes [.][H],
// E8M0 scales [.][H/32]; 4 lanes hold one 32-element block), the operand form
// the MXFP8 data gradient takes, so no separate quantization pass reads it.
template <bool BF16, bool MX>
__global__ __launch_bounds__(256) void k_combine_backward(int T, int K, int H, const uint8_t* __restrict__ dout,
                                                          const uint8_t* __restrict__ y,
                                                          const int32_t* __restrict__ s2r,
                                                          const float* __restrict__ probs,
                                                          uint8_t* __restrict__ dy, float* __restrict__ dprobs,
                                                          uint8_t* __restrict__ dyq, uint8_t* __restrict__ dyqs) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  int r = -1;
  float p = 0.f;
  if (l < K) {
    r = s2r[(long)t * K + l];
    p = probs[(long)t * K + l];
    if (r < 0) dprobs[(long)t * K + l] = 0.f;
  }
  const uint64_t bits = wave_ballot(r >= 0);
  const int row_bytes = H * (BF16 ? 2 : 4);
  const int npiece = (row_bytes + 1023) / 1024;
  const uint8_t* src_g = dout + (long)t * row_bytes;
  uint64_t b = bits;
  while (b) {  // k order
    const int k = __builtin_ctzll(b);
    b &= b - 1;
    const int d = readlane_i(r, k);
    const float pk = readlane_f(p, k);
    const uint8_t* src_y = y + (long)d * row_bytes;
    uint8_t* dst = dy + (long)d * row_bytes;
    float part = 0.f;
    for (int p0 = 0; p0 < npiece; p0 += 8) {
      u32x4 gv[8], yv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (p0 + j) * 1024 + l * 16;
        const bool in = p0 + j < npiece && off < row_bytes;
        gv[j] = in ? *(const u32x4*)(src_g + off) : u32x4{0, 0, 0, 0};
        yv[j] = in ? *(const u32x4*)(src_y + off) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (p0 + j) * 1024 + l * 16;
        u32x4 o;
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g0 = bf16_to_f32(gv[j][q] & 0xffffu), g1 = bf16_to_f32(gv[j][q] >> 16);
            part = fmaf(g0, bf16_to_f32(yv[j][q] & 0xffffu), part);
            part = fmaf(g1, bf16_to_f32(yv[j][q] >> 16), part);
            o[q] = f32_to_bf16(pk * g0) | (f32_to_bf16(pk * g1) << 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g0 = __uint_as_float(gv[j][q]);
            part = fmaf(g0, __uint_as_float(yv[j][q]), part);
            o[q] = __float_as_uint(pk * g0);
          }
        }
        if (p0 + j < npiece && off < row_bytes) *(u32x4*)(dst + off) = o;
        if (MX) {  // H % 32 == 0: the 4 lanes of a block are all in the row or all past it
          uint32_t am = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) am = max(am, max(o[q] & 0x7fffu, (o[q] >> 16) & 0x7fffu));
          am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
          am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
          const int E = mx_scale_exp(am);
          const uint32_t lo = mx_e4m3x4(o[0], o[1], E), hi = mx_e4m3x4(o[2], o[3], E);
          if (p0 + j < npiece && off < row_bytes) {
            *(uint2*)(dyq + (long)d * H + (off >> 1)) = make_uint2(lo, hi);
            if ((l & 3) == 0) dyqs[(long)d * (H >> 5) + (off >> 6)] = (uint8_t)(E + 127);
          }
        }
      }
    }
    const float dot = wave_sum_f(part);
    if (l == 0) dprobs[(long)t * K + k] = dot;
  }
}

// Backward of the route's gates for a fixed selection, one thread per token:
// d_z[t,k] = dL/dz at expert ids[t,k] (z = logit + score_bias).  Softmax over
// the selected keys: d_z_k = p_k (g_k - sum_j p_j g_j).  Normalized sigmoid,
// p_k = scale s_k / S with s = sigma(z): d_z_k = s_k (1 - s_k) (scale g_k -
// sum_j g_j p_j) / S.  Slots with id -1 give 0.
__global__ __launch_bounds__(256) void k_route_backward(int T, int E, int K, int score, float scale,
                                                        const int16_t* __restrict__ ids,
                                                        const float* __restrict__ probs,
                                                        const float* __restrict__ dprobs,
                                                        const float* __restrict__ logits,
                                                        const float* __restrict__ score_bias,
                                                        float* __restrict__ dz) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int16_t* id = ids + (long)t * K;
  const float* g = dprobs + (long)t * K;
  float* o = dz + (long)t * K;
  if (score == MOE_SCORE_SOFTMAX) {
    const float* p = probs + (long)t * K;
    float gp = 0.f;
    for (int k = 0; k < K; ++k)
      if (id[k] >= 0) gp = fmaf(p[k], g[k], gp);
    for (int k = 0; k < K; ++k) o[k] = id[k] >= 0 ? p[k] * (g[k] - gp) : 0.f;
  } else {
    float S = 0.f;
    for (int k = 0; k < K; ++k) {
      if (id[k] < 0) continue;
      float z = logits[(long)t * E + id[k]];
      if (score_bias) z += score_bias[id[k]];
      S += 1.0f / (1.0f + expf(-z));
    }
    const float inv = S > 0.f ? 1.0f / S : 0.f;
    float gp = 0.f;
    for (int k = 0; k < K; ++k) {
      if (id[k] < 0) continue;
      float z = logits[(long)t * E + id[k]];
      if (score_bias) z += score_bias[id[k]];
      const float sg = 1.0f / (1.0f + expf(-z));
      gp = fmaf(g[k], scale * sg * inv, gp);
    }
    for (int k = 0; k < K; ++k) {
      if (id[k] < 0) { o[k] = 0.f; continue; }
      float z = logits[(long)t * E + id[k]];
      if (score_bias) z += score_bias[id[k]];
      const float sg = 1.0f / (1.0f + expf(-z));
      o[k] = sg * (1.0f - sg) * (scale * g[k] - gp) * inv;
    }
  }
}

hipError_t launch_combine_backward(int T, int K, int H, int dtype, const void* dout, const void* y,
                                   const int32_t* s2r, const float* probs, void* dy, float* dprobs, uint8_t* dyq,
                                   uint8_t* dyqs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g((T + 3) / 4), b(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL((k_combine_backward<false, false>), g, b, 0, s, T, K, H, (const uint8_t*)dout,
                       (const uint8_t*)y, s2r, probs, (uint8_t*)dy, dprobs, (uint8_t*)nullptr, (uint8_t*)nullptr);
  else if (dyq)
    hipLaunchKernelGGL((k_combine_backward<true, true>), g, b, 0, s, T, K, H, (const uint8_t*)dout,
                       (const uint8_t*)y, s2r, probs, (uint8_t*)dy, dprobs, dyq, dyqs);
  else
    hipLaunchKernelGGL((k_combine_backward<true, false>), g, b, 0, s, T, K, H, (const uint8_t*)dout,
                       (const uint8_t*)y, s2r, probs, (uint8_t*)dy, dprobs, (uint8_t*)nullptr, (uint8_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_route_backward(int T, int E, int K, int score, float scale, const int16_t* ids,
                                 const float* probs, const float* dprobs, const float* logits,
                                 const float* score_bias, float* dz, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_route_backward, dim3((T + 255) / 256), dim3(256), 0, s, T, E, K, score, scale, ids, probs,
                     dprobs, logits, score_bias, dz);
  return hipGetLastError();
}

hipError_t launch_combine(int T, int K, int H, int dtype, const void* y, const int32_t* s2r,
                          const float* probs, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g((T + 3) / 4), b(256);
  const int npiece = (int)(((long)H * (dtype == MOE_F32 ? 4 : 2) + 1023) / 1024);
#define MOE_COMBINE(BF, PCS)                                                                             \
  hipLaunchKernelGGL((k_combine<BF, PCS>), g, b, 0, s, T, K, H, (const uint8_t*)y, s2r, probs, (uint8_t*)out)
  if (dtype == MOE_F32) {
    if (npiece == 1) MOE_COMBINE(false, 1);
    else if (npiece == 2) MOE_COMBINE(false, 2);
    else if (npiece <= 4) MOE_COMBINE(false, 4);
    else MOE_COMBINE(false, 8);
  } else {
    if (npiece == 1) MOE_COMBINE(true, 1);
    else if (npiece == 2) MOE_COMBINE(true, 2);
    else if (npiece <= 4) MOE_COMBINE(true, 4);
    else MOE_COMBINE(true, 8);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
