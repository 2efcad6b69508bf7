// Unpermute + probability-weighted combine back into token order.
//
// bpdata article, layer figure: the combine restores token order.  Sparser-MoE
// page, "Remove work that has no selected route": post-processing visits only
// the selected slots (a wavefront ballot over the token's K slots).
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One wavefront per token, 4 per workgroup.  Each lane owns 16 bytes of every
// 1 KiB piece of the row; up to 8 pieces are accumulated at once.
template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(int T, int K, int H, const uint8_t* __restrict__ y,
                                                 const int32_t* __restrict__ s2r,
                                                 const float* __restrict__ probs, uint8_t* __restrict__ out) {
  constexpr int EPL = BF16 ? 8 : 4;  // elements per lane per piece
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  int r = -1;
  float p = 0.f;
  if (l < K) {
    r = s2r[(long)t * K + l];
    p = probs[(long)t * K + l];
  }
  const uint64_t bits = wave_ballot(r >= 0);
  const int row_bytes = H * (BF16 ? 2 : 4);
  const int npiece = (row_bytes + 1023) / 1024;
  uint8_t* dst = out + (long)t * row_bytes;
  for (int p0 = 0; p0 < npiece; p0 += 8) {
    float acc[8][EPL];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[j][i] = 0.f;
    uint64_t b = bits;
    while (b) {  // k order
      const int k = __builtin_ctzll(b);
      b &= b - 1;
      const int d = readlane_i(r, k);
      const float pk = readlane_f(p, k);
      const uint8_t* src = y + (long)d * row_bytes;
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (p0 + j) * 1024 + l * 16;
        v[j] = (p0 + j < npiece && off < row_bytes) ? *(const u32x4*)(src + off) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[j][2 * q] = fmaf(pk, bf16_to_f32(v[j][q] & 0xffffu), acc[j][2 * q]);
            acc[j][2 * q + 1] = fmaf(pk, bf16_to_f32(v[j][q] >> 16), acc[j][2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(pk, __uint_as_float(v[j][q]), acc[j][q]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
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

hipError_t launch_combine(int T, int K, int H, int dtype, const void* y, const int32_t* s2r,
                          const float* probs, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g((T + 3) / 4), b(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(k_combine<false>, g, b, 0, s, T, K, H, (const uint8_t*)y, s2r, probs, (uint8_t*)out);
  else
    hipLaunchKernelGGL(k_combine<true>, g, b, 0, s, T, K, H, (const uint8_t*)y, s2r, probs, (uint8_t*)out);
  return hipGetLastError();
}

}  // namespace moe
