// Calibration kernels: the chip's achievable ceilings, measured the same way
// the layer's kernels are, so that their rates can be stated as fractions of
// what this MI355X actually sustains next to the datasheet peaks.
//
//  k_calib_copy   streaming copy, 16 bytes per lane, 4 loads in flight per lane
//  k_calib_read   streaming read (an xor of every word, one word per workgroup out)
//  k_calib_write  streaming write of a constant
//  k_calib_mfma   back-to-back matrix-core instructions on register operands:
//                 v_mfma_f32_32x32x16_bf16 (bf16) or
//                 v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 with E8M0 scales), four
//                 independent accumulators per wavefront, 8 wavefronts per CU
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// n16 = 16-byte words; grid-stride over groups of 4 words per lane
__global__ __launch_bounds__(256) void k_calib_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, long n16) {
  const long stride = (long)gridDim.x * 256 * 4;
  for (long i = (long)blockIdx.x * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j * 256 < n16) v[j] = __builtin_nontemporal_load(src + i + j * 256);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j * 256 < n16) __builtin_nontemporal_store(v[j], dst + i + j * 256);
  }
}

__global__ __launch_bounds__(256) void k_calib_read(const u32x4* __restrict__ src, long n16, uint32_t* __restrict__ out) {
  const long stride = (long)gridDim.x * 256 * 4;
  uint32_t acc = 0;
  for (long i = (long)blockIdx.x * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = i + j * 256 < n16 ? __builtin_nontemporal_load(src + i + j * 256) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  __shared__ uint32_t s[4];
  acc = wave_max_u(acc) ^ (uint32_t)wave_sum_i((int)acc);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

__global__ __launch_bounds__(256) void k_calib_write(u32x4* __restrict__ dst, long n16, uint32_t v) {
  const long stride = (long)gridDim.x * 256;
  const u32x4 w{v, v, v, v};
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) __builtin_nontemporal_store(w, dst + i);
}

// FP8 = 0: bf16 32x32x16 (32768 flops per instruction); FP8 = 1: E4M3
// 32x32x64 with unit scales (131072 flops per instruction)
template <int FP8>
__global__ __launch_bounds__(512, 1) void k_calib_mfma(int iters, float* __restrict__ out) {
  const int l = threadIdx.x & 63;
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  if constexpr (FP8) {
    // codes 0x38 (1.0) and 0x30 (0.5) varied by lane: finite operands
    i32x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = 0x38383838 ^ ((l + k) & 7);
      b[k] = 0x30303030 ^ ((l * 3 + k) & 7);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = (__bf16)(1.0f + 0.125f * ((l + k) & 7));
      b[k] = (__bf16)(0.5f - 0.0625f * ((l * 3 + k) & 7));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  out[(long)blockIdx.x * 512 + threadIdx.x] = s;
}

static int calib_grid(long n16, int per_block) {
  const long g = (n16 + per_block - 1) / per_block;
  const long cap = (long)2048;  // 8 workgroups of 256 threads on each of 256 CUs
  return (int)(g < 1 ? 1 : (g < cap ? g : cap));
}

hipError_t launch_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const long n16 = (long)(bytes / 16);
  hipLaunchKernelGGL(k_calib_copy, dim3(calib_grid(n16, 1024)), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* out, int* blocks, hipStream_t s) {
  const long n16 = (long)(bytes / 16);
  const int g = calib_grid(n16, 1024);
  *blocks = g;
  if (out) hipLaunchKernelGGL(k_calib_read, dim3(g), dim3(256), 0, s, (const u32x4*)src, n16, out);
  return hipGetLastError();
}

hipError_t launch_calib_write(void* dst, size_t bytes, uint32_t v, hipStream_t s) {
  const long n16 = (long)(bytes / 16);
  hipLaunchKernelGGL(k_calib_write, dim3(calib_grid(n16, 256)), dim3(256), 0, s, (u32x4*)dst, n16, v);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int fp8, int blocks, int iters, float* out, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL(k_calib_mfma<1>, dim3(blocks), dim3(512), 0, s, iters, out);
  else
    hipLaunchKernelGGL(k_calib_mfma<0>, dim3(blocks), dim3(512), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace moe
