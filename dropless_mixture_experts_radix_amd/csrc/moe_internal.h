// Internal helpers shared by the HIP kernels of the MoE hot path (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WAVE 64

typedef uint16_t bf16_t;  // raw bfloat16 bits

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Order-preserving uint32 keys of fp32 values (larger float -> larger key).
// -0.0 is read as +0.0 first, so equal floats give equal keys.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ __forceinline__ bool key_finite(uint32_t k) {
  float f = key_float(k);
  return (__float_as_uint(f) & 0x7f800000u) != 0x7f800000u;
}

// ---------------------------------------------------------------------------
// Wavefront helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// number of set bits of m below this lane
__device__ __forceinline__ int mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

// inclusive prefix sum over the wave
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int w = __shfl_up(v, o, 64);
    if (l >= o) v += w;
  }
  return v;
}

__device__ __forceinline__ int readlane_i(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ void set_err(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

// ---------------------------------------------------------------------------
// OCP MX (v1.0) E4M3 block quantization of bf16 values, integer arithmetic.
//   scale exponent E = clamp(floor(log2 amax) - 8, -127, 127)  (-127 if amax==0)
//   code = E4M3(v * 2^-E): round to nearest, ties to even, saturate to 448,
//   the sign of zero kept.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int bf16_floor_log2(uint32_t absbits) {  // absbits != 0
  uint32_t ef = absbits >> 7;
  if (ef) return (int)ef - 127;
  return -133 + (31 - __clz(absbits));
}

__device__ __forceinline__ int mx_scale_exp(uint32_t amax_abs_bits) {
  if (amax_abs_bits == 0) return -127;
  int e = bf16_floor_log2(amax_abs_bits) - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ float mx_scaled(uint32_t b, int E) {
  // bf16 value times 2^-E, clamped to the largest E4M3 magnitude (448): the
  // power-of-two scaling is exact (results below 2^-126 all become zero codes)
  const float y = __builtin_amdgcn_ldexpf(__uint_as_float(b << 16), -E);
  return fminf(fmaxf(y, -448.0f), 448.0f);
}
// E4M3 code of bf16 value b (bits) under block scale 2^E: round to nearest
// even, saturate at 448, keep the sign of zero.  The hardware conversion does
// the rounding; it agrees bit for bit with a step-by-step integer conversion
// of the OCP rules for every finite bf16 pattern and every E in [-127, 127].
__device__ __forceinline__ uint32_t mx_e4m3(uint32_t b, int E) {
  const float y = mx_scaled(b, E);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xffu;
}
// four codes (bytes 0..3) of the bf16 pairs p0 = (e0 | e1 << 16), p1 = (e2 | e3 << 16)
__device__ __forceinline__ uint32_t mx_e4m3x4(uint32_t p0, uint32_t p1, int E) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(p0 & 0xffffu, E), mx_scaled(p0 >> 16, E), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(p1 & 0xffffu, E), mx_scaled(p1 >> 16, E), lo, true);
}

// MXFP4 (OCP MX E2M1 elements): the block exponent is floor(log2 amax) - 2
// (6 = 1.5 * 2^2 is E2M1's largest normal), clamped to the E8M0 range.
__device__ __forceinline__ int mx4_scale_exp(uint32_t amax_abs_bits) {
  if (amax_abs_bits == 0) return -127;
  int e = bf16_floor_log2(amax_abs_bits) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// E2M1 code (4 bits) of bf16 value b (bits) under block scale 2^E: the
// magnitude |b| * 2^-E (exact) is compared with the midpoints of the grid
// 0, 0.5, 1, 1.5, 2, 3, 4, 6; a value on a midpoint goes to the neighbour with
// the even code (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4) and everything above 5 to 6 (saturation).  The sign bit is
// the value's, zeros included.
__device__ __forceinline__ uint32_t mx_e2m1(uint32_t b, int E) {
  const float a = __builtin_amdgcn_ldexpf(__uint_as_float((b & 0x7fffu) << 16), -E);
  const uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return m | ((b >> 12) & 8u);
}

// ---------------------------------------------------------------------------
// Host-side launchers (one per kernel family, defined in the kernel sources).
// All return hipError_t of the launch.
// ---------------------------------------------------------------------------
namespace moe {

struct RouteSplit {
  int S;         // number of H chunks (partial logit sets) of the wavefront projection
  int Hc;        // chunk length
  int C;         // prepared router rows (multiple of 32)
  int Sg;        // pieces of the GEMM projection (bf16 x and weights), 0: not used
};
RouteSplit route_split(int T, int E, int H, int x_dtype);
int router_gemm_pieces(int T, int E, int H);
hipError_t launch_router_gemm_bf16(int T, int E, int H, int S, const bf16_t* x, const bf16_t* wp, float* partial,
                                   hipStream_t s);

hipError_t launch_prepare_router(const void* w, int w_dtype, int x_dtype, int H, int E, void* out,
                                 hipStream_t s);
hipError_t launch_router_proj(int T, int E, int H, int x_dtype, int w_dtype, const void* x,
                              const void* wp, float* partial, hipStream_t s);
bool route_fused_ok(int E, int H, int x_dtype, int w_dtype);
hipError_t launch_route_fused(int T, int E, int K, int H, int score, int w_dtype, const void* x, const void* wp,
                              const float* bias, const uint8_t* mask, int16_t* ids, float* probs,
                              float* logits_out, int32_t* err, hipStream_t s);
// Group-limited routing with a selection-only bias (moe_route_topk_grouped):
// n_group groups of E/n_group experts, the topk_group best kept, a group
// scored by the fp32 sum of its m = K/topk_group largest keys; gates scaled.
struct RouteGroups {
  int n_group, topk_group, m;
  float scale;
};
#define ROUTE_GRP_MAX_E 1024   // experts of the grouped selection
#define ROUTE_GRP_MAX_M 8      // keys summed per group

hipError_t launch_route_select(int T, int E, int K, int S, int score, const float* partial,
                               const float* bias, const uint8_t* mask, int16_t* ids, float* probs,
                               float* logits_out, int32_t* err, hipStream_t s,
                               const RouteGroups* grp = nullptr, float* scores_out = nullptr);

int permute_tile_tokens(int T, int K, int L);
size_t permute_workspace_bytes(int T, int K, int L);
size_t permute_state_bytes(int T, int K, int L);  // the zero-between-calls prefix
size_t permute_noalloc_max_bytes();
hipError_t launch_permute_noalloc(int T, int H, int K, int E_global, int e0, int L, int64_t capacity, int x_dtype,
                                  int out_dtype, const void* x, const int16_t* ids, int32_t* counts,
                                  int32_t* offsets, void* x_perm, uint8_t* x_scales, int32_t* row_to_slot,
                                  int32_t* slot_to_row, int32_t* err, hipStream_t s);
hipError_t launch_permute(int T, int H, int K, int E_global, int e0, int L, int64_t capacity,
                          int x_dtype, int out_dtype, const void* x, const int16_t* ids,
                          int32_t* counts, int32_t* offsets, void* x_perm, uint8_t* x_scales,
                          int32_t* row_to_slot, int32_t* slot_to_row, int32_t* err, void* ws,
                          hipStream_t s);

hipError_t launch_prepare_weights(int L, int H, int F, int dtype, const void* w1, const void* w2,
                                  void* w1p, void* w2p, uint8_t* w1s, uint8_t* w2s, hipStream_t s);

hipError_t launch_grouped_mlp_f32(int L, int H, int F, int64_t capacity, const float* x,
                                  const int32_t* offsets, const float* w1p, const float* w2p,
                                  float* act, float* y, hipStream_t s);
size_t grouped_mlp_bf16_part_bytes();
hipError_t launch_grouped_mlp_bf16(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* w1p, const bf16_t* w2p,
                                   bf16_t* act, float* part, bf16_t* y, hipStream_t s);
hipError_t launch_grouped_mlp_bf16_backward(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                            const int32_t* offsets, const bf16_t* w1p, const bf16_t* w1t,
                                            const bf16_t* w2t, const bf16_t* dy, bf16_t* hbuf, bf16_t* dhbuf,
                                            float* part, bf16_t* dx, hipStream_t s);
hipError_t launch_grouped_mlp_mx_backward(int L, int H, int F, int64_t capacity, const bf16_t* x,
                                          const int32_t* offsets, const uint8_t* w1p, const uint8_t* w1s,
                                          const uint8_t* w1t, const uint8_t* w1ts, const uint8_t* w2t,
                                          const uint8_t* w2ts, const bf16_t* dy, uint8_t* xq, uint8_t* xqs,
                                          uint8_t* dyq, uint8_t* dyqs, bf16_t* hbuf, bf16_t* dhbuf, uint8_t* dhq,
                                          uint8_t* dhqs, float* da, float* part, bf16_t* dx, bool x_given,
                                          bool dy_given, hipStream_t s);
hipError_t launch_prepare_weights_backward(int L, int H, int F, int dtype, const void* w1, const void* w2,
                                           void* w1t, void* w2t, uint8_t* w1ts, uint8_t* w2ts, hipStream_t s);
hipError_t launch_mx_columns_grouped(int L, int64_t capacity, int C, int nbmax, const bf16_t* in,
                                     const int32_t* offsets, int32_t* pb, uint8_t* codes, uint8_t* scales,
                                     hipStream_t s);
hipError_t launch_wgrad_mx_layouts(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf,
                                   const bf16_t* dhbuf, int32_t* pk, int32_t* png, uint8_t* xa, uint8_t* xas,
                                   uint8_t* dhb, uint8_t* dhbs, uint8_t* aa, uint8_t* aas, uint8_t* dyb,
                                   uint8_t* dybs, float* dW1, float* dW2, hipStream_t s);
hipError_t launch_grouped_mlp_mx_wgrad(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                       const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf,
                                       const bf16_t* dhbuf, int32_t* pk, int32_t* png, uint8_t* xa, uint8_t* xas,
                                       uint8_t* dhb, uint8_t* dhbs, uint8_t* aa, uint8_t* aas, uint8_t* dyb,
                                       uint8_t* dybs, float* dW1, float* dW2, hipStream_t s);
hipError_t launch_wgrad_layouts(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf, const bf16_t* dhbuf,
                                int32_t* pb, bf16_t* xt, bf16_t* dht, bf16_t* at, bf16_t* dyt, float* dW1,
                                float* dW2, hipStream_t s);
hipError_t launch_grouped_mlp_bf16_wgrad(int L, int H, int F, int64_t capacity, int nbmax, const bf16_t* x,
                                         const int32_t* offsets, const bf16_t* dy, const bf16_t* hbuf,
                                         const bf16_t* dhbuf, int32_t* pb, bf16_t* xt, bf16_t* dht, bf16_t* at,
                                         bf16_t* dyt, float* dW1, float* dW2, hipStream_t s);
size_t grouped_mlp_mx_part_bytes();
hipError_t launch_grouped_mlp_mx(int L, int H, int F, int64_t capacity, bool fp4, const uint8_t* x,
                                 const uint8_t* xs, const int32_t* offsets, const uint8_t* w1p,
                                 const uint8_t* w1s, const uint8_t* w2p, const uint8_t* w2s,
                                 uint8_t* act, uint8_t* act_s, float* part, bf16_t* y, bf16_t* act_bf16,
                                 hipStream_t s);

hipError_t launch_combine(int T, int K, int H, int dtype, const void* y, const int32_t* s2r,
                          const float* probs, void* out, hipStream_t s);
hipError_t launch_combine_backward(int T, int K, int H, int dtype, const void* dout, const void* y,
                                   const int32_t* s2r, const float* probs, void* dy, float* dprobs, uint8_t* dyq,
                                   uint8_t* dyqs, hipStream_t s);
hipError_t launch_route_backward(int T, int E, int K, int score, float scale, const int16_t* ids,
                                 const float* probs, const float* dprobs, const float* logits,
                                 const float* score_bias, float* dz, hipStream_t s);

hipError_t launch_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* out, int* blocks, hipStream_t s);
hipError_t launch_calib_write(void* dst, size_t bytes, uint32_t v, hipStream_t s);
hipError_t launch_calib_mfma(int fp8, int blocks, int iters, float* out, hipStream_t s);

hipError_t launch_mx_quantize(int64_t rows, int cols, const bf16_t* in, const int32_t* row_limit,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);

}  // namespace moe
