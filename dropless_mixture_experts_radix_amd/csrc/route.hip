// Router: fused projection (x . W_r) and top-K selection with probabilities.
//
// Sparser-MoE page (harryzhou2000), "Preserve a compact route": selection
// by bounded histogram passes over a narrowed candidate range instead of K
// repeated full-row scans; the result is a compact int16 [T,K] id list;
// small top-K shapes keep a direct path.
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Experts per 32-row tile of the prepared router weights: P terms per expert.
static __host__ __device__ inline int router_terms(int w_dtype) { return w_dtype == MOE_F32 ? 3 : 1; }
static __host__ __device__ inline int router_ept(int P) { return 32 / P; }

RouteSplit route_split(int T, int E, int H, int x_dtype) {
  RouteSplit r;
  r.S = 1;
  r.Hc = H;
  r.C = 0;
  if (x_dtype != MOE_BF16) return r;
  const int ttiles = (T + 63) / 64;
  const int ctiles = (E + 31) / 32;  // the split depends on (T, E, H) only
  long waves = (long)ttiles * ctiles;
  // split H into S chunks (S a power of two, chunk a multiple of 64) until there
  // are enough wavefronts to cover the chip
  while (waves * r.S < 2048 && r.S < 16 && H % (r.S * 2 * 64) == 0) r.S *= 2;
  r.Hc = H / r.S;
  return r;
}

// ---------------------------------------------------------------------------
// Router weight preparation: W_r [H,E] -> bf16 [C][H] term rows (bf16 x) or a
// plain fp32 copy (fp32 x).  For fp32 W_r each weight w = hi + mid + lo with
// hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); both differences
// are exact in fp32.
// ---------------------------------------------------------------------------
__global__ void k_prepare_router_bf16(const void* __restrict__ w, int w_dtype, int H, int E, int C,
                                      bf16_t* __restrict__ out) {
  const int P = router_terms(w_dtype), ept = router_ept(P);
  const long total = (long)C * H;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const int row = (int)(i / H), h = (int)(i % H);
    const int tile = row / 32, r = row % 32, p = r / ept, el = r % ept;
    const int e = tile * ept + el;
    uint32_t v = 0;
    if (p < P && e < E) {
      if (w_dtype == MOE_BF16) {
        v = ((const bf16_t*)w)[(long)h * E + e];
      } else {
        float x = ((const float*)w)[(long)h * E + e];
        uint32_t hi = f32_to_bf16(x);
        float r1 = x - bf16_to_f32(hi);
        uint32_t mid = f32_to_bf16(r1);
        float r2 = r1 - bf16_to_f32(mid);
        uint32_t lo = f32_to_bf16(r2);
        v = p == 0 ? hi : (p == 1 ? mid : lo);
      }
    }
    out[i] = (bf16_t)v;
  }
}

__global__ void k_copy_f32(const float* __restrict__ in, float* __restrict__ out, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) out[i] = in[i];
}

hipError_t launch_prepare_router(const void* w, int w_dtype, int x_dtype, int H, int E, void* out,
                                 hipStream_t s) {
  if (x_dtype == MOE_BF16) {
    const int P = router_terms(w_dtype), ept = router_ept(P);
    const int C = ((E + ept - 1) / ept) * 32;
    const long total = (long)C * H;
    const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_prepare_router_bf16, dim3(blocks), dim3(256), 0, s, w, w_dtype, H, E, C,
                       (bf16_t*)out);
  } else {
    const long n = (long)H * E;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_copy_f32, dim3(blocks), dim3(256), 0, s, (const float*)w, (float*)out, n);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Projection, bf16 activations: partial[s][t][e] = sum over the s-th H chunk of
// x[t,h] * W_r[h,e], on bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation.  One wavefront computes 64 tokens x 32 prepared rows; each lane
// streams 64 contiguous bytes of a token row per 64-wide k step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_router_proj_bf16(int T, int E, int H, int Hc, int C, int S,
                                                          int P, const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wp,
                                                          float* __restrict__ partial) {
  __shared__ float s_tile[4][64][33];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int ctiles = C / 32, ttiles = (T + 63) / 64;
  const long task = (long)blockIdx.x * 4 + w;
  const int ct = (int)(task % ctiles);
  const int s = (int)((task / ctiles) % S);
  const int tt = (int)(task / ((long)ctiles * S));
  const bool active = tt < ttiles;
  const int g = l >> 5, r = l & 31;
  f32x16 acc0 = {}, acc1 = {};
  if (active) {
    const int t0 = tt * 64;
    int ra = t0 + r, rb = t0 + 32 + r;
    ra = ra < T ? ra : T - 1;
    rb = rb < T ? rb : T - 1;
    const bf16_t* pa = x + (long)ra * H + (long)s * Hc + 32 * g;
    const bf16_t* pb = x + (long)rb * H + (long)s * Hc + 32 * g;
    const bf16_t* pw = wp + (long)(ct * 32 + r) * H + (long)s * Hc + 32 * g;
    // unrolled so that the loads of several k steps are in flight together
#pragma unroll 4
    for (int k0 = 0; k0 < Hc; k0 += 64) {
      bf16x8 a0[4], a1[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0[j] = *(const bf16x8*)(pa + k0 + 8 * j);
        a1[j] = *(const bf16x8*)(pb + k0 + 8 * j);
        b[j] = *(const bf16x8*)(pw + k0 + 8 * j);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[j], b[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[j], b[j], acc1, 0, 0, 0);
      }
    }
    // D layout: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * g + (i & 3);
      s_tile[w][row][r] = acc0[i];
      s_tile[w][32 + row][r] = acc1[i];
    }
  }
  __syncthreads();
  if (!active) return;
  // sum the P terms of each expert column and store
  const int ept = router_ept(P);
  const int t0 = tt * 64;
  for (int idx = l; idx < 64 * ept; idx += 64) {
    const int row = idx / ept, el = idx % ept;
    const int e = ct * ept + el, t = t0 + row;
    if (e < E && t < T) {
      float v = 0.f;
      for (int p = 0; p < P; ++p) v += s_tile[w][row][p * ept + el];
      partial[((long)s * T + t) * E + e] = v;
    }
  }
}

// Projection, fp32 activations (small shapes): one thread per (token, expert),
// plain fp32 FMA in h order.
__global__ void k_router_proj_f32(int T, int E, int H, const float* __restrict__ x,
                                  const float* __restrict__ w, float* __restrict__ out) {
  const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (i >= (long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (long)t * H;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(xr[h], w[(long)h * E + e], acc);
  out[i] = acc;
}

hipError_t launch_router_proj(int T, int E, int H, int x_dtype, int w_dtype, const void* x,
                              const void* wp, float* partial, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (x_dtype == MOE_BF16) {
    const RouteSplit sp = route_split(T, E, H, MOE_BF16);
    const int P = router_terms(w_dtype), ept = router_ept(P);
    const int C = ((E + ept - 1) / ept) * 32;
    const long tasks = (long)((T + 63) / 64) * (C / 32) * sp.S;
    hipLaunchKernelGGL(k_router_proj_bf16, dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, s, T, E, H,
                       sp.Hc, C, sp.S, P, (const bf16_t*)x, (const bf16_t*)wp, partial);
  } else {
    const long n = (long)T * E;
    hipLaunchKernelGGL(k_router_proj_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, E, H,
                       (const float*)x, (const float*)wp, partial);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float score_of(float z, float zmax, int score) {
  return score == MOE_SCORE_SOFTMAX ? __expf(z - zmax) : 1.0f / (1.0f + __expf(-z));
}

// Small-E path (E <= 32): one thread per token, keys in registers, each key's
// output position is its rank (number of keys that beat it).
// Selection for one token of a small-E router (E <= EMAX <= 32): z holds the
// token's E logits.  Writes logits_out, applies the bias, and writes the K ids
// (descending key, lower index first on ties) and their probabilities; each
// key's output position is its rank (the number of keys that beat it).
template <int EMAX>
__device__ __forceinline__ void select_small_token(int t, int E, int K, int score, float (&z)[EMAX],
                                                   const float* __restrict__ bias,
                                                   const uint8_t* __restrict__ mask, int16_t* __restrict__ ids,
                                                   float* __restrict__ probs, float* __restrict__ logits_out,
                                                   int32_t* err) {
  uint32_t key[EMAX];
  bool bad = false;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    float v = z[e];
    if (e < E) {
      if (logits_out) logits_out[(long)t * E + e] = v;
      if (bias) v += bias[e];
    }
    key[e] = e < E ? float_key(v) : 0u;
    if (e < E && !key_finite(key[e])) bad = true;
  }
  if (bad) set_err(err, MOE_DEVERR_NONFINITE);
  if (mask && mask[t]) {
    for (int k = 0; k < K; ++k) { ids[(long)t * K + k] = -1; probs[(long)t * K + k] = 0.f; }
    return;
  }
  int rank[EMAX];
  float zmax = 0.f;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    int rk = 0;
#pragma unroll
    for (int j = 0; j < EMAX; ++j)
      rk += (j < E) && (key[j] > key[e] || (key[j] == key[e] && j < e));
    rank[e] = e < E ? rk : EMAX + 1;
    if (rank[e] == 0) zmax = key_float(key[e]);
  }
  float sum = 0.f;
  float sc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    sc[e] = 0.f;
    if (rank[e] < K) { sc[e] = score_of(key_float(key[e]), zmax, score); }
  }
  // sum in selection order (k = 0..K-1)
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) if (rank[e] == k) sum += sc[e];
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (rank[e] < K) {
      ids[(long)t * K + rank[e]] = (int16_t)e;
      probs[(long)t * K + rank[e]] = sc[e] * inv;
    }
  }
}

// Small-E path from logits or split-H partials (E <= 32): one thread per token.
template <int EMAX>
__global__ __launch_bounds__(64) void k_route_select_small(int T, int E, int K, int S, int score,
                                                            const float* __restrict__ partial,
                                                            const float* __restrict__ bias,
                                                            const uint8_t* __restrict__ mask,
                                                            int16_t* __restrict__ ids, float* __restrict__ probs,
                                                            float* __restrict__ logits_out, int32_t* err) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float z[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) z[e] = 0.f;
  // the S partial sets in order; a token's E logits of one set are contiguous
  if ((E & 3) == 0) {
    for (int s = 0; s < S; ++s) {
      const float4* ps = (const float4*)(partial + ((long)s * T + t) * E);
#pragma unroll
      for (int c = 0; c < EMAX / 4; ++c) {
        if (4 * c < E) {
          const float4 q = ps[c];
          z[4 * c] += q.x; z[4 * c + 1] += q.y; z[4 * c + 2] += q.z; z[4 * c + 3] += q.w;
        }
      }
    }
  } else {
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < E) z[e] += partial[((long)s * T + t) * E + e];
    }
  }
  select_small_token<EMAX>(t, E, K, score, z, bias, mask, ids, probs, logits_out, err);
}

// Fused projection + selection for a small router (bf16 x, all P*E prepared
// rows in one 32-row tile): a workgroup of 8 wavefronts takes 16 tokens; each
// wavefront computes the 16 x 32 logit tile over its eighth of H on
// v_mfma_f32_16x16x32_bf16 (two 16-column tiles); the eight partial tiles are
// summed in LDS in wavefront order, the P terms of each expert in term order,
// and one thread per token selects.  No partial logits go through HBM.  With
// the 16-row instruction four lanes share a token row, so one 16-byte-per-lane
// load covers 64 contiguous bytes of each of 16 rows.
template <int EMAX>
__global__ __launch_bounds__(512) void k_route_fused_small(int T, int E, int K, int H, int P, int score,
                                                           const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ wp,
                                                           const float* __restrict__ bias,
                                                           const uint8_t* __restrict__ mask,
                                                           int16_t* __restrict__ ids, float* __restrict__ probs,
                                                           float* __restrict__ logits_out, int32_t* err) {
  __shared__ float s_part[8][16][33];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, q = l >> 4, r = l & 15;
  const int t0 = blockIdx.x * 16;
  const int ra = min(t0 + r, T - 1);
  // 32-wide k slices of this wavefront: [k0s, k1s)
  const int nks = H / 32, per = (nks + 7) / 8;
  const int k0s = min(w * per, nks), k1s = min(k0s + per, nks);
  // lane (q, r): token row r (A) or prepared rows r and 16 + r (B), k = 8q..8q+7 of a slice
  const bf16_t* pa = x + (long)ra * H + 8 * q;
  const bf16_t* pw0 = wp + (long)r * H + 8 * q;
  const bf16_t* pw1 = wp + (long)(16 + r) * H + 8 * q;
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  f32x4v acc[2][2] = {};  // [slice parity][column tile]
  int ks = k0s;
  // eight slices at a time; the fence keeps all their loads ahead of the MFMAs
  for (; ks + 8 <= k1s; ks += 8) {
    bf16x8 a[8], b0[8], b1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = *(const bf16x8*)(pa + (ks + u) * 32);
      b0[u] = *(const bf16x8*)(pw0 + (ks + u) * 32);
      b1[u] = *(const bf16x8*)(pw1 + (ks + u) * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc[u & 1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc[u & 1][0], 0, 0, 0);
      acc[u & 1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc[u & 1][1], 0, 0, 0);
    }
  }
  for (; ks < k1s; ++ks) {
    const bf16x8 a = *(const bf16x8*)(pa + ks * 32);
    const bf16x8 b0 = *(const bf16x8*)(pw0 + ks * 32);
    const bf16x8 b1 = *(const bf16x8*)(pw1 + ks * 32);
    acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[0][1], 0, 0, 0);
  }
  // D layout: lane l holds column l%16, rows 4*(l/16) + i
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const f32x4v v = acc[0][c] + acc[1][c];
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[w][4 * q + i][16 * c + r] = v[i];
  }
  __syncthreads();
  // sum the eight partial tiles in wavefront order (one value per thread)
  {
    const int row = threadIdx.x >> 5, col = threadIdx.x & 31;
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) v += s_part[u][row][col];
    __syncthreads();
    s_part[0][row][col] = v;
  }
  __syncthreads();
  const int t = t0 + threadIdx.x;
  if (threadIdx.x >= 16 || t >= T) return;
  const int ept = router_ept(P);
  float z[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    float v = 0.f;
    if (e < E)
      for (int p = 0; p < P; ++p) v += s_part[0][threadIdx.x][p * ept + e];
    z[e] = v;
  }
  select_small_token<EMAX>(t, E, K, score, z, bias, mask, ids, probs, logits_out, err);
}

bool route_fused_ok(int E, int H, int x_dtype, int w_dtype) {
  const int P = router_terms(w_dtype), ept = router_ept(P);
  return x_dtype == MOE_BF16 && E <= ept && E <= 32 && H % 32 == 0;
}

hipError_t launch_route_fused(int T, int E, int K, int H, int score, int w_dtype, const void* x, const void* wp,
                              const float* bias, const uint8_t* mask, int16_t* ids, float* probs,
                              float* logits_out, int32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int P = router_terms(w_dtype);
  const dim3 g((T + 15) / 16), b(512);
  if (E <= 8)
    hipLaunchKernelGGL(k_route_fused_small<8>, g, b, 0, s, T, E, K, H, P, score, (const bf16_t*)x,
                       (const bf16_t*)wp, bias, mask, ids, probs, logits_out, err);
  else if (E <= 16)
    hipLaunchKernelGGL(k_route_fused_small<16>, g, b, 0, s, T, E, K, H, P, score, (const bf16_t*)x,
                       (const bf16_t*)wp, bias, mask, ids, probs, logits_out, err);
  else
    hipLaunchKernelGGL(k_route_fused_small<32>, g, b, 0, s, T, E, K, H, P, score, (const bf16_t*)x,
                       (const bf16_t*)wp, bias, mask, ids, probs, logits_out, err);
  return hipGetLastError();
}

// Large-E path: one wavefront per token, VPL keys per lane (element index of
// key j of lane l: (j/4)*256 + 4*l + j%4, so keys are read with 16-byte loads).
//  1. Candidate bound: lb = K-th largest of the 64 per-lane maxima; at least K
//     keys are >= lb, so the K selected keys all satisfy key >= lb.
//  2. If at most CMAX keys are >= lb, they are gathered (in index order) and
//     ranked directly.
//  3. Otherwise radix threshold select: 4 histogram passes over 8-bit digits
//     (most significant first, 256 LDS bins per wave) narrow the candidates to
//     the K-th key tau; the keys > tau and the first keys == tau in index order
//     are gathered and ranked.
#define SEL_CMAX 256
template <int VPL>
__global__ __launch_bounds__(256) void k_route_select_wave(int T, int E, int K, int S, int score,
                                                           const float* __restrict__ partial,
                                                           const float* __restrict__ bias,
                                                           const uint8_t* __restrict__ mask,
                                                           int16_t* __restrict__ ids, float* __restrict__ probs,
                                                           float* __restrict__ logits_out, int32_t* err) {
  __shared__ uint32_t s_hist[4][256];
  __shared__ uint32_t s_ckey[4][SEL_CMAX];
  __shared__ int s_cidx[4][SEL_CMAX];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;  // wave-uniform; no block-wide barrier below
  constexpr int NC = VPL / 4;
  uint32_t key[VPL];
  bool bad = false;
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e0 = c * 256 + 4 * l;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (vec && e0 < E) {
      for (int s = 0; s < S; ++s) {
        const float4 q = *(const float4*)(partial + ((long)s * T + t) * E + e0);
        v[0] += q.x; v[1] += q.y; v[2] += q.z; v[3] += q.w;
      }
    } else if (!vec) {
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e0 + q < E) v[q] += partial[((long)s * T + t) * E + e0 + q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + q;
      if (e < E) {
        if (logits_out) logits_out[(long)t * E + e] = v[q];
        float zz = bias ? v[q] + bias[e] : v[q];
        key[c * 4 + q] = float_key(zz);
        if (!key_finite(key[c * 4 + q])) bad = true;
      } else {
        key[c * 4 + q] = 0u;
      }
    }
  }
  if (wave_ballot(bad) != 0 && l == 0) set_err(err, MOE_DEVERR_NONFINITE);
  if (mask && mask[t]) {
    if (l < K) { ids[(long)t * K + l] = -1; probs[(long)t * K + l] = 0.f; }
    return;
  }
  auto valid = [&](int j) { return ((j >> 2) * 256 + 4 * l + (j & 3)) < E; };

  // 1. bound from the per-lane maxima (bitonic sort of 64 values, descending)
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) m = (valid(j) && key[j] > m) ? key[j] : m;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, j, 64);
      const bool asc = (l & k) == 0, lower = (l & j) == 0;
      m = (asc == lower) ? (m > o ? m : o) : (m < o ? m : o);
    }
  }
  const uint32_t lb = (uint32_t)readlane_i((int)m, K - 1);
  int mine = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) mine += (valid(j) && key[j] >= lb);
  const int ncand = wave_sum_i(mine);

  uint32_t tau;
  int need_eq;  // keys == tau taken (first ones in index order); keys > tau always taken
  bool direct = ncand <= SEL_CMAX;
  if (direct) {
    tau = lb;  // gather every key >= lb
    need_eq = 1 << 30;
  } else {
    // 3. radix threshold select
    uint32_t prefix = 0, pmask = 0;
    int krem = K;
    for (int d = 3; d >= 0; --d) {
      const int sh = 8 * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) s_hist[w][4 * l + i] = 0;
      wave_sync();
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (valid(j) && (key[j] & pmask) == prefix) atomicAdd(&s_hist[w][(key[j] >> sh) & 255u], 1u);
      wave_sync();
      // lane l owns bins 255-4l, 254-4l, 253-4l, 252-4l (descending)
      int c4[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c4[i] = (int)s_hist[w][255 - 4 * l - i]; tot += c4[i]; }
      const int incl = wave_incl_scan(tot);
      int run = incl - tot, hit_bin = -1, hit_above = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (hit_bin < 0 && run < krem && run + c4[i] >= krem) { hit_bin = 255 - 4 * l - i; hit_above = run; }
        run += c4[i];
      }
      const uint64_t hb = wave_ballot(hit_bin >= 0);
      if (hb == 0) break;  // cannot happen: the candidates always hold >= krem keys
      const int src = __builtin_ctzll(hb);
      const int bin = readlane_i(hit_bin, src);
      const int above = readlane_i(hit_above, src);
      krem -= above;
      prefix |= (uint32_t)bin << sh;
      pmask |= 0xffu << sh;
      wave_sync();
    }
    tau = prefix;
    need_eq = krem;
  }

  // gather: keys > tau (all, in index order), then keys == tau (all of them on
  // the direct path; the first need_eq in index order on the radix path)
  int cgt = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) cgt += valid(j) && key[j] > tau;
  const int ngt_tot = wave_sum_i(cgt);
  int base = 0, eqbase = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int ngt = 0, neq = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = c * 4 + q;
      const bool v = valid(j);
      ngt += v && key[j] > tau;
      neq += v && key[j] == tau;
    }
    const int igt = wave_incl_scan(ngt), ieq = wave_incl_scan(neq);
    int pg = base + igt - ngt, pe = eqbase + ieq - neq;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = c * 4 + q;
      const int e = c * 256 + 4 * l + q;
      if (!valid(j)) continue;
      if (key[j] > tau) {
        const int pos = pg++;
        if (pos < SEL_CMAX) { s_ckey[w][pos] = key[j]; s_cidx[w][pos] = e; }
      } else if (key[j] == tau) {
        const int er = pe++;
        const int pos = ngt_tot + er;
        if (er < need_eq && pos < SEL_CMAX) { s_ckey[w][pos] = key[j]; s_cidx[w][pos] = e; }
      }
    }
    base += readlane_i(igt, 63);
    eqbase += readlane_i(ieq, 63);
  }
  wave_sync();
  int ncan = ngt_tot + (eqbase < need_eq ? eqbase : need_eq);
  ncan = ncan < SEL_CMAX ? ncan : SEL_CMAX;

  // rank every candidate; ranks < K are the output positions
  uint32_t selkey = 0;
  int selidx = -1;
  for (int i = l; i < ncan; i += 64) {
    const uint32_t ki = s_ckey[w][i];
    const int ii = s_cidx[w][i];
    int rk = 0;
    for (int j = 0; j < ncan; ++j) {
      const uint32_t kj = s_ckey[w][j];
      const int ij = s_cidx[w][j];
      rk += (kj > ki) || (kj == ki && ij < ii);
    }
    if (rk < K) {
      // stash by rank in the histogram area (free now)
      s_hist[w][rk] = ki;
      s_hist[w][128 + rk] = (uint32_t)ii;
    }
  }
  wave_sync();
  if (l < K) {
    selkey = s_hist[w][l];
    selidx = (int)s_hist[w][128 + l];
  }
  const float zmax = key_float(s_hist[w][0]);
  const float sc = l < K ? score_of(key_float(selkey), zmax, score) : 0.f;
  const float sum = wave_sum_f(sc);
  if (l < K) {
    ids[(long)t * K + l] = (int16_t)selidx;
    probs[(long)t * K + l] = sc / sum;
  }
}

hipError_t launch_route_select(int T, int E, int K, int S, int score, const float* partial,
                               const float* bias, const uint8_t* mask, int16_t* ids, float* probs,
                               float* logits_out, int32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 32) {
    const dim3 g((T + 63) / 64), b(64);  // one thread per token, many small workgroups
    if (E <= 8)
      hipLaunchKernelGGL(k_route_select_small<8>, g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err);
    else if (E <= 16)
      hipLaunchKernelGGL(k_route_select_small<16>, g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err);
    else
      hipLaunchKernelGGL(k_route_select_small<32>, g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err);
  } else {
    const dim3 g((T + 3) / 4), b(256);
    if (E <= 256)
      hipLaunchKernelGGL(k_route_select_wave<4>, g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err);
    else if (E <= 1024)
      hipLaunchKernelGGL(k_route_select_wave<16>, g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err);
    else
      hipLaunchKernelGGL(k_route_select_wave<64>, g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err);
  }
  return hipGetLastError();
}

}  // namespace moe
