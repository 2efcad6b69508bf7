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
  r.Sg = 0;
  if (x_dtype != MOE_BF16) return r;
  // bf16 weights and at least 128 experts: the projection is one dense GEMM on
  // the grouped GEMM's matrix-core pipeline (256 x 256 tiles, pieces along H)
  if (E >= 128 && H % 128 == 0) r.Sg = router_gemm_pieces(T, E, H);
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
// are exact in fp32.  A single 32-row tile (C = 32, H % 32 == 0: the fused
// small-router path) is stored k-blocked, [H/32][32 rows][32], so that the 16
// rows x 32 k of one MFMA operand load are one contiguous KiB.
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
    const long o = (C == 32 && H % 32 == 0) ? ((long)(h >> 5) * 32 + row) * 32 + (h & 31) : i;
    out[o] = (bf16_t)v;
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
  // the S partial sets in order, four sets' loads in flight at a time; a
  // token's E logits of one set are contiguous
  if ((E & 3) == 0) {
    for (int s0 = 0; s0 < S; s0 += 4) {
      float4 q[4][EMAX / 4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < EMAX / 4; ++c)
          q[j][c] = (s0 + j < S && 4 * c < E) ? ((const float4*)(partial + ((long)(s0 + j) * T + t) * E))[c]
                                              : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < EMAX / 4; ++c) {
          if (s0 + j < S && 4 * c < E) {
            z[4 * c] += q[j][c].x; z[4 * c + 1] += q[j][c].y; z[4 * c + 2] += q[j][c].z; z[4 * c + 3] += q[j][c].w;
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
// rows in one 32-row tile): a workgroup of RF_WAVES wavefronts takes 16
// tokens; each wavefront computes the 16 x 32 logit tile over its share of H
// on v_mfma_f32_16x16x32_bf16 (two 16-column tiles); the partial tiles are
// summed in LDS in wavefront order, the P terms of each expert in term order,
// and one thread per token selects.  No partial logits go through HBM.  With
// the 16-row instruction four lanes share a token row, so one 16-byte-per-lane
// load covers 64 contiguous bytes of each of 16 rows.  The prepared rows past
// the last term row in use ((P-1)*ept + E) are zero and are not read.
#define RF_WAVES 16
template <int EMAX>
__global__ __launch_bounds__(64 * RF_WAVES) void k_route_fused_small(int T, int E, int K, int H, int P, int score,
                                                           const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ wp,
                                                           const float* __restrict__ bias,
                                                           const uint8_t* __restrict__ mask,
                                                           int16_t* __restrict__ ids, float* __restrict__ probs,
                                                           float* __restrict__ logits_out, int32_t* err) {
  __shared__ float s_part[RF_WAVES][16][33];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, q = l >> 4, r = l & 15;
  const int t0 = blockIdx.x * 16;
  const int ra = min(t0 + r, T - 1);
  const int PE = (P - 1) * router_ept(P) + E;  // prepared rows in use: term p of expert e is row p * ept + e
  // 32-wide k slices of this wavefront: [k0s, k1s)
  const int nks = H / 32, per = (nks + RF_WAVES - 1) / RF_WAVES;
  const int k0s = min(w * per, nks), k1s = min(k0s + per, nks);
  // lane (q, r): token row r (A) or prepared rows r and 16 + r (B), k = 8q..8q+7 of a slice
  const bf16_t* pa = x + (long)ra * H + 8 * q;
  // prepared rows k-blocked [H/32][32][32]: slice ks of row r at (ks*32 + r)*32
  const bf16_t* pw0 = wp + r * 32 + 8 * q;
  const bf16_t* pw1 = wp + (16 + r) * 32 + 8 * q;
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  f32x4v acc[2][2] = {};  // [slice parity][column tile]
  int ks = k0s;
  // eight slices at a time; the fence keeps all their loads ahead of the MFMAs
  for (; ks + 8 <= k1s; ks += 8) {
    bf16x8 a[8], b0[8], b1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = *(const bf16x8*)(pa + (ks + u) * 32);
      b0[u] = r < PE ? *(const bf16x8*)(pw0 + (ks + u) * 1024) : bf16x8{};
      b1[u] = 16 + r < PE ? *(const bf16x8*)(pw1 + (ks + u) * 1024) : bf16x8{};
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
    const bf16x8 b0 = r < PE ? *(const bf16x8*)(pw0 + ks * 1024) : bf16x8{};
    const bf16x8 b1 = 16 + r < PE ? *(const bf16x8*)(pw1 + ks * 1024) : bf16x8{};
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
  // sum the partial tiles in wavefront order (one value per thread)
  {
    const int row = (threadIdx.x >> 5) & 15, col = threadIdx.x & 31;
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < RF_WAVES; ++u) v += s_part[u][row][col];
    __syncthreads();
    if (threadIdx.x < 512) s_part[0][row][col] = v;
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
  const dim3 g((T + 15) / 16), b(64 * RF_WAVES);
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
// key j of lane l: (j/4)*256 + 4*l + j%4, so keys are read with 16-byte loads;
// slots past E hold key 0, below every real key).
//  1. Candidate bound: lb = K-th largest of the 128 keys formed by the two
//     largest keys of every lane.  They are keys of distinct elements, so at
//     least K keys are >= lb and the K selected keys all satisfy key >= lb.
//  2. If at most CMAX keys are >= lb, they are the candidates.
//  3. Otherwise (many equal keys) radix threshold select over the keys >= lb:
//     4 histogram passes over 8-bit digits (most significant first, 256 LDS
//     bins per wave) find the K-th key tau; the keys > tau and the first keys
//     == tau in index order are the candidates (exactly K).
//  4. The candidates are sorted by a wavefront bitonic network of 64 or 128
//     slots (key descending, lower index first); the first K are the output.
// For K <= 64 the bound of step 1 leaves at most a few dozen keys beyond K on
// continuous logits; step 3 is for logits with many equal values.
#define SEL_CMAX 128

// a before b: larger key, or equal key and lower index
__device__ __forceinline__ bool sel_better(uint32_t ka, int ia, uint32_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Bitonic sort of the 64*SL slots of one wavefront (slot p = SL*lane + s) into
// "better first" order; with IDX false the keys alone are sorted, descending.
template <int SL, bool IDX>
__device__ __forceinline__ void wave_bitonic(uint32_t (&k)[SL], int (&ix)[SL], int l) {
  auto better = [](uint32_t ka, int ia, uint32_t kb, int ib) {
    return IDX ? sel_better(ka, ia, kb, ib) : ka > kb;
  };
#pragma unroll
  for (int kk = 2; kk <= 64 * SL; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j < SL) {
#pragma unroll
        for (int a = 0; a < SL; ++a) {
          const int b = a ^ j;
          if (b <= a) continue;
          const bool desc = ((SL * l + a) & kk) == 0;  // a is the lower slot of the pair
          if (desc == better(k[b], ix[b], k[a], ix[a])) {
            const uint32_t tk = k[a]; k[a] = k[b]; k[b] = tk;
            if (IDX) { const int ti = ix[a]; ix[a] = ix[b]; ix[b] = ti; }
          }
        }
      } else {
        const int lx = j / SL;
#pragma unroll
        for (int a = 0; a < SL; ++a) {
          const uint32_t ok = (uint32_t)__shfl_xor((int)k[a], lx, 64);
          const int oi = IDX ? __shfl_xor(ix[a], lx, 64) : 0;
          const int p = SL * l + a;
          const bool lower = (p & j) == 0, desc = (p & kk) == 0;
          if ((lower == desc) != better(k[a], ix[a], ok, oi)) {
            k[a] = ok;
            if (IDX) ix[a] = oi;
          }
        }
      }
    }
  }
}

// sorts the ncan candidates of one wavefront in LDS and leaves the first K
// (key, index) in lanes 0..K-1 of (selkey, selidx)
template <int SL>
__device__ __forceinline__ void sel_sort_take(const uint32_t* ck, const int* ci, int ncan, int l,
                                              uint32_t& selkey, int& selidx) {
  uint32_t k[SL];
  int ix[SL];
#pragma unroll
  for (int a = 0; a < SL; ++a) {
    const int p = SL * l + a;
    k[a] = p < ncan ? ck[p] : 0u;  // empty slots sort last
    ix[a] = p < ncan ? ci[p] : 0x7fffffff;
  }
  wave_bitonic<SL, true>(k, ix, l);
  // element q of the sorted order is slot q % SL of lane q / SL
#pragma unroll
  for (int a = 0; a < SL; ++a) {
    const uint32_t vk = (uint32_t)__shfl((int)k[a], l / SL, 64);
    const int vi = __shfl(ix[a], l / SL, 64);
    if (l % SL == a) { selkey = vk; selidx = vi; }
  }
}

// GRP: group-limited routing with a selection-only bias (DeepSeek-V3
// Technical Report, section "DeepSeekMoE with Auxiliary-Loss-Free Load
// Balancing"): the keys are s + bias with s = sigmoid(logit) in fp32; before
// step 1 the keys of experts outside the topk_group best groups are set to 0
// (below every real key).  A group's score is the fp32 sum of its m largest
// keys, largest first; lane g scores group g from the keys in LDS, and every
// lane ranks its group against all others (ties: lower group index).  The
// gates are scale * s_k / sum_j s_j over the selected, s from LDS.
template <int VPL, bool GRP>
__global__ __launch_bounds__(256) void k_route_select_wave(int T, int E, int K, int S, int score,
                                                           const float* __restrict__ partial,
                                                           const float* __restrict__ bias,
                                                           const uint8_t* __restrict__ mask,
                                                           int16_t* __restrict__ ids, float* __restrict__ probs,
                                                           float* __restrict__ logits_out, int32_t* err,
                                                           RouteGroups grp, float* __restrict__ scores_out) {
  __shared__ uint32_t s_hist[4][256];
  __shared__ uint32_t s_ckey[4][SEL_CMAX];
  __shared__ int s_cidx[4][SEL_CMAX];
  constexpr int GE = GRP ? ROUTE_GRP_MAX_E : 1;
  __shared__ uint32_t s_gkey[4][GE];  // GRP: keys by expert
  __shared__ float s_sig[4][GE];      // GRP: sigmoid scores by expert
  __shared__ float s_gsc[4][GRP ? 64 : 1];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;  // wave-uniform; no block-wide barrier below
  constexpr int NC = VPL / 4;
  // logits (+ bias): every chunk's loads are issued before any is used
  float4 v[NC];
  const bool vec = (E & 3) == 0;
  if (vec) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = c * 256 + 4 * l;
      v[c] = e0 < E ? *(const float4*)(partial + (long)t * E + e0) : float4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s = 1; s < S; ++s)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int e0 = c * 256 + 4 * l;
        if (e0 < E) {
          const float4 q = *(const float4*)(partial + ((long)s * T + t) * E + e0);
          v[c].x += q.x; v[c].y += q.y; v[c].z += q.z; v[c].w += q.w;
        }
      }
  } else {  // rows not 16-byte aligned
#pragma unroll
    for (int c = 0; c < NC; ++c) v[c] = float4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int e0 = c * 256 + 4 * l;
        const float* r = partial + ((long)s * T + t) * E + e0;
        if (e0 < E) v[c].x += r[0];
        if (e0 + 1 < E) v[c].y += r[1];
        if (e0 + 2 < E) v[c].z += r[2];
        if (e0 + 3 < E) v[c].w += r[3];
      }
  }
  if (logits_out) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = c * 256 + 4 * l;
      float* o = logits_out + (long)t * E + e0;
      if (vec && e0 < E) {
        *(float4*)o = v[c];
      } else if (!vec) {
        if (e0 < E) o[0] = v[c].x;
        if (e0 + 1 < E) o[1] = v[c].y;
        if (e0 + 2 < E) o[2] = v[c].z;
        if (e0 + 3 < E) o[3] = v[c].w;
      }
    }
  }
  bool nfl = false;  // GRP: a non-finite logit (its sigmoid would be finite)
  if constexpr (GRP) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float zz[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = c * 256 + 4 * l + q;
        nfl |= e < E && (__float_as_uint(zz[q]) << 1) >= 0xff000000u;
        zz[q] = 1.0f / (1.0f + expf(-zz[q]));
        if (e < E) {
          s_sig[w][e] = zz[q];
          if (scores_out) scores_out[(long)t * E + e] = zz[q];
        }
      }
      v[c] = float4{zz[0], zz[1], zz[2], zz[3]};
    }
  }
  if (bias) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = c * 256 + 4 * l;
      float4 b = float4{0.f, 0.f, 0.f, 0.f};
      if (vec && e0 < E) {
        b = *(const float4*)(bias + e0);
      } else if (!vec) {
        if (e0 < E) b.x = bias[e0];
        if (e0 + 1 < E) b.y = bias[e0 + 1];
        if (e0 + 2 < E) b.z = bias[e0 + 2];
        if (e0 + 3 < E) b.w = bias[e0 + 3];
      }
      v[c].x += b.x; v[c].y += b.y; v[c].z += b.z; v[c].w += b.w;
    }
  }
  // order-preserving keys (-0 taken as +0); slots past E get 0
  uint32_t key[VPL];
  uint32_t emax = 0;  // largest (bits << 1): >= 0xff000000 for inf and NaN
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float z[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t u = __float_as_uint(z[q] + 0.0f);
      const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      const bool in = c * 256 + 4 * l + q < E;
      emax = max(emax, in ? u << 1 : 0u);
      key[c * 4 + q] = in ? k : 0u;
    }
  }
  const bool bad = emax >= 0xff000000u || nfl;
  if (wave_ballot(bad) != 0 && l == 0) set_err(err, MOE_DEVERR_NONFINITE);
  if (mask && mask[t]) {
    if (l < K) { ids[(long)t * K + l] = -1; probs[(long)t * K + l] = 0.f; }
    return;
  }
  if constexpr (GRP) {
    const int gs = E / grp.n_group;
    float gsc = 0.f;
    if (grp.m <= 2 && (gs & 3) == 0 && gs <= 256 && ((gs >> 2) & ((gs >> 2) - 1)) == 0) {
      // a group is gs/4 aligned lanes of one 256-expert chunk: the top two of
      // each lane's 4 keys, merged across the group's lanes by xor shuffles
      const int lanes = gs >> 2;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t a0 = 0u, a1 = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = key[c * 4 + q];
          a1 = max(a1, min(a0, x));
          a0 = max(a0, x);
        }
        for (int o = 1; o < lanes; o <<= 1) {
          const uint32_t b0 = (uint32_t)__shfl_xor((int)a0, o, 64), b1 = (uint32_t)__shfl_xor((int)a1, o, 64);
          const uint32_t n1 = max(min(a0, b0), max(a1, b1));
          a0 = max(a0, b0);
          a1 = n1;
        }
        const int e = c * 256 + 4 * l;
        if ((l & (lanes - 1)) == 0 && e < E)
          s_gsc[w][e / gs] = grp.m == 2 ? key_float(a0) + key_float(a1) : key_float(a0);
      }
      wave_sync();
      if (l < grp.n_group) gsc = s_gsc[w][l];
    } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = (j >> 2) * 256 + 4 * l + (j & 3);
      if (e < E) s_gkey[w][e] = key[j];
    }
    wave_sync();
    // lane g: the m largest keys of group g, descending, then their fp32 sum
    if (l < grp.n_group) {
      uint32_t tk[ROUTE_GRP_MAX_M];
#pragma unroll
      for (int i = 0; i < ROUTE_GRP_MAX_M; ++i) tk[i] = 0u;
      for (int e = l * gs; e < (l + 1) * gs; ++e) {
        uint32_t x = s_gkey[w][e];
#pragma unroll
        for (int i = 0; i < ROUTE_GRP_MAX_M; ++i) {  // insert, keeping tk descending
          if (i < grp.m && x > tk[i]) { const uint32_t y = tk[i]; tk[i] = x; x = y; }
        }
      }
      gsc = key_float(tk[0]);
#pragma unroll
      for (int i = 1; i < ROUTE_GRP_MAX_M; ++i)
        if (i < grp.m) gsc += key_float(tk[i]);
      s_gsc[w][l] = gsc;
    }
    wave_sync();
    }
    int rank = 0;
    for (int h = 0; h < grp.n_group; ++h) {
      const float o = s_gsc[w][h];
      rank += (o > gsc) || (o == gsc && h < l);
    }
    const uint64_t kept = wave_ballot(l < grp.n_group && rank < grp.topk_group);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = (j >> 2) * 256 + 4 * l + (j & 3);
      if (e < E && !((kept >> (e / gs)) & 1)) key[j] = 0u;
    }
  }

  // 1. bound: the K-th largest of the lanes' top-two keys (K <= 64 < 128)
  uint32_t top[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    top[1] = max(top[1], min(top[0], key[j]));
    top[0] = max(top[0], key[j]);
  }
  {
    int dummy[2] = {0, 0};
    wave_bitonic<2, false>(top, dummy, l);
  }
  const uint32_t lbs = (uint32_t)readlane_i((int)top[(K - 1) & 1], (K - 1) >> 1);
  const uint32_t lb = lbs > 1u ? lbs : 1u;  // at least K real keys are >= 1
  // 2. every key >= lb (if they are few), appended in (slot, lane) order: the
  // sort breaks ties by index, so the order is free
  int ncand = 0;  // wave-uniform
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool c = key[j] >= lb;
    const uint64_t b = wave_ballot(c);
    if (b != 0) {
      const int pos = ncand + mask_rank(b);
      if (c && pos < SEL_CMAX) {
        s_ckey[w][pos] = key[j];
        s_cidx[w][pos] = (j >> 2) * 256 + 4 * l + (j & 3);
      }
      ncand += __popcll(b);
    }
  }
  int ncan;
  if (ncand <= SEL_CMAX) {
    ncan = ncand;
  } else {
    // 3. radix threshold select over the keys >= lb
    uint32_t prefix = 0, pmask = 0;
    int krem = K;
    for (int d = 3; d >= 0; --d) {
      const int sh = 8 * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) s_hist[w][4 * l + i] = 0;
      wave_sync();
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (key[j] >= lb && (key[j] & pmask) == prefix) atomicAdd(&s_hist[w][(key[j] >> sh) & 255u], 1u);
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
      if (hb == 0) break;  // cannot happen: the keys >= lb always number >= krem
      const int src = __builtin_ctzll(hb);
      const int bin = readlane_i(hit_bin, src);
      const int above = readlane_i(hit_above, src);
      krem -= above;
      prefix |= (uint32_t)bin << sh;
      pmask |= 0xffu << sh;
      wave_sync();
    }
    const uint32_t tau = prefix;  // the K-th largest key; >= lb >= 1
    const int need_eq = krem;     // keys == tau taken, first in index order
    const int ngt = K - krem;     // keys > tau, at [0, ngt); then the keys == tau
    int base = 0, eqbase = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      int ng = 0, neq = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ng += key[c * 4 + q] > tau;
        neq += key[c * 4 + q] == tau;
      }
      const int ig = wave_incl_scan(ng), ieq = wave_incl_scan(neq);
      int pg = base + ig - ng, pe = eqbase + ieq - neq;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t kq = key[c * 4 + q];
        const int e = c * 256 + 4 * l + q;
        if (kq > tau) {
          const int at = pg++;
          if (at < SEL_CMAX) { s_ckey[w][at] = kq; s_cidx[w][at] = e; }
        } else if (kq == tau) {
          const int er = pe++;
          if (er < need_eq && ngt + er < SEL_CMAX) { s_ckey[w][ngt + er] = kq; s_cidx[w][ngt + er] = e; }
        }
      }
      base += readlane_i(ig, 63);
      eqbase += readlane_i(ieq, 63);
    }
    ncan = ngt + (eqbase < need_eq ? eqbase : need_eq);
    ncan = ncan < SEL_CMAX ? ncan : SEL_CMAX;
  }
  wave_sync();

  // 4. sort the candidates (at least K of them); lanes 0..K-1 take the first K
  uint32_t selkey = 0;
  int selidx = -1;
  if (ncan <= 64)
    sel_sort_take<1>(s_ckey[w], s_cidx[w], ncan, l, selkey, selidx);
  else
    sel_sort_take<2>(s_ckey[w], s_cidx[w], ncan, l, selkey, selidx);
  if constexpr (GRP) {
    const float sc = l < K ? s_sig[w][selidx] : 0.f;
    const float sum = wave_sum_f(sc);
    if (l < K) {
      ids[(long)t * K + l] = (int16_t)selidx;
      probs[(long)t * K + l] = grp.scale * (sc / sum);
    }
  } else {
    const float zmax = key_float((uint32_t)readlane_i((int)selkey, 0));
    const float sc = l < K ? score_of(key_float(selkey), zmax, score) : 0.f;
    const float sum = wave_sum_f(sc);
    if (l < K) {
      ids[(long)t * K + l] = (int16_t)selidx;
      probs[(long)t * K + l] = sc / sum;
    }
  }
}

hipError_t launch_route_select(int T, int E, int K, int S, int score, const float* partial,
                               const float* bias, const uint8_t* mask, int16_t* ids, float* probs,
                               float* logits_out, int32_t* err, hipStream_t s, const RouteGroups* grp,
                               float* scores_out) {
  if (T == 0) return hipSuccess;
  const RouteGroups g0 = grp ? *grp : RouteGroups{1, 1, 1, 1.f};
  if (grp) {  // 32 < E <= ROUTE_GRP_MAX_E, checked by the caller
    const dim3 g((T + 3) / 4), b(256);
    if (E <= 256)
      hipLaunchKernelGGL((k_route_select_wave<4, true>), g, b, 0, s, T, E, K, S, score, partial, bias, mask, ids,
                         probs, logits_out, err, g0, scores_out);
    else
      hipLaunchKernelGGL((k_route_select_wave<16, true>), g, b, 0, s, T, E, K, S, score, partial, bias, mask,
                         ids, probs, logits_out, err, g0, scores_out);
    return hipGetLastError();
  }
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
      hipLaunchKernelGGL((k_route_select_wave<4, false>), g, b, 0, s, T, E, K, S, score, partial, bias, mask,
                         ids, probs, logits_out, err, g0, nullptr);
    else if (E <= 1024)
      hipLaunchKernelGGL((k_route_select_wave<16, false>), g, b, 0, s, T, E, K, S, score, partial, bias, mask,
                         ids, probs, logits_out, err, g0, nullptr);
    else if (E <= 2304)
      hipLaunchKernelGGL((k_route_select_wave<36, false>), g, b, 0, s, T, E, K, S, score, partial, bias, mask,
                         ids, probs, logits_out, err, g0, nullptr);
    else if (E <= 2560)
      hipLaunchKernelGGL((k_route_select_wave<40, false>), g, b, 0, s, T, E, K, S, score, partial, bias, mask,
                         ids, probs, logits_out, err, g0, nullptr);
    else
      hipLaunchKernelGGL((k_route_select_wave<64, false>), g, b, 0, s, T, E, K, S, score, partial, bias, mask,
                         ids, probs, logits_out, err, g0, nullptr);
  }
  return hipGetLastError();
}

}  // namespace moe
