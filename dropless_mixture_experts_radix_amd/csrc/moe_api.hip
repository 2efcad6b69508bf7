// C ABI entry points: argument checks (before any HIP call), workspace
// carving, kernel dispatch by shape and dtype.
#include "moe_internal.h"

using namespace moe;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of the supported range";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

// ---------------------------------------------------------------------------
// Route
// ---------------------------------------------------------------------------
size_t moe_router_prepared_bytes(int H, int E, int w_dtype, int x_dtype) {
  if (H <= 0 || E <= 0) return 0;
  if (x_dtype == MOE_BF16) {
    const int P = w_dtype == MOE_F32 ? 3 : 1, ept = 32 / P;
    const size_t C = (size_t)((E + ept - 1) / ept) * 32;
    return C * (size_t)H * 2;
  }
  return (size_t)H * E * 4;
}

int moe_prepare_router(const void* w_router, int w_dtype, int x_dtype, int H, int E, void* prepared,
                       void* stream) {
  if (!w_router || !prepared) return MOE_ERR_NULL;
  if (H <= 0 || E <= 0 || E > MOE_MAX_E) return MOE_ERR_SHAPE;
  if (!((x_dtype == MOE_BF16 && (w_dtype == MOE_F32 || w_dtype == MOE_BF16)) ||
        (x_dtype == MOE_F32 && w_dtype == MOE_F32)))
    return MOE_ERR_DTYPE;
  if (!aligned16(w_router) || !aligned16(prepared)) return MOE_ERR_ALIGN;
  return launch_status(launch_prepare_router(w_router, w_dtype, x_dtype, H, E, prepared, (hipStream_t)stream));
}

size_t moe_route_workspace_bytes(int T, int E, int H, int x_dtype) {
  if (T <= 0 || E <= 0) return 0;
  const RouteSplit sp = route_split(T, E, H > 0 ? H : 64, x_dtype);
  const int S = sp.S > sp.Sg ? sp.S : sp.Sg;  // either projection may run (it depends on the weights' type)
  return round_up((size_t)S * T * E * sizeof(float), 256);
}

// moe_route_topk and moe_route_topk_grouped (grp != nullptr: score checked
// by the caller, no fused small-router path)
static int route_topk(int T, int E, int K, int H, int score, int x_dtype, int w_dtype, const void* x,
                      const void* w_prepared, const float* logits, const float* bias, const uint8_t* mask,
                      int16_t* ids, float* probs, float* logits_out, int32_t* err, void* workspace,
                      size_t workspace_bytes, void* stream, const RouteGroups* grp, float* scores_out) {
  if (T < 0 || E <= 0 || E > MOE_MAX_E || K < 1 || K > E || K > MOE_MAX_K) return MOE_ERR_SHAPE;
  const bool from_x = logits == nullptr;
  if (T > 0 && (!ids || !probs)) return MOE_ERR_NULL;
  if (from_x) {
    if (T > 0 && (!x || !w_prepared)) return MOE_ERR_NULL;
    if (H <= 0) return MOE_ERR_SHAPE;
    if (x_dtype == MOE_BF16) {
      if (H % 64 != 0) return MOE_ERR_SHAPE;
      if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) return MOE_ERR_DTYPE;
    } else if (x_dtype == MOE_F32) {
      if (w_dtype != MOE_F32) return MOE_ERR_DTYPE;
    } else {
      return MOE_ERR_DTYPE;
    }
    if (!aligned16(x) || !aligned16(w_prepared)) return MOE_ERR_ALIGN;
    if (T > 0 && (!workspace || workspace_bytes < moe_route_workspace_bytes(T, E, H, x_dtype)))
      return MOE_ERR_WORKSPACE;
    if (T > 0 && !aligned16(workspace)) return MOE_ERR_ALIGN;
  } else {
    if (!aligned16(logits)) return MOE_ERR_ALIGN;
  }
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const float* partial = logits;
  int S = 1;
  if (from_x && !grp && route_fused_ok(E, H, x_dtype, w_dtype))
    return launch_status(launch_route_fused(T, E, K, H, score, w_dtype, x, w_prepared, bias, mask, ids, probs,
                                            logits_out, err, s));
  if (from_x) {
    float* ws = (float*)workspace;
    const RouteSplit sp = route_split(T, E, H, x_dtype);
    hipError_t e;
    if (x_dtype == MOE_BF16 && w_dtype == MOE_BF16 && sp.Sg > 0) {
      e = launch_router_gemm_bf16(T, E, H, sp.Sg, (const bf16_t*)x, (const bf16_t*)w_prepared, ws, s);
      S = sp.Sg;
    } else {
      e = launch_router_proj(T, E, H, x_dtype, w_dtype, x, w_prepared, ws, s);
      S = sp.S;
    }
    if (e != hipSuccess) return MOE_ERR_LAUNCH;
    partial = ws;
  }
  return launch_status(launch_route_select(T, E, K, S, score, partial, bias, mask, ids, probs,
                                           logits_out, err, s, grp, scores_out));
}

int moe_route_topk(int T, int E, int K, int H, int score, int x_dtype, int w_dtype, const void* x,
                   const void* w_prepared, const float* logits, const float* bias, const uint8_t* mask,
                   int16_t* ids, float* probs, float* logits_out, int32_t* err, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_DTYPE;
  return route_topk(T, E, K, H, score, x_dtype, w_dtype, x, w_prepared, logits, bias, mask, ids, probs,
                    logits_out, err, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int moe_route_topk_grouped(int T, int E, int K, int H, int n_group, int topk_group, float scale, int x_dtype,
                           int w_dtype, const void* x, const void* w_prepared, const float* logits,
                           const float* bias, const uint8_t* mask, int16_t* ids, float* probs,
                           float* logits_out, float* scores_out, int32_t* err, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (E <= 32 || E > ROUTE_GRP_MAX_E || n_group < 1 || n_group > 64 || E % n_group || topk_group < 1 ||
      topk_group > n_group || K < 1 || K % topk_group || K / topk_group > ROUTE_GRP_MAX_M ||
      K / topk_group > E / n_group || K > topk_group * (E / n_group))
    return MOE_ERR_SHAPE;
  if (!(scale > 0.f) || scale > 3.0e38f) return MOE_ERR_SHAPE;
  if (scores_out && !aligned16(scores_out)) return MOE_ERR_ALIGN;
  const RouteGroups g{n_group, topk_group, K / topk_group, scale};
  return route_topk(T, E, K, H, MOE_SCORE_SIGMOID, x_dtype, w_dtype, x, w_prepared, logits, bias, mask, ids,
                    probs, logits_out, err, workspace, workspace_bytes, stream, &g, scores_out);
}

// ---------------------------------------------------------------------------
// Permute
// ---------------------------------------------------------------------------
size_t moe_permute_workspace_bytes(int T, int K, int L) {
  if (T < 0 || K <= 0 || L <= 0) return 0;
  return permute_workspace_bytes(T, K, L);
}

// argument checks shared by moe_permute and moe_permute_noalloc
static int permute_check(int T, int H, int K, int E_global, int e0, int L, int64_t capacity, int x_dtype,
                         int out_dtype, const void* x, const int16_t* ids, int32_t* counts, int32_t* offsets,
                         void* x_perm, uint8_t* x_perm_scales, int32_t* row_to_slot, int32_t* slot_to_row) {
  if (T < 0 || H <= 0 || K < 1 || K > MOE_MAX_K || E_global <= 0 || E_global > 32767 || L < 1 ||
      L > MOE_MAX_L || e0 < 0 || e0 + L > E_global || capacity < 0)
    return MOE_ERR_SHAPE;
  if ((int64_t)T * K >= ((int64_t)1 << 30)) return MOE_ERR_SHAPE;  // counts fit the 30-bit published tile counts
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F32) return MOE_ERR_DTYPE;
  const bool mx_out = out_dtype == MOE_MXFP8 || out_dtype == MOE_MXFP4;
  if (!(out_dtype == x_dtype || (mx_out && x_dtype == MOE_BF16))) return MOE_ERR_DTYPE;
  if ((x_dtype == MOE_BF16 && H % 8) || (x_dtype == MOE_F32 && H % 4)) return MOE_ERR_SHAPE;
  if (mx_out && H % 32) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!x || !ids || !slot_to_row)) return MOE_ERR_NULL;
  if (capacity > 0 && (!x_perm || !row_to_slot)) return MOE_ERR_NULL;
  if (mx_out && capacity > 0 && !x_perm_scales) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int moe_permute(int T, int H, int K, int E_global, int e0, int L, int64_t capacity, int x_dtype,
                int out_dtype, const void* x, const int16_t* ids, int32_t* counts, int32_t* offsets,
                void* x_perm, uint8_t* x_perm_scales, int32_t* row_to_slot, int32_t* slot_to_row,
                int32_t* err, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = permute_check(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, x, ids, counts, offsets,
                               x_perm, x_perm_scales, row_to_slot, slot_to_row);
  if (st != MOE_OK) return st;
  if (!workspace || workspace_bytes < moe_permute_workspace_bytes(T, K, L)) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  return launch_status(launch_permute(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, x, ids, counts,
                                      offsets, x_perm, x_perm_scales, row_to_slot, slot_to_row, err, workspace,
                                      (hipStream_t)stream));
}

size_t moe_permute_noalloc_max_workspace_bytes(void) { return permute_noalloc_max_bytes(); }

int moe_permute_noalloc(int T, int H, int K, int E_global, int e0, int L, int64_t capacity, int x_dtype,
                        int out_dtype, const void* x, const int16_t* ids, int32_t* counts, int32_t* offsets,
                        void* x_perm, uint8_t* x_perm_scales, int32_t* row_to_slot, int32_t* slot_to_row,
                        int32_t* err, void* stream) {
  const int st = permute_check(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, x, ids, counts, offsets,
                               x_perm, x_perm_scales, row_to_slot, slot_to_row);
  if (st != MOE_OK) return st;
  if (moe_permute_workspace_bytes(T, K, L) > permute_noalloc_max_bytes()) return MOE_ERR_WORKSPACE;
  return launch_status(launch_permute_noalloc(T, H, K, E_global, e0, L, capacity, x_dtype, out_dtype, x, ids,
                                              counts, offsets, x_perm, x_perm_scales, row_to_slot, slot_to_row, err,
                                              (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Weights
// ---------------------------------------------------------------------------
size_t moe_prepared_weight_bytes(int L, int H, int F, int dtype, int which) {
  if (L <= 0 || H <= 0 || F <= 0) return 0;
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_MXFP8 && dtype != MOE_MXFP4) return 0;
  const bool mx = dtype == MOE_MXFP8 || dtype == MOE_MXFP4;
  size_t n1 = (size_t)L * 2 * F * H, n2 = (size_t)L * H * F;  // elements
  if (dtype != MOE_F32) {  // whole 256-row panels
    n1 = (size_t)L * ((2 * (size_t)F + 255) / 256 * 256) * H;
    n2 = (size_t)L * (((size_t)H + 255) / 256 * 256) * F;
  }
  auto bytes = [&](size_t n) {
    return dtype == MOE_F32 ? n * 4 : dtype == MOE_BF16 ? n * 2 : dtype == MOE_MXFP8 ? n : n / 2;
  };
  switch (which) {
    case 1: return bytes(n1);
    case 2: return bytes(n2);
    // MX scales: 16 bytes per prepared row and 512-wide k group
    case 3: return mx ? n1 / H * (((size_t)H + 511) / 512) * 16 : 0;
    case 4: return mx ? n2 / F * (((size_t)F + 511) / 512) * 16 : 0;
    // the backward's bf16 panels: W1^T (ceil(H/256) panels over 2F), W2^T (ceil(F/256) panels over H)
    case 5: return dtype == MOE_BF16 || dtype == MOE_MXFP8
                       ? (size_t)L * (((size_t)H + 255) / 256 * 256) * 2 * F * (dtype == MOE_BF16 ? 2 : 1) : 0;
    case 6: return dtype == MOE_BF16 || dtype == MOE_MXFP8
                       ? (size_t)L * (((size_t)F + 255) / 256 * 256) * H * (dtype == MOE_BF16 ? 2 : 1) : 0;
    // scales of the backward's MXFP8 panels
    case 7: return dtype == MOE_MXFP8 ? (size_t)L * (((size_t)H + 255) / 256 * 256) * ((2 * (size_t)F + 511) / 512) * 16 : 0;
    case 8: return dtype == MOE_MXFP8 ? (size_t)L * (((size_t)F + 255) / 256 * 256) * (((size_t)H + 511) / 512) * 16 : 0;
    default: return 0;
  }
}

int moe_prepare_weights(int L, int H, int F, int in_dtype, int dtype, const void* w1, const void* w2,
                        void* w1p, void* w2p, uint8_t* w1p_scales, uint8_t* w2p_scales, void* stream) {
  if (L < 1 || L > MOE_MAX_L || H <= 0 || F <= 0 || H % 32 || F % 32) return MOE_ERR_SHAPE;
  if (dtype == MOE_BF16 && (H % 128 || F % 128)) return MOE_ERR_SHAPE;  // groups of 4 32-wide k steps
  if (dtype == MOE_MXFP8 && (H % 256 || F % 256)) return MOE_ERR_SHAPE;  // groups of 4 64-wide k stages
  if (dtype == MOE_MXFP4 && (H % 512 || F % 512)) return MOE_ERR_SHAPE;  // groups of 4 128-wide k stages
  if (!((dtype == MOE_F32 && in_dtype == MOE_F32) || (dtype == MOE_BF16 && in_dtype == MOE_BF16) ||
        ((dtype == MOE_MXFP8 || dtype == MOE_MXFP4) && in_dtype == MOE_BF16)))
    return MOE_ERR_DTYPE;
  if (!w1 || !w2 || !w1p || !w2p) return MOE_ERR_NULL;
  if ((dtype == MOE_MXFP8 || dtype == MOE_MXFP4) && (!w1p_scales || !w2p_scales)) return MOE_ERR_NULL;
  if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1p) || !aligned16(w2p)) return MOE_ERR_ALIGN;
  return launch_status(launch_prepare_weights(L, H, F, dtype, w1, w2, w1p, w2p, w1p_scales, w2p_scales,
                                              (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Grouped MLP
// ---------------------------------------------------------------------------
size_t moe_grouped_mlp_workspace_bytes(int64_t capacity, int F, int dtype) {
  if (capacity <= 0 || F <= 0) return 256;
  size_t a;
  if (dtype == MOE_F32) a = (size_t)capacity * F * 4;
  else if (dtype == MOE_BF16) a = round_up((size_t)capacity * F * 2, 256) + grouped_mlp_bf16_part_bytes();
  else a = round_up((size_t)capacity * (dtype == MOE_MXFP4 ? F / 2 : F), 256) +
           round_up((size_t)capacity * (F / 32), 256) + grouped_mlp_mx_part_bytes();
  return round_up(a, 256);
}

static int grouped_mlp(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                       const uint8_t* x_perm_scales, const int32_t* offsets, const void* w1p, const uint8_t* w1p_scales,
                       const void* w2p, const uint8_t* w2p_scales, void* y_perm, void* workspace, size_t workspace_bytes,
                       void* act_bf16, void* stream) {
  if (L < 1 || L > MOE_MAX_L || H <= 0 || F <= 0 || capacity < 0 || capacity > (int64_t)1 << 31)
    return MOE_ERR_SHAPE;
  if (dtype == MOE_F32) {
    if (H % 16 || F % 32) return MOE_ERR_SHAPE;
  } else if (dtype == MOE_BF16) {
    if (H % 128 || F % 128) return MOE_ERR_SHAPE;
    // byte offsets of the activation buffers stay within 31 bits
    if (capacity * (int64_t)(H > F ? H : F) * 2 > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  } else if (dtype == MOE_MXFP8) {
    if (H % 256 || F % 256) return MOE_ERR_SHAPE;
    if (capacity * (int64_t)(H > F ? H : F) > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  } else if (dtype == MOE_MXFP4) {
    if (H % 512 || F % 512) return MOE_ERR_SHAPE;
    if (capacity * (int64_t)(H > F ? H : F) / 2 > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  } else {
    return MOE_ERR_DTYPE;
  }
  const bool mx = dtype == MOE_MXFP8 || dtype == MOE_MXFP4;
  if (act_bf16 && !mx) return MOE_ERR_DTYPE;  // the bf16 / fp32 workspace already holds `a`
  if (!offsets) return MOE_ERR_NULL;
  if (capacity > 0 && (!x_perm || !w1p || !w2p || !y_perm)) return MOE_ERR_NULL;
  if (mx && capacity > 0 && (!x_perm_scales || !w1p_scales || !w2p_scales)) return MOE_ERR_NULL;
  if (!aligned16(x_perm) || !aligned16(w1p) || !aligned16(w2p) || !aligned16(y_perm) || !aligned16(act_bf16))
    return MOE_ERR_ALIGN;
  if (mx && (((uintptr_t)x_perm_scales | (uintptr_t)w1p_scales | (uintptr_t)w2p_scales) & 3u))
    return MOE_ERR_ALIGN;  // scale words are read 4 bytes at a time
  if (!workspace || workspace_bytes < moe_grouped_mlp_workspace_bytes(capacity, F, dtype))
    return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == MOE_F32) {
    e = launch_grouped_mlp_f32(L, H, F, capacity, (const float*)x_perm, offsets, (const float*)w1p,
                               (const float*)w2p, (float*)workspace, (float*)y_perm, s);
  } else if (dtype == MOE_BF16) {
    float* part = (float*)((uint8_t*)workspace + round_up((size_t)capacity * F * 2, 256));
    e = launch_grouped_mlp_bf16(L, H, F, capacity, (const bf16_t*)x_perm, offsets, (const bf16_t*)w1p,
                                (const bf16_t*)w2p, (bf16_t*)workspace, part, (bf16_t*)y_perm, s);
  } else {
    const bool fp4 = dtype == MOE_MXFP4;
    uint8_t* act = (uint8_t*)workspace;
    uint8_t* act_s = act + round_up((size_t)capacity * (fp4 ? F / 2 : F), 256);
    float* part = (float*)(act_s + round_up((size_t)capacity * (F / 32), 256));
    e = launch_grouped_mlp_mx(L, H, F, capacity, fp4, (const uint8_t*)x_perm, x_perm_scales, offsets,
                              (const uint8_t*)w1p, w1p_scales, (const uint8_t*)w2p, w2p_scales, act, act_s,
                              part, (bf16_t*)y_perm, (bf16_t*)act_bf16, s);
  }
  return launch_status(e);
}

int moe_grouped_mlp(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                    const uint8_t* x_perm_scales, const int32_t* offsets, const void* w1p,
                    const uint8_t* w1p_scales, const void* w2p, const uint8_t* w2p_scales, void* y_perm,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_mlp(L, H, F, capacity, dtype, x_perm, x_perm_scales, offsets, w1p, w1p_scales, w2p, w2p_scales,
                     y_perm, workspace, workspace_bytes, nullptr, stream);
}

int moe_grouped_mlp_with_act(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                             const uint8_t* x_perm_scales, const int32_t* offsets, const void* w1p,
                             const uint8_t* w1p_scales, const void* w2p, const uint8_t* w2p_scales, void* y_perm,
                             void* workspace, size_t workspace_bytes, void* act_bf16, void* stream) {
  if (!act_bf16) return MOE_ERR_NULL;
  return grouped_mlp(L, H, F, capacity, dtype, x_perm, x_perm_scales, offsets, w1p, w1p_scales, w2p, w2p_scales,
                     y_perm, workspace, workspace_bytes, act_bf16, stream);
}

// ---------------------------------------------------------------------------
// Combine
// ---------------------------------------------------------------------------
int moe_unpermute_combine(int T, int K, int H, int dtype, const void* y_perm, const int32_t* slot_to_row,
                          const float* probs, void* out, void* stream) {
  if (T < 0 || K < 1 || K > MOE_MAX_K || H <= 0 || H % 8) return MOE_ERR_SHAPE;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (T > 0 && (!slot_to_row || !probs || !out)) return MOE_ERR_NULL;
  if (!aligned16(y_perm) || !aligned16(out)) return MOE_ERR_ALIGN;
  return launch_status(launch_combine(T, K, H, dtype, y_perm, slot_to_row, probs, out, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Data gradient of the grouped MLP
// ---------------------------------------------------------------------------
int moe_prepare_weights_backward(int L, int H, int F, int dtype, const void* w1, const void* w2, void* w1t,
                                 void* w2t, uint8_t* w1t_scales, uint8_t* w2t_scales, void* stream) {
  if (L < 1 || L > MOE_MAX_L || H <= 0 || F <= 0 || H % 128 || F % 128) return MOE_ERR_SHAPE;
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (dtype == MOE_MXFP8 && (H % 256 || F % 256)) return MOE_ERR_SHAPE;  // groups of 4 64-wide k stages
  if (!w1 || !w2 || !w1t || !w2t) return MOE_ERR_NULL;
  if (dtype == MOE_MXFP8 && (!w1t_scales || !w2t_scales)) return MOE_ERR_NULL;
  if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1t) || !aligned16(w2t)) return MOE_ERR_ALIGN;
  return launch_status(launch_prepare_weights_backward(L, H, F, dtype, w1, w2, w1t, w2t, w1t_scales, w2t_scales,
                                                       (hipStream_t)stream));
}

// MXFP8 data gradient: row-wise MX codes and scales of x_perm, d_y (C = H) and d_h (C = 2F)
static size_t mx_rows_bytes(int64_t capacity, int C) {
  return round_up((size_t)capacity * C, 256) + round_up((size_t)capacity * (C / 32), 256);
}

size_t moe_grouped_mlp_backward_workspace_bytes(int64_t capacity, int H, int F, int dtype) {
  if (capacity <= 0 || H <= 0 || F <= 0 || (dtype != MOE_BF16 && dtype != MOE_MXFP8)) return 256;
  // h and d_h ([2F/32][capacity][32] bf16 each), the split-K partials, then
  // (MXFP8) the MX operands of x_perm, d_y and d_h
  const size_t part = grouped_mlp_bf16_part_bytes() > grouped_mlp_mx_part_bytes() ? grouped_mlp_bf16_part_bytes()
                                                                                  : grouped_mlp_mx_part_bytes();
  size_t b = 2 * round_up((size_t)capacity * 2 * F * 2, 256) + round_up(part, 256);
  if (dtype == MOE_MXFP8)  // (and d_a, fp32 [capacity][F])
    b += 2 * mx_rows_bytes(capacity, H) + mx_rows_bytes(capacity, 2 * F) + round_up((size_t)capacity * F * 4, 256);
  return b;
}

int moe_grouped_mlp_backward_data(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                                  const int32_t* offsets, const void* w1p, const uint8_t* w1p_scales,
                                  const void* w1t, const uint8_t* w1t_scales, const void* w2t,
                                  const uint8_t* w2t_scales, const void* d_y_perm, void* d_x_perm,
                                  const uint8_t* x_perm_q, const uint8_t* x_perm_q_scales, const uint8_t* d_y_perm_q,
                                  const uint8_t* d_y_perm_q_scales, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (L < 1 || L > MOE_MAX_L || H <= 0 || F <= 0 || capacity < 0 || capacity > (int64_t)1 << 31)
    return MOE_ERR_SHAPE;
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (H % 128 || F % 128) return MOE_ERR_SHAPE;
  if (dtype == MOE_MXFP8 && (H % 256 || F % 256)) return MOE_ERR_SHAPE;
  if (dtype == MOE_MXFP8 && (!w1p_scales || !w1t_scales || !w2t_scales)) return MOE_ERR_NULL;
  if (dtype == MOE_MXFP8 && (((uintptr_t)w1p_scales | (uintptr_t)w1t_scales | (uintptr_t)w2t_scales) & 3u))
    return MOE_ERR_ALIGN;  // scale words are read 4 bytes at a time, as in the forward
  // byte offsets of the k-blocked h / d_h buffers and of the rows stay within 31 bits
  if (capacity * (int64_t)(H > 2 * F ? H : 2 * F) * 2 > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (!offsets || !w1p || !w1t || !w2t) return MOE_ERR_NULL;
  // MXFP8: row-wise MX operands of x_perm and d_y may come from their producers
  const bool xq_given = x_perm_q || x_perm_q_scales, dyq_given = d_y_perm_q || d_y_perm_q_scales;
  if ((xq_given || dyq_given) && dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if ((xq_given && (!x_perm_q || !x_perm_q_scales)) || (dyq_given && (!d_y_perm_q || !d_y_perm_q_scales)))
    return MOE_ERR_NULL;
  if (capacity > 0 && ((!x_perm && !xq_given) || (!d_y_perm && !dyq_given) || !d_x_perm || !workspace))
    return MOE_ERR_NULL;
  if (!aligned16(x_perm) || !aligned16(w1p) || !aligned16(w1t) || !aligned16(w2t) || !aligned16(d_y_perm) ||
      !aligned16(d_x_perm) || !aligned16(workspace) || !aligned16(x_perm_q) || !aligned16(d_y_perm_q))
    return MOE_ERR_ALIGN;
  if (((uintptr_t)x_perm_q_scales | (uintptr_t)d_y_perm_q_scales) & 3u) return MOE_ERR_ALIGN;
  if (capacity > 0 && workspace_bytes < moe_grouped_mlp_backward_workspace_bytes(capacity, H, F, dtype))
    return MOE_ERR_WORKSPACE;
  bf16_t* hbuf = (bf16_t*)workspace;
  bf16_t* dhbuf = (bf16_t*)((uint8_t*)workspace + round_up((size_t)capacity * 2 * F * 2, 256));
  float* part = (float*)((uint8_t*)workspace + 2 * round_up((size_t)capacity * 2 * F * 2, 256));
  if (dtype == MOE_MXFP8) {
    uint8_t* w = (uint8_t*)part + round_up(grouped_mlp_bf16_part_bytes() > grouped_mlp_mx_part_bytes()
                                               ? grouped_mlp_bf16_part_bytes()
                                               : grouped_mlp_mx_part_bytes(), 256);
    uint8_t* xq = w;   w += round_up((size_t)capacity * H, 256);
    uint8_t* xqs = w;  w += round_up((size_t)capacity * (H / 32), 256);
    uint8_t* dyq = w;  w += round_up((size_t)capacity * H, 256);
    uint8_t* dyqs = w; w += round_up((size_t)capacity * (H / 32), 256);
    uint8_t* dhq = w;  w += round_up((size_t)capacity * 2 * F, 256);
    uint8_t* dhqs = w; w += round_up((size_t)capacity * (2 * F / 32), 256);
    float* da = (float*)w;
    if (xq_given) {
      xq = (uint8_t*)x_perm_q;
      xqs = (uint8_t*)x_perm_q_scales;
    }
    if (dyq_given) {
      dyq = (uint8_t*)d_y_perm_q;
      dyqs = (uint8_t*)d_y_perm_q_scales;
    }
    return launch_status(launch_grouped_mlp_mx_backward(
        L, H, F, capacity, (const bf16_t*)x_perm, offsets, (const uint8_t*)w1p, w1p_scales, (const uint8_t*)w1t,
        w1t_scales, (const uint8_t*)w2t, w2t_scales, (const bf16_t*)d_y_perm, xq, xqs, dyq, dyqs, hbuf, dhbuf, dhq,
        dhqs, da, part, (bf16_t*)d_x_perm, xq_given, dyq_given, (hipStream_t)stream));
  }
  return launch_status(launch_grouped_mlp_bf16_backward(L, H, F, capacity, (const bf16_t*)x_perm, offsets,
                                                        (const bf16_t*)w1p, (const bf16_t*)w1t, (const bf16_t*)w2t,
                                                        (const bf16_t*)d_y_perm, hbuf, dhbuf, part,
                                                        (bf16_t*)d_x_perm, (hipStream_t)stream));
}

// weight gradient: 32-token blocks of all experts' rows, each expert padded to 128
static int64_t wgrad_blocks_max(int L, int64_t capacity) { return (capacity + 128 * (int64_t)L + 31) / 32; }

int64_t moe_mx_columns_grouped_max_blocks(int L, int64_t capacity) {
  if (L < 1 || capacity < 0) return 0;
  return wgrad_blocks_max(L, capacity);
}

int moe_mx_quantize_columns_grouped(int L, int64_t capacity, int C, const void* in, const int32_t* offsets,
                                    int32_t* pb, uint8_t* codes, uint8_t* scales, void* stream) {
  if (L < 1 || L > MOE_MAX_L || capacity < 0 || capacity > (int64_t)1 << 31 || C <= 0 || C % 64) return MOE_ERR_SHAPE;
  const int64_t nbmax = wgrad_blocks_max(L, capacity);
  if (nbmax * 32 * (int64_t)C > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (!offsets || !pb) return MOE_ERR_NULL;
  if (capacity > 0 && (!in || !codes || !scales)) return MOE_ERR_NULL;
  if (!aligned16(in) || !aligned16(codes)) return MOE_ERR_ALIGN;
  return launch_status(launch_mx_columns_grouped(L, capacity, C, capacity > 0 ? (int)nbmax : 0, (const bf16_t*)in,
                                                 offsets, pb, codes, scales, (hipStream_t)stream));
}

// MXFP8 weight gradient: rows of all experts, each padded to a multiple of
// 256, and their 512-row scale groups
static int64_t wgrad_mx_rows_max(int L, int64_t capacity) { return capacity + 256 * (int64_t)L; }
static int64_t wgrad_mx_groups_max(int L, int64_t capacity) { return capacity / 512 + L + 1; }

// byte sizes of the MXFP8 operands: A-form (rows = C columns) and B-form (256-column panels)
static size_t mx_a_codes(int L, int64_t cap, int C) { return round_up((size_t)wgrad_mx_rows_max(L, cap) * C, 256); }
static size_t mx_a_scales(int L, int64_t cap, int C) { return round_up((size_t)wgrad_mx_rows_max(L, cap) / 32 * C, 256); }
static size_t mx_b_codes(int L, int64_t cap, int C) {
  return round_up((size_t)wgrad_mx_rows_max(L, cap) * ((C + 255) / 256 * 256), 256);
}
static size_t mx_b_scales(int L, int64_t cap, int C) {
  return round_up((size_t)wgrad_mx_groups_max(L, cap) * ((C + 255) / 256 * 256) * 16, 256);
}

size_t moe_grouped_mlp_backward_weights_workspace_bytes(int L, int64_t capacity, int H, int F, int dtype) {
  if (L <= 0 || capacity <= 0 || H <= 0 || F <= 0 || (dtype != MOE_BF16 && dtype != MOE_MXFP8)) return 256;
  if (dtype == MOE_MXFP8)
    return 2 * round_up((size_t)(L + 1) * 4, 256) + mx_a_codes(L, capacity, H) + mx_a_scales(L, capacity, H) +
           mx_b_codes(L, capacity, 2 * F) + mx_b_scales(L, capacity, 2 * F) + mx_a_codes(L, capacity, F) +
           mx_a_scales(L, capacity, F) + mx_b_codes(L, capacity, H) + mx_b_scales(L, capacity, H);
  const size_t tok = (size_t)wgrad_blocks_max(L, capacity) * 32 * 2;  // bytes per column of a token-blocked operand
  return round_up((size_t)(L + 1) * 4, 256) + round_up(tok * H, 256) + round_up(tok * 2 * F, 256) +
         round_up(tok * F, 256) + round_up(tok * H, 256);
}

int moe_grouped_mlp_backward_weights(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                                     const int32_t* offsets, const void* d_y_perm, const void* data_workspace,
                                     size_t data_workspace_bytes, float* dW1, float* dW2, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (L < 1 || L > MOE_MAX_L || H <= 0 || F <= 0 || capacity < 0 || capacity > (int64_t)1 << 31)
    return MOE_ERR_SHAPE;
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (H % 128 || F % 128) return MOE_ERR_SHAPE;
  if (capacity * (int64_t)(H > 2 * F ? H : 2 * F) * 2 > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (dtype == MOE_MXFP8 && wgrad_mx_rows_max(L, capacity) * (int64_t)((2 * F > H ? 2 * F : H) + 255) > (int64_t)INT32_MAX)
    return MOE_ERR_SHAPE;
  // token-blocked operands and the per-expert weight slices stay within 31-bit byte offsets
  const int64_t nbmax = wgrad_blocks_max(L, capacity);
  if (nbmax * 32 * (int64_t)(H > 2 * F ? H : 2 * F) * 2 > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (!offsets || !dW1 || !dW2) return MOE_ERR_NULL;
  if (capacity > 0 && (!x_perm || !d_y_perm || !data_workspace || !workspace)) return MOE_ERR_NULL;
  if (!aligned16(x_perm) || !aligned16(d_y_perm) || !aligned16(data_workspace) || !aligned16(dW1) ||
      !aligned16(dW2) || !aligned16(workspace))
    return MOE_ERR_ALIGN;
  if (capacity > 0 && (data_workspace_bytes < moe_grouped_mlp_backward_workspace_bytes(capacity, H, F, MOE_BF16) ||
                       workspace_bytes < moe_grouped_mlp_backward_weights_workspace_bytes(L, capacity, H, F, dtype)))
    return MOE_ERR_WORKSPACE;
  if (capacity == 0) return MOE_OK;
  const bf16_t* hbuf = (const bf16_t*)data_workspace;
  const bf16_t* dhbuf = (const bf16_t*)((const uint8_t*)data_workspace + round_up((size_t)capacity * 2 * F * 2, 256));
  if (dtype == MOE_MXFP8) {
    uint8_t* w = (uint8_t*)workspace;
    int32_t* pk = (int32_t*)w;
    w += round_up((size_t)(L + 1) * 4, 256);
    int32_t* png = (int32_t*)w;
    w += round_up((size_t)(L + 1) * 4, 256);
    uint8_t* xa = w;   w += mx_a_codes(L, capacity, H);
    uint8_t* xas = w;  w += mx_a_scales(L, capacity, H);
    uint8_t* dhb = w;  w += mx_b_codes(L, capacity, 2 * F);
    uint8_t* dhbs = w; w += mx_b_scales(L, capacity, 2 * F);
    uint8_t* aa = w;   w += mx_a_codes(L, capacity, F);
    uint8_t* aas = w;  w += mx_a_scales(L, capacity, F);
    uint8_t* dyb = w;  w += mx_b_codes(L, capacity, H);
    uint8_t* dybs = w;
    const int nbmx = (int)(wgrad_mx_rows_max(L, capacity) / 32);
    return launch_status(launch_grouped_mlp_mx_wgrad(L, H, F, capacity, nbmx, (const bf16_t*)x_perm, offsets,
                                                     (const bf16_t*)d_y_perm, hbuf, dhbuf, pk, png, xa, xas, dhb, dhbs,
                                                     aa, aas, dyb, dybs, dW1, dW2, (hipStream_t)stream));
  }
  const size_t tok = (size_t)nbmax * 32 * 2;
  uint8_t* w = (uint8_t*)workspace;
  int32_t* pb = (int32_t*)w;
  w += round_up((size_t)(L + 1) * 4, 256);
  bf16_t* xt = (bf16_t*)w;
  w += round_up(tok * H, 256);
  bf16_t* dht = (bf16_t*)w;
  w += round_up(tok * 2 * F, 256);
  bf16_t* at = (bf16_t*)w;
  w += round_up(tok * F, 256);
  bf16_t* dyt = (bf16_t*)w;
  return launch_status(launch_grouped_mlp_bf16_wgrad(L, H, F, capacity, (int)nbmax, (const bf16_t*)x_perm, offsets,
                                                     (const bf16_t*)d_y_perm, hbuf, dhbuf, pb, xt, dht, at, dyt, dW1,
                                                     dW2, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Backward of the routing steps
// ---------------------------------------------------------------------------
int moe_unpermute_combine_backward(int T, int K, int H, int dtype, const void* dout, const void* y_perm,
                                   const int32_t* slot_to_row, const float* probs, void* d_y_perm,
                                   float* d_probs, uint8_t* d_y_perm_q, uint8_t* d_y_perm_q_scales, void* stream) {
  if (T < 0 || K < 1 || K > MOE_MAX_K || H <= 0 || H % 8) return MOE_ERR_SHAPE;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (T > 0 && (!dout || !slot_to_row || !probs || !d_probs)) return MOE_ERR_NULL;
  if (!aligned16(dout) || !aligned16(y_perm) || !aligned16(d_y_perm)) return MOE_ERR_ALIGN;
  if (d_y_perm_q || d_y_perm_q_scales) {  // the MX operand form of d_y as well
    if (dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (H % 32) return MOE_ERR_SHAPE;
    if (!d_y_perm_q || !d_y_perm_q_scales) return MOE_ERR_NULL;
    if (!aligned16(d_y_perm_q)) return MOE_ERR_ALIGN;
  }
  return launch_status(launch_combine_backward(T, K, H, dtype, dout, y_perm, slot_to_row, probs, d_y_perm,
                                               d_probs, d_y_perm_q, d_y_perm_q_scales, (hipStream_t)stream));
}

int moe_permute_backward(int T, int K, int H, int dtype, const void* d_x_perm, const int32_t* slot_to_row,
                         void* d_x, void* stream) {
  if (T < 0 || K < 1 || K > MOE_MAX_K || H <= 0 || H % 8) return MOE_ERR_SHAPE;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (T > 0 && (!slot_to_row || !d_x)) return MOE_ERR_NULL;
  if (!aligned16(d_x_perm) || !aligned16(d_x)) return MOE_ERR_ALIGN;
  return launch_status(launch_combine(T, K, H, dtype, d_x_perm, slot_to_row, nullptr, d_x, (hipStream_t)stream));
}

int moe_route_backward(int T, int E, int K, int score, float scale, const int16_t* ids, const float* probs,
                       const float* d_probs, const float* logits, const float* score_bias, float* d_z,
                       void* stream) {
  if (T < 0 || E <= 0 || E > MOE_MAX_E || K < 1 || K > E || K > MOE_MAX_K) return MOE_ERR_SHAPE;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_DTYPE;
  if (!(scale > 0.f) || scale > 3.0e38f) return MOE_ERR_SHAPE;
  if (T > 0 && (!ids || !d_probs || !d_z)) return MOE_ERR_NULL;
  if (T > 0 && score == MOE_SCORE_SOFTMAX && !probs) return MOE_ERR_NULL;
  if (T > 0 && score == MOE_SCORE_SIGMOID && !logits) return MOE_ERR_NULL;
  return launch_status(launch_route_backward(T, E, K, score, scale, ids, probs, d_probs, logits, score_bias, d_z,
                                             (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Size queries (host only: no HIP call)
// ---------------------------------------------------------------------------
int moe_query_sizes(const moe_shape* sh, moe_sizes* out) {
  if (!sh || !out) return MOE_ERR_NULL;
  const int T = sh->T, H = sh->H, E = sh->E, K = sh->K, F = sh->F, dt = sh->dtype;
  const int L = sh->L > 0 ? sh->L : E;
  if (T < 0 || H <= 0 || E <= 0 || E > MOE_MAX_E || K < 1 || K > E || K > MOE_MAX_K || F <= 0 || L > E ||
      L > MOE_MAX_L)
    return MOE_ERR_SHAPE;
  if (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_MXFP8 && dt != MOE_MXFP4) return MOE_ERR_DTYPE;
  if (sh->x_dtype != MOE_F32 && sh->x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (sh->w_dtype != MOE_F32 && sh->w_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  moe_sizes z = {};
  // moe_route_topk gives each token K distinct experts, so at most min(K, L)
  // of its slots are local; caller-supplied ids may repeat an expert (each
  // slot then has its own row), which needs T * K rows
  z.capacity = (int64_t)T * (K < L ? K : L);
  z.capacity_any_ids = (int64_t)T * K;
  const int64_t cap = z.capacity;
  z.router_prepared_bytes = moe_router_prepared_bytes(H, E, sh->w_dtype, sh->x_dtype);
  z.route_workspace_bytes = moe_route_workspace_bytes(T, E, H, sh->x_dtype);
  z.permute_workspace_bytes = moe_permute_workspace_bytes(T, K, L);
  z.permute_state_bytes = permute_state_bytes(T, K, L);
  z.w1p_bytes = moe_prepared_weight_bytes(L, H, F, dt, 1);
  z.w2p_bytes = moe_prepared_weight_bytes(L, H, F, dt, 2);
  z.w1p_scales_bytes = moe_prepared_weight_bytes(L, H, F, dt, 3);
  z.w2p_scales_bytes = moe_prepared_weight_bytes(L, H, F, dt, 4);
  z.mlp_workspace_bytes = moe_grouped_mlp_workspace_bytes(cap, F, dt);
  z.mlp_act_offset = 0;
  if (dt == MOE_MXFP8 || dt == MOE_MXFP4)
    z.mlp_act_scales_offset = round_up((size_t)cap * (dt == MOE_MXFP4 ? F / 2 : F), 256);
  if (dt == MOE_BF16 || dt == MOE_MXFP8) {
    z.w1t_bytes = moe_prepared_weight_bytes(L, H, F, dt, 5);
    z.w2t_bytes = moe_prepared_weight_bytes(L, H, F, dt, 6);
    z.w1t_scales_bytes = moe_prepared_weight_bytes(L, H, F, dt, 7);
    z.w2t_scales_bytes = moe_prepared_weight_bytes(L, H, F, dt, 8);
    z.mlp_backward_workspace_bytes = moe_grouped_mlp_backward_workspace_bytes(cap, H, F, dt);
    z.bwd_h_offset = 0;
    z.bwd_dh_offset = round_up((size_t)cap * 2 * F * 2, 256);
    if (dt == MOE_MXFP8) {
      const size_t part = grouped_mlp_bf16_part_bytes() > grouped_mlp_mx_part_bytes() ? grouped_mlp_bf16_part_bytes()
                                                                                      : grouped_mlp_mx_part_bytes();
      const size_t w = 2 * z.bwd_dh_offset + round_up(part, 256) + 2 * mx_rows_bytes(cap, H);
      z.bwd_dh_codes_offset = w;
      z.bwd_dh_scales_offset = w + round_up((size_t)cap * 2 * F, 256);
    }
    z.mlp_backward_weights_workspace_bytes = moe_grouped_mlp_backward_weights_workspace_bytes(L, cap, H, F, dt);
  }
  *out = z;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Standalone MX quantizer
// ---------------------------------------------------------------------------
int moe_mx_quantize(int64_t rows, int cols, const void* in, const int32_t* row_limit, uint8_t* codes,
                    uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return MOE_ERR_SHAPE;
  if (rows > 0 && (!in || !codes || !scales)) return MOE_ERR_NULL;
  if (!aligned16(in) || !aligned16(codes)) return MOE_ERR_ALIGN;
  return launch_status(launch_mx_quantize(rows, cols, (const bf16_t*)in, row_limit, codes, scales,
                                          (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Calibration kernels (measurement support)
// ---------------------------------------------------------------------------
int moe_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_NULL;
  if (bytes % 16) return MOE_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
  return launch_status(launch_calib_copy(src, dst, bytes, (hipStream_t)stream));
}

size_t moe_calib_read_out_words(size_t bytes) {
  int blocks = 0;
  (void)launch_calib_read(nullptr, bytes, nullptr, &blocks, nullptr);
  return (size_t)blocks;
}

int moe_calib_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !out) return MOE_ERR_NULL;
  if (bytes % 16) return MOE_ERR_SHAPE;
  if (!aligned16(src)) return MOE_ERR_ALIGN;
  int blocks = 0;
  return launch_status(launch_calib_read(src, bytes, out, &blocks, (hipStream_t)stream));
}

int moe_calib_write(void* dst, size_t bytes, uint32_t value, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!dst) return MOE_ERR_NULL;
  if (bytes % 16) return MOE_ERR_SHAPE;
  if (!aligned16(dst)) return MOE_ERR_ALIGN;
  return launch_status(launch_calib_write(dst, bytes, value, (hipStream_t)stream));
}

int moe_calib_mfma(int dtype, int blocks, int iters, float* out, void* stream) {
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return MOE_ERR_SHAPE;
  if (!out) return MOE_ERR_NULL;
  return launch_status(launch_calib_mfma(dtype == MOE_MXFP8, blocks, iters, out, (hipStream_t)stream));
}

}  // extern "C"
