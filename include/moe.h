/*
 * moe.h -- C ABI of the single-GPU dropless mixture-of-experts layer hot path
 * for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The layer (bpdata article on dropless MoE in JAX with Transformer Engine,
 * figure "an expert-parallel MoE layer across two GPUs"): a router assigns each
 * token to K experts, token rows are grouped by expert, a grouped MLP runs two
 * grouped GEMMs on the variable-length groups, and a combine restores the
 * original token order.  One GPU's share of that path is four calls:
 *
 *   moe_route_topk         logits (or x . W_r) -> int16 [T,K] expert ids + fp32 probs
 *   moe_permute            per-expert count, scan and permute of the token rows
 *   moe_grouped_mlp        ragged grouped SwiGLU MLP (fp32, bf16, MXFP8 or MXFP4)
 *   moe_unpermute_combine  probability-weighted sum back in token order
 *
 * and the backward of the routing steps (combine, permute, route gates) and
 * the data and weight gradients of the grouped MLP,
 * plus one-time weight preparation and a standalone MX quantizer.
 *
 * Conventions shared by every call
 *  - Pointers named as device pointers must point to device memory (HBM) the
 *    caller owns; the library never allocates or frees memory.  Every tensor is
 *    row-major and contiguous, 16-byte aligned.
 *  - Host arguments are shapes only.  Data-dependent sizes (expert counts,
 *    offsets, the number N of routed rows) stay on the device: no call copies
 *    anything to the host or synchronises, so a whole layer can be captured in
 *    one HIP graph (bpdata article, "Optimization 1: Grouped GEMM": GEMM loops
 *    that needed device-to-host token counts broke graph capture).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it in order; nothing else is waited for.
 *  - Return value: MOE_OK, or an error status when an argument is invalid or a
 *    launch fails.  A non-zero status other than MOE_ERR_LAUNCH means nothing
 *    was enqueued; argument checks run before any HIP call, so they work on a
 *    machine without a GPU.
 *  - Data errors found on the device (an expert id out of range, more routed
 *    rows than `capacity`, a non-finite logit) set bits of the optional device
 *    word `err` with an atomic OR; the caller reads it whenever it likes.
 *  - Outputs are bitwise deterministic: no floating-point atomics, no split
 *    reductions whose order depends on scheduling.
 *  - Calls may be issued from several host threads; calls on one stream run in
 *    order, calls on different streams that share buffers race.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is out of the supported range */
  MOE_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  MOE_ERR_DTYPE = 4,     /* unsupported dtype or dtype combination */
  MOE_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
  MOE_ERR_LAUNCH = 6     /* a kernel launch failed (hipGetLastError) */
};

/* Element types. */
enum {
  MOE_F32 = 0,   /* IEEE fp32 */
  MOE_BF16 = 1,  /* bfloat16 (16-bit, fp32 exponent range) */
  MOE_MXFP8 = 2, /* OCP MX: E4M3 codes (uint8) + one E8M0 scale byte per 32
                    consecutive elements of a row (value = code * 2^(scale-127)) */
  MOE_MXFP4 = 3  /* OCP MX: E2M1 codes, two per byte (element 2i in the low
                    nibble, 2i+1 in the high nibble), + one E8M0 scale byte per
                    32 consecutive elements of a row */
};

/* Router score functions. */
enum {
  MOE_SCORE_SOFTMAX = 0, /* p_k = exp(z_k) / sum_j exp(z_j) over the K selected keys */
  MOE_SCORE_SIGMOID = 1  /* p_k = sigma(z_k) / sum_j sigma(z_j) over the K selected keys */
};

/* Device error-word bits. */
enum {
  MOE_DEVERR_BAD_ID = 1,    /* an expert id < -1 or >= E_global reached moe_permute */
  MOE_DEVERR_OVERFLOW = 2,  /* more routed local rows than `capacity` */
  MOE_DEVERR_NONFINITE = 4, /* a router key was NaN or +-inf */
  MOE_DEVERR_WORKSPACE = 8  /* moe_permute found its workspace not zero-filled
                               (its outputs are then unspecified) */
};

/* Limits of this implementation (checked; MOE_ERR_SHAPE otherwise). */
#define MOE_MAX_K 64          /* routes per token */
#define MOE_MAX_E 4096        /* experts seen by the router */
#define MOE_MAX_L 2048        /* local experts */

int moe_abi_version(void);
const char* moe_status_str(int status);

/* ------------------------------------------------------------------------
 * Sizes of every buffer of one layer shape (host only: no HIP call, so it
 * works on a machine without a GPU).
 *
 * bpdata article, "How to get started" (reproduction settings): buffers are
 * pre-sized and an overflow is checked for; "Optimization 1: Grouped GEMM":
 * the grouped GEMM computes only valid regions with no worst-case padding.
 * On one GPU the routed rows have an exact bound, so `capacity` never drops
 * a route: moe_route_topk gives a token K distinct experts, at most
 * min(K, L) of them local, hence capacity = T * min(K, L); ids supplied by
 * the caller may repeat an expert within a token (each slot gets its own
 * row), which needs capacity_any_ids = T * K.
 *
 * shape: T tokens, H hidden, E experts seen by the router, K routes per
 * token, L local experts (0 = all E), F expert FFN width, x_dtype (token
 * rows, MOE_BF16 / MOE_F32), w_dtype (router weights, MOE_F32 / MOE_BF16),
 * dtype (expert path: MOE_F32, MOE_BF16, MOE_MXFP8, MOE_MXFP4).
 * out: byte sizes for the calls below with capacity = out->capacity, and
 * the byte offsets of the documented parts of the MLP workspaces (the
 * activations `a` and their MX scales in moe_grouped_mlp's workspace; h,
 * d_h and, for MOE_MXFP8, d_h's row-wise MX codes and scales in
 * moe_grouped_mlp_backward_data's workspace).  Sizes of parts a dtype does
 * not have are 0.  Returns MOE_ERR_NULL, MOE_ERR_SHAPE or MOE_ERR_DTYPE for
 * bad arguments (out untouched).
 * ------------------------------------------------------------------------ */
typedef struct moe_shape {
  int T, H, E, K, L, F;
  int x_dtype, w_dtype, dtype;
} moe_shape;

typedef struct moe_sizes {
  int64_t capacity;          /* T * min(K, L): rows for ids from moe_route_topk */
  int64_t capacity_any_ids;  /* T * K: rows for any ids, repeats included */
  size_t router_prepared_bytes, route_workspace_bytes, permute_workspace_bytes;
  size_t permute_state_bytes;  /* the permute workspace's first bytes, zero between calls */
  size_t w1p_bytes, w2p_bytes, w1p_scales_bytes, w2p_scales_bytes;
  size_t mlp_workspace_bytes, mlp_act_offset, mlp_act_scales_offset;
  size_t w1t_bytes, w2t_bytes, w1t_scales_bytes, w2t_scales_bytes;
  size_t mlp_backward_workspace_bytes, bwd_h_offset, bwd_dh_offset, bwd_dh_codes_offset, bwd_dh_scales_offset;
  size_t mlp_backward_weights_workspace_bytes;
} moe_sizes;

int moe_query_sizes(const moe_shape* shape, moe_sizes* out);

/* ------------------------------------------------------------------------
 * Route: score + top-K selection (+ optional fused router projection)
 *
 * Sparser-MoE page (harryzhou2000), sections "Preserve a compact route" and
 * "The workload changes the bottleneck": the selected experts are carried as a
 * dense int16 [T,K] list instead of a [T,E] boolean map, selection uses bounded
 * histogram passes over a narrowed candidate range instead of K full-row
 * scans, invalid routes are -1, and small top-K shapes keep a direct path.
 *
 * Keys: z[t,e] = logit[t,e] (+ bias[e], one fp32 add), -0.0 read as +0.0.
 * Selection: the K largest keys per token, ties broken by the lower expert
 * index; ids[t,0..K-1] list them by descending key (ties: ascending index).
 * probs[t,k]: MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID over the K selected keys,
 * fp32.  A token with mask[t] != 0 gets ids -1 and probs 0.
 *
 * Logit source (exactly one):
 *  - logits  [T,E] fp32 device pointer, or
 *  - x [T,H] (x_dtype MOE_BF16 or MOE_F32) with router weights prepared by
 *    moe_prepare_router: logits = x . W_r accumulated in fp32 (for bf16 x and
 *    fp32 W_r each weight is split into three bf16 terms, which keeps fp32
 *    accuracy on bf16 matrix cores).
 * Optional (NULL = absent): bias [E] fp32, mask [T] uint8, logits_out [T,E]
 * fp32 (receives the logits before the bias), err.
 * Outputs: ids [T,K] int16, probs [T,K] fp32.
 * Limits: 1 <= K <= min(E, 64); E <= 4096; H % 32 == 0 for the projection.
 * Workspace: moe_route_workspace_bytes(T, E, H, x_dtype) bytes (0 allowed when
 * logits are given).
 * ------------------------------------------------------------------------ */
size_t moe_router_prepared_bytes(int H, int E, int w_dtype, int x_dtype);

/* Lay out the router weights W_r [H,E] (w_dtype MOE_F32 or MOE_BF16, device)
 * for moe_route_topk with activations of type x_dtype.  Output `prepared`
 * (device) has moe_router_prepared_bytes(...) bytes:
 *  x_dtype MOE_BF16: bf16 [C][H] in tiles of 32 rows.  With P terms per
 *    weight (P = 3, hi/mid/lo with W = hi + mid + lo, for fp32 W_r; P = 1 for
 *    bf16 W_r) a tile holds ept = floor(32/P) experts: row 32*t + p*ept + j
 *    holds term p of column e = t*ept + j of W_r.  C = ceil(E/ept)*32; rows
 *    with p >= P or e >= E are zero.  When C == 32 and H % 32 == 0 (one
 *    tile: the fused small-router path) the tile is k-blocked instead:
 *    element (row, h) at ((h/32)*32 + row)*32 + h%32.
 *  x_dtype MOE_F32: fp32 W_r [H,E] copied unchanged. */
int moe_prepare_router(const void* w_router, int w_dtype, int x_dtype, int H, int E,
                       void* prepared, void* stream);

size_t moe_route_workspace_bytes(int T, int E, int H, int x_dtype);

int moe_route_topk(int T, int E, int K, int H, int score, int x_dtype, int w_dtype,
                   const void* x, const void* w_prepared, const float* logits,
                   const float* bias, const uint8_t* mask,
                   int16_t* ids, float* probs, float* logits_out, int32_t* err,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Route, group-limited with a selection-only bias (a router refinement the
 * pages list as next work; the definition is the DeepSeek-V3 Technical
 * Report's, section "DeepSeekMoE with Auxiliary-Loss-Free Load Balancing")
 *
 * s[t,e] = sigmoid(logit[t,e]) in fp32.  Keys: s + bias[e] (one fp32 add;
 * bias optional) steer the choice only.  The E experts form n_group groups of
 * E/n_group consecutive ids; a group's score is the fp32 sum of its
 * m = K/topk_group largest keys, largest first; the topk_group groups with the
 * highest scores stay (ties: lower group index), and the K largest keys among
 * their experts are selected (ties: lower id), listed by descending key.
 * probs[t,k] = scale * s_k / sum_j s_j over the selected (bias not included).
 * Masked tokens: ids -1, probs 0.  Logit source, bias, mask, logits_out,
 * err, workspace: as moe_route_topk (no fused small-router path).
 * scores_out (optional, 16-byte aligned) [T,E] fp32 receives s.
 * Limits: 32 < E <= 1024; 1 <= n_group <= 64, n_group | E; 1 <= topk_group
 * <= n_group; topk_group | K; K/topk_group <= min(8, E/n_group);
 * 0 < scale < 3e38.  MOE_ERR_SHAPE otherwise.
 * ------------------------------------------------------------------------ */
int moe_route_topk_grouped(int T, int E, int K, int H, int n_group, int topk_group, float scale,
                           int x_dtype, int w_dtype, const void* x, const void* w_prepared,
                           const float* logits, const float* bias, const uint8_t* mask,
                           int16_t* ids, float* probs, float* logits_out, float* scores_out,
                           int32_t* err, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Permute: device count, single-pass scan and permute to expert order
 *
 * Sparser-MoE page, section "Remove work that has no selected route": local
 * pre-processing visits only the selected local slots of a token (a wavefront
 * ballot over its K slots, iterating set bits).  bpdata article, "Optimization
 * 1: Grouped GEMM": no device-to-host counts, no padding, no dropping.
 *
 * Local experts are ids e0 .. e0+L-1 of E_global.  For each valid local slot
 * (t,k), in flat order f = t*K + k:
 *   counts[e]      number of local slots of expert e0+e               int32 [L]
 *   offsets[e]     exclusive prefix of counts; offsets[L] = N          int32 [L+1]
 *   row r of expert e = offsets[e] + (number of earlier flat slots of e)
 *   x_perm[r]      = x[t]                                   [capacity,H]
 *   row_to_slot[r] = f                                      int32 [capacity]
 *   slot_to_row[t,k] = r, or -1 for -1 / non-local slots      int32 [T,K]
 * Rows r >= N of x_perm and row_to_slot are never written.  If N > capacity,
 * MOE_DEVERR_OVERFLOW is set in err, offsets still report the true counts and
 * rows >= capacity are dropped from x_perm/row_to_slot (their slot_to_row is
 * -1).  Ids < -1 or >= E_global set MOE_DEVERR_BAD_ID and count as -1.
 * x_dtype MOE_BF16 or MOE_F32; out_dtype = x_dtype, or MOE_MXFP8 with bf16 x:
 * x_perm then receives E4M3 codes [capacity,H] uint8 and x_perm_scales the
 * E8M0 scales [capacity,H/32] uint8 of 32-element blocks along H (OCP MX v1.0
 * rule: scale exponent floor(log2 max|v|) - 8, round to nearest even,
 * saturate at 448), which requires H % 32 == 0; or MOE_MXFP4 with bf16 x:
 * x_perm receives packed E2M1 codes [capacity,H/2] uint8 and x_perm_scales
 * the E8M0 scales [capacity,H/32] (scale exponent floor(log2 max|v|) - 2,
 * round to nearest even, saturate at 6).
 * Batches of at most 16384 slots (T * K) with at most 64 local experts run
 * one kernel that leaves the workspace untouched: each workgroup of 16
 * tokens counts every slot of the batch itself while its rows load, then
 * moves them.  Larger batches run two kernels: the first counts tiles of
 * consecutive tokens (one workgroup per tile, ids staged in LDS), gives each
 * local slot its row within its tile and expert, and publishes the tile's
 * counts; the workgroup that finishes last scans all tiles' counts (each
 * tile's base row per expert, the expert counts and offsets: a single-pass
 * scan in which no workgroup waits for another).  The second moves (or
 * MX-quantizes) each token's row to its rows.  Both give the same rows.
 * Workspace: moe_permute_workspace_bytes(T, K, L) bytes, zero-filled before
 * its first use; each call returns its state (a counter and the tile counts,
 * the first bytes) to zero when its kernels end, so one workspace serves any
 * number of calls, on one stream at a time, of any shape whose size fits.
 * A workspace found not zero-filled sets MOE_DEVERR_WORKSPACE: the outputs
 * are then unspecified, the call still ends, and the workspace must be
 * zero-filled again before the next call.  Limit: T * K < 2^30.
 * ------------------------------------------------------------------------ */
size_t moe_permute_workspace_bytes(int T, int K, int L);

int moe_permute(int T, int H, int K, int E_global, int e0, int L, int64_t capacity,
                int x_dtype, int out_dtype,
                const void* x, const int16_t* ids,
                int32_t* counts, int32_t* offsets, void* x_perm, uint8_t* x_perm_scales,
                int32_t* row_to_slot, int32_t* slot_to_row, int32_t* err,
                void* workspace, size_t workspace_bytes, void* stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and errors without the workspace, which is instead
 * a fixed array of moe_permute_noalloc_max_workspace_bytes() (16 MiB) that
 * the library holds on each GPU it runs on until the process ends.  Shapes
 * whose moe_permute_workspace_bytes(T, K, L) exceed it return
 * MOE_ERR_WORKSPACE before any launch.  No call allocates or frees memory;
 * each first clears the array's counters and flags with a fill kernel.  Calls
 * on one GPU share that GPU's array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must be ordered by the caller. */
size_t moe_permute_noalloc_max_workspace_bytes(void);
int moe_permute_noalloc(int T, int H, int K, int E_global, int e0, int L, int64_t capacity,
                        int x_dtype, int out_dtype, const void* x, const int16_t* ids,
                        int32_t* counts, int32_t* offsets, void* x_perm, uint8_t* x_perm_scales,
                        int32_t* row_to_slot, int32_t* slot_to_row, int32_t* err, void* stream);

/* ------------------------------------------------------------------------
 * Expert weights: one-time layout (+ MX quantization)
 *
 * bpdata article, reproduction settings: expert weights are pre-fused once.
 * Logical weights (device): W1 [L,H,2F] (gate columns [0,F), up columns
 * [F,2F)), W2 [L,F,H], in_dtype MOE_BF16 or MOE_F32.  Prepared layout, one
 * contiguous block per expert:
 *   W1p [L][2F][H]: row p holds column c(p) of W1[e] along H, where
 *       c(p) = (p/64)*32 + p%32 + ((p/32)%2 ? F : 0)   (gate/up chunks of 32
 *       interleaved so one output tile holds matching gate and up columns)
 *   W2p [L][H][F]: row n holds column n of W2[e] along F.
 * dtype MOE_F32: values in fp32, rows exactly as above.
 * dtype MOE_BF16: the rows above padded with zero rows to whole panels of 256
 *   (W1p [L][ceil(2F/256)*256][H], W2p [L][ceil(H/256)*256][F]), each panel
 *   k-blocked: [panel][k/32][256 rows][32 k], so one 32-wide k step of a panel
 *   is a contiguous 16 KiB block.  Requires H % 128 == 0 and F % 128 == 0.
 * dtype MOE_MXFP8 (in_dtype MOE_BF16): E4M3 codes (uint8) of the rows above
 *   with one E8M0 scale per 32 consecutive elements along a row, padded with
 *   zero rows (codes and scales) to whole panels of 256 rows and k-blocked:
 *   codes [L][panel][k/64][256 rows][64 k] (W1p: ceil(2F/256) panels over
 *   H, W2p: ceil(H/256) panels over F), scales [L][panel][ceil(k/512)][256
 *   rows][16] (w1p_scales, w2p_scales; the bytes past the last 32-block of a
 *   short final group are left as they are).  Requires H % 256 == 0 and
 *   F % 256 == 0.
 * dtype MOE_MXFP4 (in_dtype MOE_BF16): E2M1 codes of the rows above, two per
 *   byte (element 2i of a row in the low nibble), in the same zero-padded
 *   256-row panels, k-blocked by 128 elements: [L][panel][k/128][256 rows][64
 *   bytes]; scales exactly as for MOE_MXFP8.  Requires H % 512 == 0 and
 *   F % 512 == 0.
 * Requires H % 32 == 0 and F % 32 == 0 (MOE_F32).  Byte sizes:
 * moe_prepared_weight_bytes(L, H, F, dtype, which) with which = 1 (W1p),
 * 2 (W2p), 3 (W1p scales), 4 (W2p scales), and for the backward's panels
 * (moe_prepare_weights_backward) 5 (W1t), 6 (W2t), 7 (W1t scales), 8 (W2t
 * scales).
 * ------------------------------------------------------------------------ */
size_t moe_prepared_weight_bytes(int L, int H, int F, int dtype, int which);

int moe_prepare_weights(int L, int H, int F, int in_dtype, int dtype,
                        const void* w1, const void* w2,
                        void* w1p, void* w2p, uint8_t* w1p_scales, uint8_t* w2p_scales,
                        void* stream);

/* ------------------------------------------------------------------------
 * Grouped SwiGLU MLP over the expert-ordered rows
 *
 * bpdata article, "Optimization 1: Grouped GEMM": all expert matmuls in one
 * kernel, each with its actual token count, computing only valid regions;
 * "Transformer Engine building blocks": MXFP8 grouped GEMM for the expert
 * matmuls with group-aware MXFP8 quantization.
 *
 * For each local expert e with rows [offsets[e], offsets[e+1]) (clipped to
 * capacity):  h = x_perm[rows] . W1[e]  (fp32 accumulation),
 *             a = silu(h[:, :F]) * h[:, F:],  silu(g) = g * sigma(g),
 *             y_perm[rows] = a . W2[e].
 * dtype MOE_F32: x_perm, a, y_perm fp32.  MOE_BF16: x_perm, a, y_perm bf16.
 * MOE_MXFP8: x_perm as E4M3 codes + x_perm_scales (from moe_permute), `a`
 *   rounded to bf16 and then MX-quantized along F, y_perm bf16.
 * MOE_MXFP4: the same with packed E2M1 codes (x_perm [capacity][H/2] bytes,
 *   `a` quantized to E2M1 along F).
 * The schedule of output tiles is built on the device from `offsets`: empty
 * experts get no tiles.  Requires H % 128 == 0 and F % 128 == 0 for MOE_BF16,
 * H % 256 == 0 and F % 256 == 0 for MOE_MXFP8, H % 512 == 0 and F % 512 == 0
 * for MOE_MXFP4 (MX scale pointers 4-byte aligned), H % 16 == 0 and
 * F % 32 == 0 for MOE_F32.
 * Workspace: moe_grouped_mlp_workspace_bytes(capacity, F, dtype) bytes; it
 * starts with `a`: MOE_F32 [capacity][F] fp32; MOE_BF16 k-blocked
 * [F/32][capacity][32] bf16, followed at the next 256-byte boundary by 72 MiB
 * of fp32 split-K partial tiles (the tiles of a last, partial round of the
 * CUs are split along the contraction and summed in a fixed order); MOE_MXFP8
 * the codes [capacity][F], then at the next 256-byte boundary the scales
 * [capacity][F/32], then at the next 256-byte boundary 72 MiB of split-K
 * partial tiles; MOE_MXFP4 the same with packed codes [capacity][F/2].
 * ------------------------------------------------------------------------ */
size_t moe_grouped_mlp_workspace_bytes(int64_t capacity, int F, int dtype);

int moe_grouped_mlp(int L, int H, int F, int64_t capacity, int dtype,
                    const void* x_perm, const uint8_t* x_perm_scales, const int32_t* offsets,
                    const void* w1p, const uint8_t* w1p_scales,
                    const void* w2p, const uint8_t* w2p_scales,
                    void* y_perm, void* workspace, size_t workspace_bytes, void* stream);

/* moe_grouped_mlp for MOE_MXFP8 / MOE_MXFP4 that also stores the bf16 values
 * of `a` the GEMM1 epilogue quantizes, row-major [capacity][F] bf16 in
 * act_bf16 (device, 16-byte aligned; rows < N written).  A test hook: with
 * it the MX codes and scales of `a` can be checked bit for bit against the
 * quantizer's definition applied to the GPU's own `a` (for MOE_BF16 and
 * MOE_F32 the workspace already holds `a`: MOE_ERR_DTYPE).  act_bf16 NULL:
 * MOE_ERR_NULL. */
int moe_grouped_mlp_with_act(int L, int H, int F, int64_t capacity, int dtype,
                             const void* x_perm, const uint8_t* x_perm_scales, const int32_t* offsets,
                             const void* w1p, const uint8_t* w1p_scales,
                             const void* w2p, const uint8_t* w2p_scales,
                             void* y_perm, void* workspace, size_t workspace_bytes, void* act_bf16,
                             void* stream);

/* ------------------------------------------------------------------------
 * Unpermute + probability-weighted combine
 *
 * bpdata article, layer figure: the combine restores token order.
 *   out[t] = sum over k = 0..K-1 with slot_to_row[t,k] >= 0 (in k order, fp32
 *            accumulation) of probs[t,k] * y_perm[slot_to_row[t,k]]
 * A token with no such slot gets a zero row.  dtype MOE_BF16 (y_perm, out
 * bf16) or MOE_F32.  H % 8 == 0.
 * ------------------------------------------------------------------------ */
int moe_unpermute_combine(int T, int K, int H, int dtype,
                          const void* y_perm, const int32_t* slot_to_row, const float* probs,
                          void* out, void* stream);

/* ------------------------------------------------------------------------
 * Data gradient of the grouped SwiGLU MLP (bf16), the first part of the
 * grouped-GEMM backward (the pages' expert MLP is two grouped GEMMs on
 * variable-length groups, bpdata article, "Optimization 1: Grouped GEMM"; its
 * backward is the chain rule through them and SwiGLU).  For the rows of each
 * expert e: h = x_perm . W1[e] is recomputed and stored as bf16; d_a =
 * d_y_perm . W2[e]^T (fp32; MOE_BF16 keeps it in registers, MOE_MXFP8 stores
 * it in the workspace); d_h = [d_a * u * silu'(g),
 * d_a * silu(g)] with g = h[:, :F], u = h[:, F:], silu'(g) = sigma(g)
 * (1 + g (1 - sigma(g))), stored as bf16; d_x_perm = d_h . W1[e]^T (bf16).
 * All three are ragged grouped GEMMs on the device-built tile schedule.
 *
 * moe_prepare_weights_backward: from the logical W1 [L][H][2F] and W2
 *   [L][F][H] (bf16, as for moe_prepare_weights) lays out the W1^T panels
 *   (w1t: columns h of H, k = j of 2F in natural order, gate columns then up
 *   columns) and the W2^T panels (w2t: columns f of F, k = h of H), both
 *   bf16 [L][panel][k/32][256 rows][32 k], zero-padded to whole 256-row
 *   panels; sizes moe_prepared_weight_bytes(..., 5) and (..., 6).  dtype
 *   MOE_MXFP8 (H % 256 == 0, F % 256 == 0): the same panels as E4M3 codes and
 *   E8M0 scales in the layout of moe_prepare_weights' MOE_MXFP8 (codes
 *   [L][panel][k/64][256][64], scales [L][panel][ceil(k/512)][256][16] in
 *   w1t_scales / w2t_scales, sizes (..., 7) and (..., 8)); NULL for bf16.
 * moe_grouped_mlp_backward_data: x_perm, d_y_perm, d_x_perm [capacity][H]
 *   bf16 device; offsets as moe_grouped_mlp; w1p = moe_prepare_weights' W1p,
 *   w1t / w2t = moe_prepare_weights_backward's panels, all of `dtype`; the
 *   three scale pointers are NULL for MOE_BF16.  rows >= offsets[L] of
 *   d_x_perm are not written.  Workspace:
 *   moe_grouped_mlp_backward_workspace_bytes(capacity, H, F, dtype) bytes (h,
 *   d_h k-blocked bf16 at its start, which the weight gradient reads; the
 *   split-K partials; for MOE_MXFP8 the row-wise MX operands).  dtype
 *   MOE_BF16 (H % 128 == 0, F % 128 == 0) or MOE_MXFP8 (H % 256 == 0,
 *   F % 256 == 0, the three scale pointers 4-byte aligned: x_perm and d_y are
 *   MX-quantized along H; the d_a GEMM stores d_a as fp32 [capacity][F] in
 *   the workspace, and one elementwise kernel forms d_h from d_a and h,
 *   stores it as bf16 and MX-quantizes it along 2F in the same pass; fp32
 *   accumulation); capacity * max(H, 2F) * 2 < 2^31.  The byte offsets of h,
 *   d_h and (MOE_MXFP8) d_h's MX codes [capacity][2F] and scales
 *   [capacity][2F/32] (gates, then ups) in the workspace are given by
 *   moe_query_sizes.
 *   x_perm_q / x_perm_q_scales and d_y_perm_q / d_y_perm_q_scales (MOE_MXFP8
 *   only; NULL otherwise): the row-wise MX operands of x_perm and d_y along H
 *   (E4M3 codes [capacity][H], E8M0 scales [capacity][H/32]) as their
 *   producers write them: moe_permute with MOE_MXFP8 output (the forward's
 *   operand of GEMM1) and moe_unpermute_combine_backward with its MX output.
 *   Given, they are used as they are (the bf16 operand may then be NULL) and
 *   the call runs no quantization pass of its own over that operand
 *   (quantization fused with the kernels that produce the operands: the
 *   pages' planned "quantization fused with GEMM", bpdata article, closing
 *   paragraph of "Measured training impact"); not given, the call quantizes
 *   the bf16 operand into its workspace first.  Codes 16-byte and scales
 *   4-byte aligned.
 * ------------------------------------------------------------------------ */
int moe_prepare_weights_backward(int L, int H, int F, int dtype, const void* w1, const void* w2, void* w1t,
                                 void* w2t, uint8_t* w1t_scales, uint8_t* w2t_scales, void* stream);
size_t moe_grouped_mlp_backward_workspace_bytes(int64_t capacity, int H, int F, int dtype);
int moe_grouped_mlp_backward_data(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                                  const int32_t* offsets, const void* w1p, const uint8_t* w1p_scales,
                                  const void* w1t, const uint8_t* w1t_scales, const void* w2t,
                                  const uint8_t* w2t_scales, const void* d_y_perm, void* d_x_perm,
                                  const uint8_t* x_perm_q, const uint8_t* x_perm_q_scales, const uint8_t* d_y_perm_q,
                                  const uint8_t* d_y_perm_q_scales, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Weight gradient of the grouped SwiGLU MLP (bf16 or MXFP8 operands, fp32
 * results):
 * for each expert e with rows X_e (of x_perm), dW1[e] = X_e^T d_h_e [H][2F]
 * and dW2[e] = a_e^T d_y_e [F][H], contracted over the expert's own rows,
 * with a = bf16(silu(g) * u) and h, d_h as moe_grouped_mlp_backward_data
 * computed them: call this after that call, on the same stream, passing its
 * workspace as `data_workspace` (it holds h and d_h).  dW1 [L][H][2F] and dW2
 * [L][F][H] fp32 device; experts without rows get zeros.  The operands are
 * regrouped into 32-token blocks with the contraction index contiguous, each
 * expert's rows padded with zeros to a multiple of 128; the GEMMs run on the
 * grouped GEMM's pipeline, one tile per (expert, 256 x 256 block of dW).
 * dtype MOE_MXFP8: the four operands are quantized group-aware and column-wise
 * (as moe_mx_quantize_columns_grouped: MX blocks of 32 rows of one expert in
 * one column; each expert padded to a multiple of 256 rows here) and the
 * GEMMs run on the MX matrix-core instruction (fp32 accumulation).  h and d_h
 * are the ones the preceding moe_grouped_mlp_backward_data call left in
 * data_workspace, whichever its dtype: after a MOE_MXFP8 data pass they are
 * the values computed from MX operands, as a quantized training step uses
 * them (a is formed from that h).
 * Workspace: moe_grouped_mlp_backward_weights_workspace_bytes(L, capacity, H,
 * F, dtype) bytes.  Limits as moe_grouped_mlp_backward_data, and
 * (capacity + 128 L) * max(H, 2F) * 2 < 2^31 (MOE_MXFP8 also
 * (capacity + 256 L) * (max(H, 2F) + 255) < 2^31).
 * ------------------------------------------------------------------------ */
size_t moe_grouped_mlp_backward_weights_workspace_bytes(int L, int64_t capacity, int H, int F, int dtype);

/* Group-aware column-wise MX quantization, the operand form of an MXFP8
 * weight gradient (the pages' group-aware MXFP8 quantization; bpdata
 * article, "Transformer Engine building blocks for dropless MoE in JAX"): the
 * rows [offsets[e], offsets[e+1]) (bounded by capacity) of each expert group
 * of in [capacity][C] bf16 are cut into blocks of 32 consecutive rows of that
 * group alone (zero rows pad each group to a multiple of 128, so no block
 * holds rows of two groups), and each column of a block is one MX block (OCP
 * MX v1.0: E8M0 scale E = floor(log2 amax) - 8 clamped to [-127, 127], E4M3
 * codes rounded to nearest even, saturating).  Outputs (device): pb [L+1]
 * int32, the first block of each group (pb[L] = blocks written); codes
 * [blocks][C][32] uint8 (row 32 j + i of group e, column c at [pb[e] + j][c][i]);
 * scales [blocks][C] uint8 (E + 127).  codes and scales must hold
 * moe_mx_columns_grouped_max_blocks(L, capacity) blocks.  C % 64 == 0. */
int64_t moe_mx_columns_grouped_max_blocks(int L, int64_t capacity);
int moe_mx_quantize_columns_grouped(int L, int64_t capacity, int C, const void* in, const int32_t* offsets,
                                    int32_t* pb, uint8_t* codes, uint8_t* scales, void* stream);
int moe_grouped_mlp_backward_weights(int L, int H, int F, int64_t capacity, int dtype, const void* x_perm,
                                     const int32_t* offsets, const void* d_y_perm, const void* data_workspace,
                                     size_t data_workspace_bytes, float* dW1, float* dW2, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the routing steps (the pages' router work covered forward and
 * backward kernels; sparser-MoE page, "The workload changes the bottleneck").
 * For a fixed selection, with slot (t,k) routed to row r = slot_to_row[t,k]:
 *
 * moe_unpermute_combine_backward: gradients of moe_unpermute_combine's
 *   out[t] = sum_k probs[t,k] * y_perm[r]:
 *   d_y_perm[r] = probs[t,k] * dout[t] (dtype as y_perm, rounded once from
 *   fp32; rows without a slot untouched); d_probs[t,k] = <dout[t], y_perm[r]>
 *   (fp32, each lane's fixed-order sum then a fixed tree: deterministic), 0 for
 *   slots without a row.  dout [T,H], y_perm and d_y_perm [capacity,H] device.
 *   d_y_perm_q, d_y_perm_q_scales (optional, bf16 only, H % 32 == 0; NULL
 *   for none): each d_y_perm row written is also MX-quantized along H as it
 *   is formed (E4M3 codes [capacity][H], E8M0 scales [capacity][H/32], OCP MX
 *   v1.0 as moe_mx_quantize) -- the d_y operand of the MXFP8 data gradient.
 * moe_permute_backward: gradient of moe_permute's x_perm[r] = x[t]:
 *   d_x[t] = sum over the token's slots with a row (k order, fp32) of
 *   d_x_perm[r]; tokens without one get a zero row.
 * moe_route_backward: gradient of the gates with respect to the selected keys
 *   z = logit (+ score_bias), d_z [T,K] fp32 aligned with ids; the gradient
 *   of logit[t, ids[t,k]] is d_z[t,k] and of every other logit 0 (the choice
 *   is piecewise constant).  MOE_SCORE_SOFTMAX (probs needed): d_z_k = p_k
 *   (g_k - sum_j p_j g_j), g = d_probs.  MOE_SCORE_SIGMOID (logits [T,E]
 *   needed): p_k = scale s_k / S, s = sigma(z), S = sum_j s_j, d_z_k = s_k
 *   (1 - s_k) (scale g_k - sum_j g_j p_j) / S.  score_bias: moe_route_topk's
 *   bias (it enters the scores); NULL for moe_route_topk_grouped, whose bias
 *   only steers the choice (pass its scale).  Slots with id -1 give 0.
 * Limits as the forward calls; dtype MOE_BF16 or MOE_F32; H % 8 == 0;
 * 0 < scale < 3e38.
 * ------------------------------------------------------------------------ */
int moe_unpermute_combine_backward(int T, int K, int H, int dtype, const void* dout, const void* y_perm,
                                   const int32_t* slot_to_row, const float* probs, void* d_y_perm,
                                   float* d_probs, uint8_t* d_y_perm_q, uint8_t* d_y_perm_q_scales, void* stream);
int moe_permute_backward(int T, int K, int H, int dtype, const void* d_x_perm, const int32_t* slot_to_row,
                         void* d_x, void* stream);
int moe_route_backward(int T, int E, int K, int score, float scale, const int16_t* ids, const float* probs,
                       const float* d_probs, const float* logits, const float* score_bias, float* d_z,
                       void* stream);

/* ------------------------------------------------------------------------
 * Standalone MX quantization of bf16 rows (OCP MX v1.0, E4M3 + E8M0, blocks
 * of 32 along a row): in [rows][cols] bf16 -> codes [rows][cols] uint8,
 * scales [rows][cols/32] uint8.  If row_limit (device int32, may be NULL) is
 * given, only rows < *row_limit are quantized (ragged rows bounded by a device
 * value such as offsets[L]).  cols % 32 == 0.
 * ------------------------------------------------------------------------ */
int moe_mx_quantize(int64_t rows, int cols, const void* in, const int32_t* row_limit,
                    uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------
 * Calibration kernels: measurement support, not an operation of the layer.
 * The pages state their results as kernel times and rates; these kernels
 * measure the rates this GPU actually sustains, so that the layer's kernels
 * can be given as fractions of them next to the datasheet peaks.
 *
 * moe_calib_copy: dst = src, `bytes` (a multiple of 16; both 16-byte
 *   aligned, device) with streaming 16-byte loads and stores.
 * moe_calib_read: reads `bytes` of src (multiple of 16, 16-byte aligned) and
 *   writes one word per workgroup (an xor fold) to out, which holds
 *   moe_calib_read_out_words(bytes) words.
 * moe_calib_write: fills `bytes` of dst (multiple of 16, 16-byte aligned)
 *   with the 32-bit `value`.
 * moe_calib_mfma: `blocks` workgroups of 8 wavefronts, each wavefront `iters`
 *   rounds of 4 independent matrix-core instructions on register operands:
 *   MOE_BF16 v_mfma_f32_32x32x16_bf16 (32768 flops each), MOE_MXFP8
 *   v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes with unit E8M0 scales
 *   (131072 flops each); flops = blocks * 8 * 4 * iters * that.  out [blocks *
 *   512] fp32 (device) receives the accumulators' sums.
 * Zero bytes: a no-op.  Errors as for the other calls.
 * ------------------------------------------------------------------------ */
int moe_calib_copy(const void* src, void* dst, size_t bytes, void* stream);
size_t moe_calib_read_out_words(size_t bytes);
int moe_calib_read(const void* src, size_t bytes, uint32_t* out, void* stream);
int moe_calib_write(void* dst, size_t bytes, uint32_t value, void* stream);
int moe_calib_mfma(int dtype, int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
