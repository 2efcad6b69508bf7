"""CPU oracle of the dropless MoE layer hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke entry
point and the CPU-baseline leg of the benchmark may import or call this module.
The HIP library never routes through it, and it shares no code, table or helper
with the HIP path: every conversion below (bf16 rounding, E4M3 coding, the MX
block scale) is written out here from its definition.

Precision: float64 throughout.  Results are rounded only where the layer
stores a value in a narrower type (fp32 logits/probabilities, bf16 or fp32
activations and outputs, MXFP8 codes and scales).

The layer, as the pages describe it (bpdata article "Dropless MoE ... JAX ...
Transformer Engine", figure "an expert-parallel MoE layer across two GPUs"):
the router assigns each token to K experts, token rows are grouped by expert,
a grouped MLP runs two grouped GEMMs on the variable-length groups, and the
combine restores the original token order.  The single-GPU share of that path
is computed here by plain definitions:

  route_topk            sort-based top-K with lowest-index tie-break
  route_topk_repeated_argmax   the K-repeated-scan selection the "Preserve a
                        compact route" section of the sparser-MoE page names as
                        the original path (kept as an independent second
                        oracle for the pins)
  route_grouped         group-limited routing with a selection-only bias (the
                        DeepSeek-style router refinement; its definition is
                        the DeepSeek-V3 Technical Report's, not the pages')
  count_and_permute     stable counting sort of the valid local routes
  mx_quantize_rows      OCP Microscaling (MX) v1.0 block quantization, E4M3
  mx_quantize_columns_grouped  the same along columns, blocked per expert group
  mx4_quantize_rows     the same with E2M1 (MXFP4) elements
  grouped_mlp           per-expert dense SwiGLU MLP in float64
  combine               probability-weighted sum in k order
  combine_backward, permute_backward, route_backward
                        the gradients of those routing steps (by definition:
                        the adjoint sums and the derivative of the scores)
  grouped_mlp_backward_data   the data gradient of the grouped MLP (chain rule
                        through both GEMMs and SwiGLU, h recomputed)
  grouped_mlp_backward_weights the weight gradient (per-expert contractions
                        over the expert's own rows)

Every function is parity-pinned by tests/test_oracle_*.py (pages' worked sizes,
closed forms, brute force, a second algorithm, library reductions); the whole
layer against the pages is "parity unpinned" because the pages print no layer
values (only its parts are pinned).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Number formats (written from their definitions)
# ---------------------------------------------------------------------------

BF16_MAX = float.fromhex("0x1.fep127")


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 |a|) for finite non-zero a, read exactly from frexp."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range: the spacing of
    representable values near |v| is 2^(max(floor(log2|v|), -126) - 7).
    Values beyond the largest finite bf16 become +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    e = np.maximum(_floor_log2(np.where(nz, v, 1.0)), -126)
    q = np.ldexp(1.0, (e - 7).astype(np.int64))
    r = np.round(v / q) * q  # np.round is round-half-to-even; v/q is exact
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)
    out[nz] = r[nz]
    out[~nz] = v[~nz]  # keeps the sign of zero
    return out


def bf16_to_bits(v) -> np.ndarray:
    """Bit patterns (uint16) of values that are already exact bf16 values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bits_to_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# OCP 8-bit floating point E4M3 ("fn" variant): bias 7, 3 mantissa bits, no
# infinities, S.1111.111 is NaN, largest finite magnitude 448, smallest normal
# 2^-6, smallest subnormal 2^-9.
E4M3_MAX = 448.0
E4M3_EMIN = -6
E4M3_MBITS = 3
E4M3_EMAX_ELEM = 8  # exponent of the largest normal (448 = 1.75 * 2^8)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte codes -> float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    ex = (c >> 3) & 15
    m = c & 7
    sub = np.ldexp(m / 8.0, E4M3_EMIN)
    nrm = np.ldexp(1.0 + m / 8.0, (ex - 7))
    val = s * np.where(ex == 0, sub, nrm)
    return np.where((ex == 15) & (m == 7), np.nan, val)


def e4m3_round(q) -> np.ndarray:
    """Round float64 values to the E4M3 grid, ties to even, saturating at +-448.

    The spacing near |q| is 2^(max(floor(log2|q|), -6) - 3); magnitudes that
    round above 448 are clamped to 448 (the MX conversion saturates normals).
    The sign of zero is kept.
    """
    q = np.asarray(q, dtype=np.float64)
    nz = q != 0
    e = np.maximum(_floor_log2(np.where(nz, q, 1.0)), E4M3_EMIN)
    quantum = np.ldexp(1.0, (e - E4M3_MBITS).astype(np.int64))
    r = np.round(q / quantum) * quantum
    r = np.where(np.abs(r) > E4M3_MAX, np.copysign(E4M3_MAX, q), r)
    r = np.where(nz, r, q)
    # a non-zero value that rounds to zero keeps its sign
    return np.where((r == 0) & np.signbit(q), -0.0, r)


def e4m3_encode(r) -> np.ndarray:
    """Exact E4M3 grid values (from e4m3_round) -> byte codes."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.int64) << 7
    a = np.abs(r)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = (a > 0) & (a < np.ldexp(1.0, E4M3_EMIN))
    code = np.where(sub, np.round(a / np.ldexp(1.0, E4M3_EMIN - E4M3_MBITS)).astype(np.int64), code)
    nrm = a >= np.ldexp(1.0, E4M3_EMIN)
    e = _floor_log2(np.where(nrm, a, 1.0))
    man = np.round((np.where(nrm, a, 1.0) / np.ldexp(1.0, e) - 1.0) * 8).astype(np.int64)
    code = np.where(nrm, ((e + 7) << 3) | man, code)
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# MX block quantization (OCP Microscaling Formats Specification v1.0)
# ---------------------------------------------------------------------------

MX_BLOCK = 32


def mx_quantize_rows(v):
    """Quantize each row of v (bf16 values as float64) in blocks of 32.

    Follows the OCP MX v1.0 conversion with E4M3 elements: for each block of
    32 consecutive elements along the row (the contraction dimension), the
    shared exponent is E = floor(log2(max|v|)) - 8 (8 = exponent of E4M3's
    largest normal), clamped to the E8M0 range [-127, 127] (E = -127 for an
    all-zero block).  Each element is v * 2^-E rounded to E4M3 (nearest, ties
    to even, saturating at 448).  Returns (codes uint8 [R,C], scales uint8
    [R,C/32] holding E + 127).

    The pages name group-aware MXFP8 quantization as a building block
    (bpdata article, "Transformer Engine building blocks for dropless MoE in
    JAX"; "Optimization 1: Grouped GEMM" for MXFP8 block scaling of the expert
    matmuls); the block rule is the published MX specification's.
    """
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blk = v.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blk).max(axis=2)
    E = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - E4M3_EMAX_ELEM, -127)
    E = np.clip(E, -127, 127)
    q = blk * np.ldexp(1.0, -E)[:, :, None]  # exact: a power-of-two scaling
    codes = e4m3_encode(e4m3_round(q)).reshape(R, C)
    scales = (E + 127).astype(np.uint8)
    return codes, scales


def mx_quantize_columns_grouped(v, offsets, pad_rows=128):
    """Group-aware column-wise MX quantization (E4M3 elements, E8M0 scales):
    MX blocks of 32 consecutive rows of one column, the rows of each expert
    group [offsets[e], offsets[e+1]) blocked on their own (padded with zero
    rows to a multiple of pad_rows), so no block holds rows of two groups.
    This is the form the expert GEMMs' weight gradient contracts over (the
    pages' group-aware MXFP8 building block; bpdata article, "Transformer
    Engine building blocks for dropless MoE in JAX").
    Returns (pb [L+1] first block of each group, codes [nb][C][32] uint8 with
    the code of the group's row 32*j + i of column c at [pb[e] + j][c][i],
    scales [nb][C] uint8)."""
    v = np.asarray(v, dtype=np.float64)
    C = v.shape[1]
    L = len(offsets) - 1
    pb = [0]
    codes, scales = [], []
    for e in range(L):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        m = hi - lo
        mp = -(-m // pad_rows) * pad_rows
        blk = np.zeros((mp, C))
        blk[:m] = v[lo:hi]
        nb = mp // 32
        pb.append(pb[-1] + nb)
        if nb:
            # [nb, 32, C] -> [nb, C, 32]: each column of a block is one row for the row quantizer
            t = blk.reshape(nb, 32, C).transpose(0, 2, 1).reshape(nb * C, 32)
            c, s_ = mx_quantize_rows(t)
            codes.append(c.reshape(nb, C, 32))
            scales.append(s_.reshape(nb, C))
    codes = np.concatenate(codes) if codes else np.zeros((0, C, 32), np.uint8)
    scales = np.concatenate(scales) if scales else np.zeros((0, C), np.uint8)
    return np.array(pb, np.int64), codes, scales


def mx_dequantize_rows(codes, scales) -> np.ndarray:
    codes = np.asarray(codes)
    R, C = codes.shape
    vals = e4m3_decode(codes).reshape(R, C // MX_BLOCK, MX_BLOCK)
    s = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (vals * s[:, :, None]).reshape(R, C)


# OCP 4-bit floating point E2M1 (OCP MX v1.0, FP4 element): 1 sign bit, 2
# exponent bits with bias 1, 1 mantissa bit, no infinities or NaN.  Magnitudes
# 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6; largest normal 6 = 1.5 * 2^2,
# smallest normal 1 = 2^0.
E2M1_MAX = 6.0
E2M1_EMIN = 0
E2M1_MBITS = 1
E2M1_EMAX_ELEM = 2  # exponent of the largest normal


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (low 4 bits of each byte) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 15
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    ex = (c >> 1) & 3
    m = c & 1
    sub = np.ldexp(m / 2.0, E2M1_EMIN)
    nrm = np.ldexp(1.0 + m / 2.0, ex - 1)
    return s * np.where(ex == 0, sub, nrm)


def e2m1_round(q) -> np.ndarray:
    """Round float64 values to the E2M1 grid, ties to even, saturating at +-6.

    The spacing near |q| is 2^(max(floor(log2|q|), 0) - 1); magnitudes that
    round above 6 are clamped to 6 (the MX conversion saturates).  The sign of
    zero is kept."""
    q = np.asarray(q, dtype=np.float64)
    nz = q != 0
    e = np.maximum(_floor_log2(np.where(nz, q, 1.0)), E2M1_EMIN)
    quantum = np.ldexp(1.0, (e - E2M1_MBITS).astype(np.int64))
    r = np.round(q / quantum) * quantum
    r = np.where(np.abs(r) > E2M1_MAX, np.copysign(E2M1_MAX, q), r)
    r = np.where(nz, r, q)
    return np.where((r == 0) & np.signbit(q), -0.0, r)


def e2m1_encode(r) -> np.ndarray:
    """Exact E2M1 grid values (from e2m1_round) -> codes 0..15 (uint8)."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.int64) << 3
    a = np.abs(r)
    code = np.where(a == 0.5, 1, 0).astype(np.int64)
    nrm = a >= 1.0
    e = _floor_log2(np.where(nrm, a, 1.0))
    man = np.round((np.where(nrm, a, 1.0) / np.ldexp(1.0, e) - 1.0) * 2).astype(np.int64)
    code = np.where(nrm, ((e + 1) << 1) | man, code)
    return (code | sign).astype(np.uint8)


def mx4_quantize_rows(v):
    """MXFP4: quantize each row of v (bf16 values as float64) in blocks of 32.

    The OCP MX v1.0 conversion with E2M1 elements: per block of 32 consecutive
    elements along the row, E = floor(log2(max|v|)) - 2 (2 = exponent of
    E2M1's largest normal), clamped to [-127, 127] (E = -127 for an all-zero
    block); each element is v * 2^-E rounded to E2M1 (nearest, ties to even,
    saturating at 6).  Returns (codes uint8 [R,C] holding one 4-bit code each,
    scales uint8 [R,C/32] holding E + 127).  pack_fp4 gives the two-per-byte
    storage form."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blk = v.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blk).max(axis=2)
    E = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - E2M1_EMAX_ELEM, -127)
    E = np.clip(E, -127, 127)
    q = blk * np.ldexp(1.0, -E)[:, :, None]  # exact: a power-of-two scaling
    codes = e2m1_encode(e2m1_round(q)).reshape(R, C)
    scales = (E + 127).astype(np.uint8)
    return codes, scales


def mx4_dequantize_rows(codes, scales) -> np.ndarray:
    codes = np.asarray(codes)
    R, C = codes.shape
    vals = e2m1_decode(codes).reshape(R, C // MX_BLOCK, MX_BLOCK)
    s = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (vals * s[:, :, None]).reshape(R, C)


def pack_fp4(codes) -> np.ndarray:
    """[R,C] codes 0..15 -> [R,C/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 15) | ((c[:, 1::2] & 15) << 4)


def unpack_fp4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# Route: projection, score, top-K, probabilities
# ---------------------------------------------------------------------------

def router_logits(x, w_router) -> np.ndarray:
    """logits[T,E] = x[T,H] . W_r[H,E], exact products summed in float64,
    stored as fp32 (the router works in fp32; the pages' layer figure starts
    with the router assigning tokens to experts)."""
    return (np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)).astype(np.float32)


def selection_keys(logits, bias=None) -> np.ndarray:
    """z = logit (+ per-expert bias, one fp32 rounding), -0.0 replaced by +0.0."""
    z = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        z = (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    z = np.where(z == 0, np.float32(0.0), z).astype(np.float32)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite router logits")
    return z


def _probabilities(zs, score):
    zs = np.asarray(zs, dtype=np.float64)
    if score == "softmax":
        e = np.exp(zs - zs[:, :1])
        p = e / e.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-zs))
        p = s / s.sum(axis=1, keepdims=True)
    else:
        raise ValueError(score)
    return p.astype(np.float32)


def route_topk(logits, K, score="softmax", bias=None, mask=None):
    """Top-K experts per token and their probabilities.

    Selection: the K largest keys z (logit plus optional bias), ties broken by
    the lower expert index; the IDs are listed in that order (descending key).
    The result is the compact [T,K] int16 ID list of the sparser-MoE page,
    "Preserve a compact route"; masked tokens carry -1 routes (same section:
    invalid -1 routes are preserved).
    Probabilities: softmax over the K selected keys, or for score="sigmoid"
    sigma(z_k) / sum_j sigma(z_j) over the selected keys; fp32.
    """
    z = selection_keys(logits, bias)
    T, E = z.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    order = np.argsort(-z, axis=1, kind="stable")  # stable: equal keys keep index order
    ids = order[:, :K].astype(np.int64)
    zs = np.take_along_axis(z, ids, axis=1)
    p = _probabilities(zs, score)
    ids = ids.astype(np.int16)
    if mask is not None:
        m = np.asarray(mask).astype(bool)
        ids[m] = -1
        p[m] = 0.0
    return ids, p


def route_topk_repeated_argmax(logits, K, score="softmax", bias=None, mask=None):
    """Second, independent selection: K passes, each scanning the whole row
    for the next maximum (np.argmax returns the first, i.e. lowest-index,
    maximum).  This is the T x E x K scan the sparser-MoE page ("Preserve a
    compact route") says the radix/threshold selection replaced."""
    z = selection_keys(logits, bias).astype(np.float64)
    T, E = z.shape
    ids = np.zeros((T, K), dtype=np.int64)
    work = z.copy()
    for k in range(K):
        j = np.argmax(work, axis=1)
        ids[:, k] = j
        work[np.arange(T), j] = -np.inf
    zs = np.take_along_axis(z, ids, axis=1)
    p = _probabilities(zs, score)
    ids = ids.astype(np.int16)
    if mask is not None:
        m = np.asarray(mask).astype(bool)
        ids[m] = -1
        p[m] = 0.0
    return ids, p


def sigmoid_scores(logits) -> np.ndarray:
    """s = 1 / (1 + exp(-logit)) in float64, stored as fp32."""
    z = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite router logits")
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def _fp32_sum_desc(v):
    """fp32 left fold of the values along the last axis, taken in descending order."""
    v = -np.sort(-np.asarray(v, dtype=np.float32), axis=-1)
    acc = v[..., 0].astype(np.float32)
    for i in range(1, v.shape[-1]):
        acc = (acc + v[..., i]).astype(np.float32)
    return acc


def route_grouped(logits, K, n_group, topk_group, bias=None, scale=1.0, mask=None, scores=None):
    """Group-limited routing with a selection-only bias.

    Not from the pages: the pages' next steps name router refinements, and this
    is the DeepSeek-style form they point to, as the DeepSeek-V3 Technical
    Report defines it (section "DeepSeekMoE with Auxiliary-Loss-Free Load
    Balancing": sigmoid affinities, a per-expert bias that only steers the
    top-K choice, gates normalized over the selected affinities, and routing
    limited to the groups (nodes) whose experts score highest, a group scored
    by the sum of its K/topk_group highest affinities).

    s = sigmoid(logit), fp32 (or `scores`: given fp32 values of s, so that a
    check can take the selection on another implementation's own fp32 s).
    Keys: k = s + bias (one fp32 add; bias optional).  The E experts form
    n_group groups of E/n_group consecutive ids; a group's score is the fp32
    sum of its m = K/topk_group largest keys, largest first.  The topk_group
    groups with the highest scores stay (ties: lower group index); the K
    largest keys among their experts are selected (ties: lower expert id) and
    listed by descending key.  probs = scale * s_k / sum_j s_j over the
    selected (fp32).  Masked tokens get -1 and 0.
    """
    s = sigmoid_scores(logits) if scores is None else np.asarray(scores, dtype=np.float32)
    T, E = s.shape
    if n_group < 1 or E % n_group or not (1 <= topk_group <= n_group) or K % topk_group:
        raise ValueError("need n_group | E, 1 <= topk_group <= n_group, topk_group | K")
    gs, m = E // n_group, K // topk_group
    if not (1 <= K <= topk_group * gs) or m > gs:
        raise ValueError("need 1 <= K <= topk_group * E / n_group")
    key = s if bias is None else (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    key = np.where(key == 0, np.float32(0.0), key).astype(np.float32)
    if not np.all(np.isfinite(key)):
        raise ValueError("non-finite selection keys")
    gk = key.reshape(T, n_group, gs)
    gscore = _fp32_sum_desc(-np.sort(-gk, axis=2)[:, :, :m])          # [T, n_group]
    gkeep = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]  # stable: lower group first
    keep = np.zeros((T, n_group), dtype=bool)
    keep[np.arange(T)[:, None], gkeep] = True
    allowed = np.repeat(keep, gs, axis=1)
    masked = np.where(allowed, key, np.float32(-np.inf)).astype(np.float32)
    ids = np.argsort(-masked, axis=1, kind="stable")[:, :K].astype(np.int64)
    ssel = np.take_along_axis(s, ids, axis=1).astype(np.float64)
    p = (scale * ssel / ssel.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = ids.astype(np.int16)
    if mask is not None:
        mk = np.asarray(mask).astype(bool)
        ids[mk] = -1
        p[mk] = 0.0
    return ids, p


# ---------------------------------------------------------------------------
# Count / scan / permute
# ---------------------------------------------------------------------------

def count_and_permute(ids, e0, L, x=None, E_global=None):
    """Group the valid local routes by expert (a stable counting sort).

    A slot (t,k) is local when e0 <= ids[t,k] < e0+L; -1 slots and other
    ranks' experts are skipped (sparser-MoE page, "Remove work that has no
    selected route": only selected local slots are visited).  Rows are ordered
    by local expert, and within an expert by flat slot index f = t*K + k.

    Returns counts [L], offsets [L+1] (offsets[L] = N), row_to_slot [N]
    (= f), slot_to_row [T,K] (-1 where not local) and, when x is given,
    x_perm [N,H] = x[f // K].  Nothing is padded and nothing is dropped
    (bpdata article, "Optimization 1: Grouped GEMM": only valid regions).
    """
    ids = np.asarray(ids).astype(np.int64)
    T, K = ids.shape
    if E_global is not None and ((ids < -1) | (ids >= E_global)).any():
        raise ValueError("expert id out of range")
    flat_ids = ids.ravel()
    valid = (flat_ids >= e0) & (flat_ids < e0 + L)
    f = np.flatnonzero(valid)
    le = flat_ids[f] - e0
    order = np.argsort(le, kind="stable")
    row_to_slot = f[order].astype(np.int64)
    counts = np.bincount(le, minlength=L).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    slot_to_row = np.full(T * K, -1, dtype=np.int64)
    slot_to_row[row_to_slot] = np.arange(row_to_slot.size)
    out = {
        "counts": counts,
        "offsets": offsets,
        "row_to_slot": row_to_slot,
        "slot_to_row": slot_to_row.reshape(T, K),
    }
    if x is not None:
        out["x_perm"] = np.asarray(x)[row_to_slot // K]
    return out


# ---------------------------------------------------------------------------
# Grouped SwiGLU MLP
# ---------------------------------------------------------------------------

def swiglu(h, F):
    """a = silu(gate) * up with gate = h[:, :F], up = h[:, F:], silu(g) = g*sigma(g)
    (Shazeer 2020, "GLU Variants Improve Transformer")."""
    g = h[:, :F]
    u = h[:, F:]
    return g / (1.0 + np.exp(-g)) * u


def round_to(v, dtype):
    if dtype == "f32":
        return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
    if dtype in ("bf16", "mxfp8", "mxfp4"):
        return bf16_round(v)
    if dtype == "f64":
        return np.asarray(v, np.float64)
    raise ValueError(dtype)


def expert_mlp(X, W1e, W2e, dtype):
    """One expert's SwiGLU MLP on rows X (float64 values of the stored rows).

    dtype "f32"/"bf16": h = X.W1e (float64), a = swiglu(h) stored in dtype,
    y = a.W2e stored in dtype.
    dtype "mxfp8" / "mxfp4": X, W1e (per column, along H), a (after bf16
    rounding, along F) and W2e (per column, along F) are MX-quantized (E4M3 /
    E2M1 elements) and dequantized exactly before each float64 product; y is
    stored as bf16.
    Returns (y, a_stored) with a_stored the activations as stored before GEMM2
    (bf16 values for the MX types, before their quantization).
    """
    X = np.asarray(X, np.float64)
    W1e = np.asarray(W1e, np.float64)
    W2e = np.asarray(W2e, np.float64)
    F = W2e.shape[0]
    if dtype in ("mxfp8", "mxfp4"):
        quant, dequant = ((mx_quantize_rows, mx_dequantize_rows) if dtype == "mxfp8"
                          else (mx4_quantize_rows, mx4_dequantize_rows))
        Xq = dequant(*quant(X))
        W1q = dequant(*quant(W1e.T)).T
        h = Xq @ W1q
        a = bf16_round(swiglu(h, F))
        aq = dequant(*quant(a))
        W2q = dequant(*quant(W2e.T)).T
        y = bf16_round(aq @ W2q)
        return y, a
    h = X @ W1e
    a = round_to(swiglu(h, F), dtype)
    y = round_to(a @ W2e, dtype)
    return y, a


def grouped_mlp(x_perm, offsets, W1, W2, dtype):
    """Grouped MLP over the expert-ordered rows (bpdata article, "Optimization
    1: Grouped GEMM": every expert's matmuls use its actual token count and only
    valid regions are computed).  Rows [offsets[e], offsets[e+1]) go through
    expert e's MLP; empty experts produce nothing.  W1[e], W2[e] may be any
    indexable sequence of per-expert matrices.  Returns (y_perm, a)."""
    x_perm = np.asarray(x_perm, np.float64)
    N = int(offsets[-1])
    H = x_perm.shape[1] if x_perm.ndim == 2 else 0
    y = np.zeros((N, H), np.float64)
    a_all = None
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ye, ae = expert_mlp(x_perm[lo:hi], W1[e], W2[e], dtype)
        if a_all is None:
            a_all = np.zeros((N, ae.shape[1]), np.float64)
        y[lo:hi] = ye
        a_all[lo:hi] = ae
    return y, a_all


# ---------------------------------------------------------------------------
# Unpermute + probability-weighted combine
# ---------------------------------------------------------------------------

def combine(y_perm, slot_to_row, probs, out_dtype):
    """out[t] = sum over k (in k order) of probs[t,k] * y_perm[slot_to_row[t,k]]
    for the slots with a row; tokens without one get a zero row.  This restores
    the original token order (bpdata article, layer figure: "combine restores
    token order")."""
    y_perm = np.asarray(y_perm, np.float64)
    s2r = np.asarray(slot_to_row)
    p = np.asarray(probs, np.float64)
    T, K = s2r.shape
    H = y_perm.shape[1]
    out = np.zeros((T, H), np.float64)
    for k in range(K):
        r = s2r[:, k]
        ok = r >= 0
        out[ok] += p[ok, k][:, None] * y_perm[r[ok]]
    return round_to(out, out_dtype)


# ---------------------------------------------------------------------------
# Backward of the routing steps (the gradients of route, permute and combine;
# the pages' router work spans forward and backward kernels)
# ---------------------------------------------------------------------------

def combine_backward(dout, y_perm, slot_to_row, probs, out_dtype):
    """Gradients of out[t] = sum_k probs[t,k] * y_perm[slot_to_row[t,k]]:
    d_y_perm[r] = probs[t,k] * dout[t] for the row r of slot (t,k), rounded to
    out_dtype; d_probs[t,k] = <dout[t], y_perm[r]> (fp32), 0 without a row.
    Returns (d_y_perm over rows [0, N), d_probs); N = the rows in use."""
    dout = np.asarray(dout, np.float64)
    y_perm = np.asarray(y_perm, np.float64)
    s2r = np.asarray(slot_to_row)
    p = np.asarray(probs, np.float64)
    T, K = s2r.shape
    N = int(s2r.max()) + 1 if (s2r >= 0).any() else 0
    dy = np.zeros((N, dout.shape[1]), np.float64)
    dp = np.zeros((T, K), np.float64)
    for k in range(K):
        r = s2r[:, k]
        ok = r >= 0
        dy[r[ok]] = p[ok, k][:, None] * dout[ok]
        dp[ok, k] = np.einsum("th,th->t", dout[ok], y_perm[r[ok]])
    return round_to(dy, out_dtype), dp.astype(np.float32)


def permute_backward(d_x_perm, slot_to_row, out_dtype):
    """Gradient of x_perm[r] = x[t] for the row r of each slot (t,k):
    d_x[t] = sum over the token's slots with a row (k order) of d_x_perm[r]."""
    d = np.asarray(d_x_perm, np.float64)
    s2r = np.asarray(slot_to_row)
    T, K = s2r.shape
    out = np.zeros((T, d.shape[1]), np.float64)
    for k in range(K):
        r = s2r[:, k]
        ok = r >= 0
        out[ok] += d[r[ok]]
    return round_to(out, out_dtype)


def route_backward(ids, d_probs, score="softmax", probs=None, logits=None, score_bias=None, scale=1.0):
    """Gradient of the probabilities with respect to the selected keys, for a
    fixed selection (the choice itself is piecewise constant in the logits):
    d_z[t,k] = dL/dz at expert ids[t,k], where z = logit (+ score_bias, the
    bias that entered the scores: moe_route_topk's bias; none for the
    group-limited route, whose bias only steers the choice).
      softmax over the K selected keys (p given): d_z_k = p_k (g_k - sum_j p_j g_j);
      normalized sigmoid, p_k = scale * s_k / S, s = sigma(z), S = sum_j s_j:
        d_z_k = s_k (1 - s_k) (scale g_k - sum_j g_j p_j) / S.
    Every other logit's gradient is 0.  Slots with id -1 give 0.  fp32."""
    ids = np.asarray(ids).astype(np.int64)
    g = np.asarray(d_probs, np.float64)
    T, K = ids.shape
    ok = ids >= 0
    dz = np.zeros((T, K), np.float64)
    if score == "softmax":
        p = np.where(ok, np.asarray(probs, np.float64), 0.0)
        dz = p * (g - (p * np.where(ok, g, 0.0)).sum(axis=1, keepdims=True))
    elif score == "sigmoid":
        lg = np.asarray(logits, np.float32)
        z = np.take_along_axis(lg, np.where(ok, ids, 0), axis=1)
        if score_bias is not None:
            z = (z + np.asarray(score_bias, np.float32)[np.where(ok, ids, 0)]).astype(np.float32)
        sg = np.where(ok, 1.0 / (1.0 + np.exp(-z.astype(np.float64))), 0.0)
        S = sg.sum(axis=1, keepdims=True)
        Ss = np.where(S > 0, S, 1.0)
        p = scale * sg / Ss
        gp = (np.where(ok, g, 0.0) * p).sum(axis=1, keepdims=True)
        dz = sg * (1.0 - sg) * (scale * g - gp) / Ss
    else:
        raise ValueError(score)
    return np.where(ok, dz, 0.0).astype(np.float32)


def swiglu_backward(h, d_a, F):
    """Gradient of a = silu(g) * u (g = h[:, :F], u = h[:, F:]) with respect to
    h: d_g = d_a * u * silu'(g), silu'(g) = sigma(g) (1 + g (1 - sigma(g))),
    d_u = d_a * silu(g); returns [d_g, d_u]."""
    g = h[:, :F]
    u = h[:, F:]
    sg = 1.0 / (1.0 + np.exp(-g))
    return np.concatenate([d_a * u * sg * (1.0 + g * (1.0 - sg)), d_a * g * sg], axis=1)


def mlp_backward_intermediates(X, dY, W1e, W2e, dtype):
    """One expert's data pass on its rows X with output gradient dY: returns
    (h, d_a, d_h) as the data gradient computes them, with h = X . W1e
    recomputed, d_a = dY . W2e^T and d_h = swiglu'(h, d_a).

    "bf16": h and d_h are stored as bf16 (d_a is not rounded).  "f64": nothing
    is rounded.  "mxfp8": every contraction takes MX (E4M3) operands blocked
    along its own contraction dimension, as the forward's (bpdata article,
    "Optimization 1: Grouped GEMM", MXFP8 block scaling): X and W1e's columns
    along H for h; dY and W2e's rows along H for d_a; h and d_h are bf16."""
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    W1e = np.asarray(W1e, np.float64)
    W2e = np.asarray(W2e, np.float64)
    F = W2e.shape[0]
    if dtype == "mxfp8":
        h = bf16_round(_mx_rows_roundtrip(X) @ _mx_rows_roundtrip(W1e.T).T)
        d_a = _mx_rows_roundtrip(dY) @ _mx_rows_roundtrip(W2e).T
        return h, d_a, bf16_round(swiglu_backward(h, d_a, F))
    rnd = (lambda v: v) if dtype == "f64" else bf16_round
    h = rnd(X @ W1e)
    d_a = dY @ W2e.T
    return h, d_a, rnd(swiglu_backward(h, d_a, F))


def _mx_rows_roundtrip(V):
    """V after row-wise MX (E4M3) quantization along its last axis and exact
    dequantization."""
    return mx_dequantize_rows(*mx_quantize_rows(V))


def grouped_mlp_backward_data(x_perm, offsets, W1, W2, d_y, dtype):
    """Data gradient of the grouped SwiGLU MLP: for each expert's rows,
    d_x = d_h . W1[e]^T with d_h, h as mlp_backward_intermediates computes
    them.  Rounding points of the bf16 path: h and d_h are stored as bf16,
    d_x is bf16; "f64" rounds nothing; "mxfp8": d_h (after its bf16
    rounding) and W1[e]'s rows are MX operands along 2F for d_x, as the
    other two contractions' operands are along H.  Returns d_x over rows
    [0, N)."""
    x_perm = np.asarray(x_perm, np.float64)
    d_y = np.asarray(d_y, np.float64)
    N = int(offsets[-1])
    H = x_perm.shape[1]
    out = np.zeros((N, H), np.float64)
    rnd = (lambda v: v) if dtype == "f64" else bf16_round
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        W1e = np.asarray(W1[e], np.float64)
        _, _, d_h = mlp_backward_intermediates(x_perm[lo:hi], d_y[lo:hi], W1e, W2[e], dtype)
        if dtype == "mxfp8":
            out[lo:hi] = bf16_round(_mx_rows_roundtrip(d_h) @ _mx_rows_roundtrip(W1e).T)
        else:
            out[lo:hi] = rnd(d_h @ W1e.T)
    return out


def weight_gradient_operands(X, dY, W1e, W2e, data_dtype):
    """The four operands of one expert's weight gradient as the weight GEMMs
    take them (before any quantization of their own): the rows X and dY, and
    a = silu(g) u and d_h from the data pass of type data_dtype ("bf16",
    "mxfp8" or "f64"; see mlp_backward_intermediates), a rounded to bf16
    (not rounded for "f64").  Returns (X, a, d_h, dY)."""
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    F = np.asarray(W2e).shape[0]
    h, _, d_h = mlp_backward_intermediates(X, dY, W1e, W2e, data_dtype)
    a = swiglu(h, F)
    return X, (a if data_dtype == "f64" else bf16_round(a)), d_h, dY


def weight_gradient_quantize(V):
    """The MXFP8 operand form of a weight-gradient operand V [m][C] (the rows
    of one expert group): each column is cut into blocks of 32 consecutive
    rows of the group and each block is one MX block (group-aware column-wise
    quantization, mx_quantize_columns_grouped); returns the dequantized values
    [m][C] (exact)."""
    return _mx_columns_roundtrip(V)


def weight_gradient_contract(X, a, d_h, dY, dtype):
    """One expert's weight gradients from its four operands: dW1 = X^T d_h
    [H][2F] and dW2 = a^T dY [F][H], contracted over the expert's rows in
    float64.  "mxfp8": each of the four operands first goes through
    weight_gradient_quantize.  The results are fp32 ("f64": not rounded)."""
    X, a, d_h, dY = (np.asarray(v, np.float64) for v in (X, a, d_h, dY))
    if dtype == "mxfp8":
        X, a, d_h, dY = (weight_gradient_quantize(v) for v in (X, a, d_h, dY))
    out = (lambda v: v) if dtype == "f64" else (lambda v: v.astype(np.float32).astype(np.float64))
    return out(X.T @ d_h), out(a.T @ dY)


def grouped_mlp_backward_weights(x_perm, offsets, W1, W2, d_y, dtype, data_dtype=None):
    """Weight gradient of the grouped SwiGLU MLP: for each expert's rows X,
    dW1[e] = X^T d_h and dW2[e] = a^T d_y (contractions over the expert's own
    rows), with h = X W1[e] recomputed, a = silu(g) u, d_a = d_y W2[e]^T and
    d_h = swiglu'(h, d_a) from the data pass of type data_dtype (default: the
    bf16 one; "f64" for dtype "f64"), the operands taken by
    weight_gradient_contract of type dtype ("bf16", "mxfp8" or "f64").  Empty
    experts get zero gradients.  Returns (dW1 [L][H][2F], dW2 [L][F][H])."""
    x_perm = np.asarray(x_perm, np.float64)
    d_y = np.asarray(d_y, np.float64)
    if data_dtype is None:
        data_dtype = "f64" if dtype == "f64" else "bf16"
    dW1, dW2 = [], []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        ops = weight_gradient_operands(x_perm[lo:hi], d_y[lo:hi], W1[e], W2[e], data_dtype)
        g1, g2 = weight_gradient_contract(*ops, dtype)
        dW1.append(g1)
        dW2.append(g2)
    return np.stack(dW1), np.stack(dW2)


def _mx_columns_roundtrip(V):
    """Values of the rows V [m][C] after column-wise MX quantization in
    32-row blocks (one group) and dequantization."""
    m, C = V.shape
    if m == 0:
        return V
    pb, codes, scales = mx_quantize_columns_grouped(V, np.array([0, m]), pad_rows=32)
    nb = int(pb[-1])
    deq = mx_dequantize_rows(codes.reshape(nb * C, 32), scales.reshape(nb * C, 1))
    return deq.reshape(nb, C, 32).transpose(0, 2, 1).reshape(nb * 32, C)[:m]


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def layer(x, K, W1, W2, dtype, *, w_router=None, logits=None, score="softmax",
          bias=None, mask=None, e0=0, L=None):
    """Route -> count/permute -> grouped MLP -> combine on the CPU.

    x: float64 values of the token rows [T,H]; W1/W2 per expert (float64).
    Either w_router (the projection is computed) or logits is given.
    """
    x = np.asarray(x, np.float64)
    if logits is None:
        logits = router_logits(x, w_router)
    E = logits.shape[1]
    L = E if L is None else L
    ids, probs = route_topk(logits, K, score, bias, mask)
    perm = count_and_permute(ids, e0, L, x, E_global=E)
    y, a = grouped_mlp(perm["x_perm"], perm["offsets"], W1, W2, dtype)
    out_dtype = dtype if dtype in ("f32", "f64") else "bf16"
    out = combine(y, perm["slot_to_row"], probs, out_dtype)
    return {"logits": logits, "ids": ids, "probs": probs, "y_perm": y, "a": a, "out": out, **perm}
