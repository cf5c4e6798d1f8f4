"""AWQ per-linear-layer oracle: plain CPU reference (TEST INFRASTRUCTURE ONLY).

This module is the independent checker for the GPU library.  Only tests,
``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import it.  It shares no code, table or helper with the GPU path.

Sources (the AWQ pages; each function names the passage it follows):
  [CA] compassingai, "AWQ (Activation-aware Weight Quantization)"
  [MR] mudrobot, "【论文笔记】AWQ" (notes on the MLSys 2024 AWQ paper)
  [LQ] laojiahuo2003, "LLM Quantization（大模型量化）：GPTQ、AWQ、SmoothQuant 的核心思路"
  [RC] robocikowo, "AWQ"

Layout follows [CA] "一、AWQ 的核心機制": Y = X·W with X [N x D_in] and
W [D_in x D_out]; the per-input-channel scale multiplies the rows of W
(S·W) and divides the columns of X (X·S⁻¹).

Precision (readings of where the pages are silent):
  * activation magnitudes: float64 column sums, one rounding to float32;
  * scales s = a**alpha: float64 ``pow`` rounded once to float32; channels
    whose magnitude is zero or below the smallest normal float32 get s = 1;
  * the quantiser runs in IEEE float32 exactly as written: product s·w,
    group absmax, Δ = m / qmax (true division), q = round-half-even(W'/Δ)
    clamped to [-qmax, qmax]; an all-zero group has Δ = 0 and q = 0;
  * the search loss is evaluated literally, ||X·S⁻¹·Ŵ' − X·W||², in float64.

Every function here is pinned by tests/test_oracle_*.py against closed forms,
exact rational brute force and invariants the pages state.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "FLT_MIN",
    "act_stats",
    "weight_stats",
    "scales_for_alpha",
    "quantize_group_absmax",
    "dequantize",
    "search_loss",
    "search_layer",
    "argmin_first",
    "quantize_group_clipped",
    "quantize_group_asym",
    "dequantize_asym",
    "clip_search",
    "PACK_ORDER",
    "pack_int4",
    "unpack_int4",
    "round_to_bf16",
    "round_to_f16",
    "w4a16_gemm",
]

FLT_MIN = float(np.finfo(np.float32).tiny)  # 2**-126, smallest normal float32


def act_stats(X: np.ndarray, statistic: str = "mean") -> np.ndarray:
    """Per-input-channel activation magnitude.

    statistic "mean": a_j = mean_n |X[n, j]|.  [CA] "重要通道識別的統計依據":
    activation_scale[j] is the mean of |X_calib[:, j]| over the calibration
    samples; [MR] "搜索最优比例": s_X is the per-channel mean activation
    magnitude.  Reading: accumulate in float64, divide by N, round once to
    float32.

    statistic "max": a_j = max_n |X[n, j]|.  [CA] "重要通道識別的統計依據"
    allows the max in place of the mean, and [CA] "二、縮放因子的搜尋" writes
    s_j = (max|X_j|)^α.  The maximum of float32 values is exact; a NaN in a
    column makes that channel's statistic NaN.
    """
    X = np.asarray(X)
    N = X.shape[0]
    if N == 0:
        raise ValueError("act_stats needs at least one calibration row")
    if statistic == "max":
        return np.abs(X.astype(np.float64)).max(axis=0).astype(np.float32)
    if statistic != "mean":
        raise ValueError("statistic must be 'mean' or 'max'")
    col_sum = np.abs(X.astype(np.float64)).sum(axis=0)
    return (col_sum / np.float64(N)).astype(np.float32)


def weight_stats(W: np.ndarray) -> np.ndarray:
    """Per-input-channel weight magnitude b_j = mean over outputs of |W[j, o]|.

    [LQ] "4.4 怎么做：不是留 FP16，而是「缩放」" divides by (mean|W_j|)^(1−α),
    where W_j holds the weights that input channel j feeds; with W stored
    [D_in x D_out] here, that is row j.  Reading, as for the activation mean:
    float64 sum, divide by D_out, round once to float32.
    """
    W = np.asarray(W)
    if W.shape[1] == 0:
        raise ValueError("weight_stats needs at least one output column")
    row_sum = np.abs(W.astype(np.float64)).sum(axis=1)
    return (row_sum / np.float64(W.shape[1])).astype(np.float32)


def scales_for_alpha(a: np.ndarray, alpha: float, b: np.ndarray | None = None) -> np.ndarray:
    """Candidate per-channel scale s_j(α) = a_j ** α, or a_j ** α / b_j ** (1−α).

    [CA] "縮放因子最佳化的完整流程" step 3 and [MR] "搜索最优比例" (s = s_X^α).
    Reading: α is the caller's float32 grid value; the power is taken in
    float64 (C library ``pow``) and rounded once to float32.  A channel whose
    magnitude is 0 or below FLT_MIN is dead (it contributes nothing
    representable to X·W) and keeps s = 1, which avoids 1/0.

    With a weight statistic b ([LQ] "4.4 怎么做：不是留 FP16，而是「缩放」"):
    s_j = a_j^α / b_j^(1−α), both powers and the quotient in float64 with
    1−α formed exactly in float64, rounded once to float32.  A channel with
    a_j or b_j zero or below FLT_MIN keeps s = 1 (an all-zero weight row
    quantises to zero whatever its scale).
    """
    al = float(np.float32(alpha))
    a = np.asarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.float32)
    flat_a = a.ravel()
    flat_o = out.ravel()
    flat_b = None if b is None else np.asarray(b, dtype=np.float32).ravel()
    for j in range(flat_a.size):
        aj = float(flat_a[j])
        if not (aj >= FLT_MIN):
            flat_o[j] = np.float32(1.0)
        elif flat_b is None:
            flat_o[j] = np.float32(math.pow(aj, al))
        else:
            bj = float(flat_b[j])
            if not (bj >= FLT_MIN):
                flat_o[j] = np.float32(1.0)
            else:
                flat_o[j] = np.float32(math.pow(aj, al) / math.pow(bj, 1.0 - al))
    return out


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Nearest IEEE binary16 value (ties to even), as float32.

    [MR] "通过激活感知缩放保护显著权重" keeps the scaling factors Δ in FP16.
    NumPy's float16 cast rounds to nearest even (including subnormals and
    overflow to inf); the result is exact in float32.
    """
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def quantize_group_absmax(Wp: np.ndarray, bits: int, group: int, f16_steps: bool = False):
    """Symmetric absmax INT-b quantisation per group of ``group`` input rows.

    [CA] "量化數學基礎": per group, step = max|w| / (2^(b-1) - 1),
    w_q = round(w / step) clipped to [-2^(b-1)+1, 2^(b-1)-1].
    Groups run along D_in (the reduction axis): rows [k·g, (k+1)·g) of one
    output column.  Reading: float32 IEEE arithmetic, true division (twice),
    round-half-to-even; an all-zero group gets step 0 and codes 0.

    With ``f16_steps`` the step is stored in FP16: step = fl16(fl32(m/qmax))
    (round to nearest even), and the codes are taken against that stored step.

    Returns (q int8 [D_in x D_out], delta float32 [D_in/g x D_out]).
    """
    Wp = np.asarray(Wp, dtype=np.float32)
    D_in, D_out = Wp.shape
    if D_in % group:
        raise ValueError("D_in must be a multiple of the group size")
    qmax = np.float32(2 ** (bits - 1) - 1)
    G = D_in // group
    m = np.abs(Wp).reshape(G, group, D_out).max(axis=1)          # float32, exact
    delta = (m / qmax).astype(np.float32)                           # IEEE float32 division
    if f16_steps:
        delta = round_to_f16(delta)
    dfull = np.repeat(delta, group, axis=0)
    safe = np.where(dfull > 0, dfull, np.float32(1.0))
    ratio = (Wp / safe).astype(np.float32)                          # IEEE float32 division
    q = np.rint(ratio)                                              # half to even
    q = np.where(dfull > 0, q, np.float32(0.0))
    q = np.clip(q, -qmax, qmax)
    return q.astype(np.int8), delta


def quantize_group_asym(Wp: np.ndarray, bits: int, group: int, f16_steps: bool = False):
    """Asymmetric (zero-point) INT-b quantisation per group of ``group`` input rows.

    [CA] "三、量化方案細節" allows symmetric or asymmetric quantisation and
    gives only the symmetric formulas.  Reading (min-max affine with the
    range widened to contain zero, so that 0 stays exactly representable):
      lo = min(min w', 0), hi = max(max w', 0)   over the group (float32)
      step = fl32(fl32(hi − lo) / (2^b − 1))     (IEEE division)
      z    = rint(fl32(−lo / step))              in [0, 2^b − 1]
      q    = clamp(rint(fl32(w' / step)) + z, 0, 2^b − 1)
    and ŵ = (q − z)·step.  An all-zero group gets step 0, z 0 and q 0.
    ``f16_steps`` rounds the step to FP16 before z and q are taken.
    Returns (q uint8 [D_in x D_out], step float32 [G x D_out], z uint8 [G x D_out]).
    """
    Wp = np.asarray(Wp, dtype=np.float32)
    D_in, D_out = Wp.shape
    if D_in % group:
        raise ValueError("D_in must be a multiple of the group size")
    qu = np.float32(2 ** bits - 1)
    G = D_in // group
    blocks = Wp.reshape(G, group, D_out)
    lo = np.minimum(blocks.min(axis=1), np.float32(0.0))
    hi = np.maximum(blocks.max(axis=1), np.float32(0.0))
    rng = (hi - lo).astype(np.float32)                                # float32 difference
    step = (rng / qu).astype(np.float32)                                # IEEE float32 division
    if f16_steps:
        step = round_to_f16(step)
    safe = np.where(step > 0, step, np.float32(1.0))
    z = np.where(step > 0, np.rint((-lo / safe).astype(np.float32)), np.float32(0.0))
    z = np.clip(z, np.float32(0.0), qu)
    sfull = np.repeat(safe, group, axis=0)
    zfull = np.repeat(z, group, axis=0)
    q = np.rint((Wp / sfull).astype(np.float32)) + zfull
    q = np.where(np.repeat(step, group, axis=0) > 0, q, np.float32(0.0))
    q = np.clip(q, np.float32(0.0), qu)
    return q.astype(np.uint8), step, z.astype(np.uint8)


def dequantize_asym(q: np.ndarray, step: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    """ŵ = (q − z)·step in float64 (exact)."""
    zf = np.repeat(np.asarray(z, dtype=np.float64), group, axis=0)
    return (q.astype(np.float64) - zf) * np.repeat(step.astype(np.float64), group, axis=0)


def dequantize(q: np.ndarray, delta: np.ndarray, group: int) -> np.ndarray:
    """ŵ = w_q · step in float64 (exact: |q| < 2^7, step is float32).

    [CA] "量化數學基礎" step 3.
    """
    return q.astype(np.float64) * np.repeat(delta.astype(np.float64), group, axis=0)


def search_loss(X: np.ndarray, W: np.ndarray, s: np.ndarray, What: np.ndarray,
                Y: np.ndarray | None = None) -> float:
    """L = || (X·S⁻¹)·Ŵ' − X·W ||² (sum of squares), float64.

    [CA] "縮放因子最佳化的完整流程" step 4c gives this squared norm; [MR]
    "搜索最优比例" writes the same objective unsquared (same argmin).  Reading:
    report the plain sum of squares over all N x D_out outputs.
    ``Y`` may carry a precomputed X·W (float64).
    """
    X64 = np.asarray(X, dtype=np.float64)
    if Y is None:
        Y = X64 @ np.asarray(W, dtype=np.float64)
    Xs = X64 / np.asarray(s, dtype=np.float64)[None, :]
    E = Xs @ What - Y
    return float(np.sum(E * E))


def argmin_first(losses) -> int:
    """α* = argmin L; exact ties go to the first (smallest) grid index.

    [CA] "縮放因子最佳化的完整流程" step 5.
    """
    best = 0
    for k in range(1, len(losses)):
        if losses[k] < losses[best]:
            best = k
    return best


def search_layer(X: np.ndarray, W: np.ndarray, alphas, bits: int = 4, group: int = 128,
                 *, keep_all: bool = False, a: np.ndarray | None = None,
                 b: np.ndarray | None = None, asym: bool = False, f16_steps: bool = False) -> dict:
    """The per-layer AWQ grid search, steps in the pages' order.

    [CA] "縮放因子最佳化的完整流程": statistics, candidate scales s(α)=a^α,
    W' = diag(s)·W, per-group quantisation to Ŵ', loss
    ||X·S⁻¹·Ŵ' − X·W||², α* = argmin, record s* = a^α*;
    [CA] "推論時的等效實現": the kept weights are Quantize(diag(s*)·W) with s*
    as metadata.  [MR] "搜索最优比例" states the same search.

    ``a`` overrides the statistic (e.g. the max of :func:`act_stats`); ``b``
    (e.g. :func:`weight_stats`) switches to the weight-term candidates of
    [LQ] "4.4 怎么做：不是留 FP16，而是「缩放」" (see :func:`scales_for_alpha`).

    ``asym`` quantises with :func:`quantize_group_asym` (codes uint8 in
    [0, 2^b − 1] and zero points, dequantised as (q − z)·step).
    ``f16_steps`` stores the steps in FP16 ([MR] "通过激活感知缩放保护显著权重"),
    with codes taken against the stored step (see :func:`quantize_group_absmax`).

    Returns a dict with a, losses (float64 [n_alpha]), best, s_best, codes
    (int8 [D_in x D_out], uint8 with ``asym``) and scales (float32
    [D_in/g x D_out]), plus zeros with ``asym``; with ``keep_all`` also per-α
    lists s_all, codes_all, scales_all (and zeros_all).
    """
    X = np.asarray(X, dtype=np.float32)
    W = np.asarray(W, dtype=np.float32)
    if a is None:
        a = act_stats(X)
    Y = X.astype(np.float64) @ W.astype(np.float64)
    losses = []
    s_all, q_all, d_all, z_all = [], [], [], []
    for alpha in np.asarray(alphas, dtype=np.float32):
        s = scales_for_alpha(a, alpha, b)
        Wp = (s[:, None] * W).astype(np.float32)                     # float32 product
        if asym:
            q, delta, z = quantize_group_asym(Wp, bits, group, f16_steps)
            What = dequantize_asym(q, delta, z, group)
            z_all.append(z)
        else:
            q, delta = quantize_group_absmax(Wp, bits, group, f16_steps)
            What = dequantize(q, delta, group)
        losses.append(search_loss(X, W, s, What, Y))
        s_all.append(s)
        q_all.append(q)
        d_all.append(delta)
    best = argmin_first(losses)
    out = {
        "a": a,
        "losses": np.asarray(losses, dtype=np.float64),
        "best": best,
        "s_best": s_all[best],
        "codes": q_all[best],
        "scales": d_all[best],
    }
    if asym:
        out["zeros"] = z_all[best]
    if keep_all:
        out.update(s_all=s_all, codes_all=q_all, scales_all=d_all)
        if asym:
            out["zeros_all"] = z_all
    return out


# Weight clipping -------------------------------------------------------------

def quantize_group_clipped(Wp: np.ndarray, bits: int, group: int, ratio: float):
    """Absmax quantiser with the group maximum clipped to ratio · max.

    Reading of [MR] "搜索最优比例" (weight clipping to lower the quantisation
    MSE): per group, m = max|w'| (float32, exact), the clip threshold
    m_r = fl32(ratio · m), step = fl32(m_r / qmax) (IEEE division),
    q = round-half-even(w' / step) clamped to [-qmax, qmax], so weights
    beyond the threshold saturate.  ratio = 1 is :func:`quantize_group_absmax`.
    An all-zero group gets step 0 and codes 0.
    """
    Wp = np.asarray(Wp, dtype=np.float32)
    D_in, D_out = Wp.shape
    if D_in % group:
        raise ValueError("D_in must be a multiple of the group size")
    qmax = np.float32(2 ** (bits - 1) - 1)
    G = D_in // group
    m = np.abs(Wp).reshape(G, group, D_out).max(axis=1)
    mr = (np.float32(ratio) * m).astype(np.float32)                   # float32 product
    delta = (mr / qmax).astype(np.float32)                              # IEEE float32 division
    dfull = np.repeat(delta, group, axis=0)
    safe = np.where(dfull > 0, dfull, np.float32(1.0))
    q = np.rint((Wp / safe).astype(np.float32))
    q = np.where(dfull > 0, q, np.float32(0.0))
    q = np.clip(q, -qmax, qmax)
    return q.astype(np.int8), delta


def clip_search(X: np.ndarray, W: np.ndarray, s: np.ndarray, ratios, bits: int = 4,
                group: int = 128) -> dict:
    """Per-group clip-ratio search after the scale search.

    Reading of [MR] "搜索最优比例" (one sentence: weight clipping is applied to
    minimise the quantisation MSE): with s fixed (s* of the α search), every
    group of every output column takes the first ratio of the grid that
    minimises the group's own contribution to the layer's output error,
      E_g,o(r) = sum_n ( sum_{k in g} X[n, k] · (q_k·step_r / s_k − W[k, o]) )²,
    i.e. the loss of [CA] "縮放因子最佳化的完整流程" step 4c restricted to one
    group (cross-group terms left out, so the groups are chosen
    independently).  Float64 loss, float32 quantiser (as in the α search).

    Returns ratio_idx (int32 [G x D_out]), errors (float64 [n_r x G x D_out]),
    codes (int8 [D_in x D_out]) and scales (float32 [G x D_out]) at the
    chosen ratios.
    """
    X = np.asarray(X, dtype=np.float32)
    W = np.asarray(W, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    D_in, D_out = W.shape
    G = D_in // group
    Wp = (s[:, None] * W).astype(np.float32)
    X64 = X.astype(np.float64)
    s64 = s.astype(np.float64)
    W64 = W.astype(np.float64)
    ratios = np.asarray(ratios, dtype=np.float32)
    errors = np.zeros((len(ratios), G, D_out), np.float64)
    q_all, d_all = [], []
    for k, r in enumerate(ratios):
        q, delta = quantize_group_clipped(Wp, bits, group, float(r))
        What = dequantize(q, delta, group)                               # float64, exact
        D = What / s64[:, None] - W64                                    # S⁻¹·Ŵ' − W
        for g in range(G):
            rows = slice(g * group, (g + 1) * group)
            E = X64[:, rows] @ D[rows, :]
            errors[k, g, :] = np.sum(E * E, axis=0)
        q_all.append(q)
        d_all.append(delta)
    ratio_idx = np.zeros((G, D_out), np.int32)
    for g in range(G):
        for o in range(D_out):
            ratio_idx[g, o] = argmin_first(errors[:, g, o])
    codes = np.zeros((D_in, D_out), np.int8)
    scales = np.zeros((G, D_out), np.float32)
    for g in range(G):
        rows = slice(g * group, (g + 1) * group)
        for k in range(len(ratios)):
            cols = ratio_idx[g] == k
            codes[rows, cols] = q_all[k][rows, cols]
            scales[g, cols] = d_all[k][g, cols]
    return {"ratio_idx": ratio_idx, "errors": errors, "codes": codes, "scales": scales}


# Packing -------------------------------------------------------------------

#: [MR] "SIMD 感知权重打包": on GPUs every 8 weights go into 32 bits in the
#: order w0, w2, w4, w6, w1, w3, w5, w7.  Reading: nibble slot i (bits
#: 4i..4i+3, least significant first) holds input row PACK_ORDER[i] of the
#: 8-row block, stored as offset binary q + 8.
PACK_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def pack_int4(q: np.ndarray, offset: int = 8) -> np.ndarray:
    """Pack int codes [D_in x D_out] (|q| <= 7) into uint32 [D_in/8 x D_out].

    word[kw, o] = sum_i (q[8·kw + PACK_ORDER[i], o] + offset) << (4·i):
    offset 8 for signed symmetric codes, 0 for the unsigned codes of the
    zero-point quantiser.  [MR] "SIMD 感知权重打包"; [RC] "Komponenty"
    (4-bit integers with a per-group scale).
    """
    q = np.asarray(q)
    D_in, D_out = q.shape
    if D_in % 8:
        raise ValueError("D_in must be a multiple of 8 to pack")
    nib = (q.astype(np.int64) + offset).reshape(D_in // 8, 8, D_out)
    if nib.size and (nib.min() < 0 or nib.max() > 15):
        raise ValueError("codes out of 4-bit range")
    word = np.zeros((D_in // 8, D_out), dtype=np.uint64)
    for slot, row in enumerate(PACK_ORDER):
        word |= nib[:, row, :].astype(np.uint64) << np.uint64(4 * slot)
    return word.astype(np.uint32)


def unpack_int4(words: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4` -> int8 codes [8·rows x D_out]."""
    words = np.asarray(words, dtype=np.uint32)
    R, D_out = words.shape
    q = np.zeros((R, 8, D_out), dtype=np.int16)
    for slot, row in enumerate(PACK_ORDER):
        q[:, row, :] = ((words >> np.uint32(4 * slot)) & np.uint32(0xF)).astype(np.int16) - 8
    return q.reshape(R * 8, D_out).astype(np.int8)


# Inference GEMM --------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32.

    Written from the bfloat16 format definition (1 sign, 8 exponent, 7
    fraction bits): keep the top 16 bits of the float32 pattern after adding
    half an ulp of the kept part with ties to the even kept pattern.  Finite
    inputs only.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    keep = bits >> np.uint64(16)
    rest = bits & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    keep = keep + up.astype(np.uint64)
    out = (keep << np.uint64(16)).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def w4a16_gemm(X: np.ndarray, words: np.ndarray, scales: np.ndarray, group: int,
               inv_s: np.ndarray | None = None, zeros: np.ndarray | None = None) -> np.ndarray:
    """Y = (X · diag(1/s*)) · Dequant(W_q), float64.

    [CA] "推論時的等效實現": online, Y = (X·diag(1/s*))·Dequant(W_quantized); the
    activation scaling may be fused into the kernel.  Reading: when ``inv_s``
    is given, the scaled activations are float32 X·inv_s rounded once to
    bfloat16 (the 16-bit activation format of W4A16); otherwise X is used
    as given.  Dequant(W_q)[j, o] = q[j, o] · scales[j // group, o]; with
    ``zeros`` (zero-point codes, packed with offset 0) it is
    (n[j, o] − z[j // group, o]) · scales[j // group, o] for the stored nibble n.
    """
    X = np.asarray(X, dtype=np.float32)
    if inv_s is not None:
        Xe = round_to_bf16((X * np.asarray(inv_s, dtype=np.float32)[None, :]).astype(np.float32))
    else:
        Xe = X
    q = unpack_int4(words)
    if zeros is None:
        Wd = dequantize(q, np.asarray(scales, dtype=np.float32), group)
    else:
        # zero-point codes: the nibble itself is q, dequantised as (q − z)·step
        Wd = dequantize_asym(q.astype(np.int64) + 8, np.asarray(scales, dtype=np.float32), zeros, group)
    return Xe.astype(np.float64) @ Wd
