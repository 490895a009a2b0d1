"""Plain CPU reference of the AWQ W4A16 group-quantized linear layer (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``weight_only_int4_awq_amd``) never imports, calls or links it, and this module
imports nothing from the product path.  It is deliberately slow and literal:
every function follows one step of the method in the order the sources give it,
with float64 arithmetic and no blocking, fusion or reordering.

Sources (web pages about AWQ; cited by title and section):

* [jsqmd] "从Java转行大模型应用，大模型量化实现，AWQ 与 GPTQ 算法" (jsqmd.com),
  section 二.1 "核心原理": (2) weight importance from the per-channel mean absolute
  activation E[|X_j|]; (3) channel-scaling protection: salient input channels
  of W are multiplied by s and the activation is divided by s at inference so
  the product is unchanged, and s is chosen to minimise the output error of the
  quantized layer.  Section 二.2 (pseudocode) contributes only the statistic
  mean(|activation|, dim=0); its symmetric per-row rule is not followed.
  Section 五.3 warns that scale factors can overflow and asks for a clip.
* [csdn] "LLM-AWQ学术影响力：激活感知量化被引用文献的研究主题分析" (CSDN blog),
  section "量化流程优化": search-and-dump of scales, then real quantization with
  4-bit weights and group size 128 into a packed checkpoint.
* [bjdmk] "大模型量化技术极速优化：开启AI效能革命的显存优化之道" (bjdmk.com.cn),
  section "量化实施四步法 / 量化参数配置": 4-bit weights, group size 128 by
  default, zero point enabled, GEMV mode for batch-1 and GEMM mode for long
  inputs.
* [zeeklog] "LLM-AWQ多模态基准…" (zeeklog.com): W4A16 (4-bit weights, 16-bit
  activations) kernels.

The pages leave the scale parametrisation, the alpha grid, the zero-point
arithmetic, the rounding mode and the nibble layout open.  The readings used
here (all listed with their reasons in the design notes of this repository):

* s = a ** alpha with a = mean|x| per input channel and alpha_i = i / n_grid,
  i = 0 .. n_grid-1 (20 points in [0, 1) by default); s is rounded to fp16
  after a lower clamp of 2**-14 (the clip the jsqmd page asks for).
* W' = fp16_rn(W * s); per (row, group of g along K): min-max range
  r = max(mx - mn, 2**-16), step D = fp16_rn(r / 15),
  zero z = clamp(RNE(-mn / D), 0, 15), code q = clamp(RNE(W' / D) + z, 0, 15);
  dequantised value (q - z) * D.  RNE = round half to even.
* search loss L_i = sum_{t,n} (sum_k ((q - z) D / s_ik - W_nk) X_tk)^2;
  chosen index = first minimum over finite losses (-1 if none is finite).
* packed layout v1: qweight[n][k/8] holds q_nk in bits 4*(k%8)..+3;
  scales[n][j] = D_nj (fp16); qzeros[n][j/8] holds z_nj in bits 4*(j%8)..+3,
  each row padded to whole 32-bit words with zero nibbles.

Non-finite handling (a reading; the pages are silent): a group whose W'
contains inf or NaN is "non-finite"; pack writes q = 0, z = 0 and the fp16
NaN 0x7E00 as its scale and counts it.  In the search such an alpha gets an
infinite loss.

Mixed-precision baseline (a reading; the pages give the ratio only): the
protected channels are the round(frac * K) largest a_k (ties to the lower
index); the rest of W is quantized with the same RTN quantizer (s = 1, groups
over all channels) and the protected columns keep their fp16 values.

Parity status of each function is stated in its docstring ("pinned by ..." or
"parity unpinned").
"""
from __future__ import annotations

import numpy as np

F16_NAN_BITS = 0x7E00
MIN_NORMAL_F16 = 2.0 ** -14      # lower clamp on s
MIN_RANGE = 2.0 ** -16           # floor on a group's range (degenerate groups)


# ----------------------------------------------------------------------------
# rounding helpers


def fp16_rn(v) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of float64 values (subnormals kept,
    overflow to +-inf).  numpy's float64 -> float16 conversion rounds once,
    directly from the float64 bits.

    Pinned by tests/test_oracle_pins.py::test_fp16_rn_matches_exact_rounding
    (exact rational rounding of random and tie values).
    """
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def rne(v) -> np.ndarray:
    """Round half to even to an integer (float64 in, float64 out)."""
    return np.rint(np.asarray(v, dtype=np.float64))


# ----------------------------------------------------------------------------
# a1: activation statistic  ([jsqmd] 二.1(2), 二.2 first statement)


def calib_stats(x16: np.ndarray) -> np.ndarray:
    """Per-input-channel mean absolute activation a_k = (1/M) sum_t |x_tk|.

    x16: fp16 [M, K] calibration tokens.  Returns float64 [K].
    Every |fp16| is a multiple of 2**-24 below 2**16, so for M <= 8192 the
    float64 sum is exact in any order and a_k is the exact mean rounded once.

    Pinned by test_calib_stats_exact_integer_sum and
    test_calib_stats_closed_form.
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    m = x.shape[0]
    return np.abs(x).sum(axis=0) / float(m)


# ----------------------------------------------------------------------------
# a2: scale candidates  (s = mean|x|^alpha over an alpha grid; clip of [jsqmd] 五.3)


def alpha_grid(n_grid: int = 20) -> np.ndarray:
    """alpha_i = i / n_grid for i = 0 .. n_grid-1 (n_grid points in [0, 1))."""
    return np.array([float(i) / float(n_grid) for i in range(n_grid)], dtype=np.float64)


def scale_candidate(a: np.ndarray, alpha: float) -> np.ndarray:
    """s_k = fp16_rn(max(a_k ** alpha, 2**-14)); a NaN power stays NaN.

    0 ** 0 = 1 and x ** 0 = 1 for every x (C pow semantics), so alpha = 0
    gives s = 1 everywhere: plain round-to-nearest quantization.
    """
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(all="ignore"):
        p = np.power(a, np.float64(alpha))
    clamped = np.where(np.isnan(p), p, np.maximum(p, MIN_NORMAL_F16))
    return fp16_rn(clamped)


# ----------------------------------------------------------------------------
# a3 building blocks: asymmetric INT4 group quantization along K
# ([bjdmk] 量化参数配置: 4 bit, group 128, zero point; [csdn] 量化流程优化)


def scale_weights(w16: np.ndarray, s16: np.ndarray | None) -> np.ndarray:
    """W'_nk = fp16_rn(W_nk * s_k) (the fp16 x fp16 product is exact in float64).

    s16 = None means s = 1 (W' = W).
    """
    w = np.asarray(w16, dtype=np.float16)
    if s16 is None:
        return w.copy()
    with np.errstate(over="ignore", invalid="ignore"):
        return fp16_rn(w.astype(np.float64) * np.asarray(s16, np.float16).astype(np.float64)[None, :])


def group_view(a: np.ndarray, g: int) -> np.ndarray:
    """[N, K] -> [N, K/g, g] (group j covers k in [j*g, (j+1)*g))."""
    n, k = a.shape
    assert k % g == 0
    return a.reshape(n, k // g, g)


def group_params(wp16: np.ndarray, g: int, max_int: int = 15):
    """Per (row, group): step D16 (fp16), zero z (int, 0..max_int) and a flag
    for groups holding a non-finite W'.  max_int = 2**w_bit - 1 (15 for the
    4-bit weights of the method; 7 and 255 for the 3- and 8-bit variants).

    mx, mn = max, min of W' over the group (the range is not forced to hold 0);
    r = max(mx - mn, 2**-16) (exact in float64); D16 = fp16_rn(r / max_int);
    z = clamp(RNE(-mn / D16), 0, max_int).  Non-finite groups get D16 = NaN, z = 0.

    Pinned by test_codes_brute_force_all_levels, test_known_answer_groups,
    test_invariants.
    """
    wg = group_view(np.asarray(wp16, np.float16).astype(np.float64), g)
    bad = ~np.isfinite(wg).all(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        mx = wg.max(axis=2)
        mn = wg.min(axis=2)
        r = np.maximum(mx - mn, MIN_RANGE)
        d16 = fp16_rn(r / float(max_int))
        d = d16.astype(np.float64)
        z = np.clip(rne(-mn / d), 0.0, float(max_int))
    d16 = np.where(bad, np.float16(np.nan), d16)
    z = np.where(bad, 0.0, z).astype(np.int64)
    return d16, z, bad


def quantize_codes(wp16: np.ndarray, d16: np.ndarray, z: np.ndarray, g: int,
                   bad: np.ndarray | None = None, max_int: int = 15) -> np.ndarray:
    """q_nk = clamp(RNE(W'_nk / D16_nj) + z_nj, 0, max_int) (quotient in
    float64, which is exact-then-rounded for fp16 operands); non-finite groups
    get q = 0.
    """
    wg = group_view(np.asarray(wp16, np.float16).astype(np.float64), g)
    d = np.asarray(d16, np.float16).astype(np.float64)[:, :, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.clip(rne(wg / d) + np.asarray(z, np.float64)[:, :, None], 0.0, float(max_int))
    if bad is not None:
        q = np.where(bad[:, :, None], 0.0, q)
    q = np.nan_to_num(q, nan=0.0)
    n, ng, _ = wg.shape
    return q.astype(np.int64).reshape(n, ng * g)


def dequantize(q: np.ndarray, z: np.ndarray, d16: np.ndarray, g: int) -> np.ndarray:
    """(q - z) * D16 in float64 (exact: a small integer times an fp16)."""
    n, k = q.shape
    qg = q.reshape(n, k // g, g).astype(np.float64)
    d = np.asarray(d16, np.float16).astype(np.float64)[:, :, None]
    return ((qg - np.asarray(z, np.float64)[:, :, None]) * d).reshape(n, k)


def fake_quantize(w16: np.ndarray, s16: np.ndarray | None, g: int, max_int: int = 15):
    """Scale, quantize and dequantize: returns (W'16, q, z, D16, bad, deq)."""
    wp = scale_weights(w16, s16)
    d16, z, bad = group_params(wp, g, max_int)
    q = quantize_codes(wp, d16, z, g, bad, max_int)
    deq = dequantize(q, z, d16, g)
    return wp, q, z, d16, bad, deq


# ----------------------------------------------------------------------------
# a3/a4: the search  ([jsqmd] 二.1(3): minimise the output error of the scaled,
# quantized layer; the objective ||Q(W diag(s)) (diag(s)^-1 X) - W X||^2)


def search_loss(w16: np.ndarray, x16: np.ndarray, s16: np.ndarray, g: int,
                max_int: int = 15) -> float:
    """L = sum_{t,n} (sum_k ((q - z) D16 / s_k - W_nk) X_tk)^2 in float64.

    Infinite or NaN when a group of W' is non-finite.

    Pinned by test_loss_matches_exact_fractions (tiny shapes, exact rational
    evaluation) and test_alpha0_is_plain_rtn.
    """
    w = np.asarray(w16, np.float16).astype(np.float64)
    x = np.asarray(x16, np.float16).astype(np.float64)
    s = np.asarray(s16, np.float16).astype(np.float64)
    wp, q, z, d16, bad, deq = fake_quantize(w16, s16, g, max_int)
    if bad.any():
        return float("inf")
    dw = deq / s[None, :] - w                  # [N, K]
    e = dw @ x.T                               # [N, M]
    return float(np.sum(e * e))


def select_best(losses: np.ndarray) -> int:
    """Index of the first minimum over finite losses; -1 if none is finite."""
    best, best_v = -1, None
    for i, v in enumerate(np.asarray(losses, np.float64)):
        if not np.isfinite(v):
            continue
        if best_v is None or v < best_v:
            best, best_v = i, v
    return best


def search_scale(w16: np.ndarray, x16: np.ndarray, a: np.ndarray, g: int = 128,
                 n_grid: int = 20, w_bit: int = 4):
    """Grid search of s = a^alpha.  Returns (best, s16, inv_s16, losses).

    s16 = candidate at the chosen alpha; inv_s16 = fp16_rn(1 / s16) (float64
    quotient, one fp16 rounding).  When no loss is finite: best = -1 and
    s16 = inv_s16 = 1.

    Parity unpinned against any published search result (the pages print no
    numbers for it); its parts are pinned as stated above, and the property
    L[best] <= L[0] is checked.
    """
    alphas = alpha_grid(n_grid)
    max_int = (1 << w_bit) - 1
    losses = np.array([search_loss(w16, x16, scale_candidate(a, al), g, max_int) for al in alphas])
    best = select_best(losses)
    k = np.asarray(w16).shape[1]
    if best < 0:
        s16 = np.ones(k, np.float16)
    else:
        s16 = scale_candidate(a, alphas[best])
    with np.errstate(divide="ignore"):
        inv = fp16_rn(1.0 / s16.astype(np.float64))
    return best, s16, inv, losses


# ----------------------------------------------------------------------------
# shared scale over projections that read one input, with 1/s folded into the
# operation that produces that input ([bjdmk] 融合模块优化: merging steps into
# one operation; [jsqmd] 二.1 (3): the activation is divided by s at inference)


def fold_inv_scale(v16: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """Per-channel weight of the elementwise operation that produces a linear's
    input (for example a normalisation weight), with the linear's division by s
    folded in: fp16_rn(v_k / s_k), the float64 quotient of two fp16 values
    rounded once to fp16.  The linear then runs with inv_s16 = None on the
    activations that operation produces.

    A shared s for several projections of one input is search_scale on their
    weights stacked along N (the loss sums over all their output rows).

    Pinned by: s = 1 (identity), s a power of two (exact scaling), the exact
    rational quotient rounded once for random pairs, and the joint loss equal
    to the sum of the stacked projections' losses (tests/test_oracle_pins.py).
    """
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return fp16_rn(np.asarray(v16, np.float16).astype(np.float64) /
                       np.asarray(s16, np.float16).astype(np.float64))


def fold_inv_scale_rows(w16: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """The same fold when the operation producing a linear's input is itself a
    linear whose output channel j feeds input channel j (in a decoder block
    the up projection, whose output multiplies the activated gate output and
    is the down projection's input): row j of its weight [N, K] becomes
    fp16_rn(W_jk / s_j), each the float64 quotient of two fp16 values rounded
    once.  The downstream linear then runs with inv_s16 = None.

    Pinned by: s = 1 (identity), s a power of two (exact scaling), the exact
    rational quotient rounded once for random pairs, and rows equal to
    fold_inv_scale of each row with its s_j repeated (tests/test_oracle_pins.py).
    """
    w = np.asarray(w16, np.float16).astype(np.float64)
    s = np.asarray(s16, np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return fp16_rn(w / s[:, None])


# ----------------------------------------------------------------------------
# a5: real quantization and packing (layout v1)  ([csdn] 量化流程优化)


def pack_int4(w16: np.ndarray, s16: np.ndarray | None, g: int = 128):
    """Returns (qweight u32 [N, K/8], scales f16 [N, K/g],
    qzeros u32 [N, ceil(K/(8g))], n_nonfinite_groups).

    Pinned by test_pack_roundtrip and the known-answer groups.
    """
    wp, q, z, d16, bad, _ = fake_quantize(w16, s16, g)
    n, k = q.shape
    assert k % 8 == 0
    qw = np.zeros((n, k // 8), dtype=np.uint64)
    for i in range(8):
        qw |= (q[:, i::8].astype(np.uint64) & 0xF) << np.uint64(4 * i)
    ng = k // g
    nzw = (ng + 7) // 8
    zpad = np.zeros((n, nzw * 8), dtype=np.uint64)
    zpad[:, :ng] = z
    qz = np.zeros((n, nzw), dtype=np.uint64)
    for i in range(8):
        qz |= (zpad[:, i::8] & 0xF) << np.uint64(4 * i)
    scales = d16.astype(np.float16)
    return qw.astype(np.uint32), scales, qz.astype(np.uint32), int(bad.sum())


def unpack_int4(qweight: np.ndarray, qzeros: np.ndarray, k: int, g: int):
    """Inverse of the nibble layout: returns (q [N, K] int, z [N, K/g] int)."""
    qw = np.asarray(qweight, np.uint32).astype(np.uint64)
    n = qw.shape[0]
    q = np.zeros((n, k), dtype=np.int64)
    for i in range(8):
        q[:, i::8] = ((qw >> np.uint64(4 * i)) & 0xF).astype(np.int64)
    ng = k // g
    qz = np.asarray(qzeros, np.uint32).astype(np.uint64)
    zall = np.zeros((n, qz.shape[1] * 8), dtype=np.int64)
    for i in range(8):
        zall[:, i::8] = ((qz >> np.uint64(4 * i)) & 0xF).astype(np.int64)
    return q, zall[:, :ng]


# ----------------------------------------------------------------------------
# other weight widths ([csdn] 量化流程优化: the w_bit option; [jsqmd] 五: 3- and
# 4-bit quantization; [zeeklog]: the INT3 result; [bjdmk]: INT4 / INT8).  The
# same rule with max_int = 2**w_bit - 1, packed (layouts of this library):
#   w_bit 8: qweight[n][k/4] uint32, byte k%4 of word k/4 holds q_nk;
#            qzeros[n][ceil(ng/4)] uint32, byte j%4 holds z_nj (unused bytes 0).
#   w_bit 3: qweight[n][3k/32] uint32: the 32 codes of k in [32p, 32p+32) fill
#            words 3p..3p+2, code k at bit 3(k%32) of their 96-bit
#            little-endian value; qzeros as for 4 bits (nibbles; z <= 7).


def pack_weights(w16: np.ndarray, s16: np.ndarray | None, g: int = 128, w_bit: int = 4):
    """pack_int4 for w_bit 4, the layouts above for 3 and 8.  Returns
    (qweight u32, scales f16 [N, K/g], qzeros u32, n_nonfinite_groups).

    Pinned by test_pack_wbit_roundtrip and the brute-force / known-answer
    tests at 3 and 8 bits.
    """
    if w_bit == 4:
        return pack_int4(w16, s16, g)
    max_int = (1 << w_bit) - 1
    wp, q, z, d16, bad, _ = fake_quantize(w16, s16, g, max_int)
    n, k = q.shape
    ng = k // g
    if w_bit == 8:
        qw = np.zeros((n, k // 4), dtype=np.uint64)
        for i in range(4):
            qw |= (q[:, i::4].astype(np.uint64) & 0xFF) << np.uint64(8 * i)
        nzw = (ng + 3) // 4
        zpad = np.zeros((n, nzw * 4), dtype=np.uint64)
        zpad[:, :ng] = z
        qz = np.zeros((n, nzw), dtype=np.uint64)
        for i in range(4):
            qz |= (zpad[:, i::4] & 0xFF) << np.uint64(8 * i)
    elif w_bit == 3:
        assert k % 32 == 0
        qw = np.zeros((n, 3 * k // 32), dtype=np.uint64)
        for kk in range(32):                      # code kk of every pack of 32
            bit = 3 * kk
            word, off = bit // 32, bit % 32
            code = q[:, kk::32].astype(np.uint64)
            qw[:, word::3] |= (code << np.uint64(off)) & np.uint64(0xFFFFFFFF)
            if off > 29:                          # the code straddles into the next word
                qw[:, word + 1::3] |= code >> np.uint64(32 - off)
        nzw = (ng + 7) // 8
        zpad = np.zeros((n, nzw * 8), dtype=np.uint64)
        zpad[:, :ng] = z
        qz = np.zeros((n, nzw), dtype=np.uint64)
        for i in range(8):
            qz |= (zpad[:, i::8] & 0xF) << np.uint64(4 * i)
    else:
        raise ValueError("w_bit must be 3, 4 or 8")
    return qw.astype(np.uint32), d16.astype(np.float16), qz.astype(np.uint32), int(bad.sum())


def unpack_weights(qweight: np.ndarray, qzeros: np.ndarray, k: int, g: int, w_bit: int = 4):
    """Inverse of pack_weights: (q [N, K] int, z [N, K/g] int)."""
    if w_bit == 4:
        return unpack_int4(qweight, qzeros, k, g)
    qw = np.asarray(qweight, np.uint32).astype(np.uint64)
    qz = np.asarray(qzeros, np.uint32).astype(np.uint64)
    n = qw.shape[0]
    ng = k // g
    q = np.zeros((n, k), dtype=np.int64)
    if w_bit == 8:
        for i in range(4):
            q[:, i::4] = ((qw >> np.uint64(8 * i)) & 0xFF).astype(np.int64)
        zall = np.zeros((n, qz.shape[1] * 4), dtype=np.int64)
        for i in range(4):
            zall[:, i::4] = ((qz >> np.uint64(8 * i)) & 0xFF).astype(np.int64)
    elif w_bit == 3:
        for kk in range(32):
            bit = 3 * kk
            word, off = bit // 32, bit % 32
            v = qw[:, word::3] >> np.uint64(off)
            if off > 29:
                v |= qw[:, word + 1::3] << np.uint64(32 - off)
            q[:, kk::32] = (v & 0x7).astype(np.int64)
        zall = np.zeros((n, qz.shape[1] * 8), dtype=np.int64)
        for i in range(8):
            zall[:, i::8] = ((qz >> np.uint64(4 * i)) & 0xF).astype(np.int64)
    else:
        raise ValueError("w_bit must be 3, 4 or 8")
    return q, zall[:, :ng]


# ----------------------------------------------------------------------------
# a6-a8: the W4A16 linear  ([bjdmk] GEMV / GEMM modes; [zeeklog] W4A16)


def dequantized_weight(qweight, scales, qzeros, k: int, g: int, w_bit: int = 4) -> np.ndarray:
    """Unpacked (q - z) * D as float64 [N, K]."""
    q, z = unpack_weights(qweight, qzeros, k, g, w_bit)
    return dequantize(q, z, np.asarray(scales, np.float16), g)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) as float64: a bf16 value is the upper half
    of an IEEE binary32, so the conversion is exact.  Pinned by
    test_bf16_decode (values fixed by the format's definition)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def exact_f64(a) -> np.ndarray:
    """A float array's values as float64: fp16 arrays convert exactly, float32
    and float64 arrays are taken as the exact values they hold (bf16 inputs
    arrive decoded by bf16_to_f64)."""
    a = np.asarray(a)
    if a.dtype in (np.float16, np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"expected a float array, got {a.dtype}")


def linear_ref(x16, qweight, scales, qzeros, inv_s16, k: int, g: int, w_bit: int = 4) -> np.ndarray:
    """y_ref[t, n] = sum_k xt_tk (q_nk - z) D in float64, with
    xt = x * inv_s16 (exact: a product of two fp16, or of a bf16 and an fp16)
    or xt = x when inv_s16 is None.  x is an fp16 array, or float64 holding
    the exact values (bf16 activations).

    Pinned by test_linear_ref_identity (scaling identity) and the fact that it
    is one float64 matrix product of the unpacked weights.
    """
    x = exact_f64(x16)
    if inv_s16 is not None:
        x = x * np.asarray(inv_s16, np.float16).astype(np.float64)[None, :]
    wd = dequantized_weight(qweight, scales, qzeros, k, g, w_bit)
    return x @ wd.T


def linear_ref_rows(x16, qweight, scales, qzeros, inv_s16, k: int, g: int,
                    rows: np.ndarray, w_bit: int = 4) -> np.ndarray:
    """linear_ref restricted to output columns ``rows`` (used for sampled
    checks at full size)."""
    rows = np.asarray(rows)
    return linear_ref(x16, np.asarray(qweight)[rows], np.asarray(scales)[rows],
                      np.asarray(qzeros)[rows], inv_s16, k, g, w_bit)


def check_linear(y16, y_ref, tol: float = 5e-3):
    """Floored relative check: |y - y_ref| <= tol * max(|y_ref|, rms_t(y_ref))
    for every output, where rms_t is the RMS of row t of y_ref.

    Returns (passed, worst_ratio, raw_max_rel) where worst_ratio is the largest
    |y - y_ref| / (tol * floor) and raw_max_rel the plain relative error over
    outputs with |y_ref| >= rms_t.
    """
    y = exact_f64(y16)
    yr = np.asarray(y_ref, np.float64)
    if y.size == 0:
        return True, 0.0, 0.0
    rms = np.sqrt(np.mean(yr * yr, axis=1, keepdims=True))
    floor = np.maximum(np.abs(yr), rms)
    floor = np.where(floor > 0, floor, 1.0)
    err = np.abs(y - yr)
    ratio = err / (tol * floor)
    big = np.abs(yr) >= rms
    raw = float(np.max(err[big] / np.abs(yr[big]))) if big.any() else 0.0
    worst = float(np.max(ratio))
    return bool(np.all(np.isfinite(y)) and worst <= 1.0), worst, raw


# ----------------------------------------------------------------------------
# mixed-precision baseline ([jsqmd] 二.1(1): a small share (0.1 - 1 %) of the
# weights, on the input channels with large activations, matters most and
# loses accuracy under direct quantization; 五.1: protection ratio 0.1 - 1 %
# by default.  [csdn]: mixed-precision optimisation named beside the scaling.)
# The contrasting approach to the search: keep those channels in fp16 and
# quantize the rest with plain round-to-nearest.

def salient_count(k: int, frac: float) -> int:
    """Number of protected channels: round(frac * k), at least 0, at most k."""
    return int(min(max(int(np.floor(frac * k + 0.5)), 0), k))


def salient_channels(a: np.ndarray, count: int) -> np.ndarray:
    """Indices (ascending) of the ``count`` channels with the largest a_k; among
    equal a_k the lower index wins.  NaN ranks above +inf.

    Pinned by test_salient_channels_brute_force (every subset of tiny inputs)
    and its special cases.
    """
    a = np.asarray(a, np.float64)
    key = np.where(np.isnan(a), np.inf, a)
    nan_first = np.isnan(a).astype(np.int64)
    # sort by (NaN first, a descending, index ascending)
    order = np.lexsort((np.arange(a.size), -key, -nan_first))
    return np.sort(order[:count]).astype(np.int32)


def mixed_weight(w16: np.ndarray, idx: np.ndarray, g: int, max_int: int = 15) -> np.ndarray:
    """The mixed-precision weight as float64 [N, K]: plain RTN (s = 1, the
    quantizer of every other step) of the whole W, then the protected columns
    ``idx`` restored to their fp16 values.  Groups are formed over all
    channels, protected ones included (the plainest reading: quantize, then
    keep the protected channels).

    Pinned by test_mixed_loss_two_ways (against the masked-activation form of
    the loss) and test_mixed_extremes (no channel / every channel protected).
    """
    w = np.asarray(w16, np.float16).astype(np.float64)
    deq = fake_quantize(w16, None, g, max_int)[5].copy()
    deq[:, np.asarray(idx, np.int64)] = w[:, np.asarray(idx, np.int64)]
    return deq


def mixed_loss(w16: np.ndarray, x16: np.ndarray, idx: np.ndarray, g: int,
               max_int: int = 15) -> float:
    """L_mixed = sum_{t,n} (sum_k (Wm_nk - W_nk) X_tk)^2 in float64, the search's
    output-error objective for the mixed-precision weight.

    Pinned by test_mixed_loss_two_ways and test_mixed_extremes.
    """
    w = np.asarray(w16, np.float16).astype(np.float64)
    x = np.asarray(x16, np.float16).astype(np.float64)
    if fake_quantize(w16, None, g, max_int)[4].any():
        return float("inf")
    e = (mixed_weight(w16, idx, g, max_int) - w) @ x.T
    return float(np.sum(e * e))


def linear_mixed_ref(x16, qweight, scales, qzeros, w16, idx, k: int, g: int) -> np.ndarray:
    """y_ref = x Wm^T in float64 for the packed RTN weights with the protected
    columns ``idx`` taken from the fp16 weight w16 [N, K] instead.

    Pinned by test_linear_mixed_ref_exact_small (rational sum).
    """
    x = exact_f64(x16)
    wd = dequantized_weight(qweight, scales, qzeros, k, g)
    ii = np.asarray(idx, np.int64)
    wd[:, ii] = np.asarray(w16, np.float16).astype(np.float64)[:, ii]
    return x @ wd.T
