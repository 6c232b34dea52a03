"""Plain CPU oracle for the SVDQuant W4A4 + low-rank linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code, tables or helpers with the HIP path.

What the method computes (sources are the five web pages on SVDQuant):

* The layer is Y ~= Xhat.L1.L2 + Q(Xhat).Q(R) + b, with Xhat = X.diag(lam)^-1.
  Smoothing moves activation outliers onto the weights; the smoothed weight
  diag(lam).W is split by an SVD into a 16-bit low-rank branch L1.L2 and a
  residual R; both Xhat and R are quantized to 4 bits
  (chattools.cn overview, section "SVDQuant的技术原理" (technical principles),
  items on outlier handling and the low-rank branch; SVDQuant paper abstract
  on ai-digest.ru).
* Dropping the dominant singular values is optimal in the Frobenius norm
  (Eckart-Young-Mirsky; chattools.cn overview, same section, EYM item).
* LoRA adapters join the low-rank branch without re-quantizing R
  (chattools.cn overview, section "SVDQuant的主要功能" (main features), LoRA
  item; SVDQuant abstract).

The pages print no formulas, group size or rounding rule. The readings taken
here, each applied in exactly one function below, are:

* lam_j = sqrt(max_i |X_ij| / max_n |W_jn|) (migration strength 1/2), 1 where
  either max is 0, rounded to fp32; inv_lam = fp32(1/lam).
* Sigma is split as Sigma^(1/2) on each side; L1, L2 are rounded to fp16 once
  from fp64; the residual is formed from the *stored* fp16 factors.
* Quantizer Q over each group of 64 consecutive input channels: symmetric,
  scale s = fp16(min(absmax/7, 65504)) (fp32 division, then fp16 RNE),
  codes q = clamp(rint(v * fp32(1/s)), -7, 7), s == 0 -> all codes 0.
  X-hat groups run along each token row; R groups run down K for each output
  column.
* Codes are 4-bit two's complement, element 2j in the low nibble of byte j.
* The low-rank branch is fp16 x fp16: Xhat and D are rounded to fp16 where
  they enter a product.

Data are fp64 except at the rounding points named in each function.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
QMAX = 7
F16_MAX = 65504.0


# --------------------------------------------------------------------------
# rounding helpers


def to_f16(x) -> np.ndarray:
    """Round to IEEE binary16, nearest-even, in one step from the input type
    (numpy converts float64 -> float16 directly, without passing through
    float32)."""
    return np.asarray(x).astype(np.float16)


def to_f32(x) -> np.ndarray:
    return np.asarray(x).astype(np.float32)


# --------------------------------------------------------------------------
# smoothing (chattools.cn overview, technical principles, outlier item;
# SVDQuant abstract: outliers are first moved from activations to weights)


def channel_absmax(X) -> np.ndarray:
    """max_i |X_ij| per input channel j, as float64 (exact)."""
    return np.max(np.abs(np.asarray(X, dtype=np.float64)), axis=0)


def smoothing_factors(x_absmax, W) -> np.ndarray:
    """lam_j = sqrt(max|X_j| / max|W_j|) in fp64, rounded to fp32; 1 if either is 0."""
    xa = np.asarray(x_absmax, dtype=np.float64)
    wa = np.max(np.abs(np.asarray(W, dtype=np.float64)), axis=1)
    ok = (xa > 0) & (wa > 0)
    lam = np.ones_like(xa)
    lam[ok] = np.sqrt(xa[ok] / wa[ok])
    return to_f32(lam)


def inv_smoothing(lam32) -> np.ndarray:
    """inv_lam = 1/lam as a correctly rounded fp32 division."""
    lam32 = to_f32(lam32)
    return (np.float32(1.0) / lam32).astype(np.float32)


def smooth_weight(W, lam32) -> np.ndarray:
    """What = diag(lam).W in fp64 (exact: fp32 x fp32 fits in 53 bits)."""
    return np.asarray(lam32, dtype=np.float64)[:, None] * np.asarray(W, dtype=np.float64)


# --------------------------------------------------------------------------
# SVD split (chattools.cn overview, technical principles, low-rank-branch and
# EYM items)


def svd_canonical(What):
    """What = U diag(S) Vt (LAPACK, fp64), with a fixed sign per singular pair:
    the entry of largest magnitude in each column of U is positive (first such
    index on ties)."""
    U, S, Vt = np.linalg.svd(np.asarray(What, dtype=np.float64), full_matrices=False)
    idx = np.argmax(np.abs(U), axis=0)
    sgn = np.sign(U[idx, np.arange(U.shape[1])])
    sgn[sgn == 0] = 1.0
    return U * sgn[None, :], S, Vt * sgn[:, None]


def lowrank_factors_f64(U, S, Vt, r: int):
    """L1 = U_r Sigma_r^(1/2) (K x r), L2 = Sigma_r^(1/2) Vt_r (r x N), in fp64."""
    h = np.sqrt(S[:r])
    return U[:, :r] * h[None, :], h[:, None] * Vt[:r, :]


def lowrank_factors(U, S, Vt, r: int):
    """The 16-bit branch: the fp64 factors rounded once to fp16."""
    L1, L2 = lowrank_factors_f64(U, S, Vt, r)
    return to_f16(L1), to_f16(L2)


def residual(What, L1, L2) -> np.ndarray:
    """R = What - L1.L2 from the stored factors, in fp64."""
    return np.asarray(What, dtype=np.float64) - (
        np.asarray(L1, dtype=np.float64) @ np.asarray(L2, dtype=np.float64))


# --------------------------------------------------------------------------
# 4-bit group quantizer (chattools.cn overview, main features: weights and
# activations at 4 bits; technical principles: the residual is quantized to
# 4 bits)


def quantize_groups(v32, group: int = GROUP):
    """Q along the last axis, in groups of ``group`` consecutive values.

    v32 is rounded to fp32 first. Returns (codes int8 in [-7, 7], scales fp16)
    with scales shaped (..., K/group)."""
    v = to_f32(v32)
    *lead, K = v.shape
    assert K % group == 0
    vg = v.reshape(*lead, K // group, group)
    a = np.max(np.abs(vg), axis=-1)                                   # exact
    s32 = np.minimum(a / np.float32(QMAX), np.float32(F16_MAX))       # fp32 division
    s16 = s32.astype(np.float16)                                      # RNE
    sf = s16.astype(np.float32)
    zero = sf == 0
    inv = np.where(zero, np.float32(0.0),
                   np.float32(1.0) / np.where(zero, np.float32(1.0), sf)).astype(np.float32)
    prod = (vg * inv[..., None]).astype(np.float32)                   # fp32 multiply
    q = np.clip(np.rint(prod), -QMAX, QMAX).astype(np.int8)           # half to even
    return q.reshape(*lead, K), s16


def dequantize_groups(q, s16, group: int = GROUP) -> np.ndarray:
    """s * q in fp64 (exact)."""
    q = np.asarray(q, dtype=np.float64)
    *lead, K = q.shape
    s = np.asarray(s16, dtype=np.float64)
    return (q.reshape(*lead, K // group, group) * s[..., None]).reshape(*lead, K)


def pack_nibbles(q) -> np.ndarray:
    """int8 codes (..., K) -> uint8 (..., K/2); element 2j in the low nibble."""
    q = np.asarray(q, dtype=np.int16)
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b) -> np.ndarray:
    """uint8 (..., K/2) -> int8 codes (..., K), sign-extending each nibble."""
    b = np.asarray(b, dtype=np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def quantize_weight(R, group: int = GROUP):
    """Q of R (K x N) down K for each output column: (w_codes N x K/2, w_scales N x K/group)."""
    q, s = quantize_groups(to_f32(R).T, group)
    return pack_nibbles(q), s


def smooth_activation(X, inv_lam32) -> np.ndarray:
    """Xhat = fp32(float(x) * inv_lam[k]) per element (fp32 multiply)."""
    return (to_f32(X) * to_f32(inv_lam32)[None, :]).astype(np.float32)


def quantize_activation(X, inv_lam32, group: int = GROUP):
    """(a_codes M x K/2, a_scales M x K/group, Xhat fp32)."""
    xh = smooth_activation(X, inv_lam32)
    q, s = quantize_groups(xh, group)
    return pack_nibbles(q), s, xh


# --------------------------------------------------------------------------
# online part of the layer


def down_projection(xhat32, L1) -> np.ndarray:
    """D = fp16(Xhat) . L1, accumulated in fp64 (the products of fp16 values are exact)."""
    return to_f16(xhat32).astype(np.float64) @ np.asarray(L1, dtype=np.float64)


def group_partials(a_codes, w_codes, group: int = GROUP) -> np.ndarray:
    """P[m, n, g] = sum over k in group g of qx[m,k] * qw[n,k], exact integers (int64)."""
    qx = unpack_nibbles(a_codes).astype(np.int64)
    qw = unpack_nibbles(w_codes).astype(np.int64)
    M, K = qx.shape
    N = qw.shape[0]
    G = K // group
    P = np.empty((M, N, G), dtype=np.int64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        # float64 matmul of small integers: every partial sum is an integer
        # below 2^53, so the result is exact
        P[:, :, g] = np.rint(qx[:, sl].astype(np.float64) @ qw[:, sl].astype(np.float64).T)
    return P


def scaled_group_sum(P, a_scales, w_scales) -> np.ndarray:
    """sum_g s_x[m,g] * s_w[n,g] * P[m,n,g] in fp64."""
    sx = np.asarray(a_scales, dtype=np.float64)
    sw = np.asarray(w_scales, dtype=np.float64)
    return np.einsum("mng,mg,ng->mn", np.asarray(P, dtype=np.float64), sx, sw, optimize=True)


def lowrank_up(D, L2) -> np.ndarray:
    """fp16(D) . L2 in fp64."""
    return to_f16(D).astype(np.float64) @ np.asarray(L2, dtype=np.float64)


def finalize(acc, lr, bias, out_dtype: str) -> np.ndarray:
    y = np.asarray(acc, dtype=np.float64) + np.asarray(lr, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y.astype(np.float16 if out_dtype == "f16" else np.float32)


# --------------------------------------------------------------------------
# whole steps


def prepare(W, lam32, rank: int, group: int = GROUP, svd=None):
    """Offline prep: dict with inv_smooth, L1 (K x r fp16), L2 (r x N fp16),
    w_codes, w_scales, sigma, and the fp64 What/R."""
    What = smooth_weight(W, lam32)
    U, S, Vt = svd if svd is not None else svd_canonical(What)
    L1, L2 = lowrank_factors(U, S, Vt, rank)
    R = residual(What, L1, L2)
    w_codes, w_scales = quantize_weight(R, group)
    return dict(inv_smooth=inv_smoothing(lam32), L1=L1, L2=L2, w_codes=w_codes,
                w_scales=w_scales, sigma=S, What=What, R=R)


def quantize_residual_from_factors(W, lam32, L1, L2, group: int = GROUP):
    """(w_codes, w_scales) for given fp16 factors: the codes a prep with these
    factors must produce, whatever SVD produced them."""
    R = residual(smooth_weight(W, lam32), L1, L2)
    return quantize_weight(R, group)


def linear(X, inv_lam32, L1, L2, w_codes, w_scales, bias=None, out_dtype: str = "f16",
           group: int = GROUP, return_parts: bool = False, activation=None):
    """Y = act(sum_g s_x s_w P + fp16(D).L2 + b), rounded once to ``out_dtype``.
    ``activation``: None or "gelu_tanh" (the GELU of a DiT MLP's first layer,
    applied to the unrounded sum)."""
    a_codes, a_scales, xh = quantize_activation(X, inv_lam32, group)
    D = down_projection(xh, L1)
    P = group_partials(a_codes, w_codes, group)
    acc = scaled_group_sum(P, a_scales, w_scales)
    lr = lowrank_up(D, L2)
    if activation is None:
        Y = finalize(acc, lr, bias, out_dtype)
    elif activation == "gelu_tanh":
        y = np.asarray(acc, dtype=np.float64) + np.asarray(lr, dtype=np.float64)
        if bias is not None:
            y = y + np.asarray(bias, dtype=np.float64)[None, :]
        Y = gelu_tanh_f64(y).astype(np.float16 if out_dtype == "f16" else np.float32)
    else:
        raise ValueError(f"unknown activation {activation!r}")
    if return_parts:
        return Y, dict(a_codes=a_codes, a_scales=a_scales, xhat=xh, D=D, P=P, acc=acc, lr=lr)
    return Y


def linear_rows(X_rows, inv_lam32, L1, L2, w_codes, w_scales, bias=None,
                out_dtype: str = "f16", group: int = GROUP):
    """``linear`` on a subset of rows (rows are independent)."""
    return linear(X_rows, inv_lam32, L1, L2, w_codes, w_scales, bias, out_dtype, group)


# --------------------------------------------------------------------------
# LoRA (chattools.cn overview, main features, LoRA item; SVDQuant abstract:
# off-the-shelf LoRAs without re-quantization)


def concat_lora(L1, L2, lam32, A, B, scale: float = 1.0):
    """L1' = [L1 | fp16(lam (.) A * scale)], L2' = [L2 ; B].

    The branch multiplies the smoothed activation, so row j of A is scaled by
    lam_j to give Xhat.(lam (.) A) = X.A. The product lam*A is exact in fp64;
    the scale multiply rounds once in fp64; the result rounds once to fp16."""
    lam = np.asarray(lam32, dtype=np.float32).astype(np.float64)
    t = lam[:, None] * np.asarray(A, dtype=np.float64)
    t = t * np.float64(np.float32(scale))
    L1n = np.concatenate([np.asarray(L1, dtype=np.float16), to_f16(t)], axis=1)
    L2n = np.concatenate([np.asarray(L2, dtype=np.float16), np.asarray(B, dtype=np.float16)], axis=0)
    return L1n, L2n


# --------------------------------------------------------------------------
# glue between the two layers of a DiT MLP (textbook GELU, tanh form; the
# pages do not describe it)


def gelu_tanh_f64(x) -> np.ndarray:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in fp64, not rounded."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def gelu_tanh(x) -> np.ndarray:
    """The GELU above, rounded to fp16."""
    return to_f16(gelu_tanh_f64(x))


# --------------------------------------------------------------------------
# MXFP4 variant of the 4-bit part.
#
# The pages name a 4-bit floating-point variant of the method for the newest
# hardware of one vendor (taicenter.com news page on SVDQuant, section on
# hardware co-design for Blackwell GPUs, NVFP4 item); they give no format
# details. Its counterpart on CDNA4 is the OCP Microscaling format MXFP4 (OCP
# "Microscaling Formats (MX) Specification" v1.0, sections on the scale and
# element data types and on conversion): blocks of 32 values share one
# power-of-two scale (E8M0) and each value is an FP4 E2M1 number.
# Smoothing, the SVD split and the fp16 low-rank branch are unchanged; X-hat
# and R are quantized with this block quantizer instead of Q above. Readings:
#
# * shared exponent e = floor(log2(max|v|)) - 2 (2 is the largest exponent of
#   E2M1, whose largest value is 6 = 1.5 * 2^2), clamped to [-127, 127];
#   stored as the E8M0 byte e + 127; an all-zero block gets e = -127.
# * each value is v / 2^e rounded to the nearest E2M1 value (0, 0.5, 1, 1.5,
#   2, 3, 4, 6) with ties to the even encoding and magnitudes above 6
#   saturated to 6; the sign is kept (negative values that round to 0 give
#   the code of -0).
# * the code is the E2M1 bit pattern s e1 e0 m; codes pack two per byte like
#   the INT4 codes (element 2j in the low nibble). Blocks run along K: along
#   each token row for X-hat, down K for each output column of R.

MX_BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit E2M1 code (bit 3 is the sign)."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_round(x) -> np.ndarray:
    """Nearest E2M1 code of each x (fp64): ties to the even encoding (even
    mantissa bit), magnitudes above 6 saturate to 6, sign kept."""
    x = np.asarray(x, dtype=np.float64)
    m = np.abs(x)
    d = np.abs(m[..., None] - E2M1_VALUES)                 # distance to each magnitude
    cand = d == np.min(d, axis=-1, keepdims=True)          # one or two nearest
    # two nearest only at a midpoint: take the even encoding (even index)
    pick_even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(pick_even.any(-1), np.argmax(pick_even, -1), np.argmax(cand, -1))
    idx = np.where(m > 6.0, 7, idx)
    sign = np.signbit(x).astype(np.int64) * 8
    return (idx + sign).astype(np.uint8)


def mx_quantize_blocks(v32, block: int = MX_BLOCK):
    """MXFP4 quantization of the last axis in blocks of ``block`` values.
    Returns (codes (..., n) uint8 in 0..15, e8m0 (..., n/block) uint8)."""
    v = np.asarray(v32, dtype=np.float32)
    sh = v.shape
    vb = v.reshape(sh[:-1] + (sh[-1] // block, block)).astype(np.float64)
    amax = np.max(np.abs(vb), axis=-1)
    mant, ex = np.frexp(amax)                 # amax = mant * 2^ex, mant in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    scale = np.ldexp(1.0, e)                  # 2^e (exact in fp64)
    codes = e2m1_round(vb / scale[..., None])
    return codes.reshape(sh), (e + 127).astype(np.uint8)


def mx_dequantize_blocks(codes, e8m0, block: int = MX_BLOCK) -> np.ndarray:
    c = np.asarray(codes)
    sh = c.shape
    vals = e2m1_decode(c).reshape(sh[:-1] + (sh[-1] // block, block))
    s = np.ldexp(1.0, np.asarray(e8m0, dtype=np.int64) - 127)
    return (vals * s[..., None]).reshape(sh)


def pack_codes4(codes) -> np.ndarray:
    """Two 4-bit codes per byte, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8) & 15
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes4(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def mx_quantize_activation(X, inv_lam32):
    """Xhat rows in MXFP4: packed codes (M x K/2), E8M0 exponents (M x K/32), Xhat."""
    xh = smooth_activation(X, inv_lam32)
    codes, e8 = mx_quantize_blocks(xh)
    return pack_codes4(codes), e8, xh


def mx_quantize_residual_from_factors(W, lam32, L1, L2):
    """R (from the stored fp16 factors, rounded to fp32) in MXFP4 down K for each
    output column: packed codes (N x K/2), E8M0 exponents (N x K/32)."""
    R32 = to_f32(residual(smooth_weight(W, lam32), L1, L2))
    codes, e8 = mx_quantize_blocks(R32.T)
    return pack_codes4(codes), e8


def mx_prepare(W, lam32, rank: int, svd=None):
    """Offline prep of the MXFP4 variant: the same smoothing and SVD split as
    ``prepare``, then R in MXFP4 (w_codes N x K/2, w_e8m0 N x K/32)."""
    What = smooth_weight(W, lam32)
    U, S, Vt = svd if svd is not None else svd_canonical(What)
    L1, L2 = lowrank_factors(U, S, Vt, rank)
    w_codes, w_e8m0 = mx_quantize_residual_from_factors(W, lam32, L1, L2)
    return dict(inv_smooth=inv_smoothing(lam32), L1=L1, L2=L2, w_codes=w_codes,
                w_e8m0=w_e8m0, sigma=S)


def mx_linear(X, inv_lam32, L1, L2, w_codes, w_e8m0, bias=None, out_dtype: str = "f16",
              activation=None, return_parts: bool = False):
    """Y = act(deq(Q_mx(Xhat)).deq(Q_mx(R))^T + fp16(D).L2 + b), exact in fp64
    and rounded once. Products of E2M1 values and powers of two are exact, and
    so is their fp64 sum over K while the block exponents of a row and a column
    span fewer than about 40 binades (true of every input used here)."""
    a_codes, a_e8, xh = mx_quantize_activation(X, inv_lam32)
    A = mx_dequantize_blocks(unpack_codes4(a_codes), a_e8)
    B = mx_dequantize_blocks(unpack_codes4(w_codes), w_e8m0)
    acc = A @ B.T
    D = down_projection(xh, L1)
    lr = lowrank_up(D, L2)
    if activation is None:
        Y = finalize(acc, lr, bias, out_dtype)
    elif activation == "gelu_tanh":
        y = acc + np.asarray(lr, dtype=np.float64)
        if bias is not None:
            y = y + np.asarray(bias, dtype=np.float64)[None, :]
        Y = gelu_tanh_f64(y).astype(np.float16 if out_dtype == "f16" else np.float32)
    else:
        raise ValueError(f"unknown activation {activation!r}")
    if return_parts:
        return Y, dict(a_codes=a_codes, a_e8m0=a_e8, xhat=xh, D=D, acc=acc, lr=lr)
    return Y


# --------------------------------------------------------------------------
# 4-bit weight-only baseline (W4A16).
#
# The SVDQuant abstract (ai-digest.ru page) measures the method against a
# baseline that quantizes only the weights to 4 bits, and gives no format for
# it. The reading taken here: the same symmetric 4-bit group quantizer Q as
# above, applied to W itself (per output column, groups of 64 along K; no
# smoothing, no low-rank branch); activations stay fp16; each weight enters
# the product dequantized to fp16, fp16(s * q), one rounding (what a fp16
# weight-only kernel feeds its fp16 matrix unit); fp32-or-better accumulation,
# one rounding of the output.


def w4a16_prepare(W):
    """(w_codes N x K/2, w_scales N x K/64 fp16): Q of W, down K per column."""
    return quantize_weight(np.asarray(W, dtype=np.float64))


def w4a16_dequant(w_codes, w_scales, group: int = GROUP) -> np.ndarray:
    """N x K fp16 weights fp16(s * q) (the product is exact in fp64, then one
    rounding to fp16)."""
    q = unpack_nibbles(w_codes).astype(np.float64)
    s = np.asarray(w_scales, dtype=np.float16).astype(np.float64)
    N, K = q.shape
    prod = q.reshape(N, K // group, group) * s[:, :, None]
    return to_f16(prod.reshape(N, K))


def w4a16_linear(X, w_codes, w_scales, bias=None, out_dtype: str = "f16") -> np.ndarray:
    """Y = fp16(X) . fp16(s q)^T + b, exact in fp64 (each product of two fp16
    values is exact, and so is their sum at these sizes), rounded once to
    out_dtype ("f16", "f32", or "f64" for the unrounded value)."""
    Xh = to_f16(X).astype(np.float64)
    Wd = w4a16_dequant(w_codes, w_scales).astype(np.float64)
    y = Xh @ Wd.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if out_dtype == "f64":
        return y
    return y.astype(np.float16 if out_dtype == "f16" else np.float32)


# --------------------------------------------------------------------------
# Convolutions as implicit GEMMs (UNet layers).
#
# The pages say the method applies to UNet backbones as well as DiT ones
# (chattools.cn overview, main features, architectures item;
# disruptive-concepts.com post) without saying how a convolution is treated.
# Reading: a KH x KW convolution over an NHWC image (zero padding, one stride
# for both axes) is the linear layer applied to the matrix of its patches,
# X_col (batch*OH*OW x KH*KW*C), whose row (b, oh, ow) holds, at column
# (kh*KW + kw)*C + c, the input value at (b, oh*stride + kh - pad,
# ow*stride + kw - pad, c), or 0 outside the image; the weight (KH, KW, C, N)
# becomes the (KH*KW*C) x N matrix in the same order. Smoothing, the split,
# quantization and everything else are those of the linear layer on X_col.


def im2col_nhwc(X, KH: int, KW: int, stride: int, pad: int) -> np.ndarray:
    """The patch matrix X_col of an NHWC image, in the image's dtype."""
    X = np.asarray(X)
    B, H, W, C = X.shape
    OH = (H + 2 * pad - KH) // stride + 1
    OW = (W + 2 * pad - KW) // stride + 1
    Xp = np.zeros((B, H + 2 * pad, W + 2 * pad, C), dtype=X.dtype)
    Xp[:, pad:pad + H, pad:pad + W, :] = X
    cols = np.empty((B, OH, OW, KH, KW, C), dtype=X.dtype)
    for kh in range(KH):
        for kw in range(KW):
            cols[:, :, :, kh, kw, :] = Xp[:, kh:kh + stride * (OH - 1) + 1:stride,
                                          kw:kw + stride * (OW - 1) + 1:stride, :]
    return cols.reshape(B * OH * OW, KH * KW * C)


def conv_weight_matrix(Wc) -> np.ndarray:
    """(KH, KW, C, N) -> (KH*KW*C) x N, rows in the order of X_col's columns."""
    Wc = np.asarray(Wc)
    KH, KW, C, N = Wc.shape
    return Wc.reshape(KH * KW * C, N)
