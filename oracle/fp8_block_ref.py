"""CPU oracle: E4M3 decode, bf16 rounding, block dequant, block quantize and
the exact linear, written plainly from the definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing here is tuned
or blocked; every step is the definition written out with numpy.

Notation: Q[N,K] uint8 E4M3 codes (row-major, K contiguous), S[GN,GK] fp32
``weight_scale_inv`` with GN = ceil(N/128), GK = ceil(K/128), X[M,K] and the
output Y[M,N] as bf16 bit patterns held in uint16.
"""

from __future__ import annotations

import math

import numpy as np

# Block edge of the scale grid. FastVideo PR #1829, "Changes", converter
# bullet: one weight_scale_inv per 128x128 block, grid [N/128, K/128].
BLOCK = 128

# Largest finite E4M3 magnitude (code 0x7E): (1 + 6/8) * 2^8.
E4M3_MAX = 448.0

# The one NaN pattern the oracle emits for a bf16 NaN (sign clear, quiet bit).
BF16_CANONICAL_NAN = 0x7FC0


# ---------------------------------------------------------------------------
# E4M3 (OCP E4M3FN): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
# no infinities, NaN only where exponent and mantissa are all ones.
# The pages name the format "E4M3" (FastVideo PR #1829, "Changes"); the
# closed-form facts used to fix the variant are: largest magnitude 448, NaN
# at 0x7F/0xFF, subnormal step 2^-9.
# ---------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Exact value of one E4M3FN code, from the closed form."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code out of range")
    sign = code >> 7
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = man * 2.0 ** -9            # subnormal: m/8 * 2^(1-7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return -mag if sign else mag


def e4m3_table() -> np.ndarray:
    """The 256-entry decode table, fp64, indexed by code."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


# ---------------------------------------------------------------------------
# bf16 round-to-nearest-even from fp32. Two independent implementations:
# the integer one is what the oracle uses; the fp64 "pick the nearer
# neighbour" one exists only to cross-check it.
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even; NaN -> 0x7FC0.

    Adding 0x7FFF plus the lowest kept bit to the fp32 pattern and dropping
    the low 16 bits rounds the magnitude to nearest with ties to even; a carry
    out of the mantissa moves to the next binade, and past the largest finite
    value it lands on infinity, as IEEE rounding requires.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    out[np.isnan(x32)] = BF16_CANONICAL_NAN
    return out


def bf16_rne_bits_nearest(x32: np.ndarray) -> np.ndarray:
    """Second fp32 -> bf16 RNE: compare distances to both neighbours in fp64.

    ``lo`` is the bf16 value toward zero (the fp32 pattern with its low 16
    bits cleared), ``hi`` the next bf16 value away from zero (2^128 stands
    for the step past the largest finite value). Both distances are exact in
    fp64. The nearer wins; on a tie the one with an even last mantissa bit.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    mag = u & np.uint32(0x7FFFFFFF)
    lo_bits = mag & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x10000)
    a = np.abs(x32.astype(np.float64))
    lo = lo_bits.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        hi = np.where(hi_bits >= np.uint32(0x7F800000), 2.0 ** 128,
                      hi_bits.view(np.float32).astype(np.float64))
        d_lo = a - lo
        d_hi = hi - a
    lo_odd = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 1
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)
    res = np.where(take_hi, hi_bits, lo_bits)
    res = np.where(np.isinf(x32), np.uint32(0x7F800000), res)  # inf stays inf
    out = ((res | sign) >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(x32)] = BF16_CANONICAL_NAN
    return out


# ---------------------------------------------------------------------------
# Block dequant.  FastVideo PR #1829, "Purpose" and "Changes":
#   W_hat[n,k] = bf16( fl32( e4m3(Q[n,k]) * S[n//128, k//128] ) )
# The scale grid is expanded over its blocks and trimmed to [N,K] (the
# broadcast form the tests bullet compares against), multiplied in fp32,
# then rounded to bf16: two roundings, in that order.
# ---------------------------------------------------------------------------

def scale_grid_shape(n: int, k: int) -> tuple[int, int]:
    """[ceil(N/128), ceil(K/128)]; the last row/column block may be partial."""
    return (-(-n // BLOCK), -(-k // BLOCK))


def _expand_scales(scale_inv: np.ndarray, n: int, k: int) -> np.ndarray:
    s = np.asarray(scale_inv, dtype=np.float32)
    if s.shape != scale_grid_shape(n, k):
        raise ValueError(f"scale grid {s.shape} != {scale_grid_shape(n, k)}")
    return np.repeat(np.repeat(s, BLOCK, axis=0), BLOCK, axis=1)[:n, :k]


def dequant(q: np.ndarray, scale_inv: np.ndarray) -> np.ndarray:
    """Q uint8 [N,K], S fp32 [GN,GK] -> W_hat as bf16 bits uint16 [N,K]."""
    q = np.asarray(q, dtype=np.uint8)
    n, k = q.shape
    vals = e4m3_table().astype(np.float32)[q]     # every E4M3 value is exact in fp32
    s_full = _expand_scales(scale_inv, n, k)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = vals * s_full                       # IEEE fp32 multiply, RNE, no FTZ
    return bf16_rne_bits(prod)


def dequant_rows(q: np.ndarray, scale_inv: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """The same definition restricted to the weight rows ``rows`` (for sampling)."""
    q = np.asarray(q, dtype=np.uint8)
    n, k = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    s = np.asarray(scale_inv, dtype=np.float32)
    if s.shape != scale_grid_shape(n, k):
        raise ValueError("scale grid shape")
    vals = e4m3_table().astype(np.float32)[q[rows]]
    s_rows = np.repeat(s[rows // BLOCK], BLOCK, axis=1)[:, :k]
    with np.errstate(invalid="ignore", over="ignore"):
        prod = vals * s_rows
    return bf16_rne_bits(prod)


# ---------------------------------------------------------------------------
# Block quantize.  FastVideo PR #1829, "Changes", converter bullet (E4M3
# weight plus weight_scale_inv per 128x128 block). Reading of the unstated
# arithmetic: S = fl32(amax / 448) over the present elements of the block
# (1.0 for an all-zero block); v = fl32(w / S); the code is the nearest
# finite E4M3 value, ties to the even code, saturating at +-448, sign kept.
# ---------------------------------------------------------------------------

def e4m3_encode_nearest(v: np.ndarray) -> np.ndarray:
    """Encode fp32 values by searching the sorted table of the 127
    non-negative finite codes (0x00..0x7E) for the nearest one."""
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("encoder input must be finite")
    mags = e4m3_table()[:0x7F]                     # strictly increasing
    a = np.abs(v.astype(np.float64))
    idx = np.searchsorted(mags, a, side="left")    # first code with value >= a
    hi = np.minimum(idx, 0x7E)
    lo = np.maximum(idx - 1, 0)
    d_lo = a - mags[lo]                             # exact in fp64
    d_hi = mags[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)      # saturate at +-448
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def e4m3_encode_bits(v: np.ndarray) -> np.ndarray:
    """Second encoder, for cross-checking only: round the fp32 significand to
    3 bits (normal range) or |v| * 2^9 to an integer (subnormal range)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("encoder input must be finite")
    u = v.view(np.uint32)
    mag = (u & np.uint32(0x7FFFFFFF)).astype(np.int64)
    sign = (u >> np.uint32(31)).astype(np.int64) << 7
    a = np.abs(v.astype(np.float64))
    sub = np.rint(a * 512.0).astype(np.int64)               # exact product; rint is RNE
    normal = ((mag + 0x7FFFF + ((mag >> 20) & 1)) >> 20) - (120 << 3)
    code = np.where(a < 2.0 ** -6, sub, normal)
    code = np.minimum(code, 0x7E)
    return (code | sign).astype(np.uint8)


def quantize(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp32 W [N,K] -> (Q uint8 [N,K], S fp32 [GN,GK]). W must be finite."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    gn, gk = scale_grid_shape(n, k)
    q = np.empty((n, k), dtype=np.uint8)
    s = np.empty((gn, gk), dtype=np.float32)
    for i in range(gn):
        for j in range(gk):
            rs = slice(i * BLOCK, min((i + 1) * BLOCK, n))
            cs = slice(j * BLOCK, min((j + 1) * BLOCK, k))
            blk = w[rs, cs]
            amax = np.float32(np.max(np.abs(blk)))
            if amax == 0:
                sc = np.float32(1.0)
            else:
                sc = np.float32(amax / np.float32(E4M3_MAX))  # fp32 IEEE division
            s[i, j] = sc
            q[rs, cs] = e4m3_encode_nearest(blk / sc)        # fp32 IEEE division
    return q, s


def quantize_bf16(w_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The converter reading a bf16 weight: every bf16 value is exactly an
    fp32 value, so the block quantization is the fp32 one on the widened
    weight."""
    return quantize(bf16_bits_to_f32(w_bits))


# ---------------------------------------------------------------------------
# Linear.  FastVideo PR #1829, "Purpose": an ordinary matmul with the
# dequantized bf16 weight, Y = X W_hat^T; LightX2V PR #1657 "Walkthrough": accumulation in
# FP32 (the GPU side). The oracle forms the exact-arithmetic target in fp64
# and grades against it with the stated bound
#   |y - Y*| <= 2^-7 |Y*| + 1e-4 * sum_k |x_k w_k|.
# ---------------------------------------------------------------------------

def linear_exact(x_bits: np.ndarray, w_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """X bf16 bits [M,K], W_hat bf16 bits [N,K] -> (Y* fp64 [M,N], A fp64 [M,N])
    with A = sum_k |X[m,k] W_hat[n,k]|."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    y = x @ w.T
    a = np.abs(x) @ np.abs(w).T
    return y, a


def linear_value(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Y* = X W_hat^T in fp64 alone (no A), for preparing derived inputs."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    return x @ w.T


def linear_sampled(x_bits: np.ndarray, q: np.ndarray, scale_inv: np.ndarray,
                   ms: np.ndarray, ns: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Y*[ms[i], ns[i]] and A[ms[i], ns[i]] one output at a time (fp64), for
    shapes too large for the full product."""
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    x = bf16_bits_to_f32(np.asarray(x_bits)[ms]).astype(np.float64)
    w = bf16_bits_to_f32(dequant_rows(q, scale_inv, ns)).astype(np.float64)
    y = np.einsum("pk,pk->p", x, w)
    a = np.einsum("pk,pk->p", np.abs(x), np.abs(w))
    return y, a


def gemm_bound_ratio(y_bits: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray) -> np.ndarray:
    """|y - Y*| / (2^-7 |Y*| + 1e-4 A), elementwise; <= 1 passes.

    Where the tolerance is zero (all products zero) the ratio is 0 if y is
    zero and inf otherwise. A NaN or infinite y gives inf.
    """
    y = bf16_bits_to_f32(y_bits).astype(np.float64)
    tol = 2.0 ** -7 * np.abs(y_ref) + 1e-4 * a_ref
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0),
                         np.where(err == 0, 0.0, np.inf))
    ratio = np.where(np.isfinite(y), ratio, np.inf)
    return ratio


def linear_bf16(x_bits: np.ndarray, q: np.ndarray, scale_inv: np.ndarray) -> np.ndarray:
    """A representative correct output: bf16 bits of the exact Y* (rounded
    through fp32, i.e. within the bound)."""
    y, _ = linear_exact(x_bits, dequant(q, scale_inv))
    return bf16_rne_bits(y.astype(np.float32))


def swiglu_bf16(g_bits: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """Input of the MLP down projection, rounded where eager bf16 ops round
    (FastVideo fasth3_omniref_b200 README, "What --lossless-accel turns on"):
    h = bf16( bf16(silu(g)) * u ), silu(g) = g / (1 + e^-g) evaluated in fp64
    and rounded to fp32 and then to bf16; the product of two bf16 values is
    exact in fp32 and rounded once to bf16."""
    g = bf16_bits_to_f32(g_bits).astype(np.float64)
    u = bf16_bits_to_f32(u_bits)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    silu_b = bf16_bits_to_f32(bf16_rne_bits(silu.astype(np.float32)))
    return bf16_rne_bits(silu_b * u)


# ---------------------------------------------------------------------------
# Gate/up pair with the SwiGLU epilogue (one launch on the GPU). Target:
# h* = silu(G*) U* in fp64 from the exact gate and up products. The GPU's h
# differs from it by the two GEMM errors carried through SwiGLU plus two bf16
# roundings; the bound below adds them up.
# ---------------------------------------------------------------------------

SILU_SLOPE_MAX = 1.1  # max |d silu / dx| = 1.0998... (at x ~ 2.3994)


def silu_exact(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + e^-g) in fp64 (0 for g -> -inf)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_bound_ratio(h_bits: np.ndarray, g_ref: np.ndarray, a_g: np.ndarray,
                       u_ref: np.ndarray, a_u: np.ndarray) -> np.ndarray:
    """|h - silu(G*) U*| / tol, elementwise; <= 1 passes.

    With each GEMM error E = 2^-7 |Y*| + 1e-4 A (the linear's bound) and
    s = |silu(G*)| + 1.1 E_g, v = |U*| + E_u:
      tol = 1.1 E_g v + s E_u + 2^-6 s v
    The first two terms carry the gate and up errors through silu (slope at
    most 1.1) and the product; 2^-6 s v covers bf16 rounding of silu (one ulp,
    2^-7 relative, allowing the fp32 evaluation to land on the other side of
    a tie) and of the product (half an ulp), with room to spare. A NaN or
    infinite h gives inf; where tol is zero, h must be zero.
    """
    h = bf16_bits_to_f32(h_bits).astype(np.float64)
    e_g = 2.0 ** -7 * np.abs(g_ref) + 1e-4 * a_g
    e_u = 2.0 ** -7 * np.abs(u_ref) + 1e-4 * a_u
    s = np.abs(silu_exact(g_ref)) + SILU_SLOPE_MAX * e_g
    v = np.abs(u_ref) + e_u
    tol = SILU_SLOPE_MAX * e_g * v + s * e_u + 2.0 ** -6 * s * v
    err = np.abs(h - silu_exact(g_ref) * u_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0),
                         np.where(err == 0, 0.0, np.inf))
    return np.where(np.isfinite(h), ratio, np.inf)


# ---------------------------------------------------------------------------
# W8A8 variant (both operands E4M3). FastVideo PR #1829, "Changes", first
# bullet: on Blackwell the loader also needs a Triton quantizer next to the
# FlashInfer groupwise GEMM. The pages do not say what that quantizer does;
# the reading taken here is per-token activation quantization in 1x128
# groups along K, with the weight's own arithmetic (S = fl32(amax / 448),
# 1.0 for an all-zero group, nearest finite E4M3 of fl32(x / S)), and a GEMM
# that multiplies E4M3 codes exactly and applies x_scale * w_scale to the
# sum of each 128-wide K block. Activation scales are stored K-block-major,
# x_scale[GK, M], so that one K block's scales for consecutive rows are
# contiguous.
# ---------------------------------------------------------------------------

def act_quantize(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 X bits [M,K] -> (XQ uint8 [M,K], x_scale fp32 [GK, M]).

    Every 1x128 group of a row (the last one may be shorter) gets its own
    scale S = fl32(amax / 448) (1.0 if the group is all zero) and codes
    e4m3_nearest(fl32(x / S)). X must be finite."""
    x = bf16_bits_to_f32(np.asarray(x_bits))
    if not np.all(np.isfinite(x)):
        raise ValueError("activation must be finite")
    m, k = x.shape
    gk = (k + BLOCK - 1) // BLOCK
    xq = np.empty((m, k), dtype=np.uint8)
    xs = np.empty((gk, m), dtype=np.float32)
    for j in range(gk):
        cs = slice(j * BLOCK, min((j + 1) * BLOCK, k))
        grp = x[:, cs]                                          # [M, <=128]
        amax = np.max(np.abs(grp), axis=1).astype(np.float32)   # per row
        sc = np.where(amax == 0, np.float32(1.0),
                      (amax / np.float32(E4M3_MAX)).astype(np.float32)).astype(np.float32)
        xs[j] = sc
        xq[:, cs] = e4m3_encode_nearest((grp / sc[:, None]).astype(np.float32))
    return xq, xs


def act_dequant_f64(xq: np.ndarray, x_scale: np.ndarray) -> np.ndarray:
    """XQ [M,K] and x_scale [GK,M] -> the exact values e4m3(XQ) * S in fp64."""
    m, k = xq.shape
    t = e4m3_table()[xq]
    s = np.repeat(np.asarray(x_scale, np.float64).T, BLOCK, axis=1)[:, :k]
    return t * s


def weight_dequant_f64(q: np.ndarray, scale_inv: np.ndarray) -> np.ndarray:
    """Q [N,K] and S [GN,GK] -> the exact values e4m3(Q) * S in fp64 (no bf16
    rounding: in the W8A8 product the codes meet the scales only after the
    exact per-block sums)."""
    n, k = q.shape
    return e4m3_table()[q] * _expand_scales(scale_inv, n, k).astype(np.float64)


def linear_w8a8_exact(xq: np.ndarray, x_scale: np.ndarray, q: np.ndarray,
                      scale_inv: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Y*[m,n] = sum_kb x_scale[kb,m] S[n/128,kb] sum_{k in kb} e4m3(XQ[m,k]) e4m3(Q[n,k])
    in fp64, and A = the same sum over absolute values."""
    xv = act_dequant_f64(xq, x_scale)
    wv = weight_dequant_f64(q, scale_inv)
    return xv @ wv.T, np.abs(xv) @ np.abs(wv).T


def linear_w8a8_sampled(xq: np.ndarray, x_scale: np.ndarray, q: np.ndarray,
                        scale_inv: np.ndarray, ms: np.ndarray, ns: np.ndarray
                        ) -> tuple[np.ndarray, np.ndarray]:
    """Y*[ms[i], ns[i]] and A[ms[i], ns[i]] one output at a time (fp64)."""
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    n, k = q.shape
    gk = (k + BLOCK - 1) // BLOCK
    xv = e4m3_table()[np.asarray(xq)[ms]] * np.repeat(
        np.asarray(x_scale, np.float64)[:, ms].T, BLOCK, axis=1)[:, :k]
    wrows = np.asarray(q)[ns]
    srows = np.asarray(scale_inv, np.float64)[ns // BLOCK]           # [P, GK]
    wv = e4m3_table()[wrows] * np.repeat(srows, BLOCK, axis=1)[:, :k]
    assert srows.shape[1] == gk
    return np.einsum("pk,pk->p", xv, wv), np.einsum("pk,pk->p", np.abs(xv), np.abs(wv))
