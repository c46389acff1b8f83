"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself (closed forms, exact rational arithmetic, exhaustive or
structured enumeration, hand-worked values, host library routines). Some
tests plant a mistake in a copy of an oracle step to show the pin catches it.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import generate, random_problem


def f32_from_bits(b):
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------------------
# E4M3 decode table
# ---------------------------------------------------------------------------

def test_e4m3_closed_form_facts():
    t = O.e4m3_table()
    nan_codes = [c for c in range(256) if math.isnan(t[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9           # subnormal step
    assert t[0x08] == 2.0 ** -6           # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9       # largest subnormal
    assert t[0x38] == 1.0
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)       # strictly increasing over 0x00..0x7E
    for c in range(0x7F):
        assert t[c | 0x80] == -t[c]
    finite = t[np.isfinite(t)]
    assert finite.size == 254
    assert np.unique(finite).size == 253  # +0 and -0 coincide


def test_e4m3_enumeration_by_binade():
    """Independent construction: 8 subnormals, 14 full binades of 8, and the
    top binade with its last (NaN) slot removed: 127 non-negative codes."""
    vals = [Fraction(m, 512) for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    assert len(vals) == 127
    t = O.e4m3_table()
    assert [Fraction(float(v)) for v in t[:0x7F]] == vals


def test_e4m3_values_exact_in_bf16():
    t = O.e4m3_table()
    finite = t[np.isfinite(t)].astype(np.float32)
    assert np.array_equal(O.bf16_bits_to_f32(O.bf16_rne_bits(finite)), finite)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = O.e4m3_table()
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    fin = ~np.isnan(t)
    assert np.array_equal(ref[fin], t[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(t[fin]))


# ---------------------------------------------------------------------------
# bf16 round to nearest even
# ---------------------------------------------------------------------------

def _structured_f32_patterns():
    """Every (sign, exponent, top-7-mantissa) prefix with 16 chosen low
    halves (exact zero, the tie, one either side of it, the extremes...)."""
    highs = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0x8002,
                     0xBFFF, 0xFFFE, 0xFFFF, 0x1234, 0x4000, 0xC000, 0x00FF, 0xFF00],
                    dtype=np.uint32)
    return (highs[:, None] | lows[None, :]).ravel()


def test_bf16_two_implementations_agree_structured():
    pats = _structured_f32_patterns()
    rng = np.random.default_rng(123)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint32)])
    x = pats.view(np.float32)
    a = O.bf16_rne_bits(x)
    b = O.bf16_rne_bits_nearest(x)
    assert np.array_equal(a, b)


@pytest.mark.skipif(os.environ.get("FP8BL_EXHAUSTIVE") != "1",
                    reason="all 2^32 fp32 patterns; set FP8BL_EXHAUSTIVE=1 (minutes)")
def test_bf16_two_implementations_agree_exhaustive():
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        pats = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        x = pats.view(np.float32)
        assert np.array_equal(O.bf16_rne_bits(x), O.bf16_rne_bits_nearest(x)), hex(start)


@pytest.mark.skipif(os.environ.get("FP8BL_EXHAUSTIVE") != "1",
                    reason="all fp32 patterns with |v| <= 480; set FP8BL_EXHAUSTIVE=1 (minutes)")
def test_e4m3_two_encoders_agree_exhaustive():
    """Table search and bit manipulation give the same code for every fp32
    bit pattern of magnitude <= 480 (both signs): past 448 both saturate."""
    top = int(np.array([480.0], np.float32).view(np.uint32)[0])
    step = 1 << 24
    for sign in (0, 0x80000000):
        for start in range(0, top + 1, step):
            stop = min(start + step, top + 1)
            pats = (np.arange(start, stop, dtype=np.uint64) | sign).astype(np.uint32)
            v = pats.view(np.float32)
            a, b = O.e4m3_encode_nearest(v), O.e4m3_encode_bits(v)
            assert np.array_equal(a, b), (hex(sign), hex(start), np.argwhere(a != b)[:3])


def test_bf16_spot_values():
    cases = {
        0x3F800000: 0x3F80,   # 1.0
        0x3F808000: 0x3F80,   # tie, lower neighbour even
        0x3F818000: 0x3F82,   # tie, upper neighbour even
        0x3F808001: 0x3F81,   # just above the tie
        0x3F807FFF: 0x3F80,   # just below the tie
        0x80000000: 0x8000,   # -0
        0x00000000: 0x0000,
        0x7F7FFFFF: 0x7F80,   # largest fp32 rounds to +inf
        0x7F7F7FFF: 0x7F7F,   # stays finite
        0x7F7F8000: 0x7F80,   # tie at the top, odd lower -> inf
        0xFF7F8000: 0xFF80,
        0x00008000: 0x0000,   # subnormal tie to even (zero)
        0x00018000: 0x0002,   # subnormal tie to even (2)
        0x00010000: 0x0001,   # smallest bf16 subnormal
        0x7F800000: 0x7F80,   # +inf
        0xFF800000: 0xFF80,   # -inf
        0x7FC00001: 0x7FC0,   # NaN -> canonical
        0xFFFFFFFF: 0x7FC0,
    }
    x = np.array(list(cases.keys()), dtype=np.uint32).view(np.float32)
    exp = np.array(list(cases.values()), dtype=np.uint16)
    assert np.array_equal(O.bf16_rne_bits(x), exp)
    assert np.array_equal(O.bf16_rne_bits_nearest(x), exp)


def test_bf16_matches_torch_cast_on_finite():
    torch = pytest.importorskip("torch")
    pats = _structured_f32_patterns()
    x = pats.view(np.float32)
    keep = ~np.isnan(x)
    x = x[keep]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_rne_bits(x), ref)


# ---------------------------------------------------------------------------
# Dequant
# ---------------------------------------------------------------------------

def _exact_dequant_one(code, scale32):
    """R(fl32(e4m3(code) * s)): the fp64 product of a 4-bit and a 24-bit
    significand is exact (or an exact overflow/underflow-free value), then one
    rounding to fp32 and the second bf16 implementation."""
    v = O.e4m3_value(code)
    s = float(scale32)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.float32(v * s)
    return int(O.bf16_rne_bits_nearest(np.array([p], dtype=np.float32))[0])


def _scale_set():
    rng = np.random.default_rng(7)
    s = [1.0, 0.5, 2.0, 3.0, 1.0 / 448, 0.02 / 448, 1e-3, 7.5e-5]
    s += [2.0 ** e for e in range(-30, 31, 3)]
    s += list(rng.uniform(1e-6, 1e-2, size=40))
    s += list(rng.standard_normal(10) * 1e-3)            # negative scales too
    s += [2.0 ** -127, 2.0 ** -140, 2.0 ** -149, 1e-39]  # subnormal scales
    s += [2.0 ** 120, 3.0e38]                            # overflow for big codes
    s += [f32_from_bits(0x3FEB8E39), f32_from_bits(0x3DCCCCCD)]
    s += [math.inf, 0.0, -0.0, math.nan]
    return np.array(s, dtype=np.float32)


def test_dequant_exhaustive_codes_times_scales():
    scales = _scale_set()
    codes = np.arange(256, dtype=np.uint8)
    for s in scales:
        q = codes.reshape(1, 256)
        got = O.dequant(q, np.full((1, 2), s, dtype=np.float32))[0]
        exp = np.array([_exact_dequant_one(c, s) for c in range(256)], dtype=np.uint16)
        assert np.array_equal(got, exp), (float(s), np.nonzero(got != exp))


def test_dequant_golden_worked_examples(golden_dir):
    path = os.path.join(golden_dir, "dequant_worked_examples.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, sbits, want = (int(t, 16) for t in line.split()[:3])
        got = O.dequant(np.array([[code]], dtype=np.uint8),
                        np.array([[f32_from_bits(sbits)]], dtype=np.float32))
        assert int(got[0, 0]) == want, (hex(code), hex(sbits), hex(int(got[0, 0])), hex(want))
        n += 1
    assert n >= 10


def test_dequant_power_of_two_scales_are_exact_and_follow_blocks():
    """A ragged grid where each block has its own power-of-two scale: every
    element must equal e4m3(code) * 2^j exactly, with j taken from the block
    (n//128, k//128). A transposed or shifted grid fails this."""
    n, k = 300, 272                       # 3x3 grid, partial last row and column block
    gn, gk = O.scale_grid_shape(n, k)
    assert (gn, gk) == (3, 3)
    exps = np.arange(gn * gk).reshape(gn, gk) - 4
    s = (2.0 ** exps).astype(np.float32)
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11          # no NaN codes here
    got = O.bf16_bits_to_f32(O.dequant(q, s)).astype(np.float64)
    t = O.e4m3_table()
    for i in range(n):
        for j in range(0, k, 17):
            assert got[i, j] == t[q[i, j]] * 2.0 ** exps[i // 128, j // 128]


def test_dequant_matches_torch_reference_broadcast():
    """The broadcast comparison taken literally: decode with the library's
    float8_e4m3fn, expand the scale grid, multiply in fp32, cast to bf16."""
    torch = pytest.importorskip("torch")
    wl = generate("tiny")
    lin = wl.linears[0]
    q, s = O.quantize(lin.w)
    qt = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
    st = torch.from_numpy(s).repeat_interleave(128, 0).repeat_interleave(128, 1)[: q.shape[0], : q.shape[1]]
    ref = (qt * st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.dequant(q, s), ref)
    # ragged shape with random codes and random scales
    rng = np.random.default_rng(11)
    q = rng.integers(0, 256, size=(200, 144), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    s = rng.uniform(1e-5, 1e-1, size=(2, 2)).astype(np.float32)
    qt = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
    st = torch.from_numpy(s).repeat_interleave(128, 0).repeat_interleave(128, 1)[:200, :144]
    ref = (qt * st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.dequant(q, s), ref)


def test_planted_single_rounding_is_caught():
    """Plant a mistake in a copy of the dequant step: round the exact product
    straight to bf16 (one rounding instead of fp32 then bf16). The exhaustive
    scale set must contain cases where the two differ."""
    mismatches = 0
    for s in _scale_set():
        if not np.isfinite(s) or s == 0:
            continue
        for c in range(256):
            if c & 0x7F == 0x7F:
                continue
            p = O.e4m3_value(c) * float(s)
            if p == 0 or not (2.0 ** -120 < abs(p) < 3.0e38):
                continue
            if _round_f64_to_bf16(p) != _exact_dequant_one(c, s):
                mismatches += 1
    assert mismatches > 0


def _round_f64_to_bf16(p):
    """Direct RNE of an fp64 value to bf16 (single rounding), by brute force
    over the two bf16 neighbours with exact rationals."""
    if p == 0:
        return 0x8000 if math.copysign(1, p) < 0 else 0
    f = Fraction(p)
    sgn = 0x8000 if p < 0 else 0
    a = abs(f)
    # find the bf16 pattern below a
    bits = int(np.array([abs(p)], dtype=np.float32).view(np.uint32)[0]) >> 16
    for b in (bits - 1, bits, bits + 1):
        lo = Fraction(float(O.bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0]))
        hi = Fraction(float(O.bf16_bits_to_f32(np.array([b + 1], dtype=np.uint16))[0]))
        if lo <= a < hi:
            if a - lo < hi - a or (a - lo == hi - a and b % 2 == 0):
                return sgn | b
            return sgn | (b + 1)
    raise AssertionError("neighbour search failed")


# ---------------------------------------------------------------------------
# Quantize
# ---------------------------------------------------------------------------

def _encode_probe_values():
    t = O.e4m3_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2                       # 5 significant bits: exact in fp32
    pts = np.concatenate([t, mids, [448.0, 456.0, 464.0, 470.0, 480.0]]).astype(np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    offs = np.arange(-40, 41)
    near = (bits[:, None] + offs[None, :]).ravel()
    near = near[(near >= 0) & (near <= 0x43F00000)].astype(np.uint32)
    rng = np.random.default_rng(5)
    rnd = rng.integers(0, 0x43F00001, size=3_000_000, dtype=np.uint32)
    sub = np.arange(0, 1 << 20, dtype=np.uint32)      # fp32 subnormals and tiny normals
    v = np.concatenate([near, rnd, sub]).view(np.float32)
    return np.concatenate([v, -v])


def test_encoders_agree():
    v = _encode_probe_values()
    assert np.array_equal(O.e4m3_encode_nearest(v), O.e4m3_encode_bits(v))


def test_encoder_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    v = _encode_probe_values()
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode_nearest(v), ref)


def test_encoder_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 464.0, 465.0, 1e6, -1e30, -0.0, 0.0, -1e-30, 1e-30,
                  2.0 ** -10, 2.0 ** -10 + 2.0 ** -30, 3 * 2.0 ** -10], dtype=np.float32)
    got = O.e4m3_encode_nearest(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80, 0x00,
                         0x00, 0x01, 0x02]


def test_quantize_scales_codes_and_round_trip():
    wl = generate("tiny")
    w = wl.linears[0].w
    q, s = O.quantize(w)
    assert s.shape == (3, 2)
    t = O.e4m3_table()
    assert not np.any((q & 0x7F) == 0x7F)             # never a NaN code
    for i in range(3):
        for j in range(2):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].astype(np.float64)
            qb = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert s[i, j] == 1.0 and np.all(qb == 0)
                continue
            # fl32(amax/448): fp64 quotient then fp32 is the correctly rounded
            # fp32 quotient (53 >= 2*24 + 2)
            assert s[i, j] == np.float32(amax / 448.0)
            assert np.any((qb & 0x7F) == 0x7E)
            recon = t[qb] * float(s[i, j])                 # exact in fp64
            # E4M3's normal range starts at 2^-6; below it the step is 2^-9
            normal = np.abs(blk) >= 2.0 ** -6 * float(s[i, j])
            assert np.all(np.abs(recon - blk)[normal] <= 2.0 ** -4 * np.abs(blk)[normal])
            assert np.all(np.abs(recon - blk)[~normal] <= 2.0 ** -10 * float(s[i, j]))
    # the zero block and the saturating block of this workload
    assert s[0, 0] == 1.0 and np.all(q[:128, :128] == 0)
    sat = q[256:384, 128:256]
    n_idx, k_idx = np.meshgrid(np.arange(256, 384), np.arange(128, 256), indexing="ij")
    assert np.all((sat[((n_idx + k_idx) % 2) == 0] & 0x7F) == 0x7E)


def test_quantize_ragged_grid_uses_present_elements_only():
    _, w = random_problem(9, 1, 200, 160)
    w[128:, :] *= 10.0                 # the partial last row block has its own amax
    q, s = O.quantize(w)
    assert s.shape == (2, 2)
    for i, rs in enumerate([slice(0, 128), slice(128, 200)]):
        for j, cs in enumerate([slice(0, 128), slice(128, 160)]):
            assert s[i, j] == np.float32(float(np.max(np.abs(w[rs, cs]))) / 448.0)


def test_full_round_trip_within_e4m3_precision():
    """Quantize then dequantize: within 2^-4 + 2^-8 relative for normal codes
    (the E4M3 step is bounded by 2^-4; the bf16 step adds at most 2^-8)."""
    _, w = random_problem(21, 1, 384, 512)
    q, s = O.quantize(w)
    wd = O.bf16_bits_to_f32(O.dequant(q, s)).astype(np.float64)
    s_full = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:384, :512]
    normal = np.abs(w) >= 2.0 ** -6 * s_full
    rel = np.abs(wd - w)[normal] / np.abs(w.astype(np.float64))[normal]
    assert rel.max() <= 2.0 ** -4 + 2.0 ** -8


def test_quantize_bf16_input_pins():
    """bf16 weights: the widening used by the oracle agrees with the
    library's bfloat16 -> float32 cast, and the quantized blocks keep the
    invariants (scale = fl32(amax/448), a +-448 code per non-zero block)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    w32 = (rng.standard_normal((200, 272)) * 0.05).astype(np.float32)
    bits = O.bf16_rne_bits(w32)
    widened = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(widened.view(np.uint32), O.bf16_bits_to_f32(bits).view(np.uint32))
    q, s = O.quantize_bf16(bits)
    q2, s2 = O.quantize(widened)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    for i in range(2):
        for j in range(3):
            blk = widened[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].astype(np.float64)
            assert s[i, j] == np.float32(np.max(np.abs(blk)) / 448.0)
            assert np.any((q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] & 0x7F) == 0x7E)


# ---------------------------------------------------------------------------
# Linear (fp64 matmul) and the bound
# ---------------------------------------------------------------------------

def _bf16_fraction(bits):
    return Fraction(float(O.bf16_bits_to_f32(np.array([bits], dtype=np.uint16))[0]))


@pytest.mark.parametrize("m,n,k", [(3, 5, 16), (8, 8, 32), (16, 12, 48)])
def test_linear_exact_brute_force(m, n, k):
    x, w = random_problem(m * 100 + n, m, n, k, w_std=0.5)
    q, s = O.quantize(w)
    wb = O.dequant(q, s)
    y, a = O.linear_exact(x, wb)
    u = 2.0 ** -53
    for i in range(m):
        for j in range(n):
            ex = sum(_bf16_fraction(x[i, kk]) * _bf16_fraction(wb[j, kk]) for kk in range(k))
            ab = sum(abs(_bf16_fraction(x[i, kk]) * _bf16_fraction(wb[j, kk])) for kk in range(k))
            assert abs(Fraction(y[i, j]) - ex) <= k * u * ab
            assert abs(Fraction(a[i, j]) - ab) <= k * u * ab


def test_planted_transpose_is_caught():
    """A copy of the linear step that forgets the transpose (X W instead of
    X W^T, square shapes so it runs) must fail the brute-force comparison."""
    x, w = random_problem(5, 16, 16, 16, w_std=0.5)
    q, s = O.quantize(w)
    wb = O.dequant(q, s)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    wf = O.bf16_bits_to_f32(wb).astype(np.float64)
    wrong = xf @ wf
    exact = np.array([[float(sum(_bf16_fraction(x[i, kk]) * _bf16_fraction(wb[j, kk])
                                 for kk in range(16))) for j in range(16)] for i in range(16)])
    assert not np.allclose(wrong, exact)
    y, _ = O.linear_exact(x, wb)
    assert np.allclose(y, exact, rtol=0, atol=1e-12)


def test_linear_sampled_agrees_with_full():
    x, w = random_problem(8, 20, 300, 256)
    q, s = O.quantize(w)
    y, a = O.linear_exact(x, O.dequant(q, s))
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 20, 50)
    ns = rng.integers(0, 300, 50)
    assert np.array_equal(O.linear_value(x, O.dequant(q, s)), y)
    ys, as_ = O.linear_sampled(x, q, s, ms, ns)
    assert np.allclose(ys, y[ms, ns], rtol=1e-13, atol=1e-13)
    assert np.allclose(as_, a[ms, ns], rtol=1e-13, atol=1e-13)


def test_bound_accepts_rounded_and_rejects_wrong():
    x, w = random_problem(4, 32, 64, 256)
    q, s = O.quantize(w)
    y, a = O.linear_exact(x, O.dequant(q, s))
    yb = O.linear_bf16(x, q, s)
    assert O.gemm_bound_ratio(yb, y, a).max() <= 1.0
    # a dropped k-block (the last 128 of K) must fail somewhere
    y2, _ = O.linear_exact(x[:, :128], O.dequant(q, s)[:, :128])
    bad = O.bf16_rne_bits(y2.astype(np.float32))
    assert O.gemm_bound_ratio(bad, y, a).max() > 1.0
    # sign flip fails
    assert O.gemm_bound_ratio(bad ^ np.uint16(0x8000), y, a).max() > 1.0
    # zero inputs: tolerance zero, only zero passes
    z = np.zeros((2, 2))
    assert O.gemm_bound_ratio(np.zeros((2, 2), np.uint16), z, z).max() == 0.0
    assert O.gemm_bound_ratio(np.full((2, 2), 0x3F80, np.uint16), z, z).max() == np.inf


# ---------------------------------------------------------------------------
# SwiGLU helper (input preparation for the MLP down projection)
# ---------------------------------------------------------------------------

def test_swiglu_against_torch_and_closed_form():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    g = O.bf16_rne_bits(rng.standard_normal(20000).astype(np.float32) * 4)
    u = O.bf16_rne_bits(rng.standard_normal(20000).astype(np.float32))
    h = O.swiglu_bf16(g, u)
    gt = torch.from_numpy(O.bf16_bits_to_f32(g).astype(np.float64))
    silu = torch.nn.functional.silu(gt).to(torch.float32).to(torch.bfloat16)
    ref = (silu * torch.from_numpy(O.bf16_bits_to_f32(u)).to(torch.bfloat16))
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)
    # silu(0) = 0
    assert O.swiglu_bf16(np.array([0], np.uint16), np.array([0x3F80], np.uint16))[0] == 0


# ---------------------------------------------------------------------------
# SwiGLU target and bound (gate/up pair in one launch)
# ---------------------------------------------------------------------------

def test_silu_exact_closed_forms_and_torch():
    torch = pytest.importorskip("torch")
    x = np.linspace(-40.0, 40.0, 8001)
    s = O.silu_exact(x)
    # silu(x) - silu(-x) = x, silu(0) = 0, silu(x) -> x and -> 0 in the tails
    assert np.allclose(s - O.silu_exact(-x), x, rtol=0, atol=1e-12)
    assert O.silu_exact(np.array([0.0]))[0] == 0.0
    assert abs(O.silu_exact(np.array([40.0]))[0] - 40.0) < 1e-15 * 40 + 40 * np.exp(-40)
    assert O.silu_exact(np.array([-1e4]))[0] == 0.0
    assert np.allclose(s, torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-15, atol=0)


def test_silu_slope_bound():
    # d silu / dx = sig(x) (1 + x (1 - sig(x))) in closed form; its maximum is
    # about 1.0998 and its minimum about -0.0998, so 1.1 bounds |slope|.
    x = np.linspace(-30.0, 30.0, 600001)
    sig = 1.0 / (1.0 + np.exp(-x))
    d = sig * (1.0 + x * (1.0 - sig))
    assert np.abs(d).max() < O.SILU_SLOPE_MAX
    assert np.abs(d).max() > 1.09
    # and the secant slope never exceeds it either
    sl = np.abs(np.diff(O.silu_exact(x)) / np.diff(x))
    assert sl.max() < O.SILU_SLOPE_MAX


def _mlp_case(seed=5, m=48, n=96, k=512):
    rng = np.random.default_rng(seed)
    x = O.bf16_rne_bits(rng.standard_normal((m, k)).astype(np.float32))
    wg = O.bf16_rne_bits((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    wu = O.bf16_rne_bits((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    g, ag = O.linear_exact(x, wg)
    u, au = O.linear_exact(x, wu)
    # An fp32-accumulating emulation of the GPU side: fp32 matmul, bf16
    # outputs, then SwiGLU with the eager rounding points.
    xf = O.bf16_bits_to_f32(x)
    g32 = xf @ O.bf16_bits_to_f32(wg).T
    u32 = xf @ O.bf16_bits_to_f32(wu).T
    h = O.swiglu_bf16(O.bf16_rne_bits(g32.astype(np.float32)),
                      O.bf16_rne_bits(u32.astype(np.float32)))
    return x, wg, wu, g, ag, u, au, g32, u32, h


def test_swiglu_bound_accepts_fp32_emulation():
    *_, g, ag, u, au, g32, u32, h = _mlp_case()
    r = O.swiglu_bound_ratio(h, g, ag, u, au)
    assert r.max() <= 1.0
    # the bound is not vacuous: typical elements use a small part of it
    assert np.median(r) < 0.5


def test_swiglu_bound_rejects_planted_mistakes():
    *_, g, ag, u, au, g32, u32, h = _mlp_case()
    bf = lambda a: O.bf16_rne_bits(np.asarray(a, np.float32))  # noqa: E731
    gb, ub = bf(g32), bf(u32)
    wrong = {
        "gate and up swapped": O.swiglu_bf16(ub, gb),
        "silu dropped": bf(O.bf16_bits_to_f32(gb) * O.bf16_bits_to_f32(ub)),
        "sign flipped": bf(-O.bf16_bits_to_f32(h)),
        "sigmoid instead of silu": bf(1.0 / (1.0 + np.exp(-O.bf16_bits_to_f32(gb).astype(np.float64)))
                                      * O.bf16_bits_to_f32(ub)),
        "transposed output": h.T.copy() if h.shape[0] == h.shape[1] else h[:, ::-1].copy(),
    }
    for name, hb in wrong.items():
        assert O.swiglu_bound_ratio(hb, g, ag, u, au).max() > 1.0, name


def test_swiglu_bound_special_values():
    z = np.zeros((2, 2))
    zero = np.zeros((2, 2), np.uint16)
    assert O.swiglu_bound_ratio(zero, z, z, z, z).max() == 0.0
    one = np.full((2, 2), 0x3F80, np.uint16)
    assert O.swiglu_bound_ratio(one, z, z, z, z).max() == np.inf
    nan = np.full((2, 2), 0x7FC0, np.uint16)
    assert O.swiglu_bound_ratio(nan, z + 1, z + 1, z + 1, z + 1).max() == np.inf


# ---------------------------------------------------------------------------
# W8A8 variant: activation quantizer and the exact block-scaled product
# ---------------------------------------------------------------------------

def _bf16_rows(seed, m, k, scale=1.0):
    rng = np.random.default_rng(seed)
    return O.bf16_rne_bits((rng.standard_normal((m, k)) * scale).astype(np.float32))


def test_act_quantize_equals_weight_quantizer_per_row():
    # A [1,K] matrix's 128x128 blocks are exactly the 1x128 groups of that
    # row, so the (separately pinned) weight quantizer fixes every row.
    x = _bf16_rows(21, 9, 400, 3.0)
    x[2, 128:256] = 0                       # an all-zero group -> scale 1, codes 0
    x[4, :5] = 0x0001                       # subnormal bf16 values in a group
    xq, xs = O.act_quantize(x)
    assert xq.shape == (9, 400) and xs.shape == (4, 9)
    xf = O.bf16_bits_to_f32(x)
    for r in range(9):
        q, s = O.quantize(xf[r:r + 1])
        assert np.array_equal(xq[r], q[0]), r
        assert np.array_equal(xs[:, r], s[0]), r
    assert xs[1, 2] == 1.0 and np.all(xq[2, 128:256] == 0)


def test_act_quantize_group_max_hits_448_and_roundtrip():
    x = _bf16_rows(22, 16, 1024, 0.5)
    xq, xs = O.act_quantize(x)
    mag = xq & 0x7F
    for j in range(8):
        assert np.all(mag[:, j * 128:(j + 1) * 128].max(axis=1) == 0x7E)
    xv = O.act_dequant_f64(xq, xs)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    # normal range: |err| <= 2^-4 |x| (half of the 3-bit mantissa step);
    # subnormal range: |err| <= 2^-10 S (half the subnormal step 2^-9 S)
    s_full = np.repeat(xs.T.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(xv - xf) <= np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * s_full) * (1 + 1e-12))


def test_w8a8_product_exact_rational_brute_force():
    from fractions import Fraction
    rng = np.random.default_rng(23)
    m, n, k = 3, 130, 272                   # two N blocks, three K blocks (last ragged)
    xq = rng.integers(0, 256, (m, k)).astype(np.uint8)
    q = rng.integers(0, 256, (n, k)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3A          # no NaN codes
    q[(q & 0x7F) == 0x7F] = 0x41
    xs = rng.uniform(1e-3, 2.0, (3, m)).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-1, (2, 3)).astype(np.float32)
    y, a = O.linear_w8a8_exact(xq, xs, q, ws)
    tab = {c: Fraction(O.e4m3_value(c)) for c in range(256) if (c & 0x7F) != 0x7F}
    for mi in range(m):
        for ni in (0, 1, 127, 128, 129):
            tot, ab = Fraction(0), Fraction(0)
            for kb in range(3):
                part = sum((tab[xq[mi, kk]] * tab[q[ni, kk]]
                            for kk in range(kb * 128, min(kb * 128 + 128, k))), Fraction(0))
                pab = sum((abs(tab[xq[mi, kk]] * tab[q[ni, kk]])
                           for kk in range(kb * 128, min(kb * 128 + 128, k))), Fraction(0))
                sc = Fraction(float(xs[kb, mi])) * Fraction(float(ws[ni // 128, kb]))
                tot += sc * part
                ab += abs(sc) * pab
            assert abs(Fraction(y[mi, ni]) - tot) <= Fraction(1, 10 ** 12) * ab + Fraction(1, 10 ** 300)
            assert abs(Fraction(a[mi, ni]) - ab) <= Fraction(1, 10 ** 12) * ab
    # sampled form agrees with the full product
    ms = np.array([0, 2, 1]); ns = np.array([129, 0, 64])
    ys, as_ = O.linear_w8a8_sampled(xq, xs, q, ws, ms, ns)
    assert np.allclose(ys, y[ms, ns], rtol=1e-13, atol=0) and np.allclose(as_, a[ms, ns], rtol=1e-13)


def test_w8a8_reduces_to_w8a16_when_exact_in_bf16():
    # With power-of-two scales every e4m3 * scale is exact in bf16 (4-bit
    # significand), so the W8A8 target equals the W8A16 one on those values.
    rng = np.random.default_rng(24)
    m, n, k = 5, 140, 300
    xq = rng.integers(0, 0x7F, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) << 7).astype(np.uint8)
    q = rng.integers(0, 0x7F, (n, k)).astype(np.uint8)
    xs = (2.0 ** rng.integers(-8, 3, (3, m))).astype(np.float32)
    ws = (2.0 ** rng.integers(-12, -4, (2, 3))).astype(np.float32)
    x_bits = O.bf16_rne_bits(O.act_dequant_f64(xq, xs).astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(x_bits).astype(np.float64), O.act_dequant_f64(xq, xs))
    y8, a8 = O.linear_w8a8_exact(xq, xs, q, ws)
    y16, a16 = O.linear_exact(x_bits, O.dequant(q, ws))
    assert np.allclose(y8, y16, rtol=1e-14, atol=1e-300)
    assert np.allclose(a8, a16, rtol=1e-14, atol=1e-300)


def test_w8a8_planted_scale_mistakes_detected():
    rng = np.random.default_rng(25)
    m, n, k = 4, 256, 384
    x = _bf16_rows(26, m, k)
    xq, xs = O.act_quantize(x)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[:128] *= 8.0                          # the two N blocks get different scales
    q, ws = O.quantize(w)
    y, a = O.linear_w8a8_exact(xq, xs, q, ws)
    # the W8A8 target tracks the unquantized product within E4M3 error
    ref = O.bf16_bits_to_f32(x).astype(np.float64) @ w.astype(np.float64).T
    assert np.all(np.abs(y - ref) <= 0.15 * a)
    wrong_x = O.linear_w8a8_exact(xq, xs[::-1].copy(), q, ws)[0]        # K blocks swapped
    wrong_w = O.linear_w8a8_exact(xq, xs, q, ws[::-1].copy())[0]        # N blocks swapped
    for bad in (wrong_x, wrong_w):
        assert O.gemm_bound_ratio(O.bf16_rne_bits(bad.astype(np.float32)), y, a).max() > 1.0
