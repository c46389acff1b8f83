"""Seeded random ragged shapes through every entry point, against the oracle.

The other parity files use fixed shape lists chosen by hand. This one draws
M, N and K at random (K a multiple of 16, the format's only constraint on
the reduction length) so that partial tiles, partial 128-blocks, odd N and
every M below and above the skinny threshold are hit in combinations nobody
picked. Each case prints its seed and shape before any GPU work.

Bars: dequant, both quantizers and the activation quantizer bit for bit;
the linears within |y - Y*| <= 2^-7 |Y*| + 1e-4 sum |x w| of the oracle's
fp64 Y*; the gated MLP within the SwiGLU bound built from the same two sums.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from workloads import random_problem  # noqa: E402

from gpu_util import bits, f32, say, to_bf16, to_f32, to_u8, u8  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

import block_scaled_fp8_linear_amd as F  # noqa: E402

N_CASES = 24


def _shape(seed):
    """M in [1, 600] (half the cases at M <= 32), N in [1, 1200], K in 16 * [1, 160]."""
    rng = np.random.default_rng(10_000 + seed)
    m = int(rng.integers(1, 33)) if seed % 2 == 0 else int(rng.integers(33, 601))
    n = int(rng.integers(1, 1201))
    k = 16 * int(rng.integers(1, 161))
    return m, n, k


CASES = [(seed, *_shape(seed)) for seed in range(N_CASES)]
IDS = [f"s{seed}-{m}x{n}x{k}" for seed, m, n, k in CASES]


def test_case_list_spans_the_regimes():
    ms = [m for _, m, _, _ in CASES]
    ns = [n for _, _, n, _ in CASES]
    ks = [k for _, _, _, k in CASES]
    assert min(ms) <= 32 < max(ms)
    assert any(n % 128 for n in ns) and any(k % 128 for k in ks)
    assert max(ns) > 256 and max(ks) > 512


def _assert_ratio(ratio, label):
    worst = float(ratio.max()) if ratio.size else 0.0
    say(label, "max bound ratio", worst)
    assert worst <= 1.0, (label, worst, np.unravel_index(np.argmax(ratio), ratio.shape))


@pytest.mark.parametrize("seed,m,n,k", CASES, ids=IDS)
def test_random_quantize_dequant(seed, m, n, k):
    _, w = random_problem(seed, m, n, k)
    say("random quantize/dequant", seed, n, k)
    qg, sg = F.fp8_block_quantize(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = O.quantize(w)
    assert np.array_equal(u8(qg), q_ref)
    assert np.array_equal(f32(sg).view(np.uint32), s_ref.view(np.uint32))
    wd = F.fp8_block_dequant(to_u8(q_ref), to_f32(s_ref))
    assert np.array_equal(bits(wd), O.dequant(q_ref, s_ref))
    # a bf16 checkpoint: the high halves of the same fp32 patterns
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    qb, sb = F.fp8_block_quantize(to_bf16(wb))
    torch.cuda.synchronize()
    qb_ref, sb_ref = O.quantize(O.bf16_bits_to_f32(wb))
    assert np.array_equal(u8(qb), qb_ref)
    assert np.array_equal(f32(sb).view(np.uint32), sb_ref.view(np.uint32))


@pytest.mark.parametrize("path", ["tiled", "skinny"])
@pytest.mark.parametrize("seed,m,n,k", CASES, ids=IDS)
def test_random_linear(seed, m, n, k, path):
    x, w = random_problem(seed, m, n, k)
    q, s = O.quantize(w)
    say("random linear", path, seed, m, n, k)
    mode = F.PATH_TILED if path == "tiled" else F.PATH_SKINNY
    y = F.fp8_block_linear(to_bf16(x), to_u8(q), to_f32(s), path=mode)
    torch.cuda.synchronize()
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    _assert_ratio(O.gemm_bound_ratio(bits(y), yr, ar), f"{path} s{seed} {m}x{n}x{k}")


@pytest.mark.parametrize("seed,m,n,k", CASES, ids=IDS)
def test_random_mlp_gate_up(seed, m, n, k):
    x, wg = random_problem(seed, m, n, k, w_std=0.05)
    _, wu = random_problem(seed + 5000, m, n, k, w_std=0.05)
    qg, sg = O.quantize(wg)
    qu, su = O.quantize(wu)
    say("random mlp gate/up", seed, m, n, k)
    h = F.fp8_block_mlp_gate_up(to_bf16(x), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
    torch.cuda.synchronize()
    g, ag = O.linear_exact(x, O.dequant(qg, sg))
    u, au = O.linear_exact(x, O.dequant(qu, su))
    _assert_ratio(O.swiglu_bound_ratio(bits(h), g, ag, u, au), f"mlp s{seed} {m}x{n}x{k}")


@pytest.mark.parametrize("seed,m,n,k", CASES, ids=IDS)
def test_random_w8a8(seed, m, n, k):
    x, w = random_problem(seed, m, n, k)
    q, s = O.quantize(w)
    say("random w8a8", seed, m, n, k)
    xq, xs = F.fp8_act_quantize(to_bf16(x))
    torch.cuda.synchronize()
    xq_ref, xs_ref = O.act_quantize(x)
    assert np.array_equal(u8(xq), xq_ref)
    assert np.array_equal(f32(xs).view(np.uint32), xs_ref.view(np.uint32))
    y = F.fp8_block_linear_w8a8(to_u8(xq_ref), to_f32(xs_ref), to_u8(q), to_f32(s))
    y2 = F.fp8_block_linear_w8a8_bf16(to_bf16(x), to_u8(q), to_f32(s))
    torch.cuda.synchronize()
    yr, ar = O.linear_w8a8_exact(xq_ref, xs_ref, q, s)
    _assert_ratio(O.gemm_bound_ratio(bits(y), yr, ar), f"w8a8 s{seed} {m}x{n}x{k}")
    assert np.array_equal(bits(y2), bits(y))
