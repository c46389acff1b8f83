"""GPU parity of the gate/up pair with the SwiGLU epilogue (one launch),
through the C ABI, against the oracle's exact target silu(G*) U* and the
bound in ``oracle.swiglu_bound_ratio``. Weights are quantized by the oracle;
the gate and up products are the oracle's fp64 ones."""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from workloads import generate, random_problem  # noqa: E402

from gpu_util import bits, say, to_bf16, to_f32, to_u8  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

import block_scaled_fp8_linear_amd as F  # noqa: E402


def run_mlp(x_bits, qg, sg, qu, su, path=F.PATH_AUTO):
    h = F.fp8_block_mlp_gate_up(to_bf16(x_bits), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su),
                                path=path)
    torch.cuda.synchronize()
    return bits(h)


def _pair(seed, m, n, k):
    x, wg = random_problem(seed, m, n, k, w_std=0.05)
    _, wu = random_problem(seed + 1000, m, n, k, w_std=0.05)
    qg, sg = O.quantize(wg)
    qu, su = O.quantize(wu)
    return x, qg, sg, qu, su


def _check_full(x, qg, sg, qu, su, h, label):
    g, ag = O.linear_exact(x, O.dequant(qg, sg))
    u, au = O.linear_exact(x, O.dequant(qu, su))
    r = O.swiglu_bound_ratio(h, g, ag, u, au)
    worst = float(r.max()) if r.size else 0.0
    say(label, "max swiglu bound ratio", worst)
    assert worst <= 1.0, (label, worst, np.unravel_index(np.argmax(r), r.shape))


# The kernels evaluate silu in fp32 with the hardware exp2 and reciprocal:
# relative error at most (|g| + 4) 2^-23, below 2^-16 for every g >= -87. Past
# about -87 the exponential overflows fp32 and silu comes out as zero.
SILU_REL = 2.0 ** -16
SILU_ZERO_BELOW = -87.0


def _swiglu_consistent(h, g_bits, u_bits):
    """Where h can differ from the oracle's SwiGLU of the same bf16 g and u:
    only through the bf16 rounding of silu(g), which may land on the other
    neighbour when silu(g) is within SILU_REL of a rounding boundary. True
    where h is bf16(s' u) for s' a bf16 rounding of a value within SILU_REL of
    the exact silu(g), or zero for g below SILU_ZERO_BELOW."""
    g = O.bf16_bits_to_f32(g_bits).astype(np.float64)
    u = O.bf16_bits_to_f32(u_bits)
    sil = O.silu_exact(g)
    ok = np.zeros(h.shape, dtype=bool)
    for f in (1.0 - SILU_REL, 1.0 + SILU_REL):
        sb = O.bf16_rne_bits((sil * f).astype(np.float32))
        ok |= h == O.bf16_rne_bits(O.bf16_bits_to_f32(sb) * u)
    ok |= (g < SILU_ZERO_BELOW) & ((h & 0x7FFF) == 0)
    return ok


def _check_against_linears(h, g, u, label):
    ref = O.swiglu_bf16(g, u)
    differ = int((h != ref).sum())
    say(label, "differing from the SwiGLU of the two linears:", differ, "of", h.size)
    assert differ <= 1e-4 * h.size
    ok = _swiglu_consistent(h, g, u)
    assert ok.all(), (label, np.argwhere(~ok)[:5])


@pytest.mark.parametrize("m,n,k", [
    (1, 8, 16), (5, 130, 48), (37, 200, 272), (64, 384, 256),
    (130, 300, 1040), (256, 256, 512), (300, 520, 784),
])
def test_mlp_small_shapes(m, n, k):
    x, qg, sg, qu, su = _pair(m * 7 + n + k, m, n, k)
    say("mlp gate/up", m, n, k)
    h = run_mlp(x, qg, sg, qu, su)
    _check_full(x, qg, sg, qu, su, h, f"mlp {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [
    (1000, 5000, 272),    # below 2048 rows, many tiles: the 256-row paired tile
    (2100, 300, 528),     # from 2048 rows: the tile with both weights in every wave
])
def test_mlp_larger_shapes_each_kernel(m, n, k):
    """Ragged shapes (partial row and column tiles, K not a multiple of 64)
    that the tiled gate/up planner sends to the kernels the small shapes
    above do not reach, compared in full."""
    x, qg, sg, qu, su = _pair(m + 3 * n + k, m, n, k)
    say("mlp gate/up tiled", m, n, k)
    h = run_mlp(x, qg, sg, qu, su, F.PATH_TILED)
    _check_full(x, qg, sg, qu, su, h, f"mlp tiled {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [
    (1, 8, 16),            # one row, one partial column tile, one K chunk
    (37, 200, 272),        # ragged everything; the second wave pair past N
    (256, 256, 512),       # exact tiles
    (300, 520, 784),       # partial row and column tiles, K % 64 = 16
    (700, 1032, 1040),     # 3 x 9 tiles, N % 128 = 8
    (2100, 384, 3088),     # many steps, the last one partial
])
def test_mlp_large_kernel_shapes(m, n, k):
    """The large kernel's gated form (N % 8 == 0), compared in full."""
    x, qg, sg, qu, su = _pair(m * 5 + n + k, m, n, k)
    say("mlp gate/up large", m, n, k)
    h = run_mlp(x, qg, sg, qu, su, F.PATH_LARGE)
    _check_full(x, qg, sg, qu, su, h, f"mlp large {m}x{n}x{k}")


def test_mlp_large_matches_large_linears():
    """At a shape where the large kernel's plain form does not split K, its g
    and u are the gated form's g and u bit for bit (same tile rows, same K
    order), so h must be the SwiGLU of the two plain outputs up to silu's fp32
    evaluation: equal almost everywhere, and elsewhere only where the bf16
    rounding of silu can go the other way. The shape has partial row and
    column tiles. (Workgroups walking several units: the full 512 x 25600 x
    5120 pair in test_gpu_fullsize.py, 400 units.)"""
    m, n, k = 1000, 4088, 768
    x, qg, sg, qu, su = _pair(12, m, n, k)
    say("mlp large vs large linears", m, n, k)
    h = run_mlp(x, qg, sg, qu, su, F.PATH_LARGE)
    g = bits(F.fp8_block_linear(to_bf16(x), to_u8(qg), to_f32(sg), path=F.PATH_LARGE))
    u = bits(F.fp8_block_linear(to_bf16(x), to_u8(qu), to_f32(su), path=F.PATH_LARGE))
    _check_against_linears(h, g, u, "mlp large vs large linears")


def test_mlp_large_path_rejects_ragged_n():
    x, qg, sg, qu, su = _pair(5, 64, 132, 128)
    with pytest.raises(F.Fp8blError):
        run_mlp(x, qg, sg, qu, su, F.PATH_LARGE)
    with pytest.raises(F.Fp8blError):
        run_mlp(x, qg, sg, qu, su, F.PATH_SKINNY)


def test_mlp_matches_separate_linears():
    """At a shape where the plain linear does not split K, its g and u are the
    fused kernel's g and u bit for bit (every tile shape accumulates an output
    in the same order), so the
    fused h must be the SwiGLU of the two plain outputs up to silu's fp32
    evaluation: equal almost everywhere, and elsewhere only where the bf16
    rounding of silu can go the other way."""
    m, n, k = 1024, 4096, 1024
    x, qg, sg, qu, su = _pair(11, m, n, k)
    say("mlp vs separate linears", m, n, k)
    h = run_mlp(x, qg, sg, qu, su, F.PATH_TILED)
    g = bits(F.fp8_block_linear(to_bf16(x), to_u8(qg), to_f32(sg), path=F.PATH_TILED))
    u = bits(F.fp8_block_linear(to_bf16(x), to_u8(qu), to_f32(su), path=F.PATH_TILED))
    _check_against_linears(h, g, u, "mlp tiled vs tiled linears")


@pytest.mark.parametrize("path", ["tiled", "large"])
def test_mlp_silu_values(path):
    """silu pinned value by value: x picks one column of each weight (x[i, i]
    = 1), the up weight is all ones there, so h[i, j] is bf16(silu(g)) of
    g = the gate weight's dequantized element (j, i). The gate codes run
    through every finite E4M3 code, under eight scales (six powers of two
    from 2^-9 to 2^5, 3.7 and 0.013), so g spans about +-1e-5 .. +-1.4e4,
    the exponential's overflow below -87 included."""
    m, n, k = 4, 1024, 128
    j = np.arange(n)[:, None]
    c = np.arange(k)[None, :]
    codes = ((4 * j + c) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0            # no NaN codes
    qg = np.where(c < m, codes, 0).astype(np.uint8)
    sg = np.array([[2.0 ** -9], [2.0 ** -6], [2.0 ** -3], [1.0], [3.7], [2.0 ** 3],
                   [2.0 ** 5], [0.013]], dtype=np.float32)
    qu = np.where(c < m, 0x38, 0).astype(np.uint8).repeat(n, axis=0)   # E4M3 1.0
    su = np.ones((n // 128, 1), dtype=np.float32)
    x = np.zeros((m, k), dtype=np.uint16)
    x[np.arange(m), np.arange(m)] = 0x3F80                               # bf16 1.0
    say("mlp silu values", path)
    h = run_mlp(x, qg, sg, qu, su, F.PATH_LARGE if path == "large" else F.PATH_TILED)
    # g from the oracle's product: the one nonzero term, exact in bf16 (a -0
    # weight element sums with the zero terms to +0)
    g = O.bf16_rne_bits(O.linear_value(x, O.dequant(qg, sg)).astype(np.float32))
    u = np.full(h.shape, 0x3F80, dtype=np.uint16)
    gv = O.bf16_bits_to_f32(g)
    say("g range", float(gv.min()), float(gv.max()), "overflow cases", int((gv < SILU_ZERO_BELOW).sum()))
    assert gv.min() < SILU_ZERO_BELOW and gv.max() > 1e4
    ok = _swiglu_consistent(h, g, u)
    assert ok.all(), np.argwhere(~ok)[:5]
    ref = O.swiglu_bf16(g, u)
    live = gv >= SILU_ZERO_BELOW
    say("silu values off the oracle's rounding", int((h != ref)[live].sum()), "of", int(live.sum()))
    # (a CPU emulation of the kernels' fp32 silu puts 10 of these 4096 on the
    # other rounding: the large-|g| cases, where the exponent's rounding counts)
    assert (h != ref)[live].sum() <= 0.01 * live.sum()


def test_mlp_zero_input_and_zero_weight():
    m, n, k = 96, 256, 384
    x, qg, sg, qu, su = _pair(3, m, n, k)
    say("mlp zero input")
    h = run_mlp(np.zeros_like(x), qg, sg, qu, su)
    assert np.all((h & 0x7FFF) == 0)
    say("mlp zero up weight")
    h = run_mlp(x, qg, sg, np.zeros_like(qu), su)
    assert np.all((h & 0x7FFF) == 0)


def test_mlp_empty_shapes():
    x, qg, sg, qu, su = _pair(4, 8, 64, 128)
    h = F.fp8_block_mlp_gate_up(to_bf16(x[:0]), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
    torch.cuda.synchronize()
    assert tuple(h.shape) == (0, 64)


def test_mlp_reproducible():
    x, qg, sg, qu, su = _pair(6, 200, 640, 1024)
    say("mlp reproducible")
    a = run_mlp(x, qg, sg, qu, su)
    b = run_mlp(x, qg, sg, qu, su)
    assert np.array_equal(a, b)


def _sample_idx(size, block, rng, n_rand):
    edges = {0, size - 1, min(block - 1, size - 1), min(block, size - 1)}
    return np.array(sorted(edges | set(rng.integers(0, size, n_rand).tolist())), dtype=np.int64)


def test_mlp_pair_workload_sampled():
    """Full text-encoder gate/up shape (512 x 25600 x 5120), sampled outputs."""
    wl = generate("mlp_pair")
    gate, up, _ = wl.linears
    qg, sg = O.quantize(gate.w)
    qu, su = O.quantize(up.w)
    say("mlp workload mlp_pair gate/up", gate.m, gate.n, gate.k)
    h = run_mlp(gate.x, qg, sg, qu, su)
    rng = np.random.default_rng(99)
    ms = _sample_idx(gate.m, 128, rng, 24)
    ns = _sample_idx(gate.n, 128, rng, 24)
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    mm, nn = mm.ravel(), nn.ravel()
    g, ag = O.linear_sampled(gate.x, qg, sg, mm, nn)
    u, au = O.linear_sampled(gate.x, qu, su, mm, nn)
    r = O.swiglu_bound_ratio(h[mm, nn], g, ag, u, au)
    say("mlp_pair sampled", mm.size, "max swiglu bound ratio", float(r.max()))
    assert r.max() <= 1.0
    # the full output has no NaN/inf
    assert np.all((h & 0x7F80) != 0x7F80)


@pytest.mark.parametrize("path", ["tiled", "large"])
def test_mlp_graph_replay_matches_eager(path):
    """Each gate/up kernel captured in a HIP graph and replayed with eager
    work between the replays gives the eager bits every time."""
    m, n, k = 256, 640, 1024
    pid = F.PATH_TILED if path == "tiled" else F.PATH_LARGE
    x, qg, sg, qu, su = _pair(8, m, n, k)
    args = (to_bf16(x), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
    say("mlp graph replay", path, m, n, k)
    eager = bits(F.fp8_block_mlp_gate_up(*args, path=pid))
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.fp8_block_mlp_gate_up(*args, out=out, path=pid)
    for rep in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), rep
        F.fp8_block_mlp_gate_up(*args, path=pid)
        torch.cuda.synchronize()
