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


def run_mlp(x_bits, qg, sg, qu, su):
    h = F.fp8_block_mlp_gate_up(to_bf16(x_bits), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
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
    that the gate/up planner sends to the kernels the small shapes above do
    not reach, compared in full."""
    x, qg, sg, qu, su = _pair(m + 3 * n + k, m, n, k)
    say("mlp gate/up", m, n, k)
    h = run_mlp(x, qg, sg, qu, su)
    _check_full(x, qg, sg, qu, su, h, f"mlp {m}x{n}x{k}")


def test_mlp_matches_separate_linears():
    """At a shape where the plain linear does not split K, its g and u are the
    fused kernel's g and u bit for bit (every tile shape accumulates an output
    in the same order), so the
    fused h must be the SwiGLU of the two plain outputs up to silu's fp32
    evaluation: equal almost everywhere, never more than one bf16 ulp off."""
    m, n, k = 1024, 4096, 1024
    x, qg, sg, qu, su = _pair(11, m, n, k)
    say("mlp vs separate linears", m, n, k)
    h = run_mlp(x, qg, sg, qu, su)
    g = bits(F.fp8_block_linear(to_bf16(x), to_u8(qg), to_f32(sg), path=F.PATH_TILED))
    u = bits(F.fp8_block_linear(to_bf16(x), to_u8(qu), to_f32(su), path=F.PATH_TILED))
    ref = O.swiglu_bf16(g, u)
    diff = np.abs(h.astype(np.int32) - ref.astype(np.int32))
    same_sign = (h >> 15) == (ref >> 15)
    say("mlp vs separate: differing", int((diff != 0).sum()), "of", diff.size)
    assert (diff != 0).mean() < 1e-3
    both_zero = ((h & 0x7FFF) == 0) & ((ref & 0x7FFF) == 0)
    one_ulp = (diff <= 1) & same_sign
    assert np.all(one_ulp | both_zero)


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


def test_mlp_graph_replay_matches_eager():
    m, n, k = 256, 640, 1024
    x, qg, sg, qu, su = _pair(8, m, n, k)
    args = (to_bf16(x), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
    say("mlp graph replay", m, n, k)
    eager = bits(F.fp8_block_mlp_gate_up(*args))
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.fp8_block_mlp_gate_up(*args, out=out)
    for rep in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), rep
        F.fp8_block_mlp_gate_up(*args)
        torch.cuda.synchronize()
