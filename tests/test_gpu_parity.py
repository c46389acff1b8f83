"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Dequant and quantize must match bit for bit; the linear must satisfy the
bound |y - Y*| <= 2^-7 |Y*| + 1e-4 sum_k |x_k w_k| against the oracle's fp64
Y*, plus exact invariants (one-hot identity, zero input, power-of-two
scaling, run-to-run reproducibility). Inputs come from the seeded workload
generators; weights are quantized by the oracle for every linear/dequant
test, never by the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from workloads import generate, random_problem  # noqa: E402

from gpu_util import bits, f32, say, to_bf16, to_f32, to_u8, u8  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

import block_scaled_fp8_linear_amd as F  # noqa: E402

PATHS = {"auto": F.PATH_AUTO, "tiled": F.PATH_TILED, "skinny": F.PATH_SKINNY, "large": F.PATH_LARGE}


def run_linear(x_bits, q, s, path=F.PATH_AUTO):
    xt, qt, st = to_bf16(x_bits), to_u8(q), to_f32(s)
    y = F.fp8_block_linear(xt, qt, st, path=path)
    torch.cuda.synchronize()
    return bits(y)


def assert_bound(y_bits, y_ref, a_ref, label):
    ratio = O.gemm_bound_ratio(y_bits, y_ref, a_ref)
    worst = float(ratio.max()) if ratio.size else 0.0
    say(label, "max bound ratio", worst)
    assert worst <= 1.0, (label, worst, np.unravel_index(np.argmax(ratio), ratio.shape))


# ---------------------------------------------------------------------------
# device gate
# ---------------------------------------------------------------------------

def test_device_is_gfx950():
    say("device", torch.cuda.get_device_name(0))
    assert F.device_supported(0)


# ---------------------------------------------------------------------------
# dequant: bit-exact
# ---------------------------------------------------------------------------

def _scale_set():
    rng = np.random.default_rng(7)
    s = [1.0, 0.5, 2.0, 3.0, 1.0 / 448, 0.02 / 448, 1e-3, 7.5e-5]
    s += [2.0 ** e for e in range(-30, 31, 3)]
    s += list(rng.uniform(1e-6, 1e-2, size=40))
    s += list(rng.standard_normal(10) * 1e-3)
    s += [2.0 ** -127, 2.0 ** -140, 2.0 ** -149, 1e-39, 2.0 ** 120, 3.0e38]
    s += [np.array([0x3FEB8E39], np.uint32).view(np.float32)[0]]
    s += [np.inf, 0.0, -0.0, np.nan]
    return np.array(s, dtype=np.float32)


def test_dequant_all_codes_times_scales():
    scales = _scale_set()
    g = len(scales)
    q = np.tile(np.arange(256, dtype=np.uint8), (128 * g, 1))          # [128g, 256]
    s = np.repeat(scales[:, None], 2, axis=1).astype(np.float32)        # [g, 2]
    say("dequant codes x scales", q.shape)
    got = bits(F.fp8_block_dequant(to_u8(q), to_f32(s)))
    exp = O.dequant(q, s)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


@pytest.mark.parametrize("n,k", [(1, 16), (300, 272), (129, 4096), (128, 128), (7, 2064)])
def test_dequant_ragged_random(n, k):
    rng = np.random.default_rng(n * 7 + k)
    q = rng.integers(0, 256, size=(n, k), dtype=np.uint8)             # NaN codes included
    s = rng.uniform(1e-5, 1e-1, size=O.scale_grid_shape(n, k)).astype(np.float32)
    say("dequant ragged", n, k)
    got = bits(F.fp8_block_dequant(to_u8(q), to_f32(s)))
    assert np.array_equal(got, O.dequant(q, s))


@pytest.mark.parametrize("name", ["tiny", "attn_proj", "skinny"])
def test_dequant_workloads(name):
    wl = generate(name)
    lin = wl.linears[0]
    q, s = O.quantize(lin.w)
    say("dequant workload", name, q.shape)
    got = bits(F.fp8_block_dequant(to_u8(q), to_f32(s)))
    assert np.array_equal(got, O.dequant(q, s))


# ---------------------------------------------------------------------------
# quantize: bit-exact codes and scales
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "attn_proj", "skinny"])
def test_quantize_workloads(name):
    lin = generate(name).linears[0]
    say("quantize workload", name, lin.w.shape)
    qt, st = F.fp8_block_quantize(to_f32(lin.w))
    torch.cuda.synchronize()
    q, s = O.quantize(lin.w)
    assert np.array_equal(f32(st).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(u8(qt), q)


@pytest.mark.parametrize("n,k,std", [(200, 160, 0.02), (1, 16, 1.0), (129, 272, 1e-30),
                                     (300, 400, 1e3), (64, 1024, 0.02)])
def test_quantize_ragged(n, k, std):
    _, w = random_problem(n + k, 1, n, k, w_std=std)
    w[: min(n, 5), :16] = 0.0
    w[0, 0] = -0.0
    if n > 128 and k > 128:
        w[128:, 128:] = 0.0                                            # an all-zero block
    say("quantize ragged", n, k, std)
    qt, st = F.fp8_block_quantize(to_f32(w))
    torch.cuda.synchronize()
    q, s = O.quantize(w)
    assert np.array_equal(f32(st).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(u8(qt), q)


@pytest.mark.parametrize("n,k", [(384, 256), (5120, 5120), (200, 160), (1, 16), (129, 272)])
def test_quantize_bf16_input(n, k):
    _, w = random_problem(n * 5 + k, 1, n, k)
    bits_w = O.bf16_rne_bits(w)
    if n > 128 and k > 128:
        bits_w[128:256, 128:256] = 0                                  # an all-zero block
    say("quantize bf16 input", n, k)
    qt, st = F.fp8_block_quantize(to_bf16(bits_w))
    torch.cuda.synchronize()
    q, s = O.quantize_bf16(bits_w)
    assert np.array_equal(f32(st).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(u8(qt), q)


def test_quantize_subnormal_and_tie_values():
    """Values placed on E4M3 midpoints (ties) and deep in the subnormal
    range of both formats, after the per-block scale is applied."""
    t = O.e4m3_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    w = np.zeros((128, 256), dtype=np.float32)
    w[0, :] = 448.0                                  # amax 448 -> S = 1 exactly
    w[1:, :] = np.resize(np.concatenate([mids, -mids, t.astype(np.float32)]), (127, 256))
    w[100:110, :] = np.float32(2.0 ** -140)          # fp32 subnormal inputs
    say("quantize ties/subnormals")
    qt, st = F.fp8_block_quantize(to_f32(w))
    torch.cuda.synchronize()
    q, s = O.quantize(w)
    assert s[0, 0] == 1.0
    assert np.array_equal(f32(st).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(u8(qt), q)


def test_quantize_codes_around_every_midpoint():
    """With S = 1 (a block holding 448) the codes are the E4M3 encoding of
    the fp32 inputs themselves: every midpoint between neighbouring codes and
    the 8 fp32 values on each side of it, both signs, plus every code value
    and its fp32 neighbours, bit for bit against the oracle."""
    t = O.e4m3_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, t.astype(np.float32)])
    bits_ = pts.view(np.uint32).astype(np.int64)
    near = np.concatenate([bits_ + d for d in range(-8, 9)])
    near = near[(near >= 0) & (near < 0x80000000)].astype(np.uint32).view(np.float32)
    near = near[np.isfinite(near) & (np.abs(near) <= 448.0)]
    vals = np.concatenate([near, -near, [0.0, -0.0]]).astype(np.float32)
    rows = -(-vals.size // 254)
    flat = np.zeros(rows * 254, dtype=np.float32)
    flat[:vals.size] = vals
    flat = flat.reshape(rows, 254)
    w = np.zeros((rows, 256), dtype=np.float32)
    w[:, 0] = w[:, 128] = 448.0                    # both column blocks hold amax 448 -> S = 1
    w[:, 1:128], w[:, 129:] = flat[:, :127], flat[:, 127:]
    say("quantize around midpoints", w.shape)
    qt, st = F.fp8_block_quantize(to_f32(w))
    torch.cuda.synchronize()
    q, s = O.quantize(w)
    assert np.all(s == 1.0)
    assert np.array_equal(f32(st).view(np.uint32), s.view(np.uint32))
    bad = np.argwhere(u8(qt) != q)
    assert bad.size == 0, [(float(w[r, c]), int(u8(qt)[r, c]), int(q[r, c])) for r, c in bad[:8]]


def test_quantize_hardware_encode_wide():
    """The hardware E4M3 encode behind both quantizers, with S = 1 (every
    block holds 448), against the oracle's integer nearest-even encoder:
    every fp32 value that is a bf16 pattern up to 448 in magnitude, and every
    fp32 pattern within 4096 ulp of each midpoint between neighbouring codes
    and of each code, both signs (about 4.2 M inputs)."""
    t = O.e4m3_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, t.astype(np.float32)]).view(np.uint32).astype(np.int64)
    near = (pts[:, None] + np.arange(-4096, 4097, dtype=np.int64)[None, :]).ravel()
    near = near[(near >= 0) & (near < 0x7F800000)].astype(np.uint32)
    bf = (np.arange(0, 0x7F80, dtype=np.uint32) << np.uint32(16))
    mags = np.unique(np.concatenate([near, bf])).view(np.float32)
    mags = mags[mags <= 448.0]
    vals = np.concatenate([mags, -mags]).astype(np.float32)
    rows = -(-vals.size // 254)
    flat = np.zeros(rows * 254, dtype=np.float32)
    flat[:vals.size] = vals
    flat = flat.reshape(rows, 254)
    w = np.zeros((rows, 256), dtype=np.float32)
    w[:, 0] = w[:, 128] = 448.0                    # both column blocks hold amax 448 -> S = 1
    w[:, 1:128], w[:, 129:] = flat[:, :127], flat[:, 127:]
    say("quantize hardware encode, wide", w.shape, vals.size, "inputs")
    qt, st = F.fp8_block_quantize(to_f32(w))
    torch.cuda.synchronize()
    q, s = O.quantize(w)
    assert np.all(s == 1.0)
    assert np.array_equal(f32(st).view(np.uint32), s.view(np.uint32))
    bad = np.argwhere(u8(qt) != q)
    assert bad.size == 0, [(float(w[r, c]), int(u8(qt)[r, c]), int(q[r, c])) for r, c in bad[:8]]


# ---------------------------------------------------------------------------
# linear: bound against the fp64 oracle, both kernels forced on small shapes
# ---------------------------------------------------------------------------

SMALL_SHAPES = [
    (64, 384, 256),      # the tiny workload's shape
    (1, 384, 256),
    (16, 200, 272),      # ragged N and K (K % 128 != 0)
    (33, 300, 1040),     # just past the skinny threshold
    (130, 513, 528),
    (257, 640, 384),
    (512, 256, 2048),
    (5, 8, 16),          # smallest legal K
]


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_linear_small_shapes(m, n, k, path):
    x, w = random_problem(m * 131 + n * 7 + k, m, n, k)
    q, s = O.quantize(w)
    say("linear", path, m, n, k)
    y = run_linear(x, q, s, PATHS[path])
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    assert_bound(y, yr, ar, f"{path} {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [
    (129, 2500, 4112), (1100, 2000, 2512), (1000, 4000, 2000), (1500, 4100, 784), (2047, 2500, 784),
])
def test_linear_wide_tile_shapes(m, n, k):
    """Shapes the tile planner sends to the 128x256 tile (eight waves of one
    32-column block each), with 8, 3, 2 and no K splits; M, N and K all end
    in partial tiles or steps. Full compare against the oracle."""
    x, w = random_problem(m + 5 * n + k, m, n, k)
    q, s = O.quantize(w)
    say("linear wide tile", m, n, k)
    y = run_linear(x, q, s, F.PATH_AUTO)
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    assert_bound(y, yr, ar, f"wide tile {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [
    (3000, 1300, 2000), (2049, 2000, 2512), (700, 4100, 4112), (3000, 4100, 784), (2500, 5000, 784),
])
def test_linear_square_tile_shapes(m, n, k):
    """Shapes the tile planner sends to the 256x256 tile (eight waves of one
    32-column block each, 256 rows), with 3, 5 and no K splits; M, N and K
    all end in partial tiles or steps. Full compare against the oracle."""
    x, w = random_problem(m + 3 * n + 2 * k, m, n, k)
    q, s = O.quantize(w)
    say("linear square tile", m, n, k)
    y = run_linear(x, q, s, F.PATH_AUTO)
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    assert_bound(y, yr, ar, f"square tile {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [
    (256, 256, 64), (300, 520, 1040), (513, 300, 4112), (100, 700, 5200),
    (257, 1000, 2576), (1000, 300, 784), (600, 2048, 3072), (40, 130, 16), (2304, 2560, 512),
])
def test_linear_large_tile_shapes(m, n, k):
    """The 256x256 four-wave kernel forced on shapes with partial tiles in M
    and N, K tails inside a 64-wide step and a 16-wide sub-step, N % 4 != 0
    (element stores) and 8 and 4 K splits (100x700x5200, 257x1000x2576).
    Full compare against the oracle. (Workgroups walking several units are
    compared in full on the DiT shapes, 768 and 3072 tiles, in
    test_gpu_fullsize.py.)"""
    x, w = random_problem(m * 3 + n * 11 + k, m, n, k)
    q, s = O.quantize(w)
    say("linear large tile", m, n, k)
    y = run_linear(x, q, s, F.PATH_LARGE)
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    assert_bound(y, yr, ar, f"large tile {m}x{n}x{k}")


@pytest.mark.parametrize("path", ["tiled", "skinny", "large"])
def test_linear_tiny_workload(path):
    lin = generate("tiny").linears[0]
    q, s = O.quantize(lin.w)
    say("linear tiny workload", path)
    y = run_linear(lin.x, q, s, PATHS[path])
    yr, ar = O.linear_exact(lin.x, O.dequant(q, s))
    assert_bound(y, yr, ar, f"tiny {path}")


@pytest.mark.parametrize("path", ["tiled", "skinny", "large"])
def test_linear_one_hot_identity(path):
    """X = I (M = K = 256): every output is a single exact product, so Y must
    equal W_hat^T bit for bit: the GEMM consumes exactly the dequant's bf16."""
    lin = generate("tiny").linears[0]
    q, s = O.quantize(lin.w)
    x = np.zeros((256, 256), dtype=np.uint16)
    x[np.arange(256), np.arange(256)] = 0x3F80                    # bf16 1.0
    say("one-hot identity", path)
    y = run_linear(x, q, s, PATHS[path])
    assert np.array_equal(y, O.dequant(q, s).T)


@pytest.mark.parametrize("path", ["tiled", "skinny", "large"])
def test_linear_zero_input_gives_positive_zero(path):
    _, w = random_problem(3, 1, 300, 512)
    q, s = O.quantize(w)
    x = np.zeros((40, 512), dtype=np.uint16)
    say("zero input", path)
    y = run_linear(x, q, s, PATHS[path])
    assert np.all(y == 0)


@pytest.mark.parametrize("path", ["tiled", "skinny", "large"])
def test_linear_power_of_two_scaling_is_exact(path):
    x, w = random_problem(12, 48, 320, 768)
    q, s = O.quantize(w)
    x2 = O.bf16_rne_bits(O.bf16_bits_to_f32(x) * np.float32(4.0))   # exact
    say("power-of-two scaling", path)
    y1 = run_linear(x, q, s, PATHS[path])
    y2 = run_linear(x2, q, s, PATHS[path])
    assert np.array_equal(O.bf16_rne_bits(O.bf16_bits_to_f32(y1) * np.float32(4.0)), y2)


@pytest.mark.parametrize("path", ["tiled", "skinny", "large"])
def test_linear_reproducible(path):
    x, w = random_problem(44, 24, 1000, 4096)
    q, s = O.quantize(w)
    say("reproducible", path)
    xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
    ys = [bits(F.fp8_block_linear(xt, qt, st, path=PATHS[path])) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


@pytest.mark.parametrize("m,n,k", [(16, 384, 256), (1, 384, 256), (32, 1000, 16), (64, 384, 256),
                                   (5, 300, 4112), (16, 5120, 5120)])
def test_skinny_short_k_ranges_reproducible(m, n, k):
    """The skinny kernel where a wave's K range is one or a few super-steps
    (its loop ends before a whole round of ring slots), or a K split or tail
    leaves the waves unequal shares: within the bound and the same bits on
    every call. These are the cases where a code slot could be read before
    its loads had landed."""
    x, w = random_problem(m * 7 + n + k, m, n, k)
    q, s = O.quantize(w)
    say("skinny short k ranges", m, n, k)
    xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
    ys = [bits(F.fp8_block_linear(xt, qt, st, path=F.PATH_SKINNY)) for _ in range(4)]
    for y in ys[1:]:
        assert np.array_equal(ys[0], y)
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    assert_bound(ys[0], yr, ar, f"skinny {m}x{n}x{k}")


def test_linear_shared_workspace_reused():
    """Split-K shapes of several sizes through one workspace filled with
    garbage, twice: the partials need no initialisation and every result
    stays within the bound."""
    shapes = [(512, 256, 2048), (130, 513, 528), (64, 384, 4096), (512, 640, 5120)]
    need = max(F.workspace_size(m, n, k) for m, n, k in shapes)
    assert need > 0
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")
    for rep in range(2):
        for m, n, k in shapes:
            x, w = random_problem(m + n + k + rep, m, n, k)
            q, s = O.quantize(w)
            say("shared workspace", rep, m, n, k)
            y = F.fp8_block_linear(to_bf16(x), to_u8(q), to_f32(s), workspace=ws,
                                   path=F.PATH_TILED)
            torch.cuda.synchronize()
            yr, ar = O.linear_exact(x, O.dequant(q, s))
            assert_bound(bits(y), yr, ar, f"shared ws {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(512, 640, 5120), (16, 8000, 1024), (300, 1024, 512)])
def test_linear_graph_replay_matches_eager(m, n, k):
    """The call captured into a HIP graph and replayed several times, with
    eager work and synchronisations between replays, gives the eager bits
    every time (split-K and skinny shapes included)."""
    x, w = random_problem(m * 3 + n + k, m, n, k)
    q, s = O.quantize(w)
    xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
    ws = torch.empty(max(F.workspace_size(m, n, k), 1), dtype=torch.uint8, device="cuda:0")
    say("graph replay", m, n, k)
    eager = bits(F.fp8_block_linear(xt, qt, st, workspace=ws))
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.fp8_block_linear(xt, qt, st, out=out, workspace=ws)
    for rep in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), rep
        F.fp8_block_linear(xt, qt, st, workspace=ws)     # eager work in between
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["tiled", "skinny", "large"])
def test_linear_largest_k_sampled(path):
    """K at the interface's limit (2^20): 16384 tiled K steps or 4096 skinny
    super-steps, 8192 scale blocks per row; outputs sampled against Y*."""
    m, n, k = 32, 256, 1 << 20
    rng = np.random.default_rng(38)
    x = O.bf16_rne_bits(rng.standard_normal((m, k), dtype=np.float32)) & np.uint16(0xFFFF)
    w = (rng.standard_normal((n, k), dtype=np.float32) * 0.02).astype(np.float32)
    q, s = O.quantize(w)
    say("largest K", path, m, n, k)
    y = run_linear(x, q, s, PATHS[path])
    ms = np.array([0, 7, 31, 16]); ns = np.array([0, 255, 128, 3])
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    yr, ar = O.linear_sampled(x, q, s, mm.ravel(), nn.ravel())
    assert_bound(y[mm.ravel(), nn.ravel()], yr, ar, f"largest K {path}")


def test_linear_empty_shapes():
    say("empty shapes")
    q = to_u8(np.zeros((8, 32), np.uint8))
    s = to_f32(np.ones((1, 1), np.float32))
    y = F.fp8_block_linear(to_bf16(np.zeros((0, 32), np.uint16)), q, s)
    assert tuple(y.shape) == (0, 8)
    y = F.fp8_block_linear(to_bf16(np.zeros((4, 32), np.uint16)),
                           to_u8(np.zeros((0, 32), np.uint8)), to_f32(np.ones((0, 1), np.float32)))
    assert tuple(y.shape) == (4, 0)


# ---------------------------------------------------------------------------
# linear on the full workload sizes, in the launch configuration the
# benchmark uses (AUTO path)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,idx", [("attn_proj", 0), ("skinny", 0), ("skinny", 1)])
def test_linear_workload_full_compare(name, idx):
    wl = generate(name)
    lin = wl.linears[idx]
    q, s = O.quantize(lin.w)
    say("linear workload", name, lin.name, lin.m, lin.n, lin.k)
    y = run_linear(lin.x, q, s)
    yr, ar = O.linear_exact(lin.x, O.dequant(q, s))
    assert_bound(y, yr, ar, f"{name}/{lin.name}")


def _sample_idx(size, tile, rng, n_rand):
    edges = {0, 1, size - 1, size - 2}
    for b in range(tile, size, tile):
        edges |= {b - 1, b}
    edges = sorted(e for e in edges if 0 <= e < size)
    if len(edges) > 24:
        edges = list(rng.choice(edges, 24, replace=False))
    return np.unique(np.concatenate([edges, rng.integers(0, size, n_rand)])).astype(np.int64)


def _check_sampled(x_bits, q, s, y, label, n_rand=24):
    m, n = y.shape
    rng = np.random.default_rng(m + n)
    ms = _sample_idx(m, 256, rng, n_rand)
    ns = _sample_idx(n, 256, rng, n_rand)
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    mm, nn = mm.ravel(), nn.ravel()
    yr, ar = O.linear_sampled(x_bits, q, s, mm, nn)
    assert_bound(y[mm, nn], yr, ar, label + f" ({mm.size} sampled outputs)")


@pytest.mark.parametrize("idx", [0, 1])
def test_linear_dit_large_m_sampled(idx):
    wl = generate("dit_large_m")
    lin = wl.linears[idx]
    q, s = O.quantize(lin.w)
    say("linear workload dit_large_m", lin.name, lin.m, lin.n, lin.k)
    y = run_linear(lin.x, q, s)
    _check_sampled(lin.x, q, s, y, f"dit_large_m/{lin.name}")


def test_linear_mlp_pair_sampled():
    wl = generate("mlp_pair")
    gate, up, down = wl.linears
    qg, sg = O.quantize(gate.w)
    qu, su = O.quantize(up.w)
    qd, sd = O.quantize(down.w)
    say("linear workload mlp_pair gate/up", gate.m, gate.n, gate.k)
    yg = run_linear(gate.x, qg, sg)
    _check_sampled(gate.x, qg, sg, yg, "mlp_pair/gate")
    yu = run_linear(up.x, qu, su)
    _check_sampled(up.x, qu, su, yu, "mlp_pair/up")
    # The down input is the SwiGLU of the ORACLE's gate/up outputs.
    g_ref = O.bf16_rne_bits(O.linear_value(gate.x, O.dequant(qg, sg)).astype(np.float32))
    u_ref = O.bf16_rne_bits(O.linear_value(up.x, O.dequant(qu, su)).astype(np.float32))
    h = O.swiglu_bf16(g_ref, u_ref)
    say("linear workload mlp_pair down", down.m, down.n, down.k)
    yd = run_linear(h, qd, sd)
    _check_sampled(h, qd, sd, yd, "mlp_pair/down", n_rand=12)
