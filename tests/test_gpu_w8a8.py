"""GPU parity of the W8A8 route through the C ABI: the per-token activation
quantizer bit for bit against the oracle, and the E4M3 x E4M3 block-scaled
GEMM against the oracle's exact fp64 target with the bound
|y - Y*| <= 2^-7 |Y*| + 1e-4 sum_k |x_k w_k|. The GEMM's inputs (activation
codes and scales, weight codes and scales) come from the oracle."""

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


def gpu_act_quantize(x_bits):
    xq, xs = F.fp8_act_quantize(to_bf16(x_bits))
    torch.cuda.synchronize()
    return u8(xq), f32(xs)


def run_w8a8(xq, xs, q, s, path=F.PATH_AUTO):
    y = F.fp8_block_linear_w8a8(to_u8(xq), to_f32(xs), to_u8(q), to_f32(s), path=path)
    torch.cuda.synchronize()
    return bits(y)


# the kernels a shape can be forced onto (the 256-row-tile kernel needs N % 8 == 0)
def _paths(n):
    return [F.PATH_TILED, F.PATH_LARGE] if n % 8 == 0 else [F.PATH_TILED]


def assert_bound(y_bits, y_ref, a_ref, label):
    ratio = O.gemm_bound_ratio(y_bits, y_ref, a_ref)
    worst = float(ratio.max()) if ratio.size else 0.0
    say(label, "max bound ratio", worst)
    assert worst <= 1.0, (label, worst, np.unravel_index(np.argmax(ratio), ratio.shape))


# ---------------------------------------------------------------------------
# activation quantizer: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 16), (3, 144), (17, 272), (64, 1024), (130, 784), (513, 5120)])
def test_act_quantize_shapes(m, k):
    x, _ = random_problem(m * 31 + k, m, 8, k)
    say("act quantize", m, k)
    xq, xs = gpu_act_quantize(x)
    exq, exs = O.act_quantize(x)
    assert np.array_equal(xs.view(np.uint32), exs.view(np.uint32)), np.argwhere(xs != exs)[:5]
    assert np.array_equal(xq, exq), np.argwhere(xq != exq)[:5]


def test_act_quantize_special_groups():
    m, k = 8, 512
    rng = np.random.default_rng(31)
    xf = rng.standard_normal((m, k)).astype(np.float32)
    xf[0] = 0.0                                   # all-zero row: scales 1, codes 0
    xf[1, :128] = 0.0
    xf[2] *= 1e-30                                # tiny values (bf16 keeps them)
    xf[3, 128:256] = -0.0
    # exact ties: amax = 448 * 2^-3 makes S = 2^-3, so x / S is exact and the
    # midpoints between E4M3 codes must round to the even code
    tab = O.e4m3_table()[:0x7F]
    mids = (tab[1:] + tab[:-1]) / 2.0
    row = np.resize(np.concatenate([mids, -mids]), 128).astype(np.float64)
    row[0] = 448.0
    xf[4, :128] = (row * 2.0 ** -3).astype(np.float32)
    xf[5, 256:384] = np.float32(2.0 ** -133)      # bf16 subnormal, single group
    x = O.bf16_rne_bits(xf)
    assert np.array_equal(O.bf16_bits_to_f32(x[4, :128]).astype(np.float64), row * 2.0 ** -3)
    say("act quantize special groups")
    xq, xs = gpu_act_quantize(x)
    exq, exs = O.act_quantize(x)
    assert np.array_equal(xs.view(np.uint32), exs.view(np.uint32))
    assert np.array_equal(xq, exq), np.argwhere(xq != exq)[:5]


@pytest.mark.parametrize("name,idx", [("attn_proj", 0), ("dit_large_m", 0)])
def test_act_quantize_workloads(name, idx):
    lin = generate(name).linears[idx]
    say("act quantize workload", name, lin.m, lin.k)
    xq, xs = gpu_act_quantize(lin.x)
    exq, exs = O.act_quantize(lin.x)
    assert np.array_equal(xs.view(np.uint32), exs.view(np.uint32))
    assert np.array_equal(xq, exq)


# ---------------------------------------------------------------------------
# W8A8 GEMM: bound against the exact target
# ---------------------------------------------------------------------------

def _w8a8_inputs(seed, m, n, k):
    x, w = random_problem(seed, m, n, k)
    xq, xs = O.act_quantize(x)
    q, s = O.quantize(w)
    return xq, xs, q, s


@pytest.mark.parametrize("m,n,k", [
    (1, 8, 16), (5, 130, 48), (37, 200, 272), (64, 384, 256), (130, 300, 1040),
    (256, 256, 512), (300, 520, 784), (129, 129, 4096), (512, 1024, 5120),
])
def test_w8a8_small_shapes(m, n, k):
    xq, xs, q, s = _w8a8_inputs(m * 13 + n * 7 + k, m, n, k)
    yr, ar = O.linear_w8a8_exact(xq, xs, q, s)
    for path in [F.PATH_AUTO] + _paths(n):
        say("w8a8", m, n, k, "path", path)
        y = run_w8a8(xq, xs, q, s, path)
        assert_bound(y, yr, ar, f"w8a8 {m}x{n}x{k} path {path}")


@pytest.mark.parametrize("m,n,k", [
    (193, 264, 400),       # one row past a tile, the last wave past N, K % 128 = 16
    (2000, 8192, 256),     # 16 x 32 = 512 tiles: several units per workgroup's walk
    (700, 1544, 3088),     # many K blocks, the last partial; N % 256 = 8; split K
    (512, 5120, 5120),     # split K
    (1500, 8184, 400),     # 192-row tiles (256 of them fill one round), ragged rows and N
    (190, 12280, 4000),    # 192-row tiles with a 4-way K split, ragged rows, N and K
])
def test_w8a8_large_kernel_shapes(m, n, k):
    """The large-tile kernel forced (its planner picks 128 or 192 X rows per
    tile; the last two shapes take 192), compared in full."""
    xq, xs, q, s = _w8a8_inputs(m * 11 + n + k, m, n, k)
    say("w8a8 large", m, n, k)
    y = run_w8a8(xq, xs, q, s, F.PATH_LARGE)
    yr, ar = O.linear_w8a8_exact(xq, xs, q, s)
    assert_bound(y, yr, ar, f"w8a8 large {m}x{n}x{k}")


def test_w8a8_large_path_rejects_ragged_n():
    xq, xs, q, s = _w8a8_inputs(37, 64, 132, 128)
    with pytest.raises(F.Fp8blError):
        run_w8a8(xq, xs, q, s, F.PATH_LARGE)
    with pytest.raises(F.Fp8blError):
        run_w8a8(xq, xs, q, s, F.PATH_SKINNY)


def test_w8a8_all_codes_pow2_scales():
    # every finite code on both sides, power-of-two scales that differ per block
    m, n, k = 256, 256, 512
    rng = np.random.default_rng(33)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    xq = np.resize(finite, m * k).reshape(m, k).copy()
    rng.shuffle(xq, axis=1)
    q = np.resize(finite[::-1], n * k).reshape(n, k).copy()
    xs = (2.0 ** rng.integers(-10, 4, (4, m))).astype(np.float32)
    s = (2.0 ** rng.integers(-12, -2, (2, 4))).astype(np.float32)
    yr, ar = O.linear_w8a8_exact(xq, xs, q, s)
    for path in _paths(n):
        say("w8a8 all codes, path", path)
        y = run_w8a8(xq, xs, q, s, path)
        assert_bound(y, yr, ar, f"w8a8 all codes path {path}")


def test_w8a8_one_hot_exact():
    # one non-zero code per row of X: every output is one product, exact
    m, n, k = 128, 256, 384
    rng = np.random.default_rng(34)
    xq = np.zeros((m, k), np.uint8)
    cols = rng.integers(0, k, m)
    xq[np.arange(m), cols] = 0x38                  # 1.0
    xs = np.ones((3, m), np.float32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = O.quantize(w)
    yr, _ = O.linear_w8a8_exact(xq, xs, q, s)
    # y = bf16(fl32(e4m3(q) * s)) exactly: one product, one rounding
    exp = O.bf16_rne_bits(yr.astype(np.float32))
    for path in _paths(n):
        say("w8a8 one-hot, path", path)
        y = run_w8a8(xq, xs, q, s, path)
        assert np.array_equal(y, exp)


def test_w8a8_zero_and_empty():
    xq, xs, q, s = _w8a8_inputs(35, 64, 256, 512)
    for path in _paths(256):
        y = run_w8a8(np.zeros_like(xq), xs, q, s, path)
        assert np.all((y & 0x7FFF) == 0)
    y = F.fp8_block_linear_w8a8(to_u8(xq[:0]), to_f32(xs[:, :0]), to_u8(q), to_f32(s))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 256)


def test_w8a8_bf16_entry_equals_two_calls_and_reproducible():
    m, n, k = 512, 5120, 5120                      # split-K shape
    x, w = random_problem(36, m, n, k)
    q, s = O.quantize(w)
    xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
    say("w8a8 bf16 entry", m, n, k)
    ws = torch.empty(F.w8a8_workspace_size(m, n, k), dtype=torch.uint8, device="cuda:0")
    ws.fill_(0xFF)                                 # garbage must not matter
    y1 = F.fp8_block_linear_w8a8_bf16(xt, qt, st, workspace=ws)
    xq, xs = F.fp8_act_quantize(xt)
    y2 = F.fp8_block_linear_w8a8(xq, xs, qt, st, workspace=ws)
    y3 = F.fp8_block_linear_w8a8_bf16(xt, qt, st, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    # and the activation codes are the oracle's
    exq, exs = O.act_quantize(x)
    assert np.array_equal(u8(xq), exq) and np.array_equal(f32(xs), exs)


def _sample_idx(size, rng, n_rand):
    edges = {0, size - 1, min(127, size - 1), min(128, size - 1)}
    return np.array(sorted(edges | set(rng.integers(0, size, n_rand).tolist())), dtype=np.int64)


@pytest.mark.parametrize("name,idx", [("attn_proj", 0), ("mlp_pair", 0), ("dit_large_m", 0),
                                      ("dit_large_m", 1)])
def test_w8a8_workloads_sampled(name, idx):
    lin = generate(name).linears[idx]
    xq, xs = O.act_quantize(lin.x)
    q, s = O.quantize(lin.w)
    say("w8a8 workload", name, lin.name, lin.m, lin.n, lin.k)
    y = run_w8a8(xq, xs, q, s)
    rng = np.random.default_rng(lin.m + lin.n)
    ms = _sample_idx(lin.m, rng, 24)
    ns = _sample_idx(lin.n, rng, 24)
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    mm, nn = mm.ravel(), nn.ravel()
    yr, ar = O.linear_w8a8_sampled(xq, xs, q, s, mm, nn)
    assert_bound(y[mm, nn], yr, ar, f"w8a8 {name}/{lin.name} ({mm.size} sampled)")
    assert np.all((y & 0x7F80) != 0x7F80)


@pytest.mark.parametrize("m,n,k", [(512, 5120, 5120), (300, 1024, 1040)])
def test_w8a8_graph_replay_matches_eager(m, n, k):
    """The bf16-input W8A8 call (quantizer + GEMM + reduce when split)
    captured in a HIP graph and replayed with eager work in between gives the
    eager bits every time."""
    x, w = random_problem(m + n + k, m, n, k)
    q, s = O.quantize(w)
    xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
    ws = torch.empty(F.w8a8_workspace_size(m, n, k), dtype=torch.uint8, device="cuda:0")
    say("w8a8 graph replay", m, n, k)
    eager = bits(F.fp8_block_linear_w8a8_bf16(xt, qt, st, workspace=ws))
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.fp8_block_linear_w8a8_bf16(xt, qt, st, out=out, workspace=ws)
    for rep in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), rep
        F.fp8_block_linear_w8a8_bf16(xt, qt, st, workspace=ws)
        torch.cuda.synchronize()


def test_w8a8_largest_k_sampled():
    """K at the interface's limit (2^20): 8192 scale blocks per row."""
    m, n, k = 32, 256, 1 << 20
    rng = np.random.default_rng(37)
    x = O.bf16_rne_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = (rng.standard_normal((n, k), dtype=np.float32) * 0.02).astype(np.float32)
    xq, xs = O.act_quantize(x)
    q, s = O.quantize(w)
    say("w8a8 largest K", m, n, k)
    y = run_w8a8(xq, xs, q, s)
    ms = np.array([0, 5, 31, 17]); ns = np.array([0, 255, 128, 77])
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    yr, ar = O.linear_w8a8_sampled(xq, xs, q, s, mm.ravel(), nn.ravel())
    assert_bound(y[mm.ravel(), nn.ravel()], yr, ar, "w8a8 largest K")


# ---------------------------------------------------------------------------
# activation quantizer: the quotient near E4M3 rounding midpoints
# ---------------------------------------------------------------------------

def _bf16_f32(bits16):
    return (np.asarray(bits16, np.uint32) << 16).view(np.float32)


def _groups(amax_bits, x_bits):
    """Rows of one 1x128 group each: element 0 is the amax (+a), the other
    127 are the given bf16 values (all |x| <= a), zero-padded."""
    per = 127
    rows = max(1, -(-len(x_bits) // per))
    flat = np.zeros(rows * per, np.uint16)
    flat[:len(x_bits)] = x_bits
    out = np.empty((rows, 128), np.uint16)
    out[:, 0] = amax_bits
    out[:, 1:] = flat.reshape(rows, per)
    return out


def _near_midpoint_x(ab, count):
    """The `count` positive bf16 x <= a whose IEEE quotient fl32(x / S) lies
    closest (in ulps of the quotient) to a midpoint between E4M3 values: the
    inputs where a quotient one ulp off would change the code."""
    s = np.float32(_bf16_f32(ab)) / np.float32(448.0)
    xb = np.arange(0, ab + 1, dtype=np.uint32)
    q = (_bf16_f32(xb) / s).astype(np.float32).astype(np.float64)
    tab = O.e4m3_table()[:0x7F]
    mids = (tab[1:] + tab[:-1]) / 2.0
    i = np.clip(np.searchsorted(mids, q), 1, len(mids) - 1)
    d = np.minimum(np.abs(q - mids[i - 1]), np.abs(q - mids[i]))
    d /= np.spacing(q.astype(np.float32)).astype(np.float64)
    return xb[np.argsort(d, kind="stable")[:count]].astype(np.uint16)


def test_act_quantize_near_midpoints():
    """Codes of quotients within a few ulps of E4M3 midpoints, for amax over
    the whole bf16 range, with every mantissa at the exponents where the
    scale crosses 2^-64 (the kernel changes its division method there),
    both signs, bit for bit against the oracle."""
    rng = np.random.default_rng(47)
    amax = [int(e << 7 | m) for e in range(0, 255, 3) for m in rng.integers(0, 128, 2)]
    amax += [int(e << 7 | m) for e in (70, 71, 72, 73) for m in range(128)]   # a ~ 2^-57 .. 2^-54
    amax = sorted({a for a in amax if 0 < a <= 0x7F7F})
    rows = []
    for ab in amax:
        xb = _near_midpoint_x(ab, 200)
        rows.append(_groups(ab, np.concatenate([xb, xb | np.uint16(0x8000)])))
    x = np.concatenate(rows)
    say("act quantize near midpoints", x.shape, len(amax), "amax values")
    xq, xs = gpu_act_quantize(x)
    exq, exs = O.act_quantize(x)
    assert np.array_equal(xs.view(np.uint32), exs.view(np.uint32))
    bad = np.argwhere(xq != exq)
    assert bad.size == 0, [(hex(x[r, 0]), hex(x[r, c]), xq[r, c], exq[r, c]) for r, c in bad[:8]]


def test_act_quantize_exhaustive_pairs():
    """Every positive finite bf16 amax and every bf16 x with |x| <= amax,
    both signs, through the GPU quantizer, bit for bit against the oracle."""
    lo = 1
    total = 0
    while lo <= 0x7F7F:
        hi, n = lo, 0
        while hi <= 0x7F7F and n < 24_000_000:
            n += 2 * (hi + 1)
            hi += 1
        rows = []
        for ab in range(lo, hi):
            xb = np.arange(0, ab + 1, dtype=np.uint16)
            rows.append(_groups(ab, np.concatenate([xb, xb | np.uint16(0x8000)])))
        x = np.concatenate(rows)
        say("act quantize exhaustive amax", hex(lo), "..", hex(hi - 1), x.shape)
        xq, xs = gpu_act_quantize(x)
        exq, exs = O.act_quantize(x)
        assert np.array_equal(xs.view(np.uint32), exs.view(np.uint32))
        bad = np.argwhere(xq != exq)
        assert bad.size == 0, [(hex(x[r, 0]), hex(x[r, c]), xq[r, c], exq[r, c]) for r, c in bad[:8]]
        total += x.size
        lo = hi
    say("act quantize exhaustive codes checked", total)
