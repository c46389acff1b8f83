"""The allocation-free linear (fp8_block_linear_noalloc) through the C ABI.

Its split-K partials live in the library's own per-device scratch. Each case
makes two calls in a row on one stream, the second on a smaller shape, so the
scratch still holds the first call's (larger) partials when the second runs.
Both outputs must equal fp8_block_linear's (same kernels, same summation
order: bit for bit) and lie within the oracle's bound.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from workloads import random_problem  # noqa: E402

from gpu_util import bits, say, to_bf16, to_f32, to_u8  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

import block_scaled_fp8_linear_amd as F  # noqa: E402


def _problem(seed, m, n, k):
    x, w = random_problem(seed, m, n, k)
    q, s = O.quantize(w)
    return x, q, s


@pytest.mark.parametrize("first,second", [
    ((512, 5120, 5120), (300, 1000, 4096)),     # tiled path, split K both times
    ((32, 8000, 8192), (16, 3000, 8192)),       # skinny path, split K both times
    ((1024, 5120, 5120), (200, 640, 2048)),     # 60 MiB of partials, then a small split
])
def test_noalloc_matches_linear_twice(first, second):
    outs = []
    for seed, (m, n, k) in ((71, first), (72, second)):
        assert F.workspace_size(m, n, k) <= F._lib.NOALLOC_SCRATCH_BYTES
        x, q, s = _problem(seed, m, n, k)
        xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        say("noalloc", m, n, k)
        F.fp8_block_linear_noalloc(xt, qt, st, out=y)
        outs.append((x, q, s, xt, qt, st, y))
    torch.cuda.synchronize()
    for x, q, s, xt, qt, st, y in outs:
        m, n = y.shape
        k = x.shape[1]
        ref = F.fp8_block_linear(xt, qt, st)
        torch.cuda.synchronize()
        yb = bits(y)
        assert np.array_equal(yb, bits(ref)), ("noalloc differs from fp8_block_linear", m, n, k)
        yr, ar = O.linear_exact(x, O.dequant(q, s))
        worst = float(O.gemm_bound_ratio(yb, yr, ar).max())
        say("noalloc", m, n, k, "max bound ratio", worst)
        assert worst <= 1.0


def test_noalloc_rejects_oversized_partials():
    """A shape whose partials exceed the scratch comes back as FP8BL_WORKSPACE
    before anything is launched (the device stays usable)."""
    m, n, k = 768, 8192, 65536
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda:0")
    q = torch.zeros((n, k), dtype=torch.uint8, device="cuda:0")
    s = torch.ones(F.scale_grid_shape(n, k), dtype=torch.float32, device="cuda:0")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(F.Fp8blError) as e:
        F.fp8_block_linear_noalloc(x, q, s, out=y)
    assert e.value.status == F._lib.FP8BL_WORKSPACE
    torch.cuda.synchronize()
