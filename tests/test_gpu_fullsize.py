"""Every output of the large workloads against the oracle, at full size, in
the launch configuration the benchmark uses (AUTO path).

The oracle's fp64 product runs in row blocks so its memory stays bounded;
each block's outputs are held to the bound |y - Y*| <= 2^-7 |Y*| +
1e-4 sum_k |x_k w_k| (the fused gate/up pair to the SwiGLU bound built on
the same per-linear bounds). Weights are quantized by the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from workloads import generate  # noqa: E402

from gpu_util import bits, say, to_bf16, to_f32, to_u8  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

import block_scaled_fp8_linear_amd as F  # noqa: E402

ROWS = 2048          # oracle row block


def _full_compare(x_bits, q, s, y_bits, label):
    wd = O.dequant(q, s)
    worst, where = 0.0, None
    for r0 in range(0, x_bits.shape[0], ROWS):
        yr, ar = O.linear_exact(x_bits[r0:r0 + ROWS], wd)
        ratio = O.gemm_bound_ratio(y_bits[r0:r0 + ROWS], yr, ar)
        i = int(np.argmax(ratio))
        if ratio.flat[i] > worst:
            worst = float(ratio.flat[i])
            where = (r0 + i // ratio.shape[1], i % ratio.shape[1])
    say(label, "max bound ratio over all", y_bits.size, "outputs", worst, "at", where)
    assert worst <= 1.0, (label, worst, where)


def _run(x_bits, q, s):
    y = F.fp8_block_linear(to_bf16(x_bits), to_u8(q), to_f32(s))
    torch.cuda.synchronize()
    return bits(y)


@pytest.mark.parametrize("idx", [0, 1])
def test_dit_large_m_full(idx):
    """16384x3072x3072 (QKV/out) and 16384x12288x3072 (MLP up): all 50 M and
    201 M outputs."""
    lin = generate("dit_large_m").linears[idx]
    q, s = O.quantize(lin.w)
    say("full-size", lin.name, lin.m, lin.n, lin.k)
    _full_compare(lin.x, q, s, _run(lin.x, q, s), f"dit_large_m/{lin.name}")


@pytest.fixture(scope="module")
def mlp_pair():
    """The MLP pair's linears with the oracle's codes and scales."""
    gate, up, down = generate("mlp_pair").linears
    return [(lin,) + O.quantize(lin.w) for lin in (gate, up, down)]


def test_mlp_pair_full(mlp_pair):
    """512x25600x5120 gate and up, 512x5120x25600 down (its input the bf16
    SwiGLU of the oracle's gate/up outputs): every output of all three."""
    (gate, qg, sg), (up, qu, su), (down, qd, sd) = mlp_pair
    for lin, q, s in ((gate, qg, sg), (up, qu, su)):
        say("full-size", lin.name, lin.m, lin.n, lin.k)
        _full_compare(lin.x, q, s, _run(lin.x, q, s), f"mlp_pair/{lin.name}")
    g_ref = O.bf16_rne_bits(O.linear_value(gate.x, O.dequant(qg, sg)).astype(np.float32))
    u_ref = O.bf16_rne_bits(O.linear_value(up.x, O.dequant(qu, su)).astype(np.float32))
    h = O.swiglu_bf16(g_ref, u_ref)
    say("full-size", down.name, down.m, down.n, down.k)
    _full_compare(h, qd, sd, _run(h, qd, sd), "mlp_pair/down")


def test_mlp_gate_up_fused_full(mlp_pair):
    """The fused gate/up pair with the SwiGLU epilogue on 512x25600x5120:
    all 13 M outputs against the SwiGLU bound."""
    (gate, qg, sg), (up, qu, su), _ = mlp_pair
    say("full-size fused gate/up", gate.m, gate.n, gate.k)
    h = F.fp8_block_mlp_gate_up(to_bf16(gate.x), to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
    torch.cuda.synchronize()
    hb = bits(h)
    g_ref, g_a = O.linear_exact(gate.x, O.dequant(qg, sg))
    u_ref, u_a = O.linear_exact(up.x, O.dequant(qu, su))
    ratio = O.swiglu_bound_ratio(hb, g_ref, g_a, u_ref, u_a)
    worst = float(ratio.max())
    say("fused gate/up max SwiGLU bound ratio over all", hb.size, "outputs", worst)
    assert worst <= 1.0, (worst, np.unravel_index(int(np.argmax(ratio)), ratio.shape))
