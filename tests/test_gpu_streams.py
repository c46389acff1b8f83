"""Calls on streams other than the default one.

Every entry point takes a HIP stream and launches all of a call's kernels on
it (the split-K reduce included); the binding passes torch's current stream.
Here a call on a side stream must give the default stream's result bit for
bit, and calls with their own workspaces on two streams at once must each
give their own default-stream result. Inputs are quantized by the oracle and
each result is also held to the oracle's bound.
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


def _assert_bound(y, x, q, s, label):
    yr, ar = O.linear_exact(x, O.dequant(q, s))
    ratio = O.gemm_bound_ratio(bits(y), yr, ar)
    worst = float(ratio.max()) if ratio.size else 0.0
    say(label, "max bound ratio", worst)
    assert worst <= 1.0, (label, worst)


@pytest.mark.parametrize("m,n,k", [(512, 1024, 5120), (16, 4096, 4096), (300, 520, 784)])
def test_linear_on_side_stream_equals_default(m, n, k):
    x, q, s = _problem(m + 3 * n + k, m, n, k)
    xt, qt, st = to_bf16(x), to_u8(q), to_f32(s)
    say("side stream linear", m, n, k)
    y0 = F.fp8_block_linear(xt, qt, st)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1 = F.fp8_block_linear(xt, qt, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y0))
    _assert_bound(y1, x, q, s, f"side {m}x{n}x{k}")


def test_two_streams_at_once_with_own_workspaces():
    # both shapes split K, so each call writes and reduces partials in its
    # own workspace while the other stream runs
    shapes = [(512, 640, 5120), (16, 2048, 8192)]
    probs = [_problem(100 + i, *shp) for i, shp in enumerate(shapes)]
    dev = torch.device("cuda:0")
    ins = [(to_bf16(x), to_u8(q), to_f32(s)) for x, q, s in probs]
    ref = []
    for (m, n, k), (xt, qt, st) in zip(shapes, ins):
        assert F.workspace_size(m, n, k) > 0
        ref.append(bits(F.fp8_block_linear(xt, qt, st)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for stm in streams:
        stm.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for rep in range(4):
        say("two streams, round", rep)
        for i, ((m, n, k), (xt, qt, st)) in enumerate(zip(shapes, ins)):
            with torch.cuda.stream(streams[i]):
                ws = torch.empty(F.workspace_size(m, n, k), dtype=torch.uint8, device=dev)
                outs[i].append(F.fp8_block_linear(xt, qt, st, workspace=ws))
    for stm in streams:
        torch.cuda.current_stream().wait_stream(stm)
    torch.cuda.synchronize()
    for i, (m, n, k) in enumerate(shapes):
        for y in outs[i]:
            assert np.array_equal(bits(y), ref[i]), (m, n, k)
        x, q, s = probs[i]
        _assert_bound(outs[i][-1], x, q, s, f"two streams {m}x{n}x{k}")


def test_mlp_and_w8a8_on_side_stream_equal_default():
    m, n, k = 130, 300, 1040
    x, wg = random_problem(7, m, n, k, w_std=0.05)
    _, wu = random_problem(8, m, n, k, w_std=0.05)
    qg, sg = O.quantize(wg)
    qu, su = O.quantize(wu)
    xt = to_bf16(x)
    args = (xt, to_u8(qg), to_f32(sg), to_u8(qu), to_f32(su))
    say("side stream mlp and w8a8", m, n, k)
    h0 = F.fp8_block_mlp_gate_up(*args)
    w0 = F.fp8_block_linear_w8a8_bf16(xt, args[1], args[2])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h1 = F.fp8_block_mlp_gate_up(*args)
        w1 = F.fp8_block_linear_w8a8_bf16(xt, args[1], args[2])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h1), bits(h0))
    assert np.array_equal(bits(w1), bits(w0))
