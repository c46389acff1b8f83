"""Seeded synthetic inputs for the block-scaled FP8 linear layer.

This module is shared by the tests, the smoke check and the benchmark. It
holds no step of the method: it draws activations and full-precision weights
only. Quantizing those weights is the method's own first step and is done
either by the CPU oracle (tests) or by the GPU quantizer (benchmark).

Recipe (every workload):

* ``rng = numpy.random.default_rng(seed)`` (PCG64); draws happen in the order
  X, then each weight matrix in the order listed, then any masks.
* X: fp32 standard normal, narrowed to bf16 by dropping the low 16 bits of
  each fp32 pattern (round toward zero). The generator keeps away from the
  method's own round-to-nearest-even; truncation leaves the distribution
  N(0,1) to within bf16 resolution.
* W: ``float32(0.02) * standard_normal`` in fp32, i.e. N(0, 0.02^2).

The shapes stand in for the text-encoder linears (FastVideo PR #1829: the
block-FP8 Qwen3-VL text encoder, whose largest dequantized layer is about
0.26 GB = 25600 x 5120 bf16) and for DiT-projection and decode-time
skinny shapes. No public dataset or checkpoint is involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Linear", "Workload", "WORKLOADS", "bf16_trunc_bits", "draw_x", "draw_w",
    "generate", "random_problem",
]


def bf16_trunc_bits(x32: np.ndarray) -> np.ndarray:
    """High 16 bits of each fp32 pattern (bf16 rounded toward zero)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    return (x32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def draw_x(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    return bf16_trunc_bits(rng.standard_normal((m, k), dtype=np.float32))


def draw_w(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    return np.float32(0.02) * rng.standard_normal((n, k), dtype=np.float32)


@dataclass
class Linear:
    """One linear layer of a workload: Y[M,N] = X[M,K] W[N,K]^T."""
    name: str
    m: int
    n: int
    k: int
    w: np.ndarray | None = None          # fp32 [N,K] before quantization
    x: np.ndarray | None = None          # bf16 bits [M,K]; None when derived


@dataclass
class Workload:
    name: str
    seed: int
    description: str
    linears: list[Linear] = field(default_factory=list)


def _tiny(seed: int = 0) -> Workload:
    """64x256 activations, 384x256 weight (3x2 scale grid); block (0,0) all
    zero; in block (2,1) every entry with n+k even set to +-1.0 (random sign),
    so that block's largest magnitude sits exactly on the E4M3 maximum."""
    rng = np.random.default_rng(seed)
    x = draw_x(rng, 64, 256)
    w = draw_w(rng, 384, 256)
    w[0:128, 0:128] = 0.0
    rows, cols = np.meshgrid(np.arange(256, 384), np.arange(128, 256), indexing="ij")
    even = ((rows + cols) % 2) == 0
    signs = np.where(rng.integers(0, 2, size=even.shape) == 1, 1.0, -1.0).astype(np.float32)
    blk = w[256:384, 128:256]
    blk[even] = signs[even]
    return Workload("tiny", seed, "tiny block-FP8 linear, 64x384x256",
                    [Linear("tiny", 64, 384, 256, w=w, x=x)])


def _attn_proj(seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    x = draw_x(rng, 512, 5120)
    w = draw_w(rng, 5120, 5120)
    return Workload("attn_proj", seed,
                    "text-encoder attention projection, M=512 N=5120 K=5120",
                    [Linear("proj", 512, 5120, 5120, w=w, x=x)])


def _mlp_pair(seed: int = 2) -> Workload:
    """Gate and up [25600,5120] share X; the down [5120,25600] input is the
    bf16 SwiGLU of the gate/up outputs, which the caller derives."""
    rng = np.random.default_rng(seed)
    x = draw_x(rng, 512, 5120)
    w_gate = draw_w(rng, 25600, 5120)
    w_up = draw_w(rng, 25600, 5120)
    w_down = draw_w(rng, 5120, 25600)
    return Workload("mlp_pair", seed,
                    "text-encoder MLP: gate/up 512x25600x5120, down 512x5120x25600",
                    [Linear("gate", 512, 25600, 5120, w=w_gate, x=x),
                     Linear("up", 512, 25600, 5120, w=w_up, x=x),
                     Linear("down", 512, 5120, 25600, w=w_down, x=None)])


def _dit_large_m(seed: int = 3) -> Workload:
    """1% of the weight entries (Bernoulli mask) multiplied by 20."""
    rng = np.random.default_rng(seed)
    x = draw_x(rng, 16384, 3072)
    w_qkv = draw_w(rng, 3072, 3072)
    w_up = draw_w(rng, 12288, 3072)
    for w in (w_qkv, w_up):
        mask = rng.random(w.shape) < 0.01
        w[mask] *= np.float32(20.0)
    return Workload("dit_large_m", seed,
                    "DiT projections, M=16384: 3072x3072 and 12288x3072",
                    [Linear("qkv", 16384, 3072, 3072, w=w_qkv, x=x),
                     Linear("mlp_up", 16384, 12288, 3072, w=w_up, x=x)])


def _skinny(seed: int = 4) -> Workload:
    """M=16 and M=1 (row 0 of the same X) against an 8000x8192 weight whose
    last 128-row scale block holds only 64 rows."""
    rng = np.random.default_rng(seed)
    x = draw_x(rng, 16, 8192)
    w = draw_w(rng, 8000, 8192)
    return Workload("skinny", seed, "skinny-M, M=16 and M=1, N=8000 K=8192",
                    [Linear("m16", 16, 8000, 8192, w=w, x=x),
                     Linear("m1", 1, 8000, 8192, w=w, x=x[:1].copy())])


WORKLOADS = {
    "tiny": _tiny,
    "attn_proj": _attn_proj,
    "mlp_pair": _mlp_pair,
    "dit_large_m": _dit_large_m,
    "skinny": _skinny,
}


def generate(name: str) -> Workload:
    return WORKLOADS[name]()


def random_problem(seed: int, m: int, n: int, k: int, w_std: float = 0.02):
    """A seeded (X bits, W fp32) pair of any shape, drawn like the workloads."""
    rng = np.random.default_rng(seed)
    x = draw_x(rng, m, k)
    w = (np.float32(w_std) * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    return x, w
