"""Block-scaled FP8 linear layer for MI355X (gfx950).

Weights live as E4M3 bytes Q[N,K] plus one fp32 weight_scale_inv per
128x128 block, S[ceil(N/128), ceil(K/128)] (FastVideo PR #1829, "[feat]
MiniMax H3: block-FP8 text encoder on Hopper, its converter, and a 4xH100
FastH3 profile", "Changes"). The library behind this module (libfp8bl.so,
hand-written HIP) provides:

* ``fp8_block_quantize(w)``  -> (q, s)     the converter's quantization (fp32 or bf16 w)
* ``fp8_block_dequant(q, s)`` -> bf16 W_hat  bit-exact dequant
* ``fp8_block_linear(x, q, s)`` -> bf16 Y = X W_hat^T, fp32 accumulation
  (``fp8_block_linear_noalloc(x, q, s, out)``: the same with no allocation)
* ``fp8_block_mlp_gate_up(x, qg, sg, qu, su)`` -> bf16 swiglu(X Wg^T, X Wu^T)
  in one launch (the MLP's gate/up pair)
* ``fp8_act_quantize(x)`` -> (xq, x_scale)  per-token 1x128 activation quantizer
* ``fp8_block_linear_w8a8(xq, x_scale, q, s)`` / ``fp8_block_linear_w8a8_bf16(x, q, s)``
  -> bf16 Y from E4M3 x E4M3 products on the FP8 matrix cores (W8A8 route)
* ``fp8_block_stream_read(buf)`` -> a plain streaming read of device memory
  (measurement aid: the practical HBM ceiling)

``block_scaled_fp8_linear_amd.checkpoint`` converts a state dict into the
serialized block-FP8 checkpoint (quantization on the GPU, safetensors shards,
index and ``quantization_config``).

The functions here only marshal torch tensors (device memory and the current
stream) into the C ABI declared in include/fp8bl.h; all arithmetic runs in
the HIP kernels. There is no CPU fallback: without the built library every
call raises.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import (  # noqa: F401
    PATH_AUTO, PATH_LARGE, PATH_SKINNY, PATH_TILED, Fp8blError, abi_version, device_supported,
    status_string, w8a8_workspace_size, workspace_size,
)

BLOCK = 128

__all__ = [
    "fp8_block_quantize", "fp8_block_dequant", "fp8_block_linear", "fp8_block_mlp_gate_up",
    "fp8_act_quantize", "fp8_block_linear_w8a8", "fp8_block_linear_w8a8_bf16",
    "fp8_block_linear_noalloc",
    "workspace_size", "w8a8_workspace_size",
    "device_supported", "abi_version", "status_string", "Fp8blError",
    "PATH_AUTO", "PATH_TILED", "PATH_SKINNY", "PATH_LARGE", "scale_grid_shape", "fp8_block_stream_read",
]


def scale_grid_shape(n: int, k: int) -> tuple[int, int]:
    return ((n + BLOCK - 1) // BLOCK, (k + BLOCK - 1) // BLOCK)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int, where: str) -> None:
    if status != _lib.FP8BL_OK:
        raise Fp8blError(status, where)


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fp8_block_quantize(w: torch.Tensor, q: torch.Tensor | None = None,
                       s: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """fp32 or bf16 w [N,K] -> (q uint8 [N,K], s fp32 [ceil(N/128), ceil(K/128)])."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"w must be float32 or bfloat16, got {w.dtype}")
    _need(w, w.dtype, "w")
    n, k = w.shape
    if q is None:
        q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty(scale_grid_shape(n, k), dtype=torch.float32, device=w.device)
    _need(q, torch.uint8, "q")
    _need(s, torch.float32, "s")
    if tuple(q.shape) != (n, k) or tuple(s.shape) != scale_grid_shape(n, k):
        raise ValueError("output shapes do not match w")
    raw = _lib.quantize_raw if w.dtype == torch.float32 else _lib.quantize_bf16_raw
    with torch.cuda.device(w.device):
        _check(raw(w.data_ptr(), q.data_ptr(), s.data_ptr(), n, k, _stream(w.device)),
               "fp8_block_quantize")
    return q, s


def fp8_block_dequant(q: torch.Tensor, s: torch.Tensor,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """q uint8 [N,K] + s fp32 grid -> bf16 [N,K] (bit-exact)."""
    _need(q, torch.uint8, "q")
    _need(s, torch.float32, "s")
    n, k = q.shape
    if tuple(s.shape) != scale_grid_shape(n, k):
        raise ValueError(f"scale grid must be {scale_grid_shape(n, k)}, got {tuple(s.shape)}")
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != (n, k):
        raise ValueError("out shape")
    with torch.cuda.device(q.device):
        _check(_lib.dequant_raw(q.data_ptr(), s.data_ptr(), out.data_ptr(), n, k,
                                _stream(q.device)), "fp8_block_dequant")
    return out


def fp8_block_linear(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     path: int = PATH_AUTO) -> torch.Tensor:
    """bf16 x [M,K], q uint8 [N,K], s fp32 grid -> bf16 y [M,N] = x W_hat^T.

    ``workspace``, when given, must hold at least ``workspace_size(M, N, K)``
    bytes (fp32 split-K partials; no initialisation needed); calls sharing it
    must be ordered."""
    _need(x, torch.bfloat16, "x")
    _need(q, torch.uint8, "q")
    _need(s, torch.float32, "s")
    m, k = x.shape
    n, kq = q.shape
    if kq != k:
        raise ValueError(f"K mismatch: x has {k}, q has {kq}")
    if tuple(s.shape) != scale_grid_shape(n, k):
        raise ValueError(f"scale grid must be {scale_grid_shape(n, k)}, got {tuple(s.shape)}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out shape")
    need = workspace_size(m, n, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(x.device):
        _check(_lib.linear_raw(x.data_ptr(), q.data_ptr(), s.data_ptr(), out.data_ptr(),
                               m, n, k, ws_ptr, ws_bytes, path, _stream(x.device)),
               "fp8_block_linear")
    return out


def fp8_block_linear_noalloc(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor,
                             out: torch.Tensor) -> torch.Tensor:
    """fp8_block_linear into a caller-given ``out``, with the split-K partials
    in the library's own per-device scratch (64 MiB): nothing is allocated,
    here or in the library. Calls on one device share that scratch and must
    be ordered (one stream)."""
    _need(x, torch.bfloat16, "x")
    _need(q, torch.uint8, "q")
    _need(s, torch.float32, "s")
    _need(out, torch.bfloat16, "out")
    m, k = x.shape
    n, kq = q.shape
    if kq != k:
        raise ValueError(f"K mismatch: x has {k}, q has {kq}")
    if tuple(s.shape) != scale_grid_shape(n, k):
        raise ValueError(f"scale grid must be {scale_grid_shape(n, k)}, got {tuple(s.shape)}")
    if tuple(out.shape) != (m, n):
        raise ValueError("out shape")
    with torch.cuda.device(x.device):
        _check(_lib.linear_noalloc_raw(x.data_ptr(), q.data_ptr(), s.data_ptr(), out.data_ptr(),
                                       m, n, k, _stream(x.device)),
               "fp8_block_linear_noalloc")
    return out


def fp8_block_mlp_gate_up(x: torch.Tensor, q_gate: torch.Tensor, s_gate: torch.Tensor,
                          q_up: torch.Tensor, s_up: torch.Tensor,
                          out: torch.Tensor | None = None, path: int = PATH_AUTO) -> torch.Tensor:
    """bf16 x [M,K] and two block-FP8 weights [N,K] -> bf16 h [M,N] with
    h = bf16(bf16(silu(g)) * u), g and u the two linears' bf16 outputs.
    ``path``: PATH_AUTO, PATH_TILED or PATH_LARGE (N % 8 == 0)."""
    _need(x, torch.bfloat16, "x")
    for t, name in ((q_gate, "q_gate"), (q_up, "q_up")):
        _need(t, torch.uint8, name)
    for t, name in ((s_gate, "s_gate"), (s_up, "s_up")):
        _need(t, torch.float32, name)
    m, k = x.shape
    n, kq = q_gate.shape
    if kq != k or tuple(q_up.shape) != (n, k):
        raise ValueError(f"weights must both be [{n}, {k}] to match x")
    grid = scale_grid_shape(n, k)
    if tuple(s_gate.shape) != grid or tuple(s_up.shape) != grid:
        raise ValueError(f"scale grids must be {grid}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out shape")
    with torch.cuda.device(x.device):
        _check(_lib.mlp_gate_up_ex_raw(x.data_ptr(), q_gate.data_ptr(), s_gate.data_ptr(),
                                       q_up.data_ptr(), s_up.data_ptr(), out.data_ptr(),
                                       m, n, k, int(path), _stream(x.device)),
               "fp8_block_mlp_gate_up")
    return out


def x_scale_shape(m: int, k: int) -> tuple[int, int]:
    """Activation scales are K-block-major: [ceil(K/128), M]."""
    return ((k + BLOCK - 1) // BLOCK, m)


def fp8_act_quantize(x: torch.Tensor, xq: torch.Tensor | None = None,
                     x_scale: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 x [M,K] -> (xq uint8 [M,K], x_scale fp32 [ceil(K/128), M])."""
    _need(x, torch.bfloat16, "x")
    m, k = x.shape
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(x_scale_shape(m, k), dtype=torch.float32, device=x.device)
    _need(xq, torch.uint8, "xq")
    _need(x_scale, torch.float32, "x_scale")
    if tuple(xq.shape) != (m, k) or tuple(x_scale.shape) != x_scale_shape(m, k):
        raise ValueError("output shapes do not match x")
    with torch.cuda.device(x.device):
        _check(_lib.act_quantize_raw(x.data_ptr(), xq.data_ptr(), x_scale.data_ptr(), m, k,
                                     _stream(x.device)), "fp8_act_quantize")
    return xq, x_scale


def _w8a8_workspace(m, n, k, workspace, dev):
    need = w8a8_workspace_size(m, n, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return workspace, ws_ptr, ws_bytes


def fp8_block_linear_w8a8(xq: torch.Tensor, x_scale: torch.Tensor, q: torch.Tensor,
                          s: torch.Tensor, out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None,
                          path: int = PATH_AUTO) -> torch.Tensor:
    """E4M3 xq [M,K] + x_scale [ceil(K/128), M], block-FP8 weight -> bf16 y [M,N].
    ``path``: PATH_AUTO, PATH_TILED (128x128 tiles) or PATH_LARGE (256x256
    tiles, N % 8 == 0)."""
    _need(xq, torch.uint8, "xq")
    _need(x_scale, torch.float32, "x_scale")
    _need(q, torch.uint8, "q")
    _need(s, torch.float32, "s")
    m, k = xq.shape
    n, kq = q.shape
    if kq != k:
        raise ValueError(f"K mismatch: xq has {k}, q has {kq}")
    if tuple(x_scale.shape) != x_scale_shape(m, k):
        raise ValueError(f"x_scale must be {x_scale_shape(m, k)}, got {tuple(x_scale.shape)}")
    if tuple(s.shape) != scale_grid_shape(n, k):
        raise ValueError(f"scale grid must be {scale_grid_shape(n, k)}, got {tuple(s.shape)}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out shape")
    workspace, ws_ptr, ws_bytes = _w8a8_workspace(m, n, k, workspace, xq.device)
    with torch.cuda.device(xq.device):
        _check(_lib.linear_w8a8_ex_raw(xq.data_ptr(), x_scale.data_ptr(), q.data_ptr(),
                                       s.data_ptr(), out.data_ptr(), m, n, k, ws_ptr, ws_bytes,
                                       int(path), _stream(xq.device)), "fp8_block_linear_w8a8")
    return out


def fp8_block_linear_w8a8_bf16(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor,
                               out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 x [M,K] -> quantize per token (1x128) -> W8A8 GEMM -> bf16 y [M,N]."""
    _need(x, torch.bfloat16, "x")
    _need(q, torch.uint8, "q")
    _need(s, torch.float32, "s")
    m, k = x.shape
    n, kq = q.shape
    if kq != k:
        raise ValueError(f"K mismatch: x has {k}, q has {kq}")
    if tuple(s.shape) != scale_grid_shape(n, k):
        raise ValueError(f"scale grid must be {scale_grid_shape(n, k)}, got {tuple(s.shape)}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out shape")
    workspace, ws_ptr, ws_bytes = _w8a8_workspace(m, n, k, workspace, x.device)
    with torch.cuda.device(x.device):
        _check(_lib.linear_w8a8_bf16_raw(x.data_ptr(), q.data_ptr(), s.data_ptr(), out.data_ptr(),
                                         m, n, k, ws_ptr, ws_bytes, _stream(x.device)),
               "fp8_block_linear_w8a8_bf16")
    return out


def fp8_block_stream_read(buf: torch.Tensor, blocks: int = 2048,
                          sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement aid: a plain streaming read of a contiguous device tensor
    (its byte size a multiple of 16) by ``blocks`` workgroups; returns the
    int32 sink [blocks * 256] whose XOR is the XOR of the tensor's words."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    _need(sink, torch.int32, "sink")
    if sink.numel() < blocks * 256:
        raise ValueError("sink must hold blocks * 256 words")
    nbytes = buf.numel() * buf.element_size()
    with torch.cuda.device(buf.device):
        _check(_lib.stream_read_raw(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                    _stream(buf.device)), "fp8_block_stream_read")
    return sink
