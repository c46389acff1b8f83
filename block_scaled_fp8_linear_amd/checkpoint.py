"""Block-FP8 checkpoint converter: quantize a model's linear weights on the GPU
and write the serialized format the FP8 loader reads.

FastVideo PR #1829, "[feat] MiniMax H3: block-FP8 text encoder on Hopper, its
converter, and a 4xH100 FastH3 profile", "Changes", converter bullet: every
quantized linear is stored as an E4M3 weight plus a [N/128, K/128] fp32
``weight_scale_inv``, ``config.json`` carries a ``quantization_config`` and
the shard index is regenerated.

Format written here:

* for a quantized ``<prefix>.weight`` [N, K]: ``<prefix>.weight`` as
  ``float8_e4m3fn`` [N, K] and ``<prefix>.weight_scale_inv`` as fp32
  [ceil(N/128), ceil(K/128)]; every other tensor is copied unchanged;
* safetensors shards ``model-XXXXX-of-YYYYY.safetensors`` of at most
  ``max_shard_bytes`` each (a tensor is never split), tensors in name order;
* ``model.safetensors.index.json`` with ``metadata.total_size`` (bytes of
  tensor data) and ``weight_map`` (tensor name -> shard file);
* ``config.json``: the given model config with ``quantization_config`` set
  to block FP8 (E4M3, 128x128 weight blocks, dynamic activation scales).

The quantization itself runs in the HIP library (``fp8_block_quantize``); this
module only moves tensors and writes files.
"""

from __future__ import annotations

import json
import os
from typing import Callable, Iterable

import torch

BLOCK = 128

QUANTIZATION_CONFIG = {
    "quant_method": "fp8",
    "fmt": "e4m3",
    "activation_scheme": "dynamic",
    "weight_block_size": [BLOCK, BLOCK],
}

INDEX_NAME = "model.safetensors.index.json"


def scale_name(weight_name: str) -> str:
    """``<prefix>.weight`` -> ``<prefix>.weight_scale_inv``."""
    if not weight_name.endswith(".weight"):
        raise ValueError(f"not a weight name: {weight_name}")
    return weight_name + "_scale_inv"


def default_selector(name: str, t: torch.Tensor) -> bool:
    """Quantize 2-D floating ``*.weight`` tensors whose K is a multiple of 16
    (the library's constraint); everything else (norms, embeddings given as
    1-D, biases) stays as it is."""
    return (name.endswith(".weight") and t.dim() == 2 and t.dtype in (torch.float32, torch.bfloat16)
            and t.shape[1] % 16 == 0 and t.shape[0] > 0)


def quantize_state_dict(state_dict: dict[str, torch.Tensor],
                        select: Callable[[str, torch.Tensor], bool] = default_selector,
                        device: str | torch.device = "cuda:0") -> dict[str, torch.Tensor]:
    """Quantize the selected weights on ``device`` (one at a time, so only one
    layer is resident) and return CPU tensors: codes as ``float8_e4m3fn``,
    scales as fp32, untouched tensors as given."""
    from . import fp8_block_quantize

    out: dict[str, torch.Tensor] = {}
    for name in sorted(state_dict):
        t = state_dict[name]
        if not select(name, t):
            out[name] = t
            continue
        sname = scale_name(name)
        if sname in state_dict:
            raise ValueError(f"{sname} already present: {name} looks quantized")
        w = t.to(device).contiguous()
        q, s = fp8_block_quantize(w)
        out[name] = q.cpu().view(torch.float8_e4m3fn)
        out[sname] = s.cpu()
        del w, q, s
    return out


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def plan_shards(tensors: dict[str, torch.Tensor], max_shard_bytes: int) -> list[list[str]]:
    """Greedy shards in name order; a tensor larger than the limit gets a
    shard of its own."""
    if max_shard_bytes <= 0:
        raise ValueError("max_shard_bytes must be positive")
    shards: list[list[str]] = []
    cur: list[str] = []
    size = 0
    for name in sorted(tensors):
        b = _nbytes(tensors[name])
        if cur and size + b > max_shard_bytes:
            shards.append(cur)
            cur, size = [], 0
        cur.append(name)
        size += b
    if cur:
        shards.append(cur)
    return shards


def write_checkpoint(out_dir: str, tensors: dict[str, torch.Tensor], config: dict | None = None,
                     max_shard_bytes: int = 5 << 30) -> dict:
    """Write shards, the index and ``config.json`` into ``out_dir`` (created if
    needed). Returns the index dictionary."""
    from safetensors.torch import save_file

    os.makedirs(out_dir, exist_ok=True)
    shards = plan_shards(tensors, max_shard_bytes)
    n = len(shards)
    weight_map: dict[str, str] = {}
    total = 0
    for i, names in enumerate(shards):
        fname = f"model-{i + 1:05d}-of-{n:05d}.safetensors"
        part = {k: tensors[k].contiguous() for k in names}
        save_file(part, os.path.join(out_dir, fname), metadata={"format": "pt"})
        for k in names:
            weight_map[k] = fname
            total += _nbytes(tensors[k])
    index = {"metadata": {"total_size": total}, "weight_map": dict(sorted(weight_map.items()))}
    with open(os.path.join(out_dir, INDEX_NAME), "w") as f:
        json.dump(index, f, indent=2)
        f.write("\n")
    cfg = dict(config or {})
    cfg["quantization_config"] = dict(QUANTIZATION_CONFIG)
    with open(os.path.join(out_dir, "config.json"), "w") as f:
        json.dump(cfg, f, indent=2)
        f.write("\n")
    return index


def read_checkpoint(ckpt_dir: str, names: Iterable[str] | None = None) -> dict[str, torch.Tensor]:
    """Read tensors back through the index (all, or only ``names``)."""
    from safetensors import safe_open

    with open(os.path.join(ckpt_dir, INDEX_NAME)) as f:
        index = json.load(f)
    wanted = sorted(index["weight_map"]) if names is None else list(names)
    by_file: dict[str, list[str]] = {}
    for k in wanted:
        by_file.setdefault(index["weight_map"][k], []).append(k)
    out: dict[str, torch.Tensor] = {}
    for fname, keys in by_file.items():
        with safe_open(os.path.join(ckpt_dir, fname), framework="pt") as f:
            for k in keys:
                out[k] = f.get_tensor(k)
    return out


def convert(state_dict: dict[str, torch.Tensor], out_dir: str, config: dict | None = None,
            select: Callable[[str, torch.Tensor], bool] = default_selector,
            max_shard_bytes: int = 5 << 30, device: str | torch.device = "cuda:0") -> dict:
    """Quantize on the GPU, then write the checkpoint. Returns the index."""
    return write_checkpoint(out_dir, quantize_state_dict(state_dict, select, device), config,
                            max_shard_bytes)
