"""Host-side tests of the block-FP8 checkpoint writer: shard planning, index,
config, naming and a bit-exact round trip of oracle-quantized tensors (no GPU:
the quantization here is the oracle's, the file handling is the writer's)."""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytest.importorskip("safetensors")

import oracle as O  # noqa: E402
from block_scaled_fp8_linear_amd import checkpoint as C  # noqa: E402


def _quantized_dict(seed=0):
    rng = np.random.default_rng(seed)
    out = {}
    for name, (n, k) in {"layers.0.mlp.up.weight": (300, 256), "layers.0.attn.q.weight": (128, 384),
                         "layers.1.mlp.up.weight": (64, 144)}.items():
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        q, s = O.quantize(w)
        out[name] = torch.from_numpy(q).view(torch.float8_e4m3fn)
        out[C.scale_name(name)] = torch.from_numpy(s)
    out["layers.0.norm.weight"] = torch.from_numpy(rng.standard_normal(256).astype(np.float32))
    out["embed.weight"] = torch.from_numpy(rng.standard_normal((10, 8)).astype(np.float32)).to(torch.bfloat16)
    return out


def test_scale_name_and_selector():
    assert C.scale_name("a.b.weight") == "a.b.weight_scale_inv"
    with pytest.raises(ValueError):
        C.scale_name("a.b.bias")
    f32 = torch.zeros(8, 32)
    assert C.default_selector("x.weight", f32)
    assert C.default_selector("x.weight", f32.to(torch.bfloat16))
    assert not C.default_selector("x.bias", f32)
    assert not C.default_selector("x.weight", torch.zeros(32))            # 1-D
    assert not C.default_selector("x.weight", torch.zeros(8, 24))         # K % 16 != 0
    assert not C.default_selector("x.weight", torch.zeros(8, 32, dtype=torch.float16))


def test_plan_shards():
    t = {"a": torch.zeros(100, dtype=torch.uint8), "b": torch.zeros(300, dtype=torch.uint8),
         "c": torch.zeros(50, dtype=torch.uint8), "d": torch.zeros(60, dtype=torch.uint8)}
    assert C.plan_shards(t, 200) == [["a"], ["b"], ["c", "d"]]
    assert C.plan_shards(t, 10_000) == [["a", "b", "c", "d"]]
    assert C.plan_shards(t, 1) == [["a"], ["b"], ["c"], ["d"]]
    with pytest.raises(ValueError):
        C.plan_shards(t, 0)


def test_write_read_round_trip(tmp_path):
    tensors = _quantized_dict()
    cfg = {"model_type": "qwen3_vl", "hidden_size": 256}
    index = C.write_checkpoint(str(tmp_path), tensors, cfg, max_shard_bytes=40_000)
    files = sorted(f for f in os.listdir(tmp_path) if f.endswith(".safetensors"))
    assert len(files) >= 2
    assert all(f.startswith("model-") and f.endswith(f"-of-{len(files):05d}.safetensors") for f in files)
    on_disk = json.load(open(tmp_path / C.INDEX_NAME))
    assert on_disk == index
    assert set(index["weight_map"]) == set(tensors)
    assert set(index["weight_map"].values()) == set(files)
    assert index["metadata"]["total_size"] == sum(t.numel() * t.element_size() for t in tensors.values())
    cfg_out = json.load(open(tmp_path / "config.json"))
    assert cfg_out["model_type"] == "qwen3_vl" and cfg_out["hidden_size"] == 256
    assert cfg_out["quantization_config"] == {"quant_method": "fp8", "fmt": "e4m3",
                                              "activation_scheme": "dynamic",
                                              "weight_block_size": [128, 128]}
    back = C.read_checkpoint(str(tmp_path))
    assert set(back) == set(tensors)
    for k, v in tensors.items():
        assert back[k].dtype == v.dtype and back[k].shape == v.shape, k
        assert torch.equal(back[k].view(torch.uint8) if v.dtype == torch.float8_e4m3fn else back[k],
                           v.view(torch.uint8) if v.dtype == torch.float8_e4m3fn else v), k
    # the stored format is what the oracle dequantizes: codes + [N/128, K/128] scales
    q = back["layers.0.mlp.up.weight"].view(torch.uint8).numpy()
    s = back["layers.0.mlp.up.weight_scale_inv"].numpy()
    assert s.shape == O.scale_grid_shape(*q.shape) == (3, 2)
    assert O.dequant(q, s).shape == (300, 256)
    # a subset read touches only what it names
    part = C.read_checkpoint(str(tmp_path), ["embed.weight"])
    assert list(part) == ["embed.weight"]
