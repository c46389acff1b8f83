"""GPU conversion of a state dict into the block-FP8 checkpoint: the codes and
scales written are the oracle's bit for bit, and the reloaded weight
dequantizes (on the GPU) to the oracle's bf16 weight."""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytest.importorskip("safetensors")

import oracle as O  # noqa: E402

from gpu_util import bits, say, to_f32, to_u8  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

import block_scaled_fp8_linear_amd as F  # noqa: E402
from block_scaled_fp8_linear_amd import checkpoint as C  # noqa: E402


def test_convert_state_dict_bit_exact(tmp_path):
    rng = np.random.default_rng(41)
    w32 = (rng.standard_normal((300, 272)) * 0.05).astype(np.float32)
    wb = O.bf16_rne_bits((rng.standard_normal((130, 256)) * 0.02).astype(np.float32))
    sd = {
        "enc.layers.0.q.weight": torch.from_numpy(w32),
        "enc.layers.0.k.weight": torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16),
        "enc.layers.0.norm.weight": torch.ones(272),
        "enc.layers.0.odd.weight": torch.zeros(4, 24),          # K % 16 != 0: kept as is
    }
    say("checkpoint convert")
    index = C.convert(sd, str(tmp_path), {"model_type": "test"}, max_shard_bytes=64_000)
    assert "enc.layers.0.q.weight_scale_inv" in index["weight_map"]
    back = C.read_checkpoint(str(tmp_path))
    q1, s1 = O.quantize(w32)
    q2, s2 = O.quantize_bf16(wb)
    assert np.array_equal(back["enc.layers.0.q.weight"].view(torch.uint8).numpy(), q1)
    assert np.array_equal(back["enc.layers.0.q.weight_scale_inv"].numpy().view(np.uint32), s1.view(np.uint32))
    assert np.array_equal(back["enc.layers.0.k.weight"].view(torch.uint8).numpy(), q2)
    assert np.array_equal(back["enc.layers.0.k.weight_scale_inv"].numpy().view(np.uint32), s2.view(np.uint32))
    assert torch.equal(back["enc.layers.0.norm.weight"], sd["enc.layers.0.norm.weight"])
    assert torch.equal(back["enc.layers.0.odd.weight"], sd["enc.layers.0.odd.weight"])
    # reloaded weight, dequantized on the GPU, is the oracle's bf16 weight
    q = back["enc.layers.0.q.weight"].view(torch.uint8).numpy()
    s = back["enc.layers.0.q.weight_scale_inv"].numpy()
    got = bits(F.fp8_block_dequant(to_u8(q), to_f32(s)))
    assert np.array_equal(got, O.dequant(q1, s1))
