"""Helpers for the GPU parity tests: numpy <-> device tensors (bit patterns
only, no arithmetic) and a flushed progress print naming each case."""

from __future__ import annotations

import sys

import numpy as np
import torch


def dev() -> torch.device:
    return torch.device("cuda:0")


def say(*parts) -> None:
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def to_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def to_bf16(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).view(torch.bfloat16).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()
