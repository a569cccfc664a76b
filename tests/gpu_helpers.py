"""Shared helpers for the GPU parity tests (marshalling host inputs to the device)."""

import numpy as np
import torch

from synth import HostTensor


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_device(h, dev=None) -> torch.Tensor:
    """HostTensor (or a float32 / bf16-bits array with a dtype tag) -> GPU tensor."""
    dev = dev or device()
    if isinstance(h, HostTensor):
        data, dtype = h.data, h.dtype
    else:
        data, dtype = h
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(data, dtype=np.float32)).to(dev)
    bits = np.ascontiguousarray(data, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(dev).view(torch.bfloat16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32).view(np.uint32)


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
