"""Device-memory plumbing for the library: allocate cache buffers and workspaces with PyTorch,
move numpy arrays (fp32 / fp16 / bf16 bit patterns) to the device and back. No computation of
the method happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import (BF16, F16, F32, Q43, Cache, Layer, starkv_cache_bytes,
               starkv_decode_workspace_bytes)


def to_device(a: np.ndarray, device="cuda", bf16: bool = False) -> torch.Tensor:
    """Upload a numpy array; uint16 arrays with ``bf16=True`` become torch.bfloat16 tensors."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(device)
        return t.view(torch.bfloat16) if bf16 else t
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Download; bfloat16 tensors come back as uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def elem_torch_dtype(code: int):
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, Q43: torch.float16}[code]


def alloc_cache(layer: Layer, batch: int, capacity: int, device="cuda", fill=None) -> Cache:
    """Allocate the six cache buffers (byte tensors sized by starkv_cache_bytes). ``fill``: None
    leaves them uninitialised, a float fills the value latents' bytes with that byte value (used
    to poison caches in tests)."""
    sizes = starkv_cache_bytes(layer, batch, capacity)
    bufs = []
    for n in sizes:
        if n == 0:
            bufs.append(None)
            continue
        t = torch.empty(n, dtype=torch.uint8, device=device)
        if fill is not None:
            t.fill_(int(fill))
        bufs.append(t)
    return Cache(batch, capacity, *bufs)


def alloc_workspace(layer: Layer, batch: int, seq_len: int, num_splits: int = 0, device="cuda"):
    n = starkv_decode_workspace_bytes(layer, batch, seq_len, num_splits)
    if n == 0:
        raise ValueError("invalid layer / shape for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=device), n
