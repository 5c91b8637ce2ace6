"""Device plumbing shared by the bench and the GPU tests: storage arrays from
``workloads`` to torch device tensors and back.  Holds no attention arithmetic;
torch is imported on first use (a GPU is needed only to call these)."""

import numpy as np

from . import bf16_bits_to_f64


def _torch():
    import torch
    return torch


def to_dev(storage, dtype):
    """Device copy of a storage array (float32, float16, uint16 bf16 bits or uint8)."""
    torch = _torch()
    a = np.ascontiguousarray(storage)
    if dtype == "bf16":
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def empty(shape, dtype):
    """Zero-filled device tensor of a storage dtype (bf16 as int16 bits)."""
    torch = _torch()
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.int16}[dtype]
    return torch.full(shape, 0, dtype=tdt, device="cuda")


def from_dev(t, dtype):
    """float64 host copy of a device tensor of a storage dtype."""
    a = t.detach().cpu().numpy()
    if dtype == "bf16":
        return bf16_bits_to_f64(a.view(np.uint16))
    return a.astype(np.float64)
