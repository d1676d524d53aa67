"""Host <-> device helpers for the GPU parity tests (no codec arithmetic here)."""
import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous GPU tensor with the same bytes (uint16 goes as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint64:
        a = a.view(np.int64)
    return torch.from_numpy(a.copy()).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def zeros(n, dtype):
    return torch.zeros(max(int(n), 1), dtype=dtype, device="cuda")


def u16(t):
    return host(t, np.uint16)
