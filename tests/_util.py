"""Helpers shared by the parity tests: torch <-> numpy views of bf16 / uint32
data and the GPU device handle."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (numpy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def np_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def u32_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def host(t: torch.Tensor) -> np.ndarray:
    """Tensor -> numpy in the oracle's convention (bf16 as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return bf16_np(t)
    return t.detach().cpu().contiguous().numpy()


def row_norms(a: np.ndarray) -> np.ndarray:
    return np.sqrt((a.astype(np.float64) ** 2).sum(axis=1))
