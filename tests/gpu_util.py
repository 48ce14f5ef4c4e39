"""Helpers for GPU tests: host numpy <-> device torch, no arithmetic."""
import numpy as np
import torch

DEV = "cuda:0"


def gpu_available() -> bool:
    return torch.cuda.is_available()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).copy()).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def announce(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
