"""Helpers for the GPU tests: move packed numpy inputs onto the device."""

import numpy as np
import torch


def dev_codes(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).cuda()


def dev_steps(steps: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(steps).view(np.int16)).cuda().view(torch.bfloat16)


def dev_act(bits: np.ndarray, dtype: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if dtype == 0 else torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def within_bound(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, rel: float = 1e-3):
    """max |y - y_ref| <= rel * sum|w x| per output (zero-bound outputs must be
    exactly zero).  Returns (ok, worst ratio)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    ok = np.all(err <= rel * a_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(a_ref > 0, err / a_ref, np.where(err > 0, np.inf, 0.0))
    return bool(ok), float(ratio.max()) if ratio.size else 0.0
