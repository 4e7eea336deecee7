"""Shared helpers of the GPU tests: upload inputs, read back results, compare codes."""
import sys

import numpy as np
import torch

import oracle


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def np_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def codes_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)


def compare_codes(gpu: np.ndarray, ref: np.ndarray, y: np.ndarray):
    """Codes must agree bit for bit except where the oracle's pre-sign value is near
    zero; returns the number of exempt bits that differ."""
    diff = gpu ^ ref
    exempt = oracle.near_zero_mask(y)
    bad = diff & ~exempt
    assert not bad.any(), f"{int(np.bitwise_count(bad).sum())} code bits differ outside the near-zero exemption"
    return int(np.bitwise_count(diff).sum())


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()
