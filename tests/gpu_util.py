"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

from trellis_coded_bit_amd import binding as tb

# Tolerance for floating-point outputs: relative L2 over the whole output tensor.
REL_L2_TOL = 2e-3


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_linear(lin) -> tb.TrellisLinear:
    return tb.TrellisLinear.from_host(lin, "cuda")


def as_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def rel_l2(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def log_case(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
