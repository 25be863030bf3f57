"""Shared helpers of the GPU parity tests (no method arithmetic here: the references come
from the oracle, the products from the library)."""
import numpy as np
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb

# Tolerance for floating-point outputs: relative L2 over the whole output tensor.
REL_L2_TOL = 2e-3


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_linear(lin, null_scales: bool = False) -> tb.TrellisLinear:
    """The layer on the device; null_scales passes s_in = s_out = NULL (all ones)."""
    L = tb.TrellisLinear.from_host(lin, "cuda")
    if null_scales:
        L = tb.TrellisLinear(L.code, L.rin, L.rout, None, None, L.K, L.cb)
    return L


def as_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def rel_l2(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def log_case(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


# The oracle's decoded matrices, one decode per (workload, name) for the whole session: the
# full-size tests compare complete outputs, and several of them read the same matrix.
_W_HAT = {}


def oracle_w_hat(key, lin) -> np.ndarray:
    if key not in _W_HAT:
        _W_HAT[key] = O.decode_tiles(lin.code, lin.K, getattr(lin, "cb", 1))
    return _W_HAT[key]


def oracle_forward_full(key, lin, x, null_scales: bool = False, act_e4m3: bool = False) -> np.ndarray:
    """The oracle's whole output for this layer and input (its decode cached under key);
    act_e4m3 selects the FP8 prefill's per-row E4M3 activations."""
    w = oracle_w_hat(key, lin)
    s_in, s_out = (None, None) if null_scales else (lin.s_in, lin.s_out)
    return O.forward_decoded(w, lin.rin, lin.rout, s_in, s_out, x, act_e4m3=act_e4m3)


def worst_block_rel_l2(y: np.ndarray, ref: np.ndarray, rows: int = 512, cols: int = 128) -> float:
    """The largest relative L2 over row bands x column blocks: no part of the output may be
    off on its own while the whole tensor passes."""
    worst = 0.0
    for r0 in range(0, ref.shape[0], rows):
        for c0 in range(0, ref.shape[1], cols):
            worst = max(worst, rel_l2(y[r0:r0 + rows, c0:c0 + cols], ref[r0:r0 + rows, c0:c0 + cols]))
    return worst
