"""Helpers for the GPU parity tests (device buffers, packing, error norms)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dequant_matmul_iq4_amd as iq4

DEV = "cuda"


def note(msg: str):
    """Print and flush a line naming the case about to run on the GPU."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pack(blocks: np.ndarray | torch.Tensor, n: int, k: int) -> torch.Tensor:
    b = blocks if isinstance(blocks, torch.Tensor) else dev(blocks.reshape(-1))
    nbytes = iq4.iq4_packed_bytes(n, k)
    assert nbytes > 0 and b.numel() == nbytes, (n, k, b.numel())
    packed = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    iq4.iq4_pack_weights(b, n, k, packed)
    return packed


def normwise(y: np.ndarray, r: np.ndarray) -> float:
    """max |y - r| / max |r| (the tolerance measure used throughout)."""
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(np.asarray(y, dtype=np.float64) - r)) / (den if den > 0 else 1.0))


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.dtype == b.dtype and a.shape == b.shape and a.tobytes() == b.tobytes()


_WS = {}


def qmv_workspace(n: int, k: int):
    """A zero-filled workspace for iq4_qmv_multi on an n x k matrix (cached per shape)."""
    nbytes = iq4.iq4_qmv_workspace_size(n, k)
    if nbytes == 0:
        return None, 0
    if (n, k) not in _WS:
        _WS[(n, k)] = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    return _WS[(n, k)], nbytes
