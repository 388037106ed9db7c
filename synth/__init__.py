"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds random-number generation only: no block format, no codebook, no
quantisation, no routing and no matrix product.  Everything the method computes lives
either in the HIP library or, independently, in the CPU oracle.

Generator
---------
SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014), used counter-style: output i of a stream with start state ``s0`` is
``mix64(s0 + (i + 1) * GAMMA)``, so any range of a stream can be produced on its own
and in parallel.  A stream is keyed by (seed, tag): ``s0 = mix64(mix64(seed) ^ tag)``.

* uniform in [0, 1):        ``(x >> 11) * 2**-53``
* open uniform in (0, 1):   ``((x >> 11) + 0.5) * 2**-53``
* standard normal:          Box-Muller on consecutive pairs (u1, u2):
                            ``r = sqrt(-2 ln(1 - u1))``, outputs ``r cos(2 pi u2)``,
                            ``r sin(2 pi u2)``, computed in float64.

Workload recipes (sizes from the five workloads these kernels are measured on):

* source weights   ``float32(0.02 * z)``  (standard deviation 0.02)
* fp32 activations ``float32(z)``
* f16 activations  ``float16(z)`` (round to nearest even)
* decode routing logits ``float32(z)``
* prefill routing logits: Zipf(s) popularity through the Gumbel-top-k trick,
  ``L[t, e] = ln p_e + G[t, e]`` with ``p_e ~ (e + 1)**-s`` and
  ``G = -ln(-ln U)``; taking the k largest logits of a row draws k experts without
  replacement with probabilities proportional to p.

Seeds: plumbing matvec 101, verify-window matvec 102, expert bank 103 (shared by the
decode step and the prefill layer), decode step 103, prefill layer 104, long-prompt
projection 105, IQ4_XS matvec shapes 106 and 107.  Tensor tags: dense weight 0; expert e gate/up/down 3e, 3e+1, 3e+2;
activations 1000; decode logits 1001; Gumbel noise 1002.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

SEED_PLUMBING = 101
SEED_VERIFY = 102
SEED_EXPERTS = 103
SEED_DECODE = 103
SEED_PREFILL = 104
SEED_LONG = 105
# the IQ4_XS super-block matvec on the two shapes of page 2's cold/hot table
# (2560 x 6144 and 6144 x 2560, read as N x K)
SEED_XS_Z = 106
SEED_XS_OUT = 107

TAG_WEIGHT = 0
TAG_X = 1000
TAG_LOGITS = 1001
TAG_GUMBEL = 1002


def tag_expert(e: int, which: str) -> int:
    """Tag of expert ``e``'s gate / up / down matrix."""
    return 3 * e + {"gate": 0, "up": 1, "down": 2}[which]


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tag: int) -> int:
    """Start state of the (seed, tag) stream."""
    return _mix64_int(_mix64_int(seed) ^ (tag & _MASK64))


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def raw_u64(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the (seed, tag) SplitMix64 stream."""
    s0 = np.uint64(stream_key(seed, tag))
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(s0 + i * GAMMA)


_CHUNK = 1 << 22


def _parallel(fn, count: int, out: np.ndarray) -> np.ndarray:
    """Fill ``out`` (flat, length ``count``) chunk by chunk, chunks in parallel."""
    starts = list(range(0, count, _CHUNK))
    if len(starts) <= 1:
        if count:
            fn(0, count)
        return out
    workers = min(len(starts), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda s: fn(s, min(count, s + _CHUNK)), starts))
    return out


def uniform(seed: int, tag: int, count: int, open_interval: bool = False) -> np.ndarray:
    """``count`` float64 uniforms from the (seed, tag) stream."""
    out = np.empty(count, dtype=np.float64)
    off = 0.5 if open_interval else 0.0

    def fill(a, b):
        x = raw_u64(seed, tag, a, b - a)
        out[a:b] = ((x >> np.uint64(11)).astype(np.float64) + off) * (2.0 ** -53)

    return _parallel(fill, count, out)


def normal(seed: int, tag: int, count: int) -> np.ndarray:
    """``count`` standard normals (float64) from the (seed, tag) stream, Box-Muller."""
    npair = (count + 1) // 2
    out = np.empty(2 * npair, dtype=np.float64)

    def fill(a, b):
        # a, b index pairs; pair j uses stream outputs 2j, 2j+1
        x = raw_u64(seed, tag, 2 * a, 2 * (b - a))
        u = (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log1p(-u1))
        th = (2.0 * np.pi) * u2
        out[2 * a:2 * b:2] = r * np.cos(th)
        out[2 * a + 1:2 * b:2] = r * np.sin(th)

    _parallel(fill, npair, out)
    return out[:count]


def weights_f32(seed: int, tag: int, rows: int, cols: int) -> np.ndarray:
    """Source weights ~ N(0, 0.02^2) as float32 [rows, cols]."""
    return (0.02 * normal(seed, tag, rows * cols)).astype(np.float32).reshape(rows, cols)


def acts_f32(seed: int, tag: int, rows: int, cols: int) -> np.ndarray:
    """Activations ~ N(0, 1) as float32 [rows, cols] (token-major)."""
    return normal(seed, tag, rows * cols).astype(np.float32).reshape(rows, cols)


def acts_f16(seed: int, tag: int, rows: int, cols: int) -> np.ndarray:
    """Activations ~ N(0, 1) rounded to float16 [rows, cols] (token-major)."""
    return normal(seed, tag, rows * cols).astype(np.float16).reshape(rows, cols)


def logits_normal(seed: int, tag: int, n_tok: int, n_expert: int) -> np.ndarray:
    """Router logits ~ N(0, 1), float32 [n_tok, n_expert]."""
    return normal(seed, tag, n_tok * n_expert).astype(np.float32).reshape(n_tok, n_expert)


def logits_zipf_gumbel(seed: int, tag: int, n_tok: int, n_expert: int, s: float = 1.1) -> np.ndarray:
    """Router logits whose top-k is a Zipf(s)-weighted draw without replacement.

    ``L[t, e] = ln p_e + G[t, e]`` with ``p_e = (e+1)**-s / sum`` and Gumbel(0, 1)
    noise ``G = -ln(-ln U)``, U open-uniform; float64 arithmetic, stored as float32.
    """
    e = np.arange(n_expert, dtype=np.float64)
    p = (e + 1.0) ** (-s)
    lp = np.log(p / p.sum())
    u = uniform(seed, tag, n_tok * n_expert, open_interval=True).reshape(n_tok, n_expert)
    g = -np.log(-np.log(u))
    return (lp[None, :] + g).astype(np.float32)


# ----------------------------------------------------------------------------------
# The same streams produced with torch (CPU or GPU), for large inputs.  The 64-bit
# integer stream is bit-identical to the numpy version; the float64 Box-Muller step may
# differ from it in the last bit (device libm), which leaves the float32/float16
# results equal except, rarely, at a rounding boundary.  Parity tests use the numpy
# version; the benchmark uses this one to build its 600M-weight expert bank quickly.

def _as_i64(v: int) -> int:
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(z, s: int):
    import torch
    return torch.bitwise_and(torch.bitwise_right_shift(z, s), (1 << (64 - s)) - 1)


def _mix64_t(z):
    z = torch_bitxor(z, _lsr(z, 30)) * _as_i64(0xBF58476D1CE4E5B9)
    z = torch_bitxor(z, _lsr(z, 27)) * _as_i64(0x94D049BB133111EB)
    return torch_bitxor(z, _lsr(z, 31))


def torch_bitxor(a, b):
    import torch
    return torch.bitwise_xor(a, b)


def raw_u64_torch(seed: int, tag: int, start: int, count: int, device="cpu"):
    """Same values as ``raw_u64`` as a torch int64 tensor (two's complement bits)."""
    import torch
    s0 = _as_i64(stream_key(seed, tag))
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _mix64_t(i * _as_i64(int(GAMMA)) + s0)


def normal_torch(seed: int, tag: int, count: int, device="cpu"):
    """``count`` standard normals (float64 torch tensor), Box-Muller as in ``normal``."""
    import torch
    npair = (count + 1) // 2
    out = torch.empty(2 * npair, dtype=torch.float64, device=device)
    chunk = 1 << 24
    for a in range(0, npair, chunk):
        b = min(npair, a + chunk)
        x = raw_u64_torch(seed, tag, 2 * a, 2 * (b - a), device)
        u = _lsr(x, 11).to(torch.float64) * (2.0 ** -53)
        u1, u2 = u[0::2], u[1::2]
        r = torch.sqrt(-2.0 * torch.log1p(-u1))
        th = (2.0 * torch.pi) * u2
        out[2 * a:2 * b:2] = r * torch.cos(th)
        out[2 * a + 1:2 * b:2] = r * torch.sin(th)
    return out[:count]


def weights_f32_torch(seed: int, tag: int, rows: int, cols: int, device="cpu"):
    return (0.02 * normal_torch(seed, tag, rows * cols, device)).to(__import__("torch").float32).reshape(rows, cols)


def acts_f32_torch(seed: int, tag: int, rows: int, cols: int, device="cpu"):
    return normal_torch(seed, tag, rows * cols, device).to(__import__("torch").float32).reshape(rows, cols)


def acts_f16_torch(seed: int, tag: int, rows: int, cols: int, device="cpu"):
    return normal_torch(seed, tag, rows * cols, device).to(__import__("torch").float16).reshape(rows, cols)
