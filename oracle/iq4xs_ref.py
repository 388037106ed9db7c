"""Plain CPU reference (numpy, float64) of the IQ4_XS super-block format: decode, a
test-input encoder, and the T-column matrix-vector product.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``; the HIP
library never imports it and shares no code with it.

Source.  Page 2 (the Strata pull request "sm_80 (GA100) tuning") names this format
three times: the wide-dequant commit message lists it among the dense weight types
decoded every prompt chunk; the MMVQ-IL harness commit message times its matvec cold
and hot on two shapes (2560 x 6144 and 6144 x 2560); and the MMVQ-IL_PF commit message
states its integer block dot: the sum of codebook levels times 8-bit activations is
multiplied by the float of ``ls - 32``, exact below 2^24.  So each 32-weight sub-block
carries an unsigned scale code ``ls`` whose signed value is ``ls - 32``.  The pages
never print the byte layout; this module takes the format's public definition:

* a super-block holds 256 weights (8 sub-blocks of 32) in 136 bytes;
* bytes 0-1: the super-block scale ``d``, little-endian IEEE binary16;
* bytes 2-3: a little-endian 16-bit word whose bits ``2i, 2i+1`` are the two high
  bits of sub-block i's 6-bit code ``ls_i``;
* bytes 4-7: byte ``4 + i // 2`` holds the four low bits of ``ls_i`` in its low nibble
  (i even) or high nibble (i odd);
* bytes 8-135: sub-block i's 32 indices in bytes ``8 + 16 i + m`` (m < 16): element
  ``32 i + m`` in the low nibble and element ``32 i + 16 + m`` in the high nibble (the
  split-half order of the 18-byte blocks);
* weight ``32 i + j`` decodes to ``d * (ls_i - 32) * c[q]`` with the same 16-level
  codebook as the 18-byte blocks.  Its significand needs at most 11 + 5 + 7 bits, so
  the product is exact in binary32 (and in float64 here).

The encoder is a generator of test inputs only (the pages describe none; weights reach
the library already encoded): per sub-block the binary32 scale ``s_i = absmax_i / 127``;
``d = f16_rne(f32(max_i s_i / 31))``; ``ls_i - 32 = m_i``, the nearest integer of
``s_i / d`` (halves up), clamped to [0, 31] (0 when d is 0); each weight takes the
level nearest to ``w / (d m_i)`` in exact arithmetic, ties to the lower index, and
index 8 where ``d m_i`` is zero.

Parity pins: hand-worked golden super-blocks, the reduction to the 18-byte block
decoder when every ``ls`` is 33, bit-position pins of the scale fields, exact rational
brute force on tiny products, and an integer-exact product.
"""
from __future__ import annotations

import numpy as np

from .iq4_ref import CODEBOOK

__all__ = ["XS_QK", "XS_SUB", "XS_BYTES", "xs_subscales", "xs_indices", "xs_scales",
           "decode_xs", "decode_xs_f16", "encode_xs", "qmv_xs"]

#: Weights per super-block, per sub-block, and bytes per super-block.
XS_QK = 256
XS_SUB = 32
XS_BYTES = 136


def _as_superblocks(sb) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(sb, dtype=np.uint8))
    return b.reshape(-1, XS_BYTES)


def xs_scales(sb: np.ndarray) -> np.ndarray:
    """The binary16 super-block scale ``d`` of every super-block, as float64 (exact)."""
    b = _as_superblocks(sb)
    return b[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)


def xs_subscales(sb) -> np.ndarray:
    """The unsigned 6-bit codes ``ls_i`` (0..63) of the 8 sub-blocks ([nsb, 8] int)."""
    b = _as_superblocks(sb).astype(np.int64)
    high_word = b[:, 2] | (b[:, 3] << 8)
    ls = np.empty((b.shape[0], 8), dtype=np.int64)
    for i in range(8):
        low4 = (b[:, 4 + i // 2] >> (4 * (i % 2))) & 0xF
        high2 = (high_word >> (2 * i)) & 0x3
        ls[:, i] = low4 | (high2 << 4)
    return ls


def xs_indices(sb) -> np.ndarray:
    """The 256 codebook indices of every super-block, in element order ([nsb, 256])."""
    b = _as_superblocks(sb).astype(np.int64)
    q = np.empty((b.shape[0], XS_QK), dtype=np.int64)
    for i in range(8):
        qs = b[:, 8 + 16 * i: 8 + 16 * i + 16]
        q[:, 32 * i: 32 * i + 16] = qs & 0xF
        q[:, 32 * i + 16: 32 * i + 32] = qs >> 4
    return q


def decode_xs(sb) -> np.ndarray:
    """Decoded weights ``d * (ls_i - 32) * codebook[q]`` as float32 ``[nsb, 256]``
    (exact: at most 23 significant bits)."""
    b = _as_superblocks(sb)
    cb = np.asarray(CODEBOOK, dtype=np.float64)
    sub = (xs_subscales(b) - 32).astype(np.float64)                  # [nsb, 8]
    lev = cb[xs_indices(b)].reshape(-1, 8, XS_SUB)                   # [nsb, 8, 32]
    w = xs_scales(b)[:, None, None] * sub[:, :, None] * lev
    return w.reshape(-1, XS_QK).astype(np.float32)


def decode_xs_f16(sb) -> np.ndarray:
    """Decoded weights rounded to binary16 (round to nearest even, subnormals kept)."""
    return decode_xs(sb).astype(np.float16)


_ENCODE_CHUNK = 4096


def encode_xs(w) -> np.ndarray:
    """Test-input encoder: float32 weights ``[nsb, 256]`` -> super-blocks ``[nsb, 136]``
    (uint8), by the rule in the module docstring.  Inputs must be finite with
    ``max|w| / (127 * 31) <= 65504``."""
    w32 = np.ascontiguousarray(np.asarray(w, dtype=np.float32)).reshape(-1, 8, XS_SUB)
    nsb = w32.shape[0]
    if nsb > _ENCODE_CHUNK:  # bound the [sb, 8, 32, 16] distance array; same result
        return np.concatenate([encode_xs(w32[i:i + _ENCODE_CHUNK]) for i in range(0, nsb, _ENCODE_CHUNK)])
    s = (np.max(np.abs(w32), axis=2) / np.float32(127.0)).astype(np.float32)   # [nsb, 8]
    d16 = (np.max(s, axis=1) / np.float32(31.0)).astype(np.float32).astype(np.float16)
    d = d16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.floor(s.astype(np.float64) / d[:, None] + 0.5)
    m = np.where(d[:, None] > 0, np.clip(m, 0, 31), 0).astype(np.int64)
    step = d[:, None] * m                                                      # exact
    cb = np.asarray(CODEBOOK, dtype=np.float64)
    dist = np.abs(w32.astype(np.float64)[:, :, :, None] - step[:, :, None, None] * cb)
    q = np.argmin(dist, axis=3)                                                # first minimum
    q[step == 0.0] = 8
    ls = m + 32
    out = np.zeros((nsb, XS_BYTES), dtype=np.uint8)
    out[:, 0:2] = d16.astype("<f2").view(np.uint8).reshape(nsb, 2)
    high = np.zeros(nsb, dtype=np.int64)
    for i in range(8):
        high |= (ls[:, i] >> 4) << (2 * i)
        out[:, 4 + i // 2] |= ((ls[:, i] & 0xF) << (4 * (i % 2))).astype(np.uint8)
        out[:, 8 + 16 * i: 8 + 16 * i + 16] = (q[:, i, :16] | (q[:, i, 16:] << 4)).astype(np.uint8)
    out[:, 2] = (high & 0xFF).astype(np.uint8)
    out[:, 3] = (high >> 8).astype(np.uint8)
    return out


def qmv_xs(sb, n: int, k: int, x) -> np.ndarray:
    """T-column product ``Y[t][r] = sum_k W[r][k] * X[t][k]`` with W the decoded
    ``n x k`` matrix (row r = k/256 consecutive super-blocks), summed in float64 and
    rounded once to float32 (``[T, n]``)."""
    b = _as_superblocks(sb)
    if k % XS_QK or b.shape[0] != n * (k // XS_QK):
        raise ValueError("super-block count does not match N x K (K a multiple of 256)")
    W = decode_xs(b).astype(np.float64).reshape(n, k)
    X = np.asarray(x, dtype=np.float64).reshape(-1, k)
    return (X @ W.T).astype(np.float32)
