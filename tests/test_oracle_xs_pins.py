"""Pins of the oracle's IQ4_XS super-block functions to facts fixed outside them (CPU).

* hand-worked golden super-blocks (tests/golden/xs_superblocks.txt): decoded values,
  signs of zero, a subnormal scale with its binary16 roundings, and three products;
* the reduction to the 18-byte block decoder (itself pinned by golden blocks and its
  closed form) when every sub-block code is 33, i.e. ``ls - 32 = 1``;
* every 6-bit code in every sub-block position, with bytes packed here by hand;
* exact rational brute force of the encoder and of the product on tiny shapes.

The ``planted`` tests plant plausible mistakes (an offset of 31, the wrong bit pair,
swapped nibble halves, a transposed product)
and check that a pin fails on each.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle.iq4_ref as R
import oracle.iq4xs_ref as X
from conftest import read_golden
from exact import f16, f16_bits, f32

CB = [int(v) for v in read_golden("codebook.txt")["codebook"]]
G = read_golden("xs_superblocks.txt")


def _hex(tokens) -> bytes:
    return bytes(int(t, 16) for t in tokens)


def _bits32(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def golden_superblock(name: str) -> np.ndarray:
    hdr = _hex(G[f"{name}.header"])
    if name == "X1":
        qs = _hex(G["X1.qs_of_each_subblock"]) * 8
    elif name == "X2":
        qs = b"".join(bytes([b]) * 16 for b in _hex(G["X2.qs_byte_of_subblock"]))
    else:
        qs = _hex(G["X3.qs_byte"]) * 128
    assert len(hdr) == 8 and len(qs) == 128
    return np.frombuffer(hdr + qs, dtype=np.uint8).reshape(1, 136).copy()


def pack_superblock(d16_bits: int, ls: list, q: list) -> bytes:
    """Pack by hand: d, the high-bit word, the low-nibble bytes, then the indices."""
    high = 0
    low = [0, 0, 0, 0]
    for i, v in enumerate(ls):
        high |= (v >> 4) << (2 * i)
        low[i // 2] |= (v & 0xF) << (4 * (i % 2))
    out = struct.pack("<HH", d16_bits, high) + bytes(low)
    for i in range(8):
        sub = q[32 * i: 32 * i + 32]
        out += bytes(sub[m] | (sub[16 + m] << 4) for m in range(16))
    return out


# ----------------------------------------------------------------------------------


def pin_xs_sizes():
    assert (X.XS_QK, X.XS_SUB, X.XS_BYTES) == (256, 32, 136)
    assert X.XS_BYTES == 2 + 2 + 4 + 128   # d, high bits, low bits, 256 indices


def pin_xs_decode_golden():
    for name in ("X1", "X2"):
        got = X.decode_xs(golden_superblock(name)).reshape(-1)
        want = [float(v) for i in range(8) for v in G[f"{name}.sub{i}"]]
        assert [_bits32(v) for v in got] == [_bits32(v) for v in want], name  # signs of zero too
    sb = golden_superblock("X3")
    got32, got16 = X.decode_xs(sb).reshape(8, 32), X.decode_xs_f16(sb).reshape(8, 32)
    lo32, hi32 = (float(Fraction(G[f"X3.f32_{h}_half"][0])) for h in ("low", "high"))
    lo16, hi16 = (float(Fraction(G[f"X3.f16_{h}_half"][0])) for h in ("low", "high"))
    assert np.all(got32[:, :16] == lo32) and np.all(got32[:, 16:] == hi32)
    assert np.all(got16[:, :16].astype(np.float64) == lo16) and np.all(got16[:, 16:].astype(np.float64) == hi16)


def pin_xs_qmv_golden():
    sb = golden_superblock("X1")
    ones = np.ones((1, 256), np.float32)
    low = np.zeros((1, 256), np.float32)
    for i in range(8):
        low[0, 32 * i: 32 * i + 16] = 1
    sub5 = np.zeros((1, 256), np.float32)
    sub5[0, 160:192] = 1
    for x, key in ((ones, "y_ones"), (low, "y_low_halves"), (sub5, "y_sub5")):
        assert X.qmv_xs(sb, 1, 256, x)[0, 0] == float(G[f"X1.{key}"][0]), key


def pin_xs_unit_scale_is_the_block_decoder():
    """With every code 33 (ls - 32 = 1) sub-block i is an 18-byte block with the same d
    and the 16 index bytes 8 + 16i .. 8 + 16i + 15."""
    rng = np.random.default_rng(5)
    nsb = 64
    sb = rng.integers(0, 256, (nsb, 136), dtype=np.uint8)
    d = (rng.standard_normal(nsb) * 0.01).astype(np.float16)
    d[:4] = [0.0, -0.0, np.float16(6e-8), np.float16(-65504)]
    sb[:, 0:2] = d.view(np.uint8).reshape(nsb, 2)
    sb[:, 2:4] = 0xAA          # high bits 2 everywhere
    sb[:, 4:8] = 0x11          # low bits 1 everywhere
    blocks = np.empty((nsb * 8, 18), dtype=np.uint8)
    for i in range(8):
        blocks[i::8, 0:2] = sb[:, 0:2]
        blocks[i::8, 2:18] = sb[:, 8 + 16 * i: 8 + 16 * i + 16]
    a = X.decode_xs(sb).reshape(-1)
    b = R.decode_blocks(blocks).reshape(-1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def pin_xs_every_code_in_every_position():
    """Each of the 64 codes in each of the 8 positions, bytes packed by hand: with d = 1
    and every index 8 (level 1), sub-block i decodes to ls - 32 and the others, at code
    32, to +0."""
    q = [8] * 256
    for pos in range(8):
        for code in range(64):
            ls = [32] * 8
            ls[pos] = code
            sb = np.frombuffer(pack_superblock(0x3C00, ls, q), dtype=np.uint8).reshape(1, 136)
            w = X.decode_xs(sb).reshape(8, 32)
            assert np.all(w[pos] == code - 32), (pos, code)
            others = np.delete(w, pos, axis=0)
            assert np.all(others.view(np.uint32) == 0), (pos, code)


def bf_encode_xs(w: list) -> bytes:
    """Encode 256 float32 values by hand in exact arithmetic (the encoder's stated rule)."""
    wf = [Fraction(float(v)) for v in w]
    s = [f32(max(abs(v) for v in wf[32 * i: 32 * i + 32]) / 127) for i in range(8)]
    d = f16(Fraction(f32(Fraction(max(s)) / 31)))
    ms, q = [], []
    for i in range(8):
        if d == 0:
            m = 0
        else:
            t = Fraction(s[i]) / Fraction(d)
            m = min(31, max(0, int((t + Fraction(1, 2)).__floor__())))
        ms.append(m)
        step = Fraction(d) * m
        for v in wf[32 * i: 32 * i + 32]:
            if step == 0:
                q.append(8)
                continue
            best, bj = None, None
            for j, c in enumerate(CB):
                dist = abs(v - step * c)
                if best is None or dist < best:       # strict: ties keep the lower index
                    best, bj = dist, j
            q.append(bj)
    return pack_superblock(f16_bits(d), [m + 32 for m in ms], q)


def xs_encode_cases(seed=13):
    rng = np.random.default_rng(seed)
    cases = [(rng.standard_normal((3, 256)) * 0.02).astype(np.float32)]
    skew = (rng.standard_normal((2, 256)) * 0.02).astype(np.float32)
    skew[:, 0:32] *= 40.0                   # one loud sub-block: the others get small codes
    skew[1, 64:96] = 0.0                     # an all-zero sub-block
    cases.append(skew)
    z = np.zeros((1, 256), np.float32)
    cases.append(z)
    # values on the level grid of a chosen scale, and midpoints between two levels
    d, m = np.float16(2.0 ** -8), 3
    g = np.array([c * float(d) * m for c in CB] * 16, np.float32).reshape(1, 256)
    g[0, 0] = 127 * 31 * float(d) / m * m    # pins d through max|w|
    cases.append(g)
    mid = g.copy()
    mid[0, 1:16] = [(CB[j] + CB[j + 1]) / 2 * float(d) * m for j in range(15)]
    cases.append(mid)
    return np.concatenate(cases)


def pin_xs_encode_bruteforce():
    w = xs_encode_cases()
    got = X.encode_xs(w)
    for r in range(w.shape[0]):
        assert bytes(got[r]) == bf_encode_xs(list(w[r])), r


def pin_xs_encode_idempotent():
    """Weights already of the form d * m_i * c (d a binary16 value, every m_i >= 1, one
    of them 31, level -127 in every sub-block) encode back to the same bytes."""
    rng = np.random.default_rng(21)
    for _ in range(12):
        d = np.float16(rng.uniform(2.0 ** -12, 2.0 ** -4))
        ms = list(rng.integers(1, 32, 8))
        ms[int(rng.integers(0, 8))] = 31
        q = [int(v) for v in rng.integers(0, 16, 256)]
        for i in range(8):
            q[32 * i + int(rng.integers(0, 32))] = 0
        sb = np.frombuffer(pack_superblock(f16_bits(float(d)), [m + 32 for m in ms], q), np.uint8).reshape(1, 136)
        assert bytes(X.encode_xs(X.decode_xs(sb))[0]) == bytes(sb[0])


def pin_xs_qmv_fraction():
    rng = np.random.default_rng(17)
    n, k, T = 3, 512, 2
    sb = rng.integers(0, 256, (n * k // 256, 136), dtype=np.uint8)
    sb[:, 0:2] = (rng.standard_normal(sb.shape[0]) * 0.01).astype(np.float16).view(np.uint8).reshape(-1, 2)
    x = rng.standard_normal((T, k)).astype(np.float32)
    got = X.qmv_xs(sb, n, k, x)
    for r in range(n):
        w = []
        for b in range(k // 256):
            blk = bytes(sb[r * (k // 256) + b])
            d = Fraction(struct.unpack("<e", blk[0:2])[0])
            hi = struct.unpack("<H", blk[2:4])[0]
            for i in range(8):
                ls = ((blk[4 + i // 2] >> (4 * (i % 2))) & 0xF) | (((hi >> (2 * i)) & 3) << 4)
                qs = blk[8 + 16 * i: 8 + 16 * i + 16]
                idx = [v & 0xF for v in qs] + [v >> 4 for v in qs]
                w += [d * (ls - 32) * CB[j] for j in idx]
        for t in range(T):
            exact = sum(wv * Fraction(float(xv)) for wv, xv in zip(w, x[t]))
            want = f32(exact)
            assert abs(float(got[t, r]) - want) <= abs(want) * 2.0 ** -23, (t, r)


def pin_xs_qmv_one_hot():
    rng = np.random.default_rng(3)
    n, k = 4, 512
    sb = X.encode_xs((rng.standard_normal((n * k // 256, 256)) * 0.02).astype(np.float32))
    W = X.decode_xs(sb).reshape(n, k)
    for j in (0, 17, 255, 256, 300, 511):
        x = np.zeros((1, k), np.float32)
        x[0, j] = 1
        assert np.array_equal(X.qmv_xs(sb, n, k, x)[0], W[:, j])


PINS = [pin_xs_sizes, pin_xs_decode_golden, pin_xs_qmv_golden, pin_xs_unit_scale_is_the_block_decoder,
        pin_xs_every_code_in_every_position, pin_xs_encode_bruteforce, pin_xs_encode_idempotent,
        pin_xs_qmv_fraction, pin_xs_qmv_one_hot]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail

_orig_sub = X.xs_subscales
_orig_idx = X.xs_indices


def _offset31(sb):
    return _orig_sub(sb) + 1          # decode then uses ls - 31


def _high_bits_wrong_pair(sb):
    b = np.ascontiguousarray(np.asarray(sb, dtype=np.uint8)).reshape(-1, 136).astype(np.int64)
    hw = b[:, 2] | (b[:, 3] << 8)
    ls = np.empty((b.shape[0], 8), dtype=np.int64)
    for i in range(8):
        ls[:, i] = ((b[:, 4 + i // 2] >> (4 * (i % 2))) & 0xF) | (((hw >> (2 * (7 - i))) & 3) << 4)
    return ls


def _low_nibbles_swapped(sb):
    b = np.ascontiguousarray(np.asarray(sb, dtype=np.uint8)).reshape(-1, 136).astype(np.int64)
    hw = b[:, 2] | (b[:, 3] << 8)
    ls = np.empty((b.shape[0], 8), dtype=np.int64)
    for i in range(8):
        ls[:, i] = ((b[:, 4 + i // 2] >> (4 * (1 - i % 2))) & 0xF) | (((hw >> (2 * i)) & 3) << 4)
    return ls


def _xs_halves_swapped(sb):
    q = _orig_idx(sb).reshape(-1, 8, 2, 16)
    return q[:, :, ::-1, :].reshape(-1, 256)


def _xs_qmv_transposed(sb, n, k, x):
    W = X.decode_xs(sb).astype(np.float64).reshape(k, n)
    return (np.asarray(x, dtype=np.float64).reshape(-1, k) @ W).astype(np.float32)


_orig_encode_xs = X.encode_xs


def _encode_codes_floor(w):
    # sub-block codes truncated instead of rounded to nearest
    out = _orig_encode_xs(w)
    w32 = np.asarray(w, dtype=np.float32).reshape(-1, 8, 32)
    s = (np.max(np.abs(w32), axis=2) / np.float32(127)).astype(np.float32)
    d = out[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.where(d[:, None] > 0, np.clip(np.floor(s / d[:, None]), 0, 31), 0).astype(np.int64)
    ls = m + 32
    high = np.zeros(out.shape[0], dtype=np.int64)
    out[:, 4:8] = 0
    for i in range(8):
        high |= (ls[:, i] >> 4) << (2 * i)
        out[:, 4 + i // 2] |= ((ls[:, i] & 0xF) << (4 * (i % 2))).astype(np.uint8)
    out[:, 2] = (high & 0xFF).astype(np.uint8)
    out[:, 3] = (high >> 8).astype(np.uint8)
    return out


PLANTED = {
    "encoder truncates the sub-block codes": ("encode_xs", _encode_codes_floor),
    "sub-scale offset 31": ("xs_subscales", _offset31),
    "high bits from the mirrored pair": ("xs_subscales", _high_bits_wrong_pair),
    "low nibbles of a code byte swapped": ("xs_subscales", _low_nibbles_swapped),
    "index halves swapped": ("xs_indices", _xs_halves_swapped),
    "product transposed": ("qmv_xs", _xs_qmv_transposed),
}


def _fails(pins):
    failed = []
    for p in pins:
        try:
            with np.errstate(all="ignore"):
                p()
        except Exception:
            failed.append(p.__name__)
    return failed


@pytest.mark.parametrize("name", list(PLANTED))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, value = PLANTED[name]
    monkeypatch.setattr(X, attr, value)
    assert _fails(PINS), f"no pin caught the planted mistake: {name}"
