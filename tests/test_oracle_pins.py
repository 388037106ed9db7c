"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Every oracle function is checked against something other than itself: hand-worked
golden blocks, the decode closed form over every index and special scale, exact
rational brute force (``fractions.Fraction``) on tiny shapes, closed forms and
invariants.  The ``planted`` tests at the end plant a plausible mistake in the oracle
(a flipped codebook sign, swapped nibble halves, a transposed operand, the wrong tie
rule, a dropped gate weight, ...) and check that at least one pin fails on it.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle.iq4_ref as R
from conftest import read_golden
from exact import f16, f16_bits, f32, f32_bits, f32_ulp

CB = [int(v) for v in read_golden("codebook.txt")["codebook"]]


# ----------------------------------------------------------------------------------
# independent helpers (pure Python; the codebook comes from the golden file)


def bf_decode_block(b: bytes) -> list:
    """Decode one 18-byte block by hand: exact rationals, or IEEE double products
    where the scale is zero or not finite (to keep signed zeros, infinities, NaN)."""
    d = struct.unpack("<e", bytes(b[0:2]))[0]
    q = [b[2 + i] & 0xF for i in range(16)] + [b[2 + i] >> 4 for i in range(16)]
    if d == 0 or not math.isfinite(d):
        return [d * CB[v] for v in q]
    return [Fraction(d) * CB[v] for v in q]


def bf_encode_block(w: list) -> bytes:
    """Encode 32 float32 values by hand in exact arithmetic."""
    wf = [Fraction(float(v)) for v in w]
    a = max(abs(v) for v in wf)
    d32 = f32(a / 127)
    d = f16(Fraction(d32))
    q = []
    for v in wf:
        if d == 0:
            q.append(8)
            continue
        best, bj = None, None
        for j, c in enumerate(CB):
            dist = abs(v - Fraction(d) * c)
            if best is None or dist < best:  # strict: ties keep the lower index
                best, bj = dist, j
        q.append(bj)
    out = struct.pack("<H", f16_bits(d))
    out += bytes(q[i] | (q[i + 16] << 4) for i in range(16))
    return out


def rand_blocks(rng: np.random.Generator, nb: int, scale: float = 0.02) -> np.ndarray:
    """Random valid blocks: random indices and random positive fp16 scales."""
    b = np.empty((nb, 18), dtype=np.uint8)
    d = (rng.uniform(0.3, 1.0, nb) * scale / 127 * 4).astype(np.float16)
    b[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    b[:, 2:] = rng.integers(0, 256, (nb, 16), dtype=np.uint8)
    return b


def bf_matrix(blocks: np.ndarray, n: int, k: int) -> list:
    rows = []
    nbr = k // 32
    for r in range(n):
        row = []
        for j in range(nbr):
            row += bf_decode_block(bytes(blocks[r * nbr + j]))
        rows.append(row)
    return rows


def assert_f32_close_to_exact(got: float, exact: Fraction, ulps: int = 1):
    assert abs(Fraction(float(got)) - exact) <= ulps * Fraction(f32_ulp(float(exact))), (got, float(exact))


# ----------------------------------------------------------------------------------
# pins: format


def pin_codebook():
    assert list(R.CODEBOOK) == CB


def pin_block_size():
    g = read_golden("ple_compact.txt")
    n, nbytes = int(g["values"][0]), int(g["iq4_bytes"][0])
    assert n // R.QK * R.BLOCK_BYTES == nbytes
    w = np.linspace(-1, 1, n, dtype=np.float32).reshape(-1, 32)
    assert R.encode_blocks(w).size == nbytes
    assert int(g["fp32_bytes"][0]) == 4 * n


def pin_decode_golden():
    g = read_golden("block_decode.txt")
    for name in "ABC":
        b = np.array([int(x, 16) for x in g[name + ".bytes"]], dtype=np.uint8)
        want = np.array([float(x) for x in g[name + ".values"]], dtype=np.float32)
        got = R.decode_blocks(b).reshape(-1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name


SPECIAL_D = [0.0, -0.0, 2.0 ** -24, 2.0 ** -14, 0.5, 1.0, -1.5, 65504.0, math.inf, -math.inf, math.nan]


def special_blocks():
    """Every index at every position, under every special scale."""
    blocks = []
    for d in SPECIAL_D:
        for shift in range(16):
            b = bytearray(struct.pack("<e", d))
            for i in range(16):
                lo = (i + shift) % 16
                hi = (i + 3 * shift + 5) % 16
                b.append(lo | (hi << 4))
            blocks.append(bytes(b))
    return blocks


def pin_decode_closed_form():
    blocks = special_blocks()
    got = R.decode_blocks(np.frombuffer(b"".join(blocks), dtype=np.uint8))
    for r, b in enumerate(blocks):
        want = bf_decode_block(b)
        for i in range(32):
            wv = float(want[i])
            g = float(got[r, i])
            if math.isnan(wv):
                assert math.isnan(g)
            else:
                # exact, including the sign of zero
                assert f32_bits(g) == f32_bits(wv), (r, i, g, wv)


def pin_decode_f16():
    rng = np.random.default_rng(5)
    blocks = list(special_blocks())
    for _ in range(64):
        d = float(np.float16(rng.uniform(-3, 3) * 10.0 ** rng.integers(-6, 3)))
        blocks.append(struct.pack("<e", d) + bytes(rng.integers(0, 256, 16, dtype=np.uint8).tolist()))
    got = R.decode_blocks_f16(np.frombuffer(b"".join(blocks), dtype=np.uint8))
    for r, b in enumerate(blocks):
        for i, v in enumerate(bf_decode_block(b)):
            if isinstance(v, float):
                continue  # non-finite scales: covered by the f32 closed form
            want = f16(v)
            g = float(got[r, i])
            assert (g == want and math.copysign(1, g) == math.copysign(1, want)) or (
                math.isinf(want) and g == want), (r, i, g, want)


def pin_encode_golden():
    g = read_golden("block_encode.txt")
    w = np.array([float(m) * 2.0 ** -7 for m in g["m"]], dtype=np.float32)
    want = bytes(int(x, 16) for x in g["bytes"])
    assert bytes(R.encode_blocks(w).reshape(-1)) == want


def encode_cases(seed=11):
    rng = np.random.default_rng(seed)
    cases = []
    for s in [1e-3, 0.02, 1.0, 300.0, 1e-6]:
        for _ in range(6):
            cases.append((rng.standard_normal(32) * s).astype(np.float32))
    # ties: multiples of a power-of-two scale placed on level midpoints
    for p in (-7, 0, 3):
        m = [CB[0]] + [(CB[j] + CB[j + 1]) / 2 for j in range(15)] + [CB[j] for j in range(16)]
        cases.append((np.array(m) * 2.0 ** p).astype(np.float32))
    # positive-max blocks (saturate at the top level), all-zero and near-zero blocks
    cases.append(np.abs(rng.standard_normal(32)).astype(np.float32))
    cases.append(np.zeros(32, dtype=np.float32))
    z = np.zeros(32, dtype=np.float32)
    z[3] = 1e-9
    cases.append(z)
    return cases


def pin_encode_bruteforce():
    cases = encode_cases()
    got = R.encode_blocks(np.stack(cases))
    for r, w in enumerate(cases):
        assert bytes(got[r]) == bf_encode_block(list(w)), r


def pin_encode_idempotent():
    rng = np.random.default_rng(3)
    b = rand_blocks(rng, 64)
    b[:, 2] = (b[:, 2] & 0xF0)  # q_0 = 0: the block's absmax is 127 d, so d is recovered
    w = R.decode_blocks(b)
    assert np.array_equal(R.encode_blocks(w), b)


def pin_encode_zero():
    b = R.encode_blocks(np.zeros((2, 32), dtype=np.float32))
    assert np.all(b[:, 0:2] == 0) and np.all(b[:, 2:] == 0x88)


# ----------------------------------------------------------------------------------
# pins: products


def pin_qmv_one_hot():
    rng = np.random.default_rng(1)
    n, k = 6, 96
    b = rand_blocks(rng, n * k // 32)
    W = bf_matrix(b, n, k)
    for col in (0, 1, 15, 16, 17, 31, 32, 63, 95):
        x = np.zeros((1, k), dtype=np.float32)
        x[0, col] = 1.0
        y = R.qmv(b, n, k, x)
        assert y.shape == (1, n)
        for r in range(n):
            assert Fraction(float(y[0, r])) == W[r][col], (col, r)


def pin_qmv_fraction():
    rng = np.random.default_rng(2)
    n, k, T = 5, 64, 3
    b = rand_blocks(rng, n * k // 32)
    x = rng.standard_normal((T, k)).astype(np.float32)
    W = bf_matrix(b, n, k)
    y = R.qmv(b, n, k, x)
    assert y.shape == (T, n)
    for t in range(T):
        for r in range(n):
            ex = sum(W[r][c] * Fraction(float(x[t, c])) for c in range(k))
            assert_f32_close_to_exact(y[t, r], ex)


def integer_exact_blocks(rng, nb, s):
    b = np.empty((nb, 18), dtype=np.uint8)
    d = np.full(nb, 2.0 ** -s, dtype=np.float16)
    b[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    b[:, 2:] = rng.integers(0, 256, (nb, 16), dtype=np.uint8)
    return b


def pin_qmv_integer_exact():
    rng = np.random.default_rng(4)
    n, k, T = 7, 128, 2
    b = integer_exact_blocks(rng, n * k // 32, 6)
    x = rng.integers(-8, 9, (T, k)).astype(np.float32)
    W = bf_matrix(b, n, k)
    y = R.qmv(b, n, k, x)
    for t in range(T):
        for r in range(n):
            ex = sum(W[r][c] * int(x[t, c]) for c in range(k))
            assert Fraction(float(y[t, r])) == ex


def pin_gemm_fraction():
    rng = np.random.default_rng(6)
    n, k, m = 3, 64, 4
    b = rand_blocks(rng, n * k // 32)
    x = rng.standard_normal((m, k)).astype(np.float16)
    W = bf_matrix(b, n, k)
    y = R.gemm(b, n, k, x)
    assert y.shape == (m, n)
    for i in range(m):
        for r in range(n):
            ex = sum(W[r][c] * Fraction(float(x[i, c])) for c in range(k))
            assert_f32_close_to_exact(y[i, r], ex)


def pin_gemm_integer_exact():
    rng = np.random.default_rng(7)
    n, k, m = 5, 96, 6
    b = integer_exact_blocks(rng, n * k // 32, 3)
    x = rng.integers(-8, 9, (m, k)).astype(np.float16)
    W = bf_matrix(b, n, k)
    y = R.gemm(b, n, k, x)
    for i in range(m):
        for r in range(n):
            assert Fraction(float(y[i, r])) == sum(W[r][c] * int(x[i, c]) for c in range(k))


# ----------------------------------------------------------------------------------
# pins: routing and gather


def pin_route_golden():
    g = read_golden("route_example.txt")
    L = np.array([[float(v) for v in g["logits"]]], dtype=np.float32)
    ids, w = R.route_topk(L, len(g["ids"]))
    assert ids.dtype == np.int32 and ids.tolist() == [[int(v) for v in g["ids"]]]
    assert np.allclose(w[0], [float(v) for v in g["weights"]], rtol=2e-7, atol=0)


def bf_route(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]
    z = [float(row[e]) for e in order]
    m = max(z)
    ex = [math.exp(v - m) for v in z]
    s = math.fsum(ex)
    return order, [v / s for v in ex]


def pin_route_bruteforce():
    rng = np.random.default_rng(8)
    L = rng.integers(-3, 4, (40, 7)).astype(np.float32) * 0.5  # many ties
    ids, w = R.route_topk(L, 3)
    for t in range(L.shape[0]):
        order, ww = bf_route(L[t], 3)
        assert ids[t].tolist() == order
        assert np.allclose(w[t], ww, rtol=1e-6, atol=0)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) < 1e-6


def pin_gather_bruteforce():
    rng = np.random.default_rng(9)
    n, k, E = 13, 3, 5
    ids = np.stack([rng.permutation(E)[:k] for _ in range(n)]).astype(np.int32)
    counts, offsets, pairs, slot_row = R.gather(ids, E)
    flat = ids.reshape(-1).tolist()
    want_pairs = [p for _, p in sorted((e, p) for p, e in enumerate(flat))]
    assert pairs.tolist() == want_pairs
    assert counts.tolist() == [flat.count(e) for e in range(E)]
    assert offsets.tolist() == [sum(flat.count(x) for x in range(e)) for e in range(E + 1)]
    assert all(pairs[slot_row[p]] == p for p in range(n * k))
    for e in range(E):
        seg = pairs[offsets[e]:offsets[e + 1]].tolist()
        assert all(flat[p] == e for p in seg) and seg == sorted(seg)


# ----------------------------------------------------------------------------------
# pins: SwiGLU and the MoE combine


def pin_silu():
    g = np.array([-30.0, -2.5, -1.0, -0.25, 0.0, 0.25, 1.0, 2.5, 30.0])
    s = R.silu(g)
    assert s[4] == 0.0
    # silu(x) - silu(-x) = x exactly in real arithmetic
    assert np.allclose(s - R.silu(-g), g, rtol=0, atol=1e-14)
    # silu(ln 3) = (3/4) ln 3
    assert abs(R.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(s[-1] - 30.0) < 1e-11 and abs(s[0]) < 1e-11


def tiny_moe(seed=10, n=5, k=2, E=4, H=64, I=32, x_dtype=np.float32):
    rng = np.random.default_rng(seed)
    gate = [rand_blocks(rng, I * H // 32, 0.1) for _ in range(E)]
    up = [rand_blocks(rng, I * H // 32, 0.1) for _ in range(E)]
    down = [rand_blocks(rng, H * I // 32, 0.1) for _ in range(E)]
    x = rng.standard_normal((n, H)).astype(x_dtype)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(n)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), n).astype(np.float32)
    return x, ids, w, gate, up, down, H, I


def pin_moe_single_expert_is_dense_ffn():
    """k = 1, w = 1: the MoE output is the dense FFN of the routed expert, composed
    here from the (separately pinned) qmv oracle and an explicit SwiGLU."""
    x, ids, w, gate, up, down, H, I = tiny_moe(k=1)
    w = np.ones_like(w)
    out = R.moe(x, ids, w, gate, up, down, H, I)
    for t in range(x.shape[0]):
        e = ids[t, 0]
        g = R.qmv(gate[e], I, H, x[t:t + 1]).astype(np.float64)
        u = R.qmv(up[e], I, H, x[t:t + 1]).astype(np.float64)
        h = g / (1 + np.exp(-g)) * u
        y = R.qmv(down[e], H, I, h.astype(np.float32))
        assert np.allclose(out[t], y[0], rtol=1e-5, atol=1e-6 * np.abs(y).max())


def pin_moe_weight_summed_dense():
    """The MoE output equals the weight-summed dense products of all experts, where
    an expert a token was not routed to carries weight zero (computed densely, every
    token through every expert, in exact rationals except for the exponential)."""
    x, ids, w, gate, up, down, H, I = tiny_moe(n=3, E=3, H=32, I=32)
    out = R.moe(x, ids, w, gate, up, down, H, I)
    Wg = [bf_matrix(gate[e], I, H) for e in range(3)]
    Wu = [bf_matrix(up[e], I, H) for e in range(3)]
    Wd = [bf_matrix(down[e], H, I) for e in range(3)]
    for t in range(x.shape[0]):
        xt = [Fraction(float(v)) for v in x[t]]
        acc = [Fraction(0)] * H
        for e in range(3):
            weight = Fraction(0)
            for j in range(ids.shape[1]):
                if ids[t, j] == e:
                    weight = Fraction(float(w[t, j]))
            g = [sum(Wg[e][i][c] * xt[c] for c in range(H)) for i in range(I)]
            u = [sum(Wu[e][i][c] * xt[c] for c in range(H)) for i in range(I)]
            h = [Fraction(float(gi) / (1 + math.exp(-float(gi)))) * ui for gi, ui in zip(g, u)]
            y = [sum(Wd[e][r][i] * h[i] for i in range(I)) for r in range(H)]
            acc = [a + weight * v for a, v in zip(acc, y)]
        ref = np.array([float(v) for v in acc])
        assert np.allclose(out[t], ref, rtol=1e-6, atol=1e-9 * np.abs(ref).max())


def pin_moe_gate_up_bruteforce():
    """The kept first products: with power-of-two scales and small-integer activations
    every product and sum is exact, so each g and u must equal the exact rational
    product of the routed expert's closed-form decoded matrix with the token's row."""
    rng = np.random.default_rng(23)
    n, k, E, H, I = 4, 2, 3, 64, 32
    gate = [integer_exact_blocks(rng, I * H // 32, 5) for _ in range(E)]
    up = [integer_exact_blocks(rng, I * H // 32, 4) for _ in range(E)]
    x = rng.integers(-8, 9, (n, H)).astype(np.float16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(n)]).astype(np.int32)
    g, u = R.moe_gate_up(x, ids, gate, up, H, I)
    assert g.shape == u.shape == (n * k, I)
    Wg = [bf_matrix(gate[e], I, H) for e in range(E)]
    Wu = [bf_matrix(up[e], I, H) for e in range(E)]
    for t in range(n):
        for j in range(k):
            e, p = ids[t, j], t * k + j
            for i in range(I):
                assert Fraction(float(g[p, i])) == sum(Wg[e][i][c] * int(x[t, c]) for c in range(H))
                assert Fraction(float(u[p, i])) == sum(Wu[e][i][c] * int(x[t, c]) for c in range(H))


def pin_moe_gate_up_composes_to_moe():
    """silu(g) * u through each pair's down matrix, weighted and summed over the slots,
    is the (separately pinned) MoE output."""
    x, ids, w, gate, up, down, H, I = tiny_moe(seed=24)
    g, u = R.moe_gate_up(x, ids, gate, up, H, I)
    h = R.silu(g) * u
    n, k = ids.shape
    out = np.zeros((n, H))
    for t in range(n):
        for j in range(k):
            e, p = ids[t, j], t * k + j
            out[t] += float(w[t, j]) * (R._matrix(down[e], H, I) @ h[p])
    ref = R.moe(x, ids, w, gate, up, down, H, I)
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())


def pin_moe_shared_bruteforce():
    """moe_shared = the routed sum plus the shared expert's SwiGLU FFN with weight 1,
    recomputed in exact rationals (except for the exponential) from the closed-form
    decoded matrices."""
    x, ids, w, gate, up, down, H, I = tiny_moe(seed=21, n=2, E=3, H=32, I=32)
    rng = np.random.default_rng(22)
    sg, su, sd = (rand_blocks(rng, I * H // 32, 0.1), rand_blocks(rng, I * H // 32, 0.1),
                  rand_blocks(rng, H * I // 32, 0.1))
    out = R.moe_shared(x, ids, w, gate, up, down, sg, su, sd, H, I)
    mats = [(bf_matrix(gate[e], I, H), bf_matrix(up[e], I, H), bf_matrix(down[e], H, I)) for e in range(3)]
    shared = (bf_matrix(sg, I, H), bf_matrix(su, I, H), bf_matrix(sd, H, I))

    def ffn(m, xt):
        Wg, Wu, Wd = m
        g = [sum(Wg[i][c] * xt[c] for c in range(H)) for i in range(I)]
        u = [sum(Wu[i][c] * xt[c] for c in range(H)) for i in range(I)]
        h = [Fraction(float(gi) / (1 + math.exp(-float(gi)))) * ui for gi, ui in zip(g, u)]
        return [sum(Wd[r][i] * h[i] for i in range(I)) for r in range(H)]

    for t in range(x.shape[0]):
        xt = [Fraction(float(v)) for v in x[t]]
        acc = ffn(shared, xt)
        for j in range(ids.shape[1]):
            y = ffn(mats[ids[t, j]], xt)
            acc = [a + Fraction(float(w[t, j])) * v for a, v in zip(acc, y)]
        ref = np.array([float(v) for v in acc])
        assert np.allclose(out[t], ref, rtol=1e-6, atol=1e-9 * np.abs(ref).max())


def pin_moe_shared_is_an_always_on_expert():
    """The shared expert is a routed expert that every token takes with weight 1: the
    (separately pinned) routed oracle on the bank extended by it, with it appended to
    every token's routing, gives the same result."""
    x, ids, w, gate, up, down, H, I = tiny_moe(seed=23, n=4, k=2, E=4)
    rng = np.random.default_rng(24)
    sg, su, sd = (rand_blocks(rng, I * H // 32, 0.1), rand_blocks(rng, I * H // 32, 0.1),
                  rand_blocks(rng, H * I // 32, 0.1))
    out = R.moe_shared(x, ids, w, gate, up, down, sg, su, sd, H, I, tokens=[3, 0, 2])
    ids2 = np.concatenate([ids, np.full((ids.shape[0], 1), 4, np.int32)], axis=1)
    w2 = np.concatenate([w, np.ones((w.shape[0], 1), np.float32)], axis=1)
    ref = R.moe(x, ids2, w2, gate + [sg], up + [su], down + [sd], H, I, tokens=[3, 0, 2])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def pin_moe_subset_rows():
    x, ids, w, gate, up, down, H, I = tiny_moe(n=6)
    full = R.moe(x, ids, w, gate, up, down, H, I)
    sub = R.moe(x, ids, w, gate, up, down, H, I, tokens=[4, 1])
    assert np.array_equal(sub, full[[4, 1]])


# ----------------------------------------------------------------------------------
# pins: 8-bit activations (quantize_q8_1, qmv_q8)


def bf_quantize_q8_block(xs):
    """Quantise 32 float32 values by hand: exact rationals, each IEEE step rounded
    explicitly (binary32 division, reciprocal and product; binary16 scale)."""
    xf = [Fraction(float(v)) for v in xs]
    a = max(abs(v) for v in xf)
    d32 = f32(a / 127)
    d16 = f16(Fraction(d32))
    if d16 == 0:
        return [0] * 32, d16
    r = f32(1 / Fraction(d32))
    q = []
    for v in xf:
        p = Fraction(f32(v * Fraction(r)))
        n = (abs(p) + Fraction(1, 2)).__floor__()  # halves away from zero
        n = min(n, 127)
        q.append(int(n if p >= 0 else -n))
    return q, d16


def q8_special_blocks():
    blocks = [np.zeros(32, np.float32)]
    # absmax 127: d = r = 1, so every value below is its own product; halves go away
    # from zero
    ties = [127.0, -127.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5, 0.49999997, -0.49999997]
    blocks.append(np.array(ties + [0.0] * (32 - len(ties)), np.float32))
    blocks.append(np.full(32, 3.0e-6, np.float32))        # stored scale rounds to zero
    blocks.append(np.linspace(-1e-3, 2e-3, 32, dtype=np.float32))
    blocks.append(np.linspace(-6e4, 5e4, 32, dtype=np.float32))
    return blocks


def pin_q8_quantize_bruteforce():
    rng = np.random.default_rng(7)
    xs = [rng.standard_normal(32).astype(np.float32) * s for s in (1.0, 1e-3, 300.0)]
    xs += [rng.standard_normal(32).astype(np.float32) for _ in range(20)]
    xs += q8_special_blocks()
    x = np.stack(xs).reshape(1, -1)
    q, d = R.quantize_q8_1(x)
    for b, xb in enumerate(xs):
        wq, wd = bf_quantize_q8_block(xb)
        assert list(q[0, 32 * b:32 * b + 32]) == wq, b
        assert f16_bits(float(d[0, b])) == f16_bits(wd), b


def pin_q8_quantize_ties():
    x = q8_special_blocks()[1].reshape(1, 32)
    q, d = R.quantize_q8_1(x)
    assert float(d[0, 0]) == 1.0
    want = [127, -127, 1, -1, 2, -2, 3, -3, 127, -127, 0, 0] + [0] * 20
    assert list(q[0]) == want


def pin_qmv_q8_fraction():
    rng = np.random.default_rng(8)
    n, k, T = 3, 64, 2
    blocks = rand_blocks(rng, n * k // 32)
    x = rng.standard_normal((T, k)).astype(np.float32)
    q, d = R.quantize_q8_1(x)
    y = R.qmv_q8(blocks, n, k, q, d)
    W = bf_matrix(blocks, n, k)
    for t in range(T):
        xh = [Fraction(float(d[t, c // 32])) * int(q[t, c]) for c in range(k)]
        for r in range(n):
            assert_f32_close_to_exact(y[t, r], sum(W[r][c] * xh[c] for c in range(k)))


def pin_qmv_q8_on_grid_equals_fp32():
    # activations already on the 8-bit grid of their blocks (integers, each block's
    # absmax 127, so d = r = 1): the 8-bit product equals the float product
    rng = np.random.default_rng(9)
    n, k, T = 8, 256, 3
    blocks = rand_blocks(rng, n * k // 32)
    x = rng.integers(-127, 128, (T, k)).astype(np.float32)
    x[:, ::32] = 127.0
    q, d = R.quantize_q8_1(x)
    assert np.all(d == 1.0) and np.array_equal(q.astype(np.float32), x)
    assert np.array_equal(R.qmv_q8(blocks, n, k, q, d), R.qmv(blocks, n, k, x))


PINS = [
    pin_codebook, pin_block_size, pin_decode_golden, pin_decode_closed_form, pin_decode_f16,
    pin_encode_golden, pin_encode_bruteforce, pin_encode_idempotent, pin_encode_zero,
    pin_qmv_one_hot, pin_qmv_fraction, pin_qmv_integer_exact, pin_gemm_fraction,
    pin_gemm_integer_exact, pin_route_golden, pin_route_bruteforce, pin_gather_bruteforce,
    pin_silu, pin_moe_single_expert_is_dense_ffn, pin_moe_weight_summed_dense, pin_moe_subset_rows,
    pin_moe_shared_bruteforce, pin_moe_shared_is_an_always_on_expert,
    pin_moe_gate_up_bruteforce, pin_moe_gate_up_composes_to_moe,
    pin_q8_quantize_bruteforce, pin_q8_quantize_ties, pin_qmv_q8_fraction, pin_qmv_q8_on_grid_equals_fp32,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail


def _fails(pins):
    failed = []
    for p in pins:
        try:
            with np.errstate(all="ignore"):
                p()
        except Exception:  # an assertion, or a crash on nonsense values
            failed.append(p.__name__)
    return failed


def _swap_halves(blocks):
    qs = blocks[:, 2:18].astype(np.int64)
    q = np.empty((blocks.shape[0], 32), dtype=np.int64)
    q[:, :16] = qs >> 4
    q[:, 16:] = qs & 0xF
    return q


def _interleaved(blocks):
    qs = blocks[:, 2:18].astype(np.int64)
    q = np.empty((blocks.shape[0], 32), dtype=np.int64)
    q[:, 0::2] = qs & 0xF
    q[:, 1::2] = qs >> 4
    return q


def _qmv_transposed(blocks, n, k, x):
    # reads the block rows as the K x N orientation of the matrix
    W = R.decode_blocks(blocks).astype(np.float64).reshape(k, n)
    X = np.asarray(x, dtype=np.float64).reshape(-1, k)
    return (X @ W).astype(np.float32)


def _route_ties_high(logits, top_k):
    L = np.asarray(logits, dtype=np.float32)
    ids = np.empty((L.shape[0], top_k), dtype=np.int32)
    w = np.empty((L.shape[0], top_k), dtype=np.float32)
    for t in range(L.shape[0]):
        order = (L.shape[1] - 1 - np.argsort(-L[t, ::-1].astype(np.float64), kind="stable"))[:top_k]
        ids[t] = order
        z = L[t, order].astype(np.float64)
        e = np.exp(z - z.max())
        w[t] = e / e.sum()
    return ids, w


def _silu_wrong_sign(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(g))


def _encode_round_half_up(w):
    out = _orig_encode(w)
    w32 = np.asarray(w, dtype=np.float32).reshape(-1, 32)
    # re-pick ties toward the higher level
    d = out[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)
    cb = np.asarray(R.CODEBOOK, dtype=np.float64)
    dist = np.abs(w32.astype(np.float64)[:, :, None] - d[:, None, None] * cb)
    q = 15 - np.argmin(dist[:, :, ::-1], axis=2)
    q[d == 0, :] = 8
    out[:, 2:18] = (q[:, :16] | (q[:, 16:] << 4)).astype(np.uint8)
    return out


_orig_encode = R.encode_blocks
_orig_moe = R.moe


def _moe_drop_weight(x, ids, w, *a, **kw):
    return _orig_moe(x, ids, np.ones_like(np.asarray(w)), *a, **kw)


_orig_quantize_q8 = R.quantize_q8_1
_orig_qmv_q8 = R.qmv_q8


def _q8_ties_to_even(x):
    X = np.asarray(x, dtype=np.float32).reshape(np.asarray(x).shape[0], -1)
    q, d = _orig_quantize_q8(X)
    B = X.reshape(X.shape[0], -1, 32)
    d32 = np.max(np.abs(B), axis=2) / np.float32(127)
    with np.errstate(divide="ignore"):
        r = np.where(d != 0, np.float32(1) / d32, np.float32(0)).astype(np.float32)
    v = (B * r[:, :, None]).astype(np.float32)
    return np.clip(np.rint(v), -127, 127).astype(np.int8).reshape(X.shape), d


def _q8_reciprocal_of_stored_scale(x):
    X = np.asarray(x, dtype=np.float32).reshape(np.asarray(x).shape[0], -1)
    q, d = _orig_quantize_q8(X)
    B = X.reshape(X.shape[0], -1, 32)
    with np.errstate(divide="ignore"):
        r = np.where(d != 0, np.float32(1) / d.astype(np.float32), np.float32(0)).astype(np.float32)
    v = (B * r[:, :, None]).astype(np.float32)
    return np.clip(R._round_half_away(v), -127, 127).astype(np.int8).reshape(X.shape), d


def _qmv_q8_no_act_scale(blocks, n, k, q, d):
    return _orig_qmv_q8(blocks, n, k, q, np.ones_like(np.asarray(d)))


_orig_moe_shared = R.moe_shared


def _moe_shared_dropped(x, ids, w, gate, up, down, sg, su, sd, H, I, tokens=None):
    return R.moe(x, ids, w, gate, up, down, H, I, tokens=tokens)


def _moe_shared_gate_up_swapped(x, ids, w, gate, up, down, sg, su, sd, H, I, tokens=None):
    return _orig_moe_shared(x, ids, w, gate, up, down, su, sg, sd, H, I, tokens=tokens)


_orig_moe_gate_up = R.moe_gate_up


def _moe_gate_up_swapped(x, ids, gate, up, H, I):
    g, u = _orig_moe_gate_up(x, ids, gate, up, H, I)
    return u, g


def _moe_gate_up_sorted_rows(x, ids, gate, up, H, I):
    g, u = _orig_moe_gate_up(x, ids, gate, up, H, I)
    order = np.argsort(np.asarray(ids).reshape(-1), kind="stable")  # pair-sorted, not pair-id order
    return g[order], u[order]


PLANTED = {
    "codebook sign": ("CODEBOOK", tuple(-c for c in R.CODEBOOK)),
    "codebook off by one": ("CODEBOOK", tuple(R.CODEBOOK[1:]) + (127,)),
    "nibble halves swapped": ("_indices", _swap_halves),
    "nibbles interleaved": ("_indices", _interleaved),
    "scale big-endian": ("_scales", lambda b: b[:, 0:2].copy().view(">f2").astype(np.float64).reshape(-1)),
    "qmv transposed output": ("qmv", _qmv_transposed),
    "route ties to higher id": ("route_topk", _route_ties_high),
    "silu sign": ("silu", _silu_wrong_sign),
    "encode ties upward": ("encode_blocks", _encode_round_half_up),
    "moe drops gate weight": ("moe", _moe_drop_weight),
    "q8 ties to even": ("quantize_q8_1", _q8_ties_to_even),
    "q8 reciprocal of the stored scale": ("quantize_q8_1", _q8_reciprocal_of_stored_scale),
    "q8 product drops the activation scale": ("qmv_q8", _qmv_q8_no_act_scale),
    "shared expert dropped": ("moe_shared", _moe_shared_dropped),
    "shared expert gate and up swapped": ("moe_shared", _moe_shared_gate_up_swapped),
    "kept products gate and up swapped": ("moe_gate_up", _moe_gate_up_swapped),
    "kept products in sorted order": ("moe_gate_up", _moe_gate_up_sorted_rows),
}


@pytest.mark.parametrize("name", list(PLANTED))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, value = PLANTED[name]
    monkeypatch.setattr(R, attr, value)
    assert _fails(PINS), f"no pin caught the planted mistake: {name}"
