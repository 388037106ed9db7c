"""8-bit-activation matvec and activation quantisation on the GPU against the oracle.

The quantised activations (codes and binary16 scales) are integer decisions and must
match the oracle bit for bit.  The product's block dots are exact integers on the GPU
too, so the only freedom is the fp32 accumulation of the scaled block dots: normwise
max|y - r| / max|r| <= 1e-3 (the stated tolerance for the fp32 paths).  Exact cases
(power-of-two weight scales, activations already on their 8-bit grid) must match
bitwise, and every column of a T-column call must equal the 1-column call bitwise.
"""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
from gpu_util import bits_equal, dev, host, normwise, note, pack, qmv_workspace
from test_gpu_qmv import run_qmv
from test_oracle_pins import integer_exact_blocks, q8_special_blocks
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-3


def run_quantize(x: np.ndarray, ldx=None):
    T, k = x.shape
    ldx = ldx or k
    xb = np.zeros((T, ldx), dtype=np.float32)
    xb[:, :k] = x
    q = torch.full((T, k), 99, dtype=torch.int8, device="cuda")
    d = torch.full((T, k // 32), 0x7E00, dtype=torch.int16, device="cuda")
    iq4.iq4_quantize_q8_1(dev(xb), T, k, ldx, q, d)
    return host(q), host(d).view(np.float16)


def run_q8(packed, n, k, q: np.ndarray, d: np.ndarray, ldy=None) -> np.ndarray:
    T = q.shape[0]
    ldy = ldy or n
    y = torch.full((T, ldy), float("nan"), dtype=torch.float32, device="cuda")
    ws, wsb = qmv_workspace(n, k)
    iq4.iq4_qmv_q8(packed, n, k, dev(np.ascontiguousarray(q)), dev(np.ascontiguousarray(d).view(np.int16)), T, y,
                   ldy, ws, wsb)
    out = host(y)
    if ldy > n:
        assert np.all(np.isnan(out[:, n:])), "wrote outside [0, n)"
    return out[:, :n]


def test_quantize_bit_exact():
    note("q8: quantize verify-window activations (8 x 4096) and edge blocks")
    _, _, k, x = workloads.cfg2(8)
    q, d = run_quantize(x)
    rq, rd = oracle.quantize_q8_1(x)
    assert np.array_equal(q, rq) and bits_equal(d, rd)
    rng = np.random.default_rng(11)
    edge = q8_special_blocks() + [rng.standard_normal(32).astype(np.float32) * s for s in (1e-5, 1e-2, 7.0, 3e3, 0.5)]
    assert len(edge) % 2 == 0
    xe = np.stack(edge).reshape(2, -1)
    q, d = run_quantize(xe, ldx=xe.shape[1] + 12)
    rq, rd = oracle.quantize_q8_1(xe)
    assert np.array_equal(q, rq) and bits_equal(d, rd)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8])
def test_q8_verify_window(T):
    note(f"q8: verify window 4096 x 4096, T = {T}")
    b, n, k, x = workloads.cfg2(T)
    q, d = oracle.quantize_q8_1(x)
    y = run_q8(pack(b, n, k), n, k, q, d)
    r = oracle.qmv_q8(b, n, k, q, d)
    assert normwise(y, r) <= TOL
    for t in range(T):
        assert normwise(y[t], r[t]) <= TOL


def test_q8_columns_equal_single_column_bitwise():
    note("q8: T-column vs 1-column bitwise, T = 1..8")
    b, n, k, x8 = workloads.cfg2(8)
    packed = pack(b, n, k)
    q8, d8 = oracle.quantize_q8_1(x8)
    single = [run_q8(packed, n, k, q8[t:t + 1], d8[t:t + 1]) for t in range(8)]
    for T in range(1, 9):
        y = run_q8(packed, n, k, q8[:T], d8[:T])
        for t in range(T):
            assert bits_equal(y[t], single[t][0]), (T, t)


@pytest.mark.parametrize("n,k,T", [(16, 128, 1), (48, 384, 3), (64, 768, 5), (32, 1152, 8), (160, 2048, 2)])
def test_q8_on_grid_integer_exact_bitwise(n, k, T):
    """Power-of-two weight scales and integer activations with block absmax 127 (so the
    activation scale is 1): every partial sum is exact, and the 8-bit product equals the
    oracle's and the float matvec's bitwise."""
    note(f"q8: on-grid integer-exact n={n} k={k} T={T}")
    rng = np.random.default_rng(n * 5 + k + T)
    b = integer_exact_blocks(rng, n * k // 32, 6)
    x = rng.integers(-127, 128, (T, k)).astype(np.float32)
    x[:, ::32] = -127.0
    q, d = run_quantize(x)
    assert np.all(d == 1.0) and np.array_equal(q.astype(np.float32), x)
    packed = pack(b, n, k)
    y = run_q8(packed, n, k, q, d)
    assert bits_equal(y, oracle.qmv_q8(b, n, k, q, d))
    assert bits_equal(y, run_qmv(packed, n, k, x))


@pytest.mark.parametrize("n,k,T", [(16, 128, 8), (48, 384, 4), (64, 768, 2), (32, 1152, 7), (256, 14336, 3),
                                   (256, 14336, 8)])
def test_q8_ragged_shapes(n, k, T):
    note(f"q8: ragged n={n} k={k} T={T}")
    rng = np.random.default_rng(n + 3 * k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    b = oracle.encode_blocks(w.reshape(-1, 32))
    x = rng.standard_normal((T, k)).astype(np.float32)
    q, d = run_quantize(x)
    y = run_q8(pack(b, n, k), n, k, q, d, ldy=n + 16 * (T % 2))
    assert normwise(y, oracle.qmv_q8(b, n, k, q, d)) <= TOL


def test_q8_and_float_share_a_split_k_workspace():
    """Both matvecs on one split-K workspace, interleaved: each call leaves the shared
    arrival counters at zero, so every result equals its first run bitwise."""
    note("q8: shared split-K workspace with the float matvec")
    n, k = 256, 14336
    rng = np.random.default_rng(12)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((4, k)).astype(np.float32)
    q, d = oracle.quantize_q8_1(x)
    packed = pack(b, n, k)
    f1, q1 = run_qmv(packed, n, k, x), run_q8(packed, n, k, q, d)
    f2, q2 = run_qmv(packed, n, k, x), run_q8(packed, n, k, q, d)
    assert bits_equal(f1, f2) and bits_equal(q1, q2)
    assert normwise(q1, oracle.qmv_q8(b, n, k, q, d)) <= TOL
