"""T-column quantised matvec on the GPU against the oracle.

Tolerance: fp32 activations and accumulation, normwise max|y - r| / max|r| <= 1e-3
(the stated tolerance for the fp32 paths).  Exact cases (one-hot columns, power-of-two
scales with small-integer activations) must match bitwise, and every column of a
T-column call must equal the 1-column call on that column bitwise (page 1, verify.hpp
header: each window token reproduces single-token decode bit for bit).
"""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
from gpu_util import bits_equal, dev, host, normwise, note, pack, qmv_workspace
from test_oracle_pins import integer_exact_blocks
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-3


def run_qmv(packed, n, k, x: np.ndarray, ldx=None, ldy=None) -> np.ndarray:
    T = x.shape[0]
    ldx = ldx or k
    ldy = ldy or n
    xb = np.zeros((T, ldx), dtype=np.float32)
    xb[:, :k] = x
    xd = dev(xb)
    y = torch.full((T, ldy), float("nan"), dtype=torch.float32, device="cuda")
    ws, wsb = qmv_workspace(n, k)
    iq4.iq4_qmv_multi(packed, n, k, xd, ldx, T, y, ldy, ws, wsb)
    out = host(y)
    if ldy > n:
        assert np.all(np.isnan(out[:, n:])), "wrote outside [0, n)"
    return out[:, :n]


def test_plumbing_matvec():
    note("qmv: plumbing 512 x 2048, T = 1")
    b, n, k, x = workloads.cfg1()
    y = run_qmv(pack(b, n, k), n, k, x)
    r = oracle.qmv(b, n, k, x)
    assert normwise(y, r) <= TOL


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8])
def test_verify_window_matvec(T):
    note(f"qmv: verify window 4096 x 4096, T = {T}")
    b, n, k, x = workloads.cfg2(T)
    y = run_qmv(pack(b, n, k), n, k, x)
    r = oracle.qmv(b, n, k, x)
    err = normwise(y, r)
    assert err <= TOL, err
    # also every column on its own scale
    for t in range(T):
        assert normwise(y[t], r[t]) <= TOL


def test_columns_equal_single_column_bitwise():
    note("qmv: T-column vs 1-column bitwise, T = 1..8")
    b, n, k, x8 = workloads.cfg2(8)
    packed = pack(b, n, k)
    single = [run_qmv(packed, n, k, x8[t:t + 1]) for t in range(8)]
    for T in range(1, 9):
        y = run_qmv(packed, n, k, x8[:T])
        for t in range(T):
            assert bits_equal(y[t], single[t][0]), (T, t)


def test_column_position_does_not_matter():
    note("qmv: the same column in every slot of an 8-column call")
    b, n, k, x8 = workloads.cfg2(8)
    packed = pack(b, n, k)
    one = run_qmv(packed, n, k, x8[3:4])[0]
    rep = run_qmv(packed, n, k, np.repeat(x8[3:4], 8, axis=0))
    for t in range(8):
        assert bits_equal(rep[t], one)


def test_one_hot_columns_exact():
    note("qmv: one-hot columns read back the decoded matrix exactly")
    b, n, k, _ = workloads.cfg2(1)
    packed = pack(b, n, k)
    W = oracle.decode_blocks(b).reshape(n, k)
    cols = [0, 1, 15, 16, 17, 31, 32, 127, 128, 2047, 4095]
    for i in range(0, len(cols), 8):
        cs = cols[i:i + 8]
        x = np.zeros((len(cs), k), dtype=np.float32)
        for t, c in enumerate(cs):
            x[t, c] = 1.0
        y = run_qmv(packed, n, k, x)
        for t, c in enumerate(cs):
            assert bits_equal(y[t], W[:, c]), c


@pytest.mark.parametrize("n,k,T", [(16, 128, 1), (48, 384, 3), (64, 768, 5), (32, 1152, 8), (160, 2048, 2)])
def test_integer_exact_bitwise(n, k, T):
    """Power-of-two scales and integer activations: every partial sum is exact, so the
    GPU must equal the oracle bitwise whatever its summation order."""
    note(f"qmv: integer-exact n={n} k={k} T={T}")
    rng = np.random.default_rng(n * 7 + k + T)
    b = integer_exact_blocks(rng, n * k // 32, 6)
    x = rng.integers(-8, 9, (T, k)).astype(np.float32)
    y = run_qmv(pack(b, n, k), n, k, x)
    assert bits_equal(y, oracle.qmv(b, n, k, x))


@pytest.mark.parametrize("n,k,T", [(16, 128, 1), (48, 384, 4), (64, 768, 2), (32, 1152, 7), (256, 14336, 3)])
def test_ragged_shapes(n, k, T):
    """Tile-edge shapes: one tile, uneven K split over the waves, a long K."""
    note(f"qmv: ragged n={n} k={k} T={T}")
    rng = np.random.default_rng(n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    b = oracle.encode_blocks(w.reshape(-1, 32))
    x = rng.standard_normal((T, k)).astype(np.float32)
    y = run_qmv(pack(b, n, k), n, k, x, ldx=k + 4 * (T % 3), ldy=n + 16 * (T % 2))
    assert normwise(y, oracle.qmv(b, n, k, x)) <= TOL


def test_wide_dynamic_range_activations():
    """Activations spanning many binades: the two bf16 parts of each activation carry it
    to within 2^-18 of its magnitude, so the result is well inside 1e-5 normwise."""
    note("qmv: wide dynamic range")
    rng = np.random.default_rng(5)
    n, k = 64, 1024
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = (rng.standard_normal((4, k)) * 2.0 ** rng.integers(-60, 60, (4, k))).astype(np.float32)
    y = run_qmv(pack(b, n, k), n, k, x)
    r = oracle.qmv(b, n, k, x)
    assert normwise(y, r) <= 1e-5


def test_deterministic():
    note("qmv: run-to-run determinism")
    b, n, k, x = workloads.cfg2(4)
    packed = pack(b, n, k)
    assert bits_equal(run_qmv(packed, n, k, x), run_qmv(packed, n, k, x))


def test_split_k_workspace_is_reusable():
    """A shape whose K is split over workgroups leaves its workspace ready: back-to-back
    calls (different T) through one workspace match fresh ones bitwise, and the result
    matches the oracle."""
    note("qmv: split-K workspace reuse across calls")
    n, k = 256, 14336
    assert iq4.iq4_qmv_workspace_size(n, k) > 0
    rng = np.random.default_rng(9)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((4, k)).astype(np.float32)
    packed = pack(b, n, k)
    first = [run_qmv(packed, n, k, x[:T]) for T in (1, 4, 2, 3)]
    again = [run_qmv(packed, n, k, x[:T]) for T in (1, 4, 2, 3)]
    for a_, b_ in zip(first, again):
        assert bits_equal(a_, b_)
    assert normwise(first[1], oracle.qmv(b, n, k, x)) <= TOL
    for t in range(4):
        assert bits_equal(first[1][t], first[0][0] if t == 0 else run_qmv(packed, n, k, x[t:t + 1])[0])


def test_split_k_two_passes():
    """T = 5..8 on a split-K shape: the second pass of 4 columns has partial slots and an
    arrival counter of its own, so no slice of one pass can overwrite what the other
    pass's last arriver reads.  Every column is bitwise its 1-column run and within the
    tolerance of the oracle, and repeated calls through one workspace agree bitwise."""
    note("qmv: split-K, two passes (T = 5..8), n=256 k=14336")
    n, k = 256, 14336
    rng = np.random.default_rng(11)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((8, k)).astype(np.float32)
    packed = pack(b, n, k)
    single = [run_qmv(packed, n, k, x[t:t + 1])[0] for t in range(8)]
    r = oracle.qmv(b, n, k, x)
    for T in (5, 6, 7, 8, 8, 5):
        y = run_qmv(packed, n, k, x[:T])
        assert normwise(y, r[:T]) <= TOL, T
        for t in range(T):
            assert bits_equal(y[t], single[t]), (T, t)
    # the workspace is left ready: a 1-column call after them still matches
    assert bits_equal(run_qmv(packed, n, k, x[2:3])[0], single[2])


@pytest.mark.parametrize("n,k,T", [(16, 128, 1), (48, 384, 3), (32, 640, 4), (64, 896, 2)])
def test_short_k_after_other_kernels(n, k, T):
    """K of 1 to 7 quads runs a workgroup of fewer than 8 waves, which must build the
    whole level table itself.  Before each call another kernel (the 8-bit matvec, the
    IQ4_XS decode) leaves different contents in LDS, so a table built only in part would
    read their leftovers and show here (right after a full-size float matvec the
    leftovers happen to be a complete table)."""
    note(f"qmv: short K after other kernels n={n} k={k} T={T}")
    rng = np.random.default_rng(3 * n + k)
    b = integer_exact_blocks(rng, n * k // 32, 6)
    x = rng.integers(-8, 9, (T, k)).astype(np.float32)
    packed = pack(b, n, k)
    ref = oracle.qmv(b, n, k, x)
    # other kernels first: the 8-bit matvec of the same shape, an IQ4_XS decode
    xq = rng.integers(-127, 128, (T, k)).astype(np.float32)
    q = torch.from_numpy(xq.astype(np.int8)).cuda()
    d = torch.ones((T, k // 32), dtype=torch.float16, device="cuda")
    yq = torch.empty((T, n), dtype=torch.float32, device="cuda")
    ws, wsb = qmv_workspace(n, k)
    for rep in range(3):
        iq4.iq4_qmv_q8(packed, n, k, q, d.view(torch.int16), T, yq, n, ws, wsb)
        sb = dev(rng.integers(0, 256, (64, 136), dtype=np.uint8).reshape(-1))
        out = torch.empty(64 * 256, dtype=torch.float32, device="cuda")
        iq4.iq4_xs_dequant(sb, 64, iq4.IQ4_F32, out)
        assert bits_equal(run_qmv(packed, n, k, x), ref), rep
