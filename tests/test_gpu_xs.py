"""IQ4_XS super-blocks on the GPU vs the oracle: decode (bitwise) and the T-column
matvec (normwise <= 1e-3, the stated tolerance of the fp32 decode paths; bitwise where
every product and partial sum is exact; each column bitwise equal to its T = 1 call).

Shapes: page 2's cold/hot table times the format's matvec on 2560 x 6144 and
6144 x 2560 (read as N x K); 4096 x 4096 as the verify-window size; small and ragged
shapes (one super-block per row, row counts that leave a partial workgroup, K past one
pass of the workgroup's lanes)."""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
import synth
import workloads
from gpu_util import bits_equal, dev, host, normwise, note

pytestmark = pytest.mark.gpu

TOL = 1e-3


def gpu_xs_decode(sb: np.ndarray, f16: bool, guard: int = 64) -> np.ndarray:
    nsb = sb.shape[0]
    dt = torch.float16 if f16 else torch.float32
    out = torch.full((nsb * 256 + guard,), float("nan"), dtype=dt, device="cuda")
    iq4.iq4_xs_dequant(dev(sb.reshape(-1)), nsb, iq4.IQ4_F16 if f16 else iq4.IQ4_F32, out)
    got = host(out)
    assert np.all(np.isnan(got[nsb * 256:])), "wrote past the output"
    return got[:nsb * 256].reshape(nsb, 256)


def same_with_nan(got, ref, dtype):
    """Bitwise equal, NaN positions compared as positions; prints the first mismatches."""
    nan = np.isnan(ref)
    ok = np.array_equal(nan, np.isnan(got)) and bits_equal(np.where(nan, 0, got).astype(dtype),
                                                           np.where(nan, 0, ref).astype(dtype))
    if not ok:
        g, r = np.asarray(got, dtype), np.asarray(ref, dtype)
        ui = np.uint16 if dtype == np.float16 else np.uint32
        bad = np.argwhere((g.view(ui) != r.view(ui)) & ~(np.isnan(g) & np.isnan(r)))
        for idx in bad[:8]:
            idx = tuple(idx)
            note(f"  mismatch at {idx}: got {g[idx]!r} ({int(g.view(ui)[idx]):#x}) "
                 f"want {r[idx]!r} ({int(r.view(ui)[idx]):#x})")
        note(f"  {len(bad)} mismatches")
    return ok


def random_superblocks(rng, nsb: int) -> np.ndarray:
    """Every byte uniform (all 64 codes, all indices), with finite scales of the
    workload's magnitude."""
    sb = rng.integers(0, 256, (nsb, 136), dtype=np.uint8)
    d = (rng.standard_normal(nsb) * 2e-4).astype(np.float16)
    sb[:, 0:2] = d.view(np.uint8).reshape(nsb, 2)
    return sb


def special_superblocks(rng) -> np.ndarray:
    specials = np.array([0.0, -0.0, 6e-8, -6e-8, 6.1e-5, 1.0, -1.0, 65504.0, -65504.0,
                         np.inf, -np.inf, np.nan], dtype=np.float16)
    sb = random_superblocks(rng, len(specials) * 4)
    sb[:, 0:2] = np.repeat(specials, 4).view(np.uint8).reshape(-1, 2)
    sb[0::4, 2:8] = 0x00          # every code 0  (ls - 32 = -32)
    sb[1::4, 2:8] = 0xFF          # every code 63 (ls - 32 = 31)
    sb[2::4, 2:4] = 0xAA          # every code 32 (ls - 32 = 0): zeros, and NaN for an infinite d
    sb[2::4, 4:8] = 0x00
    return sb


def golden_superblocks() -> np.ndarray:
    from test_oracle_xs_pins import golden_superblock
    return np.concatenate([golden_superblock(n) for n in ("X1", "X2", "X3")])


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_decode_golden_special_random(f16):
    note(f"xs decode: golden + special + random, f16={f16}")
    rng = np.random.default_rng(31)
    sb = np.concatenate([golden_superblocks(), special_superblocks(rng), random_superblocks(rng, 1001)])
    got = gpu_xs_decode(sb, f16)
    ref = oracle.decode_xs_f16(sb) if f16 else oracle.decode_xs(sb)
    assert same_with_nan(got, ref, np.float16 if f16 else np.float32)


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_decode_workload_matrix(f16):
    note(f"xs decode: 6144 x 2560 workload matrix (seed 106), f16={f16}")
    _, sb = workloads.xs_weights(synth.SEED_XS_Z, 6144, 2560)
    got = gpu_xs_decode(sb, f16)
    ref = oracle.decode_xs_f16(sb) if f16 else oracle.decode_xs(sb)
    assert bits_equal(got, ref)


def test_decode_ragged_counts():
    note("xs decode: counts 1, 15, 17, 255")
    rng = np.random.default_rng(32)
    for nsb in (1, 15, 17, 255):
        sb = random_superblocks(rng, nsb)
        assert bits_equal(gpu_xs_decode(sb, False), oracle.decode_xs(sb)), nsb
        assert bits_equal(gpu_xs_decode(sb, True), oracle.decode_xs_f16(sb)), nsb


def run_xs_qmv(sb, n, k, x, T, ldx=None, ldy=None) -> np.ndarray:
    ldx = ldx or k
    ldy = ldy or n + 8
    xb = np.zeros((T, ldx), np.float32)
    xb[:, :k] = x[:T]
    y = torch.full((T, ldy), float("nan"), dtype=torch.float32, device="cuda")
    iq4.iq4_xs_qmv_multi(dev(sb.reshape(-1)), n, k, dev(xb), ldx, T, y, ldy)
    out = host(y)
    assert np.all(np.isnan(out[:, n:])), "wrote outside [0, n)"
    return out[:, :n]


@pytest.mark.parametrize("n,k,seed", [(6144, 2560, synth.SEED_XS_Z), (2560, 6144, synth.SEED_XS_OUT),
                                      (4096, 4096, synth.SEED_XS_Z)])
def test_qmv_workload_shapes_every_T(n, k, seed):
    """Every output of T = 1..8 against the oracle; each column of a T-column call
    bitwise equal to the T = 1 call on that column."""
    note(f"xs qmv: {n} x {k} (seed {seed}), T = 1..8")
    _, sb = workloads.xs_weights(seed, n, k)
    x = synth.acts_f32(seed, synth.TAG_X, 8, k)
    ref = oracle.qmv_xs(sb, n, k, x)
    singles = [run_xs_qmv(sb, n, k, x[t:t + 1], 1)[0] for t in range(8)]
    for T in range(1, 9):
        got = run_xs_qmv(sb, n, k, x, T)
        assert np.isfinite(got).all(), T
        err = normwise(got, ref[:T])
        note(f"  T={T} normwise {err:.2e}")
        assert err <= TOL, (T, err)
        for t in range(T):
            assert bits_equal(got[t], singles[t]), (T, t)


@pytest.mark.parametrize("n,k", [(1, 256), (37, 768), (9, 1280), (300, 16640), (1000, 8448)])
def test_qmv_small_and_ragged(n, k):
    """One super-block per row; a partial last workgroup; K past one pass of the lanes
    (16,640 = 1,040 chunks over 512 lanes, 8,448 = 528 chunks)."""
    note(f"xs qmv: ragged {n} x {k}, T = 1, 3, 8")
    rng = np.random.default_rng(n + k)
    sb = random_superblocks(rng, n * k // 256)
    x = rng.standard_normal((8, k)).astype(np.float32)
    ref = oracle.qmv_xs(sb, n, k, x)
    for T in (1, 3, 8):
        got = run_xs_qmv(sb, n, k, x, T, ldx=k + 4, ldy=n + 3)
        assert normwise(got, ref[:T]) <= TOL, T


@pytest.mark.parametrize("n,k", [(4112, 1024), (4128, 2048), (4100, 3072), (2500, 6144), (33, 6400), (17, 256)])
def test_qmv_launch_shapes(n, k):
    """The matrix-core form's launch shapes: more row tiles than CUs with 1, 2 and 3
    super-blocks per wave (4-wave workgroups, two per CU), 24 super-blocks with a
    partial last row tile, and the first K past it (the vector form); each at T = 1, 4, 8
    against the oracle, columns bitwise equal to their T = 1 call."""
    note(f"xs qmv: launch shape {n} x {k}, T = 1, 4, 8")
    rng = np.random.default_rng(n * 7 + k)
    sb = random_superblocks(rng, n * k // 256)
    x = rng.standard_normal((8, k)).astype(np.float32)
    ref = oracle.qmv_xs(sb, n, k, x)
    one = run_xs_qmv(sb, n, k, x[:1], 1, ldx=k + 4, ldy=n + 3)
    for T in (1, 4, 8):
        got = run_xs_qmv(sb, n, k, x, T, ldx=k + 4, ldy=n + 3)
        assert normwise(got, ref[:T]) <= TOL, T
        assert bits_equal(got[0], one[0]), T


def test_qmv_integer_exact_bitwise():
    """d = 2^-s, every code, integer activations in [-4, 4], K = 1024: every product and
    partial sum is an exact binary32 value (|sum| <= 4064 * 4 * 1024 < 2^24), so the
    result is the oracle's bit for bit whatever the order."""
    note("xs qmv: integer-exact 64 x 1024, T = 1..8")
    rng = np.random.default_rng(41)
    n, k = 64, 1024
    sb = rng.integers(0, 256, (n * k // 256, 136), dtype=np.uint8)
    d = np.float16(2.0) ** -rng.integers(0, 6, sb.shape[0]).astype(np.float16)
    sb[:, 0:2] = d.astype(np.float16).view(np.uint8).reshape(-1, 2)
    x = rng.integers(-4, 5, (8, k)).astype(np.float32)
    ref = oracle.qmv_xs(sb, n, k, x)
    for T in range(1, 9):
        assert bits_equal(run_xs_qmv(sb, n, k, x, T), ref[:T]), T


def test_qmv_one_hot_columns():
    note("xs qmv: one-hot activations, 48 x 512")
    rng = np.random.default_rng(43)
    n, k = 48, 512
    sb = random_superblocks(rng, n * k // 256)
    W = oracle.decode_xs(sb).reshape(n, k)
    cols = [0, 15, 16, 31, 255, 256, 300, 511]
    x = np.zeros((8, k), np.float32)
    for t, j in enumerate(cols):
        x[t, j] = 1.0
    got = run_xs_qmv(sb, n, k, x, 8)
    for t, j in enumerate(cols):
        assert np.array_equal(got[t], W[:, j]), j
