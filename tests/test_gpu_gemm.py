"""Dense dequant-fused GEMM (prompt projection in chunks) on the GPU vs the oracle.

Tolerance: binary16 activations, weights decoded to binary16, fp32 accumulation:
normwise max|y - r| / max|r| <= 5e-3 (the stated tolerance for the f16 matrix-core
paths).  Power-of-two scales with small-integer activations make every product and
partial sum exact, so those cases must match bitwise; results must not depend on the
chunk size (bitwise).
"""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
import synth
from gpu_util import bits_equal, dev, host, normwise, note, pack
from test_oracle_pins import integer_exact_blocks
import workloads

pytestmark = pytest.mark.gpu

TOL = 5e-3


def run_qgemm(packed, n, k, x16: np.ndarray, chunk=512, ldy=None) -> np.ndarray:
    m = x16.shape[0]
    ldy = ldy or n
    xd = dev(x16.astype(np.float16))
    y = torch.full((m, ldy), float("nan"), dtype=torch.float32, device="cuda")
    iq4.iq4_qgemm(packed, n, k, xd, m, k, y, ldy, chunk)
    out = host(y)
    if ldy > n:
        assert np.all(np.isnan(out[:, n:])), "wrote outside [0, n)"
    return out[:, :n]


@pytest.mark.parametrize("n,k,m", [(256, 256, 200), (48, 128, 5), (272, 384, 129), (512, 768, 640)])
def test_small_shapes(n, k, m):
    note(f"qgemm: n={n} k={k} m={m}")
    rng = np.random.default_rng(n + k + m)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float16)
    y = run_qgemm(pack(b, n, k), n, k, x, ldy=n + 16)
    assert normwise(y, oracle.gemm(b, n, k, x)) <= TOL


@pytest.mark.parametrize("n,k,m", [(256, 256, 130), (48, 384, 17)])
def test_integer_exact_bitwise(n, k, m):
    note(f"qgemm: integer-exact n={n} k={k} m={m}")
    rng = np.random.default_rng(7 * n + k)
    b = integer_exact_blocks(rng, n * k // 32, 4)
    x = rng.integers(-8, 9, (m, k)).astype(np.float16)
    y = run_qgemm(pack(b, n, k), n, k, x)
    assert bits_equal(y, oracle.gemm(b, n, k, x))


def test_unaligned_output_rows_bitwise():
    """Output rows that do not allow 16-byte stores (ldy not a multiple of 4, base 4 bytes
    past a 16-byte boundary) take the scalar stores: the same values, and nothing
    written outside the n columns of each row."""
    note("qgemm: unaligned output rows (ldy = n + 3, base + 4 bytes)")
    n, k, m = 48, 256, 37
    rng = np.random.default_rng(23)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float16)
    packed = pack(b, n, k)
    ref = run_qgemm(packed, n, k, x)  # ldy = n: 16-byte stores
    ldy = n + 3
    xd = dev(x)
    buf = torch.full((m * ldy + 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = buf[1:1 + m * ldy]  # 4 bytes past the (256-byte aligned) allocation
    iq4.iq4_qgemm(packed, n, k, xd, m, k, y, ldy, 512)
    out = host(buf)
    assert np.isnan(out[0]) and np.all(np.isnan(out[1 + m * ldy:]))
    rows = out[1:1 + m * ldy].reshape(m, ldy)
    assert np.all(np.isnan(rows[:, n:])), "wrote outside [0, n)"
    assert bits_equal(rows[:, :n], ref)
    assert normwise(rows[:, :n], oracle.gemm(b, n, k, x)) <= TOL


def test_chunk_invariance_bitwise():
    note("qgemm: chunk 512 / 256 / 100 / one launch, bitwise")
    n, k, m = 512, 512, 1100
    rng = np.random.default_rng(11)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float16)
    packed = pack(b, n, k)
    ref = run_qgemm(packed, n, k, x, chunk=512)
    for chunk in (256, 100, 0):
        assert bits_equal(run_qgemm(packed, n, k, x, chunk=chunk), ref), chunk


def test_long_prompt_projection_full():
    """The full long-prompt workload: W 14,336 x 4,096 (seed 105), 13,056 f16 tokens in
    512-token chunks (25 full chunks and a 256-token tail), exactly as the benchmark
    launches it.  The output starts as NaN and every one of the 13,056 x 14,336 outputs
    is compared with the oracle (5e-3)."""
    import time
    note("qgemm: long prompt 13056 x 4096 x 14336, chunk 512, every output")
    n, k, m = 14336, 4096, 13056
    _, b = workloads.dense_weights(synth.SEED_LONG, n, k)
    x = workloads.acts16(synth.SEED_LONG, m, k)
    packed = pack(b, n, k)
    xd = dev(x)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    iq4.iq4_qgemm(packed, n, k, xd, m, k, y, n, 512)
    got = host(y)
    del y
    t0 = time.perf_counter()
    ref = oracle.gemm(b, n, k, x)
    note(f"  oracle {time.perf_counter() - t0:.1f} s")
    assert np.isfinite(got).all()
    err = normwise(got, ref)
    note(f"  normwise {err:.2e}")
    assert err <= TOL
