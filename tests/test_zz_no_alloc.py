"""The matvec entry point that allocates nothing (iq4_qmv_multi_noalloc), through the C
ABI, against iq4_qmv_multi with a caller workspace: bitwise equal on two calls in a row,
the second with a smaller input, both on split-K shapes (k > 4096) so that the library's
own scratch array carries the partial sums and arrival counters; then a shape without
split K, and the oracle's tolerance on the first call.  Runs last (its file name sorts
after the other GPU tests) and also alone in a fresh process."""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
from gpu_util import bits_equal, dev, host, normwise, note, pack, qmv_workspace

pytestmark = pytest.mark.gpu


def _inputs(seed, n, k, T):
    rng = np.random.default_rng(seed)
    b = oracle.encode_blocks((rng.standard_normal((n * k // 32, 32)) * 0.02).astype(np.float32))
    x = rng.standard_normal((T, k)).astype(np.float32)
    return b, x


def _both(packed, n, k, x):
    T = x.shape[0]
    xd = dev(x)
    y_ws = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    y_na = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    ws, wsb = qmv_workspace(n, k)
    iq4.iq4_qmv_multi(packed, n, k, xd, k, T, y_ws, n, ws, wsb)
    iq4.iq4_qmv_multi_noalloc(packed, n, k, xd, k, T, y_na, n)
    return host(y_ws), host(y_na)


def test_noalloc_matches_workspace_call_twice_then_smaller():
    cases = [(256, 14336, 8, 1), (128, 8192, 3, 2), (512, 2048, 4, 3)]
    for i, (n, k, T, seed) in enumerate(cases):
        note(f"qmv noalloc: call {i + 1}: n={n} k={k} T={T} (split-K scratch: {k > 4096})")
        b, x = _inputs(seed, n, k, T)
        packed = pack(b, n, k)
        ref, got = _both(packed, n, k, x)
        assert np.isfinite(got).all()
        assert bits_equal(got, ref), (n, k, T)
        if i == 0:
            assert normwise(got, oracle.qmv(b, n, k, x)) <= 1e-3


def test_noalloc_rejects_shapes_beyond_its_scratch():
    note("qmv noalloc: a shape above the scratch size is rejected")
    n, k = 1 << 15, 1 << 17
    assert iq4.iq4_qmv_workspace_size(n, k) > iq4.IQ4_QMV_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    rc = iq4.lib().iq4_qmv_multi_noalloc(fake, n, k, fake, k, 1, fake, n, None)
    assert rc == iq4.IQ4_E_WORKSPACE and "scratch" in iq4.iq4_last_error()
