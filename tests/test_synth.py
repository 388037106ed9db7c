"""The seeded input generator (CPU only)."""
import numpy as np

import synth


def test_splitmix64_reference_sequence():
    # SplitMix64 started from state 0 (Steele, Lea & Flood 2014): its first three
    # outputs are the widely published values below.
    assert synth.stream_key(0, 0) == 0
    got = synth.raw_u64(0, 0, 0, 3).tolist()
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_ranges_are_consistent():
    whole = synth.raw_u64(7, 3, 0, 1000)
    assert np.array_equal(whole[250:700], synth.raw_u64(7, 3, 250, 450))
    # a large request is filled in parallel chunks; it must equal the serial stream
    n = (1 << 22) + 12345
    z = synth.normal(9, 1, n)
    assert np.array_equal(z[-1000:], synth.normal(9, 1, n)[-1000:])
    head = synth.normal(9, 1, 4096)
    assert np.array_equal(z[:4096], head)


def test_streams_differ_by_tag_and_seed():
    a = synth.raw_u64(1, 0, 0, 64)
    assert not np.array_equal(a, synth.raw_u64(1, 1, 0, 64))
    assert not np.array_equal(a, synth.raw_u64(2, 0, 0, 64))


def test_distributions():
    z = synth.normal(5, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    u = synth.uniform(5, 1, 1 << 20)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 2e-3
    w = synth.weights_f32(5, 0, 256, 256)
    assert w.dtype == np.float32 and abs(w.std() - 0.02) < 5e-4
    x = synth.acts_f16(5, 1000, 8, 64)
    assert x.dtype == np.float16


def test_zipf_gumbel_logits_skew():
    L = synth.logits_zipf_gumbel(104, synth.TAG_GUMBEL, 3256, 128)
    top = np.argsort(-L, axis=1, kind="stable")[:, :8]
    counts = np.bincount(top.reshape(-1), minlength=128)
    assert counts.sum() == 3256 * 8
    assert counts[0] > counts[10] > counts[100]
    assert counts.max() <= 3256


def test_torch_stream_matches_numpy():
    import torch
    a = synth.raw_u64(103, 7, 100, 5000)
    b = synth.raw_u64_torch(103, 7, 100, 5000).numpy().view(np.uint64)
    assert np.array_equal(a, b)
    z = synth.normal(103, 7, 10001)
    zt = synth.normal_torch(103, 7, 10001).numpy()
    assert np.allclose(z, zt, rtol=1e-13, atol=1e-13)
    w = synth.weights_f32(104, 3, 64, 128)
    wt = synth.weights_f32_torch(104, 3, 64, 128).numpy()
    assert np.mean(w == wt) > 0.9999
