"""Block format on the GPU: the device encoder and decoder are bitwise equal to the
oracle's (page 2, PLE-compact commit: device dequant = host dequant, bit for bit)."""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
import synth
from gpu_util import bits_equal, dev, host, note
from test_oracle_pins import encode_cases, special_blocks
import workloads

pytestmark = pytest.mark.gpu


def gpu_quantize(w32: np.ndarray) -> np.ndarray:
    w = dev(w32.reshape(-1, 32).astype(np.float32))
    nb = w.shape[0]
    out = torch.empty(nb * 18, dtype=torch.uint8, device="cuda")
    iq4.iq4_quantize_blocks(w, nb, out)
    return host(out).reshape(nb, 18)


def gpu_dequant(blocks: np.ndarray, f16: bool) -> np.ndarray:
    b = dev(blocks.reshape(-1))
    nb = blocks.reshape(-1, 18).shape[0]
    out = torch.full((nb * 32,), float("nan"), dtype=torch.float16 if f16 else torch.float32, device="cuda")
    iq4.iq4_dequant_blocks(b, nb, iq4.IQ4_F16 if f16 else iq4.IQ4_F32, out)
    return host(out).reshape(nb, 32)


def test_quantize_edge_cases_bitwise():
    note("quantize: tie / zero / tiny / positive-max blocks")
    cases = np.stack(encode_cases(seed=21))
    assert bits_equal(gpu_quantize(cases), oracle.encode_blocks(cases))


@pytest.mark.parametrize("cfg", ["plumbing", "verify"])
def test_quantize_workload_bitwise(cfg):
    note(f"quantize: {cfg} weights")
    if cfg == "plumbing":
        w, b = workloads.dense_weights(synth.SEED_PLUMBING, 512, 2048)
    else:
        w, b = workloads.dense_weights(synth.SEED_VERIFY, 4096, 4096)
    assert bits_equal(gpu_quantize(w), b)


def test_quantize_expert_bitwise():
    note("quantize: expert 0 gate of the expert bank")
    w = synth.weights_f32(synth.SEED_EXPERTS, synth.tag_expert(0, "gate"), 768, 2048)
    assert bits_equal(gpu_quantize(w), oracle.encode_blocks(w.reshape(-1, 32)))


def test_dequant_special_blocks_bitwise():
    note("dequant: every index x special scales (f32 and f16)")
    blocks = np.frombuffer(b"".join(special_blocks()), dtype=np.uint8).reshape(-1, 18)
    ref32 = oracle.decode_blocks(blocks)
    got32 = gpu_dequant(blocks, False)
    nan = np.isnan(ref32)
    assert np.array_equal(nan, np.isnan(got32))
    assert bits_equal(np.where(nan, 0, got32).astype(np.float32), np.where(nan, 0, ref32).astype(np.float32))
    with np.errstate(all="ignore"):
        ref16 = oracle.decode_blocks_f16(blocks)
    got16 = gpu_dequant(blocks, True)
    nan = np.isnan(ref16)
    assert np.array_equal(nan, np.isnan(got16))
    assert bits_equal(np.where(nan, 0, got16).astype(np.float16), np.where(nan, 0, ref16).astype(np.float16))


def test_dequant_workload_bitwise():
    note("dequant: verify-window matrix (f32 and f16)")
    _, b = workloads.dense_weights(synth.SEED_VERIFY, 4096, 4096)
    assert bits_equal(gpu_dequant(b, False), oracle.decode_blocks(b))
    assert bits_equal(gpu_dequant(b, True), oracle.decode_blocks_f16(b))


def test_dequant_odd_count():
    note("dequant: 7 blocks")
    rng = np.random.default_rng(3)
    b = oracle.encode_blocks(rng.standard_normal((7, 32)).astype(np.float32))
    assert bits_equal(gpu_dequant(b, False), oracle.decode_blocks(b))


@pytest.mark.parametrize("nb", [197, 453])
def test_dequant_staged_and_direct_paths(nb):
    """197 blocks: three one-group workgroups of 64 blocks plus a direct tail when 16-byte
    aligned; 453 blocks: one four-group workgroup, three one-group workgroups and a
    direct tail; all direct when the same blocks start 2 bytes into an allocation."""
    note(f"dequant: {nb} blocks, aligned and at a 2-byte offset (f32 and f16)")
    rng = np.random.default_rng(21 + nb)
    b = oracle.encode_blocks((rng.standard_normal((nb, 32)) * 0.02).astype(np.float32))
    for f16, ref in ((False, oracle.decode_blocks(b)), (True, oracle.decode_blocks_f16(b))):
        assert bits_equal(gpu_dequant(b, f16), ref)
        raw = torch.zeros(b.size + 16, dtype=torch.uint8, device="cuda")
        raw[2:2 + b.size] = dev(b.reshape(-1))
        out = torch.full((nb * 32,), float("nan"), dtype=torch.float16 if f16 else torch.float32, device="cuda")
        iq4.iq4_dequant_blocks(raw.data_ptr() + 2, nb, iq4.IQ4_F16 if f16 else iq4.IQ4_F32, out)
        assert bits_equal(host(out).reshape(ref.shape), ref)
