"""The C ABI on the CPU: the library loads, exports every entry point that
include/iq4.h declares, and rejects bad arguments on the host before touching a GPU.
(No call here reaches a launch.)"""
import ctypes
import os
import re

import pytest

import dequant_matmul_iq4_amd as iq4
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "iq4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(iq4_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = iq4.lib()
    names = declared_functions()
    assert len(names) >= 11
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(iq4.SIGNATURES), "binding and header disagree"


def test_abi_version():
    assert iq4.iq4_abi_version() == 1


def test_packed_bytes():
    assert iq4.iq4_packed_bytes(4096, 4096) == 4096 * 4096 // 32 * 18
    assert iq4.iq4_packed_bytes(768, 2048) == 768 * 2048 // 32 * 18
    assert iq4.iq4_packed_bytes(15, 128) == -1
    assert iq4.iq4_packed_bytes(16, 96) == -1
    assert iq4.iq4_packed_bytes(0, 128) == -1


def _rc(name, *args):
    return getattr(iq4.lib(), name)(*args)


FAKE = 1 << 20  # a 256-byte-aligned non-null address that no call may dereference


def test_validation_errors_never_launch():
    assert _rc("iq4_qmv_multi", FAKE, 16, 128, FAKE, 128, 0, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    assert "T must be" in iq4.iq4_last_error()
    assert _rc("iq4_qmv_multi", FAKE, 16, 128, FAKE, 128, 9, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_qmv_multi", FAKE, 17, 128, FAKE, 128, 1, FAKE, 17, None, 0, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc("iq4_qmv_multi", FAKE, 16, 96, FAKE, 128, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc("iq4_qmv_multi", FAKE, 16, 128, FAKE, 127, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_qmv_multi", FAKE, 16, 128, FAKE + 4, 128, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_qmv_multi", FAKE + 16, 16, 128, FAKE, 128, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_qmv_multi", None, 16, 128, FAKE, 128, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_dequant_blocks", FAKE, 4, 7, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_dequant_blocks", FAKE + 1, 4, 0, FAKE, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_dequant_blocks", FAKE, -1, 0, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_quantize_blocks", FAKE + 4, 4, FAKE, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_pack_weights", FAKE, 16, 128, FAKE, None) == iq4.IQ4_E_ARG  # overlap
    assert _rc("iq4_pack_weights", FAKE, 16, 100, FAKE * 2, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc("iq4_route_topk", FAKE, 4, 8, 9, FAKE, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_route_topk", FAKE, 4, 2000, 8, FAKE, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_moe_gather", FAKE, -1, 8, FAKE, FAKE, FAKE, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_moe_gather", FAKE, 8, 0, FAKE, FAKE, FAKE, FAKE, None) == iq4.IQ4_E_ARG


def test_qmv_workspace_rules():
    # K up to 4096 is one slice per workgroup: no workspace
    assert iq4.iq4_qmv_workspace_size(768, 768) == 0
    assert iq4.iq4_qmv_workspace_size(4096, 4096) == 0
    need = iq4.iq4_qmv_workspace_size(256, 14336)  # K split over workgroups
    assert need > 0
    assert _rc("iq4_qmv_multi", FAKE, 256, 14336, FAKE, 14336, 1, FAKE, 256, None, 0, None) == iq4.IQ4_E_WORKSPACE
    assert _rc("iq4_qmv_multi", FAKE, 256, 14336, FAKE, 14336, 1, FAKE, 256, FAKE, need - 1, None) == iq4.IQ4_E_WORKSPACE
    assert _rc("iq4_qmv_multi", FAKE, 256, 14336, FAKE, 14336, 1, FAKE, 256, FAKE + 64, need, None) == iq4.IQ4_E_ALIGN


def test_moe_and_gemm_validation():
    ws = iq4.iq4_moe_workspace_size(3256, 8, 128, 2048, 768, iq4.IQ4_F16)
    assert ws > 3256 * 8 * (2048 + 768) * 2  # binary16 slot rows and h (prefill)
    assert iq4.iq4_moe_workspace_size(4, 8, 128, 2048, 768, iq4.IQ4_F32) > 4 * 8 * (2048 + 768) * 4  # fp32 (decode)
    rc = _rc("iq4_moe_expert_gemm", FAKE, iq4.IQ4_F16, 16, 2048, FAKE, FAKE, 8, 128, 2048, 768,
             FAKE, FAKE, FAKE, FAKE, 2048, FAKE, 16, 0, None)
    assert rc == iq4.IQ4_E_WORKSPACE
    rc = _rc("iq4_moe_expert_gemm", FAKE, iq4.IQ4_F32, 16, 2048, FAKE, FAKE, 8, 128, 2048, 5000,
             FAKE, FAKE, FAKE, FAKE, 2048, FAKE, 1 << 30, 0, None)
    assert rc == iq4.IQ4_E_UNSUPPORTED  # fp32 path: inter above 4096
    rc = _rc("iq4_moe_expert_gemm", FAKE, iq4.IQ4_F16, 16, 2048, FAKE, FAKE, 9, 8, 2048, 768,
             FAKE, FAKE, FAKE, FAKE, 2048, FAKE, 1 << 30, 0, None)
    assert rc == iq4.IQ4_E_ARG  # top_k > n_expert
    rc = _rc("iq4_moe_expert_gemm", FAKE, iq4.IQ4_F16, 16, 2048, FAKE, FAKE, 17, 128, 2048, 768,
             FAKE, FAKE, FAKE, FAKE, 2048, FAKE, 1 << 30, 0, None)
    assert rc == iq4.IQ4_E_ARG  # top_k > 16
    nb = ctypes.c_size_t(0)
    assert iq4.lib().iq4_moe_workspace_size(16, 17, 128, 2048, 768, iq4.IQ4_F16, ctypes.byref(nb)) == iq4.IQ4_E_ARG
    rc = _rc("iq4_moe_expert_gemm", FAKE, iq4.IQ4_F16, 16, 2048, FAKE, FAKE, 8, 128, 2048, 768,
             FAKE, FAKE, FAKE, FAKE, 2048, FAKE, 1 << 30, 4, None)
    assert rc == iq4.IQ4_E_ARG  # unknown flag
    assert _rc("iq4_qgemm", FAKE, 256, 256, FAKE, 10, 252, FAKE, 256, 512, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_qgemm", FAKE, 256, 256, FAKE + 8, 10, 256, FAKE, 256, 512, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_qgemm", FAKE, 256, 256, FAKE, 0, 256, FAKE, 256, 512, None) == iq4.IQ4_OK


def test_moe_shared_validation():
    """The shared-expert call is validated as the routed call with one more expert and
    slot; none of these launches."""
    plain = iq4.iq4_moe_workspace_size(3256, 8, 128, 2048, 768, iq4.IQ4_F16)
    ws = iq4.iq4_moe_shared_workspace_size(3256, 8, 128, 2048, 768, iq4.IQ4_F16)
    assert ws >= iq4.iq4_moe_workspace_size(3256, 9, 129, 2048, 768, iq4.IQ4_F16) > plain
    nb = ctypes.c_size_t(0)
    L = iq4.lib()
    assert L.iq4_moe_shared_workspace_size(16, 16, 128, 2048, 768, iq4.IQ4_F16, ctypes.byref(nb)) == iq4.IQ4_E_ARG
    assert L.iq4_moe_shared_workspace_size(16, 8, 1024, 2048, 768, iq4.IQ4_F16, ctypes.byref(nb)) == iq4.IQ4_E_ARG
    assert L.iq4_moe_shared_workspace_size(16, 15, 1023, 2048, 768, iq4.IQ4_F32, ctypes.byref(nb)) == iq4.IQ4_OK

    def call(top_k=8, n_expert=128, shared=(FAKE, FAKE, FAKE), ws_bytes=1 << 30, flags=0):
        return _rc("iq4_moe_expert_gemm_shared", FAKE, iq4.IQ4_F16, 16, 2048, FAKE, FAKE, top_k, n_expert, 2048,
                   768, FAKE, FAKE, FAKE, *shared, FAKE, 2048, FAKE, ws_bytes, flags, None)
    assert call(top_k=16) == iq4.IQ4_E_ARG  # the shared expert takes a 17th slot
    assert call(n_expert=1024) == iq4.IQ4_E_ARG  # and a 1025th expert
    assert call(shared=(FAKE, None, FAKE)) == iq4.IQ4_E_ARG
    assert call(shared=(FAKE, FAKE, FAKE + 16)) == iq4.IQ4_E_ALIGN
    need = iq4.iq4_moe_shared_workspace_size(16, 8, 128, 2048, 768, iq4.IQ4_F16)
    assert need > iq4.iq4_moe_workspace_size(16, 8, 128, 2048, 768, iq4.IQ4_F16)
    assert call(ws_bytes=need - 1) == iq4.IQ4_E_WORKSPACE
    assert call(flags=4) == iq4.IQ4_E_ARG


def test_zero_sized_calls_are_no_ops():
    assert _rc("iq4_quantize_blocks", None, 0, None, None) == iq4.IQ4_OK
    assert _rc("iq4_dequant_blocks", None, 0, 0, None, None) == iq4.IQ4_OK
    assert _rc("iq4_route_topk", None, 0, 8, 2, None, None, None) == iq4.IQ4_OK


def test_binding_raises_with_message():
    with pytest.raises(iq4.IQ4Error) as ei:
        iq4.iq4_qmv_multi(FAKE, 16, 128, FAKE, 128, 0, FAKE, 16, None, 0, stream=0)
    assert ei.value.code == iq4.IQ4_E_ARG and "T must be" in str(ei.value)


def test_q8_validation_errors_never_launch():
    # quantize: k % 32, ldx, alignment, null
    assert _rc("iq4_quantize_q8_1", FAKE, 2, 48, 48, FAKE, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_quantize_q8_1", FAKE, 2, 64, 60, FAKE, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_quantize_q8_1", FAKE, -1, 64, 64, FAKE, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_quantize_q8_1", FAKE + 4, 2, 64, 64, FAKE, FAKE, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_quantize_q8_1", FAKE, 2, 64, 64, FAKE + 4, FAKE, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_quantize_q8_1", FAKE, 2, 64, 64, None, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_quantize_q8_1", None, 0, 64, 64, None, None, None) == iq4.IQ4_OK  # T = 0: no-op
    # matvec: T range, shape, ldy, alignment, workspace
    assert _rc("iq4_qmv_q8", FAKE, 16, 128, FAKE, FAKE, 0, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    assert "T must be" in iq4.iq4_last_error()
    assert _rc("iq4_qmv_q8", FAKE, 16, 128, FAKE, FAKE, 9, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_qmv_q8", FAKE, 17, 128, FAKE, FAKE, 1, FAKE, 17, None, 0, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc("iq4_qmv_q8", FAKE, 16, 96, FAKE, FAKE, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc("iq4_qmv_q8", FAKE, 16, 128, FAKE, FAKE, 1, FAKE, 15, None, 0, None) == iq4.IQ4_E_ARG
    assert _rc("iq4_qmv_q8", FAKE, 16, 128, FAKE + 4, FAKE, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_qmv_q8", FAKE, 16, 128, FAKE, FAKE + 1, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ALIGN
    assert _rc("iq4_qmv_q8", None, 16, 128, FAKE, FAKE, 1, FAKE, 16, None, 0, None) == iq4.IQ4_E_ARG
    need = iq4.iq4_qmv_workspace_size(256, 14336)
    assert _rc("iq4_qmv_q8", FAKE, 256, 14336, FAKE, FAKE, 1, FAKE, 256, FAKE, need - 1, None) == iq4.IQ4_E_WORKSPACE


def test_noalloc_matvec_validation_never_launches():
    """The no-allocation matvec validates as iq4_qmv_multi and rejects shapes whose
    split-K scratch would exceed its fixed device array, before any set-up or launch."""
    assert _rc("iq4_qmv_multi_noalloc", FAKE, 16, 128, FAKE, 128, 0, FAKE, 16, None) == iq4.IQ4_E_ARG
    assert "T must be" in iq4.iq4_last_error()
    assert _rc("iq4_qmv_multi_noalloc", FAKE, 17, 128, FAKE, 128, 1, FAKE, 17, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc("iq4_qmv_multi_noalloc", FAKE, 16, 128, FAKE + 4, 128, 1, FAKE, 16, None) == iq4.IQ4_E_ALIGN
    n, k = 1 << 15, 1 << 17
    assert iq4.iq4_qmv_workspace_size(n, k) > iq4.IQ4_QMV_NOALLOC_SCRATCH_BYTES
    assert _rc("iq4_qmv_multi_noalloc", FAKE, n, k, FAKE, k, 1, FAKE, n, None) == iq4.IQ4_E_WORKSPACE
    assert "scratch" in iq4.iq4_last_error()


def test_moe_keep_intermediate_layout():
    """The kept-intermediates layout: regions in order, each inside the total, g and u
    after everything a plain call uses; a keeping call with only the plain workspace is
    rejected before any launch."""
    for act in (iq4.IQ4_F16, iq4.IQ4_F32):
        L = iq4.iq4_moe_intermediate_layout(3256, 8, 128, 2048, 768, act)
        plain = iq4.iq4_moe_workspace_size(3256, 8, 128, 2048, 768, act)
        P = 3256 * 8
        assert L["g"] >= plain and L["u"] >= L["g"] + P * 768 * 4 and L["total"] >= L["u"] + P * 768 * 4
        assert L["counts"] < L["offsets"] < L["pairs"] < L["slot_row"] < L["h"] < L["rows"] < L["g"]
        assert all(v % 256 == 0 for v in L.values())
    Ls = iq4.iq4_moe_intermediate_layout(16, 8, 128, 2048, 768, iq4.IQ4_F16, 1)
    assert Ls["total"] > iq4.iq4_moe_intermediate_layout(16, 8, 128, 2048, 768, iq4.IQ4_F16)["total"]
    plain = iq4.iq4_moe_workspace_size(16, 8, 128, 2048, 768, iq4.IQ4_F16)
    rc = _rc("iq4_moe_expert_gemm", FAKE, iq4.IQ4_F16, 16, 2048, FAKE, FAKE, 8, 128, 2048, 768,
             FAKE, FAKE, FAKE, FAKE, 2048, FAKE, plain, iq4.IQ4_MOE_KEEP_INTERMEDIATE, None)
    assert rc == iq4.IQ4_E_WORKSPACE
    with pytest.raises(iq4.IQ4Error):
        iq4.iq4_moe_intermediate_layout(16, 17, 128, 2048, 768, iq4.IQ4_F16)


def test_xs_validation_errors_never_launch():
    """The IQ4_XS calls: sizes, T range, alignment and pointers are checked on the host."""
    assert iq4.iq4_xs_bytes(6144, 2560) == 6144 * 10 * 136
    assert iq4.iq4_xs_bytes(1, 256) == 136
    assert iq4.iq4_xs_bytes(4, 128) == -1 and iq4.iq4_xs_bytes(0, 256) == -1
    q = "iq4_xs_qmv_multi"
    assert _rc(q, FAKE, 16, 256, FAKE, 256, 0, FAKE, 16, None) == iq4.IQ4_E_ARG
    assert "T must be" in iq4.iq4_last_error()
    assert _rc(q, FAKE, 16, 256, FAKE, 256, 9, FAKE, 16, None) == iq4.IQ4_E_ARG
    assert _rc(q, FAKE, 16, 384, FAKE, 384, 1, FAKE, 16, None) == iq4.IQ4_E_UNSUPPORTED
    assert _rc(q, FAKE, 0, 256, FAKE, 256, 1, FAKE, 16, None) == iq4.IQ4_E_ARG
    assert _rc(q, FAKE, 16, 256, FAKE, 252, 1, FAKE, 16, None) == iq4.IQ4_E_ARG       # ldx < k
    assert _rc(q, FAKE, 16, 256, FAKE, 256, 1, FAKE, 15, None) == iq4.IQ4_E_ARG       # ldy < n
    assert _rc(q, FAKE + 4, 16, 256, FAKE, 256, 1, FAKE, 16, None) == iq4.IQ4_E_ALIGN
    assert _rc(q, FAKE, 16, 256, FAKE + 8, 256, 1, FAKE, 16, None) == iq4.IQ4_E_ALIGN
    assert _rc(q, FAKE, 16, 256, FAKE, 258, 1, FAKE, 16, None) == iq4.IQ4_E_ALIGN     # ldx % 4
    assert _rc(q, None, 16, 256, FAKE, 256, 1, FAKE, 16, None) == iq4.IQ4_E_ARG
    d = "iq4_xs_dequant"
    assert _rc(d, FAKE, 4, 7, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc(d, FAKE, -1, 0, FAKE, None) == iq4.IQ4_E_ARG
    assert _rc(d, FAKE + 4, 4, 0, FAKE, None) == iq4.IQ4_E_ALIGN
    assert _rc(d, FAKE, 4, 0, FAKE + 8, None) == iq4.IQ4_E_ALIGN
    assert _rc(d, FAKE, 0, 0, None, None) == iq4.IQ4_OK                                # nothing to do
