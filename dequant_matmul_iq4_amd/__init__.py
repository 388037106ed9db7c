"""Thin Python binding of the IQ4 C ABI (``include/iq4.h``).

Each function has the C entry point's name and argument order; device buffers are
passed as ``torch.Tensor`` (or raw integer addresses) and ``stream`` defaults to
torch's current stream.  The binding only marshals arguments: every step of the
computation runs in the HIP kernels of ``libiq4.so``.  There is no fallback: if the
library has not been built (``python -m dequant_matmul_iq4_amd.build``) or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libiq4.so")

IQ4_OK = 0
IQ4_E_ARG = -1
IQ4_E_ALIGN = -2
IQ4_E_UNSUPPORTED = -3
IQ4_E_HIP = -4
IQ4_E_WORKSPACE = -5
IQ4_F32 = 0
IQ4_F16 = 1
IQ4_MOE_ATOMIC_COMBINE = 1
IQ4_MOE_KEEP_INTERMEDIATE = 2
# iq4_moe_intermediate_layout indices
MOE_LAYOUT = {"total": 0, "counts": 1, "offsets": 2, "pairs": 3, "slot_row": 4, "h": 5, "rows": 6, "g": 7, "u": 8}
IQ4_QMV_NOALLOC_SCRATCH_BYTES = 4 << 20

_c_i64, _c_i32, _c_u32, _c_p, _c_sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes) exactly as declared in include/iq4.h
SIGNATURES = {
    "iq4_last_error": (ctypes.c_char_p, []),
    "iq4_abi_version": (ctypes.c_int, []),
    "iq4_quantize_blocks": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_p]),
    "iq4_dequant_blocks": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p]),
    "iq4_packed_bytes": (_c_i64, [_c_i64, _c_i64]),
    "iq4_pack_weights": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "iq4_qmv_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "iq4_qmv_multi": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_i32, _c_p, _c_i64, _c_p, _c_sz,
                                     _c_p]),
    "iq4_qmv_multi_noalloc": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_i32, _c_p, _c_i64, _c_p]),
    "iq4_xs_bytes": (_c_i64, [_c_i64, _c_i64]),
    "iq4_xs_dequant": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p]),
    "iq4_xs_qmv_multi": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_i32, _c_p, _c_i64, _c_p]),
    "iq4_quantize_q8_1": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "iq4_qmv_q8": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i32, _c_p, _c_i64, _c_p, _c_sz, _c_p]),
    "iq4_route_topk": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "iq4_moe_gather": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "iq4_moe_workspace_size": (ctypes.c_int, [_c_i64, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32,
                                              ctypes.POINTER(_c_sz)]),
    "iq4_moe_intermediate_layout": (ctypes.c_int, [_c_i64, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32,
                                                   ctypes.POINTER(_c_i64)]),
    "iq4_moe_expert_gemm": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_i32, _c_i32,
                                           _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p,
                                           _c_sz, _c_u32, _c_p]),
    "iq4_moe_shared_workspace_size": (ctypes.c_int, [_c_i64, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32,
                                                     ctypes.POINTER(_c_sz)]),
    "iq4_moe_expert_gemm_shared": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_i32, _c_i32,
                                                  _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                  _c_i64, _c_p, _c_sz, _c_u32, _c_p]),
    "iq4_qgemm": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_i64, _c_p]),
}

_lib = None


class IQ4Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded ``libiq4.so`` (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m dequant_matmul_iq4_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != IQ4_OK:
        raise IQ4Error(name, rc, lib().iq4_last_error().decode())
    return rc


def iq4_last_error() -> str:
    return lib().iq4_last_error().decode()


def iq4_abi_version() -> int:
    return lib().iq4_abi_version()


def iq4_quantize_blocks(src, n_blocks, blocks, stream=None):
    _call("iq4_quantize_blocks", _ptr(src), n_blocks, _ptr(blocks), _stream(stream))


def iq4_dequant_blocks(blocks, n_blocks, out_dtype, out, stream=None):
    _call("iq4_dequant_blocks", _ptr(blocks), n_blocks, out_dtype, _ptr(out), _stream(stream))


def iq4_packed_bytes(n, k) -> int:
    return lib().iq4_packed_bytes(n, k)


def iq4_pack_weights(blocks, n, k, packed, stream=None):
    _call("iq4_pack_weights", _ptr(blocks), n, k, _ptr(packed), _stream(stream))


def iq4_qmv_workspace_size(n, k) -> int:
    out = _c_sz(0)
    _call("iq4_qmv_workspace_size", n, k, ctypes.byref(out))
    return out.value


def iq4_qmv_multi(packed, n, k, x, ldx, T, y, ldy, workspace=None, ws_bytes=0, stream=None):
    _call("iq4_qmv_multi", _ptr(packed), n, k, _ptr(x), ldx, T, _ptr(y), ldy, _ptr(workspace), ws_bytes,
          _stream(stream))


def iq4_qmv_multi_noalloc(packed, n, k, x, ldx, T, y, ldy, stream=None):
    _call("iq4_qmv_multi_noalloc", _ptr(packed), n, k, _ptr(x), ldx, T, _ptr(y), ldy, _stream(stream))


def iq4_xs_bytes(n, k) -> int:
    return lib().iq4_xs_bytes(n, k)


def iq4_xs_dequant(sb, n_superblocks, out_dtype, out, stream=None):
    _call("iq4_xs_dequant", _ptr(sb), n_superblocks, out_dtype, _ptr(out), _stream(stream))


def iq4_xs_qmv_multi(w, n, k, x, ldx, T, y, ldy, stream=None):
    _call("iq4_xs_qmv_multi", _ptr(w), n, k, _ptr(x), ldx, T, _ptr(y), ldy, _stream(stream))


def iq4_quantize_q8_1(x, T, k, ldx, q, d, stream=None):
    _call("iq4_quantize_q8_1", _ptr(x), T, k, ldx, _ptr(q), _ptr(d), _stream(stream))


def iq4_qmv_q8(packed, n, k, q, d, T, y, ldy, workspace=None, ws_bytes=0, stream=None):
    _call("iq4_qmv_q8", _ptr(packed), n, k, _ptr(q), _ptr(d), T, _ptr(y), ldy, _ptr(workspace), ws_bytes,
          _stream(stream))


def iq4_route_topk(logits, n_tok, n_expert, top_k, ids, w, stream=None):
    _call("iq4_route_topk", _ptr(logits), n_tok, n_expert, top_k, _ptr(ids), _ptr(w), _stream(stream))


def iq4_moe_gather(ids, n_pairs, n_expert, counts, offsets, pairs, slot_row, stream=None):
    _call("iq4_moe_gather", _ptr(ids), n_pairs, n_expert, _ptr(counts), _ptr(offsets), _ptr(pairs),
          _ptr(slot_row), _stream(stream))


def iq4_moe_workspace_size(n_tok, top_k, n_expert, hidden, inter, act_dtype) -> int:
    out = _c_sz(0)
    _call("iq4_moe_workspace_size", n_tok, top_k, n_expert, hidden, inter, act_dtype, ctypes.byref(out))
    return out.value


def iq4_moe_intermediate_layout(n_tok, top_k, n_expert, hidden, inter, act_dtype, shared=0) -> dict:
    """Byte offsets of the kept intermediates (and the workspace size a keeping call needs)."""
    out = (_c_i64 * 9)()
    _call("iq4_moe_intermediate_layout", n_tok, top_k, n_expert, hidden, inter, act_dtype, shared, out)
    return {name: int(out[i]) for name, i in MOE_LAYOUT.items()}


def iq4_moe_expert_gemm(x, act_dtype, n_tok, ldx, ids, w, top_k, n_expert, hidden, inter,
                        w_gate, w_up, w_down, out, ldo, workspace, ws_bytes, flags=0, stream=None):
    _call("iq4_moe_expert_gemm", _ptr(x), act_dtype, n_tok, ldx, _ptr(ids), _ptr(w), top_k, n_expert,
          hidden, inter, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out), ldo, _ptr(workspace),
          ws_bytes, flags, _stream(stream))


def iq4_moe_shared_workspace_size(n_tok, top_k, n_expert, hidden, inter, act_dtype) -> int:
    out = _c_sz(0)
    _call("iq4_moe_shared_workspace_size", n_tok, top_k, n_expert, hidden, inter, act_dtype, ctypes.byref(out))
    return out.value


def iq4_moe_expert_gemm_shared(x, act_dtype, n_tok, ldx, ids, w, top_k, n_expert, hidden, inter,
                               w_gate, w_up, w_down, s_gate, s_up, s_down, out, ldo, workspace, ws_bytes,
                               flags=0, stream=None):
    _call("iq4_moe_expert_gemm_shared", _ptr(x), act_dtype, n_tok, ldx, _ptr(ids), _ptr(w), top_k, n_expert,
          hidden, inter, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down),
          _ptr(out), ldo, _ptr(workspace), ws_bytes, flags, _stream(stream))


def iq4_qgemm(packed, n, k, x, m, ldx, y, ldy, chunk, stream=None):
    _call("iq4_qgemm", _ptr(packed), n, k, _ptr(x), m, ldx, _ptr(y), ldy, chunk, _stream(stream))
