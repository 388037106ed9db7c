"""Plain, slow, obviously-correct CPU reference (numpy, float64) of the IQ4 hot path.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the HIP library never imports it and shares no
code with it.

Sources.  The method is described on three web pages: the Strata commit "wire
multi-token kernels into Verifier and MtpDrafter CUDA graphs" (page 1, the
``verify.hpp`` header), the Strata pull request "sm_80 (GA100) tuning" (page 2, its
commit messages and description) and the DSpark ``tp2.py`` drafter file (page 3).
The pages never print the block layout; the workload definition fixes it as 32 weights
per block, an fp16 scale ``d = absmax / 127`` and 4-bit indices into the 16-level int8
codebook below, each index the nearest level after scaling.  Page 2's PLE-compact
commit message (2,560 values in 1,440 bytes) fixes the block at 18 bytes.

Readings where the pages are silent (each also listed in the design notes):

* byte layout: bytes 0-1 hold ``d`` as little-endian IEEE binary16; byte ``2 + i``
  (i < 16) holds index ``q_i`` in its low nibble and ``q_{i+16}`` in its high nibble;
* ``d = f16_rne(f32(absmax) / 127)`` with an IEEE binary32 division;
* nearest level in exact arithmetic, ties to the lower index; a block whose ``d`` is
  zero stores index 8 everywhere (the level nearest zero);
* SwiGLU is ``silu(gate) * up`` with no clamp; gate weights are the softmax over the
  k selected logits; routing takes the k largest logits, ties to the lower expert id
  (page 3: the module docstring of the TP-2 layout and the ``markov_local_argmax``
  docstring both break ties toward the smaller index);
* every output is float32, computed here as the float64 result rounded once;
* 8-bit activations (page 1's ``verify.hpp`` holds the window's T activation columns
  in the q8_1 format for the decode products; the pages name the format but never
  print it): per column and per block
  of 32 consecutive k, ``d = f32(absmax) / 127`` (binary32 division), ``r = 1 / d``
  (binary32 division; 0 when f16(d) is 0), ``q_i = round_half_away(f32(x_i * r))`` clamped
  to [-127, 127], and the stored scale is ``f16_rne(d)``; the product of a weight block
  and an activation block is ``d_w * d_x * sum_i c[q_w,i] * q_i``.  This is the public
  definition of that 8-bit block format; its sum field serves zero-offset formats only
  and is not produced;
* a shared expert (page 3's cooperative decode adds it after the routed sum, weight 1)
  has the routed experts' sizes and the same SwiGLU form.

Parity pins: the test-suite checks each function here against something other than
itself (closed forms, brute force in exact rationals, invariants, hand-written golden
blocks); no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "CODEBOOK", "QK", "BLOCK_BYTES",
    "decode_blocks", "decode_blocks_f16", "encode_blocks",
    "qmv", "route_topk", "gather", "silu", "moe", "gemm",
    "quantize_q8_1", "qmv_q8", "moe_shared", "moe_gate_up",
]

#: The fixed 16-level int8 codebook of the block format (workload definition).
CODEBOOK = (-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113)
#: Weights per block.
QK = 32
#: Bytes per block: a 2-byte fp16 scale plus 32 four-bit indices (page 2, PLE-compact
#: commit message: a 2,560-value row takes 1,440 bytes, so 18 bytes per 32 values).
BLOCK_BYTES = 18


def _as_blocks(blocks) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(blocks, dtype=np.uint8))
    return b.reshape(-1, BLOCK_BYTES)


def _indices(blocks: np.ndarray) -> np.ndarray:
    """The 32 codebook indices of every block, in element order ([nb, 32] int)."""
    qs = blocks[:, 2:18].astype(np.int64)
    q = np.empty((blocks.shape[0], QK), dtype=np.int64)
    q[:, :16] = qs & 0xF        # element i      <- low nibble of byte 2+i
    q[:, 16:] = qs >> 4         # element i + 16 <- high nibble of byte 2+i
    return q


def _scales(blocks: np.ndarray) -> np.ndarray:
    """The fp16 scale of every block as float64 (exact)."""
    return blocks[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)


def decode_blocks(blocks) -> np.ndarray:
    """Decoded weights ``w = d * codebook[q]`` as float32 ``[nb, 32]``.

    The product of an 11-bit fp16 significand and a 7-bit integer is exact in
    float32, so this is the closed form with no rounding.
    """
    b = _as_blocks(blocks)
    cb = np.asarray(CODEBOOK, dtype=np.float64)
    w = _scales(b)[:, None] * cb[_indices(b)]
    return w.astype(np.float32)


def decode_blocks_f16(blocks) -> np.ndarray:
    """Decoded weights rounded to binary16 (round to nearest even, subnormals kept)."""
    return decode_blocks(blocks).astype(np.float16)


_ENCODE_CHUNK = 1 << 15


def encode_blocks(w) -> np.ndarray:
    """Quantise float32 weights ``[nb, 32]`` to 18-byte blocks ``[nb, 18]`` (uint8).

    ``d = f16(f32(max|w|) / 127)``; each element takes the codebook level nearest
    to ``w / d`` (exact comparison, ties to the lower index); ``d == 0`` gives index 8.
    Inputs must be finite with ``max|w| / 127 <= 65504``.
    """
    w32 = np.ascontiguousarray(np.asarray(w, dtype=np.float32)).reshape(-1, QK)
    nb = w32.shape[0]
    if nb > _ENCODE_CHUNK:  # bound the [blocks, 32, 16] distance array; same result
        return np.concatenate([encode_blocks(w32[i:i + _ENCODE_CHUNK])
                               for i in range(0, nb, _ENCODE_CHUNK)])
    amax = np.max(np.abs(w32), axis=1)
    d16 = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    d = d16.astype(np.float64)
    cb = np.asarray(CODEBOOK, dtype=np.float64)
    # |w - c_j d| in float64: c_j d is exact, and wherever two levels are close to a
    # tie both differences are exact too, so argmin (first minimum) is the exact
    # nearest level with ties to the lower index.
    dist = np.abs(w32.astype(np.float64)[:, :, None] - d[:, None, None] * cb[None, None, :])
    q = np.argmin(dist, axis=2)
    q[d == 0.0, :] = 8
    out = np.empty((nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = d16.astype("<f2").view(np.uint8).reshape(nb, 2)
    out[:, 2:18] = (q[:, :16] | (q[:, 16:] << 4)).astype(np.uint8)
    return out


def _matrix(blocks, n: int, k: int) -> np.ndarray:
    """Decoded ``n x k`` weight matrix (rows of k/32 consecutive blocks), float64."""
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    b = _as_blocks(blocks)
    if b.shape[0] != n * (k // QK):
        raise ValueError("block count does not match N x K")
    return decode_blocks(b).astype(np.float64).reshape(n, k)


def qmv(blocks, n: int, k: int, x) -> np.ndarray:
    """T-column quantised matrix-vector product.

    ``Y[t][r] = sum_k W[r][k] * X[t][k]`` for the decoded ``n x k`` matrix W and the
    token-major activations X (``[T, k]``), summed in float64, returned as float32
    ``[T, n]`` -- the multi-column product of page 1's verify window (file header of
    ``verify.hpp``: one read of the dense weights serves all T tokens), each column its
    own single-token product.
    """
    W = _matrix(blocks, n, k)
    X = np.asarray(x, dtype=np.float64).reshape(-1, k)
    return (X @ W.T).astype(np.float32)


def route_topk(logits, top_k: int):
    """Top-k routing: ids of the k largest logits per token (value descending, ties to
    the lower expert id) and their softmax gate weights (over the k selected, float64,
    stored as float32).  Returns ``(ids int32 [n, k], w float32 [n, k])``."""
    L = np.asarray(logits, dtype=np.float32)
    n, E = L.shape
    ids = np.empty((n, top_k), dtype=np.int32)
    w = np.empty((n, top_k), dtype=np.float32)
    for t in range(n):
        # stable sort on -L keeps equal logits in ascending id order
        order = np.argsort(-L[t].astype(np.float64), kind="stable")[:top_k]
        ids[t] = order
        z = L[t, order].astype(np.float64)
        e = np.exp(z - z.max())
        w[t] = (e / e.sum()).astype(np.float32)
    return ids, w


def gather(ids, n_expert: int):
    """Token gather of the routed pairs.

    Pair ``p = t * k + j`` is token t's j-th routed slot.  Returns
    ``counts [E]`` (pairs per expert), ``offsets [E+1]`` (exclusive prefix sum),
    ``pairs [n*k]`` (pair ids grouped by expert, ascending within an expert) and
    ``slot_row [n*k]`` (position of pair p in ``pairs``), all int32 -- the per-expert
    counts / start / token lists of page 1's expert plan block.
    """
    I = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = I.shape[0]
    counts = np.zeros(n_expert, dtype=np.int64)
    for e in I:
        counts[e] += 1
    offsets = np.zeros(n_expert + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    pairs = np.empty(P, dtype=np.int64)
    fill = offsets[:-1].copy()
    for p in range(P):
        e = I[p]
        pairs[fill[e]] = p
        fill[e] += 1
    slot_row = np.empty(P, dtype=np.int64)
    slot_row[pairs] = np.arange(P)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            pairs.astype(np.int32), slot_row.astype(np.int32))


def silu(g: np.ndarray) -> np.ndarray:
    """``g / (1 + exp(-g))`` in float64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def moe(x, ids, w, gate_blocks, up_blocks, down_blocks, hidden: int, inter: int,
        tokens=None, return_pair_rows: bool = False):
    """Mixture-of-experts FFN over the routed pairs.

    For token t and slot j with expert ``e = ids[t][j]``:
    ``g = Wg_e x_t``, ``u = Wu_e x_t``, ``h = silu(g) * u``, ``y_tj = Wd_e h``, and
    ``out[t] = sum_j w[t][j] * y_tj`` added in j order -- page 1's ``PoolMultiFn``
    contract (x (n_tok, n_embd), ids (n_tok, k) -> per-slot rows (n_tok*k, n_embd),
    then summed per token).  Gate/up are ``inter x hidden`` and down ``hidden x inter``
    block matrices per expert (``*_blocks[e]``).  Everything in float64; ``out`` is
    returned as float32 ``[len(tokens), hidden]``.  ``tokens`` restricts the
    computation to a subset of token rows (for sampled checks at full size).
    """
    out, rows = _moe64(x, ids, w, gate_blocks, up_blocks, down_blocks, hidden, inter, tokens)
    if return_pair_rows:
        return out.astype(np.float32), rows
    return out.astype(np.float32)


def moe_gate_up(x, ids, gate_blocks, up_blocks, hidden: int, inter: int):
    """The first products of every routed pair: ``g[p] = Wg_e x_t`` and ``u[p] = Wu_e x_t``
    for pair ``p = t * k + j`` with ``e = ids[t][j]``, summed in float64, returned as
    float64 ``[n_tok * k, inter]`` arrays in pair-id order -- the per-slot layout of page
    1's ``PoolMultiFn`` (x (n_tok, n_embd), ids (n_tok, k) -> (n_tok * k, ...) rows)."""
    X = np.asarray(x).astype(np.float64)
    ids = np.asarray(ids)
    n_tok, k = ids.shape
    flat = ids.reshape(-1)
    g = np.zeros((n_tok * k, inter), dtype=np.float64)
    u = np.zeros((n_tok * k, inter), dtype=np.float64)
    for e in np.unique(flat):
        ps = np.nonzero(flat == e)[0]
        xi = X[ps // k]
        g[ps] = xi @ _matrix(gate_blocks[e], inter, hidden).T
        u[ps] = xi @ _matrix(up_blocks[e], inter, hidden).T
    return g, u


def _expert_ffn(X, gate_b, up_b, down_b, hidden: int, inter: int) -> np.ndarray:
    """One SwiGLU expert on float64 rows X: ``Wd (silu(Wg x) * (Wu x))``."""
    Wg = _matrix(gate_b, inter, hidden)
    Wu = _matrix(up_b, inter, hidden)
    Wd = _matrix(down_b, hidden, inter)
    h = silu(X @ Wg.T) * (X @ Wu.T)
    return h @ Wd.T


def _moe64(x, ids, w, gate_blocks, up_blocks, down_blocks, hidden, inter, tokens):
    """``moe`` in float64: (out [len(tokens), hidden], pair rows [len(tokens), k, hidden])."""
    X = np.asarray(x).astype(np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n_tok, k = ids.shape
    toks = np.arange(n_tok) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), hidden), dtype=np.float64)
    rows = np.zeros((len(toks), k, hidden), dtype=np.float64)
    experts = np.unique(ids[toks])
    for e in experts:
        sel = [(i, j) for i, t in enumerate(toks) for j in range(k) if ids[t, j] == e]
        if not sel:
            continue
        xi = X[[toks[i] for i, _ in sel]]
        y = _expert_ffn(xi, gate_blocks[e], up_blocks[e], down_blocks[e], hidden, inter)
        for r, (i, j) in enumerate(sel):
            rows[i, j] = y[r]
    for j in range(k):
        out += w[toks, j][:, None] * rows[:, j, :]
    return out, rows


def moe_shared(x, ids, w, gate_blocks, up_blocks, down_blocks, shared_gate, shared_up, shared_down,
               hidden: int, inter: int, tokens=None):
    """``moe`` plus a shared expert that every token passes through with weight 1:
    ``out[t] = sum_j w[t][j] * y_tj + ys_t`` with ``ys_t`` the shared expert's SwiGLU FFN
    of ``x_t`` (the same sizes as the routed experts).  Page 3 (the DSpark drafter
    file, its cooperative decode with the shared expert): the shared expert's output is
    added, with weight 1, to the routed sum.  float64, returned as float32."""
    out, _ = _moe64(x, ids, w, gate_blocks, up_blocks, down_blocks, hidden, inter, tokens)
    X = np.asarray(x).astype(np.float64)
    toks = np.arange(X.shape[0]) if tokens is None else np.asarray(tokens)
    ys = _expert_ffn(X[toks], shared_gate, shared_up, shared_down, hidden, inter)
    return (out + ys).astype(np.float32)


def gemm(blocks, n: int, k: int, x) -> np.ndarray:
    """Dense product against the decoded weights: ``Y[m][r] = sum_k X[m][k] W[r][k]``
    (X token-major ``[M, k]``, any float dtype taken exactly), float64 sums,
    float32 ``[M, n]`` result."""
    W = _matrix(blocks, n, k)
    X = np.asarray(x).reshape(-1, k)
    Y = np.empty((X.shape[0], n), dtype=np.float32)
    for i in range(0, X.shape[0], 512):  # rows are independent: bounds the float64 temporaries
        Y[i:i + 512] = (X[i:i + 512].astype(np.float64) @ W.T).astype(np.float32)
    return Y


def _round_half_away(v: np.ndarray) -> np.ndarray:
    """Nearest integer of float32 values, halves away from zero (C ``roundf``), done
    in exact steps: ``v - trunc(v)`` is exact in float32 for |v| < 2^23."""
    v = np.asarray(v, dtype=np.float32)
    t = np.trunc(v)
    frac = np.abs(v - t)
    return t + np.where(frac >= np.float32(0.5), np.sign(v), np.float32(0)).astype(np.float32)


def quantize_q8_1(x):
    """8-bit block quantisation of float32 activations ``x`` ([T, k], k % 32 == 0).

    Per column t and block b of 32 consecutive k: ``d = f32(absmax) / 127`` and
    ``r = 1 / d`` as IEEE binary32 divisions, ``q_i`` the
    nearest integer of the binary32 product ``x_i * r`` (halves away from zero), clamped
    to [-127, 127]; the stored scale is d rounded to binary16, and a block whose stored
    scale is zero gets zero codes (r = 0).  Non-finite x are not defined.  Returns ``q``
    (int8 ``[T, k]``) and ``d`` (float16 ``[T, k/32]``): the activation side of page 1's
    decode products (``verify.hpp`` member declarations).
    """
    X = np.asarray(x, dtype=np.float32)
    T, k = X.reshape(X.shape[0] if X.ndim > 1 else 1, -1).shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    B = X.reshape(T, k // QK, QK)
    amax = np.max(np.abs(B), axis=2)
    d = (amax / np.float32(127)).astype(np.float32)
    d16 = d.astype(np.float16)
    # a block whose stored scale is zero (absmax < 127 * 2^-25) contributes nothing:
    # its codes are zero (this also keeps 1/d finite)
    with np.errstate(divide="ignore"):
        r = np.where(d16 != 0, np.float32(1) / d, np.float32(0)).astype(np.float32)
    v = (B * r[:, :, None]).astype(np.float32)
    q = np.clip(_round_half_away(v), -127, 127).astype(np.int8)
    return q.reshape(T, k), d16


def qmv_q8(blocks, n: int, k: int, q, d) -> np.ndarray:
    """T-column product with 8-bit activations: ``Y[t][r] = sum_b dw[r][b] * dx[t][b] *
    sum_i c[qw[r][32b+i]] * q[t][32b+i]`` (integer block dots, each scaled by the
    product of the two binary16 scales), summed in float64 and rounded once to float32
    (``[T, n]``).  ``q``, ``d`` as :func:`quantize_q8_1` returns them."""
    b = _as_blocks(blocks)
    if k % QK or b.shape[0] != n * (k // QK):
        raise ValueError("block count does not match N x K")
    nb = k // QK
    cb = np.asarray(CODEBOOK, dtype=np.int64)
    lev = cb[_indices(b)].reshape(n, nb, QK)              # integer levels
    dw = _scales(b).reshape(n, nb)                         # float64 (exact)
    Q = np.asarray(q, dtype=np.int64).reshape(-1, nb, QK)
    dx = np.asarray(d, dtype=np.float16).astype(np.float64).reshape(-1, nb)
    dots = np.einsum("rbi,tbi->trb", lev, Q)               # exact integers
    return np.einsum("trb,rb,tb->tr", dots.astype(np.float64), dw, dx).astype(np.float32)
