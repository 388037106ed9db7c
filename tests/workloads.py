"""Seeded workloads for the parity tests: source floats from ``synth``, encoded by the
oracle's encoder (never by the HIP path), cached per process."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth


@functools.lru_cache(maxsize=None)
def dense_weights(seed: int, n: int, k: int, tag: int = synth.TAG_WEIGHT):
    """(source float32 [n, k], oracle-encoded blocks [n*k/32, 18])."""
    w = synth.weights_f32(seed, tag, n, k)
    return w, oracle.encode_blocks(w.reshape(-1, 32))


@functools.lru_cache(maxsize=None)
def xs_weights(seed: int, n: int, k: int):
    """(source float32 [n, k], oracle-encoded IQ4_XS super-blocks [n*k/256, 136])."""
    w = synth.weights_f32(seed, synth.TAG_WEIGHT, n, k)
    return w, oracle.encode_xs(w.reshape(-1, 256))


@functools.lru_cache(maxsize=None)
def acts32(seed: int, t: int, k: int):
    return synth.acts_f32(seed, synth.TAG_X, t, k)


@functools.lru_cache(maxsize=None)
def acts16(seed: int, m: int, k: int):
    return synth.acts_f16(seed, synth.TAG_X, m, k)


def cfg1():
    """Plumbing matvec: W 512 x 2048 (seed 101), one fp32 column."""
    w, b = dense_weights(synth.SEED_PLUMBING, 512, 2048)
    return b, 512, 2048, acts32(synth.SEED_PLUMBING, 1, 2048)


def cfg2(T: int = 4):
    """Verify-window matvec: W 4096 x 4096 (seed 102), T fp32 columns."""
    w, b = dense_weights(synth.SEED_VERIFY, 4096, 4096)
    return b, 4096, 4096, acts32(synth.SEED_VERIFY, 8, 4096)[:T]


def _expert_matrix(seed: int, e: int, which: str, n: int, k: int) -> np.ndarray:
    w = synth.weights_f32(seed, synth.tag_expert(e, which), n, k)
    return oracle.encode_blocks(w.reshape(-1, 32))


@functools.lru_cache(maxsize=None)
def expert_blocks(seed: int, experts: tuple, hidden: int, inter: int):
    """Oracle-encoded blocks of the listed experts of a bank: {e: (gate, up, down)},
    gate/up inter x hidden, down hidden x inter.  Encoded in a thread pool (numpy
    releases the GIL in the heavy loops)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(e, which, inter if which != "down" else hidden, hidden if which != "down" else inter)
            for e in experts for which in ("gate", "up", "down")]
    with ThreadPoolExecutor(max_workers=16) as ex:
        mats = list(ex.map(lambda j: _expert_matrix(seed, *j), jobs))
    return {e: tuple(mats[3 * i:3 * i + 3]) for i, e in enumerate(experts)}
