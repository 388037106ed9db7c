"""Mixture-of-experts path on the GPU vs the oracle: routing, the bit-exact gather, the
fp32 decode path (tolerance 1e-3) and the binary16 prefill path (tolerance 5e-3)."""
import numpy as np
import pytest
import torch

import dequant_matmul_iq4_amd as iq4
import oracle
import synth
from gpu_util import bits_equal, dev, host, normwise, note, pack
from test_oracle_pins import integer_exact_blocks

pytestmark = pytest.mark.gpu


def make_bank(rng, E, H, I, scale=0.02):
    gate = [oracle.encode_blocks((rng.standard_normal((I * H // 32, 32)) * scale).astype(np.float32)) for _ in range(E)]
    up = [oracle.encode_blocks((rng.standard_normal((I * H // 32, 32)) * scale).astype(np.float32)) for _ in range(E)]
    down = [oracle.encode_blocks((rng.standard_normal((H * I // 32, 32)) * scale).astype(np.float32)) for _ in range(E)]
    return gate, up, down


def pack_bank(blocks, n, k):
    return torch.cat([pack(b, n, k) for b in blocks])


def run_moe(x, ids, w, banks, H, I, E, flags=0, dtype="f16"):
    """One call of the MoE layer.  The output and the whole workspace start as NaN bytes
    (0xFF: a NaN in every float field, -1 in every integer one), so a row that no kernel
    writes, or a stale workspace row that a kernel reads, shows up in the comparison."""
    n_tok, top_k = ids.shape
    f16 = dtype == "f16"
    xd = dev(x.astype(np.float16 if f16 else np.float32))
    out = torch.full((n_tok, H), float("nan"), dtype=torch.float32, device="cuda")
    act = iq4.IQ4_F16 if f16 else iq4.IQ4_F32
    wsb = iq4.iq4_moe_workspace_size(n_tok, top_k, E, H, I, act)
    ws = torch.full((max(wsb, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    g, u, d = banks
    iq4.iq4_moe_expert_gemm(xd, act, n_tok, H, dev(ids.astype(np.int32)), dev(w.astype(np.float32)), top_k, E,
                            H, I, g, u, d, out, H, ws, wsb, flags)
    return host(out), ws


def routing(rng, n_tok, E, k):
    logits = rng.standard_normal((n_tok, E)).astype(np.float32)
    return oracle.route_topk(logits, k)


def test_route_topk_matches_oracle():
    note("route: top-8 of 128, ties")
    rng = np.random.default_rng(1)
    L = rng.standard_normal((300, 128)).astype(np.float32)
    L[::7, 5] = L[::7, 9]  # ties
    L[3] = 0.25  # a fully tied row
    ids_r, w_r = oracle.route_topk(L, 8)
    ids = torch.empty((300, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((300, 8), dtype=torch.float32, device="cuda")
    iq4.iq4_route_topk(dev(L), 300, 128, 8, ids, w)
    assert bits_equal(host(ids), ids_r)
    assert np.allclose(host(w), w_r, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("n_tok,k,E", [(3256, 8, 128), (4, 8, 128), (1, 1, 1), (37, 3, 7)])
def test_gather_bit_exact(n_tok, k, E):
    note(f"gather: n_tok={n_tok} k={k} E={E}")
    rng = np.random.default_rng(n_tok + E)
    if E == 128 and n_tok > 100:
        L = synth.logits_zipf_gumbel(synth.SEED_PREFILL, synth.TAG_GUMBEL, n_tok, E)
        ids, _ = oracle.route_topk(L, k)
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(n_tok)]).astype(np.int32)
    P = n_tok * k
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    o = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    p = torch.empty(P, dtype=torch.int32, device="cuda")
    s = torch.empty(P, dtype=torch.int32, device="cuda")
    iq4.iq4_moe_gather(dev(ids), P, E, c, o, p, s)
    rc, ro, rp, rs = oracle.gather(ids, E)
    assert bits_equal(host(c), rc) and bits_equal(host(o), ro)
    assert bits_equal(host(p), rp) and bits_equal(host(s), rs)


@pytest.fixture(scope="module")
def small_bank():
    rng = np.random.default_rng(42)
    E, H, I = 8, 256, 128
    gate, up, down = make_bank(rng, E, H, I)
    banks = (pack_bank(gate, I, H), pack_bank(up, I, H), pack_bank(down, H, I))
    return dict(E=E, H=H, I=I, gate=gate, up=up, down=down, banks=banks)


@pytest.mark.parametrize("n_tok,k", [(300, 2), (129, 3), (5, 8), (1, 1)])
def test_prefill_small(small_bank, n_tok, k):
    note(f"moe prefill: n_tok={n_tok} k={k}")
    B = small_bank
    rng = np.random.default_rng(n_tok * 10 + k)
    ids, w = routing(rng, n_tok, B["E"], k)
    x = rng.standard_normal((n_tok, B["H"])).astype(np.float16)
    got, ws = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"])
    ref = oracle.moe(x, ids, w, B["gate"], B["up"], B["down"], B["H"], B["I"])
    assert normwise(got, ref) <= 5e-3
    # the call leaves the gather at the start of its workspace
    rc, ro, rp, rs = oracle.gather(ids, B["E"])
    wsn = host(ws)
    cnt = wsn[:4 * B["E"]].view(np.int32)
    assert bits_equal(cnt, rc)


@pytest.mark.parametrize("n_tok,k", [(4, 2), (8, 8), (1, 3), (13, 4)])
def test_decode_small(small_bank, n_tok, k):
    note(f"moe decode: n_tok={n_tok} k={k}")
    B = small_bank
    rng = np.random.default_rng(n_tok * 100 + k)
    ids, w = routing(rng, n_tok, B["E"], k)
    x = rng.standard_normal((n_tok, B["H"])).astype(np.float32)
    got, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"], dtype="f32")
    ref = oracle.moe(x, ids, w, B["gate"], B["up"], B["down"], B["H"], B["I"])
    assert normwise(got, ref) <= 1e-3


@pytest.mark.parametrize("H,I,E,n_tok,k", [(512, 1024, 4, 3, 2), (4096, 128, 3, 2, 2), (1280, 1152, 5, 8, 3),
                                           (512, 1024, 16, 8, 12)])
def test_decode_other_shapes(H, I, E, n_tok, k):
    """Decode shapes off the workload's: a down product with K above 7 quads (the grouped
    form, 8 and 9 quads, direct and gathered), a 4,096-wide gate|up (4 quads per wave)
    and a 10-quad gate|up over 5 waves."""
    note(f"moe decode: H={H} I={I} E={E} n_tok={n_tok} k={k}")
    rng = np.random.default_rng(H + I + E + k)
    gate, up, down = make_bank(rng, E, H, I)
    banks = (pack_bank(gate, I, H), pack_bank(up, I, H), pack_bank(down, H, I))
    ids, w = routing(rng, n_tok, E, k)
    x = rng.standard_normal((n_tok, H)).astype(np.float32)
    got, _ = run_moe(x, ids, w, banks, H, I, E, dtype="f32")
    assert normwise(got, oracle.moe(x, ids, w, gate, up, down, H, I)) <= 1e-3
    one, _ = run_moe(x[:1], ids[:1], w[:1], banks, H, I, E, dtype="f32")
    assert bits_equal(got[0], one[0])


def test_decode_batch_invariance(small_bank):
    """Each token of a 4-token decode step equals that token run alone, bitwise (the
    verify window's per-token property, for the expert path)."""
    note("moe decode: batch invariance")
    B = small_bank
    rng = np.random.default_rng(5)
    ids, w = routing(rng, 4, B["E"], 4)
    ids[1] = ids[0]  # two tokens sharing all their experts
    x = rng.standard_normal((4, B["H"])).astype(np.float32)
    full, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"], dtype="f32")
    for t in range(4):
        one, _ = run_moe(x[t:t + 1], ids[t:t + 1], w[t:t + 1], B["banks"], B["H"], B["I"], B["E"], dtype="f32")
        assert bits_equal(full[t], one[0]), t


def test_decode_direct_and_gathered_paths_agree():
    """A decode call with at most 64 routed pairs finds each expert's pairs from the ids
    inside its matvecs; above 64 it runs the gather first.  Both give the oracle's result
    within the fp32 tolerance, and each token's row is bitwise the same on either path
    (8 tokens x top-12 = 96 pairs, gathered; the same tokens 5 + 3 at a time, direct)."""
    note("moe decode: direct (<= 64 pairs) vs gathered (> 64 pairs)")
    rng = np.random.default_rng(77)
    E, H, I, k = 16, 256, 128, 12
    gate, up, down = make_bank(rng, E, H, I)
    banks = (pack_bank(gate, I, H), pack_bank(up, I, H), pack_bank(down, H, I))
    ids, w = routing(rng, 8, E, k)
    ids[3] = ids[2]  # two tokens on the same experts
    x = rng.standard_normal((8, H)).astype(np.float32)
    full, _ = run_moe(x, ids, w, banks, H, I, E, dtype="f32")
    ref = oracle.moe(x, ids, w, gate, up, down, H, I)
    assert normwise(full, ref) <= 1e-3
    for lo, hi in [(0, 5), (5, 8)]:
        part, _ = run_moe(x[lo:hi], ids[lo:hi], w[lo:hi], banks, H, I, E, dtype="f32")
        assert bits_equal(full[lo:hi], part), (lo, hi)
    # exactly 64 pairs (direct), every expert present
    ids64 = np.stack([rng.permutation(E) for _ in range(4)]).astype(np.int32)
    w64 = rng.random((4, E)).astype(np.float32)
    x64 = rng.standard_normal((4, H)).astype(np.float32)
    got, _ = run_moe(x64, ids64, w64, banks, H, I, E, dtype="f32")
    assert normwise(got, oracle.moe(x64, ids64, w64, gate, up, down, H, I)) <= 1e-3


def run_moe_shared(x, ids, w, banks, shared, H, I, E, dtype="f16", flags=0):
    n_tok, top_k = ids.shape
    f16 = dtype == "f16"
    xd = dev(x.astype(np.float16 if f16 else np.float32))
    out = torch.full((n_tok, H), float("nan"), dtype=torch.float32, device="cuda")
    act = iq4.IQ4_F16 if f16 else iq4.IQ4_F32
    wsb = iq4.iq4_moe_shared_workspace_size(n_tok, top_k, E, H, I, act)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    g, u, d = banks
    sg, su, sd = shared
    iq4.iq4_moe_expert_gemm_shared(xd, act, n_tok, H, dev(ids.astype(np.int32)), dev(w.astype(np.float32)), top_k,
                                   E, H, I, g, u, d, sg, su, sd, out, H, ws, wsb, flags)
    return host(out)


@pytest.mark.parametrize("dtype,n_tok,k", [("f32", 4, 3), ("f32", 8, 8), ("f16", 300, 2), ("f16", 5, 8)])
def test_shared_expert(small_bank, dtype, n_tok, k):
    """A shared expert added after the routed sum: against the oracle, and bitwise equal
    to the routed call on the bank extended by the shared expert, with it appended to
    every token's routing at weight 1 (decode: 16 pairs direct, 72 pairs gathered)."""
    note(f"moe shared expert: {dtype} n_tok={n_tok} k={k}")
    B = small_bank
    E, H, I = B["E"], B["H"], B["I"]
    rng = np.random.default_rng(900 + n_tok * 10 + k)
    sgate, sup, sdown = make_bank(rng, 1, H, I)
    shared = (pack(sgate[0], I, H), pack(sup[0], I, H), pack(sdown[0], H, I))
    ids, w = routing(rng, n_tok, E, k)
    x = rng.standard_normal((n_tok, H)).astype(np.float16 if dtype == "f16" else np.float32)
    got = run_moe_shared(x, ids, w, B["banks"], shared, H, I, E, dtype=dtype)
    ref = oracle.moe_shared(x, ids, w, B["gate"], B["up"], B["down"], sgate[0], sup[0], sdown[0], H, I)
    assert normwise(got, ref) <= (5e-3 if dtype == "f16" else 1e-3)
    ext = (pack_bank(B["gate"] + sgate, I, H), pack_bank(B["up"] + sup, I, H), pack_bank(B["down"] + sdown, H, I))
    ids2 = np.concatenate([ids, np.full((n_tok, 1), E, np.int32)], axis=1)
    w2 = np.concatenate([w, np.ones((n_tok, 1), np.float32)], axis=1)
    same, _ = run_moe(x, ids2, w2, ext, H, I, E + 1, dtype=dtype)
    assert bits_equal(got, same)


def test_shared_expert_atomic_combine(small_bank):
    """The shared expert with the atomic combine (prefill): within the f16 tolerance."""
    note("moe shared expert: atomic combine")
    B = small_bank
    E, H, I = B["E"], B["H"], B["I"]
    rng = np.random.default_rng(31)
    sgate, sup, sdown = make_bank(rng, 1, H, I)
    shared = (pack(sgate[0], I, H), pack(sup[0], I, H), pack(sdown[0], H, I))
    ids, w = routing(rng, 200, E, 3)
    x = rng.standard_normal((200, H)).astype(np.float16)
    got = run_moe_shared(x, ids, w, B["banks"], shared, H, I, E, flags=iq4.IQ4_MOE_ATOMIC_COMBINE)
    ref = oracle.moe_shared(x, ids, w, B["gate"], B["up"], B["down"], sgate[0], sup[0], sdown[0], H, I)
    assert normwise(got, ref) <= 5e-3


def test_prefill_batch_invariance(small_bank):
    note("moe prefill: batch invariance")
    B = small_bank
    rng = np.random.default_rng(6)
    ids, w = routing(rng, 200, B["E"], 2)
    x = rng.standard_normal((200, B["H"])).astype(np.float16)
    full, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"])
    sub = [0, 77, 199]
    part, _ = run_moe(x[sub], ids[sub], w[sub], B["banks"], B["H"], B["I"], B["E"])
    assert bits_equal(full[sub], part)


def test_prefill_atomic_combine(small_bank):
    """The atomic combine adds the fp32 slot rows r_j; the ordered combine adds them
    rounded to binary16.  Elementwise the two differ by at most that rounding, 2^-11 |r_j|
    per row (2^-25 where r_j is subnormal), plus the two fp32 summations' rounding, at
    most 2 (k - 1) 2^-24 sum_j |r_j|.  The kept binary16 rows give sum_j |r_j| to within
    a factor 1 + 2^-11.  Both results are within the f16 tolerance of the oracle."""
    note("moe prefill: atomic combine")
    B = small_bank
    rng = np.random.default_rng(8)
    n_tok, k = 150, 3
    ids, w = routing(rng, n_tok, B["E"], k)
    x = rng.standard_normal((n_tok, B["H"])).astype(np.float16)
    det, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"])
    atom, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"], flags=iq4.IQ4_MOE_ATOMIC_COMBINE)
    kept_out, r = run_moe_keep(x, ids, w, B["banks"], B["H"], B["I"], B["E"])
    assert bits_equal(kept_out, det)
    row_abs = np.abs(r["rows"].astype(np.float64)).reshape(n_tok, k, B["H"]).sum(axis=1) * (1 + 2.0 ** -11)
    bound = 2.0 ** -11 * row_abs + 2 * (k - 1) * 2.0 ** -24 * row_abs + k * 2.0 ** -25
    assert np.all(np.abs(atom.astype(np.float64) - det) <= bound)
    ref = oracle.moe(x, ids, w, B["gate"], B["up"], B["down"], B["H"], B["I"])
    assert normwise(atom, ref) <= 5e-3 and normwise(det, ref) <= 5e-3


def test_prefill_deterministic(small_bank):
    note("moe prefill: run-to-run determinism")
    B = small_bank
    rng = np.random.default_rng(9)
    ids, w = routing(rng, 300, B["E"], 2)
    x = rng.standard_normal((300, B["H"])).astype(np.float16)
    a, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"])
    b, _ = run_moe(x, ids, w, B["banks"], B["H"], B["I"], B["E"])
    assert bits_equal(a, b)


# ---- full-size workloads: the 128-expert bank (hidden 2048, inter 768, seed 103) ----------

H_FULL, I_FULL, E_FULL, K_FULL = 2048, 768, 128, 8


@pytest.fixture(scope="module")
def full_bank():
    """Every expert of the bank encoded by the oracle, and the same bank packed on the
    GPU (expert-major), as the benchmark lays it out."""
    import workloads
    blocks = workloads.expert_blocks(synth.SEED_EXPERTS, tuple(range(E_FULL)), H_FULL, I_FULL)
    gate = {e: b[0] for e, b in blocks.items()}
    up = {e: b[1] for e, b in blocks.items()}
    down = {e: b[2] for e, b in blocks.items()}
    banks = (pack_bank([gate[e] for e in range(E_FULL)], I_FULL, H_FULL),
             pack_bank([up[e] for e in range(E_FULL)], I_FULL, H_FULL),
             pack_bank([down[e] for e in range(E_FULL)], H_FULL, I_FULL))
    return dict(gate=gate, up=up, down=down, banks=banks)


def test_decode_step_full_size(full_bank):
    """The decode step at its real shape: 4 fp32 tokens, top-8 of 128 experts with softmax
    gate weights from N(0,1) logits; every output against the oracle (1e-3), and the
    on-device router bit-exact against the oracle's."""
    note("moe decode full size: 4 tokens, top-8 of 128, hidden 2048, inter 768")
    logits = synth.logits_normal(synth.SEED_DECODE, synth.TAG_LOGITS, 4, E_FULL)
    ids, w = oracle.route_topk(logits, K_FULL)
    ids_d = torch.empty((4, K_FULL), dtype=torch.int32, device="cuda")
    w_d = torch.empty((4, K_FULL), dtype=torch.float32, device="cuda")
    iq4.iq4_route_topk(dev(logits), 4, E_FULL, K_FULL, ids_d, w_d)
    assert bits_equal(host(ids_d), ids.astype(np.int32))
    x = synth.acts_f32(synth.SEED_DECODE, synth.TAG_X, 4, H_FULL)
    B = full_bank
    got, _ = run_moe(x, ids, w, B["banks"], H_FULL, I_FULL, E_FULL, dtype="f32")
    ref = oracle.moe(x, ids, w, B["gate"], B["up"], B["down"], H_FULL, I_FULL)
    err = normwise(got, ref)
    note(f"  unique experts {len(np.unique(ids))}, normwise {err:.2e}")
    assert err <= 1e-3


def test_prefill_layer_full_size(full_bank):
    """The prefill layer at its real shape and launch configuration: 3,256 f16 tokens with
    Zipf(1.1)-skewed top-8 routing (experts of 27 to about 2,950 rows, so the grouped
    GEMM's tile list, its partial tiles and its XCD order are all at their real sizes).
    Every one of the 3,256 x 2,048 outputs against the oracle (5e-3), with the output and
    the workspace NaN-filled before the call."""
    import time
    n_tok = 3256
    note("moe prefill full size: 3256 tokens, Zipf 1.1, top-8 of 128, every output")
    logits = synth.logits_zipf_gumbel(synth.SEED_PREFILL, synth.TAG_GUMBEL, n_tok, E_FULL)
    ids, w = oracle.route_topk(logits, K_FULL)
    x = synth.acts_f16(synth.SEED_PREFILL, synth.TAG_X, n_tok, H_FULL)
    B = full_bank
    got, _ = run_moe(x, ids, w, B["banks"], H_FULL, I_FULL, E_FULL, dtype="f16")
    t0 = time.perf_counter()
    ref = oracle.moe(x, ids, w, B["gate"], B["up"], B["down"], H_FULL, I_FULL)
    note(f"  oracle {time.perf_counter() - t0:.1f} s")
    assert np.isfinite(got).all()
    err = normwise(got, ref)
    worst = np.max(np.abs(got.astype(np.float64) - ref), axis=1) / np.max(np.abs(ref))
    note(f"  normwise {err:.2e}; worst token {int(np.argmax(worst))}")
    assert err <= 5e-3


def test_prefill_three_quad_shapes():
    """A prefill bank whose products span several K quads at shapes off the workload's:
    hidden 1,280 (10 quads in gate|up, not a multiple of 256 rows in down's output tile
    walk) and inter 1,152 (9 quads in down); every output against the oracle."""
    note("moe prefill: H=1280 I=1152 E=6 n_tok=260 k=3, every output")
    rng = np.random.default_rng(1280)
    E, H, I = 6, 1280, 1152
    gate, up, down = make_bank(rng, E, H, I)
    banks = (pack_bank(gate, I, H), pack_bank(up, I, H), pack_bank(down, H, I))
    ids, w = routing(rng, 260, E, 3)
    x = rng.standard_normal((260, H)).astype(np.float16)
    got, _ = run_moe(x, ids, w, banks, H, I, E)
    assert normwise(got, oracle.moe(x, ids, w, gate, up, down, H, I)) <= 5e-3


# ---- the kept intermediates (IQ4_MOE_KEEP_INTERMEDIATE) ------------------------------------

def run_moe_keep(x, ids, w, banks, H, I, E, dtype="f16"):
    """A call with the intermediates kept: (out, {g, u, h, rows, pairs, counts, offsets}),
    read back from the offsets iq4_moe_intermediate_layout gives; the workspace starts as
    0xFF bytes."""
    n_tok, top_k = ids.shape
    f16 = dtype == "f16"
    act = iq4.IQ4_F16 if f16 else iq4.IQ4_F32
    L = iq4.iq4_moe_intermediate_layout(n_tok, top_k, E, H, I, act)
    assert L["total"] > iq4.iq4_moe_workspace_size(n_tok, top_k, E, H, I, act)
    ws = torch.full((L["total"],), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((n_tok, H), float("nan"), dtype=torch.float32, device="cuda")
    g_, u_, d_ = banks
    iq4.iq4_moe_expert_gemm(dev(x.astype(np.float16 if f16 else np.float32)), act, n_tok, H,
                            dev(ids.astype(np.int32)), dev(w.astype(np.float32)), top_k, E, H, I, g_, u_, d_, out,
                            H, ws, L["total"], iq4.IQ4_MOE_KEEP_INTERMEDIATE)
    P = n_tok * top_k
    # a view of each region on the device, copied back one at a time
    def region(name, count, dtype, shape):
        nbytes = count * np.dtype(dtype).itemsize
        return host(ws[L[name]:L[name] + nbytes]).view(dtype).reshape(shape)
    r = {"pairs": region("pairs", P, np.int32, (P,)), "counts": region("counts", E, np.int32, (E,)),
         "offsets": region("offsets", E + 1, np.int32, (E + 1,)),
         "g": region("g", P * I, np.float32, (P, I)), "u": region("u", P * I, np.float32, (P, I)),
         "h": region("h", P * I, np.float16 if f16 else np.float32, (P, I)),
         "rows": region("rows", P * H, np.float16 if f16 else np.float32, (P, H))}
    return host(out), r


def integer_exact_bank(rng, E, H, I, s):
    return ([integer_exact_blocks(rng, I * H // 32, s) for _ in range(E)],
            [integer_exact_blocks(rng, I * H // 32, s) for _ in range(E)],
            [integer_exact_blocks(rng, H * I // 32, s) for _ in range(E)])


def check_kept(x, ids, w, blocks, H, I, E, out, r, dtype):
    gate, up, down = blocks
    P = ids.size
    rc, ro, rp, _ = oracle.gather(ids, E)
    assert bits_equal(r["pairs"], rp) and bits_equal(r["counts"], rc) and bits_equal(r["offsets"], ro)
    # power-of-two scales and small-integer activations: g and u are exact, so bitwise
    g, u = oracle.moe_gate_up(x, ids, gate, up, H, I)
    assert bits_equal(r["g"], g[rp].astype(np.float32)), "g"
    assert bits_equal(r["u"], u[rp].astype(np.float32)), "u"
    h = oracle.silu(g) * u
    assert normwise(r["h"].astype(np.float64), h[rp]) <= (5e-3 if dtype == "f16" else 1e-3)
    ref_out, y = oracle.moe(x, ids, w, gate, up, down, H, I, return_pair_rows=True)
    rows_ref = (np.asarray(w, dtype=np.float64)[:, :, None] * y).reshape(P, H)
    assert normwise(r["rows"].astype(np.float64), rows_ref) <= (5e-3 if dtype == "f16" else 1e-3)
    assert normwise(out, ref_out) <= (5e-3 if dtype == "f16" else 1e-3)
    # the output is the kept rows (binary16 for the prefill, widened exactly) added in
    # fp32 in slot order, bit for bit
    rows = r["rows"].astype(np.float32).reshape(ids.shape[0], ids.shape[1], H)
    acc = rows[:, 0].copy()
    for j in range(1, ids.shape[1]):
        acc = (acc + rows[:, j]).astype(np.float32)
    assert bits_equal(out, acc), "combine"


def test_keep_intermediate_prefill_full_size_integer_exact():
    """The prefill layer at its real shape (3,256 tokens, Zipf(1.1) top-8 of 128 experts,
    hidden 2048, inter 768) on power-of-two-scale weights and small-integer f16
    activations: the kept gate and up products equal the oracle's bitwise (every partial
    sum is exact whatever the order), h, the per-slot rows and the output match within
    the f16 tolerance, and keeping the intermediates leaves the output bitwise unchanged."""
    n_tok, E, H, I, k = 3256, E_FULL, H_FULL, I_FULL, K_FULL
    note("moe keep intermediates: prefill full size, integer-exact")
    rng = np.random.default_rng(104)
    blocks = integer_exact_bank(rng, E, H, I, 10)
    banks = (pack_bank(blocks[0], I, H), pack_bank(blocks[1], I, H), pack_bank(blocks[2], H, I))
    logits = synth.logits_zipf_gumbel(synth.SEED_PREFILL, synth.TAG_GUMBEL, n_tok, E)
    ids, w = oracle.route_topk(logits, k)
    x = rng.integers(-8, 9, (n_tok, H)).astype(np.float16)
    out, r = run_moe_keep(x, ids, w, banks, H, I, E)
    plain, _ = run_moe(x, ids, w, banks, H, I, E)
    assert bits_equal(out, plain)
    check_kept(x, ids, w, blocks, H, I, E, out, r, "f16")


def test_keep_intermediate_decode_integer_exact():
    """The fp32 decode path with the intermediates kept (the gather then always runs):
    g and u bitwise, the rest within the fp32 tolerance, the output bitwise the plain
    (gather-free) call's."""
    note("moe keep intermediates: decode, integer-exact")
    rng = np.random.default_rng(31)
    E, H, I, n_tok, k = 8, 256, 128, 4, 3
    blocks = integer_exact_bank(rng, E, H, I, 8)
    banks = (pack_bank(blocks[0], I, H), pack_bank(blocks[1], I, H), pack_bank(blocks[2], H, I))
    ids, w = routing(rng, n_tok, E, k)
    x = rng.integers(-8, 9, (n_tok, H)).astype(np.float32)
    out, r = run_moe_keep(x, ids, w, banks, H, I, E, dtype="f32")
    plain, _ = run_moe(x, ids, w, banks, H, I, E, dtype="f32")
    assert bits_equal(out, plain)
    check_kept(x, ids, w, blocks, H, I, E, out, r, "f32")
