"""Pins for the CPU oracle, checked against things other than the oracle itself.

Runs on the CPU only.  Each test names what fixes the expected value: a
hand-worked example, a library routine (numpy's stable argsort, torch's
tanh-GELU, numpy matmul), a closed form, an invariant, or a brute-force dense
recomputation that routes nothing.
"""
import math
import os

import numpy as np
import pytest
import torch

import moe_synth as ms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------- helpers
def unpack_codes(P: np.ndarray) -> np.ndarray:
    """Independent nibble unpack: view the little-endian words as bytes; byte i
    of a word holds codes 2i (low nibble) and 2i+1 (high nibble)."""
    b = np.ascontiguousarray(P).view(np.uint8)
    lo = b & 0x0F
    hi = b >> 4
    q = np.stack([lo, hi], axis=-1).reshape(*P.shape[:-1], P.shape[-1] * 8)
    return q.astype(np.float64)


def unpack_bytes(P: np.ndarray) -> np.ndarray:
    """8-bit codes: the words' bytes in memory order (little-endian: low byte
    first), through numpy's byte view rather than shifts."""
    b = np.ascontiguousarray(P).astype("<u4").view(np.uint8)
    return b.reshape(*P.shape[:-1], P.shape[-1] * 4).astype(np.float64)


def dense_weights(P, S, B, gs, bits=4):
    q = unpack_codes(P) if bits == 4 else unpack_bytes(P)
    s = np.repeat(ms.bf16_bits_to_f32(S).astype(np.float64), gs, axis=-1)
    b = np.repeat(ms.bf16_bits_to_f32(B).astype(np.float64), gs, axis=-1)
    return s * q + b


def torch_gelu_tanh(v: np.ndarray) -> np.ndarray:
    return torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()


def torch_silu(v: np.ndarray) -> np.ndarray:
    return torch.nn.functional.silu(torch.from_numpy(v)).numpy()


def brute_force_out(p, act="gelu") -> np.ndarray:
    """Dense, unrouted recomputation: every token through every expert, then
    out[t] = sum_e C[t, e] * FFN_e(x_t) with C[t, e] = sum_j [ids[t,j] == e] w[t,j]."""
    x = ms.bf16_bits_to_f32(p.x).astype(np.float64)
    Wgu = dense_weights(p.w_gateup, p.s_gateup, p.b_gateup, p.gs, p.bits)
    Wd = dense_weights(p.w_down, p.s_down, p.b_down, p.gs, p.bits)
    C = np.zeros((p.T, p.E))
    for j in range(p.k):
        valid = (p.topk_ids[:, j] >= 0) & (p.topk_ids[:, j] < p.E)
        t = np.nonzero(valid)[0]
        np.add.at(C, (t, p.topk_ids[t, j]), p.topk_weights[t, j].astype(np.float64))
    out = np.zeros((p.T, p.H))
    for e in range(p.E):
        gu = x @ Wgu[e].T
        gate = gu[:, : p.I]
        hid = (torch_gelu_tanh(gate) if act == "gelu" else torch_silu(gate)) * gu[:, p.I:]
        out += C[:, e: e + 1] * (hid @ Wd[e].T)
    return out


def rel_err(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def read_worked_example():
    d = {"tile": []}
    with open(os.path.join(GOLDEN, "route_worked_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, val = [s.strip() for s in line.split("=")]
            vals = [int(v) for v in val.split()]
            if key == "tile":
                d["tile"].append(vals)
            else:
                d[key] = np.array(vals, np.int32)
    d["tile"] = np.array(d["tile"], np.int32)
    return d


# ----------------------------------------------------------------- route
def test_route_worked_example(oracle_lib):
    ex = read_worked_example()
    counts, offsets, perm, inv, bad = oracle_lib.route(ex["ids"], 4)
    assert bad == 0
    np.testing.assert_array_equal(counts, ex["counts"])
    np.testing.assert_array_equal(offsets, ex["offsets"])
    np.testing.assert_array_equal(perm, ex["perm"])
    np.testing.assert_array_equal(inv, ex["inv_perm"])
    tiles = oracle_lib.tiles(counts, offsets, bm_big=2, bm_small=1)
    np.testing.assert_array_equal(tiles, ex["tile"])


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_stable_argsort(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([1, 3, 8, 128]))
    A = int(rng.integers(0, 3000))
    ids = rng.integers(-2, E + 2, size=A).astype(np.int32)
    if seed % 2 == 0:
        ids = np.clip(ids, 0, E - 1).astype(np.int32)
    counts, offsets, perm, inv, bad = oracle_lib.route(ids, E)
    valid = (ids >= 0) & (ids < E)
    key = np.where(valid, ids, E)
    np.testing.assert_array_equal(perm, np.argsort(key, kind="stable"))
    np.testing.assert_array_equal(counts, np.bincount(ids[valid], minlength=E))
    assert bad == int((~valid).sum())
    assert offsets[0] == 0 and offsets[E] == A - bad
    np.testing.assert_array_equal(np.diff(offsets), counts)
    # bijection and inverse
    np.testing.assert_array_equal(np.sort(perm), np.arange(A))
    np.testing.assert_array_equal(inv[perm], np.arange(A))
    # sortedness as the PR #4 review defines it: adjacent pairs non-decreasing
    sorted_ids = key[perm]
    assert np.all(sorted_ids[1:] >= sorted_ids[:-1])
    # stable: within one expert, ascending flat index
    same = sorted_ids[1:] == sorted_ids[:-1]
    assert np.all(perm[1:][same] > perm[:-1][same])


@pytest.mark.parametrize("bm_big,bm_small", [(32, 16), (64, 16), (16, 16), (128, 32)])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill8k", "prefill16k"])
def test_tiles_invariants(oracle_lib, name, bm_big, bm_small):
    c = ms.CONFIGS[name]
    rng = np.random.default_rng(0)
    p_logits = ms._router_logits(rng, c["router"], c["T"], c["E"])
    ids, _ = ms.route_topk(p_logits, c["k"])
    counts, offsets, perm, inv, bad = oracle_lib.route(ids, c["E"])
    tiles = oracle_lib.tiles(counts, offsets, bm_big, bm_small)
    A = ids.size
    assert len(tiles) == int(np.sum((counts + bm_big - 1) // bm_big))
    assert len(tiles) <= A // bm_big + min(c["E"], A)
    # disjoint, in-order cover of [0, A)
    assert tiles[0, 1] == 0
    np.testing.assert_array_equal(tiles[1:, 1], tiles[:-1, 1] + tiles[:-1, 2])
    assert tiles[-1, 1] + tiles[-1, 2] == A
    assert np.all(tiles[:, 2] >= 1) and np.all(tiles[:, 2] <= bm_big)
    np.testing.assert_array_equal(tiles[:, 3] == bm_small, tiles[:, 2] <= bm_small)
    assert set(np.unique(tiles[:, 3])) <= {bm_small, bm_big}
    # expert-major; every row of a tile belongs to its expert; only the last
    # tile of an expert may be short
    assert np.all(np.diff(tiles[:, 0]) >= 0)
    for e, rb, rc, _ in tiles:
        assert np.all(ids.ravel()[perm[rb: rb + rc]] == e)
    last_of_expert = np.r_[tiles[1:, 0] != tiles[:-1, 0], True]
    assert np.all(tiles[~last_of_expert, 2] == bm_big)


def test_route_empty_and_all_invalid(oracle_lib):
    counts, offsets, perm, inv, bad = oracle_lib.route(np.zeros(0, np.int32), 5)
    assert perm.size == 0 and bad == 0 and np.all(offsets == 0)
    assert oracle_lib.tiles(counts, offsets).shape == (0, 4)
    ids = np.array([7, -1, 5, 9], np.int32)
    counts, offsets, perm, inv, bad = oracle_lib.route(ids, 5)
    assert bad == 4 and offsets[-1] == 0
    np.testing.assert_array_equal(perm, [0, 1, 2, 3])


# --------------------------------------------------------------- dequant
def test_unit_scale_gives_codes(oracle_lib):
    rng = np.random.default_rng(1)
    E, R, K, gs = 2, 3, 128, 64
    P = rng.integers(0, 2**32, size=(E, R, K // 8), dtype=np.uint32)
    S = np.full((E, R, K // gs), 0x3F80, np.uint16)   # bf16 1.0
    B = np.zeros((E, R, K // gs), np.uint16)
    q = unpack_codes(P)
    for e in range(E):
        for n in range(R):
            for c in range(0, K, 5):
                assert oracle_lib.weight(P, S, B, gs, e, n, c) == q[e, n, c]


def test_group_indexing(oracle_lib):
    """Scale g+1 and bias -(g+1)/2 on group g: fixes which group a column uses."""
    rng = np.random.default_rng(2)
    E, R, K, gs = 1, 2, 256, 64
    P = rng.integers(0, 2**32, size=(E, R, K // 8), dtype=np.uint32)
    g = np.arange(K // gs, dtype=np.float32)
    S = np.broadcast_to(ms.f32_to_bf16_bits(g + 1), (E, R, K // gs)).copy()
    B = np.broadcast_to(ms.f32_to_bf16_bits(-(g + 1) / 2), (E, R, K // gs)).copy()
    q = unpack_codes(P)
    for n in range(R):
        for c in range(K):
            want = (c // gs + 1) * q[0, n, c] - (c // gs + 1) / 2
            assert oracle_lib.weight(P, S, B, gs, 0, n, c) == want


def test_dequant_matches_independent_unpack(oracle_lib):
    p = ms.make_problem(E=3, H=128, I=64, T=1, k=1, seed=3)
    W = dense_weights(p.w_gateup, p.s_gateup, p.b_gateup, p.gs)
    rng = np.random.default_rng(4)
    for _ in range(200):
        e, n, c = rng.integers(0, 3), rng.integers(0, 128), rng.integers(0, 128)
        assert oracle_lib.weight(p.w_gateup, p.s_gateup, p.b_gateup, p.gs, e, n, c) == W[e, n, c]


def test_8bit_byte_order(oracle_lib):
    """Hand-made words: 8-bit code c sits in byte c % 4 of word c / 4, low
    byte first; scale 1 and bias 0 give the code itself."""
    P = np.array([[[0x04030201, 0xFF00807F]]], np.uint32)
    S = np.full((1, 1, 1), 0x3F80, np.uint16)   # bf16 1.0
    B = np.zeros((1, 1, 1), np.uint16)
    want = [1, 2, 3, 4, 0x7F, 0x80, 0x00, 0xFF]
    got = [oracle_lib.weight(P, S, B, 8, 0, 0, c, bits=8) for c in range(8)]
    assert got == want


@pytest.mark.parametrize("gs,shape", [(64, (3, 128, 64, 6, 2)), (32, (2, 96, 64, 4, 2)),
                                      (128, (3, 256, 128, 5, 2))])
def test_8bit_matches_brute_force(oracle_lib, gs, shape):
    E, H, I, T, k = shape
    p = ms.make_problem(E, H, I, T, k, seed=gs + T + 1, gs=gs, bits=8)
    assert p.w_gateup.shape[-1] == H // 4 and p.w_down.shape[-1] == I // 4
    r = oracle_lib.ffn_tokens(p)
    ref = brute_force_out(p)
    assert rel_err(r["out"], ref) < 1e-12
    # the generator's 8-bit weights keep the 4-bit spread
    W = dense_weights(p.w_gateup, p.s_gateup, p.b_gateup, gs, 8)
    W4 = dense_weights(*[getattr(ms.make_problem(E, H, I, T, k, seed=1, gs=gs), f)
                         for f in ("w_gateup", "s_gateup", "b_gateup")], gs)
    assert 0.5 < W.std() / W4.std() < 2


def test_8bit_symmetric_code_gives_zero_output(oracle_lib):
    """q = 128 everywhere with B = -128 S dequantises to exactly zero."""
    p = ms.make_problem(E=4, H=128, I=64, T=6, k=2, seed=5, bits=8)
    p.w_gateup[:] = 0x80808080
    r = oracle_lib.ffn_tokens(p)
    assert np.all(r["h"] == 0) and np.all(r["out"] == 0)


def test_symmetric_code_gives_zero_output(oracle_lib):
    """q = 8 everywhere with B = -8 S dequantises to exactly zero."""
    p = ms.make_problem(E=4, H=128, I=64, T=6, k=2, seed=5)
    p.w_gateup[:] = 0x88888888
    r = oracle_lib.ffn_tokens(p)
    assert np.all(r["h"] == 0) and np.all(r["out"] == 0)


# ------------------------------------------------------------------ GELU
def test_gelu_closed_forms(oracle_lib):
    assert oracle_lib.gelu_tanh(0.0) == 0.0
    for v in np.linspace(-6, 6, 97):
        # odd identity of x * Phi-like gates: gelu(x) - gelu(-x) = x
        assert abs(oracle_lib.gelu_tanh(v) - oracle_lib.gelu_tanh(-v) - v) <= 4e-15 * max(1, abs(v))
    assert oracle_lib.gelu_tanh(30.0) == 30.0
    assert oracle_lib.gelu_tanh(-30.0) == 0.0


def test_gelu_matches_torch_tanh_approximation(oracle_lib):
    v = np.linspace(-8, 8, 1001)
    ref = torch_gelu_tanh(v)
    got = np.array([oracle_lib.gelu_tanh(t) for t in v])
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)
    # and it is the tanh form, not erf: the two differ by at most ~4.7e-4
    erf = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in v])
    d = np.abs(got - erf).max()
    assert 3e-4 < d < 5e-4


# ------------------------------------------------------------------- SiLU
def test_silu_closed_forms(oracle_lib):
    assert oracle_lib.silu(0.0) == 0.0
    for v in np.linspace(-6, 6, 97):
        # v sigmoid(v) - (-v) sigmoid(-v) = v (sigmoid(v) + sigmoid(-v)) = v
        assert abs(oracle_lib.silu(v) - oracle_lib.silu(-v) - v) <= 4e-15 * max(1, abs(v))
    assert oracle_lib.silu(50.0) == 50.0
    assert abs(oracle_lib.silu(-50.0)) < 1e-19
    # the slope at 0 is sigmoid(0) = 1/2
    assert abs(oracle_lib.silu(1e-8) / 1e-8 - 0.5) < 1e-8


def test_silu_matches_torch(oracle_lib):
    v = np.linspace(-12, 12, 1001)
    got = np.array([oracle_lib.silu(t) for t in v])
    np.testing.assert_allclose(got, torch_silu(v), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("seed", [0, 3])
def test_swiglu_matches_brute_force(oracle_lib, seed):
    p = ms.make_config("tiny", seed=seed)
    r = oracle_lib.ffn_tokens(p, act="silu")
    ref = brute_force_out(p, act="silu")
    assert rel_err(r["out"], ref) < 1e-12
    # and it is not the GeGLU result
    assert rel_err(r["out"], brute_force_out(p)) > 1e-2


# ------------------------------------------------------------------- FFN
def test_single_expert_is_dense_ffn(oracle_lib):
    """E = 1, k = 1: the routed FFN reduces to a dense quantised FFN."""
    p = ms.make_problem(E=1, H=192, I=128, T=5, k=1, seed=6)
    x = ms.bf16_bits_to_f32(p.x).astype(np.float64)
    Wgu = dense_weights(p.w_gateup, p.s_gateup, p.b_gateup, p.gs)[0]
    Wd = dense_weights(p.w_down, p.s_down, p.b_down, p.gs)[0]
    gate = x @ Wgu[: p.I].T
    up = x @ Wgu[p.I:].T
    h = torch_gelu_tanh(gate) * up
    y = h @ Wd.T
    r = oracle_lib.ffn_tokens(p)
    assert rel_err(r["h"], h) < 1e-12
    assert rel_err(r["y"], y) < 1e-12
    np.testing.assert_allclose(r["out"], y * p.topk_weights[:, :1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_config_matches_brute_force(oracle_lib, seed):
    p = ms.make_config("tiny", seed=seed)
    r = oracle_lib.ffn_tokens(p)
    ref = brute_force_out(p)
    assert rel_err(r["out"], ref) < 1e-12
    assert np.abs(r["out"] - ref).max() < 1e-10 * np.sqrt((ref ** 2).mean())


@pytest.mark.parametrize("shape", [(3, 64, 64, 7, 2), (5, 128, 192, 3, 5), (2, 64, 128, 1, 2)])
def test_fuzz_shapes_match_brute_force(oracle_lib, shape):
    E, H, I, T, k = shape
    p = ms.make_problem(E, H, I, T, k, seed=E * 7 + T)
    r = oracle_lib.ffn_tokens(p)
    assert rel_err(r["out"], brute_force_out(p)) < 1e-12


@pytest.mark.parametrize("gs,shape", [(32, (3, 96, 64, 6, 2)), (32, (2, 64, 160, 4, 2)),
                                      (128, (3, 256, 128, 5, 2)), (128, (2, 128, 384, 3, 1))])
def test_group_sizes_match_brute_force(oracle_lib, gs, shape):
    """Groups of 32 and 128 columns: one scale and bias per gs columns."""
    E, H, I, T, k = shape
    p = ms.make_problem(E, H, I, T, k, seed=gs + T, gs=gs)
    assert p.s_gateup.shape[-1] == H // gs and p.s_down.shape[-1] == I // gs
    r = oracle_lib.ffn_tokens(p)
    assert rel_err(r["out"], brute_force_out(p)) < 1e-12


def test_invalid_ids_contribute_zero(oracle_lib):
    p = ms.make_problem(E=4, H=64, I=64, T=4, k=2, seed=8)
    ref = brute_force_out(p)
    p.topk_ids[1, 0] = 4
    p.topk_ids[2, 1] = -3
    r = oracle_lib.ffn_tokens(p)
    bf = brute_force_out(p)       # brute force drops the same copies
    assert rel_err(r["out"], bf) < 1e-12
    assert np.all(r["h"][2] == 0) and np.all(r["y"][2] == 0)
    assert rel_err(r["out"][[0, 3]], ref[[0, 3]]) < 1e-12


def test_combine_linear_in_weights(oracle_lib):
    p = ms.make_problem(E=4, H=64, I=64, T=5, k=3, seed=9)
    r1 = oracle_lib.ffn_tokens(p)
    p.topk_weights = (p.topk_weights * np.float32(2)).astype(np.float32)
    r2 = oracle_lib.ffn_tokens(p)
    np.testing.assert_array_equal(r2["out"], 2 * r1["out"])
    np.testing.assert_array_equal(r2["y"], r1["y"])


def test_identical_experts_give_plain_ffn(oracle_lib):
    """All experts equal and weights summing to one: out = FFN(x)."""
    p = ms.make_problem(E=4, H=64, I=64, T=6, k=3, seed=10)
    for arr in (p.w_gateup, p.s_gateup, p.b_gateup, p.w_down, p.s_down, p.b_down):
        arr[:] = arr[0:1]
    r = oracle_lib.ffn_tokens(p)
    ffn = r["y"].reshape(p.T, p.k, p.H)[:, 0]
    wsum = p.topk_weights.astype(np.float64).sum(1, keepdims=True)
    assert np.abs(wsum - 1).max() < 1e-6
    np.testing.assert_allclose(r["out"], ffn * wsum, rtol=1e-12, atol=1e-12)


def test_token_subset_is_consistent(oracle_lib):
    p = ms.make_config("tiny")
    full = oracle_lib.ffn_tokens(p)
    toks = np.array([63, 0, 17, 17], np.int32)
    sub = oracle_lib.ffn_tokens(p, toks)
    np.testing.assert_array_equal(sub["out"], full["out"][toks])
    rows = (toks[:, None] * p.k + np.arange(p.k)[None, :]).ravel()
    np.testing.assert_array_equal(sub["h"], full["h"][rows])
    np.testing.assert_array_equal(sub["y"], full["y"][rows])


# ----------------------------------------------------------------- router
def test_router_hand_example(oracle_lib):
    """Ties go to the lower id; weights are the renormalised softmax of the
    chosen logits: [1, 1, e^-2] / (2 + e^-2)."""
    ids, w = oracle_lib.router_topk(np.array([[0.0, 3.0, 3.0, 1.0]], np.float32), 3)
    assert ids.tolist() == [[1, 2, 3]]
    d = 2 + math.exp(-2)
    np.testing.assert_allclose(w[0], [1 / d, 1 / d, math.exp(-2) / d], rtol=1e-15)


def test_router_full_k_is_softmax(oracle_lib):
    rng = np.random.default_rng(21)
    logits = rng.standard_normal((33, 8)).astype(np.float32) * 3
    ids, w = oracle_lib.router_topk(logits, 8)
    ref = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), axis=1),
                               rtol=1e-13)


@pytest.mark.parametrize("E,k", [(128, 8), (64, 1), (1024, 64), (5, 5)])
def test_router_matches_library_routines(oracle_lib, E, k):
    rng = np.random.default_rng(E + k)
    logits = rng.standard_normal((40, E)).astype(np.float32)
    logits[::7, : E // 2] = 0.5  # ties inside and across the chosen set
    ids, w = oracle_lib.router_topk(logits, k)
    ref_ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref_ids)
    sel = np.take_along_axis(logits, ref_ids, axis=1).astype(np.float64)
    ref_w = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    np.testing.assert_allclose(w, ref_w, rtol=1e-13)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    # a constant shift of a row changes nothing
    ids2, w2 = oracle_lib.router_topk(logits + np.float32(4.0), k)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_allclose(w2, w, rtol=1e-6)


# ---------------------------------------------------- forward tile lists
def test_forward_tiles_hand_example(oracle_lib):
    """bm_big 64, bm_small 16; counts 0, 5, 16, 17, 64, 65, 130 (offsets are
    their running sum): experts 1 and 2 are short tiles; 17 and 64 one tile
    each; 65 -> 33 + 32; 130 -> 44 + 43 + 43."""
    counts = np.array([0, 5, 16, 17, 64, 65, 130], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wide, short = oracle_lib.forward_tiles(counts, offsets, 64, 16)
    assert short.tolist() == [[1, 0, 5, 16], [2, 5, 16, 16]]
    assert wide.tolist() == [[3, 21, 17, 64], [4, 38, 64, 64], [5, 102, 33, 64], [5, 135, 32, 64],
                             [6, 167, 44, 64], [6, 211, 43, 64], [6, 254, 43, 64]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_tiles_invariants(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 300, size=50).astype(np.int32)
    counts[rng.integers(0, 50, 10)] = rng.integers(0, 17, 10)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wide, short = oracle_lib.forward_tiles(counts, offsets, 64, 16)
    for e, c in enumerate(counts):
        w = wide[wide[:, 0] == e]
        s = short[short[:, 0] == e]
        if c == 0:
            assert len(w) == len(s) == 0
        elif c <= 16:
            assert len(w) == 0 and s.tolist() == [[e, offsets[e], c, 16]]
        else:
            assert len(s) == 0 and len(w) == -(-c // 64)
            assert np.all(w[:, 2] > 16) and np.all(w[:, 2] <= 64)
            assert w[:, 2].max() - w[:, 2].min() <= 1
            # consecutive, covering the expert's rows exactly
            assert w[0, 1] == offsets[e] and np.all(w[1:, 1] == w[:-1, 1] + w[:-1, 2])
            assert w[:, 2].sum() == c


def test_forward_tiles_one_operand_path_per_expert(oracle_lib):
    """The bf16 gate|up launch picks its operand format per tile (fp8 from
    32 rows up).  With 64-row tiles every tile of an expert falls on the same
    side of 32 rows, and the side is that of the expert's own count, so a
    row's bits never depend on where it sits among its expert's rows."""
    counts = np.arange(17, 1025, dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wide, _ = oracle_lib.forward_tiles(counts, offsets, 64, 16)
    for e, c in enumerate(counts):
        rows = wide[wide[:, 0] == e, 2]
        assert np.all((rows >= 32) == (c >= 32)), (c, rows)


# ------------------------------------------------- whole-batch entry point
@pytest.mark.parametrize("case", ["tiny", "invalid", "silu", "gs32-8bit", "gs128-indep"])
def test_ffn_all_same_bits_as_per_token_path(oracle_lib, case):
    """The expert-major whole-batch entry computes the same sums in the same
    order as the per-token path: identical bits for h, y and out."""
    act = "gelu"
    if case == "tiny":
        p = ms.make_config("tiny")
    elif case == "invalid":
        p = ms.make_problem(6, 128, 64, 30, 3, seed=4, name="inv")
        p.topk_ids[2, 1] = -1
        p.topk_ids[7, :] = 6
    elif case == "silu":
        p = ms.make_problem(5, 192, 128, 20, 2, seed=5, name="silu")
        act = "silu"
    elif case == "gs32-8bit":
        p = ms.make_problem(4, 128, 64, 16, 2, seed=6, gs=32, bits=8, name="g32b8")
    else:
        p = ms.make_problem(4, 256, 128, 16, 2, seed=7, gs=128, bias="independent", name="g128")
    a = oracle_lib.ffn_tokens(p, act=act)
    b = oracle_lib.ffn_all(p, act=act)
    for key in ("h", "y", "out"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 32)])
def test_independent_biases_match_brute_force(oracle_lib, bits, gs):
    """Biases drawn independently of the scales (the general affine format):
    the whole-batch entry against the dense, unrouted recomputation."""
    p = ms.make_problem(6, 256, 128, 24, 3, seed=8 + bits, gs=gs, bits=bits, bias="independent",
                        name="indep")
    s = ms.bf16_bits_to_f32(p.s_gateup).astype(np.float64)
    b = ms.bf16_bits_to_f32(p.b_gateup).astype(np.float64)
    assert np.mean(b + 2 ** (bits - 1) * s == 0) < 0.01  # not the centred draw
    ref = brute_force_out(p)
    got = oracle_lib.ffn_all(p)["out"]
    assert np.abs(got - ref).max() <= 1e-10 * np.abs(ref).max()


def test_down_rows_same_bits_as_whole_forward(oracle_lib):
    """The down projection for a given h reproduces the whole forward's y
    bit for bit when handed the forward's own h; its magnitude sum bounds |y|
    and equals it for a one-column matrix of non-negative terms."""
    p = ms.make_problem(6, 128, 64, 30, 3, seed=12, name="down")
    p.topk_ids[4, 2] = -3
    r = oracle_lib.ffn_all(p)
    y, ya = oracle_lib.down_rows(p, p.topk_ids.ravel(), r["h"])
    np.testing.assert_array_equal(y, r["y"])
    assert np.all(ya >= np.abs(y))
    assert not np.any(y[4 * 3 + 2]) and not np.any(ya[4 * 3 + 2])
    q = ms.make_problem(1, 64, 64, 1, 1, seed=1, name="one")
    q.s_down[:] = ms.f32_to_bf16_bits(np.array([1.0], np.float32))
    q.b_down[:] = 0
    h = np.full((1, 64), 0.5)
    y, ya = oracle_lib.down_rows(q, np.zeros(1, np.int32), h)
    np.testing.assert_array_equal(y, ya)
