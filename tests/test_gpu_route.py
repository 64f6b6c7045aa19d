"""Route / sort / tile kernel against the oracle: bit-exact (GPU)."""
import numpy as np
import pytest
import torch

import bit_gathered_quantized_amd as bgq
import moe_synth as ms
from gpu_util import log

pytestmark = pytest.mark.gpu


def gpu_route(ids_np, E, bm_big=32, bm_small=16):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    if ids.dim() == 1:
        ids = ids.view(-1, 1)
    r = bgq.sort_build_tiles(ids, E, bm_big, bm_small)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def check_route(oracle_lib, ids, E, bm_big=32, bm_small=16):
    flat = np.ascontiguousarray(ids, dtype=np.int32).ravel()
    log(f"route: A={flat.size} E={E} bm=({bm_big},{bm_small})")
    g = gpu_route(ids, E, bm_big, bm_small)
    counts, offsets, perm, inv, bad = oracle_lib.route(flat, E)
    tiles = oracle_lib.tiles(counts, offsets, bm_big, bm_small)
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["perm"], perm)
    np.testing.assert_array_equal(g["inv_perm"], inv)
    assert int(g["num_tiles"][0]) == len(tiles)
    assert int(g["num_tiles"][1]) == bad
    np.testing.assert_array_equal(g["tiles"][: len(tiles)], tiles)
    return g


@pytest.mark.parametrize("name", ms.CONFIG_ORDER)
def test_route_configs(oracle_lib, name):
    c = ms.CONFIGS[name]
    rng = np.random.default_rng(0)
    ids, _ = ms.route_topk(ms._router_logits(rng, c["router"], c["T"], c["E"]), c["k"])
    check_route(oracle_lib, ids, c["E"])


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (3, 2, 8), (17, 8, 128), (64, 1, 3),
                                   (1000, 8, 128), (4096, 4, 1024), (5000, 2, 7),
                                   (20000, 8, 128)])
def test_route_fuzz(oracle_lib, T, k, E):
    rng = np.random.default_rng(T * 31 + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    check_route(oracle_lib, ids, E)


@pytest.mark.parametrize("T,k,E,lo,hi", [(8, 8, 128, 0, 128), (7, 9, 1024, -2, 1030), (64, 1, 1, 0, 1),
                                         (5, 3, 2, -1, 3), (1, 64, 64, 0, 64), (2, 32, 4, 0, 4),
                                         (1, 63, 1000, 990, 1001)])
def test_route_one_row(oracle_lib, T, k, E, lo, hi):
    """At most 64 assignments (one wave does the whole sort), with repeated
    and out-of-range ids."""
    rng = np.random.default_rng(T * 131 + k * 7 + E)
    ids = rng.integers(lo, hi, size=(T, k)).astype(np.int32)
    for bm in [(32, 16), (64, 16), (1, 1)]:
        check_route(oracle_lib, ids, E, *bm)


@pytest.mark.parametrize("bm_big,bm_small", [(64, 16), (16, 16), (128, 32), (1, 1), (7, 3)])
def test_route_tile_sizes(oracle_lib, bm_big, bm_small):
    c = ms.CONFIGS["prefill16k"]
    rng = np.random.default_rng(0)
    ids, _ = ms.route_topk(ms._router_logits(rng, c["router"], c["T"], c["E"]), c["k"])
    check_route(oracle_lib, ids, c["E"], bm_big, bm_small)


def test_route_all_to_one_expert(oracle_lib):
    ids = np.full((777, 2), 5, np.int32)
    g = check_route(oracle_lib, ids, 8)
    assert g["counts"][5] == 1554


def test_route_invalid_ids(oracle_lib):
    rng = np.random.default_rng(7)
    ids = rng.integers(-3, 12, size=(300, 3)).astype(np.int32)
    g = check_route(oracle_lib, ids, 9)
    assert g["num_tiles"][1] > 0


def test_route_empty(oracle_lib):
    ids = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    r = bgq.sort_build_tiles(ids, 16)
    torch.cuda.synchronize()
    assert int(r["num_tiles"][0]) == 0 and int(r["num_tiles"][1]) == 0
    assert torch.all(r["counts"] == 0) and torch.all(r["offsets"] == 0)
