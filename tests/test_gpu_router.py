"""Device router (softmax top-k, renormalised weights) against the oracle.

ids bit-exact; weights within 4e-6 relative (fp32 exp and one fp32 division
against a double-precision reference: a few ulps)."""
import numpy as np
import pytest
import torch

import bit_gathered_quantized_amd as bgq
import moe_synth as ms
from gpu_util import log
from test_gpu_forward import compare

pytestmark = pytest.mark.gpu


def _logits(T, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        l = np.round(l * 2).astype(np.float32)  # many equal logits per row
    return l


@pytest.mark.parametrize("T,E,k,ties", [(2048, 128, 8, False), (2048, 128, 8, True),
                                        (64, 8, 2, False), (7, 1024, 64, True), (33, 5, 5, False),
                                        (1, 300, 1, True)])
def test_router_matches_oracle(oracle_lib, T, E, k, ties):
    log(f"router T={T} E={E} k={k} ties={ties}")
    l = _logits(T, E, seed=T + E + k, ties=ties)
    ids, w = bgq.router_topk(torch.from_numpy(l).cuda(), k)
    torch.cuda.synchronize()
    rid, rw = oracle_lib.router_topk(l, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), rw, rtol=4e-6, atol=0)


def test_router_empty_and_errors():
    l = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    ids, w = bgq.router_topk(l, 2)
    assert ids.shape == (0, 2)
    with pytest.raises(bgq.MoeError):
        bgq.router_topk(torch.zeros((4, 8), dtype=torch.float32, device="cuda"), 9)
    with pytest.raises(bgq.MoeError):
        bgq.router_topk(torch.zeros((4, 128), dtype=torch.float32, device="cuda"), 65)


def test_router_feeds_forward(oracle_lib):
    """Device-routed ids give the same expert choice as the workload
    generator's router, and the forward on them matches the oracle."""
    p = ms.make_config("decode")
    rng = np.random.default_rng(99)
    l = rng.standard_normal((p.T, p.E)).astype(np.float32)
    ids, w = bgq.router_topk(torch.from_numpy(l).cuda(), p.k)
    gid, gw = ms.route_topk(l, p.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), gid)
    p.topk_ids = ids.cpu().numpy()
    p.topk_weights = w.cpu().numpy()
    compare(oracle_lib, p, False)
