"""The pre-sorted entry: a caller's order sorted by expert is used as given
(any order within an expert), results equal the regular forward bit for bit;
orders that are not sorted, out of range or not a permutation are detected
on the device (workspace num_tiles[4]) and sorted there, again with equal
results."""
import numpy as np
import pytest
import torch

import bit_gathered_quantized_amd as bgq
import moe_synth as ms
from gpu_util import dev_arrays, log, ws_view
from test_gpu_forward import compare

pytestmark = pytest.mark.gpu


def _run(p, d, order=None):
    prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, 0, group_size=p.gs, bits=p.bits)
    ws = torch.zeros(bgq.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    so = None if order is None else torch.from_numpy(np.ascontiguousarray(order, np.int32)).cuda()
    out = bgq.expert_ffn_forward(d["x"], d["ids"], d["w"], d["w_gu"], d["s_gu"], d["b_gu"],
                                 d["w_d"], d["s_d"], d["b_d"], workspace=ws, sorted_order=so)
    torch.cuda.synchronize()
    lay = bgq.workspace_layout(prob)
    status = int(ws_view(ws, lay.num_tiles, 8, np.int32)[4]) if order is not None else None
    perm = ws_view(ws, lay.perm, p.T * p.k, np.int32)
    return out.clone(), status, perm


def _sorted_orders(p, oracle_lib):
    _, _, stable, _, _ = oracle_lib.route(p.topk_ids, p.E)
    rng = np.random.default_rng(17)
    keys = np.where((p.topk_ids.ravel() >= 0) & (p.topk_ids.ravel() < p.E), p.topk_ids.ravel(), p.E)
    # a sorted order with each expert's rows shuffled
    shuffled = stable.copy()
    ks = keys[stable]
    for e in np.unique(ks):
        idx = np.nonzero(ks == e)[0]
        shuffled[idx] = rng.permutation(stable[idx])
    return stable, shuffled


def _problem(name):
    if name == "prefill4k-8bit-gs32":
        return ms.make_problem(128, 2816, 704, 512, 8, seed=0, gs=32, bits=8, name=name)
    return ms.make_config(name)


@pytest.mark.parametrize("name", ["decode", "prefill16k", "prefill4k-8bit-gs32"])
def test_presorted_orders_used_and_bitwise_equal(oracle_lib, name):
    p = _problem(name)
    d = dev_arrays(p)
    ref, _, _ = _run(p, d)
    stable, shuffled = _sorted_orders(p, oracle_lib)
    for order in (stable, shuffled):
        out, status, perm = _run(p, d, order)
        log(f"  {name}: status {status}")
        assert status == 0
        np.testing.assert_array_equal(perm, order)
        assert torch.equal(out, ref)


def test_presorted_bad_orders_fall_back(oracle_lib):
    p = ms.make_config("prefill4k")
    d = dev_arrays(p)
    ref, _, _ = _run(p, d)
    stable, _ = _sorted_orders(p, oracle_lib)
    A = p.T * p.k
    rng = np.random.default_rng(2)
    unsorted = rng.permutation(A).astype(np.int32)
    out_of_range = stable.copy()
    out_of_range[A // 2] = A + 5
    negative = stable.copy()
    negative[-1] = -1
    dup = stable.copy()
    dup[1] = dup[0]  # same expert (the first slots share one), still sorted: not a permutation
    assert p.topk_ids.ravel()[stable[0]] == p.topk_ids.ravel()[stable[1]]
    for order, want in ((unsorted, 1), (out_of_range, 1), (negative, 1), (dup, 2)):
        out, status, perm = _run(p, d, order)
        log(f"  bad order: status {status} (want {want})")
        assert status == want
        np.testing.assert_array_equal(perm, stable)  # the device sorted by itself
        assert torch.equal(out, ref)


@pytest.mark.parametrize("name", ["decode", "prefill4k", "prefill16k"])
@pytest.mark.parametrize("fp32", [False, True])
def test_presorted_against_oracle(oracle_lib, name, fp32):
    """The pre-sorted entry, given a sorted order with each expert's rows
    shuffled, against the oracle (every token, intermediates included)."""
    p = ms.make_config(name)
    _, shuffled = _sorted_orders(p, oracle_lib)
    d = dev_arrays(p)
    flags = (bgq.MOE_F_FP32_OUT | bgq.MOE_F_FP32_INTERMEDIATE) if fp32 else 0
    prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, flags, group_size=p.gs, bits=p.bits)
    lay = bgq.workspace_layout(prob)

    def run(p_, fp32_, swiglu_):
        ws = torch.zeros(lay.total, dtype=torch.uint8, device="cuda")
        so = torch.from_numpy(shuffled).cuda()
        out = bgq.expert_ffn_forward(d["x"], d["ids"], d["w"], d["w_gu"], d["s_gu"], d["b_gu"],
                                     d["w_d"], d["s_d"], d["b_d"], fp32_out=fp32_,
                                     fp32_intermediate=fp32_, workspace=ws, sorted_order=so)
        torch.cuda.synchronize()
        assert int(ws_view(ws, lay.num_tiles, 8, np.int32)[4]) == 0
        np.testing.assert_array_equal(ws_view(ws, lay.perm, p.T * p.k, np.int32), shuffled)
        return out.float().cpu().numpy().astype(np.float64), ws, lay

    compare(oracle_lib, p, fp32, run=run)
