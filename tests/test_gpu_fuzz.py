"""Seeded random problems against the oracle (GPU): geometry (E, H, I, T, k),
group size, code width, router, bias recipe, mode (bf16 or fp32),
activation (GeGLU or SwiGLU), batches of at most 16 tokens (the skinny-only
launch), repeated and out-of-range expert ids, drawn per case from a fixed
seed; every token compared (h, y and out, with the same bounds as the named
cases).  Every third case also runs the pre-sorted entry with each expert's
rows shuffled, which must give the same bits."""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth as ms
from gpu_util import dev_arrays, log
from test_gpu_forward import compare
from test_gpu_presorted import _run, _sorted_orders

pytestmark = pytest.mark.gpu

N_CASES = 96


def fuzz_case(i: int):
    """Case i: (problem, fp32, swiglu), all drawn from seed 7000 + i."""
    rng = np.random.default_rng(7000 + i)
    gs = int(rng.choice([32, 64, 128]))
    bits = int(rng.choice([4, 8]))
    unit = max(64, gs)  # H and I: multiples of 64 and of the group size
    H = unit * int(rng.integers(1, 1024 // unit + 1))
    I = unit * int(rng.integers(1, 768 // unit + 1))
    small = i % 4 == 3  # at most 16 tokens: every expert on the skinny path
    E = int(rng.integers(1, 129 if small else 41))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 17 if small else 401))
    router = str(rng.choice(["normal", "biased", "zipf"]))
    bias = str(rng.choice(["centred", "independent"]))
    fp32 = bool(rng.integers(0, 2))
    swiglu = bool(rng.integers(0, 2))
    p = ms.make_problem(E, H, I, T, k, seed=7000 + i, router=router, gs=gs, bits=bits, bias=bias,
                        name=f"fuzz{i}")
    ids = p.topk_ids.copy()
    if k > 1 and rng.random() < 0.25:
        # repeated ids: some slots take the id of the token's first slot
        rep_ = rng.random(ids.shape) < 0.1
        rep_[:, 0] = False
        ids[rep_] = np.broadcast_to(ids[:, :1], ids.shape)[rep_]
    if rng.random() < 0.3:
        # a few out-of-range ids (negative or >= E), which must contribute 0
        bad = rng.random(ids.shape) < 0.05
        ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + rng.integers(0, 5, int(bad.sum())))
    p = dataclasses.replace(p, topk_ids=ids.astype(np.int32))
    return p, fp32, swiglu


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_against_oracle(oracle_lib, i):
    p, fp32, swiglu = fuzz_case(i)
    compare(oracle_lib, p, fp32, swiglu=swiglu)


@pytest.mark.parametrize("i", range(0, N_CASES, 3))
def test_fuzz_presorted_bitwise(oracle_lib, i):
    p, _, _ = fuzz_case(i)
    d = dev_arrays(p)
    ref, _, _ = _run(p, d)
    _, shuffled = _sorted_orders(p, oracle_lib)
    out, status, _ = _run(p, d, shuffled)
    log(f"  fuzz{i}: pre-sorted status {status}, equal {torch.equal(out, ref)}")
    assert status == 0 and torch.equal(out, ref)
