"""Seeded random problems against the oracle (GPU): geometry (E, H, I, T, k),
group size, code width, router, bias recipe, mode (bf16 or fp32),
activation (GeGLU or SwiGLU) and out-of-range expert ids drawn per case from
a fixed seed, every token compared (h, y and out, with the same bounds as the
named cases)."""
import dataclasses

import numpy as np
import pytest

import moe_synth as ms
from test_gpu_forward import compare

pytestmark = pytest.mark.gpu

N_CASES = 24


def fuzz_case(i: int):
    """Case i: (problem, fp32, swiglu), all drawn from seed 7000 + i."""
    rng = np.random.default_rng(7000 + i)
    gs = int(rng.choice([32, 64, 128]))
    bits = int(rng.choice([4, 8]))
    unit = max(64, gs)  # H and I: multiples of 64 and of the group size
    H = unit * int(rng.integers(1, 1024 // unit + 1))
    I = unit * int(rng.integers(1, 768 // unit + 1))
    E = int(rng.integers(1, 41))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 401))
    router = str(rng.choice(["normal", "biased", "zipf"]))
    bias = str(rng.choice(["centred", "independent"]))
    fp32 = bool(rng.integers(0, 2))
    swiglu = bool(rng.integers(0, 2))
    p = ms.make_problem(E, H, I, T, k, seed=7000 + i, router=router, gs=gs, bits=bits, bias=bias,
                        name=f"fuzz{i}")
    if rng.random() < 0.3:
        # a few out-of-range ids (negative or >= E), which must contribute 0
        ids = p.topk_ids.copy()
        bad = rng.random(ids.shape) < 0.05
        ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + rng.integers(0, 5, int(bad.sum())))
        p = dataclasses.replace(p, topk_ids=ids.astype(np.int32))
    return p, fp32, swiglu


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_against_oracle(oracle_lib, i):
    p, fp32, swiglu = fuzz_case(i)
    compare(oracle_lib, p, fp32, swiglu=swiglu)
