"""The seeded input generator: a routing-only draw gives the same routing as
the full draw (the emulation tests use it), and full draws are repeatable."""
import numpy as np
import pytest

import moe_synth as ms


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill8k"])
def test_routing_only_draw_matches_full_draw(name):
    full = ms.make_config(name)
    part = ms.make_config(name, routing_only=True)
    np.testing.assert_array_equal(part.topk_ids, full.topk_ids)
    np.testing.assert_array_equal(part.topk_weights, full.topk_weights)
    assert part.x is None and part.w_gateup is None and part.w_down is None


def test_full_draw_repeats():
    a, b = ms.make_config("tiny"), ms.make_config("tiny")
    for f in ("x", "topk_ids", "w_gateup", "s_gateup", "b_gateup", "w_down", "s_down", "b_down"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
