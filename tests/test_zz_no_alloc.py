"""The allocation-free entry point (moe_expert_ffn_forward_noalloc): its
output equals the regular entry point's, bit for bit, on two calls in a row
(the second smaller than the first, on the scratch array the first left
behind), in both modes; a problem too large for its scratch array is refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import bit_gathered_quantized_amd as bgq
import moe_synth as ms
from gpu_util import dev_arrays, log

pytestmark = pytest.mark.gpu


def _call(p, d, fp32, no_alloc):
    out = torch.empty((p.T, p.H), dtype=torch.float32 if fp32 else torch.bfloat16, device="cuda")
    kw = dict(fp32_out=fp32, fp32_intermediate=fp32, out=out)
    if no_alloc:
        bgq.expert_ffn_forward(*[d[n] for n in ("x", "ids", "w", "w_gu", "s_gu", "b_gu", "w_d", "s_d",
                                                 "b_d")], no_alloc=True, **kw)
    else:
        prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, (3 if fp32 else 0), group_size=p.gs, bits=p.bits)
        ws = torch.empty(bgq.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
        bgq.expert_ffn_forward(*[d[n] for n in ("x", "ids", "w", "w_gu", "s_gu", "b_gu", "w_d", "s_d",
                                                 "b_d")], workspace=ws, **kw)
    torch.cuda.synchronize()
    return out.clone()


@pytest.mark.parametrize("fp32", [False, True])
def test_noalloc_matches_regular_entry(fp32):
    big = ms.make_problem(128, 2816, 704, 96, 8, seed=5, name="noalloc-96")   # wide and skinny tiles
    small = ms.make_config("decode")                                           # 8 tokens, skinny only
    for p in (big, small):
        prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, (3 if fp32 else 0))
        assert bgq.workspace_bytes(prob) <= bgq.NOALLOC_SCRATCH_BYTES
        d = dev_arrays(p)
        got = _call(p, d, fp32, True)
        ref = _call(p, d, fp32, False)
        log(f"  {p.name} fp32={fp32}: equal={torch.equal(got, ref)}")
        assert torch.equal(got, ref)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    p = ms.make_problem(128, 2816, 704, 400, 8, seed=1, name="too-big")
    prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, 0)
    assert bgq.workspace_bytes(prob) > bgq.NOALLOC_SCRATCH_BYTES
    d = dev_arrays(p)
    out = torch.full((p.T, p.H), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bgq.MoeError) as ei:
        bgq.expert_ffn_forward(*[d[n] for n in ("x", "ids", "w", "w_gu", "s_gu", "b_gu", "w_d", "s_d",
                                                 "b_d")], out=out, no_alloc=True)
    assert ei.value.status == bgq.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was enqueued
