"""The forward captured in a HIP graph (the analogue of a whole-forward
compile): every replay, with new inputs copied into the captured buffers and
eager work and synchronisations between replays, matches the oracle on those
inputs and equals the eager forward bit for bit.  The forward records no memset, allocates nothing and never
synchronises, so it captures as six kernel nodes."""
import numpy as np
import pytest
import torch

import bit_gathered_quantized_amd as bgq
import moe_synth as ms
import dataclasses

from gpu_util import dev_arrays, log
from test_gpu_forward import compare

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,swiglu", [("decode", False), ("prefill4k", True),
                                         ("prefill4k-8bit-gs128", False)])
def test_graph_replays_match_eager(oracle_lib, name, swiglu):
    if name == "prefill4k-8bit-gs128":
        p = ms.make_problem(128, 2816, 768, 512, 8, seed=0, gs=128, bits=8, name=name)
    else:
        p = ms.make_config(name)
    d = dev_arrays(p)
    prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, bgq.MOE_F_SWIGLU if swiglu else 0, group_size=p.gs,
                       bits=p.bits)
    ws = torch.zeros(bgq.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device="cuda")
    args = [d[n] for n in ("x", "ids", "w", "w_gu", "s_gu", "b_gu", "w_d", "s_d", "b_d")]

    def fwd():
        bgq.expert_ffn_forward(*args, swiglu=swiglu, out=out, workspace=ws)

    fwd()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fwd()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    rng = np.random.default_rng(3)
    for rep in range(4):
        # new activations and routing in the captured buffers
        x = ms.f32_to_bf16_bits(rng.standard_normal((p.T, p.H)).astype(np.float32))
        ids, w = ms.route_topk(rng.standard_normal((p.T, p.E)).astype(np.float32), p.k)
        d["x"].copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        d["ids"].copy_(torch.from_numpy(ids))
        d["w"].copy_(torch.from_numpy(w))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        q = dataclasses.replace(p, x=x, topk_ids=ids, topk_weights=w, name=f"{name}-replay{rep}")
        lay = bgq.workspace_layout(prob)
        compare(oracle_lib, q, False, swiglu=swiglu,
                run=lambda *_: (got.float().cpu().numpy().astype(np.float64), ws, lay))
        _ = (d["x"].float() * 2).sum()  # unrelated eager work between replays
        fwd()
        torch.cuda.synchronize()
        log(f"  {name} replay {rep}: equal={torch.equal(got, out)}")
        assert torch.equal(got, out)
