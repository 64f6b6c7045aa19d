"""Host-side logic of bench.py: the algorithmic byte and flop counts that the
roofline figures divide by, the roofline classification, the committed
counter summaries, and the one-GPU guard.  No GPU needed."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import moe_synth as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _expert_bytes(H, I, bits, gs):
    """Codes plus bf16 scales and biases of one expert, written out per matrix."""
    gate_up = (2 * I) * (H * bits // 8) + 2 * (2 * I) * (H // gs) * 2
    down = H * (I * bits // 8) + 2 * H * (I // gs) * 2
    return gate_up, down


@pytest.mark.parametrize("bits,gs,I", [(4, 64, 704), (8, 64, 704), (4, 32, 704), (4, 128, 768)])
def test_decode_algorithmic_bytes(bits, gs, I):
    p = ms.make_problem(128, 2816, I, 8, 8, seed=0, gs=gs, bits=bits)
    work, fwd, split = bench.algorithmic_work(p)
    touched = np.unique(p.topk_ids).size
    gu, d = _expert_bytes(p.H, p.I, bits, gs)
    A = p.T * p.k
    # at 8 tokens every expert is a skinny tile; x rows once, h rows once
    assert work["moe_gateup_skinny"]["bytes"] == touched * gu + p.T * p.H * 2 + A * p.I * 2
    assert work["moe_down_skinny"]["bytes"] == touched * d + A * p.I * 2 + A * p.H * 4
    assert work["moe_gateup_wide"]["bytes"] == 0 and work["moe_down_wide"]["flops"] == 0
    assert work["moe_gateup_skinny"]["flops"] == A * 4 * p.H * p.I
    assert fwd["flops"] == A * 6 * p.H * p.I
    assert split["skinny_rows"] == A and split["wide_rows"] == 0


def test_published_geometry_per_expert_bytes():
    gu, d = _expert_bytes(2816, 704, 4, 64)
    assert (gu, d) == (1982464 + 247808, 991232 + 123904)
    assert gu + d == 3345408


def test_prefill_rows_split_between_paths():
    p = ms.make_config("prefill16k")
    work, fwd, split = bench.algorithmic_work(p)
    counts = np.bincount(p.topk_ids.ravel(), minlength=p.E)
    small = counts[(counts > 0) & (counts <= 16)]
    assert split["skinny_rows"] == small.sum() and split["experts_with_skinny_tile"] == small.size
    assert split["skinny_rows"] + split["wide_rows"] == p.T * p.k
    # 64-row near-equal tiles per large expert
    assert split["wide_tiles"] == int(sum(-(-c // 64) for c in counts if c > 16))
    assert work["moe_gateup_wide"]["flops"] == split["wide_rows"] * 4 * p.H * p.I


def test_roofline_classification():
    w = dict(bytes=8e9, flops=1e12)          # 1 s of HBM, 0.4 ms of MFMA
    e = bench.roofline_entry(w, 2.0)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["achieved"] == 4.0 and e["frac"] == 0.0005
    w = dict(bytes=1e6, flops=2.5e15)
    e = bench.roofline_entry(w, 2.0)
    assert e["bound"] == "mfma" and e["achieved"] == 1250.0 and e["frac"] == 0.5


def test_committed_traffic_summaries():
    """Each committed counter summary names its kernel, workload and the source
    digest it was taken on; the benchmark reports its traffic only while that
    digest matches the sources."""
    from bit_gathered_quantized_amd.build import source_digest
    for k, w in (("moe_gateup_skinny", "decode"), ("moe_gateup_wide", "prefill16k"), ("moe_gateup_wide", "prefill4k")):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"{k}_{w}_traffic.json")))
        assert rec["kernel"] == k and rec["workload"] == w and rec["bytes_per_launch"] > 0
        assert len(rec["commands"]) == 2 and rec["fetch_scale"] > 0
        want = rec["bytes_per_launch"] if rec["source_digest"] == source_digest() else None
        assert bench.load_traffic(k, w) == want


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
