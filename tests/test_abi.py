"""The C ABI on the CPU: the library loads, exports every declared entry
point, and rejects bad arguments before enqueueing anything (no GPU needed:
every call here fails a host-side check first)."""
import ctypes
import os
import re

import pytest

import bit_gathered_quantized_amd as bgq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "moe_ffn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 7
    L = bgq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(bgq.EXPORTED_SYMBOLS) == names


def test_max_tiles():
    assert bgq.max_tiles(16384, 128, 32) == 512 + 128
    assert bgq.max_tiles(64, 128, 32) == 2 + 64
    assert bgq.max_tiles(0, 8, 32) == 0
    assert bgq.max_tiles(-1, 8, 32) == -1
    assert bgq.max_tiles(10, 0, 32) == -1


def test_workspace_layout_and_sizes():
    p = bgq.problem(2048, 8, 128, 2816, 704)
    lay = bgq.workspace_layout(p)
    A = 2048 * 8
    assert lay.total == bgq.workspace_bytes(p)
    offs = [lay.counts, lay.offsets, lay.perm, lay.inv_perm, lay.tiles, lay.tiles_skinny,
            lay.num_tiles, lay.x_perm, lay.x_sums, lay.h, lay.h_sums, lay.y, lay.route_hist]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.x_sums - lay.x_perm >= 2048 * 2816 * 2
    assert lay.h_sums - lay.h >= A * 704 * 2 and lay.route_hist - lay.y >= A * 2816 * 4
    # per-key counts of each 1024-assignment segment for the route launches
    assert lay.total - lay.route_hist >= (A // 1024) * 129 * 4
    small = bgq.workspace_layout(bgq.problem(256, 8, 128, 2816, 704))
    assert small.x8_hi == small.route_hist  # 2048 assignments: one workgroup sorts
    # x as e4m3 hi + lo with a scale byte per 32 columns (rows padded to 4 bytes)
    assert lay.x8_lo - lay.x8_hi >= 2048 * 2816 and lay.x8_scales - lay.x8_lo >= 2048 * 2816
    assert lay.total - lay.x8_scales >= 2048 * 88
    assert lay.x8_hi >= lay.route_hist
    assert lay.y - lay.h_sums >= A * (704 // 16) * 4  # 16-column block sums of h
    assert lay.bm_big == 64 and lay.bm_small == 16
    assert lay.max_tiles == A // 64 + 128
    assert lay.tiles_skinny - lay.tiles >= 16 * lay.max_tiles
    assert lay.num_tiles - lay.tiles_skinny >= 16 * lay.max_skinny
    # the short list holds every expert in 16-row pieces when T <= 16
    assert lay.max_skinny == bgq.max_tiles(p.T * p.k, p.E, lay.bm_small)
    p32 = bgq.problem(2048, 8, 128, 2816, 704, bgq.MOE_F_FP32_INTERMEDIATE)
    l32 = bgq.workspace_layout(p32)
    assert l32.h_sums - l32.h >= A * 704 * 4


@pytest.mark.parametrize("T,flags,gs,bits,fp8", [
    (17, 0, 64, 4, True), (2048, 0, 128, 4, True), (16, 0, 64, 4, False),
    (2048, 2, 64, 4, False), (2048, 0, 32, 4, False), (2048, 0, 64, 8, False)])
def test_fp8_activation_layout(T, flags, gs, bits, fp8):
    """The fp8 copies of x exist exactly when the wide gate|up matmul takes
    fp8 operands: more than 16 tokens, bf16 mode, 4-bit codes in groups of
    64 or 128."""
    I = 768 if gs == 128 else 704
    lay = bgq.workspace_layout(bgq.problem(T, 8, 128, 2816, I, flags, group_size=gs, bits=bits))
    size = lay.total - lay.x8_hi
    assert (size > 0) == fp8
    if fp8:
        assert size >= T * 2816 * 2 + T * 88


@pytest.mark.parametrize("kw,status", [
    (dict(bits=2), -3), (dict(bits=16), -3), (dict(bits=3), -3), (dict(group_size=16), -3), (dict(group_size=256), -3),
    (dict(group_size=48), -3), (dict(E=2000), -3), (dict(flags=8), -3), (dict(flags=16), -3),
    (dict(group_size=128, H=192), -2), (dict(group_size=128, I=320), -2),
    (dict(group_size=32, H=96), -2),
    (dict(H=100), -2), (dict(I=96), -2), (dict(H=8192), -3), (dict(I=4160), -3), (dict(k=0), -2), (dict(k=9, E=8), -2), (dict(T=-1), -2),
])
def test_bad_problem(kw, status):
    base = dict(T=4, k=2, E=8, H=256, I=128, flags=0, group_size=64, bits=4)
    base.update(kw)
    p = bgq.problem(**base)
    assert bgq.workspace_bytes(p) == 0
    with pytest.raises(bgq.MoeError) as e:
        bgq.workspace_layout(p)
    assert e.value.status == status


def _forward(p, ptrs, out, ws, ws_bytes):
    L = bgq.lib()
    return L.moe_expert_ffn_forward(ctypes.byref(p), *ptrs, out, ws, ws_bytes, None)


def test_forward_host_checks():
    p = bgq.problem(4, 2, 8, 256, 128)
    need = bgq.workspace_bytes(p)
    good = [ctypes.c_void_p(0x10000)] * 9
    out = ctypes.c_void_p(0x20000)
    ws = ctypes.c_void_p(0x40000)
    # null pointer
    assert _forward(p, [None] + good[1:], out, ws, need) == -1
    assert _forward(p, good, None, ws, need) == -1
    # workspace missing / too small
    assert _forward(p, good, out, None, need) == -5
    assert _forward(p, good, out, ws, need - 1) == -5
    # misaligned x, weights, out, workspace
    assert _forward(p, [ctypes.c_void_p(0x10002)] + good[1:], out, ws, need) == -4
    bad_w = list(good)
    bad_w[3] = ctypes.c_void_p(0x10008)
    assert _forward(p, bad_w, out, ws, need) == -4
    # scales and biases are read in 16-byte pieces
    for i in (4, 5, 7, 8):
        bad_s = list(good)
        bad_s[i] = ctypes.c_void_p(0x10002)
        assert _forward(p, bad_s, out, ws, need) == -4
    assert _forward(p, good, ctypes.c_void_p(0x20002), ws, need) == -4
    assert _forward(p, good, out, ctypes.c_void_p(0x40080), need) == -4
    # zero tokens: nothing to do, nothing touched
    p0 = bgq.problem(0, 2, 8, 256, 128)
    assert _forward(p0, [None] * 9, None, None, 0) == 0
    # bad problem wins over pointers
    assert _forward(bgq.problem(4, 2, 8, 256, 128, 0, 64, 3), good, out, ws, need) == -3


def test_sort_host_checks():
    L = bgq.lib()
    P = ctypes.c_void_p
    d = P(0x10000)
    mt = bgq.max_tiles(40, 8, 32)
    # bm_small > bm_big
    assert L.moe_sort_build_tiles(d, 10, 4, 8, 16, 32, d, d, d, d, d, mt, d, None) == -2
    # too few tiles
    assert L.moe_sort_build_tiles(d, 10, 4, 8, 32, 16, d, d, d, d, d, mt - 1, d, None) == -5
    # null outputs
    assert L.moe_sort_build_tiles(d, 10, 4, 8, 32, 16, None, d, d, d, d, mt, d, None) == -1
    assert L.moe_sort_build_tiles(None, 10, 4, 8, 32, 16, d, d, d, d, d, mt, d, None) == -1
    # too many experts
    assert L.moe_sort_build_tiles(d, 10, 4, 5000, 32, 16, d, d, d, d, d, mt, d, None) == -3
    # misaligned tile buffer
    assert L.moe_sort_build_tiles(d, 10, 4, 8, 32, 16, d, d, d, d, P(0x10004), mt, d, None) == -4


def test_status_strings():
    for s in range(-6, 1):
        assert bgq.status_string(s) and "unknown" not in bgq.status_string(s)
    assert "unknown" in bgq.status_string(-99)


def test_router_host_checks():
    L = bgq.lib()
    P = ctypes.c_void_p
    d = P(0x10000)
    assert L.moe_router_topk(d, -1, 8, 2, d, d, None) == -2
    assert L.moe_router_topk(d, 4, 8, 9, d, d, None) == -2
    assert L.moe_router_topk(d, 4, 8, 0, d, d, None) == -2
    assert L.moe_router_topk(d, 4, 2000, 8, d, d, None) == -3
    assert L.moe_router_topk(d, 4, 128, 65, d, d, None) == -3
    assert L.moe_router_topk(None, 4, 8, 2, d, d, None) == -1
    assert L.moe_router_topk(d, 4, 8, 2, P(0x10002), d, None) == -4
    assert L.moe_router_topk(None, 0, 8, 2, None, None, None) == 0


def test_presorted_host_checks():
    L = bgq.lib()
    p = bgq.problem(4, 2, 8, 256, 128)
    need = bgq.workspace_bytes(p)
    good = [ctypes.c_void_p(0x10000)] * 9
    out, ws = ctypes.c_void_p(0x20000), ctypes.c_void_p(0x40000)
    P = ctypes.c_void_p

    def call(order):
        return L.moe_expert_ffn_forward_presorted(ctypes.byref(p), *good[:3], order, *good[3:],
                                                  out, ws, need, None)
    assert call(None) == -1
    assert call(P(0x10002)) == -4


@pytest.mark.parametrize("gs,bits", [(32, 4), (64, 4), (128, 4), (32, 8), (64, 8), (128, 8)])
def test_layout_other_geometries(gs, bits):
    """Group sums take H/gs floats per token; 8-bit codes use 32-row wide tiles."""
    T, k, E, H, I = 300, 4, 16, 1024, 256
    lay = bgq.workspace_layout(bgq.problem(T, k, E, H, I, 0, group_size=gs, bits=bits))
    assert lay.h - lay.x_sums >= T * (H // gs) * 4
    assert lay.bm_big == (32 if bits == 8 else 64) and lay.bm_small == 16
    assert lay.max_tiles == bgq.max_tiles(T * k, E, lay.bm_big)

