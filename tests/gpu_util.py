"""Helpers for the GPU parity tests: upload a problem, run the library, read
its workspace, and the tolerance rules.

Tolerances (from the target statement of this path):
  * integer outputs (sort, tiles): bit-exact;
  * bf16 outputs: max_i(|gpu_i - ref_i| - half_ulp_bf16(max(|gpu_i|, |ref_i|)))
    <= 2e-2 * rms(ref) -- the half-ulp allowance is the rounding of the
    output itself, which even an exact result pays;
  * the fp32-intermediate, fp32-output path: ||gpu - ref||_2 / ||ref||_2 <= 1e-3.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import torch

import bit_gathered_quantized_amd as bgq
import moe_synth as ms

BF16_MAX_REL_RMS = 2e-2
FP32_L2_REL = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_arrays(p, dev="cuda"):
    def t(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
    return dict(
        x=t(p.x, np.int16).view(torch.bfloat16),
        ids=t(p.topk_ids, np.int32),
        w=t(p.topk_weights, np.float32),
        w_gu=t(p.w_gateup, np.int32),
        s_gu=t(p.s_gateup, np.int16),
        b_gu=t(p.b_gateup, np.int16),
        w_d=t(p.w_down, np.int32),
        s_d=t(p.s_down, np.int16),
        b_d=t(p.b_down, np.int16),
    )


def run_forward(p, fp32=False, d=None, workspace=None, swiglu=False):
    """Run the forward; return (out as float64 numpy, workspace tensor, layout)."""
    if d is None:
        d = dev_arrays(p)
    flags = (bgq.MOE_F_FP32_OUT | bgq.MOE_F_FP32_INTERMEDIATE) if fp32 else 0
    flags |= bgq.MOE_F_SWIGLU if swiglu else 0
    prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, flags, group_size=p.gs, bits=p.bits)
    lay = bgq.workspace_layout(prob)
    if workspace is None:
        workspace = torch.zeros(max(lay.total, 256), dtype=torch.uint8, device="cuda")
    out = bgq.expert_ffn_forward(d["x"], d["ids"], d["w"], d["w_gu"], d["s_gu"], d["b_gu"],
                                 d["w_d"], d["s_d"], d["b_d"], fp32_out=fp32,
                                 fp32_intermediate=fp32, swiglu=swiglu, workspace=workspace)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    return o, workspace, lay


def ws_view(ws, offset, count, dtype):
    itemsize = np.dtype(dtype).itemsize
    raw = ws[offset: offset + count * itemsize].cpu().numpy()
    return raw.view(dtype)


OPERAND_ORDER = np.array([0, 4, 1, 5, 2, 6, 3, 7])


def from_operand_order(a: np.ndarray) -> np.ndarray:
    """Undo the operand order of the last axis: within every 8 columns the
    stored order is 0,4,1,5,2,6,3,7."""
    n = a.shape[-1]
    src = np.empty(n, np.int64)
    for b in range(0, n, 8):
        src[b + OPERAND_ORDER] = b + np.arange(8)
    return a[..., src]


def ws_h(ws, lay, p, fp32):
    """h [A, I] in sorted order, natural column order, as float64."""
    A = p.T * p.k
    if fp32:
        bits = ws_view(ws, lay.h, 2 * A * p.I, np.uint16).reshape(2, A, p.I)
        h = (ms.bf16_bits_to_f32(bits[0]).astype(np.float64)
             + ms.bf16_bits_to_f32(bits[1]).astype(np.float64))
    else:
        bits = ws_view(ws, lay.h, A * p.I, np.uint16).reshape(A, p.I)
        h = ms.bf16_bits_to_f32(bits).astype(np.float64)
    return from_operand_order(h)


def ws_y_rows(ws, lay, p, rows):
    """Rows (flat assignment indices) of the weighted y buffer."""
    rows = np.asarray(rows, dtype=np.int64)
    A = p.T * p.k
    if rows.size > A // 4:
        return ws_view(ws, lay.y, A * p.H, np.float32).reshape(A, p.H)[rows].astype(np.float64)
    out = np.zeros((len(rows), p.H))
    for i, a in enumerate(rows):
        out[i] = ws_view(ws, lay.y + int(a) * p.H * 4, p.H, np.float32)
    return out


def dense_codes(P: np.ndarray, bits: int) -> np.ndarray:
    """Codes of packed words, through numpy's little-endian byte view."""
    b = np.ascontiguousarray(P).astype("<u4").view(np.uint8)
    if bits == 8:
        return b.reshape(*P.shape[:-1], P.shape[-1] * 4)
    return np.stack([b & 0x0F, b >> 4], axis=-1).reshape(*P.shape[:-1], P.shape[-1] * 8)


def code_offset(p, fp32):
    """The kernels' code offset: the 4-bit operand is off + q (16 in the fp32
    intermediate mode, 128 in the bf16 mode), the 8-bit one q."""
    return (16.0 if fp32 else 128.0) if p.bits == 4 else 0.0


def bias_magnitude(p, experts, h, fp32):
    """sum_g (|B[m, g]| + off |S[m, g]|) sum_{n in g} |h[n]| per row and output
    column (off: code_offset): the size of the bias contraction the down
    kernels evaluate, sum_g (B - off S) X_g, with both factors split into
    bf16 hi + lo."""
    off = code_offset(p, fp32)
    G = p.I // p.gs
    out = np.zeros((len(experts), p.H))
    xa = np.abs(h).reshape(len(experts), G, p.gs).sum(-1)
    for e in np.unique(experts):
        if e < 0 or e >= p.E:
            continue
        sel = experts == e
        c = (np.abs(ms.bf16_bits_to_f32(p.b_down[e]).astype(np.float64))
             + off * np.abs(ms.bf16_bits_to_f32(p.s_down[e]).astype(np.float64)))
        out[sel] = xa[sel] @ c.T
    return out


def h_model_bound(p, rows, fp32):
    """Per-element bound on |h_kernel - h_exact| before h's own rounding, for
    the given flat rows (valid ids): the kernels' g and u carry the same
    error model as y, |dg| <= 2^-14 (sum_k |x W_g| + sum_g (|B| + off |S|)
    sum_{k in g} |x|) (likewise du), and with |act(g)| <= |g| and |act'| <=
    1.13 (GELU and SiLU), |dh| <= 1.13 |u| dg + |g| du + 1.13 dg du.  The
    bias contraction (hi + lo factors) dominates where its term is large
    against g: few groups and cancelling offsets.  g and u come from numpy
    here only to size the bound; the reference h is the oracle's."""
    rows = np.asarray(rows, dtype=np.int64)
    ids = p.topk_ids.ravel()[rows]
    x = ms.bf16_bits_to_f32(p.x).astype(np.float64)[rows // p.k]
    off = code_offset(p, fp32)
    G = p.H // p.gs
    bound = np.zeros((len(rows), p.I))
    for e in np.unique(ids):
        sel = ids == e
        q = dense_codes(p.w_gateup[e], p.bits).astype(np.float64)           # [2I, H]
        S = ms.bf16_bits_to_f32(p.s_gateup[e]).astype(np.float64)            # [2I, G]
        B = ms.bf16_bits_to_f32(p.b_gateup[e]).astype(np.float64)
        W = q * np.repeat(S, p.gs, axis=1) + np.repeat(B, p.gs, axis=1)
        xs = x[sel]
        gu = xs @ W.T
        mag = np.abs(xs) @ np.abs(W).T
        xg = np.abs(xs).reshape(len(xs), G, p.gs).sum(-1)
        mag += xg @ (np.abs(B) + off * np.abs(S)).T
        d = 2.0 ** -14 * mag
        g, u, dg, du = gu[:, :p.I], gu[:, p.I:], d[:, :p.I], d[:, p.I:]
        bound[sel] = 1.13 * np.abs(u) * dg + np.abs(g) * du + 1.13 * dg * du
    return bound


# Worst-case relative rounding of the kernels' fp32 sums against the sum of
# the terms' magnitudes: n * 2^-24 for n <= 1024 terms is below 2^-14, and
# the bias contraction's bf16 hi + lo factors are each within 2^-17.
Y_MODEL_REL = 2.0 ** -14


def check_y_model(oracle_lib, p, rows, h_gpu, y_gpu, fp32, what="y"):
    """Per-element check of the weighted down output of the given flat rows
    against the oracle's down projection of the kernel's own h (bf16, or
    bf16 hi + lo in fp32 mode): |y_gpu - w y_model| <= 2^-14 w (sum_n |W h| +
    bias magnitude).  Returns (w * y_model, bound) for the valid rows."""
    ids = p.topk_ids.ravel()[rows]
    valid = (ids >= 0) & (ids < p.E)
    w = p.topk_weights.ravel()[rows].astype(np.float64)[:, None]
    ym, ya = oracle_lib.down_rows(p, np.where(valid, ids, p.E), h_gpu)
    bound = Y_MODEL_REL * w * (ya + bias_magnitude(p, ids, h_gpu, fp32))
    model = w * ym
    err = np.abs(y_gpu - model)[valid]
    worst = float(np.max(err / np.maximum(bound[valid], 1e-300))) if err.size else 0.0
    log(f"  {what}: per element |y - model| / bound max = {worst:.3g}")
    assert np.all(err <= bound[valid]), f"{what}: per-element model bound exceeded ({worst})"
    return model, bound


def fp8_wide_gateup(p, fp32: bool) -> bool:
    """Whether some wide gate|up tile of the forward takes fp8 operands (x as
    e4m3 hi + lo, the codes as e4m3 bytes): bf16 mode, 4-bit codes in groups
    of 64 or 128, more than 16 tokens, and a tile of at least 32 rows (the
    forward cuts an expert of c > 16 rows into ceil(c / 64) near-equal
    tiles, so that is an expert of at least 32 rows).  Such rows differ in
    the last bits from the exact bf16 operand."""
    if fp32 or p.bits != 4 or p.gs not in (64, 128) or p.T <= 16:
        return False
    ids = p.topk_ids.ravel()
    counts = np.bincount(ids[(ids >= 0) & (ids < p.E)], minlength=p.E)
    return bool((counts >= 32).any())


def assert_same_or_within(a, b, same_path: bool, bound, what=""):
    """Outputs of the same tokens from two forwards: the same bits when both
    took paths of one arithmetic; otherwise within the sum of the two runs'
    per-element model bounds (each already checked against the oracle)."""
    if same_path:
        np.testing.assert_array_equal(a, b)
        return
    d = np.abs(a - b)
    log(f"  {what}: paths differ; {int(np.count_nonzero(d))} of {d.size} elements differ, "
        f"max |a - b| / bound = {float(np.max(d / np.maximum(bound, 1e-300))):.3g}")
    assert np.all(d <= bound), f"{what}: apart by more than the two model bounds"


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    v = np.abs(v)
    e = np.floor(np.log2(np.maximum(v, 1e-38)))
    return np.where(v > 0, np.exp2(e - 8), 0.0)


def bf16_excess(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max(|gpu - ref| - half_ulp(max(|gpu|, |ref|))) / rms(ref)."""
    rms = float(np.sqrt(np.mean(ref ** 2)))
    allow = half_ulp_bf16(np.maximum(np.abs(gpu), np.abs(ref)))
    return float(np.max(np.abs(gpu - ref) - allow)) / max(rms, 1e-300)


def max_rel_rms(gpu, ref) -> float:
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(gpu - ref))) / max(rms, 1e-300)


def l2_rel(gpu, ref) -> float:
    return float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_bf16_close(gpu, ref, what=""):
    ex = bf16_excess(gpu, ref)
    log(f"  {what}: bf16 excess/rms={ex:.4g} (literal max/rms={max_rel_rms(gpu, ref):.4g}, "
        f"l2rel={l2_rel(gpu, ref):.3g})")
    assert ex <= BF16_MAX_REL_RMS, f"{what}: {ex} > {BF16_MAX_REL_RMS}"


def assert_fp32_close(gpu, ref, what="", tol=FP32_L2_REL):
    e = l2_rel(gpu, ref)
    log(f"  {what}: fp32 l2rel={e:.3g} max/rms={max_rel_rms(gpu, ref):.3g}")
    assert e <= tol, f"{what}: {e} > {tol}"


def sample_tokens(p, n=24, seed=1):
    """A spread of tokens: first, last, random, and ones routed to the most
    and least loaded experts (tile tails)."""
    rng = np.random.default_rng(seed)
    counts = np.bincount(p.topk_ids[(p.topk_ids >= 0) & (p.topk_ids < p.E)], minlength=p.E)
    hot = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    cold = int(nz[np.argmin(counts[nz])])
    pick = {0, p.T - 1}
    for e in (hot, cold):
        rows = np.nonzero((p.topk_ids == e).any(axis=1))[0]
        pick.update(rows[:2].tolist())
        pick.update(rows[-2:].tolist())
    extra = rng.choice(p.T, size=min(p.T, n), replace=False)
    for t in extra:
        if len(pick) >= n:
            break
        pick.add(int(t))
    return np.array(sorted(pick), np.int32)


def ctypes_ptr(t):
    return ctypes.c_void_p(t.data_ptr())
