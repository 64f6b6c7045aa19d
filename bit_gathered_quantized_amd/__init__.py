"""Python binding of libmoeffn, the routed 4-bit (or 8-bit) MoE expert FFN for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmoeffn.so``.  PyTorch supplies device memory and the stream.
The binding raises if the library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "MoeError", "lib", "LIB_PATH", "MOE_F_FP32_OUT", "MOE_F_FP32_INTERMEDIATE", "MOE_F_SWIGLU",
    "max_tiles", "workspace_bytes", "workspace_layout", "sort_build_tiles",
    "expert_ffn_forward", "router_topk", "status_string", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoeffn.so")

MOE_OK = 0
# kernels of one forward, in launch order; the timed forward takes a start
# and a stop event per kernel
KERNELS = ("moe_route_sort_tiles", "moe_gateup_skinny", "moe_gateup_wide", "moe_down_skinny",
           "moe_down_wide", "moe_combine")
N_EVENTS = 2 * len(KERNELS)
MOE_F_FP32_OUT = 1
MOE_F_FP32_INTERMEDIATE = 2
MOE_F_SWIGLU = 4

EXPORTED_SYMBOLS = (
    "moe_max_tiles", "moe_sort_build_tiles", "moe_ffn_workspace_bytes",
    "moe_ffn_workspace_layout", "moe_expert_ffn_forward",
    "moe_expert_ffn_forward_timed", "moe_expert_ffn_forward_presorted", "moe_router_topk",
    "moe_status_string", "moe_expert_ffn_forward_noalloc",
)
MOE_ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("k", ctypes.c_int32), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class MoeWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("counts", "offsets", "perm", "inv_perm", "tiles", "num_tiles", "x_perm", "x_sums",
                 "h", "h_sums", "y", "total")] + \
               [(n, ctypes.c_int32) for n in ("max_tiles", "bm_big", "bm_small", "max_skinny")] + \
               [("tiles_skinny", ctypes.c_size_t), ("route_hist", ctypes.c_size_t),
                ("x8_hi", ctypes.c_size_t), ("x8_lo", ctypes.c_size_t), ("x8_scales", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded HIP library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_gathered_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_max_tiles.argtypes = [i64, i32, i32]
        L.moe_max_tiles.restype = i32
        L.moe_sort_build_tiles.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, i32, P, P]
        L.moe_sort_build_tiles.restype = i32
        L.moe_ffn_workspace_bytes.argtypes = [ctypes.POINTER(MoeProblem)]
        L.moe_ffn_workspace_bytes.restype = sz
        L.moe_ffn_workspace_layout.argtypes = [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeWsLayout)]
        L.moe_ffn_workspace_layout.restype = i32
        fwd = [ctypes.POINTER(MoeProblem)] + [P] * 10 + [P, sz, P]
        L.moe_expert_ffn_forward.argtypes = fwd
        L.moe_expert_ffn_forward.restype = i32
        L.moe_expert_ffn_forward_timed.argtypes = fwd + [P]
        L.moe_expert_ffn_forward_timed.restype = i32
        L.moe_expert_ffn_forward_presorted.argtypes = fwd[:4] + [P] + fwd[4:]
        L.moe_expert_ffn_forward_presorted.restype = i32
        L.moe_expert_ffn_forward_noalloc.argtypes = [ctypes.POINTER(MoeProblem)] + [P] * 10 + [P]
        L.moe_expert_ffn_forward_noalloc.restype = i32
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_router_topk.argtypes = [P, i32, i32, i32, P, P, P]
        L.moe_router_topk.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def problem(T: int, k: int, E: int, H: int, I: int, flags: int = 0,
            group_size: int = 64, bits: int = 4) -> MoeProblem:
    return MoeProblem(T, k, E, H, I, group_size, bits, flags)


def max_tiles(A: int, E: int, bm_big: int = 32) -> int:
    return int(lib().moe_max_tiles(A, E, bm_big))


def workspace_bytes(p: MoeProblem) -> int:
    return int(lib().moe_ffn_workspace_bytes(ctypes.byref(p)))


def workspace_layout(p: MoeProblem) -> MoeWsLayout:
    lay = MoeWsLayout()
    _check(lib().moe_ffn_workspace_layout(ctypes.byref(p), ctypes.byref(lay)),
           "moe_ffn_workspace_layout")
    return lay


# ------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dev_ptr(t, name: str, itemsize: Optional[int] = None, shape: Optional[Sequence[int]] = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def router_topk(logits, k: int, ids=None, weights=None, stream=None):
    """Softmax top-k routing on the GPU: logits fp32 [T, E] -> (ids int32 [T, k],
    weights fp32 [T, k])."""
    torch = _torch()
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise ValueError("logits must be float32")
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    st = lib().moe_router_topk(_dev_ptr(logits, "logits", 4, (T, E)), T, E, k,
                               _dev_ptr(ids, "ids", 4, (T, k)),
                               _dev_ptr(weights, "weights", 4, (T, k)),
                               ctypes.c_void_p(_stream(stream)))
    if st != 0:
        raise MoeError(st, "moe_router_topk")
    return ids, weights


def sort_build_tiles(topk_ids, E: int, bm_big: int = 32, bm_small: int = 16, stream=None):
    """Route/sort/tile on the GPU.  Returns a dict of device tensors:
    counts [E], offsets [E+1], perm [A], inv_perm [A], tiles [max_tiles, 4],
    num_tiles [2] (tile count, out-of-range ids)."""
    torch = _torch()
    if topk_ids.dtype != torch.int32:
        raise ValueError("topk_ids must be int32")
    T, k = topk_ids.shape
    A = T * k
    dev = topk_ids.device
    mt = max(max_tiles(A, E, bm_big), 1)
    out = dict(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm=torch.empty(max(A, 1), dtype=torch.int32, device=dev),
        inv_perm=torch.empty(max(A, 1), dtype=torch.int32, device=dev),
        tiles=torch.empty((mt, 4), dtype=torch.int32, device=dev),
        num_tiles=torch.empty(2, dtype=torch.int32, device=dev),
    )
    st = lib().moe_sort_build_tiles(
        _dev_ptr(topk_ids, "topk_ids", 4), T, k, E, bm_big, bm_small,
        _dev_ptr(out["counts"], "counts"), _dev_ptr(out["offsets"], "offsets"),
        _dev_ptr(out["perm"], "perm"), _dev_ptr(out["inv_perm"], "inv_perm"),
        _dev_ptr(out["tiles"], "tiles"), mt, _dev_ptr(out["num_tiles"], "num_tiles"),
        ctypes.c_void_p(_stream(stream)))
    _check(st, "moe_sort_build_tiles")
    out["perm"] = out["perm"][:A]
    out["inv_perm"] = out["inv_perm"][:A]
    return out


def expert_ffn_forward(x, topk_ids, topk_weights, w_gateup, s_gateup, b_gateup,
                       w_down, s_down, b_down, *, fp32_out: bool = False,
                       fp32_intermediate: bool = False, swiglu: bool = False, out=None,
                       workspace=None, stream=None, events=None, sorted_order=None,
                       no_alloc: bool = False):
    """Expert FFN forward.  Shapes: x [T, H] (2-byte), topk_ids int32 [T, k],
    topk_weights fp32 [T, k], w_gateup 4-byte [E, 2I, H*bits/32], s/b_gateup
    2-byte [E, 2I, H/gs], w_down 4-byte [E, H, I*bits/32], s/b_down 2-byte
    [E, H, I/gs]; the code width (4 or 8 bits) is read off the weight shapes
    and the group size gs (32, 64 or 128) off the scale shapes.
    Returns out [T, H] (bf16, or fp32 with fp32_out); swiglu selects
    h = silu(g) * u instead of gelu_tanh(g) * u.  With sorted_order (int32
    [T*k], slot -> flat assignment, sorted by expert) the pre-sorted entry is
    used.  `workspace` is a uint8
    device tensor of at least workspace_bytes() bytes (allocated if None).
    With no_alloc the allocation-free entry point runs on the library's
    built-in scratch array instead (no workspace; `out` must then be given
    for the call itself to allocate nothing)."""
    torch = _torch()
    T, H = x.shape
    k = topk_ids.shape[1]
    E, I2, hw = w_gateup.shape
    I = I2 // 2
    flags = ((MOE_F_FP32_OUT if fp32_out else 0) | (MOE_F_FP32_INTERMEDIATE if fp32_intermediate else 0)
             | (MOE_F_SWIGLU if swiglu else 0))
    if w_gateup.shape[-1] * 8 == H:
        bits = 4
    elif w_gateup.shape[-1] * 4 == H:
        bits = 8
    else:
        raise ValueError(f"w_gateup has {w_gateup.shape[-1]} words per row: neither 4-bit nor 8-bit codes of H={H}")
    ng = s_gateup.shape[-1]
    if ng < 1 or H % ng:
        raise ValueError(f"s_gateup has {ng} groups per row, which does not divide H={H}")
    gs = H // ng
    p = problem(T, k, E, H, I, flags, group_size=gs, bits=bits)
    if topk_ids.dtype != torch.int32 or topk_weights.dtype != torch.float32:
        raise ValueError("topk_ids must be int32 and topk_weights float32")
    G = ng
    ptrs = [
        _dev_ptr(x, "x", 2, (T, H)),
        _dev_ptr(topk_ids, "topk_ids", 4, (T, k)),
        _dev_ptr(topk_weights, "topk_weights", 4, (T, k)),
        _dev_ptr(w_gateup, "w_gateup", 4, (E, 2 * I, H * bits // 32)),
        _dev_ptr(s_gateup, "s_gateup", 2, (E, 2 * I, G)),
        _dev_ptr(b_gateup, "b_gateup", 2, (E, 2 * I, G)),
        _dev_ptr(w_down, "w_down", 4, (E, H, I * bits // 32)),
        _dev_ptr(s_down, "s_down", 2, (E, H, I // gs)),
        _dev_ptr(b_down, "b_down", 2, (E, H, I // gs)),
    ]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32 if fp32_out else torch.bfloat16, device=x.device)
    optr = _dev_ptr(out, "out", 4 if fp32_out else 2, (T, H))
    if no_alloc:
        if workspace is not None or events is not None or sorted_order is not None:
            raise ValueError("no_alloc takes no workspace, events or sorted_order")
        st = lib().moe_expert_ffn_forward_noalloc(ctypes.byref(p), *ptrs, optr,
                                                  ctypes.c_void_p(_stream(stream)))
        _check(st, "moe_expert_ffn_forward_noalloc")
        return out
    need = workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    wptr = _dev_ptr(workspace, "workspace", 1)
    s = ctypes.c_void_p(_stream(stream))
    if sorted_order is not None:
        if events is not None:
            raise ValueError("events are not supported with sorted_order")
        if sorted_order.dtype != torch.int32:
            raise ValueError("sorted_order must be int32")
        sp = _dev_ptr(sorted_order, "sorted_order", 4, (T * k,))
        st = lib().moe_expert_ffn_forward_presorted(ctypes.byref(p), *ptrs[:3], sp, *ptrs[3:],
                                                    optr, wptr, workspace.numel(), s)
        _check(st, "moe_expert_ffn_forward_presorted")
        return out
    if events is None:
        st = lib().moe_expert_ffn_forward(ctypes.byref(p), *ptrs, optr, wptr,
                                          workspace.numel(), s)
    else:
        if len(events) != N_EVENTS:
            raise ValueError(f"events must hold {N_EVENTS} event handles")
        arr = (ctypes.c_void_p * N_EVENTS)(*[ctypes.c_void_p(int(e)) for e in events])
        st = lib().moe_expert_ffn_forward_timed(ctypes.byref(p), *ptrs, optr, wptr,
                                                workspace.numel(), s, arr)
    _check(st, "moe_expert_ffn_forward")
    return out
