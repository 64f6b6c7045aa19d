"""Python handle on the CPU oracle (``oracle/moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
loads or runs anything in this directory.

All floating-point results come back as float64 numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-O2", "-fno-fast-math",
               "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_route.argtypes = [P, i64, i32, P, P, P, P, P]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_tiles.argtypes = [P, P, i32, i32, i32, P, i64, P]
        lib.oracle_tiles.restype = ctypes.c_int
        lib.oracle_weight.argtypes = [P, P, P, i64, i64, i32, i32, i64, i64, i64]
        lib.oracle_weight.restype = dbl
        lib.oracle_gelu_tanh.argtypes = [dbl]
        lib.oracle_gelu_tanh.restype = dbl
        lib.oracle_silu.argtypes = [dbl]
        lib.oracle_silu.restype = dbl
        lib.oracle_router_topk.argtypes = [P, i32, i32, i32, P, P]
        lib.oracle_router_topk.restype = ctypes.c_int
        lib.oracle_ffn_tokens.argtypes = [i32] * 7 + [P] * 9 + [P, i32, i32, P, P, P]
        lib.oracle_ffn_tokens.restype = ctypes.c_int
        lib.oracle_ffn_all.argtypes = [i32] * 7 + [P] * 9 + [i32, P, P, P]
        lib.oracle_ffn_all.restype = ctypes.c_int
        lib.oracle_down_rows.argtypes = [i32] * 5 + [P] * 4 + [i64] + [P] * 3
        lib.oracle_down_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the following calls (timing only: every result is the same
    for any thread count)."""
    _load().oracle_set_num_threads(int(n))


def route(ids: np.ndarray, E: int):
    """Stable counting sort of the flat assignments by expert id.

    Returns (counts[E], offsets[E+1], perm[A], inv_perm[A], n_invalid).
    """
    ids = np.ascontiguousarray(ids, dtype=np.int32).ravel()
    A = ids.size
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(max(A, 1), np.int32)
    inv = np.zeros(max(A, 1), np.int32)
    bad = np.zeros(1, np.int32)
    rc = _load().oracle_route(_ptr(ids), A, E, _ptr(counts), _ptr(offsets),
                              _ptr(perm), _ptr(inv), _ptr(bad))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return counts, offsets, perm[:A], inv[:A], int(bad[0])


def tiles(counts: np.ndarray, offsets: np.ndarray, bm_big: int = 32, bm_small: int = 16):
    """Tile descriptors [n, 4] = {expert, row_begin, row_count, bm}."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = counts.size
    nt = np.zeros(1, np.int32)
    lib = _load()
    rc = lib.oracle_tiles(_ptr(counts), _ptr(offsets), E, bm_big, bm_small, None, 0, _ptr(nt))
    n = int(nt[0])
    out = np.zeros((max(n, 1), 4), np.int32)
    rc = lib.oracle_tiles(_ptr(counts), _ptr(offsets), E, bm_big, bm_small, _ptr(out), n, _ptr(nt))
    if rc != 0:
        raise ValueError(f"oracle_tiles failed ({rc})")
    return out[:n]


def forward_tiles(counts: np.ndarray, offsets: np.ndarray, bm_big: int, bm_small: int,
                  short_only: bool = False):
    """The forward's own tile lists, written out plainly: an expert of
    1..bm_small rows is one short tile; a larger one is cut into
    n = ceil(count / bm_big) tiles, tile j holding count // n rows plus one
    if j < count % n, consecutively.  With short_only (the forward's choice
    for batches of at most bm_small tokens) every expert goes to the short
    list instead, as consecutive tiles of bm_small rows, the last one
    shorter.  Returns (wide [m, 4], short [s, 4])."""
    wide, short = [], []
    for e, c in enumerate(np.asarray(counts).tolist()):
        o = int(offsets[e])
        if c == 0:
            continue
        if c <= bm_small or short_only:
            for r0 in range(0, c, bm_small):
                short.append([e, o + r0, min(bm_small, c - r0), bm_small])
            continue
        n = -(-c // bm_big)
        base, extra = divmod(c, n)
        row = o
        for j in range(n):
            r = base + (1 if j < extra else 0)
            wide.append([e, row, r, bm_big])
            row += r
    return (np.array(wide, np.int32).reshape(-1, 4), np.array(short, np.int32).reshape(-1, 4))


def weight(P: np.ndarray, S: np.ndarray, B: np.ndarray, gs: int, e: int, n: int, c: int,
           bits: int = 4) -> float:
    """One dequantised weight W[e, n, c] of a packed [E, rows, K * bits / 32] matrix."""
    E, rows, kw = P.shape
    return float(_load().oracle_weight(_ptr(P), _ptr(S), _ptr(B), rows, kw * 32 // bits, gs, bits,
                                       e, n, c))


def gelu_tanh(v: float) -> float:
    return float(_load().oracle_gelu_tanh(float(v)))


def silu(v: float) -> float:
    return float(_load().oracle_silu(float(v)))


ACTIVATIONS = {"gelu": 0, "silu": 1}


def router_topk(logits: np.ndarray, k: int):
    """Softmax top-k routing: (ids int32 [T, k], weights float64 [T, k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((max(T, 1), k), np.int32)
    w = np.zeros((max(T, 1), k))
    rc = _load().oracle_router_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError(f"oracle_router_topk failed ({rc})")
    return ids[:T], w[:T]


def ffn_tokens(p, tokens=None, want_h: bool = True, want_y: bool = True,
               want_out: bool = True, act: str = "gelu"):
    """Expert FFN for a list of tokens of problem ``p`` (a moe_synth.Problem);
    act "gelu" (GeGLU, h = gelu_tanh(g) u) or "silu" (SwiGLU, h = silu(g) u).

    Returns dict with h [n*k, I], y [n*k, H] (unweighted), out [n, H]; row
    i*k + j belongs to assignment tokens[i]*k + j.
    """
    if tokens is None:
        tokens = np.arange(p.T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = tokens.size
    h = np.zeros((n * p.k, p.I)) if want_h else None
    y = np.zeros((n * p.k, p.H)) if want_y else None
    out = np.zeros((n, p.H)) if want_out else None
    arrs = [np.ascontiguousarray(a) for a in (p.x, p.topk_ids, p.topk_weights, p.w_gateup,
                                              p.s_gateup, p.b_gateup, p.w_down, p.s_down,
                                              p.b_down)]
    assert arrs[1].dtype == np.int32 and arrs[2].dtype == np.float32
    rc = _load().oracle_ffn_tokens(p.T, p.k, p.E, p.H, p.I, p.gs, p.bits, *[_ptr(a) for a in arrs],
                                   _ptr(tokens), n, ACTIVATIONS[act], _ptr(h), _ptr(y),
                                   _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_ffn_tokens failed ({rc})")
    return dict(h=h, y=y, out=out, tokens=tokens)


def ffn_all(p, want_h: bool = True, want_y: bool = True, act: str = "gelu"):
    """Expert FFN for every assignment of problem ``p``, organised by expert
    (each expert dequantised once): the same sums in the same order as
    :func:`ffn_tokens`, hence the same bits, fast enough for a whole 16384-
    assignment batch.

    Returns dict with h [T*k, I] and y [T*k, H] (unweighted) in flat order
    a = t*k + j, and out [T, H].
    """
    A = p.T * p.k
    h = np.zeros((A, p.I)) if want_h else None
    y = np.zeros((A, p.H)) if want_y else None
    out = np.zeros((p.T, p.H))
    arrs = [np.ascontiguousarray(a) for a in (p.x, p.topk_ids, p.topk_weights, p.w_gateup,
                                              p.s_gateup, p.b_gateup, p.w_down, p.s_down,
                                              p.b_down)]
    assert arrs[1].dtype == np.int32 and arrs[2].dtype == np.float32
    rc = _load().oracle_ffn_all(p.T, p.k, p.E, p.H, p.I, p.gs, p.bits, *[_ptr(a) for a in arrs],
                                ACTIVATIONS[act], _ptr(h), _ptr(y), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_ffn_all failed ({rc})")
    return dict(h=h, y=y, out=out)


def down_rows(p, experts: np.ndarray, h: np.ndarray, want_abs: bool = True):
    """The down projection of problem ``p``'s weights for rows with a given h:
    y[r] = W_d[experts[r]] . h[r] (unweighted, fp64, ascending-n sums), and
    yabs[r] = sum_n |W_d[experts[r], :, n] h[r, n]|.  Returns (y, yabs)."""
    experts = np.ascontiguousarray(experts, dtype=np.int32).ravel()
    h = np.ascontiguousarray(h, dtype=np.float64)
    n = experts.size
    assert h.shape == (n, p.I)
    y = np.zeros((max(n, 1), p.H))
    ya = np.zeros((max(n, 1), p.H)) if want_abs else None
    rc = _load().oracle_down_rows(p.E, p.H, p.I, p.gs, p.bits, _ptr(np.ascontiguousarray(p.w_down)),
                                  _ptr(np.ascontiguousarray(p.s_down)),
                                  _ptr(np.ascontiguousarray(p.b_down)), _ptr(experts), n, _ptr(h),
                                  _ptr(y), _ptr(ya))
    if rc != 0:
        raise ValueError(f"oracle_down_rows failed ({rc})")
    return y[:n], (ya[:n] if ya is not None else None)
