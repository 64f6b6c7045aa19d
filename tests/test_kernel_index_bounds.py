"""CPU emulation of the HIP kernels' index arithmetic and work coverage.

For a routing (the tile lists of the forward's rule, `oracle.forward_tiles`,
which the GPU tests pin bit-exactly to the route kernel's output), this
recomputes, with numpy, every global-memory index and every LDS offset that
the kernels of libmoeffn form, for every work item and every thread, and
checks them against the sizes of the buffers and of the LDS structures.  It
also checks that the launch grids cover every (tile, column block) item of
both tile lists exactly once.  The formulas are transcriptions of the kernel
source (csrc/gemm_kernels.h, route.hip, combine.hip); each block below names
the function it follows.  No GPU is needed.

Buffer-resource loads (weights, scale and bias tables, bias rows) read zeros
past the resource's size without touching memory, so for them the check is
that the resource itself (base and size) lies inside its buffer.
"""
import numpy as np
import pytest

import moe_synth as ms

# --------------------------------------------------------------- constants
# (csrc/moe_internal.h, csrc/gemm_kernels.h)
K_BM_BIG, K_BM_BIG_F32, K_BM_SMALL = 64, 32, 16
K_MAX_DIM = 4096
K_THREADS = 256
K_XCDS = 8
K_ASTRIDE = 2 * 32 + 4          # u32 per staged activation row
K_ROUTE_THREADS = 1024
K_ROUTE_WAVES = 16
K_ROUTE_SEGMENT = 1024
K_ROUTE_MULTI_MIN = 2048
K_SKINNY_DOWN_BLOCKS = 2
EMU_BATCH = 256                   # items emulated at once
K_PRE_G = 22                      # down wide: group sums read in the prologue up to this many groups
K_LDS_BIAS_G = 16                 # down wide: bias rows in LDS up to this many groups


def max_groups(gs):
    return K_MAX_DIM // gs


def kchain(gs):
    return gs if gs < 64 else 64


def word(gs, s, q):
    """Geo<GS>::word: chunk word that lane group q feeds to slice s."""
    return 8 * (s >> 1) + 2 * q + (s & 1) if kchain(gs) == 64 else 4 * s + q


class Checker:
    def __init__(self, label):
        self.label = label
        self.bad = []

    def within(self, what, idx, size):
        idx = np.asarray(idx)
        if idx.size == 0:
            return
        lo, hi = int(idx.min()), int(idx.max())
        if lo < 0 or hi >= size:
            self.bad.append(f"{what}: index range [{lo}, {hi}] outside [0, {size})")

    def resource(self, what, base, nbytes, size_bytes):
        base = np.asarray(base, dtype=np.int64)
        if base.size == 0:
            return
        if int(base.min()) < 0 or int((base + nbytes).max()) > size_bytes:
            self.bad.append(f"{what}: resource [{int(base.min())}, {int((base + nbytes).max())}) "
                            f"outside [0, {size_bytes})")

    def true(self, what, cond):
        if not cond:
            self.bad.append(what)

    def done(self):
        assert not self.bad, self.label + ":\n  " + "\n  ".join(self.bad)


def wide_smem_u32(RB, P, NBUF, MAXG, BITS):
    """Sizes of WideSmem's fields: a (u32), w (u32), ts (u16), dst, wt."""
    return dict(a=NBUF * P * RB * 16 * K_ASTRIDE, a_per_buf_part=RB * 16 * K_ASTRIDE,
                w=4 * 64 * 4 * BITS, w_per_wave=64 * 4 * BITS,
                ts=4 * 64 * MAXG, ts_per_wave=64 * MAXG, dst=RB * 16)


class Setup:
    """Everything the host side (api.hip make_layout / forward_impl, the
    launchers in gemm_kernels.h) derives for one problem."""

    def __init__(self, oracle, p, fp32):
        self.p, self.fp32 = p, fp32
        self.T, self.k, self.E, self.H, self.I = p.T, p.k, p.E, p.H, p.I
        self.gs, self.bits = p.gs, p.bits
        self.A = p.T * p.k
        self.bm_big = K_BM_BIG_F32 if (fp32 or p.bits == 8) else K_BM_BIG
        self.max_tiles = self.A // self.bm_big + min(self.E, self.A)
        self.max_skinny = self.A // K_BM_SMALL + min(self.E, self.A)
        self.skinny_only = p.T <= K_BM_SMALL
        counts, offsets, perm, inv, bad = oracle.route(p.topk_ids, p.E)
        self.counts, self.offsets, self.perm = counts, offsets, perm
        self.wide, self.short = oracle.forward_tiles(counts, offsets, self.bm_big, K_BM_SMALL,
                                                     short_only=self.skinny_only)
        self.Gh, self.Gi = p.H // p.gs, p.I // p.gs
        # grids (skinny_grid / wide_grid)
        self.skinny_grid = min(self.max_skinny, min(self.E, self.A) +
                               (self.A // K_BM_SMALL if self.skinny_only else 0))
        self.wide_grid = 0 if self.skinny_only else self.max_tiles
        self.RB = (K_BM_BIG_F32 if (fp32 or p.bits == 8) else K_BM_BIG) // 16
        self.hbytes = 4 if fp32 else 2
        # buffer sizes in elements of their own type
        self.size = dict(
            ids=self.A, w=self.A, perm=self.A, inv=self.A,
            x_u32x4=p.T * p.H // 8, xs=p.T * self.Gh,
            w_gu=p.E * 2 * p.I * p.H * p.bits // 32, s_gu=p.E * 2 * p.I * self.Gh,
            w_d=p.E * p.H * p.I * p.bits // 32, s_d=p.E * p.H * self.Gi,
            tiles=4 * self.max_tiles, tiles_skinny=4 * self.max_skinny,
            h_u16=(2 if fp32 else 1) * self.A * p.I, hs=self.A * p.I // 16,
            y=self.A * p.H, out=p.T * p.H,
            hist=(-(-self.A // K_ROUTE_SEGMENT) if self.A > K_ROUTE_MULTI_MIN else 0) * (p.E + 2))
        # fp8_wide_gateup: x as e4m3 hi + lo and a scale byte per 32 columns
        self.fp8 = (p.T > K_BM_SMALL and p.bits == 4 and p.gs in (64, 128) and not fp32)
        self.S8 = (p.H // 32 + 3) // 4 * 4
        self.size.update(x8=p.T * p.H if self.fp8 else 0, x8s=p.T * self.S8 if self.fp8 else 0)

    def maxg_wide(self, K, kind="gateup"):
        big = max_groups(self.gs)
        small = 3 * big // 4
        if kind == "down" and K // self.gs <= K_LDS_BIAS_G:
            return K_LDS_BIAS_G
        return small if K // self.gs <= small else big


# ------------------------------------------------------------ work mapping
def wide_items(s, ncol):
    """wide_work over the whole grid: the (tile, column block) of each live
    workgroup."""
    nw = min(len(s.wide), s.max_tiles)
    total = nw * ncol
    grid = -(-s.wide_grid * ncol // K_XCDS) * K_XCDS if s.wide_grid else 0
    share = -(-total // K_XCDS)
    L = np.arange(grid)
    i = L // K_XCDS
    item = (L % K_XCDS) * share + i
    live = (i < share) & (item < total)
    return item[live] // ncol, item[live] % ncol, total


def skinny_items(s, ncb):
    """load_skinny_tile over the skinny grid: (tile, column block) of each live
    workgroup, and every tile index read."""
    grid = s.skinny_grid * ncb
    item = np.arange(grid)
    ti, cb = item // ncb, item % ncb
    n = min(len(s.short), s.max_skinny)
    live = ti < n
    return ti, ti[live], cb[live], n


def check_coverage(c, s):
    for name, ncol in (("gate|up wide", -(-s.I // 128)), ("down wide", -(-s.H // 256))):
        ti, col, total = wide_items(s, ncol)
        c.true(f"{name}: {len(s.wide)} wide tiles exceed max_tiles {s.max_tiles}",
               len(s.wide) <= s.max_tiles)
        hit = np.bincount(ti * ncol + col, minlength=total) if total else np.zeros(0, int)
        c.true(f"{name}: items covered {np.count_nonzero(hit == 1)} of {total} exactly once",
               total == 0 or (hit.size == total and np.all(hit == 1)))
    for name, ncb in (("gate|up skinny", s.I // 16), ("down skinny", s.H // (16 * K_SKINNY_DOWN_BLOCKS))):
        all_ti, ti, cb, n = skinny_items(s, ncb)
        c.true(f"{name}: {len(s.short)} short tiles exceed max_skinny {s.max_skinny}",
               len(s.short) <= s.max_skinny)
        c.within(f"{name}: tile entry read", 4 * all_ti + 3, s.size["tiles_skinny"])
        hit = np.bincount(ti * ncb + cb, minlength=n * ncb) if n else np.zeros(0, int)
        c.true(f"{name}: items covered exactly once", n == 0 or np.all(hit == 1))


# --------------------------------------------------------------- wide paths
def thread_ids():
    tid = np.arange(K_THREADS)
    wave, lane = tid >> 6, tid & 63
    return tid, wave, lane, lane >> 4, lane & 15


def check_wide(c, s, kind):
    """gateup_wide / down_wide with Stager, Tables, WaveW, BiasRows,
    wide_kloop, wide_bias and the epilogues."""
    p = s.p
    P = 2 if (kind == "down" and s.fp32) else 1
    NBUF = 1 if (kind == "down" and s.fp32) else 2
    RB, BITS, GS = s.RB, s.bits, s.gs
    K = s.H if kind == "gateup" else s.I    # K of the matmul
    N = 2 * s.I if kind == "gateup" else s.H  # weight rows per expert
    G = K // GS
    MAXG = s.maxg_wide(K, kind)
    sm = wide_smem_u32(RB, P, NBUF, MAXG, BITS)
    ncol = -(-s.I // 128) if kind == "gateup" else -(-s.H // 256)
    ti, by, _ = wide_items(s, ncol)
    if ti.size == 0:
        return
    # items in batches: small arrays keep the emulation's memory (and page
    # faults) low
    for b0 in range(0, ti.size, EMU_BATCH):
        _wide_batch(c, s, kind, P, NBUF, RB, BITS, GS, K, N, G, MAXG, sm, ti[b0:b0 + EMU_BATCH],
                    by[b0:b0 + EMU_BATCH])


def _wide_batch(c, s, kind, P, NBUF, RB, BITS, GS, K, N, G, MAXG, sm, ti, by):
    p = s.p
    e, rbeg, rows = (s.wide[ti, j].astype(np.int64)[:, None] for j in range(3))
    by = by.astype(np.int64)[:, None]
    tid, wave, lane, q, lr = thread_ids()
    if kind == "gateup":
        n0 = by * 128
        active = n0 + 32 * wave < s.I
        base = np.where(active, n0 + 32 * wave, 0)
        row0 = [e * 2 * s.I + base + 16 * (cb & 1) + (cb >> 1) * s.I for cb in range(4)]
    else:
        n0 = by * 256
        active = n0 + 64 * wave < s.H
        base = np.where(active, n0 + 64 * wave, 0)
        row0 = [e * s.H + base + 16 * cb for cb in range(4)]
    row_words = K // 32 * BITS
    wbuf, sbuf = ("w_gu", "s_gu") if kind == "gateup" else ("w_d", "s_d")
    for cb in range(4):
        # Tables::load and BiasRows::load: 16 rows of G bf16 from row0
        c.resource(f"{kind} wide: scale/bias table rows", row0[cb] * G * 2, 32 * G, s.size[sbuf] * 2)
        # WaveW::init: 16 weight rows of row_words u32
        c.resource(f"{kind} wide: weight block", row0[cb] * row_words * 4, 64 * row_words,
                   s.size[wbuf] * 4)
        c.within(f"{kind} wide: weight row", row0[cb] + 15, N * s.E)
    # activation rows staged by thread t: rows (t >> 4) + 16 i
    r = (tid >> 4)[None, :, None] + 16 * np.arange(RB)[None, None, :]
    srow = rbeg[:, :, None] + np.minimum(r, rows[:, :, None] - 1)
    c.within(f"{kind} wide: sorted row of a staged activation", srow, s.A)
    pc = tid & 15
    nh = K // 64
    nch = -(-K // 128)
    for cc in (0, nch - 1):
        hf = np.minimum(2 * cc + (pc >> 3), nh - 1)
        piece = 8 * hf + (pc & 7)  # 16-byte piece of the row
        if kind == "gateup":
            tok = s.perm[srow] // s.k
            c.within("gate|up wide: token of a staged row", tok, s.T)
            c.within("gate|up wide: x_perm piece", tok * (K // 8) + piece[None, :, None], s.size["x_u32x4"])
        else:
            for pp in range(P):
                u16 = pp * s.A * s.I + srow * s.I + 8 * piece[None, :, None] + 7
                c.within("down wide: h piece", u16, s.size["h_u16"])
    # Stager::store and lds_frag: rows below RB * 16, pieces below 16
    c.true("wide: staged activation row stays in its buffer",
           (RB * 16 - 1) * K_ASTRIDE + 4 * 15 + 3 < sm["a_per_buf_part"])
    # Tables::store into ts[wave] (and, down with G <= kLdsBiasG, tb[wave] of
    # the same size): entries cb * 16 G + 8 idx + 7, idx < 2 G
    c.true("wide: scale table fits", 3 * 16 * G + 8 * (2 * G - 1) + 7 < sm["ts_per_wave"])
    if kind == "down" and G <= K_LDS_BIAS_G:
        c.true("down wide: bias table fits", 3 * 16 * G + 8 * (2 * G - 1) + 7 < 64 * MAXG)
        # bias_from_table reads 8 entries from (16 cb + lr) G + 8 q + 32 st of the
        # wave's rows (masked past G): at most 32 entries past the last row,
        # inside the struct (the next wave's rows, or the group sums after)
        c.true("down wide: bias table reads", 63 * G + 8 * 3 + 32 * (-(-G // 32) - 1) + 7 < 64 * MAXG + 32)
    # WaveW put/get rows: 64 rows of 16 * (BITS / 4) u32
    c.true("wide: weight transpose buffer", 64 * 16 * (BITS // 4) <= sm["w_per_wave"])
    # BiasRows::store into the wave's weight buffer (as u16): 16 rows of G
    c.true("wide: bias rows fit the wave's buffer", 8 * (2 * G - 1) + 7 < 2 * sm["w_per_wave"])
    # wide_bias: group sums in a[0][0] with row stride XS = kMaxG + 4 floats
    XS = max_groups(GS) + 4
    c.true("wide: group sums fit the activation buffer", RB * 16 * XS <= sm["a"])
    steps = -(-G // 32)
    c.true("wide: row operand reads stay in the row", 32 * (steps - 1) + 31 < XS)
    if kind == "gateup":
        tok = s.perm[srow] // s.k
        c.within("gate|up wide: x group sums", tok * G + (G - 1), s.size["xs"])
        # epilogue (store_h): rows r < rows, columns hbase + 16 half + lr
        rr = 16 * np.arange(RB)[:, None] + 4 * q[None, :]  # [RB, 256] (v = 0..3 added)
        for v in range(4):
            rowv = rr + v
            ok = (rowv[None] < rows[:, None, :]) & active[:, None, :]
            srow_e = rbeg[:, None, :] + rowv[None]
            for half in range(2):
                hcol = base[:, None, :] + 16 * half + lr[None, None, :]
                pos = srow_e * s.I + hcol
                if s.fp32:
                    pos = pos + s.A * s.I
                c.within("gate|up wide: h store", np.where(ok, pos, 0), s.size["h_u16"])
                c.within("gate|up wide: h column", np.where(ok, hcol, 0), s.I)
                hs = srow_e * (s.I // 16) + base[:, None, :] // 16 + half
                c.within("gate|up wide: h block sums store", np.where(ok, hs, 0), s.size["hs"])
    else:
        # destinations and weights of the rows (tid < RB * 16)
        dsrc = rbeg + np.minimum(tid[None, :], rows - 1)
        c.within("down wide: destination read", np.where(tid[None, :] < RB * 16, dsrc, 0), s.A)
        c.within("down wide: h block sums", srow * (s.I // 16) + (GS // 16) * (G - 1) + GS // 16 - 1,
                 s.size["hs"])
        if G <= K_PRE_G:
            # the same sums read in the prologue into DownSmem::xg (entry
            # idx = row * G + g of RB * 16 * kPreG), read back per staged row
            idx = tid[:, None] + 256 * np.arange(-(-RB * 16 * K_PRE_G // 256))[None, :]
            ok = idx < RB * 16 * G
            c.within("down wide: prefetched sum row", np.where(ok, idx // G, 0), RB * 16)
            c.within("down wide: prefetched sum entry", np.where(ok, idx, 0), RB * 16 * K_PRE_G)
            c.within("down wide: prefetched sum read", ((tid >> 4)[:, None] + 16 * np.arange(RB)[None, :]) * G + G - 1,
                     RB * 16 * K_PRE_G)
        rr = 16 * np.arange(RB)[:, None] + 4 * q[None, :]
        for v in range(4):
            rowv = rr + v
            ok = (rowv[None] < rows[:, None, :]) & active[:, None, :]
            dst = s.perm[np.where(ok, rbeg[:, None, :] + rowv[None], 0)]
            for cb in range(4):
                col = base[:, None, :] + lr[None, None, :] + 16 * cb
                c.within("down wide: y store", np.where(ok, dst * s.H + col, 0), s.size["y"])
                c.within("down wide: y column", np.where(ok, col, 0), s.H)


# ------------------------------------------------------------- skinny paths
def check_skinny(c, s, kind):
    """moe_gateup_skinny / moe_down_skinny (Tables, WaveW, load_a, RowSums,
    store_h, the weighted unsort)."""
    p = s.p
    GS, BITS = s.gs, s.bits
    if kind == "gateup":
        NB, ncb, K, N = 2, s.I // 16, s.H, 2 * s.I
    else:
        NB, ncb, K, N = K_SKINNY_DOWN_BLOCKS, s.H // (16 * K_SKINNY_DOWN_BLOCKS), s.I, s.H
    G = K // GS
    _, ti, cb, _ = skinny_items(s, ncb)
    if ti.size == 0:
        return
    for b0 in range(0, ti.size, EMU_BATCH):
        _skinny_batch(c, s, kind, GS, BITS, NB, ncb, K, N, G, ti[b0:b0 + EMU_BATCH], cb[b0:b0 + EMU_BATCH])


def _skinny_batch(c, s, kind, GS, BITS, NB, ncb, K, N, G, ti, cb):
    p = s.p
    e, rbeg, rows = (s.short[ti, j].astype(np.int64)[:, None] for j in range(3))
    cb = cb.astype(np.int64)[:, None]
    lane = np.arange(64)
    q, lr = lane >> 4, lane & 15
    row_words = K // 32 * BITS
    MAXG = max_groups(GS)
    wbuf, sbuf = ("w_gu", "s_gu") if kind == "gateup" else ("w_d", "s_d")
    if kind == "gateup":
        hcol0 = cb * 16
        row0 = [e * 2 * s.I + hcol0, e * 2 * s.I + hcol0 + s.I]
    else:
        cbase = cb * 16 * NB
        nb = np.minimum(NB, (s.H - cbase) // 16)
        row0 = [e * s.H + cbase + 16 * np.minimum(b, nb - 1) for b in range(NB)]
    for b in range(NB):
        c.resource(f"{kind} skinny: scale/bias table rows", row0[b] * G * 2, 32 * G, s.size[sbuf] * 2)
        c.resource(f"{kind} skinny: weight block", row0[b] * row_words * 4, 64 * row_words,
                   s.size[wbuf] * 4)
        c.within(f"{kind} skinny: weight row", row0[b] + 15, N * s.E)
    # SkinnySmem: w [NB * 16 * 4 * BITS] u32, ts/tb [NB * 16 * MAXG] u16, dst/wt [16]
    c.true("skinny: table store fits", (NB - 1) * 16 * G + 8 * (2 * G - 1) + 7 < NB * 16 * MAXG)
    # bias_from_table: lane q reads entries 8 q + 32 st + [0, 8) of every row
    # of both tables for st < ceil(G / 32), masked at or past G: the reads of
    # tb's last row go up to 62 bytes past its G entries and must stay inside
    # the struct (tb's spare entries, then dst/wt)
    steps = -(-G // 32)
    last_read = NB * 16 * MAXG + (NB * 16 - 1) * G + 8 * 3 + 32 * (steps - 1) + 7  # u16 past ts
    c.within("skinny: bias table read (u16 past ts)", last_read, 2 * NB * 16 * MAXG + 2 * 16 * 2)
    arow = rbeg + np.minimum(lr[None, :], rows - 1)  # the lane's activation row
    c.within(f"{kind} skinny: sorted row", arow, s.A)
    kc64 = kchain(GS) == 64
    last = 32 * (K // 64 - 1) + (8 * 3 + 4 + 3 if kc64 else 4 * 3 + 16 + 3)
    if kind == "gateup":
        tok = s.perm[arow] // s.k
        c.within("gate|up skinny: token", tok, s.T)
        c.within("gate|up skinny: x_perm u32", tok * (s.H // 2) + last, s.size["x_u32x4"] * 4)
        c.within("gate|up skinny: x group sums", tok * G + (G - 1), s.size["xs"])
        for v in range(4):
            rr = 4 * q + v
            ok = rr[None, :] < rows
            srow = rbeg + rr[None, :]
            pos = srow * s.I + hcol0 + lr[None, :]
            if s.fp32:
                pos = pos + s.A * s.I
            c.within("gate|up skinny: h store", np.where(ok, pos, 0), s.size["h_u16"])
            c.within("gate|up skinny: h block sums", np.where(ok, srow * (s.I // 16) + cb, 0), s.size["hs"])
    else:
        P = 2 if s.fp32 else 1
        for pp in range(P):
            c.within("down skinny: h u32", pp * s.A * (s.I // 2) + arow * (s.I // 2) + last,
                     s.size["h_u16"] // 2)
        c.within("down skinny: h block sums", arow * (s.I // 16) + (GS // 16) * G - 1, s.size["hs"])
        dsrc = rbeg + np.minimum(lane[None, :16], rows - 1)
        c.within("down skinny: destination read", dsrc, s.A)
        for v in range(4):
            rr = 4 * q + v
            ok = rr[None, :] < rows
            dst = s.perm[np.where(ok, rbeg + rr[None, :], 0)]
            for b in range(NB):
                col = cbase + lr[None, :] + 16 * b
                okb = ok & (b < nb)
                c.within("down skinny: y store", np.where(okb, dst * s.H + col, 0), s.size["y"])


# ------------------------------------------------------------ route, combine
def check_route_and_combine(c, s):
    """launch_route / prepare_x / emit_tiles and moe_combine."""
    p = s.p
    E = s.E
    nkeys = E + 1
    lds_words = K_ROUTE_WAVES * nkeys + nkeys + 3 * (nkeys + 1) + K_ROUTE_WAVES + 1
    # s_tab [waves][nkeys] then s_cnt, s_off, s_toff, s_soff, s_wsum
    c.true("route: LDS layout fits", K_ROUTE_WAVES * nkeys + nkeys + 3 * (nkeys + 1) + K_ROUTE_WAVES + 1
           <= lds_words)
    # two lists: s_ns = s_tab + nkeys holds E entries
    c.true("route: per-list tile counts fit s_tab", 2 * nkeys <= K_ROUTE_WAVES * nkeys)
    # block_exclusive_scan handles n <= 2 * 1024 entries
    c.true("route: scan length", nkeys <= 2 * K_ROUTE_THREADS)
    # prepare_x: thread piece index below T * H / 8, group sum index p / lanes
    lanes = s.gs // 8
    n_pieces = s.T * s.H // 8
    prep = -(-n_pieces // K_ROUTE_THREADS)
    pieces = np.arange(prep * K_ROUTE_THREADS)
    live = pieces < n_pieces
    c.within("route: prepare_x piece", pieces[live], s.size["x_u32x4"])
    c.within("route: prepare_x group sum", pieces[live] // lanes, s.size["xs"])
    count_wgs = -(-s.A // K_ROUTE_SEGMENT) if s.A > K_ROUTE_MULTI_MIN else 0
    if count_wgs:
        ai = np.arange(count_wgs * K_ROUTE_SEGMENT)
        c.within("route: assignment read", ai[ai < s.A], s.A)
        # the extra scatter workgroup sums hist [count_wgs][nkeys] for the tile lists
        w, kk = np.meshgrid(np.arange(count_wgs), np.arange(nkeys), indexing="ij")
        c.within("route: emitter hist read", w * nkeys + kk, s.size["hist"])
        # pre-sorted entry: slot s reads order[s] and order[s + 1] (s + 1 < A),
        # writes inv_perm only for an assignment in range, and one status per
        # segment after hist
        sl = ai[ai < s.A]
        c.within("route: order read", np.minimum(sl + 1, s.A - 1), s.A)
        c.within("route: segment status", count_wgs * nkeys + np.arange(count_wgs), s.size["hist"])
    if s.A <= 64:
        # one row of keys: wave 1's counts, offsets and emit scratch inside s_tab
        used = nkeys + (nkeys + 1) + 2 * nkeys + 2 * (nkeys + 1)
        c.true("route: wave 1 scratch fits s_tab", used <= K_ROUTE_WAVES * nkeys)
    if len(s.wide):
        c.within("route: wide tile store", 4 * (min(len(s.wide), s.max_tiles) - 1) + 3, s.size["tiles"])
    if len(s.short):
        c.within("route: short tile store", 4 * (min(len(s.short), s.max_skinny) - 1) + 3,
                 s.size["tiles_skinny"])
    # combine: thread (t, c4), slot rows t * k + min(j, k - 1)
    t = np.arange(s.T)
    j = np.arange(-(-s.k // 8) * 8)
    asg = t[:, None] * s.k + np.minimum(j[None, :], s.k - 1)
    c.within("combine: ids read", asg, s.A)
    c.within("combine: y read", asg * s.H + s.H - 1, s.size["y"])
    c.within("combine: out store", (s.T - 1) * s.H + s.H - 1, s.size["out"])


K_FP8_SMEM_SW = 2 * 64                  # GateupFp8Smem::sw8, u32


def check_fp8_gateup(c, s):
    """prepare_x's fp8 split (route.hip) and gateup_wide_fp8 with Stager8,
    put_fp8 / get_fp8, wide_bias_fp8 (csrc/gemm_kernels.h)."""
    if not s.fp8:
        return
    T, H = s.T, s.H
    # prepare_x: piece p (8 columns) writes bytes 8p .. 8p + 7 of hi and lo,
    # and the first of every 4 pieces one scale byte t * S8 + block
    pieces = np.arange(T * H // 8)
    c.within("x8: hi/lo piece store", 8 * pieces + 7, s.size["x8"])
    t = pieces // (H // 8)
    blk = (pieces - t * (H // 8)) // 4
    c.within("x8: scale store", t * s.S8 + blk, s.size["x8s"])
    c.true("x8: the scale row holds every block", H // 32 <= s.S8 and s.S8 % 4 == 0)
    ti, by, _ = wide_items(s, -(-s.I // 128))
    if ti.size == 0:
        return
    nh, nch = H // 64, -(-H // 128)
    # Stager8: row token tok, chunk c: hi/lo bytes at 64 min(2c + h, nh - 1) + 16 q .. + 15
    cc = np.arange(nch)
    col_last = 64 * np.minimum(2 * cc + 1, nh - 1) + 16 * 3 + 15
    c.within("fp8 gate|up: x8 row read", int(col_last.max()), H)
    c.within("fp8 gate|up: scale word read (bytes)", 4 * (nch - 1) + 3, s.S8)
    tok = s.perm[s.wide[ti, 1].astype(np.int64) + np.minimum(63, s.wide[ti, 2].astype(np.int64) - 1)] // s.k
    c.within("fp8 gate|up: token", tok, T)
    # LDS: staged rows 0..63, pieces 0..15 (hi 0..7, lo 8..15); the MFMA reads
    # pieces 4 j + kh, + 2 and 8 + those; scale words sw8[buf][0..63]
    j, kh = np.meshgrid(np.arange(2), np.arange(2), indexing="ij")
    c.within("fp8 gate|up: activation piece read", 10 + 4 * j + kh, 16)
    c.within("fp8 gate|up: staged row read", 32 + 31, 64)
    c.true("fp8 gate|up: scale words fit", 64 <= K_FP8_SMEM_SW // 2)
    # weights: row 16 cb + lane / 4 (< 64), slot (2 (pc / 2) + {0, 1}) ^ ((r >> 1) & 3) < 4,
    # 16 u32 per row: the wave's 64 x 16 u32 buffer
    r = np.arange(64)[:, None]
    pc = np.arange(4)[None, :]
    for s0 in (2 * (pc >> 1), 2 * (pc >> 1) + 1):
        c.within("fp8 gate|up: weight slot store", 16 * r + 4 * (s0 ^ ((r >> 1) & 3)) + 2 * (pc & 1) + 1, 64 * 16)
    c.within("fp8 gate|up: weight slot read", 16 * 63 + 4 * 3 + 3, 64 * 16)
    # bias rows of the four blocks in the scale table: 64 rows of G (G <= MAXG)
    maxg = s.maxg_wide(H, "gateup")
    c.true("fp8 gate|up: bias rows fit the scale table", 64 * s.Gh <= 64 * maxg)
    ns = -(-max_groups(s.gs) // 16)
    xs_stride = max_groups(s.gs) + 4
    c.within("fp8 gate|up: group sum read", 63 * xs_stride + 16 * ns - 1, 64 * xs_stride)


def check_problem(oracle, p, fp32):
    s = Setup(oracle, p, fp32)
    c = Checker(f"{p.name} fp32={fp32} gs={p.gs} bits={p.bits}")
    check_coverage(c, s)
    for kind in ("gateup", "down"):
        check_skinny(c, s, kind)
        check_wide(c, s, kind)
    check_fp8_gateup(c, s)
    check_route_and_combine(c, s)
    c.done()
    return s


def _problem(name, gs=64, bits=4, I=None):
    cfg = ms.CONFIGS[name]
    return ms.make_problem(cfg["E"], cfg["H"], I or cfg["I"], cfg["T"], cfg["k"], seed=0,
                           router=cfg["router"], gs=gs, bits=bits, name=name, routing_only=True)


@pytest.mark.parametrize("name", ms.CONFIG_ORDER)
@pytest.mark.parametrize("fp32", [False, True])
def test_named_workloads(oracle_lib, name, fp32):
    """The five workloads (8192 assignments included), both modes."""
    check_problem(oracle_lib, ms.make_config(name, routing_only=True), fp32)


@pytest.mark.parametrize("gs,bits,I", [(32, 4, 704), (128, 4, 768), (64, 8, 704), (32, 8, 704),
                                       (128, 8, 768)])
@pytest.mark.parametrize("name", ["decode", "prefill8k", "prefill16k"])
@pytest.mark.parametrize("fp32", [False, True])
def test_other_geometries(oracle_lib, gs, bits, I, name, fp32):
    check_problem(oracle_lib, _problem(name, gs, bits, I), fp32)


@pytest.mark.parametrize("fp32,bits", [(False, 4), (True, 4), (False, 8)])
def test_every_expert_33_rows(oracle_lib, fp32, bits):
    """Tiles of 17 and 16 rows at bm_big = 32: more wide tiles than A / 17,
    all covered by the grid."""
    E, T, k = 128, 528, 8
    ids = (np.arange(T * k, dtype=np.int32) % E).reshape(T, k)
    p = ms.make_problem(E, 2816, 704, T, k, seed=34, topk_ids=ids, bits=bits, name="e33", routing_only=True)
    s = check_problem(oracle_lib, p, fp32)
    assert len(s.wide) == (2 * E if s.bm_big == 32 else E)
    if s.bm_big == 32:
        # the former grid, min(max_tiles, A / 17) tiles' worth, leaves items out
        s.wide_grid = min(s.max_tiles, s.A // 17)
        c = Checker("former grid")
        check_coverage(c, s)
        assert any("exactly once" in b for b in c.bad)


@pytest.mark.parametrize("c_rows", list(range(17, 300)))
def test_wide_tile_count_bound_every_expert_size(oracle_lib, c_rows):
    """For every expert size the wide list stays within max_tiles and the
    grid covers it (E experts all of c_rows rows, both tile heights)."""
    E = 4
    counts = np.full(E, c_rows, np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(offsets[-1])
    for bm in (K_BM_BIG, K_BM_BIG_F32):
        wide, _ = oracle_lib.forward_tiles(counts, offsets, bm, K_BM_SMALL)
        max_tiles = A // bm + min(E, A)
        assert len(wide) <= max_tiles
        assert wide[:, 2].min() >= (16 if bm == 32 else 17)


def test_invalid_ids_and_tiny_batches(oracle_lib):
    p = ms.make_config("tiny", routing_only=True)
    p.topk_ids[3, 0] = p.E
    p.topk_ids[10, 1] = -1
    check_problem(oracle_lib, p, False)
    for T in (1, 5, 16, 17):
        q = ms.make_problem(128, 2816, 704, T, 8, seed=T, name=f"T{T}", routing_only=True)
        check_problem(oracle_lib, q, False)
        check_problem(oracle_lib, q, True)


def test_checker_catches_a_planted_overrun(oracle_lib):
    """The emulation is not vacuous: the same formulas with a wide grid for
    half the tiles, or a y index one row too far, are reported."""
    p = ms.make_config("prefill4k", routing_only=True)
    s = Setup(oracle_lib, p, False)
    c = Checker("planted grid")
    s.wide_grid = len(s.wide) // 2
    check_coverage(c, s)
    assert any("exactly once" in b for b in c.bad)
    c = Checker("planted y")
    c.within("y", s.A * s.H, s.size["y"])
    assert c.bad
