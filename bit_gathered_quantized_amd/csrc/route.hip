// Route / sort / tile kernel: one workgroup of 1024 threads (16 waves).
//
// Prior art: the descriptor builder of the Layr-Labs/mlx PR #4 page ("What"),
// which runs on one 128-thread threadgroup over *pre-sorted* expert indices:
// a binary search of each expert's range, a Hillis-Steele exclusive scan of
// per-expert tile counts and a strided upper-bound emission of the tiles.
// Here the input is the raw top-k id array, so the kernel also sorts:
//
//   1. each wave owns a contiguous segment of the assignments and counts the
//      keys in it with LDS atomic adds (counts do not depend on their order);
//   2. per-key totals and an exclusive scan give counts and offsets, and a
//      scan over waves gives each (wave, key) its first sorted slot;
//   3. each wave walks its segment again in order and scatters every
//      assignment to base + (rank among equal keys in lower lanes, from a
//      wave match-any: one ballot per key bit): a stable counting sort;
//   4. tiles per expert = ceil(count / bm_big), scanned; thread i emits tile i
//      after an upper-bound search of the scanned tile offsets.  The forward
//      asks for two lists instead, with balanced tiles: experts of at most
//      bm_small rows get one short tile, larger experts ceil(count / bm_big)
//      tiles of near-equal size, so that each matmul launch only covers its
//      own tiles and no expert's weights are read again for a short tail.
//
// In the forward, the other workgroups of the same launch prepare the
// activations for the matmuls (prepare_x).
//
// Keys are expert ids; ids outside [0, E) get key E, which sorts after all
// experts and gets no tiles.
#include "moe_internal.h"

namespace moe {
namespace {


constexpr int kBatch = 16;  // rows of 64 keys loaded ahead per wave

// Sort key of assignment ai: its expert id, or E for an out-of-range id.
__device__ __forceinline__ uint32_t load_key(const RouteArgs& a, int ai, int end, int E) {
    if (ai >= end) return 0;
    const int32_t id = a.ids[ai];
    return (id >= 0 && id < E) ? static_cast<uint32_t>(id) : static_cast<uint32_t>(E);
}

// Lanes of the wave whose key equals this lane's key, among `active` lanes.
__device__ __forceinline__ uint64_t match_any(uint32_t key, int nbits, uint64_t active) {
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// Exclusive scan of in[0, n) into out[0, n], out[n] = total.  n <= 2 * 1024.
// Every thread of the block must call it.
__device__ void block_exclusive_scan(const int32_t* in, int32_t* out, int n, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = 2 * tid, i1 = 2 * tid + 1;
    const int32_t v0 = i0 < n ? in[i0] : 0;
    const int32_t v1 = i1 < n ? in[i1] : 0;
    const int32_t s = v0 + v1;
    int32_t inc = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t t = __shfl_up(inc, d);
        if (lane >= d) inc += t;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const int32_t w = lane < kRouteWaves ? wsum[lane] : 0;
        int32_t winc = w;
#pragma unroll
        for (int d = 1; d < kRouteWaves; d <<= 1) {
            const int32_t t = __shfl_up(winc, d);
            if (lane >= d) winc += t;
        }
        if (lane < kRouteWaves) wsum[lane] = winc - w;
        if (lane == kRouteWaves - 1) wsum[kRouteWaves] = winc;
    }
    __syncthreads();
    const int32_t excl = inc - s + wsum[wave];
    if (i0 < n) out[i0] = excl;
    if (i1 < n) out[i1] = excl + v0;
    if (tid == 0) out[n] = wsum[kRouteWaves];
    __syncthreads();
}

// The same by one wave alone (lane l scans a contiguous run of n / 64 entries);
// in and out must not overlap.
__device__ void wave_exclusive_scan(const int32_t* in, int32_t* out, int n) {
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) / 64;
    const int b = min(n, lane * per), e = min(n, b + per);
    int32_t s = 0;
    for (int i = b; i < e; ++i) s += in[i];
    int32_t inc = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t t = __shfl_up(inc, d);
        if (lane >= d) inc += t;
    }
    int32_t run = inc - s;
    for (int i = b; i < e; ++i) {
        const int32_t v = in[i];
        out[i] = run;
        run += v;
    }
    if (lane == 63) out[n] = inc;
}

// Activation preparation, run by workgroups 1.. of the same launch: x in MFMA
// operand order (each 8-column piece reordered by permute8) and the fp32 sum
// of each (token, quantisation group), which the matmuls use for the bias
// term.  Thread p handles piece p of the [T, H/8] piece grid; the gs/8 pieces
// of a group are that many consecutive lanes (gs divides H, so a group never
// straddles two rows).
// Four values (already scaled) as e4m3 hi bytes (.x) and the e4m3 bytes of
// their remainders v - hi (.y), value i in byte i, rounded to nearest even.
__device__ __forceinline__ uint2 fp8_quad(float v0, float v1, float v2, float v3) {
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, h, true);
    int l = __builtin_amdgcn_cvt_pk_fp8_f32(v0 - __builtin_amdgcn_cvt_f32_fp8(h, 0),
                                            v1 - __builtin_amdgcn_cvt_f32_fp8(h, 1), 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32(v2 - __builtin_amdgcn_cvt_f32_fp8(h, 2),
                                        v3 - __builtin_amdgcn_cvt_f32_fp8(h, 3), l, true);
    return make_uint2(static_cast<uint32_t>(h), static_cast<uint32_t>(l));
}

__device__ void prepare_x(const RouteArgs& a, int block) {
    const int pieces_per_row = a.H / 8;
    const int lanes = a.gs / 8;  // 4, 8 or 16
    const int64_t p = static_cast<int64_t>(block) * kRouteThreads + threadIdx.x;
    const int64_t total = static_cast<int64_t>(a.T) * pieces_per_row;
    const bool ok = p < total;
    u32x4 v = {0, 0, 0, 0};
    if (ok) v = reinterpret_cast<const u32x4*>(a.x)[p];
    float s = sum8_bf16(v);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (lanes >= 8) s += __shfl_xor(s, 4);
    if (lanes >= 16) s += __shfl_xor(s, 8);
    // x as e4m3 hi + lo (fp8 wide path): the block of 32 columns (4 lanes)
    // takes the scale 2^e with max |x| * 2^-e in [128, 256) (e4m3 holds up to
    // 448); hi = e4m3(x 2^-e) to nearest even, lo = e4m3(x 2^-e - hi), exact
    // down to |x 2^-e| = 1/4 (the remainder has at most 4 significant bits)
    float m = 0.f;
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(static_cast<uint16_t>(v[i] & 0xFFFFu));
        f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(v[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    if (!ok) return;
    reinterpret_cast<u32x4*>(a.xp)[p] = permute8(v);
    if ((p & (lanes - 1)) == 0) a.xs[p / lanes] = s;
    if (a.x8hi != nullptr) {
        int ex = 0;
        if (m > 0.f) {
            (void)frexpf(m, &ex);
            ex -= 8;
        }
        ex = min(max(ex, -127), 127);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = ldexpf(f[i], -ex);
        // piece order 0,2,4,6 | 1,3,5,7: the even and odd nibbles of a code word
        const uint2 ev = fp8_quad(f[0], f[2], f[4], f[6]), od = fp8_quad(f[1], f[3], f[5], f[7]);
        reinterpret_cast<u32x2*>(a.x8hi)[p] = u32x2{ev.x, od.x};
        reinterpret_cast<u32x2*>(a.x8lo)[p] = u32x2{ev.y, od.y};
        if ((p & 3) == 0) {
            const int64_t t = p / pieces_per_row, blk = (p - t * pieces_per_row) / 4;
            a.x8s[t * x8_stride(a.H) + blk] = static_cast<uint8_t>(127 + ex);
        }
    }
}

// Key of flat assignment a (its expert id, or E for an out-of-range id).
__device__ __forceinline__ int32_t key_of(const RouteArgs& a, int32_t ai) {
    const int32_t id = a.ids[ai];
    return (id >= 0 && id < a.E) ? id : a.E;
}

// A caller's sorted order: every slot names an assignment in [0, A) and the
// keys along it never decrease (the adjacent-pair scan of the Layr-Labs/mlx
// PR #4 page's fail-safe, "Deep-review round": a strided scan of adjacent
// pairs holds exactly when the whole order is non-decreasing).  Every thread
// of the block calls it.
__device__ bool presorted_order_ok(const RouteArgs& a) {
    const int A = a.A;
    bool ok = true;
    for (int s = threadIdx.x; s < A; s += kRouteThreads) {
        const int32_t a0 = a.presorted[s];
        if (a0 < 0 || a0 >= A) {
            ok = false;
            continue;
        }
        if (s + 1 < A) {
            const int32_t a1 = a.presorted[s + 1];
            if (a1 < 0 || a1 >= A || key_of(a, a0) > key_of(a, a1)) ok = false;
        }
    }
    return __syncthreads_and(ok);
}

// First index in [0, n) with v[index] > x (v ascending), n if none.
__device__ __forceinline__ int upper_bound(const int32_t* v, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (v[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ void write_tile(int32_t* t, int e, int row_begin, int rows, int bm) {
    t[0] = e;
    t[1] = row_begin;
    t[2] = rows;
    t[3] = bm;
}

// Counts, offsets and the tile lists from the per-key totals (s_cnt) and
// their exclusive scan (s_off), by NT threads: the whole block, or one wave
// (NT = 64, no barriers).
template <int NT>
__device__ void emit_tiles(const RouteArgs& a, int32_t* s_tab, const int32_t* s_cnt, const int32_t* s_off,
                           int32_t* s_toff, int32_t* s_soff, int32_t* s_wsum, int32_t order_status) {
    static_assert((NT & (NT - 1)) == 0, "NT: a power of two");
    const int tid = static_cast<int>(threadIdx.x) & (NT - 1), E = a.E, nkeys = E + 1;
    auto sync = [] {
        if constexpr (NT == 64) __builtin_amdgcn_wave_barrier(); else __syncthreads();
    };
    auto scan = [&](const int32_t* in, int32_t* out, int n) {
        if constexpr (NT == 64) {
            wave_exclusive_scan(in, out, n);
            __builtin_amdgcn_wave_barrier();
        } else {
            block_exclusive_scan(in, out, n, s_wsum);
        }
    };
    for (int e = tid; e < E; e += NT) {
        a.counts[e] = s_cnt[e];
        a.offsets[e] = s_off[e];
    }
    if (tid == 0) {
        a.offsets[E] = s_off[E];
        a.num_tiles[1] = s_cnt[E];
        if (a.presorted != nullptr) a.num_tiles[4] = order_status;
    }
    sync();
    if (a.tiles_skinny == nullptr) {
        // one list in expert order: tiles per expert into s_tab's first row
        // (no longer needed), scan, upper-bound emission
        for (int e = tid; e < E; e += NT) s_tab[e] = (s_cnt[e] + a.bm_big - 1) / a.bm_big;
        sync();
        scan(s_tab, s_toff, E);
        const int total = s_toff[E];
        for (int i = tid; i < total && i < a.max_tiles; i += NT) {
            const int e = upper_bound(s_toff, E + 1, i) - 1;
            const int row0 = (i - s_toff[e]) * a.bm_big;
            const int rows = min(a.bm_big, s_cnt[e] - row0);
            write_tile(a.tiles + 4 * i, e, s_off[e] + row0, rows,
                       rows <= a.bm_small ? a.bm_small : a.bm_big);
        }
        if (tid == 0) a.num_tiles[0] = total;
    } else {
        // two lists, each in expert order.  An expert of at most bm_small rows
        // is one short tile; a larger one is cut into ceil(c / bm_big) tiles
        // of near-equal size (the first c % n one row longer), every one of
        // them above bm_small rows: no expert ends in a short tail that would
        // read its weights once more for a few rows.
        // Experts of more than skinny_max_rows rows are wide (normally
        // skinny_max_rows = bm_small; when it is larger, the short list holds
        // consecutive tiles of bm_small rows, the last one shorter).
        int32_t* s_ns = s_tab + nkeys;
        for (int e = tid; e < E; e += NT) {
            const int c = s_cnt[e];
            const bool wide = c > a.skinny_max_rows;
            s_tab[e] = wide ? (c + a.bm_big - 1) / a.bm_big : 0;
            s_ns[e] = wide ? 0 : (c + a.bm_small - 1) / a.bm_small;
        }
        sync();
        scan(s_tab, s_toff, E);
        scan(s_ns, s_soff, E);
        const int nw = s_toff[E], ns = s_soff[E];
        for (int i = tid; i < nw && i < a.max_tiles; i += NT) {
            const int e = upper_bound(s_toff, E + 1, i) - 1;
            const int c = s_cnt[e], n = s_toff[e + 1] - s_toff[e], j = i - s_toff[e];
            const int base = c / n, extra = c - base * n;
            const int row0 = j * base + min(j, extra);
            write_tile(a.tiles + 4 * i, e, s_off[e] + row0, base + (j < extra ? 1 : 0), a.bm_big);
        }
        for (int i = tid; i < ns && i < a.max_skinny; i += NT) {
            const int e = upper_bound(s_soff, E + 1, i) - 1;
            const int row0 = (i - s_soff[e]) * a.bm_small;
            write_tile(a.tiles_skinny + 4 * i, e, s_off[e] + row0, min(a.bm_small, s_cnt[e] - row0),
                       a.bm_small);
        }
        if (tid == 0) {
            a.num_tiles[0] = nw + ns;
            a.num_tiles[2] = nw;
            a.num_tiles[3] = ns;
        }
    }
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_sort_tiles(RouteArgs a) {
    if (blockIdx.x > 0) {
        prepare_x(a, blockIdx.x - 1);
        return;
    }
    // LDS sized by E at launch (route_lds_bytes), so that the activation
    // workgroups of the same launch are not held to one per CU
    extern __shared__ int32_t route_lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, A = a.A;
    const int nkeys = E + 1;
    int32_t* const s_tab = route_lds;                       // [waves][nkeys] counts, then bases
    int32_t* const s_cnt = s_tab + kRouteWaves * nkeys;     // [nkeys]
    int32_t* const s_off = s_cnt + nkeys;                   // [nkeys + 1]
    int32_t* const s_toff = s_off + nkeys + 1;              // [nkeys + 1]
    int32_t* const s_soff = s_toff + nkeys + 1;             // [nkeys + 1]
    int32_t* const s_wsum = s_soff + nkeys + 1;             // [waves + 1]
    const int nbits = 32 - __clz(E);  // bits of the largest key, E
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    if (A <= 64 && a.presorted == nullptr) {
        // one row of keys: a match-any gives each key's count (at its lowest
        // lane) and each assignment's rank among equal keys.  Waves 0 and 1
        // both count, in LDS of their own; wave 0 then scatters while wave 1
        // writes counts, offsets and the tile lists.
        if (wave > 1) return;
        int32_t* const cnt = wave == 0 ? s_cnt : s_tab;
        int32_t* const off = wave == 0 ? s_off : s_tab + nkeys;
        for (int i = lane; i < nkeys; i += 64) cnt[i] = 0;
        const bool act = lane < A;
        const uint32_t key = act ? load_key(a, lane, A, E) : static_cast<uint32_t>(E);
        const uint64_t m = match_any(key, nbits, __ballot(act));
        __builtin_amdgcn_wave_barrier();
        if (act && (m & below) == 0) cnt[key] = __popcll(m);
        __builtin_amdgcn_wave_barrier();
        wave_exclusive_scan(cnt, off, nkeys);
        __builtin_amdgcn_wave_barrier();
        if (wave == 0) {
            if (act) {
                const int32_t slot = off[key] + __popcll(m & below);
                a.perm[slot] = lane;
                a.inv_perm[lane] = slot;
            }
        } else {
            // wave 1's scratch follows its counts and offsets in s_tab
            int32_t* const tab = off + nkeys + 1;  // [2 nkeys]
            int32_t* const toff = tab + 2 * nkeys;  // [nkeys + 1]
            int32_t* const soff = toff + nkeys + 1; // [nkeys + 1]
            emit_tiles<64>(a, tab, cnt, off, toff, soff, s_wsum, 0);
        }
        return;
    }

    for (int i = tid; i < kRouteWaves * nkeys; i += kRouteThreads) s_tab[i] = 0;
    __syncthreads();

    // Contiguous, 64-aligned segment of the assignments per wave.
    const int per = ((A + kRouteWaves - 1) / kRouteWaves + 63) & ~63;
    const int beg = wave * per;
    const int end = min(A, beg + per);
    int32_t* tab = s_tab + wave * nkeys;

    // 1. per-wave histogram: LDS atomic adds (a count does not depend on the
    // order of the adds).  Keys are loaded kBatch rows of 64 at a time, all
    // loads issued before the first is used.
    for (int base0 = beg; base0 < end; base0 += 64 * kBatch) {
        uint32_t keys[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) keys[b] = load_key(a, base0 + 64 * b + lane, end, E);
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (base0 + 64 * b + lane < end) atomicAdd(&tab[keys[b]], 1);
    }
    __syncthreads();

    // 2. totals, offsets, per-(wave, key) bases
    for (int key = tid; key < nkeys; key += kRouteThreads) {
        int32_t s = 0;
        for (int w = 0; w < kRouteWaves; ++w) s += s_tab[w * nkeys + key];
        s_cnt[key] = s;
    }
    __syncthreads();
    block_exclusive_scan(s_cnt, s_off, nkeys, s_wsum);
    for (int key = tid; key < nkeys; key += kRouteThreads) {
        int32_t run = s_off[key];
        for (int w = 0; w < kRouteWaves; ++w) {
            const int32_t c = s_tab[w * nkeys + key];
            s_tab[w * nkeys + key] = run;
            run += c;
        }
    }
    __syncthreads();

    // 3. the caller's sorted order, if it is one (it must also be a
    // permutation: checked after writing inv_perm), else the stable scatter
    int32_t order_status = 0;
    if (a.presorted != nullptr) {
        order_status = presorted_order_ok(a) ? 0 : 1;
        if (order_status == 0) {
            for (int s = tid; s < A; s += kRouteThreads) {
                const int32_t ai = a.presorted[s];
                a.perm[s] = ai;
                a.inv_perm[ai] = s;
            }
            __threadfence_block();
            __syncthreads();
            bool bij = true;
            for (int s = tid; s < A; s += kRouteThreads)
                if (a.inv_perm[a.presorted[s]] != s) bij = false;
            order_status = __syncthreads_and(bij) ? 0 : 2;
        }
    }
    if (a.presorted == nullptr || order_status != 0)
    for (int base0 = beg; base0 < end; base0 += 64 * kBatch) {
        uint32_t keys[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) keys[b] = load_key(a, base0 + 64 * b + lane, end, E);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int base = base0 + 64 * b;
            if (base >= end) break;
            const int ai = base + lane;
            const bool act = ai < end;
            const uint64_t m = match_any(keys[b], nbits, __ballot(act));
            if (act) {
                const int32_t slot = tab[keys[b]] + __popcll(m & below);
                a.perm[slot] = ai;
                a.inv_perm[ai] = slot;
            }
            if (act && (m & below) == 0) tab[keys[b]] += __popcll(m);
        }
    }

    // 4. counts, offsets, tiles
    emit_tiles<kRouteThreads>(a, s_tab, s_cnt, s_off, s_toff, s_soff, s_wsum, order_status);
}

// ---------------------------------------------------------------------------
// Large A (the forward, without a caller's order): the sort spreads over
// count_wgs workgroups of kRouteSegment assignments each (one row of 64 per
// wave), in two launches.  moe_route_count: each workgroup's per-key counts of
// its segment into hist[wg][key]; the activation workgroups of the forward
// ride in the same launch.  moe_route_scatter: each workgroup forms the totals
// and its own base per key from hist (sums in workgroup order, so the sort is
// the same stable sort), ranks its rows with a wave match-any and scatters;
// one more workgroup writes counts, offsets and the tile lists meanwhile.
//
// With a caller's order (the pre-sorted entry) the same segments, of slots,
// check it in three steps, one per launch (each needs the last one's writes
// from every workgroup): moe_route_count also checks its slots' range and
// order and writes inv_perm from the order; moe_route_verify checks that
// inv_perm maps every slot back to itself (a permutation); moe_route_scatter
// then uses the order if every segment passed, else sorts as without one.
// Segment status (after hist): 0 ok, 1 not sorted or out of range, 2 not a
// permutation.
__device__ __forceinline__ int32_t* seg_status(const RouteArgs& a) {
    return a.hist + static_cast<size_t>(a.count_wgs) * (a.E + 1);
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_count(RouteArgs a) {
    if (static_cast<int>(blockIdx.x) >= a.count_wgs) {
        prepare_x(a, blockIdx.x - a.count_wgs);
        return;
    }
    extern __shared__ int32_t route_lds[];
    const int tid = threadIdx.x, E = a.E, nkeys = E + 1;
    int32_t* const s_cnt = route_lds;  // [nkeys]
    for (int i = tid; i < nkeys; i += kRouteThreads) s_cnt[i] = 0;
    __syncthreads();
    const int ai = blockIdx.x * kRouteSegment + tid;
    if (ai < a.A) atomicAdd(&s_cnt[load_key(a, ai, a.A, E)], 1);
    if (a.presorted != nullptr) {
        // slot ai of the caller's order (the adjacent-pair check of
        // presorted_order_ok, spread over the segments)
        bool bad = false;
        if (ai < a.A) {
            const int32_t a0 = a.presorted[ai];
            if (a0 < 0 || a0 >= a.A) {
                bad = true;
            } else {
                a.inv_perm[a0] = ai;
                if (ai + 1 < a.A) {
                    const int32_t a1 = a.presorted[ai + 1];
                    bad = a1 < 0 || a1 >= a.A || key_of(a, a0) > key_of(a, a1);
                }
            }
        }
        bad = __syncthreads_or(bad);
        if (tid == 0) seg_status(a)[blockIdx.x] = bad ? 1 : 0;
    }
    __syncthreads();
    int32_t* const h = a.hist + static_cast<size_t>(blockIdx.x) * nkeys;
    for (int i = tid; i < nkeys; i += kRouteThreads) h[i] = s_cnt[i];
}

// Pre-sorted entry, second step: every slot of the segment maps back to
// itself through inv_perm (two slots naming one assignment cannot both).
__global__ __launch_bounds__(kRouteThreads) void moe_route_verify(RouteArgs a) {
    const int s = blockIdx.x * kRouteSegment + threadIdx.x;
    bool bad = false;
    if (s < a.A) {
        const int32_t a0 = a.presorted[s];
        bad = a0 >= 0 && a0 < a.A && a.inv_perm[a0] != s;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0 && bad && seg_status(a)[blockIdx.x] == 0) seg_status(a)[blockIdx.x] = 2;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_scatter(RouteArgs a) {
    extern __shared__ int32_t route_lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, nkeys = E + 1, wg = blockIdx.x;
    int32_t* const s_tab = route_lds;                       // [waves][nkeys]
    int32_t* const s_cnt = s_tab + kRouteWaves * nkeys;     // [nkeys]
    int32_t* const s_off = s_cnt + nkeys;                   // [nkeys + 1]
    int32_t* const s_toff = s_off + nkeys + 1;              // [nkeys + 1]
    int32_t* const s_soff = s_toff + nkeys + 1;             // [nkeys + 1]
    int32_t* const s_wsum = s_soff + nkeys + 1;             // [waves + 1]
    // a caller's order: used if every segment passed (1 before 2 if not)
    int32_t order_status = 0;
    if (a.presorted != nullptr) {
        int32_t st = 0;
        for (int w = tid; w < a.count_wgs; w += kRouteThreads) st |= 1 << seg_status(a)[w];
        st = __syncthreads_or(st & 2) ? 1 : (__syncthreads_or(st & 4) ? 2 : 0);
        order_status = st;
    }
    if (wg == a.count_wgs) {
        // the last workgroup writes counts, offsets and the tile lists (from
        // the same totals), while the others scatter
        for (int k = tid; k < nkeys; k += kRouteThreads) {
            int32_t tot = 0;
#pragma unroll 16
            for (int w = 0; w < a.count_wgs; ++w) tot += a.hist[static_cast<size_t>(w) * nkeys + k];
            s_cnt[k] = tot;
        }
        __syncthreads();
        block_exclusive_scan(s_cnt, s_off, nkeys, s_wsum);
        emit_tiles<kRouteThreads>(a, s_tab, s_cnt, s_off, s_toff, s_soff, s_wsum, order_status);
        return;
    }
    if (a.presorted != nullptr && order_status == 0) {
        // the order as given (inv_perm came with the first step)
        const int s = wg * kRouteSegment + tid;
        if (s < a.A) a.perm[s] = a.presorted[s];
        return;
    }
    const int nbits = 32 - __clz(E);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = tid; i < kRouteWaves * nkeys; i += kRouteThreads) s_tab[i] = 0;
    __syncthreads();
    // this workgroup's rows: wave w owns row w (assignments beg + 64 w + lane)
    const int ai = wg * kRouteSegment + tid;
    const bool act = ai < a.A;
    const uint32_t key = act ? load_key(a, ai, a.A, E) : static_cast<uint32_t>(E);
    if (act) atomicAdd(&s_tab[wave * nkeys + key], 1);
    // totals, and the rows of this key in the workgroups before this one
    for (int k = tid; k < nkeys; k += kRouteThreads) {
        int32_t tot = 0, before = 0;
#pragma unroll 16
        for (int w = 0; w < a.count_wgs; ++w) {  // unrolled: the loads go out together
            const int32_t c = a.hist[static_cast<size_t>(w) * nkeys + k];
            tot += c;
            before += w < wg ? c : 0;
        }
        s_cnt[k] = tot;
        s_toff[k] = before;  // scratch until the tile emission
    }
    __syncthreads();
    block_exclusive_scan(s_cnt, s_off, nkeys, s_wsum);
    for (int k = tid; k < nkeys; k += kRouteThreads) {
        int32_t run = s_off[k] + s_toff[k];
        for (int w = 0; w < kRouteWaves; ++w) {
            const int32_t c = s_tab[w * nkeys + k];
            s_tab[w * nkeys + k] = run;
            run += c;
        }
    }
    __syncthreads();
    const uint64_t m = match_any(key, nbits, __ballot(act));
    if (act) {
        const int32_t slot = s_tab[wave * nkeys + key] + __popcll(m & below);
        a.perm[slot] = ai;
        a.inv_perm[ai] = slot;
    }
}

}  // namespace

size_t route_lds_bytes(int E) {
    const size_t nkeys = static_cast<size_t>(E) + 1;
    return sizeof(int32_t) * (kRouteWaves * nkeys + nkeys + 3 * (nkeys + 1) + kRouteWaves + 1);
}

int route_count_wgs(int64_t A) {
    return A > kRouteMultiMin ? static_cast<int>((A + kRouteSegment - 1) / kRouteSegment) : 0;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream, const KTiming& t) {
    int prep = 0;
    if (a.x != nullptr) {
        const int64_t pieces = static_cast<int64_t>(a.T) * (a.H / 8);
        prep = static_cast<int>((pieces + kRouteThreads - 1) / kRouteThreads);
    }
    const size_t lds = route_lds_bytes(a.E);
    if (a.count_wgs > 0) {
        if (a.hist == nullptr || a.count_wgs != route_count_wgs(a.A)) return hipErrorInvalidValue;
        if (lds > 64 * 1024) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_route_scatter),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     static_cast<int>(lds));
            if (e != hipSuccess) return e;
        }
        if (t.start != nullptr && hipEventRecord(t.start, stream) != hipSuccess) return hipGetLastError();
        const size_t lds1 = sizeof(int32_t) * (static_cast<size_t>(a.E) + 1);
        hipLaunchKernelGGL(moe_route_count, dim3(a.count_wgs + prep), dim3(kRouteThreads), lds1, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.presorted != nullptr) {
            hipLaunchKernelGGL(moe_route_verify, dim3(a.count_wgs), dim3(kRouteThreads), 0, stream, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(moe_route_scatter, dim3(a.count_wgs + 1), dim3(kRouteThreads), lds, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (t.stop != nullptr) return hipEventRecord(t.stop, stream);
        return hipSuccess;
    }
    const int blocks = 1 + prep;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_route_sort_tiles),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    return launch_kernel_lds(moe_route_sort_tiles, dim3(blocks), dim3(kRouteThreads), lds, stream,
                             t, a);
}

}  // namespace moe
