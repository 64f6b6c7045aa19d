// C ABI of libmoeffn: argument checks, workspace layout and the launch
// sequence of the forward.  Nothing here allocates, frees or waits on the
// device; everything is enqueued on the caller's stream.
#include <limits.h>
#include <stddef.h>

#include <mutex>

#include "moe_internal.h"

// The built-in workspace of moe_expert_ffn_forward_noalloc: one copy per
// GPU, alive until the process ends.  Host code never passes `scratch`
// itself to a kernel or a copy (in host code it is a stand-in, not a device
// address): it takes the device address from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device), or nullptr with *err set.
void* scratch_for_current_device(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by the forward's size queries and the forward itself.
moe_status check_problem(const moe_problem* p) {
    if (!p) return MOE_ERR_NULL;
    if (p->bits != 4 && p->bits != 8) return MOE_ERR_UNSUPPORTED;
    if (p->group_size != 32 && p->group_size != 64 && p->group_size != 128)
        return MOE_ERR_UNSUPPORTED;
    if (p->flags & ~(MOE_F_FP32_OUT | MOE_F_FP32_INTERMEDIATE | MOE_F_SWIGLU))
        return MOE_ERR_UNSUPPORTED;
    if (p->T < 0 || p->k < 1 || p->E < 1 || p->H < 1 || p->I < 1) return MOE_ERR_SHAPE;
    if (p->E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (p->k > p->E) return MOE_ERR_SHAPE;
    // The kernels step through K in 64-column halves of 128-column chunks;
    // a group never straddles two of those steps.
    if (p->H % 64 || p->I % 64) return MOE_ERR_SHAPE;
    if (p->H % p->group_size || p->I % p->group_size) return MOE_ERR_SHAPE;
    if (p->H > moe::kMaxDim || p->I > moe::kMaxDim) return MOE_ERR_UNSUPPORTED;
    const int64_t A = static_cast<int64_t>(p->T) * p->k;
    if (A > INT32_MAX / 2) return MOE_ERR_SHAPE;
    return MOE_OK;
}

moe_ws_layout make_layout(const moe_problem* p) {
    moe_ws_layout l = {};
    const int64_t A = static_cast<int64_t>(p->T) * p->k;
    // Wide tiles of at most 64 rows (4 row blocks per wave), or 32 with an
    // fp32 h (the down matmul carries two activation parts) or 8-bit codes
    // (twice the weight words in flight).
    l.bm_big = (p->flags & MOE_F_FP32_INTERMEDIATE) || p->bits == 8 ? moe::kBmBigF32 : moe::kBmBig;
    l.bm_small = moe::kBmSmall;
    l.max_tiles = moe_max_tiles(A, p->E, l.bm_big);
    l.max_skinny = moe_max_tiles(A, p->E, l.bm_small);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    const size_t hbytes = (p->flags & MOE_F_FP32_INTERMEDIATE) ? 4 : 2;
    const size_t G = p->H / p->group_size;
    l.counts = take(sizeof(int32_t) * p->E);
    l.offsets = take(sizeof(int32_t) * (p->E + 1));
    l.perm = take(sizeof(int32_t) * A);
    l.inv_perm = take(sizeof(int32_t) * A);
    l.tiles = take(sizeof(moe_tile) * l.max_tiles);
    l.tiles_skinny = take(sizeof(moe_tile) * l.max_skinny);
    l.num_tiles = take(sizeof(int32_t) * 8);
    l.x_perm = take(sizeof(uint16_t) * p->T * p->H);
    l.x_sums = take(sizeof(float) * p->T * G);
    l.h = take(hbytes * A * p->I);
    l.h_sums = take(sizeof(float) * A * (p->I / 16));
    l.y = take(sizeof(float) * A * p->H);
    // per-segment key counts, then one order check per segment (pre-sorted entry)
    l.route_hist = take(sizeof(int32_t) * moe::route_count_wgs(A) * (static_cast<size_t>(p->E) + 2));
    // x as e4m3 hi + lo with block scales, for the wide gate|up kernel's fp8 operands
    const bool fp8 = moe::fp8_wide_gateup(p->T, p->group_size, p->bits, p->flags);
    l.x8_hi = take(fp8 ? static_cast<size_t>(p->T) * p->H : 0);
    l.x8_lo = take(fp8 ? static_cast<size_t>(p->T) * p->H : 0);
    l.x8_scales = take(fp8 ? static_cast<size_t>(p->T) * moe::x8_stride(p->H) : 0);
    l.total = off;
    return l;
}

moe_status forward_impl(const moe_problem* p, const void* x, const int32_t* ids,
                        const float* topk_w, const uint32_t* w_gu, const void* s_gu,
                        const void* b_gu, const uint32_t* w_d, const void* s_d,
                        const void* b_d, void* out, void* ws, size_t ws_bytes, void* stream,
                        void* const* events, const int32_t* presorted, bool want_presorted) {
    const moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->T == 0) return MOE_OK;
    if (!x || !ids || !topk_w || !w_gu || !s_gu || !b_gu || !w_d || !s_d || !b_d || !out)
        return MOE_ERR_NULL;
    if (want_presorted && !presorted) return MOE_ERR_NULL;
    if (presorted && !aligned(presorted, 4)) return MOE_ERR_ALIGN;
    if (!ws) return MOE_ERR_WORKSPACE;
    const moe_ws_layout l = make_layout(p);
    if (ws_bytes < l.total) return MOE_ERR_WORKSPACE;
    const bool f32out = p->flags & MOE_F_FP32_OUT;
    if (!aligned(x, 16) || !aligned(w_gu, 16) || !aligned(w_d, 16) || !aligned(ids, 4) ||
        !aligned(topk_w, 4) || !aligned(s_gu, 16) || !aligned(b_gu, 16) || !aligned(s_d, 16) ||
        !aligned(b_d, 16) || !aligned(out, f32out ? 16 : 8) || !aligned(ws, kAlign))
        return MOE_ERR_ALIGN;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    // events[2i], events[2i+1]: start and stop of kernel i
    auto kt = [&](int i) {
        moe::KTiming t;
        if (events != nullptr) {
            t.start = static_cast<hipEvent_t>(events[2 * i]);
            t.stop = static_cast<hipEvent_t>(events[2 * i + 1]);
        }
        return t;
    };

    moe::RouteArgs r;
    r.ids = ids;
    r.A = p->T * p->k;
    r.E = p->E;
    r.bm_big = l.bm_big;
    r.bm_small = l.bm_small;
    r.max_tiles = l.max_tiles;
    r.max_skinny = l.max_skinny;
    // At most bm_small tokens: no expert has more rows unless a token repeats
    // an id, so every expert takes the skinny path (in tiles of bm_small) and
    // the wide launches are left out.
    const bool skinny_only = p->T <= l.bm_small;
    r.skinny_max_rows = skinny_only ? INT32_MAX : l.bm_small;
    r.counts = reinterpret_cast<int32_t*>(base + l.counts);
    r.offsets = reinterpret_cast<int32_t*>(base + l.offsets);
    r.perm = reinterpret_cast<int32_t*>(base + l.perm);
    r.inv_perm = reinterpret_cast<int32_t*>(base + l.inv_perm);
    r.tiles = reinterpret_cast<int32_t*>(base + l.tiles);
    r.tiles_skinny = reinterpret_cast<int32_t*>(base + l.tiles_skinny);
    r.num_tiles = reinterpret_cast<int32_t*>(base + l.num_tiles);
    r.presorted = presorted;
    r.count_wgs = moe::route_count_wgs(r.A);
    r.hist = reinterpret_cast<int32_t*>(base + l.route_hist);
    r.x = static_cast<const uint16_t*>(x);
    r.T = p->T;
    r.H = p->H;
    r.gs = p->group_size;
    r.xp = reinterpret_cast<uint16_t*>(base + l.x_perm);
    r.xs = reinterpret_cast<float*>(base + l.x_sums);
    const bool fp8 = moe::fp8_wide_gateup(p->T, p->group_size, p->bits, p->flags);
    r.x8hi = fp8 ? reinterpret_cast<uint8_t*>(base + l.x8_hi) : nullptr;
    r.x8lo = fp8 ? reinterpret_cast<uint8_t*>(base + l.x8_lo) : nullptr;
    r.x8s = fp8 ? reinterpret_cast<uint8_t*>(base + l.x8_scales) : nullptr;

    moe::FfnArgs f;
    f.T = p->T;
    f.k = p->k;
    f.E = p->E;
    f.H = p->H;
    f.I = p->I;
    f.gs = p->group_size;
    f.bits = p->bits;
    f.max_tiles = l.max_tiles;
    f.max_skinny = l.max_skinny;
    f.skinny_only = skinny_only ? 1 : 0;
    f.flags = p->flags;
    f.zero = 0;
    f.x = static_cast<const uint16_t*>(x);
    f.xp = r.xp;
    f.xs = r.xs;
    f.x8hi = r.x8hi;
    f.x8lo = r.x8lo;
    f.x8s = r.x8s;
    f.hs = reinterpret_cast<float*>(base + l.h_sums);
    f.ids = ids;
    f.topk_w = topk_w;
    f.w_gu = w_gu;
    f.s_gu = static_cast<const uint16_t*>(s_gu);
    f.b_gu = static_cast<const uint16_t*>(b_gu);
    f.w_d = w_d;
    f.s_d = static_cast<const uint16_t*>(s_d);
    f.b_d = static_cast<const uint16_t*>(b_d);
    f.perm = r.perm;
    f.tiles = r.tiles;
    f.tiles_skinny = r.tiles_skinny;
    f.num_tiles = r.num_tiles;
    f.h = base + l.h;
    f.y = reinterpret_cast<float*>(base + l.y);
    f.out = out;

    if (moe::launch_route(r, s, kt(0)) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_gateup_skinny(f, s, kt(1)) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_gateup_wide(f, s, kt(2)) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_down_skinny(f, s, kt(3)) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_down_wide(f, s, kt(4)) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_combine(f, s, kt(5)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_max_tiles(int64_t A, int32_t E, int32_t bm_big) {
    if (A < 0 || E < 1 || bm_big < 1) return -1;
    const int64_t v = A / bm_big + (A < E ? A : E);
    return v > INT32_MAX ? -1 : static_cast<int32_t>(v);
}

moe_status moe_sort_build_tiles(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                int32_t bm_big, int32_t bm_small, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                moe_tile* tiles, int32_t max_tiles, int32_t* num_tiles,
                                void* stream) {
    if (T < 0 || k < 1 || E < 1) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (bm_small < 1 || bm_big < bm_small) return MOE_ERR_SHAPE;
    const int64_t A = static_cast<int64_t>(T) * k;
    if (A > INT32_MAX / 2) return MOE_ERR_SHAPE;
    if (!counts || !offsets || !num_tiles || !tiles) return MOE_ERR_NULL;
    if (A > 0 && (!topk_ids || !perm || !inv_perm)) return MOE_ERR_NULL;
    const int32_t need = moe_max_tiles(A, E, bm_big);
    if (need < 0 || max_tiles < need) return MOE_ERR_WORKSPACE;
    if (!aligned(tiles, 16) || !aligned(counts, 4) || !aligned(offsets, 4) ||
        !aligned(num_tiles, 4) || (A > 0 && (!aligned(topk_ids, 4) || !aligned(perm, 4) ||
                                             !aligned(inv_perm, 4))))
        return MOE_ERR_ALIGN;
    moe::RouteArgs r;
    r.ids = topk_ids;
    r.A = static_cast<int32_t>(A);
    r.E = E;
    r.bm_big = bm_big;
    r.bm_small = bm_small;
    r.max_tiles = max_tiles;
    r.counts = counts;
    r.offsets = offsets;
    r.perm = perm;
    r.inv_perm = inv_perm;
    r.tiles = reinterpret_cast<int32_t*>(tiles);
    r.tiles_skinny = nullptr;
    r.max_skinny = 0;
    r.skinny_max_rows = bm_small;
    r.presorted = nullptr;
    r.count_wgs = 0;
    r.hist = nullptr;
    r.num_tiles = num_tiles;
    r.x = nullptr;
    r.gs = 0;
    r.T = T;
    r.H = 0;
    r.xp = nullptr;
    r.xs = nullptr;
    r.x8hi = nullptr;
    r.x8lo = nullptr;
    r.x8s = nullptr;
    return moe::launch_route(r, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK
                                                                               : MOE_ERR_HIP;
}

size_t moe_ffn_workspace_bytes(const moe_problem* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return make_layout(p).total;
}

moe_status moe_ffn_workspace_layout(const moe_problem* p, moe_ws_layout* layout) {
    if (!layout) return MOE_ERR_NULL;
    const moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    *layout = make_layout(p);
    return MOE_OK;
}

moe_status moe_expert_ffn_forward(const moe_problem* p, const void* x, const int32_t* topk_ids,
                                  const float* topk_weights, const uint32_t* w_gateup,
                                  const void* s_gateup, const void* b_gateup,
                                  const uint32_t* w_down, const void* s_down, const void* b_down,
                                  void* out, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(p, x, topk_ids, topk_weights, w_gateup, s_gateup, b_gateup, w_down,
                        s_down, b_down, out, ws, ws_bytes, stream, nullptr, nullptr, false);
}

moe_status moe_expert_ffn_forward_noalloc(const moe_problem* p, const void* x,
                                          const int32_t* topk_ids, const float* topk_weights,
                                          const uint32_t* w_gateup, const void* s_gateup,
                                          const void* b_gateup, const uint32_t* w_down,
                                          const void* s_down, const void* b_down, void* out,
                                          void* stream) {
    const moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->T == 0) return MOE_OK;
    if (make_layout(p).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    hipError_t err = hipSuccess;
    void* ws = scratch_for_current_device(&err);
    if (ws == nullptr) return MOE_ERR_HIP;
    return forward_impl(p, x, topk_ids, topk_weights, w_gateup, s_gateup, b_gateup, w_down, s_down,
                        b_down, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, false);
}

moe_status moe_expert_ffn_forward_presorted(const moe_problem* p, const void* x,
                                            const int32_t* topk_ids, const float* topk_weights,
                                            const int32_t* sorted_order,
                                            const uint32_t* w_gateup, const void* s_gateup,
                                            const void* b_gateup, const uint32_t* w_down,
                                            const void* s_down, const void* b_down, void* out,
                                            void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(p, x, topk_ids, topk_weights, w_gateup, s_gateup, b_gateup, w_down,
                        s_down, b_down, out, ws, ws_bytes, stream, nullptr, sorted_order, true);
}

moe_status moe_expert_ffn_forward_timed(const moe_problem* p, const void* x,
                                        const int32_t* topk_ids, const float* topk_weights,
                                        const uint32_t* w_gateup, const void* s_gateup,
                                        const void* b_gateup, const uint32_t* w_down,
                                        const void* s_down, const void* b_down, void* out,
                                        void* ws, size_t ws_bytes, void* stream,
                                        void* const* events) {
    return forward_impl(p, x, topk_ids, topk_weights, w_gateup, s_gateup, b_gateup, w_down,
                        s_down, b_down, out, ws, ws_bytes, stream, events, nullptr, false);
}

moe_status moe_router_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                           int32_t* topk_ids, float* topk_weights, void* stream) {
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > moe::kRouterMaxK) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
        return MOE_ERR_ALIGN;
    if (static_cast<int64_t>(T) * E > INT32_MAX) return MOE_ERR_SHAPE;
    const hipError_t e = moe::launch_router_topk(logits, T, E, k, topk_ids, topk_weights,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "invalid or inconsistent sizes";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration (bits, group size, flags or expert count)";
        case MOE_ERR_ALIGN: return "a pointer is misaligned";
        case MOE_ERR_WORKSPACE: return "workspace or tile buffer missing or too small";
        case MOE_ERR_HIP: return "HIP runtime error while enqueueing work";
        case MOE_ERR_SCRATCH:
            return "problem needs more workspace than the built-in scratch buffer of the allocation-free entry point holds";
        default: return "unknown status";
    }
}

}  // extern "C"
