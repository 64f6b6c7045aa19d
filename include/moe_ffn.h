/*
 * moe_ffn.h -- C ABI of libmoeffn, the routed 4-bit (or 8-bit) MoE expert FFN for AMD
 * MI355X (gfx950).
 *
 * The operation (switch-GLU expert FFN with a tanh-GELU product):
 *
 *   for every token t and slot j < k, with e = topk_ids[t, j]:
 *     g = x[t] . Wg[e]^T,  u = x[t] . Wu[e]^T          (one packed gate|up
 *         projection; mlx-node PR #168 page: the "MLP gate|up" split)
 *     h = gelu_tanh(g) * u                              (SwiftLM issue #236,
 *         "Still missing": activation(xGate) * xUp, activation =
 *         geluApproximate)
 *     y = h . Wd[e]^T
 *   out[t] = sum_j topk_weights[t, j] * y(t, j)         (SwiftLM issue #236,
 *         "Already on main": weightedExpertSum; Layr-Labs/mlx PR #4,
 *         "Measured standing": direct weighted unsort)
 *
 * with gelu_tanh(v) = 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).
 *
 * Weights are affine 4-bit in groups of gs = group_size columns (64 on the
 * pages; 32 and 128 are the other common choices), in the layout of the
 * Layr-Labs/mlx PR #4 page ("What": packed gate/up [128, 1408, 352] and down
 * [128, 2816, 88] uint32 for 128 experts, hidden 2816, intermediate 704):
 *
 *   w_gateup uint32 [E, 2I, H/8]  rows [0, I) gate, [I, 2I) up; K contiguous
 *   s_gateup bf16   [E, 2I, H/gs] b_gateup bf16 [E, 2I, H/gs]
 *   w_down   uint32 [E, H, I/8]   s_down bf16 [E, H, I/gs]  b_down bf16 [E, H, I/gs]
 *
 * Element c of a row is the 4-bit code q at bits 4*(c%8) of word c/8 (low
 * nibble first) and dequantises to  W = S[c/gs] * q + B[c/gs]  in fp32.
 * With bits = 8 the same format holds 8-bit codes: H/4 (I/4) words per row,
 * code c at bits 8*(c%4) of word c/4 (low byte first).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL is the default stream) and is stream-ordered.
 *  - Entry points never throw and never abort.  Host-checkable errors are
 *    returned before anything is enqueued.
 *  - Apart from the scratch arrays of moe_expert_ffn_forward_noalloc (one per
 *    GPU, see there), the library keeps no mutable global state; concurrent
 *    calls on distinct buffers are safe.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL                    */
    MOE_ERR_SHAPE = -2,       /* a size is negative, inconsistent or overflows */
    MOE_ERR_UNSUPPORTED = -3, /* bits not 4/8, group_size not 32/64/128, E too large, ... */
    MOE_ERR_ALIGN = -4,       /* a pointer is not aligned as required          */
    MOE_ERR_WORKSPACE = -5,   /* workspace missing or too small                */
    MOE_ERR_HIP = -6,         /* the HIP runtime rejected a launch             */
    MOE_ERR_SCRATCH = -7      /* too large for moe_expert_ffn_forward_noalloc  */
};

/* One tile of sorted rows of a single expert: rows
 * [row_begin, row_begin + row_count) of the sorted order.  bm is the tile
 * height class: bm_small when row_count <= bm_small, else bm_big
 * (Layr-Labs/mlx PR #4, "What": BM32 expert tiles with BM16 fallback rows). */
typedef struct {
    int32_t expert;
    int32_t row_begin;
    int32_t row_count;
    int32_t bm;
} moe_tile;

/* Problem description.  Append-only: new fields go at the end. */
typedef struct {
    int32_t T;          /* tokens, >= 0                                  */
    int32_t k;          /* experts per token, 1 <= k <= E                */
    int32_t E;          /* experts, 1 <= E <= MOE_MAX_EXPERTS            */
    int32_t H;          /* hidden size, multiple of 64 and of group_size, <= 4096 */
    int32_t I;          /* intermediate size, same rules as H            */
    int32_t group_size; /* 32, 64 or 128 columns per scale and bias      */
    int32_t bits;       /* 4 or 8 (8: wide tiles of at most 32 rows)     */
    uint32_t flags;     /* MOE_F_* below                                 */
} moe_problem;

#define MOE_MAX_EXPERTS 1024
/* out is fp32 [T, H] instead of bf16 */
#define MOE_F_FP32_OUT 1u
/* the GeGLU intermediate h is kept to 16 significant bits (bf16 hi + lo)
 * instead of bf16 (the fp32-accumulator path); combine with MOE_F_FP32_OUT
 * for a full-fp32 result.  Without it h is bf16, the dtype of x (SwiftLM
 * issue #236, "What #27 set out to do" (3): the switch-GLU intermediates stay
 * in the original dtype).  The weighted down output y is fp32 either way: a
 * bf16 y costs more than the bf16 output's error budget on a 16384-assignment
 * batch. */
#define MOE_F_FP32_INTERMEDIATE 2u
/* SwiGLU instead of GeGLU: h = silu(g) * u with silu(v) = v / (1 + exp(-v))
 * (SwiftLM issue #236, "What #27 set out to do" (2) and "Already on main":
 * the compiled SiLU product; mlx-node PR #168: the MoE switch GLU through the
 * fused SwiGLU kernel) */
#define MOE_F_SWIGLU 4u

/* Upper bound on the number of tiles for A assignments over E experts with
 * tile height bm_big: floor(A / bm_big) + min(E, A) (every expert's tiles
 * are full bm_big-row tiles plus at most one shorter tile: the BM32 expert
 * tiles with BM16 fallback rows of the Layr-Labs/mlx PR #4 page, "What").
 * Sizes the tile arrays of moe_sort_build_tiles.  Returns -1 on bad input. */
int32_t moe_max_tiles(int64_t A, int32_t E, int32_t bm_big);

/*
 * Route the T*k assignments by expert and cut them into tiles
 * (Layr-Labs/mlx PR #4, "What": sorted expert indices and the parallel tile
 * descriptor builder -- binary search, exclusive scan, upper-bound emission).
 *
 *   topk_ids  int32 [T*k]  expert of flat assignment a = t*k + j
 *   counts    int32 [E]    rows per expert (valid ids only)
 *   offsets   int32 [E+1]  exclusive scan of counts; offsets[E] = valid rows
 *   perm      int32 [T*k]  sorted slot -> flat assignment.  Stable: within an
 *                          expert, ascending a.  Assignments whose id is
 *                          outside [0, E) follow all valid rows, ascending a.
 *   inv_perm  int32 [T*k]  flat assignment -> sorted slot
 *   tiles     moe_tile [max_tiles]  in expert order; per expert, tiles of
 *                          bm_big rows, the last one possibly short
 *   num_tiles int32 [2]    [0] = number of tiles written, [1] = number of
 *                          assignments with an out-of-range expert id
 *
 * Requires 1 <= bm_small <= bm_big, E <= MOE_MAX_EXPERTS and
 * max_tiles >= moe_max_tiles(T*k, E, bm_big).  T = 0 is valid (counts and
 * offsets are zeroed).  All outputs are bit-exact and deterministic.  It
 * takes no workspace: one workgroup sorts in its LDS (per-key counts, scan
 * and ranks never leave the chip), so the only device memory written is the
 * caller's outputs above.
 */
moe_status moe_sort_build_tiles(const int32_t* topk_ids, int32_t T, int32_t k,
                                int32_t E, int32_t bm_big, int32_t bm_small,
                                int32_t* counts, int32_t* offsets, int32_t* perm,
                                int32_t* inv_perm, moe_tile* tiles,
                                int32_t max_tiles, int32_t* num_tiles,
                                void* stream);

/*
 * Device router: softmax top-k with renormalised weights, feeding
 * moe_sort_build_tiles / moe_expert_ffn_forward.  The pages do not define the
 * router; this is the usual top-k softmax gate (the fused top-k candidate
 * selection of the mlx-node PR #168 page is its nearest relative there).
 *
 *   logits        fp32 [T, E]   4-byte aligned; NaN ranks as -inf
 *   topk_ids      int32 [T, k]  the k largest logits of each row, in order of
 *                               descending logit, the lower id first on ties
 *   topk_weights  fp32 [T, k]   exp(l_j - m) / sum_i exp(l_i - m) over the k
 *                               chosen (m the row's largest logit): the
 *                               softmax over E renormalised over the k
 *
 * Requires 1 <= k <= min(E, 64), E <= MOE_MAX_EXPERTS.  T = 0 is valid.
 * Deterministic; enqueued on `stream`, nothing allocated.
 */
moe_status moe_router_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                           int32_t* topk_ids, float* topk_weights, void* stream);

/* Bytes of device workspace moe_expert_ffn_forward needs for problem p
 * (0 on invalid p).  The pages' forward keeps its sorted indices, tile
 * descriptors and switch-GLU intermediates in buffers of its own (Layr-Labs/
 * mlx PR #4, "What"; SwiftLM issue #236, "What #27 set out to do" (3)); here
 * they live in one caller-owned workspace, laid out by
 * moe_ffn_workspace_layout. */
size_t moe_ffn_workspace_bytes(const moe_problem* p);

/* Byte offsets of the forward's intermediates inside its workspace, so that
 * callers and tests can inspect them after a forward on the same stream.
 * "Operand order": within every run of 8 consecutive columns, the values are
 * stored in the order 0,4,1,5,2,6,3,7 (the column order of the matmul
 * operands). */
typedef struct {
    size_t counts;    /* int32 [E]                                        */
    size_t offsets;   /* int32 [E+1]                                      */
    size_t perm;      /* int32 [A]                                        */
    size_t inv_perm;  /* int32 [A]                                        */
    size_t tiles;     /* moe_tile [max_tiles]: the tiles of the experts of
                         more than bm_small rows, ceil(count / bm_big) of
                         near-equal size per expert, in expert order
                         (empty when T <= bm_small)                       */
    size_t num_tiles; /* int32 [8]: total tiles, out-of-range ids, tiles
                         in `tiles`, tiles in `tiles_skinny`, and the
                         order check of the pre-sorted entry (0 used,
                         1 not sorted or out of range, 2 not a
                         permutation; the route launch then sorted by
                         itself); [5..7] unused                           */
    size_t x_perm;    /* bf16 [T, H]: x in operand order                  */
    size_t x_sums;    /* fp32 [T, H/gs]: sum of x over each group      */
    size_t h;         /* GeGLU output in sorted order, operand order:
                         bf16 [A, I]; with MOE_F_FP32_INTERMEDIATE two bf16
                         arrays [2, A, I], h = hi + lo                    */
    size_t h_sums;    /* fp32 [A, I/16]: sum of h (hi + lo) over each
                         16-column block (in column order); the sum of a
                         group adds its blocks left to right, e.g.
                         ((b0 + b1) + b2) + b3 at gs = 64                */
    size_t y;         /* fp32 [A, H] flat order a = t*k + j, already
                         multiplied by topk_weights (the direct weighted
                         unsort of the Layr-Labs/mlx PR #4 page,
                         "Measured standing"); rows of assignments with an
                         out-of-range id are not written                  */
    size_t total;     /* == moe_ffn_workspace_bytes(p)                    */
    int32_t max_tiles;
    int32_t bm_big;
    int32_t bm_small;
    int32_t max_skinny;
    size_t tiles_skinny; /* moe_tile [max_skinny]: tiles of at most bm_small
                            rows, in expert order: one per expert of 1 to
                            bm_small rows.  When T <= bm_small (no expert
                            can have more rows unless a token repeats an
                            id) every expert is put here instead, in
                            consecutive tiles of bm_small rows, the last
                            one shorter, and `tiles` stays empty         */
    size_t route_hist;   /* int32 [ceil(A/1024), E+1] when A > 2048 (else
                            empty): per-key counts of each 1024-assignment
                            segment, for the route launches; then int32
                            [ceil(A/1024)]: each segment's check of a
                            caller's order (pre-sorted entry)            */
    size_t x8_hi;        /* e4m3 [T, H] and                                 */
    size_t x8_lo;        /* e4m3 [T, H]: x * 2^-e = hi + lo, each 8-column
                            piece in the order 0,2,4,6,1,3,5,7, with one e
                            per 32 columns                                 */
    size_t x8_scales;    /* uint8 [T, H/32 rounded up to 4]: 127 + e.
                            These three are empty unless the wide gate|up
                            matmul takes fp8 operands: more than bm_small
                            tokens, 4-bit codes in groups of 64 or 128,
                            without MOE_F_FP32_INTERMEDIATE                */
} moe_ws_layout;

moe_status moe_ffn_workspace_layout(const moe_problem* p, moe_ws_layout* layout);

/*
 * Full expert FFN forward: route/sort/tile, gathered quantised gate|up matmul
 * with the fused GeGLU product, gathered quantised down matmul with the
 * weighted unsort, and the combine back to tokens (codes of p->bits bits in
 * groups of p->group_size columns).  Defined by: the expert-tile gathered
 * QMM over sorted indices (Layr-Labs/mlx PR #4, "What"), the GeGLU product
 * activation(xGate) * xUp with the approximate GELU (SwiftLM issue #236,
 * "Still missing"), the weighted unsort (PR #4, "Measured standing") and
 * the weighted expert sum (issue #236, "Already on main").
 *
 *   x            bf16 [T, H]        16-byte aligned
 *   topk_ids     int32 [T, k]
 *   topk_weights fp32 [T, k]        used as given (no renormalisation)
 *   w_gateup ... b_down             see the layout above; all six 16-byte aligned
 *   out          [T, H] bf16, or fp32 with MOE_F_FP32_OUT
 *   ws           device workspace of at least moe_ffn_workspace_bytes(p)
 *                bytes, 256-byte aligned
 *
 * Assignments with an expert id outside [0, E) contribute zero (they are
 * counted in the workspace's num_tiles[1]).  The host never waits on the
 * device: the tile count stays in device memory.  Results are deterministic
 * and independent of the order of tokens.
 */
moe_status moe_expert_ffn_forward(const moe_problem* p, const void* x,
                                  const int32_t* topk_ids, const float* topk_weights,
                                  const uint32_t* w_gateup, const void* s_gateup,
                                  const void* b_gateup, const uint32_t* w_down,
                                  const void* s_down, const void* b_down, void* out,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * The forward on assignments the caller has already sorted by expert, the
 * input the expert-tile kernel of the Layr-Labs/mlx PR #4 page takes ("What":
 * sorted indices).  Arguments as moe_expert_ffn_forward, plus
 *
 *   sorted_order  int32 [T*k]  slot -> flat assignment a = t*k + j, with the
 *                              expert ids topk_ids[sorted_order[s]]
 *                              non-decreasing in s (ids outside [0, E) last);
 *                              any order within an expert; 4-byte aligned
 *
 * The route launches check the order on the device, as the page's fail-safe
 * does ("Deep-review round": a strided adjacent-pair scan, which holds exactly
 * when the order is globally non-decreasing), and also that it is a
 * permutation (above 2048 assignments in three launches over 1024-slot
 * segments, else in one workgroup).  If a check fails they record why in
 * the workspace's num_tiles[4] (1 not sorted or out of range, 2 not a
 * permutation) and sort by themselves, so the result is always correct and
 * the host never waits.  Results are bit-identical to moe_expert_ffn_forward's
 * (they do not depend on the order of rows within an expert).
 */
moe_status moe_expert_ffn_forward_presorted(const moe_problem* p, const void* x,
                                            const int32_t* topk_ids, const float* topk_weights,
                                            const int32_t* sorted_order,
                                            const uint32_t* w_gateup, const void* s_gateup,
                                            const void* b_gateup, const uint32_t* w_down,
                                            const void* s_down, const void* b_down, void* out,
                                            void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_forward without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It calls no hipMalloc, hipFree
 * or allocating routine: its workspace is a scratch array built into the
 * library, MOE_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library
 * runs on holds until the process ends (its device address is looked up
 * once per device, on the first call there).
 *
 * Arguments as moe_expert_ffn_forward, minus ws and ws_bytes.  Problems whose
 * workspace (moe_ffn_workspace_bytes) exceeds MOE_NOALLOC_SCRATCH_BYTES
 * return MOE_ERR_SCRATCH before anything is enqueued (at hidden 2816 and
 * intermediate 704 the limit is about 2400 assignments, e.g. 300 tokens at
 * top-8).  Every call on a
 * GPU shares that GPU's scratch array: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  Nothing in
 * the scratch array needs clearing between calls.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_expert_ffn_forward_noalloc(const moe_problem* p, const void* x,
                                          const int32_t* topk_ids, const float* topk_weights,
                                          const uint32_t* w_gateup, const void* s_gateup,
                                          const void* b_gateup, const uint32_t* w_down,
                                          const void* s_down, const void* b_down, void* out,
                                          void* stream);

/* Same as moe_expert_ffn_forward, with per-kernel timing: events[2i] and
 * events[2i+1] (hipEvent_t, created by the caller) are recorded at the start
 * and the end of kernel i, with the kernel's dispatch itself, on `stream`.
 * The kernels, in launch order: 0 route, 1 gate|up skinny (tiles of <= 16
 * rows), 2 gate|up wide, 3 down skinny, 4 down wide, 5 combine.  A kernel
 * whose pair holds a NULL is not timed; events may be NULL. */
moe_status moe_expert_ffn_forward_timed(const moe_problem* p, const void* x,
                                        const int32_t* topk_ids,
                                        const float* topk_weights,
                                        const uint32_t* w_gateup, const void* s_gateup,
                                        const void* b_gateup, const uint32_t* w_down,
                                        const void* s_down, const void* b_down,
                                        void* out, void* ws, size_t ws_bytes,
                                        void* stream, void* const* events);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
