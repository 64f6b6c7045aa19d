// Gathered 4-bit quantised matmuls over expert tiles.
//
//   moe_gateup_geglu  h[s, n] = gelu_tanh(x[tok(s)] . Wg[e, n]) * (x[tok(s)] . Wu[e, n])
//   moe_down          y[perm[s], m] = w[perm[s]] * (h[s] . Wd[e, m])
//
// Prior art: the expert-tile QMM of the Layr-Labs/mlx PR #4 page ("What":
// BM32 expert tiles with BM16 fallback rows over sorted indices, one private
// row count per tile), the compiled gelu-product of SwiftLM issue #236
// ("Still missing"), and the direct weighted unsort of the PR #4 page
// ("Measured standing").  Design for gfx950:
//
//  * One workgroup = 4 waves = one tile x one block of output columns.  All
//    products run on v_mfma_f32_16x16x32_bf16: a tile of at most 16 rows is
//    one 16-row block (decode-sized tiles pay for 16 rows, not 32), a 32-row
//    tile two.  Each output row sees the same MFMA sequence in every tile, so
//    results are bitwise independent of how rows are grouped into tiles.
//  * The activation tile is staged through LDS in chunks of 4 quantisation
//    groups (256 columns), double-buffered; the gather through perm happens
//    in the staging loads, so no gathered copy of x is ever written.
//  * Weights go straight from HBM to registers (16-byte loads), are never
//    staged, and are turned into MFMA operands in registers: each 4-bit code
//    q becomes the bf16 value 128 + q exactly (codes_as_bf16).  The MFMA
//    operand therefore carries q exactly; scale and bias are applied in fp32
//    once per 64-column group:
//        acc += s * P + (b - 128 s) * X,
//    P = MFMA partial sum over the group, X = sum of the group's activations
//    (computed while staging).  Rounding the dequantised weights to bf16
//    instead would cost accuracy the fp32 path cannot afford.
//  * The gate and up rows of one output column are loaded by the same wave,
//    so the GeGLU product is formed in registers and h is written once.
//  * The down kernel scales each row by its routing weight and writes it to
//    its original (token, slot) position: the weighted unsort.
//  * Workgroups past the device-side tile count exit at once, so the host
//    never reads the tile count back.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkGroups = 4;                 // groups per staged K chunk
constexpr int kARows = 32;                      // staged activation rows
constexpr int kAStride = kChunkGroups * kGroup / 2 + 4;  // u32 per LDS row (+16 B pad)

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- staging
// Activation rows of one tile, staged chunk by chunk.  Thread t handles row
// t / 8 and, for each group i of the chunk, the 8 columns 8 * (t % 8) of it.
// LDS row layout: per group 8 pieces of 8 bf16, each piece reordered by
// permute8 to match the code order of codes_as_bf16.  Alongside, the fp32
// sum of each (row, group) for the bias term.
template <bool kF32>
struct Stager {
    // bf16 source: one 16-byte piece per group; fp32 source: two.
    u32x4 v[kChunkGroups][kF32 ? 2 : 1];
};

template <bool kF32>
__device__ __forceinline__ void stage_load(Stager<kF32>& st, const void* row_ptr, bool valid,
                                           int g0, int G, int sub) {
#pragma unroll
    for (int i = 0; i < kChunkGroups; ++i) {
        const bool ok = valid && (g0 + i) < G;
        const size_t col = static_cast<size_t>(g0 + i) * kGroup + 8 * sub;
        if constexpr (kF32) {
            const float* p = static_cast<const float*>(row_ptr) + col;
            st.v[i][0] = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
            st.v[i][1] = ok ? *reinterpret_cast<const u32x4*>(p + 4) : u32x4{0, 0, 0, 0};
        } else {
            const uint16_t* p = static_cast<const uint16_t*>(row_ptr) + col;
            st.v[i][0] = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
        }
    }
}

__device__ __forceinline__ float group_sum8(float s) {
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    return s;
}

// bf16 source -> one LDS array.
__device__ __forceinline__ void stage_store(const Stager<false>& st, uint32_t* sA, uint32_t*,
                                            float (*sX)[kARows], int r, int sub) {
#pragma unroll
    for (int i = 0; i < kChunkGroups; ++i) {
        *reinterpret_cast<u32x4*>(sA + r * kAStride + 32 * i + 4 * sub) = permute8(st.v[i][0]);
        const float s = group_sum8(sum8_bf16(st.v[i][0]));
        if (sub == 0) sX[i][r] = s;
    }
}

// fp32 source -> hi and lo bf16 LDS arrays, value = hi + lo to 16 bits.
__device__ __forceinline__ void stage_store(const Stager<true>& st, uint32_t* sAh, uint32_t* sAl,
                                            float (*sX)[kARows], int r, int sub) {
#pragma unroll
    for (int i = 0; i < kChunkGroups; ++i) {
        u32x4 hi, lo;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f0 = __uint_as_float(st.v[i][w >> 1][2 * (w & 1)]);
            const float f1 = __uint_as_float(st.v[i][w >> 1][2 * (w & 1) + 1]);
            const uint16_t h0 = f32_to_bf16(f0), h1 = f32_to_bf16(f1);
            const float r0 = f0 - bf16_to_f32(h0), r1 = f1 - bf16_to_f32(h1);
            const uint16_t l0 = f32_to_bf16(r0), l1 = f32_to_bf16(r1);
            hi[w] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
            lo[w] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
            s += bf16_to_f32(h0) + bf16_to_f32(l0);
            s += bf16_to_f32(h1) + bf16_to_f32(l1);
        }
        *reinterpret_cast<u32x4*>(sAh + r * kAStride + 32 * i + 4 * sub) = permute8(hi);
        *reinterpret_cast<u32x4*>(sAl + r * kAStride + 32 * i + 4 * sub) = permute8(lo);
        s = group_sum8(s);
        if (sub == 0) sX[i][r] = s;
    }
}

__device__ __forceinline__ u32x4 lds_piece(const uint32_t* sA, int row, int piece) {
    return *reinterpret_cast<const u32x4*>(sA + row * kAStride + 4 * piece);
}

// ------------------------------------------------------------ gate | up
// Grid: (max_tiles, I / 64).  Wave w owns h columns n0 + 16 w + [0, 16): its
// 16 gate rows and the matching 16 up rows, as two 16-column MFMA blocks, so
// gate and up of one output land in the same lane.  A tile of up to 16 rows
// is one 16-row block, a 32-row tile two.  Every row goes through the same
// sequence of 16x16x32 MFMAs whatever tile it sits in, so results do not
// depend on the tile layout (and hence not on the order of the tokens).
template <int RB, bool kF32H>
__device__ __forceinline__ void gateup_tile(const FfnArgs& a, uint32_t (*sA)[kARows * kAStride],
                                            float (*sX)[kChunkGroups][kARows], int e,
                                            int row_begin, int rows, int n0) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int H = a.H, I = a.I, G = H / kGroup;
    const int nchunks = (G + kChunkGroups - 1) / kChunkGroups;

    // staging role
    const int sr = tid >> 3, sub = tid & 7;
    const bool svalid = sr < rows;
    const uint16_t* xrow = a.x;
    if (svalid) xrow = a.x + static_cast<size_t>(a.perm[row_begin + sr] / a.k) * H;

    const int q = lane >> 4, lr = lane & 15;
    const int hcol = n0 + 16 * wave + lr;
    const size_t row_words = static_cast<size_t>(H) / 8;
    const size_t grow = static_cast<size_t>(e) * 2 * I + hcol;   // gate row
    const size_t urow = grow + I;                                // up row
    const uint32_t* wg = a.w_gu + grow * row_words + 2 * q;
    const uint32_t* wu = a.w_gu + urow * row_words + 2 * q;
    const uint16_t* sg_p = a.s_gu + grow * G;
    const uint16_t* bg_p = a.b_gu + grow * G;
    const uint16_t* su_p = a.s_gu + urow * G;
    const uint16_t* bu_p = a.b_gu + urow * G;

    Stager<false> st;
    stage_load<false>(st, xrow, svalid, 0, G, sub);
    stage_store(st, sA[0], nullptr, sX[0], sr, sub);

    f32x4 accg[RB] = {}, accu[RB] = {};
    // per group: gate words [0,1], up words [2,3]; scale/bias of gate, up
    u32x4 wcur[kChunkGroups], wnext[kChunkGroups];
    uint32_t sbc[kChunkGroups][4], sbn[kChunkGroups][4];
    auto load_w = [&](int c, u32x4 (&wv)[kChunkGroups], uint32_t (&sb)[kChunkGroups][4]) {
#pragma unroll
        for (int i = 0; i < kChunkGroups; ++i) {
            const int g = c * kChunkGroups + i;
            if (g < G) {
                const u32x2 gw = *reinterpret_cast<const u32x2*>(wg + 8 * g);
                const u32x2 uw = *reinterpret_cast<const u32x2*>(wu + 8 * g);
                wv[i] = u32x4{gw[0], gw[1], uw[0], uw[1]};
                sb[i][0] = sg_p[g];
                sb[i][1] = bg_p[g];
                sb[i][2] = su_p[g];
                sb[i][3] = bu_p[g];
            }
        }
    };
    load_w(0, wcur, sbc);
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < nchunks;
        if (more) {
            stage_load<false>(st, xrow, svalid, (c + 1) * kChunkGroups, G, sub);
            load_w(c + 1, wnext, sbn);
        }
        const uint32_t* A = sA[buf];
#pragma unroll
        for (int i = 0; i < kChunkGroups; ++i) {
            if (c * kChunkGroups + i >= G) break;
            f32x4 pg[RB] = {}, pu[RB] = {};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 bg = codes_as_bf16(wcur[i][s]);
                const u32x4 bu = codes_as_bf16(wcur[i][2 + s]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const u32x4 av = lds_piece(A, 16 * rb + lr, 8 * i + 2 * q + s);
                    pg[rb] = mfma16(av, bg, pg[rb]);
                    pu[rb] = mfma16(av, bu, pu[rb]);
                }
            }
            const float sg = bf16_to_f32(sbc[i][0]), bgv = bf16_to_f32(sbc[i][1]);
            const float su = bf16_to_f32(sbc[i][2]), buv = bf16_to_f32(sbc[i][3]);
            const float cg = fmaf(-kCodeOffset, sg, bgv), cu = fmaf(-kCodeOffset, su, buv);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float X = sX[buf][i][16 * rb + 4 * q + v];
                    accg[rb][v] = fmaf(cg, X, fmaf(sg, pg[rb][v], accg[rb][v]));
                    accu[rb][v] = fmaf(cu, X, fmaf(su, pu[rb][v], accu[rb][v]));
                }
            }
        }
        if (more) stage_store(st, sA[buf ^ 1], nullptr, sX[buf ^ 1], sr, sub);
        __syncthreads();
        if (more) {
#pragma unroll
            for (int i = 0; i < kChunkGroups; ++i) {
                wcur[i] = wnext[i];
#pragma unroll
                for (int z = 0; z < 4; ++z) sbc[i][z] = sbn[i][z];
            }
        }
    }

    // GeGLU epilogue: h = gelu_tanh(gate) * up, written once.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * rb + 4 * q + v;
            if (r < rows) {
                const float hv = gelu_tanh(accg[rb][v]) * accu[rb][v];
                const size_t o = static_cast<size_t>(row_begin + r) * I + hcol;
                if constexpr (kF32H) static_cast<float*>(a.h)[o] = hv;
                else static_cast<uint16_t*>(a.h)[o] = f32_to_bf16(hv);
            }
        }
    }
}

template <bool kF32H>
__global__ __launch_bounds__(kThreads) void moe_gateup_geglu(FfnArgs a) {
    __shared__ uint32_t sA[2][kARows * kAStride];
    __shared__ float sX[2][kChunkGroups][kARows];
    const int tile_idx = blockIdx.x;
    if (tile_idx >= min(a.num_tiles[0], a.max_tiles)) return;
    const int4 tile = reinterpret_cast<const int4*>(a.tiles)[tile_idx];
    const int n0 = blockIdx.y * 64;
    if (tile.z <= 16)
        gateup_tile<1, kF32H>(a, sA, sX, tile.x, tile.y, tile.z, n0);
    else
        gateup_tile<2, kF32H>(a, sA, sX, tile.x, tile.y, tile.z, n0);
}

// ------------------------------------------------------------------ down
// Grid: (max_tiles, ceil(H / 128)).  Wave w owns output columns
// n0 + 32 w + [0, 32) as two 16-column MFMA blocks (skipped past H); one or
// two 16-row blocks as above.  With an fp32 h the activation operand is split
// into bf16 hi + lo and both halves go through the MFMAs.
template <int RB, bool kF32H>
__device__ __forceinline__ void down_tile(const FfnArgs& a,
                                          uint32_t (*sA)[kF32H ? 2 : 1][kARows * kAStride],
                                          float (*sX)[kChunkGroups][kARows], const int32_t* sDst,
                                          const float* sW, int e, int row_begin, int rows,
                                          int n0) {
    constexpr int kParts = kF32H ? 2 : 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int H = a.H, I = a.I, G = I / kGroup;
    const int nchunks = (G + kChunkGroups - 1) / kChunkGroups;
    const int ncol0 = n0 + 32 * wave;
    const bool wave_active = ncol0 < H;

    const int sr = tid >> 3, sub = tid & 7;
    const bool svalid = sr < rows;
    const size_t elt = kF32H ? 4 : 2;
    const char* hbase = static_cast<const char*>(a.h);
    const void* hrow = hbase + static_cast<size_t>(row_begin + (svalid ? sr : 0)) * I * elt;

    const int q = lane >> 4, lr = lane & 15;
    const int c0 = ncol0 + lr, c1 = c0 + 16;
    const size_t row_words = static_cast<size_t>(I) / 8;
    const size_t r0 = static_cast<size_t>(e) * H + (wave_active ? c0 : 0);
    const size_t r1 = static_cast<size_t>(e) * H + (wave_active ? c1 : 0);
    const uint32_t* w0 = a.w_d + r0 * row_words + 2 * q;
    const uint32_t* w1 = a.w_d + r1 * row_words + 2 * q;
    const uint16_t* s0 = a.s_d + r0 * G;
    const uint16_t* b0 = a.b_d + r0 * G;
    const uint16_t* s1 = a.s_d + r1 * G;
    const uint16_t* b1 = a.b_d + r1 * G;

    Stager<kF32H> st;
    stage_load<kF32H>(st, hrow, svalid, 0, G, sub);
    stage_store(st, sA[0][0], sA[0][kParts - 1], sX[0], sr, sub);

    f32x4 acc0[RB] = {}, acc1[RB] = {};
    u32x4 wcur[kChunkGroups], wnext[kChunkGroups];
    uint32_t sbc[kChunkGroups][4], sbn[kChunkGroups][4];
    auto load_w = [&](int c, u32x4 (&wv)[kChunkGroups], uint32_t (&sb)[kChunkGroups][4]) {
#pragma unroll
        for (int i = 0; i < kChunkGroups; ++i) {
            const int g = c * kChunkGroups + i;
            if (g < G && wave_active) {
                const u32x2 x0 = *reinterpret_cast<const u32x2*>(w0 + 8 * g);
                const u32x2 x1 = *reinterpret_cast<const u32x2*>(w1 + 8 * g);
                wv[i] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                sb[i][0] = s0[g];
                sb[i][1] = b0[g];
                sb[i][2] = s1[g];
                sb[i][3] = b1[g];
            }
        }
    };
    load_w(0, wcur, sbc);
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < nchunks;
        if (more) {
            stage_load<kF32H>(st, hrow, svalid, (c + 1) * kChunkGroups, G, sub);
            load_w(c + 1, wnext, sbn);
        }
        if (wave_active) {
#pragma unroll
            for (int i = 0; i < kChunkGroups; ++i) {
                if (c * kChunkGroups + i >= G) break;
                f32x4 p0[RB] = {}, p1[RB] = {};
#pragma unroll
                for (int part = 0; part < kParts; ++part) {
                    const uint32_t* A = sA[buf][part];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const u32x4 bw0 = codes_as_bf16(wcur[i][s]);
                        const u32x4 bw1 = codes_as_bf16(wcur[i][2 + s]);
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            const u32x4 av = lds_piece(A, 16 * rb + lr, 8 * i + 2 * q + s);
                            p0[rb] = mfma16(av, bw0, p0[rb]);
                            p1[rb] = mfma16(av, bw1, p1[rb]);
                        }
                    }
                }
                const float sa = bf16_to_f32(sbc[i][0]), ba = bf16_to_f32(sbc[i][1]);
                const float sb = bf16_to_f32(sbc[i][2]), bb = bf16_to_f32(sbc[i][3]);
                const float ca = fmaf(-kCodeOffset, sa, ba), cb = fmaf(-kCodeOffset, sb, bb);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float X = sX[buf][i][16 * rb + 4 * q + v];
                        acc0[rb][v] = fmaf(ca, X, fmaf(sa, p0[rb][v], acc0[rb][v]));
                        acc1[rb][v] = fmaf(cb, X, fmaf(sb, p1[rb][v], acc1[rb][v]));
                    }
                }
            }
        }
        if (more) stage_store(st, sA[buf ^ 1][0], sA[buf ^ 1][kParts - 1], sX[buf ^ 1], sr, sub);
        __syncthreads();
        if (more) {
#pragma unroll
            for (int i = 0; i < kChunkGroups; ++i) {
                wcur[i] = wnext[i];
#pragma unroll
                for (int z = 0; z < 4; ++z) sbc[i][z] = sbn[i][z];
            }
        }
    }

    // weighted unsort: row s goes back to assignment perm[s], times its weight
    if (!wave_active) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * rb + 4 * q + v;
            if (r < rows) {
                float* yrow = a.y + static_cast<size_t>(sDst[r]) * H;
                const float wt = sW[r];
                yrow[c0] = wt * acc0[rb][v];
                yrow[c1] = wt * acc1[rb][v];
            }
        }
    }
}

template <bool kF32H>
__global__ __launch_bounds__(kThreads) void moe_down(FfnArgs a) {
    __shared__ uint32_t sA[2][kF32H ? 2 : 1][kARows * kAStride];
    __shared__ float sX[2][kChunkGroups][kARows];
    __shared__ int32_t sDst[kARows];
    __shared__ float sW[kARows];
    const int tile_idx = blockIdx.x;
    if (tile_idx >= min(a.num_tiles[0], a.max_tiles)) return;
    const int4 tile = reinterpret_cast<const int4*>(a.tiles)[tile_idx];
    const int tid = threadIdx.x;
    if (tid < tile.z) {
        const int32_t dst = a.perm[tile.y + tid];
        sDst[tid] = dst;
        sW[tid] = a.topk_w[dst];
    }
    const int n0 = blockIdx.y * 128;
    if (tile.z <= 16)
        down_tile<1, kF32H>(a, sA, sX, sDst, sW, tile.x, tile.y, tile.z, n0);
    else
        down_tile<2, kF32H>(a, sA, sX, sDst, sW, tile.x, tile.y, tile.z, n0);
}

}  // namespace

hipError_t launch_gateup(const FfnArgs& a, hipStream_t stream) {
    const dim3 grid(a.max_tiles, a.I / 64);
    if (a.flags & MOE_F_FP32_INTERMEDIATE)
        hipLaunchKernelGGL(moe_gateup_geglu<true>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(moe_gateup_geglu<false>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_down(const FfnArgs& a, hipStream_t stream) {
    const dim3 grid(a.max_tiles, (a.H + 127) / 128);
    if (a.flags & MOE_F_FP32_INTERMEDIATE)
        hipLaunchKernelGGL(moe_down<true>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(moe_down<false>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moe
