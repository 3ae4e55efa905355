// bf16 / fp16 batched GEMM on gfx950 MFMA.
//
// Computes Y = alpha * A' B' + beta * C (Gemm, since version 13) and the
// numpy.matmul product with broadcast batch dims (MatMul, since version 13):
// fp32 accumulation, one round-to-nearest-even conversion to the output type.
// Kernels, chosen on the host by shape:
//   dense16_t16_kernel   256x256 tiles, operands by LDS-DMA, 16x16x32 MFMAs
//                        (v_mfma_f32_16x16x32_{bf16,f16}); whole tiles without
//                        bounds checks, ragged tiles and any C form checked
//   dense16_kernel       128x128 tiles on 32x32x16 MFMAs for shapes with few
//                        tiles, its split-K partial-product mode, and the
//                        register-staged mode for unaligned operands
//   skinny*_kernel       decode-like products (a few rows): B streamed once
//   splitk_reduce_kernel fixed-order sum of split-K partials + the epilogue
// The K loops are the shared MFMA core (gemm16_core.hpp); this file adds the
// batch / tile mapping and the alpha-beta-C epilogues.
#include <algorithm>
#include <mutex>

#include "gemm16_core.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

using namespace core16;

// Y = alpha * acc + beta * C.  A C that does not vary along m (bias vector or
// scalar) is loaded once per lane for all its columns before any store, so the
// loads are in flight together; a C that varies along m is loaded per row block.
template <int BM, int BN, int DT, bool VEC>
__device__ __forceinline__ void epilogue16(const DenseArgs& p, const f32x16_t (&acc)[BM / 64][BN / 64],
                                           uint16_t* __restrict__ Y, int64_t m0, int64_t n0, int lane, int wm,
                                           int wn) {
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    const float alpha = p.alpha, beta = p.beta;
    const int64_t M = p.M, N = p.N;
    const uint16_t* __restrict__ Cp = (const uint16_t*)p.C;
    const bool vec_store = VEC && (N % 4 == 0) && (p.ldy % 4 == 0);
    const bool c_cols = Cp && p.c_sm == 0;  // C constant along m
    const int64_t nl = n0 + wn * WN + 4 * (lane >> 5);
    const int64_t ml = m0 + wm * WM + (lane & 31);

    // beta * C for the lane's columns: once for a C constant along m, per row
    // block otherwise
    float cb[TN][4][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) cb[j][q][e] = 0.0f;
    if (c_cols) {
        const bool c_vec = VEC && p.c_sn == 1 && (N % 4 == 0) && (((uintptr_t)Cp & 7) == 0);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = nl + 32 * j + 8 * q;
                if (c_vec && n < N) {
                    const u32x2_t c2 = *(const u32x2_t*)(Cp + n);
                    cb[j][q][0] = from_bits<DT>((uint16_t)c2.x);
                    cb[j][q][1] = from_bits<DT>((uint16_t)(c2.x >> 16));
                    cb[j][q][2] = from_bits<DT>((uint16_t)c2.y);
                    cb[j][q][3] = from_bits<DT>((uint16_t)(c2.y >> 16));
                } else if (!c_vec) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) cb[j][q][e] = from_bits<DT>(Cp[(n + e) * p.c_sn]);
                }
            }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) cb[j][q][e] *= beta;
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = ml + 32 * i;
        if (m >= M) continue;
        uint16_t* __restrict__ yr = Y + m * p.ldy;
        // a C that varies along m: this row block's values, all loads first
        if (Cp && !c_cols) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t n = nl + 32 * j + 8 * q + e;
                        cb[j][q][e] = n < N ? beta * from_bits<DT>(Cp[m * p.c_sm + n * p.c_sn]) : 0.0f;
                    }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = nl + 32 * j + 8 * q;
                if (n >= N) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = alpha * acc[i][j][4 * q + e] + cb[j][q][e];
                if (vec_store) {
                    u32x2_t o;
                    o.x = pack2<DT>(v[0], v[1]);
                    o.y = pack2<DT>(v[2], v[3]);
                    *(u32x2_t*)(yr + n) = o;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) yr[n + e] = to_bits<DT>(v[e]);
                }
            }
        }
    }
}

// fp32 partial sums of a split-K workgroup: the lane's 4 consecutive columns
// of each (i, j, q) go to ws[split][z] (row-major M x N)
template <int BM, int BN>
__device__ __forceinline__ void store_partial(const DenseArgs& p, const f32x16_t (&acc)[BM / 64][BN / 64],
                                              float* __restrict__ ws, int64_t m0, int64_t n0, int lane, int wm,
                                              int wn) {
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    const int64_t M = p.M, N = p.N;
    const int64_t nl = n0 + wn * WN + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + 32 * i + (lane & 31);
        if (m >= M) continue;
        float* __restrict__ row = ws + m * N;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = nl + 32 * j + 8 * q;
                if (N % 4 == 0 && n < N) {
                    *(f32x4_t*)(row + n) = f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                   acc[i][j][4 * q + 3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) row[n + e] = acc[i][j][4 * q + e];
                }
            }
    }
}

// MODE 0: register-staged loads, any shape.  MODE 1: DMA loads, ragged edge
// tiles handled in the loads and the epilogue.  MODE 2 / 3: DMA loads, every
// tile full and K a multiple of the K step (checked on the host), epilogue
// without bounds checks, with no C (2) or a bias row C (3).  MODE 4: split-K,
// DMA loads over one K range, fp32 partial tile to the workspace (the
// reduction kernel applies alpha, beta and C).
template <int BM, int BN, int DT, bool AK, bool BKM, int MODE>
__global__ __launch_bounds__(NT) void dense16_kernel(DenseArgs p, int tiles_m, int tiles_n) {
    constexpr bool VEC = MODE != 0;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int STAGE = (BM + BN) * KSTEP * 2;
    __shared__ __attribute__((aligned(1024))) char smem0[STAGE];
    __shared__ __attribute__((aligned(1024))) char smem1[STAGE];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int T = tiles_m * tiles_n;
    const int w = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    int z = w / T;
    int tm, tn;
    grouped_order(w - z * T, tiles_m, tiles_n, 4, tm, tn);
    int split = 0;
    if constexpr (MODE == 4) {
        const int NB = (int)(p.nb0 * p.nb1);
        split = z / NB;
        z -= split * NB;
    }
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const uint16_t* __restrict__ A = (const uint16_t*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1;
    const uint16_t* __restrict__ B = (const uint16_t*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1;
    uint16_t* __restrict__ Y = (uint16_t*)p.Y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t M = p.M, N = p.N;
    int64_t K = p.K;
    if constexpr (MODE == 4) {
        // this workgroup's K range; the operands start at its first k
        const int64_t k0 = split * p.kchunk;
        K = min(p.K - k0, p.kchunk);
        A += AK ? k0 : k0 * p.lda;
        B += BKM ? k0 : k0 * p.ldb;
    }

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (int)((K + KSTEP - 1) / KSTEP);
    if constexpr (VEC) {
        DmaSrc<BM, AK> srcA;
        DmaSrc<BN, BKM> srcB;
        srcA.init(A, p.lda, m0, M, K, lane);
        srcB.init(B, p.ldb, n0, N, K, lane);
        if constexpr (MODE == 2 || MODE == 3)
            mainloop_dma<BM, BN, DT, AK, BKM, false>(acc, smem0, smem1, srcA, srcB, nk, lane, wm, wn, wave);
        else if ((m0 + BM <= M) && (n0 + BN <= N) && (K % KSTEP == 0))
            mainloop_dma<BM, BN, DT, AK, BKM, false>(acc, smem0, smem1, srcA, srcB, nk, lane, wm, wn, wave);
        else
            mainloop_dma<BM, BN, DT, AK, BKM, true>(acc, smem0, smem1, srcA, srcB, nk, lane, wm, wn, wave);
    } else {
        TileSrc<BM, AK> srcA;
        TileSrc<BN, BKM> srcB;
        srcA.init(A, p.lda, m0, M, K, t);
        srcB.init(B, p.ldb, n0, N, K, t);
        mainloop<BM, BN, DT, AK, BKM, 2>(acc, smem0, smem1, srcA, srcB, nk, t, lane, wm, wn);
    }

    // Epilogue: for each (i, j, q) a lane holds row m = m0 + wm*WM + 32 i + l%32 and
    // the 4 columns n .. n+3, n = n0 + wn*WN + 32 j + 8 q + 4 (l/32).
    if constexpr (MODE == 4) {
        const int64_t NB = p.nb0 * p.nb1;
        store_partial<BM, BN>(p, acc, p.ws + ((int64_t)split * NB + z) * M * N, m0, n0, lane, wm, wn);
    } else if constexpr (MODE >= 2) {
        static_assert(BM == 256 && BN == 256, "four 32 KiB wave blocks in the two stage buffers");
        __syncthreads();  // every wave is done reading the last stage
        // full tile, no bounds checks; the results leave through LDS as whole
        // row segments.  MODE 3: C is a bias row (constant along m, contiguous
        // along n).
        char* stage = (wave < 2 ? smem0 : smem1) + (wave & 1) * (STAGE / 2);
        const int64_t col0 = n0 + wn * (BN / 2);
        const uint16_t* bias = MODE == 3 ? (const uint16_t*)p.C + col0 : nullptr;
        uint16_t* yb = Y + (m0 + wm * (BM / 2)) * p.ldy + col0;
        const int64_t ldy = p.ldy;
        wave_epilogue_lds<DT, MODE == 3>(acc, p.alpha, bias, p.beta, stage, lane,
                              [&](int r) -> uint16_t* { return yb + r * ldy; });
    } else
        epilogue16<BM, BN, DT, VEC>(p, acc, Y, m0, n0, lane, wm, wn);
}

// The same epilogue in the 16x16 accumulator layout (tile (i, j), register e
// of lane l: row 16 i + l%16, column 16 j + 4 (l/16) + e of the wave's
// 16 TM x 16 TN block); operands and output as the DMA path requires (Y
// 8-byte aligned).
template <int DT, int TM, int TN>
__device__ __forceinline__ void epilogue_t16(const DenseArgs& p, const f32x4_t (&acc)[TM][TN], uint16_t* __restrict__ Y,
                                             int64_t m0, int64_t n0, int lane, int wm, int wn) {
    const float alpha = p.alpha, beta = p.beta;
    const int64_t M = p.M, N = p.N;
    const uint16_t* __restrict__ Cp = (const uint16_t*)p.C;
    const bool vec_store = (N % 4 == 0) && (p.ldy % 4 == 0);
    const bool c_cols = Cp && p.c_sm == 0;  // C constant along m
    const int64_t nl = n0 + wn * (16 * TN) + 4 * (lane >> 4);
    const int64_t ml = m0 + wm * (16 * TM) + (lane & 15);
    float cb[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) cb[j][e] = 0.0f;
    if (c_cols) {
        const bool c_vec = p.c_sn == 1 && (N % 4 == 0) && (((uintptr_t)Cp & 7) == 0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = nl + 16 * j;
            if (c_vec && n < N) {
                const u32x2_t c2 = *(const u32x2_t*)(Cp + n);
                cb[j][0] = from_bits<DT>((uint16_t)c2.x);
                cb[j][1] = from_bits<DT>((uint16_t)(c2.x >> 16));
                cb[j][2] = from_bits<DT>((uint16_t)c2.y);
                cb[j][3] = from_bits<DT>((uint16_t)(c2.y >> 16));
            } else if (!c_vec) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) cb[j][e] = from_bits<DT>(Cp[(n + e) * p.c_sn]);
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) cb[j][e] *= beta;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = ml + 16 * i;
        if (m >= M) continue;
        uint16_t* __restrict__ yr = Y + m * p.ldy;
        if (Cp && !c_cols) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t n = nl + 16 * j + e;
                    cb[j][e] = n < N ? beta * from_bits<DT>(Cp[m * p.c_sm + n * p.c_sn]) : 0.0f;
                }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = nl + 16 * j;
            if (n >= N) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][e] + cb[j][e];
            if (vec_store) {
                u32x2_t o;
                o.x = pack2<DT>(v[0], v[1]);
                o.y = pack2<DT>(v[2], v[3]);
                *(u32x2_t*)(yr + n) = o;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) yr[n + e] = to_bits<DT>(v[e]);
            }
        }
    }
}

// BT x BT tiles (256, or 128 for shapes with too few 256-tiles to fill the
// chip) on the DMA path in the 16x16x32 MFMA form (mainloop_dma16): MODE 2 / 3
// as in dense16_kernel (every tile full, no C or a bias row C, the LDS-staged
// epilogue; BT = 256 only); MODE 1 any shape and C (checked loads on ragged
// tiles; 256-tiles leave through LDS where they can, else epilogue_t16).  Same
// work per stage as the 32x32x16 form, but measured on gfx950 the chip holds a
// higher shader clock under it (~1.55 against ~1.35 GHz on one box at 8192^3
// with both operands k-major), which more than pays for its lower
// matrix-pipe busy share.
template <int DT, int MODE, bool AK, bool BKM, int BT>
__global__ __launch_bounds__(NT) void dense16_t16_kernel(DenseArgs p, int tiles_m, int tiles_n) {
    static_assert(BT == 256 || (BT == 128 && MODE == 1), "128-tiles: any-shape mode only");
    constexpr int BM = BT, BN = BT;
    constexpr int STAGE = (BM + BN) * KSTEP * 2;
    __shared__ __attribute__((aligned(1024))) char smem0[STAGE];
    __shared__ __attribute__((aligned(1024))) char smem1[STAGE];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int T = tiles_m * tiles_n;
    const int w = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int z = w / T;
    int tm, tn;
    grouped_order(w - z * T, tiles_m, tiles_n, 4, tm, tn);
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const uint16_t* __restrict__ A = (const uint16_t*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1;
    const uint16_t* __restrict__ B = (const uint16_t*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1;
    uint16_t* __restrict__ Y = (uint16_t*)p.Y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    f32x4_t acc[BM / 32][BN / 32];  // written by the first k-block (K > 0 on this path)
    const int nk = (int)((p.K + KSTEP - 1) / KSTEP);
    DmaSrc<BM, AK> srcA;
    DmaSrc<BN, BKM> srcB;
    srcA.init(A, p.lda, m0, p.M, p.K, lane);
    srcB.init(B, p.ldb, n0, p.N, p.K, lane);
    // the loop runs at least two stages: unchecked loads only for whole tiles and K > 0
    if (MODE != 1 || (m0 + BM <= p.M && n0 + BN <= p.N && p.K % KSTEP == 0 && p.K > 0))
        mainloop_dma16<BM, BN, DT, AK, BKM, false>(acc, smem0, smem1, srcA, srcB, nk, lane, wm, wn, wave);
    else
        mainloop_dma16<BM, BN, DT, AK, BKM, true>(acc, smem0, smem1, srcA, srcB, nk, lane, wm, wn, wave);
    if constexpr (BT == 128) {
        epilogue_t16<DT, BM / 32, BN / 32>(p, acc, Y, m0, n0, lane, wm, wn);
        return;
    } else if constexpr (MODE == 1) {
        // whole tiles with no C or a bias row C leave through LDS as whole row
        // segments (16-byte stores: Y and its row stride 16-byte aligned); edge
        // tiles and a C that varies along m use the 4-value stores
        const bool staged = m0 + BM <= p.M && n0 + BN <= p.N && p.ldy % 8 == 0 && ((uintptr_t)Y & 15) == 0 &&
                            (!p.C || (p.c_sm == 0 && p.c_sn == 1 && ((uintptr_t)p.C & 7) == 0));
        if (!staged) {
            epilogue_t16<DT, 8, 8>(p, acc, Y, m0, n0, lane, wm, wn);
            return;
        }
    }
    if constexpr (BT == 256) {
        __syncthreads();
        char* stage = (wave < 2 ? smem0 : smem1) + (wave & 1) * (STAGE / 2);
        const int64_t col0 = n0 + wn * (BN / 2);
        uint16_t* yb = Y + (m0 + wm * (BM / 2)) * p.ldy + col0;
        const int64_t ldy = p.ldy;
        auto st = [&](int, int r, int c, const u32x4_t& d) { *(u32x4_t*)(yb + r * ldy + 8 * c) = d; };
        if (MODE == 3 || (MODE == 1 && p.C))
            wave_epilogue_lds16<DT, true>(acc, p.alpha, (const uint16_t*)p.C + col0, p.beta, stage, lane, st);
        else
            wave_epilogue_lds16<DT, false>(acc, p.alpha, nullptr, p.beta, stage, lane, st);
    }
}


// Split-K reduction: Y = alpha * sum_s ws[s] + beta * C, the partial sums
// added in split order (deterministic), one output element per thread.
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(DenseArgs p) {
    const int64_t MN = p.M * p.N, NB = p.nb0 * p.nb1;
    const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (f >= NB * MN) return;
    const int64_t z = f / MN, mn = f - z * MN, m = mn / p.N, n = mn - m * p.N;
    float acc = 0.0f;
    for (int s = 0; s < p.splits; ++s) acc += p.ws[(s * NB + z) * MN + mn];
    float v = p.alpha * acc;
    if (p.C) v += p.beta * from_bits<DT>(((const uint16_t*)p.C)[m * p.c_sm + n * p.c_sn]);
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    ((uint16_t*)p.Y)[z0 * p.y_bs0 + z1 * p.y_bs1 + m * p.ldy + n] = to_bits<DT>(v);
}

// ---------------------------------------------------------------------------
// Skinny products (M <= 16 rows, A and B both k-contiguous: a decode-like
// activation block against weights stored (N, K)).  The work is one read of
// B, so the kernel is built to stream B from HBM: each wave owns 16 columns
// and loads its B operand straight from global memory in the
// v_mfma_f32_16x16x32 operand layout (lane l: column l%16, 8 consecutive k at
// 8 (l/16)), one batch of SK_U k-steps of 32 in flight while the previous
// batch multiplies; A (16 rows, zero past M) sits in LDS for the workgroup's
// K range and is shared by its 4 waves.  K is split over gridDim.y ranges so
// that every CU streams; the fp32 partial products go to the split-K
// workspace and splitk_reduce_kernel adds them in a fixed order and applies
// the epilogue.  (skinny1_kernel below covers shapes with enough columns in
// one pass.)
constexpr int SK_COLS = 64;      // columns per workgroup (4 waves x 16)
constexpr int SK_U = 16;         // k-steps of 32 per batch of loads
constexpr int SK_KMAX = 2048;    // k per workgroup (A rows in LDS: 16 x 2048 x 2 bytes)
constexpr int SK_ROWB = SK_KMAX * 2 + 64;  // LDS row pitch of A (bytes)

// Branch-free 16-byte loads for the streaming kernels: through a buffer
// resource, an offset at or past 2^31 reads zeros, so masked lanes need no
// branch (a branch around a load makes the compiler wait for every load in
// flight before the next use) and the loads of a batch stay in flight together.
constexpr uint32_t SK_OOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4_t sk_load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    if constexpr (DT == 0)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                     c, 0, 0, 0);
}

template <int DT>
__global__ __launch_bounds__(256) void skinny_kernel(DenseArgs p) {
    __shared__ __attribute__((aligned(16))) char As[16 * SK_ROWB];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t z = blockIdx.z, z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const int split = blockIdx.y;
    const int64_t M = p.M, N = p.N, K = p.K, NB = p.nb0 * p.nb1;
    const int64_t k0 = (int64_t)split * p.kchunk;
    const int64_t kn = min(p.kchunk, K - k0);  // > 0: the launcher sizes the splits
    const uint16_t* __restrict__ A = (const uint16_t*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1 + k0;
    const uint16_t* __restrict__ B = (const uint16_t*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1 + k0;
    const int64_t n = (int64_t)blockIdx.x * SK_COLS + 16 * wave + (lane & 15);
    const int kl = 8 * (lane >> 4);  // this lane's k offset inside a k-step
    const bool nok = n < N;
    const __amdgpu_buffer_rsrc_t rb = sk_rsrc(B);
    const uint32_t boff = (uint32_t)((n * p.ldb + kl) * 2);
    const int nsteps = (int)((kn + 31) / 32);

    // B of one batch of k-steps (zeros past K or N); 16-byte loads, K % 8 == 0
    auto load_b = [&](u32x4_t (&r)[SK_U], int j0) {
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int64_t k = 32 * (int64_t)(j0 + u) + kl;
            r[u] = sk_load(rb, nok && k < kn ? boff + 64u * (uint32_t)(j0 + u) : SK_OOB);
        }
    };
    u32x4_t bcur[SK_U], bnxt[SK_U];
    load_b(bcur, 0);

    // A rows 0..15 of this K range into LDS (rows past M: zeros), 4 loads in
    // flight per thread
    {
        const int kc = (int)((kn + 7) / 8);  // 16-byte chunks per row
        const __amdgpu_buffer_rsrc_t rsa = sk_rsrc(A);
        for (int c0 = 0; c0 < 16 * kc; c0 += 1024) {
            u32x4_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + t + 256 * u, m = c / kc, q = c - m * kc;
                v[u] = sk_load(rsa, c < 16 * kc && m < M ? (uint32_t)((m * p.lda + 8 * q) * 2) : SK_OOB);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + t + 256 * u, m = c / kc, q = c - m * kc;
                if (c < 16 * kc) *(u32x4_t*)(As + m * SK_ROWB + 16 * q) = v[u];
            }
        }
    }
    __syncthreads();

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const char* Arow = As + (lane & 15) * SK_ROWB + 2 * kl;
    // batch j0 of MFMAs on buffer r (A fragment: row l%16, k = 32 j + 8 (l/16)
    // .. +7; k past kn reads zeros: LDS there was never written, B is zero too)
    auto mma = [&](const u32x4_t (&r)[SK_U], int j0) {
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int j = j0 + u;
            u32x4_t av = {0u, 0u, 0u, 0u};
            if (32 * j + kl < kn) av = *(const u32x4_t*)(Arow + 64 * j);
            acc = mfma16x16x32<DT>(av, r[u], acc);
        }
    };
    // two buffers in turn (no register copies, which would wait for the loads):
    // one batch of loads in flight while the other batch multiplies
    for (int j0 = 0; j0 < nsteps; j0 += 2 * SK_U) {
        load_b(bnxt, j0 + SK_U);
        mma(bcur, j0);
        load_b(bcur, j0 + 2 * SK_U);
        mma(bnxt, j0 + SK_U);
    }

    // result register r of lane l: row 4 (l/16) + r, column l%16
    if (!nok) return;
    float* __restrict__ ws = p.ws + ((int64_t)split * NB + z) * M * N;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t m = 4 * (lane >> 4) + r;
        if (m < M) ws[m * N + n] = acc[r];
    }
}

// Single-pass variant (one launch, no workspace): a workgroup owns 16 CG
// columns, each of its NW waves (4 or 8) takes one contiguous K range for all
// of them; A fragments come straight from global memory too (the A rows, at
// most 16, are small and stay in L2); the NW partial tiles are added in LDS
// in a fixed order and wave 0 applies alpha * acc + beta * C and stores Y.
// CG = 2 lets each A fragment feed two MFMAs, so the workgroup reads A once
// per 32 columns: the choice once A has more than 8 rows, where A's reads
// are as many as B's.  SB keeps each batch of loads issued ahead of the
// MFMAs on the other batch (scheduling barriers), which the CG = 2 form
// needs to keep both batches in flight.  SK1_U: k-steps per batch of loads.
template <int DT, int CG, int NW, bool SB, int SK1_U>
__global__ __launch_bounds__(64 * NW) void skinny1_kernel(DenseArgs p) {
    __shared__ float red[NW - 1][CG][64][4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t z = blockIdx.y, z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const int64_t M = p.M, N = p.N, K = p.K;
    // this wave's K range: steps of 32, split as evenly as whole steps allow
    const int64_t steps = (K + 31) / 32;
    const int64_t s0 = steps * wave / NW, s1 = steps * (wave + 1) / NW;
    const int nst = (int)(s1 - s0);
    const int64_t kbase = 32 * s0;
    const int64_t m = lane & 15;
    const int kl = 8 * (lane >> 4);
    const bool mok = m < M;
    int64_t n[CG];
    bool nok[CG];
    uint32_t boff[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        n[c] = (int64_t)blockIdx.x * (16 * CG) + 16 * c + (lane & 15);
        nok[c] = n[c] < N;
        boff[c] = (uint32_t)((n[c] * p.ldb + kbase + kl) * 2);
    }
    const __amdgpu_buffer_rsrc_t rsb = sk_rsrc((const uint16_t*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1);
    const __amdgpu_buffer_rsrc_t rsa = sk_rsrc((const uint16_t*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1);
    const uint32_t aoff = (uint32_t)((m * p.lda + kbase + kl) * 2);
    // step j of this wave reads k = kbase + 32 j + kl .. + 7, inside the
    // wave's range and below K (K % 8 == 0) for j < jl; the row and column
    // bounds fold into per-lane limits (0: nothing to read)
    const int64_t kn = K - kbase - kl;
    const int jl = kn <= 0 ? 0 : (kn + 31) / 32 < nst ? (int)((kn + 31) / 32) : nst;
    const int jla = mok ? jl : 0;
    int jlb[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) jlb[c] = nok[c] ? jl : 0;

    auto load = [&](u32x4_t (&rb)[CG][SK1_U], u32x4_t (&ra)[SK1_U], int j0) {
#pragma unroll
        for (int u = 0; u < SK1_U; ++u) {
            const int j = j0 + u;
#pragma unroll
            for (int c = 0; c < CG; ++c) rb[c][u] = sk_load(rsb, j < jlb[c] ? boff[c] + 64u * (uint32_t)j : SK_OOB);
            ra[u] = sk_load(rsa, j < jla ? aoff + 64u * (uint32_t)j : SK_OOB);
        }
    };
    f32x4_t acc[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto mma = [&](const u32x4_t (&rb)[CG][SK1_U], const u32x4_t (&ra)[SK1_U]) {
#pragma unroll
        for (int u = 0; u < SK1_U; ++u)
#pragma unroll
            for (int c = 0; c < CG; ++c) acc[c] = mfma16x16x32<DT>(ra[u], rb[c][u], acc[c]);
    };
    u32x4_t b0[CG][SK1_U], a0[SK1_U], b1[CG][SK1_U], a1[SK1_U];
    load(b0, a0, 0);
    // straight-line ping-pong (steps past the range load zeros)
    for (int j0 = 0; j0 < nst; j0 += 2 * SK1_U) {
        load(b1, a1, j0 + SK1_U);
        if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
        mma(b0, a0);
        if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
        load(b0, a0, j0 + 2 * SK1_U);
        if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
        mma(b1, a1);
        if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
    }
    // waves 1.. hand their tiles to wave 0, which adds them in wave order
    if (wave > 0) {
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave - 1][c][lane][r] = acc[c][r];
    }
    __syncthreads();
    if (wave != 0) return;
    uint16_t* __restrict__ Y = (uint16_t*)p.Y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const uint16_t* Cp = (const uint16_t*)p.C;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
#pragma unroll
        for (int w = 0; w < NW - 1; ++w)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[c][r] += red[w][c][lane][r];
        // result register r of lane l: row 4 (l/16) + r, column l%16
        if (!nok[c]) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t mm = 4 * (lane >> 4) + r;
            if (mm < M) {
                float v = p.alpha * acc[c][r];
                if (Cp) v += p.beta * from_bits<DT>(Cp[mm * p.c_sm + n[c] * p.c_sn]);
                Y[mm * p.ldy + n[c]] = to_bits<DT>(v);
            }
        }
    }
}

// Skinny products with n-contiguous B (MatMul's own layout: a few activation
// rows against weights stored (K, N)), M <= 4.  B rows are read as 16-byte
// chunks of 8 columns (a wave reads RPI rows x CW columns per instruction)
// and multiplied on the vector ALU: each lane keeps MR x 8 fp32 sums for its
// 8 columns over its rows (the work per B byte is MR/2 multiply-adds, well
// under the ALU rate at the HBM rate).  A is held in LDS transposed to (K,
// MR) so one small LDS read per row gives all MR values.  A workgroup owns CW
// columns over the whole of K, split in NW ranges over its waves (4, or 8
// when there are few workgroups); the partial sums are reduced across the
// lanes that share columns (shuffles) and across the waves in LDS in a fixed
// order; wave 0 applies the epilogue.
template <int DT, int MR, int CW, int NW>
__global__ __launch_bounds__(64 * NW) void skinny_nmaj_kernel(DenseArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint16_t At[];  // (K, MR)
    __shared__ float red[NW - 1][CW / 8][MR][8];
    constexpr int LPR = CW / 8, RPI = 64 / LPR, U = 8;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t z = blockIdx.y, z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint16_t* __restrict__ A = (const uint16_t*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1;
    // Workgroups of neighbouring columns share B's cache lines: keep them on
    // one XCD (workgroup b runs on XCD b % 8), so each line leaves HBM once.
    const int cg = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int c = lane % LPR, r = lane / LPR;
    const int64_t n = (int64_t)cg * CW + 8 * c;
    const bool nok = n < N;  // N % 8 == 0: whole chunks
    const int64_t groups = (K + RPI - 1) / RPI;
    const int64_t g0 = groups * wave / NW, g1 = groups * (wave + 1) / NW;
    const int ng = (int)(g1 - g0);
    const __amdgpu_buffer_rsrc_t rsb = sk_rsrc((const uint16_t*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1);
    // this lane's first row; K fits in LDS, so rows are 32-bit
    const int kb = (int)(g0 * RPI) + r, Ki = (int)K;
    // step i reads row kb + RPI i: inside the wave's range and below K for
    // i < il (0 for masked columns); offsets advance by a fixed stride
    const int il = !nok || kb >= Ki ? 0 : min(ng, (Ki - kb + RPI - 1) / RPI);
    const uint32_t boff = (uint32_t)(((int64_t)kb * p.ldb + n) * 2), bstep = (uint32_t)(RPI * p.ldb * 2);

    float acc[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] = 0.0f;
    auto load = [&](u32x4_t (&rb)[U], int i0) {
#pragma unroll
        for (int u = 0; u < U; ++u) rb[u] = sk_load(rsb, i0 + u < il ? boff + bstep * (uint32_t)(i0 + u) : SK_OOB);
    };
    auto fma_rows = [&](const u32x4_t (&rb)[U], int i0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // rows past this wave's range or K hold B = 0: read any valid A row
            const int k = min(kb + RPI * (i0 + u), Ki - 1);
            float av[MR];
            if constexpr (MR == 1) {
                av[0] = from_bits<DT>(At[k]);
            } else if constexpr (MR == 2) {
                const uint32_t w = *(const uint32_t*)(At + 2 * k);
                av[0] = from_bits<DT>((uint16_t)w);
                av[1] = from_bits<DT>((uint16_t)(w >> 16));
            } else {
                const u32x2_t w = *(const u32x2_t*)(At + 4 * k);
                av[0] = from_bits<DT>((uint16_t)w.x);
                av[1] = from_bits<DT>((uint16_t)(w.x >> 16));
                av[2] = from_bits<DT>((uint16_t)w.y);
                av[3] = from_bits<DT>((uint16_t)(w.y >> 16));
            }
            const uint32_t bw[4] = {rb[u].x, rb[u].y, rb[u].z, rb[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float bv = from_bits<DT>((uint16_t)(bw[e >> 1] >> (16 * (e & 1))));
#pragma unroll
                for (int m = 0; m < MR; ++m) acc[m][e] = __builtin_fmaf(av[m], bv, acc[m][e]);
            }
        }
    };
    u32x4_t b0[U], b1[U];
    load(b0, 0);  // the first B rows are on their way while A is staged
    {
        // A rows as 16-byte chunks (K % 8 == 0), UA loads in flight per thread
        // (one load then store per iteration would wait out every load);
        // rows MR > M hold zeros
        constexpr int UA = 4;
        const __amdgpu_buffer_rsrc_t rsa = sk_rsrc(A);
        const int64_t kc = K / 8, total = kc * MR;
        for (int64_t c0 = 0; c0 < total; c0 += 64 * NW * UA) {
            u32x4_t v[UA];
#pragma unroll
            for (int u = 0; u < UA; ++u) {
                const int64_t c = c0 + t + 64 * NW * u, m = c / kc, q = c - m * kc;
                v[u] = sk_load(rsa, c < total && m < M ? (uint32_t)((m * p.lda + 8 * q) * 2) : SK_OOB);
            }
#pragma unroll
            for (int u = 0; u < UA; ++u) {
                const int64_t c = c0 + t + 64 * NW * u, m = c / kc, q = c - m * kc;
                if (c < total) {
                    if constexpr (MR == 1) {
                        *(u32x4_t*)(At + 8 * q) = v[u];
                    } else {
                        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) At[(8 * q + e) * MR + m] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
    }
    __syncthreads();
    // straight-line ping-pong: loads past the range are out of bounds (no
    // memory access, zeros), so the loop needs no exits in the middle
    for (int i0 = 0; i0 < ng; i0 += 2 * U) {
        load(b1, i0 + U);
        fma_rows(b0, i0);
        load(b0, i0 + 2 * U);
        fma_rows(b1, i0 + U);
    }
    // lanes with the same c hold the same columns: add over r (lane bits >= log2 LPR)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][e] += __shfl_xor(acc[m][e], off);
    if (wave > 0 && r == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave - 1][c][m][e] = acc[m][e];
    }
    __syncthreads();
    if (wave != 0 || r != 0 || !nok) return;
    uint16_t* __restrict__ Y = (uint16_t*)p.Y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const uint16_t* Cp = (const uint16_t*)p.C;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= M) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[m][e];
#pragma unroll
            for (int w = 0; w < NW - 1; ++w) v += red[w][c][m][e];
            v *= p.alpha;
            if (Cp) v += p.beta * from_bits<DT>(Cp[m * p.c_sm + (n + e) * p.c_sn]);
            Y[m * p.ldy + n + e] = to_bits<DT>(v);
        }
    }
}

template <int DT, int MR>
hipError_t launch_skinny_nmaj(const DenseArgs& a, hipStream_t s) {
    const int64_t NB = a.nb0 * a.nb1;
    // at least 60 KB of LDS per workgroup, so that at most two share a CU
    // (its ~100 VGPRs would let four in; measured at M = 1, N = 28672,
    // K = 8192: 0.135 ms with four resident, 0.108 with three, 0.105 with two)
    const size_t lds = std::max<size_t>((size_t)a.K * MR * 2, 61440);
    // 32-column groups (64-byte row pieces) once there is one per CU: at M = 1,
    // N = K = 8192 (256 groups) 30 against 35 us with 16-column groups; fewer
    // than 256 groups of 16 columns: 8 waves per workgroup
    const int64_t g16 = (a.N + 15) / 16;
    if ((a.N + 31) / 32 * NB >= 256) {
        hipLaunchKernelGGL((skinny_nmaj_kernel<DT, MR, 32, 4>), dim3((unsigned)((a.N + 31) / 32), (unsigned)NB),
                           dim3(256), lds, s, a);
    } else if (g16 * NB >= 256) {
        hipLaunchKernelGGL((skinny_nmaj_kernel<DT, MR, 16, 4>), dim3((unsigned)g16, (unsigned)NB), dim3(256), lds, s, a);
    } else {
        hipLaunchKernelGGL((skinny_nmaj_kernel<DT, MR, 16, 8>), dim3((unsigned)g16, (unsigned)NB), dim3(512), lds, s, a);
    }
    return hipGetLastError();
}

template <int BM, int BN, int DT, bool AK, bool BKM, int MODE>
hipError_t launch_cfg(const DenseArgs& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1 * (MODE == 4 ? a.splits : 1);
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dense16_kernel<BM, BN, DT, AK, BKM, MODE>), dim3((unsigned)total), dim3(NT), 0, s, a,
                       (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

template <int DT, int MODE, bool AK, bool BKM, int BT>
hipError_t launch_t16(const DenseArgs& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + BT - 1) / BT, tiles_n = (a.N + BT - 1) / BT;
    const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dense16_t16_kernel<DT, MODE, AK, BKM, BT>), dim3((unsigned)total), dim3(NT), 0, s, a,
                       (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

template <int BM, int BN, int DT, int MODE>
hipError_t launch_layout(const DenseArgs& a, hipStream_t s) {
    if constexpr ((BM == 256 && MODE >= 1 && MODE <= 3) || (BM == 128 && MODE == 1)) {
        if (a.a_kmajor && a.b_kmajor) return launch_t16<DT, MODE, true, true, BM>(a, s);
        if (a.a_kmajor) return launch_t16<DT, MODE, true, false, BM>(a, s);
        if (a.b_kmajor) return launch_t16<DT, MODE, false, true, BM>(a, s);
        return launch_t16<DT, MODE, false, false, BM>(a, s);
    } else {  // (an else, so that the 32x32 kernel is not instantiated for these modes)
        if (a.a_kmajor && a.b_kmajor) return launch_cfg<BM, BN, DT, true, true, MODE>(a, s);
        if (a.a_kmajor && !a.b_kmajor) return launch_cfg<BM, BN, DT, true, false, MODE>(a, s);
        if (!a.a_kmajor && a.b_kmajor) return launch_cfg<BM, BN, DT, false, true, MODE>(a, s);
        return launch_cfg<BM, BN, DT, false, false, MODE>(a, s);
    }
}

// The kernel choice for one launch and the split-K workspace it needs.
struct Plan16 {
    enum Kind { T16_FULL, T16_BIAS, T16_ANY, SKINNY_NMAJ, SKINNY1, SKINNY_SPLIT, SPLIT128, T128_VEC, T128_REG } kind;
    int mr = 0;           // SKINNY_NMAJ: rows per workgroup pass (1, 2, 4)
    int64_t splits = 0;   // SKINNY_SPLIT / SPLIT128: K ranges
    int64_t kchunk = 0;   // their length
    int64_t groups = 0;   // SKINNY_SPLIT: 64-column workgroups
    size_t ws_bytes = 0;  // fp32 partial products, splits x batches x M x N
};

Plan16 plan16(const DenseArgs& a) {
    Plan16 pl;
    // 16-byte loads need 16-byte aligned bases, row strides that are multiples
    // of 8 elements and a contiguous extent (K, M or N) that is a multiple of 8.
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    const bool a_ok = al16(a.A) && a.lda % 8 == 0 && (a.a_kmajor ? a.K % 8 == 0 : a.M % 8 == 0) &&
                      a.a_bs0 % 8 == 0 && a.a_bs1 % 8 == 0;
    const bool b_ok = al16(a.B) && a.ldb % 8 == 0 && (a.b_kmajor ? a.K % 8 == 0 : a.N % 8 == 0) &&
                      a.b_bs0 % 8 == 0 && a.b_bs1 % 8 == 0;
    const bool y_ok = ((uintptr_t)a.Y & 7) == 0 && a.y_bs0 % 4 == 0 && a.y_bs1 % 4 == 0;
    // DMA byte offsets are 32-bit: one tile's rows must span < 2 GiB per operand
    const bool span_ok = (a.a_kmajor ? 256 * a.lda * 2 : 64 * a.lda * 2) < (1LL << 31) &&
                         (a.b_kmajor ? 256 * a.ldb * 2 : 64 * a.ldb * 2) < (1LL << 31);
    const bool vec = a_ok && b_ok && y_ok && span_ok;
    const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256) * a.nb0 * a.nb1;
    const int forced = tile_override();
    if (vec && forced == 128) {
        pl.kind = Plan16::T128_VEC;
        return pl;
    }
    if (vec && (big_tiles >= 256 || forced == 256)) {
        // every tile full: epilogue without bounds checks (8-byte stores need
        // N and the row stride to be multiples of 4)
        const bool full = a.M % 256 == 0 && a.N % 256 == 0 && a.K % KSTEP == 0 && a.K > 0 && a.ldy % 4 == 0;
        if (full && !a.C) pl.kind = Plan16::T16_FULL;
        else if (full && a.c_sm == 0 && a.c_sn == 1 && ((uintptr_t)a.C & 7) == 0) pl.kind = Plan16::T16_BIAS;
        else pl.kind = Plan16::T16_ANY;
        return pl;
    }
    const int64_t NB = a.nb0 * a.nb1;
    // Skinny (M <= 16) with both operands k-contiguous: stream B, split K.
    // Skinny (M <= 4) against n-contiguous B, A (K x MR x 2 bytes) within 60 KB
    // of LDS, with enough columns to fill the chip with 16-column workgroups
    // or K short enough for fewer workgroups of 8 waves.
    // (buffer offsets are 32-bit: one batch entry of B below 2 GiB)
    const bool b_span = (a.b_kmajor ? a.N * a.ldb : a.K * a.ldb) * 2 < (1LL << 31);
    const bool a_span = a.M * a.lda * 2 < (1LL << 31);
    // (measured: ahead of the split-K path for M <= 2 at any K and for M <= 4
    // up to K = 4096; behind it for 3-4 rows and longer K; with fewer than
    // 256 groups and K <= 8192, M = 1-4, N = 512-2048: 9.1-16.1 us per call
    // against 22-23 us split-K)
    if (vec && b_span && a_span && (a.M <= 2 || (a.M <= 4 && a.K <= 4096)) && a.a_kmajor && !a.b_kmajor &&
        a.K >= 1024 && NB <= 65535 &&
        ((a.N + 15) / 16 * NB >= 256 || a.K <= 8192) && (a.N + 15) / 16 <= 0x7fffffff) {
        const int mr = a.M <= 1 ? 1 : a.M <= 2 ? 2 : 4;
        if (a.K * mr * 2 <= 61440) {
            pl.kind = Plan16::SKINNY_NMAJ;
            pl.mr = mr;
            return pl;
        }
    }
    // Single pass (no workspace, one launch) with at least 512 groups of 16
    // columns, or fewer groups of 8 waves each while K is short enough that
    // one workgroup streams its columns' K in less time than the split-K path
    // takes (measured per call: 10-13 us at K <= 8192 and 15-21 us at
    // K = 9000-16384, against 26-30 us split-K; 33 against 26 us at K = 28672)
    const int64_t g16 = (a.N + 15) / 16;
    if (vec && b_span && a_span && a.M <= 16 && a.a_kmajor && a.b_kmajor && a.K >= 1024 && NB <= 65535 &&
        g16 <= 0x7fffffff && (g16 * NB >= 512 || a.K <= 16384)) {
        pl.kind = Plan16::SKINNY1;
        return pl;
    }
    if (vec && b_span && a_span && a.M <= 16 && a.a_kmajor && a.b_kmajor && a.K >= 1024 && NB <= 65535) {
        const int64_t groups = (a.N + SK_COLS - 1) / SK_COLS;
        int64_t S = std::max<int64_t>((512 + groups * NB - 1) / (groups * NB), (a.K + SK_KMAX - 1) / SK_KMAX);
        S = std::min<int64_t>(S, (a.K + 255) / 256);
        const int64_t kchunk = std::min<int64_t>(((a.K + S - 1) / S + 255) / 256 * 256, SK_KMAX);
        S = (a.K + kchunk - 1) / kchunk;
        if (groups <= 0x7fffffff && S <= 65535) {
            pl.kind = Plan16::SKINNY_SPLIT;
            pl.groups = groups;
            pl.splits = S;
            pl.kchunk = kchunk;
            pl.ws_bytes = (size_t)(S * NB * a.M * a.N) * sizeof(float);
            return pl;
        }
    }
    // Few output tiles and a long K: split K over several workgroups per tile
    // so that the whole chip streams the operands, then reduce.
    const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128) * NB;
    if (vec && t128 < 128 && a.K >= 2048) {
        int64_t S = std::min<int64_t>(std::min<int64_t>(512 / t128, a.K / 512), 32);
        if (S >= 2) {
            const int64_t kchunk = ((a.K + S - 1) / S + KSTEP - 1) / KSTEP * KSTEP;
            S = (a.K + kchunk - 1) / kchunk;
            pl.kind = Plan16::SPLIT128;
            pl.splits = S;
            pl.kchunk = kchunk;
            pl.ws_bytes = (size_t)(S * NB * a.M * a.N) * sizeof(float);
            return pl;
        }
    }
    pl.kind = vec ? Plan16::T128_VEC : Plan16::T128_REG;
    return pl;
}

// Launches the planned kernels; ws holds pl.ws_bytes when the plan splits K.
template <int DT>
hipError_t run16(const DenseArgs& a, const Plan16& pl, float* ws, hipStream_t s) {
    const int64_t NB = a.nb0 * a.nb1;
    switch (pl.kind) {
        case Plan16::T16_FULL: return launch_layout<256, 256, DT, 2>(a, s);
        case Plan16::T16_BIAS: return launch_layout<256, 256, DT, 3>(a, s);
        case Plan16::T16_ANY: return launch_layout<256, 256, DT, 1>(a, s);
        case Plan16::SKINNY_NMAJ:
            if (pl.mr == 1) return launch_skinny_nmaj<DT, 1>(a, s);
            if (pl.mr == 2) return launch_skinny_nmaj<DT, 2>(a, s);
            return launch_skinny_nmaj<DT, 4>(a, s);
        case Plan16::SKINNY1:
            // fewer than 512 groups of 16 columns: 8 waves per workgroup, so a
            // CU keeps as many loads in flight as two workgroups of 4 would;
            // else, more than 8 rows: 32 columns per workgroup of 4 waves
            // (measured 10-20% ahead with B in the last-level cache, even
            // with it in HBM); else 16 columns per workgroup of 8 waves with
            // batches of 4 k-steps (69 VGPRs, three workgroups per CU; with B
            // from HBM 6-9% ahead of 4 waves with batches of 8 at N = K = 8192
            // and N = 28672)
            if ((a.N + 15) / 16 * NB < 512)
                hipLaunchKernelGGL((skinny1_kernel<DT, 1, 8, true, 8>), dim3((unsigned)((a.N + 15) / 16), (unsigned)NB),
                                   dim3(512), 0, s, a);
            else if (a.M > 8 && (a.N + 31) / 32 * NB >= 256)
                hipLaunchKernelGGL((skinny1_kernel<DT, 2, 4, true, 8>), dim3((unsigned)((a.N + 31) / 32), (unsigned)NB),
                                   dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((skinny1_kernel<DT, 1, 8, false, 4>), dim3((unsigned)((a.N + 15) / 16), (unsigned)NB),
                                   dim3(512), 0, s, a);
            return hipGetLastError();
        case Plan16::SKINNY_SPLIT:
        case Plan16::SPLIT128: {
            DenseArgs b = a;
            b.kchunk = pl.kchunk;
            b.splits = (int)pl.splits;
            b.ws = ws;
            hipError_t e;
            if (pl.kind == Plan16::SKINNY_SPLIT) {
                hipLaunchKernelGGL(skinny_kernel<DT>, dim3((unsigned)pl.groups, (unsigned)pl.splits, (unsigned)NB),
                                   dim3(256), 0, s, b);
                e = hipGetLastError();
            } else {
                e = launch_layout<128, 128, DT, 4>(b, s);
            }
            if (e != hipSuccess) return e;
            const int64_t elems = NB * a.M * a.N;
            hipLaunchKernelGGL(splitk_reduce_kernel<DT>, dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, s, b);
            return hipGetLastError();
        }
        case Plan16::T128_VEC: return launch_layout<128, 128, DT, 1>(a, s);
        case Plan16::T128_REG: return launch_layout<128, 128, DT, 0>(a, s);
    }
    return hipErrorInvalidValue;
}

// scratch == nullptr: split-K partials in stream-ordered memory taken and
// returned around the launch; otherwise the caller's scratch (its size checked
// against the plan before anything is enqueued).
const char* plan_name(const Plan16& pl) {
    switch (pl.kind) {
        case Plan16::T16_FULL: return "256x256x64 tiles, 16x16x32 MFMA, DMA, whole tiles, no C";
        case Plan16::T16_BIAS: return "256x256x64 tiles, 16x16x32 MFMA, DMA, whole tiles, bias row";
        case Plan16::T16_ANY: return "256x256x64 tiles, 16x16x32 MFMA, DMA, ragged tiles / any C";
        case Plan16::SKINNY_NMAJ: return "skinny rows against n-contiguous B (vector ALU, B streamed once)";
        case Plan16::SKINNY1: return "skinny rows against k-contiguous B (16 or 32 columns per workgroup)";
        case Plan16::SKINNY_SPLIT: return "skinny rows, K split over workgroups + fixed-order reduction";
        case Plan16::SPLIT128: return "128x128x64 tiles, K split over workgroups + fixed-order reduction";
        case Plan16::T128_VEC: return "128x128x64 tiles, 16x16x32 MFMA, DMA";
        case Plan16::T128_REG: return "128x128x64 tiles, 32x32x16 MFMA, register-staged loads";
    }
    return "?";
}

// Split-K partials outside graph capture: one workspace per GPU, kept for
// the life of the process and grown on demand (stream-ordered: the old buffer
// is freed and the new one taken on the calling stream), and an event that
// orders every call using it after the previous one, whatever its stream.
// This replaces a hipMallocAsync / hipFreeAsync pair per call, whose host
// cost (~15 us in hipFreeAsync) exceeded the kernels' time on small shapes.
// Under graph capture the partials stay in per-call stream-ordered memory.
struct SplitWorkspace {
    std::mutex mu;
    float* ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t last = nullptr;
};
constexpr int WS_DEVICES = 64;
SplitWorkspace split_ws[WS_DEVICES];

template <int DT>
hipError_t run_split_cached(const DenseArgs& a, const Plan16& pl, hipStream_t s, SplitWorkspace& w) {
    std::lock_guard<std::mutex> lock(w.mu);
    hipError_t e;
    if (!w.last && (e = hipEventCreateWithFlags(&w.last, hipEventDisableTiming)) != hipSuccess) {
        w.last = nullptr;
        return e;
    }
    if ((e = hipStreamWaitEvent(s, w.last, 0)) != hipSuccess) return e;
    if (pl.ws_bytes > w.bytes) {
        if (w.ptr && (e = hipFreeAsync(w.ptr, s)) != hipSuccess) return e;
        w.ptr = nullptr;
        w.bytes = 0;
        if ((e = hipMallocAsync((void**)&w.ptr, pl.ws_bytes, s)) != hipSuccess) {
            w.ptr = nullptr;
            return e;
        }
        w.bytes = pl.ws_bytes;
    }
    e = run16<DT>(a, pl, w.ptr, s);
    const hipError_t f = hipEventRecord(w.last, s);
    return e != hipSuccess ? e : f;
}

template <int DT>
hipError_t launch_dt(const DenseArgs& a, hipStream_t s, const DenseScratch* scratch) {
    const Plan16 pl = plan16(a);
    if (log_enabled())
        log_choice("%s M=%lld N=%lld K=%lld batches=%lld A %s B %s: %s%s splits=%lld scratch=%s", DT == 0 ? "bf16" : "fp16",
                   (long long)a.M, (long long)a.N, (long long)a.K, (long long)(a.nb0 * a.nb1),
                   a.a_kmajor ? "k-contiguous" : "m-contiguous", a.b_kmajor ? "k-contiguous" : "n-contiguous",
                   plan_name(pl), tile_override() ? " (OMM_TILE)" : "", (long long)pl.splits,
                   pl.ws_bytes == 0 ? "none" : scratch ? "static" : "stream-ordered");
    if (pl.ws_bytes == 0) return run16<DT>(a, pl, nullptr, s);
    if (scratch) {
        if (!scratch->ptr || pl.ws_bytes > scratch->bytes) return hipErrorInvalidValue;
        return run16<DT>(a, pl, (float*)scratch->ptr, s);
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    int dev = -1;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone && dev >= 0 && dev < WS_DEVICES)
        return run_split_cached<DT>(a, pl, s, split_ws[dev]);
    float* ws = nullptr;
    if ((e = hipMallocAsync((void**)&ws, pl.ws_bytes, s)) != hipSuccess) return e;
    e = run16<DT>(a, pl, ws, s);
    const hipError_t f = hipFreeAsync(ws, s);
    return e != hipSuccess ? e : f;
}

}  // namespace

hipError_t launch_dense16(const DenseArgs& a, int dt, hipStream_t s, const DenseScratch* scratch) {
    return dt == 0 ? launch_dt<0>(a, s, scratch) : launch_dt<1>(a, s, scratch);
}

size_t dense16_scratch_bytes(const DenseArgs& a) { return plan16(a).ws_bytes; }

}  // namespace omm
