// GroupedMatMul (version 29) on gfx950.
//
//   output[m, i, :] = input[m, :] @ weights[g] (+ bias[g, :]),  g = group_indices[m, i]
//
// The page defines the result through Gather + Expand + MatMul and asks
// runtimes for a fused grouped product that never forms the gathered
// (M*S, K, N) weights.  Here the (m, i) pairs are counting-sorted by group on
// the device and every group's pairs run as the rows of one GEMM against
// weights[g]:
//   1. routing, four short kernels: zero the counters; per-workgroup LDS
//      histograms of the M*S indices over the G groups folded into global
//      counts (invalid indices are counted, not routed); exclusive scans of
//      the counts and of the per-group tile counts into the tile table
//      (group, first sorted pair, end of the group's pairs, walk run); the
//      scatter of pair ids p = m*S + i
//      into group order, each workgroup reserving its range per group with
//      one global atomic;
//   2. grouped16_kernel: one 256x256 output tile per workgroup (128x256 for a
//      group's last tile of at most 128 rows), rows gathered
//      from input[p / S], B = weights[g] (n contiguous, read through the
//      transposing LDS path), 16x16x32 MFMAs (32x32x16 on the element-wise
//      path for unaligned operands), epilogue adds bias[g] in fp32, rounds
//      once and writes each row to output[p].  The grid is the upper bound
//      (M*S/BM + G) x (N/BN); the routed tiles, walked in runs aligned to the
//      groups, are split evenly over the 8 XCDs and each XCD's surplus
//      workgroups exit.
//   Weight-only quantised experts (int8/uint8 weights with block scales) run
//   the same routing and grouped16_dq_dma_kernel / grouped16_dq_kernel, which
//   dequantise each weight tile on its way into the MFMAs; fp32 / fp64 run it
//   with 128-row tiles and grouped_fp_kernel.
// No host synchronisation between the two.  Each output row depends only on
// its own pair, so the order of pairs inside a group never changes a value.
#include "gemm16_core.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

constexpr int ROUTE_THREADS = 1024;
constexpr int GBM = 256, GBN = 256;  // grouped tile
// Tile order of every grouped kernel (run_tile): runs of row tiles that the
// router aligns to the groups -- a group of at most RUN_MAX row tiles is one
// run, a larger one is cut into balanced runs of at most RUN_ROWS -- each
// walked column tile by column tile, so the 32 tiles an XCD runs at once
// share the weight panels of one group.  Measured on the benchmark routing
// (64 experts of 8 or 9 row tiles) against fixed runs of 8 (4 for the
// quantised-expert kernels) that straddle two experts: 3-4 % faster for the
// bf16, quantised-expert, fp32 and fp64 kernels; capping runs at 4 rows was
// slower.
constexpr int RUN_MAX = 12, RUN_ROWS = 8;
constexpr int MAX_G = 8192;          // groups handled by the single-workgroup router

// workspace layout (bytes, from a 256-byte aligned base)
//   [0, 64)                   header: int32 num_tiles, int32 invalid_count
//   [64, 64 + 4G)             per-group pair counts
//   [64 + 4G, 64 + 8G)        per-group scatter cursors
//   [tiles, + 16 TT)          tile table: int4 (group, first sorted pair, end of the group's pairs,
//                             run: first row tile << 4 | rows - 1), TT = P/BM_MIN + G + 1
//   [sorted, + 4P)            pair ids p = m*S + i in group order
constexpr int BM_MIN = 128;
constexpr int ROUTE_CHUNK = 1024;  // pairs per routing workgroup
__host__ __device__ inline int64_t tiles_cap(int64_t P, int64_t G) { return P / BM_MIN + G + 1; }
__host__ __device__ inline int64_t off_counts() { return 64; }
__host__ __device__ inline int64_t off_cursor(int64_t G) { return 64 + 4 * G; }
__host__ __device__ inline int64_t off_tiles(int64_t G) { return (64 + 8 * G + 255) / 256 * 256; }
__host__ __device__ inline int64_t off_sorted(int64_t P, int64_t G) {
    return (off_tiles(G) + 16 * tiles_cap(P, G) + 255) / 256 * 256;
}

__device__ __forceinline__ int64_t load_idx(const void* idx, int64_t p, int idx64) {
    return idx64 ? ((const int64_t*)idx)[p] : (int64_t)((const int32_t*)idx)[p];
}

// (group, first sorted pair, rows) of a tile-table entry for bm-row tiles
__device__ __forceinline__ int4 tile_entry(const int4& e, int bm) { return make_int4(e.x, e.y, min(bm, e.z - e.y), 0); }

// Linear tile w of the run order: the row tile q = w / tiles_n lies in the
// run that holds w (a run of h row tiles starting at row tile c0 covers
// linear tiles c0 * tiles_n .. (c0 + h) * tiles_n - 1), whose tiles it walks
// column by column.  Returns (group, first sorted pair, rows) of row tile tm
// from q's entry alone (tiles of one run are consecutive bm-row slices of one
// group), and its column tile.
__device__ __forceinline__ int4 run_tile(const int4* tiles, int w, int tiles_n, int bm, int& tn) {
    const int q = w / tiles_n;
    const int4 e = tiles[q];
    const int c0 = e.w >> 4, h = (e.w & 15) + 1;
    const int r = w - c0 * tiles_n;
    const int tm = c0 + r % h;
    tn = r / h;
    const int start = e.y + (tm - q) * bm;
    return make_int4(e.x, start, min(bm, e.z - start), 0);
}

// exclusive scan of v[0..n) in LDS by one workgroup; returns the total
__device__ int block_exclusive_scan(int* v, int n, int* part) {
    const int t = threadIdx.x, nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    const int lo = min(n, t * per), hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += v[i];
    part[t] = s;
    __syncthreads();
    for (int d = 1; d < nt; d <<= 1) {
        const int x = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int run = part[t] - s;  // exclusive prefix of this thread's range
    for (int i = lo; i < hi; ++i) {
        const int c = v[i];
        v[i] = run;
        run += c;
    }
    const int total = part[nt - 1];
    __syncthreads();
    return total;
}

// 1. zero the counts and the header
__global__ void route_zero_kernel(char* ws, int G) {
    int* c = (int*)(ws + off_counts());
    for (int g = threadIdx.x; g < G; g += blockDim.x) c[g] = 0;
    if (threadIdx.x < 16) ((int*)ws)[threadIdx.x] = 0;
}

// 2. per-group pair counts: an LDS histogram per workgroup, one global add per used group
__global__ __launch_bounds__(256) void route_hist_kernel(const void* idx, int idx64, int64_t P, int G, char* ws) {
    __shared__ int h[MAX_G];
    __shared__ int bad;
    for (int g = threadIdx.x; g < G; g += 256) h[g] = 0;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * ROUTE_CHUNK, p1 = min(P, p0 + ROUTE_CHUNK);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
        const int64_t g = load_idx(idx, p, idx64);
        if (g >= 0 && g < G) atomicAdd(&h[g], 1);
        else atomicAdd(&bad, 1);
    }
    __syncthreads();
    int* c = (int*)(ws + off_counts());
    for (int g = threadIdx.x; g < G; g += 256)
        if (h[g]) atomicAdd(&c[g], h[g]);
    if (threadIdx.x == 0 && bad) atomicAdd(&((int*)ws)[1], bad);
}

// 3. scans: first sorted position and first tile of each group, the tile table, the cursors
__global__ __launch_bounds__(ROUTE_THREADS) void route_scan_kernel(int64_t P, int G, int BM, char* ws) {
    __shared__ int tile0[MAX_G];
    __shared__ int row0[MAX_G];
    __shared__ int part[ROUTE_THREADS];
    const int t = threadIdx.x;
    const int* cnt = (const int*)(ws + off_counts());
    for (int g = t; g < G; g += ROUTE_THREADS) {
        tile0[g] = (cnt[g] + BM - 1) / BM;
        row0[g] = cnt[g];
    }
    __syncthreads();
    const int ntiles = block_exclusive_scan(tile0, G, part);
    block_exclusive_scan(row0, G, part);
    int4* tiles = (int4*)(ws + off_tiles(G));
    int* cur = (int*)(ws + off_cursor(G));
    for (int g = t; g < G; g += ROUTE_THREADS) {
        const int c = cnt[g], nt = (c + BM - 1) / BM, end = row0[g] + c;
        const int nrun = nt <= RUN_MAX ? 1 : (nt + RUN_ROWS - 1) / RUN_ROWS;
        for (int ru = 0; ru < nrun; ++ru) {
            const int lo = (int)((int64_t)ru * nt / nrun), hi = (int)((int64_t)(ru + 1) * nt / nrun);
            const int run = ((tile0[g] + lo) << 4) | (hi - lo - 1);
            for (int tt = lo; tt < hi; ++tt) tiles[tile0[g] + tt] = make_int4(g, row0[g] + tt * BM, end, run);
        }
        cur[g] = row0[g];
    }
    if (t == 0) ((int*)ws)[0] = ntiles;
}

// 4. scatter pair ids into group order: each workgroup reserves its range per
//    group with one global add, then places its pairs with LDS cursors
__global__ __launch_bounds__(256) void route_scatter_kernel(const void* idx, int idx64, int64_t P, int G, char* ws) {
    __shared__ int h[MAX_G];
    for (int g = threadIdx.x; g < G; g += 256) h[g] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * ROUTE_CHUNK, p1 = min(P, p0 + ROUTE_CHUNK);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
        const int64_t g = load_idx(idx, p, idx64);
        if (g >= 0 && g < G) atomicAdd(&h[g], 1);
    }
    __syncthreads();
    int* cur = (int*)(ws + off_cursor(G));
    for (int g = threadIdx.x; g < G; g += 256)
        if (h[g]) h[g] = atomicAdd(&cur[g], h[g]);
    __syncthreads();
    int* sorted = (int*)(ws + off_sorted(P, G));
    for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
        const int64_t g = load_idx(idx, p, idx64);
        if (g >= 0 && g < G) sorted[atomicAdd(&h[g], 1)] = (int)p;
    }
}

// Epilogue of one grouped tile: + bias[g], one rounding to T, each row to
// output[pair].  VEC: output and bias 8-byte aligned and N % 8 == 0 (4-value
// stores; whole 256-column tiles of a 16-byte aligned output go through LDS as
// whole row segments, orow_s holding the tile's output rows, filled before
// the K loop's barriers).
template <int DT, bool VEC>
__device__ __forceinline__ void grouped_epilogue(const f32x16_t (&acc)[4][4], const GroupedArgs& a, int g, int rows,
                                                 int start, const int* sorted, int64_t n0, int lane, int wave,
                                                 char* s0, char* s1, const int* orow_s) {
    using namespace core16;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t N = a.N;
    if constexpr (VEC) {
        if (n0 + GBN <= N && N % 8 == 0 && ((uintptr_t)a.output & 15) == 0) {
            __syncthreads();  // every wave is done reading the last stage
            char* stage = (wave < 2 ? s0 : s1) + (wave & 1) * (GBM * KSTEP * 2);
            const int64_t col0 = n0 + wn * (GBN / 2);
            uint16_t* out = (uint16_t*)a.output + col0;
            const int* orow_w = orow_s + wm * (GBM / 2);
            auto rowp = [&](int r) -> uint16_t* {
                const int o = orow_w[r];
                return o >= 0 ? out + (int64_t)o * N : nullptr;
            };
            if (a.bias)
                wave_epilogue_lds<DT, true>(acc, 1.0f, (const uint16_t*)a.bias + (int64_t)g * N + col0, 1.0f, stage,
                                            lane, rowp);
            else
                wave_epilogue_lds<DT, false>(acc, 1.0f, nullptr, 1.0f, stage, lane, rowp);
            return;
        }
    }
    const uint16_t* __restrict__ bias = a.bias ? (const uint16_t*)a.bias + (int64_t)g * N : nullptr;
    uint16_t* __restrict__ out = (uint16_t*)a.output;
    const bool vec_store = VEC && (N % 4 == 0);
    const int64_t nl = n0 + wn * 128 + 4 * (lane >> 5);
    int orow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + 32 * i + (lane & 31);
        orow[i] = r < rows ? sorted[start + r] : -1;
    }
    // one 32-column block at a time, so only its 16 bias values are live
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float bv[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = nl + 32 * j + 8 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[q][e] = 0.0f;
            if (bias && vec_store && n < N) {
                const u32x2_t b2 = *(const u32x2_t*)(bias + n);
                bv[q][0] = from_bits<DT>((uint16_t)b2.x);
                bv[q][1] = from_bits<DT>((uint16_t)(b2.x >> 16));
                bv[q][2] = from_bits<DT>((uint16_t)b2.y);
                bv[q][3] = from_bits<DT>((uint16_t)(b2.y >> 16));
            } else if (bias) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) bv[q][e] = from_bits<DT>(bias[n + e]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (orow[i] < 0) continue;
            uint16_t* __restrict__ yr = out + (int64_t)orow[i] * N;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = nl + 32 * j + 8 * q;
                if (n >= N) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] + bv[q][e];
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

// One 256x256 tile of the grouped product with element-wise register-staged
// loads (any alignment and shape; the DMA form is grouped_body16).
template <int DT>
__device__ __forceinline__ void grouped_body(const GroupedArgs& a, const char* ws, int4 te, int tn, char* s0,
                                             char* s1, int* orow_s) {
    const int g = te.x, start = te.y, rows = te.z;
    const int* sorted = (const int*)(ws + off_sorted(a.M * a.S, a.G));
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = a.K, N = a.N, S = a.S;
    const int64_t n0 = (int64_t)tn * GBN;

    using namespace core16;
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int nk = (int)((K + KSTEP - 1) / KSTEP);
    const uint16_t* wg = (const uint16_t*)a.weights + (int64_t)g * K * N;
    orow_s[t] = t < rows ? sorted[start + t] : -1;  // output row (token * S + slot) of tile row t

    GatherSrc<GBM> srcA;
    srcA.base = (const uint16_t*)a.input;
    srcA.K = K;
    int r0, lk;
    Chunks<GBM, true>::coords(t, 0, r0, lk);
    srcA.lk = lk;
    srcA.valid = 0;
#pragma unroll
    for (int i = 0; i < GatherSrc<GBM>::NC; ++i) {
        const int r = r0 + 32 * i;
        int64_t off = 0;
        if (r < rows) {
            srcA.valid |= 1u << i;
            off = (int64_t)(sorted[start + r] / S) * K;
        }
        srcA.roff[i] = off + srcA.lk;
    }
    TileSrc<GBN, false> srcB;
    srcB.init(wg, N, n0, N, K, t);
    mainloop<GBM, GBN, DT, true, false, 2>(acc, s0, s1, srcA, srcB, nk, t, lane, wm, wn);
    grouped_epilogue<DT, false>(acc, a, g, rows, start, sorted, n0, lane, wave, s0, s1, orow_s);
}

// The same tile in the 16x16x32 MFMA form (DMA operands, K > 0): accumulator
// tile (i, j), register e of lane l holds row 16 i + l%16, column
// 16 j + 4 (l/16) + e of the wave's 128 x 128 block.  Whole 256-column tiles
// leave through LDS as whole row segments; a ragged column tile (N % 8 == 0
// here, so a lane's 4 columns are all in range or all out) stores 4 values
// per row.
template <int DT, int TM>
__device__ __forceinline__ void grouped_epilogue16(const f32x4_t (&acc)[TM][8], const GroupedArgs& a, int g, int rows,
                                                   int start, const int* sorted, int64_t n0, int lane, int wave,
                                                   char* s0, char* s1, const int* orow_s) {
    using namespace core16;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t N = a.N;
    if (n0 + GBN <= N && ((uintptr_t)a.output & 15) == 0) {
        __syncthreads();  // every wave is done reading the last stage
        char* stage = (wave < 2 ? s0 : s1) + (wave & 1) * (GBM * KSTEP * 2);
        const int64_t col0 = n0 + wn * (GBN / 2);
        uint16_t* out = (uint16_t*)a.output + col0;
        const int* orow_w = orow_s + wm * (16 * TM);
        auto st = [&](int, int r, int c, const u32x4_t& d) {
            const int o = orow_w[r];
            if (o >= 0) *(u32x4_t*)(out + (int64_t)o * N + 8 * c) = d;
        };
        if (a.bias)
            wave_epilogue_lds16<DT, true>(acc, 1.0f, (const uint16_t*)a.bias + (int64_t)g * N + col0, 1.0f, stage,
                                          lane, st);
        else
            wave_epilogue_lds16<DT, false>(acc, 1.0f, nullptr, 1.0f, stage, lane, st);
        return;
    }
    const uint16_t* __restrict__ bias = a.bias ? (const uint16_t*)a.bias + (int64_t)g * N : nullptr;
    uint16_t* __restrict__ out = (uint16_t*)a.output;
    const int64_t nl = n0 + wn * 128 + 4 * (lane >> 4);
    int orow[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * (16 * TM) + 16 * i + (lane & 15);
        orow[i] = r < rows ? sorted[start + r] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t n = nl + 16 * j;
        if (n >= N) continue;
        float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias) {
            const u32x2_t b2 = *(const u32x2_t*)(bias + n);
            bv[0] = from_bits<DT>((uint16_t)b2.x);
            bv[1] = from_bits<DT>((uint16_t)(b2.x >> 16));
            bv[2] = from_bits<DT>((uint16_t)b2.y);
            bv[3] = from_bits<DT>((uint16_t)(b2.y >> 16));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (orow[i] < 0) continue;
            u32x2_t o;
            o.x = pack2<DT>(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]);
            o.y = pack2<DT>(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]);
            *(u32x2_t*)(out + (int64_t)orow[i] * N + n) = o;
        }
    }
}

// BM = 256, or 128 for a group's last tile of at most 128 rows (4 row blocks
// of 16 per wave: about half the MFMAs and A traffic of a 256-row tile).
template <int DT, int BM>
__device__ __forceinline__ void grouped_body16(const GroupedArgs& a, const char* ws, int4 te, int tn, char* s0,
                                               char* s1, int* orow_s, uint32_t* roff_s, uint16_t* bias_s) {
    const int g = te.x, start = te.y, rows = te.z;
    const int* sorted = (const int*)(ws + off_sorted(a.M * a.S, a.G));
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = a.K, N = a.N, S = a.S;
    const int64_t n0 = (int64_t)tn * GBN;

    using namespace core16;
    static_assert(BM == 256 || BM == 128, "tile height");
    f32x4_t acc[BM / 32][8];  // written by the first k-block
    const int nk = (int)((K + KSTEP - 1) / KSTEP);
    const uint16_t* wg = (const uint16_t*)a.weights + (int64_t)g * K * N;
    const int srow = t < rows ? sorted[start + t] : -1;  // output row (token * S + slot) of tile row t
    if (t < BM) orow_s[t] = srow;
    // Whole-tile epilogue with 32-bit row offsets: the tile's bias columns and
    // its output row byte offsets are staged in LDS now, so the epilogue
    // neither waits on global loads nor branches per row.  Row r of wave
    // block wm (BM / 2 rows) goes to roff_s[(BM / 2) wm + (BM / 8) (r % 4) + r / 4]:
    // the BM / 8 rows a lane stores are contiguous.
    const bool fast = n0 + GBN <= N && ((uintptr_t)a.output & 15) == 0 && (int64_t)a.M * S * N * 2 < (1LL << 31);
    if (fast) {
        const int rr = t % (BM / 2);
        if (t < BM)
            roff_s[(t / (BM / 2)) * (BM / 2) + (BM / 8) * (rr & 3) + (rr >> 2)] =
                srow >= 0 ? (uint32_t)srow * (uint32_t)(N * 2) : DMA_OOB;
        if (a.bias && t < GBN / 4)
            *(u32x2_t*)(bias_s + 4 * t) = *(const u32x2_t*)((const uint16_t*)a.bias + (int64_t)g * N + n0 + 4 * t);
    }
    GatherDma<BM> srcA;
    srcA.base = (const char*)a.input;
    srcA.K = K;
    srcA.lane = lane;
#pragma unroll
    for (int j = 0; j < GatherDma<BM>::PER_WAVE; ++j) {
        const int r = GatherDma<BM>::row_of(wave, j, lane);
        srcA.roff[j] = r < rows ? (uint32_t)((int64_t)(sorted[start + r] / S) * K * 2) + (GatherDma<BM>::chunk(j, lane) << 4)
                                : DMA_OOB;
    }
    DmaSrc<GBN, false> srcB;
    srcB.init(wg, N, n0, N, K, lane);
    // (rows past the tile's end read zeros through their out-of-range offsets either way)
    if ((BM == GBM ? rows == GBM : true) && n0 + GBN <= N && K % KSTEP == 0)
        mainloop_dma16<BM, GBN, DT, true, false, false>(acc, s0, s1, srcA, srcB, nk, lane, wm, wn, wave);
    else
        mainloop_dma16<BM, GBN, DT, true, false, true>(acc, s0, s1, srcA, srcB, nk, lane, wm, wn, wave);

    if (fast) {
        __syncthreads();  // every wave is done reading the last stage
        char* stage = (wave < 2 ? s0 : s1) + (wave & 1) * (GBM * KSTEP * 2);  // 16 BM bytes x 128 rows fit
        const uint64_t ob = (uint64_t)((uint16_t*)a.output + n0 + wn * (GBN / 2));
        const uint64_t obu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ob) |
                             ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ob >> 32)) << 32);
        const __amdgpu_buffer_rsrc_t out =
            __builtin_amdgcn_make_buffer_rsrc((void*)obu, (short)0, 0x7fffffff, 0x00020000);
        uint32_t ro[BM / 8];
        const u32x4_t* rw = (const u32x4_t*)(roff_s + (BM / 2) * wm + (BM / 8) * (lane >> 4));
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const u32x4_t v = rw[i];
            ro[4 * i] = v.x;
            ro[4 * i + 1] = v.y;
            ro[4 * i + 2] = v.z;
            ro[4 * i + 3] = v.w;
        }
        auto st = [&](int k, int, int c, const u32x4_t& d) {
            __builtin_amdgcn_raw_buffer_store_b128(d, out, (int)(ro[k] + 16 * c), 0, 0);
        };
        if (a.bias)
            wave_epilogue_lds16<DT, true>(acc, 1.0f, bias_s + wn * (GBN / 2), 1.0f, stage, lane, st);
        else
            wave_epilogue_lds16<DT, false>(acc, 1.0f, nullptr, 1.0f, stage, lane, st);
        return;
    }
    grouped_epilogue16<DT, BM / 32>(acc, a, g, rows, start, sorted, n0, lane, wave, s0, s1, orow_s);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void grouped16_kernel(GroupedArgs a, const char* ws, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) char s0[(GBM + GBN) * core16::KSTEP * 2];
    __shared__ __attribute__((aligned(1024))) char s1[(GBM + GBN) * core16::KSTEP * 2];
    __shared__ int orow_s[GBM];
    __shared__ __attribute__((aligned(16))) uint32_t roff_s[GBM];
    __shared__ __attribute__((aligned(16))) uint16_t bias_s[GBN];
    // The grid is sized for the most row tiles any routing can produce; the
    // routed count is known only here.  Workgroup b runs on XCD b % 8, so the
    // routed tiles are split evenly over the 8 XCDs (each takes one contiguous
    // run of the tile order) and the surplus workgroups of every XCD exit.
    const int ntiles = ((const int*)ws)[0];
    const int total = ntiles * tiles_n;
    const int b = (int)blockIdx.x, x = b & 7, l = b >> 3;
    const int per = total >> 3, extra = total & 7;
    if (l >= per + (x < extra ? 1 : 0)) return;
    const int w = x * per + min(x, extra) + l;
    int tn;
    const int4 te = run_tile((const int4*)(ws + off_tiles(a.G)), w, tiles_n, GBM, tn);
    if constexpr (VEC) {
        if (te.z <= GBM / 2)
            grouped_body16<DT, GBM / 2>(a, ws, te, tn, s0, s1, orow_s, roff_s, bias_s);
        else
            grouped_body16<DT, GBM>(a, ws, te, tn, s0, s1, orow_s, roff_s, bias_s);
    } else
        grouped_body<DT>(a, ws, te, tn, s0, s1, orow_s);
}

// ---------------------------------------------------------------------------
// Weight-only quantised experts: the weights arrive as int8 / uint8 q (G, K, N)
// with scales (G, nkb, N) of T and optional zero points (G, nkb, N) of q's
// type, one per block of bs consecutive k and per column; the weight the
// product uses is w = T((q - zp) * scale) (DequantizeLinear, its output in the
// scale's type), formed in registers as each tile is staged: the dequantised
// (G, K, N) tensor never exists.

// Register-staged source of one dequantised 256-column weight tile, in the
// MN-major chunks of Chunks<GBN, false> (8 columns of one k row per chunk;
// chunk i of thread t is row t/32 + 8 i of the stage, columns (t%32)*8 ..).
//  FAST: N % 8 == 0, q rows 8-byte and scale rows 16-byte aligned, bs a
//        multiple of the 64-deep stage (a stage lies in one block): load()
//        issues 8-byte loads of the int8 bytes and one scale / zero-point
//        chunk per stage; convert() dequantises when the stage is stored, so
//        the loads have the whole stage of MFMAs to land.
//  else: element loads with element range checks, dequantised in load().
// (q - zp) * scale is exact in fp32 (|q - zp| <= 255, 8- or 11-bit scale
// significand), so the one rounding is the conversion to T.
template <int DT, bool QU8, bool FAST>
struct DeqSrc {
    static constexpr int NC = core16::Chunks<GBN, false>::NC;
    const uint8_t* q;    // this group's q, (K, N)
    const uint16_t* sc;  // this group's scales, (nkb, N)
    const uint8_t* zp;   // this group's zero points, or nullptr
    int64_t N, K, bs, n;
    int r0;
    u32x2_t raw[NC];
    u32x4_t sraw;
    u32x2_t zraw;
    u32x4_t out[NC];

    __device__ void init(const GroupedArgs& a, int g, int64_t n0, int t) {
        const int64_t nkb = a.nkb;
        q = (const uint8_t*)a.weights + (int64_t)g * a.K * a.N;
        sc = (const uint16_t*)a.wscale + (int64_t)g * nkb * a.N;
        zp = a.wzp ? (const uint8_t*)a.wzp + (int64_t)g * nkb * a.N : nullptr;
        N = a.N;
        K = a.K;
        bs = a.bs;
        int lmn, lk;
        core16::Chunks<GBN, false>::coords(t, 0, lmn, lk);
        n = n0 + lmn;
        r0 = lk;
    }

    __device__ static float elem(uint32_t qb, uint32_t zb, float s) {
        const int qi = QU8 ? (int)qb : (int)(int8_t)qb, zi = QU8 ? (int)zb : (int)(int8_t)zb;
        return (float)(qi - zi) * s;
    }

    __device__ __forceinline__ void load(int kt) {
        const int64_t k0 = (int64_t)kt * core16::KSTEP + r0;
        if constexpr (FAST) {
            const bool nok = n < N;
            const int64_t kb = (int64_t)kt * core16::KSTEP / bs;
            sraw = u32x4_t{0u, 0u, 0u, 0u};
            zraw = u32x2_t{0u, 0u};
            if (nok) {
                sraw = *(const u32x4_t*)(sc + kb * N + n);
                if (zp) zraw = *(const u32x2_t*)(zp + kb * N + n);
            }
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int64_t k = k0 + 8 * i;
                u32x2_t v = {0u, 0u};
                if (nok && k < K) v = *(const u32x2_t*)(q + k * N + n);
                raw[i] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int64_t k = k0 + 8 * i;
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = 0.0f;
                if (k < K) {
                    const int64_t kb = k / bs;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (n + e < N) {
                            const uint32_t qb = q[k * N + n + e];
                            const uint32_t zb = zp ? zp[kb * N + n + e] : 0u;
                            w[e] = elem(qb, zb, from_bits<DT>(sc[kb * N + n + e]));
                        }
                    }
                }
                out[i] = u32x4_t{pack2<DT>(w[0], w[1]), pack2<DT>(w[2], w[3]), pack2<DT>(w[4], w[5]),
                                 pack2<DT>(w[6], w[7])};
            }
        }
    }

    __device__ __forceinline__ void convert(u32x4_t (&reg)[NC], int kt) const {
        if constexpr (FAST) {
            // int8 bytes are shifted to q + 128 (one xor per 4 bytes) so that
            // every byte converts as unsigned; the shift moves into the offset:
            // w = (q + 128) * s - (zp + 128) * s, both products exact
            float sf[8], cf[8];
            const uint32_t sw[4] = {sraw.x, sraw.y, sraw.z, sraw.w}, zw[2] = {zraw.x, zraw.y};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sf[e] = from_bits<DT>((uint16_t)(sw[e >> 1] >> (16 * (e & 1))));
                const uint32_t zb = (zw[e >> 2] >> (8 * (e & 3))) & 0xffu;
                const int zs = QU8 ? (int)zb : (int)(int8_t)zb + 128;
                cf[e] = -(float)zs * sf[e];
            }
            const int64_t k0 = (int64_t)kt * core16::KSTEP + r0;
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                uint32_t u[2] = {raw[i].x, raw[i].y};
                if constexpr (!QU8) {
                    u[0] ^= 0x80808080u;
                    u[1] ^= 0x80808080u;
                }
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = __builtin_fmaf((float)((u[e >> 2] >> (8 * (e & 3))) & 0xffu), sf[e], cf[e]);
                u32x4_t v = {pack2<DT>(w[0], w[1]), pack2<DT>(w[2], w[3]), pack2<DT>(w[4], w[5]), pack2<DT>(w[6], w[7])};
                // rows past K (and columns past N, whose scales are 0) hold zeros
                if (!(k0 + 8 * i < K)) v = u32x4_t{0u, 0u, 0u, 0u};
                reg[i] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NC; ++i) reg[i] = out[i];
        }
    }
};

// Register-staged K loop with a dequantising B source: stage kt+1's loads are
// issued before stage kt's MFMAs and dequantised + stored after them.
template <int DT, int MODE, class SA, class SB>
__device__ __forceinline__ void mainloop_deq(f32x16_t (&acc)[4][4], char* smem0, char* smem1, const SA& srcA, SB& srcB,
                                             int nk, int t, int lane, int wm, int wn) {
    using namespace core16;
    constexpr int A_BYTES = GBM * KSTEP * 2;
    u32x4_t ra[Chunks<GBM, true>::NC], rb[Chunks<GBN, false>::NC];
    if (nk > 0) {
        srcA.template load<MODE>(ra, 0);
        srcB.load(0);
        srcB.convert(rb, 0);
        store_tile<GBM, true>(smem0, ra, t);
        store_tile<GBN, false>(smem0 + A_BYTES, rb, t);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            srcA.template load<MODE>(ra, kt + 1);
            srcB.load(kt + 1);
        }
        const char* sa = buf ? smem1 : smem0;
        const char* sb = sa + A_BYTES;
#pragma unroll
        for (int s = 0; s < KSTEP / 16; ++s) {
            u32x4_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = read_frag<GBM, true>(sa, wm * 128 + 32 * i, s, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = read_frag<GBN, false>(sb, wn * 128 + 32 * j, s, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16<DT>(bfr[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk) {
            char* so = buf ? smem0 : smem1;
            srcB.convert(rb, kt + 1);
            store_tile<GBM, true>(so, ra, t);
            store_tile<GBN, false>(so + A_BYTES, rb, t);
        }
        __syncthreads();
    }
}

// FAST variant: the gathered input rows go global -> LDS by DMA (as in
// grouped16_kernel), the dequantised weights through registers.  Stage kt+1's
// DMA and weight loads are issued before stage kt's MFMAs; its weights are
// dequantised and stored after them; one wait + barrier per stage.
template <int DT, class SB>
__device__ __forceinline__ void mainloop_deq_dma(f32x16_t (&acc)[4][4], char* s0, char* s1,
                                                 const core16::GatherDma<GBM>& srcA, SB& srcB, int nk, int t,
                                                 int lane, int wm, int wn, int wave) {
    using namespace core16;
    constexpr int A_BYTES = GBM * KSTEP * 2;
    u32x4_t rb[Chunks<GBN, false>::NC];
    if (nk > 0) {
        srcA.template issue<true>(s0, 0, wave);
        srcB.load(0);
        srcB.convert(rb, 0);
        store_tile<GBN, false>(s0 + A_BYTES, rb, t);
    }
    wait_vm<0>();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const char* sa = buf ? s1 : s0;
        char* so = buf ? s0 : s1;
        // so held stage kt-1, whose reads ended before the last barrier
        if (kt + 1 < nk) {
            srcA.template issue<true>(so, kt + 1, wave);
            srcB.load(kt + 1);
        }
        const char* sb = sa + A_BYTES;
#pragma unroll
        for (int s = 0; s < KSTEP / 16; ++s) {
            u32x4_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = read_frag<GBM, true>(sa, wm * 128 + 32 * i, s, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = read_frag<GBN, false>(sb, wn * 128 + 32 * j, s, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16<DT>(bfr[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk) {
            srcB.convert(rb, kt + 1);
            store_tile<GBN, false>(so + A_BYTES, rb, t);
        }
        wait_vm<0>();  // this wave's DMA of stage kt+1 has landed
        __syncthreads();
    }
}

// ---- DMA variant: the int8 weight tile itself goes global -> LDS by DMA (64
// k rows x 256 bytes per stage, the 8-bit MN-major layout) and each lane
// dequantises its MFMA operand after the transposing read: ds_read_b64_tr_b8
// gives lane l the 8 k-values k = 16 s + 8 (l/32) + 0..7 of column
// colb + l%32, exactly the bf16 operand layout, so one scale and one zero
// point (of that column and the stage's block) serve all 8.  LDS holds half
// the weight bytes of the bf16 kernel and the weights never pass through
// registers on their way in.

template <int DT, bool QU8>
__device__ __forceinline__ u32x4_t dq8(u32x2_t raw, float sf, float cf) {
    uint32_t u[2] = {raw.x, raw.y};
    if constexpr (!QU8) {
        u[0] ^= 0x80808080u;  // q + 128 in every byte
        u[1] ^= 0x80808080u;
    }
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = __builtin_fmaf((float)((u[e >> 2] >> (8 * (e & 3))) & 0xffu), sf, cf);
    return u32x4_t{pack2<DT>(w[0], w[1]), pack2<DT>(w[2], w[3]), pack2<DT>(w[4], w[5]), pack2<DT>(w[6], w[7])};
}

__device__ __forceinline__ u32x2_t read_frag_q8(const char* lds, int colb, int s, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int krow = 16 * s + 8 * (g >> 1) + (i >> 1);
    const int ncol = colb + 16 * (g & 1) + 8 * (i & 1);
    const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(OMM_LDS(i32x2_t, lds + mmaj8_off<GBN>(krow, ncol)));
    return __builtin_bit_cast(u32x2_t, v);
}

// Wave layout of the dequantising kernel: TM row blocks x TN column blocks of
// 32 per wave, rows row0 + 32 i, columns col0 + 32 j (1x4: each wave all 256
// rows and its own 64 columns, so every weight fragment is dequantised by one
// wave only).
template <int TM, int TN>
struct FragsDQ {
    u32x4_t a[TM], b[TN];
    u32x2_t braw[TN];
};

// reads of a k-block in order of first use (frag_order), read r after MFMA
// slot dq_read_slot(r); weight fragment j converted 4 MFMAs after its read
constexpr int dq_read_slot(int TM, int TN, int r) {
    const int NM = TM * TN, NR = TM + TN;
    for (int x = 0; x < NM; ++x)
        if (r < ((x + 1) * NR + NM - 1) / NM) return x;
    return NM - 1;
}
constexpr int dq_conv_slot(int TM, int TN, int j) {
    for (int r = 0; r < TM + TN; ++r)
        if (core16::frag_order(TM, TN, r) == TM + j) return dq_read_slot(TM, TN, r) + 4;
    return -1;
}

// per-stage dequantisation constants of this lane's TN columns: w = fma(q', sf, cf)
template <int TN>
struct DqScales {
    float sf[TN], cf[TN];
};

template <int DT, bool QU8, int TM, int TN, int X>
__device__ __forceinline__ void dq_slot_reads(FragsDQ<TM, TN>& nxt, const char* lds, int s, int lane, int row0,
                                              int col0, const DqScales<TN>& sc) {
    using namespace core16;
    constexpr int A_BYTES = GBM * KSTEP * 2;
    static_for<0, TM + TN>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (dq_read_slot(TM, TN, r) == X) {
            constexpr int f = frag_order(TM, TN, r);
            if constexpr (f < TM)
                nxt.a[f] = read_frag<GBM, true>(lds, row0 + 32 * f, s, lane);
            else
                nxt.braw[f - TM] = read_frag_q8(lds + A_BYTES, col0 + 32 * (f - TM), s, lane);
        }
    });
    static_for<0, TN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (dq_conv_slot(TM, TN, j) == X) nxt.b[j] = dq8<DT, QU8>(nxt.braw[j], sc.sf[j], sc.cf[j]);
    });
}

// One k-block of MFMAs on `cur`, the reads (and conversions) of k-block s of
// `lds` into `nxt`, and this wave's DMA instructions D0 .. D1-1 of stage kt
// into buffer Xb spread between the MFMAs (none when D0 == D1).
template <int DT, bool QU8, int TM, int TN, int D0, int D1, class SA, class SB>
__device__ __forceinline__ void kblock_dq(f32x16_t (&acc)[TM][TN], const FragsDQ<TM, TN>& cur,
                                          FragsDQ<TM, TN>& nxt, const char* lds, int s, char* Xb, const SA& srcA,
                                          const SB& srcB, int kt, bool live, int lane, int row0, int col0, int wave,
                                          const DqScales<TN>& sc) {
    using namespace core16;
    constexpr int A_BYTES = GBM * KSTEP * 2;
    constexpr int NM = TM * TN, ND = D1 - D0, LA = SA::PER_WAVE;
    static_assert(dq_conv_slot(TM, TN, TN - 1) < NM, "every conversion inside the k-block");
    DmaCtx ca{}, cb{};
    if constexpr (ND > 0) {
        ca = srcA.ctx(Xb, kt, live);
        cb = srcB.ctx(Xb + A_BYTES, kt, live);
    }
    static_for<0, NM>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        acc[x / TN][x % TN] = mfma32x32x16<DT>(cur.b[x % TN], cur.a[x / TN], acc[x / TN][x % TN]);
        if constexpr (ND > 0)
            static_for<D0 + (x * ND + NM - 1) / NM, D0 + ((x + 1) * ND + NM - 1) / NM>(
                [&](auto dc) { dma_one<true, LA, decltype(dc)::value>(srcA, srcB, ca, cb, kt, wave); });
        dq_slot_reads<DT, QU8, TM, TN, x>(nxt, lds, s, lane, row0, col0, sc);
        fence_sched();
    });
}

// One stage's scales and zero points (the block of the stage's k, the tile's
// 256 columns) go to the stage's LDS buffer by DMA next to the tiles: wave 0
// loads the 512 bytes of scales, wave 1 the 256 bytes of zero points (no zero
// points, or columns past N: zeros).  After the stage's barrier each lane
// reads the 4 values of its columns from LDS.
constexpr int DQ_SC_OFF = GBM * core16::KSTEP * 2 + GBN * core16::KSTEP;  // after the A and int8 B tiles
struct DqParams {
    const char* sc;  // this group's scales (N per block, 2 bytes each)
    const char* zp;  // this group's zero points, or nullptr
    int64_t N, bs, n0;
    __device__ __forceinline__ void issue(char* buf, int kt, bool live, int wave, int lane) const {
        using namespace core16;
        const int w = __builtin_amdgcn_readfirstlane(wave);  // uniform: the buffer resource lives in SGPRs
        if (w >= 2) return;
        const bool isz = w == 1;
        const char* base = isz ? zp : sc;
        const int es = isz ? 1 : 2;
        const bool lv = __builtin_amdgcn_readfirstlane((int)(live && base != nullptr)) != 0;
        const int64_t kb = lv ? (int64_t)kt * KSTEP / bs : 0;
        const i32x4_t r = make_rsrc(lv ? base + (kb * N + n0) * es : sc, lv);
        const int nl = isz ? 16 : 32;  // lanes with data: 16 bytes = 8 scales or 16 zero points each
        const uint32_t voff = (lane < nl && n0 + (int64_t)lane * (16 / es) < N) ? (uint32_t)lane * 16u : DMA_OOB;
        dma16u(r, lds_addr(buf + DQ_SC_OFF + (isz ? 1024 : 0)), voff);
    }
    // this lane's columns: col0 + 32 j + lane % 32
    template <int DT, bool QU8, int TN>
    __device__ __forceinline__ void to_scales(const char* buf, int col0, int lane, DqScales<TN>& o) const {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int c = col0 + 32 * j + (lane & 31);
            o.sf[j] = from_bits<DT>(*(const uint16_t*)(buf + DQ_SC_OFF + 2 * c));
            const uint32_t zb = *(const uint8_t*)(buf + DQ_SC_OFF + 1024 + c);
            const int zs = QU8 ? (int)zb : (int)(int8_t)zb + 128;
            o.cf[j] = -(float)zs * o.sf[j];
        }
    }
};

template <int DT, bool QU8, int TM, int TN, class SA, class SB>
__device__ __forceinline__ void dq_stage(f32x16_t (&acc)[TM][TN], FragsDQ<TM, TN>& fc, FragsDQ<TM, TN>& fn, char* X,
                                         char* Y, const SA& srcA, const SB& srcB, DqParams& prm, DqScales<TN>& sc,
                                         int kt, int nk, int lane, int row0, int col0, int wave) {
    using namespace core16;
    constexpr int LD = SA::PER_WAVE + SB::PER_WAVE, H = LD / 2;
    fence_sched();
    prm.issue(Y, kt + 1, kt + 1 < nk, wave, lane);
    kblock_dq<DT, QU8, TM, TN, H, LD>(acc, fc, fn, X, 1, Y, srcA, srcB, kt + 1, kt + 1 < nk, lane, row0, col0, wave,
                                      sc);
    kblock_dq<DT, QU8, TM, TN, 0, 0>(acc, fn, fc, X, 2, Y, srcA, srcB, kt, false, lane, row0, col0, wave, sc);
    kblock_dq<DT, QU8, TM, TN, 0, 0>(acc, fc, fn, X, 3, Y, srcA, srcB, kt, false, lane, row0, col0, wave, sc);
    wait_vm<0>();     // stage kt+1 (tiles and scales) has landed
    __syncthreads();  // ... for every wave; every read of X is done
    prm.template to_scales<DT, QU8, TN>(Y, col0, lane, sc);
    fence_sched();
    kblock_dq<DT, QU8, TM, TN, 0, H>(acc, fn, fc, Y, 0, X, srcA, srcB, kt + 2, kt + 2 < nk, lane, row0, col0, wave,
                                     sc);
}

template <int DT, bool QU8, int TM, int TN, class SA, class SB>
__device__ __forceinline__ void mainloop_dq_dma(f32x16_t (&acc)[TM][TN], char* __restrict__ s0, char* __restrict__ s1,
                                                const SA& srcA, const SB& srcB, DqParams& prm, int nk, int lane,
                                                int row0, int col0, int wave) {
    using namespace core16;
    constexpr int A_BYTES = GBM * KSTEP * 2;
    constexpr int LA = SA::PER_WAVE, LD = SA::PER_WAVE + SB::PER_WAVE, H = LD / 2;
    if (nk <= 0) return;
    prm.issue(s0, 0, true, wave, lane);
    {
        const DmaCtx a0 = srcA.ctx(s0, 0, true), b0 = srcB.ctx(s0 + A_BYTES, 0, true);
        static_for<0, LD>([&](auto dc) { dma_one<true, LA, decltype(dc)::value>(srcA, srcB, a0, b0, 0, wave); });
        const DmaCtx a1 = srcA.ctx(s1, 1, nk > 1), b1 = srcB.ctx(s1 + A_BYTES, 1, nk > 1);
        static_for<0, H>([&](auto dc) { dma_one<true, LA, decltype(dc)::value>(srcA, srcB, a1, b1, 1, wave); });
    }
    wait_vm<H>();
    __syncthreads();
    DqScales<TN> sc;
    prm.template to_scales<DT, QU8, TN>(s0, col0, lane, sc);
    fence_sched();
    FragsDQ<TM, TN> fc, fn;
#pragma unroll
    for (int i = 0; i < TM; ++i) fc.a[i] = read_frag<GBM, true>(s0, row0 + 32 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j)
        fc.b[j] = dq8<DT, QU8>(read_frag_q8(s0 + A_BYTES, col0 + 32 * j, 0, lane), sc.sf[j], sc.cf[j]);
    for (int kt = 0; kt < nk; kt += 2) {
        dq_stage<DT, QU8, TM, TN>(acc, fc, fn, s0, s1, srcA, srcB, prm, sc, kt, nk, lane, row0, col0, wave);
        dq_stage<DT, QU8, TM, TN>(acc, fc, fn, s1, s0, srcA, srcB, prm, sc, kt + 1, nk, lane, row0, col0, wave);
    }
    wait_vm<0>();
}

// Epilogue of a TM x TN block of 32x32 results (rows row0 + 32 i, columns
// col0 + 32 j of the tile): + bias[g], one rounding to T, 4-value stores to
// each row's output[pair] (output and bias 8-byte aligned, N % 8 == 0).
template <int DT, int TM, int TN>
__device__ __forceinline__ void grouped_epilogue_blocks(const f32x16_t (&acc)[TM][TN], const GroupedArgs& a, int g,
                                                        int64_t n0, int row0, int col0, int lane, const int* orow_s) {
    const int64_t N = a.N;
    const uint16_t* __restrict__ bias = a.bias ? (const uint16_t*)a.bias + (int64_t)g * N : nullptr;
    uint16_t* __restrict__ out = (uint16_t*)a.output;
    const int64_t nl = n0 + col0 + 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        float bv[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = nl + 32 * j + 8 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[q][e] = 0.0f;
            if (bias && n < N) {
                const u32x2_t b2 = *(const u32x2_t*)(bias + n);
                bv[q][0] = from_bits<DT>((uint16_t)b2.x);
                bv[q][1] = from_bits<DT>((uint16_t)(b2.x >> 16));
                bv[q][2] = from_bits<DT>((uint16_t)b2.y);
                bv[q][3] = from_bits<DT>((uint16_t)(b2.y >> 16));
            }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int o = orow_s[row0 + 32 * i + (lane & 31)];
            if (o < 0) continue;
            uint16_t* __restrict__ yr = out + (int64_t)o * N;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = nl + 32 * j + 8 * q;
                if (n >= N) continue;
                u32x2_t st;
                st.x = pack2<DT>(acc[i][j][4 * q + 0] + bv[q][0], acc[i][j][4 * q + 1] + bv[q][1]);
                st.y = pack2<DT>(acc[i][j][4 * q + 2] + bv[q][2], acc[i][j][4 * q + 3] + bv[q][3]);
                *(u32x2_t*)(yr + n) = st;
            }
        }
    }
}

// Epilogue of the 1x4 wave layout (each wave: all 256 rows, 64 columns) for a
// tile wholly inside the output with 32-bit row offsets: the bias columns
// (bias_s, the tile's 256) and the output row byte offsets (roff_s, row r at
// 32 (r % 8) + r / 8, so the 32 rows a lane stores are contiguous; rows past
// the tile's valid rows hold an offset beyond the buffer's range and their
// stores are dropped) were staged in LDS at tile start.  Each wave converts
// its block into its 32 KiB of `stage` (row r: 128 bytes, 16-byte chunk c in
// slot c ^ (r % 8)) and stores whole 128-byte row segments, 8 rows per
// instruction.
template <int DT>
__device__ __forceinline__ void dq_epilogue_lds(const f32x16_t (&acc)[8][2], const GroupedArgs& a, int64_t n0,
                                                int col0, int lane, int wave, char* stage, const uint32_t* roff_s,
                                                const uint16_t* bias_s) {
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (a.bias) {
                const u32x2_t b2 = *(const u32x2_t*)(bias_s + col0 + 32 * j + 8 * q + 4 * h);
                bv[0] = from_bits<DT>((uint16_t)b2.x);
                bv[1] = from_bits<DT>((uint16_t)(b2.x >> 16));
                bv[2] = from_bits<DT>((uint16_t)b2.y);
                bv[3] = from_bits<DT>((uint16_t)(b2.y >> 16));
            }
            const int c = 4 * j + q;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 32 * i + (lane & 31);
                u32x2_t o;
                o.x = pack2<DT>(acc[i][j][4 * q + 0] + bv[0], acc[i][j][4 * q + 1] + bv[1]);
                o.y = pack2<DT>(acc[i][j][4 * q + 2] + bv[2], acc[i][j][4 * q + 3] + bv[3]);
                *(u32x2_t*)(stage + r * 128 + ((c ^ (r & 7)) << 4) + 8 * h) = o;
            }
        }
    }
    uint32_t ro[32];
    const u32x4_t* rw = (const u32x4_t*)(roff_s + 32 * (lane >> 3));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4_t v = rw[i];
        ro[4 * i] = v.x;
        ro[4 * i + 1] = v.y;
        ro[4 * i + 2] = v.z;
        ro[4 * i + 3] = v.w;
    }
    // the base made visibly wave-uniform, so that the resource sits in scalar registers
    const uint64_t ob = (uint64_t)((uint16_t*)a.output + n0 + 64 * wave);
    const uint64_t obu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ob) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ob >> 32)) << 32);
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc((void*)obu, (short)0, 0x7fffffff, 0x00020000);
    const int c = lane & 7;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const int r = 8 * k + (lane >> 3);
        const u32x4_t d = *(const u32x4_t*)(stage + r * 128 + ((c ^ (r & 7)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(d, out, (int)(ro[k] + 16 * c), 0, 0);
    }
}

// Weights by DMA: K % 64 == 0, N % 16 == 0, 16-byte aligned q, scale and
// zero-point rows (16-byte aligned bases), block size a multiple of 64 (one
// block per stage).
template <int DT, bool QU8>
__global__ __launch_bounds__(256) void grouped16_dq_dma_kernel(GroupedArgs a, const char* ws, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) char s0[(GBM + GBN) * core16::KSTEP * 2];
    __shared__ __attribute__((aligned(1024))) char s1[(GBM + GBN) * core16::KSTEP * 2];
    __shared__ int orow_s[GBM];
    __shared__ __attribute__((aligned(16))) uint32_t roff_s[GBM];
    __shared__ __attribute__((aligned(16))) uint16_t bias_s[GBN];
    using namespace core16;
    const int ntiles = ((const int*)ws)[0];
    const int total = ntiles * tiles_n;
    const int b = (int)blockIdx.x, x = b & 7, l = b >> 3;
    const int per = total >> 3, extra = total & 7;
    if (l >= per + (x < extra ? 1 : 0)) return;
    int tn;

    const int4 te = run_tile((const int4*)(ws + off_tiles(a.G)), x * per + min(x, extra) + l, tiles_n, GBM, tn);
    const int g = te.x, start = te.y, rows = te.z;
    const int* sorted = (const int*)(ws + off_sorted(a.M * a.S, a.G));
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t K = a.K, N = a.N, S = a.S;
    const int64_t n0 = (int64_t)tn * GBN;
    // 1x4 wave layout: all 256 rows, 64 columns per wave
    constexpr int TM = 8, TN = 2;
    const int row0 = 0, col0 = 64 * wave;
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int nk = (int)(K / KSTEP);
    const int srow = t < rows ? sorted[start + t] : -1;  // output row of tile row t
    orow_s[t] = srow;
    const bool fast = n0 + GBN <= N && N % 8 == 0 && ((uintptr_t)a.output & 15) == 0 &&
                      (!a.bias || ((uintptr_t)a.bias & 7) == 0) && (int64_t)a.M * S * N * 2 < (1LL << 31);
    if (fast) {
        roff_s[32 * (t & 7) + (t >> 3)] = srow >= 0 ? (uint32_t)srow * (uint32_t)(N * 2) : DMA_OOB;
        if (a.bias && t < GBN / 4)
            *(u32x2_t*)(bias_s + 4 * t) = *(const u32x2_t*)((const uint16_t*)a.bias + (int64_t)g * N + n0 + 4 * t);
    }

    GatherDma<GBM> srcA;
    srcA.base = (const char*)a.input;
    srcA.K = K;
    srcA.lane = lane;
#pragma unroll
    for (int j = 0; j < GatherDma<GBM>::PER_WAVE; ++j) {
        const int r = GatherDma<GBM>::row_of(wave, j, lane);
        srcA.roff[j] = r < rows ? (uint32_t)((int64_t)(sorted[start + r] / S) * K * 2) +
                                      (GatherDma<GBM>::chunk(j, lane) << 4)
                                : DMA_OOB;
    }
    DmaSrcMN8<GBN, KSTEP> srcB;
    srcB.init((const uint8_t*)a.weights + (int64_t)g * K * N, N, n0, N, K, lane);
    DqParams prm;
    prm.sc = (const char*)a.wscale + (int64_t)g * a.nkb * N * 2;
    prm.zp = a.wzp ? (const char*)a.wzp + (int64_t)g * a.nkb * N : nullptr;
    prm.N = N;
    prm.bs = a.bs;
    prm.n0 = n0;
    mainloop_dq_dma<DT, QU8, TM, TN>(acc, s0, s1, srcA, srcB, prm, nk, lane, row0, col0, wave);
    __syncthreads();  // the LDS tables complete even when the K loop ran no stage (K = 0); stages free
    if (fast)
        dq_epilogue_lds<DT>(acc, a, n0, col0, lane, wave, (wave < 2 ? s0 : s1) + (wave & 1) * (GBM * 128), roff_s,
                            bias_s);
    else
        grouped_epilogue_blocks<DT, TM, TN>(acc, a, g, n0, row0, col0, lane, orow_s);
}

template <int DT, bool QU8, bool FAST>
__global__ __launch_bounds__(256) void grouped16_dq_kernel(GroupedArgs a, const char* ws, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) char s0[(GBM + GBN) * core16::KSTEP * 2];
    __shared__ __attribute__((aligned(1024))) char s1[(GBM + GBN) * core16::KSTEP * 2];
    __shared__ int orow_s[GBM];
    using namespace core16;
    // routed tiles split evenly over the 8 XCDs, as in grouped16_kernel
    const int ntiles = ((const int*)ws)[0];
    const int total = ntiles * tiles_n;
    const int b = (int)blockIdx.x, x = b & 7, l = b >> 3;
    const int per = total >> 3, extra = total & 7;
    if (l >= per + (x < extra ? 1 : 0)) return;
    int tn;

    const int4 te = run_tile((const int4*)(ws + off_tiles(a.G)), x * per + min(x, extra) + l, tiles_n, GBM, tn);
    const int g = te.x, start = te.y, rows = te.z;
    const int* sorted = (const int*)(ws + off_sorted(a.M * a.S, a.G));
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = a.K, S = a.S;
    const int64_t n0 = (int64_t)tn * GBN;
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int nk = (int)((K + KSTEP - 1) / KSTEP);
    if (t < GBM) orow_s[t] = t < rows ? sorted[start + t] : -1;

    DeqSrc<DT, QU8, FAST> srcB;
    srcB.init(a, g, n0, t);
    if constexpr (FAST) {
        GatherDma<GBM> srcA;
        srcA.base = (const char*)a.input;
        srcA.K = K;
        srcA.lane = lane;
#pragma unroll
        for (int j = 0; j < GatherDma<GBM>::PER_WAVE; ++j) {
            const int r = GatherDma<GBM>::row_of(wave, j, lane);
            srcA.roff[j] = r < rows ? (uint32_t)((int64_t)(sorted[start + r] / S) * K * 2) +
                                          (GatherDma<GBM>::chunk(j, lane) << 4)
                                    : DMA_OOB;
        }
        mainloop_deq_dma<DT>(acc, s0, s1, srcA, srcB, nk, t, lane, wm, wn, wave);
    } else {
        GatherSrc<GBM> srcA;
        srcA.base = (const uint16_t*)a.input;
        srcA.K = K;
        int r0, lk;
        Chunks<GBM, true>::coords(t, 0, r0, lk);
        srcA.lk = lk;
        srcA.valid = 0;
#pragma unroll
        for (int i = 0; i < GatherSrc<GBM>::NC; ++i) {
            const int r = r0 + 32 * i;
            int64_t off = 0;
            if (r < rows) {
                srcA.valid |= 1u << i;
                off = (int64_t)(sorted[start + r] / S) * K;
            }
            srcA.roff[i] = off + srcA.lk;
        }
        mainloop_deq<DT, 2>(acc, s0, s1, srcA, srcB, nk, t, lane, wm, wn);
    }
    grouped_epilogue<DT, FAST>(acc, a, g, rows, start, sorted, n0, lane, wave, s0, s1, orow_s);
}

// ---------------------------------------------------------------------------
// fp32 / fp64 grouped product on the matrix cores: v_mfma_f32_16x16x4f32 and
// v_mfma_f64_16x16x4f64 (fp32 accumulation for fp32, fp64 for fp64), over the
// same routing with 128-row tiles.  One 128x128 output tile per workgroup of 4
// waves (each 64x64: 4x4 MFMA tiles of 16x16); its 128 rows are the tile's
// sorted pairs, gathered from input[pair / S]; B is weights[g] (n
// contiguous).  K is staged 16 values at a time through three LDS buffers:
// stage k+2 is loaded into registers while stage k multiplies and written to
// LDS at the end of stage k (into the buffer stage k-1 left), so stage k+1 is
// in LDS a whole stage before it starts and its first fragments are read
// ahead of the barrier.  Element loads with range checks (any K, N, alignment).
// WQ = 0: weights of type F.  WQ = 1 / 2 (fp32 only): int8 / uint8 weights
// dequantised on load, w = fp32((q - zp) * scale) with the scale and zero
// point of block k / bs and column n (one rounding, as DequantizeLinear to fp32).
constexpr int FT = 128;  // output tile edge
constexpr int FKS = 16;  // k per stage
constexpr int FNB = 3;   // LDS stage buffers
constexpr int FNL = FT * FKS / 256;  // elements per thread per operand and stage
// LDS tiles (elements): A as 128 rows of 16 k at a stride of 18 (the 16 lanes
// reading one k of 16 consecutive rows hit distinct banks), B as 16 k rows of
// 128 n at a stride of 130
constexpr int FA_ELEMS = FT * 18, FB_ELEMS = FKS * 130;

template <class F>
struct FpMfma;
template <>
struct FpMfma<double> {
    typedef double v4 __attribute__((ext_vector_type(4)));
    __device__ static v4 mma(double a, double b, v4 c) { return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0); }
    // result register r of lane l: row l/16 + 4 r, column l%16
    __device__ static int row(int lane, int r) { return (lane >> 4) + 4 * r; }
};
template <>
struct FpMfma<float> {
    typedef float v4 __attribute__((ext_vector_type(4)));
    __device__ static v4 mma(float a, float b, v4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
    // result register r of lane l: row 4 (l/16) + r, column l%16
    __device__ static int row(int lane, int r) { return 4 * (lane >> 4) + r; }
};

template <class F, int WQ>
__global__ __launch_bounds__(256) void grouped_fp_kernel(GroupedArgs a, const char* ws, int tiles_n) {
    typedef typename FpMfma<F>::v4 v4;
    __shared__ F As[FNB * FA_ELEMS];
    __shared__ F Bs[FNB * FB_ELEMS];
    __shared__ int orow_s[FT];
    // routed tiles split evenly over the 8 XCDs, surplus workgroups exit (as grouped16_kernel)
    const int ntiles = ((const int*)ws)[0];
    const int total = ntiles * tiles_n;
    const int bid = (int)blockIdx.x, x = bid & 7, l = bid >> 3;
    const int per = total >> 3, extra = total & 7;
    if (l >= per + (x < extra ? 1 : 0)) return;
    int tn;

    const int4 te = run_tile((const int4*)(ws + off_tiles(a.G)), x * per + min(x, extra) + l, tiles_n, FT, tn);
    const int g = te.x, start = te.y, rows = te.z;
    const int* sorted = (const int*)(ws + off_sorted(a.M * a.S, a.G));
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = a.K, N = a.N, S = a.S;
    const int64_t n0 = (int64_t)tn * FT;
    if (t < FT) orow_s[t] = t < rows ? sorted[start + t] : -1;

    // A: thread t loads k = t % 16 of tile rows t / 16 + 16 i (gathered token rows)
    const F* __restrict__ in = (const F*)a.input;
    const int ka = t & 15;
    int64_t aoff[FNL];
    uint32_t avalid = 0;
#pragma unroll
    for (int i = 0; i < FNL; ++i) {
        const int r = (t >> 4) + 16 * i;
        aoff[i] = 0;
        if (r < rows) {
            avalid |= 1u << i;
            aoff[i] = (int64_t)(sorted[start + r] / S) * K + ka;
        }
    }
    // B: thread t loads column n0 + t % 128 of k rows t / 128 + 2 i
    const int nb = t & 127, kb = t >> 7;
    const int64_t ncol = n0 + nb;
    const bool nok = ncol < N;
    const int64_t wbase = (int64_t)g * K * N + ncol;
    const float* wsc = WQ ? (const float*)a.wscale + (int64_t)g * a.nkb * N + ncol : nullptr;
    const uint8_t* wzp = (WQ && a.wzp) ? (const uint8_t*)a.wzp + (int64_t)g * a.nkb * N + ncol : nullptr;

    auto load = [&](F (&ra)[FNL], F (&rb)[FNL], int kt) {
        const int64_t k0 = (int64_t)kt * FKS;
#pragma unroll
        for (int i = 0; i < FNL; ++i) ra[i] = (((avalid >> i) & 1u) && k0 + ka < K) ? in[aoff[i] + k0] : (F)0;
#pragma unroll
        for (int i = 0; i < FNL; ++i) {
            const int64_t k = k0 + kb + 2 * i;
            F v = (F)0;
            if (nok && k < K) {
                if constexpr (WQ == 0) {
                    v = ((const F*)a.weights)[wbase + k * N];
                } else {
                    const uint8_t qb = ((const uint8_t*)a.weights)[wbase + k * N];
                    const int64_t po = (k / a.bs) * N;
                    const uint8_t zb = wzp ? wzp[po] : (uint8_t)0;
                    const int qi = WQ == 2 ? (int)qb : (int)(int8_t)qb, zi = WQ == 2 ? (int)zb : (int)(int8_t)zb;
                    v = (F)((float)(qi - zi) * wsc[po]);
                }
            }
            rb[i] = v;
        }
    };
    auto store = [&](int buf, const F (&ra)[FNL], const F (&rb)[FNL]) {
        F* A_ = As + buf * FA_ELEMS;
        F* B_ = Bs + buf * FB_ELEMS;
#pragma unroll
        for (int i = 0; i < FNL; ++i) A_[((t >> 4) + 16 * i) * 18 + ka] = ra[i];
#pragma unroll
        for (int i = 0; i < FNL; ++i) B_[(kb + 2 * i) * 130 + nb] = rb[i];
    };
    // lane l supplies A[m = l%16][k = kk + l/16] and B[k = kk + l/16][n = l%16]
    struct Fr {
        F a[4], b[4];
    };
    auto read = [&](Fr& f, int buf, int kk) {
        const F* A_ = As + buf * FA_ELEMS;
        const F* B_ = Bs + buf * FB_ELEMS;
#pragma unroll
        for (int i = 0; i < 4; ++i) f.a[i] = A_[(wm * 64 + 16 * i + (lane & 15)) * 18 + kk + (lane >> 4)];
#pragma unroll
        for (int j = 0; j < 4; ++j) f.b[j] = B_[(kk + (lane >> 4)) * 130 + wn * 64 + 16 * j + (lane & 15)];
    };
    v4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4{0, 0, 0, 0};
    auto mma = [&](const Fr& f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = FpMfma<F>::mma(f.a[i], f.b[j], acc[i][j]);
    };

    const int nk = (int)((K + FKS - 1) / FKS);
    F ra[FNL], rb[FNL];
    for (int s2 = 0; s2 < 2 && s2 < nk; ++s2) {
        load(ra, rb, s2);
        store(s2, ra, rb);
    }
    __syncthreads();
    Fr fc, fn;
    if (nk > 0) read(fc, 0, 0);
    int b0 = 0;  // buffer of stage kt
    for (int kt = 0; kt < nk; ++kt) {
        const int b1 = b0 == FNB - 1 ? 0 : b0 + 1, b2 = b1 == FNB - 1 ? 0 : b1 + 1;
        const bool more = kt + 2 < nk;
        if (more) load(ra, rb, kt + 2);
        read(fn, b0, 4);
        mma(fc);
        read(fc, b0, 8);
        mma(fn);
        read(fn, b0, 12);
        mma(fc);
        // stage kt+1 has been in LDS since the last barrier (unused junk past the last stage)
        read(fc, b1, 0);
        mma(fn);
        if (more) store(b2, ra, rb);  // the buffer stage kt-1 used, retired at the last barrier
        __syncthreads();
        b0 = b1;
    }

    // + bias[g], each row to output[pair]
    const F* bias = a.bias ? (const F*)a.bias + (int64_t)g * N : nullptr;
    F* __restrict__ out = (F*)a.output;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
        if (n >= N) continue;
        const F bv = bias ? bias[n] : (F)0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = wm * 64 + 16 * i + FpMfma<F>::row(lane, r);
                if (tr < rows) out[(int64_t)orow_s[tr] * N + n] = acc[i][j][r] + bv;
            }
    }
}

}  // namespace

size_t grouped_workspace_bytes(int64_t M, int64_t S, int64_t G) {
    const int64_t P = M * S;
    return (size_t)(off_sorted(P, G) + 4 * P + 255) / 256 * 256;
}

namespace {
// Routing kernels: counts, tile table and the pairs sorted by group in `ws`.
hipError_t launch_routing(const GroupedArgs& a, void* ws, hipStream_t s, int bm) {
    const int64_t P = a.M * a.S;
    char* w = (char*)ws;
    const unsigned nchunk = (unsigned)((P + ROUTE_CHUNK - 1) / ROUTE_CHUNK);
    hipLaunchKernelGGL(route_zero_kernel, dim3(1), dim3(256), 0, s, w, (int)a.G);
    if (nchunk) {
        hipLaunchKernelGGL(route_hist_kernel, dim3(nchunk), dim3(256), 0, s, a.idx, a.idx64, P, (int)a.G, w);
    }
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(ROUTE_THREADS), 0, s, P, (int)a.G, bm, w);
    if (nchunk) {
        hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunk), dim3(256), 0, s, a.idx, a.idx64, P, (int)a.G, w);
    }
    return hipGetLastError();
}
bool al(const void* q, uintptr_t n) { return ((uintptr_t)q & (n - 1)) == 0; }

// fp32 (dt 2) / fp64 (dt 3) grouped product: routing into 128-row tiles, then
// grouped_fp_kernel; wq = 1 / 2: int8 / uint8 weights dequantised on load (fp32)
hipError_t launch_grouped_fp(const GroupedArgs& a, int dt, int wq, void* ws, hipStream_t s) {
    const int64_t P = a.M * a.S;
    hipError_t e = launch_routing(a, ws, s, FT);
    if (e != hipSuccess) return e;
    if (P == 0 || a.N == 0) return hipSuccess;
    const int64_t max_mtiles = P / FT + a.G;
    const int64_t tiles_n = (a.N + FT - 1) / FT;
    if (max_mtiles * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(max_mtiles * tiles_n));
    const char* wsc = (const char*)ws;
    const int tn = (int)tiles_n;
    log_choice("grouped %s%s M=%lld S=%lld K=%lld N=%lld G=%lld: 128x128x16 routed tiles, %s MFMA",
               dt == 3 ? "fp64" : "fp32", wq ? " (int8/uint8 weights, dequantised on load)" : "", (long long)a.M,
               (long long)a.S, (long long)a.K, (long long)a.N, (long long)a.G,
               dt == 3 ? "16x16x4 fp64" : "16x16x4 fp32");
    if (dt == 3)
        hipLaunchKernelGGL((grouped_fp_kernel<double, 0>), grid, dim3(256), 0, s, a, wsc, tn);
    else if (wq == 0)
        hipLaunchKernelGGL((grouped_fp_kernel<float, 0>), grid, dim3(256), 0, s, a, wsc, tn);
    else if (wq == 1)
        hipLaunchKernelGGL((grouped_fp_kernel<float, 1>), grid, dim3(256), 0, s, a, wsc, tn);
    else
        hipLaunchKernelGGL((grouped_fp_kernel<float, 2>), grid, dim3(256), 0, s, a, wsc, tn);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_grouped_dq(const GroupedArgs& a, int dt, void* ws, hipStream_t s) {
    const int64_t P = a.M * a.S;
    if (a.G > MAX_G || P > 0x7fffffff || a.bs < 1) return hipErrorInvalidValue;
    const int qu8 = a.q_kind == 2;
    if (dt == 2) return launch_grouped_fp(a, dt, qu8 ? 2 : 1, ws, s);
    hipError_t e = launch_routing(a, ws, s, GBM);
    if (e != hipSuccess) return e;
    if (P == 0 || a.N == 0) return hipSuccess;
    const int64_t max_mtiles = P / GBM + a.G;
    const int64_t tiles_n = (a.N + GBN - 1) / GBN;
    if (max_mtiles * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    // the gathered input goes by DMA (32-bit offsets: it must span < 2 GiB)
    const bool fast = al(a.input, 16) && a.K % 8 == 0 && a.M * a.K * 2 < (1LL << 31) && a.N % 8 == 0 &&
                      al(a.weights, 8) && al(a.wscale, 16) && (!a.wzp || al(a.wzp, 8)) &&
                      a.bs % core16::KSTEP == 0 && al(a.output, 8) && (!a.bias || al(a.bias, 8));
    dim3 grid((unsigned)(max_mtiles * tiles_n));
    const char* wsc = (const char*)ws;
    const int tn = (int)tiles_n;
    // weights by DMA as well: whole stages (K % 64 == 0), 16-byte weight rows
    const bool dma = fast && a.K % core16::KSTEP == 0 && a.N % 16 == 0 && al(a.weights, 16) &&
                     (!a.wzp || al(a.wzp, 16)) && core16::KSTEP * a.N < (1LL << 31) &&
                     a.nkb * a.N * 2 < (1LL << 31);
    log_choice("grouped %s over %s weights, block %lld, M=%lld S=%lld K=%lld N=%lld G=%lld: 256x256x64 routed tiles, %s",
               dt == 0 ? "bf16" : "fp16", qu8 ? "uint8" : "int8", (long long)a.bs, (long long)a.M, (long long)a.S,
               (long long)a.K, (long long)a.N, (long long)a.G,
               dma ? "weights by DMA, dequantised in LDS fragments" : fast ? "weights register-staged" : "element-wise");
    if (dma) {
        if (dt == 0) {
            if (qu8) hipLaunchKernelGGL((grouped16_dq_dma_kernel<0, true>), grid, dim3(256), 0, s, a, wsc, tn);
            else hipLaunchKernelGGL((grouped16_dq_dma_kernel<0, false>), grid, dim3(256), 0, s, a, wsc, tn);
        } else {
            if (qu8) hipLaunchKernelGGL((grouped16_dq_dma_kernel<1, true>), grid, dim3(256), 0, s, a, wsc, tn);
            else hipLaunchKernelGGL((grouped16_dq_dma_kernel<1, false>), grid, dim3(256), 0, s, a, wsc, tn);
        }
        return hipGetLastError();
    }
#define OMM_DQ(D, U, F) hipLaunchKernelGGL((grouped16_dq_kernel<D, U, F>), grid, dim3(256), 0, s, a, wsc, tn)
    if (dt == 0) {
        if (qu8) { if (fast) OMM_DQ(0, true, true); else OMM_DQ(0, true, false); }
        else { if (fast) OMM_DQ(0, false, true); else OMM_DQ(0, false, false); }
    } else {
        if (qu8) { if (fast) OMM_DQ(1, true, true); else OMM_DQ(1, true, false); }
        else { if (fast) OMM_DQ(1, false, true); else OMM_DQ(1, false, false); }
    }
#undef OMM_DQ
    return hipGetLastError();
}

hipError_t launch_grouped(const GroupedArgs& a, int dt, void* ws, hipStream_t s) {
    const int64_t P = a.M * a.S;
    if (a.G > MAX_G || P > 0x7fffffff) return hipErrorInvalidValue;
    if (dt >= 2) return launch_grouped_fp(a, dt, 0, ws, s);
    hipError_t e = launch_routing(a, ws, s, GBM);
    if (e != hipSuccess) return e;
    if (P == 0 || a.N == 0) return hipSuccess;
    const int64_t max_mtiles = P / GBM + a.G;
    const int64_t tiles_n = (a.N + GBN - 1) / GBN;
    if (max_mtiles * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    // DMA offsets are 32-bit: the gathered input and one k-stage of a group's weights must span < 2 GiB
    const bool vec = al(a.input, 16) && al(a.weights, 16) && al(a.output, 8) && (!a.bias || al(a.bias, 8)) &&
                     a.K % 8 == 0 && a.N % 8 == 0 && a.M * a.K * 2 < (1LL << 31) && 64 * a.N * 2 < (1LL << 31) &&
                     a.K > 0;  // the DMA K loop runs at least one stage
    dim3 grid((unsigned)(max_mtiles * tiles_n));
    const char* wsc = (const char*)ws;
    log_choice("grouped %s M=%lld S=%lld K=%lld N=%lld G=%lld: 256x256x64 routed tiles, %s", dt == 0 ? "bf16" : "fp16",
               (long long)a.M, (long long)a.S, (long long)a.K, (long long)a.N, (long long)a.G,
               vec ? "16x16x32 MFMA, DMA (gathered rows)" : "32x32x16 MFMA, element-wise loads");
    if (dt == 0) {
        if (vec) hipLaunchKernelGGL((grouped16_kernel<0, true>), grid, dim3(256), 0, s, a, wsc, (int)tiles_n);
        else hipLaunchKernelGGL((grouped16_kernel<0, false>), grid, dim3(256), 0, s, a, wsc, (int)tiles_n);
    } else {
        if (vec) hipLaunchKernelGGL((grouped16_kernel<1, true>), grid, dim3(256), 0, s, a, wsc, (int)tiles_n);
        else hipLaunchKernelGGL((grouped16_kernel<1, false>), grid, dim3(256), 0, s, a, wsc, (int)tiles_n);
    }
    return hipGetLastError();
}

hipError_t grouped_invalid_count(const void* ws, hipStream_t s, int64_t* count) {
    int hdr[2] = {0, 0};
    hipError_t e = hipMemcpyAsync(hdr, ws, sizeof hdr, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    *count = hdr[1];
    return hipSuccess;
}

}  // namespace omm
