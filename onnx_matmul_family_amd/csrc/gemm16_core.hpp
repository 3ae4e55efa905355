// MFMA core shared by the bf16 / fp16 GEMM kernels (dense and grouped): the
// operand tile sources, the swizzled LDS tile layouts, the MFMA fragment reads
// and the double-buffered K loops.
//
// Per workgroup of 256 threads = 4 waves on the CU's 4 SIMDs: output tile
// BM x BN (256x256 or 128x128), K consumed 64 values per stage, each wave owns
// a (BM/2) x (BN/2) sub-tile in fp32 accumulators (AGPRs at 256x256).
// The main path moves tiles global -> LDS directly (buffer_load ... lds, no
// register staging), double-buffered, the DMA of stage k+2 in flight while
// stage k multiplies (mainloop_dma16: 16x16x32 MFMAs; mainloop_dma: 32x32x16).
// Unaligned operands take a register-staged loop (mainloop: 16-byte or element
// loads into registers, then LDS stores, one barrier per stage).  Operands with
// k contiguous sit in LDS as XOR-swizzled 128-byte rows read with ds_read_b128;
// operands with m/n contiguous are copied as they are (swizzled 32-byte
// granules) and read with the transposing ds_read_b64_tr_b16, so no register
// transpose.
#pragma once
#include <type_traits>

#include "device_common.hpp"

namespace omm {
namespace core16 {

constexpr int NT = 256;
constexpr int KSTEP = 64;  // k-values per LDS stage

// Position of chunk i (16 bytes = 8 elements) of thread t in an operand tile
// with R rows along m/n.  K-major: (mn row, k offset); MN-major: (k row, mn offset).
template <int R, bool KMAJ>
struct Chunks {
    static constexpr int NC = R * KSTEP / 8 / NT;
    static constexpr int PER_ROW_MN = R / 8;  // MN-major: chunks per k row
    __device__ static void coords(int t, int i, int& lmn, int& lk) {
        if constexpr (KMAJ) {
            // a wave's 64 lanes cover 8 rows x 8 chunks; lanes 8c..8c+7 take
            // chunk c of 8 consecutive rows (conflict-free LDS stores)
            lmn = ((t >> 6) << 3) + (t & 7) + 32 * i;
            lk = ((t >> 3) & 7) * 8;
        } else {
            lk = t / PER_ROW_MN + (NT / PER_ROW_MN) * i;
            lmn = (t % PER_ROW_MN) * 8;
        }
    }
    // byte offset of that chunk inside the LDS tile
    __device__ static int lds_off(int lmn, int lk) {
        if constexpr (KMAJ)
            return kmaj_off<R>(lmn, lk >> 3);
        else
            return mmaj16_off<R * 2>(lk, lmn * 2);
    }
};

// Global -> register copy of one operand tile.  A thread's chunk i sits at
// p0 + i * si (si uniform), and the tile advances by `step` elements per stage.
//  MODE 0: whole tile in range, 16-byte loads.
//  MODE 1: 16-byte loads, chunk-granular range checks (contiguous extent % 8 == 0).
//  MODE 2: element loads with element range checks (any shape / alignment).
template <int R, bool KMAJ>
struct TileSrc {
    const uint16_t* p0;  // chunk 0 of this thread at stage 0
    int64_t si;          // element distance between a thread's consecutive chunks
    int64_t step;        // element advance per K stage
    int64_t mn_first;    // global m/n index of chunk 0's first element
    int64_t k_first;     // global k index of chunk 0's first element (stage 0)
    int64_t MN, K;

    __device__ void init(const uint16_t* base, int64_t ld, int64_t mn0, int64_t MN_, int64_t K_, int t) {
        int lmn, lk;
        Chunks<R, KMAJ>::coords(t, 0, lmn, lk);
        mn_first = mn0 + lmn;
        k_first = lk;
        MN = MN_;
        K = K_;
        if constexpr (KMAJ) {
            p0 = base + mn_first * ld + lk;
            si = 32 * ld;
            step = KSTEP;
        } else {
            p0 = base + (int64_t)lk * ld + mn_first;
            si = (int64_t)(NT / Chunks<R, KMAJ>::PER_ROW_MN) * ld;
            step = (int64_t)KSTEP * ld;
        }
    }

    template <int MODE, int NC>
    __device__ __forceinline__ void load(u32x4_t (&reg)[NC], int kt) const {
        const uint16_t* p = p0 + (int64_t)kt * step;
        const int64_t k0 = k_first + (int64_t)kt * KSTEP;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const uint16_t* q = p + i * si;
            // chunk i covers (mn, k .. k+7) [K-major] or (k, mn .. mn+7) [MN-major]
            const int64_t mn = KMAJ ? mn_first + 32 * i : mn_first;
            const int64_t k = KMAJ ? k0 : k0 + (int64_t)(NT / Chunks<R, KMAJ>::PER_ROW_MN) * i;
            if constexpr (MODE == 0) {
                reg[i] = *(const u32x4_t*)q;
            } else if constexpr (MODE == 1) {
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (mn < MN && k < K) v = *(const u32x4_t*)q;
                reg[i] = v;
            } else {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    uint32_t lo = 0, hi = 0;
                    if (KMAJ) {
                        if (mn < MN && k + e < K) lo = q[e];
                        if (mn < MN && k + e + 1 < K) hi = q[e + 1];
                    } else {
                        if (k < K && mn + e < MN) lo = q[e];
                        if (k < K && mn + e + 1 < MN) hi = q[e + 1];
                    }
                    w[e >> 1] = lo | (hi << 16);
                }
                reg[i] = u32x4_t{w[0], w[1], w[2], w[3]};
            }
        }
    }
};

// K-major A source whose rows are gathered through a row-offset table (the
// grouped product reads token rows input[pair / S]).  Chunk i of thread t is
// the tile row Chunks<R, true>::coords gives; rows >= `rows` read as zero.
template <int R>
struct GatherSrc {
    static constexpr int NC = Chunks<R, true>::NC;
    const uint16_t* base;
    int64_t roff[NC];  // element offset of each chunk's row (+ its k offset)
    uint32_t valid;    // bit i: chunk i's row exists
    int64_t K;
    int lk;

    template <int MODE, int NC_>
    __device__ __forceinline__ void load(u32x4_t (&reg)[NC_], int kt) const {
        const int64_t k = (int64_t)kt * KSTEP + lk;
#pragma unroll
        for (int i = 0; i < NC_; ++i) {
            const uint16_t* q = base + roff[i] + (int64_t)kt * KSTEP;
            const bool rok = (valid >> i) & 1u;
            if constexpr (MODE == 0) {
                reg[i] = *(const u32x4_t*)q;
            } else if constexpr (MODE == 1) {
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (rok && k < K) v = *(const u32x4_t*)q;
                reg[i] = v;
            } else {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    uint32_t lo = 0, hi = 0;
                    if (rok && k + e < K) lo = q[e];
                    if (rok && k + e + 1 < K) hi = q[e + 1];
                    w[e >> 1] = lo | (hi << 16);
                }
                reg[i] = u32x4_t{w[0], w[1], w[2], w[3]};
            }
        }
    }
};

template <int R, bool KMAJ, int NC>
__device__ __forceinline__ void store_tile(char* lds, const u32x4_t (&reg)[NC], int t) {
    using C = Chunks<R, KMAJ>;
#pragma unroll
    for (int i = 0; i < C::NC; ++i) {
        int lmn, lk;
        C::coords(t, i, lmn, lk);
        *(u32x4_t*)(lds + C::lds_off(lmn, lk)) = reg[i];
    }
}

// MFMA operand fragment for rows/columns [mnb, mnb+32) and k-block s (16 values)
// of an LDS tile: lane l gets mn = mnb + l%32, k = 16 s + 8 (l/32) + 0..7.
template <int R, bool KMAJ>
__device__ __forceinline__ u32x4_t read_frag(const char* lds, int mnb, int s, int lane) {
    if constexpr (KMAJ) {
        return *(const u32x4_t*)(lds + mnb * 128 + kmaj_lane(lane, s));
    } else {
        const int g = lane >> 4, i = lane & 15;
        const int krow = 16 * s + 8 * (g >> 1) + (i >> 2);
        const int n = mnb + 16 * (g & 1) + 4 * (i & 3);
        const int off = mmaj16_off<R * 2>(krow, n * 2), off4 = mmaj16_off<R * 2>(krow + 4, n * 2);
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OMM_LDS(i16x4_t, lds + off));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OMM_LDS(i16x4_t, lds + off4));
        u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        return u32x4_t{l2.x, l2.y, h2.x, h2.y};
    }
}

// Register-staged K loop (element-wise loads, any shape / alignment).
template <int BM, int BN, int DT, bool AK, bool BKM, int MODE, class SA, class SB>
__device__ __forceinline__ void mainloop(f32x16_t (&acc)[BM / 64][BN / 64], char* smem0, char* smem1,
                                         const SA& srcA, const SB& srcB, int nk, int t, int lane, int wm, int wn) {
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int A_BYTES = BM * KSTEP * 2;
    u32x4_t ra[Chunks<BM, AK>::NC], rb[Chunks<BN, BKM>::NC];
    if (nk > 0) {
        srcA.template load<MODE>(ra, 0);
        srcB.template load<MODE>(rb, 0);
        store_tile<BM, AK>(smem0, ra, t);
        store_tile<BN, BKM>(smem0 + A_BYTES, rb, t);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            srcA.template load<MODE>(ra, kt + 1);
            srcB.template load<MODE>(rb, kt + 1);
        }
        const char* sa = buf ? smem1 : smem0;
        const char* sb = sa + A_BYTES;
#pragma unroll
        for (int s = 0; s < KSTEP / 16; ++s) {
            u32x4_t af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = read_frag<BM, AK>(sa, wm * WM + 32 * i, s, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = read_frag<BN, BKM>(sb, wn * WN + 32 * j, s, lane);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<DT>(bfr[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk) {
            char* so = buf ? smem0 : smem1;
            store_tile<BM, AK>(so, ra, t);
            store_tile<BN, BKM>(so + A_BYTES, rb, t);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS path: buffer_load_dwordx4 ... lds.  Each wave
// instruction fills one contiguous 1 KiB LDS block (lane p -> bytes 16p..16p+15),
// so a lane chooses which global 16-byte chunk lands in its slot; the tile
// layouts above are produced by that choice.  Out-of-range lanes get a byte
// offset past the buffer's range and the hardware writes zeros, which pads
// ragged tiles and K tails without branches.  Offsets are 32-bit: a tile's
// rows must span less than 2 GiB (checked on the host).
constexpr uint32_t DMA_OOB = 0x80000000u;

// Raw buffer resource (gfx9 family): base, stride 0, 2^31-1 bytes in range, or
// an empty range (every access out of range: no memory access, zeros into LDS).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, bool live = true) {
    const uint64_t a = (uint64_t)base;
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)), live ? 0x7fffffff : 0, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)OMM_LDS(const char, p));
}
// The DMA load is issued from inline assembly on purpose: the compiler's
// wait-count pass cannot tell which LDS buffer an LDS-DMA intrinsic writes and
// would make every later ds_read wait for all DMA traffic in flight (the
// prefetch of the next stage included).  The kernels wait for their own DMA
// (s_waitcnt vmcnt) before the barrier that publishes a stage.  M0 is set per
// instruction, followed by the one wait state an M0 write needs before an
// LDS-DMA read of it.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds),
        "v"(voff), "s"(rsrc)
        : "memory", "m0");
}
__device__ __forceinline__ void dma16u(i32x4_t rsrc, uint32_t lds, uint32_t voff) {
    dma16(rsrc, (uint32_t)__builtin_amdgcn_readfirstlane((int)lds), voff);
}
// buffer resource and LDS base of one stage's DMA
struct DmaCtx {
    i32x4_t r;
    uint32_t l0;
};

// One operand tile (R rows along m/n, 128 bytes of k per stage) loaded by DMA.
// ES = element size in bytes (2: bf16/fp16, 1: int8; MN-major needs ES = 2).
//  K-major: LDS block b = rows 8b .. 8b+7; lane p -> row 8b + p/8, slot p%8,
//           logical chunk (p%8) ^ kswz(row): 8 whole 128-byte row segments
//           (kswz(row) = 4 (b & 1) + p/16 depends on the block's parity).
//  MN-major: LDS block b = k rows RPB b .. RPB b + RPB-1 (RPB = 1024 / (2R));
//           lane p -> row p / LPR, physical 16-byte chunk p % LPR (LPR = R/8),
//           logical 32-byte granule = physical ^ mswz16(row).
template <int R, bool KMAJ, int ES = 2>
struct DmaSrc {
    static_assert(KMAJ || ES == 2, "8-bit MN-major tiles use DmaSrcMN8");
    static_assert((R / 32) % 2 == 0, "block parity == parity of the wave-local block index");
    static constexpr int NBLK = R / 8;  // 1 KiB blocks per stage
    static constexpr int PER_WAVE = NBLK / 4;
    static constexpr int RPB = KMAJ ? 8 : 1024 / (2 * R);
    static constexpr int LPR = R / 8;
    // MN-major: the swizzle repeats every 16 rows, so blocks come in 16 / RPB phases
    static constexpr int NQ = KMAJ ? 2 : (16 / RPB > 1 ? 16 / RPB : 1);
    static_assert(KMAJ || PER_WAVE % NQ == 0, "block phase == phase of the wave-local block index");
    static constexpr int KE = 128 / ES;  // k elements per stage
    const char* base;   // tile origin at stage 0 (bytes)
    int64_t step;       // bytes per stage
    uint32_t ldb;       // row stride as stored (bytes)
    uint32_t lane_off[NQ];
    int64_t MN, K, mn0;
    int lane;

    __device__ void init(const void* b, int64_t ld, int64_t mn0_, int64_t MN_, int64_t K_, int lane_) {
        lane = lane_;
        MN = MN_;
        K = K_;
        mn0 = mn0_;
        ldb = (uint32_t)(ld * ES);
        if constexpr (KMAJ) {
            base = (const char*)b + mn0 * ld * ES;
            step = 128;
#pragma unroll
            for (int q = 0; q < 2; ++q) lane_off[q] = (uint32_t)(lane >> 3) * ldb + (kchunk(q) << 4);
        } else {
            base = (const char*)b + mn0 * ES;
            step = (int64_t)KE * ld * ES;
#pragma unroll
            for (int q = 0; q < NQ; ++q) lane_off[q] = (uint32_t)(lane / LPR) * ldb + (chunk(q) << 4);
        }
    }
    // K-major: logical 16-byte chunk (along k) of this lane in a block of parity q
    __device__ uint32_t kchunk(int q) const { return (uint32_t)((lane & 7) ^ kswz(8 * q + (lane >> 3))); }
    // MN-major: logical 16-byte chunk (along m/n) of this lane in a block of phase q
    __device__ uint32_t chunk(int q) const {
        const int row = q * RPB + lane / LPR, C = lane % LPR;
        return (uint32_t)(2 * ((C >> 1) ^ mswz16(row)) + (C & 1));
    }

    __device__ __forceinline__ DmaCtx ctx(char* lds, int kt, bool live = true) const {
        return DmaCtx{make_rsrc(base + (live ? (int64_t)kt * step : 0), live), lds_addr(lds)};
    }
    template <bool CHECKED>
    __device__ __forceinline__ void issue(char* lds, int kt, int wave, bool live = true) const {
        const DmaCtx c = ctx(lds, kt, live);
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) one<CHECKED>(c, kt, wave, j);
    }
    // block j (0 .. PER_WAVE-1) of this wave's share of stage kt
    template <bool CHECKED>
    __device__ __forceinline__ void one(const DmaCtx& c, int kt, int wave, int j) const {
        {
            const int b = wave * PER_WAVE + j;
            uint32_t voff;
            if constexpr (KMAJ) {
                voff = lane_off[j & 1] + (uint32_t)(b * 8) * ldb;
                if (CHECKED) {
                    // a select, not a branch: exec-mask writes between the
                    // MFMAs stall their issue
                    const int64_t row = mn0 + b * 8 + (lane >> 3);
                    const int64_t k = (int64_t)kt * KE + (16 / ES) * kchunk(j & 1);
                    voff = ((row < MN) & (k < K)) ? voff : DMA_OOB;
                }
            } else {
                voff = lane_off[j % NQ] + (uint32_t)(b * RPB) * ldb;
                if (CHECKED) {
                    const int64_t k = (int64_t)kt * KE + b * RPB + lane / LPR;
                    const int64_t mn = mn0 + 8 * (int64_t)chunk(j % NQ);
                    voff = ((k < K) & (mn < MN)) ? voff : DMA_OOB;
                }
            }
            dma16u(c.r, c.l0 + b * 1024, voff);
        }
    }
};

// 8-bit MN-major tile (int8 b, n contiguous): KR k rows of R bytes per stage,
// 16-byte chunk c of row k stored at chunk c ^ mswz8(k).  LDS block b = rows
// 4b..4b+3 (R = 256); lane p -> row p / 16, physical chunk p % 16.
template <int R, int KR = 128>
struct DmaSrcMN8 {
    static_assert(R == 256, "256-byte rows");
    static constexpr int PER_WAVE = KR / 16;  // KR / 4 blocks per stage
    static_assert(PER_WAVE % 2 == 0, "block phase == parity of the wave-local block index");
    const char* base;
    int64_t step;
    uint32_t ldb;
    uint32_t lane_off[2];
    int64_t MN, K, mn0;
    int lane;

    __device__ uint32_t chunk(int q) const {
        const int row = 4 * q + (lane >> 4);
        return (uint32_t)((lane & 15) ^ mswz8(row));
    }
    __device__ void init(const void* b, int64_t ld, int64_t mn0_, int64_t MN_, int64_t K_, int lane_) {
        lane = lane_;
        MN = MN_;
        K = K_;
        mn0 = mn0_;
        ldb = (uint32_t)ld;
        base = (const char*)b + mn0;
        step = (int64_t)KR * ld;
#pragma unroll
        for (int q = 0; q < 2; ++q) lane_off[q] = (uint32_t)(lane >> 4) * ldb + (chunk(q) << 4);
    }
    __device__ __forceinline__ DmaCtx ctx(char* lds, int kt, bool live = true) const {
        return DmaCtx{make_rsrc(base + (live ? (int64_t)kt * step : 0), live), lds_addr(lds)};
    }
    template <bool CHECKED>
    __device__ __forceinline__ void issue(char* lds, int kt, int wave, bool live = true) const {
        const DmaCtx c = ctx(lds, kt, live);
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) one<CHECKED>(c, kt, wave, j);
    }
    template <bool CHECKED>
    __device__ __forceinline__ void one(const DmaCtx& c, int kt, int wave, int j) const {
        const int b = wave * PER_WAVE + j;
        uint32_t voff = lane_off[j & 1] + (uint32_t)(b * 4) * ldb;
        if (CHECKED) {
            const int64_t k = (int64_t)kt * KR + b * 4 + (lane >> 4);
            const int64_t mn = mn0 + 16 * (int64_t)chunk(j & 1);
            voff = ((k < K) & (mn < MN)) ? voff : DMA_OOB;
        }
        dma16u(c.r, c.l0 + b * 1024, voff);
    }
};

// K-major A tile whose rows are gathered (grouped product: token rows
// input[pair / S]), same layout as DmaSrc K-major.  Wave w fills blocks
// w*PER_WAVE + j; roff[j] = byte offset of the row this lane loads in block j
// (DMA_OOB for rows past the tile's valid rows) plus the lane's chunk.
template <int R>
struct GatherDma {
    static constexpr int NBLK = R / 8;
    static constexpr int PER_WAVE = NBLK / 4;
    static_assert(PER_WAVE % 2 == 0, "block parity == parity of the wave-local block index");
    const char* base;
    uint32_t roff[PER_WAVE];
    int64_t K;
    int lane;

    // tile row loaded by this lane in block j of wave w, and its chunk's byte offset
    __device__ static int row_of(int w, int j, int lane) { return 8 * (w * PER_WAVE + j) + (lane >> 3); }
    // logical chunk of this lane in block j (kswz of its row depends on j's parity)
    __device__ static uint32_t chunk(int j, int lane) { return (uint32_t)((lane & 7) ^ kswz(8 * (j & 1) + (lane >> 3))); }

    __device__ __forceinline__ DmaCtx ctx(char* lds, int kt, bool live = true) const {
        return DmaCtx{make_rsrc(base + (live ? (int64_t)kt * KSTEP * 2 : 0), live), lds_addr(lds)};
    }
    template <bool CHECKED>
    __device__ __forceinline__ void issue(char* lds, int kt, int wave, bool live = true) const {
        const DmaCtx c = ctx(lds, kt, live);
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) one<CHECKED>(c, kt, wave, j);
    }
    template <bool CHECKED>
    __device__ __forceinline__ void one(const DmaCtx& c, int kt, int wave, int j) const {
        const int b = wave * PER_WAVE + j;
        uint32_t voff = roff[j];
        if (CHECKED) {
            const int64_t k = (int64_t)kt * KSTEP + 8 * chunk(j, lane);
            voff = k < K ? voff : DMA_OOB;
        }
        dma16u(c.r, c.l0 + b * 1024, voff);
    }
};

template <int BM, int BN, bool AK, bool BKM>
struct Frags {
    static constexpr int TM = BM / 64, TN = BN / 64;
    u32x4_t a[TM], b[TN];
    __device__ __forceinline__ void read(const char* st, int s, int lane, int wm, int wn) {
        constexpr int A_BYTES = BM * KSTEP * 2;
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = read_frag<BM, AK>(st, wm * (BM / 2) + 32 * i, s, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = read_frag<BN, BKM>(st + A_BYTES, wn * (BN / 2) + 32 * j, s, lane);
    }
    // fragment R of k-block s: R < TM -> a[R], else b[R - TM]
    template <int R>
    __device__ __forceinline__ void read_one(const char* st, int s, int lane, int wm, int wn) {
        constexpr int A_BYTES = BM * KSTEP * 2;
        if constexpr (R < TM)
            a[R] = read_frag<BM, AK>(st, wm * (BM / 2) + 32 * R, s, lane);
        else
            b[R - TM] = read_frag<BN, BKM>(st + A_BYTES, wn * (BN / 2) + 32 * (R - TM), s, lane);
    }
};

template <int DT, int TM, int TN, class F>
__device__ __forceinline__ void mma_step(f32x16_t (&acc)[TM][TN], const F& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<DT>(f.b[j], f.a[i], acc[i][j]);
}

__device__ __forceinline__ void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

// Wait until at most n of this wave's vector-memory ops are outstanding (gfx9
// s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left unrestricted).
template <int n>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1, so every
// register-array index below is a constant.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Fragment read order within a k-block.  MFMA X of a k-block uses A fragment
// X / TN (first needed by MFMA i*TN) and B fragment X % TN (first needed by
// MFMA j); reading the next k-block's fragments in order of first use (B
// before A on ties) leaves every read the most MFMAs to land.  Fragment ids:
// 0 .. TM-1 = A, TM .. TM+TN-1 = B.
constexpr int frag_order(int TM, int TN, int r) {
    int done[16] = {};
    int pick = 0;
    for (int n = 0; n <= r; ++n) {
        int best = -1, bt = 1 << 20;
        for (int f = 0; f < TM + TN; ++f) {
            if (done[f]) continue;
            const int t = f < TM ? 2 * (f * TN) + 1 : 2 * (f - TM);  // B first on equal times
            if (t < bt) { bt = t; best = f; }
        }
        done[best] = 1;
        pick = best;
    }
    return pick;
}

// MFMA number X (0 .. TM*TN-1) of a k-block: tile (X / TN, X % TN).
template <int X, int DT, int TM, int TN, class F>
__device__ __forceinline__ void mma_one(f32x16_t (&acc)[TM][TN], const F& f) {
    acc[X / TN][X % TN] = mfma32x32x16<DT>(f.b[X % TN], f.a[X / TN], acc[X / TN][X % TN]);
}

// One k-block of MFMAs on `cur`, with the TM+TN fragment reads of k-block s of
// `lds` into `nxt` spread evenly between them (read r after MFMA r*NM/NR), so
// the LDS sees a steady stream instead of bursts.
template <int DT, int TM, int TN, class F>
__device__ __forceinline__ void kblock_read(f32x16_t (&acc)[TM][TN], const F& cur, F& nxt, const char* lds, int s,
                                            int lane, int wm, int wn) {
    constexpr int NM = TM * TN, NR = TM + TN;
    static_for<0, NM>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        mma_one<x, DT>(acc, cur);
        static_for<(x * NR + NM - 1) / NM, ((x + 1) * NR + NM - 1) / NM>([&](auto rc) {
            nxt.template read_one<frag_order(TM, TN, decltype(rc)::value)>(lds, s, lane, wm, wn);
        });
        fence_sched();
    });
}

// DMA instruction d (0 .. LA+LB-1) of this wave's share of one stage: the
// first LA go to operand A, the rest to operand B.
template <bool CHECKED, int LA, int d, class SA, class SB>
__device__ __forceinline__ void dma_one(const SA& srcA, const SB& srcB, const DmaCtx& ca, const DmaCtx& cb, int kt,
                                        int wave) {
    if constexpr (d < LA)
        srcA.template one<CHECKED>(ca, kt, wave, d);
    else
        srcB.template one<CHECKED>(cb, kt, wave, d - LA);
}

// One k-block of MFMAs on `cur` with the fragment reads of k-block s of `lds`
// into `nxt`, and this wave's DMA instructions D0 .. D1-1 of stage kt (into
// buffer X) spread evenly between the MFMAs: issuing them back to back would
// stall the wave on the memory pipeline.
template <int DT, int TM, int TN, bool CHECKED, int D0, int D1, class F, class SA, class SB>
__device__ __forceinline__ void kblock_read_dma(f32x16_t (&acc)[TM][TN], const F& cur, F& nxt, const char* lds, int s,
                                                char* X, int A_BYTES, const SA& srcA, const SB& srcB, int kt,
                                                bool live, int lane, int wm, int wn, int wave) {
    constexpr int NM = TM * TN, NR = TM + TN, ND = D1 - D0;
    constexpr int LA = SA::PER_WAVE;
    const DmaCtx ca = srcA.ctx(X, kt, live), cb = srcB.ctx(X + A_BYTES, kt, live);
    static_for<0, NM>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        mma_one<x, DT>(acc, cur);
        static_for<D0 + (x * ND + NM - 1) / NM, D0 + ((x + 1) * ND + NM - 1) / NM>(
            [&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(srcA, srcB, ca, cb, kt, wave); });
        static_for<(x * NR + NM - 1) / NM, ((x + 1) * NR + NM - 1) / NM>([&](auto rc) {
            nxt.template read_one<frag_order(TM, TN, decltype(rc)::value)>(lds, s, lane, wm, wn);
        });
        fence_sched();
    });
}

// One stage of the DMA K loop.  On entry stage kt is complete in X (barrier
// passed), fc holds its k-block 0 fragments (requested), and the first half of
// stage kt+1's DMA into Y is in flight.  The second half of stage kt+1's DMA
// goes out during k-block 0, the barrier after k-block 2 retires X and lands
// Y, and the first half of stage kt+2's DMA into X goes out during k-block 3.
// Each DMA thus has at least two k-blocks of MFMAs to land before its barrier.
// Past the last stage the DMA targets an empty range (zeros into a buffer no
// later stage reads) and the reads of Y fetch values nobody uses: the stage
// has no data-dependent branches, so the accumulators flow through
// straight-line code.
template <int BM, int BN, int DT, bool AK, bool BKM, bool CHECKED, class SA, class SB, class F>
__device__ __forceinline__ void dma_stage(f32x16_t (&acc)[BM / 64][BN / 64], F& fc, F& fn, char* X, char* Y,
                                          const SA& srcA, const SB& srcB, int kt, int nk, int lane, int wm, int wn,
                                          int wave) {
    constexpr int A_BYTES = BM * KSTEP * 2;
    constexpr int LD = SA::PER_WAVE + SB::PER_WAVE, H = LD / 2;
    constexpr int TM = BM / 64, TN = BN / 64;
    fence_sched();
    kblock_read_dma<DT, TM, TN, CHECKED, H, LD>(acc, fc, fn, X, 1, Y, A_BYTES, srcA, srcB, kt + 1, kt + 1 < nk,
                                                lane, wm, wn, wave);
    kblock_read<DT>(acc, fn, fc, X, 2, lane, wm, wn);
    kblock_read<DT>(acc, fc, fn, X, 3, lane, wm, wn);
    wait_vm<0>();     // this wave's DMA of stage kt+1 has landed
    __syncthreads();  // ... every wave's; and every read of X is done
    fence_sched();
    kblock_read_dma<DT, TM, TN, CHECKED, 0, H>(acc, fn, fc, Y, 0, X, A_BYTES, srcA, srcB, kt + 2, kt + 2 < nk, lane,
                                               wm, wn, wave);
}

// DMA K loop over nk stages; stage kt lives in buffer kt & 1 (s0 / s1).  The
// loop body covers two stages so that each LDS access names its buffer
// statically; an odd stage count runs one more stage of zeros.  On return no
// DMA is in flight.
template <int BM, int BN, int DT, bool AK, bool BKM, bool CHECKED, class SA, class SB>
__device__ __forceinline__ void mainloop_dma(f32x16_t (&acc)[BM / 64][BN / 64], char* __restrict__ s0,
                                             char* __restrict__ s1, const SA& srcA, const SB& srcB, int nk, int lane,
                                             int wm, int wn, int wave) {
    constexpr int A_BYTES = BM * KSTEP * 2;
    constexpr int LA = SA::PER_WAVE, LD = SA::PER_WAVE + SB::PER_WAVE, H = LD / 2;
    if (nk <= 0) return;
    {
        // stage 0 whole, the first half of stage 1
        const DmaCtx a0 = srcA.ctx(s0, 0, true), b0 = srcB.ctx(s0 + A_BYTES, 0, true);
        static_for<0, LD>([&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(srcA, srcB, a0, b0, 0, wave); });
        const DmaCtx a1 = srcA.ctx(s1, 1, nk > 1), b1 = srcB.ctx(s1 + A_BYTES, 1, nk > 1);
        static_for<0, H>([&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(srcA, srcB, a1, b1, 1, wave); });
    }
    wait_vm<H>();
    __syncthreads();
    Frags<BM, BN, AK, BKM> fc, fn;
    fc.read(s0, 0, lane, wm, wn);
    for (int kt = 0; kt < nk; kt += 2) {
        dma_stage<BM, BN, DT, AK, BKM, CHECKED>(acc, fc, fn, s0, s1, srcA, srcB, kt, nk, lane, wm, wn, wave);
        dma_stage<BM, BN, DT, AK, BKM, CHECKED>(acc, fc, fn, s1, s0, srcA, srcB, kt + 1, nk, lane, wm, wn, wave);
    }
    wait_vm<0>();
}

// Epilogue of one wave's 128 x 128 block of 16-bit results through LDS.  The
// values alpha * acc + beta * bias[col] are converted and written to `stage`
// (this wave's 32 KiB: row-major, 256 bytes per row, 16-byte chunk c of row r
// in slot c ^ (r % 16)), then read back as 16-byte lanes, 16 lanes per row,
// and stored to rowp(r) (the block row's first column; nullptr skips the row)
// so that every store instruction writes 4 whole 256-byte row segments
// (store(k, r, c, d): lane chunk c of row r, the k-th of the lane's 32 rows).
// BIAS: bias holds the block's 128 column values; otherwise no term is added
// (not even beta * 0).  The caller has synchronised the workgroup since the
// last read of `stage` as a K buffer.
template <int DT, bool BIAS, class StoreRow>
__device__ __forceinline__ void wave_epilogue_lds_f(const f32x16_t (&acc)[4][4], float alpha, const uint16_t* bias,
                                                    float beta, char* stage, int lane, StoreRow&& store) {
    constexpr int ROWB = 256, NCH = 16;
    const int h = lane >> 5;
    // the bias stays packed (two 16-bit values per register) until its column
    // block is converted
    u32x2_t craw[4][4];
    if constexpr (BIAS) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) craw[j][q] = *(const u32x2_t*)(bias + 32 * j + 8 * q + 4 * h);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float cb[4][4];
        if constexpr (BIAS) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cb[q][0] = beta * from_bits<DT>((uint16_t)craw[j][q].x);
                cb[q][1] = beta * from_bits<DT>((uint16_t)(craw[j][q].x >> 16));
                cb[q][2] = beta * from_bits<DT>((uint16_t)craw[j][q].y);
                cb[q][3] = beta * from_bits<DT>((uint16_t)(craw[j][q].y >> 16));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 32 * i + (lane & 31);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = BIAS ? alpha * acc[i][j][4 * q + e] + cb[q][e] : alpha * acc[i][j][4 * q + e];
                u32x2_t o;
                o.x = pack2<DT>(v[0], v[1]);
                o.y = pack2<DT>(v[2], v[3]);
                const int c = 4 * j + q;
                *(u32x2_t*)(stage + r * ROWB + ((c ^ (r % NCH)) << 4) + (h << 3)) = o;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const int r = 4 * k + (lane >> 4), c = lane & 15;
        const u32x4_t d = *(const u32x4_t*)(stage + r * ROWB + ((c ^ (r % NCH)) << 4));
        store(k, r, c, d);
    }
}
// ... storing row r to rowp(r) (its first column; nullptr skips the row)
template <int DT, bool BIAS, class RowPtr>
__device__ __forceinline__ void wave_epilogue_lds(const f32x16_t (&acc)[4][4], float alpha, const uint16_t* bias,
                                                  float beta, char* stage, int lane, RowPtr&& rowp) {
    wave_epilogue_lds_f<DT, BIAS>(acc, alpha, bias, beta, stage, lane, [&](int, int r, int c, const u32x4_t& d) {
        uint16_t* dst = rowp(r);
        if (dst) *(u32x4_t*)(dst + 8 * c) = d;
    });
}


// ---------------------------------------------------------------------------
// 16x16x32 form of the K loop.  Each wave's 128 x 128
// sub-tile is 8 x 8 MFMA tiles of 16 x 16; a 64-k stage is two k-blocks of 32,
// each 64 MFMAs.  Operand fragment of rows [mnb, mnb+16), k-block s: lane l
// gets mn = mnb + l%16, k = 32 s + 8 (l/16) + 0..7 (one swizzled chunk).
//
// The MFMAs are issued from inline assembly with the accumulator tied to its
// AGPRs: with 64 separate 4-register accumulators filling the AGPR file the
// compiler picks the untied MFMA form for some of them and then shuffles
// accumulators between register files every iteration (measured: ~150 move
// instructions per two stages and a 10 % slower kernel).  The compiler does
// not see inside the assembly, so the hazards it would guard are fenced by
// hand: the first k-block writes the accumulators with C = 0 instead of
// reading zeroed registers, and acc_fence (a few wait states, with every
// accumulator as an operand so that no read moves above it) separates the
// last MFMA from the first read of its result.
// Z: the first k-block, C = 0 (the accumulators are never zeroed by VALU
// writes, which an MFMA must not read too soon after).
template <int DT, bool Z>
__device__ __forceinline__ void mfma16_tied(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
    if constexpr (Z && DT == 0)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
    else if constexpr (Z)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
    else if constexpr (DT == 0)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int TM>
__device__ __forceinline__ void acc_fence(f32x4_t (&acc)[TM][8]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                     : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                       "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
}
template <int TM>
__device__ __forceinline__ void acc_fence(f32x4_t (&acc)[TM][4]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
}
template <int R, bool KMAJ>
__device__ __forceinline__ u32x4_t read_frag16(const char* lds, int mnb, int s, int lane) {
    if constexpr (KMAJ) {
        // 16 lanes on 16 consecutive rows of one chunk: 16 distinct bank quads
        const int r = lane & 15, c = 4 * s + (lane >> 4);
        return *(const u32x4_t*)(lds + (mnb + r) * 128 + ((c ^ kswz(r)) << 4));
    } else {
        // group g = l/16 takes k rows 32 s + 8 g + (0..3, then 4..7); lane i of a
        // group reads columns mnb + 4 (i%4) .. +3 of row i/4, and the transposing
        // read hands lane i column mnb + i of the group's 4 rows
        const int g = lane >> 4, i = lane & 15;
        const int krow = 32 * s + 8 * g + (i >> 2);
        const int n = mnb + 4 * (i & 3);
        const int off = mmaj16_off<R * 2>(krow, n * 2), off4 = mmaj16_off<R * 2>(krow + 4, n * 2);
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OMM_LDS(i16x4_t, lds + off));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OMM_LDS(i16x4_t, lds + off4));
        u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        return u32x4_t{l2.x, l2.y, h2.x, h2.y};
    }
}
template <int BM, int BN, bool AK, bool BKM>
struct Frags16 {
    static constexpr int TM = BM / 32, TN = BN / 32;
    u32x4_t a[TM], b[TN];
    template <int R>
    __device__ __forceinline__ void read_one(const char* st, int s, int lane, int wm, int wn) {
        constexpr int A_BYTES = BM * KSTEP * 2;
        if constexpr (R < TM)
            a[R] = read_frag16<BM, AK>(st, wm * (BM / 2) + 16 * R, s, lane);
        else
            b[R - TM] = read_frag16<BN, BKM>(st + A_BYTES, wn * (BN / 2) + 16 * (R - TM), s, lane);
    }
    __device__ __forceinline__ void read(const char* st, int s, int lane, int wm, int wn) {
        static_for<0, TM + TN>([&](auto rc) { read_one<decltype(rc)::value>(st, s, lane, wm, wn); });
    }
};

// One 32-k block of MFMAs on `cur`; the fragment reads of k-block s of `lds`
// into `nxt` and (D1 > D0) this wave's DMA instructions D0 .. D1-1 of stage kt
// into buffer X, each spread evenly over the MFMAs.
template <int DT, int TM, int TN, bool CHECKED, int D0, int D1, bool Z, class F, class SA, class SB>
__device__ __forceinline__ void kblock16(f32x4_t (&acc)[TM][TN], const F& cur, F& nxt, const char* lds, int s,
                                         char* X, int A_BYTES, const SA& srcA, const SB& srcB, int kt, bool live,
                                         int lane, int wm, int wn, int wave) {
    constexpr int NM = TM * TN, NR = TM + TN, ND = D1 - D0;
    constexpr int LA = SA::PER_WAVE;
    DmaCtx ca, cb;
    if constexpr (ND > 0) {
        ca = srcA.ctx(X, kt, live);
        cb = srcB.ctx(X + A_BYTES, kt, live);
    }
    static_for<0, NM>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        mfma16_tied<DT, Z>(acc[x / TN][x % TN], cur.b[x % TN], cur.a[x / TN]);
        if constexpr (ND > 0)
            static_for<D0 + (x * ND + NM - 1) / NM, D0 + ((x + 1) * ND + NM - 1) / NM>(
                [&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(srcA, srcB, ca, cb, kt, wave); });
        static_for<(x * NR + NM - 1) / NM, ((x + 1) * NR + NM - 1) / NM>([&](auto rc) {
            nxt.template read_one<frag_order(TM, TN, decltype(rc)::value)>(lds, s, lane, wm, wn);
        });
        fence_sched();
    });
}

// One stage: k-block 0 (reads of k-block 1 of X), the barrier that retires X
// and publishes Y (stage kt+1, whose DMA went out a whole k-block earlier),
// k-block 1 (reads of Y's k-block 0, stage kt+2's DMA into X).
template <int BM, int BN, int DT, bool CHECKED, bool Z, class SA, class SB, class F>
__device__ __forceinline__ void dma_stage16(f32x4_t (&acc)[BM / 32][BN / 32], F& fc, F& fn, char* X, char* Y,
                                            const SA& srcA, const SB& srcB, int kt, int nk, int lane, int wm, int wn,
                                            int wave) {
    constexpr int A_BYTES = BM * KSTEP * 2;
    constexpr int LD = SA::PER_WAVE + SB::PER_WAVE;
    constexpr int TM = BM / 32, TN = BN / 32;
    fence_sched();
    kblock16<DT, TM, TN, CHECKED, 0, 0, Z>(acc, fc, fn, X, 1, X, A_BYTES, srcA, srcB, kt, false, lane, wm, wn, wave);
    wait_vm<0>();
    __syncthreads();
    fence_sched();
    kblock16<DT, TM, TN, CHECKED, 0, LD, false>(acc, fn, fc, Y, 0, X, A_BYTES, srcA, srcB, kt + 2, kt + 2 < nk, lane, wm, wn,
                                         wave);
}

template <int BM, int BN, int DT, bool AK, bool BKM, bool CHECKED, class SA, class SB>
__device__ __forceinline__ void mainloop_dma16(f32x4_t (&acc)[BM / 32][BN / 32], char* __restrict__ s0,
                                               char* __restrict__ s1, const SA& srcA, const SB& srcB, int nk, int lane,
                                               int wm, int wn, int wave) {
    constexpr int A_BYTES = BM * KSTEP * 2;
    constexpr int LA = SA::PER_WAVE, LD = SA::PER_WAVE + SB::PER_WAVE;
    // nk >= 1: the first two stages run unconditionally
    {
        const DmaCtx a0 = srcA.ctx(s0, 0, true), b0 = srcB.ctx(s0 + A_BYTES, 0, true);
        static_for<0, LD>([&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(srcA, srcB, a0, b0, 0, wave); });
        const DmaCtx a1 = srcA.ctx(s1, 1, nk > 1), b1 = srcB.ctx(s1 + A_BYTES, 1, nk > 1);
        static_for<0, LD>([&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(srcA, srcB, a1, b1, 1, wave); });
    }
    wait_vm<LD>();
    __syncthreads();
    Frags16<BM, BN, AK, BKM> fc, fn;
    fc.read(s0, 0, lane, wm, wn);
    dma_stage16<BM, BN, DT, CHECKED, true>(acc, fc, fn, s0, s1, srcA, srcB, 0, nk, lane, wm, wn, wave);
    dma_stage16<BM, BN, DT, CHECKED, false>(acc, fc, fn, s1, s0, srcA, srcB, 1, nk, lane, wm, wn, wave);
    for (int kt = 2; kt < nk; kt += 2) {
        dma_stage16<BM, BN, DT, CHECKED, false>(acc, fc, fn, s0, s1, srcA, srcB, kt, nk, lane, wm, wn, wave);
        dma_stage16<BM, BN, DT, CHECKED, false>(acc, fc, fn, s1, s0, srcA, srcB, kt + 1, nk, lane, wm, wn, wave);
    }
    wait_vm<0>();
    acc_fence(acc);
}

// Epilogue of one wave's 16 TM x 128 block in the 16x16 accumulator layout
// (tile (i, j), register e of lane l: row 16 i + l%16, column 16 j + 4 (l/16) + e),
// through the same LDS staging and row-segment stores as wave_epilogue_lds_f
// (store(k, r, c, d): row r = 4 k + l/16 of the block, 16-byte chunk c).
template <int DT, bool BIAS, int TM, class StoreRow>
__device__ __forceinline__ void wave_epilogue_lds16(const f32x4_t (&acc)[TM][8], float alpha, const uint16_t* bias,
                                                    float beta, char* stage, int lane, StoreRow&& store) {
    constexpr int ROWB = 256, NCH = 16;
    const int g = lane >> 4, h = g & 1;
    u32x2_t craw[8];
    if constexpr (BIAS) {
#pragma unroll
        for (int j = 0; j < 8; ++j) craw[j] = *(const u32x2_t*)(bias + 16 * j + 4 * g);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float cb[4];
        if constexpr (BIAS) {
            cb[0] = beta * from_bits<DT>((uint16_t)craw[j].x);
            cb[1] = beta * from_bits<DT>((uint16_t)(craw[j].x >> 16));
            cb[2] = beta * from_bits<DT>((uint16_t)craw[j].y);
            cb[3] = beta * from_bits<DT>((uint16_t)(craw[j].y >> 16));
        }
        const int c = 2 * j + (g >> 1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = 16 * i + (lane & 15);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = BIAS ? alpha * acc[i][j][e] + cb[e] : alpha * acc[i][j][e];
            u32x2_t o;
            o.x = pack2<DT>(v[0], v[1]);
            o.y = pack2<DT>(v[2], v[3]);
            *(u32x2_t*)(stage + r * ROWB + ((c ^ (r % NCH)) << 4) + (h << 3)) = o;
        }
    }
#pragma unroll
    for (int k = 0; k < 4 * TM; ++k) {
        const int r = 4 * k + (lane >> 4), c = lane & 15;
        const u32x4_t d = *(const u32x4_t*)(stage + r * ROWB + ((c ^ (r % NCH)) << 4));
        store(k, r, c, d);
    }
}

}  // namespace core16
}  // namespace omm
