// MFMA core shared by the bf16 / fp16 GEMM kernels (dense and grouped): the
// operand tile sources (global -> registers), the swizzled LDS tile stores,
// the MFMA fragment reads and the double-buffered K loop.
//
// Per workgroup of 256 threads = 4 waves on the CU's 4 SIMDs: output tile
// BM x BN (256x256 or 128x128), K consumed 64 values per stage, each wave owns
// a (BM/2) x (BN/2) sub-tile in fp32 accumulators (AGPRs at 256x256).
// Tiles go global -> registers (16-byte loads, coalesced along the contiguous
// dim) -> LDS, double-buffered with one barrier per stage; stage k+1's global
// loads are in flight while stage k's MFMAs run.  Operands with k contiguous
// sit in LDS as XOR-swizzled 128-byte rows read with ds_read_b128; operands
// with m/n contiguous are copied as they are (swizzled 32-byte granules) and
// read with the transposing ds_read_b64_tr_b16, so no register transpose.
#pragma once
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
        return *(const u32x4_t*)(lds + s * (R * 32) + mnb * 32 + kmaj_lane(lane));
    } else {
        const int g = lane >> 4, i = lane & 15;
        const int krow = 16 * s + 8 * (g >> 1) + (i >> 2);
        const int n = mnb + 16 * (g & 1) + 4 * (i & 3);
        const int off = mmaj16_off<R * 2>(krow, n * 2);
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OMM_LDS(i16x4_t, lds + off));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OMM_LDS(i16x4_t, lds + off + 4 * R * 2));
        u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        return u32x4_t{l2.x, l2.y, h2.x, h2.y};
    }
}

template <int BM, int BN, int DT, bool AK, bool BKM, int MODE, class SA, class SB>
__device__ __forceinline__ void mainloop(f32x16_t (&acc)[BM / 64][BN / 64], char* smem, const SA& srcA,
                                         const SB& srcB, int nk, int t, int lane, int wm, int wn) {
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int A_BYTES = BM * KSTEP * 2, B_BYTES = BN * KSTEP * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    u32x4_t ra[Chunks<BM, AK>::NC], rb[Chunks<BN, BKM>::NC];
    if (nk > 0) {
        srcA.template load<MODE>(ra, 0);
        srcB.template load<MODE>(rb, 0);
        store_tile<BM, AK>(smem, ra, t);
        store_tile<BN, BKM>(smem + A_BYTES, rb, t);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            srcA.template load<MODE>(ra, kt + 1);
            srcB.template load<MODE>(rb, kt + 1);
        }
        const char* sa = smem + buf * STAGE;
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
            char* so = smem + (buf ^ 1) * STAGE;
            store_tile<BM, AK>(so, ra, t);
            store_tile<BN, BKM>(so + A_BYTES, rb, t);
        }
        __syncthreads();
    }
}

}  // namespace core16
}  // namespace omm
