// QLinearMatMul (version 10) on gfx950: int8 MFMA with an exact int32
// accumulator and the fused requantisation -- v_mfma_i32_16x16x64_i8 on whole
// 256x256 tiles (qlinear16_kernel), v_mfma_i32_32x32x32_i8 on ragged or
// unaligned shapes (qlinear_kernel); at most 4 rows of a stream b on the
// vector ALU instead (qlinear_skinny_kernel).
//
// Per output element the operator asks for
//   acc = sum_k (a - za)(b - zb)                      (int32, wraps mod 2^32)
//   y   = saturate(rint(fp32(acc) * fp32(fp32(sa * sb) / sy)) + zy)
// a - za does not fit in int8, so the product runs on the raw bytes and the
// zero points enter through the expansion (exact mod 2^32)
//   acc = sum ab - zb * sum_k a[m,k] - za * sum_k b[k,n] + K * za * zb.
// The row sums of a and column sums of b come from the MFMA operand fragments
// already in registers, so no extra pass over memory: each dword of 4 signed
// bytes is biased to unsigned (xor 0x80) and summed with v_sad_u8 against
// zero, and the bias is taken off at the end; of the two waves that read a
// fragment, only one sums it.  (The v_dot4 instructions would do it in one
// step, but on gfx950 they hold up the MFMAs issued around them; v_sad_u8 and
// v_xor cost issue slots only.)  uint8 operands are mapped to int8 by flipping the top bit
// (a - 128) and their zero points shifted by 128, which leaves every a - za
// unchanged.  The requantisation uses IEEE fp32 multiply, correctly rounded
// division and round-half-even, in the order above, with no contraction.
//
// Tiles: 256x256 outputs per workgroup of 4 waves (128x128 each), K in stages
// of 128 bytes, double-buffered LDS.  a (k contiguous) is stored as swizzled
// 128-byte rows and read with ds_read_b128; b (n contiguous) is copied as is
// (swizzled 16-byte chunks) and read with the transposing ds_read_b64_tr_b8.
#include "gemm16_core.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

constexpr int NT = 256;
constexpr int BMQ = 256, BNQ = 256;
constexpr int KB = 128;                 // k (bytes) per stage
constexpr int A_BYTES = BMQ * KB;       // 32 KiB
constexpr int B_BYTES = BNQ * KB;       // 32 KiB
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int NC = 8;                   // 16-byte chunks per thread per operand per stage

// a: chunk i of thread t = row 8 (t >> 6) + (t & 7) + 32 i, k bytes 16 ((t >> 3) & 7) .. +15
// b: chunk i of thread t = k row (t >> 4) + 16 i, n bytes (t & 15) * 16 .. +15
template <bool KMAJ, bool U8>
struct QSrc {
    const uint8_t* p0;
    int64_t si, step;
    int64_t mn_first, k_first, MN, K;

    __device__ void init(const uint8_t* base, int64_t ld, int64_t mn0, int64_t MN_, int64_t K_, int t) {
        MN = MN_;
        K = K_;
        if constexpr (KMAJ) {
            mn_first = mn0 + ((t >> 6) << 3) + (t & 7);
            k_first = ((t >> 3) & 7) * 16;
            p0 = base + mn_first * ld + k_first;
            si = 32 * ld;
            step = KB;
        } else {
            k_first = t >> 4;
            mn_first = mn0 + (t & 15) * 16;
            p0 = base + k_first * ld + mn_first;
            si = 16 * ld;
            step = (int64_t)KB * ld;
        }
    }

    template <int MODE>
    __device__ __forceinline__ void load(u32x4_t (&reg)[NC], int kt) const {
        const uint8_t* p = p0 + (int64_t)kt * step;
        const int64_t k0 = k_first + (int64_t)kt * KB;
        const uint32_t flip = U8 ? 0x80808080u : 0u;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const uint8_t* q = p + i * si;
            const int64_t mn = KMAJ ? mn_first + 32 * i : mn_first;
            const int64_t k = KMAJ ? k0 : k0 + 16 * i;
            if constexpr (MODE == 0) {
                reg[i] = *(const u32x4_t*)q ^ flip;
            } else if constexpr (MODE == 1) {
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (mn < MN && k < K) v = *(const u32x4_t*)q ^ flip;
                reg[i] = v;
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const bool ok = KMAJ ? (mn < MN && k + e < K) : (k < K && mn + e < MN);
                    if (ok) w[e >> 2] |= (uint32_t)(q[e] ^ (U8 ? 0x80 : 0)) << (8 * (e & 3));
                }
                reg[i] = u32x4_t{w[0], w[1], w[2], w[3]};
            }
        }
    }
};

__device__ __forceinline__ void stash(char* s, const u32x4_t (&ra)[NC], const u32x4_t (&rb)[NC], int t) {
#pragma unroll
    for (int i = 0; i < NC; ++i)
        *(u32x4_t*)(s + kmaj_off<BMQ>(((t >> 6) << 3) + (t & 7) + 32 * i, (t >> 3) & 7)) = ra[i];
#pragma unroll
    for (int i = 0; i < NC; ++i) *(u32x4_t*)(s + A_BYTES + mmaj8_off<BNQ>((t >> 4) + 16 * i, (t & 15) * 16)) = rb[i];
}

__device__ __forceinline__ i32x4_t frag_a(const char* s, int rowb, int ks, int lane) {
    return *(const i32x4_t*)(s + rowb * 128 + kmaj_lane(lane, ks));
}
// lane l gets column colb + l%32, k = 32 ks + 16 (l/32) + 0..15
__device__ __forceinline__ i32x4_t frag_b(const char* s, int colb, int ks, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int krow = 32 * ks + 16 * (g >> 1) + (i >> 1);
    const int ncol = colb + 16 * (g & 1) + 8 * (i & 1);
    const int off = A_BYTES + mmaj8_off<BNQ>(krow, ncol);
    i32x2_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(OMM_LDS(i32x2_t, s + off));
    i32x2_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(OMM_LDS(i32x2_t, s + off + 8 * BNQ));
    return i32x4_t{lo.x, lo.y, hi.x, hi.y};
}

// acc + sum of the 4 bytes of v taken as int8, each biased by +128 (the bias,
// 128 per byte summed, is removed once after the K loop)
__device__ __forceinline__ int bytesum1(int v, int acc) {
    // plain C: for uint8 operands v comes out of the opaque flip below, so the
    // compiler cannot fold the two xors (and keep both copies of the fragment
    // live), and a known instruction needs no hazard padding before v_sad_u8
    const uint32_t u = (uint32_t)v ^ 0x80808080u;
    return (int)__builtin_amdgcn_sad_u8(u, 0u, (uint32_t)acc);
}
__device__ __forceinline__ int bytesum(i32x4_t v, int acc) {
    acc = bytesum1(v.x, acc);
    acc = bytesum1(v.y, acc);
    acc = bytesum1(v.z, acc);
    return bytesum1(v.w, acc);
}

template <bool AU8, bool BU8, int MODE>
__device__ __forceinline__ void qloop(i32x16_t (&acc)[4][4], int (&rs)[4], int (&cs)[4], char* smem,
                                      char* smem1, const QSrc<true, AU8>& sa, const QSrc<false, BU8>& sb, int nk, int t,
                                      int lane, int wm, int wn) {
    u32x4_t ra[NC], rb[NC];
    if (nk > 0) {
        sa.template load<MODE>(ra, 0);
        sb.template load<MODE>(rb, 0);
        stash(smem, ra, rb, t);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            sa.template load<MODE>(ra, kt + 1);
            sb.template load<MODE>(rb, kt + 1);
        }
        const char* s = buf ? smem1 : smem;
#pragma unroll
        for (int ks = 0; ks < KB / 32; ++ks) {
            i32x4_t af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = frag_a(s, wm * 128 + 32 * i, ks, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = frag_b(s, wn * 128 + 32 * j, ks, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) rs[i] = bytesum(af[i], rs[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) cs[j] = bytesum(bf[j], cs[j]);
        }
        if (kt + 1 < nk) stash(buf ? smem : smem1, ra, rb, t);
        __syncthreads();
    }
}

// uint8 -> int8 (a - 128) in place: the top bit of each byte flipped with the
// three-input bit operation (table 0x3c: src0 xor src1), which the compiler
// does not fold into the xor of a later byte sum, so one copy of each
// fragment stays live
__device__ __forceinline__ void flip(i32x4_t& v, uint32_t mask = 0x80808080u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (int)__builtin_amdgcn_bitop3_b32((uint32_t)v[e], mask, 0u, 0x3c);
}

// sum of the 4 bytes of v taken as uint8
__device__ __forceinline__ int bytesum_u8(int v, int acc) {
    return (int)__builtin_amdgcn_sad_u8((uint32_t)v, 0u, (uint32_t)acc);
}

// int8 MFMA operand fragments of one 32-value k-block, ids 0-3: a, 4-7: b.
// The DMA copies uint8 operands as they are; a uint8 fragment is flipped to
// int8 (flip_one) shortly before its first use, at least one MFMA ahead (b j
// is first used by MFMA j, a i by MFMA 4i): the fragments of MFMAs 0 and 1
// near the end of the k-block before, the others within their own k-block.
// Every fragment's read went out a k-block earlier, so no flip waits on LDS,
// and no MFMA waits on the flip of its operand.
template <bool AU8, bool BU8>
struct QFrags {
    static constexpr bool A_U8 = AU8;
    i32x4_t a[4], b[4];
    template <int R>
    __device__ __forceinline__ void read_one(const char* st, int ks, int lane, int wm, int wn) {
        if constexpr (R < 4)
            a[R] = frag_a(st, wm * 128 + 32 * R, ks, lane);
        else
            b[R - 4] = frag_b(st, wn * 128 + 32 * (R - 4), ks, lane);
    }
    template <int R>
    __device__ __forceinline__ void flip_one() {
        if constexpr (R < 4) {
            if constexpr (AU8) flip(a[R]);
        } else {
            if constexpr (BU8) flip(b[R - 4]);
        }
    }
    // the fragments MFMAs 0 and 1 of the k-block need
    __device__ __forceinline__ void flip_first() {
        flip_one<4>();
        flip_one<0>();
        flip_one<5>();
    }
    __device__ __forceinline__ void read(const char* st, int ks, int lane, int wm, int wn) {
        core16::static_for<0, 8>([&](auto rc) { read_one<decltype(rc)::value>(st, ks, lane, wm, wn); });
    }
};

// The fragment flipped right after MFMA x of its k-block, -1 if none (b 2, b 3,
// a 1, a 2, a 3; flip_first does b 0, a 0, b 1 near the end of the k-block
// before, after MFMA FLIP_FIRST_AT).
constexpr int flip_after(int x) { return x == 0 ? 6 : x == 1 ? 7 : x == 2 ? 1 : x == 6 ? 2 : x == 10 ? 3 : -1; }
constexpr int FLIP_FIRST_AT = 13;
// MFMA after which fragment f is flipped (-1: in the k-block before)
constexpr int flipped_after(int f) {
    for (int x = 0; x < 16; ++x)
        if (flip_after(x) == f) return x;
    return -1;
}
// MFMA X uses a-fragment X / 4 and b-fragment X % 4 (q_one): fragment f is
// first used by MFMA 4f (a) or f - 4 (b); every flip lands at least one MFMA
// before that, and every fragment is flipped exactly once.
constexpr bool flip_table_ok() {
    for (int f = 0; f < 8; ++f) {
        const int use = f < 4 ? 4 * f : f - 4;
        int n = 0;
        for (int x = 0; x < 16; ++x) n += flip_after(x) == f;
        const bool first = f == 4 || f == 0 || f == 5;
        if (n + (first ? 1 : 0) != 1) return false;
        if (!first && flipped_after(f) > use - 2) return false;
        if (first && use > 1) return false;
    }
    return FLIP_FIRST_AT < 15;
}
static_assert(flip_table_ok(), "each uint8 fragment is flipped once, at least one MFMA before its first use");

// MFMA X of a k-block (tile (X/4, X%4)) plus one dword of the byte sums.
// The two waves that read the same a-fragments (same wm) have different roles
// R = wm ^ wn, and so do the two that read the same b-fragments (same wn):
// a wave sums only a-fragments 2R, 2R+1 (during MFMAs 0-7) and b-fragments
// 2R, 2R+1 (MFMAs 8-15), so every fragment's bytes are summed once per
// workgroup, 16 dwords per wave and k-block.  A uint8 a-fragment not yet
// flipped is summed as it is; every other dword is int8 (raw or flipped) and
// is biased first.  Then the flip scheduled after MFMA X.
template <int X, int R, class F>
__device__ __forceinline__ void q_one(i32x16_t (&acc)[4][4], int (&rs)[4], int (&cs)[4], F& f) {
    acc[X / 4][X % 4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.b[X % 4], f.a[X / 4], acc[X / 4][X % 4], 0, 0, 0);
    constexpr int I = 2 * R + (X & 7) / 4;
    if constexpr (X < 8) {
        if constexpr (F::A_U8 && flipped_after(I) >= X)
            rs[I] = bytesum_u8(f.a[I][X % 4], rs[I]);
        else
            rs[I] = bytesum1(f.a[I][X % 4], rs[I]);
    } else {
        static_assert(X < 8 || flipped_after(4 + (2 * R + (X & 7) / 4)) < 8, "b-fragments are int8 when summed");
        cs[I] = bytesum1(f.b[I][X % 4], cs[I]);
    }
    if constexpr (flip_after(X) >= 0) f.template flip_one<flip_after(X)>();
}

template <int R, class F>
__device__ __forceinline__ void q_kblock(i32x16_t (&acc)[4][4], int (&rs)[4], int (&cs)[4], F& cur, F& nxt,
                                         const char* lds, int ks, int lane, int wm, int wn) {
    using namespace core16;
    static_for<0, 16>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        q_one<x, R>(acc, rs, cs, cur);
        if constexpr ((x & 1) == 0) nxt.template read_one<core16::frag_order(4, 4, x / 2)>(lds, ks, lane, wm, wn);
        if constexpr (x == FLIP_FIRST_AT) nxt.flip_first();
        fence_sched();
    });
}

// A k-block of MFMAs on `cur`, the reads of k-block ks of `lds` into `nxt`,
// and this wave's DMA instructions D0 .. D1-1 of stage kt (into buffer X)
// spread evenly between the MFMAs.
template <bool CHECKED, int R, int D0, int D1, class F, class SA, class SB>
__device__ __forceinline__ void q_kblock_dma(i32x16_t (&acc)[4][4], int (&rs)[4], int (&cs)[4], F& cur, F& nxt,
                                             const char* lds, int ks, char* X, const SA& sa, const SB& sb, int kt,
                                             bool live, int lane, int wm, int wn, int wave) {
    using namespace core16;
    constexpr int LA = SA::PER_WAVE, ND = D1 - D0;
    const DmaCtx ca = sa.ctx(X, kt, live), cb = sb.ctx(X + A_BYTES, kt, live);
    static_for<0, 16>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        q_one<x, R>(acc, rs, cs, cur);
        static_for<D0 + (x * ND + 15) / 16, D0 + ((x + 1) * ND + 15) / 16>(
            [&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(sa, sb, ca, cb, kt, wave); });
        if constexpr ((x & 1) == 0) nxt.template read_one<core16::frag_order(4, 4, x / 2)>(lds, ks, lane, wm, wn);
        if constexpr (x == FLIP_FIRST_AT) nxt.flip_first();
        fence_sched();
    });
}

// One stage of the DMA loop, on the schedule of the bf16 core: fragments one
// k-block ahead; the second half of stage kt+1's DMA (into Y) during k-block
// 0, the barrier after k-block 2, the first half of stage kt+2's DMA (into X)
// during k-block 3; no data-dependent branches.
template <bool CHECKED, int R, class SA, class SB, class F>
__device__ __forceinline__ void q_stage(i32x16_t (&acc)[4][4], int (&rs)[4], int (&cs)[4], F& fc, F& fn, char* X,
                                        char* Y, const SA& sa, const SB& sb, int kt, int nk, int lane, int wm, int wn,
                                        int wave) {
    using namespace core16;
    constexpr int LD = SA::PER_WAVE + SB::PER_WAVE, H = LD / 2;
    fence_sched();
    q_kblock_dma<CHECKED, R, H, LD>(acc, rs, cs, fc, fn, X, 1, Y, sa, sb, kt + 1, kt + 1 < nk, lane, wm, wn, wave);
    q_kblock<R>(acc, rs, cs, fn, fc, X, 2, lane, wm, wn);
    q_kblock<R>(acc, rs, cs, fc, fn, X, 3, lane, wm, wn);
    wait_vm<0>();
    __syncthreads();
    fence_sched();
    q_kblock_dma<CHECKED, R, 0, H>(acc, rs, cs, fn, fc, Y, 0, X, sa, sb, kt + 2, kt + 2 < nk, lane, wm, wn, wave);
}

// An odd stage count runs one more stage of zeros (no effect on the products;
// the sums count its bytes like any other).  On return no DMA is in flight and
// every wave is done with LDS.
template <bool AU8, bool BU8, bool CHECKED, int R, class SA, class SB>
__device__ __forceinline__ void qloop_dma(i32x16_t (&acc)[4][4], int (&rs)[4], int (&cs)[4], char* __restrict__ s0,
                                          char* __restrict__ s1, const SA& sa, const SB& sb, int nk, int lane, int wm,
                                          int wn, int wave) {
    using namespace core16;
    constexpr int LA = SA::PER_WAVE, LD = SA::PER_WAVE + SB::PER_WAVE, H = LD / 2;
    if (nk <= 0) return;
    {
        // stage 0 whole, the first half of stage 1
        const DmaCtx a0 = sa.ctx(s0, 0, true), b0 = sb.ctx(s0 + A_BYTES, 0, true);
        static_for<0, LD>([&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(sa, sb, a0, b0, 0, wave); });
        const DmaCtx a1 = sa.ctx(s1, 1, nk > 1), b1 = sb.ctx(s1 + A_BYTES, 1, nk > 1);
        static_for<0, H>([&](auto dc) { dma_one<CHECKED, LA, decltype(dc)::value>(sa, sb, a1, b1, 1, wave); });
    }
    wait_vm<H>();
    __syncthreads();
    QFrags<AU8, BU8> fc, fn;
    fc.read(s0, 0, lane, wm, wn);
    fc.flip_first();
    for (int kt = 0; kt < nk; kt += 2) {
        q_stage<CHECKED, R>(acc, rs, cs, fc, fn, s0, s1, sa, sb, kt, nk, lane, wm, wn, wave);
        q_stage<CHECKED, R>(acc, rs, cs, fc, fn, s1, s0, sa, sb, kt + 1, nk, lane, wm, wn, wave);
    }
    wait_vm<0>();
    __syncthreads();
}

__device__ __forceinline__ int ldzp(const void* p, int64_t i, bool u8) {
    return u8 ? (int)((const uint8_t*)p)[i] - 128 : (int)((const int8_t*)p)[i];
}

// Requantisation of the lane's 4 x 64 outputs.  Per element:
//   acc  = sum ab - zb * U[m] - za[m] * colsum[n]          (int32, mod 2^32)
//   mult = fp32(fp32(sa[m] * sb[n]) / sy)                   (correctly rounded divide)
//   y    = saturate(rint(fp32(acc) * mult) + zy)
// rint(.) + zy and the saturation run in fp32: the sum is exact below 2^24 and
// beyond it the result saturates either way, so this equals the integer add
// and clamp.  Per-column terms are read once per group of 4 columns and reused
// for the 4 row blocks.
template <bool SMALL, bool VEC>
__device__ __forceinline__ void q_epilogue(const QArgs& p, const i32x16_t (&acc)[4][4], uint8_t* __restrict__ y,
                                           const uint32_t* U, const int* ZA, const float* SA, const uint32_t* CB,
                                           const int* ZB, const float* SB, int64_t m0, int64_t n0, int lane, int wm,
                                           int wn, float sy, float zyf, float lo, float hi, bool vec_store) {
    const int64_t M = p.M, N = p.N;
    uint32_t Um[4];
    int za[4];
    float sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int mloc = wm * 128 + 32 * i + (lane & 31);
        Um[i] = U[mloc];
        za[i] = ZA[mloc];
        sa[i] = SA[mloc];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nloc = wn * 128 + 32 * j + 8 * q + 4 * (lane >> 5);
            const int64_t n = n0 + nloc;
            if (n >= N) continue;
            const u32x4_t cb = *(const u32x4_t*)(CB + nloc);
            const i32x4_t zb = *(const i32x4_t*)(ZB + nloc);
            const f32x4_t sb = *(const f32x4_t*)(SB + nloc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = m0 + wm * 128 + 32 * i + (lane & 31);
                if (m >= M) continue;
                uint32_t packed = 0;
                int outv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int32_t s32;
                    if constexpr (SMALL)  // exact 24-bit products, wrapping 32-bit sums
                        s32 = (int32_t)((uint32_t)acc[i][j][4 * q + e] - (uint32_t)__mul24(zb[e], (int)Um[i]) -
                                        (uint32_t)__mul24(za[i], (int)cb[e]));
                    else
                        s32 = (int32_t)((uint32_t)acc[i][j][4 * q + e] - (uint32_t)zb[e] * Um[i] -
                                        (uint32_t)za[i] * cb[e]);
                    const float prod = sa[i] * sb[e];
                    const float mult = prod / sy;
                    const float x = (float)s32 * mult;
                    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(x) + zyf, lo, hi);
                    const int qv = (int)r;
                    outv[e] = qv;
                    packed |= ((uint32_t)qv & 0xffu) << (8 * e);
                }
                uint8_t* yr = y + m * p.ldy + n;
                if (vec_store) {
                    *(uint32_t*)yr = packed;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) yr[e] = (uint8_t)outv[e];
                }
            }
        }
    }
}

// Requantisation of a tile that lies wholly inside y (K <= 32768, 4-byte
// aligned rows), without bounds checks.  Per element, with the per-row terms
// U, za, sa and per-column terms colsum, zb, sb of the tile in LDS:
//   acc  = sum ab - zb * U - za * colsum        (24-bit products, int32 wrap)
//   mult = fp32(fp32(sa * sb) / sy)
//   t    = (fp32(acc) * mult + 1.5*2^23) + zy, clamped to 1.5*2^23 + [lo, hi]
// MODE 0: register-staged loads, any shape.  MODE 1: DMA loads, ragged tiles
// handled in the loads and the epilogue.  (Whole tiles go to qlinear16_kernel.)
template <bool AU8, bool BU8, int MODE>
__global__ __launch_bounds__(NT) void qlinear_kernel(QArgs p, int tiles_m, int tiles_n) {
    constexpr bool VEC = MODE != 0;
    __shared__ __attribute__((aligned(1024))) char smem[STAGE];
    __shared__ __attribute__((aligned(1024))) char smem1[STAGE];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int T = tiles_m * tiles_n;
    const int w = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int z = w / T;
    int tm, tn;
    grouped_order(w - z * T, tiles_m, tiles_n, 4, tm, tn);
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const uint8_t* a = (const uint8_t*)p.a + z0 * p.a_bs0 + z1 * p.a_bs1;
    const uint8_t* b = (const uint8_t*)p.b + z0 * p.b_bs0 + z1 * p.b_bs1;
    uint8_t* y = (uint8_t*)p.y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const int64_t m0 = (int64_t)tm * BMQ, n0 = (int64_t)tn * BNQ;
    const int64_t M = p.M, N = p.N, K = p.K;

    i32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    int rs[4] = {0, 0, 0, 0}, cs[4] = {0, 0, 0, 0};

    const int nk = (int)((K + KB - 1) / KB);
    int nk_run;  // stages the loop ran: every lane summed 64 biased bytes per stage
    if constexpr (VEC) {
        core16::DmaSrc<BMQ, true, 1> sa;
        core16::DmaSrcMN8<BNQ> sb;
        sa.init(a, p.lda, m0, M, K, lane);
        sb.init(b, p.ldb, n0, N, K, lane);
        // the wave's role (which fragments it sums) is a template argument
        // so that the loop has no role-dependent branches
        auto run = [&](auto checked) {
            constexpr bool C = decltype(checked)::value;
            if ((wm ^ wn) == 0)
                qloop_dma<AU8, BU8, C, 0>(acc, rs, cs, smem, smem1, sa, sb, nk, lane, wm, wn, wave);
            else
                qloop_dma<AU8, BU8, C, 1>(acc, rs, cs, smem, smem1, sa, sb, nk, lane, wm, wn, wave);
        };
        if (m0 + BMQ <= M && n0 + BNQ <= N && K % KB == 0)
            run(std::false_type{});
        else
            run(std::true_type{});
        nk_run = nk > 0 ? (nk + 1) & ~1 : 0;
    } else {
        QSrc<true, AU8> sa;
        QSrc<false, BU8> sb;
        sa.init(a, p.lda, m0, M, K, t);
        sb.init(b, p.ldb, n0, N, K, t);
        qloop<AU8, BU8, 2>(acc, rs, cs, smem, smem1, sa, sb, nk, t, lane, wm, wn);
        nk_run = nk;
    }
    const uint32_t bias = 128u * 64u * (uint32_t)nk_run;

    // full row / column sums: lanes l and l^32 hold the two k-halves.  The
    // DMA loop sums fragments 2R, 2R+1 of each operand in the wave of role
    // R = wm ^ wn; the register loop sums every fragment in every wave.
    int* rowsum = (int*)smem;        // 256 tile rows
    int* colsum = (int*)smem + 256;  // 256 tile columns
    const int role = wm ^ wn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t r = (uint32_t)rs[i] - bias;
        const int rr = (int)(r + (uint32_t)__shfl_xor((int)r, 32));
        if ((VEC ? (i >> 1) == role : wn == 0) && lane < 32) rowsum[wm * 128 + 32 * i + lane] = rr;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t c = (uint32_t)cs[j] - bias;
        const int cc = (int)(c + (uint32_t)__shfl_xor((int)c, 32));
        if ((VEC ? (j >> 1) == role : wm == 0) && lane < 32) colsum[wn * 128 + 32 * j + lane] = cc;
    }
    __syncthreads();

    // Per-row terms U = rowsum - K*za, za, sa and per-column terms colsum, zb, sb,
    // one row and one column per thread, so that
    //   acc = sum ab - zb * U - za * colsum   (mod 2^32)
    uint32_t* U = (uint32_t*)smem + 512;
    int* ZA = (int*)smem + 768;
    float* SA = (float*)smem + 1024;
    uint32_t* CB = (uint32_t*)smem + 1280;
    int* ZB = (int*)smem + 1536;
    float* SB = (float*)smem + 1792;
    const uint32_t Ku = (uint32_t)K;
    // fp16 scales are exactly representable in fp32
    auto ldscale = [&](const void* q, int64_t i) {
        return p.scale_f16 ? from_bits<1>(((const uint16_t*)q)[i]) : ((const float*)q)[i];
    };
    const float sy = ldscale(p.y_scale, 0);
    // scales inside [2^-30, 2^30] (or zero) keep the fast division exact
    auto tame = [](float v) {
        const float av = __builtin_fabsf(v);
        return av == 0.0f || (av >= 0x1p-30f && av <= 0x1p30f);
    };
    int scales_ok;
    {
        const int64_t m = m0 + t, n = n0 + t;
        int za = 0, zb = 0;
        float sa = 0.0f, sb = 0.0f;
        if (m < M) {
            const int64_t apo = z0 * p.ap_bs0 + z1 * p.ap_bs1 + m * p.ap_sm;
            za = ldzp(p.a_zp, apo, AU8);
            sa = ldscale(p.a_scale, apo);
        }
        if (n < N) {
            const int64_t bpo = z0 * p.bp_bs0 + z1 * p.bp_bs1 + n * p.bp_sn;
            zb = ldzp(p.b_zp, bpo, BU8);
            sb = ldscale(p.b_scale, bpo);
        }
        U[t] = (uint32_t)rowsum[t] - Ku * (uint32_t)za;
        ZA[t] = za;
        SA[t] = sa;
        CB[t] = (uint32_t)colsum[t];
        ZB[t] = zb;
        SB[t] = sb;
        scales_ok = tame(sa) && tame(sb) && sy != 0.0f && tame(sy);
    }
    scales_ok = __syncthreads_and(scales_ok);

    const float zyf = (float)(p.y_u8 ? (int)((const uint8_t*)p.y_zp)[0] : (int)((const int8_t*)p.y_zp)[0]);
    const float lo = p.y_u8 ? 0.0f : -128.0f, hi = p.y_u8 ? 255.0f : 127.0f;
    const bool vec_store = VEC && (N % 4 == 0) && (p.ldy % 4 == 0);
    // |U| <= 256 K and |colsum| <= 128 K: below 2^23 for K <= 32768, where the
    // 24-bit multiply-adds are exact
    if (K <= 32768)
        q_epilogue<true, VEC>(p, acc, y, U, ZA, SA, CB, ZB, SB, m0, n0, lane, wm, wn, sy, zyf, lo, hi, vec_store);
    else
        q_epilogue<false, VEC>(p, acc, y, U, ZA, SA, CB, ZB, SB, m0, n0, lane, wm, wn, sy, zyf, lo, hi, vec_store);
}

// ---------------------------------------------------------------------------
// 16x16x64 form for whole tiles (v_mfma_i32_16x16x64_i8).  The
// same 256x256 tile and 4 waves, each wave's 128x128 block as 8 x 8 MFMA
// tiles of 16x16; a 128-byte stage is two k-blocks of 64, each 64 MFMAs, on
// the pipeline of the bf16 / fp16 16x16x32 loop (fragments one k-block ahead,
// the barrier between the two k-blocks, stage kt+2's DMA spread over the
// second).  On gfx950 the chip holds a higher shader clock under the 16x16
// MFMAs than under the 32x32 ones (measured on the bf16 loops).
//   a fragment (rows mnb .. mnb+15, k-block kb): lane l reads the 16 bytes of
//     row mnb + l%16 at k 64 kb + 16 (l/16) -- the bf16 read, byte for byte.
//   b fragment (columns nb .. nb+15): lane l holds column nb + l%16 at the same
//     16 k: two transposing 8-row reads, 16-lane group g on rows 64 kb + 16 g
//     (+ 0..7, + 8..15).  The two groups of a half-wave sit 16 rows apart, so
//     the b tile's 16-byte chunk c of row r lives at c ^ bswz(r), bswz(r) =
//     2 (r % 8) + (r / 16) % 2: rows 16 apart take chunks of opposite parity
//     and the half-wave touches every bank once.
// The MFMAs are tied inline assembly (the accumulators stay in their AGPRs,
// as in the bf16 loop).  int8 fragments come straight from LDS, so no VALU
// instruction writes one; uint8 fragments are flipped to int8 in their
// registers on a fixed schedule that keeps every flip at least three MFMAs
// ahead of the fragment's use (see the flip plan below).  The byte sums for
// the zero points are the 32x32 kernel's: each fragment is summed (v_xor +
// v_sad_u8) by one of the two waves that read it, one dword after every
// other MFMA, always after its flip.
namespace q16 {
using namespace core16;

constexpr int NF = 8;  // fragments per wave and operand per k-block

__device__ __forceinline__ int bswz(int r) { return ((r & 7) << 1) | ((r >> 4) & 1); }

// DMA of the n-contiguous b tile: 128 k rows x 256 bytes per stage.  Block b =
// rows 4b .. 4b+3 (one instruction, 1 KiB); lane p -> row 4b + p/16, physical
// chunk p%16, which takes logical chunk (p%16) ^ bswz(row).  A wave fills
// blocks 8 w + j; bswz of their rows depends on j only.
struct BDma {
    static constexpr int PER_WAVE = 8;
    const char* base;
    int64_t step;
    uint32_t ldb;
    uint32_t lane_off[PER_WAVE];

    __device__ void init(const void* b, int64_t ld, int64_t n0, int lane) {
        ldb = (uint32_t)ld;
        base = (const char*)b + n0;
        step = (int64_t)KB * ld;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int row = 4 * j + (lane >> 4);
            lane_off[j] = (uint32_t)(lane >> 4) * ldb + ((uint32_t)((lane & 15) ^ bswz(row)) << 4);
        }
    }
    __device__ __forceinline__ DmaCtx ctx(char* lds, int kt, bool live = true) const {
        return DmaCtx{make_rsrc(base + (live ? (int64_t)kt * step : 0), live), lds_addr(lds)};
    }
    template <bool CHECKED>
    __device__ __forceinline__ void one(const DmaCtx& c, int kt, int wave, int j) const {
        static_assert(!CHECKED, "whole tiles only");
        const int b = wave * PER_WAVE + j;
        dma16u(c.r, c.l0 + b * 1024, lane_off[j] + (uint32_t)(b * 4) * ldb);
    }
};

// U8: an operand may be uint8; ma / mb are 0x80808080 for a uint8 a / b and 0
// for int8 (a flip with mask 0 leaves the fragment as it is)
template <bool U8_>
struct Frags {
    static constexpr bool U8 = U8_;
    i32x4_t a[NF], b[NF];
    uint32_t ma, mb;
    // fragment R of k-block kb: R < 8 -> a[R], else b[R - 8]
    template <int R>
    __device__ __forceinline__ void read_one(const char* st, int kb, int lane, int wm, int wn) {
        if constexpr (R < NF) {
            a[R] = __builtin_bit_cast(i32x4_t, read_frag16<BMQ, true>(st, wm * 128 + 16 * R, kb, lane));
        } else {
            const int g = lane >> 4, i = lane & 15;
            const int krow = 64 * kb + 16 * g + (i >> 1);
            const int ncol = wn * 128 + 16 * (R - NF) + 8 * (i & 1);
            const int off = A_BYTES + krow * BNQ + ((((ncol >> 4) ^ bswz(krow))) << 4) + (ncol & 15);
            // rows krow + 8 share krow's swizzle (same r % 8, same 16-row half)
            const i32x2_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(OMM_LDS(i32x2_t, st + off));
            const i32x2_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(OMM_LDS(i32x2_t, st + off + 8 * BNQ));
            b[R - NF] = i32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
    }
    __device__ __forceinline__ void read(const char* st, int kb, int lane, int wm, int wn) {
        static_for<0, 2 * NF>([&](auto rc) { read_one<decltype(rc)::value>(st, kb, lane, wm, wn); });
    }
    // dword D of a uint8 fragment F (F < 8: a[F], else b[F - 8]) to int8 in place
    template <int F, int D>
    __device__ __forceinline__ void flip_dw() {
        if constexpr (F < NF)
            a[F][D] = (int)__builtin_amdgcn_bitop3_b32((uint32_t)a[F][D], ma, 0u, 0x3c);
        else
            b[F - NF][D] = (int)__builtin_amdgcn_bitop3_b32((uint32_t)b[F - NF][D], mb, 0u, 0x3c);
    }
};

template <bool Z>
__device__ __forceinline__ void mfma_i8(i32x4_t& acc, const i32x4_t& a, const i32x4_t& b) {
    if constexpr (Z)
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void acc_fence(i32x4_t (&acc)[NF][NF]) {
#pragma unroll
    for (int i = 0; i < NF; ++i)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                     : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                       "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
}

// Position of fragment f in the read order of a k-block (frag_order(8, 8, .)).
constexpr int read_pos(int f) {
    for (int r = 0; r < 2 * NF; ++r)
        if (frag_order(NF, NF, r) == f) return r;
    return -1;
}
// The d-th (0..31) dword a wave of role R sums in a k-block: its 8 fragments
// (a 4R .. 4R+3, b 4R .. 4R+3) in the order they were read, 4 dwords each.
// Returns fragment id (0..7 a, 8..15 b) * 4 + dword.
constexpr int sum_slot(int R, int d) {
    int ids[8] = {}, n = 0;
    for (int r = 0; r < 2 * NF; ++r) {
        const int f = frag_order(NF, NF, r);
        const int q = f < NF ? f : f - NF;
        if (q / 4 == R) ids[n++] = f;
    }
    return ids[d / 4] * 4 + d % 4;
}

// uint8 operands: the DMA copies the bytes as they are, and each fragment is
// mapped to int8 (x - 128: flip) in its registers, one dword after every MFMA
// (a wave64 VALU instruction holds the issue for 4 of the MFMA's 16 cycles, so
// more than a few between two MFMAs would delay the second).  Fragment r of
// the read order (read after MFMA 4r of the k-block before) is flipped there,
// after MFMAs 4r + 16 .. 4r + 19, for r < 12; the last four (a4 .. a7, first
// used by MFMAs 32 .. 56) in their own k-block, after MFMAs 0 .. 15.  An MFMA
// issued from inline assembly gets no wait states from the compiler after a
// VALU write of its sources: every flip lands at least three MFMAs ahead of
// the fragment's first use (MFMA x of a k-block uses a[x / 8] and b[x % 8]).
constexpr int first_use(int f) { return f < NF ? NF * f : f - NF; }
constexpr int NXT_FLIPS = 12;
// fragment * 4 + dword of `cur` / `nxt` flipped after MFMA x, -1 if none
constexpr int cur_flip(int x) { return x < 16 ? 4 * frag_order(NF, NF, NXT_FLIPS + x / 4) + x % 4 : -1; }
constexpr int nxt_flip(int x) { return x >= 16 ? 4 * frag_order(NF, NF, (x - 16) / 4) + x % 4 : -1; }
struct FlipPlan {
    int cur[NF * NF], nxt[NF * NF];
};
constexpr FlipPlan make_flip_plan() {
    FlipPlan p{};
    for (int x = 0; x < NF * NF; ++x) {
        p.cur[x] = cur_flip(x);
        p.nxt[x] = nxt_flip(x);
    }
    return p;
}
constexpr FlipPlan FLIPS = make_flip_plan();
constexpr bool flip_plan_ok() {
    int seen[2 * NF * 4] = {};
    int at[2 * NF * 4] = {};  // slot of the flip; nxt flips as slot - 64
    for (int x = 0; x < NF * NF; ++x) {
        if (FLIPS.cur[x] >= 0) {
            ++seen[FLIPS.cur[x]];
            at[FLIPS.cur[x]] = x;
        }
        if (FLIPS.nxt[x] >= 0) {
            const int fd = FLIPS.nxt[x];
            ++seen[fd];
            at[fd] = x - NF * NF;
            if (4 * read_pos(fd / 4) + 16 > x) return false;  // 16 MFMAs after the fragment's read
        }
    }
    for (int fd = 0; fd < 2 * NF * 4; ++fd) {
        if (seen[fd] != 1) return false;                      // every dword flipped once
        if (first_use(fd / 4) - at[fd] - 1 < 3) return false;  // >= 3 MFMAs before the first use
    }
    for (int R = 0; R < 2; ++R)
        for (int d = 0; d < 32; ++d)  // every byte sum (after MFMA 2d + 1) sees an int8 dword
            if (at[sum_slot(R, d)] >= 2 * d + 1) return false;
    return true;
}
static_assert(flip_plan_ok(), "uint8 flips: each dword once, >= 3 MFMAs ahead of its use, before its byte sum");

// One k-block: MFMA x on tile (x/8, x%8) of `cur`; the 16 fragment reads of
// k-block kb of `lds` into `nxt` and this wave's DMA instructions D0 .. D1-1
// of stage kt (into buffer X) spread evenly; one dword of byte sums after
// every other MFMA; then the uint8 flips scheduled after MFMA x.
template <int R, bool Z, int D0, int D1, class SA, class SB, class FR>
__device__ __forceinline__ void kblock(i32x4_t (&acc)[NF][NF], int (&rs)[4], int (&cs)[4], FR& cur, FR& nxt,
                                       const char* lds, int kb, char* X, const SA& sa, const SB& sb, int kt,
                                       bool live, int lane, int wm, int wn, int wave) {
    constexpr int NM = NF * NF, NR = 2 * NF, ND = D1 - D0, LA = SA::PER_WAVE;
    DmaCtx ca, cb;
    if constexpr (ND > 0) {
        ca = sa.ctx(X, kt, live);
        cb = sb.ctx(X + A_BYTES, kt, live);
    }
    static_for<0, NM>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        mfma_i8<Z>(acc[x / NF][x % NF], cur.b[x % NF], cur.a[x / NF]);
        if constexpr (ND > 0)
            static_for<D0 + (x * ND + NM - 1) / NM, D0 + ((x + 1) * ND + NM - 1) / NM>(
                [&](auto dc) { dma_one<false, LA, decltype(dc)::value>(sa, sb, ca, cb, kt, wave); });
        static_for<(x * NR + NM - 1) / NM, ((x + 1) * NR + NM - 1) / NM>([&](auto rc) {
            nxt.template read_one<frag_order(NF, NF, decltype(rc)::value)>(lds, kb, lane, wm, wn);
        });
        if constexpr (x % 2 == 1) {
            constexpr int slot = sum_slot(R, x / 2), f = slot / 4, w = slot % 4;
            if constexpr (f < NF)
                rs[f % 4] = bytesum1(cur.a[f][w], rs[f % 4]);
            else
                cs[(f - NF) % 4] = bytesum1(cur.b[f - NF][w], cs[(f - NF) % 4]);
        }
        if constexpr (FR::U8 && FLIPS.cur[x] >= 0) cur.template flip_dw<FLIPS.cur[x] / 4, FLIPS.cur[x] % 4>();
        if constexpr (FR::U8 && FLIPS.nxt[x] >= 0) nxt.template flip_dw<FLIPS.nxt[x] / 4, FLIPS.nxt[x] % 4>();
        fence_sched();
    });
}

template <int R, bool Z, class SA, class SB, class FR>
__device__ __forceinline__ void stage(i32x4_t (&acc)[NF][NF], int (&rs)[4], int (&cs)[4], FR& fc, FR& fn,
                                      char* X, char* Y, const SA& sa, const SB& sb, int kt, int nk, int lane, int wm,
                                      int wn, int wave) {
    constexpr int LD = SA::PER_WAVE + SB::PER_WAVE;
    fence_sched();
    kblock<R, Z, 0, 0>(acc, rs, cs, fc, fn, X, 1, X, sa, sb, kt, false, lane, wm, wn, wave);
    wait_vm<0>();     // this wave's DMA of stage kt+1 has landed
    __syncthreads();  // ... every wave's; every read of X is done
    fence_sched();
    kblock<R, false, 0, LD>(acc, rs, cs, fn, fc, Y, 0, X, sa, sb, kt + 2, kt + 2 < nk, lane, wm, wn, wave);
}

// nk >= 1 stages; an odd count runs one more stage of zeros.  On return no
// DMA is in flight and the accumulators are safe to read.
template <int R, bool U8, class SA, class SB>
__device__ __forceinline__ void loop(i32x4_t (&acc)[NF][NF], int (&rs)[4], int (&cs)[4], char* __restrict__ s0,
                                     char* __restrict__ s1, const SA& sa, const SB& sb, int nk, uint32_t ma,
                                     uint32_t mb, int lane, int wm, int wn, int wave) {
    constexpr int LA = SA::PER_WAVE, LD = SA::PER_WAVE + SB::PER_WAVE;
    {
        const DmaCtx a0 = sa.ctx(s0, 0, true), b0 = sb.ctx(s0 + A_BYTES, 0, true);
        static_for<0, LD>([&](auto dc) { dma_one<false, LA, decltype(dc)::value>(sa, sb, a0, b0, 0, wave); });
        const DmaCtx a1 = sa.ctx(s1, 1, nk > 1), b1 = sb.ctx(s1 + A_BYTES, 1, nk > 1);
        static_for<0, LD>([&](auto dc) { dma_one<false, LA, decltype(dc)::value>(sa, sb, a1, b1, 1, wave); });
    }
    wait_vm<LD>();
    __syncthreads();
    Frags<U8> fc, fn;
    fc.ma = fn.ma = ma;
    fc.mb = fn.mb = mb;
    fc.read(s0, 0, lane, wm, wn);
    if constexpr (U8) {
        // the fragments a k-block before would have flipped, flipped here; then
        // wait states before the first MFMA reads them
        static_for<0, NF * NF>([&](auto c) {
            constexpr int fd = FLIPS.nxt[decltype(c)::value];
            if constexpr (fd >= 0) fc.template flip_dw<fd / 4, fd % 4>();
        });
        fence_sched();
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
        fence_sched();
    }
    stage<R, true>(acc, rs, cs, fc, fn, s0, s1, sa, sb, 0, nk, lane, wm, wn, wave);
    stage<R, false>(acc, rs, cs, fc, fn, s1, s0, sa, sb, 1, nk, lane, wm, wn, wave);
    for (int kt = 2; kt < nk; kt += 2) {
        stage<R, false>(acc, rs, cs, fc, fn, s0, s1, sa, sb, kt, nk, lane, wm, wn, wave);
        stage<R, false>(acc, rs, cs, fc, fn, s1, s0, sa, sb, kt + 1, nk, lane, wm, wn, wave);
    }
    wait_vm<0>();
    acc_fence(acc);
}

// An accumulator register read where it is used (the register allocator
// would otherwise copy most of the AGPRs into VGPRs right after the K loop and
// run short of VGPRs for the epilogue).  The loop's closing fence provides the
// wait states between the last MFMA and these reads.
__device__ __forceinline__ int aread(int a) {
    int v;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// c + a * b on 24-bit signed operands, low 32 bits (v_mad_i32_i24; the
// compiler would otherwise issue two multiplies and a three-way add for two
// of these)
__device__ __forceinline__ int mad24(int a, int b, int c) {
    int r;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Requantisation of the wave's 128 x 128 block (lane l, tile (i, j), register
// e: row 16 i + l%16, column 16 j + 4 (l/16) + e) with the per-row / per-
// column terms in LDS; the arithmetic of q_epilogue.  Adding 1.5 * 2^23 (an
// even integer, where the fp32 spacing is 1) rounds the product to the
// nearest integer, ties to even, exactly like rint; adding the integer zy
// afterwards is exact; the clamp saturates, also for products too large for
// the trick; the result is the low byte of t's bits.  (zy is added after the
// rounding constant, not folded into it: x + (1.5 * 2^23 + zy) would break
// ties towards an even sum, which differs from rint(x) + zy for odd zy.)
// MARK: the division as q0 = prod * r, r = fp32(1 / sy) once, corrected by
// one fused step q0 + fma(-q0, sy, prod) * r, which is the correctly rounded
// quotient (Markstein) when nothing underflows or overflows; the caller takes
// this branch only when every scale of the tile and sy lie in [2^-30, 2^30]
// in magnitude (or are zero), which keeps every intermediate normal.  The
// bytes go through this wave's 16 KiB of `stage` (row r of 128 bytes, 16-byte
// chunk c in slot c ^ (r / 2 % 8)) and leave as whole 128-byte row segments.
// ZY0: y_zero_point is 0 (adding it is skipped; adding 0.0f is exact, so the
// result is the same either way).
template <bool MARK, bool ZY0>
__device__ __forceinline__ void epilogue(const QArgs& p, const i32x4_t (&acc)[NF][NF], uint8_t* __restrict__ y,
                                         const uint32_t* U, const int* ZA, const float* SA, const uint32_t* CB,
                                         const int* ZB, const float* SB, int64_t m0, int64_t n0, int lane, int wm,
                                         int wn, float sy, float zyf, float lo, float hi, char* stage) {
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    const float r = 1.0f / sy;
    const float tlo = MAGIC + lo, thi = MAGIC + hi;
    const int g = lane >> 4;
    int Um[NF], nza[NF];
    float sa[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int mloc = wm * 128 + 16 * i + (lane & 15);
        Um[i] = (int)U[mloc];
        nza[i] = -ZA[mloc];
        sa[i] = SA[mloc];
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        const int nloc = wn * 128 + 16 * j + 4 * g;
        const i32x4_t cb = *(const i32x4_t*)(CB + nloc);
        const i32x4_t zb = *(const i32x4_t*)(ZB + nloc);
        const f32x4_t sb = *(const f32x4_t*)(SB + nloc);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            uint32_t bytes[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // |U| <= 2^23, |colsum| <= 2^22, |z| <= 128: exact 24-bit products
                const int s32 = mad24(nza[i], cb[e], mad24(-zb[e], Um[i], aread(acc[i][j][e])));
                const float prod = sa[i] * sb[e];
                float mult;
                if constexpr (MARK) {
                    const float q0 = prod * r;
                    mult = __builtin_fmaf(__builtin_fmaf(-q0, sy, prod), r, q0);
                } else {
                    mult = prod / sy;
                }
                const float x = (float)s32 * mult;
                const float t = __builtin_amdgcn_fmed3f(ZY0 ? x + MAGIC : (x + MAGIC) + zyf, tlo, thi);
                bytes[e] = __float_as_uint(t);
            }
            const uint32_t lo2 = __builtin_amdgcn_perm(bytes[1], bytes[0], 0x0c0c0400u);
            const uint32_t hi2 = __builtin_amdgcn_perm(bytes[3], bytes[2], 0x0c0c0400u);
            const int row = 16 * i + (lane & 15);
            *(uint32_t*)(stage + row * 128 + ((j ^ ((row >> 1) & 7)) << 4) + 4 * g) = lo2 | (hi2 << 16);
            // two 16x16 tiles at a time: their eight outputs' chains interleave
            if (i % 2 == 1) fence_sched();
        }
    }
    uint8_t* __restrict__ yb = y + (m0 + wm * 128) * p.ldy + n0 + wn * 128;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int row = 8 * k + (lane >> 3), c = lane & 7;
        const u32x4_t d = *(const u32x4_t*)(stage + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
        *(u32x4_t*)(yb + (int64_t)row * p.ldy + 16 * c) = d;
    }
}

}  // namespace q16

// Everything after the set-up of qlinear16_kernel, for the waves of role R =
// wm ^ wn (which fragments a wave sums is a template argument, and the
// accumulators never meet a branch merge, which would copy all 256 of them).
template <int R, bool U8>
__device__ __forceinline__ void qlinear16_tile(const QArgs& p, char* smem, char* smem1, const uint8_t* a,
                                               const uint8_t* b, uint8_t* y, int64_t m0, int64_t n0, int za_t,
                                               int zb_t, float sa_t, float sb_t, float sy, float zyf, int t,
                                               int lane, int wave, int wm, int wn) {
    const int64_t M = p.M, K = p.K;
    i32x4_t acc[q16::NF][q16::NF];
    int rs[4] = {0, 0, 0, 0}, cs[4] = {0, 0, 0, 0};
    const int nk = (int)(K / KB);
    {
        core16::DmaSrc<BMQ, true, 1> sa;
        q16::BDma sb;
        sa.init(a, p.lda, m0, M, K, lane);
        sb.init(b, p.ldb, n0, lane);
        q16::loop<R, U8>(acc, rs, cs, smem, smem1, sa, sb, nk, p.a_u8 ? 0x80808080u : 0u,
                         p.b_u8 ? 0x80808080u : 0u, lane, wm, wn, wave);
    }
    // every lane summed 32 bytes (each +128) per stage into each of rs / cs
    const int nk_run = (nk + 1) & ~1;
    const uint32_t bias = 128u * 32u * (uint32_t)nk_run;
    __syncthreads();  // every wave is done with the K buffers

    // full row / column sums: the 4 lane groups hold 4 k-slices of each row /
    // column.  The wave of role R summed a fragments 4R .. 4R+3 and b
    // fragments 4R .. 4R+3.
    int* rowsum = (int*)smem;
    int* colsum = (int*)smem + 256;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t r = (uint32_t)rs[q] - bias;
        r += (uint32_t)__shfl_xor((int)r, 16);
        r += (uint32_t)__shfl_xor((int)r, 32);
        if (lane < 16) rowsum[wm * 128 + 16 * (4 * R + q) + lane] = (int)r;
        uint32_t c = (uint32_t)cs[q] - bias;
        c += (uint32_t)__shfl_xor((int)c, 16);
        c += (uint32_t)__shfl_xor((int)c, 32);
        if (lane < 16) colsum[wn * 128 + 16 * (4 * R + q) + lane] = (int)c;
    }
    __syncthreads();

    uint32_t* U = (uint32_t*)smem + 512;
    int* ZA = (int*)smem + 768;
    float* SA = (float*)smem + 1024;
    uint32_t* CB = (uint32_t*)smem + 1280;
    int* ZB = (int*)smem + 1536;
    float* SB = (float*)smem + 1792;
    auto tame = [](float v) {
        const float av = __builtin_fabsf(v);
        return av == 0.0f || (av >= 0x1p-30f && av <= 0x1p30f);
    };
    U[t] = (uint32_t)rowsum[t] - (uint32_t)K * (uint32_t)za_t;
    ZA[t] = za_t;
    SA[t] = sa_t;
    CB[t] = (uint32_t)colsum[t];
    ZB[t] = zb_t;
    SB[t] = sb_t;
    const int scales_ok = __syncthreads_and(tame(sa_t) && tame(sb_t) && sy != 0.0f && tame(sy));
    const float lo = p.y_u8 ? 0.0f : -128.0f, hi = p.y_u8 ? 255.0f : 127.0f;
    char* stg = smem1 + wave * (STAGE / 4);
    if (scales_ok && zyf == 0.0f)
        q16::epilogue<true, true>(p, acc, y, U, ZA, SA, CB, ZB, SB, m0, n0, lane, wm, wn, sy, zyf, lo, hi, stg);
    else if (scales_ok)
        q16::epilogue<true, false>(p, acc, y, U, ZA, SA, CB, ZB, SB, m0, n0, lane, wm, wn, sy, zyf, lo, hi, stg);
    else
        q16::epilogue<false, false>(p, acc, y, U, ZA, SA, CB, ZB, SB, m0, n0, lane, wm, wn, sy, zyf, lo, hi, stg);
}

// int8 / uint8 x int8 / uint8 -> int8 / uint8 on whole tiles (M, N multiples of
// 256, K a multiple of 128 up to 32768 -- of 256 with a uint8 operand, whose
// zero-padded stage would not flip to zero -- 16-byte aligned operands, checked
// on the host), the 16x16x64 loop.  A uint8 zero point enters as zp - 128.
template <bool U8>
__global__ __launch_bounds__(NT) void qlinear16_kernel(QArgs p, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) char smem[STAGE];
    __shared__ __attribute__((aligned(1024))) char smem1[STAGE];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int T = tiles_m * tiles_n;
    const int w = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int z = w / T;
    int tm, tn;
    grouped_order(w - z * T, tiles_m, tiles_n, 4, tm, tn);
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const uint8_t* a = (const uint8_t*)p.a + z0 * p.a_bs0 + z1 * p.a_bs1;
    const uint8_t* b = (const uint8_t*)p.b + z0 * p.b_bs0 + z1 * p.b_bs1;
    uint8_t* y = (uint8_t*)p.y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const int64_t m0 = (int64_t)tm * BMQ, n0 = (int64_t)tn * BNQ;

    // this thread's row (m0 + t) and column (n0 + t) parameters and the output
    // scale / zero point, loaded now so that their latency hides behind the K loop
    auto ldscale = [&](const void* q, int64_t i) {
        return p.scale_f16 ? from_bits<1>(((const uint16_t*)q)[i]) : ((const float*)q)[i];
    };
    const int64_t apo = z0 * p.ap_bs0 + z1 * p.ap_bs1 + (m0 + t) * p.ap_sm;
    const int64_t bpo = z0 * p.bp_bs0 + z1 * p.bp_bs1 + (n0 + t) * p.bp_sn;
    const int za_t = ldzp(p.a_zp, apo, U8 && p.a_u8), zb_t = ldzp(p.b_zp, bpo, U8 && p.b_u8);
    const float sa_t = ldscale(p.a_scale, apo), sb_t = ldscale(p.b_scale, bpo);
    const float sy = ldscale(p.y_scale, 0);
    const float zyf = (float)(p.y_u8 ? (int)((const uint8_t*)p.y_zp)[0] : (int)((const int8_t*)p.y_zp)[0]);
    if ((wm ^ wn) == 0)
        qlinear16_tile<0, U8>(p, smem, smem1, a, b, y, m0, n0, za_t, zb_t, sa_t, sb_t, sy, zyf, t, lane, wave, wm, wn);
    else
        qlinear16_tile<1, U8>(p, smem, smem1, a, b, y, m0, n0, za_t, zb_t, sa_t, sb_t, sy, zyf, t, lane, wave, wm, wn);
}

template <bool AU8, bool BU8, int MODE>
hipError_t launch_q(const QArgs& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + BMQ - 1) / BMQ, tiles_n = (a.N + BNQ - 1) / BNQ;
    const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qlinear_kernel<AU8, BU8, MODE>), dim3((unsigned)total), dim3(NT), 0, s, a, (int)tiles_m,
                       (int)tiles_n);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_q_types(const QArgs& a, hipStream_t s) {
    if (a.a_u8 && a.b_u8) return launch_q<true, true, MODE>(a, s);
    if (a.a_u8) return launch_q<true, false, MODE>(a, s);
    if (a.b_u8) return launch_q<false, true, MODE>(a, s);
    return launch_q<false, false, MODE>(a, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// Decode-like QLinearMatMul: at most 4 rows of a against b stored (K, N), one
// batch.  The whole cost is one read of b, so b is streamed once on the vector
// ALU instead of in 256x256 MFMA tiles (of which such a shape has a handful):
// a workgroup owns 16 columns; each lane of its NW waves reads the 16 bytes
// of one b row per step (64 rows per wave instruction, the waves on disjoint
// K ranges) and keeps, per column, the int32 sums of a[m,k] * b[k,n] over its
// rows (24-bit multiply-adds, exact) and of b[k,n] itself.  a is staged in LDS
// transposed to (K, MR) bytes and its row sums taken on the way.  Lanes and waves
// are then summed (integer, so the order does not matter) and the outputs
// requantised exactly as in q_epilogue, bytes taken as they are (uint8 as
// 0..255 with their own zero points: (a - za)(b - zb) is unchanged).
constexpr int QSK_NW = 8;
// steps of 64 rows per wave: K <= 8192 gives at most 16, all loaded at once
constexpr int QSK_STEPS = 16;

__device__ __forceinline__ u32x4_t qsk_load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

template <bool U8>
__device__ __forceinline__ int qsk_byte(uint32_t w, int e) {
    return U8 ? (int)((w >> (8 * e)) & 0xffu) : (int)(int8_t)(w >> (8 * e));
}

// Each phase waits for memory once: the lane's b rows (all its steps), its
// share of a, and, for the lanes that write an output, that output's
// parameters are all requested before the first wait.
template <int MR, bool AU8, bool BU8>
__global__ __launch_bounds__(64 * QSK_NW) void qlinear_skinny_kernel(QArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t At[];  // (K, MR) bytes
    __shared__ int red[QSK_NW][MR + 1][16];
    __shared__ int rowsum[MR];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint8_t* __restrict__ A = (const uint8_t*)p.a;
    // neighbouring column groups share b's 128-byte lines: keep them on one XCD
    const int64_t n0 = (int64_t)xcd_remap((int)blockIdx.x, (int)gridDim.x) * 16;

    // b: this wave's rows in steps of 64 (groups split as evenly as whole
    // groups allow); step i of the lane reads row kb + 64 i, below K for i < il
    const int64_t groups = (K + 63) / 64;
    const int g0 = (int)(groups * wave / QSK_NW), g1 = (int)(groups * (wave + 1) / QSK_NW);
    const int ns = g1 - g0;  // <= QSK_STEPS
    const int kb = 64 * g0 + lane, Ki = (int)K;
    const int il = kb >= Ki ? 0 : min(ns, (Ki - kb + 63) / 64);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.b), (short)0, 0x7fffffff,
                                                                        0x00020000);
    const uint32_t boff = (uint32_t)((int64_t)kb * p.ldb + n0), bstep = (uint32_t)(64 * p.ldb);
    u32x4_t v[QSK_STEPS];
#pragma unroll
    for (int i = 0; i < QSK_STEPS; ++i) v[i] = qsk_load(rb, i < il ? boff + bstep * (uint32_t)i : 0x80000000u);

    // a: 16-byte pieces (at most 4 per thread for K <= 8192); rows >= M are 0
    constexpr int QA = 4;
    const int kc = Ki / 16;
    u32x4_t va[QA];
#pragma unroll
    for (int u = 0; u < QA; ++u) {
        const int c = t + 64 * QSK_NW * u, m = c / kc, q = c - m * kc;
        va[u] = c < kc * MR && m < M ? *(const u32x4_t*)(A + m * p.lda + 16 * q) : u32x4_t{0u, 0u, 0u, 0u};
    }

    // the output parameters of lane (m, e) of wave 0
    const int om = lane >> 4, oe = lane & 15;
    const bool writer = wave == 0 && lane < 16 * MR && om < M && n0 + oe < N;
    int za = 0, zb = 0, zy = 0;
    float sa = 0.0f, sb = 0.0f, sy = 1.0f;
    if (writer) {
        auto ldscale = [&](const void* q, int64_t i) {
            return p.scale_f16 ? from_bits<1>(((const uint16_t*)q)[i]) : ((const float*)q)[i];
        };
        za = AU8 ? (int)((const uint8_t*)p.a_zp)[om * p.ap_sm] : (int)((const int8_t*)p.a_zp)[om * p.ap_sm];
        zb = BU8 ? (int)((const uint8_t*)p.b_zp)[(n0 + oe) * p.bp_sn]
                 : (int)((const int8_t*)p.b_zp)[(n0 + oe) * p.bp_sn];
        sa = ldscale(p.a_scale, om * p.ap_sm);
        sb = ldscale(p.b_scale, (n0 + oe) * p.bp_sn);
        sy = ldscale(p.y_scale, 0);
        zy = p.y_u8 ? (int)((const uint8_t*)p.y_zp)[0] : (int)((const int8_t*)p.y_zp)[0];
    }

    // a -> LDS transposed (K, MR), row sums from the same bytes
    if (t < MR) rowsum[t] = 0;
    __syncthreads();
    {
        int part[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) part[m] = 0;
#pragma unroll
        for (int u = 0; u < QA; ++u) {
            const int c = t + 64 * QSK_NW * u, m = c / kc, q = c - m * kc;
            if (c < kc * MR) {
                const uint32_t w[4] = {va[u].x, va[u].y, va[u].z, va[u].w};
                int sum = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    At[(16 * q + e) * MR + m] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
                    sum += qsk_byte<AU8>(w[e >> 2], e & 3);
                }
#pragma unroll
                for (int mm = 0; mm < MR; ++mm)
                    if (mm == m) part[mm] += sum;
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) part[m] += __shfl_xor(part[m], off);
            if (lane == 0) atomicAdd(&rowsum[m], part[m]);
        }
    }
    __syncthreads();

    // per column: sum over the lane's rows of a[m,k] b[k,n] (24-bit products,
    // exact) and of b[k,n]; rows past the range read as zero bytes
    int acc[MR][16], cs[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        cs[e] = 0;
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m][e] = 0;
    }
#pragma unroll
    for (int i = 0; i < QSK_STEPS; ++i) {
        if (i < ns) {
            const int k = min(kb + 64 * i, Ki - 1);
            int av[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) av[m] = qsk_byte<AU8>(At[k * MR + m], 0);
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int bv = qsk_byte<BU8>(w[e >> 2], e & 3);
                cs[e] += bv;
#pragma unroll
                for (int m = 0; m < MR; ++m) acc[m][e] = __mul24(av[m], bv) + acc[m][e];
            }
        }
    }
    // sum over the wave's lanes, then over the waves (integers: any order)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            cs[e] += __shfl_xor(cs[e], off);
#pragma unroll
            for (int m = 0; m < MR; ++m) acc[m][e] += __shfl_xor(acc[m][e], off);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            red[wave][MR][e] = cs[e];
#pragma unroll
            for (int m = 0; m < MR; ++m) red[wave][m][e] = acc[m][e];
        }
    }
    __syncthreads();
    if (!writer) return;
    int sab = 0, cb = 0;
#pragma unroll
    for (int w = 0; w < QSK_NW; ++w) {
        sab += red[w][om][oe];
        cb += red[w][MR][oe];
    }
    // requantised as in q_epilogue, with the bytes and zero points as stored:
    // sum (a - za)(b - zb) = sab - zb * (rowsum - K za) - za * cb   (mod 2^32)
    const uint32_t U = (uint32_t)rowsum[om] - (uint32_t)K * (uint32_t)za;
    const int32_t s32 = (int32_t)((uint32_t)sab - (uint32_t)zb * U - (uint32_t)za * (uint32_t)cb);
    const float prod = sa * sb;
    const float mult = prod / sy;
    const float x = (float)s32 * mult;
    const float lo = p.y_u8 ? 0.0f : -128.0f, hi = p.y_u8 ? 255.0f : 127.0f;
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(x) + (float)zy, lo, hi);
    ((uint8_t*)p.y)[om * p.ldy + n0 + oe] = (uint8_t)(int)r;
}

template <int MR>
hipError_t launch_qlinear_skinny(const QArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.N / 16)), block(64 * QSK_NW);
    const size_t lds = (size_t)a.K * MR;
    if (a.a_u8 && a.b_u8) hipLaunchKernelGGL((qlinear_skinny_kernel<MR, true, true>), grid, block, lds, s, a);
    else if (a.a_u8) hipLaunchKernelGGL((qlinear_skinny_kernel<MR, true, false>), grid, block, lds, s, a);
    else if (a.b_u8) hipLaunchKernelGGL((qlinear_skinny_kernel<MR, false, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((qlinear_skinny_kernel<MR, false, false>), grid, block, lds, s, a);
    return hipGetLastError();
}

hipError_t launch_qlinear(const QArgs& a, hipStream_t s) {
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    const bool vec = al16(a.a) && al16(a.b) && ((uintptr_t)a.y & 3) == 0 && a.lda % 16 == 0 && a.ldb % 16 == 0 &&
                     a.K % 16 == 0 && a.N % 16 == 0 && a.a_bs0 % 16 == 0 && a.a_bs1 % 16 == 0 &&
                     a.b_bs0 % 16 == 0 && a.b_bs1 % 16 == 0 && a.y_bs0 % 4 == 0 && a.y_bs1 % 4 == 0 &&
                     256 * a.lda < (1LL << 31) && 128 * a.ldb < (1LL << 31) &&
                     // the DMA path zero-pads a K tail and an odd stage count in LDS, and a
                     // flipped uint8 zero is not zero: uint8 needs an even number of full stages
                     (a.K % (2 * KB) == 0 || (!a.a_u8 && !a.b_u8));
    const bool full = vec && a.M % BMQ == 0 && a.N % BNQ == 0 && a.K % KB == 0 && a.K > 0 && a.K <= 32768 &&
                      a.ldy % 16 == 0 && ((uintptr_t)a.y & 15) == 0 && a.y_bs0 % 16 == 0 && a.y_bs1 % 16 == 0;
    // decode-like: at most 4 rows, one batch, a (K x 4 bytes) within 32 KB of
    // LDS; a and b read as 16-byte pieces (b in whole 16-column groups, with
    // 32-bit offsets)
    const bool skinny = al16(a.a) && al16(a.b) && a.lda % 16 == 0 && a.ldb % 16 == 0 && a.K % 16 == 0 &&
                        a.N % 16 == 0 && a.M <= 4 && a.nb0 * a.nb1 == 1 && a.K >= 256 && a.K <= 8192 &&
                        a.K * a.ldb < (1LL << 31) && a.N / 16 <= 0x7fffffff;
    log_choice("qlinear %s x %s -> %s M=%lld N=%lld K=%lld batches=%lld: %s", a.a_u8 ? "u8" : "i8",
               a.b_u8 ? "u8" : "i8", a.y_u8 ? "u8" : "i8", (long long)a.M, (long long)a.N, (long long)a.K,
               (long long)(a.nb0 * a.nb1),
               skinny ? "b streamed on the vector ALU, 16 columns per workgroup"
               : !vec ? "256x256x128 tiles, 32x32x32 MFMA, register-staged loads"
               : full ? "256x256x128 tiles, 16x16x64 MFMA, DMA, whole tiles"
                      : "256x256x128 tiles, 32x32x32 MFMA, DMA, ragged tiles");
    if (skinny) {
        if (a.M == 1) return launch_qlinear_skinny<1>(a, s);
        if (a.M == 2) return launch_qlinear_skinny<2>(a, s);
        return launch_qlinear_skinny<4>(a, s);
    }
    if (!vec) return launch_q_types<0>(a, s);
    if (full) {
        // (vec holds K % 256 == 0 when an operand is uint8)
        const int64_t tiles_m = a.M / BMQ, tiles_n = a.N / BNQ;
        const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1;
        if (total > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 grid((unsigned)total);
        if (a.a_u8 || a.b_u8)
            hipLaunchKernelGGL((qlinear16_kernel<true>), grid, dim3(NT), 0, s, a, (int)tiles_m, (int)tiles_n);
        else
            hipLaunchKernelGGL((qlinear16_kernel<false>), grid, dim3(NT), 0, s, a, (int)tiles_m, (int)tiles_n);
        return hipGetLastError();
    }
    return launch_q_types<1>(a, s);
}

}  // namespace omm
