// fp64 batched GEMM on gfx950 MFMA (v_mfma_f64_16x16x4f64).
//
// MatMul and Gemm (since version 13) allow double tensors; the semantics are
// those of the other types with double accumulation and a double epilogue
// (alpha and beta are the operator's float attributes, taken exactly).  Structure:
// any layout and extents, element loads with range checks, one 128x128
// output tile per workgroup of 4 waves (each wave 64x64 as 4x4 MFMA tiles of
// 16x16), K staged through three LDS buffers 16 values at a time.  Stage k+2
// is loaded into registers while stage k multiplies and stored to LDS at the
// end of stage k (into the buffer stage k-1 left), so stage k+1 has been in
// LDS for a whole stage when it starts: its first fragments are read before
// the stage barrier and the MFMAs run across it.  Within a stage the fragments
// of the next 4-deep k step are read while the current one multiplies.
#include "device_common.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int T = 128;   // output tile edge (4 waves of 64 x 64)
constexpr int KS = 16;   // k per stage
constexpr int NB = 3;    // LDS stage buffers
constexpr int NL = T * KS / 256;  // elements per thread per operand and stage

// LDS stage tile of one operand.  M/N-major operands keep k rows of T values
// (row stride 130 doubles); k-major operands keep m/n rows of KS values (row
// stride 18 doubles = 144 bytes), so that the 16 lanes that read one k of 16
// consecutive rows hit 16 different bank pairs and the next k's 16 lanes the
// pairs beside them: no bank conflicts on fragment reads, and the 16 lanes
// that store one row write 128 contiguous bytes.
template <bool KM>
struct F64Tile {
    static constexpr int ELEMS = KM ? T * 18 : KS * 130;
    __device__ static int off(int k, int mn) { return KM ? mn * 18 + k : k * 130 + mn; }
};

// One operand's element loads: thread t owns NL elements of each stage (the
// contiguous dim of the stored operand across consecutive threads); zeros
// outside the matrix.  Addresses advance by a fixed step per stage.
template <bool KM>
struct F64Src {
    const double* p;   // element 0 of this thread at stage 0
    int64_t si;        // distance between the thread's elements
    int64_t step;      // advance per stage
    int64_t mn_first, k_first, MN, K;
    __device__ void init(const double* X, int64_t ld, int64_t mn0, int64_t MN_, int64_t K_, int t) {
        MN = MN_;
        K = K_;
        if (KM) {  // element i: k = t % 16, m/n = t / 16 + 16 i
            k_first = t & 15;
            mn_first = mn0 + (t >> 4);
            p = X + mn_first * ld + k_first;
            si = 16 * ld;
            step = KS;
        } else {   // element i: m/n = t % 128, k = t / 128 + 2 i
            k_first = t >> 7;
            mn_first = mn0 + (t & 127);
            p = X + k_first * ld + mn_first;
            si = 2 * ld;
            step = KS * ld;
        }
    }
    __device__ __forceinline__ void load(double (&r)[NL], int kt) const {
        const double* q = p + kt * step;
        const int64_t k0 = k_first + (int64_t)kt * KS;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int64_t m = KM ? mn_first + 16 * i : mn_first;
            const int64_t k = KM ? k0 : k0 + 2 * i;
            r[i] = (m < MN && k < K) ? q[i * si] : 0.0;
        }
    }
    __device__ __forceinline__ void store(double* S, const double (&r)[NL], int t) const {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int kk = KM ? (t & 15) : (t >> 7) + 2 * i;
            const int mm = KM ? (t >> 4) + 16 * i : (t & 127);
            S[F64Tile<KM>::off(kk, mm)] = r[i];
        }
    }
};

// lane l supplies A[m = l%16][k = l/16] and B[k = l/16][n = l%16] of a 4-deep k step
template <bool AK, bool BK>
struct F64Frags {
    double a[4], b[4];
    __device__ __forceinline__ void read(const double* As, const double* Bs, int kk, int lane, int wm, int wn) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[F64Tile<AK>::off(kk + (lane >> 4), wm * 64 + 16 * i + (lane & 15))];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[F64Tile<BK>::off(kk + (lane >> 4), wn * 64 + 16 * j + (lane & 15))];
    }
};

template <class F>
__device__ __forceinline__ void f64_mma(f64x4_t (&acc)[4][4], const F& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

template <bool AK, bool BK>
__global__ __launch_bounds__(256) void dense_f64_kernel(DenseArgs p, int tiles_m, int tiles_n) {
    constexpr int EA = F64Tile<AK>::ELEMS, EB = F64Tile<BK>::ELEMS;
    __shared__ double As[NB * EA];
    __shared__ double Bs[NB * EB];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles = tiles_m * tiles_n;
    const int w = blockIdx.x;
    const int z = w / tiles;
    const int tm = (w - z * tiles) / tiles_n, tn = (w - z * tiles) % tiles_n;
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const double* A = (const double*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1;
    const double* B = (const double*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1;
    double* Y = (double*)p.Y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const int64_t m0 = (int64_t)tm * T, n0 = (int64_t)tn * T;
    const int64_t M = p.M, N = p.N, K = p.K;

    f64x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};

    const int nk = (int)((K + KS - 1) / KS);
    F64Src<AK> sa;
    F64Src<BK> sb;
    sa.init(A, p.lda, m0, M, K, t);
    sb.init(B, p.ldb, n0, N, K, t);
    double ra[NL], rb[NL];
    // stages 0 and 1 into buffers 0 and 1
    for (int s = 0; s < 2 && s < nk; ++s) {
        sa.load(ra, s);
        sb.load(rb, s);
        sa.store(As + s * EA, ra, t);
        sb.store(Bs + s * EB, rb, t);
    }
    __syncthreads();
    F64Frags<AK, BK> fc, fn;
    if (nk > 0) fc.read(As, Bs, 0, lane, wm, wn);
    int b0 = 0;  // buffer of stage kt
    for (int kt = 0; kt < nk; ++kt) {
        const int b1 = b0 == NB - 1 ? 0 : b0 + 1, b2 = b1 == NB - 1 ? 0 : b1 + 1;
        const bool more = kt + 2 < nk;
        if (more) {
            sa.load(ra, kt + 2);
            sb.load(rb, kt + 2);
        }
        const double* Ac = As + b0 * EA;
        const double* Bc = Bs + b0 * EB;
        fn.read(Ac, Bc, 4, lane, wm, wn);
        f64_mma(acc, fc);
        fc.read(Ac, Bc, 8, lane, wm, wn);
        f64_mma(acc, fn);
        fn.read(Ac, Bc, 12, lane, wm, wn);
        f64_mma(acc, fc);
        // stage kt+1 has been in LDS since the last barrier (junk past the last stage, unused)
        fc.read(As + b1 * EA, Bs + b1 * EB, 0, lane, wm, wn);
        f64_mma(acc, fn);
        if (more) {
            // the buffer stage kt-1 used: every wave finished reading it before the last barrier
            sa.store(As + b2 * EA, ra, t);
            sb.store(Bs + b2 * EB, rb, t);
        }
        __syncthreads();
        b0 = b1;
    }
    // result register r of lane l in a 16x16 tile: row l/16 + 4 r, column l%16
    const double* Cp = (const double*)p.C;
    const double alpha = (double)p.alpha, beta = (double)p.beta;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + 16 * i + (lane >> 4) + 4 * r;
                if (m < M) {
                    double v = alpha * acc[i][j][r];
                    if (Cp) v += beta * Cp[m * p.c_sm + n * p.c_sn];
                    Y[m * p.ldy + n] = v;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_dense_f64(const DenseArgs& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + T - 1) / T, tiles_n = (a.N + T - 1) / T;
    const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)total);
    log_choice("fp64 M=%lld N=%lld K=%lld batches=%lld: 128x128x16 tiles, 16x16x4 fp64 MFMA, %lld workgroups",
               (long long)a.M, (long long)a.N, (long long)a.K, (long long)(a.nb0 * a.nb1), (long long)total);
    if (a.a_kmajor && a.b_kmajor)
        hipLaunchKernelGGL((dense_f64_kernel<true, true>), grid, dim3(256), 0, s, a, (int)tiles_m, (int)tiles_n);
    else if (a.a_kmajor)
        hipLaunchKernelGGL((dense_f64_kernel<true, false>), grid, dim3(256), 0, s, a, (int)tiles_m, (int)tiles_n);
    else if (a.b_kmajor)
        hipLaunchKernelGGL((dense_f64_kernel<false, true>), grid, dim3(256), 0, s, a, (int)tiles_m, (int)tiles_n);
    else
        hipLaunchKernelGGL((dense_f64_kernel<false, false>), grid, dim3(256), 0, s, a, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace omm
