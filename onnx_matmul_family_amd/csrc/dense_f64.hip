// fp64 batched GEMM on gfx950 MFMA (v_mfma_f64_16x16x4f64).
//
// MatMul and Gemm (since version 13) allow double tensors; the semantics are
// those of the other types with double accumulation and a double epilogue
// (alpha and beta are the operator's float attributes, taken exactly).  Structure:
// any layout and extents, element loads with range checks, one 128x128
// output tile per workgroup of 4 waves (each wave 64x64 as 4x4 MFMA tiles of
// 16x16), K staged through two LDS buffers 16 values at a time with the next
// stage's loads in flight during the current stage's MFMAs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int T = 128;   // output tile edge (4 waves of 64 x 64)
constexpr int KS = 16;   // k per stage
constexpr int PAD = 130; // LDS row stride (doubles)
constexpr int NL = T * KS / 256;  // elements per thread per operand and stage

// Element loads of one operand's stage (KS x T values), the contiguous dim of
// the stored operand across consecutive threads; zeros outside the matrix.
__device__ __forceinline__ void f64_load(double (&r)[NL], const double* X, int64_t ld, bool kmajor, int64_t mn0,
                                         int64_t MN, int64_t k0, int64_t K, int t) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        int kk, mm;
        if (kmajor) { kk = t & 15; mm = (t >> 4) + 16 * i; }
        else { mm = t & 127; kk = (t >> 7) + 2 * i; }
        const int64_t m = mn0 + mm, k = k0 + kk;
        r[i] = (m < MN && k < K) ? (kmajor ? X[m * ld + k] : X[k * ld + m]) : 0.0;
    }
}
__device__ __forceinline__ void f64_store(double (*S)[PAD], const double (&r)[NL], bool kmajor, int t) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        int kk, mm;
        if (kmajor) { kk = t & 15; mm = (t >> 4) + 16 * i; }
        else { mm = t & 127; kk = (t >> 7) + 2 * i; }
        S[kk][mm] = r[i];
    }
}

__global__ __launch_bounds__(256) void dense_f64_kernel(DenseArgs p, int tiles_m, int tiles_n) {
    __shared__ double As[2][KS][PAD];
    __shared__ double Bs[2][KS][PAD];
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
    const bool ak = p.a_kmajor, bk = p.b_kmajor;

    f64x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};

    // stage k+1 is loaded into registers while stage k multiplies from LDS
    const int nk = (int)((K + KS - 1) / KS);
    double ra[NL], rb[NL];
    if (nk > 0) {
        f64_load(ra, A, p.lda, ak, m0, M, 0, K, t);
        f64_load(rb, B, p.ldb, bk, n0, N, 0, K, t);
        f64_store(As[0], ra, ak, t);
        f64_store(Bs[0], rb, bk, t);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            f64_load(ra, A, p.lda, ak, m0, M, (int64_t)(kt + 1) * KS, K, t);
            f64_load(rb, B, p.ldb, bk, n0, N, (int64_t)(kt + 1) * KS, K, t);
        }
        // lane l supplies A[m = l%16][k = l/16] and B[k = l/16][n = l%16]
#pragma unroll
        for (int kk = 0; kk < KS; kk += 4) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[buf][kk + (lane >> 4)][wm * 64 + 16 * i + (lane & 15)];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[buf][kk + (lane >> 4)][wn * 64 + 16 * j + (lane & 15)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            f64_store(As[buf ^ 1], ra, ak, t);
            f64_store(Bs[buf ^ 1], rb, bk, t);
        }
        __syncthreads();
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
    hipLaunchKernelGGL(dense_f64_kernel, dim3((unsigned)total), dim3(256), 0, s, a, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace omm
