// fp64 batched GEMM on gfx950 MFMA (v_mfma_f64_16x16x4f64).
//
// MatMul and Gemm (since version 13) allow double tensors; the semantics are
// those of the other types with double accumulation and a double epilogue
// (alpha and beta are the operator's float attributes, taken exactly).  Same
// structure as the fp32 kernel: any layout and extents, element loads with
// range checks, one 64x64 output tile per workgroup of 4 waves (each wave
// 32x32 as 2x2 MFMA tiles of 16x16), K staged through LDS 16 values at a time.
#include "device_common.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int T = 64;    // output tile edge
constexpr int KS = 16;   // k per stage
constexpr int PAD = 65;  // LDS row stride (doubles)

__global__ __launch_bounds__(256) void dense_f64_kernel(DenseArgs p, int tiles_m, int tiles_n) {
    __shared__ double As[KS][PAD];
    __shared__ double Bs[KS][PAD];
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

    f64x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};

    for (int64_t k0 = 0; k0 < K; k0 += KS) {
        // 16 x 64 elements per operand, 4 per thread; the contiguous dim of
        // the stored operand runs across consecutive threads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int kk, mm;
            if (p.a_kmajor) { kk = t & 15; mm = (t >> 4) + 16 * i; }
            else { mm = t & 63; kk = (t >> 6) + 4 * i; }
            const int64_t m = m0 + mm, k = k0 + kk;
            double v = 0.0;
            if (m < M && k < K) v = p.a_kmajor ? A[m * p.lda + k] : A[k * p.lda + m];
            As[kk][mm] = v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int kk, nn;
            if (p.b_kmajor) { kk = t & 15; nn = (t >> 4) + 16 * i; }
            else { nn = t & 63; kk = (t >> 6) + 4 * i; }
            const int64_t n = n0 + nn, k = k0 + kk;
            double v = 0.0;
            if (n < N && k < K) v = p.b_kmajor ? B[n * p.ldb + k] : B[k * p.ldb + n];
            Bs[kk][nn] = v;
        }
        __syncthreads();
        // lane l supplies A[m = l%16][k = l/16] and B[k = l/16][n = l%16]
#pragma unroll
        for (int kk = 0; kk < KS; kk += 4) {
            double a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = As[kk + (lane >> 4)][wm * 32 + 16 * i + (lane & 15)];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = Bs[kk + (lane >> 4)][wn * 32 + 16 * j + (lane & 15)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // result register r of lane l in a 16x16 tile: row l/16 + 4 r, column l%16
    const double* Cp = (const double*)p.C;
    const double alpha = (double)p.alpha, beta = (double)p.beta;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 32 + 16 * j + (lane & 15);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 32 + 16 * i + (lane >> 4) + 4 * r;
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
