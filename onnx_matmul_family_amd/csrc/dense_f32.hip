// fp32 batched GEMM on gfx950 MFMA (v_mfma_f32_32x32x2f32).
//
// Same operator semantics as the bf16/fp16 path (Gemm / MatMul, since version
// 13) for fp32 tensors.  fp32 problems in this library are small (the Gemm
// with transA = transB = 1 and a (1, N) bias takes one workgroup), so the
// kernel is built for latency: one 64x64 output tile per workgroup of 4 waves
// (one 32x32 MFMA tile each), any layout and extent (element loads with range
// checks), K staged through LDS 64 values at a time.  Every load of a stage is
// issued before the first of them is stored to LDS, the next stage's loads
// are in flight while the current stage multiplies, and the C values a lane
// needs are fetched at the start, so a K <= 64 product costs one round trip to
// memory for its operands.
#include "device_common.hpp"
#include "kernels.hpp"

namespace omm {

namespace {

constexpr int T = 64;   // output tile edge
constexpr int KS = 64;  // k per stage
constexpr int PAD = 65; // LDS row stride (floats): column writes hit distinct banks
constexpr int NL = T * KS / 256;  // elements per thread per operand and stage

__global__ __launch_bounds__(256) void dense_f32_kernel(DenseArgs p, int tiles_m, int tiles_n) {
    __shared__ float As[KS][PAD];
    __shared__ float Bs[KS][PAD];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles = tiles_m * tiles_n;
    const int w = blockIdx.x;
    const int z = w / tiles;
    const int tm = (w - z * tiles) / tiles_n, tn = (w - z * tiles) % tiles_n;
    const int64_t z0 = z / p.nb1, z1 = z - z0 * p.nb1;
    const float* A = (const float*)p.A + z0 * p.a_bs0 + z1 * p.a_bs1;
    const float* B = (const float*)p.B + z0 * p.b_bs0 + z1 * p.b_bs1;
    float* Y = (float*)p.Y + z0 * p.y_bs0 + z1 * p.y_bs1;
    const int64_t m0 = (int64_t)tm * T, n0 = (int64_t)tn * T;
    const int64_t M = p.M, N = p.N, K = p.K;

    // result register r of lane l: row 8(r/4) + 4(l/32) + r%4, column l%32
    const float* Cp = (const float*)p.C;
    const int64_t n = n0 + wn * 32 + (lane & 31);
    float cv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        cv[r] = (Cp && m < M && n < N) ? Cp[m * p.c_sm + n * p.c_sn] : 0.0f;
    }

    // Thread t's element i of a stage: the contiguous dim of the stored operand
    // runs across consecutive threads.
    float ra[NL], rb[NL];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            int kk, mm;
            if (p.a_kmajor) { kk = t & 63; mm = (t >> 6) + 4 * i; }
            else { mm = t & 63; kk = (t >> 6) + 4 * i; }
            const int64_t m = m0 + mm, k = k0 + kk;
            ra[i] = (m < M && k < K) ? (p.a_kmajor ? A[m * p.lda + k] : A[k * p.lda + m]) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            int kk, nn;
            if (p.b_kmajor) { kk = t & 63; nn = (t >> 6) + 4 * i; }
            else { nn = t & 63; kk = (t >> 6) + 4 * i; }
            const int64_t nb = n0 + nn, k = k0 + kk;
            rb[i] = (nb < N && k < K) ? (p.b_kmajor ? B[nb * p.ldb + k] : B[k * p.ldb + nb]) : 0.0f;
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (p.a_kmajor) As[t & 63][(t >> 6) + 4 * i] = ra[i];
            else As[(t >> 6) + 4 * i][t & 63] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (p.b_kmajor) Bs[t & 63][(t >> 6) + 4 * i] = rb[i];
            else Bs[(t >> 6) + 4 * i][t & 63] = rb[i];
        }
    };

    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    if (K > 0) load(0);
    for (int64_t k0 = 0; k0 < K; k0 += KS) {
        store();
        __syncthreads();
        if (k0 + KS < K) load(k0 + KS);
        // k-steps of 2 past K hold zeros: skip them (uniform across the workgroup)
        const int ksteps = (int)((min((int64_t)KS, K - k0) + 1) >> 1);
        for (int s2 = 0; s2 < ksteps; ++s2) {
            const int kk = 2 * s2;
            const float a = As[kk + (lane >> 5)][wm * 32 + (lane & 31)];
            const float b = Bs[kk + (lane >> 5)][wn * 32 + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }

    if (n >= N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M) {
            float v = p.alpha * acc[r];
            if (Cp) v += p.beta * cv[r];
            Y[m * p.ldy + n] = v;
        }
    }
}

}  // namespace

hipError_t launch_dense_f32(const DenseArgs& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + T - 1) / T, tiles_n = (a.N + T - 1) / T;
    const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    log_choice("fp32 M=%lld N=%lld K=%lld batches=%lld: 64x64x64 tiles, 32x32x2 fp32 MFMA, %lld workgroups",
               (long long)a.M, (long long)a.N, (long long)a.K, (long long)(a.nb0 * a.nb1), (long long)total);
    hipLaunchKernelGGL(dense_f32_kernel, dim3((unsigned)total), dim3(256), 0, s, a, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace omm
