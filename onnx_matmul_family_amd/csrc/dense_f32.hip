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
constexpr uint32_t OOB = 0x80000000u;  // buffer offset past the range: loads read 0, stores are dropped

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// AK / BK: A / B stored with k contiguous.  BUF: every operand of one batch
// entry spans < 2 GiB, so elements are read and written through buffer
// resources with 32-bit byte offsets, an out-of-range element taking an offset
// past the range (no branch per element); otherwise plain loads under range
// checks.
template <bool AK, bool BK, bool BUF>
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
    const __amdgpu_buffer_rsrc_t rA = rsrc(A), rB = rsrc(B), rY = rsrc(Y);

    // result register r of lane l: row 8(r/4) + 4(l/32) + r%4, column l%32
    const float* Cp = (const float*)p.C;
    const int64_t n = n0 + wn * 32 + (lane & 31);
    const int64_t mr = m0 + wm * 32 + 4 * (lane >> 5);  // + 8 (r/4) + r%4
    // rows of this lane's outputs inside the matrix: the r with 8 (r/4) + r%4 < mrows
    const int mrows = (int)max((int64_t)0, min(M - mr, (int64_t)32));
    const bool nok = n < N;
    float cv[16];
    if (Cp) {
        const __amdgpu_buffer_rsrc_t rC = rsrc(Cp);
        const uint32_t c0 = (uint32_t)((mr * p.c_sm + n * p.c_sn) * 4), cs = (uint32_t)(p.c_sm * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dm = 8 * (r >> 2) + (r & 3);
            if constexpr (BUF)
                cv[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      rC, (nok && dm < mrows) ? c0 + (uint32_t)dm * cs : OOB, 0, 0));
            else
                cv[r] = (nok && dm < mrows) ? Cp[(mr + dm) * p.c_sm + n * p.c_sn] : 0.0f;
        }
    }

    // Thread t's element i of a stage: the contiguous dim of the stored operand
    // runs across consecutive threads (t % 64), the other dim is t / 64 + 4 i.
    const int tc = t & 63, tr = t >> 6;
    float ra[NL], rb[NL];
    // one operand: stored (R, C) with row stride ld; this thread reads rows
    // r0 + 4 i (i < NL) of column c0; rlim = rows left from r0, cok = c0 inside
    auto load_op = [&](float (&reg)[NL], const float* X, __amdgpu_buffer_rsrc_t rx, int64_t r0, int64_t c0,
                       int64_t R, int64_t C, int64_t ld) {
        // rows left from r0, clamped to the stage (32-bit compares below)
        const int rlim = (int)max((int64_t)0, min(R - r0, (int64_t)KS));
        const bool cok = c0 < C;
        if constexpr (BUF) {
            const uint32_t base = (uint32_t)((r0 * ld + c0) * 4), step = (uint32_t)(16 * ld);
#pragma unroll
            for (int i = 0; i < NL; ++i)
                reg[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       rx, (cok && 4 * i < rlim) ? base + (uint32_t)i * step : OOB, 0, 0));
        } else {
#pragma unroll
            for (int i = 0; i < NL; ++i) reg[i] = (cok && 4 * i < rlim) ? X[(r0 + 4 * i) * ld + c0] : 0.0f;
        }
    };
    auto load = [&](int64_t k0) {
        if constexpr (AK) load_op(ra, A, rA, m0 + tr, k0 + tc, M, K, p.lda);
        else load_op(ra, A, rA, k0 + tr, m0 + tc, K, M, p.lda);
        if constexpr (BK) load_op(rb, B, rB, n0 + tr, k0 + tc, N, K, p.ldb);
        else load_op(rb, B, rB, k0 + tr, n0 + tc, K, N, p.ldb);
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (AK) As[tc][tr + 4 * i] = ra[i];
            else As[tr + 4 * i][tc] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (BK) Bs[tc][tr + 4 * i] = rb[i];
            else Bs[tr + 4 * i][tc] = rb[i];
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

    const uint32_t y0 = (uint32_t)((mr * p.ldy + n) * 4), ys = (uint32_t)(p.ldy * 4);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int dm = 8 * (r >> 2) + (r & 3);
        const bool ok = nok && dm < mrows;
        float v = p.alpha * acc[r];
        if (Cp) v += p.beta * cv[r];
        if constexpr (BUF)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rY, ok ? y0 + (uint32_t)dm * ys : OOB,
                                                  0, 0);
        else if (ok)
            Y[(mr + dm) * p.ldy + n] = v;
    }
}

template <bool AK, bool BK>
void launch_f32(const DenseArgs& a, bool buf, dim3 grid, int tiles_m, int tiles_n, hipStream_t s) {
    if (buf)
        hipLaunchKernelGGL((dense_f32_kernel<AK, BK, true>), grid, dim3(256), 0, s, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((dense_f32_kernel<AK, BK, false>), grid, dim3(256), 0, s, a, tiles_m, tiles_n);
}

}  // namespace

hipError_t launch_dense_f32(const DenseArgs& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + T - 1) / T, tiles_n = (a.N + T - 1) / T;
    const int64_t total = tiles_m * tiles_n * a.nb0 * a.nb1;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    // 32-bit byte offsets: every operand of one batch entry spans < 2 GiB
    const int64_t lim = (1LL << 31) / 4;
    const int64_t a_span = a.a_kmajor ? (a.M - 1) * a.lda + a.K : (a.K - 1) * a.lda + a.M;
    const int64_t b_span = a.b_kmajor ? (a.N - 1) * a.ldb + a.K : (a.K - 1) * a.ldb + a.N;
    const int64_t c_span = a.C ? (a.M - 1) * a.c_sm + (a.N - 1) * a.c_sn + 1 : 0;
    const bool buf = a_span < lim && b_span < lim && c_span < lim && (a.M - 1) * a.ldy + a.N < lim;
    log_choice("fp32 M=%lld N=%lld K=%lld batches=%lld: 64x64x64 tiles, 32x32x2 fp32 MFMA, %s, %lld workgroups",
               (long long)a.M, (long long)a.N, (long long)a.K, (long long)(a.nb0 * a.nb1),
               buf ? "buffer loads" : "element loads", (long long)total);
    const dim3 grid((unsigned)total);
    const int tm = (int)tiles_m, tn = (int)tiles_n;
    if (a.a_kmajor && a.b_kmajor) launch_f32<true, true>(a, buf, grid, tm, tn, s);
    else if (a.a_kmajor) launch_f32<true, false>(a, buf, grid, tm, tn, s);
    else if (a.b_kmajor) launch_f32<false, true>(a, buf, grid, tm, tn, s);
    else launch_f32<false, false>(a, buf, grid, tm, tn, s);
    return hipGetLastError();
}

}  // namespace omm
