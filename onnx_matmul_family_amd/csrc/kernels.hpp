// Kernel argument blocks and launcher entry points (host side of the kernels).
// The launchers only enqueue work; shape validation happens in api.cpp before
// any of them is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace omm {

// A batched product Y[z] = op(A[z]) x op(B[z]) with up to two batch levels:
// batch z in [0, nb0*nb1) has z0 = z / nb1, z1 = z % nb1 and element offsets
// z0*bs0 + z1*bs1 per operand.  Layout flags say which dim is contiguous.
struct DenseArgs {
    const void* A;
    const void* B;
    void* Y;
    const void* C;         // Gemm C (nullptr = none)
    int64_t M, N, K;
    int64_t lda, ldb, ldy;  // row strides (elements) of A, B, Y as stored
    int64_t a_bs0, a_bs1, b_bs0, b_bs1, y_bs0, y_bs1;
    int64_t nb0, nb1;
    int64_t c_sm, c_sn;     // C element strides along m and n (0 = broadcast)
    float alpha, beta;
    int a_kmajor;           // 1: A stored (M,K) with k contiguous; 0: stored (K,M)
    int b_kmajor;           // 1: B stored (N,K) with k contiguous; 0: stored (K,N)
    // split-K (set by the launcher): partial products of K range
    // [s*kchunk, (s+1)*kchunk) go to ws[s][batch][M][N] (fp32)
    float* ws;
    int64_t kchunk;
    int splits;
};

// Quantised product.  Parameter offsets follow the same two batch levels plus
// an m (row side) or n (column side) stride of 0 or 1.
struct QArgs {
    const void* a;
    const void* b;
    void* y;
    const void* a_scale;   // fp32, or fp16 when scale_f16 (all three scales alike)
    const void* a_zp;
    const void* b_scale;
    const void* b_zp;
    const void* y_scale;
    const void* y_zp;
    int64_t M, N, K;
    int64_t lda, ldb, ldy;
    int64_t a_bs0, a_bs1, b_bs0, b_bs1, y_bs0, y_bs1;
    int64_t ap_bs0, ap_bs1, bp_bs0, bp_bs1;  // parameter batch strides
    int64_t ap_sm, bp_sn;                    // parameter stride along m / n
    int64_t nb0, nb1;
    int a_u8, b_u8, y_u8;                    // 1 = uint8
    int scale_f16;                           // 1 = the scales are fp16 (upcast exactly)
};

struct GroupedArgs {
    const void* input;      // (M, K)
    const void* weights;    // (G, K, N)
    const void* idx;        // (M, S) int32 or int64
    const void* bias;       // (G, N) or nullptr
    void* output;           // (M, S, N)
    int64_t M, K, N, G, S;
    int idx64;
    // weight-only quantised weights (launch_grouped_dq): weights are int8 /
    // uint8 q (G, K, N), w = T((q - zp) * scale) per block of bs k and column
    const void* wscale;  // (G, nkb, N) of T
    const void* wzp;     // (G, nkb, N) of q's type, or nullptr (zero)
    int64_t bs, nkb;
    int q_kind;          // 1 = int8, 2 = uint8
};

// Device memory a caller lends a launch for split-K partial products.
struct DenseScratch {
    void* ptr;
    size_t bytes;
};

// Host-side diagnostics and tuning, read from the environment once per process:
//   OMM_LOG=1          every launch prints its kernel choice to stderr
//   OMM_TILE=MxNxK     bf16 / fp16 MatMul / Gemm: force the 256x256x64 or the
//                      128x128x64 tile path (bench sweeps; honoured where the
//                      16-byte-load path applies, ignored otherwise)
bool log_enabled();
void log_choice(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
int tile_override();  // 0 (none), 256 or 128

// dt: 0 = bf16, 1 = fp16.  scratch == nullptr: split-K partials go to the
// library's per-GPU workspace (grown stream-ordered on s, calls ordered by an
// event), or under graph capture to stream-ordered memory taken and returned
// on s; otherwise to scratch, which must hold dense16_scratch_bytes(a).
hipError_t launch_dense16(const DenseArgs& a, int dt, hipStream_t s, const DenseScratch* scratch = nullptr);
// bytes of split-K partials launch_dense16 needs for a (0: no split)
size_t dense16_scratch_bytes(const DenseArgs& a);
hipError_t launch_dense_f32(const DenseArgs& a, hipStream_t s);
hipError_t launch_dense_f64(const DenseArgs& a, hipStream_t s);
hipError_t launch_qlinear(const QArgs& a, hipStream_t s);
// dt: 0 = bf16, 1 = fp16, 2 = fp32, 3 = fp64
size_t grouped_workspace_bytes(int64_t M, int64_t S, int64_t G);
hipError_t launch_grouped(const GroupedArgs& a, int dt, void* ws, hipStream_t s);
hipError_t launch_grouped_dq(const GroupedArgs& a, int dt, void* ws, hipStream_t s);
hipError_t grouped_invalid_count(const void* ws, hipStream_t s, int64_t* count);

}  // namespace omm
