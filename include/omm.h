/*
 * omm.h -- C ABI of the ONNX MatMul-family operators for AMD Instinct MI355X (gfx950).
 *
 * Four operators, each one call, each computing what its ONNX operator page
 * defines:
 *   omm_matmul           MatMul (since version 13): a matrix product that
 *                        behaves like numpy.matmul.
 *   omm_gemm             Gemm (since version 13): Y = alpha * A' * B' + beta * C.
 *   omm_qlinear_matmul   QLinearMatMul (version 10): quantised 8-bit matmul with
 *                        32-bit accumulation and a round-half-even requantisation.
 *   omm_grouped_matmul   GroupedMatMul (version 29):
 *                        output[m, i] = input[m] @ weights[group_indices[m, i]] (+ bias[g]).
 *   omm_grouped_matmul_dequant  the same over int8/uint8 weights with block
 *                        scales (DequantizeLinear fused into the weight load).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense and row-major (the last dim is contiguous), described by
 *    omm_tensor: a DEVICE pointer, a dtype and a shape.  The caller owns every
 *    buffer -- inputs, outputs and the grouped workspace -- allocates the
 *    output at the shape the matching *_output_shape call reports, and keeps
 *    all of them alive until the enqueued work has finished.  The library
 *    keeps no per-call state and never frees caller memory.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued: a call returns as soon as its kernels are launched, without a
 *    host synchronisation (omm_grouped_matmul_check is the one exception).
 *  - Return value: OMM_OK (0) when the arguments were valid and every kernel
 *    launched; a negative OMM_ERR_* code otherwise.  Argument errors are found
 *    on the host before anything is launched, so on error nothing was written.
 *  - Empty outputs (any output dim 0) return OMM_OK without launching.  An empty
 *    contraction (K = 0) writes the epilogue of a zero accumulator.
 *  - Data pointers must be at least element-aligned.  16-byte-aligned bases and
 *    row lengths that are multiples of 16 bytes take the vectorised path; other
 *    layouts are still computed correctly by an element-wise path.
 *  - Concurrent calls on different streams may run in parallel; they share
 *    nothing but the caller's buffers (omm_gemm_noalloc and the split-K
 *    workspace below excepted).
 *  - Scratch: omm_matmul and omm_gemm with bf16 / fp16 operands split K over
 *    several workgroups for shapes with few output tiles and a long K
 *    (decode-like rows, narrow outputs).  The fp32 partial products of such a
 *    call (splits x batches x M x N x 4 bytes) live in a workspace the
 *    library keeps per GPU until the process ends: taken with hipMallocAsync
 *    on the calling stream and, when a call needs more, freed with
 *    hipFreeAsync and taken again larger on that stream.  An event recorded
 *    after each such call makes the next one (on any stream) wait for it, so
 *    split-K calls on one GPU run one after another.  Under HIP graph capture
 *    the partials instead live in stream-ordered memory taken and returned
 *    around the call's kernels.  If the memory pool cannot supply the
 *    workspace the call returns OMM_ERR_HIP with nothing launched.  No other
 *    entry point allocates device memory.
 */
#ifndef OMM_H_
#define OMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum omm_dtype {
    OMM_F32 = 0,
    OMM_F16 = 1,
    OMM_BF16 = 2,
    OMM_F64 = 3,
    OMM_I8 = 4,
    OMM_U8 = 5,
    OMM_I32 = 6,
    OMM_I64 = 7
} omm_dtype;

#define OMM_MAX_DIMS 8

typedef struct omm_tensor {
    void* data;                   /* device pointer to element 0 (may be NULL if numel == 0) */
    int32_t dtype;                /* an omm_dtype                                            */
    int32_t ndim;                 /* 0 .. OMM_MAX_DIMS; 0 = scalar                           */
    int64_t shape[OMM_MAX_DIMS];  /* extents, all >= 0; entries past ndim are ignored        */
} omm_tensor;

#define OMM_OK 0
#define OMM_ERR_NULL (-1)        /* a required tensor/pointer argument is NULL               */
#define OMM_ERR_DTYPE (-2)       /* dtype not allowed, or dtypes that must agree differ      */
#define OMM_ERR_SHAPE (-3)       /* ranks/extents inconsistent (e.g. inner dims differ)      */
#define OMM_ERR_BROADCAST (-4)   /* batch dims, C or a quantisation parameter don't broadcast */
#define OMM_ERR_UNSUPPORTED (-5) /* valid for the operator but not implemented here          */
#define OMM_ERR_WORKSPACE (-6)   /* grouped workspace NULL or smaller than required          */
#define OMM_ERR_HIP (-7)         /* a HIP runtime call or kernel launch failed               */
#define OMM_ERR_SCRATCH (-8)     /* omm_gemm_noalloc: the shape needs more than its scratch   */

/* Human-readable text for a status code (static storage, never NULL). */
const char* omm_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int omm_version(void);

/* ------------------------------------------------------------------------
 * MatMul.  Defined as "matrix product that behaves like numpy.matmul"
 * (MatMul since version 13, Summary; inputs A, B and output Y of type T).
 *   - A 1-D A (K) is read as (1, K) and a 1-D B (K) as (K, 1); the added dim
 *     is removed from Y (so 1-D x 1-D gives a 0-d Y).
 *   - Dims before the last two are batch dims: right-aligned, each pair equal
 *     or one of them 1 (broadcast); Y's batch dims are the broadcast shape.
 *   - T: OMM_BF16, OMM_F16, OMM_F32 or OMM_F64 (A, B and Y all the same).
 *     bf16/fp16 accumulate in fp32 and round once (nearest-even) to T; fp64
 *     accumulates in fp64.  The integer types the page allows (int32/64,
 *     uint32/64) return OMM_ERR_UNSUPPORTED.
 * Errors: OMM_ERR_NULL, OMM_ERR_DTYPE, OMM_ERR_SHAPE (ndim 0, inner dims
 * differ, or Y's shape is not the computed one), OMM_ERR_BROADCAST.
 */
int omm_matmul_output_shape(const omm_tensor* A, const omm_tensor* B, int32_t* ndim, int64_t* shape);
int omm_matmul(const omm_tensor* A, const omm_tensor* B, omm_tensor* Y, void* stream);

/* ------------------------------------------------------------------------
 * Gemm.  Y = alpha * A' * B' + beta * C with A' = transpose(A) if transA,
 * B' = transpose(B) if transB (Gemm since version 13, formula and Inputs).
 *   - A is (M, K), or (K, M) when transA != 0; B is (K, N), or (N, K) when
 *     transB != 0; Y is (M, N).
 *   - C may be NULL (computed as if C were a scalar 0); otherwise it must be
 *     unidirectionally broadcastable to (M, N): shape (), (1), (N), (1, N),
 *     (M, 1) or (M, N) (and the equivalents with extents 1).
 *   - alpha and beta are the operator's float attributes; the ONNX defaults
 *     are alpha = 1, beta = 1, transA = transB = 0 and are the caller's to pass.
 *   - T: OMM_BF16, OMM_F16, OMM_F32 or OMM_F64 for A, B, C and Y alike.  The
 *     epilogue is computed in fp32 from the fp32 accumulator and rounded once
 *     to T (fp64: in fp64, alpha and beta taken exactly).
 * Errors: as omm_matmul, plus OMM_ERR_BROADCAST for a C that does not fit.
 */
int omm_gemm_output_shape(const omm_tensor* A, const omm_tensor* B, int transA, int transB,
                          int32_t* ndim, int64_t* shape);
int omm_gemm(const omm_tensor* A, const omm_tensor* B, const omm_tensor* C, float alpha, float beta,
             int transA, int transB, omm_tensor* Y, void* stream);

/* ------------------------------------------------------------------------
 * omm_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as omm_gemm, computed by the same kernels;
 * the split-K partial products that omm_gemm takes from stream-ordered memory
 * go instead to a static device array of OMM_GEMM_NOALLOC_SCRATCH_BYTES per
 * GPU (reserved when the library's device code is loaded on that GPU, held
 * until the process ends; its address is looked up on the first call that
 * runs on the GPU).  The call allocates and frees nothing.
 *   - A shape whose partials need more than the scratch (bf16 / fp16 split-K
 *     with splits x M x N x 4 bytes > OMM_GEMM_NOALLOC_SCRATCH_BYTES) returns
 *     OMM_ERR_SCRATCH with nothing launched.  Shapes that do not split K
 *     (and every fp32 / fp64 shape) use no scratch.
 *   - The array's address on a GPU is looked up once (hipGetSymbolAddress);
 *     a failure there returns OMM_ERR_HIP, a device ordinal of 64 or more
 *     OMM_ERR_UNSUPPORTED.
 *   - Every call on one GPU shares that GPU's array and leaves its last
 *     contents there (each call writes every partial it reads, nothing needs
 *     clearing).  Calls that overlap on one GPU -- on different streams, or
 *     from several host threads -- race on the array: the caller serialises
 *     them (one stream, or events).
 */
#define OMM_GEMM_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int omm_gemm_noalloc(const omm_tensor* A, const omm_tensor* B, const omm_tensor* C, float alpha, float beta,
                     int transA, int transB, omm_tensor* Y, void* stream);

/* ------------------------------------------------------------------------
 * QLinearMatMul (version 10, Summary, Inputs, Type Constraints).
 *   a (T1), b (T2): int8/uint8 matrices with numpy.matmul shape rules (as
 *   omm_matmul).  y (T3): int8/uint8, dtype taken from y_zero_point.
 *   Per output element:
 *     acc  = sum_k (a - a_zero_point) * (b - b_zero_point)   int32, wraps mod 2^32
 *     mult = fp32( fp32(a_scale * b_scale) / y_scale )         each op rounded to nearest even
 *     x    = fp32( fp32(acc) * mult )
 *     y    = saturate( round_half_even(x) + y_zero_point )     to T3's range
 *   Scales are fp32 (OMM_F32) or fp16 (OMM_F16) device tensors, all three of
 *   one dtype (fp16 values are taken exactly as fp32; the page's examples use
 *   both).  Scale and zero point of one
 *   operand have the same shape: a single element (per tensor), or per row of
 *   a -- (M), or (..., M, 1) broadcastable to a's batch dims -- or per column
 *   of b -- (N), or (..., 1, N) broadcastable to b's batch dims.  The zero
 *   point's dtype equals its operand's.  y_scale and y_zero_point hold one
 *   element each.
 * Errors: OMM_ERR_NULL, OMM_ERR_DTYPE (also scales of mixed or other dtypes),
 * OMM_ERR_SHAPE, OMM_ERR_BROADCAST.  Non-positive or non-finite scales
 * are outside the operator's domain; the result is then unspecified.
 */
int omm_qlinear_matmul_output_shape(const omm_tensor* a, const omm_tensor* b, int32_t* ndim, int64_t* shape);
int omm_qlinear_matmul(const omm_tensor* a, const omm_tensor* a_scale, const omm_tensor* a_zero_point,
                       const omm_tensor* b, const omm_tensor* b_scale, const omm_tensor* b_zero_point,
                       const omm_tensor* y_scale, const omm_tensor* y_zero_point, omm_tensor* y, void* stream);

/* ------------------------------------------------------------------------
 * GroupedMatMul (version 29, Summary and Inputs).
 *   input (M, K), weights (G, K, N), group_indices (M, S) of OMM_I32 or
 *   OMM_I64, optional bias (G, N) (NULL = absent), output (M, S, N):
 *     output[m, i, :] = input[m, :] @ weights[g] (+ bias[g, :]), g = group_indices[m, i]
 *   T: OMM_BF16, OMM_F16, OMM_F32 or OMM_F64 (input, weights, bias, output
 *   alike); fp32 accumulation (fp64 for OMM_F64), one rounding to T of
 *   (accumulator + bias).
 *   The (m, i) pairs are counting-sorted by group on the device and each
 *   group's rows run as one GEMM against weights[g]; the gathered
 *   (M*S, K, N) weights are never formed.
 *   workspace: device memory of at least omm_grouped_matmul_workspace_size(M,
 *   S, G) bytes, 256-byte aligned, owned by the caller, used only during the
 *   call's kernels (reuse it once the stream has passed them).
 *   Indices outside [0, G) -- negative ones included, they do not wrap -- are
 *   invalid input for the operator.  Here such a pair's output row is left
 *   unwritten and the pair is counted; omm_grouped_matmul_check reads the count.
 * Errors: OMM_ERR_NULL, OMM_ERR_DTYPE, OMM_ERR_SHAPE, OMM_ERR_WORKSPACE.
 */
size_t omm_grouped_matmul_workspace_size(int64_t M, int64_t S, int64_t G);
int omm_grouped_matmul_output_shape(const omm_tensor* input, const omm_tensor* weights,
                                    const omm_tensor* group_indices, int32_t* ndim, int64_t* shape);
int omm_grouped_matmul(const omm_tensor* input, const omm_tensor* weights, const omm_tensor* group_indices,
                       const omm_tensor* bias, omm_tensor* output, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * GroupedMatMul over weight-only quantised experts (GroupedMatMul version 29,
 * Summary: quantised weights passed through DequantizeLinear and then to
 * GroupedMatMul, a composition runtimes may fuse so the dequantised
 * (G, K, N) weights are never materialised).  Computes exactly
 *     w[g, k, n] = T( (q[g, k, n] - zp[g, k / block_size, n]) * scale[g, k / block_size, n] )
 *     output[m, i, :] = input[m, :] @ w[g] (+ bias[g, :]),  g = group_indices[m, i]
 * i.e. DequantizeLinear blocked along K (its output in the scale's type T,
 * rounded once, nearest-even; (q - zp) * scale is exact before that rounding
 * for 16-bit T) followed by omm_grouped_matmul.  The dequantised weights are
 * formed in registers as each weight tile is staged.
 *   input (M, K) of T; qweights (G, K, N) OMM_I8 or OMM_U8; w_scale
 *   (G, ceil(K / block_size), N) of T; w_zero_point NULL (zero) or like
 *   w_scale with qweights' dtype; block_size >= 1 (block_size >= K: one scale
 *   per group and column); group_indices, bias, output, workspace, stream and
 *   invalid indices as omm_grouped_matmul.  T: OMM_BF16, OMM_F16 or OMM_F32
 *   (OMM_F64 returns OMM_ERR_UNSUPPORTED).
 *   The fast path needs 16-byte aligned input / 8-byte aligned q, zp, bias and
 *   output / 16-byte aligned scales, K and N multiples of 8 and block_size a
 *   multiple of 64; other layouts use an element-wise path.
 * Errors: OMM_ERR_NULL, OMM_ERR_DTYPE, OMM_ERR_SHAPE (also block_size < 1 or
 * a scale / zero-point shape that is not (G, ceil(K / block_size), N)),
 * OMM_ERR_WORKSPACE.
 */
int omm_grouped_matmul_dequant(const omm_tensor* input, const omm_tensor* qweights, const omm_tensor* w_scale,
                               const omm_tensor* w_zero_point, int64_t block_size, const omm_tensor* group_indices,
                               const omm_tensor* bias, omm_tensor* output, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Waits for `stream`, then reports how many (m, i) pairs of the last
 * omm_grouped_matmul that used `workspace` had an index outside [0, G).
 * Returns OMM_OK or OMM_ERR_NULL / OMM_ERR_HIP. */
int omm_grouped_matmul_check(const void* workspace, void* stream, int64_t* invalid_count);

#ifdef __cplusplus
}
#endif

#endif /* OMM_H_ */
