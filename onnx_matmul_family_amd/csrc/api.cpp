// C ABI of the MatMul-family operators: argument validation, numpy.matmul
// broadcast resolution and kernel dispatch.  Everything here runs on the host
// before any launch; the kernels live in the .hip files.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "omm.h"
#include "kernels.hpp"

namespace omm {

bool log_enabled() {
    static const bool on = [] {
        const char* v = getenv("OMM_LOG");
        return v && *v && strcmp(v, "0") != 0;
    }();
    return on;
}

void log_choice(const char* fmt, ...) {
    if (!log_enabled()) return;
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    fprintf(stderr, "omm: %s\n", buf);
}

int tile_override() {
    static const int t = [] {
        const char* v = getenv("OMM_TILE");
        if (!v) return 0;
        if (strcmp(v, "256x256x64") == 0) return 256;
        if (strcmp(v, "128x128x64") == 0) return 128;
        return 0;
    }();
    return t;
}

}  // namespace omm

using omm::DenseArgs;
using omm::GroupedArgs;
using omm::QArgs;

namespace {

bool numel(const omm_tensor* t, int64_t* n) {
    int64_t v = 1;
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] < 0) return false;
        v *= t->shape[i];
    }
    *n = v;
    return true;
}

// structural checks shared by every tensor argument
int check_tensor(const omm_tensor* t) {
    if (!t) return OMM_ERR_NULL;
    if (t->ndim < 0 || t->ndim > OMM_MAX_DIMS) return OMM_ERR_SHAPE;
    int64_t n;
    if (!numel(t, &n)) return OMM_ERR_SHAPE;
    if (n > 0 && !t->data) return OMM_ERR_NULL;
    return OMM_OK;
}

int elem_size(int dt) {
    switch (dt) {
        case OMM_F32: case OMM_I32: return 4;
        case OMM_F16: case OMM_BF16: return 2;
        case OMM_F64: case OMM_I64: return 8;
        case OMM_I8: case OMM_U8: return 1;
    }
    return 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? OMM_OK : OMM_ERR_HIP; }

// ---------------------------------------------------------------------------
// numpy.matmul geometry: 1-D promotion, right-aligned batch broadcast, and the
// element strides of each operand along each output batch dim.
struct MMGeom {
    int64_t M = 0, N = 0, K = 0;
    bool drop_m = false, drop_n = false;
    int nb = 0;
    int64_t bsh[OMM_MAX_DIMS];
    int64_t as[OMM_MAX_DIMS], bs[OMM_MAX_DIMS], ys[OMM_MAX_DIMS];  // batch strides (elements)
    int a_nb = 0, b_nb = 0;  // operands' own batch ranks after promotion
    int y_nd = 0;
    int64_t y_sh[OMM_MAX_DIMS];
};

int mm_resolve(const omm_tensor* A, const omm_tensor* B, MMGeom* g) {
    if (A->ndim < 1 || B->ndim < 1) return OMM_ERR_SHAPE;
    int64_t ash[OMM_MAX_DIMS + 1], bsh[OMM_MAX_DIMS + 1];
    int an = A->ndim, bn = B->ndim;
    if (an == 1) { ash[0] = 1; ash[1] = A->shape[0]; an = 2; g->drop_m = true; }
    else for (int i = 0; i < an; ++i) ash[i] = A->shape[i];
    if (bn == 1) { bsh[0] = B->shape[0]; bsh[1] = 1; bn = 2; g->drop_n = true; }
    else for (int i = 0; i < bn; ++i) bsh[i] = B->shape[i];
    g->M = ash[an - 2];
    g->K = ash[an - 1];
    g->N = bsh[bn - 1];
    if (bsh[bn - 2] != g->K) return OMM_ERR_SHAPE;
    const int na = an - 2, nbb = bn - 2;
    g->a_nb = na;
    g->b_nb = nbb;
    g->nb = std::max(na, nbb);
    int64_t astr = g->M * g->K, bstr = g->K * g->N, ystr = g->M * g->N;
    for (int i = g->nb - 1; i >= 0; --i) {
        const int ia = i - (g->nb - na), ib = i - (g->nb - nbb);
        const int64_t da = ia >= 0 ? ash[ia] : 1, db = ib >= 0 ? bsh[ib] : 1;
        if (da != db && da != 1 && db != 1) return OMM_ERR_BROADCAST;
        const int64_t d = (da == 0 || db == 0) ? 0 : std::max(da, db);
        g->bsh[i] = d;
        g->as[i] = da == 1 ? 0 : astr;
        g->bs[i] = db == 1 ? 0 : bstr;
        g->ys[i] = ystr;
        astr *= da;
        bstr *= db;
        ystr *= d;
    }
    g->y_nd = 0;
    for (int i = 0; i < g->nb; ++i) g->y_sh[g->y_nd++] = g->bsh[i];
    if (!g->drop_m) g->y_sh[g->y_nd++] = g->M;
    if (!g->drop_n) g->y_sh[g->y_nd++] = g->N;
    return OMM_OK;
}

// Batch dims after dropping extents of 1 and merging neighbours that every
// operand walks contiguously.  `extra` holds further per-operand stride sets
// that must merge the same way (quantisation parameters).
struct Batch {
    int nb = 0;
    int64_t sh[OMM_MAX_DIMS];
    int64_t st[6][OMM_MAX_DIMS];  // stride sets: 0 = A, 1 = B, 2 = Y, 3.. = extra
    int nsets = 3;
};

void fold_batch(Batch* b) {
    int n = 0;
    for (int i = 0; i < b->nb; ++i) {
        if (b->sh[i] == 1) continue;
        b->sh[n] = b->sh[i];
        for (int s = 0; s < b->nsets; ++s) b->st[s][n] = b->st[s][i];
        ++n;
    }
    b->nb = n;
    n = 0;
    for (int i = 0; i < b->nb; ++i) {
        if (n > 0) {
            bool mergeable = true;
            for (int s = 0; s < b->nsets; ++s)
                if (b->st[s][n - 1] != b->st[s][i] * b->sh[i]) mergeable = false;
            if (mergeable) {
                b->sh[n - 1] *= b->sh[i];
                for (int s = 0; s < b->nsets; ++s) b->st[s][n - 1] = b->st[s][i];
                continue;
            }
        }
        b->sh[n] = b->sh[i];
        for (int s = 0; s < b->nsets; ++s) b->st[s][n] = b->st[s][i];
        ++n;
    }
    b->nb = n;
}

// Calls launch(offsets, nb0, nb1, strides of the two innermost batch levels)
// once per combination of the outer batch levels (normally exactly once).
template <class F>
int for_each_outer(const Batch& b, F&& launch) {
    const int inner = std::min(b.nb, 2);
    const int outer = b.nb - inner;
    int64_t nouter = 1;
    for (int i = 0; i < outer; ++i) nouter *= b.sh[i];
    for (int64_t o = 0; o < nouter; ++o) {
        int64_t off[6] = {0, 0, 0, 0, 0, 0};
        int64_t r = o;
        for (int i = outer - 1; i >= 0; --i) {
            const int64_t c = r % b.sh[i];
            r /= b.sh[i];
            for (int s = 0; s < b.nsets; ++s) off[s] += c * b.st[s][i];
        }
        int64_t nb0 = 1, nb1 = 1, s0[6] = {0, 0, 0, 0, 0, 0}, s1[6] = {0, 0, 0, 0, 0, 0};
        if (inner == 2) {
            nb0 = b.sh[outer];
            nb1 = b.sh[outer + 1];
            for (int s = 0; s < b.nsets; ++s) { s0[s] = b.st[s][outer]; s1[s] = b.st[s][outer + 1]; }
        } else if (inner == 1) {
            nb1 = b.sh[outer];
            for (int s = 0; s < b.nsets; ++s) s1[s] = b.st[s][outer];
        }
        const int rc = launch(off, nb0, nb1, s0, s1);
        if (rc != OMM_OK) return rc;
    }
    return OMM_OK;
}

bool is_dense_float(int dt) { return dt == OMM_BF16 || dt == OMM_F16 || dt == OMM_F32 || dt == OMM_F64; }

hipError_t launch_dense(const DenseArgs& a, int dt, hipStream_t s, const omm::DenseScratch* scratch = nullptr) {
    if (dt == OMM_F32) return omm::launch_dense_f32(a, s);
    if (dt == OMM_F64) return omm::launch_dense_f64(a, s);
    return omm::launch_dense16(a, dt == OMM_BF16 ? 0 : 1, s, scratch);
}

// ---------------------------------------------------------------------------
// Static scratch of omm_gemm_noalloc: one array per GPU, reserved when the
// library's device code is loaded on that GPU and held until the process
// ends.  On the host `scratch` only names the symbol; its device address on
// each GPU comes from hipGetSymbolAddress with that GPU current, looked up on
// the first call that runs on the GPU and kept in scratch_dev.
static __device__ __align__(256) char scratch[OMM_GEMM_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES] = {};

// device address of `scratch` on the GPU that runs `s`
int scratch_address(hipStream_t s, void** out) {
    int dev = -1;
    if (s) {
        if (hipStreamGetDevice(s, &dev) != hipSuccess) return OMM_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return OMM_ERR_HIP;
    }
    if (dev < 0 || dev >= MAX_DEVICES) return OMM_ERR_UNSUPPORTED;  // more GPUs than the table holds
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return OMM_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return OMM_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return OMM_ERR_HIP;
        if (e != hipSuccess || !p) return OMM_ERR_HIP;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return OMM_OK;
}

int check_out(const omm_tensor* Y, int ndim, const int64_t* shape) {
    if (Y->ndim != ndim) return OMM_ERR_SHAPE;
    for (int i = 0; i < ndim; ++i)
        if (Y->shape[i] != shape[i]) return OMM_ERR_SHAPE;
    return OMM_OK;
}

const char* byte_ptr(const void* p, int64_t elems, int dt) { return (const char*)p + elems * elem_size(dt); }

}  // namespace

extern "C" {

const char* omm_status_string(int status) {
    switch (status) {
        case OMM_OK: return "ok";
        case OMM_ERR_NULL: return "required argument is NULL";
        case OMM_ERR_DTYPE: return "dtype not allowed or dtypes disagree";
        case OMM_ERR_SHAPE: return "shapes are inconsistent";
        case OMM_ERR_BROADCAST: return "dims do not broadcast";
        case OMM_ERR_UNSUPPORTED: return "valid for the operator but not implemented";
        case OMM_ERR_WORKSPACE: return "workspace missing or too small";
        case OMM_ERR_HIP: return "HIP runtime or launch failure";
        case OMM_ERR_SCRATCH: return "split-K partials exceed the static scratch of omm_gemm_noalloc (32 MiB)";
    }
    return "unknown status";
}

int omm_version(void) { return 100; }

// ------------------------------------------------------------------ MatMul

int omm_matmul_output_shape(const omm_tensor* A, const omm_tensor* B, int32_t* ndim, int64_t* shape) {
    int rc;
    if ((rc = check_tensor(A)) || (rc = check_tensor(B))) return rc;
    if (!ndim || !shape) return OMM_ERR_NULL;
    MMGeom g;
    if ((rc = mm_resolve(A, B, &g))) return rc;
    *ndim = g.y_nd;
    for (int i = 0; i < g.y_nd; ++i) shape[i] = g.y_sh[i];
    return OMM_OK;
}

int omm_matmul(const omm_tensor* A, const omm_tensor* B, omm_tensor* Y, void* stream) {
    int rc;
    if ((rc = check_tensor(A)) || (rc = check_tensor(B)) || (rc = check_tensor(Y))) return rc;
    if (A->dtype != B->dtype || A->dtype != Y->dtype) return OMM_ERR_DTYPE;
    const int dt = A->dtype;
    if (elem_size(dt) == 0) return OMM_ERR_DTYPE;
    if (!is_dense_float(dt)) return OMM_ERR_UNSUPPORTED;
    MMGeom g;
    if ((rc = mm_resolve(A, B, &g))) return rc;
    if ((rc = check_out(Y, g.y_nd, g.y_sh))) return rc;
    int64_t ny;
    numel(Y, &ny);
    if (ny == 0) return OMM_OK;

    Batch b;
    b.nb = g.nb;
    for (int i = 0; i < g.nb; ++i) {
        b.sh[i] = g.bsh[i];
        b.st[0][i] = g.as[i];
        b.st[1][i] = g.bs[i];
        b.st[2][i] = g.ys[i];
    }
    fold_batch(&b);
    int64_t M = g.M;
    // B shared by every batch and A, Y walked contiguously: one taller GEMM
    if (b.nb == 1 && b.st[1][0] == 0 && b.st[0][0] == g.M * g.K && b.st[2][0] == g.M * g.N) {
        M *= b.sh[0];
        b.nb = 0;
    }
    hipStream_t s = (hipStream_t)stream;
    return for_each_outer(b, [&](const int64_t* off, int64_t nb0, int64_t nb1, const int64_t* s0,
                                 const int64_t* s1) -> int {
        DenseArgs a;
        memset(&a, 0, sizeof a);
        a.A = byte_ptr(A->data, off[0], dt);
        a.B = byte_ptr(B->data, off[1], dt);
        a.Y = (void*)byte_ptr(Y->data, off[2], dt);
        a.C = nullptr;
        a.M = M;
        a.N = g.N;
        a.K = g.K;
        a.lda = g.K;
        a.ldb = g.N;
        a.ldy = g.N;
        a.a_bs0 = s0[0]; a.a_bs1 = s1[0];
        a.b_bs0 = s0[1]; a.b_bs1 = s1[1];
        a.y_bs0 = s0[2]; a.y_bs1 = s1[2];
        a.nb0 = nb0;
        a.nb1 = nb1;
        a.alpha = 1.0f;
        a.beta = 0.0f;
        a.a_kmajor = 1;
        a.b_kmajor = 0;
        return hip_status(launch_dense(a, dt, s));
    });
}

// ------------------------------------------------------------------ Gemm

int omm_gemm_output_shape(const omm_tensor* A, const omm_tensor* B, int transA, int transB, int32_t* ndim,
                          int64_t* shape) {
    int rc;
    if ((rc = check_tensor(A)) || (rc = check_tensor(B))) return rc;
    if (!ndim || !shape) return OMM_ERR_NULL;
    if (A->ndim != 2 || B->ndim != 2) return OMM_ERR_SHAPE;
    const int64_t K = transA ? A->shape[0] : A->shape[1];
    const int64_t Kb = transB ? B->shape[1] : B->shape[0];
    if (K != Kb) return OMM_ERR_SHAPE;
    *ndim = 2;
    shape[0] = transA ? A->shape[1] : A->shape[0];
    shape[1] = transB ? B->shape[0] : B->shape[1];
    return OMM_OK;
}

}  // extern "C"

namespace {

// Gemm with split-K partials in stream-ordered memory (noalloc = false) or in
// this GPU's static scratch (noalloc = true: nothing allocated, shapes needing
// more than the scratch rejected before any launch).
int gemm_impl(const omm_tensor* A, const omm_tensor* B, const omm_tensor* C, float alpha, float beta, int transA,
              int transB, omm_tensor* Y, void* stream, bool noalloc) {
    int rc;
    if ((rc = check_tensor(A)) || (rc = check_tensor(B)) || (rc = check_tensor(Y))) return rc;
    if (C && (rc = check_tensor(C))) return rc;
    const int dt = A->dtype;
    if (B->dtype != dt || Y->dtype != dt || (C && C->dtype != dt)) return OMM_ERR_DTYPE;
    if (elem_size(dt) == 0) return OMM_ERR_DTYPE;
    if (!is_dense_float(dt)) return OMM_ERR_UNSUPPORTED;
    int32_t nd;
    int64_t ysh[2];
    if ((rc = omm_gemm_output_shape(A, B, transA, transB, &nd, ysh))) return rc;
    if ((rc = check_out(Y, 2, ysh))) return rc;
    const int64_t M = ysh[0], N = ysh[1], K = transA ? A->shape[0] : A->shape[1];
    int64_t c_sm = 0, c_sn = 0;
    if (C) {
        if (C->ndim > 2) return OMM_ERR_BROADCAST;
        const int64_t cN = C->ndim >= 1 ? C->shape[C->ndim - 1] : 1;
        const int64_t cM = C->ndim == 2 ? C->shape[0] : 1;
        if ((cM != 1 && cM != M) || (cN != 1 && cN != N)) return OMM_ERR_BROADCAST;
        c_sn = cN == 1 ? 0 : 1;
        c_sm = cM == 1 ? 0 : cN;
    }
    if (M == 0 || N == 0) return OMM_OK;
    DenseArgs a;
    memset(&a, 0, sizeof a);
    a.A = A->data;
    a.B = B->data;
    a.Y = Y->data;
    a.C = C ? C->data : nullptr;
    a.M = M;
    a.N = N;
    a.K = K;
    a.lda = A->shape[1];
    a.ldb = B->shape[1];
    a.ldy = N;
    a.nb0 = 1;
    a.nb1 = 1;
    a.c_sm = c_sm;
    a.c_sn = c_sn;
    a.alpha = alpha;
    a.beta = beta;
    a.a_kmajor = transA ? 0 : 1;
    a.b_kmajor = transB ? 1 : 0;
    if (!noalloc) return hip_status(launch_dense(a, dt, (hipStream_t)stream));
    omm::DenseScratch sc{nullptr, OMM_GEMM_NOALLOC_SCRATCH_BYTES};
    if (dt == OMM_BF16 || dt == OMM_F16) {
        const size_t need = omm::dense16_scratch_bytes(a);
        if (need > OMM_GEMM_NOALLOC_SCRATCH_BYTES) return OMM_ERR_SCRATCH;
        // shapes that split nothing never touch the array (launch_dense16 checks
        // the pointer only when the plan needs scratch)
        if (need > 0 && (rc = scratch_address((hipStream_t)stream, &sc.ptr))) return rc;
    }
    return hip_status(launch_dense(a, dt, (hipStream_t)stream, &sc));
}

}  // namespace

extern "C" {

int omm_gemm(const omm_tensor* A, const omm_tensor* B, const omm_tensor* C, float alpha, float beta, int transA,
             int transB, omm_tensor* Y, void* stream) {
    return gemm_impl(A, B, C, alpha, beta, transA, transB, Y, stream, false);
}

int omm_gemm_noalloc(const omm_tensor* A, const omm_tensor* B, const omm_tensor* C, float alpha, float beta,
                     int transA, int transB, omm_tensor* Y, void* stream) {
    return gemm_impl(A, B, C, alpha, beta, transA, transB, Y, stream, true);
}

// ------------------------------------------------------------------ QLinearMatMul

namespace {

// Strides of a quantisation parameter over the operand's own batch dims, and
// along m (row side) or n (column side).  Per tensor: one element.  1-D of
// length MN: the per-row (a) / per-column (b) vector.  Otherwise (..., MN, 1)
// for the row side or (..., 1, MN) for the column side, leading dims
// broadcastable to the operand's batch dims.
int qparam_strides(const omm_tensor* p, int op_nb, const int64_t* op_bsh, int64_t MN, bool row_side,
                   int64_t* pst, int64_t* pmn) {
    int64_t n;
    numel(p, &n);
    for (int i = 0; i < op_nb; ++i) pst[i] = 0;
    *pmn = 0;
    if (n == 1) return OMM_OK;
    if (p->ndim == 1) {
        if (p->shape[0] != MN) return OMM_ERR_BROADCAST;
        *pmn = 1;
        return OMM_OK;
    }
    if (p->ndim < 2) return OMM_ERR_BROADCAST;
    const int64_t dm = row_side ? p->shape[p->ndim - 2] : p->shape[p->ndim - 1];
    const int64_t d1 = row_side ? p->shape[p->ndim - 1] : p->shape[p->ndim - 2];
    if (d1 != 1 || (dm != MN && dm != 1)) return OMM_ERR_BROADCAST;
    if (p->ndim - 2 > op_nb) return OMM_ERR_BROADCAST;
    *pmn = dm == 1 ? 0 : 1;
    int64_t str = dm == 1 ? 1 : MN;
    for (int i = p->ndim - 3; i >= 0; --i) {
        const int ob = op_nb - (p->ndim - 2) + i;
        if (p->shape[i] != 1 && p->shape[i] != op_bsh[ob]) return OMM_ERR_BROADCAST;
        pst[ob] = p->shape[i] == 1 ? 0 : str;
        str *= p->shape[i];
    }
    return OMM_OK;
}

bool same_shape(const omm_tensor* x, const omm_tensor* y) {
    if (x->ndim != y->ndim) return false;
    for (int i = 0; i < x->ndim; ++i)
        if (x->shape[i] != y->shape[i]) return false;
    return true;
}

}  // namespace

int omm_qlinear_matmul_output_shape(const omm_tensor* a, const omm_tensor* b, int32_t* ndim, int64_t* shape) {
    return omm_matmul_output_shape(a, b, ndim, shape);
}

int omm_qlinear_matmul(const omm_tensor* a, const omm_tensor* a_scale, const omm_tensor* a_zero_point,
                       const omm_tensor* b, const omm_tensor* b_scale, const omm_tensor* b_zero_point,
                       const omm_tensor* y_scale, const omm_tensor* y_zero_point, omm_tensor* y, void* stream) {
    const omm_tensor* all[9] = {a, a_scale, a_zero_point, b, b_scale, b_zero_point, y_scale, y_zero_point, y};
    int rc;
    for (const omm_tensor* t : all)
        if ((rc = check_tensor(t))) return rc;
    auto is8 = [](int d) { return d == OMM_I8 || d == OMM_U8; };
    if (!is8(a->dtype) || !is8(b->dtype) || !is8(y_zero_point->dtype)) return OMM_ERR_DTYPE;
    if (a_zero_point->dtype != a->dtype || b_zero_point->dtype != b->dtype || y->dtype != y_zero_point->dtype)
        return OMM_ERR_DTYPE;
    // scales: fp32, or fp16 (upcast exactly); the three alike
    if (a_scale->dtype != OMM_F32 && a_scale->dtype != OMM_F16) return OMM_ERR_DTYPE;
    if (b_scale->dtype != a_scale->dtype || y_scale->dtype != a_scale->dtype) return OMM_ERR_DTYPE;
    const int64_t ses = elem_size(a_scale->dtype);
    if (!same_shape(a_scale, a_zero_point) || !same_shape(b_scale, b_zero_point)) return OMM_ERR_BROADCAST;
    int64_t n;
    numel(y_scale, &n);
    if (n != 1) return OMM_ERR_UNSUPPORTED;
    numel(y_zero_point, &n);
    if (n != 1) return OMM_ERR_UNSUPPORTED;
    MMGeom g;
    if ((rc = mm_resolve(a, b, &g))) return rc;
    if ((rc = check_out(y, g.y_nd, g.y_sh))) return rc;
    // each operand's own batch shape
    int64_t a_bsh[OMM_MAX_DIMS], b_bsh[OMM_MAX_DIMS];
    for (int i = 0; i < g.a_nb; ++i) a_bsh[i] = a->shape[i];
    for (int i = 0; i < g.b_nb; ++i) b_bsh[i] = b->shape[i];
    int64_t apst[OMM_MAX_DIMS], bpst[OMM_MAX_DIMS], apm, bpn;
    if ((rc = qparam_strides(a_scale, g.a_nb, a_bsh, g.M, true, apst, &apm))) return rc;
    if ((rc = qparam_strides(b_scale, g.b_nb, b_bsh, g.N, false, bpst, &bpn))) return rc;
    int64_t ny;
    numel(y, &ny);
    if (ny == 0) return OMM_OK;

    Batch bt;
    bt.nb = g.nb;
    bt.nsets = 5;
    for (int i = 0; i < g.nb; ++i) {
        const int ia = i - (g.nb - g.a_nb), ib = i - (g.nb - g.b_nb);
        bt.sh[i] = g.bsh[i];
        bt.st[0][i] = g.as[i];
        bt.st[1][i] = g.bs[i];
        bt.st[2][i] = g.ys[i];
        bt.st[3][i] = (ia >= 0 && a_bsh[ia] != 1) ? apst[ia] : 0;
        bt.st[4][i] = (ib >= 0 && b_bsh[ib] != 1) ? bpst[ib] : 0;
    }
    fold_batch(&bt);
    hipStream_t s = (hipStream_t)stream;
    return for_each_outer(bt, [&](const int64_t* off, int64_t nb0, int64_t nb1, const int64_t* s0,
                                  const int64_t* s1) -> int {
        QArgs q;
        memset(&q, 0, sizeof q);
        q.a = (const char*)a->data + off[0];
        q.b = (const char*)b->data + off[1];
        q.y = (char*)y->data + off[2];
        q.a_scale = (const char*)a_scale->data + off[3] * ses;
        q.a_zp = (const char*)a_zero_point->data + off[3];
        q.b_scale = (const char*)b_scale->data + off[4] * ses;
        q.b_zp = (const char*)b_zero_point->data + off[4];
        q.y_scale = y_scale->data;
        q.scale_f16 = a_scale->dtype == OMM_F16;
        q.y_zp = y_zero_point->data;
        q.M = g.M;
        q.N = g.N;
        q.K = g.K;
        q.lda = g.K;
        q.ldb = g.N;
        q.ldy = g.N;
        q.a_bs0 = s0[0]; q.a_bs1 = s1[0];
        q.b_bs0 = s0[1]; q.b_bs1 = s1[1];
        q.y_bs0 = s0[2]; q.y_bs1 = s1[2];
        q.ap_bs0 = s0[3]; q.ap_bs1 = s1[3];
        q.bp_bs0 = s0[4]; q.bp_bs1 = s1[4];
        q.ap_sm = apm;
        q.bp_sn = bpn;
        q.nb0 = nb0;
        q.nb1 = nb1;
        q.a_u8 = a->dtype == OMM_U8;
        q.b_u8 = b->dtype == OMM_U8;
        q.y_u8 = y->dtype == OMM_U8;
        return hip_status(omm::launch_qlinear(q, s));
    });
}

// ------------------------------------------------------------------ GroupedMatMul

size_t omm_grouped_matmul_workspace_size(int64_t M, int64_t S, int64_t G) {
    if (M < 0 || S < 0 || G < 0) return 0;
    return omm::grouped_workspace_bytes(M, S, G);
}

int omm_grouped_matmul_output_shape(const omm_tensor* input, const omm_tensor* weights,
                                    const omm_tensor* group_indices, int32_t* ndim, int64_t* shape) {
    int rc;
    if ((rc = check_tensor(input)) || (rc = check_tensor(weights)) || (rc = check_tensor(group_indices))) return rc;
    if (!ndim || !shape) return OMM_ERR_NULL;
    if (input->ndim != 2 || weights->ndim != 3 || group_indices->ndim != 2) return OMM_ERR_SHAPE;
    if (weights->shape[1] != input->shape[1] || group_indices->shape[0] != input->shape[0]) return OMM_ERR_SHAPE;
    *ndim = 3;
    shape[0] = input->shape[0];
    shape[1] = group_indices->shape[1];
    shape[2] = weights->shape[2];
    return OMM_OK;
}

int omm_grouped_matmul(const omm_tensor* input, const omm_tensor* weights, const omm_tensor* group_indices,
                       const omm_tensor* bias, omm_tensor* output, void* workspace, size_t workspace_bytes,
                       void* stream) {
    int rc;
    if ((rc = check_tensor(output))) return rc;
    if (bias && (rc = check_tensor(bias))) return rc;
    int32_t nd;
    int64_t osh[3];
    if ((rc = omm_grouped_matmul_output_shape(input, weights, group_indices, &nd, osh))) return rc;
    const int dt = input->dtype;
    if (weights->dtype != dt || output->dtype != dt || (bias && bias->dtype != dt)) return OMM_ERR_DTYPE;
    if (elem_size(dt) == 0 || dt == OMM_I8 || dt == OMM_U8 || dt == OMM_I32 || dt == OMM_I64) return OMM_ERR_DTYPE;
    if (!is_dense_float(dt)) return OMM_ERR_UNSUPPORTED;
    if (group_indices->dtype != OMM_I32 && group_indices->dtype != OMM_I64) return OMM_ERR_DTYPE;
    const int64_t M = osh[0], S = osh[1], N = osh[2], K = input->shape[1], G = weights->shape[0];
    if (bias && (bias->ndim != 2 || bias->shape[0] != G || bias->shape[1] != N)) return OMM_ERR_SHAPE;
    if ((rc = check_out(output, 3, osh))) return rc;
    if (!workspace || workspace_bytes < omm::grouped_workspace_bytes(M, S, G) || ((uintptr_t)workspace & 255))
        return OMM_ERR_WORKSPACE;
    if (G > 8192 || M * S > 0x7fffffffLL) return OMM_ERR_UNSUPPORTED;
    GroupedArgs a;
    memset(&a, 0, sizeof a);
    a.input = input->data;
    a.weights = weights->data;
    a.idx = group_indices->data;
    a.bias = bias ? bias->data : nullptr;
    a.output = output->data;
    a.M = M;
    a.K = K;
    a.N = N;
    a.G = G;
    a.S = S;
    a.idx64 = group_indices->dtype == OMM_I64;
    const int kd = dt == OMM_BF16 ? 0 : dt == OMM_F16 ? 1 : dt == OMM_F32 ? 2 : 3;
    return hip_status(omm::launch_grouped(a, kd, workspace, (hipStream_t)stream));
}

int omm_grouped_matmul_dequant(const omm_tensor* input, const omm_tensor* qweights, const omm_tensor* w_scale,
                               const omm_tensor* w_zero_point, int64_t block_size, const omm_tensor* group_indices,
                               const omm_tensor* bias, omm_tensor* output, void* workspace, size_t workspace_bytes,
                               void* stream) {
    int rc;
    if ((rc = check_tensor(output)) || (rc = check_tensor(w_scale))) return rc;
    if (bias && (rc = check_tensor(bias))) return rc;
    if (w_zero_point && (rc = check_tensor(w_zero_point))) return rc;
    int32_t nd;
    int64_t osh[3];
    if ((rc = omm_grouped_matmul_output_shape(input, qweights, group_indices, &nd, osh))) return rc;
    const int dt = input->dtype;
    if (qweights->dtype != OMM_I8 && qweights->dtype != OMM_U8) return OMM_ERR_DTYPE;
    if (w_scale->dtype != dt || output->dtype != dt || (bias && bias->dtype != dt)) return OMM_ERR_DTYPE;
    if (w_zero_point && w_zero_point->dtype != qweights->dtype) return OMM_ERR_DTYPE;
    if (elem_size(dt) == 0 || dt == OMM_I8 || dt == OMM_U8 || dt == OMM_I32 || dt == OMM_I64) return OMM_ERR_DTYPE;
    if (!is_dense_float(dt) || dt == OMM_F64) return OMM_ERR_UNSUPPORTED;
    if (group_indices->dtype != OMM_I32 && group_indices->dtype != OMM_I64) return OMM_ERR_DTYPE;
    const int64_t M = osh[0], S = osh[1], N = osh[2], K = input->shape[1], G = qweights->shape[0];
    if (block_size < 1) return OMM_ERR_SHAPE;
    const int64_t nkb = (K + block_size - 1) / block_size;
    if (w_scale->ndim != 3 || w_scale->shape[0] != G || w_scale->shape[1] != nkb || w_scale->shape[2] != N)
        return OMM_ERR_SHAPE;
    if (w_zero_point && (w_zero_point->ndim != 3 || w_zero_point->shape[0] != G || w_zero_point->shape[1] != nkb ||
                         w_zero_point->shape[2] != N))
        return OMM_ERR_SHAPE;
    if (bias && (bias->ndim != 2 || bias->shape[0] != G || bias->shape[1] != N)) return OMM_ERR_SHAPE;
    if ((rc = check_out(output, 3, osh))) return rc;
    if (!workspace || workspace_bytes < omm::grouped_workspace_bytes(M, S, G) || ((uintptr_t)workspace & 255))
        return OMM_ERR_WORKSPACE;
    if (G > 8192 || M * S > 0x7fffffffLL) return OMM_ERR_UNSUPPORTED;
    GroupedArgs a;
    memset(&a, 0, sizeof a);
    a.input = input->data;
    a.weights = qweights->data;
    a.idx = group_indices->data;
    a.bias = bias ? bias->data : nullptr;
    a.output = output->data;
    a.M = M;
    a.K = K;
    a.N = N;
    a.G = G;
    a.S = S;
    a.idx64 = group_indices->dtype == OMM_I64;
    a.wscale = w_scale->data;
    a.wzp = w_zero_point ? w_zero_point->data : nullptr;
    a.bs = block_size;
    a.nkb = nkb;
    a.q_kind = qweights->dtype == OMM_U8 ? 2 : 1;
    const int kd = dt == OMM_BF16 ? 0 : dt == OMM_F16 ? 1 : 2;
    return hip_status(omm::launch_grouped_dq(a, kd, workspace, (hipStream_t)stream));
}

int omm_grouped_matmul_check(const void* workspace, void* stream, int64_t* invalid_count) {
    if (!workspace || !invalid_count) return OMM_ERR_NULL;
    return hip_status(omm::grouped_invalid_count(workspace, (hipStream_t)stream, invalid_count));
}

}  // extern "C"
