/*
 * Plain CPU oracle for the ONNX MatMul-family operators.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with the
 * GPU path.
 *
 * Every operator is computed straight from its definition, one output element
 * at a time, accumulating floating-point products in double and integer
 * products in int64.  No blocking, no reordering beyond "sum over k in order".
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no -ffast-math), so every float
 * operation below is a separately rounded IEEE operation.
 *
 * Definitions followed (page title, section):
 *  - MatMul (onnx-light docs, since version 13), Summary: a matrix product
 *    that behaves like numpy.matmul -- 1-D operands are promoted (a 1 is
 *    prepended to a 1-D A, appended to a 1-D B, and the added dim is removed
 *    from the result) and the leading "batch" dims broadcast numpy-style.
 *  - Gemm (onnx-light docs, since version 13), formula paragraph and Inputs:
 *    Y = alpha * A' * B' + beta * C, A' = A^T if transA, B' = B^T if transB,
 *    C optional (absent = scalar 0) and unidirectionally broadcastable to (M,N).
 *  - QLinearMatMul - version 10, Summary: int8/uint8 inputs with zero points,
 *    products accumulated in 32 bits (the only place overflow may happen),
 *    y = saturate(round_half_even(x / y_scale) + y_zero_point); scale and zero
 *    point per tensor, per row of a or per column of b.
 *  - GroupedMatMul - 29, Summary:
 *    output[m, i] = input[m] @ weights[group_indices[m, i]] (+ bias[g]),
 *    indices outside [0, G) are invalid; weight-only quantised experts are
 *    DequantizeLinear of quantised weights fed to GroupedMatMul (the page
 *    names the composition; the affine map used is the QLinearMatMul
 *    page's (q - zero_point) * scale).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_F64 3
#define ORC_I8 4
#define ORC_U8 5
#define ORC_I32 6
#define ORC_I64 7

#define ORC_OK 0
#define ORC_ESHAPE -1
#define ORC_EBCAST -2
#define ORC_EDTYPE -3
#define ORC_EINDEX -4

#define ORC_MAXD 8

/* ---- exact element decoding ------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double orc_half(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1.f) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double orc_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double orc_ldf(const void* p, int dt, int64_t i) {
    switch (dt) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_F64: return ((const double*)p)[i];
    case ORC_F16: return orc_half(((const uint16_t*)p)[i]);
    case ORC_BF16: return orc_bf16(((const uint16_t*)p)[i]);
    }
    return NAN;
}

static int64_t orc_ldi(const void* p, int dt, int64_t i) {
    switch (dt) {
    case ORC_I8: return (int64_t)((const int8_t*)p)[i];
    case ORC_U8: return (int64_t)((const uint8_t*)p)[i];
    case ORC_I32: return (int64_t)((const int32_t*)p)[i];
    case ORC_I64: return ((const int64_t*)p)[i];
    }
    return 0;
}

/* a float-valued parameter (fp32, or fp16 which is exactly representable in fp32) */
static float orc_ldscale(const void* p, int dt, int64_t i) {
    if (dt == ORC_F32) return ((const float*)p)[i];
    return (float)orc_half(((const uint16_t*)p)[i]);
}

static int orc_is_float(int dt) { return dt == ORC_F32 || dt == ORC_F64 || dt == ORC_F16 || dt == ORC_BF16; }

/* ---- numpy.matmul geometry --------------------------------------------- */

typedef struct {
    int nb;                       /* number of output batch dims            */
    int64_t bsh[ORC_MAXD];        /* output batch shape                     */
    int64_t abs_[ORC_MAXD];       /* A element stride per output batch dim  */
    int64_t bbs[ORC_MAXD];        /* B element stride per output batch dim  */
    int64_t M, N, K;
    int a_nb;                     /* A's own number of batch dims (after promotion) */
    int64_t a_bsh[ORC_MAXD];      /* A's own batch shape */
    int drop_m, drop_n;
    int y_nd;
    int64_t y_sh[ORC_MAXD];
    int64_t total;
} orc_mm;

static int orc_mm_resolve(int a_nd, const int64_t* a_sh, int b_nd, const int64_t* b_sh, orc_mm* g) {
    int64_t as[ORC_MAXD + 1], bs[ORC_MAXD + 1];
    int an = a_nd, bn = b_nd, i;
    if (a_nd < 1 || b_nd < 1 || a_nd > ORC_MAXD || b_nd > ORC_MAXD) return ORC_ESHAPE;
    memset(g, 0, sizeof(*g));
    /* 1-D promotion: A (K,) -> (1,K); B (K,) -> (K,1) */
    if (a_nd == 1) { as[0] = 1; as[1] = a_sh[0]; an = 2; g->drop_m = 1; }
    else for (i = 0; i < a_nd; i++) as[i] = a_sh[i];
    if (b_nd == 1) { bs[0] = b_sh[0]; bs[1] = 1; bn = 2; g->drop_n = 1; }
    else for (i = 0; i < b_nd; i++) bs[i] = b_sh[i];
    g->M = as[an - 2];
    g->K = as[an - 1];
    g->N = bs[bn - 1];
    if (bs[bn - 2] != g->K) return ORC_ESHAPE;
    /* batch dims, right aligned; each pair equal or one of them 1 */
    int na = an - 2, nbb = bn - 2;
    g->nb = na > nbb ? na : nbb;
    g->a_nb = na;
    for (i = 0; i < na; i++) g->a_bsh[i] = as[i];
    /* contiguous element strides of each operand's batch dims */
    int64_t astr = g->M * g->K, bstr = g->K * g->N;
    for (i = g->nb - 1; i >= 0; i--) {
        int ia = i - (g->nb - na), ib = i - (g->nb - nbb);
        int64_t da = ia >= 0 ? as[ia] : 1, db = ib >= 0 ? bs[ib] : 1;
        if (da != db && da != 1 && db != 1) return ORC_EBCAST;
        g->bsh[i] = da > db ? da : db;
        if (da == 0 || db == 0) g->bsh[i] = 0;
        g->abs_[i] = (da == 1) ? 0 : astr;
        g->bbs[i] = (db == 1) ? 0 : bstr;
        astr *= da;
        bstr *= db;
    }
    g->y_nd = 0;
    for (i = 0; i < g->nb; i++) g->y_sh[g->y_nd++] = g->bsh[i];
    if (!g->drop_m) g->y_sh[g->y_nd++] = g->M;
    if (!g->drop_n) g->y_sh[g->y_nd++] = g->N;
    g->total = 1;
    for (i = 0; i < g->y_nd; i++) g->total *= g->y_sh[i];
    return ORC_OK;
}

/* Split an output flat index into (A batch offset, B batch offset, m, n, the
   batch coordinate vector).  Dropping a size-1 dim does not change flat order. */
static void orc_mm_split(const orc_mm* g, int64_t f, int64_t* aoff, int64_t* boff,
                         int64_t* m, int64_t* n, int64_t* coord) {
    *n = f % g->N;
    f /= g->N;
    *m = f % g->M;
    f /= g->M;
    *aoff = 0;
    *boff = 0;
    for (int i = g->nb - 1; i >= 0; i--) {
        int64_t c = f % g->bsh[i];
        f /= g->bsh[i];
        coord[i] = c;
        *aoff += c * g->abs_[i];
        *boff += c * g->bbs[i];
    }
}

int orc_matmul_shape(int a_nd, const int64_t* a_sh, int b_nd, const int64_t* b_sh,
                     int* y_nd, int64_t* y_sh) {
    orc_mm g;
    int r = orc_mm_resolve(a_nd, a_sh, b_nd, b_sh, &g);
    if (r) return r;
    *y_nd = g.y_nd;
    for (int i = 0; i < g.y_nd; i++) y_sh[i] = g.y_sh[i];
    return ORC_OK;
}

/*
 * MatMul: y[f] = sum_k A[b,m,k] * B[b,k,n] in double, t[f] = sum_k |A*B|.
 * sel: NULL for every output element in flat order, else n_sel flat indices.
 */
int orc_matmul(const void* a, int dt, int a_nd, const int64_t* a_sh,
               const void* b, int b_nd, const int64_t* b_sh,
               int64_t n_sel, const int64_t* sel, double* y, double* t, int nthreads) {
    orc_mm g;
    int r;
    if (!orc_is_float(dt)) return ORC_EDTYPE;
    r = orc_mm_resolve(a_nd, a_sh, b_nd, b_sh, &g);
    if (r) return r;
    int64_t cnt = sel ? n_sel : g.total;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t j = 0; j < cnt; j++) {
        int64_t f = sel ? sel[j] : j, ao, bo, m, n, coord[ORC_MAXD];
        orc_mm_split(&g, f, &ao, &bo, &m, &n, coord);
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < g.K; k++) {
            double p = orc_ldf(a, dt, ao + m * g.K + k) * orc_ldf(b, dt, bo + k * g.N + n);
            s += p;
            sa += fabs(p);
        }
        y[j] = s;
        if (t) t[j] = sa;
    }
    return ORC_OK;
}

/*
 * Gemm: y[m,n] = alpha * sum_k A'[m,k] B'[k,n] + beta * C[m,n] (C broadcast,
 * absent = 0).  alpha and beta are the operator's float attributes.
 */
int orc_gemm(const void* a, const int64_t* a_sh, const void* b, const int64_t* b_sh,
             const void* c, int c_nd, const int64_t* c_sh, int dt,
             float alpha, float beta, int transA, int transB,
             int64_t n_sel, const int64_t* sel, double* y, double* t, int nthreads) {
    if (!orc_is_float(dt)) return ORC_EDTYPE;
    int64_t M = transA ? a_sh[1] : a_sh[0];
    int64_t K = transA ? a_sh[0] : a_sh[1];
    int64_t Kb = transB ? b_sh[1] : b_sh[0];
    int64_t N = transB ? b_sh[0] : b_sh[1];
    if (K != Kb) return ORC_ESHAPE;
    int64_t cM = 1, cN = 1;
    if (c) {
        if (c_nd > 2 || c_nd < 0) return ORC_EBCAST;
        if (c_nd >= 1) cN = c_sh[c_nd - 1];
        if (c_nd == 2) cM = c_sh[0];
        if ((cM != 1 && cM != M) || (cN != 1 && cN != N)) return ORC_EBCAST;
    }
    int64_t cnt = sel ? n_sel : M * N;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t j = 0; j < cnt; j++) {
        int64_t f = sel ? sel[j] : j;
        int64_t m = f / N, n = f % N;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double av = orc_ldf(a, dt, transA ? k * M + m : m * K + k);
            double bv = orc_ldf(b, dt, transB ? n * K + k : k * N + n);
            double p = av * bv;
            s += p;
            sa += fabs(p);
        }
        double v = (double)alpha * s;
        if (c) v += (double)beta * orc_ldf(c, dt, (cM == 1 ? 0 : m) * cN + (cN == 1 ? 0 : n));
        y[j] = v;
        if (t) t[j] = sa;
    }
    return ORC_OK;
}

/* ---- QLinearMatMul ------------------------------------------------------ */

/*
 * Strides of a quantisation parameter over the operand's own (promoted) dims.
 * For a (row side) the parameter must broadcast to [*a_batch, M, 1]; a 1-D
 * parameter of length M (M > 1) is the per-row vector of the 2-D case.
 * For b (column side) it must broadcast to [*b_batch, 1, N]; a 1-D parameter of
 * length N is the per-column vector.  Per tensor = one element.
 * pst[0..nb) are strides over the operand's batch dims, *prow / *pcol the
 * stride along m (row side) or n (column side).
 */
static int orc_qparam(int p_nd, const int64_t* p_sh, int op_nb, const int64_t* op_bsh,
                      int64_t MN, int row_side, int64_t* pst, int64_t* pmn) {
    int64_t numel = 1;
    int i;
    for (i = 0; i < p_nd; i++) numel *= p_sh[i];
    for (i = 0; i < op_nb; i++) pst[i] = 0;
    *pmn = 0;
    if (numel == 1) return ORC_OK;
    if (p_nd == 1) {
        if (p_sh[0] != MN) return ORC_EBCAST;
        *pmn = 1;
        return ORC_OK;
    }
    /* full form: [..., M, 1] or [..., 1, N] */
    int64_t d_m = row_side ? p_sh[p_nd - 2] : p_sh[p_nd - 1];
    int64_t d_1 = row_side ? p_sh[p_nd - 1] : p_sh[p_nd - 2];
    if (d_1 != 1 || (d_m != MN && d_m != 1)) return ORC_EBCAST;
    if (p_nd - 2 > op_nb) return ORC_EBCAST;
    *pmn = (d_m == 1) ? 0 : 1;
    int64_t str = (d_m == 1) ? 1 : MN;
    for (i = p_nd - 3; i >= 0; i--) {
        int ob = op_nb - (p_nd - 2) + i;
        if (p_sh[i] != 1 && p_sh[i] != op_bsh[ob]) return ORC_EBCAST;
        pst[ob] = p_sh[i] == 1 ? 0 : str;
        str *= p_sh[i];
    }
    return ORC_OK;
}

int orc_qlinear_shape(int a_nd, const int64_t* a_sh, int b_nd, const int64_t* b_sh,
                      int* y_nd, int64_t* y_sh) {
    return orc_matmul_shape(a_nd, a_sh, b_nd, b_sh, y_nd, y_sh);
}

/*
 * QLinearMatMul.  Steps, per output element:
 *   acc  = sum_k (a - a_zp) * (b - b_zp)      exact in int64, then reduced mod 2^32
 *                                             to int32 (accumulation is the one
 *                                             place overflow is allowed, in 32 bits)
 *   mult = fp32( fp32(a_scale * b_scale) / y_scale )
 *   x    = fp32( fp32(acc) * mult )            int -> fp32 rounds to nearest even
 *   r    = rintf(x)                            ties to even (default rounding mode)
 *   q    = saturate(r + y_zero_point)          to T3's range
 * Writes q into y (T3 = y_dt), and acc into acc32 if non-NULL.
 */
int orc_qlinear_matmul(const void* a, int a_dt, int a_nd, const int64_t* a_sh,
                       const void* a_scale, int as_dt, const void* a_zp, int ap_nd, const int64_t* ap_sh,
                       const void* b, int b_dt, int b_nd, const int64_t* b_sh,
                       const void* b_scale, int bs_dt, const void* b_zp, int bp_nd, const int64_t* bp_sh,
                       const void* y_scale, int ys_dt, const void* y_zp, int y_dt,
                       int64_t n_sel, const int64_t* sel, void* y, int32_t* acc32, int nthreads) {
    orc_mm g;
    int r, i;
    if ((a_dt != ORC_I8 && a_dt != ORC_U8) || (b_dt != ORC_I8 && b_dt != ORC_U8) ||
        (y_dt != ORC_I8 && y_dt != ORC_U8))
        return ORC_EDTYPE;
    if ((as_dt != ORC_F32 && as_dt != ORC_F16) || (bs_dt != ORC_F32 && bs_dt != ORC_F16) ||
        (ys_dt != ORC_F32 && ys_dt != ORC_F16))
        return ORC_EDTYPE;
    r = orc_mm_resolve(a_nd, a_sh, b_nd, b_sh, &g);
    if (r) return r;
    /* each operand's own batch shape (after promotion) */
    int64_t b_bsh[ORC_MAXD];
    int b_nb = (b_nd == 1) ? 0 : b_nd - 2;
    for (i = 0; i < b_nb; i++) b_bsh[i] = b_sh[i];
    int64_t apst[ORC_MAXD], bpst[ORC_MAXD], apm, bpn;
    r = orc_qparam(ap_nd, ap_sh, g.a_nb, g.a_bsh, g.M, 1, apst, &apm);
    if (r) return r;
    r = orc_qparam(bp_nd, bp_sh, b_nb, b_bsh, g.N, 0, bpst, &bpn);
    if (r) return r;
    int64_t lo = (y_dt == ORC_I8) ? -128 : 0, hi = (y_dt == ORC_I8) ? 127 : 255;
    float sy = orc_ldscale(y_scale, ys_dt, 0);
    int64_t zy = orc_ldi(y_zp, y_dt, 0);
    int64_t cnt = sel ? n_sel : g.total;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t j = 0; j < cnt; j++) {
        int64_t f = sel ? sel[j] : j, ao, bo, m, n, coord[ORC_MAXD];
        orc_mm_split(&g, f, &ao, &bo, &m, &n, coord);
        /* parameter offsets: map the output batch coordinate into each operand */
        int64_t apo = m * apm, bpo = n * bpn;
        for (int d = 0; d < g.nb; d++) {
            int ia = d - (g.nb - g.a_nb), ib = d - (g.nb - b_nb);
            if (ia >= 0 && g.a_bsh[ia] != 1) apo += coord[d] * apst[ia];
            if (ib >= 0 && b_bsh[ib] != 1) bpo += coord[d] * bpst[ib];
        }
        int64_t za = orc_ldi(a_zp, a_dt, apo), zb = orc_ldi(b_zp, b_dt, bpo);
        int64_t acc = 0;
        for (int64_t k = 0; k < g.K; k++)
            acc += (orc_ldi(a, a_dt, ao + m * g.K + k) - za) * (orc_ldi(b, b_dt, bo + k * g.N + n) - zb);
        int32_t acc_w = (int32_t)(uint32_t)(uint64_t)acc;
        float sa = orc_ldscale(a_scale, as_dt, apo), sb = orc_ldscale(b_scale, bs_dt, bpo);
        float prod = sa * sb;
        float mult = prod / sy;
        float xf = (float)acc_w;
        float x = xf * mult;
        float rr = rintf(x);
        /* |rr| beyond the int range saturates anyway; clamp before the integer add */
        if (rr > 1.0e9f) rr = 1.0e9f;
        if (rr < -1.0e9f) rr = -1.0e9f;
        int64_t q = (int64_t)rr + zy;
        if (q < lo) q = lo;
        if (q > hi) q = hi;
        if (y_dt == ORC_I8) ((int8_t*)y)[j] = (int8_t)q;
        else ((uint8_t*)y)[j] = (uint8_t)q;
        if (acc32) acc32[j] = acc_w;
    }
    return ORC_OK;
}

/* ---- GroupedMatMul ------------------------------------------------------ */

/*
 * output[m, i, n] = sum_k input[m, k] * weights[g, k, n] (+ bias[g, n]),
 * g = group_indices[m, i].  Returns ORC_EINDEX if any visited g is outside
 * [0, G) (negative indices do not wrap).
 */
int orc_grouped_matmul(const void* input, const void* weights, const void* idx, int idx_dt,
                       const void* bias, int dt, int64_t M, int64_t K, int64_t G, int64_t N, int64_t S,
                       int64_t n_sel, const int64_t* sel, double* y, double* t, int nthreads) {
    if (!orc_is_float(dt)) return ORC_EDTYPE;
    if (idx_dt != ORC_I32 && idx_dt != ORC_I64) return ORC_EDTYPE;
    int64_t cnt = sel ? n_sel : M * S * N;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t j = 0; j < cnt; j++) {
        int64_t f = sel ? sel[j] : j;
        int64_t n = f % N, mi = f / N;          /* mi = m * S + i */
        int64_t m = mi / S;
        int64_t grp = orc_ldi(idx, idx_dt, mi);
        if (grp < 0 || grp >= G) {
            bad = 1;
            y[j] = NAN;
            if (t) t[j] = NAN;
            continue;
        }
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = orc_ldf(input, dt, m * K + k) * orc_ldf(weights, dt, (grp * K + k) * N + n);
            s += p;
            sa += fabs(p);
        }
        if (bias) s += orc_ldf(bias, dt, grp * N + n);
        y[j] = s;
        if (t) t[j] = sa;
    }
    return bad ? ORC_EINDEX : ORC_OK;
}

/* ---- GroupedMatMul over DequantizeLinear weights ------------------------ */

/*
 * Round a real value to the nearest value of float type dt, ties to even,
 * with IEEE gradual underflow and overflow to infinity: p significand bits,
 * emin the exponent of the smallest normal number, maxf the largest finite
 * value.  The value's leading-digit exponent fixes the spacing of the
 * representable numbers around it (fixed below emin: subnormals).
 */
static double orc_round_to(double v, int dt) {
    int p, emin;
    double maxf;
    switch (dt) {
    case ORC_F64: return v;
    case ORC_F32: p = 24; emin = -126; maxf = ldexp(2.0 - ldexp(1.0, -23), 127); break;
    case ORC_BF16: p = 8; emin = -126; maxf = ldexp(2.0 - ldexp(1.0, -7), 127); break;
    case ORC_F16: p = 11; emin = -14; maxf = 65504.0; break;
    default: return NAN;
    }
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int e;
    frexp(v, &e);  /* |v| in [2^(e-1), 2^e) */
    int ue = e - 1;
    if (ue < emin) ue = emin;
    double ulp = ldexp(1.0, ue - (p - 1));
    double r = nearbyint(v / ulp) * ulp;  /* default rounding mode: to nearest, ties to even */
    if (fabs(r) > maxf) return v > 0 ? INFINITY : -INFINITY;
    return r;
}

/*
 * Weight-only quantised experts, as the GroupedMatMul page describes them:
 * DequantizeLinear applied to quantised weights, its result fed to
 * GroupedMatMul.  The dequantised weight is the affine map the QLinearMatMul
 * page uses for its operands, (q - zero_point) * scale, held in the scale's
 * type T (so rounded once to T), with one scale and zero point per block of
 * block_size consecutive k and per column n of each group:
 *   w[g, k, n] = round_T((q[g, k, n] - zp[g, k / bs, n]) * scale[g, k / bs, n])
 *   output[m, i, n] = sum_k input[m, k] * w[g, k, n] (+ bias[g, n]),  g = group_indices[m, i]
 * scale and zp have shape (G, ceil(K / bs), N); zp NULL means 0.  q and zp are
 * int8 or uint8 (q_dt), scale, input, bias and the result of type dt.
 */
int orc_grouped_matmul_dq(const void* input, const void* qw, int q_dt, const void* scale, const void* zp,
                          int64_t bs, const void* idx, int idx_dt, const void* bias, int dt, int64_t M, int64_t K,
                          int64_t G, int64_t N, int64_t S, int64_t n_sel, const int64_t* sel, double* y, double* t,
                          int nthreads) {
    if (!orc_is_float(dt)) return ORC_EDTYPE;
    if (q_dt != ORC_I8 && q_dt != ORC_U8) return ORC_EDTYPE;
    if (idx_dt != ORC_I32 && idx_dt != ORC_I64) return ORC_EDTYPE;
    if (bs < 1) return ORC_ESHAPE;
    int64_t nkb = (K + bs - 1) / bs;
    int64_t cnt = sel ? n_sel : M * S * N;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t j = 0; j < cnt; j++) {
        int64_t f = sel ? sel[j] : j;
        int64_t n = f % N, mi = f / N;
        int64_t m = mi / S;
        int64_t grp = orc_ldi(idx, idx_dt, mi);
        if (grp < 0 || grp >= G) {
            bad = 1;
            y[j] = NAN;
            if (t) t[j] = NAN;
            continue;
        }
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; k++) {
            int64_t po = (grp * nkb + k / bs) * N + n;
            double q = (double)orc_ldi(qw, q_dt, (grp * K + k) * N + n);
            double z = zp ? (double)orc_ldi(zp, q_dt, po) : 0.0;
            double w = orc_round_to((q - z) * orc_ldf(scale, dt, po), dt);
            double p = orc_ldf(input, dt, m * K + k) * w;
            s += p;
            sa += fabs(p);
        }
        if (bias) s += orc_ldf(bias, dt, grp * N + n);
        y[j] = s;
        if (t) t[j] = sa;
    }
    return bad ? ORC_EINDEX : ORC_OK;
}

/* Exposed so a test can compare the rounding against library conversions. */
double orc_round(int dt, double v) { return orc_round_to(v, dt); }

/* Exposed so a test can compare the decoders against library conversions. */
double orc_decode(int dt, const void* p, int64_t i) { return orc_ldf(p, dt, i); }
