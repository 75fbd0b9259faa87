/*
 * Reference oracle for the fused row reductions: row softmax, LayerNorm and
 * RMSNorm over a dense row-major [M, N] matrix.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the GPU library is checked against.  It shares no code,
 * header, table or helper with the GPU library and never calls into it.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.
 *
 * Everything is computed in IEEE double precision from the exact input bits:
 * inputs stored as fp32, fp16 or bf16 are decoded exactly to double by this
 * file's own decoders, every row sum runs in element index order with
 * Neumaier's compensation (or_acc below), and results are returned as
 * doubles.  Rounding a result to the output storage type is done once, by the
 * caller's comparator, never here.  The compensation matters for long rows of
 * 16-bit inputs: their few distinct values make the rounding errors of a
 * plain running sum add up in one direction (2^28 bf16 values: about 1e-9
 * relative in LayerNorm's sum of squares), which a LayerNorm output that
 * nearly cancels (y = (x - mean) * rstd * gamma + beta close to 0) magnifies
 * beyond one unit in the last place of a bf16 result.
 *
 * Sources (cited by page title and section):
 *  - softmax: "Portable Triton Kernels" (Hugging Face kernel-builder
 *    triton-kernels skill), sections "Safe Softmax Pattern" and "Reference
 *    Kernel: Softmax"; stanleyjacob.dev Triton guide, Part II "Worked example:
 *    fused softmax".  y_j = exp(x_j - max_k x_k) / sum_k exp(x_k - max_k x_k).
 *  - RMSNorm: "Portable Triton Kernels", section "Reference Kernel: RMSNorm".
 *    variance = sum(x^2)/D, inv = 1/sqrt(variance + eps), y = x * inv * w,
 *    with w = 1 when no weight is given.
 *  - LayerNorm: named (not written out) in "Rebuilding Triton and Helion from
 *    Scratch in 4,000 Lines of Python", sections "Memory-bound kernels" and
 *    "deuteron".  No formula is printed on any page; the plainest reading is
 *    used: mean = sum(x)/N, biased variance = sum((x-mean)^2)/N,
 *    rstd = 1/sqrt(var + eps) (eps inside the root, as in the RMSNorm kernel),
 *    y = (x - mean) * rstd * gamma + beta, gamma = 1 and beta = 0 when absent.
 *  - residual add of a fused add + norm (or_add): named as a kernel pattern
 *    in "Portable Triton Kernels" (References), no formula printed; h = x + r
 *    stored in the input type, then the plain norm of that stored h.
 *  - causal scaled softmax (or_softmax_causal): attention-score rows whose
 *    keys after the query are masked; the plain softmax of the row with the
 *    masked scores at -inf, masked inputs never read, masked outputs 0.
 *  - online softmax: "Triton: Block-Level GPU Programming Without CUDA",
 *    section "How Flash Attention Uses Triton" (running max m and
 *    denominator l rescaled by alpha = exp(m_prev - m_new) per block; the
 *    Milakov & Gimelshein online normalizer), for the rows' (m, l).
 *  - attention forward (or_attention, or_attention_online): the same
 *    section's loop over key/value tiles, whose result is
 *    softmax(scale Q K^T) V with an optional causal mask.
 *
 * Special cases (readings where the pages are silent):
 *  - x_j = -inf gives exp(x_j - m) = 0 exactly (the masked-load identity of
 *    the "Safe Softmax Pattern").  A row that is entirely -inf yields NaN,
 *    exactly as the literal formula (-inf) - (-inf) does.
 *  - NaN anywhere in a softmax row makes the row max NaN and so the whole
 *    row NaN.  (Parity for NaN/inf inputs is not pinned.)
 *  - eps arrives as a C float and is widened exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's own storage-type codes. */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* Exact decode of one IEEE binary16 value to double. */
static double or_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);              /* zero or subnormal */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant | 0x400), expo - 25);
    return sign ? -v : v;
}

/* Exact decode of one bfloat16 value: it is the top half of a binary32. */
static double or_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double or_load(int dtype, const void *base, int64_t idx)
{
    switch (dtype) {
    case OR_F32: return (double)((const float *)base)[idx];
    case OR_F16: return or_half_to_double(((const uint16_t *)base)[idx]);
    case OR_BF16: return or_bf16_to_double(((const uint16_t *)base)[idx]);
    }
    return NAN;
}

/*
 * Compensated running sum (Neumaier's refinement of Kahan summation): the
 * rounding error of every addition is recovered exactly (two-sum) and
 * accumulated apart, and added back once at the end, so the error of the sum
 * stays about one rounding of the result instead of growing with the number
 * of terms.  Once the running sum is not finite it is returned as it is (the
 * plain sum's inf or NaN).  Needs strict IEEE evaluation (no reassociation,
 * no contraction), which the build flags ask for.
 */
typedef struct { double s, c; } or_acc;

static void or_acc_add(or_acc *a, double v)
{
    double t = a->s + v;
    if (isfinite(t)) {
        if (fabs(a->s) >= fabs(v))
            a->c += (a->s - t) + v;
        else
            a->c += (v - t) + a->s;
    }
    a->s = t;
}

static double or_acc_sum(const or_acc *a)
{
    return isfinite(a->s) ? a->s + a->c : a->s;
}

static int or_check(int64_t M, int64_t N, int dtype)
{
    if (M < 0 || N <= 0) return 1;
    if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return 2;
    return 0;
}

/* Decode a whole [M, N] array (or a length-N vector with M = 1) to doubles. */
int or_decode(int64_t count, int dtype, const void *x, double *out)
{
    if (count < 0) return 1;
    if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return 2;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = or_load(dtype, x, i);
    return 0;
}

/* Row softmax, plain definition: max, shift, exp, sum, divide. */
int or_softmax(int64_t M, int64_t N, int dtype, const void *x, double *y)
{
    int rc = or_check(M, N, dtype);
    if (rc) return rc;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        double *yr = y + base;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            double v = or_load(dtype, x, base + j);
            if (isnan(v) || isnan(m)) m = NAN;
            else if (v > m) m = v;
        }
        or_acc acc = {0.0, 0.0};
        for (int64_t j = 0; j < N; ++j) {
            double v = or_load(dtype, x, base + j);
            /* exp(-inf - m) is exactly 0 for finite m; for m = -inf the
             * difference is NaN, which is the all-masked row's result. */
            double e = exp(v - m);
            yr[j] = e;
            or_acc_add(&acc, e);
        }
        const double s = or_acc_sum(&acc);
        for (int64_t j = 0; j < N; ++j)
            yr[j] = yr[j] / s;
    }
    return 0;
}

/* LayerNorm over each row: returns y, and per-row mean and rstd. */
int or_layernorm(int64_t M, int64_t N, int dtype, float eps, const void *x,
                 const void *gamma, const void *beta, double *y, double *mean,
                 double *rstd)
{
    int rc = or_check(M, N, dtype);
    if (rc) return rc;
    const double deps = (double)eps;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        or_acc a1 = {0.0, 0.0};
        for (int64_t j = 0; j < N; ++j)
            or_acc_add(&a1, or_load(dtype, x, base + j));
        double mu = or_acc_sum(&a1) / (double)N;
        or_acc a2 = {0.0, 0.0};
        for (int64_t j = 0; j < N; ++j) {
            double d = or_load(dtype, x, base + j) - mu;
            or_acc_add(&a2, d * d);
        }
        double var = or_acc_sum(&a2) / (double)N;
        double rs = 1.0 / sqrt(var + deps);
        for (int64_t j = 0; j < N; ++j) {
            double g = gamma ? or_load(dtype, gamma, j) : 1.0;
            double b = beta ? or_load(dtype, beta, j) : 0.0;
            y[base + j] = (or_load(dtype, x, base + j) - mu) * rs * g + b;
        }
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return 0;
}

/* RMSNorm over each row: y = x / sqrt(mean(x^2) + eps) * w. */
int or_rmsnorm(int64_t M, int64_t N, int dtype, float eps, const void *x,
               const void *w, double *y)
{
    int rc = or_check(M, N, dtype);
    if (rc) return rc;
    const double deps = (double)eps;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        or_acc acc = {0.0, 0.0};
        for (int64_t j = 0; j < N; ++j) {
            double v = or_load(dtype, x, base + j);
            or_acc_add(&acc, v * v);
        }
        double inv = 1.0 / sqrt(or_acc_sum(&acc) / (double)N + deps);
        for (int64_t j = 0; j < N; ++j) {
            double wv = w ? or_load(dtype, w, j) : 1.0;
            y[base + j] = or_load(dtype, x, base + j) * inv * wv;
        }
    }
    return 0;
}

/*
 * Residual add: h = x + r elementwise over `count` stored values of one type,
 * the first half of a fused "add + norm" step.  The pages name a fused
 * add + norm pattern ("Portable Triton Kernels", References) and explain
 * fusion as reading each input once and writing each result once ("Triton:
 * Block-Level GPU Programming Without CUDA", kernel fusion), but print no
 * formula.  Reading taken: the updated residual stream h is stored in the
 * input type, rounded once from the exact sum (by the caller's comparator),
 * and the norm is the plain norm of that stored h.  The double sum returned
 * here rounds to the storage type exactly as the exact real sum does: double
 * has at least 29 more significand bits than any storage type, so when the
 * sum is not exact in double its error is far below the distance to the
 * nearest storage-type rounding boundary.
 */
int or_add(int64_t count, int dtype, const void *x, const void *r, double *h)
{
    if (count < 0 || (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16)) return 1;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        h[i] = or_load(dtype, x, i) + or_load(dtype, r, i);
    return 0;
}

/*
 * Causal, scaled row softmax (attention scores): row r holds the scores of
 * query q = r mod `queries` against N keys, and key k is visible to it iff
 * k <= q + offset.  Over the visible keys, with s = scale:
 *   m = max_k s*x[r,k],  y[r,k] = exp(s*x[r,k] - m) / sum_k exp(s*x[r,k] - m),
 * and y = 0 at masked keys, whose inputs are never read.  This is the plain
 * softmax of the row with its masked scores set to -inf: the masked-load
 * identity of "Portable Triton Kernels" ("Safe Softmax Pattern": a -inf
 * entry contributes exactly nothing), with the causal pattern of attention
 * scores (keys after the query masked, the diagonal kept).  `scale` arrives
 * as a C float and is widened exactly.
 */
int or_softmax_causal(int64_t M, int64_t N, int dtype, float scale, int64_t queries,
                      int64_t offset, const void *x, double *y)
{
    int rc = or_check(M, N, dtype);
    if (rc) return rc;
    if (queries <= 0 || offset < 0) return 1;
    const double sc = (double)scale;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        int64_t q = r % queries;
        int64_t vis = q + offset + 1;            /* keys 0 .. vis-1 are visible */
        if (vis > N) vis = N;
        double m = -INFINITY;
        for (int64_t k = 0; k < vis; ++k) {
            double v = sc * or_load(dtype, x, base + k);
            if (isnan(v) || isnan(m)) m = NAN;
            else if (v > m) m = v;
        }
        or_acc acc = {0.0, 0.0};
        for (int64_t k = 0; k < vis; ++k) {
            double v = sc * or_load(dtype, x, base + k);
            or_acc_add(&acc, (v == -INFINITY) ? 0.0 : exp(v - m));
        }
        const double s = or_acc_sum(&acc);
        for (int64_t k = 0; k < vis; ++k) {
            double v = sc * or_load(dtype, x, base + k);
            y[base + k] = ((v == -INFINITY) ? 0.0 : exp(v - m)) / s;
        }
        for (int64_t k = vis; k < N; ++k) y[base + k] = 0.0;
    }
    return 0;
}

/*
 * Online softmax: the row is visited in consecutive blocks of `block`
 * elements.  Per block, in the page's order: new running max
 * m_new = max(m_prev, max(block)); rescale factor alpha = exp(m_prev - m_new);
 * l = l_prev * alpha + sum(exp(block - m_new)).  After the last block,
 * y_j = exp(x_j - m) / l.  In real arithmetic this equals the plain softmax.
 *
 * Reading: while the running max is still -inf no mass has been seen, so
 * alpha is taken as 1 (the page's formula would give exp(-inf + inf) = NaN
 * for a fully masked leading block, a case attention kernels never reach).
 */
int or_softmax_online(int64_t M, int64_t N, int dtype, int64_t block,
                      const void *x, double *y)
{
    int rc = or_check(M, N, dtype);
    if (rc) return rc;
    if (block <= 0) return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        double m_prev = -INFINITY, l_prev = 0.0;
        for (int64_t j0 = 0; j0 < N; j0 += block) {
            int64_t j1 = j0 + block < N ? j0 + block : N;
            double bmax = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) {
                double v = or_load(dtype, x, base + j);
                if (isnan(v) || isnan(bmax)) bmax = NAN;
                else if (v > bmax) bmax = v;
            }
            double m_new = (isnan(bmax) || isnan(m_prev)) ? NAN
                           : (bmax > m_prev ? bmax : m_prev);
            double alpha = (m_prev == -INFINITY) ? 1.0 : exp(m_prev - m_new);
            double psum = 0.0;
            if (m_new != -INFINITY)
                for (int64_t j = j0; j < j1; ++j)
                    psum += exp(or_load(dtype, x, base + j) - m_new);
            l_prev = l_prev * alpha + psum;
            m_prev = m_new;
        }
        for (int64_t j = 0; j < N; ++j)
            y[base + j] = exp(or_load(dtype, x, base + j) - m_prev) / l_prev;
    }
    return 0;
}

/*
 * Attention forward, plain definition.  BH independent heads; q is
 * [BH, Lq, D], k and v are [BH, Lk, D], row-major, one storage type.  For
 * head b and query i the visible keys are j < Lk, and when `causal` only
 * j <= i + offset (offset 0: square causal attention, the diagonal kept;
 * Lk - Lq aligns the last query with the last key).  With
 *   s_j = scale * sum_c q[b,i,c] k[b,j,c]      over the visible keys,
 *   m = max_j s_j,  w_j = exp(s_j - m),
 *   o[b,i,c] = sum_j w_j v[b,j,c] / sum_j w_j.
 * "Triton: Block-Level GPU Programming Without CUDA", section "How Flash
 * Attention Uses Triton", prints the tiled loop that computes this without
 * materializing the scores (Q K^T tile, running max, rescale of the
 * accumulator, P V tile); in real arithmetic the loop's result is this
 * softmax(scale Q K^T) V, which is written out here with every sum
 * compensated and in index order.  The page's loop applies no scale; scale
 * (1/sqrt(D) in attention) is an argument and 1 gives the page's scores.
 * `rows` lists the rows b*Lq + i to compute (NULL: all BH*Lq in order);
 * o receives nrows rows of D doubles in that order.  `oabs` (NULL: not
 * computed) receives, in the same layout, sum_j w_j |v[b,j,c]| / sum_j w_j:
 * the size of the terms each output sums, the scale of the error a finite-
 * precision evaluation of the sums can make.
 */
int or_attention(int64_t BH, int64_t Lq, int64_t Lk, int64_t D, int dtype, float scale, int causal,
                 int64_t offset, const void *q, const void *k, const void *v, int64_t nrows,
                 const int64_t *rows, double *o, double *oabs)
{
    if (BH < 0 || Lq < 0 || Lk < 1 || D < 1 || offset < 0) return 1;
    if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return 2;
    if (!rows) nrows = BH * Lq;
    const double sc = (double)scale;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t n = 0; n < nrows; ++n) {
        const int64_t row = rows ? rows[n] : n;
        if (row < 0 || row >= BH * Lq) { bad = 1; continue; }
        const int64_t b = row / Lq, i = row % Lq;
        int64_t vis = Lk;
        if (causal && i + offset + 1 < vis) vis = i + offset + 1;
        double *s = (double *)malloc((size_t)vis * sizeof(double));
        if (!s) { bad = 1; continue; }
        double m = -INFINITY;
        for (int64_t j = 0; j < vis; ++j) {
            or_acc dot = {0.0, 0.0};
            for (int64_t c = 0; c < D; ++c)
                or_acc_add(&dot, or_load(dtype, q, row * D + c) * or_load(dtype, k, (b * Lk + j) * D + c));
            s[j] = sc * or_acc_sum(&dot);
            if (s[j] > m) m = s[j];
        }
        or_acc l = {0.0, 0.0};
        for (int64_t j = 0; j < vis; ++j) {
            s[j] = exp(s[j] - m);
            or_acc_add(&l, s[j]);
        }
        const double ls = or_acc_sum(&l);
        for (int64_t c = 0; c < D; ++c) {
            or_acc acc = {0.0, 0.0}, aab = {0.0, 0.0};
            for (int64_t j = 0; j < vis; ++j) {
                const double vj = or_load(dtype, v, (b * Lk + j) * D + c);
                or_acc_add(&acc, s[j] * vj);
                if (oabs) or_acc_add(&aab, s[j] * fabs(vj));
            }
            o[n * D + c] = or_acc_sum(&acc) / ls;
            if (oabs) oabs[n * D + c] = or_acc_sum(&aab) / ls;
        }
        free(s);
    }
    return bad ? 3 : 0;
}

/*
 * Attention forward in the page's tiled order ("How Flash Attention Uses
 * Triton"): per query row the visible keys are taken in consecutive blocks
 * of `block`; per block, the block's scores s_j, then m_new = max(m_prev,
 * max_j s_j), alpha = exp(m_prev - m_new), p_j = exp(s_j - m_new),
 * acc = acc * alpha + sum_j p_j v_j, l = l * alpha + sum_j p_j, m_prev =
 * m_new; finally o = acc / l.  Plain (uncompensated) sums in that order.  In
 * real arithmetic it equals or_attention; it is kept as the page's own form
 * of the algorithm and pinned against the plain definition.  Reading, as in
 * or_softmax_online: alpha = 1 while the running max is still -inf.
 */
int or_attention_online(int64_t BH, int64_t Lq, int64_t Lk, int64_t D, int dtype, float scale, int causal,
                        int64_t offset, int64_t block, const void *q, const void *k, const void *v,
                        double *o)
{
    if (BH < 0 || Lq < 0 || Lk < 1 || D < 1 || offset < 0 || block < 1) return 1;
    if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return 2;
    const double sc = (double)scale;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t row = 0; row < BH * Lq; ++row) {
        const int64_t b = row / Lq, i = row % Lq;
        int64_t vis = Lk;
        if (causal && i + offset + 1 < vis) vis = i + offset + 1;
        double *acc = (double *)calloc((size_t)D, sizeof(double));
        double *s = (double *)malloc((size_t)block * sizeof(double));
        if (!acc || !s) { free(acc); free(s); bad = 1; continue; }
        double m_prev = -INFINITY, l_prev = 0.0;
        for (int64_t j0 = 0; j0 < vis; j0 += block) {
            const int64_t j1 = j0 + block < vis ? j0 + block : vis;
            double bmax = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < D; ++c)
                    dot += or_load(dtype, q, row * D + c) * or_load(dtype, k, (b * Lk + j) * D + c);
                s[j - j0] = sc * dot;
                if (s[j - j0] > bmax) bmax = s[j - j0];
            }
            const double m_new = bmax > m_prev ? bmax : m_prev;
            const double alpha = (m_prev == -INFINITY) ? 1.0 : exp(m_prev - m_new);
            double psum = 0.0;
            for (int64_t c = 0; c < D; ++c) acc[c] *= alpha;
            for (int64_t j = j0; j < j1; ++j) {
                const double p = exp(s[j - j0] - m_new);
                psum += p;
                for (int64_t c = 0; c < D; ++c) acc[c] += p * or_load(dtype, v, (b * Lk + j) * D + c);
            }
            l_prev = l_prev * alpha + psum;
            m_prev = m_new;
        }
        for (int64_t c = 0; c < D; ++c) o[row * D + c] = acc[c] / l_prev;
        free(acc);
        free(s);
    }
    return bad ? 3 : 0;
}

/* Sets the number of OpenMP threads later parallel regions use (n >= 1);
 * timing only, the results do not depend on it. */
void or_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of OpenMP threads a parallel region of this library will use. */
int or_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
