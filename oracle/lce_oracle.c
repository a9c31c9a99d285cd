/*
 * lce_oracle.c -- the CPU oracle for vocabulary-wide cross-entropy.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link or call this file.  Only the tests,
 * the smoke check and the bench's CPU-baseline leg use it.  It shares no code,
 * header, table or constant with the GPU kernels.
 *
 * Plain, slow, obviously correct: every quantity is the textbook definition,
 * evaluated in IEEE double precision with libm (build WITHOUT -ffast-math).
 * Rows are independent, so the only parallelism is a plain OpenMP loop over
 * rows; inside a row the loops run in index order.
 *
 * What it follows (pages are cited by title and section):
 *  - "Add Megatron-LM cross-entropy integration" (Liger-Kernel PR), Summary:
 *    cross-entropy over the vocabulary with ignore_index=-100 and a
 *    label_smoothing argument; the gradient is written in place and no full
 *    softmax is kept.  Test setup: every provider computes the same operation
 *    as torch.nn.functional.cross_entropy, which fixes the smoothing form
 *    (a uniform eps/V over all V classes, the target included) and the mean
 *    over non-ignored tokens.
 *  - "Add opt-in Liger vocab-parallel cross entropy" (Megatron-LM PR), "What
 *    does this PR do?": fp32 per-token losses, an arbitrary upstream gradient,
 *    and the argmax of the original logits with smallest-index ties.
 *  - "Add Liger Kernel support for Muse Glimmer" (Liger-Kernel PR), Summary and
 *    Details/Softcap: token accuracy, the fused linear variant that never
 *    forms the [tokens, V] logits, the softcap T*tanh(x/T), and grad_weight
 *    accumulated in fp32.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *  - softcap T == 0 means "off"; its derivative is sech^2(x/T) = 1 - tanh^2(x/T)
 *    (chain rule on T*tanh(x/T)).
 *  - a label outside [0, V) that is not ignore_index is counted as "bad" and
 *    treated exactly like an ignored token.
 *  - mean over zero valid tokens gives loss 0 and all-zero gradients.
 *  - the argmax is over the raw stored logits (tanh is strictly increasing, so
 *    it is also the argmax of the capped logits) and is computed for every
 *    row, ignored rows included.
 *  - the target column of the gradient uses p_y - 1 = -sum_{j != y} p_j, the
 *    same number written without the cancellation that 1 - p_y suffers when
 *    p_y is close to 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };
enum { OR_RED_NONE = 0, OR_RED_MEAN = 1, OR_RED_SUM = 2 };

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == OR_BF16) return bf16_to_double(((const uint16_t *)base)[idx]);
    if (dtype == OR_F32) return (double)((const float *)base)[idx];
    return ((const double *)base)[idx];
}

/* Round a double to the nearest bfloat16, ties to even, in one step (no
 * intermediate float).  bf16 keeps 8 significant bits and the binary32
 * exponent range; below 2^-126 the spacing is fixed at 2^-133. */
uint16_t lce_oracle_bf16_from_double(double v)
{
    uint32_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return 0x7fc0;
    if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
    if (a == 0.0) return (uint16_t)sign;
    int e;
    frexp(a, &e);                       /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                      /* spacing of 8-bit significands */
    if (q < -133) q = -133;             /* subnormal spacing */
    double m = ldexp(a, -q);            /* exact: scaling by a power of two */
    double r = nearbyint(m);            /* default rounding mode: ties to even */
    double rv = ldexp(r, q);
    if (rv >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80u); /* past 0x1.fep127 */
    float f = (float)rv;                /* exact: rv has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7fffu));
}

void lce_oracle_round_bf16(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = lce_oracle_bf16_from_double(in[i]);
}

/* Step 1 of the definition: which tokens count.  A label equal to
 * ignore_index is ignored; a label outside [0, V) is "bad" and also
 * contributes nothing. */
static int label_is_valid(int64_t y, int64_t V, int64_t ignore_index)
{
    return y != ignore_index && y >= 0 && y < V;
}

void lce_oracle_count(const int64_t *labels, int64_t n, int64_t V, int64_t ignore_index,
                      int64_t *n_valid, int64_t *n_bad)
{
    int64_t nv = 0, nb = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t y = labels[i];
        if (label_is_valid(y, V, ignore_index)) ++nv;
        else if (y != ignore_index) ++nb;
    }
    *n_valid = nv;
    *n_bad = nb;
}

/* The per-token gradient multiplier: dL/dloss_i.  mean: g / n_valid (0 when
 * no token counts); sum: g; none: g_i.  g defaults to 1. */
static double token_scale(int reduction, const double *grad_out, int64_t i, int64_t n_valid)
{
    if (reduction == OR_RED_NONE) return grad_out ? grad_out[i] : 1.0;
    double g = grad_out ? grad_out[0] : 1.0;
    if (reduction == OR_RED_MEAN) return n_valid > 0 ? g / (double)n_valid : 0.0;
    return g;
}

/*
 * One row of the definition.  x: the raw row (V doubles).  Writes the loss,
 * the argmax and (if grad != NULL) the V gradient entries, unrounded.
 */
static void ce_row(const double *x, int64_t V, int64_t y, int valid, double eps, double T,
                   double scale, double *loss, int64_t *argmax, double *grad, double *z)
{
    /* argmax over the raw stored values; strict '>' keeps the first index. */
    int64_t am = 0;
    for (int64_t j = 1; j < V; ++j)
        if (x[j] > x[am]) am = j;
    *argmax = am;

    /* capped logits z = T*tanh(x/T), or x itself when the cap is off */
    for (int64_t j = 0; j < V; ++j) z[j] = T > 0.0 ? T * tanh(x[j] / T) : x[j];

    if (!valid) {
        *loss = 0.0;
        if (grad)
            for (int64_t j = 0; j < V; ++j) grad[j] = 0.0;
        return;
    }

    /* log-sum-exp, two plain passes: max, then sum of shifted exponentials */
    double m = z[0];
    for (int64_t j = 1; j < V; ++j)
        if (z[j] > m) m = z[j];
    double s = 0.0, s_other = 0.0, zsum = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        double e = exp(z[j] - m);
        s += e;
        if (j != y) s_other += e;
        zsum += z[j];
    }
    double lse = m + log(s);

    /* loss = (1-eps)(-log p_y) + (eps/V) sum_j (-log p_j)
     *      = lse - (1-eps) z_y - (eps/V) sum_j z_j                     */
    *loss = lse - (1.0 - eps) * z[y] - (eps / (double)V) * zsum;

    if (!grad) return;
    for (int64_t j = 0; j < V; ++j) {
        /* d loss / d z_j = p_j - (1-eps)[j==y] - eps/V */
        double dz;
        if (j == y) {
            /* p_y - (1-eps) = -(sum_{k!=y} p_k) + eps */
            dz = -(s_other / s) + eps - eps / (double)V;
        } else {
            dz = exp(z[j] - lse) - eps / (double)V;
        }
        double chain = 1.0;
        if (T > 0.0) {
            /* d(T tanh(x/T))/dx = sech^2(x/T) = 1 - tanh^2(x/T); the sech form keeps
             * its value where 1 - tanh^2 would cancel to 0 (|x/T| > ~19) */
            double c = cosh(x[j] / T);
            chain = 1.0 / (c * c);
        }
        grad[j] = scale * dz * chain;
    }
}

/*
 * Cross-entropy forward + backward over the rows listed in `rows` (all n rows
 * when rows == NULL, in which case nrows must equal n).
 *
 *   logits   : [n, ld] in dtype (0 f32, 1 bf16, 2 f64), row-major
 *   labels   : [n] int64
 *   grad_out : NULL (= 1.0), a scalar for mean/sum, or [n] for none
 *   loss_rows, argmax_rows : [nrows]   (argmax_rows may be NULL)
 *   grad_rows: [nrows, V] unrounded fp64 gradient, or NULL
 *   counts   : [3] = {n_valid over all n, n_correct over the evaluated rows,
 *                     n_bad over all n}
 * Returns 0, or -1 on an argument error.
 */
int lce_oracle_ce(const void *logits, int64_t ld, int dtype, const int64_t *labels, int64_t n,
                  int64_t V, int64_t ignore_index, double eps, double softcap, int reduction,
                  const double *grad_out, const int64_t *rows, int64_t nrows, double *loss_rows,
                  int64_t *argmax_rows, double *grad_rows, int64_t *counts, int nthreads)
{
    if (n < 0 || V < 1 || ld < V || !labels || !loss_rows || !counts) return -1;
    if (!rows && nrows != n) return -1;
    int64_t n_valid, n_bad;
    lce_oracle_count(labels, n, V, ignore_index, &n_valid, &n_bad);
    int64_t n_correct = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(+ : n_correct)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)V);
        double *z = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = rows ? rows[r] : r;
            for (int64_t j = 0; j < V; ++j) x[j] = load_elem(logits, dtype, i * ld + j);
            int64_t y = labels[i];
            int valid = label_is_valid(y, V, ignore_index);
            double scale = token_scale(reduction, grad_out, i, n_valid);
            int64_t am;
            ce_row(x, V, y, valid, eps, softcap, scale, &loss_rows[r], &am,
                   grad_rows ? grad_rows + r * V : NULL, z);
            if (argmax_rows) argmax_rows[r] = am;
            if (valid && am == y) n_correct += 1;
        }
        free(x);
        free(z);
    }
    counts[0] = n_valid;
    counts[1] = n_correct;
    counts[2] = n_bad;
    return 0;
}

/* The reduced loss: mean over valid tokens (0 when there are none) or sum. */
double lce_oracle_reduce_loss(const double *loss_tok, int64_t n, int64_t n_valid, int reduction)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += loss_tok[i];
    if (reduction == OR_RED_MEAN) return n_valid > 0 ? s / (double)n_valid : 0.0;
    return s;
}

/*
 * Fused linear cross-entropy ("Add Liger Kernel support for Muse Glimmer",
 * Summary and Memory): the loss of the logits Z = hidden * weight^T without
 * forming Z for all tokens at once.  The oracle does not chunk: it forms each
 * row of Z in fp64 (bf16 products are exact in fp64), runs the row
 * definition above on it, and accumulates
 *     grad_hidden = G * weight,   grad_weight = G^T * hidden
 * with G the unrounded fp64 logit gradient.  Any output multiplier is folded
 * into hidden by the caller (Details/Softcap), so hidden is used as given.
 *
 *   hidden [n, H] bf16, weight [V, H] bf16, labels [n]
 *   loss_tok [n], grad_hidden [n, H], grad_weight [V, H] (fp64, overwritten)
 *   counts [3] as for lce_oracle_ce (argmax over Z rows)
 */
int lce_oracle_flce(const uint16_t *hidden, const uint16_t *weight, const int64_t *labels,
                    int64_t n, int64_t H, int64_t V, int64_t ignore_index, double eps,
                    double softcap, int reduction, const double *grad_out, double *loss_tok,
                    double *loss_out, double *grad_hidden, double *grad_weight, int64_t *counts,
                    int nthreads)
{
    if (n < 0 || H < 1 || V < 1 || !hidden || !weight || !labels || !loss_tok || !counts)
        return -1;
    int64_t n_valid, n_bad;
    lce_oracle_count(labels, n, V, ignore_index, &n_valid, &n_bad);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    double *h = (double *)malloc(sizeof(double) * (size_t)(n * H));
    double *w = (double *)malloc(sizeof(double) * (size_t)(V * H));
    double *g = (double *)malloc(sizeof(double) * (size_t)(n * V));
    for (int64_t k = 0; k < n * H; ++k) h[k] = bf16_to_double(hidden[k]);
    for (int64_t k = 0; k < V * H; ++k) w[k] = bf16_to_double(weight[k]);
    int64_t n_correct = 0;
#pragma omp parallel reduction(+ : n_correct)
    {
        double *zrow = (double *)malloc(sizeof(double) * (size_t)V);
        double *ztmp = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t v = 0; v < V; ++v) {
                double acc = 0.0;
                for (int64_t k = 0; k < H; ++k) acc += h[i * H + k] * w[v * H + k];
                zrow[v] = acc;
            }
            int64_t y = labels[i];
            int valid = label_is_valid(y, V, ignore_index);
            double scale = token_scale(reduction, grad_out, i, n_valid);
            int64_t am;
            ce_row(zrow, V, y, valid, eps, softcap, scale, &loss_tok[i], &am, g + i * V, ztmp);
            if (valid && am == y) n_correct += 1;
        }
        free(zrow);
        free(ztmp);
    }
    if (grad_hidden) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t k = 0; k < H; ++k) {
                double acc = 0.0;
                for (int64_t v = 0; v < V; ++v) acc += g[i * V + v] * w[v * H + k];
                grad_hidden[i * H + k] = acc;
            }
    }
    if (grad_weight) {
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v)
            for (int64_t k = 0; k < H; ++k) {
                double acc = 0.0;
                for (int64_t i = 0; i < n; ++i) acc += g[i * V + v] * h[i * H + k];
                grad_weight[v * H + k] = acc;
            }
    }
    if (loss_out) *loss_out = lce_oracle_reduce_loss(loss_tok, n, n_valid, reduction);
    counts[0] = n_valid;
    counts[1] = n_correct;
    counts[2] = n_bad;
    free(h);
    free(w);
    free(g);
    return 0;
}

/*
 * Per-row statistics of the softmax over z = T tanh(x/T) (or x when T = 0),
 * by definition, for the rows listed in `rows` (all n rows when rows == NULL):
 *   lse_i     = log sum_j exp(z_ij)
 *   logp_i    = log p_{i,y_i} = z_{i,y_i} - lse_i      (0 for an ignored row)
 *   entropy_i = -sum_j p_ij log p_ij                   (every row)
 * The target log-probability and the entropy are the RL-side quantities of
 * labs-molt PR "Enable Liger layers" (Why attention, RoPE, and RL loss stay in
 * Molt; Validation / Correctness); lse is what a forward pass keeps for a
 * deferred backward.  Any of the three outputs may be NULL.
 */
int lce_oracle_row_stats(const void *logits, int64_t ld, int dtype, const int64_t *labels, int64_t n,
                         int64_t V, int64_t ignore_index, double softcap, const int64_t *rows,
                         int64_t nrows, double *lse_out, double *logp_out, double *entropy_out,
                         int nthreads)
{
    if (n < 0 || V < 1 || ld < V || !logits || !labels || (!rows && nrows != n)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= n)) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t row_i = rows ? rows[r] : r;
            for (int64_t j = 0; j < V; ++j) {
                double x = load_elem(logits, dtype, row_i * ld + j);
                z[j] = softcap > 0.0 ? softcap * tanh(x / softcap) : x;
            }
            double m = z[0];
            for (int64_t j = 1; j < V; ++j)
                if (z[j] > m) m = z[j];
            double s = 0.0;
            for (int64_t j = 0; j < V; ++j) s += exp(z[j] - m);
            const double lse_r = m + log(s);
            double h = 0.0;   /* -sum p log p with log p_j = z_j - lse */
            for (int64_t j = 0; j < V; ++j) {
                double lp = z[j] - lse_r;
                h -= exp(lp) * lp;
            }
            const int64_t y = labels[row_i];
            if (lse_out) lse_out[r] = lse_r;
            if (logp_out) logp_out[r] = label_is_valid(y, V, ignore_index) ? z[y] - lse_r : 0.0;
            if (entropy_out) entropy_out[r] = h;
        }
        free(z);
    }
    return 0;
}

/* Version tag so the Python side can check it loaded this file's build. */
int lce_oracle_abi_version(void) { return 2; }
