/*
 * oracle.c -- plain fp64 CPU reference for the selective state-space scan
 * (the S6 core of Mamba) and its single-token recurrent decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code with the HIP library.
 *
 * What it computes, and where the pages fix it:
 *   - zero-order-hold discretisation of a diagonal continuous SSM
 *     h'(t) = A h(t) + B x(t):  Abar = exp(delta*A),  Bbar = (Abar-1)/A * B
 *     (ultralytics glossary "State Space Models (SSM)", section "SSMの仕組み";
 *     paperlens tutorial "Mamba と状態空間モデル", eq.(2) and the prose under it;
 *     ihouse article on Mamba-3, discretisation paragraph: Mamba uses ZOH);
 *   - Delta, B and C are per token, A is fixed per (channel, state)
 *     (paperlens tutorial, section "Mamba: 状態を「選択的」にする");
 *   - the recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t, evaluated strictly in
 *     sequence over t, state updated first and read afterwards
 *     (ultralytics glossary, recurrent form of the worked example);
 *   - the readout y_t = C_t . h_t + D x_t (ultralytics glossary, intro
 *     paragraph; ihouse article, the state and output equations);
 *   - the output gate y * SiLU(z) of the Mamba block (agenticai-flow guide,
 *     section "アーキテクチャ図解": S6 output times SiLU of the z branch);
 *   - variants (oracle_scan_ex): the Euler rule Bbar = delta * B with
 *     Abar = exp(delta*A) (paperlens tutorial, the selection pseudo-code;
 *     ihouse article: Mamba-2 simplified the discretisation this way), and A
 *     as one value per channel shared by its states (ihouse article, section
 *     on Mamba-2's scalar A; ultralytics glossary, S4-to-Mamba section).
 *
 * Readings taken where the pages are silent:
 *   - A == 0 uses the continuous limit of (exp(delta*A)-1)/A, which is delta;
 *   - D and the gate are optional (NULL pointer = D of zero / no gate);
 *   - the gate multiplies the D*x term as well;
 *   - SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v)) (textbook definition).
 *
 * Precision: every quantity is widened to double on entry and all arithmetic
 * is double; results are returned as double.  Build with gcc -O2, no
 * -ffast-math, -ffp-contract=off.
 *
 * Layouts (row-major, contiguous):
 *   x, delta, z, y : [batch, seqlen, dim]
 *   B, C           : [batch, seqlen, dstate]   (shared by every channel)
 *   A              : [dim, dstate]   ([dim] with a_per_channel)
 *   Dskip          : [dim]
 *   h0, h_last, h  : [batch, dim, dstate]
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* SiLU(v) = v * sigmoid(v). */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/*
 * Zero-order hold for one diagonal entry a = A[d,n] and step size delta:
 *   *abar      = exp(delta * a)
 *   *bbar_coef = (exp(delta * a) - 1) / a      (so that Bbar = bbar_coef * B)
 * expm1 gives exp(u)-1 without cancellation for small |u|; at a == 0 the
 * coefficient takes its limit, delta.
 */
static void zoh(double delta, double a, double *abar, double *bbar_coef) {
    double u = delta * a;
    *abar = exp(u);
    *bbar_coef = (a != 0.0) ? expm1(u) / a : delta;
}

/* Exposed so that tests can check the discretisation on its own. */
void oracle_zoh(double delta, double a, double *abar, double *bbar_coef) {
    zoh(delta, a, abar, bbar_coef);
}

/*
 * Euler rule for one diagonal entry: Abar = exp(delta * a) as in the zero-
 * order hold, Bbar = delta * B.
 */
static void euler(double delta, double a, double *abar, double *bbar_coef) {
    *abar = exp(delta * a);
    *bbar_coef = delta;
}

/*
 * One channel (b, d) over the whole sequence: a plain loop over t.
 * h is the channel's state, length dstate, updated in place.  a_row points
 * at the channel's dstate values of A, a_step is 1 (A[d, n]) or 0 (one A[d]
 * for every state); disc picks the discretisation rule.
 */
static void scan_channel(int64_t b, int64_t d, int64_t seqlen, int64_t dim,
                         int64_t dstate, const double *x, const double *delta,
                         const double *a_row, int64_t a_step,
                         void (*disc)(double, double, double *, double *),
                         const double *B, const double *C,
                         const double *Dskip, const double *z, double *h,
                         double *y) {
    double dval = Dskip ? Dskip[d] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
        int64_t io = (b * seqlen + t) * dim + d;     /* [b, t, d]  */
        int64_t bc = (b * seqlen + t) * dstate;      /* [b, t, 0]  */
        double xv = x[io];
        double dv = delta[io];

        /* state update first: h_t = Abar_t h_{t-1} + Bbar_t x_t */
        for (int64_t n = 0; n < dstate; ++n) {
            double abar, bcoef;
            disc(dv, a_row[n * a_step], &abar, &bcoef);
            h[n] = abar * h[n] + bcoef * B[bc + n] * xv;
        }

        /* then the readout of the new state, the skip term and the gate */
        double s = 0.0;
        for (int64_t n = 0; n < dstate; ++n) s += C[bc + n] * h[n];
        double pre = s + dval * xv;
        y[io] = z ? pre * silu(z[io]) : pre;
    }
}

/*
 * Full scan.  Channels are independent, so they are spread over nthreads
 * host threads (nthreads <= 0 means all available); within a channel the
 * loop over t is strictly sequential.  a_per_channel: A is [dim] instead of
 * [dim, dstate]; use_euler: Bbar = delta * B instead of the zero-order hold.
 */
int oracle_scan_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                   const double *x, const double *delta, const double *A,
                   int a_per_channel, int use_euler,
                   const double *B, const double *C, const double *Dskip,
                   const double *z, const double *h0, double *y, double *h_last,
                   int nthreads) {
    if (batch < 0 || seqlen < 0 || dim < 0 || dstate <= 0) return ORACLE_EINVAL;
    if (batch == 0 || dim == 0) return ORACLE_OK;
    if (!A || (seqlen > 0 && (!x || !delta || !B || !C || !y)))
        return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    int64_t nch = batch * dim;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t b = ch / dim, d = ch % dim;
        double *h = (double *)malloc((size_t)dstate * sizeof(double));
        for (int64_t n = 0; n < dstate; ++n)
            h[n] = h0 ? h0[ch * dstate + n] : 0.0;
        const double *a_row = a_per_channel ? A + d : A + d * dstate;
        scan_channel(b, d, seqlen, dim, dstate, x, delta, a_row, a_per_channel ? 0 : 1,
                     use_euler ? euler : zoh, B, C, Dskip, z, h, y);
        if (h_last)
            for (int64_t n = 0; n < dstate; ++n) h_last[ch * dstate + n] = h[n];
        free(h);
    }
    return ORACLE_OK;
}

/* The scan of the method as written: A [dim, dstate], zero-order hold. */
int oracle_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                const double *x, const double *delta, const double *A,
                const double *B, const double *C, const double *Dskip,
                const double *z, const double *h0, double *y, double *h_last,
                int nthreads) {
    return oracle_scan_ex(batch, seqlen, dim, dstate, x, delta, A, 0, 0, B, C, Dskip, z,
                          h0, y, h_last, nthreads);
}

/*
 * One recurrent decode step: the loop body of the scan applied once per
 * channel to a resident state h [batch, dim, dstate] (updated in place).
 * x, delta, z, y are [batch, dim]; B, C are [batch, dstate].
 */
int oracle_decode_step(int64_t batch, int64_t dim, int64_t dstate, double *h,
                       const double *x, const double *delta, const double *A,
                       const double *B, const double *C, const double *Dskip,
                       const double *z, double *y) {
    if (batch < 0 || dim < 0 || dstate <= 0) return ORACLE_EINVAL;
    if (batch == 0 || dim == 0) return ORACLE_OK;
    if (!h || !x || !delta || !A || !B || !C || !y) return ORACLE_EINVAL;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < dim; ++d)
            /* a decode step is a scan of length 1 over this channel's state */
            scan_channel(0, d, 1, dim, dstate, x + b * dim, delta + b * dim,
                         A + d * dstate, 1, zoh, B + b * dstate, C + b * dstate, Dskip,
                         z ? z + b * dim : NULL, h + (b * dim + d) * dstate,
                         y + b * dim);
    return ORACLE_OK;
}

/*
 * Prologue of the selective scan inside a Mamba block (the step right before
 * the scan), evaluated on its own so that a fused GPU kernel can be checked
 * against (prologue -> scan) in fp64.
 *
 *  - causal depthwise convolution over time (paperlens tutorial, section
 *    "現場ではこう使う": a short 1-D convolution of width d_conv in front of
 *    the SSM; agenticai-flow guide, implementation example: d_conv = 4,
 *    installed as the causal-conv1d package).  Each channel d has its own
 *    d_conv taps; tap k multiplies the input d_conv-1-k steps back, so
 *    w[d, d_conv-1] multiplies the current step.  Steps before the start of
 *    the sequence are zero.  Optional bias, optional SiLU of the result (the
 *    pages do not say whether an activation follows the convolution).
 *      xc[b,t,d] = act( sum_k w[d,k] * x_raw[b, t-(d_conv-1)+k, d] + bias[d] )
 *
 *  - step size (paperlens tutorial, section "Mamba: 状態を「選択的」にする":
 *    delta is a softplus of a per-token projection plus a bias):
 *      delta[b,t,d] = softplus(delta_raw[b,t,d] + delta_bias[d]),
 *      softplus(v) = log(1 + exp(v)), evaluated as max(v,0) + log1p(exp(-|v|)).
 */
static double softplus(double v) {
    return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

/* Exposed so that tests can check the formula on its own. */
double oracle_softplus(double v) { return softplus(v); }

int oracle_conv1d(int64_t batch, int64_t seqlen, int64_t dim, int64_t d_conv,
                  const double *x_raw, const double *w, const double *bias, int silu_act,
                  double *out) {
    if (batch < 0 || seqlen < 0 || dim < 0 || d_conv <= 0) return ORACLE_EINVAL;
    if (batch == 0 || seqlen == 0 || dim == 0) return ORACLE_OK;
    if (!x_raw || !w || !out) return ORACLE_EINVAL;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t t = 0; t < seqlen; ++t)
            for (int64_t d = 0; d < dim; ++d) {
                double acc = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < d_conv; ++k) {
                    int64_t ts = t - (d_conv - 1) + k;
                    if (ts >= 0) acc += w[d * d_conv + k] * x_raw[(b * seqlen + ts) * dim + d];
                }
                out[(b * seqlen + t) * dim + d] = silu_act ? silu(acc) : acc;
            }
    return ORACLE_OK;
}

int oracle_delta_softplus(int64_t batch, int64_t seqlen, int64_t dim, const double *delta_raw,
                          const double *bias, double *out) {
    if (batch < 0 || seqlen < 0 || dim < 0) return ORACLE_EINVAL;
    if (batch == 0 || seqlen == 0 || dim == 0) return ORACLE_OK;
    if (!delta_raw || !out) return ORACLE_EINVAL;
    for (int64_t i = 0; i < batch * seqlen; ++i)
        for (int64_t d = 0; d < dim; ++d)
            out[i * dim + d] = softplus(delta_raw[i * dim + d] + (bias ? bias[d] : 0.0));
    return ORACLE_OK;
}
