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
 * Backward of the scan: the reverse-mode derivative of oracle_scan_ex with
 * respect to every input, for a loss whose gradients dy = dL/dy and
 * (optionally) dh_last = dL/dh_last are given.  The recompute-instead-of-
 * store design of the fused kernel is the GPU's business; here every state
 * of a channel is kept (paperlens tutorial, section on the hardware-aware
 * algorithm: the backward needs the states again).
 *
 * The chain rule on the forward loop, with g_t = SiLU(z_t) (1 without a
 * gate) and p_t = C_t . h_t + D x_t the gate's input:
 *   dp_t      = dy_t g_t,    dz_t = dy_t p_t SiLU'(z_t)
 *   dh_t      = dp_t C_t + Abar_{t+1} dh_{t+1}      (dh_last joins at t = L-1)
 *   dx_t      = dp_t D + sum_n dh_t[n] coef_t[n] B_t[n]
 *   ddelta_t  = sum_n dh_t[n] (dAbar/ddelta h_{t-1}[n] + dcoef/ddelta B_t[n] x_t)
 *   dA[d,n]  += dh_t[n] (dAbar/dA h_{t-1}[n] + dcoef/dA B_t[n] x_t)
 *   dB_t[n]  += dh_t[n] coef_t[n] x_t                (summed over channels)
 *   dC_t[n]  += dp_t h_t[n]                          (summed over channels)
 *   dD[d]    += dp_t x_t,   dh0 = Abar_0 dh_0
 * where coef = Bbar/B.  dA and dD are summed over batch and time; with A
 * given per channel, dA[d] is also summed over the states.
 */
typedef struct {
    double abar, coef;          /* Abar and Bbar / B */
    double dabar_dd, dabar_da;  /* dAbar/ddelta, dAbar/dA */
    double dcoef_dd, dcoef_da;  /* dcoef/ddelta, dcoef/dA */
} disc_grad;

/* Zero-order hold: Abar = exp(delta a), coef = (Abar - 1)/a, and at a = 0
 * the limits coef = delta, dcoef/da = delta^2 / 2. */
static void zoh_grad(double delta, double a, disc_grad *g) {
    double u = delta * a;
    g->abar = exp(u);
    g->dabar_dd = a * g->abar;
    g->dabar_da = delta * g->abar;
    if (a != 0.0) {
        g->coef = expm1(u) / a;
        g->dcoef_dd = g->abar;
        g->dcoef_da = (delta * g->abar - g->coef) / a;
    } else {
        g->coef = delta;
        g->dcoef_dd = 1.0;
        g->dcoef_da = 0.5 * delta * delta;
    }
}

/* Euler rule: Abar = exp(delta a), coef = delta. */
static void euler_grad(double delta, double a, disc_grad *g) {
    g->abar = exp(delta * a);
    g->dabar_dd = a * g->abar;
    g->dabar_da = delta * g->abar;
    g->coef = delta;
    g->dcoef_dd = 1.0;
    g->dcoef_da = 0.0;
}

/* SiLU'(v) = sigmoid(v) (1 + v (1 - sigmoid(v))). */
static double dsilu(double v) {
    double sg = 1.0 / (1.0 + exp(-v));
    return sg * (1.0 + v * (1.0 - sg));
}

/*
 * One channel (b, d): forward keeping every state (hist[t+1] = h_t,
 * hist[0] = h0), then the reverse loop.  e holds dL/dh_t arriving from the
 * steps after t.  dA_row (dstate entries, or 1 with a_step 0) and *dD_acc
 * receive this channel's sums; dB_acc and dC_acc ([batch, seqlen, dstate])
 * receive its share of the channel sums.
 */
static void scan_channel_bwd(int64_t b, int64_t d, int64_t seqlen, int64_t dim,
                             int64_t dstate, const double *x, const double *delta,
                             const double *a_row, int64_t a_step,
                             void (*disc)(double, double, disc_grad *),
                             const double *B, const double *C, const double *Dskip,
                             const double *z, const double *h0_row, const double *dy,
                             const double *dh_last_row, double *hist, double *e,
                             double *dx, double *ddelta, double *dz, double *dA_row,
                             double *dD_acc, double *dB_acc, double *dC_acc,
                             double *dh0_row) {
    double dval = Dskip ? Dskip[d] : 0.0;
    for (int64_t n = 0; n < dstate; ++n) hist[n] = h0_row ? h0_row[n] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
        int64_t io = (b * seqlen + t) * dim + d;
        int64_t bc = (b * seqlen + t) * dstate;
        for (int64_t n = 0; n < dstate; ++n) {
            disc_grad g;
            disc(delta[io], a_row[n * a_step], &g);
            hist[(t + 1) * dstate + n] =
                g.abar * hist[t * dstate + n] + g.coef * B[bc + n] * x[io];
        }
    }
    for (int64_t n = 0; n < dstate; ++n) e[n] = dh_last_row ? dh_last_row[n] : 0.0;
    for (int64_t t = seqlen - 1; t >= 0; --t) {
        int64_t io = (b * seqlen + t) * dim + d;
        int64_t bc = (b * seqlen + t) * dstate;
        const double *h_t = hist + (t + 1) * dstate;
        const double *h_prev = hist + t * dstate;
        double xv = x[io], dv = delta[io];
        double s = 0.0;
        for (int64_t n = 0; n < dstate; ++n) s += C[bc + n] * h_t[n];
        double p = s + dval * xv;
        double dp = z ? dy[io] * silu(z[io]) : dy[io];
        if (z && dz) dz[io] = dy[io] * p * dsilu(z[io]);
        double dxv = dp * dval, ddv = 0.0;
        for (int64_t n = 0; n < dstate; ++n) {
            disc_grad g;
            disc(dv, a_row[n * a_step], &g);
            double dh = e[n] + dp * C[bc + n];
            dC_acc[bc + n] += dp * h_t[n];
            dB_acc[bc + n] += dh * g.coef * xv;
            dxv += dh * g.coef * B[bc + n];
            ddv += dh * (g.dabar_dd * h_prev[n] + g.dcoef_dd * B[bc + n] * xv);
            dA_row[n * a_step] += dh * (g.dabar_da * h_prev[n] + g.dcoef_da * B[bc + n] * xv);
            e[n] = g.abar * dh;
        }
        dx[io] = dxv;
        ddelta[io] = ddv;
        *dD_acc += dp * xv;
    }
    if (dh0_row)
        for (int64_t n = 0; n < dstate; ++n) dh0_row[n] = e[n];
}

/*
 * Full backward.  Inputs as oracle_scan_ex plus dy [batch, seqlen, dim] and
 * dh_last [batch, dim, dstate] (NULL = 0).  Outputs: dx, ddelta, dz
 * [batch, seqlen, dim] (dz only with a gate; may be NULL), dA [dim, dstate]
 * ([dim] with a_per_channel), dB, dC [batch, seqlen, dstate], dD [dim] (may
 * be NULL), dh0 [batch, dim, dstate] (may be NULL).  Channels run on
 * nthreads threads in contiguous ranges; the channel sums of dB and dC are
 * kept per thread and added in thread order, so a result depends on
 * nthreads only through rounding.
 */
int oracle_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       const double *x, const double *delta, const double *A,
                       int a_per_channel, int use_euler, const double *B, const double *C,
                       const double *Dskip, const double *z, const double *h0,
                       const double *dy, const double *dh_last, double *dx, double *ddelta,
                       double *dA, double *dB, double *dC, double *dD, double *dz,
                       double *dh0, int nthreads) {
    if (batch < 0 || seqlen < 0 || dim < 0 || dstate <= 0) return ORACLE_EINVAL;
    if (!A || !dA) return ORACLE_EINVAL;
    if (batch > 0 && dim > 0 && seqlen > 0 &&
        (!x || !delta || !B || !C || !dy || !dx || !ddelta || !dB || !dC))
        return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const int64_t na = a_per_channel ? dim : dim * dstate;
    const int64_t nbc = batch * seqlen * dstate;
    for (int64_t i = 0; i < na; ++i) dA[i] = 0.0;
    if (dD)
        for (int64_t i = 0; i < dim; ++i) dD[i] = 0.0;
    for (int64_t i = 0; i < nbc; ++i) dB[i] = dC[i] = 0.0;
    if (batch == 0 || dim == 0) return ORACLE_OK;

    /* per (b, d) sums of dA and dD, added over b in order afterwards */
    const int64_t a_len = a_per_channel ? 1 : dstate;
    double *dA_part = (double *)calloc((size_t)(batch * dim * a_len), sizeof(double));
    double *dD_part = (double *)calloc((size_t)(batch * dim), sizeof(double));
    double **dB_thr = (double **)calloc((size_t)nthreads, sizeof(double *));
    double **dC_thr = (double **)calloc((size_t)nthreads, sizeof(double *));
    int used = 1;
    const int64_t nch = batch * dim;
#pragma omp parallel num_threads(nthreads)
    {
        int tid = omp_get_thread_num();
#pragma omp single
        used = omp_get_num_threads();
        double *dBt = (double *)calloc((size_t)nbc + 1, sizeof(double));
        double *dCt = (double *)calloc((size_t)nbc + 1, sizeof(double));
        double *hist = (double *)malloc((size_t)((seqlen + 1) * dstate) * sizeof(double));
        double *e = (double *)malloc((size_t)dstate * sizeof(double));
        dB_thr[tid] = dBt;
        dC_thr[tid] = dCt;
#pragma omp for schedule(static)
        for (int64_t ch = 0; ch < nch; ++ch) {
            int64_t b = ch / dim, d = ch % dim;
            const double *a_row = a_per_channel ? A + d : A + d * dstate;
            scan_channel_bwd(b, d, seqlen, dim, dstate, x, delta, a_row, a_per_channel ? 0 : 1,
                             use_euler ? euler_grad : zoh_grad, B, C, Dskip, z,
                             h0 ? h0 + ch * dstate : NULL, dy,
                             dh_last ? dh_last + ch * dstate : NULL, hist, e, dx, ddelta, dz,
                             dA_part + ch * a_len, dD_part + ch, dBt, dCt,
                             dh0 ? dh0 + ch * dstate : NULL);
        }
        free(hist);
        free(e);
    }
    for (int th = 0; th < used; ++th) {
        for (int64_t i = 0; i < nbc; ++i) {
            dB[i] += dB_thr[th][i];
            dC[i] += dC_thr[th][i];
        }
        free(dB_thr[th]);
        free(dC_thr[th]);
    }
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < dim; ++d) {
            for (int64_t k = 0; k < a_len; ++k) dA[d * a_len + k] += dA_part[(b * dim + d) * a_len + k];
            if (dD) dD[d] += dD_part[b * dim + d];
        }
    free(dA_part);
    free(dD_part);
    free(dB_thr);
    free(dC_thr);
    return ORACLE_OK;
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
