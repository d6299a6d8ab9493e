/*
 * gconv_oracle.c -- plain, slow, fp64 CPU oracle for grouped convolution forward
 * (and the backward of the depthwise 1-D convolution).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (read from the pages, no blocking, fusion or reordering):
 *
 *  - Grouped convolution as defined in the neon issue "Grouped convolutions"
 *    (reply by thestew42): input channels, filters and output channels are split
 *    into `groups` groups with no connection between groups.  Group k owns the
 *    contiguous input block [k*C/g, (k+1)*C/g) and the contiguous output block
 *    [k*Cout/g, (k+1)*Cout/g) -- the "usual" 111122223333 output order named in
 *    a later reply (ibmua) of the same issue.
 *  - The per-output sum is the cross-correlation of PyTorch's F.conv2d, the call
 *    the discuss.pytorch.org thread "F.conv2d runs x15 slower in
 *    mixed-precision/half-precision mode" times (its test script: padding 3//2,
 *    groups=4, weight [512,128,3,3]): no kernel flip, zero padding on both
 *    sides, taps spaced by the dilation, windows advanced by the stride.
 *  - Depthwise 1-D convolution over a (batch, steps, channels) tensor, as in the
 *    speechbrain issue "Investigate custom Triton kernels for depthwise-separable
 *    convolutions in Conformer" (#2733): groups equal to the channel count, one
 *    K-tap filter per channel, data laid out (batch, steps, channels).
 *  - The backward pass of that depthwise 1-D convolution (the same issue's
 *    follow-up comments): the gradients with respect to x, w and the bias, the
 *    chain-rule sums of the forward definition.
 *
 * Every input is fp64 (callers pass fp16/bf16/fp32 values widened exactly), every
 * product and sum is fp64, and results are returned in fp64.
 *
 * Return codes: 0 = ok, 1 = invalid argument, 2 = empty / non-positive output.
 */
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of window positions along one axis: the count of o >= 0 whose window
 * [o*s - p, o*s - p + d*(K-1)] lies inside the zero-padded range [-p, L+p-1]. */
int64_t gconv_oracle_out_len(int64_t L, int64_t K, int64_t s, int64_t p, int64_t d)
{
    if (L < 0 || K < 1 || s < 1 || p < 0 || d < 1) return -1;
    int64_t last_start = L + 2 * p - d * (K - 1) - 1; /* last admissible o*s */
    if (last_start < 0) return 0;
    return last_start / s + 1;
}

int gconv_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

typedef struct {
    int64_t N, C, H, W;        /* input  x[N][C][H][W]            */
    int64_t Cout, KH, KW;      /* weight w[Cout][C/groups][KH][KW] */
    int64_t groups;
    int64_t sh, sw, ph, pw, dh, dw;
    int64_t OH, OW;            /* output y[N][Cout][OH][OW]       */
} conv2d_geom;

static int conv2d_check(const conv2d_geom *g)
{
    if (g->N < 0 || g->C < 1 || g->H < 1 || g->W < 1) return 1;
    if (g->Cout < 1 || g->KH < 1 || g->KW < 1 || g->groups < 1) return 1;
    if (g->C % g->groups != 0 || g->Cout % g->groups != 0) return 1;
    if (g->sh < 1 || g->sw < 1 || g->ph < 0 || g->pw < 0 || g->dh < 1 || g->dw < 1) return 1;
    if (g->OH < 1 || g->OW < 1) return 2;
    return 0;
}

/* One output element y[n][o][oh][ow]: the definition written out. */
static double conv2d_one(const conv2d_geom *g, const double *x, const double *w,
                         const double *bias, int64_t n, int64_t o, int64_t oh, int64_t ow)
{
    const int64_t Cg = g->C / g->groups;         /* input channels per group  */
    const int64_t Ng = g->Cout / g->groups;      /* output channels per group */
    const int64_t k = o / Ng;                    /* the group output o is in  */
    double acc = bias ? bias[o] : 0.0;
    for (int64_t ci = 0; ci < Cg; ++ci) {
        const int64_t c = k * Cg + ci;           /* input channel of this tap */
        for (int64_t kh = 0; kh < g->KH; ++kh) {
            const int64_t ih = oh * g->sh - g->ph + kh * g->dh;
            if (ih < 0 || ih >= g->H) continue;  /* zero padding */
            for (int64_t kw = 0; kw < g->KW; ++kw) {
                const int64_t iw = ow * g->sw - g->pw + kw * g->dw;
                if (iw < 0 || iw >= g->W) continue;
                const double xv = x[((n * g->C + c) * g->H + ih) * g->W + iw];
                const double wv = w[((o * Cg + ci) * g->KH + kh) * g->KW + kw];
                acc += xv * wv;
            }
        }
    }
    return acc;
}

static int conv2d_geom_make(conv2d_geom *g, int64_t N, int64_t C, int64_t H, int64_t W,
                            int64_t Cout, int64_t Cg_w, int64_t KH, int64_t KW, int64_t groups,
                            int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw)
{
    g->N = N; g->C = C; g->H = H; g->W = W;
    g->Cout = Cout; g->KH = KH; g->KW = KW; g->groups = groups;
    g->sh = sh; g->sw = sw; g->ph = ph; g->pw = pw; g->dh = dh; g->dw = dw;
    g->OH = gconv_oracle_out_len(H, KH, sh, ph, dh);
    g->OW = gconv_oracle_out_len(W, KW, sw, pw, dw);
    if (groups < 1 || C < 1 || C % groups != 0 || Cg_w != C / groups) return 1;
    return conv2d_check(g);
}

/*
 * Full grouped conv2d, NCHW.  x: [N][C][H][W]; w: [Cout][Cg_w][KH][KW] with
 * Cg_w == C/groups; bias: [Cout] or NULL; y: [N][Cout][OH][OW] where OH and OW
 * are gconv_oracle_out_len of each axis.
 */
int gconv_oracle_conv2d(const double *x, int64_t N, int64_t C, int64_t H, int64_t W,
                        const double *w, int64_t Cout, int64_t Cg_w, int64_t KH, int64_t KW,
                        const double *bias, int64_t groups,
                        int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                        double *y)
{
    conv2d_geom g;
    int rc = conv2d_geom_make(&g, N, C, H, W, Cout, Cg_w, KH, KW, groups, sh, sw, ph, pw, dh, dw);
    if (rc) return rc;
    const int64_t planes = N * Cout;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < planes; ++p) {
        const int64_t n = p / Cout, o = p % Cout;
        for (int64_t oh = 0; oh < g.OH; ++oh)
            for (int64_t ow = 0; ow < g.OW; ++ow)
                y[((n * Cout + o) * g.OH + oh) * g.OW + ow] = conv2d_one(&g, x, w, bias, n, o, oh, ow);
    }
    return 0;
}

/*
 * The same definition evaluated only at selected outputs: idx[i] is a flat
 * index into y[N][Cout][OH][OW]; out[i] receives that element.
 */
int gconv_oracle_conv2d_at(const double *x, int64_t N, int64_t C, int64_t H, int64_t W,
                           const double *w, int64_t Cout, int64_t Cg_w, int64_t KH, int64_t KW,
                           const double *bias, int64_t groups,
                           int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                           const int64_t *idx, int64_t n_idx, double *out)
{
    conv2d_geom g;
    int rc = conv2d_geom_make(&g, N, C, H, W, Cout, Cg_w, KH, KW, groups, sh, sw, ph, pw, dh, dw);
    if (rc) return rc;
    const int64_t total = N * Cout * g.OH * g.OW;
    for (int64_t i = 0; i < n_idx; ++i)
        if (idx[i] < 0 || idx[i] >= total) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_idx; ++i) {
        int64_t r = idx[i];
        const int64_t ow = r % g.OW; r /= g.OW;
        const int64_t oh = r % g.OH; r /= g.OH;
        const int64_t o = r % Cout;
        const int64_t n = r / Cout;
        out[i] = conv2d_one(&g, x, w, bias, n, o, oh, ow);
    }
    return 0;
}

/*
 * The interleaved output order of the neon issue "Grouped convolutions" (ibmua's
 * reply on output ordering: 1234123412341234 instead of the usual 111122223333):
 * filter j of group k (filter index o = k*Ng + j, the same weights and sum as
 * above) is stored at output channel j*groups + k.  y: [N][Cout][OH][OW].
 */
int gconv_oracle_conv2d_interleaved(const double *x, int64_t N, int64_t C, int64_t H, int64_t W,
                                    const double *w, int64_t Cout, int64_t Cg_w, int64_t KH, int64_t KW,
                                    const double *bias, int64_t groups,
                                    int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                                    double *y)
{
    conv2d_geom g;
    int rc = conv2d_geom_make(&g, N, C, H, W, Cout, Cg_w, KH, KW, groups, sh, sw, ph, pw, dh, dw);
    if (rc) return rc;
    const int64_t Ng = Cout / groups;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < N * Cout; ++p) {
        const int64_t n = p / Cout, o = p % Cout;       /* o: filter index */
        const int64_t k = o / Ng, j = o % Ng;
        const int64_t oc = j * groups + k;              /* its output channel */
        for (int64_t oh = 0; oh < g.OH; ++oh)
            for (int64_t ow = 0; ow < g.OW; ++ow)
                y[((n * Cout + oc) * g.OH + oh) * g.OW + ow] = conv2d_one(&g, x, w, bias, n, o, oh, ow);
    }
    return 0;
}

/* ---- depthwise 1-D convolution over (batch, steps, channels) ---------------- */

static double dw1d_one(const double *x, int64_t T, int64_t C, const double *w, int64_t K,
                       const double *bias, int64_t s, int64_t p, int64_t d,
                       int64_t b, int64_t t, int64_t c)
{
    double acc = bias ? bias[c] : 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t ti = t * s - p + k * d;
        if (ti < 0 || ti >= T) continue;         /* zero padding */
        acc += x[(b * T + ti) * C + c] * w[c * K + k];
    }
    return acc;
}

/*
 * x: [B][T][C]; w: [C][1][K] (one filter per channel, groups == C);
 * bias: [C] or NULL; y: [B][To][C] with To = gconv_oracle_out_len(T, K, s, p, d).
 */
int gconv_oracle_dwconv1d_btc(const double *x, int64_t B, int64_t T, int64_t C,
                              const double *w, int64_t K, const double *bias,
                              int64_t s, int64_t p, int64_t d, double *y)
{
    if (B < 0 || T < 1 || C < 1 || K < 1 || s < 1 || p < 0 || d < 1) return 1;
    const int64_t To = gconv_oracle_out_len(T, K, s, p, d);
    if (To < 1) return 2;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < B * To; ++bt) {
        const int64_t b = bt / To, t = bt % To;
        for (int64_t c = 0; c < C; ++c)
            y[(b * To + t) * C + c] = dw1d_one(x, T, C, w, K, bias, s, p, d, b, t, c);
    }
    return 0;
}

/* Selected outputs of the depthwise 1-D convolution; idx[i] is a flat index
 * into y[B][To][C]. */
int gconv_oracle_dwconv1d_btc_at(const double *x, int64_t B, int64_t T, int64_t C,
                                 const double *w, int64_t K, const double *bias,
                                 int64_t s, int64_t p, int64_t d,
                                 const int64_t *idx, int64_t n_idx, double *out)
{
    if (B < 0 || T < 1 || C < 1 || K < 1 || s < 1 || p < 0 || d < 1) return 1;
    const int64_t To = gconv_oracle_out_len(T, K, s, p, d);
    if (To < 1) return 2;
    for (int64_t i = 0; i < n_idx; ++i)
        if (idx[i] < 0 || idx[i] >= B * To * C) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_idx; ++i) {
        const int64_t c = idx[i] % C;
        const int64_t t = (idx[i] / C) % To;
        const int64_t b = idx[i] / (C * To);
        out[i] = dw1d_one(x, T, C, w, K, bias, s, p, d, b, t, c);
    }
    return 0;
}

/* ---- backward of the depthwise 1-D convolution -----------------------------
 *
 * The speechbrain issue #2733 follow-up comments: its author went on to write the
 * backward pass of the (batch, steps, channels) depthwise convolution.  With
 * y = dwconv1d_btc(x, w, bias) and an upstream gradient dy [B][To][C], the chain
 * rule gives, term by term of the forward sum:
 *   dx[b][i][c] = sum over taps k and outputs t with t*s - p + k*d == i of
 *                 dy[b][t][c] * w[c][k];
 *   dw[c][0][k] = sum over b and t with 0 <= t*s - p + k*d < T of
 *                 dy[b][t][c] * x[b][t*s - p + k*d][c];
 *   db[c]       = sum over b and t of dy[b][t][c].
 * For dx the condition is solved for t: t = (i + p - k*d) / s when that is an
 * integer in [0, To).
 */
static double dw1d_bwd_data_one(const double *dy, int64_t To, int64_t C, const double *w, int64_t K,
                                int64_t s, int64_t p, int64_t d, int64_t b, int64_t i, int64_t c)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t ts = i + p - k * d;        /* = t * s */
        if (ts < 0 || ts % s != 0) continue;
        const int64_t t = ts / s;
        if (t >= To) continue;
        acc += dy[(b * To + t) * C + c] * w[c * K + k];
    }
    return acc;
}

static int dw1d_bwd_check(int64_t B, int64_t T, int64_t C, int64_t K, int64_t s, int64_t p, int64_t d)
{
    if (B < 0 || T < 1 || C < 1 || K < 1 || s < 1 || p < 0 || d < 1) return 1;
    if (gconv_oracle_out_len(T, K, s, p, d) < 1) return 2;
    return 0;
}

/* dy: [B][To][C] with To = gconv_oracle_out_len(T, K, s, p, d); w: [C][1][K];
 * dx: [B][T][C]. */
int gconv_oracle_dwconv1d_btc_bwd_data(const double *dy, int64_t B, int64_t T, int64_t C,
                                       const double *w, int64_t K, int64_t s, int64_t p, int64_t d,
                                       double *dx)
{
    const int rc = dw1d_bwd_check(B, T, C, K, s, p, d);
    if (rc) return rc;
    const int64_t To = gconv_oracle_out_len(T, K, s, p, d);
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < B * T; ++bi) {
        const int64_t b = bi / T, i = bi % T;
        for (int64_t c = 0; c < C; ++c)
            dx[(b * T + i) * C + c] = dw1d_bwd_data_one(dy, To, C, w, K, s, p, d, b, i, c);
    }
    return 0;
}

/* Selected elements of dx; idx[j] is a flat index into dx[B][T][C]. */
int gconv_oracle_dwconv1d_btc_bwd_data_at(const double *dy, int64_t B, int64_t T, int64_t C,
                                          const double *w, int64_t K, int64_t s, int64_t p, int64_t d,
                                          const int64_t *idx, int64_t n_idx, double *out)
{
    const int rc = dw1d_bwd_check(B, T, C, K, s, p, d);
    if (rc) return rc;
    const int64_t To = gconv_oracle_out_len(T, K, s, p, d);
    for (int64_t j = 0; j < n_idx; ++j)
        if (idx[j] < 0 || idx[j] >= B * T * C) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_idx; ++j) {
        const int64_t c = idx[j] % C, i = (idx[j] / C) % T, b = idx[j] / (C * T);
        out[j] = dw1d_bwd_data_one(dy, To, C, w, K, s, p, d, b, i, c);
    }
    return 0;
}

/* x: [B][T][C]; dy: [B][To][C]; dw: [C][1][K]; db: [C] or NULL. */
int gconv_oracle_dwconv1d_btc_bwd_filter(const double *x, const double *dy, int64_t B, int64_t T,
                                         int64_t C, int64_t K, int64_t s, int64_t p, int64_t d,
                                         double *dw, double *db)
{
    const int rc = dw1d_bwd_check(B, T, C, K, s, p, d);
    if (rc) return rc;
    const int64_t To = gconv_oracle_out_len(T, K, s, p, d);
#pragma omp parallel for schedule(static)
    for (int64_t ck = 0; ck < C * K; ++ck) {
        const int64_t c = ck / K, k = ck % K;
        double acc = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < To; ++t) {
                const int64_t ti = t * s - p + k * d;
                if (ti < 0 || ti >= T) continue;
                acc += dy[(b * To + t) * C + c] * x[(b * T + ti) * C + c];
            }
        dw[c * K + k] = acc;
    }
    if (db) {
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b)
                for (int64_t t = 0; t < To; ++t) acc += dy[(b * To + t) * C + c];
            db[c] = acc;
        }
    }
    return 0;
}

/* ---- grouped conv2d over channels-last (NHWC) tensors -----------------------
 *
 * The discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
 * half-precision mode" (replies 7-11) turns to the NHWC (channels_last) memory
 * format for the fp16 grouped conv.  The sum is the one above, only the element
 * addresses change: x[n][ih][iw][c], w[o][kh][kw][ci] (PyTorch's channels_last
 * weight order), y[n][oh][ow][o].
 */
static double conv2d_nhwc_one(const conv2d_geom *g, const double *x, const double *w,
                              const double *bias, int64_t n, int64_t o, int64_t oh, int64_t ow)
{
    const int64_t Cg = g->C / g->groups;
    const int64_t Ng = g->Cout / g->groups;
    const int64_t k = o / Ng;
    double acc = bias ? bias[o] : 0.0;
    for (int64_t kh = 0; kh < g->KH; ++kh) {
        const int64_t ih = oh * g->sh - g->ph + kh * g->dh;
        if (ih < 0 || ih >= g->H) continue;
        for (int64_t kw = 0; kw < g->KW; ++kw) {
            const int64_t iw = ow * g->sw - g->pw + kw * g->dw;
            if (iw < 0 || iw >= g->W) continue;
            for (int64_t ci = 0; ci < Cg; ++ci) {
                const double xv = x[((n * g->H + ih) * g->W + iw) * g->C + k * Cg + ci];
                const double wv = w[((o * g->KH + kh) * g->KW + kw) * Cg + ci];
                acc += xv * wv;
            }
        }
    }
    return acc;
}

/* x: [N][H][W][C]; w: [Cout][KH][KW][Cg_w] with Cg_w == C/groups; bias [Cout] or
 * NULL; y: [N][OH][OW][Cout]. */
int gconv_oracle_conv2d_nhwc(const double *x, int64_t N, int64_t C, int64_t H, int64_t W,
                             const double *w, int64_t Cout, int64_t Cg_w, int64_t KH, int64_t KW,
                             const double *bias, int64_t groups,
                             int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                             double *y)
{
    conv2d_geom g;
    int rc = conv2d_geom_make(&g, N, C, H, W, Cout, Cg_w, KH, KW, groups, sh, sw, ph, pw, dh, dw);
    if (rc) return rc;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < N * g.OH * g.OW; ++q) {
        const int64_t n = q / (g.OH * g.OW), oh = (q / g.OW) % g.OH, ow = q % g.OW;
        for (int64_t o = 0; o < Cout; ++o)
            y[q * Cout + o] = conv2d_nhwc_one(&g, x, w, bias, n, o, oh, ow);
    }
    return 0;
}

/* Selected outputs; idx[i] is a flat index into y[N][OH][OW][Cout]. */
int gconv_oracle_conv2d_nhwc_at(const double *x, int64_t N, int64_t C, int64_t H, int64_t W,
                                const double *w, int64_t Cout, int64_t Cg_w, int64_t KH, int64_t KW,
                                const double *bias, int64_t groups,
                                int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                                const int64_t *idx, int64_t n_idx, double *out)
{
    conv2d_geom g;
    int rc = conv2d_geom_make(&g, N, C, H, W, Cout, Cg_w, KH, KW, groups, sh, sw, ph, pw, dh, dw);
    if (rc) return rc;
    const int64_t total = N * g.OH * g.OW * Cout;
    for (int64_t i = 0; i < n_idx; ++i)
        if (idx[i] < 0 || idx[i] >= total) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_idx; ++i) {
        int64_t r = idx[i];
        const int64_t o = r % Cout; r /= Cout;
        const int64_t ow = r % g.OW; r /= g.OW;
        const int64_t oh = r % g.OH;
        const int64_t n = r / g.OH;
        out[i] = conv2d_nhwc_one(&g, x, w, bias, n, o, oh, ow);
    }
    return 0;
}
