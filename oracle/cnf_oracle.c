/*
 * cnf_oracle.c -- plain, slow, fp64 CPU definition of the fused
 * convolution + normalization forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is written straight from
 * the definitions on the four source pages and is meant to be checked by eye:
 * nested loops, no blocking, no fusion, no reordering beyond what each
 * definition states.
 *
 * Pages (cited by their title, the KernelBench level-2 problem they work on):
 *   [p27] "Kimi-K2.6__l2_p27": Conv3d(3->16, k=4) -> HardSwish -> GroupNorm(4)
 *         -> mean over D,H,W.
 *   [p17] "Kimi-K2.6__l2_p17": Conv2d(64->128, k=3) -> InstanceNorm2d -> /2.
 *   [p6]  "Kimi-K2.6__l2_p6":  Conv3d(3->16, k=3) -> softmax over channels ->
 *         MaxPool3d(2) -> MaxPool3d(2).
 *   [p19] "Kimi-K2.6__l2_p19": ConvTranspose2d(64->64, k=3, s=1) -> GELU ->
 *         GroupNorm(8).
 * The pages carry no numbered sections; each citation names the passage.
 *
 * All arithmetic is in double.  Inputs arrive as fp32 (the type the path is
 * fed) and are widened before use.  Libm supplies exp and erf.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* --------------------------------------------------------------------------
 * Convolution, stride 1, no padding, dilation 1, groups G (cross-correlation).
 *   y[n,co,d,h,w] = b[co] + sum_{c<Ci/G} sum_{a,bb,e}
 *                   x[n, g*Ci/G + c, d+a, h+bb, w+e] * wt[co, c, a, bb, e]
 * with g = co / (Co/G).  Output extent per axis is L - K + 1.
 * [p27] first trace, the opening problem statement (13x29x29 output of the
 *       k=4 Conv3d); [p17] second trace, its statement of the 3x3 conv and
 *       the 126x126 output; [p6] the trace's per-voxel conv loop.
 * 2-D convolution is the D = 1, kd = 1 case.
 * x: [N][Ci][D][H][W], wt: [Co][Ci/G][kd][kh][kw], b: [Co] or NULL,
 * y: [N][Co][D-kd+1][H-kh+1][W-kw+1].  Returns 0, or -1 on a bad shape.
 * ------------------------------------------------------------------------ */
int orc_conv(int N, int Ci, int D, int H, int W, int Co, int G,
             int kd, int kh, int kw,
             const float *x, const float *wt, const float *b, double *y)
{
    if (N < 0 || Ci < 1 || Co < 1 || G < 1 || Ci % G || Co % G) return -1;
    if (kd < 1 || kh < 1 || kw < 1) return -1;
    const int Do = D - kd + 1, Ho = H - kh + 1, Wo = W - kw + 1;
    if (Do < 1 || Ho < 1 || Wo < 1) return -1;
    const int cig = Ci / G, cog = Co / G;
    const int64_t in_plane = (int64_t)D * H * W;
    const int64_t out_plane = (int64_t)Do * Ho * Wo;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int co = 0; co < Co; ++co) {
            const int g = co / cog;
            double *yp = y + ((int64_t)n * Co + co) * out_plane;
            for (int od = 0; od < Do; ++od)
            for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow) {
                double acc = b ? (double)b[co] : 0.0;
                for (int c = 0; c < cig; ++c) {
                    const int ci = g * cig + c;
                    const float *xp = x + ((int64_t)n * Ci + ci) * in_plane;
                    const float *wp = wt + ((int64_t)co * cig + c) * kd * kh * kw;
                    for (int a = 0; a < kd; ++a)
                    for (int bb = 0; bb < kh; ++bb)
                    for (int e = 0; e < kw; ++e) {
                        const double xv = (double)xp[((int64_t)(od + a) * H + (oh + bb)) * W + (ow + e)];
                        const double wv = (double)wp[(a * kh + bb) * kw + e];
                        acc += xv * wv;
                    }
                }
                yp[((int64_t)od * Ho + oh) * Wo + ow] = acc;
            }
        }
    }
    return 0;
}

/* --------------------------------------------------------------------------
 * Transposed 2-D convolution, stride 1, no padding, groups G, written as the
 * adjoint of the convolution above: every input pixel scatters its value,
 * times the kernel, into the kh x kw output window that starts at its own
 * position.  Output extent is (H-1)*1 - 0 + (kh-1) + 0 + 1 = H + kh - 1.
 * [p19] second trace, the 1-D adjoint derivation and the 2x2-input /
 *       3x3-ones worked example; first trace, the output-size formula
 *       giving 258x258.  Weight layout is the transposed one the page states:
 *       wt: [Ci][Co/G][kh][kw].
 * x: [N][Ci][H][W], b: [Co] or NULL, y: [N][Co][H+kh-1][W+kw-1].
 * ------------------------------------------------------------------------ */
int orc_conv_transpose2d(int N, int Ci, int H, int W, int Co, int G,
                         int kh, int kw,
                         const float *x, const float *wt, const float *b,
                         double *y)
{
    if (N < 0 || Ci < 1 || Co < 1 || G < 1 || Ci % G || Co % G) return -1;
    if (kh < 1 || kw < 1 || H < 1 || W < 1) return -1;
    const int Ho = H + kh - 1, Wo = W + kw - 1;
    const int cig = Ci / G, cog = Co / G;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int co = 0; co < Co; ++co) {
            const int g = co / cog, col = co % cog;
            double *yp = y + ((int64_t)n * Co + co) * Ho * Wo;
            const double bias = b ? (double)b[co] : 0.0;
            for (int64_t p = 0; p < (int64_t)Ho * Wo; ++p) yp[p] = bias;
            for (int c = 0; c < cig; ++c) {
                const int ci = g * cig + c;
                const float *xp = x + ((int64_t)n * Ci + ci) * H * W;
                const float *wp = wt + ((int64_t)ci * cog + col) * kh * kw;
                for (int i = 0; i < H; ++i)
                for (int j = 0; j < W; ++j) {
                    const double v = (double)xp[(int64_t)i * W + j];
                    for (int a = 0; a < kh; ++a)
                    for (int e = 0; e < kw; ++e)
                        yp[(int64_t)(i + a) * Wo + (j + e)] += v * (double)wp[a * kw + e];
                }
            }
        }
    }
    return 0;
}

/* --------------------------------------------------------------------------
 * Convolution with stride s, zero padding p and dilation d along each axis
 * (s, p, dl are 3-entry arrays for D, H, W), groups G:
 *   y[n,co,o] = b[co] + sum_{c<Ci/G} sum_{a} x[n, g*Ci/G + c, o*s - p + a*dl]
 *                                           * wt[co, c, a]
 * per axis, with x taken as 0 outside [0, L).  Output extent per axis is
 * floor((L + 2p - dl*(k-1) - 1) / s) + 1.
 * [p6] the trace's integer output-size passage, which states this extent for
 *      Conv3d and MaxPool3d; [p19] the fix sequence's adjoint derivation,
 *      which writes the strided, padded, dilated conv as this gather.
 * A 2-D conv is the D = 1, kd = 1, s[0] = dl[0] = 1, p[0] = 0 case.
 * x: [N][Ci][D][H][W], wt: [Co][Ci/G][kd][kh][kw], b: [Co] or NULL,
 * y: [N][Co][Do][Ho][Wo].  Returns 0, or -1 on a bad shape.
 * ------------------------------------------------------------------------ */
static int conv_extent(int L, int k, int s, int p, int dl)
{
    const int num = L + 2 * p - dl * (k - 1) - 1;
    if (num < 0) return 0;
    return num / s + 1;
}

int orc_conv_general(int N, int Ci, int D, int H, int W, int Co, int G,
                     int kd, int kh, int kw, const int *s, const int *p, const int *dl,
                     const float *x, const float *wt, const float *b, double *y)
{
    if (N < 0 || Ci < 1 || Co < 1 || G < 1 || Ci % G || Co % G) return -1;
    if (kd < 1 || kh < 1 || kw < 1) return -1;
    for (int i = 0; i < 3; ++i)
        if (s[i] < 1 || p[i] < 0 || dl[i] < 1) return -1;
    const int Do = conv_extent(D, kd, s[0], p[0], dl[0]);
    const int Ho = conv_extent(H, kh, s[1], p[1], dl[1]);
    const int Wo = conv_extent(W, kw, s[2], p[2], dl[2]);
    if (Do < 1 || Ho < 1 || Wo < 1) return -1;
    const int cig = Ci / G, cog = Co / G;
    const int64_t in_plane = (int64_t)D * H * W;
    const int64_t out_plane = (int64_t)Do * Ho * Wo;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int co = 0; co < Co; ++co) {
            const int g = co / cog;
            double *yp = y + ((int64_t)n * Co + co) * out_plane;
            for (int od = 0; od < Do; ++od)
            for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow) {
                double acc = b ? (double)b[co] : 0.0;
                for (int c = 0; c < cig; ++c) {
                    const int ci = g * cig + c;
                    const float *xp = x + ((int64_t)n * Ci + ci) * in_plane;
                    const float *wp = wt + ((int64_t)co * cig + c) * kd * kh * kw;
                    for (int a = 0; a < kd; ++a)
                    for (int bb = 0; bb < kh; ++bb)
                    for (int e = 0; e < kw; ++e) {
                        const int id = od * s[0] - p[0] + a * dl[0];
                        const int ih = oh * s[1] - p[1] + bb * dl[1];
                        const int iw = ow * s[2] - p[2] + e * dl[2];
                        if (id < 0 || id >= D || ih < 0 || ih >= H || iw < 0 || iw >= W)
                            continue;  /* zero padding */
                        acc += (double)xp[((int64_t)id * H + ih) * W + iw] *
                               (double)wp[(a * kh + bb) * kw + e];
                    }
                }
                yp[((int64_t)od * Ho + oh) * Wo + ow] = acc;
            }
        }
    }
    return 0;
}

/* --------------------------------------------------------------------------
 * Transposed convolution with stride s, padding p, dilation dl and
 * output_padding op along each axis, groups G, written as the adjoint of
 * orc_conv_general: input position i, tap a sends x[i] * wt[ci, co, a] to the
 * output position o = i*s - p + a*dl, and contributions falling outside
 * [0, Lo) are dropped.  Output extent per axis is
 *   Lo = (L - 1)*s - 2p + dl*(k - 1) + op + 1.
 * [p19] first trace, the output-size formula with all five parameters; the
 *       fix sequence's statement that the transposed conv is the adjoint of
 *       the conv, and the conv gather it takes the adjoint of.  Weight
 *       layout as the page states: wt: [Ci][Co/G][kd][kh][kw].
 * x: [N][Ci][D][H][W], b: [Co] or NULL, y: [N][Co][Do][Ho][Wo].
 * ------------------------------------------------------------------------ */
int orc_conv_transpose_general(int N, int Ci, int D, int H, int W, int Co, int G,
                               int kd, int kh, int kw, const int *s, const int *p,
                               const int *dl, const int *op,
                               const float *x, const float *wt, const float *b, double *y)
{
    if (N < 0 || Ci < 1 || Co < 1 || G < 1 || Ci % G || Co % G) return -1;
    if (kd < 1 || kh < 1 || kw < 1 || D < 1 || H < 1 || W < 1) return -1;
    for (int i = 0; i < 3; ++i)
        if (s[i] < 1 || p[i] < 0 || dl[i] < 1 || op[i] < 0) return -1;
    const int Do = (D - 1) * s[0] - 2 * p[0] + dl[0] * (kd - 1) + op[0] + 1;
    const int Ho = (H - 1) * s[1] - 2 * p[1] + dl[1] * (kh - 1) + op[1] + 1;
    const int Wo = (W - 1) * s[2] - 2 * p[2] + dl[2] * (kw - 1) + op[2] + 1;
    if (Do < 1 || Ho < 1 || Wo < 1) return -1;
    const int cig = Ci / G, cog = Co / G;
    const int64_t in_plane = (int64_t)D * H * W;
    const int64_t out_plane = (int64_t)Do * Ho * Wo;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int co = 0; co < Co; ++co) {
            const int g = co / cog, col = co % cog;
            double *yp = y + ((int64_t)n * Co + co) * out_plane;
            const double bias = b ? (double)b[co] : 0.0;
            for (int64_t q = 0; q < out_plane; ++q) yp[q] = bias;
            for (int c = 0; c < cig; ++c) {
                const int ci = g * cig + c;
                const float *xp = x + ((int64_t)n * Ci + ci) * in_plane;
                const float *wp = wt + ((int64_t)ci * cog + col) * kd * kh * kw;
                for (int i0 = 0; i0 < D; ++i0)
                for (int i1 = 0; i1 < H; ++i1)
                for (int i2 = 0; i2 < W; ++i2) {
                    const double v = (double)xp[((int64_t)i0 * H + i1) * W + i2];
                    for (int a = 0; a < kd; ++a)
                    for (int bb = 0; bb < kh; ++bb)
                    for (int e = 0; e < kw; ++e) {
                        const int od = i0 * s[0] - p[0] + a * dl[0];
                        const int oh = i1 * s[1] - p[1] + bb * dl[1];
                        const int ow = i2 * s[2] - p[2] + e * dl[2];
                        if (od < 0 || od >= Do || oh < 0 || oh >= Ho || ow < 0 || ow >= Wo)
                            continue;
                        yp[((int64_t)od * Ho + oh) * Wo + ow] +=
                            v * (double)wp[(a * kh + bb) * kw + e];
                    }
                }
            }
        }
    }
    return 0;
}

/* HardSwish h(x) = x * min(max(x + 3, 0), 6) / 6.
 * [p27] first trace, its statement of the activation and its piecewise
 *       reading (0 below -3, x above 3). */
void orc_hardswish(double *v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        const double x = v[i];
        v[i] = x * fmin(fmax(x + 3.0, 0.0), 6.0) / 6.0;
    }
}

/* Exact GELU, gelu(x) = x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt 2)),
 * PyTorch's default (no tanh approximation).
 * [p19] second trace, the passage settling on the erf form as the default. */
void orc_gelu_erf(double *v, int64_t n)
{
    const double inv_sqrt2 = 0.70710678118654752440;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double x = v[i];
        v[i] = 0.5 * x * (1.0 + erf(x * inv_sqrt2));
    }
}

/* GELU with the tanh approximation, kept only so the tests can show how far
 * it is from the exact form ([p19] first trace quotes its constants). */
void orc_gelu_tanh(double *v, int64_t n)
{
    const double k0 = 0.79788456080286535588; /* sqrt(2/pi) */
    for (int64_t i = 0; i < n; ++i) {
        const double x = v[i];
        v[i] = 0.5 * x * (1.0 + tanh(k0 * (x + 0.044715 * x * x * x)));
    }
}

/* Softmax over the channel axis at every spatial position, with the channel
 * maximum subtracted before exponentiating.
 * [p6] the trace's per-voxel softmax over the 16 output channels.
 * y: [N][C][S], in place. */
void orc_softmax_channel(double *y, int N, int C, int64_t S)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int64_t s = 0; s < S; ++s) {
            double *p = y + (int64_t)n * C * S + s;
            double m = p[0];
            for (int c = 1; c < C; ++c) if (p[c * S] > m) m = p[c * S];
            double sum = 0.0;
            for (int c = 0; c < C; ++c) { p[c * S] = exp(p[c * S] - m); sum += p[c * S]; }
            for (int c = 0; c < C; ++c) p[c * S] = p[c * S] / sum;
        }
    }
}

/* GroupNorm over (C/G) channels x S positions per (sample, group): mean, then
 * the biased variance around it (two passes), eps inside the square root,
 * then the per-channel affine gamma_c, beta_c (NULL means 1 and 0).
 * InstanceNorm without affine is the G = C, gamma = beta = NULL case.
 * [p27] first trace, its GroupNorm statement; [p19] first trace, stats over
 *       the 8 channels of a group and all 258x258 positions; [p17] second
 *       trace, the InstanceNorm2d defaults (no affine, no running stats,
 *       biased variance, eps 1e-5).
 * y: [N][C][S], in place. */
void orc_group_norm(double *y, int N, int C, int64_t S, int G, double eps,
                    const float *gamma, const float *beta)
{
    const int cg = C / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            double *p = y + ((int64_t)n * C + (int64_t)g * cg) * S;
            const int64_t cnt = (int64_t)cg * S;
            double sum = 0.0;
            for (int64_t i = 0; i < cnt; ++i) sum += p[i];
            const double mean = sum / (double)cnt;
            double ss = 0.0;
            for (int64_t i = 0; i < cnt; ++i) { const double d = p[i] - mean; ss += d * d; }
            const double var = ss / (double)cnt;
            const double inv = 1.0 / sqrt(var + eps);
            for (int c = 0; c < cg; ++c) {
                const int ch = g * cg + c;
                const double ga = gamma ? (double)gamma[ch] : 1.0;
                const double be = beta ? (double)beta[ch] : 0.0;
                double *q = p + (int64_t)c * S;
                for (int64_t s = 0; s < S; ++s) q[s] = (q[s] - mean) * inv * ga + be;
            }
        }
    }
}

/* Element-wise true division by a constant ([p17]: the "/ 2.0" step). */
void orc_divide(double *y, int64_t n, double divisor)
{
    for (int64_t i = 0; i < n; ++i) y[i] = y[i] / divisor;
}

/* Arithmetic mean over all spatial positions ([p27]: mean over D, H, W).
 * y: [N][C][S] -> out: [N][C]. */
void orc_mean_spatial(const double *y, int N, int C, int64_t S, double *out)
{
    for (int64_t nc = 0; nc < (int64_t)N * C; ++nc) {
        double sum = 0.0;
        for (int64_t s = 0; s < S; ++s) sum += y[nc * S + s];
        out[nc] = sum / (double)S;
    }
}

/* One max-pool pass, kernel = stride = (kd, kh, kw), no padding, floor
 * mode: out extent floor(L / k) per axis.  Each window is scanned in
 * row-major (d, h, w) order and a later value replaces the running maximum
 * only when strictly larger, so among equal values the first one scanned wins.
 * The argmax of every output is carried as a flat index into the grid the
 * first pass saw: in_idx NULL means "this is the first pass" and the index
 * of an input voxel is d*H*W + h*W + w; otherwise the index is copied from
 * in_idx.  [p6] the problem statement (MaxPool3d(kernel_size=2) twice) and
 * the trace's floor-mode size chain 14x30x30 -> 7x15x15 -> 3x7x7, and its
 * output-size formula with padding 0, dilation 1, stride = kernel.  A 2-D
 * pool is the D = 1, kd = 1 case (it pools H and W only).
 * in: [N][C][D][H][W]; out, out_idx: [N][C][D/kd][H/kh][W/kw]. */
int orc_maxpool3d(const double *in, const int64_t *in_idx,
                  int N, int C, int D, int H, int W, int kd, int kh, int kw,
                  double *out, int64_t *out_idx)
{
    if (kd < 1 || kh < 1 || kw < 1) return -1;
    const int Dp = D / kd, Hp = H / kh, Wp = W / kw;
    const int64_t in_plane = (int64_t)D * H * W, out_plane = (int64_t)Dp * Hp * Wp;
    for (int64_t nc = 0; nc < (int64_t)N * C; ++nc) {
        const double *ip = in + nc * in_plane;
        const int64_t *ix = in_idx ? in_idx + nc * in_plane : NULL;
        for (int od = 0; od < Dp; ++od)
        for (int oh = 0; oh < Hp; ++oh)
        for (int ow = 0; ow < Wp; ++ow) {
            double best = 0.0;
            int64_t best_i = -1;
            for (int a = 0; a < kd; ++a)
            for (int bb = 0; bb < kh; ++bb)
            for (int e = 0; e < kw; ++e) {
                const int64_t off = ((int64_t)(od * kd + a) * H + (oh * kh + bb)) * W + (ow * kw + e);
                const double v = ip[off];
                if (best_i < 0 || v > best) {
                    best = v;
                    best_i = ix ? ix[off] : off;
                }
            }
            const int64_t o = nc * out_plane + ((int64_t)od * Hp + oh) * Wp + ow;
            out[o] = best;
            out_idx[o] = best_i;
        }
    }
    return 0;
}

/* Closed form of GroupNorm followed by a spatial mean ([p27] first trace,
 * the derivation that the mean of the normalized channel needs only the
 * channel's mean m_c and the group's mean and variance; second trace, the
 * same result via per-channel sums):
 *   out[n,c] = gamma_c * (m_c - mu_g) / sqrt(var_g + eps) + beta_c
 *   mu_g  = mean over the group's channels of m_c       (equal counts)
 *   var_g = mean over the group's channels of (v_c + (m_c - mu_g)^2)
 * with m_c, v_c the mean and biased variance of channel c (two passes).
 * h: [N][C][S] -> out: [N][C]. */
void orc_gn_mean_closed_form(const double *h, int N, int C, int64_t S, int G,
                             double eps, const float *gamma, const float *beta,
                             double *out)
{
    const int cg = C / G;
    double *m = (double *)malloc(sizeof(double) * (size_t)C);
    double *v = (double *)malloc(sizeof(double) * (size_t)C);
    for (int n = 0; n < N; ++n) {
        for (int c = 0; c < C; ++c) {
            const double *p = h + ((int64_t)n * C + c) * S;
            double sum = 0.0;
            for (int64_t s = 0; s < S; ++s) sum += p[s];
            m[c] = sum / (double)S;
            double ss = 0.0;
            for (int64_t s = 0; s < S; ++s) { const double d = p[s] - m[c]; ss += d * d; }
            v[c] = ss / (double)S;
        }
        for (int g = 0; g < G; ++g) {
            double mu = 0.0;
            for (int c = g * cg; c < (g + 1) * cg; ++c) mu += m[c];
            mu /= (double)cg;
            double var = 0.0;
            for (int c = g * cg; c < (g + 1) * cg; ++c) var += v[c] + (m[c] - mu) * (m[c] - mu);
            var /= (double)cg;
            const double inv = 1.0 / sqrt(var + eps);
            for (int c = g * cg; c < (g + 1) * cg; ++c) {
                const double ga = gamma ? (double)gamma[c] : 1.0;
                const double be = beta ? (double)beta[c] : 0.0;
                out[(int64_t)n * C + c] = ga * (m[c] - mu) * inv + be;
            }
        }
    }
    free(m);
    free(v);
}

/* Number of OpenMP threads the oracle will use (reported with CPU timings). */
int orc_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
