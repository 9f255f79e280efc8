// k_generic.hip -- the general kernel family: every descriptor the planner
// accepts that no specialised family covers.  2-D or 3-D, conv or transposed
// conv, any groups, stride, zero padding, dilation and output_padding, every
// activation, norm and reduction.
//
// What is computed (pages cited by title):
//   * conv: y[o] = b + sum over taps a and the group's input channels of
//     x[o*s - p + a*d] * w[a], x read as 0 outside the input; output extent
//     floor((L + 2p - d(k-1) - 1)/s) + 1  ("Kimi-K2.6__l2_p6", the integer
//     output-size passage; "Kimi-K2.6__l2_p19", the fix sequence's statement
//     of the strided, padded, dilated conv it takes the adjoint of);
//   * transposed conv: the adjoint of that conv.  Input i, tap a reaches
//     output o = i*s - p + a*d, so the gather form used here is
//     y[o] = b + sum_a x[(o + p - a*d)/s] * w[a] over the taps where the
//     division is exact and the quotient is inside the input; output extent
//     (L-1)s - 2p + d(k-1) + op + 1  ("Kimi-K2.6__l2_p19", first trace's
//     output-size formula and the fix sequence's adjoint derivation);
//   * activation, GroupNorm / InstanceNorm (biased variance, eps inside the
//     square root, optional per-channel affine), divide, mean over the
//     spatial axes, floor-mode max pool with kernel = stride applied
//     pool_repeats times (2-D problems pool H and W), argmax carried through
//     the passes: the same definitions the specialised families implement.
//
// Launch sequence (each step only when the descriptor needs it):
//   1. gen_conv_kernel     implicit GEMM on v_mfma_f32_16x16x4f32.  Rows = 16
//                          output channels of one conv group, columns = 16 output
//                          positions, K = (tap, four input channels of the group),
//                          gathered straight from the input through L1/L2 with
//                          per-lane bounds checks (no LDS staging: the access
//                          pattern depends on stride and dilation).  A wave owns
//                          16 channels x 64 positions (four column tiles share
//                          each weight operand); + bias + activation; writes the
//                          conv output and, for each (sample, channel, 64-position
//                          tile), (count, mean, M2) from two passes over the tile.
//   2. gen_softmax_kernel  softmax over the channels at each position, in place,
//                          and the same per-tile statistics of its result.
//   3. gen_finalize_kernel per (sample, norm group): merges the tile triples in
//                          double, in a fixed order (Chan et al.), and writes a
//                          per-channel scale and shift that fold the norm, the
//                          affine and the divide; for the mean reduction it writes
//                          the result instead (the spatial mean of an affine map
//                          of a channel is that map of the channel's mean).
//   4. gen_apply_kernel    in-place scale and shift of the conv output.
//   5. gen_pool_kernel     one floor-mode max-pool pass; the first pass applies the
//                          scale and shift and starts each argmax at the conv-grid
//                          index, later passes carry it.  A window is scanned in
//                          row-major order and only a strictly larger value
//                          replaces the running maximum.
//
// Bounds: every global access goes through a raw buffer resource whose size is
// the tensor's (per sample for x and y); masked lanes use an offset past the end,
// which reads 0 and drops stores.  The planner keeps every resource below 2 GiB
// and every coordinate below 2^20 (see generic_supported).
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.h"
#include "kernels.h"

namespace cnf {
namespace {

constexpr int GT = 256;                  // threads per workgroup (4 waves)
constexpr int PTILE = 64;                // output positions per wave task
constexpr unsigned GOOB = 0x7ff00000u;   // an offset past the end of every resource
constexpr unsigned RES_MAX = 0x7f000000u;

struct GenConv {
    const float *x, *w, *b;
    float *y;          // conv output [N][C_out][S] or nullptr
    v4f *part;         // [N][C_out][T] (count, mean, M2, 0) or nullptr
    long long tasks;   // N * T * G * cob
    int C_in, C_out, Cgi, Cgo, G, cob, T;
    int D, H, W, Do, Ho, Wo, S;
    int kd, kh, kw;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    float rsd, rsh, rsw;  // 1 / stride (transposed gather)
    unsigned in_plane, w_elems;
    float out_scale;
};

// Transposed gather: t = o + p - a*d names input position t / s when s divides
// t and the quotient lies in [0, L).  The quotient comes from a float product:
// for 0 <= t < 2^21 the fraction of (t + 0.5)/s is at least 0.5/s away from an
// integer while the float error is below 0.25/s, so the floor is exact.
__device__ __forceinline__ bool gather_src(int t, int s, float rs, int L, int &q) {
    q = (int)floorf(((float)t + 0.5f) * rs);
    return t >= 0 && q * s == t && q < L;
}

template <int ACT, bool TR>
__global__ __launch_bounds__(GT) void gen_conv_kernel(GenConv g) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const long long task = (long long)xcd_remap(blockIdx.x, gridDim.x) * 4 + wave;
    if (task >= g.tasks) return;  // whole waves leave; the kernel has no barriers
    long long t = task;
    const int cb = (int)(t % g.cob); t /= g.cob;
    const int grp = (int)(t % g.G); t /= g.G;
    const int pt = (int)(t % g.T);
    const int n = (int)(t / g.T);

    const auto xr = make_rsrc(g.x + (size_t)n * g.C_in * g.in_plane, g.C_in * g.in_plane * 4u);
    const auto wr = make_rsrc(g.w, g.w_elems * 4u);

    // This lane's output position in each of the four column tiles.
    const int HWo = g.Ho * g.Wo;
    int bz[4], by[4], bx[4], pos[4];
    bool pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        pos[u] = pt * PTILE + u * 16 + col;
        pv[u] = pos[u] < g.S;
        const int p2 = pv[u] ? pos[u] : 0;
        const int oz = p2 / HWo, rem = p2 - oz * HWo;
        const int oy = rem / g.Wo, ox = rem - oy * g.Wo;
        if (TR) { bz[u] = oz + g.pd; by[u] = oy + g.ph; bx[u] = ox + g.pw; }
        else { bz[u] = oz * g.sd - g.pd; by[u] = oy * g.sh - g.ph; bx[u] = ox * g.sw - g.pw; }
        if (!pv[u]) bz[u] = -(1 << 29);  // every tap falls outside the input
    }

    // A operand: row col = output channel co_l of the group, K entry kq = input channel.
    const int co_l = cb * 16 + col;
    const bool arow = co_l < g.Cgo;
    const int taps = g.kd * g.kh * g.kw;
    unsigned wbase, wci;
    if (TR) {  // w[C_in][Cgo][taps]
        wbase = ((unsigned)(grp * g.Cgi) * g.Cgo + co_l) * taps;
        wci = (unsigned)g.Cgo * taps;
    } else {   // w[C_out][Cgi][taps]
        wbase = (unsigned)(grp * g.Cgo + co_l) * g.Cgi * taps;
        wci = taps;
    }
    const unsigned xch0 = (unsigned)(grp * g.Cgi) * g.in_plane;

    v4f acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

    int tap = 0;
    for (int kz = 0; kz < g.kd; ++kz)
    for (int ky = 0; ky < g.kh; ++ky)
    for (int kx = 0; kx < g.kw; ++kx, ++tap) {
        unsigned sp[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int iz, iy, ix;
            if (TR) {
                const bool a = gather_src(bz[u] - kz * g.dd, g.sd, g.rsd, g.D, iz);
                const bool b = gather_src(by[u] - ky * g.dh, g.sh, g.rsh, g.H, iy);
                const bool c = gather_src(bx[u] - kx * g.dw, g.sw, g.rsw, g.W, ix);
                ok[u] = a && b && c;
            } else {
                iz = bz[u] + kz * g.dd;
                iy = by[u] + ky * g.dh;
                ix = bx[u] + kx * g.dw;
                ok[u] = (unsigned)iz < (unsigned)g.D && (unsigned)iy < (unsigned)g.H &&
                        (unsigned)ix < (unsigned)g.W;
            }
            sp[u] = ((unsigned)iz * g.H + (unsigned)iy) * g.W + (unsigned)ix;
        }
        for (int c0 = 0; c0 < g.Cgi; c0 += 4) {
            const int ci = c0 + kq;
            const bool cok = ci < g.Cgi;
            const float a = buf_load1(wr, (arow && cok) ? (wbase + ci * wci + tap) * 4u : GOOB);
            float bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                bv[u] = buf_load1(xr, (ok[u] && cok) ? (xch0 + ci * g.in_plane + sp[u]) * 4u : GOOB);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] = mfma_16x16x4(a, bv[u], acc[u]);
        }
    }

    // Epilogue: lane holds channels 4*kq + r of the block at position col of each tile.
    const int cnt = min(PTILE, g.S - pt * PTILE);
    const auto yr = make_rsrc(g.y ? g.y + (size_t)n * g.C_out * g.S : g.x,
                              g.y ? (unsigned)g.C_out * g.S * 4u : 0u);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = cb * 16 + 4 * kq + r;
        const bool cv = co < g.Cgo;
        const int cgl = grp * g.Cgo + co;
        const float bias = (g.b && cv) ? g.b[cgl] : 0.0f;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = activate<ACT>(acc[u][r] + bias);
        if (g.y) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                buf_store1(v[u] * g.out_scale, yr,
                           (cv && pv[u]) ? ((unsigned)cgl * g.S + pos[u]) * 4u : GOOB);
        }
        if (g.part) {
            float s = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) s += pv[u] ? v[u] : 0.0f;
            const float mean = row_sum16(s) / (float)cnt;
            float q = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float d = v[u] - mean;
                q += pv[u] ? d * d : 0.0f;
            }
            q = row_sum16(q);
            if (col == 0 && cv)
                g.part[((size_t)n * g.C_out + cgl) * g.T + pt] = v4f{(float)cnt, mean, q, 0.0f};
        }
    }
}

__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Softmax over C channels at every position of y[N][C][S], in place; one
// thread per position, one wave per 64-position tile.
__global__ __launch_bounds__(GT) void gen_softmax_kernel(float *y, v4f *part, int C, int S, int T,
                                                         int blocks_per_sample, float out_scale) {
    const int n = blockIdx.x / blocks_per_sample;
    const int blk = blockIdx.x - n * blocks_per_sample;
    const int pos = blk * GT + threadIdx.x;
    const int pt = blk * (GT / PTILE) + (threadIdx.x >> 6);
    if (pt * PTILE >= S) return;  // whole wave past the end
    const bool valid = pos < S;
    float *p = y + (size_t)n * C * S + (valid ? pos : 0);
    float m = -INFINITY;
    for (int c = 0; c < C; ++c) m = fmaxf(m, p[(size_t)c * S]);
    float sum = 0.0f;
    for (int c = 0; c < C; ++c) sum += expf(p[(size_t)c * S] - m);
    const float inv = 1.0f / sum;
    const int cnt = min(PTILE, S - pt * PTILE);
    for (int c = 0; c < C; ++c) {
        const float v = expf(p[(size_t)c * S] - m) * inv;
        if (part) {
            const float mean = wave_sum(valid ? v : 0.0f) / (float)cnt;
            const float d = v - mean;
            const float q = wave_sum(valid ? d * d : 0.0f);
            if ((threadIdx.x & 63) == 0)
                part[((size_t)n * C + c) * T + pt] = v4f{(float)cnt, mean, q, 0.0f};
        }
        if (valid) p[(size_t)c * S] = v * out_scale;
    }
}

__device__ __forceinline__ void chan_merge_d(double &n, double &mean, double &m2, double nb,
                                             double meanb, double m2b) {
    const double nn = n + nb;
    if (nn > 0.0) {
        const double delta = meanb - mean;
        const double f = nb / nn;
        mean += delta * f;
        m2 += m2b + delta * delta * n * f;
    }
    n = nn;
}

// One workgroup per (sample, norm group) of cpg channels.  Dynamic LDS:
// GT x 3 doubles for the tree, then cpg x 3 doubles of channel triples.
__global__ __launch_bounds__(GT) void gen_finalize_kernel(const v4f *part, int C, int T, int cpg,
                                                          int NG, int norm, const float *gamma,
                                                          const float *beta, float eps,
                                                          float inv_div, float *mean_out,
                                                          v2f *ss) {
    extern __shared__ double shd[];
    double *tr = shd;             // [3][GT]
    double *ch = shd + 3 * GT;    // [3][cpg]
    __shared__ double grp_mean, grp_rstd;
    const int n = blockIdx.x / NG, grp = blockIdx.x - n * NG;
    const int tid = threadIdx.x;
    for (int cl = 0; cl < cpg; ++cl) {
        const int c = grp * cpg + cl;
        const v4f *pp = part + ((size_t)n * C + c) * T;
        double cn = 0.0, mu = 0.0, m2 = 0.0;
        for (int t = tid; t < T; t += GT) {
            const v4f q = pp[t];
            chan_merge_d(cn, mu, m2, q[0], q[1], q[2]);
        }
        tr[tid] = cn; tr[GT + tid] = mu; tr[2 * GT + tid] = m2;
        __syncthreads();
        for (int h = GT / 2; h > 0; h >>= 1) {
            if (tid < h) {
                double a = tr[tid], b = tr[GT + tid], c2 = tr[2 * GT + tid];
                chan_merge_d(a, b, c2, tr[tid + h], tr[GT + tid + h], tr[2 * GT + tid + h]);
                tr[tid] = a; tr[GT + tid] = b; tr[2 * GT + tid] = c2;
            }
            __syncthreads();
        }
        if (tid == 0) { ch[cl] = tr[0]; ch[cpg + cl] = tr[GT]; ch[2 * cpg + cl] = tr[2 * GT]; }
        __syncthreads();
    }
    if (tid == 0) {
        double cn = 0.0, mu = 0.0, m2 = 0.0;
        for (int cl = 0; cl < cpg; ++cl) chan_merge_d(cn, mu, m2, ch[cl], ch[cpg + cl], ch[2 * cpg + cl]);
        grp_mean = mu;
        grp_rstd = 1.0 / sqrt(m2 / cn + (double)eps);
    }
    __syncthreads();
    for (int cl = tid; cl < cpg; cl += GT) {
        const int c = grp * cpg + cl;
        double scale = inv_div, shift = 0.0;
        if (norm) {
            const double ga = gamma ? (double)gamma[c] : 1.0;
            const double be = beta ? (double)beta[c] : 0.0;
            scale = ga * grp_rstd * inv_div;
            shift = (be - grp_mean * ga * grp_rstd) * inv_div;
        }
        if (mean_out) mean_out[(size_t)n * C + c] = (float)(ch[cpg + cl] * scale + shift);
        else ss[(size_t)n * C + c] = v2f{(float)scale, (float)shift};
    }
}

// y[plane][i] = y * scale[plane] + shift[plane]; blockIdx.x = plane.
constexpr int APPLY_CHUNK = GT * 8;
__global__ __launch_bounds__(GT) void gen_apply_kernel(float *y, const v2f *ss, int S) {
    const v2f sc = ss[blockIdx.x];
    float *p = y + (size_t)blockIdx.x * S;
    const int end = min(S, (int)(blockIdx.y + 1) * APPLY_CHUNK);
    for (int i = blockIdx.y * APPLY_CHUNK + threadIdx.x; i < end; i += GT) p[i] = fmaf(p[i], sc[0], sc[1]);
}

// One floor-mode max-pool pass over [N*C][Di][Hi][Wi] with kernel = stride =
// (kd, kh, kw).  first: the input is the conv output; apply the per-plane
// scale/shift (ss, or the uniform scale when ss is null) and index by the
// conv-grid position.  Otherwise carry in_idx (may be null when no argmax is
// wanted).
__global__ __launch_bounds__(GT) void gen_pool_kernel(const float *in, const int32_t *in_idx,
                                                      const v2f *ss, float uni_scale, int first,
                                                      int Di, int Hi, int Wi, int kd, int kh,
                                                      int kw, int Dq, int Hq, int Wq,
                                                      long long total, float *out,
                                                      int32_t *out_idx) {
    const long long i = (long long)blockIdx.x * GT + threadIdx.x;
    if (i >= total) return;
    const int wq = (int)(i % Wq);
    long long r = i / Wq;
    const int hq = (int)(r % Hq); r /= Hq;
    const int dq = (int)(r % Dq);
    const long long plane = r / Dq;
    const size_t in_plane = (size_t)Di * Hi * Wi;
    const float *ip = in + plane * in_plane;
    const int32_t *ix = in_idx ? in_idx + plane * in_plane : nullptr;
    v2f sc = v2f{uni_scale, 0.0f};
    if (first && ss) sc = ss[plane];
    float best = 0.0f;
    int32_t best_i = -1;
    for (int a = 0; a < kd; ++a)
    for (int b = 0; b < kh; ++b)
    for (int e = 0; e < kw; ++e) {
        const int off = ((dq * kd + a) * Hi + (hq * kh + b)) * Wi + (wq * kw + e);
        float v = ip[off];
        if (first) v = fmaf(v, sc[0], sc[1]);
        if (best_i < 0 || v > best) {
            best = v;
            best_i = first ? off : (ix ? ix[off] : 0);
        }
    }
    out[i] = best;
    if (out_idx) out_idx[i] = best_i;
}

struct GenLayout {
    bool stats, stage, softmax, finalize, apply;
    int T;
    size_t off_stage, off_part, off_ss, off_pv[2], off_pi[2], total;
    long long pool1;  // elements after the first pool pass
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

void layout(const GenericArgs &a, GenLayout &L) {
    const long long S = (long long)a.Do * a.Ho * a.Wo;
    const long long NC = (long long)a.N * a.C_out;
    L.softmax = a.act == ACT_SOFTMAX;
    L.stats = a.norm_groups > 0 || a.reduce == 1;
    L.stage = a.reduce == 2 || (a.reduce == 1 && L.softmax);
    L.finalize = L.stats;
    L.apply = a.reduce == 0 && a.norm_groups > 0;
    L.T = (int)((S + PTILE - 1) / PTILE);
    size_t off = 0;
    L.off_stage = off;
    if (L.stage) off = align256(off + (size_t)NC * S * 4);
    L.off_part = off;
    if (L.stats) off = align256(off + (size_t)NC * L.T * 16);
    L.off_ss = off;
    if (L.finalize && a.reduce != 1) off = align256(off + (size_t)NC * 8);
    L.pool1 = 0;
    if (a.reduce == 2) {
        const int kd = a.ndim == 3 ? a.pool_kernel : 1;
        L.pool1 = NC * (long long)(a.Do / kd) * (a.Ho / a.pool_kernel) * (a.Wo / a.pool_kernel);
        for (int i = 0; i < 2; ++i) {
            L.off_pv[i] = off;
            if (a.pool_repeats > 1) off = align256(off + (size_t)L.pool1 * 4);
            L.off_pi[i] = off;
            if (a.pool_repeats > 1 && a.argmax_wanted) off = align256(off + (size_t)L.pool1 * 4);
        }
    }
    L.total = off;
}

template <int ACT, bool TR>
hipError_t launch_conv(const GenConv &g, hipStream_t st) {
    const long long blocks = (g.tasks + 3) / 4;
    gen_conv_kernel<ACT, TR><<<dim3((unsigned)blocks), dim3(GT), 0, st>>>(g);
    return hipGetLastError();
}

}  // namespace

bool generic_supported(const GenericArgs &a) {
    const long long S = (long long)a.Do * a.Ho * a.Wo;
    const long long in_plane = (long long)a.D * a.H * a.W;
    const int Cgi = a.C_in / a.groups, Cgo = a.C_out / a.groups;
    const long long taps = (long long)a.kd * a.kh * a.kw;
    // every raw buffer resource below 2 GiB; coordinates below 2^20
    if ((long long)a.C_in * in_plane * 4 >= RES_MAX) return false;
    if ((long long)a.C_out * S * 4 >= RES_MAX) return false;
    const long long w_elems = a.transposed ? (long long)a.C_in * Cgo * taps
                                           : (long long)a.C_out * Cgi * taps;
    if (w_elems * 4 >= RES_MAX) return false;
    const int lim = 1 << 20;
    if (a.D >= lim || a.H >= lim || a.W >= lim || a.Do >= lim || a.Ho >= lim || a.Wo >= lim) return false;
    if (a.pd >= lim || a.ph >= lim || a.pw >= lim) return false;
    if ((long long)a.dd * a.kd >= lim || (long long)a.dh * a.kh >= lim || (long long)a.dw * a.kw >= lim)
        return false;
    // finalize keeps a group's channel triples in LDS
    const int cpg = a.norm_groups > 0 ? a.C_out / a.norm_groups : 1;
    if (cpg > 2048) return false;
    if (a.reduce == 2 && (long long)a.pool_kernel * a.pool_kernel * a.pool_kernel > (1 << 20)) return false;
    // launch grids: the apply kernel's chunk axis, and 32-bit block counts
    if (S >= (1LL << 27)) return false;
    const long long T = (S + PTILE - 1) / PTILE;
    const long long cob = (Cgo + 15) / 16;
    if ((long long)a.N * T * a.groups * cob / 4 >= (1LL << 31) - 1) return false;
    if ((long long)a.N * a.C_out * S / GT >= (1LL << 31) - 1) return false;
    return true;
}

size_t generic_workspace(const GenericArgs &a) {
    GenLayout L;
    layout(a, L);
    return L.total;
}

hipError_t launch_generic(const GenericArgs &a, hipStream_t st) {
    GenLayout L;
    layout(a, L);
    char *ws = static_cast<char *>(a.workspace);
    const int S = a.Do * a.Ho * a.Wo;
    v4f *part = L.stats ? reinterpret_cast<v4f *>(ws + L.off_part) : nullptr;
    float *stage = L.stage ? reinterpret_cast<float *>(ws + L.off_stage) : nullptr;
    v2f *ss = (L.finalize && a.reduce != 1) ? reinterpret_cast<v2f *>(ws + L.off_ss) : nullptr;
    float *y = a.reduce == 0 ? a.out : stage;  // nullptr: mean of an elementwise activation
    hipError_t e;

    // 1. conv (+ bias + elementwise activation)
    GenConv g{};
    g.x = a.x; g.w = a.w; g.b = a.b;
    g.y = y;
    g.part = L.softmax ? nullptr : part;
    g.C_in = a.C_in; g.C_out = a.C_out; g.G = a.groups;
    g.Cgi = a.C_in / a.groups; g.Cgo = a.C_out / a.groups;
    g.cob = (g.Cgo + 15) / 16;
    g.T = L.T;
    g.tasks = (long long)a.N * L.T * a.groups * g.cob;
    g.D = a.D; g.H = a.H; g.W = a.W; g.Do = a.Do; g.Ho = a.Ho; g.Wo = a.Wo; g.S = S;
    g.kd = a.kd; g.kh = a.kh; g.kw = a.kw;
    g.sd = a.sd; g.sh = a.sh; g.sw = a.sw; g.pd = a.pd; g.ph = a.ph; g.pw = a.pw;
    g.dd = a.dd; g.dh = a.dh; g.dw = a.dw;
    g.rsd = 1.0f / a.sd; g.rsh = 1.0f / a.sh; g.rsw = 1.0f / a.sw;
    g.in_plane = (unsigned)a.D * a.H * a.W;
    const unsigned taps = (unsigned)a.kd * a.kh * a.kw;
    g.w_elems = a.transposed ? (unsigned)a.C_in * g.Cgo * taps : (unsigned)a.C_out * g.Cgi * taps;
    // the conv writes the final values when nothing follows but the divide
    g.out_scale = (!L.softmax && a.norm_groups == 0 && a.reduce == 0) ? a.inv_div : 1.0f;
    const int act = L.softmax ? ACT_NONE : a.act;
#define CNF_GEN_CASE(A)                                                             \
    case A: e = a.transposed ? launch_conv<A, true>(g, st) : launch_conv<A, false>(g, st); break;
    switch (act) {
        CNF_GEN_CASE(ACT_NONE)
        CNF_GEN_CASE(ACT_HARDSWISH)
        CNF_GEN_CASE(ACT_GELU_ERF)
        CNF_GEN_CASE(ACT_GELU_TANH)
    default: return hipErrorInvalidValue;
    }
#undef CNF_GEN_CASE
    if (e != hipSuccess) return e;

    // 2. channel softmax
    if (L.softmax) {
        const int bps = (S + GT - 1) / GT;
        const float sc = (a.norm_groups == 0 && a.reduce == 0) ? a.inv_div : 1.0f;
        gen_softmax_kernel<<<dim3((unsigned)((long long)a.N * bps)), dim3(GT), 0, st>>>(
            y, part, a.C_out, S, L.T, bps, sc);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // 3. statistics -> scale / shift (or the mean itself)
    if (L.finalize) {
        const int NG = a.norm_groups > 0 ? a.norm_groups : a.C_out;
        const int cpg = a.C_out / NG;
        const size_t lds = sizeof(double) * 3 * (GT + cpg);
        gen_finalize_kernel<<<dim3((unsigned)((long long)a.N * NG)), dim3(GT), lds, st>>>(
            part, a.C_out, L.T, cpg, NG, a.norm_groups > 0, a.gamma, a.beta, a.eps, a.inv_div,
            a.reduce == 1 ? a.out : nullptr, ss);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // 4. in-place normalisation of the output
    if (L.apply) {
        const unsigned chunks = (unsigned)((S + APPLY_CHUNK - 1) / APPLY_CHUNK);
        gen_apply_kernel<<<dim3((unsigned)((long long)a.N * a.C_out), chunks), dim3(GT), 0, st>>>(
            a.out, ss, S);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // 5. max-pool passes
    if (a.reduce == 2) {
        const int kd = a.ndim == 3 ? a.pool_kernel : 1, k = a.pool_kernel;
        int Di = a.Do, Hi = a.Ho, Wi = a.Wo;
        const float *in = stage;
        const int32_t *in_idx = nullptr;
        for (int r = 0; r < a.pool_repeats; ++r) {
            const int Dq = Di / kd, Hq = Hi / k, Wq = Wi / k;
            const long long total = (long long)a.N * a.C_out * Dq * Hq * Wq;
            const bool last = r == a.pool_repeats - 1;
            float *o = last ? a.out : reinterpret_cast<float *>(ws + L.off_pv[r & 1]);
            int32_t *oi = last ? a.argmax
                               : (a.argmax_wanted ? reinterpret_cast<int32_t *>(ws + L.off_pi[r & 1])
                                                  : nullptr);
            const unsigned blocks = (unsigned)((total + GT - 1) / GT);
            gen_pool_kernel<<<dim3(blocks), dim3(GT), 0, st>>>(
                in, in_idx, ss, a.norm_groups > 0 ? 1.0f : a.inv_div, r == 0, Di, Hi, Wi, kd, k, k,
                Dq, Hq, Wq, total, o, oi);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            in = o;
            in_idx = oi;
            Di = Dq; Hi = Hq; Wi = Wq;
        }
    }
    return hipSuccess;
}

}  // namespace cnf
