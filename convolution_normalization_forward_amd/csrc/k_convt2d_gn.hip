// k_convt2d_gn.hip -- grouped ConvTranspose2d (stride 1, no padding, k = 3,
// 8 input and 8 output channels per group) + activation, writing y and one
// Welford partial per (sample, channel, row block); then an in-place
// GroupNorm pass over any norm grouping of the channels (InstanceNorm is
// GroupNorm with one channel per group), so the norm groups need not be the
// conv groups.
//
// Page "Kimi-K2.6__l2_p19": ConvTranspose2d(64 -> 64, k = 3, stride 1,
// groups 8) -> GELU -> GroupNorm(8) on 128 x 64 x 256 x 256, output 258 x 258.
// Second trace: out[i, j] = sum x[i - kh, j - kw] * W[ci, co, kh, kw] with x
// zero outside its extent, weights laid out (C_in, C_out/groups, kh, kw);
// first trace: GroupNorm statistics run over the channels of a norm group and
// all 258 x 258 positions, so they need the whole (sample, norm group) unit.
//
// Column-pair MFMA mapping.  A group has only 8 output channels, half of a
// 16-wide MFMA operand.  Output pixels (i, 2p) and (i, 2p+1) read the same
// input pixels shifted by one column, so writing the tap as v = kw - t + 1
// (t = pixel parity, v = 0..3) gives
//     y[co][i][2p + t] = sum_{ci, kh, v} x[ci][i - kh][2p + 1 - v] * A[(co,t)][(ci,kh,v)]
// with A[(co,t)][(ci,kh,v)] = W[ci][co][kh][v + t - 1] (zero outside 0..2).
// That is a 16 x 96 x 16 product per 16 column pairs: rows = (co, t), K =
// (ci, kh, v), columns = 16 column pairs.  A (72 distinct weights, padded to
// 96) stays in registers; B is read from an LDS tile of the input that is
// zero-padded on every side, so the loop has no bounds checks.  75% of the
// MFMA work is useful (72 of 96 K entries per row).
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int CG = 8;          // channels per group (in and out)
constexpr int KS = 3;
constexpr int R = 4;           // output rows per workgroup
constexpr int THREADS = 256;
constexpr int NB = 3;          // tiles in flight per wave
constexpr int PADL = 4;        // zero columns left of x inside an LDS row

__host__ __device__ constexpr int row_pitch(int W) { return ((W + 2 * PADL) + 3) & ~3; }

template <int ACT>
__global__ __launch_bounds__(THREADS, 2)
void convt2d_g8_kernel(const float *__restrict__ x, const float *__restrict__ wt,
                       const float *__restrict__ bias, float *__restrict__ y,
                       float *__restrict__ partials, int C, int H, int W, int Ho, int Wo,
                       int rblocks)
{
    extern __shared__ float lds[];
    const int RP = row_pitch(W);
    const int CSTR = (R + KS - 1) * RP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c16 = lane & 15;
    const int rb = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
    const int i0 = rb * R;
    const int G = C / CG;

    // ---- stage x rows i0-2 .. i0+R-1 of the group's 8 channels, zero padded
    const float *xg = x + ((size_t)n * C + (size_t)g * CG) * H * W;
    const int W4 = W >> 2;
    const int rows = R + KS - 1;
    for (int e = tid; e < CG * rows * (RP >> 2); e += THREADS) {
        const int c4 = e % (RP >> 2), rest = e / (RP >> 2);
        const int rr = rest % rows, ci = rest / rows;
        const int gr = i0 - (KS - 1) + rr;
        const int xc4 = c4 - PADL / 4;  // float4 column of x
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gr >= 0 && gr < H && xc4 >= 0 && xc4 < W4)
            v = reinterpret_cast<const float4 *>(xg + ((size_t)ci * H + gr) * W)[xc4];
        reinterpret_cast<float4 *>(lds + ci * CSTR + rr * RP)[c4] = v;
    }

    // ---- A operand: rows (co, t) = (l%16 / 2, l%16 % 2), K = (ci, kh, v = q)
    float wreg[CG * KS];
    {
        const int co = c16 >> 1, t = c16 & 1;
        const int kw = q + t - 1;
#pragma unroll
        for (int s = 0; s < CG * KS; ++s) {
            const int ci = s / KS, kh = s % KS;
            wreg[s] = (kw >= 0 && kw < KS)
                          ? wt[(((size_t)(g * CG + ci) * CG + co) * KS + kh) * KS + kw]
                          : 0.0f;
        }
    }
    // D rows 4q + r -> channel 2q + r/2, parity r%2
    const float b0 = bias ? bias[g * CG + 2 * q] : 0.0f;
    const float b1 = bias ? bias[g * CG + 2 * q + 1] : 0.0f;
    __syncthreads();

    const int PR = Wo >> 1;                 // column pairs per row
    const int rows_here = min(R, Ho - i0);
    const int npairs = rows_here * PR;
    const int T = (npairs + 15) >> 4;
    // per-lane sums of the lane's two channels 2q (a) and 2q+1 (b)
    float s1a = 0.f, s2a = 0.f, s1b = 0.f, s2b = 0.f;
    int cnt_i = 0;  // values per channel
    float *yg = y + ((size_t)n * C + (size_t)g * CG) * Ho * Wo;

    for (int t0 = wave; t0 < T; t0 += 4 * NB) {
        v4f acc[NB];
        int base[NB], prs[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            int p = (t0 + 4 * j) * 16 + c16;
            prs[j] = p;
            p = p < npairs ? p : npairs - 1;
            const int il = p / PR, pc = p - il * PR;
            // x column 2pc + 1 - v sits at LDS column 2pc + 1 - v + PADL
            base[j] = il * RP + 2 * pc + 1 - q + PADL;
            acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ci = 0; ci < CG; ++ci) {
#pragma unroll
            for (int kh = 0; kh < KS; ++kh) {
                const int s = ci * KS + kh;
                const int imm = ci * CSTR + (KS - 1 - kh) * RP;
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[j] = mfma_16x16x4(wreg[s], lds[base[j] + imm], acc[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int p = prs[j];
            if ((t0 + 4 * j) < T && p < npairs) {
                const int il = p / PR, pc = p - il * PR;
                const size_t o = (size_t)(i0 + il) * Wo + 2 * pc;
                float2 v0, v1;
                v0.x = activate<ACT>(acc[j][0] + b0);
                v0.y = activate<ACT>(acc[j][1] + b0);
                v1.x = activate<ACT>(acc[j][2] + b1);
                v1.y = activate<ACT>(acc[j][3] + b1);
                *reinterpret_cast<float2 *>(yg + (size_t)(2 * q) * Ho * Wo + o) = v0;
                *reinterpret_cast<float2 *>(yg + (size_t)(2 * q + 1) * Ho * Wo + o) = v1;
                s1a += v0.x + v0.y;
                s2a = fmaf(v0.x, v0.x, s2a); s2a = fmaf(v0.y, v0.y, s2a);
                s1b += v1.x + v1.y;
                s2b = fmaf(v1.x, v1.x, s2b); s2b = fmaf(v1.y, v1.y, s2b);
                cnt_i += 2;
            }
        }
    }

    // ---- one Welford triple per channel: the 16 lanes of a row share channels
    // 2q, 2q+1; rows merge in LDS, then the 4 waves in wave order
    __syncthreads();  // LDS reuse
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float s1 = j ? s1b : s1a, s2 = j ? s2b : s2a;
        float cnt = (float)cnt_i;
        float mean = cnt_i ? s1 / cnt : 0.0f;
        float m2 = cnt_i ? fmaxf(s2 - s1 * mean, 0.0f) : 0.0f;
        row_chan16(cnt, mean, m2);
        if (c16 == 0) {
            float *e = lds + (wave * CG + 2 * q + j) * 3;
            e[0] = cnt; e[1] = mean; e[2] = m2;
        }
    }
    __syncthreads();
    if (tid < CG) {
        float c2 = 0.f, m = 0.f, s2 = 0.f;
        for (int k = 0; k < 4; ++k) {
            const float *e = lds + (k * CG + tid) * 3;
            chan_merge(c2, m, s2, e[0], e[1], e[2]);
        }
        float *pp = partials + (((size_t)n * C + g * CG + tid) * rblocks + rb) * 3;
        pp[0] = c2; pp[1] = m; pp[2] = s2;
    }
    (void)G;
}

// One workgroup per (sample, channel): merge the row-block partials of every
// channel in the channel's norm group (NG groups of C / NG channels) in a
// fixed order (strided per thread, then in thread order), then normalise the
// channel's plane in place.
__global__ __launch_bounds__(256)
void convt2d_gn_pass_kernel(float *__restrict__ y, const float *__restrict__ partials,
                            const float *__restrict__ gamma, const float *__restrict__ beta,
                            int C, int NG, int plane, int rblocks, float eps, float inv_div)
{
    const int nc = blockIdx.x;
    const int n = nc / C, c = nc % C, cg = C / NG, c0 = (c / cg) * cg;
    const int tid = threadIdx.x;
    __shared__ float tri[256][3];
    __shared__ float coef[2];
    {
        // the group's channels' partials are contiguous: [c0 .. c0 + cg) x rblocks
        float cnt = 0.f, mean = 0.f, m2 = 0.f;
        const float *pp = partials + ((size_t)n * C + c0) * rblocks * 3;
        for (int r = tid; r < cg * rblocks; r += 256) chan_merge(cnt, mean, m2, pp[r * 3], pp[r * 3 + 1], pp[r * 3 + 2]);
        tri[tid][0] = cnt; tri[tid][1] = mean; tri[tid][2] = m2;
    }
    __syncthreads();
    if (tid == 0) {
        float tc = 0.f, tm = 0.f, tq = 0.f;
        for (int k = 0; k < 256; ++k) chan_merge(tc, tm, tq, tri[k][0], tri[k][1], tri[k][2]);
        const float rstd = rsqrtf(tq / tc + eps);
        const float ga = gamma ? gamma[c] : 1.0f, be = beta ? beta[c] : 0.0f;
        coef[0] = rstd * ga * inv_div;
        coef[1] = (be - tm * rstd * ga) * inv_div;
    }
    __syncthreads();
    const float sc = coef[0], sh = coef[1];
    float *p = y + (size_t)nc * plane;
    if ((plane & 3) == 0) {
        v4f *p4 = reinterpret_cast<v4f *>(p);
        const int n4 = plane / 4;
        int i = tid;
        for (; i + 3 * 256 < n4; i += 4 * 256) {
            v4f a0 = p4[i], a1 = p4[i + 256], a2 = p4[i + 512], a3 = p4[i + 768];
            p4[i] = a0 * sc + sh;
            p4[i + 256] = a1 * sc + sh;
            p4[i + 512] = a2 * sc + sh;
            p4[i + 768] = a3 * sc + sh;
        }
        for (; i < n4; i += 256) p4[i] = p4[i] * sc + sh;
    } else {
        for (int i = tid; i < plane; i += 256) p[i] = p[i] * sc + sh;
    }
}

// No norm: only the divide (when it is not 1).
__global__ __launch_bounds__(256)
void scale_kernel(float *__restrict__ y, size_t count, float sc)
{
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < count; i += (size_t)gridDim.x * 256) y[i] *= sc;
}

template <int ACT>
hipError_t launch_t(const ConvT2dArgs &a, hipStream_t st)
{
    const int rblocks = (a.Ho + R - 1) / R;
    const size_t lds = (size_t)CG * (R + KS - 1) * row_pitch(a.W) * sizeof(float);
    hipError_t e = dominant_begin(st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((convt2d_g8_kernel<ACT>), dim3(rblocks, a.groups, a.N), dim3(THREADS), lds,
                       st, a.x, a.w, a.b, a.out, a.partials, a.C_out, a.H, a.W, a.Ho, a.Wo,
                       rblocks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = dominant_end(st)) != hipSuccess) return e;
    if (a.norm_groups > 0) {
        hipLaunchKernelGGL(convt2d_gn_pass_kernel, dim3(a.N * a.C_out), dim3(256), 0, st, a.out,
                           a.partials, a.gamma, a.beta, a.C_out, a.norm_groups, a.Ho * a.Wo,
                           rblocks, a.eps, a.inv_div);
    } else if (a.inv_div != 1.0f) {
        const size_t count = (size_t)a.N * a.C_out * a.Ho * a.Wo;
        hipLaunchKernelGGL(scale_kernel, dim3(4096), dim3(256), 0, st, a.out, count, a.inv_div);
    }
    return hipGetLastError();
}

}  // namespace

bool convt2d_supported(int C_in, int C_out, int kernel, int groups, int H, int W, int act,
                       int norm, int num_groups)
{
    if (kernel != KS || groups < 1 || C_in != CG * groups || C_out != CG * groups) return false;
    if (W % 4 != 0 || H < 1) return false;
    if ((size_t)CG * (R + KS - 1) * row_pitch(W) * sizeof(float) > 64 * 1024) return false;
    if (act == ACT_SOFTMAX) return false;
    // any norm grouping of the channels: partials are per channel
    if (norm == 1 /* group */ && (num_groups < 1 || C_out % num_groups != 0)) return false;
    return true;
}

size_t convt2d_workspace(int N, int C_out, int Ho, int Wo)
{
    (void)Wo;
    const size_t rblocks = (Ho + R - 1) / R;
    return (size_t)N * C_out * rblocks * 3 * sizeof(float);
}

hipError_t launch_convt2d(const ConvT2dArgs &a, hipStream_t st)
{
    switch (a.act) {
    case ACT_NONE: return launch_t<ACT_NONE>(a, st);
    case ACT_HARDSWISH: return launch_t<ACT_HARDSWISH>(a, st);
    case ACT_GELU_ERF: return launch_t<ACT_GELU_ERF>(a, st);
    case ACT_GELU_TANH: return launch_t<ACT_GELU_TANH>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cnf
