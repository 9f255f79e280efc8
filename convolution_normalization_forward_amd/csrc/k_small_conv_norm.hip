// k_small_conv_norm.hip -- small Conv2d/Conv3d (C_out = 16) + activation +
// InstanceNorm/GroupNorm + divide, one workgroup per sample, every conv
// output kept in registers so the result is written exactly once.
//
// Page "Kimi-K2.6__l2_p17": Conv2d -> InstanceNorm2d (affine off, biased
// variance, eps 1e-5) -> divide by 2.  This family covers samples whose whole
// conv output fits in the registers of one workgroup (<= 1024 positions x 16
// channels), e.g. the 8->16, 32x32 shrunken form of that problem.
//
// Mapping (4 waves per sample):
//   * The sample's input is staged whole in LDS (layout = the tensor's own).
//   * Positions are cut into tiles of 16; wave w owns tiles w, w+4, ...; each
//     tile is one 16x16 MFMA result (rows = 16 channels, columns = 16
//     positions; K = C_in * k^ndim padded to a multiple of 4 with zero
//     weights).  Weights (A operand) live in registers; the im2col operand
//     (B) is read from LDS through a per-lane offset table.
//   * Per-channel Welford triples are merged over the 16 lanes of a row (DPP),
//     over the 4 waves (LDS), then over the channels of each norm group; each
//     lane normalises its registers and stores them.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int THREADS = 256;
constexpr int MAXT = 16;          // tiles per wave -> <= 1024 positions per sample
constexpr int MAX_LDS_FLOATS = 14 * 1024;

template <int K>
struct SmallGeom {
    static constexpr int NS = (K + 3) / 4;
};

template <int CI, int KS, int ND, int ACT>
__global__ __launch_bounds__(THREADS)
void small_conv_norm_kernel(const float *__restrict__ x, const float *__restrict__ w,
                            const float *__restrict__ bias, const float *__restrict__ gamma,
                            const float *__restrict__ beta, float *__restrict__ out,
                            int D, int H, int W, int Do, int Ho, int Wo, int norm_groups,
                            float eps, float inv_div, int reduce_mean)
{
    constexpr int KD = ND == 3 ? KS : 1;
    constexpr int K = CI * KD * KS * KS;
    constexpr int NS = SmallGeom<K>::NS;
    extern __shared__ float lds[];

    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c16 = lane & 15;
    const int HW = H * W;
    const int P = Do * Ho * Wo;
    const int T = (P + 15) >> 4;
    const int in_floats = CI * D * HW;

    // Stage the whole sample, every load of a thread in flight before its LDS
    // stores (a load-then-store loop waits out one memory latency per element
    // group).  float4 when the sample size keeps every sample 16-byte aligned
    // (x itself is), else batches of 8 scalars.
    const float *xs = x + (size_t)n * in_floats;
    if ((in_floats & 3) == 0) {
        constexpr int MAXV = (MAX_LDS_FLOATS / 4 + THREADS - 1) / THREADS;
        const int nv = in_floats >> 2;
        const v4f *xs4 = reinterpret_cast<const v4f *>(xs);
        v4f buf[MAXV];
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            const int e = tid + u * THREADS;
            buf[u] = e < nv ? xs4[e] : v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            const int e = tid + u * THREADS;
            if (e < nv) reinterpret_cast<v4f *>(lds)[e] = buf[u];
        }
    } else {
        for (int e0 = 0; e0 < in_floats; e0 += 8 * THREADS) {
            float buf[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + tid + u * THREADS;
                buf[u] = e < in_floats ? xs[e] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + tid + u * THREADS;
                if (e < in_floats) lds[e] = buf[u];
            }
        }
    }

    float wreg[NS];
    int toff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int k = 4 * s + q;
        wreg[s] = k < K ? w[c16 * K + k] : 0.0f;
        int off = 0;
        if (k < K) {
            const int kw = k % KS, kh = (k / KS) % KS, kd = (k / (KS * KS)) % KD,
                      ci = k / (KD * KS * KS);
            off = ci * D * HW + kd * HW + kh * W + kw;
        }
        toff[s] = off;
    }
    float bch[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bch[r] = bias ? bias[4 * q + r] : 0.0f;
    __syncthreads();

    v4f acc[MAXT];
    float cnt = 0.f, mean[4] = {0.f, 0.f, 0.f, 0.f}, m2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MAXT; ++i) {
        const int t = wave + 4 * i;
        acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
        if (t < T) {
            int pos = t * 16 + c16;
            const bool valid = pos < P;
            pos = valid ? pos : P - 1;
            const int ow = pos % Wo, rest = pos / Wo;
            const int oh = rest % Ho, od = rest / Ho;
            const int base = od * HW + oh * W + ow;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                acc[i] = mfma_16x16x4(wreg[s], lds[base + toff[s]], acc[i]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = activate<ACT>(acc[i][r] + bch[r]);
            if (valid) {
                cnt += 1.0f;
                const float rn = __builtin_amdgcn_rcpf(cnt);
#pragma unroll
                for (int r = 0; r < 4; ++r) welford_push(mean[r], m2[r], acc[i][r], rn);
            }
        }
    }

    // per-channel scale/shift: y_norm = y * sc + sh (then the divide)
    float *red = lds;  // reuse: [4 waves][16][3], then [16][2] coefficients
    __syncthreads();   // everyone is done reading the input
    float sc[4], sh[4];
    if (norm_groups > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float nn = cnt, mm = mean[r], qq = m2[r];
            row_chan16(nn, mm, qq);
            if (c16 == 0) {
                float *e = red + (wave * 16 + 4 * q + r) * 3;
                e[0] = nn; e[1] = mm; e[2] = qq;
            }
        }
        __syncthreads();
        float *coef = red + 4 * 16 * 3;
        if (tid < 16) {
            const int c = tid, cg = 16 / norm_groups, g0 = (c / cg) * cg;
            float nn = 0.f, mm = 0.f, qq = 0.f;
            for (int j = 0; j < cg; ++j)
                for (int wv = 0; wv < 4; ++wv) {
                    const float *e = red + (wv * 16 + g0 + j) * 3;
                    chan_merge(nn, mm, qq, e[0], e[1], e[2]);
                }
            const float rstd = rsqrtf(qq / nn + eps);
            const float ga = gamma ? gamma[c] : 1.0f, be = beta ? beta[c] : 0.0f;
            coef[c * 2 + 0] = rstd * ga * inv_div;
            coef[c * 2 + 1] = (be - mm * rstd * ga) * inv_div;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) { sc[r] = coef[(4 * q + r) * 2]; sh[r] = coef[(4 * q + r) * 2 + 1]; }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) { sc[r] = inv_div; sh[r] = 0.0f; }
    }

    if (!reduce_mean) {
        float *o = out + (size_t)n * 16 * P;
#pragma unroll
        for (int i = 0; i < MAXT; ++i) {
            const int t = wave + 4 * i;
            const int pos = t * 16 + c16;
            if (t < T && pos < P) {
#pragma unroll
                for (int r = 0; r < 4; ++r) o[(size_t)(4 * q + r) * P + pos] = acc[i][r] * sc[r] + sh[r];
            }
        }
    } else {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < MAXT; ++i) {
            const int t = wave + 4 * i;
            if (t < T && t * 16 + c16 < P) {
#pragma unroll
                for (int r = 0; r < 4; ++r) s4[r] += acc[i][r] * sc[r] + sh[r];
            }
        }
        float *sums = red + 4 * 16 * 3 + 32;  // [4 waves][16]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = row_sum16(s4[r]);
            if (c16 == 0) sums[wave * 16 + 4 * q + r] = v;
        }
        __syncthreads();
        if (tid < 16) {
            const float v = sums[tid] + sums[16 + tid] + sums[32 + tid] + sums[48 + tid];
            out[(size_t)n * 16 + tid] = v / (float)P;
        }
    }
}

template <int CI, int KS, int ND, int ACT>
hipError_t launch_t(const SmallConvNormArgs &a, hipStream_t st)
{
    const size_t floats = (size_t)a.C_in * a.D * a.H * a.W;
    const size_t lds = (floats > 4 * 16 * 3 + 32 + 64 ? floats : 4 * 16 * 3 + 32 + 64) * sizeof(float);
    hipLaunchKernelGGL((small_conv_norm_kernel<CI, KS, ND, ACT>), dim3(a.N), dim3(THREADS), lds, st,
                       a.x, a.w, a.b, a.gamma, a.beta, a.out, a.D, a.H, a.W, a.Do, a.Ho, a.Wo,
                       a.norm_groups, a.eps, a.inv_div, a.reduce_mean);
    return hipGetLastError();
}

}  // namespace

bool small_conv_norm_supported(int C_in, int C_out, int kernel, int ndim, int D, int H, int W,
                               int act)
{
    if (C_out != 16) return false;
    if (act == ACT_SOFTMAX) return false;
    const bool inst = (ndim == 2 && kernel == 3 && (C_in == 8 || C_in == 4 || C_in == 3 || C_in == 1)) ||
                      (ndim == 3 && kernel == 3 && (C_in == 3 || C_in == 1));
    if (!inst) return false;
    const int Do = ndim == 3 ? D - kernel + 1 : 1, Ho = H - kernel + 1, Wo = W - kernel + 1;
    if ((long)Do * Ho * Wo > 4L * MAXT * 16) return false;
    if ((long)C_in * D * H * W > MAX_LDS_FLOATS) return false;
    return true;
}

hipError_t launch_small_conv_norm(const SmallConvNormArgs &a, hipStream_t st)
{
    const int nd = a.D == 1 && a.Do == 1 ? 2 : 3;
#define CNF_CASE(CI, KS, ND)                                                                     \
    if (a.C_in == CI && a.kernel == KS && nd == ND) {                                            \
        switch (a.act) {                                                                         \
        case ACT_NONE: return launch_t<CI, KS, ND, ACT_NONE>(a, st);                             \
        case ACT_HARDSWISH: return launch_t<CI, KS, ND, ACT_HARDSWISH>(a, st);                   \
        case ACT_GELU_ERF: return launch_t<CI, KS, ND, ACT_GELU_ERF>(a, st);                     \
        case ACT_GELU_TANH: return launch_t<CI, KS, ND, ACT_GELU_TANH>(a, st);                   \
        default: return hipErrorInvalidValue;                                                    \
        }                                                                                        \
    }
    CNF_CASE(8, 3, 2)
    CNF_CASE(4, 3, 2)
    CNF_CASE(3, 3, 2)
    CNF_CASE(1, 3, 2)
    CNF_CASE(3, 3, 3)
    CNF_CASE(1, 3, 3)
#undef CNF_CASE
    return hipErrorInvalidValue;
}

}  // namespace cnf
