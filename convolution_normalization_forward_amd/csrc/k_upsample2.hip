// k_upsample2.hip -- the general family's conv stage for one shape: a 2-D
// ConvTranspose2d with a 3x3 kernel, stride 2, padding 1 and output_padding 1
// over conv groups of 8 input / 8 output channels (the upsampling form of the
// layer on page "Kimi-K2.6__l2_p19": 64 -> 64 channels, groups 8, H x W ->
// 2H x 2W), fp32.  It writes the conv output (bias and activation applied)
// once, plus one (count, mean, M2) record per (sample, channel, block) in the
// layout the family's finalize pass merges.
//
// Output row o takes the taps kh for which o + 1 - kh is even: kh = 1 from
// input row o / 2 when o is even; kh = 0 from row (o + 1) / 2 and kh = 2 from
// row (o - 1) / 2 when o is odd (columns alike).  So the 2 x 2 output block
// (2i + a, 2j + b) depends only on inputs (i, j), (i, j + 1), (i + 1, j) and
// (i + 1, j + 1): one thread owns that block for the group's 8 output
// channels, reading 4 inputs per input channel and doing 9 multiply-adds per
// (input, output) channel pair -- 18 per output, split into four parity
// classes of 1, 2, 2 and 4 taps.  That is too thin and too uneven for MFMA
// tiles, so it runs on the VALU; the weights are the same for the whole
// workgroup and come through scalar loads.
//
// Workgroup: 4 input rows x 64 input columns (256 threads) of one (sample,
// group); its statistics are taken over its 8 channels' 4 x 256 outputs each,
// two-pass in fp32 (mean, then summed squared deviations).
//
// When a norm follows, the conv output is never stored un-normalised: a first
// launch (MODE_STATS) only takes the statistics, the family's finalize turns
// them into a scale and shift per (sample, channel), and a second launch
// (MODE_NORM) recomputes the conv -- bit for bit the same values -- and stores
// act(conv) * scale + shift once.  The conv is 18 multiply-adds per output;
// storing, re-reading and rewriting the 4-byte output costs more.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int UT = 256;   // threads
constexpr int QC = 64;    // input columns per workgroup (one wave per input row)
constexpr int QR = UT / QC;
constexpr int G8 = 8;     // channels per conv group, in and out

__device__ __forceinline__ float wave_sum(float v)
{
    v = row_sum16(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

enum { MODE_WRITE = 0, MODE_STATS = 1, MODE_NORM = 2 };

// MODE_WRITE: store act(conv) * out_scale, and the statistics if part is set;
// MODE_STATS: statistics only; MODE_NORM: store act(conv) * ss.x + ss.y.
template <int ACT, int MODE>
__global__ __launch_bounds__(UT)
void upsample2_conv_kernel(const float *__restrict__ x, const float *__restrict__ w,
                           const float *__restrict__ bias, float *__restrict__ y,
                           v4f *__restrict__ part, const v2f *__restrict__ ss, int C, int H,
                           int W, int G, int T, float out_scale)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = blockIdx.x * QC + lane;
    const int i = blockIdx.y * QR + wave;
    const int n = blockIdx.z / G, g = blockIdx.z - (blockIdx.z / G) * G;
    const bool valid = i < H && j < W;
    const bool r1 = i + 1 < H, c1 = j + 1 < W;
    const int Ho = 2 * H, Wo = 2 * W;
    const size_t HW = (size_t)H * W;
    const float *xg = x + ((size_t)n * C + (size_t)g * G8) * HW;
    const float *wg = w + (size_t)g * G8 * G8 * 9;  // [ci][co][kh][kw] of the group

    // acc[co][p]: p = 0 (even row, even col), 1 (even, odd), 2 (odd, even), 3 (odd, odd)
    float acc[G8][4];
#pragma unroll
    for (int co = 0; co < G8; ++co) {
        const float b = bias ? bias[g * G8 + co] : 0.0f;
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[co][p] = b;
    }
    const int o00 = valid ? i * W + j : 0;
    // one input channel per iteration: its 72 weights fit the scalar registers
    // (all 576 of the group at once would spill into vector-register lanes)
#pragma unroll 1
    for (int ci = 0; ci < G8; ++ci) {
        const float *xc = xg + (size_t)ci * HW;
        const float x00 = valid ? xc[o00] : 0.0f;
        const float x01 = valid && c1 ? xc[o00 + 1] : 0.0f;
        const float x10 = valid && r1 ? xc[o00 + W] : 0.0f;
        const float x11 = valid && r1 && c1 ? xc[o00 + W + 1] : 0.0f;
#pragma unroll
        for (int co = 0; co < G8; ++co) {
            const float *k = wg + (ci * G8 + co) * 9;  // k[kh * 3 + kw]
            acc[co][0] = fmaf(x00, k[4], acc[co][0]);
            acc[co][1] = fmaf(x01, k[3], fmaf(x00, k[5], acc[co][1]));
            acc[co][2] = fmaf(x10, k[1], fmaf(x00, k[7], acc[co][2]));
            acc[co][3] = fmaf(x11, k[0], fmaf(x10, k[2], fmaf(x01, k[6], fmaf(x00, k[8], acc[co][3]))));
        }
    }
#pragma unroll
    for (int co = 0; co < G8; ++co)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[co][p] = activate<ACT>(acc[co][p]);

    if (MODE != MODE_STATS && valid) {
#pragma unroll
        for (int co = 0; co < G8; ++co) {
            const size_t c = (size_t)n * C + (size_t)g * G8 + co;
            float sc = out_scale, sh = 0.0f;
            if constexpr (MODE == MODE_NORM) {
                const v2f t = ss[c];
                sc = t[0];
                sh = t[1];
            }
            float *o = y + (c * Ho + 2 * i) * Wo + 2 * j;
            *reinterpret_cast<v2f *>(o) = v2f{fmaf(acc[co][0], sc, sh), fmaf(acc[co][1], sc, sh)};
            *reinterpret_cast<v2f *>(o + Wo) = v2f{fmaf(acc[co][2], sc, sh), fmaf(acc[co][3], sc, sh)};
        }
    }
    if (MODE == MODE_NORM || !part) return;  // workgroup-uniform

    // statistics of the block: 4 outputs per valid thread and channel
    __shared__ float red[QR][G8];
    __shared__ float mean_s[G8];
    const int rows = min(QR, H - (int)blockIdx.y * QR), cols = min(QC, W - (int)blockIdx.x * QC);
    const float cnt = 4.0f * (float)(rows * cols);
#pragma unroll
    for (int co = 0; co < G8; ++co) {
        const float s = valid ? (acc[co][0] + acc[co][1]) + (acc[co][2] + acc[co][3]) : 0.0f;
        const float t = wave_sum(s);
        if (lane == 0) red[wave][co] = t;
    }
    __syncthreads();
    if (tid < G8) {
        float s = 0.0f;
#pragma unroll
        for (int r = 0; r < QR; ++r) s += red[r][tid];
        mean_s[tid] = s / cnt;
    }
    __syncthreads();
    float q[G8];
#pragma unroll
    for (int co = 0; co < G8; ++co) {
        const float m = mean_s[co];
        float d = 0.0f;
#pragma unroll
        for (int p = 0; p < 4; ++p) d = fmaf(acc[co][p] - m, acc[co][p] - m, d);
        q[co] = wave_sum(valid ? d : 0.0f);
    }
    __syncthreads();  // every wave has read mean_s and red's first use is over
    if (lane == 0) {
#pragma unroll
        for (int co = 0; co < G8; ++co) red[wave][co] = q[co];
    }
    __syncthreads();
    if (tid < G8) {
        float m2 = 0.0f;
#pragma unroll
        for (int r = 0; r < QR; ++r) m2 += red[r][tid];
        const int tile = blockIdx.y * gridDim.x + blockIdx.x;
        part[((size_t)n * C + (size_t)g * G8 + tid) * T + tile] = v4f{cnt, mean_s[tid], m2, 0.0f};
    }
}

}  // namespace

bool upsample2_supported(const GenericArgs &a)
{
    return a.transposed && a.ndim == 2 && a.dtype == 0 && a.kh == 3 && a.kw == 3 && a.sh == 2 &&
           a.sw == 2 && a.ph == 1 && a.pw == 1 && a.dh == 1 && a.dw == 1 && a.Ho == 2 * a.H &&
           a.Wo == 2 * a.W && a.groups >= 1 && a.C_in == G8 * a.groups &&
           a.C_out == G8 * a.groups && a.reduce == 0 && a.act != ACT_SOFTMAX &&
           (long long)a.Ho * a.Wo < (1LL << 31) && (long long)a.N * a.groups < 65536 &&
           (a.H + QR - 1) / QR < 65536;
}

int upsample2_tiles(int H, int W)
{
    return ((H + QR - 1) / QR) * ((W + QC - 1) / QC);
}

hipError_t launch_upsample2(const GenericArgs &a, float *y, void *part, int T, float out_scale,
                            const void *ss, int mode, hipStream_t st)
{
    if (!upsample2_supported(a) || (part && T < upsample2_tiles(a.H, a.W))) return hipErrorInvalidValue;
    if ((mode == MODE_STATS && !part) || (mode == MODE_NORM && !ss) || mode < 0 || mode > 2)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.W + QC - 1) / QC), (unsigned)((a.H + QR - 1) / QR),
                    (unsigned)(a.N * a.groups));
    const float *x = static_cast<const float *>(a.x), *w = static_cast<const float *>(a.w);
    v4f *pp = static_cast<v4f *>(part);
    const v2f *sp = static_cast<const v2f *>(ss);
#define CNF_UP2M(A, M)                                                                            \
    hipLaunchKernelGGL((upsample2_conv_kernel<A, M>), grid, dim3(UT), 0, st, x, w, a.b, y, pp, sp, \
                       a.C_out, a.H, a.W, a.groups, T, out_scale)
#define CNF_UP2(A)                                                           \
    if (mode == MODE_WRITE) CNF_UP2M(A, MODE_WRITE);                         \
    else if (mode == MODE_STATS) CNF_UP2M(A, MODE_STATS);                    \
    else CNF_UP2M(A, MODE_NORM)
    // a pass that writes the output is the dominant launch
    hipError_t e = mode != MODE_STATS ? dominant_begin(st) : hipSuccess;
    if (e != hipSuccess) return e;
    switch (a.act) {
    case ACT_NONE: CNF_UP2(ACT_NONE); break;
    case ACT_HARDSWISH: CNF_UP2(ACT_HARDSWISH); break;
    case ACT_GELU_ERF: CNF_UP2(ACT_GELU_ERF); break;
    case ACT_GELU_TANH: CNF_UP2(ACT_GELU_TANH); break;
    default: return hipErrorInvalidValue;
    }
#undef CNF_UP2
#undef CNF_UP2M
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mode != MODE_STATS ? dominant_end(st) : hipSuccess;
}

}  // namespace cnf
