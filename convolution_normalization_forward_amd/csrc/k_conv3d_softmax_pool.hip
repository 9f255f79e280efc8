// k_conv3d_softmax_pool.hip -- Conv3d (C_out = 16, small C_in * k^3) +
// softmax over the channels + a 4x4x4 max pool with argmax.
//
// Page "Kimi-K2.6__l2_p6": Conv3d -> softmax(dim=1) -> MaxPool3d(2) ->
// MaxPool3d(2).  The trace shows that the two floor-mode 2-pools are one
// floor-mode 4-pool (same extents, same maxima), that only conv voxels inside
// the 4*Dp x 4*Hp x 4*Wp corner ever reach the output, and that the softmax
// (over channels) cannot be moved past the pools (over space).  So each pooled
// output window needs exactly 4x4x4 conv voxels x 16 channels, and nothing
// else is computed.
//
// Mapping: one wave per pooled window (n, od, oh, ow); a workgroup is one
// wave and walks WPW consecutive windows.
//   * The window's input patch (C_in x (4+k-1)^3) is staged in LDS with row
//     pitch 8.
//   * Tile j (j = 0..3) is conv depth 4*od + j: a 16x16 MFMA result with
//     rows = the 16 positions of the 4x4 (h, w) patch and columns = the 16
//     output channels (v_mfma_f32_16x16x4f32, K = C_in*k^3 padded to a
//     multiple of 4 with zero weights).  Weights (B operand) live in registers;
//     the im2col operand (A) is read from LDS through a per-lane offset table.
//   * Lane l holds positions (h = l/16, w = r) of channel l%16, so the softmax
//     over channels is a max and a sum across the 16 lanes of a DPP row.
//   * The window maximum and its argmax are reduced in-lane over (depth, w),
//     then across the four rows with lane shuffles.  Ties resolve as the
//     literal sequence of pools would (first 2x2x2 block in scan order, then
//     first voxel inside it), or in plain row-major order for a single 4-pool.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int WPW = 4;  // windows per wave
constexpr int PP = 8;   // LDS row pitch of the patch

template <int CI, int KS>
struct PatchGeom {
    static constexpr int E = 4 + KS - 1;          // patch extent per axis
    static constexpr int ROWS = CI * E * E;       // rows of E floats
    static constexpr int CH = E * E * PP;         // floats per channel
    static constexpr int FLOATS = CI * CH;
    static constexpr int K = CI * KS * KS * KS;
    static constexpr int NS = (K + 3) / 4;
};

__device__ __forceinline__ int tie_key(int a, int b, int c, int two_stage)
{
    return two_stage ? (((a >> 1) << 5) | ((b >> 1) << 4) | ((c >> 1) << 3) |
                        ((a & 1) << 2) | ((b & 1) << 1) | (c & 1))
                     : (a * 16 + b * 4 + c);
}

__device__ __forceinline__ void key_abc(int key, int two_stage, int &a, int &b, int &c)
{
    if (two_stage) {
        a = ((key >> 5) & 1) * 2 + ((key >> 2) & 1);
        b = ((key >> 4) & 1) * 2 + ((key >> 1) & 1);
        c = ((key >> 3) & 1) * 2 + (key & 1);
    } else {
        a = key >> 4;
        b = (key >> 2) & 3;
        c = key & 3;
    }
}

__device__ __forceinline__ void better(float &best, int &bkey, float v, int key)
{
    if (v > best || (v == best && key < bkey)) { best = v; bkey = key; }
}

template <int CI, int KS, int ACT>
__global__ __launch_bounds__(64)
void conv3d_softmax_pool_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                const float *__restrict__ bias, float *__restrict__ out,
                                int32_t *__restrict__ argmax, int N, int D, int H, int W,
                                int Ho, int Wo, int Dp, int Hp, int Wp, int two_stage)
{
    using G = PatchGeom<CI, KS>;
    __shared__ float patch[G::FLOATS];

    const int lane = threadIdx.x;
    const int q = lane >> 4, c16 = lane & 15;

    // B operand: w[co = l%16][k = 4s + l/16], zero past K.
    float wreg[G::NS];
    int toff[G::NS];
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
        const int k = 4 * s + q;
        wreg[s] = k < G::K ? w[c16 * G::K + k] : 0.0f;
        int off = 0;
        if (k < G::K) {
            const int kw = k % KS, kh = (k / KS) % KS, kd = (k / (KS * KS)) % KS,
                      ci = k / (KS * KS * KS);
            off = ci * G::CH + kd * (G::E * PP) + kh * PP + kw;
        }
        toff[s] = off;
    }
    const float bc = bias ? bias[c16] : 0.0f;
    // A operand row m = l%16 is patch position (h = m/4, w = m%4)
    const int lbase = (c16 >> 2) * PP + (c16 & 3);

    const int total = N * Dp * Hp * Wp;
    const int HW = H * W;
    for (int it = 0; it < WPW; ++it) {
        const int win = blockIdx.x * WPW + it;
        if (win >= total) break;  // wave-uniform
        int t = win;
        const int ow = t % Wp; t /= Wp;
        const int oh = t % Hp; t /= Hp;
        const int od = t % Dp;
        const int n = t / Dp;

        // stage the input patch: rows of E floats starting at (4od+., 4oh+., 4ow)
        const float *xs = x + (size_t)n * CI * D * HW;
        __syncthreads();  // previous window's reads are done
        for (int e = lane; e < G::ROWS * G::E; e += 64) {
            const int col = e % G::E, row = e / G::E;
            const int rh = row % G::E, rd = (row / G::E) % G::E, ci = row / (G::E * G::E);
            patch[ci * G::CH + rd * (G::E * PP) + rh * PP + col] =
                xs[((size_t)ci * D + 4 * od + rd) * HW + (size_t)(4 * oh + rh) * W + 4 * ow + col];
        }
        __syncthreads();

        v4f acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < G::NS; ++s) {
            const int a0 = lbase + toff[s];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = mfma_16x16x4(patch[a0 + j * G::E * PP], wreg[s], acc[j]);
        }

        float best = -1.0f;
        int bkey = 1 << 30;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[j][r] + bc;
                float pv;
                if constexpr (ACT == ACT_SOFTMAX) {
                    const float m = row_max16(v);
                    const float e = __expf(v - m);
                    const float sum = row_sum16(e);
                    pv = e / sum;
                } else {
                    pv = activate<ACT>(v);
                }
                if (j == 0 && r == 0) { best = pv; bkey = tie_key(j, q, r, two_stage); }
                else better(best, bkey, pv, tie_key(j, q, r, two_stage));
            }
        }
        // across the 4 rows (h = q)
#pragma unroll
        for (int sh = 16; sh <= 32; sh <<= 1) {
            const float ov = __shfl_xor(best, sh, 64);
            const int ok = __shfl_xor(bkey, sh, 64);
            better(best, bkey, ov, ok);
        }
        if (q == 0) {
            int a, b, c;
            key_abc(bkey, two_stage, a, b, c);
            const size_t o = (((size_t)n * 16 + c16) * Dp + od) * Hp * Wp + (size_t)oh * Wp + ow;
            out[o] = best;
            if (argmax)
                argmax[o] = ((4 * od + a) * Ho + (4 * oh + b)) * Wo + (4 * ow + c);
        }
    }
}

template <int CI, int KS, int ACT>
hipError_t launch_t(const Conv3dSoftmaxPoolArgs &a, hipStream_t st)
{
    const int total = a.N * a.Dp * a.Hp * a.Wp;
    const int grid = (total + WPW - 1) / WPW;
    hipLaunchKernelGGL((conv3d_softmax_pool_kernel<CI, KS, ACT>), dim3(grid), dim3(64), 0, st,
                       a.x, a.w, a.b, a.out, a.argmax, a.N, a.D, a.H, a.W, a.Ho, a.Wo, a.Dp,
                       a.Hp, a.Wp, a.two_stage);
    return hipGetLastError();
}

}  // namespace

bool conv3d_softmax_pool_supported(int C_in, int C_out, int kernel, int act, int pool_total)
{
    if (C_out != 16 || pool_total != 4) return false;
    if (!((C_in == 3 && (kernel == 3 || kernel == 2)) || (C_in == 1 && kernel == 3)))
        return false;
    return act == ACT_SOFTMAX || act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF;
}

hipError_t launch_conv3d_softmax_pool(const Conv3dSoftmaxPoolArgs &a, hipStream_t st)
{
    if ((size_t)a.N * a.Dp * a.Hp * a.Wp > (size_t)INT32_MAX) return hipErrorInvalidValue;
#define CNF_CASE(CI, KS, ACT) \
    if (a.C_in == CI && a.kernel == KS && a.act == ACT) return launch_t<CI, KS, ACT>(a, st);
    CNF_CASE(3, 3, ACT_SOFTMAX)
    CNF_CASE(3, 3, ACT_NONE)
    CNF_CASE(3, 3, ACT_HARDSWISH)
    CNF_CASE(3, 3, ACT_GELU_ERF)
    CNF_CASE(3, 2, ACT_SOFTMAX)
    CNF_CASE(1, 3, ACT_SOFTMAX)
#undef CNF_CASE
    return hipErrorInvalidValue;
}

}  // namespace cnf
