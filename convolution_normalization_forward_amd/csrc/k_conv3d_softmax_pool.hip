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
// Mapping: one wave per pooled window (n, od, oh, ow).  A workgroup is one
// wave; the grid is one wave per resident slot (16 per CU) and each wave walks
// the windows blockIdx, blockIdx + grid, ..., prefetching the next window's
// input patch into registers while the current one is multiplied.
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

constexpr int WAVES_PER_CU = 16;  // persistent grid: one wave per resident slot (4 per SIMD)
constexpr int PP = 8;   // LDS row pitch of the patch

template <int CI, int KS>
struct PatchGeom {
    static constexpr int E = 4 + KS - 1;          // patch extent per axis
    static constexpr int ROWS = CI * E * E;       // rows of E floats
    static constexpr int CH = E * E * PP;         // floats per channel
    static constexpr int FLOATS = CI * CH;
    static constexpr int K = CI * KS * KS * KS;
    static constexpr int NS = (K + 3) / 4;
    // LDS offset of tap k = (ci, kd, kh, kw) inside the patch (0 past K: zero weight)
    static constexpr int tap_off(int k) {
        return k < K ? (k / (KS * KS * KS)) * CH + ((k / (KS * KS)) % KS) * (E * PP) +
                           ((k / KS) % KS) * PP + k % KS
                     : 0;
    }
};

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

template <int CI, int KS, int ACT, bool VEC, bool TWO>
__global__ __launch_bounds__(64)
void conv3d_softmax_pool_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                const float *__restrict__ bias, float *__restrict__ out,
                                int32_t *__restrict__ argmax, int N, int D, int H, int W,
                                int Ho, int Wo, int Dp, int Hp, int Wp)
{
    using G = PatchGeom<CI, KS>;
    static_assert(G::E <= 8 && G::E > 4, "patch rows are one float4 plus a tail");
    constexpr int TAIL = G::E - 4;             // floats after the leading float4 of a row
    constexpr int LSLOTS = (G::ROWS + 63) / 64;
    __shared__ float patch[2][G::FLOATS + 8];  // + a dump row for surplus slots

    const int lane = threadIdx.x;
    const int q = lane >> 4, c16 = lane & 15;
    const int HW = H * W;

    // B operand: w[co = l%16][k = 4s + l/16], zero past K.  A operand offset of
    // tap k in the patch; the four lane rows q take compile-time values.
    float wreg[G::NS];
    int toff[G::NS];
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
        const int k = 4 * s + q;
        wreg[s] = k < G::K ? w[c16 * G::K + k] : 0.0f;
        const int t0 = G::tap_off(4 * s), t1 = G::tap_off(4 * s + 1);
        const int t2 = G::tap_off(4 * s + 2), t3 = G::tap_off(4 * s + 3);
        toff[s] = q < 2 ? (q == 0 ? t0 : t1) : (q == 2 ? t2 : t3);
    }
    const float bc = bias ? bias[c16] : 0.0f;
    // A operand row m = l%16 is patch position (h = m/4, w = m%4)
    const int lbase = (c16 >> 2) * PP + (c16 & 3);
    // tie keys of this lane's 16 voxels (j = depth, q = row, r = column)
    const int kq = TWO ? (((q >> 1) << 4) | ((q & 1) << 1)) : q * 4;

    // Patch rows (ci, rd, rh) of E floats: a float4 and a TAIL part per row.
    int gro[LSLOTS], lro[LSLOTS];
#pragma unroll
    for (int u = 0; u < LSLOTS; ++u) {
        const int row = lane + 64 * u;
        const bool rok = row < G::ROWS;
        const int rr = rok ? row : 0;
        const int rh = rr % G::E, rd = (rr / G::E) % G::E, ci = rr / (G::E * G::E);
        gro[u] = (ci * D + rd) * HW + rh * W;
        lro[u] = rok ? ci * G::CH + rd * (G::E * PP) + rh * PP : G::FLOATS;
    }

    const int total = N * Dp * Hp * Wp;
    // XCD x owns windows [lo_x, hi_x) (contiguous, so neighbouring windows share
    // its L2); its waves (ids L = x, x + NXCD, ...) stride through that range.
    // (A grid smaller than NXCD just strides over all windows.)
    const int NG = gridDim.x, L = blockIdx.x;
    const bool split = NG >= NXCD;
    const int xcd = L % NXCD, slot = L / NXCD;
    const int waves_here = NG / NXCD + (xcd < NG % NXCD ? 1 : 0);
    const int lo = split ? xcd_remap(xcd, total) : 0;
    const int hi = split ? lo + total / NXCD + (xcd < total % NXCD ? 1 : 0) : total;
    const int first = split ? lo + slot : L, stride = split ? waves_here : NG;
    auto window_base = [&](int win, int &n, int &od, int &oh, int &ow) {
        int t = win;
        ow = t % Wp; t /= Wp;
        oh = t % Hp; t /= Hp;
        od = t % Dp;
        n = t / Dp;
        return ((size_t)n * CI * D + 4 * od) * HW + (size_t)(4 * oh) * W + 4 * ow;
    };

    v4f pa[LSLOTS];
    float pt[LSLOTS][TAIL];
#define CNF_FETCH(GBASE)                                                              \
    {                                                                                 \
        const float *xb = x + (GBASE);                                                \
        _Pragma("unroll") for (int u = 0; u < LSLOTS; ++u) {                          \
            const float *src = xb + gro[u];                                           \
            if constexpr (VEC) {                                                      \
                pa[u] = *reinterpret_cast<const v4f *>(src);                       \
            } else {                                                                  \
                pa[u] = v4f{src[0], src[1], src[2], src[3]};                  \
            }                                                                         \
            _Pragma("unroll") for (int e = 0; e < TAIL; ++e) pt[u][e] = src[4 + e];   \
        }                                                                             \
    }
#define CNF_STASH(BUF)                                                                \
    {                                                                                 \
        _Pragma("unroll") for (int u = 0; u < LSLOTS; ++u) {                          \
            float *dst = &patch[BUF][lro[u]];                                         \
            *reinterpret_cast<v4f *>(dst) = pa[u];                                 \
            _Pragma("unroll") for (int e = 0; e < TAIL; ++e) dst[4 + e] = pt[u][e];   \
        }                                                                             \
    }

    int n, od, oh, ow;
    if (first >= hi) return;
    CNF_FETCH(window_base(first, n, od, oh, ow))
    CNF_STASH(0)
    int buf = 0;
    for (int win = first; win < hi; win += stride) {  // wave-uniform
        int nn, od2, oh2, ow2;
        const bool more = win + stride < hi;
        window_base(win, n, od, oh, ow);
        if (more) CNF_FETCH(window_base(win + stride, nn, od2, oh2, ow2))
        __syncthreads();  // patch[buf] is complete

        v4f acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
        const float *pb = patch[buf];
#pragma unroll
        for (int s = 0; s < G::NS; ++s) {
            const int a0 = lbase + toff[s];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = mfma_16x16x4(pb[a0 + j * G::E * PP], wreg[s], acc[j]);
        }

        // activation (softmax over the 16 channels = the 16 lanes of a row)
        float v[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float a = acc[j][r] + bc;
                if constexpr (ACT == ACT_SOFTMAX) {
                    const float m = row_max16(a);
                    const float e = __builtin_amdgcn_exp2f((a - m) * 1.4426950408889634f);
                    const float sum = row_sum16(e);
                    a = e * __builtin_amdgcn_rcpf(sum);
                } else {
                    a = activate<ACT>(a);
                }
                v[j][r] = a;
            }
        }
        // window max, then the first voxel (in tie order) that attains it
        float best = v[0][0];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) best = fmaxf(best, v[j][r]);
        best = fmaxf(best, __shfl_xor(best, 16, 64));
        best = fmaxf(best, __shfl_xor(best, 32, 64));
        int bkey = 1 << 30;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = TWO ? (kq | ((j >> 1) << 5) | ((r >> 1) << 3) |
                                       ((j & 1) << 2) | (r & 1))
                                    : (kq | (j << 4) | r);
                bkey = (v[j][r] == best) ? min(bkey, key) : bkey;
            }
        bkey = min(bkey, __shfl_xor(bkey, 16, 64));
        bkey = min(bkey, __shfl_xor(bkey, 32, 64));
        if (q == 0) {
            int a, b, c;
            key_abc(bkey, TWO, a, b, c);
            const size_t o = (((size_t)n * 16 + c16) * Dp + od) * Hp * Wp + (size_t)oh * Wp + ow;
            out[o] = best;
            if (argmax)
                argmax[o] = ((4 * od + a) * Ho + (4 * oh + b)) * Wo + (4 * ow + c);
        }
        if (more) CNF_STASH(buf ^ 1)  // buf^1 was last read in the previous iteration
        buf ^= 1;
    }
#undef CNF_FETCH
#undef CNF_STASH
}

template <int CI, int KS, int ACT, bool TWO>
hipError_t launch_t2(const Conv3dSoftmaxPoolArgs &a, hipStream_t st)
{
    const int total = a.N * a.Dp * a.Hp * a.Wp;
    static int cus[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (!cus[dev & 63]) {
        e = hipDeviceGetAttribute(&cus[dev & 63], hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    const int grid = total < cus[dev & 63] * WAVES_PER_CU ? total : cus[dev & 63] * WAVES_PER_CU;
    if (a.W % 4 == 0)
        hipLaunchKernelGGL((conv3d_softmax_pool_kernel<CI, KS, ACT, true, TWO>), dim3(grid), dim3(64),
                           0, st, a.x, a.w, a.b, a.out, a.argmax, a.N, a.D, a.H, a.W, a.Ho, a.Wo,
                           a.Dp, a.Hp, a.Wp);
    else
        hipLaunchKernelGGL((conv3d_softmax_pool_kernel<CI, KS, ACT, false, TWO>), dim3(grid),
                           dim3(64), 0, st, a.x, a.w, a.b, a.out, a.argmax, a.N, a.D, a.H, a.W,
                           a.Ho, a.Wo, a.Dp, a.Hp, a.Wp);
    return hipGetLastError();
}

template <int CI, int KS, int ACT>
hipError_t launch_t(const Conv3dSoftmaxPoolArgs &a, hipStream_t st)
{
    return a.two_stage ? launch_t2<CI, KS, ACT, true>(a, st) : launch_t2<CI, KS, ACT, false>(a, st);
}

}  // namespace

bool conv3d_softmax_pool_supported(int C_in, int C_out, int kernel, int act, int pool_total)
{
    // exactly the instantiations launch_conv3d_softmax_pool dispatches to
    if (C_out != 16 || pool_total != 4) return false;
    if (C_in == 3 && kernel == 3)
        return act == ACT_SOFTMAX || act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF ||
               act == ACT_GELU_TANH;
    return ((C_in == 3 && kernel == 2) || (C_in == 1 && kernel == 3)) && act == ACT_SOFTMAX;
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
    CNF_CASE(3, 3, ACT_GELU_TANH)
    CNF_CASE(3, 2, ACT_SOFTMAX)
    CNF_CASE(1, 3, ACT_SOFTMAX)
#undef CNF_CASE
    return hipErrorInvalidValue;
}

}  // namespace cnf
