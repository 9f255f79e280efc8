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
//     rows = the 16 output channels and columns = the 16 positions of the 4x4
//     (h, w) patch (v_mfma_f32_16x16x4f32, K = C_in*k^3 padded to a multiple
//     of 4 with zero weights).  Weights (A operand) live in registers; the
//     im2col operand (B) is read from LDS through a per-lane offset table.
//     The accumulator starts at the bias.
//   * Lane l holds channels 4*(l/16) + r (r = 0..3) of position l%16, so the
//     softmax over the 16 channels is 3 in-lane steps and two cross-row
//     exchanges (xor 16, xor 32, on the LDS pipe) per reduction, instead of a
//     16-lane DPP reduction per value.  (gfx950's permlane swaps would do the
//     exchange on the VALU, but each costs a copy and the swap there, and
//     this kernel is bound by VALU + MFMA issue: measured slower.)  For the
//     softmax, weights and bias carry the factor log2(e), so each
//     exponential is one exp2 of (logit - max).
//   * The window maximum of channel c and its argmax are reduced in-lane over
//     depth, then across the 16 lanes (positions) of the row.  Ties resolve as
//     the literal sequence of pools would (first 2x2x2 block in scan order, then
//     first voxel inside it), or in plain row-major order for a single 4-pool.
#include <atomic>
#include <type_traits>

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

    // A operand: w[co = l%16][k = 4s + l/16], zero past K (times log2 e for the
    // softmax).  B operand offset of tap k in the patch; the four lane rows q
    // take compile-time values.
    constexpr float LSCALE = ACT == ACT_SOFTMAX ? 1.4426950408889634f : 1.0f;
    float wreg[G::NS];
    int toff[G::NS];
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
        const int t0 = G::tap_off(4 * s), t1 = G::tap_off(4 * s + 1);
        const int t2 = G::tap_off(4 * s + 2), t3 = G::tap_off(4 * s + 3);
        toff[s] = q < 2 ? (q == 0 ? t0 : t1) : (q == 2 ? t2 : t3);
    }
    // accumulator rows 4q + r start at their channel's bias
    v4f bias4;
#pragma unroll
    for (int r = 0; r < 4; ++r) bias4[r] = bias ? bias[4 * q + r] * LSCALE : 0.0f;
    // B operand column m = l%16 is patch position (h = m/4, w = m%4)
    const int lbase = (c16 >> 2) * PP + (c16 & 3);
    // tie key of this lane's position (h, w) = (c16 / 4, c16 % 4); depth j adds
    // its own bits
    const int ph = c16 >> 2, pw = c16 & 3;
    const int kpos = TWO ? (((ph >> 1) << 4) | ((pw >> 1) << 3) | ((ph & 1) << 1) | (pw & 1))
                         : ((ph << 2) | pw);

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
    // Weights: every wave of the grid needs the whole (16 x K) tensor at once,
    // and per-lane 4-byte gathers from it (lane l wants w[l%16][4s + l/16])
    // pile ~20 requests per wave onto the same few L2 lines at kernel start.
    // Instead the wave reads it with contiguous float4 loads (16 * K is a
    // multiple of 4 and w is 16-byte aligned), parks it in the patch buffers
    // (not yet in use), and picks its A operands from LDS.
    {
        constexpr int WN = 16 * G::K;
        static_assert(WN % 4 == 0 && WN <= 2 * (G::FLOATS + 8), "weights fit the patch buffers");
        float *wl = &patch[0][0];
#pragma unroll
        for (int i = 4 * lane; i < WN; i += 256)
            *reinterpret_cast<v4f *>(wl + i) = *reinterpret_cast<const v4f *>(w + i);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < G::NS; ++s) {
            const int k = 4 * s + q;
            wreg[s] = k < G::K ? wl[c16 * G::K + k] * LSCALE : 0.0f;
        }
        __syncthreads();  // every lane has its weights before the patch overwrites them
    }
    CNF_STASH(0)
    // One window on patch buffer BUF (a compile-time constant, so every LDS
    // operand address is a per-lane base plus an immediate offset).
    auto window = [&](int win, auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
        int nn, od2, oh2, ow2;
        const bool more = win + stride < hi;
        window_base(win, n, od, oh, ow);
        if (more) CNF_FETCH(window_base(win + stride, nn, od2, oh2, ow2))
        __syncthreads();  // patch[BUF] is complete

        v4f acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = bias4;
        const float *pb = patch[BUF];
        // B operands one K step ahead: the reads of step s + 1 are issued before
        // the four MFMAs of step s (pinned by the scheduling groups), so a step
        // waits only for reads issued a step earlier.
        float bop[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bop[0][j] = pb[lbase + toff[0] + j * G::E * PP];
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);          // step 0's LDS reads
#pragma unroll
        for (int s = 0; s < G::NS; ++s) {
            if (s + 1 < G::NS) {
                const int a1 = lbase + toff[s + 1];
#pragma unroll
                for (int j = 0; j < 4; ++j) bop[(s + 1) & 1][j] = pb[a1 + j * G::E * PP];
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the step's LDS reads
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = mfma_16x16x4(wreg[s], bop[s & 1][j], acc[j]);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);      // then its MFMAs
        }

        // activation; the softmax at position (j, c16) runs over the lane's 4
        // channels and the same position in the other three lane rows
        float v[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (ACT == ACT_SOFTMAX) {
                float m = fmaxf(fmaxf(acc[j][0], acc[j][1]), fmaxf(acc[j][2], acc[j][3]));
                m = fmaxf(m, __shfl_xor(m, 16, 64));
                m = fmaxf(m, __shfl_xor(m, 32, 64));
                float e[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(acc[j][r] - m);
                float sum = (e[0] + e[1]) + (e[2] + e[3]);
                sum += __shfl_xor(sum, 16, 64);
                sum += __shfl_xor(sum, 32, 64);
                const float inv = __builtin_amdgcn_rcpf(sum);
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] = e[r] * inv;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] = activate<ACT>(acc[j][r]);
            }
        }
        // per channel row 4q + r: window max over depth (in-lane) and the 16
        // positions (lanes of the row), then the first voxel in tie order
        float best[4];
        int bkey[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float b = fmaxf(fmaxf(v[0][r], v[1][r]), fmaxf(v[2][r], v[3][r]));
            b = row_max16(b);
            // keys grow with depth j: the first depth holding the max wins in-lane
            int k = 1 << 30;
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                const int key = kpos | (TWO ? (((j >> 1) << 5) | ((j & 1) << 2)) : (j << 4));
                k = (v[j][r] == b) ? key : k;
            }
            k = row_min16_i(k);
            best[r] = b;
            bkey[r] = k;
        }
        // lanes c16 = 0..3 of row q store channel 4q + c16
        if (c16 < 4) {
            const float bv = c16 == 0 ? best[0] : c16 == 1 ? best[1] : c16 == 2 ? best[2] : best[3];
            const int bk = c16 == 0 ? bkey[0] : c16 == 1 ? bkey[1] : c16 == 2 ? bkey[2] : bkey[3];
            int a, b, c;
            key_abc(bk, TWO, a, b, c);
            const size_t o = (((size_t)n * 16 + 4 * q + c16) * Dp + od) * Hp * Wp +
                             (size_t)oh * Wp + ow;
            out[o] = bv;
            if (argmax)
                argmax[o] = ((4 * od + a) * Ho + (4 * oh + b)) * Wo + (4 * ow + c);
        }
        if (more) CNF_STASH(BUF ^ 1)  // BUF^1 was last read in the previous window
    };
    for (int win = first; win < hi;) {  // wave-uniform
        window(win, std::integral_constant<int, 0>{});
        win += stride;
        if (win >= hi) break;
        window(win, std::integral_constant<int, 1>{});
        win += stride;
    }
#undef CNF_FETCH
#undef CNF_STASH
}

template <int CI, int KS, int ACT, bool TWO>
hipError_t launch_t2(const Conv3dSoftmaxPoolArgs &a, hipStream_t st)
{
    const int total = a.N * a.Dp * a.Hp * a.Wp;
    // CU count per device, cached; concurrent first calls store the same value
    static std::atomic<int> cus_cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = dev >= 0 && dev < 64 ? cus_cache[dev].load(std::memory_order_relaxed) : 0;
    if (!cus) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) cus_cache[dev].store(cus, std::memory_order_relaxed);
    }
    const int grid = total < cus * WAVES_PER_CU ? total : cus * WAVES_PER_CU;
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
