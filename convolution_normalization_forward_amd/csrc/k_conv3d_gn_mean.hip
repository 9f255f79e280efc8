// k_conv3d_gn_mean.hip -- Conv3d (C_out = 16, k = 4) + activation +
// GroupNorm + mean over D,H,W, fused so that the conv output never leaves
// the compute unit.
//
// Page "Kimi-K2.6__l2_p27", first trace: the mean over D,H,W of a GroupNorm
// output needs only each channel's mean m_c and each group's mean and
// variance,   out[n,c] = gamma_c (m_c - mu_g) / sqrt(var_g + eps) + beta_c,
// so one pass that accumulates per-channel statistics is enough.  Here the
// per-channel statistics are Welford triples, merged with Chan's formula
// across lanes (DPP), waves (LDS) and finally into group statistics.
//
// Mapping (one workgroup of 4 waves per sample):
//   * The sample's input planes stream through an LDS ring of 5 depth planes
//     (all C_in channels of one depth each); output plane d reads ring slots
//     (d .. d+3) mod 5 while plane d+4 is prefetched into registers.
//   * Output plane d (Ho x Wo positions, flattened) is cut into tiles of 16
//     positions.  A tile is one 16x16 MFMA output: rows = the 16 output
//     channels, columns = the 16 positions, contraction K = C_in * 64 in
//     steps of 4 (v_mfma_f32_16x16x4f32).  The weights (A operand) sit in
//     registers for the whole kernel; the im2col operand (B) is read straight
//     from the LDS ring.  With k = 4 the tap kw equals the lane's K-quarter,
//     and the LDS row/plane pitches are compile-time, so every LDS read is the
//     lane's base address plus an immediate.
//   * Lane l of a tile result holds channels 4*(l/16)+r, r = 0..3, at
//     position l%16; bias and activation are applied in registers and the
//     value is pushed into that lane's per-channel Welford triple.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int KS = 4;        // kernel extent (cubic)
constexpr int NSLOT = 5;     // LDS ring of depth planes
constexpr int THREADS = 256;
constexpr int NB = 4;        // tiles in flight per wave
constexpr int WP = 32;       // LDS row pitch (== W)
constexpr int HWP = 32 * 32; // LDS channel pitch inside a slot (>= H * W)

template <int CI, int NBV>
__device__ __forceinline__ void tile_mfma(const float *__restrict__ lds, const int (&slot)[KS],
                                          const int (&base)[NB], const float *wreg,
                                          v4f (&acc)[NB])
{
#pragma unroll
    for (int kd = 0; kd < KS; ++kd) {
        int vb[NBV];
#pragma unroll
        for (int j = 0; j < NBV; ++j) vb[j] = slot[kd] + base[j];
#pragma unroll
        for (int ci = 0; ci < CI; ++ci) {
#pragma unroll
            for (int kh = 0; kh < KS; ++kh) {
                const int s = (ci * KS + kd) * KS + kh;
                const int imm = ci * HWP + kh * WP;
#pragma unroll
                for (int j = 0; j < NBV; ++j)
                    acc[j] = mfma_16x16x4(wreg[s], lds[vb[j] + imm], acc[j]);
            }
        }
    }
}

template <int CI, int ACT>
__global__ __launch_bounds__(THREADS, 2)
void conv3d_k4_gn_mean_kernel(const float *__restrict__ x, const float *__restrict__ w,
                              const float *__restrict__ bias, const float *__restrict__ gamma,
                              const float *__restrict__ beta, float *__restrict__ out,
                              int D, int H, int num_groups, float eps, float inv_div)
{
    constexpr int K = CI * KS * KS * KS;
    constexpr int NS = K / 4;  // MFMA steps
    constexpr int PL = CI * HWP;  // floats per ring slot
    constexpr int W = WP;
    extern __shared__ float lds[];

    const int Do = D - KS + 1, Ho = H - KS + 1, Wo = W - KS + 1;
    const int P = Ho * Wo;
    const int T = (P + 15) >> 4;
    const int HW = H * W;
    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c16 = lane & 15;

    // A operand: w[co = l%16][k = 4s + l/16] (natural PyTorch weight order).
    float wreg[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) wreg[s] = w[c16 * K + 4 * s + q];
    float bch[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bch[r] = bias ? bias[4 * q + r] : 0.0f;

    const float *xs = x + (size_t)n * CI * D * HW;

    // Depth plane p of every channel -> ring slot p % NSLOT.  A channel's
    // plane is H*W <= 1024 floats, i.e. at most one float4 per thread.
    const int hw4 = HW >> 2;
    const bool ld = tid < hw4;
    const int e4 = ld ? tid : 0;

    for (int p = 0; p < KS; ++p) {
#pragma unroll
        for (int ci = 0; ci < CI; ++ci) {
            const float4 v = reinterpret_cast<const float4 *>(xs + ((size_t)ci * D + p) * HW)[e4];
            if (ld) reinterpret_cast<float4 *>(lds + (p % NSLOT) * PL + ci * HWP)[e4] = v;
        }
    }

    float cnt = 0.0f;
    float mean[4] = {0.f, 0.f, 0.f, 0.f}, m2[4] = {0.f, 0.f, 0.f, 0.f};

    for (int d = 0; d < Do; ++d) {
        __syncthreads();  // planes d .. d+3 are in the ring
        // prefetch plane d+4 (clamped to the last plane; stored only if it exists)
        const int pn = min(d + KS, D - 1);
        float4 pf[CI];
#pragma unroll
        for (int ci = 0; ci < CI; ++ci)
            pf[ci] = reinterpret_cast<const float4 *>(xs + ((size_t)ci * D + pn) * HW)[e4];

        int slot[KS];
#pragma unroll
        for (int kd = 0; kd < KS; ++kd) slot[kd] = ((d + kd) % NSLOT) * PL;

        // The plane's T tiles go to the four waves by residue mod 4; which wave
        // takes the residue with the extra tile rotates with the plane and the
        // sample, so no SIMD carries it every plane (two workgroups share a CU).
        const int wr = (wave + d + n) & 3;
        for (int t0 = wr; t0 < T; t0 += 4 * NB) {
            v4f acc[NB];
            int base[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int t = t0 + 4 * j;
                int pos = t * 16 + c16;
                pos = pos < P ? pos : P - 1;
                const int h = pos / Wo, wv = pos - h * Wo;
                base[j] = h * WP + wv + q;  // kw == q
                acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
            const int nv = (T - t0 + 3) >> 2;  // valid tiles in this batch (wave-uniform)
            if (nv >= 4) tile_mfma<CI, 4>(lds, slot, base, wreg, acc);
            else if (nv == 3) tile_mfma<CI, 3>(lds, slot, base, wreg, acc);
            else if (nv == 2) tile_mfma<CI, 2>(lds, slot, base, wreg, acc);
            else tile_mfma<CI, 1>(lds, slot, base, wreg, acc);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int t = t0 + 4 * j;
                if (t < T && t * 16 + c16 < P) {
                    cnt += 1.0f;
                    const float rn = __builtin_amdgcn_rcpf(cnt);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = activate<ACT>(acc[j][r] + bch[r]);
                        welford_push(mean[r], m2[r], v, rn);
                    }
                }
            }
        }

        // slot (d+4)%5 == (d-1)%5 held plane d-1, which no wave reads after
        // the barrier that opened this iteration.
        if (d + KS < D && ld) {
#pragma unroll
            for (int ci = 0; ci < CI; ++ci)
                reinterpret_cast<float4 *>(lds + ((d + KS) % NSLOT) * PL + ci * HWP)[e4] = pf[ci];
        }
    }

    // ---- statistics: the 16 lanes of a row share channels 4q..4q+3
    float *red = lds + NSLOT * PL;  // [4 waves][16 ch][3]
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
    float *chs = red + 4 * 16 * 3;  // [16 ch][3] merged over waves
    if (tid < 16) {
        float nn = 0.f, mm = 0.f, qq = 0.f;
        for (int wv = 0; wv < 4; ++wv) {
            const float *e = red + (wv * 16 + tid) * 3;
            chan_merge(nn, mm, qq, e[0], e[1], e[2]);
        }
        chs[tid * 3 + 0] = nn; chs[tid * 3 + 1] = mm; chs[tid * 3 + 2] = qq;
    }
    __syncthreads();
    if (tid < 16 && num_groups <= 0) {
        // no norm: the plain spatial mean of the activation
        out[(size_t)n * 16 + tid] = chs[tid * 3 + 1] * inv_div;
    } else if (tid < 16) {
        // group statistics from equal-count channel triples, then the closed form
        const int c = tid;
        const int cg = 16 / num_groups;
        const int g0 = (c / cg) * cg;
        float mu = 0.f;
        for (int j = 0; j < cg; ++j) mu += chs[(g0 + j) * 3 + 1];
        mu = mu / (float)cg;
        float var = 0.f;
        for (int j = 0; j < cg; ++j) {
            const float mj = chs[(g0 + j) * 3 + 1];
            var += chs[(g0 + j) * 3 + 2] / chs[(g0 + j) * 3 + 0] + (mj - mu) * (mj - mu);
        }
        var = var / (float)cg;
        const float ga = gamma ? gamma[c] : 1.0f, be = beta ? beta[c] : 0.0f;
        const float mc = chs[c * 3 + 1];
        out[(size_t)n * 16 + c] = (ga * (mc - mu) * rsqrtf(var + eps) + be) * inv_div;
    }
}

template <int CI, int ACT>
hipError_t launch_t(const Conv3dGnMeanArgs &a, hipStream_t st)
{
    const size_t lds = conv3d_gn_mean_lds_bytes(CI);
    hipLaunchKernelGGL((conv3d_k4_gn_mean_kernel<CI, ACT>), dim3(a.N), dim3(THREADS), lds, st,
                       a.x, a.w, a.b, a.gamma, a.beta, a.out, a.D, a.H, a.num_groups,
                       a.eps, a.inv_div);
    return hipGetLastError();
}

}  // namespace

size_t conv3d_gn_mean_lds_bytes(int C_in)
{
    return (size_t)(NSLOT * C_in * HWP + 4 * 16 * 3 + 16 * 3) * sizeof(float);
}

// Shapes this kernel family covers: C_out 16, k 4, W == 32, 4 <= H <= 32,
// D >= 4, C_in in {1, 3}.
bool conv3d_gn_mean_supported(int C_in, int C_out, int kernel, int D, int H, int W, int act)
{
    if (C_out != 16 || kernel != KS) return false;
    if (C_in != 3 && C_in != 1) return false;
    if (W != WP || H < KS || H > HWP / WP || D < KS) return false;
    return act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF || act == ACT_GELU_TANH;
}

hipError_t launch_conv3d_gn_mean(const Conv3dGnMeanArgs &a, hipStream_t st)
{
#define CNF_CASE(CI, ACT) \
    if (a.C_in == CI && a.act == ACT) return launch_t<CI, ACT>(a, st);
    CNF_CASE(3, ACT_HARDSWISH)
    CNF_CASE(3, ACT_NONE)
    CNF_CASE(3, ACT_GELU_ERF)
    CNF_CASE(3, ACT_GELU_TANH)
    CNF_CASE(1, ACT_HARDSWISH)
    CNF_CASE(1, ACT_NONE)
    CNF_CASE(1, ACT_GELU_ERF)
    CNF_CASE(1, ACT_GELU_TANH)
#undef CNF_CASE
    return hipErrorInvalidValue;
}

}  // namespace cnf
