// k_conv2d_igemm.hip -- Conv2d (C_out = 128 or 64, k = 3, C_in a multiple of
// 4, optional zero padding) as an implicit GEMM on fp32 MFMA, with bias,
// activation and per-tile Welford partials in the epilogue, followed by a
// statistics finalize (scale and shift per channel) and an in-place
// InstanceNorm / GroupNorm + divide pass.  A dense (groups = 1)
// stride-1 ConvTranspose2d is the same GEMM on the input padded by k - 1 with
// the kernel flipped and its channel axes swapped (page "Kimi-K2.6__l2_p19",
// second trace: out[i, j] = sum x[i - kh, j - kw] W[ci, co, kh, kw]), so it
// runs here too: only the weight copy and the padding differ.
//
// Page "Kimi-K2.6__l2_p17": Conv2d(64 -> 128, k = 3) -> InstanceNorm2d ->
// divide by 2 on 128 x 64 x 128 x 128.  The second trace shows the conv is
// compute-bound (arithmetic intensity ~190 FLOP/byte) and that a workgroup
// per (sample, output channel) re-reads the input 128 times, so a tile must
// cover every output channel.  Statistics need a whole 126 x 126 plane, which
// no single tile sees; tiles publish Welford partials and a second pass merges
// them and normalises in place.
//
// Mapping:
//   * GEMM rows = the 128 output channels (A = weights), columns = output
//     positions (B = im2col of x), K = C_in * 9 ordered (tap, channel).
//   * A workgroup (8 waves) owns all CO channels x a TR-row x 32-column block
//     of output positions of one sample (TR = 8 for 128 channels, 16 for 64);
//     wave (wm, wn) computes channels 64*wm .. +63 on output rows 2*wn and
//     2*wn + 1 as 2 x 2 tiles of v_mfma_f32_32x32x2f32 (channel half x row).
//     32-column tiles keep the padding of the last column tile small for
//     widths just past a multiple of 64 (258 = 4 * 64 + 2 wasted a quarter of
//     the MFMA work with 64-column tiles).  At stride 1, widths 1 or 2 past a
//     multiple of 32 (258 again) leave those last columns to column-strip
//     tiles, whose 32 MFMA columns are 16 rows x 2 columns (32 NR rows per
//     tile), instead of tiles with 1 or 2 live columns in 32; heights 1 or 2
//     past a multiple of TR leave those last rows to row-strip tiles of 2 rows
//     x 32 NR columns, instead of tiles in which one wave has live rows.  On a
//     258 x 258 output this drops the tiles from 153 to 131 per sample and the
//     MFMA work from 1.18x to 1.00x the live positions.
//   * Stride s = 1 or 2: output position (r, c) reads input rows s r + kh and
//     columns s c + kw of the (padded) input, so a tile's halo is
//     (TR - 1) s + 3 rows of 31 s + 3 columns.
//   * K is walked in chunks of CC input channels (4 at stride 1, 2 at stride 2,
//     so two workgroups still fit a CU's LDS): the chunk's input halo
//     (CC x halo rows x halo columns) and its weights (9*CC x CO, from a [ci][tap][co] copy the
//     first kernel makes) are double-buffered in LDS; the next chunk is
//     fetched into registers while the current one is multiplied.
//   * Epilogue: bias, coalesced fp32 stores of y (32 consecutive positions per
//     register), and per-channel (count, mean, M2) of each 16-lane row taken in
//     two passes over the registers (DPP row sums, no division per lane); one
//     Chan merge per channel over the rows (LDS) leaves one partial per
//     (sample, tile, channel).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int TC = 32;                   // output tile columns
constexpr int THREADS = 512;
constexpr int NWAVES = THREADS / 64;
constexpr int MAX_CC = 4;                // input channels per K chunk at stride 1

// Padding that makes a block of `base` floats end `m` floats past a multiple
// of 64 (the next block then starts m floats into a 64-bank row).
constexpr int pad_to(int base, int m) { return base + ((m - base % 64) + 64) % 64; }

// Tile geometry for CO output channels (128 or 64) and stride SD: 64 channels x
// 64 columns (two rows of 32) per wave, so NR = 8 waves / (CO / 64) waves along
// the rows and TR = 2 * NR output rows per tile.  At stride 1 the halo row
// pitch is 36 and a channel's block starts 32 floats past a multiple of 64, so
// the two K rows of an operand (lane halves) read disjoint banks; at stride 2 a
// lane half reads every other float of a row, so the channel block starts an
// odd number of floats in and the two halves take the even and the odd banks.
template <int CO_, int SD_>
struct Geo {
    static constexpr int CO = CO_, SD = SD_;
    static constexpr int CC = SD == 1 ? MAX_CC : 2;
    static constexpr int KC = 9 * CC;
    static constexpr int WM = CO / 64, NR = NWAVES / WM, TR = 2 * NR;
    static constexpr int HR = (TR - 1) * SD + 3, HC = (TC - 1) * SD + 3;  // halo rows, columns
    static constexpr int PITCH = SD == 1 ? 36 : 68;
    static constexpr int BJ = SD * PITCH;  // LDS offset from a wave's first output row to its second
    static constexpr int CS = pad_to(HR * PITCH, SD == 1 ? 32 : 33);
    static constexpr int WPITCH = CO + 32;                                // == 32 mod 64
    static constexpr int XS_FLOATS = (CC * CS + 3) / 4 * 4;             // float4-aligned weights after it
    static constexpr int WS_FLOATS = KC * WPITCH;
    static constexpr int BUF_FLOATS = XS_FLOATS + WS_FLOATS;
    static constexpr int XIN = CC * HR * HC;                       // halo floats per chunk
    static constexpr int XPF = (XIN + THREADS - 1) / THREADS;      // per-thread prefetch (scalar)
    static constexpr int WPF = (KC * CO / 4 + THREADS - 1) / THREADS;  // (float4)
    static_assert(WPITCH % 64 == 32, "bank spread");
    static_assert(HC <= PITCH, "halo row fits its pitch");
    static_assert(NR * WM == NWAVES, "one 64-channel x 64-position block per wave");
    static_assert(2 * BUF_FLOATS * 4 <= 80 * 1024, "two workgroups per CU");
};

// Column strip (stride 1): when Wo mod 32 is 1 or 2, a tile of 32 columns would
// hold 1 or 2 live ones, so those last columns get tiles of their own in which
// a wave's two 32-column MFMA blocks are 16 rows x 2 columns each (lane i of a
// half: row i / 2, column i % 2).  A wave covers 32 rows and a tile TR = 32 NR
// rows; its halo is TR + 2 rows of 4 columns (pitch 4).  A lane half reads
// columns {0, 1} + kw of every fourth float, so a channel block starts 2 floats
// past a multiple of 64 and the two halves take the banks 4 j + {0, 1} and
// 4 j + {2, 3}.  Two input channels per K chunk keep the halo and the weights
// inside the main tile's staging buffers (the same LDS layout).
template <int CO_>
struct GeoStrip {
    static constexpr int CO = CO_, SD = 1;
    static constexpr int CC = 2, KC = 9 * CC;
    static constexpr int WM = CO / 64, NR = NWAVES / WM, TR = 32 * NR;
    static constexpr int HR = TR + 2, HC = 4, PITCH = 4;
    static constexpr int BJ = 16 * PITCH;
    static constexpr int CS = pad_to(HR * PITCH, 2);
    static constexpr int WPITCH = Geo<CO, 1>::WPITCH;
    static constexpr int XS_FLOATS = Geo<CO, 1>::XS_FLOATS, BUF_FLOATS = Geo<CO, 1>::BUF_FLOATS;
    static constexpr int XIN = CC * HR * HC;
    static constexpr int XPF = (XIN + THREADS - 1) / THREADS;
    static constexpr int WPF = (KC * CO / 4 + THREADS - 1) / THREADS;
    static_assert(CC * CS <= XS_FLOATS, "strip halo fits the main tile's halo buffer");
    static_assert(KC * WPITCH <= Geo<CO, 1>::WS_FLOATS, "strip weights fit the main tile's buffer");
};

// Row strip (stride 1): when Ho mod TR is 1 or 2, those last rows get tiles of
// 2 rows x 32 NR columns (wave wn: both rows, columns 32 wn .. + 31) instead of
// tiles in which one wave in NR has live rows.  Halo: 4 rows of 32 NR + 2
// columns; two input channels per K chunk, as in the column strip.
template <int CO_>
struct GeoRow {
    static constexpr int CO = CO_, SD = 1;
    static constexpr int CC = 2, KC = 9 * CC;
    static constexpr int WM = CO / 64, NR = NWAVES / WM, TW = 32 * NR;  // tile columns
    static constexpr int HR = 4, HC = TW + 2, PITCH = HC, BJ = PITCH;
    static constexpr int CS = pad_to(HR * PITCH, 32);
    static constexpr int WPITCH = Geo<CO, 1>::WPITCH;
    static constexpr int XS_FLOATS = Geo<CO, 1>::XS_FLOATS, BUF_FLOATS = Geo<CO, 1>::BUF_FLOATS;
    static constexpr int XIN = CC * HR * HC;
    static constexpr int XPF = (XIN + THREADS - 1) / THREADS;
    static constexpr int WPF = (KC * CO / 4 + THREADS - 1) / THREADS;
    static_assert(CC * CS <= XS_FLOATS, "row-strip halo fits the main tile's halo buffer");
    static_assert(KC * WPITCH <= Geo<CO, 1>::WS_FLOATS, "row-strip weights fit the main tile's buffer");
};

// Conv: w[co][ci][kh][kw] -> wt[ci][tap][co].  Transposed conv (weights
// [ci][co][kh][kw]): the flipped tap, wt[ci][tap][co] = w[ci][co][8 - tap].
__global__ void conv2d_weight_transpose_kernel(const float *__restrict__ w, float *__restrict__ wt,
                                               int C_in, int CO, int transposed)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int total = CO * C_in * 9;
    if (i >= total) return;
    const int co = i % CO, rest = i / CO;  // rest = ci * 9 + tap
    const int ci = rest / 9, tap = rest % 9;
    wt[i] = transposed ? w[((size_t)ci * CO + co) * 9 + (8 - tap)] : w[(size_t)co * C_in * 9 + rest];
}

// Per-thread staging slots of geometry G for the tile at (row0, col0): halo
// element e = tid + u*THREADS (clamped so every load is in bounds; out-of-image
// or surplus slots carry 0), and float4 e of the chunk's [ci][tap][co] weight rows.
template <class G>
__device__ __forceinline__ void igemm_tables(int tid, int row0, int col0, int H, int W, int pad,
                                             int (&xoff)[G::XPF], bool (&xok)[G::XPF],
                                             int (&xdst)[G::XPF], int (&wdst)[G::WPF])
{
#pragma unroll
    for (int u = 0; u < G::XPF; ++u) {
        const int e = tid + u * THREADS;
        const int ec = e < G::XIN ? e : G::XIN - 1;
        const int cc = ec % G::HC, rest = ec / G::HC;
        const int rr = rest % G::HR, c = rest / G::HR;
        // input row / column of the (zero-padded by pad) halo element
        const int gr = G::SD * row0 + rr - pad, gc = G::SD * col0 + cc - pad;
        xok[u] = e < G::XIN && gr >= 0 && gr < H && gc >= 0 && gc < W;
        xoff[u] = xok[u] ? (c * H + gr) * W + gc : 0;
        xdst[u] = e < G::XIN ? c * G::CS + rr * G::PITCH + cc : -1;
    }
#pragma unroll
    for (int u = 0; u < G::WPF; ++u) {
        const int e = tid + u * THREADS;
        const int co4 = e % (G::CO / 4), r = e / (G::CO / 4);  // r = c * 9 + tap
        const int c = r / 9, tap = r % 9;
        wdst[u] = e < G::KC * G::CO / 4 ? (tap * G::CC + c) * G::WPITCH + co4 * 4 : -1;
    }
}

template <class G>
__device__ __forceinline__ void igemm_fetch(const float *__restrict__ xn, const float *__restrict__ wt,
                                            int chunk, int H, int W, int tid,
                                            const int (&xoff)[G::XPF], const bool (&xok)[G::XPF],
                                            float (&xpf)[G::XPF], v4f (&wpf)[G::WPF])
{
    const float *xc = xn + (size_t)chunk * G::CC * H * W;
#pragma unroll
    for (int u = 0; u < G::XPF; ++u) {
        const float v = xc[xoff[u]];
        xpf[u] = xok[u] ? v : 0.0f;
    }
    const v4f *src = reinterpret_cast<const v4f *>(wt + (size_t)chunk * G::CC * 9 * G::CO);
#pragma unroll
    for (int u = 0; u < G::WPF; ++u) {
        const int e = tid + u * THREADS;
        wpf[u] = src[e < G::KC * G::CO / 4 ? e : 0];
    }
}

template <class G>
__device__ __forceinline__ void igemm_stash(float *lds, int buf, const int (&xdst)[G::XPF],
                                            const int (&wdst)[G::WPF], const float (&xpf)[G::XPF],
                                            const v4f (&wpf)[G::WPF])
{
    float *xs = lds + buf * G::BUF_FLOATS;
    float *ws = xs + G::XS_FLOATS;
#pragma unroll
    for (int u = 0; u < G::XPF; ++u)
        if (xdst[u] >= 0) xs[xdst[u]] = xpf[u];
#pragma unroll
    for (int u = 0; u < G::WPF; ++u)
        if (wdst[u] >= 0) *reinterpret_cast<v4f *>(ws + wdst[u]) = wpf[u];
}

// The K loop of one tile of geometry G: chunks of CC input channels staged in
// double-buffered LDS, the next chunk fetched into registers while the current
// one is multiplied.  xlane: LDS offset of this lane's first B operand in a
// channel block; active: false for a wave whose output rows all lie past the
// output (it still stages, but skips the MFMAs).
template <class G>
__device__ __forceinline__ void igemm_loop(const float *__restrict__ xn, const float *__restrict__ wt,
                                           float *lds, int C_in, int H, int W, int pad, int row0,
                                           int col0, int tid, int xlane, bool active, v16f (&acc)[2][2])
{
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::NR, h = lane >> 5, i32 = lane & 31;
    int xoff[G::XPF], xdst[G::XPF], wdst[G::WPF];
    bool xok[G::XPF];
    igemm_tables<G>(tid, row0, col0, H, W, pad, xoff, xok, xdst, wdst);
    float xpf[G::XPF];
    v4f wpf[G::WPF];

    const int nchunks = C_in / G::CC;
    igemm_fetch<G>(xn, wt, 0, H, W, tid, xoff, xok, xpf, wpf);
    igemm_stash<G>(lds, 0, xdst, wdst, xpf, wpf);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        if (ch + 1 < nchunks) igemm_fetch<G>(xn, wt, ch + 1, H, W, tid, xoff, xok, xpf, wpf);
        const float *xs = lds + buf * G::BUF_FLOATS;
        const float *ws = xs + G::XS_FLOATS;
        const float *wa = ws + h * G::WPITCH + 64 * wm + i32;
        const float *xb = xs + h * G::CS + xlane;
        if (active) {
#pragma unroll
            for (int tap = 0; tap < 9; ++tap) {
                const int kh = tap / 3, kw = tap % 3;
#pragma unroll
                for (int p = 0; p < G::CC / 2; ++p) {
                    const int s = tap * (G::CC / 2) + p;
                    const float a0 = wa[2 * s * G::WPITCH];
                    const float a1 = wa[2 * s * G::WPITCH + 32];
                    const float b0 = xb[2 * p * G::CS + kh * G::PITCH + kw];
                    const float b1 = xb[2 * p * G::CS + G::BJ + kh * G::PITCH + kw];
                    acc[0][0] = mfma_32x32x2(a0, b0, acc[0][0]);
                    acc[0][1] = mfma_32x32x2(a0, b1, acc[0][1]);
                    acc[1][0] = mfma_32x32x2(a1, b0, acc[1][0]);
                    acc[1][1] = mfma_32x32x2(a1, b1, acc[1][1]);
                }
            }
        }
        if (ch + 1 < nchunks)  // buf^1 was last read in iteration ch-1
            igemm_stash<G>(lds, buf ^ 1, xdst, wdst, xpf, wpf);
        __syncthreads();
    }
}

// EDGE (stride 1 only): a sample's tiles are tiles_w x tiles_h row-major
// 32-column tiles, then `row_strips` row-strip tiles of the last Ho - TR tiles_h
// rows (0 unless that is 1 or 2), then column-strip tiles of the last Wo - 32
// tiles_w columns (none unless that is 1 or 2), which cover every row; and a
// wave whose output rows all lie past the bottom edge skips its MFMAs.  Without
// EDGE every tile is a 32-column tile.
template <int CO, int ACT, int SD, bool EDGE>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4, 4)))
void conv2d_igemm_kernel(const float *__restrict__ x, const float *__restrict__ wt,
                         const float *__restrict__ bias, float *__restrict__ y,
                         float *__restrict__ partials, int C_in, int H, int W, int Ho, int Wo,
                         int pad, int tiles_w, int tiles_h, int row_strips, int tiles_per_sample)
{
    static_assert(!EDGE || SD == 1, "edge strips at stride 1");
    using G = Geo<CO, SD>;
    using GS = GeoStrip<CO>;
    using GR = GeoRow<CO>;
    constexpr int TR = G::TR, NR = G::NR, BUF_FLOATS = G::BUF_FLOATS;
    __shared__ float lds[2 * BUF_FLOATS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NR, wn = wave % NR;
    const int h = lane >> 5, i32 = lane & 31;
    // XCD-aware tile order: each XCD takes a contiguous run of (n, tile), so
    // vertically adjacent tiles share their halo rows in L2.
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int T = xcd_remap(L, gridDim.x * gridDim.y * gridDim.z);
    const int n = T / tiles_per_sample, t = T - n * tiles_per_sample;
    const int tiles_main = tiles_w * tiles_h;
    const float *xn = x + (size_t)n * C_in * H * W;

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    // Register r of acc[bi][bj] holds channel co(bi, r) (fixed per 32-lane half
    // h) at output row prow[bj], column pcol.  Statistics are taken per 16-lane
    // row s16 = (lane / 16) % 2 over both bj: mean and then summed squared
    // deviations (two passes over the registers), giving 2 * NR (count, mean,
    // M2) partials per channel that one Chan merge per channel folds into the
    // tile's partial; cnt = the live positions of the lane's 16-lane row.
    const int s16 = (lane >> 4) & 1;
    int prow[2], pcol, cnt;
    if (EDGE && t >= tiles_main + row_strips) {  // block-uniform
        const int row0 = (t - tiles_main - row_strips) * GS::TR, col0 = tiles_w * TC;
        const int rw = row0 + 32 * wn;  // the wave's first row
        igemm_loop<GS>(xn, wt, lds, C_in, H, W, pad, row0, col0, tid,
                       ((i32 >> 1) + 32 * wn) * GS::PITCH + (i32 & 1), rw < Ho, acc);
        const int sw = min(Wo - col0, 2);
        cnt = 0;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            prow[bj] = rw + 16 * bj + (i32 >> 1);
            cnt += min(max(Ho - (rw + 16 * bj + 8 * s16), 0), 8) * sw;
        }
        pcol = col0 + (i32 & 1);
    } else if (EDGE && t >= tiles_main) {
        // rows TR tiles_h .. Ho - 1; columns of the 32-column tiles only
        const int row0 = tiles_h * TR, col0 = (t - tiles_main) * GR::TW;
        const int cw = col0 + 32 * wn;  // the wave's first column
        const int cend = min(tiles_w * TC, Wo);
        igemm_loop<GR>(xn, wt, lds, C_in, H, W, pad, row0, col0, tid, 32 * wn + i32, cw < cend, acc);
        const int live = min(max(cend - (cw + 16 * s16), 0), 16);
        cnt = 0;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            prow[bj] = row0 + bj < Ho ? row0 + bj : Ho;  // Ho: not live
            cnt += row0 + bj < Ho ? live : 0;
        }
        pcol = cw + i32 < cend ? cw + i32 : Wo;  // Wo: not live
    } else {
        const int th = t / tiles_w, tw = t - th * tiles_w;
        const int row0 = th * TR, col0 = tw * TC;
        igemm_loop<G>(xn, wt, lds, C_in, H, W, pad, row0, col0, tid,
                      2 * SD * wn * G::PITCH + SD * i32, !EDGE || row0 + 2 * wn < Ho, acc);
        int rem[2];  // live columns of each of the wave's two rows
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            prow[bj] = row0 + 2 * wn + bj;
            rem[bj] = prow[bj] < Ho ? Wo - col0 : 0;
        }
        cnt = min(max(rem[0] - 16 * s16, 0), 16) + min(max(rem[1] - 16 * s16, 0), 16);
        pcol = col0 + i32;
    }

    // ---- epilogue: bias, activation, stores, statistics
    const float rcnt = cnt ? 1.0f / (float)cnt : 0.0f;
    const unsigned plane = (unsigned)Ho * Wo;
    const auto yr = make_rsrc(y + (size_t)n * CO * plane, CO * plane * 4u);
    bool ok[2];
    unsigned off[2];
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
        ok[bj] = prow[bj] < Ho && pcol < Wo;
        off[bj] = ((unsigned)(64 * wm + 4 * h) * plane + (unsigned)prow[bj] * Wo + pcol) * 4u;
    }
    float (*red)[2][CO][3] = reinterpret_cast<float (*)[2][CO][3]>(lds);
    static_assert(NR * 2 * CO * 3 <= 2 * BUF_FLOATS, "row partials fit the staging buffers");
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dc = 32 * bi + 8 * (r >> 2) + (r & 3);  // co - 64 * wm - 4 * h
            const int co = 64 * wm + 4 * h + dc;
            const float bc = bias ? bias[co] : 0.0f;
            float v[2];
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                v[bj] = activate<ACT>(acc[bi][bj][r] + bc);
                buf_store1(v[bj], yr, ok[bj] ? off[bj] + (unsigned)dc * plane * 4u : GOOB);
            }
            const float mean = row_sum16((ok[0] ? v[0] : 0.0f) + (ok[1] ? v[1] : 0.0f)) * rcnt;
            const float d0 = v[0] - mean, d1 = v[1] - mean;
            const float m2 = row_sum16((ok[0] ? d0 * d0 : 0.0f) + (ok[1] ? d1 * d1 : 0.0f));
            if ((lane & 15) == 0) {
                red[wn][s16][co][0] = (float)cnt;
                red[wn][s16][co][1] = mean;
                red[wn][s16][co][2] = m2;
            }
        }
    }
    __syncthreads();
    if (tid < CO) {
        float tc = 0.f, tm = 0.f, tq = 0.f;
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                chan_merge(tc, tm, tq, red[k][q][tid][0], red[k][q][tid][1], red[k][q][tid][2]);
        float *pp = partials + (((size_t)n * tiles_per_sample + t) * CO + tid) * 3;
        pp[0] = tc; pp[1] = tm; pp[2] = tq;
    }
}

// ---- 16-bit inputs (bf16 or fp16 x and w, fp32 accumulation): the same GEMM
// on v_mfma_f32_32x32x16_{bf16,f16}.  Lane l of that MFMA supplies A[l % 32][8
// (l / 32) .. + 7] and B[8 (l / 32) .. + 7][l % 32] (eight 16-bit values, one
// 16-byte register quad), so a K step is one tap x 16 input channels and a
// lane's eight K values are eight channels of one input pixel.  The chunk's
// input halo is therefore kept channel-innermost in LDS: pixel (row, col)
// holds its 16 channels in 32 contiguous bytes, and every B operand is one
// 16-byte LDS read (the 64 lanes of a wave read 1 KB of consecutive bytes).
// x arrives row-major per channel, so the staging threads load 8 columns of 8
// channels (eight 16-byte loads) and transpose the 8 x 8 block in registers
// with byte permutes before the 16-byte LDS writes.  Weights are copied once
// per launch into [chunk][tap][co][16 ci] order, which is exactly the LDS
// layout of the A operand.
//   * A wave owns 64 channels x 4 rows x 32 columns (2 x 4 blocks of 32 x 32);
//     the workgroup (8 waves) all CO channels x 4 NR rows x 32 columns.
//   * Zero padding is not applied here (the planner sends only unpadded
//     stride-1 convs with W % 8 == 0, so a row's 8-column groups are whole and
//     16-byte aligned); halo pixels past the input read as zeros.
//   * Epilogue and statistics as in the fp32 kernel (4 rows per wave).
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

constexpr int CC16 = 16;                 // input channels per K chunk (one K step per tap)
constexpr int HCOL16 = TC + 2;           // halo columns

template <int CO>
struct Geo16 {
    static constexpr int WM = CO / 64, NR = NWAVES / WM, TR = 4 * NR;  // 4 rows per wave
    static constexpr int HR = TR + 2;
    static constexpr int XBYTES = HR * HCOL16 * CC16 * 2;     // halo, channel-innermost
    static constexpr int WBYTES = 9 * CO * CC16 * 2;          // [tap][co][16 ci]
    static constexpr int BUF = XBYTES + WBYTES;
    static constexpr int NFULL = HR * 2 * (TC / 8);           // 8 ch x 8 col units
    static constexpr int NLEFT = HR * 2;                      // 8 ch x the last 2 columns
    static constexpr int WV = WBYTES / 16;                    // 16-byte weight vectors
    static constexpr int WPF = (WV + THREADS - 1) / THREADS;
    static_assert(NFULL + NLEFT <= THREADS, "one staging unit per thread");
    static_assert(2 * BUF <= 160 * 1024, "double buffer fits the LDS");
    static_assert(NR * 2 * CO * 3 * 4 <= 2 * BUF, "row partials fit the staging buffers");
};

// w[co][ci][3][3] (16-bit) -> [ci / 16][tap][co][ci % 16]
__global__ void conv2d_weight_pack16_kernel(const unsigned short *__restrict__ w,
                                            unsigned short *__restrict__ wt, int C_in, int CO)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= CO * C_in * 9) return;
    const int cl = i % CC16, co = (i / CC16) % CO, tap = (i / (CC16 * CO)) % 9,
              chunk = i / (CC16 * CO * 9);
    wt[i] = w[((size_t)co * C_in + chunk * CC16 + cl) * 9 + tap];
}

__device__ __forceinline__ unsigned lo_pair(unsigned a, unsigned b)  // (a.lo16, b.lo16)
{
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ unsigned hi_pair(unsigned a, unsigned b)  // (a.hi16, b.hi16)
{
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int DT>
__device__ __forceinline__ v16f mfma16(const u4v &a, const u4v &b, const v16f &c)
{
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, a),
                                                       __builtin_bit_cast(bf8v, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a),
                                                      __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}

template <int CO, int ACT, int DT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void conv2d_igemm16_kernel(const unsigned short *__restrict__ x, const unsigned short *__restrict__ wt,
                           const float *__restrict__ bias, float *__restrict__ y,
                           float *__restrict__ partials, int C_in, int H, int W, int Ho, int Wo,
                           int tiles_w, int tiles_per_sample)
{
    using G = Geo16<CO>;
    constexpr int TR = G::TR, NR = G::NR, XBYTES = G::XBYTES, BUF = G::BUF, WPF = G::WPF;
    __shared__ u4v lds4[2 * BUF / 16];
    __shared__ float sbias[CO];
    unsigned char *const lds = reinterpret_cast<unsigned char *>(lds4);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NR, wn = wave % NR;
    const int h = lane >> 5, j = lane & 31;
    const int tiles_h = gridDim.y;
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + tiles_h * blockIdx.z);
    const int T = xcd_remap(L, gridDim.x * tiles_h * gridDim.z);
    const int tw = T % tiles_w, th = (T / tiles_w) % tiles_h, n = T / (tiles_w * tiles_h);
    const int row0 = th * TR, col0 = tw * TC;
    const auto xr = make_rsrc(x + (size_t)n * C_in * H * W, (unsigned)((size_t)C_in * H * W * 2));

    // staging unit of this thread: full (8 channels x 8 columns of one halo row)
    // or left-over (8 channels x the halo's last 2 columns), or none
    const bool full = tid < G::NFULL, left = !full && tid < G::NFULL + G::NLEFT;
    const bool stager = wave * 64 < G::NFULL + G::NLEFT;  // wave-uniform
    const int u = full ? tid : tid - G::NFULL;
    const int cg = full ? u % 4 : 0, cb = full ? (u / 4) % 2 : u % 2, rr = full ? u / 8 : u / 2;
    const int gr = row0 + rr, gc = col0 + (full ? 8 * cg : TC);
    const bool uok = (full || left) && gr < H && gc < W;
    // byte offset of channel c8 of the unit in chunk 0; chunk k adds k * 16 H W * 2
    const unsigned ubase = uok ? (unsigned)(((cb * 8) * H + gr) * W + gc) * 2u : GOOB;
    const unsigned cstride = (unsigned)(H * W) * 2u;               // next channel
    const int lbase = (rr * HCOL16 + (full ? 8 * cg : TC)) * 32 + cb * 16;  // LDS byte offset

    // channel c8's 8 columns from the unit's first column (a left-over unit uses
    // the first 2; its 8-column group is whole and aligned too, since W % 8 ==
    // 0): one kind of load for every staging lane, issued without a branch
    u4v xf[8];
    u4v wf[WPF];
    auto fetch = [&](int chunk) {
        const unsigned cbase = (unsigned)chunk * CC16 * cstride;
        if (stager) {
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) {
                const unsigned off = uok ? ubase + cbase + (unsigned)c8 * cstride : GOOB;
                xf[c8] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0));
            }
        }
        const u4v *src = reinterpret_cast<const u4v *>(wt) + (size_t)chunk * G::WV;
#pragma unroll
        for (int q = 0; q < WPF; ++q) {
            const int e = tid + q * THREADS;
            wf[q] = src[e < G::WV ? e : 0];
        }
    };
    auto stash = [&](int buf) {
        unsigned char *b = lds + buf * BUF;
        if (full) {
            // column c gets dwords (ch 0,1), (2,3), (4,5), (6,7) of that column
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                u4v o0, o1;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    o0[p] = lo_pair(xf[2 * p][m], xf[2 * p + 1][m]);
                    o1[p] = hi_pair(xf[2 * p][m], xf[2 * p + 1][m]);
                }
                *reinterpret_cast<u4v *>(b + lbase + (2 * m) * 32) = o0;
                *reinterpret_cast<u4v *>(b + lbase + (2 * m + 1) * 32) = o1;
            }
        } else if (left) {
            u4v o0, o1;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                o0[p] = lo_pair(xf[2 * p][0], xf[2 * p + 1][0]);
                o1[p] = hi_pair(xf[2 * p][0], xf[2 * p + 1][0]);
            }
            *reinterpret_cast<u4v *>(b + lbase) = o0;
            *reinterpret_cast<u4v *>(b + lbase + 32) = o1;
        }
        u4v *wl = reinterpret_cast<u4v *>(b + XBYTES);
#pragma unroll
        for (int q = 0; q < WPF; ++q) {
            const int e = tid + q * THREADS;
            if (e < G::WV) wl[e] = wf[q];
        }
    };

    v16f acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int nchunks = C_in / CC16;
    if (tid < CO) sbias[tid] = bias ? bias[tid] : 0.0f;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        if (ch + 1 < nchunks) fetch(ch + 1);
        const unsigned char *xs = lds + buf * BUF;
        const unsigned char *as = xs + XBYTES + ((64 * wm + j) * CC16 + 8 * h) * 2;
        const unsigned char *bs = xs + ((4 * wn) * HCOL16 + j) * 32 + 16 * h;
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const int kh = tap / 3, kw = tap % 3;
            u4v a[2], b[4];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
                a[bi] = *reinterpret_cast<const u4v *>(as + ((tap * CO + 32 * bi) * CC16) * 2);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                b[bj] = *reinterpret_cast<const u4v *>(bs + ((bj + kh) * HCOL16 + kw) * 32);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mfma16<DT>(a[bi], b[bj], acc[bi][bj]);
        }
        if (ch + 1 < nchunks) stash(buf ^ 1);  // buf^1 was last read in iteration ch-1
        __syncthreads();
    }

    // ---- epilogue: register r of acc[bi][bj] is channel 64 wm + 32 bi +
    // 8 (r / 4) + 4 h + r % 4 at row row0 + 4 wn + bj, column col0 + j.
    // Statistics per 16-lane row s16 (columns 16 s16 .. + 15 of the wave's 4
    // rows), then one Chan merge per channel over the 2 NR row partials.  A
    // tile wholly inside the output (every tile but the last row and column
    // ones) takes the unmasked path.
    const int s16 = (lane >> 4) & 1;
    const unsigned plane = (unsigned)Ho * Wo;
    const auto yr = make_rsrc(y + (size_t)n * CO * plane, CO * plane * 4u);
    float (*red)[2][CO][3] = reinterpret_cast<float (*)[2][CO][3]>(lds);
    auto epilogue = [&](auto whole) {
        constexpr bool WHOLE = decltype(whole)::value;
        int rem[4];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) rem[bj] = WHOLE ? TC : row0 + 4 * wn + bj < Ho ? Wo - col0 : 0;
        int cnt = 0;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) cnt += min(max(rem[bj] - 16 * s16, 0), 16);
        const float rcnt = WHOLE ? 1.0f / 64.0f : cnt ? 1.0f / (float)cnt : 0.0f;
        bool ok[4];
        unsigned voff[4];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            ok[bj] = WHOLE || j < rem[bj];
            voff[bj] = ok[bj] ? ((unsigned)(64 * wm + 4 * h) * plane +
                                 (unsigned)(row0 + 4 * wn + bj) * Wo + col0 + j) * 4u
                              : GOOB;
        }
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dc = 32 * bi + 8 * (r >> 2) + (r & 3);  // co - 64 * wm - 4 * h
                const int co = 64 * wm + 4 * h + dc;
                const float bc = sbias[co];
                const unsigned so = (unsigned)dc * plane * 4u;     // uniform
                float v[4], sum = 0.0f;
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    v[bj] = activate<ACT>(acc[bi][bj][r] + bc);
                    buf_store1(v[bj], yr, voff[bj], so);
                    sum += ok[bj] ? v[bj] : 0.0f;
                }
                const float mean = row_sum16(sum) * rcnt;
                float sq = 0.0f;
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const float d = v[bj] - mean;
                    sq = ok[bj] ? fmaf(d, d, sq) : sq;
                }
                const float m2 = row_sum16(sq);
                if ((lane & 15) == 0) {
                    red[wn][s16][co][0] = (float)cnt;
                    red[wn][s16][co][1] = mean;
                    red[wn][s16][co][2] = m2;
                }
            }
        }
    };
    if (row0 + TR <= Ho && col0 + TC <= Wo)
        epilogue(std::integral_constant<bool, true>{});
    else
        epilogue(std::integral_constant<bool, false>{});
    __syncthreads();
    if (tid < CO) {
        float tc = 0.f, tm = 0.f, tq = 0.f;
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                chan_merge(tc, tm, tq, red[k][q][tid][0], red[k][q][tid][1], red[k][q][tid][2]);
        const size_t tile = (size_t)th * tiles_w + tw;
        float *pp = partials + (((size_t)n * tiles_per_sample + tile) * CO + tid) * 3;
        pp[0] = tc; pp[1] = tm; pp[2] = tq;
    }
}

// Statistics -> per-channel scale and shift.  One wave per (sample, norm
// group): lane l folds the group's (channel, tile) partials l, l + 64, ... in
// order, the 64 lane results are merged by a fixed tree (DPP rows, then the two
// row pairs, then the halves), and lane 0's result is the group's, so every
// channel of the group uses the same mean and variance.
__global__ __launch_bounds__(256)
void conv2d_norm_finalize_kernel(const float *__restrict__ partials, const float *__restrict__ gamma,
                                 const float *__restrict__ beta, v2f *__restrict__ ss, int N, int C,
                                 int tiles, int norm_groups, float eps, float inv_div)
{
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= N * norm_groups) return;  // whole waves; the kernel has no barriers
    const int n = wid / norm_groups, g = wid % norm_groups;
    const int cg = C / norm_groups, c0 = g * cg;
    const int items = cg * tiles;
    float cnt = 0.f, mean = 0.f, m2 = 0.f;
    for (int i = lane; i < items; i += 64) {
        const int j = i / tiles, t = i % tiles;
        const float *pp = partials + (((size_t)n * tiles + t) * C + c0 + j) * 3;
        chan_merge(cnt, mean, m2, pp[0], pp[1], pp[2]);
    }
    row_chan16(cnt, mean, m2);
#pragma unroll
    for (int sh = 16; sh <= 32; sh *= 2) {
        const float nb = __shfl_xor(cnt, sh, 64), mb = __shfl_xor(mean, sh, 64),
                    qb = __shfl_xor(m2, sh, 64);
        chan_merge(cnt, mean, m2, nb, mb, qb);
    }
    cnt = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cnt)));
    mean = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mean)));
    m2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, m2)));
    const float rstd = rsqrtf(m2 / cnt + eps);
    for (int j = lane; j < cg; j += 64) {
        const int c = c0 + j;
        const float ga = gamma ? gamma[c] : 1.0f, be = beta ? beta[c] : 0.0f;
        ss[(size_t)n * C + c] = v2f{rstd * ga * inv_div, (be - mean * rstd * ga) * inv_div};
    }
}

// y = y * scale + shift in place, with (scale, shift) per (sample, channel)
// plane (ss) or uniform (ss null: the divide alone).  Workgroup b covers chunk
// b % chunks of plane b / chunks: APPLY_V vectors of VEC floats per thread,
// all loads issued before the stores.  VEC = 4 needs plane % 4 == 0.
constexpr int APPLY_V = 4;
template <int VEC>
__global__ __launch_bounds__(256)
void conv2d_apply_kernel(float *__restrict__ y, const v2f *__restrict__ ss, float uscale,
                         int plane, int chunks)
{
    typedef float vt __attribute__((ext_vector_type(VEC)));
    const int p = blockIdx.x / chunks, chunk = blockIdx.x - p * chunks;
    const v2f s = ss ? ss[p] : v2f{uscale, 0.0f};
    const int nv = plane / VEC;
    vt *yp = reinterpret_cast<vt *>(y + (size_t)p * plane);
    const int i0 = chunk * (256 * APPLY_V) + threadIdx.x;
    vt v[APPLY_V];
#pragma unroll
    for (int k = 0; k < APPLY_V; ++k)
        if (i0 + k * 256 < nv) v[k] = yp[i0 + k * 256];
#pragma unroll
    for (int k = 0; k < APPLY_V; ++k)
        if (i0 + k * 256 < nv) yp[i0 + k * 256] = v[k] * s[0] + s[1];
}

// Flat form: workgroup b takes float4 vectors [b * 256 * APPLY_V, +256 * APPLY_V)
// of the whole [N * C][plane] tensor, so every cache line belongs to one
// workgroup (planes of 126^2 or 258^2 floats do not end on line boundaries).
// A chunk is no longer than a plane, so it spans at most two planes: the first
// vector's plane p0 and p0 + 1.
__global__ __launch_bounds__(256)
void conv2d_apply_flat_kernel(float *__restrict__ y, const v2f *__restrict__ ss, float uscale,
                              int plane4, int total4)
{
    const int base = blockIdx.x * (256 * APPLY_V);
    const int p0 = base / plane4, b1 = (p0 + 1) * plane4;
    const v2f s0 = ss ? ss[p0] : v2f{uscale, 0.0f};
    const v2f s1 = ss ? ss[min(p0 + 1, total4 / plane4 - 1)] : v2f{uscale, 0.0f};
    v4f *y4 = reinterpret_cast<v4f *>(y);
    v4f v[APPLY_V];
#pragma unroll
    for (int k = 0; k < APPLY_V; ++k) {
        const int i = base + threadIdx.x + k * 256;
        if (i < total4) v[k] = y4[i];
    }
#pragma unroll
    for (int k = 0; k < APPLY_V; ++k) {
        const int i = base + threadIdx.x + k * 256;
        if (i < total4) {
            const v2f s = i < b1 ? s0 : s1;
            y4[i] = v[k] * s[0] + s[1];
        }
    }
}

}  // namespace

bool conv2d_igemm_supported(int C_in, int C_out, int kernel, int groups, int H, int W, int act,
                            int stride)
{
    // (H, W: the padded input; one sample's output planes are addressed with
    // 32-bit byte offsets and its input planes with 32-bit element offsets)
    const int cc = stride == 1 ? Geo<128, 1>::CC : Geo<128, 2>::CC;
    const long long ho = H >= 3 ? (H - 3) / stride + 1 : 0, wo = W >= 3 ? (W - 3) / stride + 1 : 0;
    return (C_out == 128 || C_out == 64) && kernel == 3 && groups == 1 && (stride == 1 || stride == 2) &&
           C_in % cc == 0 && C_in >= cc && H >= 3 && W >= 3 &&
           (long long)C_out * ho * wo * 4 < (long long)RES_MAX &&
           (long long)C_in * H * W < (1LL << 31) &&
           (act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF || act == ACT_GELU_TANH);
}

bool conv2d_igemm16_supported(int C_in, int C_out, int kernel, int groups, int H, int W, int act)
{
    return (C_out == 128 || C_out == 64) && kernel == 3 && groups == 1 && C_in % CC16 == 0 &&
           C_in >= CC16 && H >= 3 && W >= 8 && W % 8 == 0 &&
           (long long)C_out * (H - 2) * (W - 2) * 4 < (long long)RES_MAX &&
           (long long)C_in * H * W * 2 < (1LL << 31) &&
           (act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF || act == ACT_GELU_TANH);
}

static int tile_rows(int C_out, int dtype)
{
    if (dtype) return C_out == 128 ? Geo16<128>::TR : Geo16<64>::TR;
    return C_out == 128 ? Geo<128, 1>::TR : Geo<64, 1>::TR;
}

static size_t tiles_of(int C_out, int Ho, int Wo, int dtype)
{
    const int tr = tile_rows(C_out, dtype);
    return (size_t)((Wo + TC - 1) / TC) * ((Ho + tr - 1) / tr);
}

// Edge strips (fp32, stride 1): the output columns left to column-strip tiles
// (Wo mod 32 when that is 1 or 2 and Wo > 32, else 0) and the rows left to
// row-strip tiles (Ho mod TR when that is 1 or 2 and Ho > TR, else 0).
struct EdgeTiles {
    int tiles_w, tiles_h, row_strips, col_strips;
    int total() const { return tiles_w * tiles_h + row_strips + col_strips; }
};
template <int CO>
static EdgeTiles edge_tiles(int Ho, int Wo, bool edges)
{
    constexpr int TR = Geo<CO, 1>::TR;
    const int rc = Wo % TC, rr = Ho % TR;
    const bool cs = edges && Wo > TC && (rc == 1 || rc == 2), rs = edges && Ho > TR && (rr == 1 || rr == 2);
    EdgeTiles e;
    e.tiles_w = cs ? Wo / TC : (Wo + TC - 1) / TC;
    e.tiles_h = rs ? Ho / TR : (Ho + TR - 1) / TR;
    e.row_strips = rs ? (e.tiles_w * TC + GeoRow<CO>::TW - 1) / GeoRow<CO>::TW : 0;
    e.col_strips = cs ? (Ho + GeoStrip<CO>::TR - 1) / GeoStrip<CO>::TR : 0;
    return e;
}

// [N][tiles][C_out][3] Welford partials, the weight copy ([ci][tap][co] fp32,
// or [ci / 16][tap][co][16] 16-bit), then [N][C_out] (scale, shift) pairs
static size_t weight_copy_bytes(int C_in, int C_out, int dtype)
{
    return (size_t)C_in * 9 * C_out * (dtype ? 2 : 4);
}

size_t conv2d_igemm_workspace(int N, int C_in, int C_out, int Ho, int Wo, int dtype)
{
    return (size_t)N * tiles_of(C_out, Ho, Wo, dtype) * C_out * 3 * sizeof(float) +
           weight_copy_bytes(C_in, C_out, dtype) + (size_t)N * C_out * 2 * sizeof(float);
}

template <int CO, int ACT>
static void launch_gemm(const Conv2dIgemmArgs &a, const float *wt, const EdgeTiles &e, hipStream_t st)
{
    static_assert(Geo<CO, 1>::TR == Geo<CO, 2>::TR, "one tile height per channel count");
    const float *x = static_cast<const float *>(a.x);
    const int tps = e.total();
    const dim3 grid(tps, 1, a.N);
#define CNF_ARGS                                                                                   \
    grid, dim3(THREADS), 0, st, x, wt, a.b, a.out, a.partials, a.C_in, a.H, a.W, a.Ho, a.Wo, a.pad, \
        e.tiles_w, e.tiles_h, e.row_strips, tps
    if (a.stride == 2)
        hipLaunchKernelGGL((conv2d_igemm_kernel<CO, ACT, 2, false>), CNF_ARGS);
    else if (e.row_strips || e.col_strips)
        hipLaunchKernelGGL((conv2d_igemm_kernel<CO, ACT, 1, true>), CNF_ARGS);
    else
        hipLaunchKernelGGL((conv2d_igemm_kernel<CO, ACT, 1, false>), CNF_ARGS);
#undef CNF_ARGS
}

template <int CO, int ACT>
static void launch_gemm16(const Conv2dIgemmArgs &a, const unsigned short *wt, int tiles_w, int tiles_h,
                          int tps, hipStream_t st)
{
    const unsigned short *x = static_cast<const unsigned short *>(a.x);
    if (a.dtype == 1)
        hipLaunchKernelGGL((conv2d_igemm16_kernel<CO, ACT, 1>), dim3(tiles_w, tiles_h, a.N), dim3(THREADS),
                           0, st, x, wt, a.b, a.out, a.partials, a.C_in, a.H, a.W, a.Ho, a.Wo, tiles_w,
                           tps);
    else
        hipLaunchKernelGGL((conv2d_igemm16_kernel<CO, ACT, 2>), dim3(tiles_w, tiles_h, a.N), dim3(THREADS),
                           0, st, x, wt, a.b, a.out, a.partials, a.C_in, a.H, a.W, a.Ho, a.Wo, tiles_w,
                           tps);
}

hipError_t launch_conv2d_igemm(const Conv2dIgemmArgs &a, hipStream_t st)
{
    if (a.stride != 1 && (a.stride != 2 || a.transposed)) return hipErrorInvalidValue;
    const int dt = a.dtype;
    if (dt != 0 && (dt > 2 || a.stride != 1 || a.transposed || a.pad != 0 || a.W % 8 != 0 ||
                    a.C_in % CC16 != 0))
        return hipErrorInvalidValue;
    const int CO = a.C_out, tr = tile_rows(CO, dt);
    const bool edges = dt == 0 && a.stride == 1;
    const EdgeTiles et = CO == 128 ? edge_tiles<128>(a.Ho, a.Wo, edges) : edge_tiles<64>(a.Ho, a.Wo, edges);
    const int tiles_w = (a.Wo + TC - 1) / TC, tiles_h = (a.Ho + tr - 1) / tr;  // (16-bit kernel)
    const int tps = dt ? tiles_w * tiles_h : et.total();
    // The strips of a sample never outnumber the 32-column tiles they replace (a
    // row strip is at least as wide as a tile row, a column strip at least as
    // tall as a tile column), so the partials fit the space tiles_of sizes.
    const size_t tps_space = tiles_of(CO, a.Ho, a.Wo, dt);  // the partials conv2d_igemm_workspace sizes
    if ((size_t)tps > tps_space) return hipErrorInvalidValue;
    float *wt = a.partials + (size_t)a.N * tps_space * CO * 3;
    {
        const int total = CO * a.C_in * 9;
        if (dt)
            hipLaunchKernelGGL(conv2d_weight_pack16_kernel, dim3((total + 255) / 256), dim3(256), 0, st,
                               static_cast<const unsigned short *>(a.w),
                               reinterpret_cast<unsigned short *>(wt), a.C_in, CO);
        else
            hipLaunchKernelGGL(conv2d_weight_transpose_kernel, dim3((total + 255) / 256), dim3(256), 0,
                               st, static_cast<const float *>(a.w), wt, a.C_in, CO, a.transposed);
    }
    hipError_t e = dominant_begin(st);
    if (e != hipSuccess) return e;
    const unsigned short *wt16 = reinterpret_cast<const unsigned short *>(wt);
#define CNF_CASE(C, A)                                                                    \
    if (CO == C && a.act == A) {                                                          \
        if (dt) launch_gemm16<C, A>(a, wt16, tiles_w, tiles_h, tps, st);                  \
        else launch_gemm<C, A>(a, wt, et, st);                                            \
    } else
    CNF_CASE(128, ACT_NONE) CNF_CASE(128, ACT_HARDSWISH) CNF_CASE(128, ACT_GELU_ERF)
    CNF_CASE(128, ACT_GELU_TANH) CNF_CASE(64, ACT_NONE) CNF_CASE(64, ACT_HARDSWISH)
    CNF_CASE(64, ACT_GELU_ERF) CNF_CASE(64, ACT_GELU_TANH)
    return hipErrorInvalidValue;
#undef CNF_CASE
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = dominant_end(st)) != hipSuccess) return e;
    if (a.norm_groups > 0 || a.inv_div != 1.0f) {
        v2f *ss = nullptr;
        if (a.norm_groups > 0) {
            ss = reinterpret_cast<v2f *>(reinterpret_cast<char *>(wt) + weight_copy_bytes(a.C_in, CO, dt));
            const int waves = a.N * a.norm_groups;
            hipLaunchKernelGGL(conv2d_norm_finalize_kernel, dim3((waves + 3) / 4), dim3(256), 0, st,
                               a.partials, a.gamma, a.beta, ss, a.N, CO, tps, a.norm_groups, a.eps,
                               a.inv_div);
        }
        const int plane = a.Ho * a.Wo;
        const int vec = plane % 4 == 0 ? 4 : 1;
        const long long total4 = (long long)a.N * CO * plane / 4;
        if (vec == 4 && plane / 4 >= 256 * APPLY_V && total4 < 0x7fffffffLL - 256 * APPLY_V) {
            const unsigned blocks = (unsigned)((total4 + 256 * APPLY_V - 1) / (256 * APPLY_V));
            hipLaunchKernelGGL(conv2d_apply_flat_kernel, dim3(blocks), dim3(256), 0, st, a.out, ss,
                               a.inv_div, plane / 4, (int)total4);
            return hipGetLastError();
        }
        const int chunks = (plane / vec + 256 * APPLY_V - 1) / (256 * APPLY_V);
        if ((long long)a.N * CO * chunks > 0x7fffffffLL) return hipErrorInvalidValue;
        const dim3 grid((unsigned)(a.N * CO * chunks));
        if (vec == 4)
            hipLaunchKernelGGL(conv2d_apply_kernel<4>, grid, dim3(256), 0, st, a.out, ss, a.inv_div,
                               plane, chunks);
        else
            hipLaunchKernelGGL(conv2d_apply_kernel<1>, grid, dim3(256), 0, st, a.out, ss, a.inv_div,
                               plane, chunks);
    }
    return hipGetLastError();
}

}  // namespace cnf
