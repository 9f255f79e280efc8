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
//                          up to 4 x 16 channels x a 4-row x 16-column block of
//                          positions (row coordinates are wave-uniform; each
//                          gathered operand feeds up to 16 MFMAs); a strided transposed
//                          conv is split into stride^ndim phases so only the taps
//                          that reach a phase are issued; + bias + activation;
//                          writes the conv output and, for each (sample, channel,
//                          64-position tile), (count, mean, M2) from two passes
//                          over the tile.
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

struct GenConv {
    const void *x, *wp;        // element type DT; wp: weights packed by gen_weight_pack_kernel
    const float *b;
    float *y;          // conv output [N][C_out][S] or nullptr
    v4f *part;         // [N][C_out][T] (count, mean, M2, 0) or nullptr
    int tasks;         // N * nph * Tq * GTn * cobN (below 2^31)
    int tpw;           // tasks per wave
    int C_in, C_out, Cgi, Cgo, G, cobN, T, Tq, CT;  // CT: column tiles per phase
    // P conv groups share one 16-row tile (groups of at most 8 output channels):
    // RPG = 16/P rows and KPG = KS/P K entries per group per step (KS = 4 K
    // entries per step for fp32, 16 for the 16-bit types); GTn = ceil(G/P)
    // group tiles; steps = ceil(Cgi/KPG) K steps per tap; KP = KS*steps.
    int P, RPG, KPG, GTn, steps, KP;
    int act;
    int D, H, W, Do, Ho, Wo, S;
    int kd, kh, kw;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    unsigned in_plane, wp_elems;
    float out_scale;
};

// A wave's 64 output positions are ROWS rows x (64 / ROWS) consecutive
// columns (four MFMA column tiles u; tile u is row u / CW, columns
// (u % CW)*16 + col).  Row coordinates are wave-uniform; columns are per lane.
// Wide outputs use one row of 64 columns, so each store instruction of a wave
// writes whole runs of a row.
//
// A conv gathers input x[o*s - p + a*d].  A transposed conv (the adjoint) reaches
// output o from input (o + p - a*d)/s where s divides o + p - a*d.  Along z and y
// the outputs are visited in phases: rows o = q*s + r with the same residue r
// are reached by the same taps (those with s | r + p - a*d) from input rows
// q + (r + p - a*d)/s, so a wave works inside one phase and skips the other taps
// with a uniform branch.  Along x each lane checks its own column: the exact
// quotient comes from a float product, exact for 0 <= t < 2^21 (the fraction of
// (t + 0.5)/s is at least 0.5/s from an integer, the float error below 0.25/s).
//
// One wave owns NB blocks of 16 output channels of one conv group: each
// gathered input operand feeds NB MFMAs, each weight operand 4.
//
// DT selects the input element type: 0 fp32 (v_mfma_f32_16x16x4f32, one K
// entry per lane per step), 1 bf16 / 2 fp16 (v_mfma_f32_16x16x16_{bf16,f16},
// four consecutive K entries per lane per step; products are exact in fp32 and
// accumulate in fp32).
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef unsigned short v4us __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float activate_rt(float x, int act) {
    switch (act) {
    case ACT_HARDSWISH: return hardswish(x);
    case ACT_GELU_ERF: return gelu_erf(x);
    case ACT_GELU_TANH: return gelu_tanh(x);
    default: return x;
    }
}

template <int DT>
__device__ __forceinline__ v4f mfma16(v4us a, v4us b, v4f c) {
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4bf, a),
                                                         __builtin_bit_cast(v4bf, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, a),
                                                     __builtin_bit_cast(v4h, b), c, 0, 0, 0);
}

template <bool TR, int NB, int ROWS, int DT>
__device__ __forceinline__ void gen_conv_task(const GenConv &g, int task, int lane) {
    constexpr unsigned ES = DT ? 2u : 4u;   // element size of x and the packed weights
    constexpr int KL = DT ? 4 : 1;          // K entries a lane supplies per step
    constexpr int CW = 4 / ROWS;  // 16-column tiles per row
    const int col = lane & 15, kq = lane >> 4;
    // Task order (fastest first): channel blocks, phase, group, tile, sample.
    const int nph = TR ? g.sd * g.sh : 1;
    int t = task;
    const int cbn = t % g.cobN; t /= g.cobN;
    const int phs = t % nph; t /= nph;
    const int gt = t % g.GTn; t /= g.GTn;
    const int pt = t % g.Tq;
    const int n = t / g.Tq;

    // Phase residues (z, y) and the phase's row grid (all rows for a conv).
    int rz = 0, ry = 0, Qz = g.Do, Qy = g.Ho;
    if (TR) {
        ry = phs % g.sh;
        rz = phs / g.sh;
        Qz = (g.Do - rz + g.sd - 1) / g.sd;
        Qy = (g.Ho - ry + g.sh - 1) / g.sh;
    }
    const int rt = pt / g.CT, ct = pt - rt * g.CT;
    const int row0 = rt * ROWS, col0 = ct * 16 * CW;
    const int nrows = min(ROWS, Qz * Qy - row0), ncols = min(16 * CW, g.Wo - col0);
    const int cnt = nrows > 0 && ncols > 0 ? nrows * ncols : 0;
    const int tile = phs * g.Tq + pt;

    // Output channel of accumulator row `row` of block b (tile rows are split
    // into P groups of RPG rows); false for padding rows.
    auto out_channel = [&](int b, int row, int &cgl) -> bool {
        const int grp = gt * g.P + row / g.RPG;
        const int co = (cbn * NB + b) * 16 + row % g.RPG;
        cgl = grp * g.Cgo + co;
        return co < g.Cgo && grp < g.G;
    };

    if (cnt <= 0) {  // this phase has fewer rows than the largest: empty statistics
        if (g.part && col == 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int cgl;
                    if (out_channel(b, 4 * kq + r, cgl))
                        g.part[((size_t)n * g.C_out + cgl) * g.T + tile] = v4f{0.f, 0.f, 0.f, 0.f};
                }
        }
        return;
    }

    // Rows (uniform): gather base along z and y, output row offset.
    int bz[ROWS], by[ROWS], orow[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const bool rv = r < nrows;
        const int rq = rv ? row0 + r : 0;
        const int qz = rq / Qy, qy = rq - qz * Qy;
        const int oz = TR ? qz * g.sd + rz : qz, oy = TR ? qy * g.sh + ry : qy;
        bz[r] = TR ? qz : oz * g.sd - g.pd;
        by[r] = TR ? qy : oy * g.sh - g.ph;
        if (!rv) bz[r] = -(1 << 29);  // every tap falls outside the input
        orow[r] = (oz * g.Ho + oy) * g.Wo;
    }
    const float rsw = 1.0f / (float)g.sw;
    // Columns (per lane): output column and the x term of the gather.  For a
    // transposed conv, (ox + pw) = bq * sw + bm; tap kx with kx*dw = kq' * sw + km
    // reaches the lane iff bm == km, from input column bq - kq'.
    int ox[4], bx[4], bm[4];
    bool pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        ox[u] = col0 + (u % CW) * 16 + col;
        pv[u] = (u / CW) < nrows && ox[u] < g.Wo;
        if (TR) {
            const int num = ox[u] + g.pw;  // >= 0, below 2^21
            bx[u] = (int)floorf(((float)num + 0.5f) * rsw);
            bm[u] = num - bx[u] * g.sw;
        } else {
            bx[u] = ox[u] * g.sw - g.pw;
            bm[u] = 0;
        }
    }

    // A operands: row col = output channel (cbn*NB + b)*16 + col, K entries
    // KL*kq .. KL*kq + KL-1.  In the packed weights a lane's NB*KL values are
    // adjacent and a (tap, K step) is one contiguous run of 64*NB*KL elements,
    // zero where the channel or the output channel is padding.
    const int taps = g.kd * g.kh * g.kw;
    const unsigned wrow = (unsigned)g.cobN * 16 * NB * KL;   // elements per lane row kq
    const unsigned woff = ((unsigned)kq * wrow + ((unsigned)cbn * 16 + col) * NB * KL) * ES;
    // B operand: K entry e of a step is channel c0 + e % KPG of group gt*P + e / KPG.
    const char *xs = static_cast<const char *>(g.x) +
                     ((size_t)n * g.C_in + (size_t)gt * g.P * g.Cgi) * g.in_plane * ES;
    const unsigned xbytes = (unsigned)(g.C_in - gt * g.P * g.Cgi) * g.in_plane * ES;
    unsigned koff[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) {
        const int e = KL * kq + i;
        koff[i] = (unsigned)((e / g.KPG) * g.Cgi + e % g.KPG) * g.in_plane * ES;
    }

    // Bias of this lane's output channels, fetched before the MFMA loop so its
    // latency overlaps the gathers.
    float bias[NB][4];
    const auto br = make_rsrc(g.b ? (const void *)g.b : g.x, g.b ? (unsigned)g.C_out * 4u : 0u);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int cgl;
            const bool cv = out_channel(b, 4 * kq + r, cgl);
            bias[b][r] = buf_load1(br, cv ? (unsigned)cgl * 4u : GOOB);
        }

    v4f acc[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[b][u] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kz = 0; kz < g.kd; ++kz) {
        int tz = kz * g.dd;
        if (TR) {
            const int num = rz + g.pd - kz * g.dd;
            if (num % g.sd) continue;
            tz = num / g.sd;
        }
        for (int ky = 0; ky < g.kh; ++ky) {
            int ty = ky * g.dh;
            if (TR) {
                const int num = ry + g.ph - ky * g.dh;
                if (num % g.sh) continue;
                ty = num / g.sh;
            }
            bool okzy[ROWS];
            unsigned rowb[ROWS];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const int iz = bz[r] + tz, iy = by[r] + ty;
                okzy[r] = (unsigned)iz < (unsigned)g.D && (unsigned)iy < (unsigned)g.H;
                rowb[r] = ((unsigned)iz * g.H + (unsigned)iy) * g.W * ES;
            }
            for (int kx = 0; kx < g.kw; ++kx) {
                const int tap = (kz * g.kh + ky) * g.kw + kx;
                const int kxd = kx * g.dw;
                const int kxq = TR ? kxd / g.sw : 0, kxm = TR ? kxd - kxq * g.sw : 0;
                unsigned xo[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    int ix;
                    bool okx;
                    if (TR) {
                        ix = bx[u] - kxq;
                        okx = bm[u] == kxm && (unsigned)ix < (unsigned)g.W;
                    } else {
                        ix = bx[u] + kxd;
                        okx = (unsigned)ix < (unsigned)g.W;
                    }
                    // (a lane's K entries add koff[i]; GOOB + koff stays past the end)
                    xo[u] = (okzy[u / CW] && okx) ? rowb[u / CW] + (unsigned)ix * ES : GOOB;
                }
                const unsigned wtap = ((unsigned)(gt * taps + tap) * g.KP) * (wrow / KL);
                for (int st = 0; st < g.steps; ++st) {
                    // buffers rebased on the step's first channel (scalar work);
                    // padding channels and other groups' rows meet zero weights
                    const int c0 = st * g.KPG;
                    const auto xr = make_rsrc(xs + (size_t)c0 * g.in_plane * ES,
                                              xbytes - (unsigned)c0 * g.in_plane * ES);
                    const unsigned wsh = wtap + (unsigned)st * 4u * wrow;   // elements
                    const auto wr = make_rsrc(static_cast<const char *>(g.wp) + (size_t)wsh * ES,
                                              (g.wp_elems - wsh) * ES);
                    if constexpr (DT == 0) {
                        float a[NB];
                        if constexpr (NB == 4) {
                            const v4f v = buf_load4(wr, woff);
                            a[0] = v[0]; a[1] = v[1]; a[2] = v[2]; a[3] = v[3];
                        } else if constexpr (NB == 2) {
                            const v2f v = buf_load2(wr, woff);
                            a[0] = v[0]; a[1] = v[1];
                        } else {
                            a[0] = buf_load1(wr, woff);
                        }
                        float bv[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) bv[u] = buf_load1(xr, xo[u] + koff[0]);
#pragma unroll
                        for (int b = 0; b < NB; ++b)
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[b][u] = mfma_16x16x4(a[b], bv[u], acc[b][u]);
                    } else {
                        // A: NB blocks x 4 consecutive K entries (8*NB bytes per lane)
                        v4us a[NB];
                        if constexpr (NB == 1) {
                            a[0] = __builtin_bit_cast(v4us, buf_load2(wr, woff));
                        } else {
#pragma unroll
                            for (int h = 0; h < NB / 2; ++h) {
                                const v4f v = buf_load4(wr, woff + 16u * h);
                                a[2 * h] = __builtin_bit_cast(v4us, v2f{v[0], v[1]});
                                a[2 * h + 1] = __builtin_bit_cast(v4us, v2f{v[2], v[3]});
                            }
                        }
                        // B: the lane's 4 K entries (channels) at each column tile
                        v4us bv[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                bv[u][i] = __builtin_amdgcn_raw_buffer_load_b16(
                                    xr, (int)(xo[u] + koff[i]), 0, 0);
#pragma unroll
                        for (int b = 0; b < NB; ++b)
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[b][u] = mfma16<DT>(a[b], bv[u], acc[b][u]);
                    }
                }
            }
        }
    }

    // Epilogue: lane holds channels 4*kq + r of block b at column tile u.
    const auto yr = make_rsrc(g.y ? g.y + (size_t)n * g.C_out * g.S : g.x,
                              g.y ? (unsigned)g.C_out * g.S * 4u : 0u);
    const float rcnt = 1.0f / (float)cnt;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int cgl;
        const bool cv = out_channel(b, 4 * kq + r, cgl);
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = activate_rt(acc[b][u][r] + bias[b][r], g.act);
        if (g.y) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                buf_store1(v[u] * g.out_scale, yr,
                           (cv && pv[u]) ? ((unsigned)cgl * g.S + orow[u / CW] + ox[u]) * 4u : GOOB);
        }
        if (g.part) {
            float sm = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) sm += pv[u] ? v[u] : 0.0f;
            const float mean = row_sum16(sm) * rcnt;
            float q = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float d = v[u] - mean;
                q += pv[u] ? d * d : 0.0f;
            }
            q = row_sum16(q);
            if (col == 0 && cv)
                g.part[((size_t)n * g.C_out + cgl) * g.T + tile] = v4f{(float)cnt, mean, q, 0.0f};
        }
    }
}

// Each wave runs g.tpw consecutive tasks (the host sizes it so a wave issues a
// few hundred MFMAs).
template <bool TR, int NB, int ROWS, int DT>
__global__ __launch_bounds__(GT) void gen_conv_kernel(GenConv g) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int first = (xcd_remap(blockIdx.x, gridDim.x) * 4 + wave) * g.tpw;
    for (int j = 0; j < g.tpw; ++j) {
        const int task = first + j;
        if (task >= g.tasks) return;  // whole waves leave; the kernel has no barriers
        gen_conv_task<TR, NB, ROWS, DT>(g, task, lane);
    }
}

// Packed weights for gen_conv_kernel: wp[gt][tap][st][kq][cbn][col][b][i] is
// the A operand entry (row (cbn*NB + b)*16 + col, K entry e = KL*kq + i) of K
// step st at that tap for group tile gt: with P groups per tile, the row
// belongs to group gt*P + row / RPG (output channel row % RPG) and the K entry
// to group gt*P + e / KPG (input channel st*KPG + e % KPG); the entry is the
// weight when both name the same existing group and real channels, else 0
// (block-diagonal A, zero padding).  KL = 1 K entry per lane for fp32, 4 for
// the 16-bit types (copied bit for bit).  Source layout: conv w[C_out][Cgi][taps],
// transposed conv w[C_in][Cgo][taps].
template <typename E>
__global__ __launch_bounds__(GT) void gen_weight_pack_kernel(const E *w, E *wp, int G, int Cgi,
                                                             int Cgo, int taps, int steps, int P,
                                                             int KL, int cobN, int NB,
                                                             int transposed, unsigned total) {
    const unsigned idx = blockIdx.x * GT + threadIdx.x;
    if (idx >= total) return;
    const int RPG = 16 / P, KPG = 4 * KL / P;
    unsigned r = idx;
    const int i = r % KL; r /= KL;
    const int b = r % NB; r /= NB;
    const int col = r % 16; r /= 16;
    const int cbn = r % cobN; r /= cobN;
    const int kq = r % 4; r /= 4;
    const int st = r % steps; r /= steps;
    const int tap = r % taps;
    const int gt = r / taps;
    const int e = KL * kq + i;
    const int grp = gt * P + col / RPG;
    const int co = (cbn * NB + b) * 16 + col % RPG;
    const int ci = st * KPG + e % KPG;
    E v = E(0);
    if (grp == gt * P + e / KPG && grp < G && co < Cgo && ci < Cgi)
        v = transposed ? w[((size_t)(grp * Cgi + ci) * Cgo + co) * taps + tap]
                       : w[((size_t)(grp * Cgo + co) * Cgi + ci) * taps + tap];
    wp[idx] = v;
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

// y[plane][i] = y * scale[plane] + shift[plane]; workgroup b takes chunk
// b % chunks (of APPLY_CHUNK elements) of plane b / chunks, so consecutive
// workgroups stream consecutive addresses.  Planes of a multiple of 4 elements
// are 16-byte aligned and go by 16-byte accesses.  Each thread issues all its
// loads before its stores (a load-store loop kept one load in flight per thread).
constexpr int APPLY_PER = 4;                    // accesses per thread
constexpr int APPLY_CHUNK = GT * APPLY_PER * 4;
template <int VEC>
__device__ __forceinline__ void apply_chunk(float *p, int lo, int hi, v2f sc) {
    typedef float vt __attribute__((ext_vector_type(VEC)));
    vt *q = reinterpret_cast<vt *>(p);
    const int i0 = lo / VEC + threadIdx.x, n = hi / VEC;
    vt v[APPLY_PER];
#pragma unroll
    for (int k = 0; k < APPLY_PER; ++k)
        if (i0 + k * GT < n) v[k] = q[i0 + k * GT];
#pragma unroll
    for (int k = 0; k < APPLY_PER; ++k) {
        if (i0 + k * GT < n) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[k][e] = fmaf(v[k][e], sc[0], sc[1]);
            q[i0 + k * GT] = v[k];
        }
    }
}
// Flat form for planes of at least one chunk (S % 4 == 0): workgroup b takes
// vectors [b * APPLY_CHUNK / 4, +APPLY_CHUNK / 4) of the whole [N * C][S] tensor,
// so no cache line is split between workgroups where planes do not end on line
// boundaries; a chunk spans at most two planes, p0 and p0 + 1.
__global__ __launch_bounds__(GT) void gen_apply_flat_kernel(float *y, const v2f *ss, int S4, int total4) {
    constexpr int CV = APPLY_CHUNK / 4;  // vectors per chunk (= GT * APPLY_PER)
    const int base = blockIdx.x * CV;
    const int p0 = base / S4, b1 = (p0 + 1) * S4;
    const v2f s0 = ss[p0], s1 = ss[min(p0 + 1, total4 / S4 - 1)];
    v4f *q = reinterpret_cast<v4f *>(y);
    v4f v[APPLY_PER];
#pragma unroll
    for (int k = 0; k < APPLY_PER; ++k) {
        const int i = base + threadIdx.x + k * GT;
        if (i < total4) v[k] = q[i];
    }
#pragma unroll
    for (int k = 0; k < APPLY_PER; ++k) {
        const int i = base + threadIdx.x + k * GT;
        if (i < total4) {
            const v2f sc = i < b1 ? s0 : s1;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[k][e] = fmaf(v[k][e], sc[0], sc[1]);
            q[i] = v[k];
        }
    }
}
__global__ __launch_bounds__(GT) void gen_apply_kernel(float *y, const v2f *ss, int S, int chunks) {
    const int plane = blockIdx.x / chunks, chunk = blockIdx.x - plane * chunks;
    const v2f sc = ss[plane];
    float *p = y + (size_t)plane * S;
    const int lo = chunk * APPLY_CHUNK, hi = min(S, lo + APPLY_CHUNK);
    if ((S & 3) == 0) {
        apply_chunk<4>(p, lo, hi, sc);
    } else {
        // scalar accesses: the chunk in APPLY_CHUNK / (GT * APPLY_PER) passes
        for (int part = lo; part < hi; part += GT * APPLY_PER)
            apply_chunk<1>(p, part, min(hi, part + GT * APPLY_PER), sc);
    }
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

int blocks_per_wave(int Cgo) {
    const int cob = (Cgo + 15) / 16;
    return cob >= 4 ? 4 : cob >= 2 ? 2 : 1;
}

struct GenLayout {
    bool stats, stage, softmax, finalize, apply;
    int nph, Tq, CT;  // conv phases (z, y), tiles per phase, column tiles per row
    int ROWS;         // rows per tile: 1 (64 columns) or 4 (16 columns)
    int NB, cobN, P, KPG, GTn, steps;
    int KL, ES;       // K entries per lane per step (1 fp32, 4 16-bit); element bytes
    size_t off_wp, wp_elems;
    int T;            // statistics tiles per (sample, channel)
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
    // A transposed conv visits its outputs in stride^ndim phases (see
    // gen_conv_kernel); each phase gets as many tiles as the largest needs.
    // Tiles are ROWS rows (over z, y) x 64/ROWS columns; a transposed conv's
    // rows are split into sd*sh phases (the largest phase has the most rows).
    L.nph = 1;
    long long Qzy = (long long)a.Do * a.Ho;
    if (a.transposed) {
        L.nph = a.sd * a.sh;
        Qzy = (long long)((a.Do + a.sd - 1) / a.sd) * ((a.Ho + a.sh - 1) / a.sh);
    }
    L.ROWS = a.Wo >= 48 ? 1 : 4;
    const int tw = PTILE / L.ROWS;
    L.CT = (a.Wo + tw - 1) / tw;
    L.Tq = (int)((Qzy + L.ROWS - 1) / L.ROWS) * L.CT;
    // the softmax pass writes the statistics over contiguous positions instead
    L.T = L.softmax ? (int)((S + PTILE - 1) / PTILE) : L.nph * L.Tq;
    const int Cgi = a.C_in / a.groups, Cgo = a.C_out / a.groups;
    // Groups of at most 8 output channels share a 16-row tile, P per tile.
    int pw2 = 1;
    while (pw2 < Cgo) pw2 <<= 1;
    L.P = (Cgo <= 8 && a.groups >= 2) ? (16 / pw2 < 4 ? 16 / pw2 : 4) : 1;
    L.KL = a.dtype ? 4 : 1;
    L.ES = a.dtype ? 2 : 4;
    L.KPG = 4 * L.KL / L.P;
    L.GTn = (a.groups + L.P - 1) / L.P;
    L.steps = (Cgi + L.KPG - 1) / L.KPG;
    L.NB = L.P > 1 ? 1 : blocks_per_wave(Cgo);
    L.cobN = L.P > 1 ? 1 : ((Cgo + 15) / 16 + L.NB - 1) / L.NB;
    L.wp_elems = (size_t)L.GTn * a.kd * a.kh * a.kw * 4 * L.steps * L.cobN * 16 * L.NB * L.KL;
    size_t off = 0;
    L.off_wp = off;
    off = align256(off + L.wp_elems * L.ES);
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

template <bool TR, int ROWS, int DT>
void launch_conv_nb(const GenConv &g, int NB, dim3 grid, hipStream_t st) {
    if (NB == 4) gen_conv_kernel<TR, 4, ROWS, DT><<<grid, dim3(GT), 0, st>>>(g);
    else if (NB == 2) gen_conv_kernel<TR, 2, ROWS, DT><<<grid, dim3(GT), 0, st>>>(g);
    else gen_conv_kernel<TR, 1, ROWS, DT><<<grid, dim3(GT), 0, st>>>(g);
}

template <int DT>
hipError_t launch_conv(const GenConv &g, bool tr, int NB, int ROWS, hipStream_t st) {
    const long long waves = ((long long)g.tasks + g.tpw - 1) / g.tpw;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (tr) {
        if (ROWS == 1) launch_conv_nb<true, 1, DT>(g, NB, grid, st);
        else launch_conv_nb<true, 4, DT>(g, NB, grid, st);
    } else {
        if (ROWS == 1) launch_conv_nb<false, 1, DT>(g, NB, grid, st);
        else launch_conv_nb<false, 4, DT>(g, NB, grid, st);
    }
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
    GenLayout L;
    layout(a, L);
    if ((long long)a.N * L.nph * L.Tq * L.GTn * L.cobN >= (1LL << 31) - 64) return false;
    if (L.wp_elems * L.ES >= RES_MAX) return false;
    if ((long long)a.N * a.C_out * S / GT >= (1LL << 31) - 1) return false;
    if ((long long)a.N * a.C_out * ((S + APPLY_CHUNK - 1) / APPLY_CHUNK) >= (1LL << 31) - 1)
        return false;
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

    // 1. conv (+ bias + elementwise activation).  The stride-2 3x3 transposed conv
    // over 8-channel groups has a direct kernel of its own (k_upsample2.hip); it
    // writes its own (coarser) statistics tiles, so the finalize reads Tst of them.
    // When a norm follows, that stage only takes statistics here and writes the
    // normalised output in step 4 (recomputing the conv instead of re-reading it).
    int Tst = L.T;
    const float out_scale0 = (!L.softmax && a.norm_groups == 0 && a.reduce == 0) ? a.inv_div : 1.0f;
    const bool up2 = !L.softmax && upsample2_supported(a) && upsample2_tiles(a.H, a.W) <= L.T;
    if (up2) {
        Tst = upsample2_tiles(a.H, a.W);
        e = launch_upsample2(a, y, part, Tst, out_scale0, nullptr, L.apply ? 1 : 0, st);
        if (e != hipSuccess) return e;
    } else {
        GenConv g{};
        g.x = a.x; g.b = a.b;
        void *wp = ws + L.off_wp;
        g.wp = wp;
        g.wp_elems = (unsigned)L.wp_elems;
        g.P = L.P; g.RPG = 16 / L.P; g.KPG = L.KPG; g.GTn = L.GTn; g.steps = L.steps;
        g.KP = 4 * L.KL * L.steps;
        g.y = y;
        g.part = L.softmax ? nullptr : part;
        g.C_in = a.C_in; g.C_out = a.C_out; g.G = a.groups;
        g.Cgi = a.C_in / a.groups; g.Cgo = a.C_out / a.groups;
        const int NB = L.NB;
        g.cobN = L.cobN;
        g.T = L.T;
        g.Tq = L.Tq;
        g.CT = L.CT;
        g.tasks = (int)((long long)a.N * L.nph * L.Tq * L.GTn * g.cobN);
        g.D = a.D; g.H = a.H; g.W = a.W; g.Do = a.Do; g.Ho = a.Ho; g.Wo = a.Wo; g.S = S;
        g.kd = a.kd; g.kh = a.kh; g.kw = a.kw;
        g.sd = a.sd; g.sh = a.sh; g.sw = a.sw; g.pd = a.pd; g.ph = a.ph; g.pw = a.pw;
        g.dd = a.dd; g.dh = a.dh; g.dw = a.dw;
        g.in_plane = (unsigned)a.D * a.H * a.W;
        {
            // ~256 MFMAs per wave, but at least 16K waves in flight
            const double taps_issued = (double)a.kd * a.kh * a.kw / L.nph;  // x taps all issued
            const double mfma = taps_issued * L.steps * 4.0 * NB * (a.dtype ? 0.5 : 1.0);
            long long tpw = (long long)(256.0 / (mfma > 1.0 ? mfma : 1.0));
            const long long cap = g.tasks / 16384;
            if (tpw > cap) tpw = cap;
            g.tpw = (int)(tpw < 1 ? 1 : tpw > 64 ? 64 : tpw);
        }
        {
            const unsigned total = (unsigned)L.wp_elems, blocks = (total + GT - 1) / GT;
            const int taps = a.kd * a.kh * a.kw;
            if (a.dtype)
                gen_weight_pack_kernel<unsigned short><<<dim3(blocks), dim3(GT), 0, st>>>(
                    static_cast<const unsigned short *>(a.w), static_cast<unsigned short *>(wp),
                    a.groups, g.Cgi, g.Cgo, taps, L.steps, L.P, L.KL, L.cobN, NB, a.transposed,
                    total);
            else
                gen_weight_pack_kernel<float><<<dim3(blocks), dim3(GT), 0, st>>>(
                    static_cast<const float *>(a.w), static_cast<float *>(wp), a.groups, g.Cgi,
                    g.Cgo, taps, L.steps, L.P, L.KL, L.cobN, NB, a.transposed, total);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        // the conv writes the final values when nothing follows but the divide
        g.out_scale = (!L.softmax && a.norm_groups == 0 && a.reduce == 0) ? a.inv_div : 1.0f;
        g.act = L.softmax ? ACT_NONE : a.act;
        if ((e = dominant_begin(st)) != hipSuccess) return e;
        if (a.dtype == 1) e = launch_conv<1>(g, a.transposed, NB, L.ROWS, st);
        else if (a.dtype == 2) e = launch_conv<2>(g, a.transposed, NB, L.ROWS, st);
        else e = launch_conv<0>(g, a.transposed, NB, L.ROWS, st);
        if (e != hipSuccess) return e;
        if ((e = dominant_end(st)) != hipSuccess) return e;
    }

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
            part, a.C_out, Tst, cpg, NG, a.norm_groups > 0, a.gamma, a.beta, a.eps, a.inv_div,
            a.reduce == 1 ? a.out : nullptr, ss);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // 4. in-place normalisation of the output
    if (L.apply && up2) {
        e = launch_upsample2(a, y, nullptr, Tst, 1.0f, ss, 2, st);
        if (e != hipSuccess) return e;
    } else if (L.apply && (S & 3) == 0 && S >= APPLY_CHUNK &&
               (long long)a.N * a.C_out * S / 4 < (1LL << 31) - APPLY_CHUNK) {
        const int total4 = (int)((long long)a.N * a.C_out * S / 4);
        const unsigned blocks = (unsigned)((total4 + APPLY_CHUNK / 4 - 1) / (APPLY_CHUNK / 4));
        gen_apply_flat_kernel<<<dim3(blocks), dim3(GT), 0, st>>>(a.out, ss, S / 4, total4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (L.apply) {
        const unsigned chunks = (unsigned)((S + APPLY_CHUNK - 1) / APPLY_CHUNK);
        gen_apply_kernel<<<dim3((unsigned)((long long)a.N * a.C_out * chunks)), dim3(GT), 0, st>>>(
            a.out, ss, S, (int)chunks);
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
