// k_convt2d_gn_fused.hip -- grouped ConvTranspose2d (stride 1, k = 3, 8 in /
// 8 out channels per group, W = 256) + activation + GroupNorm over the
// (sample, group) unit, with every output written to HBM exactly once.
//
// Page "Kimi-K2.6__l2_p19": ConvTranspose2d(64 -> 64, k 3, stride 1,
// groups 8) -> GELU -> GroupNorm(8), 128 x 64 x 256 x 256 -> 258 x 258.  The
// second trace weighs a three-kernel plan (conv + GELU writing the tensor and
// accumulating per-(n, g) sums with atomics, a finalize, then a normalize pass
// that re-reads the tensor); its minimum-traffic estimate is one read of x and
// one write of the output.  With conv groups == norm groups each (sample,
// group) unit is independent, so that minimum is reachable: a unit is cut
// into S row slices, each computed by one workgroup that keeps its post-
// activation values in registers, publishes a Welford triple, waits for the
// unit's other S-1 triples, merges them in a fixed order and writes the
// normalised slice once.
//
// Co-residency: the kernel is launched cooperatively (every workgroup of the
// grid is resident), and each round assigns whole units to groups of S
// consecutive workgroups, so a waiting workgroup only ever waits on resident
// ones.  The wait is bounded; if the bound is hit a flag in the workspace is
// raised and the kernel still terminates.
//
// Tile mapping (the column-pair MFMA form of the two-pass kernel): rows of a
// 16x16 result = (channel, pixel parity), columns = 16 column pairs, K =
// (ci, kh, v) with v = kw - t + 1.  An output row of 258 pixels is 8 row
// tiles (pixels 0..255) plus the last column pair (256, 257); the last pairs
// of 16 consecutive rows form one "column tile".  A slice of RS = 2 * NSTEP
// rows is NSTEP steps of 2 rows (16 row tiles, 4 per wave) plus NCT column
// tiles; the input rows stream through a 6-row LDS ring (one barrier per
// step), the column tiles read a small LDS strip of input columns 254..255.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int CG = 8;            // channels per group (in and out)
constexpr int KS = 3;
constexpr int W = 256;           // input width this kernel is built for
constexpr int WO = W + KS - 1;   // 258
constexpr int PADL = 4;          // zero columns left of x inside an LDS row
constexpr int RP = W + 2 * PADL; // 264: LDS row pitch
constexpr int RING = 6;          // input rows in the LDS ring
constexpr int THREADS = 256;
constexpr int NSTEP = 6;         // 2-row steps per slice
constexpr int RS = 2 * NSTEP;    // output rows per slice
constexpr int NCT = (RS + 15) / 16;          // column tiles per slice
constexpr int NACC = 4 * NSTEP + 1;          // accumulator tiles per wave (waves >= NCT use 4*NSTEP)
constexpr int STRIP_ROWS = 16 * NCT + KS - 1;
constexpr int RING_FLOATS = RING * CG * RP;
constexpr int STRIP_FLOATS = CG * STRIP_ROWS * 4;
constexpr int ROW4 = CG * (W / 4);           // float4 granules in one input row of the group
constexpr int PF = 2 * ROW4 / THREADS;       // per-thread float4 prefetch for 2 rows
static_assert(2 * ROW4 % THREADS == 0, "prefetch split");
constexpr int SPIN_LIMIT = 1 << 24;

struct FusedArgs {
    const float *x, *wt, *bias, *gamma, *beta;
    float *y;
    int *counters;   // [N*G], zero on entry
    int *flag;       // raised if a wait timed out
    float *partials; // [N*G][S][4]
    int N, C, H, G, Ho, S, units_per_round;
    float eps, inv_div;
};

// Prefetch slot u of a thread covers row (u * THREADS) / ROW4 of the pair (a
// compile-time value) and a lane-dependent (channel, float4 column).
__device__ __forceinline__ unsigned fetch_lane_off(int tid, int u, int H)
{
    const int rem = (tid + u * THREADS) % ROW4;
    const int ci = rem / (W / 4), c4 = rem % (W / 4);
    return (unsigned)((ci * H * W + 4 * c4) * 4);
}

// x rows gr0, gr0+1 of the group's 8 channels -> registers (zero outside [0, H))
__device__ __forceinline__ void fetch_rows(__amdgpu_buffer_rsrc_t xr, int H, int gr0,
                                           const unsigned (&loff)[PF], v4f (&pf)[PF])
{
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int rr = (u * THREADS) / ROW4;
        const int gr = gr0 + rr;
        const bool ok = gr >= 0 && gr < H;  // uniform
        const v4f v = buf_load4(xr, loff[u], (unsigned)((ok ? gr : 0) * W * 4));
        pf[u] = ok ? v : v4f{0.f, 0.f, 0.f, 0.f};
    }
}

__device__ __forceinline__ void stash_rows(float *ring, int slot0, int tid, const v4f (&pf)[PF])
{
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int e = tid + u * THREADS;
        const int rr = e / ROW4, rem = e % ROW4;
        const int ci = rem / (W / 4), c4 = rem % (W / 4);
        const int slot = (slot0 + rr) % RING;
        *reinterpret_cast<v4f *>(ring + (slot * CG + ci) * RP + PADL + 4 * c4) = pf[u];
    }
}

template <int ACT>
__global__ __launch_bounds__(THREADS, 2)
void convt2d_gn_fused_kernel(FusedArgs a)
{
    __shared__ float ring[RING_FLOATS];
    __shared__ float strip[STRIP_FLOATS];
    __shared__ float red[16];  // [4 waves][3] triples, then mean and rstd at [12], [13]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c16 = lane & 15;
    const int H = a.H, Ho = a.Ho, S = a.S;
    const int slice = blockIdx.x % S, ulocal = blockIdx.x / S;
    const int U = a.N * a.G;
    const int r0 = slice * RS;
    const int rs = min(RS, Ho - r0);   // rows of this slice (>= 1)
    const size_t plane_o = (size_t)Ho * WO;
    unsigned loff[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) loff[u] = fetch_lane_off(tid, u, H);

    // zero padding columns of the ring rows once (never overwritten)
    for (int e = tid; e < RING * CG; e += THREADS) {
        float *row = ring + e * RP;
#pragma unroll
        for (int c = 0; c < PADL; ++c) { row[c] = 0.f; row[PADL + W + c] = 0.f; }
    }

    for (int round = 0;; ++round) {
        const int unit = round * a.units_per_round + ulocal;
        if (unit >= U) break;
        const int n = unit / a.G, g = unit % a.G;
        const float *xg = a.x + ((size_t)n * a.C + (size_t)g * CG) * H * W;
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(xg, (unsigned)(CG * H * W * 4));
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wt + (size_t)g * CG * CG * KS * KS,
                                                    CG * CG * KS * KS * 4);

        // ---- weights (A operand), bias, affine for channels 2q, 2q+1
        float wreg[CG * KS];
        {
            const int co = c16 >> 1, t = c16 & 1;
            const int kw = q + t - 1;
#pragma unroll
            for (int s = 0; s < CG * KS; ++s) {
                const int ci = s / KS, kh = s % KS;
                const float v = buf_load1(
                    wr, (unsigned)((((ci * CG + co) * KS + kh) * KS + (kw >= 0 && kw < KS ? kw : 0)) * 4));
                wreg[s] = (kw >= 0 && kw < KS) ? v : 0.0f;
            }
        }
        const int ch0 = g * CG + 2 * q;
        const float b0 = a.bias ? a.bias[ch0] : 0.0f, b1 = a.bias ? a.bias[ch0 + 1] : 0.0f;

        // ---- stage: column strip (x cols 254, 255; 256, 257 are zero) and ring rows r0-2 .. r0+1
        __syncthreads();  // the previous round's readers of ring/strip are done
        {
            // issue every staging load first (one memory round trip), then write LDS
            v4f pa[PF], pb[PF];
            fetch_rows(xr, H, r0 - 2, loff, pa);
            fetch_rows(xr, H, r0, loff, pb);
            constexpr int SE = (CG * STRIP_ROWS + THREADS - 1) / THREADS;
            float sv[SE][2];
#pragma unroll
            for (int u = 0; u < SE; ++u) {
                const int e = tid + u * THREADS;
                const int ci = e / STRIP_ROWS, rr = e % STRIP_ROWS;
                const int gr = r0 - (KS - 1) + rr;
                const bool ok = e < CG * STRIP_ROWS && gr >= 0 && gr < H;
                const unsigned off = ok ? (unsigned)(((ci * H + gr) * W + (W - 2)) * 4) : 0u;
                const float v0 = buf_load1(xr, off), v1 = buf_load1(xr, off + 4);
                sv[u][0] = ok ? v0 : 0.0f;
                sv[u][1] = ok ? v1 : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < SE; ++u) {
                const int e = tid + u * THREADS;
                if (e < CG * STRIP_ROWS) {
                    float *dst = strip + e * 4;  // (ci, row) major, 4 columns
                    dst[0] = sv[u][0]; dst[1] = sv[u][1]; dst[2] = 0.f; dst[3] = 0.f;
                }
            }
            stash_rows(ring, 0, tid, pa);
            stash_rows(ring, 2, tid, pb);
        }

        v4f acc[NACC];
        float s1 = 0.f, s2 = 0.f;
        int cnt = 0;
        // Row tile i = wave + 4j of a step: output row 2k + (j >> 1), column block
        // rt = wave + 4 (j & 1) (wave < 4).  LDS column of x column (2 pc + 1 - v)
        // for pair pc = 16 rt + c16, v = q, is lb + 128 (j & 1).
        const int lb = 2 * c16 + 1 - q + PADL + 32 * wave;

#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
            __syncthreads();  // ring rows r0+2k-2 .. r0+2k+1 are in place
            if (2 * k < rs) {  // workgroup-uniform
                v4f pf[PF];
                const bool more = k + 1 < NSTEP && 2 * k + 2 < rs;
                if (more) fetch_rows(xr, H, r0 + 2 * k + 2, loff, pf);
                // 4 row tiles per wave, interleaved so each LDS read has 3 MFMAs of slack
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[4 * k + j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ci = 0; ci < CG; ++ci) {
#pragma unroll
                    for (int kh = 0; kh < KS; ++kh) {
                        float bv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int orow = 2 * k + (j >> 1);  // slice-relative output row
                            // input row orow - kh (slice-relative) lives in slot (orow - kh + 2) % RING
                            const int slot = (orow - kh + 2) % RING;
                            bv[j] = ring[lb + (slot * CG + ci) * RP + 128 * (j & 1)];
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[4 * k + j] = mfma_16x16x4(wreg[ci * KS + kh], bv[j], acc[4 * k + j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int orow = 2 * k + (j >> 1);
                    v4f c = acc[4 * k + j];
                    c[0] = activate<ACT>(c[0] + b0);
                    c[1] = activate<ACT>(c[1] + b0);
                    c[2] = activate<ACT>(c[2] + b1);
                    c[3] = activate<ACT>(c[3] + b1);
                    if (orow < rs) {
                        s1 += (c[0] + c[1]) + (c[2] + c[3]);
                        s2 = fmaf(c[0], c[0], s2); s2 = fmaf(c[1], c[1], s2);
                        s2 = fmaf(c[2], c[2], s2); s2 = fmaf(c[3], c[3], s2);
                        cnt += 4;
                    }
                    acc[4 * k + j] = c;
                }
                if (more) stash_rows(ring, (2 * k + 4) % RING, tid, pf);
            }
        }

        // ---- column tiles: pair 128 of rows 16*ct + c16, read from the strip
        if (wave < NCT) {
            const int ct = wave;
            const int orow = 16 * ct + c16;
            v4f c = v4f{0.f, 0.f, 0.f, 0.f};
            // x row orow - kh -> strip row orow - kh + 2; x col 257 - q -> strip col 3 - q
#pragma unroll
            for (int ci = 0; ci < CG; ++ci) {
#pragma unroll
                for (int kh = 0; kh < KS; ++kh) {
                    const float bv = strip[(ci * STRIP_ROWS + orow + 2 - kh) * 4 + 3 - q];
                    c = mfma_16x16x4(wreg[ci * KS + kh], bv, c);
                }
            }
            c[0] = activate<ACT>(c[0] + b0);
            c[1] = activate<ACT>(c[1] + b0);
            c[2] = activate<ACT>(c[2] + b1);
            c[3] = activate<ACT>(c[3] + b1);
            if (orow < rs) {
                s1 += (c[0] + c[1]) + (c[2] + c[3]);
                s2 = fmaf(c[0], c[0], s2); s2 = fmaf(c[1], c[1], s2);
                s2 = fmaf(c[2], c[2], s2); s2 = fmaf(c[3], c[3], s2);
                cnt += 4;
            }
            acc[4 * NSTEP] = c;
        }

        // ---- slice statistics -> one Welford triple
        float fn = (float)cnt;
        float mean = cnt ? s1 / fn : 0.0f;
        float m2 = cnt ? fmaxf(s2 - s1 * mean, 0.0f) : 0.0f;
        row_chan16(fn, mean, m2);
#pragma unroll
        for (int sh = 16; sh <= 32; sh <<= 1) {
            const float nb = __shfl_xor(fn, sh, 64), mb = __shfl_xor(mean, sh, 64),
                        qb = __shfl_xor(m2, sh, 64);
            chan_merge(fn, mean, m2, nb, mb, qb);
        }
        __syncthreads();  // every wave is done with the ring and with last round's red[]
        if (lane == 0) { red[wave * 3] = fn; red[wave * 3 + 1] = mean; red[wave * 3 + 2] = m2; }
        __syncthreads();
        if (tid == 0) {
            float c2 = 0.f, m = 0.f, q2 = 0.f;
            for (int k = 0; k < 4; ++k) chan_merge(c2, m, q2, red[k * 3], red[k * 3 + 1], red[k * 3 + 2]);
            float *pp = a.partials + ((size_t)unit * S + slice) * 4;
            __hip_atomic_store(pp + 0, c2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pp + 1, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pp + 2, q2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            // Spin with coherent relaxed loads (an acquire load per iteration would
            // invalidate this XCD's L2 every time); the partials are then read with
            // coherent loads, which the counter value orders after their stores.
            int it = 0;
            while (__hip_atomic_load(a.counters + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < S) {
                if (++it > SPIN_LIMIT) {
                    __hip_atomic_store(a.flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
        // read the unit's S triples in parallel (coherent loads), merge in slice order
        __syncthreads();
        if (wave == 0) {
            const int u0 = unit;
            for (int s0 = 0; s0 < S; s0 += 64) {
                const int sl = s0 + lane;
                if (sl < S) {
                    const float *ps = a.partials + ((size_t)u0 * S + sl) * 4;
                    // the strip is free until the next round re-stages it
                    strip[sl * 3 + 0] = __hip_atomic_load(ps + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    strip[sl * 3 + 1] = __hip_atomic_load(ps + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    strip[sl * 3 + 2] = __hip_atomic_load(ps + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        __syncthreads();
        if (tid == 0) {
            float uc = 0.f, um = 0.f, uq = 0.f;
            for (int sl = 0; sl < S; ++sl) chan_merge(uc, um, uq, strip[sl * 3], strip[sl * 3 + 1], strip[sl * 3 + 2]);
            red[12] = um;
            red[13] = rsqrtf(uq / uc + a.eps);
        }
        __syncthreads();
        const float mu = red[12], rstd = red[13];
        const float ga0 = a.gamma ? a.gamma[ch0] : 1.0f, be0 = a.beta ? a.beta[ch0] : 0.0f;
        const float ga1 = a.gamma ? a.gamma[ch0 + 1] : 1.0f, be1 = a.beta ? a.beta[ch0 + 1] : 0.0f;
        const float sc0 = rstd * ga0 * a.inv_div, sh0 = (be0 - mu * rstd * ga0) * a.inv_div;
        const float sc1 = rstd * ga1 * a.inv_div, sh1 = (be1 - mu * rstd * ga1) * a.inv_div;

        // ---- normalise in registers and write once (streaming stores)
        const __amdgpu_buffer_rsrc_t yr =
            make_rsrc(a.y + ((size_t)n * a.C + (size_t)g * CG) * plane_o,
                      (unsigned)(CG * plane_o * 4));
        const unsigned yo0 = (unsigned)(2 * q) * (unsigned)plane_o * 4u;
        const unsigned yo1 = yo0 + (unsigned)plane_o * 4u;
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int orow = 2 * k + (j >> 1);
                if (orow < rs) {
                    const v4f c = acc[4 * k + j];
                    const unsigned uo = (unsigned)((r0 + orow) * WO + 32 * (wave + 4 * (j & 1))) * 4u;  // uniform
                    buf_store2_nt(v2f{c[0] * sc0 + sh0, c[1] * sc0 + sh0}, yr, yo0 + 8u * c16, uo);
                    buf_store2_nt(v2f{c[2] * sc1 + sh1, c[3] * sc1 + sh1}, yr, yo1 + 8u * c16, uo);
                }
            }
        }
        if (wave < NCT) {
            const int orow = 16 * wave + c16;
            if (orow < rs) {
                const v4f c = acc[4 * NSTEP];
                const unsigned o = (unsigned)((r0 + orow) * WO + W) * 4u;
                buf_store2_nt(v2f{c[0] * sc0 + sh0, c[1] * sc0 + sh0}, yr, yo0 + o);
                buf_store2_nt(v2f{c[2] * sc1 + sh1, c[3] * sc1 + sh1}, yr, yo1 + o);
            }
        }
    }
}

__global__ void zero_ints_kernel(int *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

struct Occupancy {
    int device = -1;
    int blocks_per_cu[4] = {0, 0, 0, 0};
    int cus = 0;
};

template <int ACT>
hipError_t launch_t(const ConvT2dArgs &p, int slices, hipStream_t st)
{
    static Occupancy occ[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Occupancy &o = occ[dev & 63];
    if (o.device != dev || o.blocks_per_cu[ACT] == 0) {
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, convt2d_gn_fused_kernel<ACT>,
                                                         THREADS, 0);
        if (e != hipSuccess) return e;
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        o.device = dev;
        o.blocks_per_cu[ACT] = nb;
        o.cus = cus;
    }
    if (slices * 3 > STRIP_FLOATS) return hipErrorInvalidValue;  // partial triples are merged in the strip
    const int resident = o.blocks_per_cu[ACT] * o.cus;
    const int U = p.N * p.groups;
    int upr = resident / slices;
    if (upr < 1) return hipErrorCooperativeLaunchTooLarge;
    if (upr > U) upr = U;

    // workspace: [U] counters, flag, pad to 16 B, then [U][S][4] partials
    int *counters = reinterpret_cast<int *>(p.partials);
    int *flag = counters + U;
    float *partials = p.partials + ((U + 1 + 3) & ~3);
    hipLaunchKernelGGL(zero_ints_kernel, dim3((U + 1 + 255) / 256), dim3(256), 0, st, counters,
                       U + 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    FusedArgs fa{p.x, p.w, p.b, p.gamma, p.beta, p.out, counters, flag, partials,
                 p.N, p.C_out, p.H, p.groups, p.Ho, slices, upr, p.eps, p.inv_div};
    void *args[] = {&fa};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(convt2d_gn_fused_kernel<ACT>),
                                      dim3(upr * slices), dim3(THREADS), args, 0, st);
}

}  // namespace

int convt2d_fused_slices(int Ho) { return (Ho + RS - 1) / RS; }

bool convt2d_fused_supported(int C_in, int C_out, int groups, int H, int W_, int act, int norm,
                             int num_groups)
{
    return W_ == W && C_in == CG * groups && C_out == CG * groups && H >= 1 &&
           norm == 1 /* group */ && num_groups == groups &&
           (act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF);
}

size_t convt2d_fused_workspace(int N, int groups, int Ho)
{
    const size_t U = (size_t)N * groups;
    return (((U + 1 + 3) & ~(size_t)3) + U * convt2d_fused_slices(Ho) * 4) * sizeof(float);
}

hipError_t launch_convt2d_fused(const ConvT2dArgs &a, hipStream_t st)
{
    const int S = convt2d_fused_slices(a.Ho);
    switch (a.act) {
    case ACT_NONE: return launch_t<ACT_NONE>(a, S, st);
    case ACT_HARDSWISH: return launch_t<ACT_HARDSWISH>(a, S, st);
    case ACT_GELU_ERF: return launch_t<ACT_GELU_ERF>(a, S, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cnf
