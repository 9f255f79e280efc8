// k_convt2d_gn_fused.hip -- grouped ConvTranspose2d (stride 1, k = 3, 8 in /
// 8 out channels per group, W = 256) + activation + GroupNorm over each
// (sample, group) unit in ONE persistent, cooperative kernel.
//
// Page "Kimi-K2.6__l2_p19": ConvTranspose2d(64 -> 64, k 3, stride 1,
// groups 8) -> GELU -> GroupNorm(8), 128 x 64 x 256 x 256 -> 258 x 258.  The
// second trace weighs a three-kernel plan: conv + GELU writing the tensor and
// accumulating per-(n, g) sums, a finalize, then a normalize pass that
// re-reads the tensor.  Here the three steps run inside one kernel and are
// pipelined so that the re-read is a cache hit and nothing waits:
//   * a unit is cut into S row slices; a group of S workgroups owns one unit
//     per round (units handed out round by round; the grid is launched
//     cooperatively, so every workgroup of a group is resident);
//   * round r: each workgroup computes its slice of unit u_r (conv + bias +
//     activation), writes it to y and publishes a Welford triple of the slice
//     (release + a per-unit arrival counter);
//   * interleaved with round r's compute, the same workgroup normalises its
//     slice of u_{r-1} in place: the other S-1 slices of u_{r-1} were
//     published a round earlier, so the wait is almost always empty, and the
//     slice it rewrites is the one it wrote a round ago, still in L2 or the
//     MALL;
//   * after the last round the last unit is normalised on its own.
// The wait is bounded; on time-out a flag in the workspace is raised and the
// kernel still terminates.  Statistics are merged in slice order, so results
// do not depend on timing.
//
// Tile mapping: rows of a 16x16 MFMA result = (channel, pixel parity),
// columns = 16 column pairs, K = (ci, kh, v = kw - t + 1): pixels (2p, 2p+1)
// read the same input columns shifted by one, so 72 of every 96 K entries are
// useful (zero-padded weights fill the rest).  An output row of 258 pixels is
// 8 row tiles (pixels 0..255) plus the last column pair; the last pairs of 16
// consecutive rows form one column tile.  A slice is a loop of 2-row steps
// (16 row tiles, 4 per wave, interleaved) over a 6-row LDS ring of input rows
// (one barrier per step), plus column tiles read from a small LDS strip of
// input columns 254..255.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int CG = 8;            // channels per group (in and out)
constexpr int KS = 3;
constexpr int W = 256;           // input width this kernel is built for
constexpr int WO = W + KS - 1;   // 258
constexpr int PAIRS = WO / 2;    // 129 column pairs per output row
constexpr int PADL = 4;          // zero columns left of x inside an LDS row
constexpr int RP = W + 2 * PADL; // 264: LDS row pitch
constexpr int RING = 6;          // input rows in the LDS ring
constexpr int THREADS = 256;
constexpr int RS = 26;           // output rows per slice
constexpr int NCT = (RS + 15) / 16;           // column tiles per slice
constexpr int STRIP_ROWS = 16 * NCT + KS - 1;
constexpr int RING_FLOATS = RING * CG * RP;
constexpr int STRIP_FLOATS = CG * STRIP_ROWS * 4;
constexpr int ROW4 = CG * (W / 4);            // float4 granules in one input row of the group
constexpr int PF = 2 * ROW4 / THREADS;        // per-thread float4 prefetch for 2 rows
constexpr int SE = (CG * STRIP_ROWS + THREADS - 1) / THREADS;
constexpr int FIX_PER_STEP = 2 * CG * PAIRS;  // float2 elements per step of the fix-up
constexpr int FCT = (FIX_PER_STEP + THREADS - 1) / THREADS;
constexpr int MAX_S = 32;                     // slices per unit the merge buffer holds
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

__device__ __forceinline__ unsigned fetch_lane_off(int tid, int u, int H)
{
    const int rem = (tid + u * THREADS) % ROW4;
    const int ci = rem / (W / 4), c4 = rem % (W / 4);
    return (unsigned)((ci * H * W + 4 * c4) * 4);
}

// x rows gr0, gr0+1 of the group's 8 channels -> registers (zero outside [0, H)).
// Slot u covers row (u * THREADS) / ROW4 of the pair.
__device__ __forceinline__ void fetch_rows(__amdgpu_buffer_rsrc_t xr, int H, int gr0,
                                           const unsigned (&loff)[PF], v4f (&pf)[PF])
{
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int gr = gr0 + (u * THREADS) / ROW4;
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

// Staging of one unit's slice: ring rows r0-2 .. r0+1 and the column strip.
struct Stage {
    v4f pa[PF], pb[PF];
    float sv[SE][2];
};

__device__ __forceinline__ void stage_load(Stage &st, __amdgpu_buffer_rsrc_t xr, int H, int r0,
                                           int tid, const unsigned (&loff)[PF])
{
    fetch_rows(xr, H, r0 - 2, loff, st.pa);
    fetch_rows(xr, H, r0, loff, st.pb);
#pragma unroll
    for (int u = 0; u < SE; ++u) {
        const int e = tid + u * THREADS;
        const int ci = e / STRIP_ROWS, rr = e % STRIP_ROWS;
        const int gr = r0 - (KS - 1) + rr;
        const bool ok = e < CG * STRIP_ROWS && gr >= 0 && gr < H;
        const unsigned off = ok ? (unsigned)(((ci * H + gr) * W + (W - 2)) * 4) : 0u;
        const float v0 = buf_load1(xr, off), v1 = buf_load1(xr, off + 4);
        st.sv[u][0] = ok ? v0 : 0.0f;
        st.sv[u][1] = ok ? v1 : 0.0f;
    }
}

__device__ __forceinline__ void stage_store(const Stage &st, float *ring, float *strip, int tid)
{
#pragma unroll
    for (int u = 0; u < SE; ++u) {
        const int e = tid + u * THREADS;
        if (e < CG * STRIP_ROWS) {
            float *dst = strip + e * 4;  // (ci, row) major; columns x254, x255, 0, 0
            dst[0] = st.sv[u][0]; dst[1] = st.sv[u][1]; dst[2] = 0.f; dst[3] = 0.f;
        }
    }
    stash_rows(ring, 0, tid, st.pa);
    stash_rows(ring, 2, tid, st.pb);
}

struct Unit {
    int n, g;
    __amdgpu_buffer_rsrc_t xr, yr;
};

__device__ __forceinline__ Unit unit_of(const FusedArgs &a, int unit, unsigned plane_o)
{
    Unit u;
    u.n = unit / a.G;
    u.g = unit % a.G;
    const size_t cbase = (size_t)u.n * a.C + (size_t)u.g * CG;
    u.xr = make_rsrc(a.x + cbase * a.H * W, (unsigned)(CG * a.H * W * 4));
    u.yr = make_rsrc(a.y + cbase * plane_o, CG * plane_o * 4u);
    return u;
}

// Fix-up (in-place normalisation) of the previous unit's slice: float2
// elements e = (ch * rs + row) * PAIRS + pair, a chunk [base, base + chunk)
// at a time, loads first so the chunk can overlap with MFMA work.
struct Fix {
    v2f v[FCT];
    unsigned off[FCT];
    int ch[FCT];
};

__device__ __forceinline__ void fix_load(Fix &f, __amdgpu_buffer_rsrc_t yr, int base, int chunk,
                                         int total, int tid, int rs, unsigned rs_magic, int r0,
                                         unsigned plane_o)
{
#pragma unroll
    for (int i = 0; i < FCT; ++i) {
        const int e = base + tid + i * THREADS;
        const bool ok = e < base + chunk && e < total;
        const int ee = ok ? e : 0;
        const int rowg = ee / PAIRS, c2 = ee - rowg * PAIRS;      // rowg = ch * rs + row
        const int ch = (int)(((unsigned)rowg * rs_magic) >> 16);  // exact for rowg < 8 rs
        const int row = rowg - ch * rs;
        f.ch[i] = ok ? ch : -1;
        f.off[i] = ((unsigned)ch * plane_o + (unsigned)(r0 + row) * WO + 2u * c2) * 4u;
        f.v[i] = __builtin_bit_cast(v2f, __builtin_amdgcn_raw_buffer_load_b64(yr, (int)f.off[i], 0, 0));
    }
}

__device__ __forceinline__ void fix_store(const Fix &f, __amdgpu_buffer_rsrc_t yr,
                                          const float (*coef)[2])
{
#pragma unroll
    for (int i = 0; i < FCT; ++i) {
        if (f.ch[i] >= 0) {
            const float sc = coef[f.ch[i]][0], sh = coef[f.ch[i]][1];
            buf_store2_nt(v2f{f.v[i][0] * sc + sh, f.v[i][1] * sc + sh}, yr, f.off[i]);
        }
    }
}

template <int ACT>
__global__ __launch_bounds__(THREADS, 2)
void convt2d_gn_fused_kernel(FusedArgs a)
{
    __shared__ float ring[RING_FLOATS];
    __shared__ float strip[STRIP_FLOATS];
    __shared__ float mrg[MAX_S * 3];
    __shared__ float red[12];   // [4 waves][3] slice triple
    __shared__ float coef[CG][2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c16 = lane & 15;
    const int H = a.H, Ho = a.Ho, S = a.S;
    const int slice = blockIdx.x % S, ulocal = blockIdx.x / S;
    const int U = a.N * a.G;
    const int r0 = slice * RS;
    const int rs = min(RS, Ho - r0);   // rows of this slice (>= 1)
    const int nsteps = (rs + 1) >> 1;
    const unsigned plane_o = (unsigned)Ho * WO;
    const int fix_total = CG * rs * PAIRS;
    const int fix_chunk = (fix_total + nsteps - 1) / nsteps;            // <= FIX_PER_STEP
    const unsigned rs_magic = (65536u + (unsigned)rs - 1u) / (unsigned)rs;  // ceil(2^16 / rs)

    for (int e = tid; e < RING * CG; e += THREADS) {  // zero pad columns, never overwritten
        float *row = ring + e * RP;
#pragma unroll
        for (int c = 0; c < PADL; ++c) { row[c] = 0.f; row[PADL + W + c] = 0.f; }
    }
    unsigned loff[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) loff[u] = fetch_lane_off(tid, u, H);
    // LDS column of x column (2 pc + 1 - v), pair pc = 16 rt + c16, v = q,
    // rt = wave + 4 (j & 1) for row tile j of a step (+128 floats for j & 1)
    const int lb = 2 * c16 + 1 - q + PADL + 32 * wave;
    const int ch_lo = 2 * q;  // this lane's channels in a tile result: ch_lo, ch_lo + 1

    int prev = -1;
    Unit pu{};
    Stage st;
    bool staged = false;
    for (int round = 0;; ++round) {
        const int unit = round * a.units_per_round + ulocal;
        const bool cur = unit < U;

        // ---- statistics of the previous unit -> per-channel scale / shift in LDS
        if (prev >= 0) {
            if (tid == 0) {
                // Spin with coherent relaxed loads (an acquire load per iteration
                // would invalidate this XCD's L2 every time); the triples are then
                // read with coherent loads, ordered after the counter read.
                int it = 0;
                while (__hip_atomic_load(a.counters + prev, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) < S) {
                    if (++it > SPIN_LIMIT) {
                        __hip_atomic_store(a.flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            }
            __syncthreads();
            if (tid < S) {
                const float *ps = a.partials + ((size_t)prev * S + tid) * 4;
                mrg[tid * 3 + 0] = __hip_atomic_load(ps + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                mrg[tid * 3 + 1] = __hip_atomic_load(ps + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                mrg[tid * 3 + 2] = __hip_atomic_load(ps + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            if (tid < CG) {
                float uc = 0.f, um = 0.f, uq = 0.f;
                for (int s = 0; s < S; ++s) chan_merge(uc, um, uq, mrg[s * 3], mrg[s * 3 + 1], mrg[s * 3 + 2]);
                const float rstd = rsqrtf(uq / uc + a.eps);
                const int c = pu.g * CG + tid;
                const float ga = a.gamma ? a.gamma[c] : 1.0f, be = a.beta ? a.beta[c] : 0.0f;
                coef[tid][0] = rstd * ga * a.inv_div;
                coef[tid][1] = (be - um * rstd * ga) * a.inv_div;
            }
            // the next barrier publishes coef
        }

        if (!cur) {
            // no unit this round: normalise the previous one on its own
            if (prev >= 0) {
                __syncthreads();
                for (int base = 0; base < fix_total; base += fix_chunk) {
                    Fix f;
                    fix_load(f, pu.yr, base, fix_chunk, fix_total, tid, rs, rs_magic, r0, plane_o);
                    fix_store(f, pu.yr, coef);
                }
            }
            break;
        }

        const Unit cu = unit_of(a, unit, plane_o);
        // ---- weights (A operand) and bias for this unit's group
        float wreg[CG * KS];
        {
            const __amdgpu_buffer_rsrc_t wr =
                make_rsrc(a.wt + (size_t)cu.g * CG * CG * KS * KS, CG * CG * KS * KS * 4);
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
        const int ch0 = cu.g * CG + ch_lo;
        const float b0 = a.bias ? a.bias[ch0] : 0.0f, b1 = a.bias ? a.bias[ch0 + 1] : 0.0f;
        const unsigned yo0 = (unsigned)ch_lo * plane_o * 4u, yo1 = yo0 + plane_o * 4u;

        if (!staged) stage_load(st, cu.xr, H, r0, tid, loff);
        __syncthreads();  // last round's readers of ring / strip are done; coef is published
        stage_store(st, ring, strip, tid);
        staged = false;

        float s1 = 0.f, s2 = 0.f;
        int cnt = 0;
        for (int k = 0; k < nsteps; ++k) {
            __syncthreads();  // ring rows r0+2k-2 .. r0+2k+1 are in place
            v4f pf[PF];
            const bool more = k + 1 < nsteps;
            if (more) fetch_rows(cu.xr, H, r0 + 2 * k + 2, loff, pf);
            Fix f;
            if (prev >= 0)
                fix_load(f, pu.yr, k * fix_chunk, fix_chunk, fix_total, tid, rs, rs_magic, r0, plane_o);

            // slice-relative input row 2k - 2 + m lives in slot (2k + m) % RING
            int sb[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) sb[m] = lb + ((2 * k + m) % RING) * CG * RP;
            v4f acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ci = 0; ci < CG; ++ci) {
#pragma unroll
                for (int kh = 0; kh < KS; ++kh) {
                    float bv[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        bv[j] = ring[sb[(j >> 1) - kh + 2] + ci * RP + 128 * (j & 1)];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = mfma_16x16x4(wreg[ci * KS + kh], bv[j], acc[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int orow = 2 * k + (j >> 1);
                if (orow < rs) {
                    v4f c = acc[j];
                    c[0] = activate<ACT>(c[0] + b0);
                    c[1] = activate<ACT>(c[1] + b0);
                    c[2] = activate<ACT>(c[2] + b1);
                    c[3] = activate<ACT>(c[3] + b1);
                    s1 += (c[0] + c[1]) + (c[2] + c[3]);
                    s2 = fmaf(c[0], c[0], s2); s2 = fmaf(c[1], c[1], s2);
                    s2 = fmaf(c[2], c[2], s2); s2 = fmaf(c[3], c[3], s2);
                    cnt += 4;
                    const unsigned uo = (unsigned)((r0 + orow) * WO + 32 * (wave + 4 * (j & 1))) * 4u;
                    const unsigned lo = 8u * c16;
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v2f{c[0], c[1]}),
                                                          cu.yr, (int)(yo0 + lo), (int)uo, 0);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v2f{c[2], c[3]}),
                                                          cu.yr, (int)(yo1 + lo), (int)uo, 0);
                }
            }
            if (prev >= 0) fix_store(f, pu.yr, coef);
            if (more) stash_rows(ring, (2 * k + 4) % RING, tid, pf);
        }

        // ---- column tiles: pair 128 of rows 16 ct + c16, read from the strip
        if (wave < NCT) {
            const int orow = 16 * wave + c16;
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
            if (orow < rs) {
                c[0] = activate<ACT>(c[0] + b0);
                c[1] = activate<ACT>(c[1] + b0);
                c[2] = activate<ACT>(c[2] + b1);
                c[3] = activate<ACT>(c[3] + b1);
                s1 += (c[0] + c[1]) + (c[2] + c[3]);
                s2 = fmaf(c[0], c[0], s2); s2 = fmaf(c[1], c[1], s2);
                s2 = fmaf(c[2], c[2], s2); s2 = fmaf(c[3], c[3], s2);
                cnt += 4;
                const unsigned o = (unsigned)((r0 + orow) * WO + W) * 4u;
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v2f{c[0], c[1]}),
                                                      cu.yr, (int)(yo0 + o), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v2f{c[2], c[3]}),
                                                      cu.yr, (int)(yo1 + o), 0, 0);
            }
        }

        // ---- publish the slice's Welford triple
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
        if (lane == 0) { red[wave * 3] = fn; red[wave * 3 + 1] = mean; red[wave * 3 + 2] = m2; }
        __syncthreads();
        if (tid == 0) {
            float c2 = 0.f, m = 0.f, q2 = 0.f;
            for (int w4 = 0; w4 < 4; ++w4) chan_merge(c2, m, q2, red[w4 * 3], red[w4 * 3 + 1], red[w4 * 3 + 2]);
            float *pp = a.partials + ((size_t)unit * S + slice) * 4;
            __hip_atomic_store(pp + 0, c2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pp + 1, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pp + 2, q2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        // fetch the next unit's staging rows while the other slices finish
        {
            const int nxt = unit + a.units_per_round;
            if (nxt < U) {
                const Unit nu = unit_of(a, nxt, plane_o);
                stage_load(st, nu.xr, H, r0, tid, loff);
                staged = true;
            }
        }
        prev = unit;
        pu = cu;
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
    if (slices > MAX_S) return hipErrorInvalidValue;
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
           convt2d_fused_slices(H + KS - 1) <= MAX_S && norm == 1 /* group */ &&
           num_groups == groups &&
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
