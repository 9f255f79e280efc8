// k_convt2d_gn_fused.hip -- grouped ConvTranspose2d (stride 1, k = 3, 8 in /
// 8 out channels per group, W = 256) + activation + GroupNorm over each
// (sample, group) unit in ONE persistent, cooperative kernel that writes the
// output exactly once.
//
// Page "Kimi-K2.6__l2_p19": ConvTranspose2d(64 -> 64, k 3, stride 1,
// groups 8) -> GELU -> GroupNorm(8), 128 x 64 x 256 x 256 -> 258 x 258.  Its
// second trace weighs a three-kernel plan (conv + GELU writing the tensor and
// per-(n, g) sums, a finalize, a normalize pass re-reading the tensor).  Here
// the conv output never goes to memory un-normalised:
//   * a unit (sample, group) is cut into S row slices; S workgroups own one
//     unit per round (units handed out round by round; the launch is
//     cooperative, so all workgroups are resident at once);
//   * round r: a workgroup computes its slice of unit u_r (conv + bias +
//     activation) into an LDS bank (each lane's own values, so no barrier),
//     keeps running sums, and at the start of round r+1 publishes the
//     slice's (count, mean, M2) triple;
//   * during round r+1 the same workgroup normalises the bank of u_r and
//     stores it, one step behind its new MFMA work: the coefficients of u_r
//     are needed one step into round r+1, by which time the sibling slices
//     have normally published.  Step k of round rho lives in bank slot
//     (k - rho) mod 6, so step k of round r+1 overwrites exactly the slot of
//     step k-1 of round r, which it has just normalised and stored.
// Each triple travels as two 64-bit relaxed atomics that both carry the
// count, so a reader that sees both halves non-zero has the whole triple and
// no fence or counter is needed.  The wait is bounded; on time-out a flag in
// the workspace is raised and the kernel still terminates.  Triples are
// merged in slice order, so results do not depend on timing.
//
// Tile mapping: rows of a 16x16 MFMA result = (channel, pixel parity),
// columns = 16 column pairs, K = (ci, kh, v = kw - t + 1): pixels (2p, 2p+1)
// read the same input columns shifted by one, so 72 of every 96 K entries are
// useful (zero-padded weights fill the rest).  An output row of 258 pixels is
// 8 row tiles (pixels 0..255, one per wave) plus the last column pair; the
// last pairs of 16 consecutive rows form one column tile.  A slice is a run
// of 2-row steps; each step reads two input row pairs from a 3-pair LDS ring
// that is refilled from registers loaded three events ahead.  Each step's
// activation and sums run interleaved with the next step's MFMAs.
#include "device.h"
#include "kernels.h"

namespace cnf {

namespace {

constexpr int CG = 8;              // channels per group (in and out)
constexpr int KS = 3;
constexpr int W = 256;             // input width this kernel is built for
constexpr int WO = W + KS - 1;     // 258
constexpr int PADL = 4;            // zero columns left of x inside an LDS row
constexpr int RP = W + PADL;       // 260: LDS row pitch (reads never pass column W - 1)
constexpr int THREADS = 512;
constexpr int NWAVE = THREADS / 64;          // one 32-pixel row tile per wave
constexpr int NSLOT = 3;                     // input row pairs in the LDS ring
constexpr int PAIR_FLOATS = 2 * CG * RP;
constexpr int MAXST = 5;                     // steps per slice
constexpr int NEV = MAXST + 1;               // ring events per round (fixed)
constexpr int NBANK = MAXST + 1;             // LDS bank slots (one step of two rounds overlap)
constexpr int MAX_S = 32;                    // slices per unit
constexpr int STRIP_ROWS = 16 + KS - 1;      // input rows behind one column tile
constexpr int STRIP_ELEMS = CG * STRIP_ROWS; // (ci, row) entries of x columns 254..255
constexpr int COLWAVE = NWAVE - 1;           // wave that owns the column tile
constexpr int SPIN_LIMIT = 1 << 16;   // polls (each a memory round trip) before giving up
static_assert(NWAVE * 32 == W, "one row tile per wave");
static_assert(CG * 64 == THREADS, "one (channel, 64 float4) row chunk per wave");
static_assert(STRIP_ELEMS <= THREADS, "strip staging");

struct FusedArgs {
    const float *x, *wt, *bias, *gamma, *beta;
    float *y;
    float *partials;  // [U][S][4]: (count, mean), (M2, count); zero on entry
    int *flag;        // raised if a wait timed out
    int N, C, H, G, Ho;
    int S, SPS, TAIL, NCOL;
    int upr;          // units per round
    int xcd_units;    // units per XCD per round (0: plain workgroup order)
    float eps, inv_div;
};

// Steps [k0, k0 + ns) of a unit's NST = ceil(Ho / 2) two-row steps; the
// first TAIL slices take one step more; column tile col (or -1).
struct Slice {
    int k0, ns, col;
};

__device__ __forceinline__ Slice slice_of(const FusedArgs &a, int sg)
{
    Slice s;
    s.k0 = sg * a.SPS + min(sg, a.TAIL);
    s.ns = a.SPS + (sg < a.TAIL ? 1 : 0);
    const int c = a.S - 1 - sg;
    s.col = c < a.NCOL ? c : -1;
    return s;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const FusedArgs &a, int unit)
{
    const int n = unit / a.G, g = unit % a.G;
    return make_rsrc(a.x + ((size_t)n * a.C + (size_t)g * CG) * a.H * W, (unsigned)(CG * a.H * W * 4));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t y_rsrc(const FusedArgs &a, int unit, unsigned plane)
{
    const int n = unit / a.G, g = unit % a.G;
    return make_rsrc(a.y + ((size_t)n * a.C + (size_t)g * CG) * plane, CG * plane * 4u);
}

// One input row pair (rows row0, row0 + 1 of the group's 8 channels): this
// thread's float4 of each row (channel = wave, column 4 * lane).  Every load
// is issued (rows outside [0, H) are clamped; stash_pair writes zeros for
// them): a load under a branch would leave the register a merge of two
// values, and copying it would wait for the load.
__device__ __forceinline__ void load_pair(v4f (&pf)[2], __amdgpu_buffer_rsrc_t xr, int H, int row0,
                                          unsigned loff)
{
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = min(max(row0 + rr, 0), H - 1);
        pf[rr] = buf_load4(xr, loff, (unsigned)(row * W * 4));
    }
}

__device__ __forceinline__ void stash_pair(float *ring, int slot, const v4f (&pf)[2], int H, int row0,
                                           int wave, int lane)
{
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = row0 + rr;
        const bool ok = row >= 0 && row < H;
        *reinterpret_cast<v4f *>(ring + slot * PAIR_FLOATS + (rr * CG + wave) * RP + PADL + 4 * lane) =
            ok ? pf[rr] : v4f{0.f, 0.f, 0.f, 0.f};
    }
}

// Statistics of one unit -> this lane's two channel scale / shift pairs.
// Lanes < S read slice triples; the merge is a fixed tree over lanes, so
// every wave gets bit-identical coefficients.
struct Coef {
    float sc0, sh0, sc1, sh1;
};

__device__ __forceinline__ void probe_issue(const FusedArgs &a, int unit, int lane,
                                            unsigned long long &p0, unsigned long long &p1)
{
    // every lane loads (lanes >= S read slot 0 and are ignored): no branch
    unsigned long long *p = reinterpret_cast<unsigned long long *>(
        a.partials + ((size_t)unit * a.S + (lane < a.S ? lane : 0)) * 4);
    p0 = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p1 = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float lo_f(unsigned long long v) { return __uint_as_float((unsigned)v); }
__device__ __forceinline__ float hi_f(unsigned long long v) { return __uint_as_float((unsigned)(v >> 32)); }

// gb = (gamma, beta) of channels 2q, 2q+1 of the unit's group
__device__ __forceinline__ Coef probe_finish(const FusedArgs &a, int unit, int lane, const v4f &gb,
                                             unsigned long long p0, unsigned long long p1)
{
    int it = 0;
    for (;;) {
        const bool ok = lane >= a.S || (lo_f(p0) > 0.0f && hi_f(p1) > 0.0f);
        if (__all(ok)) break;
        if (++it > SPIN_LIMIT) {
            if (lane == 0) __hip_atomic_store(a.flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        probe_issue(a, unit, lane, p0, p1);
    }
    const bool mine = lane < a.S;
    float n = mine ? lo_f(p0) : 0.f, m = mine ? hi_f(p0) : 0.f, m2 = mine ? lo_f(p1) : 0.f;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
        const float nb = __shfl_down(n, off, 64), mb = __shfl_down(m, off, 64),
                    qb = __shfl_down(m2, off, 64);
        if (lane < off) chan_merge(n, m, m2, nb, mb, qb);
    }
    n = __shfl(n, 0, 64);
    m = __shfl(m, 0, 64);
    m2 = __shfl(m2, 0, 64);
    const float rstd = rsqrtf(m2 / n + a.eps);
    Coef c;
    c.sc0 = rstd * gb[0] * a.inv_div;
    c.sh0 = (gb[1] - m * rstd * gb[0]) * a.inv_div;
    c.sc1 = rstd * gb[2] * a.inv_div;
    c.sh1 = (gb[3] - m * rstd * gb[2]) * a.inv_div;
    return c;
}

// Normalised store of one row tile (rows of the tile: channels 2q, 2q+1,
// pixels 32 * wave + 2 * c16 + {0, 1}) of output row orow.
__device__ __forceinline__ void store_tile(__amdgpu_buffer_rsrc_t yr, const v4f &c, const Coef &k,
                                           unsigned vo0, unsigned vo1, int orow)
{
    const unsigned so = (unsigned)(orow * WO * 4);
    buf_store2_nt(v2f{c[0] * k.sc0 + k.sh0, c[1] * k.sc0 + k.sh0}, yr, vo0, so);
    buf_store2_nt(v2f{c[2] * k.sc1 + k.sh1, c[3] * k.sc1 + k.sh1}, yr, vo1, so);
}

// Events of a round with ns steps: e = 0 (round start) stashes pair 1;
// e = k + 1 (end of step k) stashes pair k + 2, or after the last step the
// next round's pair 0; events ns + 1 .. NEV - 1 stash nothing.  Loads issued
// at event e fill the register set that event e + 3 stashes (every round has
// NEV events, so event e always uses register set e % 3, and the next
// round's events 0..2 -- its pairs 1..3, as every slice has >= 3 steps -- are
// loaded during this one).  Rows are picked with selects and the loads are
// always issued; a load for an event that stashes nothing is not used.
__device__ __forceinline__ void issue_event(int e, v4f (&dst)[2], const Slice &sl,
                                            __amdgpu_buffer_rsrc_t xr, bool nhas, const Slice &nsl,
                                            __amdgpu_buffer_rsrc_t nxr, int H, unsigned loff)
{
    const int e3 = e + 3;
    const bool this_round = e3 < NEV && e3 < sl.ns;   // pair e3 + 1 of this round
    const int pair = this_round ? e3 + 1 : (e3 < NEV ? 0 : e3 - NEV + 1);
    const bool use_next = !this_round && nhas;
    load_pair(dst, use_next ? nxr : xr, H, 2 * ((use_next ? nsl.k0 : sl.k0) + pair) - 2, loff);
}

template <int ACT>
__device__ __forceinline__ v4f activate4(v4f c, float b0, float b1)
{
    c[0] = activate<ACT>(c[0] + b0);
    c[1] = activate<ACT>(c[1] + b0);
    c[2] = activate<ACT>(c[2] + b1);
    c[3] = activate<ACT>(c[3] + b1);
    return c;
}

__device__ __forceinline__ void sums4(const v4f &c, float &s1, float &s2)
{
    s1 += (c[0] + c[1]) + (c[2] + c[3]);
    s2 = fmaf(c[0], c[0], s2);
    s2 = fmaf(c[1], c[1], s2);
    s2 = fmaf(c[2], c[2], s2);
    s2 = fmaf(c[3], c[3], s2);
}

// Activation of a finished step's two row tiles (row 2 of them may lie past
// Ho: then it is kept out of the sums) -> running sums and the bank slot wp.
template <int ACT>
__device__ __forceinline__ void epilogue_to_bank(const v4f &acc0, const v4f &acc1, float b0, float b1,
                                                 bool v1, float &s1, float &s2, int &cnt, v4f *wp)
{
    const v4f e0 = activate4<ACT>(acc0, b0, b1);
    const v4f e1 = activate4<ACT>(acc1, b0, b1);
    float t1 = 0.f, t2 = 0.f;
    sums4(e0, s1, s2);
    sums4(e1, t1, t2);
    s1 += v1 ? t1 : 0.0f;
    s2 += v1 ? t2 : 0.0f;
    cnt += v1 ? 8 : 4;
    wp[0] = e0;
    wp[THREADS] = e1;
}

template <int ACT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void convt2d_gn_fused_kernel(FusedArgs a)
{
    __shared__ float ring[NSLOT * PAIR_FLOATS];
    __shared__ float strip[STRIP_ELEMS * 4];
    __shared__ float red[NWAVE * 3];
    __shared__ v4f bank[NBANK * 2 * THREADS];  // [slot][tile][thread], private to each thread

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, c16 = lane & 15;
    const int H = a.H, Ho = a.Ho, S = a.S;
    const int U = a.N * a.G;
    const unsigned plane = (unsigned)Ho * WO;
    // Waves w and w + 4 share a SIMD: one runs a step's MFMAs while the other
    // runs the previous step's activation, then they swap.
    const bool late = (wave & 4) != 0;

    int ulocal, s_base;
    if (a.xcd_units > 0) {  // a unit's S slices on one XCD: halo rows hit its L2
        const int xcd = blockIdx.x % NXCD, l = blockIdx.x / NXCD;
        ulocal = xcd * a.xcd_units + l / S;
        s_base = l % S;
    } else {
        ulocal = blockIdx.x / S;
        s_base = blockIdx.x % S;
    }

    for (int e = tid; e < NSLOT * 2 * CG; e += THREADS) {  // pad columns, never overwritten
        float *row = ring + e * RP;
#pragma unroll
        for (int c = 0; c < PADL; ++c) row[c] = 0.f;
    }
    for (int e = tid; e < STRIP_ELEMS; e += THREADS) { strip[e * 4 + 2] = 0.f; strip[e * 4 + 3] = 0.f; }

    const unsigned loff = (unsigned)((wave * H * W + 4 * lane) * 4);  // pair loads
    const int lb = PADL + 32 * wave + 2 * c16 + 1 - q;                // B operand column
    const unsigned vo0 = ((unsigned)(2 * q) * plane + 32u * wave + 2u * c16) * 4u;
    const unsigned vo1 = vo0 + plane * 4u;
    v4f *const mybank = bank + tid;
    auto slot_of = [](int k, int rho) { return (k + NBANK - rho % NBANK) % NBANK; };

    // ---- prologue: round 0's pair 0 in the ring, events 0..2 in flight
    v4f pf[3][2];
    int base = 0;  // ring slot of the current round's pair 0
    if (ulocal < U) {
        const Slice s0 = slice_of(a, s_base);
        const __amdgpu_buffer_rsrc_t xr = x_rsrc(a, ulocal);
        v4f p0[2];
        load_pair(p0, xr, H, 2 * s0.k0 - 2, loff);
        stash_pair(ring, 0, p0, H, 2 * s0.k0 - 2, wave, lane);
#pragma unroll
        for (int e = 0; e < 3; ++e) load_pair(pf[e], xr, H, 2 * (s0.k0 + e + 1) - 2, loff);
    }

    float wreg[CG * KS];
    float b0 = 0.f, b1 = 0.f;
    v4f gb = v4f{1.f, 0.f, 1.f, 0.f}, p_gb = gb;
    v4f cur_col = v4f{0.f, 0.f, 0.f, 0.f}, prv_col = v4f{0.f, 0.f, 0.f, 0.f};
    int p_unit = -1, p_sg = 0, p_k0 = 0, p_ns = 0, p_col = -1;
    Coef pc{0.f, 0.f, 0.f, 0.f};

    int r = 0;
    for (;; ++r) {
        const int unit = r * a.upr + ulocal;
        __syncthreads();  // ring readers of the last round are done; red[] is complete
        if (p_unit >= 0 && tid == 0) {
            float n = 0.f, m = 0.f, m2 = 0.f;
            for (int w = 0; w < NWAVE; ++w) chan_merge(n, m, m2, red[w * 3], red[w * 3 + 1], red[w * 3 + 2]);
            unsigned long long *p =
                reinterpret_cast<unsigned long long *>(a.partials + ((size_t)p_unit * S + p_sg) * 4);
            const unsigned long long v0 = (unsigned long long)__float_as_uint(n) |
                                          ((unsigned long long)__float_as_uint(m) << 32);
            const unsigned long long v1 = (unsigned long long)__float_as_uint(m2) |
                                          ((unsigned long long)__float_as_uint(n) << 32);
            __hip_atomic_store(p, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p + 1, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (unit >= U) break;

        const int sg = (s_base + r) % S;
        const Slice sl = slice_of(a, sg);
        const __amdgpu_buffer_rsrc_t xr = x_rsrc(a, unit);
        const int nunit = unit + a.upr;
        const bool nhas = nunit < U;
        const Slice nsl = slice_of(a, (sg + 1) % S);
        const __amdgpu_buffer_rsrc_t nxr = x_rsrc(a, nhas ? nunit : unit);
        const int nbase = base + sl.ns + 1;  // ring slot (mod 3) of the next round's pair 0
        const bool has_prev = p_unit >= 0;
        const __amdgpu_buffer_rsrc_t pyr = y_rsrc(a, has_prev ? p_unit : unit, plane);

        // ---- weights (A operand), bias, gamma / beta of the unit's group; strip
        const int g = unit % a.G;
        {
            const __amdgpu_buffer_rsrc_t wr =
                make_rsrc(a.wt + (size_t)g * CG * CG * KS * KS, CG * CG * KS * KS * 4);
            const int co = c16 >> 1, t = c16 & 1;
            const int kw = q + t - 1;
            const bool kok = kw >= 0 && kw < KS;
#pragma unroll
            for (int s = 0; s < CG * KS; ++s) {
                const int ci = s / KS, kh = s % KS;
                const float v = buf_load1(wr, (unsigned)((((ci * CG + co) * KS + kh) * KS + (kok ? kw : 0)) * 4));
                wreg[s] = kok ? v : 0.0f;
            }
            const int c0 = g * CG + 2 * q;
            b0 = a.bias ? a.bias[c0] : 0.0f;
            b1 = a.bias ? a.bias[c0 + 1] : 0.0f;
            gb = v4f{a.gamma ? a.gamma[c0] : 1.0f, a.beta ? a.beta[c0] : 0.0f,
                     a.gamma ? a.gamma[c0 + 1] : 1.0f, a.beta ? a.beta[c0 + 1] : 0.0f};
        }
        const int srow0 = sl.col >= 0 ? 16 * sl.col - (KS - 1) + tid % STRIP_ROWS : -1;
        const bool sok = sl.col >= 0 && tid < STRIP_ELEMS && srow0 >= 0 && srow0 < H;
        const v2f sv = __builtin_bit_cast(
            v2f, __builtin_amdgcn_raw_buffer_load_b64(
                     xr, (int)((((tid / STRIP_ROWS % CG) * H + min(max(srow0, 0), H - 1)) * W + (W - 2)) * 4),
                     0, 0));

        // ---- event 0: stash pair 1
        stash_pair(ring, (base + 1) % NSLOT, pf[0], H, 2 * (sl.k0 + 1) - 2, wave, lane);
        issue_event(0, pf[0], sl, xr, nhas, nsl, nxr, H, loff);
        __syncthreads();  // pairs 0, 1 in the ring

        // ---- steps.  Iteration k runs the MFMAs of step k and the activation,
        // sums and bank write of step k - 1 (before or after the MFMAs, by
        // wave); then it stores the previous unit's step k - 1 and stashes /
        // loads for event k + 1.
        float s1 = 0.f, s2 = 0.f;
        int cnt = 0;
        unsigned long long pr0 = 0ull, pr1 = 0ull;
        v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < MAXST; ++k) {
            if (k < sl.ns) {
                if (k > 0) __syncthreads();  // pair k + 1 in the ring
                const float *rA = ring + ((base + k) % NSLOT) * PAIR_FLOATS + lb;
                const float *rB = ring + ((base + k + 1) % NSLOT) * PAIR_FLOATS + lb;
                // B operands of the whole step first: input rows 2(k0+k) - 2 + m
                float xb[CG][4];
#pragma unroll
                for (int ci = 0; ci < CG; ++ci) {
                    xb[ci][0] = rA[ci * RP];
                    xb[ci][1] = rA[(CG + ci) * RP];
                    xb[ci][2] = rB[ci * RP];
                    xb[ci][3] = rB[(CG + ci) * RP];
                }
                if (k >= 1 && late)
                    epilogue_to_bank<ACT>(acc0, acc1, b0, b1, 2 * (sl.k0 + k - 1) + 1 < Ho, s1, s2, cnt,
                                          mybank + slot_of(k - 1, r) * 2 * THREADS);
                v4f n0 = v4f{0.f, 0.f, 0.f, 0.f}, n1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ci = 0; ci < CG; ++ci) {
                    // output row 2(k0+k) + j reads input row 2(k0+k) + j - kh, i.e. m = 2 + j - kh
                    n0 = mfma_16x16x4(wreg[ci * KS + 0], xb[ci][2], n0);
                    n1 = mfma_16x16x4(wreg[ci * KS + 0], xb[ci][3], n1);
                    n0 = mfma_16x16x4(wreg[ci * KS + 1], xb[ci][1], n0);
                    n1 = mfma_16x16x4(wreg[ci * KS + 1], xb[ci][2], n1);
                    n0 = mfma_16x16x4(wreg[ci * KS + 2], xb[ci][0], n0);
                    n1 = mfma_16x16x4(wreg[ci * KS + 2], xb[ci][1], n1);
                }
                if (k >= 1 && !late)
                    epilogue_to_bank<ACT>(acc0, acc1, b0, b1, 2 * (sl.k0 + k - 1) + 1 < Ho, s1, s2, cnt,
                                          mybank + slot_of(k - 1, r) * 2 * THREADS);
                acc0 = n0;
                acc1 = n1;

                if (k == 1 && has_prev) pc = probe_finish(a, p_unit, lane, p_gb, pr0, pr1);
                if (k >= 1 && has_prev) {
                    // the previous unit's step k - 1 (bank slot of this round's step k)
                    const v4f *sp = mybank + slot_of(k, r) * 2 * THREADS;
                    const int prow = 2 * (p_k0 + k - 1);
                    store_tile(pyr, sp[0], pc, vo0, vo1, prow);
                    if (prow + 1 < Ho) store_tile(pyr, sp[THREADS], pc, vo0, vo1, prow + 1);
                }
                if (k == 0) {
                    if (has_prev) probe_issue(a, p_unit, lane, pr0, pr1);
                    if (tid < STRIP_ELEMS) {
                        strip[tid * 4 + 0] = sok ? sv[0] : 0.0f;
                        strip[tid * 4 + 1] = sok ? sv[1] : 0.0f;
                    }
                }

                // ---- event k + 1: stash its pair (this round's pair k + 2, or after the
                // last step the next round's pair 0; harmless if there is none)
                const bool last = k + 1 == sl.ns;
                stash_pair(ring, last ? nbase % NSLOT : (base + k + 2) % NSLOT, pf[(k + 1) % 3], H,
                           last ? 2 * nsl.k0 - 2 : 2 * (sl.k0 + k + 2) - 2, wave, lane);
            }
            // event k + 1's loads (also for events past the last step, which only load)
            issue_event(k + 1, pf[(k + 1) % 3], sl, xr, nhas, nsl, nxr, H, loff);
        }

        // ---- last step: activation + sums -> bank; previous unit's step ns - 1
        {
            const int k = sl.ns;
            epilogue_to_bank<ACT>(acc0, acc1, b0, b1, 2 * (sl.k0 + k - 1) + 1 < Ho, s1, s2, cnt,
                                  mybank + slot_of(k - 1, r) * 2 * THREADS);
            if (has_prev && k - 1 < p_ns) {
                const v4f *sp = mybank + slot_of(k, r) * 2 * THREADS;
                const int prow = 2 * (p_k0 + k - 1);
                store_tile(pyr, sp[0], pc, vo0, vo1, prow);
                if (prow + 1 < Ho) store_tile(pyr, sp[THREADS], pc, vo0, vo1, prow + 1);
            }
        }

        // ---- column tile: pair 128 of rows 16 col + c16, read from the strip
        if (wave == COLWAVE && sl.col >= 0) {
            const int orow = 16 * sl.col + c16;
            // x row orow - kh -> strip row c16 + 2 - kh; x col 257 - q -> strip col 3 - q
            const float *sp = strip + c16 * 4 + 3 - q;
            v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ci = 0; ci < CG; ++ci) {
#pragma unroll
                for (int kh = 0; kh < KS; ++kh)
                    c = mfma_16x16x4(wreg[ci * KS + kh], sp[(ci * STRIP_ROWS + 2 - kh) * 4], c);
            }
            if (orow < Ho) {
                cur_col = activate4<ACT>(c, b0, b1);
                sums4(cur_col, s1, s2);
                cnt += 4;
            }
        }

        // ---- slice statistics -> red[wave]; published after the next barrier
        {
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
        }

        // ---- the previous unit's remaining step (if it had one more) and its column tile
        if (has_prev) {
            for (int j = sl.ns; j < p_ns; ++j) {
                const v4f *sp = mybank + slot_of(j + 1, r) * 2 * THREADS;
                const int prow = 2 * (p_k0 + j);
                store_tile(pyr, sp[0], pc, vo0, vo1, prow);
                if (prow + 1 < Ho) store_tile(pyr, sp[THREADS], pc, vo0, vo1, prow + 1);
            }
            if (wave == COLWAVE && p_col >= 0) {
                const int prow = 16 * p_col + c16;
                if (prow < Ho) {
                    const unsigned o = ((unsigned)(2 * q) * plane + (unsigned)prow * WO + W) * 4u;
                    buf_store2_nt(v2f{prv_col[0] * pc.sc0 + pc.sh0, prv_col[1] * pc.sc0 + pc.sh0}, pyr, o);
                    buf_store2_nt(v2f{prv_col[2] * pc.sc1 + pc.sh1, prv_col[3] * pc.sc1 + pc.sh1}, pyr,
                                  o + plane * 4u);
                }
            }
        }

        prv_col = cur_col;
        p_gb = gb;
        p_unit = unit;
        p_sg = sg;
        p_k0 = sl.k0;
        p_ns = sl.ns;
        p_col = sl.col;
        base = nbase % NSLOT;
    }

    // ---- the last unit: its triple was published above; wait, normalise, store
    if (p_unit >= 0) {
        const __amdgpu_buffer_rsrc_t pyr = y_rsrc(a, p_unit, plane);
        unsigned long long pr0, pr1;
        probe_issue(a, p_unit, lane, pr0, pr1);
        pc = probe_finish(a, p_unit, lane, p_gb, pr0, pr1);
        for (int j = 0; j < p_ns; ++j) {
            const v4f *sp = mybank + slot_of(j, r - 1) * 2 * THREADS;
            const int prow = 2 * (p_k0 + j);
            store_tile(pyr, sp[0], pc, vo0, vo1, prow);
            if (prow + 1 < Ho) store_tile(pyr, sp[THREADS], pc, vo0, vo1, prow + 1);
        }
        if (wave == COLWAVE && p_col >= 0) {
            const int prow = 16 * p_col + c16;
            if (prow < Ho) {
                const unsigned o = ((unsigned)(2 * q) * plane + (unsigned)prow * WO + W) * 4u;
                buf_store2_nt(v2f{prv_col[0] * pc.sc0 + pc.sh0, prv_col[1] * pc.sc0 + pc.sh0}, pyr, o);
                buf_store2_nt(v2f{prv_col[2] * pc.sc1 + pc.sh1, prv_col[3] * pc.sc1 + pc.sh1}, pyr,
                              o + plane * 4u);
            }
        }
    }
}

__global__ void zero_words_kernel(unsigned *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

struct Geometry {
    int S, SPS, TAIL, NCOL;
};

// Slices per unit: at most MAX_S and at least three steps each.
bool geometry(int Ho, Geometry &g)
{
    const int NST = (Ho + 1) / 2;
    g.S = NST / 3 < MAX_S ? NST / 3 : MAX_S;
    if (g.S < 1) return false;
    g.SPS = NST / g.S;
    g.TAIL = NST - g.S * g.SPS;
    g.NCOL = (Ho + 15) / 16;
    return g.SPS >= 3 && g.SPS + (g.TAIL > 0 ? 1 : 0) <= MAXST && g.NCOL <= g.S;
}

struct Occupancy {
    int device = -1;
    int blocks_per_cu[4] = {0, 0, 0, 0};
    int cus = 0;
};

template <int ACT>
hipError_t launch_t(const ConvT2dArgs &p, hipStream_t st)
{
    Geometry geo;
    if (!geometry(p.Ho, geo)) return hipErrorInvalidValue;
    static Occupancy occ[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Occupancy &o = occ[dev & 63];
    if (o.device != dev || o.blocks_per_cu[ACT] == 0) {
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, convt2d_gn_fused_kernel<ACT>, THREADS, 0);
        if (e != hipSuccess) return e;
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        o.device = dev;
        o.blocks_per_cu[ACT] = nb;
        o.cus = cus;
    }
    const int resident = o.blocks_per_cu[ACT] * o.cus;
    const int U = p.N * p.groups;
    int upr = resident / geo.S;
    if (upr < 1) return hipErrorCooperativeLaunchTooLarge;
    if (upr > U) upr = U;
    const int xcd_units = upr % NXCD == 0 ? upr / NXCD : 0;

    // workspace: flag word, pad to 16 B, then [U][S][4] partials (all zeroed)
    const int words = 4 + U * geo.S * 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                       reinterpret_cast<unsigned *>(p.partials), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    FusedArgs fa{p.x, p.w, p.b, p.gamma, p.beta, p.out, p.partials + 4,
                 reinterpret_cast<int *>(p.partials), p.N, p.C_out, p.H, p.groups, p.Ho,
                 geo.S, geo.SPS, geo.TAIL, geo.NCOL, upr, xcd_units, p.eps, p.inv_div};
    void *args[] = {&fa};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(convt2d_gn_fused_kernel<ACT>),
                                      dim3(upr * geo.S), dim3(THREADS), args, 0, st);
}

}  // namespace

int convt2d_fused_slices(int Ho)
{
    Geometry g;
    return geometry(Ho, g) ? g.S : 0;
}

bool convt2d_fused_supported(int C_in, int C_out, int groups, int H, int W_, int act, int norm,
                             int num_groups)
{
    Geometry g;
    return W_ == W && C_in == CG * groups && C_out == CG * groups && H >= 1 &&
           geometry(H + KS - 1, g) && norm == 1 /* group */ && num_groups == groups &&
           (act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF);
}

size_t convt2d_fused_workspace(int N, int groups, int Ho)
{
    const size_t U = (size_t)N * groups;
    return (4 + U * (size_t)convt2d_fused_slices(Ho) * 4) * sizeof(float);
}

hipError_t launch_convt2d_fused(const ConvT2dArgs &a, hipStream_t st)
{
    switch (a.act) {
    case ACT_NONE: return launch_t<ACT_NONE>(a, st);
    case ACT_HARDSWISH: return launch_t<ACT_HARDSWISH>(a, st);
    case ACT_GELU_ERF: return launch_t<ACT_GELU_ERF>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cnf
