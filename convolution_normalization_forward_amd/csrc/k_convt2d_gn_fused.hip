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
//   * a unit (sample, group) is cut into S slices of SPS two-row steps (the
//     last TAIL steps of the unit are spread over the slices as single row
//     tiles, so every slice carries the same work); S workgroups own one unit
//     per round (units handed out round by round; the launch is cooperative,
//     so all workgroups are resident at once);
//   * round r: a workgroup computes its slice of unit u_r (conv + bias +
//     activation) into an LDS bank laid out in output order, keeps running
//     sums, and early in round r+1 publishes the slice's (count, mean, M2)
//     triple;
//   * during round r+1 the same workgroup normalises the bank of u_r and
//     stores it: the coefficients of u_r are merged at the end of step 1 of
//     round r+1 (step 2 with 16-bit inputs), by which time the sibling slices
//     have normally published, and the steps after that store u_r's four
//     steps (2 and 3 two each; 3 all four).  Step k of round rho
//     lives in bank slot (rho SPS + k) mod (SPS + 1); a slot is read for its
//     store before the barrier after which a later step's epilogue rewrites
//     it (slots at risk are read into registers at the end of the step before).
//   * stores: the output row is 258 floats (1032 bytes), so a 32-pixel tile's
//     run of a row straddles two 128-byte lines in every row; such stores
//     measured ~2.7x slower than line-aligned ones.  Wave c instead writes
//     channel c's rows of a finished step, which are contiguous in memory, as
//     whole aligned lines: the line shared by two steps of a slice is written
//     by the later one, with the earlier step's floats carried in registers.
// Each triple travels as two 64-bit relaxed atomics that both carry the
// count, so a reader that sees both halves non-zero has the whole triple and
// no fence or counter is needed.  The wait is bounded: on time-out the
// caller's flag word is raised, the unit's outputs become NaN and the kernel
// still terminates.  Triples are
// merged in slice order, so results do not depend on timing.
//
// Tile mapping: rows of a 16x16 MFMA result = (channel, pixel parity),
// columns = 16 column pairs, K = (ci, kh, v = kw - t + 1): pixels (2p, 2p+1)
// read the same input columns shifted by one, so 72 of every 96 K entries are
// useful (zero-padded weights fill the rest).  An output row of 258 pixels is
// 8 row tiles (pixels 0..255, one per wave) plus the last column pair; the
// last pairs of a slice's 8 rows form its column tile (slice 0's also takes
// the rows past the slices, at most 4).  Each step reads
// two input row pairs from a 4-pair LDS ring refilled from registers loaded
// three stashes ahead; waves sharing a SIMD alternate the step's MFMAs and
// the previous step's activation.
//
// Input element type DT: 0 fp32; 1 bf16 / 2 fp16 for x and the weights (the
// second input precision).  16-bit inputs stay 16-bit in the ring and in the
// A operands, and a step's contraction runs on v_mfma_f32_16x16x32_{bf16,f16}
// with fp32 accumulation: K = 32 entries (ci, v') per kh, lane (q, c16)
// supplying ci = 2q, 2q+1 and v' = 0..3, i.e. four consecutive input columns
// 2 c16 - 2 .. 2 c16 + 1 of each channel (v' = 3 - v).  A row tile then takes
// 3 MFMAs instead of 24.  The single tiles widen to fp32 as they are loaded
// (products of 16-bit values are exact in fp32 either way).
//
// DT 3: fp32 x and w contracted on bf16 pieces.  fp32 MFMAs and the
// epilogue's vector work issue one after the other on a SIMD, bf16 MFMAs run
// beside it, so this form keeps x and w fp32 (ring and loads as DT 0) and
// splits each operand into three bf16 pieces, v = v1 + v2 + v3 exactly: the
// weights once per group, a step's two new input rows as it reads them.  The
// 16-bit tile mapping above then sums the six leading piece products per
// kernel row (18 MFMAs per tile), smallest first; the three dropped ones total
// at most about 2^-23 |w x|, two units in the last place of an fp32 product.
#include <atomic>

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
constexpr int NSLOT = 4;                     // input row pairs in the LDS ring
constexpr int PAIR_FLOATS = 2 * CG * RP;
// 16-bit ring rows: 4 zero elements left of x, pitch 272 elements (136 words:
// the four lane groups of a B read, channels 2q, start 16 q banks apart)
constexpr int RP16 = 272;
constexpr int PAIR16_WORDS = 2 * CG * RP16 / 2;
constexpr int SPS = 4;                       // steps per slice
// Bank: finished steps in output order, [slot][channel][row j * 258 + pixel]
// (CP = 528 = 16 mod 32: the four lane groups of an epilogue write land 32
// banks apart), SPS + 1 slots: step k of round rho in slot (rho SPS + k) mod
// (SPS + 1).  A slot is read (gathered for its store) at least one barrier
// before the epilogue of step k + SPS + 1 rewrites it.
constexpr int CP = 528;
constexpr int SLOT_FLOATS = CG * CP;
constexpr int BPAD = 32;                     // floats before slot 0 (line offsets start at -30)
constexpr int BTAIL = 128;                   // floats past the last slot (line slots past a range)
constexpr int NBANK = SPS + 1;
constexpr int LINE_SLOTS = 5;                // store instructions per wave per step: 20 lines >= 18
constexpr int NPOS = 6;                      // ring stash positions per round (SPS + 1, padded to 3 k)
constexpr int MAX_S = 32;                    // slices per unit
constexpr int SCH = CG * KS / 4;             // K entries of a single tile per wave (4 waves per tile)
// Per-round duties go to waves on different SIMDs (wave w runs on SIMD w % 4):
constexpr int COEFWAVE = 0;                  // merges the previous unit's slice triples
constexpr int PUBWAVE = 1;                   // publishes this workgroup's slice triple
constexpr int EXTWAVE = 3;                   // finishes the slice's extra row tile
constexpr int COLWAVE = 6;                   // finishes the slice's column tile
constexpr int SPIN_LIMIT = 1 << 16;          // polls (each a memory round trip) before giving up
constexpr unsigned OOB = 0x7ff00000u;        // buffer offset past any extent: loads return 0
static_assert(NWAVE * 32 == W, "one row tile per wave");
static_assert(CG * 64 == THREADS, "one (channel, 64 float4) row chunk per wave");
static_assert(NPOS % 3 == 0 && NPOS >= SPS + 1, "stash positions");
static_assert((EXTWAVE & 3) != (COLWAVE & 3), "extra and column tiles finish on different SIMDs");
static_assert(SPS == 4, "single tiles are computed in step 2 and finished in step 3");

struct FusedArgs {
    const void *x, *wt;  // element type DT
    const float *bias, *gamma, *beta;
    float *y;
    float *partials;  // [U][S][4]: (count, mean), (M2, count); zero on entry
    int *flag;        // raised if a wait timed out
    int spin_limit;   // polls before a wait gives up
    int never_ready;  // test hook: a wait also needs a word nobody writes
    int N, C, H, G, Ho;
    int S, NEXT;        // slices, extra row tiles (16 per tail step)
    int upr;            // units per round
    int xcd_units;      // units per XCD per round (0: plain workgroup order)
    float eps, inv_div;
};

// Element size of x and the weights, and loads that widen them to fp32.
template <int DT>
constexpr unsigned ESZ = DT == 0 ? 4u : 2u;

template <int DT>
__device__ __forceinline__ float widen16(unsigned h)
{
    if constexpr (DT == 1) return __builtin_bit_cast(float, h << 16);                       // bf16
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xffffu));       // fp16
}

// one element at a byte offset (OOB reads 0)
template <int DT>
__device__ __forceinline__ float eload1(__amdgpu_buffer_rsrc_t r, unsigned byte_off)
{
    if constexpr (DT == 0) {
        return buf_load1(r, byte_off);
    } else {
        const unsigned h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)byte_off, 0, 0);
        return widen16<DT>(h);
    }
}

// four consecutive elements at a byte offset (OOB reads 0)
template <int DT>
__device__ __forceinline__ v4f eload4(__amdgpu_buffer_rsrc_t r, unsigned byte_off)
{
    if constexpr (DT == 0) {
        return buf_load4(r, byte_off);
    } else {
        const auto raw = __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0);
        const unsigned w0 = (unsigned)raw[0], w1 = (unsigned)raw[1];
        return v4f{widen16<DT>(w0), widen16<DT>(w0 >> 16), widen16<DT>(w1), widen16<DT>(w1 >> 16)};
    }
}

// Ring staging registers: fp32 widened float4, or four raw 16-bit elements.
template <int DT>
struct Stage {
    using T = v2u;
};
template <>
struct Stage<0> {
    using T = v4f;
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// D(16x16) += A(16x32) B(32x16) on 16-bit operands: lane l supplies
// A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16], e = 0..7, two per word (low
// half first); D element [4(l/16) + r][l%16] lives in register r of lane l.
template <int DT>
__device__ __forceinline__ v4f mfma16x32(v4u a, v4u b, v4f c)
{
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// The 16-bit B operand of input row m from the fp32 ring, as three pieces:
// p points at channel 2q, column 2 c16 - 2 of the lane's tile; words 0, 1
// take that channel's four columns, words 2, 3 channel 2q + 1's.
__device__ __forceinline__ void split_row(v4u (&xp)[4][3], int m, const float *p)
{
    const v2f f0 = *reinterpret_cast<const v2f *>(p), f1 = *reinterpret_cast<const v2f *>(p + 2);
    const v2f g0 = *reinterpret_cast<const v2f *>(p + RP), g1 = *reinterpret_cast<const v2f *>(p + RP + 2);
    put_pieces(xp[m], 0, split3(f0[0], f0[1]));
    put_pieces(xp[m], 1, split3(f1[0], f1[1]));
    put_pieces(xp[m], 2, split3(g0[0], g0[1]));
    put_pieces(xp[m], 3, split3(g1[0], g1[1]));
}

// Unit (n, g) = n G + g owns channels n C + g CG .. + CG - 1, and C = G CG, so
// its first channel is unit * CG: no division by G.
template <int DT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const FusedArgs &a, int unit)
{
    return make_rsrc(static_cast<const char *>(a.x) + (size_t)unit * CG * a.H * W * ESZ<DT>,
                     (unsigned)(CG * a.H * W * ESZ<DT>));
}

// The unit's output resource, built from a base address held in scalar
// registers (readfirstlane), so that its stores take the descriptor as is.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t y_rsrc_u(const FusedArgs &a, int unit, unsigned plane)
{
    const unsigned long long p = reinterpret_cast<unsigned long long>(a.y + (size_t)unit * CG * plane);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p),
                   hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
    const unsigned long long pu = (unsigned long long)lo | ((unsigned long long)hi << 32);
    return make_rsrc(reinterpret_cast<float *>(pu), __builtin_amdgcn_readfirstlane(CG * plane * 4u));
}

// One input row pair (rows row0, row0 + 1 of the group's 8 channels): this
// thread's float4 of each row (channel = wave, column 4 * lane).  Every load
// is issued -- a load under a branch would leave the register a merge of two
// values, and copying it would wait for the load -- and a row outside [0, H)
// gets an offset past the buffer, which reads as zeros.
template <int DT>
__device__ __forceinline__ void load_pair(typename Stage<DT>::T (&pf)[2], __amdgpu_buffer_rsrc_t xr, int H,
                                          int row0, unsigned loff)
{
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = row0 + rr;
        const unsigned ro = row >= 0 && row < H ? (unsigned)(row * W) * ESZ<DT> : OOB;
        if constexpr (DT == 0)
            pf[rr] = eload4<DT>(xr, loff + ro);
        else
            pf[rr] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(xr, (int)(loff + ro), 0, 0));
    }
}

template <int DT>
__device__ __forceinline__ void stash_pair(float *ring, int slot, const typename Stage<DT>::T (&pf)[2], int wave,
                                           int lane)
{
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        if constexpr (DT == 0)
            *reinterpret_cast<v4f *>(ring + slot * PAIR_FLOATS + (rr * CG + wave) * RP + PADL + 4 * lane) = pf[rr];
        else  // 8-byte aligned: RP16 and PADL are multiples of 4 elements
            *reinterpret_cast<v2u *>(reinterpret_cast<unsigned *>(ring) + slot * PAIR16_WORDS +
                                     (rr * CG + wave) * (RP16 / 2) + PADL / 2 + 2 * lane) = pf[rr];
    }
}

// Ring stash positions of a round: p <= SPS-2 stashes pair p+2 at the end of
// step p; p = SPS-1 and SPS stash the next round's pairs 0 and 1 at the end
// of the last step; later positions stash nothing.  The loads for position
// p + 3 are issued right after position p's stash, into register set p % 3
// (NPOS is a multiple of 3, so every round starts on set 0).
template <int DT>
__device__ __forceinline__ void issue_pos(int p, typename Stage<DT>::T (&dst)[2], int k0, __amdgpu_buffer_rsrc_t xr,
                                          bool nhas, int nk0, __amdgpu_buffer_rsrc_t nxr, int H,
                                          unsigned loff)
{
    const int p3 = p + 3;
    int pair;
    bool next;
    if (p3 < NPOS) {
        next = p3 >= SPS - 1;
        pair = p3 <= SPS - 2 ? p3 + 2 : p3 - (SPS - 1);  // past SPS: unused
    } else {
        next = true;  // the next round's position p3 - NPOS <= 2 <= SPS - 2
        pair = p3 - NPOS + 2;
    }
    const bool use_next = next && nhas;
    load_pair<DT>(dst, use_next ? nxr : xr, H, 2 * ((use_next ? nk0 : k0) + pair) - 2, loff);
}

// Chan merge of Welford triples with the weight nb / (n + nb) from the
// hardware reciprocal (a merge here feeds only the statistics; counts are
// exact integers, so the weight is off by at most an ulp or so).
__device__ __forceinline__ void merge_fast(float &n, float &mean, float &m2, float nb, float meanb, float m2b)
{
    const float nn = n + nb;
    const float f = nn > 0.0f ? nb * __builtin_amdgcn_rcpf(nn) : 0.0f;
    const float delta = meanb - mean;
    mean = fmaf(delta, f, mean);
    m2 = m2 + m2b + delta * delta * n * f;
    n = nn;
}

// Every lane of a 16-lane row ends with the merge of the row's triples
// (rotations through DPP; lane 0 of the row merges in lane order 0..15 by
// halves, and every wave doing this on the same data gets the same bits).
__device__ __forceinline__ void row_merge16(float &n, float &mean, float &m2)
{
#define CNF_ROW_STEP(S)                                                                  \
    {                                                                                    \
        const float nb = row_ror<S>(n), mb = row_ror<S>(mean), qb = row_ror<S>(m2);      \
        merge_fast(n, mean, m2, nb, mb, qb);                                             \
    }
    CNF_ROW_STEP(8) CNF_ROW_STEP(4) CNF_ROW_STEP(2) CNF_ROW_STEP(1)
#undef CNF_ROW_STEP
}

// Lanes 0..31 hold triples (zeros where there is nothing): merge of lanes
// 0..15 with the merge of lanes 16..31, the same in every lane.
__device__ __forceinline__ void merge32(float &n, float &mean, float &m2)
{
    row_merge16(n, mean, m2);
    auto lane_f = [](float v, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
    };
    const float n1 = lane_f(n, 16), m1 = lane_f(mean, 16), q1 = lane_f(m2, 16);
    n = lane_f(n, 0);
    mean = lane_f(mean, 0);
    m2 = lane_f(m2, 0);
    merge_fast(n, mean, m2, n1, m1, q1);
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
    bool timed_out = false;
    for (;;) {
        const bool ok = a.never_ready == 0 && (lane >= a.S || (lo_f(p0) > 0.0f && hi_f(p1) > 0.0f));
        if (__all(ok)) break;
        if (++it > a.spin_limit) {
            // one store per wave at most, and none once the flag is up
            if (lane == 0 && __hip_atomic_load(a.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
                __hip_atomic_store(a.flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            timed_out = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        probe_issue(a, unit, lane, p0, p1);
    }
    const bool mine = lane < a.S;
    float n = mine ? lo_f(p0) : 0.f, m = mine ? hi_f(p0) : 0.f, m2 = mine ? lo_f(p1) : 0.f;
    merge32(n, m, m2);
    if (timed_out) m = __builtin_nanf("");  // the unit's outputs become NaN
    const float rstd = timed_out ? m : rsqrtf(m2 / n + a.eps);
    Coef c;
    c.sc0 = rstd * gb[0] * a.inv_div;
    c.sh0 = (gb[1] - m * rstd * gb[0]) * a.inv_div;
    c.sc1 = rstd * gb[2] * a.inv_div;
    c.sh1 = (gb[3] - m * rstd * gb[2]) * a.inv_div;
    return c;
}

// The slice triple from the 32 row triples in red[] (4 rows of 16 lanes per
// wave), stored by lane 0 as two 64-bit relaxed atomics that both carry the
// count.  Called by one whole wave.
__device__ __forceinline__ void publish(const FusedArgs &a, const float *red, int unit, int sg, int lane)
{
    const int l = lane & 31;
    float n = lane < 32 ? red[l * 3] : 0.f, m = lane < 32 ? red[l * 3 + 1] : 0.f,
          m2 = lane < 32 ? red[l * 3 + 2] : 0.f;
    merge32(n, m, m2);
    if (lane == 0) {
        unsigned long long *p =
            reinterpret_cast<unsigned long long *>(a.partials + ((size_t)unit * a.S + sg) * 4);
        const unsigned long long v0 = (unsigned long long)__float_as_uint(n) |
                                      ((unsigned long long)__float_as_uint(m) << 32);
        const unsigned long long v1 = (unsigned long long)__float_as_uint(m2) |
                                      ((unsigned long long)__float_as_uint(n) << 32);
        __hip_atomic_store(p, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p + 1, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Normalised 8-byte stores of one tile's two channel rows (voffsets vo0 /
// vo1 hold the lane's pixel pair; so = the uniform row offset).  Output rows
// are 1032 bytes, so a tile's 128-byte run straddles two cache lines whose
// other parts come from the neighbouring tiles of the same step: plain
// (L2-allocating) stores let L2 merge them before they reach HBM.
__device__ __forceinline__ void store_tile(__amdgpu_buffer_rsrc_t yr, const v4f &c, const Coef &k,
                                           unsigned vo0, unsigned vo1, unsigned so)
{
    buf_store2(v2f{c[0] * k.sc0 + k.sh0, c[1] * k.sc0 + k.sh0}, yr, vo0, so);
    buf_store2(v2f{c[2] * k.sc1 + k.sh1, c[3] * k.sc1 + k.sh1}, yr, vo1, so);
}

template <int ACT>
__device__ __forceinline__ v4f activate4(v4f c)
{
    c[0] = activate<ACT>(c[0]);
    c[1] = activate<ACT>(c[1]);
    c[2] = activate<ACT>(c[2]);
    c[3] = activate<ACT>(c[3]);
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

// Activation of a finished step's two row tiles (bias already in the
// accumulators; the second row may lie past Ho: then it is skipped) ->
// running sums and the bank slot wp.
// Bank position p = slot + 2q CP + j 258 + pixel of the lane's pair: the
// lane's channels 2q (p) and 2q + 1 (p + CP).
__device__ __forceinline__ void bank_put(float *p, const v4f &e)
{
    *reinterpret_cast<v2f *>(p) = v2f{e[0], e[1]};
    *reinterpret_cast<v2f *>(p + CP) = v2f{e[2], e[3]};
}

template <int ACT>
__device__ __forceinline__ void epilogue_to_bank(const v4f &acc0, const v4f &acc1, bool v1, float &s1,
                                                 float &s2, int &cnt, float *p)
{
    const v4f e0 = activate4<ACT>(acc0);
    sums4(e0, s1, s2);
    bank_put(p, e0);
    cnt += 4;
    if (v1) {
        const v4f e1 = activate4<ACT>(acc1);
        sums4(e1, s1, s2);
        bank_put(p + WO, e1);
        cnt += 4;
    }
}

// One finished step of the previous unit, normalised and stored by the wave
// of channel c (= wave).  Its rows are the contiguous float range [F, F + R)
// of the channel plane (R = 258 per row); t = F mod 32, so the step's lines of
// 32 floats start at offsets -t + 32 m, and lane (q, c16) of store i writes
// offsets u = 128 i + 32 q + 2 c16 - t: whole 128-byte lines.  The line that
// straddles two steps of a slice is written once, by the later step, its
// earlier floats (u < 0) taken from `carry`, which the earlier step read from
// its own slot; floats at or past `hi` are left to the next step.  Only the
// first and last lines of a slice are partial (masked lanes): their other
// floats belong to the neighbouring slices.
//
// gather_lines reads a step's values from its bank row `chan` (and the next
// step's carry), emit_lines normalises and stores them, so a slot can be read
// before the barrier after which another step's epilogue rewrites it.
struct Lines {
    v2f v[LINE_SLOTS];
};

// R2 = floats in a step's two rows (2 x 258 here, 2 x 256 for the upsampling kernel)
template <int R2>
__device__ __forceinline__ void gather_lines(Lines &L, const float *chan, int t, bool has_next, int next_t,
                                             v2f &carry, int q, int c16)
{
    const int base = 32 * q + 2 * c16 - t;
#pragma unroll
    for (int i = 0; i < LINE_SLOTS; ++i) {
        const int u = base + 128 * i;
        const v2f v = *reinterpret_cast<const v2f *>(chan + u);
        L.v[i] = i == 0 && u < 0 ? carry : v;
    }
    if (has_next) carry = *reinterpret_cast<const v2f *>(chan + R2 - next_t + 2 * c16);
}

// soff = byte offset of the step's first float; with active false every store
// goes past the buffer.  The buffer range check sees only the per-lane offset,
// so after the first step (whose lanes never go below 0) the uniform offset
// moves back one line and the lanes' offsets forward by the same amount.
__device__ __forceinline__ void emit_lines(__amdgpu_buffer_rsrc_t yr, const Lines &L, float sc, float sh, int t,
                                           int hi, bool first, unsigned soff, int q, int c16, bool active)
{
    soff = __builtin_amdgcn_readfirstlane(soff);
    const int base = 32 * q + 2 * c16 - t;
    const int lift = first ? 0 : 32;
#pragma unroll
    for (int i = 0; i < LINE_SLOTS; ++i) {
        const int u = base + 128 * i;
        bool ok = active && u < hi;
        if (i == 0) ok = ok && (!first || u >= 0);
        const v2f v = L.v[i];
        buf_store2(v2f{fmaf(v[0], sc, sh), fmaf(v[1], sc, sh)}, yr, ok ? (unsigned)(4 * (u + lift)) : OOB,
                   soff - 4u * (unsigned)lift);
    }
}

// A single tile (the extra row tile or the column tile) is split over four
// waves, each taking SCH = 6 of its 24 K entries (channels 2 chunk, 2 chunk
// + 1; kh = 0..2) and reading them straight from x (L2): lane (q, c16), entry
// (ci, kh) takes x[ci][row(c16) - kh][col(c16) - q], zero outside the input
// (the offset is pushed past the buffer, which returns 0).  Row tile:
// row(c16) = orow, col = 32 rt + 2 c16 + 1.  Column tile: row = 16 c + c16,
// col = 257.  Lanes of a wave without such a tile read past the buffer.
template <int DT>
__device__ __forceinline__ void single_load(float (&b)[SCH], __amdgpu_buffer_rsrc_t xr, int H, int chunk,
                                            bool has, int row, int col)
{
#pragma unroll
    for (int j = 0; j < SCH; ++j) {
        const int ci = 2 * chunk + j / KS, rr = row - j % KS;
        const bool ok = has && rr >= 0 && rr < H && col >= 0 && col < W;
        b[j] = eload1<DT>(xr, ok ? (unsigned)((ci * H + rr) * W + col) * ESZ<DT> : OOB);
    }
}

template <int ACT, int DT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void convt2d_gn_fused_kernel(FusedArgs a)
{
    // DT 3: x and w are fp32 in memory (load type LT = 0) and the contraction
    // runs on bf16 pieces of them (split3) in the 16-bit tile mapping
    constexpr int LT = DT == 3 ? 0 : DT;
    using PF = typename Stage<LT>::T;
    constexpr int NB = NBANK;
    // iteration at whose end the previous unit's coefficients are merged: one
    // step later with 16-bit inputs, whose steps are short, so that the sibling
    // slices have published (measured: 0.90 -> 0.85 ms; fp32, whose SIMDs are
    // MFMA-bound, loses 3% to the extra registers and the single store burst)
    constexpr int MERGE = DT == 1 || DT == 2 ? 2 : 1;
    __shared__ __align__(16) float ring[LT == 0 ? NSLOT * PAIR_FLOATS : NSLOT * PAIR16_WORDS];
    __shared__ float red[NWAVE * 4 * 3];  // [wave][row of 16 lanes] slice triples
    __shared__ v4f spart[2 * 4 * 64];     // [tile][chunk][lane] single-tile partial sums
    __shared__ float coefs[CG * 2];       // the previous unit's (scale, shift) per channel
    __shared__ __align__(16) float bank[BPAD + NB * SLOT_FLOATS + BTAIL];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, c16 = lane & 15;
    const int H = a.H, Ho = a.Ho, S = a.S;
    const int U = a.N * a.G;
    const unsigned plane = (unsigned)Ho * WO;
    const int rows_main = 2 * S * SPS;  // rows of the slices; the rest are extra row tiles
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
        if constexpr (LT == 0) {
            float *row = ring + e * RP;
#pragma unroll
            for (int c = 0; c < PADL; ++c) row[c] = 0.f;
        } else {
            unsigned *row = reinterpret_cast<unsigned *>(ring) + e * (RP16 / 2);
#pragma unroll
            for (int c = 0; c < PADL / 2; ++c) row[c] = 0u;
        }
    }

    const unsigned loff = (unsigned)(wave * H * W + 4 * lane) * ESZ<LT>;  // pair loads
    const int lb = PADL + 32 * wave + 2 * c16 + 1 - q;                // B operand column
    // 16-bit B operand: word of columns 2 c16 - 2, -1 of channel 2q in a ring row
    const int lb16 = 2 * q * (RP16 / 2) + (PADL - 2) / 2 + 16 * wave + c16;
    const int bo = 2 * q * CP + 32 * wave + 2 * c16;                   // bank position of the lane's pair
    // fp32 ring float of channel 2q, column 32 wave + 2 c16 - 2 (DT 3's B operand)
    const int lbe = 2 * q * RP + PADL - 2 + 32 * wave + 2 * c16;
    // bank slot of step k of round rho (steps numbered over rounds; rho = -1,
    // the round before the first, when a store is issued with nothing to store)
    auto slot = [&](int rho, int k) { return bank + BPAD + (((rho * SPS + k) % NB + NB) % NB) * SLOT_FLOATS; };

    // ---- prologue: round 0's pairs 0, 1 in the ring, positions 0..2 in flight
    PF pf[3][2];
    int base = 0;  // ring slot of the current round's pair 0
    {
        const int k0 = s_base * SPS;
        const __amdgpu_buffer_rsrc_t xr = x_rsrc<LT>(a, ulocal);
        PF p0[2], p1[2];
        load_pair<LT>(p0, xr, H, 2 * k0 - 2, loff);
        load_pair<LT>(p1, xr, H, 2 * k0, loff);
        stash_pair<LT>(ring, 0, p0, wave, lane);
        stash_pair<LT>(ring, 1, p1, wave, lane);
#pragma unroll
        for (int p = 0; p < 3; ++p) load_pair<LT>(pf[p], xr, H, 2 * (k0 + p + 2) - 2, loff);
    }

    float wreg[CG * KS];
    v4u a16[KS];  // 16-bit A operands, one per kh
    v4u ap[KS][3];  // DT 3: bf16 pieces of the A operands, [kh][piece]
    float wsub[SCH];  // this wave's single-tile chunk of the weights
    v4f bias4 = v4f{0.f, 0.f, 0.f, 0.f};  // accumulator start: bias of channels 2q, 2q, 2q+1, 2q+1
    v4f gb = v4f{1.f, 0.f, 1.f, 0.f}, p_gb = gb;
    int wgroup = -1;
    v4f cur_ext = v4f{0.f, 0.f, 0.f, 0.f}, prv_ext = cur_ext;  // extra row tile (wave EXTWAVE)
    v4f cur_col = cur_ext, prv_col = cur_ext;                  // column tile (wave COLWAVE)
    int p_unit = -1, p_sg = 0, p_k0 = 0, p_ext = -1;
    Coef pc{0.f, 0.f, 0.f, 0.f};
    float psc = 0.f, psh = 0.f;  // the previous unit's scale / shift of channel `wave`

    // Column tile of a slice: its own rows 2 k0 + c16 (c16 < 8); slice 0 also
    // takes the rows past the slices (c16 - 8 of them, at most 4).
    auto col_row = [&](int k0, int sg) { return c16 < 8 ? 2 * k0 + c16 : (sg == 0 ? rows_main + c16 - 8 : Ho); };

    // The previous unit's step s, by the wave of its channel `wave`: gathered
    // from its slot, then normalised and stored (active false: the same
    // instructions, every store past the buffer -- the memory waits the
    // compiler places then count the same stores on every path).
    v2f carry = v2f{0.f, 0.f};
    Lines held0, held1, held2;
    auto gather_step = [&](int rho, int s, unsigned cu, Lines &held) {
        const int prow = 2 * (p_k0 + s);
        const bool last = s == SPS - 1 || prow + 2 >= Ho;
        gather_lines<2 * WO>(held, slot(rho, s) + wave * CP, (int)((cu + 4u * s) & 31u), !last,
                     (int)((cu + 4u * s + 4u) & 31u), carry, q, c16);
    };
    auto emit_step = [&](int s, __amdgpu_buffer_rsrc_t pyr, unsigned cu, bool active, const Lines &held) {
        const int prow = 2 * (p_k0 + s);
        const int nr = prow + 1 < Ho ? 2 : 1;
        const bool last = s == SPS - 1 || prow + 2 >= Ho;
        const int t = (int)((cu + 4u * s) & 31u), nt = (int)((cu + 4u * s + 4u) & 31u);
        emit_lines(pyr, held, psc, psh, t, last ? WO * nr : 2 * WO - nt, s == 0,
                   ((unsigned)wave * plane + (unsigned)prow * WO) * 4u, q, c16, active);
    };
    // (float offset of the unit's channel-`wave` slice start) mod 32, even
    auto line_phase = [&](int unit, int k0) {
        const unsigned long long f = (reinterpret_cast<unsigned long long>(a.y) >> 2) +
                                     (unsigned long long)unit * CG * plane + (unsigned long long)wave * plane +
                                     (unsigned long long)(2 * k0) * WO;
        return (unsigned)f & 30u;
    };
    // the previous unit's tiles outside the slices' rows: its extra row tile
    // and the column pixels of those rows (slice 0's column tile, lanes c16 >= 8)
    // (issued by every wave, masked ones past the buffer, as in store_step)
    auto store_outside = [&](__amdgpu_buffer_rsrc_t pyr, bool active) {
        const int prow_e = rows_main + 2 * (p_ext >> 4) + ((p_ext >> 3) & 1);
        const bool e_ok = active && wave == EXTWAVE && p_ext >= 0 && prow_e < Ho;
        const unsigned oe = ((unsigned)(2 * q) * plane + (unsigned)prow_e * WO + 32u * (p_ext & 7) + 2u * c16) * 4u;
        store_tile(pyr, prv_ext, pc, e_ok ? oe : OOB, e_ok ? oe + plane * 4u : OOB, 0u);
        const int prow_c = rows_main + c16 - 8;
        const bool c_ok = active && wave == COLWAVE && p_sg == 0 && c16 >= 8 && prow_c < Ho;
        const unsigned oc = ((unsigned)(2 * q) * plane + (unsigned)prow_c * WO + W) * 4u;
        store_tile(pyr, prv_col, pc, c_ok ? oc : OOB, c_ok ? oc + plane * 4u : OOB, 0u);
    };
    // the column pixels (256, 257) of the previous unit's rows into its bank slots
    auto put_col = [&](int rho) {
        if (wave == COLWAVE && c16 < 8 && 2 * p_k0 + c16 < Ho)
            bank_put(slot(rho, c16 >> 1) + 2 * q * CP + (c16 & 1) * WO + W, prv_col);
    };

    // the round's slice and group, stepped once per round (no division in the loop):
    // slice (s_base + r) mod S, group (r upr + ulocal) mod G
    int sg = s_base, g = ulocal % a.G;
    const int g_step = a.upr % a.G;
    int r = 0;
    for (;; ++r) {
        const int unit = r * a.upr + ulocal;
        __syncthreads();  // pairs 0, 1 in the ring; last round's ring readers done; red[] complete
        if (unit >= U) {
            if (p_unit >= 0 && wave == PUBWAVE) publish(a, red, p_unit, p_sg, lane);
            break;
        }
        const bool has_prev = p_unit >= 0;
        if (has_prev && wave == PUBWAVE) publish(a, red, p_unit, p_sg, lane);
        if (has_prev) put_col(r - 1);

        const int k0 = sg * SPS;
        const int ext = sg < a.NEXT ? sg : -1;           // extra row tile e: tail step e/16, tile e%16
        const __amdgpu_buffer_rsrc_t xr = x_rsrc<LT>(a, unit);
        const int nunit = unit + a.upr;
        const bool nhas = nunit < U;
        const int nk0 = (sg + 1 == S ? 0 : sg + 1) * SPS;
        const __amdgpu_buffer_rsrc_t nxr = x_rsrc<LT>(a, nhas ? nunit : unit);
        const __amdgpu_buffer_rsrc_t pyr = y_rsrc_u(a, has_prev ? p_unit : unit, plane);
        const unsigned pcu = has_prev ? line_phase(p_unit, p_k0) : 0u;

        // ---- weights (A operand), bias, gamma / beta of the unit's group
        if (g != wgroup) {
            wgroup = g;
            const __amdgpu_buffer_rsrc_t wr =
                make_rsrc(static_cast<const char *>(a.wt) + (size_t)g * CG * CG * KS * KS * ESZ<LT>,
                          CG * CG * KS * KS * ESZ<LT>);
            const int co = c16 >> 1, t = c16 & 1;
            const int kw = q + t - 1;
            const bool kok = kw >= 0 && kw < KS;
            if constexpr (DT == 0) {
#pragma unroll
                for (int s = 0; s < CG * KS; ++s) {
                    const int ci = s / KS, kh = s % KS;
                    const float v = eload1<LT>(wr, (unsigned)(((ci * CG + co) * KS + kh) * KS + (kok ? kw : 0)) * ESZ<LT>);
                    wreg[s] = kok ? v : 0.0f;
                }
            } else if constexpr (DT == 3) {
                // the 16-bit mapping below, on three bf16 pieces of each fp32 weight
#pragma unroll
                for (int kh = 0; kh < KS; ++kh) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        float v[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * d + h, ci = 2 * q + e / 4, kw16 = 2 - e % 4 + t;
                            const bool ok = kw16 >= 0 && kw16 < KS;
                            v[h] = buf_load1(wr, ok ? (unsigned)((((ci * CG + co) * KS + kh) * KS + kw16) * 4) : OOB);
                        }
                        put_pieces(ap[kh], d, split3(v[0], v[1]));
                    }
                }
            } else {
                // A[(co, t)][(ci, v')] = w[ci][co][kh][2 - v' + t], ci = 2q + e / 4, v' = e % 4;
                // taps outside the kernel read past the buffer (zero)
#pragma unroll
                for (int kh = 0; kh < KS; ++kh) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        unsigned word = 0u;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * d + h, ci = 2 * q + e / 4, kw16 = 2 - e % 4 + t;
                            const bool ok = kw16 >= 0 && kw16 < KS;
                            const unsigned v = __builtin_amdgcn_raw_buffer_load_b16(
                                wr, ok ? (int)((((ci * CG + co) * KS + kh) * KS + kw16) * 2) : (int)OOB, 0, 0);
                            word |= (v & 0xffffu) << (16 * h);
                        }
                        a16[kh][d] = word;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < SCH; ++j) {
                const int ci = 2 * (wave & 3) + j / KS, kh = j % KS;
                const float v = eload1<LT>(wr, (unsigned)(((ci * CG + co) * KS + kh) * KS + (kok ? kw : 0)) * ESZ<LT>);
                wsub[j] = kok ? v : 0.0f;
            }
            const int c0 = g * CG + 2 * q;
            const float b0 = a.bias ? a.bias[c0] : 0.0f, b1 = a.bias ? a.bias[c0 + 1] : 0.0f;
            bias4 = v4f{b0, b0, b1, b1};
            gb = v4f{a.gamma ? a.gamma[c0] : 1.0f, a.beta ? a.beta[c0] : 0.0f,
                     a.gamma ? a.gamma[c0 + 1] : 1.0f, a.beta ? a.beta[c0 + 1] : 0.0f};
        }

        // ---- this slice's single tiles: B operands straight from x (L2)
        const int ext_row = rows_main + 2 * (ext >> 4) + ((ext >> 3) & 1);
        const int tsel = wave >> 2, chunk = wave & 3;  // tile (0 extra, 1 column) and K chunk
        const int crow = col_row(k0, sg);
        const bool has_t = tsel == 0 ? ext >= 0 : crow < Ho;
        // their loads: at the round top with 16-bit inputs, in iteration 1 with
        // fp32 ones (off the round boundary, where all eight waves would issue
        // these scattered loads at once; measured 1.20 -> 1.18 ms with bf16
        // pieces, 0.85 -> 0.89 ms the other way with 16-bit inputs)
        constexpr int SINGLE_AT = DT == 1 || DT == 2 ? -1 : 1;
        float sb[SCH];
        auto load_single = [&]() {
            single_load<LT>(sb, xr, H, chunk, has_t, tsel == 0 ? ext_row : crow,
                            tsel == 0 ? 32 * (ext & 7) + 2 * c16 + 1 - q : 2 * (W / 2) + 1 - q);
        };
        if constexpr (SINGLE_AT < 0) load_single();

        // ---- steps.  Iteration k runs the MFMAs of step k and the activation, sums
        // and bank write of step k - 1 (before or after the MFMAs, by wave), then
        // stashes / loads ring pairs; the iterations after MERGE also store the
        // previous unit.
        float s1 = 0.f, s2 = 0.f;
        int cnt = 0;
        unsigned long long pr0 = 0ull, pr1 = 0ull;
        v4u xp[4][3];  // DT 3: bf16 pieces of the B operands, [input row m][piece]
        v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < SPS; ++k) {
            if (k > 0) __syncthreads();  // pair k + 1 in the ring
            // B operands of the whole step first: input rows 2(k0+k) - 2 + m
            float xb[CG][4];
            v4u xb16[4];
            if constexpr (DT == 0) {
                const float *rA = ring + ((base + k) % NSLOT) * PAIR_FLOATS + lb;
                const float *rB = ring + ((base + k + 1) % NSLOT) * PAIR_FLOATS + lb;
#pragma unroll
                for (int ci = 0; ci < CG; ++ci) {
                    xb[ci][0] = rA[ci * RP];
                    xb[ci][1] = rA[(CG + ci) * RP];
                    xb[ci][2] = rB[ci * RP];
                    xb[ci][3] = rB[(CG + ci) * RP];
                }
            } else if constexpr (DT == 3) {
                // rows m = 0, 1 are the last step's rows 2, 3 (split then), except at a
                // round's first step
                const float *rA = ring + ((base + k) % NSLOT) * PAIR_FLOATS + lbe;
                const float *rB = ring + ((base + k + 1) % NSLOT) * PAIR_FLOATS + lbe;
                if (k == 0) {
                    split_row(xp, 0, rA);
                    split_row(xp, 1, rA + CG * RP);
                } else {
#pragma unroll
                    for (int pc3 = 0; pc3 < 3; ++pc3) {
                        xp[0][pc3] = xp[2][pc3];
                        xp[1][pc3] = xp[3][pc3];
                    }
                }
                split_row(xp, 2, rB);
                split_row(xp, 3, rB + CG * RP);
            } else {
                const unsigned *r16 = reinterpret_cast<const unsigned *>(ring);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const unsigned *rp = r16 + ((base + k + m / 2) % NSLOT) * PAIR16_WORDS +
                                         (m % 2) * CG * (RP16 / 2) + lb16;
                    xb16[m] = v4u{rp[0], rp[1], rp[RP16 / 2], rp[RP16 / 2 + 1]};
                }
            }
            if (k == SINGLE_AT) load_single();
            if (k == MERGE && has_prev && wave == COEFWAVE) probe_issue(a, p_unit, lane, pr0, pr1);
            if (k == MERGE + 1 && has_prev) {
                const float *cq = coefs + 4 * q;  // channels 2q, 2q+1, merged last step
                pc = Coef{cq[0], cq[1], cq[2], cq[3]};
                psc = coefs[2 * wave];
                psh = coefs[2 * wave + 1];
            }
            if (k == 3) {
                // single tiles: the four chunk partials, summed in chunk order
                const bool fin_e = wave == EXTWAVE && ext >= 0, fin_c = wave == COLWAVE;
                if (fin_e || fin_c) {
                    const v4f *pp = spart + (fin_e ? 0 : 4) * 64 + lane;
                    const v4f e = activate4<ACT>(((pp[0] + pp[64]) + pp[128]) + pp[192]);
                    // the tile's row (column tile: the lane's row) may lie past Ho
                    if (fin_e ? ext_row < Ho : crow < Ho) {
                        sums4(e, s1, s2);
                        cnt += 4;
                    }
                    if (fin_e) cur_ext = e;
                    else cur_col = e;
                }
            }
            // The previous unit's steps, in the iterations after the merge (steps
            // whose slots an epilogue rewrites are gathered before the barrier that
            // precedes the rewrite); no store is issued late in a round, so a memory
            // wait early in the next round (vmcnt counts loads and stores in issue
            // order) finds them done.
            if constexpr (MERGE == 1) {
                if (k == 2 || k == 3) {
                    emit_step(2 * (k - 2), pyr, pcu, has_prev, held0);
                    gather_step(r - 1, 2 * (k - 2) + 1, pcu, held0);
                    emit_step(2 * (k - 2) + 1, pyr, pcu, has_prev, held0);
                    if (k == 3) store_outside(pyr, has_prev);
                }
            } else if (k == 3) {
                emit_step(0, pyr, pcu, has_prev, held0);
                emit_step(1, pyr, pcu, has_prev, held1);
                emit_step(2, pyr, pcu, has_prev, held2);
                gather_step(r - 1, 3, pcu, held0);
                emit_step(3, pyr, pcu, has_prev, held0);
                store_outside(pyr, has_prev);
            }
            if (k >= 1 && late)
                epilogue_to_bank<ACT>(acc0, acc1, 2 * (k0 + k - 1) + 1 < Ho, s1, s2, cnt, slot(r, k - 1) + bo);
            v4f n0 = bias4, n1 = bias4;
            // output row 2(k0+k) + j reads input row 2(k0+k) + j - kh, i.e. m = 2 + j - kh
            if constexpr (DT == 0) {
#pragma unroll
                for (int ci = 0; ci < CG; ++ci) {
                    n0 = mfma_16x16x4(wreg[ci * KS + 0], xb[ci][2], n0);
                    n1 = mfma_16x16x4(wreg[ci * KS + 0], xb[ci][3], n1);
                    n0 = mfma_16x16x4(wreg[ci * KS + 1], xb[ci][1], n0);
                    n1 = mfma_16x16x4(wreg[ci * KS + 1], xb[ci][2], n1);
                    n0 = mfma_16x16x4(wreg[ci * KS + 2], xb[ci][0], n0);
                    n1 = mfma_16x16x4(wreg[ci * KS + 2], xb[ci][1], n1);
                }
            } else if constexpr (DT == 3) {
                // six of the nine piece products, smallest first: the three dropped
                // ones total at most about 2^-23 |w x|
                constexpr const int *PA = PIECE_A, *PB = PIECE_B;
#pragma unroll
                for (int s = 0; s < 6; ++s) {
#pragma unroll
                    for (int kh = 0; kh < KS; ++kh) {
                        n0 = mfma16x32<1>(ap[kh][PA[s]], xp[2 - kh][PB[s]], n0);
                        n1 = mfma16x32<1>(ap[kh][PA[s]], xp[3 - kh][PB[s]], n1);
                    }
                }
            } else {
                n0 = mfma16x32<DT>(a16[0], xb16[2], n0);
                n1 = mfma16x32<DT>(a16[0], xb16[3], n1);
                n0 = mfma16x32<DT>(a16[1], xb16[1], n0);
                n1 = mfma16x32<DT>(a16[1], xb16[2], n1);
                n0 = mfma16x32<DT>(a16[2], xb16[0], n0);
                n1 = mfma16x32<DT>(a16[2], xb16[1], n1);
            }
            if (k >= 1 && !late)
                epilogue_to_bank<ACT>(acc0, acc1, 2 * (k0 + k - 1) + 1 < Ho, s1, s2, cnt, slot(r, k - 1) + bo);
            acc0 = n0;
            acc1 = n1;
            if (k == MERGE && has_prev && wave == COEFWAVE) {
                // the previous unit's coefficients for the next step (one merge per workgroup)
                const Coef cw = probe_finish(a, p_unit, lane, p_gb, pr0, pr1);
                if (c16 == 0) {
                    coefs[4 * q] = cw.sc0; coefs[4 * q + 1] = cw.sh0;
                    coefs[4 * q + 2] = cw.sc1; coefs[4 * q + 3] = cw.sh1;
                }
            }
            if (k == 2 && has_t) {
                // this wave's chunk of a single tile (chunk 0 carries the bias)
                v4f c = chunk == 0 ? bias4 : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < SCH; ++j) c = mfma_16x16x4(wsub[j], sb[j], c);
                spart[(tsel * 4 + chunk) * 64 + lane] = c;
            }

            // ---- ring stashes at the end of step k, each followed by its loads
            if (k <= SPS - 2) {
                stash_pair<LT>(ring, (base + k + 2) % NSLOT, pf[k % 3], wave, lane);
                issue_pos<LT>(k, pf[k % 3], k0, xr, nhas, nk0, nxr, H, loff);
            } else {
                stash_pair<LT>(ring, (base + SPS + 1) % NSLOT, pf[(SPS - 1) % 3], wave, lane);
                issue_pos<LT>(SPS - 1, pf[(SPS - 1) % 3], k0, xr, nhas, nk0, nxr, H, loff);
                stash_pair<LT>(ring, (base + SPS + 2) % NSLOT, pf[SPS % 3], wave, lane);
                issue_pos<LT>(SPS, pf[SPS % 3], k0, xr, nhas, nk0, nxr, H, loff);
#pragma unroll
                for (int p = SPS + 1; p < NPOS; ++p) issue_pos<LT>(p, pf[p % 3], k0, xr, nhas, nk0, nxr, H, loff);
            }
            // the previous unit's steps whose slots the next iterations' epilogues
            // rewrite (0 in iteration 2, 1 in iteration 3, 2 after the loop) and
            // that are not stored before then, ahead of the barrier that precedes
            // the rewrite
            if (k == 1) gather_step(r - 1, 0, pcu, held0);
            if (k == 2) {
                if constexpr (MERGE == 2) gather_step(r - 1, 1, pcu, held1);
                gather_step(r - 1, 2, pcu, MERGE == 2 ? held2 : held0);
            }
        }

        // ---- the last step's activation -> bank (the slot of the previous unit's
        // step SPS - 2, gathered at the end of iteration 2)
        epilogue_to_bank<ACT>(acc0, acc1, 2 * (k0 + SPS - 1) + 1 < Ho, s1, s2, cnt, slot(r, SPS - 1) + bo);

        // ---- slice statistics -> red[wave][row]; published after the next barrier
        {
            float fn = (float)cnt;
            float mean = cnt ? s1 / fn : 0.0f;
            float m2 = cnt ? fmaxf(s2 - s1 * mean, 0.0f) : 0.0f;
            row_merge16(fn, mean, m2);
            if (c16 == 0) {
                float *e = red + (wave * 4 + q) * 3;
                e[0] = fn; e[1] = mean; e[2] = m2;
            }
        }

        prv_ext = cur_ext;
        prv_col = cur_col;
        p_gb = gb;
        p_unit = unit;
        p_sg = sg;
        p_k0 = k0;
        p_ext = ext;
        base = (base + SPS + 1) % NSLOT;
        sg = sg + 1 == S ? 0 : sg + 1;
        g += g_step;
        if (g >= a.G) g -= a.G;
    }

    // ---- the last unit: its triple was published above; wait, normalise, store
    if (p_unit >= 0) {
        put_col(r - 1);
        const __amdgpu_buffer_rsrc_t pyr = y_rsrc_u(a, p_unit, plane);
        unsigned long long pr0, pr1;
        probe_issue(a, p_unit, lane, pr0, pr1);
        pc = probe_finish(a, p_unit, lane, p_gb, pr0, pr1);
        // channel `wave`'s coefficients from the lane that holds them
        const int src = 16 * (wave >> 1);
        psc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                  __builtin_bit_cast(int, (wave & 1) ? pc.sc1 : pc.sc0), src));
        psh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                  __builtin_bit_cast(int, (wave & 1) ? pc.sh1 : pc.sh0), src));
        __syncthreads();  // the column pixels in the bank
        const unsigned pcu = line_phase(p_unit, p_k0);
        for (int j = 0; j < SPS; ++j) {
            gather_step(r - 1, j, pcu, held0);
            emit_step(j, pyr, pcu, true, held0);
        }
        store_outside(pyr, true);
    }
}

// ===========================================================================
// The upsampling form of the grouped transposed conv: ConvTranspose2d k 3,
// stride 2, padding 1, output_padding 1, 8 in / 8 out channels per group,
// input width 128 (output 2H x 256), + activation + GroupNorm, in the same
// single-write scheme (page "Kimi-K2.6__l2_p19", its layer at stride 2).
// Output (2i + a, 2j + b) takes inputs (i, j), (i, j + 1), (i + 1, j) and
// (i + 1, j + 1) only: kh = 1 for a = 0, kh = 2 from row i and kh = 0 from row
// i + 1 for a = 1 (columns alike).  So a step is one input row i -> output
// rows 2i, 2i + 1: wave c computes output channel c, lane l the 2 x 2 blocks
// of input columns 2l and 2l + 1 (output columns 4l .. 4l + 3), on the VALU
// (9 taps per input / output channel pair, 18 multiply-adds per output: too
// thin for MFMA tiles), with the channel's 72 weights in registers.
// A slice is SPS input rows, every unit has H / SPS slices, and the output
// rows are 256 floats, so no single tiles are needed and a step's rows start
// on a 128-byte line.  The input rows of a round (i0 .. i0 + SPS) sit in LDS
// slots 0 .. SPS, refilled from registers loaded three stashes ahead; the
// statistics exchange, the bank and the line stores are the ones above, with
// the merge at the end of step 1 and two of the previous unit's steps stored
// in each of steps 2 and 3 (measured: all four in step 3 0.85 ms, this 0.79;
// a merge at the end of step 0 spins on the siblings, 0.97).
constexpr int UW = 128;                      // input width
constexpr int UWO = 2 * UW;                  // output row
constexpr int URP = UW + 4;                  // ring row pitch: x at 0..127, zeros at 128..131
constexpr int UROW_FLOATS = CG * URP;        // one input row of the group's 8 channels
constexpr int UMAX_S = 32;
static_assert(2 * UWO + 16 == CP, "the bank's channel rows hold a step");
static_assert(CG * 64 == THREADS && UW == 2 * 64, "one row load: channel = wave, 2 columns per lane");

// One input row (row of this unit; rows past H read as zeros): this thread's
// two columns of channel `wave`.
__device__ __forceinline__ v2u load_urow(__amdgpu_buffer_rsrc_t xr, int H, int row, unsigned loff)
{
    const unsigned ro = row < H ? (unsigned)(row * UW) * 4u : OOB;
    return __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(xr, (int)(loff + ro), 0, 0));
}

__device__ __forceinline__ void stash_urow(float *ring, int slot, v2u v, int wave, int lane)
{
    *reinterpret_cast<v2u *>(ring + slot * UROW_FLOATS + wave * URP + 2 * lane) = v;
}

// Stash positions of a round: p <= SPS - 2 stashes row p + 2 at the end of
// step p; p = SPS - 1 and SPS stash the next round's rows 0 and 1 at the end
// of the last step; position SPS + 1 stashes nothing.  Position p + 3 is
// loaded right after position p's stash, into register set p % 3.
__device__ __forceinline__ v2u issue_upos(int p, int i0, __amdgpu_buffer_rsrc_t xr, bool nhas, int ni0,
                                          __amdgpu_buffer_rsrc_t nxr, int H, unsigned loff)
{
    const int p3 = p + 3;
    int row;
    bool next;
    if (p3 < NPOS) {
        next = p3 >= SPS - 1;
        row = p3 <= SPS - 2 ? p3 + 2 : p3 - (SPS - 1);
    } else {
        next = true;
        row = p3 - NPOS + 2;
    }
    const bool use_next = next && nhas;
    return load_urow(use_next ? nxr : xr, H, (use_next ? ni0 : i0) + row, loff);
}

// SPLIT (f32_math = BF16X3): the conv as 16x16x32 bf16 tiles on three pieces
// of every fp32 operand.  Wave w takes input columns j = 16 w + c16; tile b
// (output column parity) has rows (co, a) = (c16 / 2, c16 % 2) and K = (ci =
// 2q + e / 4, di = e / 2 % 2, dj = e % 2), the 2 x 2 input neighbourhood of
// 8 channels, so A[(co, a)][(ci, di, dj)] is the tap of (a, di), (b, dj) or
// zero (9 of 16 useful) and B[(ci, di, dj)][j] = x[ci][i + di][j + dj].  A step
// splits one new input row (two words per lane), issues 12 MFMAs, and the D
// rows 4q + r of tile b are channel 2q + r / 2, output row 2i + r % 2,
// column 2j + b.
template <int ACT, bool SPLIT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void upsample2_gn_fused_kernel(FusedArgs a)
{
    __shared__ __align__(16) float ring[(SPS + 1) * UROW_FLOATS];
    __shared__ float red[NWAVE * 4 * 3];
    __shared__ float coefs[CG * 2];
    __shared__ __align__(16) float bank[BPAD + NBANK * SLOT_FLOATS + BTAIL];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, c16 = lane & 15;
    const int H = a.H, Ho = a.Ho, S = a.S;
    const int U = a.N * a.G;
    const unsigned plane = (unsigned)Ho * UWO;

    int ulocal, s_base;
    if (a.xcd_units > 0) {
        const int xcd = blockIdx.x % NXCD, l = blockIdx.x / NXCD;
        ulocal = xcd * a.xcd_units + l / S;
        s_base = l % S;
    } else {
        ulocal = blockIdx.x / S;
        s_base = blockIdx.x % S;
    }
    for (int e = tid; e < (SPS + 1) * CG; e += THREADS) {  // zero columns right of x, never overwritten
        float *row = ring + e * URP + UW;
#pragma unroll
        for (int c = 0; c < URP - UW; ++c) row[c] = 0.f;
    }
    const unsigned loff = (unsigned)(wave * H * UW + 2 * lane) * 4u;
    auto slot = [&](int rho, int k) { return bank + BPAD + (((rho * SPS + k) % NBANK + NBANK) % NBANK) * SLOT_FLOATS; };
    auto xres = [&](int unit) {
        return make_rsrc(static_cast<const char *>(a.x) + (size_t)unit * CG * H * UW * 4, (unsigned)(CG * H * UW * 4));
    };

    // ---- prologue: round 0's rows 0, 1 in the ring, positions 0..2 in flight
    v2u pf[3];
    {
        const int i0 = s_base * SPS;
        const __amdgpu_buffer_rsrc_t xr = xres(ulocal);
        stash_urow(ring, 0, load_urow(xr, H, i0, loff), wave, lane);
        stash_urow(ring, 1, load_urow(xr, H, i0 + 1, loff), wave, lane);
#pragma unroll
        for (int p = 0; p < 3; ++p) pf[p] = load_urow(xr, H, i0 + p + 2, loff);
    }

    float bias1 = 0.f;
    v4f gb = v4f{1.f, 0.f, 1.f, 0.f}, p_gb = gb;
    int wgroup = -1;
    float wk[CG][KS * KS];  // w[ci][c][kh][kw] of this wave's output channel c
    v4u uwa[2][3];          // SPLIT: A pieces of tiles b = 0, 1
    v4f ubias4 = v4f{0.f, 0.f, 0.f, 0.f};  // SPLIT: bias of channels 2q, 2q, 2q+1, 2q+1
    v4u bq[3];              // SPLIT: B pieces, words d: channel 2q + d / 2, input row i + d % 2
    const int uj = 16 * wave + c16;  // SPLIT: this lane's input column
    int p_unit = -1, p_sg = 0, p_i0 = 0;
    float psc = 0.f, psh = 0.f;
    v2f carry = v2f{0.f, 0.f};
    Lines held0, held1, held2;
    // (float offset of the previous unit's channel-`wave` slice start) mod 32, even
    auto line_phase = [&](int unit, int i0) {
        const unsigned long long f = (reinterpret_cast<unsigned long long>(a.y) >> 2) +
                                     (unsigned long long)unit * CG * plane + (unsigned long long)wave * plane +
                                     (unsigned long long)(2 * i0) * UWO;
        return (unsigned)f & 30u;
    };
    // a step's rows are 512 floats (0 mod 32), so its line phase is the slice's
    auto gather_step = [&](int rho, int s, unsigned cu, Lines &held) {
        gather_lines<2 * UWO>(held, slot(rho, s) + wave * CP, (int)cu, s < SPS - 1, (int)cu, carry, q, c16);
    };
    auto emit_step = [&](int s, __amdgpu_buffer_rsrc_t pyr, unsigned cu, bool active, const Lines &held) {
        const int prow = 2 * (p_i0 + s);
        emit_lines(pyr, held, psc, psh, (int)cu, s == SPS - 1 ? 2 * UWO : 2 * UWO - (int)cu, s == 0,
                   ((unsigned)wave * plane + (unsigned)prow * UWO) * 4u, q, c16, active);
    };

    int r = 0;
    int sg = s_base, g = ulocal % a.G;  // stepped once per round, as above
    const int g_step = a.upr % a.G;
    for (;; ++r) {
        const int unit = r * a.upr + ulocal;
        __syncthreads();  // rows 0, 1 in the ring; last round's ring readers done; red[] complete
        if (unit >= U) {
            if (p_unit >= 0 && wave == PUBWAVE) publish(a, red, p_unit, p_sg, lane);
            break;
        }
        const bool has_prev = p_unit >= 0;
        if (has_prev && wave == PUBWAVE) publish(a, red, p_unit, p_sg, lane);

        const int i0 = sg * SPS;
        const __amdgpu_buffer_rsrc_t xr = xres(unit);
        const int nunit = unit + a.upr;
        const bool nhas = nunit < U;
        const int ni0 = (sg + 1 == S ? 0 : sg + 1) * SPS;
        const __amdgpu_buffer_rsrc_t nxr = xres(nhas ? nunit : unit);
        const __amdgpu_buffer_rsrc_t pyr = y_rsrc_u(a, has_prev ? p_unit : unit, plane);
        const unsigned pcu = has_prev ? line_phase(p_unit, p_i0) : 0u;

        if (g != wgroup) {
            wgroup = g;
            if constexpr (SPLIT) {
                // A[(co, aa)][(ci, di, dj)] = w[ci][co][kh][kw]: kh 1 for (aa, di) = (0, 0),
                // 2 for (1, 0), 0 for (1, 1), none for (0, 1); kw alike from (b, dj)
                const float *wg = static_cast<const float *>(a.wt) + (size_t)g * CG * CG * KS * KS;
                const int co = c16 >> 1, aa = c16 & 1;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        float v2[2];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int e = 2 * d + hh, ci = 2 * q + e / 4, di = (e >> 1) & 1, dj = e & 1;
                            const int kh = aa == 0 ? (di == 0 ? 1 : -1) : (di == 0 ? 2 : 0);
                            const int kw = b == 0 ? (dj == 0 ? 1 : -1) : (dj == 0 ? 2 : 0);
                            v2[hh] = kh >= 0 && kw >= 0 ? wg[(ci * CG + co) * KS * KS + kh * KS + kw] : 0.0f;
                        }
                        put_pieces(uwa[b], d, split3(v2[0], v2[1]));
                    }
                const int c0 = g * CG + 2 * q;
                const float b0 = a.bias ? a.bias[c0] : 0.0f, b1 = a.bias ? a.bias[c0 + 1] : 0.0f;
                ubias4 = v4f{b0, b0, b1, b1};
            } else {
                const float *wg = static_cast<const float *>(a.wt) + ((size_t)g * CG * CG + wave) * KS * KS;
#pragma unroll
                for (int ci = 0; ci < CG; ++ci)
#pragma unroll
                    for (int t = 0; t < KS * KS; ++t) wk[ci][t] = wg[ci * CG * KS * KS + t];
                bias1 = a.bias ? a.bias[g * CG + wave] : 0.0f;
            }
            const int cg = g * CG + 2 * q;  // the (gamma, beta) pairs probe_finish uses
            gb = v4f{a.gamma ? a.gamma[cg] : 1.0f, a.beta ? a.beta[cg] : 0.0f,
                     a.gamma ? a.gamma[cg + 1] : 1.0f, a.beta ? a.beta[cg + 1] : 0.0f};
        }

        float s1 = 0.f, s2 = 0.f;
        unsigned long long pr0 = 0ull, pr1 = 0ull;
#pragma unroll
        for (int k = 0; k < SPS; ++k) {
            if (k > 0) __syncthreads();  // row k + 1 in the ring
            if (k == 1 && has_prev && wave == COEFWAVE) probe_issue(a, p_unit, lane, pr0, pr1);
            if (k == 2 && has_prev) {
                psc = coefs[2 * wave];
                psh = coefs[2 * wave + 1];
            }
            if constexpr (SPLIT) {
                // ---- B pieces: rows i (words 0, 2) are the last step's rows i + 1,
                // except at a round's first step; then 12 MFMAs, the activation,
                // sums and the bank (v2f per (channel, output row): columns 2j, 2j + 1)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if (k > 0 && (d & 1) == 0) {
#pragma unroll
                        for (int pc = 0; pc < 3; ++pc) bq[pc][d] = bq[pc][d + 1];
                    } else {
                        const float *src = ring + (k + (d & 1)) * UROW_FLOATS + (2 * q + (d >> 1)) * URP + uj;
                        put_pieces(bq, d, split3(src[0], src[1]));
                    }
                }
                v4f t0 = ubias4, t1 = ubias4;
#pragma unroll
                for (int s = 0; s < 6; ++s) {
                    t0 = mfma_bf16_16x16x32(uwa[0][PIECE_A[s]], bq[PIECE_B[s]], t0);
                    t1 = mfma_bf16_16x16x32(uwa[1][PIECE_A[s]], bq[PIECE_B[s]], t1);
                }
                const v4f e0 = activate4<ACT>(t0), e1 = activate4<ACT>(t1);
                sums4(e0, s1, s2);
                sums4(e1, s1, s2);
                float *bp = slot(r, k) + 2 * q * CP + 2 * uj;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    *reinterpret_cast<v2f *>(bp + (rr >> 1) * CP + (rr & 1) * UWO) = v2f{e0[rr], e1[rr]};
            } else {
            // ---- conv of input row i0 + k (ring slots k, k + 1): acc[h][p] is the
            // block of input column 2 lane + h, p = 2a + b (output row 2i + a,
            // column 2(2 lane + h) + b)
            const float *r0 = ring + k * UROW_FLOATS + 2 * lane, *r1 = ring + (k + 1) * UROW_FLOATS + 2 * lane;
            float acc[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) acc[h][pp] = bias1;
#pragma unroll
            for (int ci = 0; ci < CG; ++ci) {
                // input columns 2 lane .. 2 lane + 2 of rows i and i + 1
                const v2f a01 = *reinterpret_cast<const v2f *>(r0 + ci * URP);
                const v2f b01 = *reinterpret_cast<const v2f *>(r1 + ci * URP);
                const float a2 = r0[ci * URP + 2], b2 = r1[ci * URP + 2];
                const float *kk = wk[ci];  // kk[kh * 3 + kw]
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float x00 = h ? a01[1] : a01[0], x01 = h ? a2 : a01[1];
                    const float x10 = h ? b01[1] : b01[0], x11 = h ? b2 : b01[1];
                    acc[h][0] = fmaf(x00, kk[4], acc[h][0]);
                    acc[h][1] = fmaf(x01, kk[3], fmaf(x00, kk[5], acc[h][1]));
                    acc[h][2] = fmaf(x10, kk[1], fmaf(x00, kk[7], acc[h][2]));
                    acc[h][3] = fmaf(x11, kk[0], fmaf(x10, kk[2], fmaf(x01, kk[6], fmaf(x00, kk[8], acc[h][3]))));
                }
            }
            // ---- activation, sums, bank (channel `wave`, output columns 4 lane .. + 3)
            {
                const v4f e0 = activate4<ACT>(v4f{acc[0][0], acc[0][1], acc[1][0], acc[1][1]});
                const v4f e1 = activate4<ACT>(v4f{acc[0][2], acc[0][3], acc[1][2], acc[1][3]});
                sums4(e0, s1, s2);
                sums4(e1, s1, s2);
                float *bp = slot(r, k) + wave * CP + 4 * lane;
                *reinterpret_cast<v4f *>(bp) = e0;
                *reinterpret_cast<v4f *>(bp + UWO) = e1;
            }
            }
            // ---- the previous unit, in the two steps after the merge: steps 0..2
            // were gathered at the ends of steps 0..2 (each iteration's epilogue
            // rewrites the slot of the previous unit's step k - 1); stores are
            // issued on every path (masked past the buffer) so that the memory
            // waits the compiler places count the same stores everywhere
            if (k == 2) {
                emit_step(0, pyr, pcu, has_prev, held0);
                emit_step(1, pyr, pcu, has_prev, held1);
            }
            if (k == 3) {
                emit_step(2, pyr, pcu, has_prev, held2);
                gather_step(r - 1, 3, pcu, held0);
                emit_step(3, pyr, pcu, has_prev, held0);
            }
            if (k == 1 && has_prev && wave == COEFWAVE) {
                const Coef cw = probe_finish(a, p_unit, lane, p_gb, pr0, pr1);
                if (c16 == 0) {
                    coefs[4 * q] = cw.sc0; coefs[4 * q + 1] = cw.sh0;
                    coefs[4 * q + 2] = cw.sc1; coefs[4 * q + 3] = cw.sh1;
                }
            }
            // ---- ring stashes at the end of step k, each followed by its loads
            if (k <= SPS - 2) {
                stash_urow(ring, k + 2, pf[k % 3], wave, lane);
                pf[k % 3] = issue_upos(k, i0, xr, nhas, ni0, nxr, H, loff);
            } else {
                stash_urow(ring, 0, pf[(SPS - 1) % 3], wave, lane);
                pf[(SPS - 1) % 3] = issue_upos(SPS - 1, i0, xr, nhas, ni0, nxr, H, loff);
                stash_urow(ring, 1, pf[SPS % 3], wave, lane);
                pf[SPS % 3] = issue_upos(SPS, i0, xr, nhas, ni0, nxr, H, loff);
#pragma unroll
                for (int p = SPS + 1; p < NPOS; ++p) pf[p % 3] = issue_upos(p, i0, xr, nhas, ni0, nxr, H, loff);
            }
            // the previous unit's step k, before the barrier after which the next
            // iteration's epilogue rewrites its slot
            if (k == 0) gather_step(r - 1, 0, pcu, held0);
            if (k == 1) gather_step(r - 1, 1, pcu, held1);
            if (k == 2) gather_step(r - 1, 2, pcu, held2);
        }

        // ---- slice statistics -> red[wave][row]; published after the next barrier
        {
            const int cnt = 8 * SPS;  // every lane: 8 outputs per step
            float fn = (float)cnt;
            float mean = s1 / fn;
            float m2 = fmaxf(s2 - s1 * mean, 0.0f);
            row_merge16(fn, mean, m2);
            if (c16 == 0) {
                float *e = red + (wave * 4 + q) * 3;
                e[0] = fn; e[1] = mean; e[2] = m2;
            }
        }
        p_gb = gb;
        p_unit = unit;
        p_sg = sg;
        p_i0 = i0;
        sg = sg + 1 == S ? 0 : sg + 1;
        g += g_step;
        if (g >= a.G) g -= a.G;
    }

    // ---- the last unit: its triple was published above; wait, normalise, store
    if (p_unit >= 0) {
        const __amdgpu_buffer_rsrc_t pyr = y_rsrc_u(a, p_unit, plane);
        unsigned long long pr0, pr1;
        probe_issue(a, p_unit, lane, pr0, pr1);
        const Coef pc = probe_finish(a, p_unit, lane, p_gb, pr0, pr1);
        const int src = 16 * (wave >> 1);
        psc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                  __builtin_bit_cast(int, (wave & 1) ? pc.sc1 : pc.sc0), src));
        psh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                  __builtin_bit_cast(int, (wave & 1) ? pc.sh1 : pc.sh0), src));
        const unsigned pcu = line_phase(p_unit, p_i0);
        for (int s = 0; s < SPS; ++s) {
            gather_step(r - 1, s, pcu, held0);
            emit_step(s, pyr, pcu, true, held0);
        }
    }
}

__global__ void zero_words_kernel(unsigned *p, long long n)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

struct Geometry {
    int S, NEXT;
};

// S slices of SPS steps; the NST - S * SPS tail steps become 16 extra row
// tiles each, at most one per slice (so at most 4 rows lie past the slices,
// whose column pixels slice 0's column tile takes).
bool geometry(int Ho, Geometry &g)
{
    const int NST = (Ho + 1) / 2;
    g.S = NST / SPS < MAX_S ? NST / SPS : MAX_S;
    if (g.S < 1) return false;
    const int tail = NST - g.S * SPS;
    g.NEXT = 16 * tail;
    return g.NEXT <= g.S;
}

// Resident workgroups per CU of each instantiation and the CU count, cached per
// device; concurrent first calls store the same values.
struct Occupancy {
    std::atomic<int> blocks_per_cu[5][4];  // [activation][input type / contraction]
    std::atomic<int> cus;
};

template <int ACT, int DT>
hipError_t launch_t(const ConvT2dArgs &p, hipStream_t st)
{
    Geometry geo;
    if (!geometry(p.Ho, geo)) return hipErrorInvalidValue;
    const LaunchHooks &hk = hooks();
    static Occupancy occ[64];  // zero-initialised (static storage)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Occupancy *o = dev >= 0 && dev < 64 ? &occ[dev] : nullptr;
    int nb = o ? o->blocks_per_cu[ACT][DT].load(std::memory_order_relaxed) : 0;
    int cus = o ? o->cus.load(std::memory_order_relaxed) : 0;
    if (nb == 0 || cus == 0) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, convt2d_gn_fused_kernel<ACT, DT>,
                                                         THREADS, 0);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (o) {
            o->blocks_per_cu[ACT][DT].store(nb, std::memory_order_relaxed);
            o->cus.store(cus, std::memory_order_relaxed);
        }
    }
    const int resident = nb * cus;
    const int U = p.N * p.groups;
    int upr = resident / geo.S;
    if (upr < 1 || hk.force_fallback) return hipErrorCooperativeLaunchTooLarge;
    if (upr > U) upr = U;
    if (hk.max_units_per_round > 0 && upr > hk.max_units_per_round) upr = hk.max_units_per_round;
    const int xcd_units = upr % NXCD == 0 ? upr / NXCD : 0;

    // workspace: [U][S][4] partials, zeroed (the flag word sits at p.flag)
    const long long words = (long long)U * geo.S * 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<unsigned *>(p.partials), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    FusedArgs fa{p.x, p.w, p.b, p.gamma, p.beta, p.out, p.partials, p.flag,
                 hk.spin_limit > 0 ? hk.spin_limit : SPIN_LIMIT, hk.never_ready,
                 p.N, p.C_out, p.H, p.groups, p.Ho,
                 geo.S, geo.NEXT, upr, xcd_units, p.eps, p.inv_div};
    void *args[] = {&fa};
    if ((e = dominant_begin(st)) != hipSuccess) return e;
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(convt2d_gn_fused_kernel<ACT, DT>),
                                   dim3(upr * geo.S), dim3(THREADS), args, 0, st);
    if (e != hipSuccess) return e;
    return dominant_end(st);
}

// Slices of the upsampling kernel: SPS input rows each, at most UMAX_S (0 if H
// does not split so).
int ups_slices(int H)
{
    return H >= SPS && H % SPS == 0 && H / SPS <= UMAX_S ? H / SPS : 0;
}

template <int ACT, bool SPLIT>
hipError_t launch_ups_t(const ConvT2dArgs &p, hipStream_t st)
{
    const int S = ups_slices(p.H);
    if (!S || p.W != UW || p.Ho != 2 * p.H) return hipErrorInvalidValue;
    const LaunchHooks &hk = hooks();
    static std::atomic<int> blocks_per_cu[64][5][2], cus_cache[64];  // zero-initialised
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cache = dev >= 0 && dev < 64;
    int nb = cache ? blocks_per_cu[dev][ACT][SPLIT].load(std::memory_order_relaxed) : 0;
    int cus = cache ? cus_cache[dev].load(std::memory_order_relaxed) : 0;
    if (nb == 0 || cus == 0) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, upsample2_gn_fused_kernel<ACT, SPLIT>, THREADS, 0);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (cache) {
            blocks_per_cu[dev][ACT][SPLIT].store(nb, std::memory_order_relaxed);
            cus_cache[dev].store(cus, std::memory_order_relaxed);
        }
    }
    const int U = p.N * p.groups;
    int upr = nb * cus / S;
    if (upr < 1 || hk.force_fallback) return hipErrorCooperativeLaunchTooLarge;
    if (upr > U) upr = U;
    if (hk.max_units_per_round > 0 && upr > hk.max_units_per_round) upr = hk.max_units_per_round;
    const int xcd_units = upr % NXCD == 0 ? upr / NXCD : 0;

    const long long words = (long long)U * S * 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<unsigned *>(p.partials), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    FusedArgs fa{p.x, p.w, p.b, p.gamma, p.beta, p.out, p.partials, p.flag,
                 hk.spin_limit > 0 ? hk.spin_limit : SPIN_LIMIT, hk.never_ready,
                 p.N, p.C_out, p.H, p.groups, p.Ho, S, 0, upr, xcd_units, p.eps, p.inv_div};
    void *args[] = {&fa};
    if ((e = dominant_begin(st)) != hipSuccess) return e;
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(upsample2_gn_fused_kernel<ACT, SPLIT>),
                                   dim3(upr * S), dim3(THREADS), args, 0, st);
    if (e != hipSuccess) return e;
    return dominant_end(st);
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
           (act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF || act == ACT_GELU_TANH);
}

size_t convt2d_fused_workspace(int N, int groups, int Ho)
{
    const size_t U = (size_t)N * groups;
    return U * (size_t)convt2d_fused_slices(Ho) * 4 * sizeof(float);
}

template <int DT>
hipError_t launch_dt(const ConvT2dArgs &a, hipStream_t st)
{
    switch (a.act) {
    case ACT_NONE: return launch_t<ACT_NONE, DT>(a, st);
    case ACT_HARDSWISH: return launch_t<ACT_HARDSWISH, DT>(a, st);
    case ACT_GELU_ERF: return launch_t<ACT_GELU_ERF, DT>(a, st);
    case ACT_GELU_TANH: return launch_t<ACT_GELU_TANH, DT>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_convt2d_fused(const ConvT2dArgs &a, hipStream_t st)
{
    switch (a.dtype) {
    case 0: return launch_dt<0>(a, st);
    case 1: return launch_dt<1>(a, st);
    case 2: return launch_dt<2>(a, st);
    case 3: return launch_dt<3>(a, st);
    default: return hipErrorInvalidValue;
    }
}

bool upsample2_fused_supported(int C_in, int C_out, int groups, int H, int W_, int act, int norm,
                               int num_groups)
{
    return W_ == UW && C_in == CG * groups && C_out == CG * groups && ups_slices(H) > 0 &&
           norm == 1 /* group */ && num_groups == groups &&
           (act == ACT_NONE || act == ACT_HARDSWISH || act == ACT_GELU_ERF || act == ACT_GELU_TANH);
}

size_t upsample2_fused_workspace(int N, int groups, int H)
{
    return (size_t)N * groups * (size_t)ups_slices(H) * 4 * sizeof(float);
}

template <bool SPLIT>
hipError_t launch_ups_act(const ConvT2dArgs &a, hipStream_t st)
{
    switch (a.act) {
    case ACT_NONE: return launch_ups_t<ACT_NONE, SPLIT>(a, st);
    case ACT_HARDSWISH: return launch_ups_t<ACT_HARDSWISH, SPLIT>(a, st);
    case ACT_GELU_ERF: return launch_ups_t<ACT_GELU_ERF, SPLIT>(a, st);
    case ACT_GELU_TANH: return launch_ups_t<ACT_GELU_TANH, SPLIT>(a, st);
    default: return hipErrorInvalidValue;
    }
}

// dtype 0: fp32 on the vector unit; 3: fp32 operands as bf16 pieces on the MFMA
hipError_t launch_upsample2_fused(const ConvT2dArgs &a, hipStream_t st)
{
    if (a.dtype == 0) return launch_ups_act<false>(a, st);
    if (a.dtype == 3) return launch_ups_act<true>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace cnf
