// device.h -- gfx950 device helpers shared by the HIP kernels of this library:
// fp32 MFMA wrappers, wave64 DPP row reductions, activations and the
// Welford / Chan statistics merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cnf {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// D(16x16) += A(16x4) * B(4x16).  Lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; D element [4*(l/16)+r][l%16] lives in register r of lane l.
__device__ __forceinline__ v4f mfma_16x16x4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D(32x32) += A(32x2) * B(2x32).  Lane l supplies A[l%32][l/32] and
// B[l/32][l%32]; D element [8*(r/4) + 4*(l/32) + r%4][l%32] lives in register r.
__device__ __forceinline__ v16f mfma_32x32x2(float a, float b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// D(16x16) += A(16x32) B(32x16) on bf16 operands: lane l supplies
// A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16], e = 0..7, two per word (low
// half first); D element [4(l/16) + r][l%16] lives in register r of lane l
// (the layout of mfma_16x16x4 above).
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v4u a, v4u b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- fp32 operands as three bf16 pieces (f32_math = BF16X3)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> one word of two bf16 (round to nearest even, low half first).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v2f{lo, hi}, bf16x2));
}

// Three bf16 pieces of each of two fp32 values, v = p1 + p2 + p3 exactly:
// p1 = bf16(v) leaves a remainder r = v - p1 that is exact (Sterbenz) and
// at most 2^-8 |v| with at most 16 significant bits; p2 = bf16(r) leaves at
// most 8 bits, which p3 holds exactly.  Words w1, w2, w3 hold the pieces of
// (lo, hi).  (Below 2^-100 in magnitude p3 can be a bf16 subnormal.)
struct Pieces {
    unsigned w1, w2, w3;
};
__device__ __forceinline__ Pieces split3(float lo, float hi)
{
    Pieces p;
    p.w1 = pack_bf16(lo, hi);
    const float rl = lo - __builtin_bit_cast(float, p.w1 << 16),
                rh = hi - __builtin_bit_cast(float, p.w1 & 0xffff0000u);
    p.w2 = pack_bf16(rl, rh);
    const float sl = rl - __builtin_bit_cast(float, p.w2 << 16),
                sh = rh - __builtin_bit_cast(float, p.w2 & 0xffff0000u);
    p.w3 = pack_bf16(sl, sh);
    return p;
}

__device__ __forceinline__ void put_pieces(v4u (&dst)[3], int d, const Pieces &p)
{
    dst[0][d] = p.w1;
    dst[1][d] = p.w2;
    dst[2][d] = p.w3;
}

// The six leading piece products, smallest first: (A piece, B piece) of
// w3x1, w2x2, w1x3, w2x1, w1x2, w1x1; the three dropped ones total at most
// about 2^-23 |w x|.
constexpr int PIECE_A[6] = {2, 1, 0, 1, 0, 0}, PIECE_B[6] = {0, 1, 2, 0, 1, 0};

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and stores past it are dropped; offsets are 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// Resources built here span fewer than RES_MAX bytes, so GOOB is past the end of
// every one of them: a lane that must not touch memory passes GOOB as its offset.
constexpr unsigned GOOB = 0x7ff00000u;
constexpr unsigned RES_MAX = 0x7f000000u;
__device__ __forceinline__ v4f buf_load4(__amdgpu_buffer_rsrc_t r, unsigned byte_off,
                                         unsigned uniform_off = 0) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off,
                                                                        (int)uniform_off, 0));
}
__device__ __forceinline__ float buf_load1(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}
__device__ __forceinline__ v2f buf_load2(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_bit_cast(v2f, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0));
}
// 4-byte store (dropped when the per-lane offset is past the end; a uniform
// offset rides in the scalar operand).
__device__ __forceinline__ void buf_store1(float v, __amdgpu_buffer_rsrc_t r, unsigned byte_off,
                                           unsigned uniform_off = 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)byte_off,
                                          (int)uniform_off, 0);
}
// 8-byte store, and its non-temporal (streaming) form.
__device__ __forceinline__ void buf_store2(v2f v, __amdgpu_buffer_rsrc_t r, unsigned byte_off,
                                           unsigned uniform_off = 0) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, (int)byte_off,
                                          (int)uniform_off, 0);
}

__device__ __forceinline__ void buf_store2_nt(v2f v, __amdgpu_buffer_rsrc_t r, unsigned byte_off,
                                              unsigned uniform_off = 0) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, (int)byte_off,
                                          (int)uniform_off, 2);
}

// Workgroups are dispatched round-robin over the XCDs (linear workgroup id
// L runs on XCD L % NXCD), and each XCD has its own L2.  xcd_remap turns L
// into a tile index such that every XCD gets one contiguous range of tiles,
// so neighbouring tiles (which share input halos) hit the same L2.
// Bijective on [0, total) for any total.
constexpr int NXCD = 8;
__device__ __forceinline__ int xcd_remap(int L, int total) {
    const int q = total / NXCD, r = total % NXCD;
    const int x = L % NXCD, k = L / NXCD;
    return x * q + (x < r ? x : r) + k;
}

// Rotate right by N lanes inside each row of 16 lanes (DPP row_ror).
// (bound_ctrl set: every lane of a row rotation has a source, and this form lets
// the compiler fold the move into the consuming VALU op as a DPP operand.)
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    static_assert(N >= 1 && N <= 15, "row_ror amount");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0x120 + N, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ int row_ror_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, 0x120 + N, 0xf, 0xf, false);
}
// Every lane of a 16-lane row gets the row's minimum (int).  bound_ctrl is set,
// as in row_ror, so each rotation folds into v_min_i32 as a DPP operand.
template <int N>
__device__ __forceinline__ int row_ror_ib(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x120 + N, 0xf, 0xf, true);
}
__device__ __forceinline__ int row_min16_i(int v) {
    v = min(v, row_ror_ib<8>(v));
    v = min(v, row_ror_ib<4>(v));
    v = min(v, row_ror_ib<2>(v));
    v = min(v, row_ror_ib<1>(v));
    return v;
}

// Every lane of a 16-lane row gets the row's max / sum.
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<2>(v));
    v = fmaxf(v, row_ror<1>(v));
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    v += row_ror<1>(v);
    return v;
}

enum : int { ACT_NONE = 0, ACT_HARDSWISH = 1, ACT_GELU_ERF = 2, ACT_SOFTMAX = 3, ACT_GELU_TANH = 4 };

__device__ __forceinline__ float hardswish(float x) {
    return x * fminf(fmaxf(x + 3.0f, 0.0f), 6.0f) * (1.0f / 6.0f);
}

// Exact (erf) GELU, gelu(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in
// logistic form x * Phi(x) ~= x * sigma(x P(x^2)): the log-odds of the
// standard normal CDF is an odd function, and an odd degree-9 polynomial
// fitted to it (minimax on |x * (sigma(f(x)) - Phi(x))| over [-12, 12],
// weighted by the GELU error it causes) keeps the result within 3.5e-6 of
// x * Phi(x) for every finite x, fp32 rounding included (the tanh form below
// is the degree-3 member of this family, 4.7e-4 off; Abramowitz & Stegun's
// erfc formula 7.1.26 reaches 1.5e-7 but costs 11 VALU ops + rcp + exp2).
// P > 0 on [0, inf), so the log-odds run to +-inf with x: the result tends to
// x and to -0, never NaN.  With -log2(e) folded into P:
// x / (1 + exp2(x P'(x^2))), 7 VALU ops + exp2 + rcp.
__device__ __forceinline__ float gelu_erf(float x) {
    const float u = x * x;
    float p = fmaf(u, -3.230937637e-06f, 8.828550199e-05f);
    p = fmaf(u, p, 3.599097254e-04f);
    p = fmaf(u, p, -1.052256599e-01f);
    p = fmaf(u, p, -2.302046299e+00f);
    const float e = __builtin_amdgcn_exp2f(x * p);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Tanh form of GELU, 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// With 1 + tanh(u) = 2 / (1 + exp(-2u)) it is x / (1 + exp2(x (a + b x^2))),
// a = -2 sqrt(2/pi) log2(e), b = 0.044715 a: 6 VALU ops + exp2 + rcp.  For
// x -> -inf the exponential overflows to +inf and the result is -0.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float e = __builtin_amdgcn_exp2f(x * fmaf(x * x, -1.029432396e-01f, -2.302208198e+00f));
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int ACT>
__device__ __forceinline__ float activate(float x) {
    if constexpr (ACT == ACT_HARDSWISH) return hardswish(x);
    else if constexpr (ACT == ACT_GELU_ERF) return gelu_erf(x);
    else if constexpr (ACT == ACT_GELU_TANH) return gelu_tanh(x);
    else return x;
}

// Chan et al. merge of Welford triples (count, mean, M2): (n, mean, m2) += (nb, meanb, m2b).
__device__ __forceinline__ void chan_merge(float &n, float &mean, float &m2,
                                           float nb, float meanb, float m2b) {
    const float nn = n + nb;
    if (nn > 0.0f) {
        const float delta = meanb - mean;
        const float f = nb / nn;
        mean = mean + delta * f;
        m2 = m2 + m2b + delta * delta * n * f;
    }
    n = nn;
}

// Welford update with one new value; rn = 1 / (count after the update).
__device__ __forceinline__ void welford_push(float &mean, float &m2, float v, float rn) {
    const float delta = v - mean;
    mean = mean + delta * rn;
    m2 = m2 + delta * (v - mean);
}

// Chan-merge of triples across the 16 lanes of each row; every lane ends
// with the row total.
__device__ __forceinline__ void row_chan16(float &n, float &mean, float &m2) {
#define CNF_ROW_STEP(S)                                                   \
    {                                                                     \
        const float nb = row_ror<S>(n), mb = row_ror<S>(mean), qb = row_ror<S>(m2); \
        chan_merge(n, mean, m2, nb, mb, qb);                              \
    }
    CNF_ROW_STEP(8) CNF_ROW_STEP(4) CNF_ROW_STEP(2) CNF_ROW_STEP(1)
#undef CNF_ROW_STEP
}

}  // namespace cnf
