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

// Rotate right by N lanes inside each row of 16 lanes (DPP row_ror).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    static_assert(N >= 1 && N <= 15, "row_ror amount");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                             0x120 + N, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ int row_ror_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, 0x120 + N, 0xf, 0xf, false);
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

enum : int { ACT_NONE = 0, ACT_HARDSWISH = 1, ACT_GELU_ERF = 2, ACT_SOFTMAX = 3 };

__device__ __forceinline__ float hardswish(float x) {
    return x * fminf(fmaxf(x + 3.0f, 0.0f), 6.0f) * (1.0f / 6.0f);
}

// Exact (erf) GELU, x * Phi(x), through the device math library's erff.
__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

template <int ACT>
__device__ __forceinline__ float activate(float x) {
    if constexpr (ACT == ACT_HARDSWISH) return hardswish(x);
    else if constexpr (ACT == ACT_GELU_ERF) return gelu_erf(x);
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
