// kernels.h -- internal interface between the plan/dispatch layer and the
// HIP kernel families.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cnf {

// ---- Per-call launch hooks, set by the C ABI for the duration of one
//      cnf_forward call on the calling thread (defaults otherwise):
//      events recorded on the launch stream right before and right after the
//      plan's dominant kernel, and test knobs of the single-write transposed
//      conv read from the environment when the plan was created.
struct LaunchHooks {
    void *before = nullptr, *after = nullptr;  // hipEvent_t or null
    int spin_limit = 0;            // > 0: polls before a cross-workgroup wait gives up
    int never_ready = 0;           // 1: every such wait also needs a word nobody writes
    int force_fallback = 0;        // 1: act as if the cooperative grid could not be resident
    int max_units_per_round = 0;   // > 0: cap on units per round (more rounds)
};
const LaunchHooks &hooks();
void set_hooks(const LaunchHooks *h);  // null: defaults
// Record hooks().before / .after on st (no-ops when unset).
hipError_t dominant_begin(hipStream_t st);
hipError_t dominant_end(hipStream_t st);

// ---- Conv3d (C_out 16, k 4) + act + GroupNorm + mean over D,H,W
struct Conv3dGnMeanArgs {
    const float *x, *w, *b, *gamma, *beta;
    float *out;
    int N, C_in, D, H, W;
    int act, num_groups;
    float eps, inv_div;
};
bool conv3d_gn_mean_supported(int C_in, int C_out, int kernel, int D, int H, int W, int act);
size_t conv3d_gn_mean_lds_bytes(int C_in);
hipError_t launch_conv3d_gn_mean(const Conv3dGnMeanArgs &a, hipStream_t st);

// ---- Conv3d (C_out 16) + channel softmax + 4x4x4 max pool (+ argmax)
struct Conv3dSoftmaxPoolArgs {
    const float *x, *w, *b;
    float *out;
    int32_t *argmax;
    int N, C_in, D, H, W, kernel;
    int Do, Ho, Wo;      // conv output extents
    int Dp, Hp, Wp;      // pooled extents
    int act;
    int two_stage;       // 1: tie order of two 2-pools; 0: one 4-pool
};
bool conv3d_softmax_pool_supported(int C_in, int C_out, int kernel, int act, int pool_total);
hipError_t launch_conv3d_softmax_pool(const Conv3dSoftmaxPoolArgs &a, hipStream_t st);

// ---- small conv (C_out 16), one workgroup per sample, norm + divide
//      applied in registers, full output written once
struct SmallConvNormArgs {
    const float *x, *w, *b, *gamma, *beta;
    float *out;
    int N, C_in, D, H, W, kernel;
    int Do, Ho, Wo;
    int act, norm_groups;  // norm_groups 0: no norm
    float eps, inv_div;
    int reduce_mean;
};
bool small_conv_norm_supported(int C_in, int C_out, int kernel, int ndim, int D, int H, int W,
                               int act);
hipError_t launch_small_conv_norm(const SmallConvNormArgs &a, hipStream_t st);

// ---- Conv2d implicit GEMM on fp32 MFMA (C_out 128 or 64, k 3) writing y and
//      per-tile Welford partials, then in-place InstanceNorm/GroupNorm + divide;
//      stride 1 or 2; also a dense stride-1 ConvTranspose2d (input padded by 2,
//      kernel flipped)
struct Conv2dIgemmArgs {
    const void *x, *w;   // element type dtype
    const float *b, *gamma, *beta;
    float *out;
    float *partials;     // workspace: [N][tiles][C_out][3], then the weight copy
    int N, C_in, C_out, H, W;
    int Ho, Wo;
    int pad;             // zero padding of the input on every side
    int transposed;      // weights are [C_in][C_out][k][k] (transposed conv)
    int act;
    int norm_groups;     // 0: no norm; C_out: instance norm
    float eps, inv_div;
    int stride = 1;      // 1 or 2 (a transposed conv: 1)
    int dtype = 0;       // 0 fp32; 1 bf16 / 2 fp16 x and w (stride 1, no padding, W % 8 == 0,
                         // C_in % 16 == 0: v_mfma_f32_32x32x16 on a channel-innermost halo)
};
// H, W: the input extents after the zero padding the kernel applies
bool conv2d_igemm_supported(int C_in, int C_out, int kernel, int groups, int H, int W, int act,
                            int stride = 1);
bool conv2d_igemm16_supported(int C_in, int C_out, int kernel, int groups, int H, int W, int act);
size_t conv2d_igemm_workspace(int N, int C_in, int C_out, int Ho, int Wo, int dtype = 0);
hipError_t launch_conv2d_igemm(const Conv2dIgemmArgs &a, hipStream_t st);

// ---- grouped ConvTranspose2d (8 in / 8 out per group, k 3, stride 1) +
//      act writing y and per-tile Welford partials, then in-place GroupNorm
struct ConvT2dArgs {
    const float *x, *w, *b, *gamma, *beta;  // x, w: element type dtype
    float *out;
    float *partials;     // workspace
    int N, C_in, C_out, H, W, groups;
    int Ho, Wo;
    int act;
    int norm_groups;     // 0: no norm; else GroupNorm groups (C_out: InstanceNorm)
    float eps, inv_div;
    int dtype = 0;       // 0 fp32; 1 bf16 / 2 fp16 x and w; 3 fp32 on bf16 pieces (single-write kernels only)
    int *flag = nullptr; // single-write kernel: raised (1) if a cross-workgroup wait gave up
};
bool convt2d_supported(int C_in, int C_out, int kernel, int groups, int H, int W, int act,
                       int norm, int num_groups);
size_t convt2d_workspace(int N, int C_out, int Ho, int Wo);  // [N][C_out][row blocks][3]
hipError_t launch_convt2d(const ConvT2dArgs &a, hipStream_t st);
// single-write variant (W == 256, GroupNorm groups == conv groups): cooperative
// persistent kernel; returns hipErrorCooperativeLaunchTooLarge (and launches
// nothing) if the grid cannot be made co-resident.  Takes fp32, bf16 or fp16 x
// and w (dtype).  The caller zeroes *flag before the launch.
bool convt2d_fused_supported(int C_in, int C_out, int groups, int H, int W, int act, int norm,
                             int num_groups);
size_t convt2d_fused_workspace(int N, int groups, int Ho);
hipError_t launch_convt2d_fused(const ConvT2dArgs &a, hipStream_t st);
// The same single-write scheme for the stride-2 upsampling form (k 3, padding
// 1, output_padding 1, 8 -> 8 channels per group, input width 128, H a
// multiple of 4 up to 128), fp32; hipErrorCooperativeLaunchTooLarge when the
// grid cannot be co-resident (the caller falls back to the general family).
bool upsample2_fused_supported(int C_in, int C_out, int groups, int H, int W, int act, int norm,
                               int num_groups);
size_t upsample2_fused_workspace(int N, int groups, int H);
hipError_t launch_upsample2_fused(const ConvT2dArgs &a, hipStream_t st);

// ---- general family: any validated descriptor (2-D or 3-D, conv or
//      transposed conv, groups, stride, padding, dilation, output_padding,
//      every activation / norm / reduction).  Up to five launches: conv
//      (MFMA implicit GEMM, gathered from L2) + act + per-tile statistics,
//      channel softmax, statistics finalize, in-place normalise, max-pool passes.
struct GenericArgs {
    const void *x, *w;           // element type `dtype` (cnf_dtype)
    const float *b, *gamma, *beta;
    float *out;
    int32_t *argmax;
    void *workspace;
    int N, C_in, C_out, groups, ndim, transposed;
    int D, H, W;                 // input extents (D = 1 for 2-D)
    int Do, Ho, Wo;              // conv output extents
    int kd, kh, kw;              // kernel extents (kd = 1 for 2-D)
    int sd, sh, sw;              // stride per axis
    int pd, ph, pw;              // zero padding per axis (transposed: the conv's padding)
    int dd, dh, dw;              // dilation per axis
    int act;
    int norm_groups;             // 0: no norm; C_out: instance norm
    float eps, inv_div;
    int reduce;                  // cnf_reduce
    int pool_kernel, pool_repeats;
    int argmax_wanted;
    int dtype;                   // 0 fp32, 1 bf16, 2 fp16 (x and w)
};
bool generic_supported(const GenericArgs &a);
// The general family's conv stage for a 2-D ConvTranspose2d, k 3, stride 2,
// padding 1, output_padding 1, conv groups of 8 in / 8 out channels, fp32, no
// softmax or reduction: direct VALU kernel.  mode 0 writes act(conv) *
// out_scale to y and, when part is not null, [N][C_out][T] (count, mean, M2, 0)
// records (T >= upsample2_tiles); mode 1 writes only the records; mode 2
// writes act(conv) * ss.x + ss.y with ss the [N][C_out] (scale, shift) pairs.
bool upsample2_supported(const GenericArgs &a);
int upsample2_tiles(int H, int W);
hipError_t launch_upsample2(const GenericArgs &a, float *y, void *part, int T, float out_scale,
                            const void *ss, int mode, hipStream_t st);
size_t generic_workspace(const GenericArgs &a);
hipError_t launch_generic(const GenericArgs &a, hipStream_t st);

}  // namespace cnf
