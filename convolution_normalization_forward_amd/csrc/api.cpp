// api.cpp -- the C ABI declared in include/cnf.h: descriptor validation,
// output-shape and workspace arithmetic, kernel-family selection and the
// launch of the chosen family on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "cnf.h"
#include "kernels.h"

namespace {

enum Family : int {
    FAM_GN_MEAN = 1,       // Conv3d k4 C_out 16 + act + GroupNorm + mean, fully fused
    FAM_SOFTMAX_POOL = 2,  // Conv3d C_out 16 + channel softmax + 4^3 max pool
    FAM_SMALL = 3,         // small conv C_out 16, one workgroup per sample
    FAM_IGEMM = 4,         // Conv2d C_out 128/64 k3 implicit GEMM (also dense stride-1 ConvTranspose2d) + norm pass
    FAM_CONVT = 5,         // grouped ConvTranspose2d 8x8 per group + act + GroupNorm pass
    FAM_CONVT_FUSED = 6,   // same, single write: cooperative kernel, cross-workgroup merge
    FAM_GENERIC = 7,       // any validated descriptor: gathered implicit GEMM + passes
    FAM_IGEMM16 = 8,       // Conv2d C_out 128/64 k3, 16-bit x and w: implicit GEMM on 32x32x16 MFMA + norm pass
    FAM_UPS2_FUSED = 9     // stride-2 upsampling grouped ConvTranspose2d + act + GroupNorm, single write
};

const char *family_name(int f)
{
    switch (f) {
    case FAM_GN_MEAN: return "conv3d_k4_gn_mean(fused,1wg/sample,mfma16x16x4)";
    case FAM_SOFTMAX_POOL: return "conv3d_softmax_pool4(1wave/window,mfma16x16x4)";
    case FAM_SMALL: return "small_conv_norm(1wg/sample,mfma16x16x4)";
    case FAM_IGEMM: return "conv2d_igemm(mfma32x32x2)+norm_finalize+apply";
    case FAM_CONVT: return "convt2d_grouped8(mfma16x16x4,column-pair)+groupnorm_pass";
    case FAM_CONVT_FUSED: return "convt2d_grouped8_gn_fused(cooperative,single-write)";
    case FAM_GENERIC: return "generic(gathered-igemm mfma16x16x4 + softmax/finalize/apply/pool passes)";
    case FAM_IGEMM16: return "conv2d_igemm16(mfma32x32x16,channel-innermost halo)+norm_finalize+apply";
    case FAM_UPS2_FUSED: return "convt2d_s2_grouped8_gn_fused(cooperative,single-write,valu)";
    default: return "none";
    }
}

}  // namespace

struct cnf_plan {
    cnf_desc d;
    int family;
    int Do, Ho, Wo;     // conv output extents (Do = 1 for 2-D)
    int Dp, Hp, Wp;     // pooled extents
    int64_t dims[5];
    int32_t rank;
    size_t workspace;
    size_t flag_offset; // single-write transposed conv: byte offset of its wait flag
    int igemm_pad;      // zero padding the implicit GEMM applies to the input
    int igemm_stride;   // its stride (1 or 2)
    cnf::LaunchHooks knobs;  // test knobs read from the environment at creation
};

namespace {
// fp32 x and w contracted as bf16 pieces: asked for, and the plan's kernel has
// that form (the two single-write transposed-conv kernels)
bool split_f32(const cnf_plan &p)
{
    return (p.family == FAM_CONVT_FUSED || p.family == FAM_UPS2_FUSED) && p.d.dtype == CNF_DTYPE_F32 &&
           p.d.f32_math == CNF_F32_BF16X3;
}
}  // namespace

namespace cnf {

namespace {
thread_local const LaunchHooks *t_hooks = nullptr;
const LaunchHooks k_default_hooks{};
}  // namespace

const LaunchHooks &hooks() { return t_hooks ? *t_hooks : k_default_hooks; }
void set_hooks(const LaunchHooks *h) { t_hooks = h; }

hipError_t dominant_begin(hipStream_t st)
{
    const LaunchHooks &h = hooks();
    return h.before ? hipEventRecord(static_cast<hipEvent_t>(h.before), st) : hipSuccess;
}

hipError_t dominant_end(hipStream_t st)
{
    const LaunchHooks &h = hooks();
    return h.after ? hipEventRecord(static_cast<hipEvent_t>(h.after), st) : hipSuccess;
}

}  // namespace cnf

namespace {

// Hooks of one cnf_forward call, in place for its duration on this thread.
struct HookScope {
    explicit HookScope(const cnf::LaunchHooks *h) { cnf::set_hooks(h); }
    ~HookScope() { cnf::set_hooks(nullptr); }
};

int env_int(const char *name)
{
    const char *v = std::getenv(name);
    return v ? std::atoi(v) : 0;
}

__global__ void clear_word_kernel(int *p) { *p = 0; }

// The general family's arguments for a plan (pointers may be null when only
// the workspace size or the limits are wanted).
cnf::GenericArgs generic_args(const cnf_plan &p, const void *x, const void *w, const float *b,
                              const float *gamma, const float *beta, float *out, int32_t *argmax,
                              void *workspace, int norm_groups)
{
    const cnf_desc &d = p.d;
    const bool three = d.ndim == 3;
    cnf::GenericArgs a{};
    a.x = x; a.w = w; a.b = b; a.gamma = gamma; a.beta = beta;
    a.out = out; a.argmax = argmax; a.workspace = workspace;
    a.N = d.N; a.C_in = d.C_in; a.C_out = d.C_out; a.groups = d.groups; a.ndim = d.ndim;
    a.transposed = d.kind == CNF_CONV_TRANSPOSE;
    a.D = d.in_dims[0]; a.H = d.in_dims[1]; a.W = d.in_dims[2];
    a.Do = p.Do; a.Ho = p.Ho; a.Wo = p.Wo;
    a.kd = three ? d.kernel : 1; a.kh = d.kernel; a.kw = d.kernel;
    a.sd = three ? d.stride : 1; a.sh = d.stride; a.sw = d.stride;
    a.pd = three ? d.padding : 0; a.ph = d.padding; a.pw = d.padding;
    a.dd = three ? d.dilation : 1; a.dh = d.dilation; a.dw = d.dilation;
    a.act = d.act;
    a.norm_groups = norm_groups;
    a.eps = d.eps;
    a.inv_div = 1.0f / d.divide_by;
    a.reduce = d.reduce;
    a.pool_kernel = d.pool_kernel; a.pool_repeats = d.pool_repeats;
    a.argmax_wanted = d.want_argmax;
    a.dtype = d.dtype;
    return a;
}

}  // namespace

extern "C" {

int32_t cnf_abi_version(void) { return CNF_ABI_VERSION; }

const char *cnf_status_string(cnf_status s)
{
    switch (s) {
    case CNF_OK: return "CNF_OK";
    case CNF_ERR_NULL: return "CNF_ERR_NULL";
    case CNF_ERR_INVALID_DESC: return "CNF_ERR_INVALID_DESC";
    case CNF_ERR_UNSUPPORTED: return "CNF_ERR_UNSUPPORTED";
    case CNF_ERR_WORKSPACE: return "CNF_ERR_WORKSPACE";
    case CNF_ERR_ALIGNMENT: return "CNF_ERR_ALIGNMENT";
    case CNF_ERR_HIP: return "CNF_ERR_HIP";
    case CNF_ERR_ABI: return "CNF_ERR_ABI";
    case CNF_ERR_NOMEM: return "CNF_ERR_NOMEM";
    case CNF_ERR_WAIT_TIMEOUT: return "CNF_ERR_WAIT_TIMEOUT";
    case CNF_ERR_SCRATCH: return "CNF_ERR_SCRATCH";
    }
    return "CNF_ERR_UNKNOWN";
}

cnf_status cnf_plan_create(const cnf_desc *desc, cnf_plan **plan)
{
    if (!plan) return CNF_ERR_NULL;
    *plan = nullptr;
    if (!desc) return CNF_ERR_NULL;
    const cnf_desc &d = *desc;
    if (d.abi_version != CNF_ABI_VERSION) return CNF_ERR_ABI;

    // ---- validation (a self-inconsistent descriptor is INVALID_DESC)
    if (d.ndim != 2 && d.ndim != 3) return CNF_ERR_INVALID_DESC;
    if (d.kind != CNF_CONV && d.kind != CNF_CONV_TRANSPOSE) return CNF_ERR_INVALID_DESC;
    if (d.N < 0 || d.C_in < 1 || d.C_out < 1 || d.kernel < 1 || d.groups < 1)
        return CNF_ERR_INVALID_DESC;
    if (d.C_in % d.groups || d.C_out % d.groups) return CNF_ERR_INVALID_DESC;
    if (d.in_dims[0] < 1 || d.in_dims[1] < 1 || d.in_dims[2] < 1) return CNF_ERR_INVALID_DESC;
    if (d.ndim == 2 && d.in_dims[0] != 1) return CNF_ERR_INVALID_DESC;
    if (d.has_bias != 0 && d.has_bias != 1) return CNF_ERR_INVALID_DESC;
    if (d.act < CNF_ACT_NONE || d.act > CNF_ACT_GELU_TANH) return CNF_ERR_INVALID_DESC;
    if (d.norm < CNF_NORM_NONE || d.norm > CNF_NORM_INSTANCE) return CNF_ERR_INVALID_DESC;
    if (d.reduce < CNF_RED_NONE || d.reduce > CNF_RED_MAXPOOL) return CNF_ERR_INVALID_DESC;
    if (d.affine != 0 && d.affine != 1) return CNF_ERR_INVALID_DESC;
    if (d.want_argmax != 0 && d.want_argmax != 1) return CNF_ERR_INVALID_DESC;
    if (d.norm == CNF_NORM_GROUP && (d.num_groups < 1 || d.C_out % d.num_groups))
        return CNF_ERR_INVALID_DESC;
    if (d.norm != CNF_NORM_NONE && !(d.eps > 0.0f)) return CNF_ERR_INVALID_DESC;
    if (!(d.divide_by == d.divide_by) || d.divide_by == 0.0f) return CNF_ERR_INVALID_DESC;
    if (d.want_argmax && d.reduce != CNF_RED_MAXPOOL) return CNF_ERR_INVALID_DESC;
    if (d.stride < 1 || d.dilation < 1 || d.padding < 0 || d.output_padding < 0)
        return CNF_ERR_INVALID_DESC;
    if (d.kind == CNF_CONV && d.output_padding != 0) return CNF_ERR_INVALID_DESC;
    if (d.dtype != CNF_DTYPE_F32 && d.dtype != CNF_DTYPE_BF16 && d.dtype != CNF_DTYPE_F16)
        return CNF_ERR_INVALID_DESC;
    if (d.f32_math != CNF_F32_NATIVE && d.f32_math != CNF_F32_BF16X3) return CNF_ERR_INVALID_DESC;
    if (d.kind == CNF_CONV_TRANSPOSE &&
        d.output_padding >= (d.stride > d.dilation ? d.stride : d.dilation))
        return CNF_ERR_INVALID_DESC;

    cnf_plan p{};
    p.d = d;
    const int k = d.kernel;
    const int D = d.in_dims[0], H = d.in_dims[1], W = d.in_dims[2];
    // Output extent per axis (64-bit, so huge descriptors are rejected, not wrapped).
    auto extent = [&](int L) -> long long {
        const long long s = d.stride, pd = d.padding, dl = d.dilation;
        if (d.kind == CNF_CONV) {
            const long long num = L + 2 * pd - dl * (k - 1) - 1;
            return num < 0 ? 0 : num / s + 1;
        }
        return (L - 1LL) * s - 2 * pd + dl * (k - 1) + d.output_padding + 1;
    };
    const long long eD = d.ndim == 3 ? extent(D) : 1, eH = extent(H), eW = extent(W);
    if (eD < 1 || eH < 1 || eW < 1) return CNF_ERR_INVALID_DESC;
    if (eD > (1 << 30) || eH > (1 << 30) || eW > (1 << 30) || eD * eH * eW > (1LL << 40))
        return CNF_ERR_UNSUPPORTED;
    p.Do = (int)eD; p.Ho = (int)eH; p.Wo = (int)eW;

    int pool_total = 1;
    p.Dp = p.Do; p.Hp = p.Ho; p.Wp = p.Wo;
    if (d.reduce == CNF_RED_MAXPOOL) {
        if (d.pool_kernel < 1 || d.pool_repeats < 1 || d.pool_repeats > 8)
            return CNF_ERR_INVALID_DESC;
        for (int r = 0; r < d.pool_repeats; ++r) {
            if (d.ndim == 3) p.Dp /= d.pool_kernel;
            p.Hp /= d.pool_kernel;
            p.Wp /= d.pool_kernel;
            pool_total *= d.pool_kernel;
            if (pool_total > 1 << 20) return CNF_ERR_INVALID_DESC;
        }
        if (p.Dp < 1 || p.Hp < 1 || p.Wp < 1) return CNF_ERR_INVALID_DESC;
    }

    if (d.reduce == CNF_RED_MEAN_SPATIAL) {
        p.rank = 2;
        p.dims[0] = d.N; p.dims[1] = d.C_out;
    } else if (d.reduce == CNF_RED_MAXPOOL) {
        p.rank = 5;
        p.dims[0] = d.N; p.dims[1] = d.C_out;
        p.dims[2] = p.Dp; p.dims[3] = p.Hp; p.dims[4] = p.Wp;
    } else {
        p.rank = d.ndim + 2;
        p.dims[0] = d.N; p.dims[1] = d.C_out;
        if (d.ndim == 3) { p.dims[2] = p.Do; p.dims[3] = p.Ho; p.dims[4] = p.Wo; }
        else { p.dims[2] = p.Ho; p.dims[3] = p.Wo; }
    }

    // ---- kernel-family selection (UNSUPPORTED rather than any slow path)
    const int norm_groups = d.norm == CNF_NORM_GROUP ? d.num_groups
                          : d.norm == CNF_NORM_INSTANCE ? d.C_out : 0;
    p.family = 0;
    // The specialised families assume stride 1, no padding, dilation 1; the
    // CNF_FORCE_GENERIC environment variable (tests) sends everything to the
    // general family.
    const char *force = std::getenv("CNF_FORCE_GENERIC");
    // (16-bit inputs: the general family, except the single-write transposed
    // conv below)
    const bool unit = d.stride == 1 && d.dilation == 1 && d.output_padding == 0 &&
                      d.dtype == CNF_DTYPE_F32 && !(force && force[0] == '1');
    const bool basic = unit && d.padding == 0;
    p.igemm_pad = d.kind == CNF_CONV_TRANSPOSE ? k - 1 : 0;
    p.igemm_stride = 1;
    if (!basic) {
        // Stride-1, dilation-1 2-D convs with padding up to k - 1 are the implicit
        // GEMM with that padding; a dense transposed conv with padding p is the
        // GEMM of the flipped kernel with padding k - 1 - p.
        const int gp = d.kind == CNF_CONV ? d.padding : k - 1 - d.padding;
        if (unit && d.ndim == 2 && d.groups == 1 && d.reduce == CNF_RED_NONE &&
            d.padding <= k - 1 &&
            cnf::conv2d_igemm_supported(d.C_in, d.C_out, k, d.groups, H + 2 * gp, W + 2 * gp,
                                        d.act)) {
            p.family = FAM_IGEMM;
            p.igemm_pad = gp;
        }
        // stride-2 2-D convs with padding up to k - 1: the same GEMM at stride 2
        if (d.kind == CNF_CONV && d.stride == 2 && d.dilation == 1 && d.dtype == CNF_DTYPE_F32 &&
            !(force && force[0] == '1') && d.ndim == 2 && d.groups == 1 &&
            d.reduce == CNF_RED_NONE && d.padding <= k - 1 &&
            cnf::conv2d_igemm_supported(d.C_in, d.C_out, k, d.groups, H + 2 * d.padding,
                                        W + 2 * d.padding, d.act, 2)) {
            p.family = FAM_IGEMM;
            p.igemm_pad = d.padding;
            p.igemm_stride = 2;
        }
    } else if (d.kind == CNF_CONV && d.groups == 1) {
        if (d.ndim == 3 && d.reduce == CNF_RED_MEAN_SPATIAL && d.act != CNF_ACT_SOFTMAX_CHANNEL &&
            cnf::conv3d_gn_mean_supported(d.C_in, d.C_out, k, D, H, W, d.act))
            p.family = FAM_GN_MEAN;
        else if (d.ndim == 3 && d.reduce == CNF_RED_MAXPOOL && d.norm == CNF_NORM_NONE &&
                 d.divide_by == 1.0f && (d.pool_kernel == 2 || d.pool_repeats == 1) &&
                 cnf::conv3d_softmax_pool_supported(d.C_in, d.C_out, k, d.act, pool_total))
            p.family = FAM_SOFTMAX_POOL;
        else if (d.reduce != CNF_RED_MAXPOOL &&
                 cnf::small_conv_norm_supported(d.C_in, d.C_out, k, d.ndim, D, H, W, d.act))
            p.family = FAM_SMALL;
        else if (d.ndim == 2 && d.reduce == CNF_RED_NONE &&
                 cnf::conv2d_igemm_supported(d.C_in, d.C_out, k, d.groups, H, W, d.act))
            p.family = FAM_IGEMM;
    } else if (d.kind == CNF_CONV_TRANSPOSE && d.ndim == 2 && d.reduce == CNF_RED_NONE) {
        // dense transposed conv: the implicit GEMM on the input padded by k - 1;
        // 8-channel groups (or a dense 8 -> 8 one): the column-pair kernels
        if (d.groups == 1 && cnf::conv2d_igemm_supported(d.C_in, d.C_out, k, d.groups,
                                                         H + 2 * (k - 1), W + 2 * (k - 1), d.act))
            p.family = FAM_IGEMM;
        else if (cnf::convt2d_supported(d.C_in, d.C_out, k, d.groups, H, W, d.act, d.norm,
                                   d.num_groups))
            p.family = FAM_CONVT;
        if (p.family == FAM_CONVT &&
            cnf::convt2d_fused_supported(d.C_in, d.C_out, d.groups, H, W, d.act, d.norm,
                                         d.num_groups))
            p.family = FAM_CONVT_FUSED;
    }
    // 16-bit x and w of an unpadded stride-1 Conv2d with 64 or 128 output
    // channels: the implicit GEMM on the 16-bit MFMA
    if (!p.family && d.dtype != CNF_DTYPE_F32 && !(force && force[0] == '1') &&
        d.kind == CNF_CONV && d.ndim == 2 && d.groups == 1 && d.reduce == CNF_RED_NONE &&
        d.stride == 1 && d.dilation == 1 && d.padding == 0 &&
        cnf::conv2d_igemm16_supported(d.C_in, d.C_out, k, d.groups, H, W, d.act))
        p.family = FAM_IGEMM16;
    // 16-bit x and w of the single-write transposed-conv shape: that kernel widens
    // them to fp32 as it loads them.  The general family stays its fallback (for a
    // grid that cannot be co-resident), so it must take the descriptor too.
    const cnf::GenericArgs ga = generic_args(p, nullptr, nullptr, nullptr, nullptr, nullptr,
                                             nullptr, nullptr, nullptr, norm_groups);
    if (!p.family && d.dtype != CNF_DTYPE_F32 && !(force && force[0] == '1') &&
        d.kind == CNF_CONV_TRANSPOSE && d.ndim == 2 && d.reduce == CNF_RED_NONE &&
        d.stride == 1 && d.dilation == 1 && d.output_padding == 0 && d.padding == 0 &&
        cnf::convt2d_supported(d.C_in, d.C_out, k, d.groups, H, W, d.act, d.norm, d.num_groups) &&
        cnf::convt2d_fused_supported(d.C_in, d.C_out, d.groups, H, W, d.act, d.norm, d.num_groups) &&
        cnf::generic_supported(ga))
        p.family = FAM_CONVT_FUSED;
    // the stride-2 upsampling transposed conv over 8-channel groups + GroupNorm:
    // the single-write kernel, with the general family as its fallback
    if (!p.family && d.dtype == CNF_DTYPE_F32 && !(force && force[0] == '1') &&
        d.kind == CNF_CONV_TRANSPOSE && d.ndim == 2 && d.reduce == CNF_RED_NONE && k == 3 &&
        d.stride == 2 && d.padding == 1 && d.output_padding == 1 && d.dilation == 1 &&
        cnf::upsample2_fused_supported(d.C_in, d.C_out, d.groups, H, W, d.act, d.norm, d.num_groups) &&
        cnf::generic_supported(ga))
        p.family = FAM_UPS2_FUSED;
    if (!p.family) {
        if (!cnf::generic_supported(ga)) return CNF_ERR_UNSUPPORTED;
        p.family = FAM_GENERIC;
    }

    p.workspace = 0;
    if (p.family == FAM_IGEMM)
        p.workspace = cnf::conv2d_igemm_workspace(d.N, d.C_in, d.C_out, p.Ho, p.Wo);
    if (p.family == FAM_IGEMM16)
        p.workspace = cnf::conv2d_igemm_workspace(d.N, d.C_in, d.C_out, p.Ho, p.Wo, (int)d.dtype);
    if (p.family == FAM_CONVT) p.workspace = cnf::convt2d_workspace(d.N, d.C_out, p.Ho, p.Wo);
    if (p.family == FAM_GENERIC)
        p.workspace = cnf::generic_workspace(generic_args(p, nullptr, nullptr, nullptr, nullptr,
                                                          nullptr, nullptr, nullptr, nullptr,
                                                          norm_groups));
    if (p.family == FAM_CONVT_FUSED) {
        // room for the fallback too (used if the grid cannot be co-resident): the
        // two-pass kernels for fp32 inputs, the general family for 16-bit ones
        const size_t a = cnf::convt2d_fused_workspace(d.N, d.groups, p.Ho);
        const size_t b = d.dtype == CNF_DTYPE_F32 ? cnf::convt2d_workspace(d.N, d.C_out, p.Ho, p.Wo)
                                                  : cnf::generic_workspace(ga);
        p.workspace = a > b ? a : b;
    }

    if (p.family == FAM_UPS2_FUSED) {
        const size_t a = cnf::upsample2_fused_workspace(d.N, d.groups, H), b = cnf::generic_workspace(ga);
        p.workspace = a > b ? a : b;
    }

    p.flag_offset = 0;
    if (p.family == FAM_CONVT_FUSED || p.family == FAM_UPS2_FUSED) {
        // the wait flag after everything either path uses, on its own 16 bytes
        p.flag_offset = (p.workspace + 15) & ~(size_t)15;
        p.workspace = p.flag_offset + 16;
    }
    // Test knobs of the single-write transposed conv (documented in cnf.h):
    // CNF_TEST_FUSED_SPIN_LIMIT, CNF_TEST_FUSED_NEVER_READY,
    // CNF_TEST_FORCE_FALLBACK, CNF_TEST_FUSED_MAX_UNITS_PER_ROUND.
    p.knobs.spin_limit = env_int("CNF_TEST_FUSED_SPIN_LIMIT");
    p.knobs.never_ready = env_int("CNF_TEST_FUSED_NEVER_READY") ? 1 : 0;
    p.knobs.force_fallback = env_int("CNF_TEST_FORCE_FALLBACK") ? 1 : 0;
    p.knobs.max_units_per_round = env_int("CNF_TEST_FUSED_MAX_UNITS_PER_ROUND");

    cnf_plan *np = new (std::nothrow) cnf_plan(p);
    if (!np) return CNF_ERR_NOMEM;
    *plan = np;
    return CNF_OK;
}

cnf_status cnf_plan_output_shape(const cnf_plan *plan, int64_t dims[5], int32_t *rank)
{
    if (!plan || !dims || !rank) return CNF_ERR_NULL;
    for (int i = 0; i < 5; ++i) dims[i] = i < plan->rank ? plan->dims[i] : 0;
    *rank = plan->rank;
    return CNF_OK;
}

cnf_status cnf_plan_workspace_size(const cnf_plan *plan, size_t *bytes)
{
    if (!plan || !bytes) return CNF_ERR_NULL;
    *bytes = plan->workspace;
    return CNF_OK;
}

cnf_status cnf_plan_describe(const cnf_plan *plan, char *buf, size_t len)
{
    if (!plan || !buf) return CNF_ERR_NULL;
    if (len == 0) return CNF_OK;
    const cnf_desc &d = plan->d;
    std::snprintf(buf, len, "family=%s N=%d C_in=%d C_out=%d in=%dx%dx%d k=%d groups=%d "
                  "stride=%d padding=%d dilation=%d output_padding=%d dtype=%s%s out_rank=%d "
                  "workspace=%zu",
                  family_name(plan->family), d.N, d.C_in, d.C_out, d.in_dims[0], d.in_dims[1],
                  d.in_dims[2], d.kernel, d.groups, d.stride, d.padding, d.dilation,
                  d.output_padding,
                  d.dtype == CNF_DTYPE_BF16 ? "bf16" : d.dtype == CNF_DTYPE_F16 ? "f16" : "f32",
                  split_f32(*plan) ? " contraction=bf16x3" : "", plan->rank, plan->workspace);
    return CNF_OK;
}

void cnf_plan_destroy(cnf_plan *plan) { delete plan; }

static bool misaligned(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

}  // extern "C"

namespace {

// cnf_forward with optional events around the plan's dominant kernel.
cnf_status forward_impl(const cnf_plan *plan, const void *xv, const void *wv, const float *b,
                        const float *gamma, const float *beta, float *out, int32_t *argmax,
                        void *workspace, size_t workspace_bytes, void *stream, void *ev_before,
                        void *ev_after)
{
    if (!plan) return CNF_ERR_NULL;
    const cnf_desc &d = plan->d;
    // fp32 views for the fp32-only families (16-bit inputs only reach the general one)
    const float *x = static_cast<const float *>(xv), *w = static_cast<const float *>(wv);
    const bool need_affine = d.norm != CNF_NORM_NONE && d.affine;
    if (!x || !w || !out) return CNF_ERR_NULL;
    if ((b != nullptr) != (d.has_bias != 0)) return CNF_ERR_NULL;
    if ((gamma != nullptr) != need_affine || (beta != nullptr) != need_affine) return CNF_ERR_NULL;
    if ((argmax != nullptr) != (d.want_argmax != 0)) return CNF_ERR_NULL;
    if (misaligned(x) || misaligned(w) || misaligned(b) || misaligned(gamma) ||
        misaligned(beta) || misaligned(out) || misaligned(argmax) || misaligned(workspace))
        return CNF_ERR_ALIGNMENT;
    if (plan->workspace > 0 && (!workspace || workspace_bytes < plan->workspace))
        return CNF_ERR_WORKSPACE;
    if (d.N == 0) return CNF_OK;

    cnf::LaunchHooks hk = plan->knobs;
    hk.before = ev_before;
    hk.after = ev_after;
    HookScope scope(&hk);

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const float inv_div = 1.0f / d.divide_by;
    const int D = d.in_dims[0], H = d.in_dims[1], W = d.in_dims[2];
    const int norm_groups = d.norm == CNF_NORM_GROUP ? d.num_groups
                          : d.norm == CNF_NORM_INSTANCE ? d.C_out : 0;
    hipError_t e = hipSuccess;
    // single-launch families: the events bracket the whole call
    auto single = [&](auto &&launch) {
        hipError_t r = cnf::dominant_begin(st);
        if (r != hipSuccess) return r;
        if ((r = launch()) != hipSuccess) return r;
        return cnf::dominant_end(st);
    };
    switch (plan->family) {
    case FAM_GN_MEAN: {
        cnf::Conv3dGnMeanArgs a{x, w, b, gamma, beta, out, d.N, d.C_in, D, H, W, d.act,
                                norm_groups ? norm_groups : d.C_out, d.eps, inv_div};
        if (!norm_groups) a.num_groups = -1;  // plain mean of the activation
        e = single([&] { return cnf::launch_conv3d_gn_mean(a, st); });
        break;
    }
    case FAM_SOFTMAX_POOL: {
        cnf::Conv3dSoftmaxPoolArgs a{x, w, b, out, argmax, d.N, d.C_in, D, H, W, d.kernel,
                                     plan->Do, plan->Ho, plan->Wo, plan->Dp, plan->Hp, plan->Wp,
                                     d.act, d.pool_repeats > 1 ? 1 : 0};
        e = single([&] { return cnf::launch_conv3d_softmax_pool(a, st); });
        break;
    }
    case FAM_SMALL: {
        cnf::SmallConvNormArgs a{x, w, b, gamma, beta, out, d.N, d.C_in, D, H, W, d.kernel,
                                 plan->Do, plan->Ho, plan->Wo, d.act, norm_groups, d.eps,
                                 inv_div, d.reduce == CNF_RED_MEAN_SPATIAL ? 1 : 0};
        e = single([&] { return cnf::launch_small_conv_norm(a, st); });
        break;
    }
    case FAM_IGEMM:
    case FAM_IGEMM16: {
        const int tr = d.kind == CNF_CONV_TRANSPOSE;
        cnf::Conv2dIgemmArgs a{xv, wv, b, gamma, beta, out, static_cast<float *>(workspace), d.N,
                               d.C_in, d.C_out, H, W, plan->Ho, plan->Wo, plan->igemm_pad, tr,
                               d.act, norm_groups, d.eps, inv_div};
        a.stride = plan->igemm_stride;
        a.dtype = plan->family == FAM_IGEMM16 ? (int)d.dtype : 0;
        e = cnf::launch_conv2d_igemm(a, st);
        break;
    }
    case FAM_CONVT:
    case FAM_CONVT_FUSED: {
        cnf::ConvT2dArgs a{x, w, b, gamma, beta, out, static_cast<float *>(workspace), d.N,
                           d.C_in, d.C_out, H, W, d.groups, plan->Ho, plan->Wo, d.act,
                           norm_groups, d.eps, inv_div, (int)d.dtype};
        e = hipErrorInvalidValue;
        if (plan->family == FAM_CONVT_FUSED) {
            // the flag reads 0 unless the single-write kernel below raises it
            int *flag = reinterpret_cast<int *>(static_cast<char *>(workspace) + plan->flag_offset);
            a.flag = flag;
            hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, st, flag);
            if ((e = hipGetLastError()) != hipSuccess) break;
            if (split_f32(*plan)) a.dtype = 3;  // the kernel's fp32-on-bf16-pieces form
            e = cnf::launch_convt2d_fused(a, st);
            a.dtype = (int)d.dtype;
            if (e == hipErrorCooperativeLaunchTooLarge) (void)hipGetLastError();
        }
        if (e == hipErrorCooperativeLaunchTooLarge && d.dtype != CNF_DTYPE_F32)
            e = cnf::launch_generic(generic_args(*plan, xv, wv, b, gamma, beta, out, argmax,
                                                 workspace, norm_groups),
                                    st);
        else if (plan->family == FAM_CONVT || e == hipErrorCooperativeLaunchTooLarge)
            e = cnf::launch_convt2d(a, st);
        break;
    }
    case FAM_UPS2_FUSED: {
        cnf::ConvT2dArgs a{x, w, b, gamma, beta, out, static_cast<float *>(workspace), d.N,
                           d.C_in, d.C_out, H, W, d.groups, plan->Ho, plan->Wo, d.act,
                           norm_groups, d.eps, inv_div, split_f32(*plan) ? 3 : 0};
        int *flag = reinterpret_cast<int *>(static_cast<char *>(workspace) + plan->flag_offset);
        a.flag = flag;
        hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, st, flag);
        if ((e = hipGetLastError()) != hipSuccess) break;
        e = cnf::launch_upsample2_fused(a, st);
        if (e == hipErrorCooperativeLaunchTooLarge) {
            (void)hipGetLastError();
            e = cnf::launch_generic(generic_args(*plan, xv, wv, b, gamma, beta, out, argmax,
                                                 workspace, norm_groups),
                                    st);
        }
        break;
    }
    case FAM_GENERIC:
        e = cnf::launch_generic(generic_args(*plan, xv, wv, b, gamma, beta, out, argmax,
                                             workspace, norm_groups),
                                st);
        break;
    default: return CNF_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? CNF_OK : CNF_ERR_HIP;
}

}  // namespace

extern "C" {

cnf_status cnf_forward(const cnf_plan *plan, const void *xv, const void *wv, const float *b,
                       const float *gamma, const float *beta, float *out, int32_t *argmax,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    return forward_impl(plan, xv, wv, b, gamma, beta, out, argmax, workspace, workspace_bytes,
                        stream, nullptr, nullptr);
}

cnf_status cnf_forward_timed(const cnf_plan *plan, const void *x, const void *w, const float *b,
                             const float *gamma, const float *beta, float *out, int32_t *argmax,
                             void *workspace, size_t workspace_bytes, void *stream,
                             void *event_before, void *event_after)
{
    if (!event_before || !event_after) return CNF_ERR_NULL;
    return forward_impl(plan, x, w, b, gamma, beta, out, argmax, workspace, workspace_bytes,
                        stream, event_before, event_after);
}

cnf_status cnf_forward_check(const cnf_plan *plan, const void *workspace, size_t workspace_bytes,
                             void *stream)
{
    if (!plan) return CNF_ERR_NULL;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((plan->family != FAM_CONVT_FUSED && plan->family != FAM_UPS2_FUSED) || plan->d.N == 0)
        return hipStreamSynchronize(st) == hipSuccess ? CNF_OK : CNF_ERR_HIP;
    if (!workspace || workspace_bytes < plan->workspace) return CNF_ERR_WORKSPACE;
    if (misaligned(workspace)) return CNF_ERR_ALIGNMENT;
    int flag = 0;
    const char *src = static_cast<const char *>(workspace) + plan->flag_offset;
    if (hipMemcpyAsync(&flag, src, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return CNF_ERR_HIP;
    return flag ? CNF_ERR_WAIT_TIMEOUT : CNF_OK;
}

}  // extern "C"

namespace {

// Workspace of cnf_forward_noalloc: one copy per device, loaded with the
// library's code object.  In host code `scratch` names a host-side stand-in,
// never the device memory: only the address hipGetSymbolAddress returns for
// a device may be handed to kernels.
static __device__ __align__(256) unsigned char scratch[CNF_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_ptr[MAX_DEVICES];  // device address of scratch, per device
std::mutex scratch_mu;

// The device address of scratch on device dev, taken once with dev current.
hipError_t scratch_address(int dev, void **out)
{
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void *ptr = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        ptr = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            int cur = 0;
            hipError_t e = hipGetDevice(&cur);
            if (e != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t r = hipSetDevice(cur);
                if (e == hipSuccess) e = r;
            }
            if (e != hipSuccess) return e;
            if (!ptr) return hipErrorInvalidSymbol;
            scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return hipSuccess;
}

}  // namespace

extern "C" {

cnf_status cnf_forward_noalloc(const cnf_plan *plan, const void *x, const void *w, const float *b,
                               const float *gamma, const float *beta, float *out, int32_t *argmax,
                               void *stream)
{
    if (!plan) return CNF_ERR_NULL;
    if (plan->workspace > CNF_NOALLOC_SCRATCH_BYTES) return CNF_ERR_SCRATCH;
    void *ws = nullptr;
    if (plan->workspace > 0 && plan->d.N > 0) {
        int dev = 0;
        if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev) != hipSuccess ||
            scratch_address(dev, &ws) != hipSuccess)
            return CNF_ERR_HIP;
    }
    return forward_impl(plan, x, w, b, gamma, beta, out, argmax, ws, plan->workspace, stream,
                        nullptr, nullptr);
}

}  // extern "C"
