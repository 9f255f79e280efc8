/*
 * cnf.h -- C ABI of the fused convolution + normalization forward library
 * for AMD MI355X (gfx950).
 *
 * The library computes, in one call on one HIP stream, the forward pass
 *
 *     y   = conv(x; w, b)           groups, stride, zero padding, dilation
 *                                   (transposed conv: also output_padding)
 *     a   = act(y)                  none | HardSwish | exact GELU | tanh GELU |
 *                                   channel softmax
 *     z   = norm(a)                 none | GroupNorm | InstanceNorm (eps inside sqrt)
 *     z   = z / divide_by
 *     out = reduce(z)               none | mean over D,H,W | p-max-pool applied r times
 *
 * as stated by four KernelBench level-2 reasoning-trace pages:
 *   "Kimi-K2.6__l2_p27"  Conv3d -> HardSwish -> GroupNorm -> mean over D,H,W
 *                        (first trace: problem statement and the closed form of
 *                        the mean of a GroupNorm output);
 *   "Kimi-K2.6__l2_p17"  Conv2d -> InstanceNorm2d -> divide by a constant
 *                        (second trace: InstanceNorm2d defaults);
 *   "Kimi-K2.6__l2_p6"   Conv3d -> softmax over channels -> MaxPool3d(2) twice
 *                        (the trace's problem statement and floor-mode size chain);
 *   "Kimi-K2.6__l2_p19"  ConvTranspose2d (stride 1, groups) -> GELU -> GroupNorm
 *                        (first trace: shapes and the output-size formula with
 *                        stride, padding, dilation and output_padding; second
 *                        trace: transposed-conv definition and weight layout;
 *                        the fix sequence: the transposed conv as the adjoint
 *                        of the strided, padded, dilated conv).
 * The conv output-size formula with stride, padding and dilation is the one
 * "Kimi-K2.6__l2_p6" states in its integer output-size passage.
 *
 * Conventions for every entry point:
 *   - Tensors are dense and contiguous, batch-major NC(D)HW.  2-D problems set
 *     ndim = 2 and in_dims[0] = 1.  x and w have the element type
 *     desc->dtype (fp32, bf16 or fp16); b, gamma, beta and out are always fp32.
 *     The contraction accumulates in fp32 whatever the input type; every
 *     step after it (activation, statistics, norm, divide, reduction) is fp32.
 *   - Every tensor pointer passed to cnf_forward is a DEVICE pointer owned by
 *     the caller (for example a torch tensor's data_ptr()); the library never
 *     allocates device memory (its only device memory is the fixed scratch
 *     array of cnf_forward_noalloc, loaded with its code), never frees caller
 *     memory and never synchronises the stream.  The plan owns only host
 *     memory.
 *   - Device pointers must be 16-byte aligned (CNF_ERR_ALIGNMENT otherwise).
 *   - No function throws; every failure is a cnf_status.  Argument errors
 *     (NULL, ALIGNMENT, WORKSPACE, ...) are found before anything is
 *     enqueued.  A CNF_ERR_HIP from a family that launches several kernels
 *     may come after some of them were enqueued; the output is then
 *     unspecified.
 *   - cnf_forward is asynchronous on `stream` (a hipStream_t; NULL is the
 *     null stream).  Calls on different streams may run concurrently if each
 *     has its own workspace and output.
 *   - Inputs and parameters must be finite: padded contraction entries and
 *     conv groups that share a matrix tile multiply zero weights by real
 *     inputs, so an Inf or NaN may reach outputs outside its receptive field.
 */
#ifndef CNF_H_
#define CNF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CNF_ABI_VERSION 5

typedef enum {
    CNF_OK = 0,
    CNF_ERR_NULL = 1,          /* a required pointer is NULL (or a forbidden one is not) */
    CNF_ERR_INVALID_DESC = 2,  /* descriptor is self-inconsistent (groups, sizes, eps...) */
    CNF_ERR_UNSUPPORTED = 3,   /* valid, but no kernel family covers it: never a slow path */
    CNF_ERR_WORKSPACE = 4,     /* workspace pointer NULL or smaller than required */
    CNF_ERR_ALIGNMENT = 5,     /* a device pointer is not 16-byte aligned */
    CNF_ERR_HIP = 6,           /* a HIP launch reported an error */
    CNF_ERR_ABI = 7,           /* desc->abi_version != CNF_ABI_VERSION */
    CNF_ERR_NOMEM = 8,         /* host memory for the plan could not be allocated */
    CNF_ERR_WAIT_TIMEOUT = 9,  /* cnf_forward_check: a bounded cross-workgroup wait gave up */
    CNF_ERR_SCRATCH = 10       /* cnf_forward_noalloc: the plan needs more than the fixed scratch */
} cnf_status;

typedef enum { CNF_CONV = 0, CNF_CONV_TRANSPOSE = 1 } cnf_conv_kind;

/* Element type of x and w.  The 16-bit types feed the 16-bit matrix
 * instructions (products exact in fp32, fp32 accumulation), or, in the
 * single-write grouped transposed-conv kernel, are widened to fp32 as they are
 * loaded; either way the epilogue is fp32.  The pages use fp32 throughout, and
 * name tensor-core input precisions only as what a vendor library would
 * pick. */
typedef enum { CNF_DTYPE_F32 = 0, CNF_DTYPE_BF16 = 1, CNF_DTYPE_F16 = 2 } cnf_dtype;

/* How fp32 x and w are contracted (ignored for 16-bit inputs).
 *   NATIVE  products of fp32 values on the fp32 matrix (or vector) units.
 *   BF16X3  each fp32 operand split into three bf16 pieces, v = v1 + v2 + v3
 *           exactly (v1 = bf16(v), v2 = bf16(v - v1), v3 = v - v1 - v2), and
 *           the six leading piece products (w1x1, w1x2, w2x1, w1x3, w2x2,
 *           w3x1) summed on the bf16 matrix instruction with fp32
 *           accumulation.  Each piece product is exact in fp32; the three
 *           dropped ones total at most about 2^-23 |w x| (two units in the
 *           last place of one fp32 product, which rounds by up to 2^-24
 *           itself), so the result keeps fp32 accuracy (values below
 *           2^-100 in magnitude can lose their last piece to bf16
 *           subnormals).  The 16-bit matrix instruction runs
 *           beside the vector unit's epilogue work, where fp32 products do
 *           not.  The two single-write grouped transposed-conv kernels
 *           (stride 1, and the stride-2 upsampling one) have this form;
 *           every other kernel contracts fp32 natively. */
typedef enum { CNF_F32_NATIVE = 0, CNF_F32_BF16X3 = 1 } cnf_f32_math;

typedef enum {
    CNF_ACT_NONE = 0,
    CNF_ACT_HARDSWISH = 1,        /* x * min(max(x + 3, 0), 6) / 6           (l2_p27) */
    CNF_ACT_GELU_ERF = 2,         /* 0.5 * x * (1 + erf(x / sqrt 2))          (l2_p19) */
    CNF_ACT_SOFTMAX_CHANNEL = 3,  /* softmax over C_out at every position     (l2_p6)  */
    CNF_ACT_GELU_TANH = 4         /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),
                                     the tanh form of GELU   (l2_p19, first trace)      */
} cnf_act;

typedef enum {
    CNF_NORM_NONE = 0,
    CNF_NORM_GROUP = 1,           /* per (n, group) over C_out/num_groups channels x all positions */
    CNF_NORM_INSTANCE = 2         /* per (n, c); num_groups is ignored */
} cnf_norm;

typedef enum {
    CNF_RED_NONE = 0,             /* out has the conv output's shape */
    CNF_RED_MEAN_SPATIAL = 1,     /* out[n][c] = mean over D, H, W */
    CNF_RED_MAXPOOL = 2           /* pool_repeats floor-mode max pools, kernel = stride = pool_kernel */
} cnf_reduce;

/* Problem descriptor.  All fields are plain 32-bit values so the struct has
 * the same layout from C, C++ and ctypes. */
typedef struct {
    int32_t abi_version;   /* must equal CNF_ABI_VERSION */
    int32_t ndim;          /* 2 or 3 spatial dims */
    int32_t kind;          /* cnf_conv_kind */
    int32_t N;             /* batch (>= 0; N == 0 is a valid no-op) */
    int32_t C_in;
    int32_t C_out;
    int32_t in_dims[3];    /* D, H, W of x (D = 1 when ndim == 2) */
    int32_t kernel;        /* cubic/square kernel extent k */
    int32_t groups;        /* conv groups; must divide C_in and C_out */
    int32_t has_bias;      /* 1: b is a [C_out] device array; 0: b must be NULL */
    int32_t act;           /* cnf_act */
    int32_t norm;          /* cnf_norm */
    int32_t num_groups;    /* GroupNorm groups; must divide C_out */
    float   eps;           /* > 0; added to the biased variance inside the sqrt */
    int32_t affine;        /* 1: per-channel gamma, beta [C_out] given; 0: both NULL */
    float   divide_by;     /* != 0; applied after the norm as a true division; 1 = none */
    int32_t reduce;        /* cnf_reduce */
    int32_t pool_kernel;   /* maxpool kernel = stride (>= 1) */
    int32_t pool_repeats;  /* number of successive pools (>= 1) */
    int32_t want_argmax;   /* maxpool only: 1 = also write int32 argmax */
    /* Conv geometry, the same on every spatial axis (added in ABI version 2). */
    int32_t stride;        /* >= 1 */
    int32_t padding;       /* >= 0; conv: zeros around the input; transposed conv:
                              rows/cols dropped from each side of the full output */
    int32_t dilation;      /* >= 1; spacing of the kernel taps */
    int32_t output_padding;/* transposed conv: 0 <= output_padding < max(stride,
                              dilation), extra extent at the high end; conv: 0 */
    int32_t dtype;         /* cnf_dtype of x and w (added in ABI version 3) */
    int32_t f32_math;      /* cnf_f32_math (added in ABI version 5) */
} cnf_desc;

typedef struct cnf_plan cnf_plan;

/* Validate `desc`, pick a kernel family and its launch geometry, and return
 * an immutable plan in *plan (host memory, freed by cnf_plan_destroy).
 * Checks: abi_version; ndim in {2,3}; N >= 0; C_in, C_out, kernel >= 1;
 * groups divides C_in and C_out; num_groups divides C_out (GroupNorm);
 * stride, dilation >= 1; padding >= 0; output_padding as stated above;
 * dtype and f32_math in range;
 * every conv output extent >= 1; pooled extents >= 1; eps > 0 when a norm is
 * requested; divide_by != 0; enum fields in range.  Shapes the specialised
 * kernel families cover take them; every other valid descriptor takes the
 * general family (cnf_plan_describe names the choice).  Returns
 * CNF_ERR_UNSUPPORTED only past the general family's size limits: a sample's
 * input or output, or the weights, at or above 2 GiB - 16 MiB; an extent,
 * padding or dilated kernel extent at or above 2^20; more than 2048 channels
 * per norm group; more than 2^27 output positions per channel.
 * On failure *plan is set to NULL. */
cnf_status cnf_plan_create(const cnf_desc *desc, cnf_plan **plan);

/* Output shape of cnf_forward's `out`: dims[0..rank-1], rank <= 5.
 *   reduce NONE    -> (N, C_out, [Do,] Ho, Wo) with, per axis,
 *                     conv:       floor((L + 2p - d(k-1) - 1) / s) + 1
 *                     transposed: (L - 1)s - 2p + d(k-1) + output_padding + 1
 *   reduce MEAN    -> (N, C_out)
 *   reduce MAXPOOL -> (N, C_out, Dp, Hp, Wp), each extent floor-divided by
 *                     pool_kernel pool_repeats times (2-D: H and W are pooled,
 *                     Dp = 1 is kept).
 * argmax, when requested, has the same shape as out. */
cnf_status cnf_plan_output_shape(const cnf_plan *plan, int64_t dims[5], int32_t *rank);

/* Bytes of device workspace cnf_forward needs (0 is possible; then NULL may
 * be passed).  The workspace holds per-tile partial statistics; its content
 * on entry is ignored and on exit is unspecified. */
cnf_status cnf_plan_workspace_size(const cnf_plan *plan, size_t *bytes);

/* Run the whole forward path on `stream`.
 *   x      [N][C_in][D][H][W]  (D absent for 2-D), element type desc->dtype
 *   w      conv: [C_out][C_in/groups][k]^ndim; transposed conv:
 *          [C_in][C_out/groups][k]^ndim (the layout l2_p19 states), element
 *          type desc->dtype
 *   b      [C_out] iff has_bias, else NULL
 *   gamma, beta  [C_out] iff a norm with affine = 1, else NULL
 *   out    the shape cnf_plan_output_shape reports
 *   argmax int32, same shape as out, iff want_argmax; flat index
 *          d*Ho*Wo + h*Wo + w of the winning voxel in its (n, c) conv grid.
 *          Among equal maxima the first one met by the literal sequence of
 *          pools (each scanning its window in row-major order) wins.
 *   workspace / workspace_bytes  at least cnf_plan_workspace_size bytes
 * Returns CNF_ERR_NULL / CNF_ERR_ALIGNMENT / CNF_ERR_WORKSPACE before any
 * launch, or CNF_ERR_HIP if a launch failed. */
cnf_status cnf_forward(const cnf_plan *plan,
                       const void *x, const void *w, const float *b,
                       const float *gamma, const float *beta,
                       float *out, int32_t *argmax,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/* cnf_forward, and also records event_before (a hipEvent_t) on `stream`
 * right before the launch of the plan's dominant kernel (the one that does
 * the contraction) and event_after right after it, so the caller can time
 * that kernel alone with hipEventElapsedTime.  Both events must be non-NULL
 * (CNF_ERR_NULL) and are owned by the caller.  Same results as cnf_forward. */
cnf_status cnf_forward_timed(const cnf_plan *plan,
                             const void *x, const void *w, const float *b,
                             const float *gamma, const float *beta,
                             float *out, int32_t *argmax,
                             void *workspace, size_t workspace_bytes,
                             void *stream, void *event_before, void *event_after);

/* Outcome of the last cnf_forward (or cnf_forward_timed) that ran `plan` on
 * this workspace.  Waits for `stream` (hipStreamSynchronize), then reads the
 * status word that call left in the workspace.  Only the single-write
 * grouped ConvTranspose2d + GroupNorm kernels (page "Kimi-K2.6__l2_p19": the
 * stride-1 layer and its stride-2 upsampling form) wait across workgroups:
 * their workgroups exchange per-slice GroupNorm statistics and each wait is
 * bounded.  If a wait gave up (for example
 * because other work on the device kept a sibling workgroup from running),
 * the affected (sample, group) units of that call's output hold NaN, never
 * values normalised with partial statistics, and this returns
 * CNF_ERR_WAIT_TIMEOUT.  Every other plan returns CNF_OK once the stream
 * is idle.  CNF_ERR_WORKSPACE / CNF_ERR_ALIGNMENT as for cnf_forward.
 *
 * Test knobs of those kernels, read from the environment by cnf_plan_create
 * (unset means off): CNF_TEST_FUSED_SPIN_LIMIT=k (give up after k polls),
 * CNF_TEST_FUSED_NEVER_READY=1 (each wait also needs a word nothing writes,
 * so every wait gives up after its polls and the kernel still ends),
 * CNF_TEST_FORCE_FALLBACK=1 (run the multi-pass fallback the plan keeps for
 * a grid that cannot be co-resident), CNF_TEST_FUSED_MAX_UNITS_PER_ROUND=k
 * (at most k units per round, so small batches run many rounds). */
cnf_status cnf_forward_check(const cnf_plan *plan, const void *workspace,
                             size_t workspace_bytes, void *stream);

/* Bytes of the fixed device scratch behind cnf_forward_noalloc. */
#define CNF_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* cnf_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the workspace is the library's own scratch array, a fixed
 * CNF_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory that each GPU the
 * library runs on holds from the library's load until the process ends.
 * Its device address is taken once per device, on the first call that
 * needs it for the device of `stream`.  Nothing is allocated or freed.
 * Arguments and results are cnf_forward's without workspace /
 * workspace_bytes.  Plans whose cnf_plan_workspace_size exceeds
 * CNF_NOALLOC_SCRATCH_BYTES return CNF_ERR_SCRATCH before anything is
 * enqueued.  Every call on one GPU shares that GPU's scratch and the kernels
 * clear what they need cleared, so consecutive calls are fine, but calls that
 * overlap in time on one GPU (other streams, other threads) race on it and
 * must not be issued.  A timed-out cross-workgroup wait of the single-write
 * kernel (see cnf_forward_check) shows here only as NaN outputs. */
cnf_status cnf_forward_noalloc(const cnf_plan *plan,
                               const void *x, const void *w, const float *b,
                               const float *gamma, const float *beta,
                               float *out, int32_t *argmax, void *stream);

/* Free a plan (NULL is ignored). */
void cnf_plan_destroy(cnf_plan *plan);

/* Static, NUL-terminated name of a status code. */
const char *cnf_status_string(cnf_status status);

/* Write a one-line, NUL-terminated description of the plan's kernel family
 * and launch geometry into buf (truncated to len).  Returns CNF_ERR_NULL if
 * plan or buf is NULL. */
cnf_status cnf_plan_describe(const cnf_plan *plan, char *buf, size_t len);

/* The ABI version the library was built with (== CNF_ABI_VERSION). */
int32_t cnf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CNF_H_ */
