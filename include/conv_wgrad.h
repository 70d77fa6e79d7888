/*
 * conv_wgrad.h -- C ABI of the MI355X (gfx950) convolution weight-gradient library.
 *
 * Operation (the weight gradient of a 2-D convolution, "weight.grad" of
 * nn.Conv2d in rocm-libraries PR #11188 "fix silent zero wgrad", section
 * Motivation; for a 1x1 filter it equals dY^T X on the [N*H*W, .] matrices,
 * the "F.linear on the reshaped tensor" equivalence of the same section):
 *
 *   dW[k, r, s, c] = sum_{n, ho, wo} dY[n, ho, wo, k]
 *                    * X[n, ho*stride + r*dilation - pad, wo*stride + s*dilation - pad, g(k)*Cg + c]
 *
 *   Cg = C / groups, Kg = K / groups, g(k) = k / Kg; X is zero outside the
 *   H x W image (the same pad on all four sides; stride and dilation are the
 *   same on both axes); Ho = (H + 2*pad - dilation*(R-1) - 1) / stride + 1,
 *   Wo likewise.
 *
 * Layouts (dense, row-major, no strides):
 *   x  : [N][H][W][C]    element type desc->dtype
 *   dy : [N][Ho][Wo][K]  element type desc->dtype
 *   dw : [K][R][S][Cg]   fp32, always (fp32 accumulation for every dtype)
 *
 * Execution: the reduction over N*Ho*Wo is cut into ks_count slices
 * ("split-K", the two-stage scheme of rocm-libraries PR #14393 "split-K
 * forward implicit-GEMM convolution on gfx1250", section "Two-stage split-K").
 * With ks_count > 1 every stage-1 workgroup writes its fp32 partial tile into
 * slab `slice` of the workspace exactly once, and a second kernel folds the
 * slabs in one fixed order that depends only on ks_count (16 consecutive
 * parts of the slab range, each summed in ascending slab order, then the part
 * sums in ascending part order; beyond 256 slabs, runs of 32 slabs are folded
 * first the same way); with ks_count == 1 stage 1 writes dw directly.  Results are therefore bit-identical from run to run for a fixed
 * split degree, and the workspace needs no clearing.  Tensor base addresses
 * and image offsets are 64-bit, so tensors larger than 4 GB are handled in
 * one launch (the failure mode of rocm-libraries PR #11188, sections
 * Motivation and Technical Details, where a truncating split computation let
 * one dispatch address more than ~4 GB and silently return zeros).
 *
 * Errors are returned, never hidden: validation is synchronous and happens
 * before anything is enqueued; on any error nothing is enqueued and dw is not
 * touched.  There is no fallback path.
 */
#ifndef CONV_WGRAD_H_
#define CONV_WGRAD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x and dy.  dw is always fp32. */
typedef enum conv_wgrad_dtype {
  CONV_WGRAD_F32 = 0,
  CONV_WGRAD_BF16 = 1,
  CONV_WGRAD_F16 = 2
} conv_wgrad_dtype_t;

/*
 * Problem descriptor.  All fields are read; the struct is copied, never kept.
 *   N, C, H, W : input batch, channels, height, width (each >= 1)
 *   K, R, S    : output channels, filter height, filter width (each >= 1)
 *   pad >= 0, stride >= 1, dilation >= 1 (same value for both spatial axes)
 *   groups >= 1, dividing both C and K
 *   dtype      : conv_wgrad_dtype_t of x and dy
 *   split_k    : -1 = choose the number of reduction slices automatically;
 *                n >= 1 = pin it.  The pinned degree is honoured except that
 *                no slice may be empty: with U reduction units the plan uses
 *                ceil(U / ceil(U / n')) slices with n' = min(n, 65536)
 *                (never more than n).  Any other
 *                value (0, < -1) is CONV_WGRAD_ERR_BAD_SPLIT, as in the
 *                split-K validators of rocm-libraries PR #14393 (section
 *                "Review follow-ups": split_k <= 0 is rejected).
 */
typedef struct conv_wgrad_desc {
  int64_t N, C, H, W, K, R, S;
  int64_t pad, stride, dilation, groups;
  int32_t dtype;
  int32_t split_k;
} conv_wgrad_desc_t;

typedef enum conv_wgrad_status {
  CONV_WGRAD_OK = 0,
  CONV_WGRAD_ERR_NULL_ARG = 1,     /* desc, x, dy, dw or a needed workspace is NULL */
  CONV_WGRAD_ERR_BAD_SHAPE = 2,    /* a dimension < 1, pad < 0, stride/dilation < 1,
                                      C or K not divisible by groups, Ho or Wo < 1,
                                      or a size that overflows int64 */
  CONV_WGRAD_ERR_BAD_DTYPE = 3,    /* dtype is not a conv_wgrad_dtype_t */
  CONV_WGRAD_ERR_BAD_SPLIT = 4,    /* split_k is 0 or < -1 */
  CONV_WGRAD_ERR_UNSUPPORTED = 5,  /* valid, but outside the library's documented
                                      limits (see conv_wgrad_get_plan) */
  CONV_WGRAD_ERR_MISALIGNED = 6,   /* x, dy, dw or workspace not 16-byte aligned */
  CONV_WGRAD_ERR_WORKSPACE = 7,    /* conv_wgrad_ex: ws_bytes smaller than required */
  CONV_WGRAD_ERR_HIP = 8           /* the HIP runtime reported an error at launch */
} conv_wgrad_status_t;

/* Which stage-1 kernel family a plan uses. */
typedef enum conv_wgrad_path {
  CONV_WGRAD_PATH_DENSE = 0,   /* implicit GEMM per group on MFMA */
  CONV_WGRAD_PATH_DIRECT = 1   /* direct per-group kernel for small groups (depthwise, <= 8 ch/group) */
} conv_wgrad_path_t;

/*
 * The execution plan the library derives from a descriptor (pure host
 * integer arithmetic; no GPU needed).  Exposed for tests and diagnostics.
 */
typedef struct conv_wgrad_plan {
  int32_t path;            /* conv_wgrad_path_t */
  int32_t variant;         /* kernel variant within the path (diagnostic) */
  int64_t Ho, Wo;          /* output extents */
  int64_t L;               /* reduction length N*Ho*Wo */
  int64_t E;               /* dW elements K*R*S*Cg */
  int64_t unit_rows;       /* reduction rows per unit (a unit is the smallest slice grain) */
  int64_t units;           /* reduction units: ceil(L / unit_rows) or per-path equivalent */
  int64_t units_per_slice; /* ceil(units / requested degree); depthwise with 2..256 slices: the
                              longest slice (slices there are balanced by the X rows each stages) */
  int32_t ks_count;        /* slices >= 1, none empty: ceil(units / units_per_slice), except for
                              balanced depthwise slices, whose count is the uniform one's */
  int32_t needs_reduce;    /* 1 iff ks_count > 1: the only condition for launching stage 2 */
  int64_t tiles;           /* output tiles per slice */
  int64_t grid;            /* stage-1 workgroups = tiles * ks_count */
  int64_t slab_stride;     /* fp32 elements between workspace slabs (multiple of 64) */
  uint64_t ws_bytes;       /* workspace bytes: ks_count * slab_stride * 4, or 0 */
  uint64_t x_bytes, dy_bytes, dw_bytes;  /* tensor sizes in bytes */
  int64_t windows_4g;      /* ceil(max(x_bytes, dy_bytes) / 2^32): 4-GiB address windows the
                              tensors span (diagnostic; one launch covers them all) */
} conv_wgrad_plan_t;

/*
 * Human-readable name of a status code (static storage; never NULL; "unknown
 * status" for a value outside the enum).  Every failure is reported as one of
 * these codes rather than as a silently wrong dW: a weight gradient that came
 * back all zeros with no error is the failure rocm-libraries PR #11188
 * ("fix silent zero wgrad", section Motivation) fixed.
 */
const char* conv_wgrad_status_string(conv_wgrad_status_t status);

/*
 * Workspace bytes conv_wgrad and conv_wgrad_bias need for desc: ks_count fp32
 * slabs (each holding one slice's partial dW, then its partial db), or 0 when
 * the plan has one slice.  The workspace is the split-K slab buffer of
 * rocm-libraries PR #14393 (section "Two-stage split-K": every workgroup stores
 * an fp32 partial tile into its slab; section "ABI, AOT and runtime": the
 * split-K form takes a workspace argument).
 *   desc  : read only
 *   bytes : host pointer, written on success only
 * Pure host function (no HIP call).  Errors: NULL_ARG (desc or bytes NULL),
 * BAD_SHAPE / BAD_DTYPE / BAD_SPLIT as for conv_wgrad, UNSUPPORTED.
 */
conv_wgrad_status_t conv_wgrad_workspace_size(const conv_wgrad_desc_t* desc, size_t* bytes);

/*
 * Fill *plan with the plan for desc: the stage-1 kernel, the reduction units,
 * the split degree (split_k = -1 resolves it automatically, n >= 1 pins it, as
 * in rocm-libraries PR #14393, section "Auto-deduced degree (split_k = -1)";
 * the slices come from exact integer ceiling divisions, the form whose
 * truncating variant under-counted the batch split in rocm-libraries
 * PR #11188, section Technical Details), the grid and the workspace size.
 *   desc : read only;  plan : host pointer, written on success only
 * Pure host function (no HIP call); the same validation and errors as
 * conv_wgrad (NULL_ARG for a NULL desc or plan).
 */
conv_wgrad_status_t conv_wgrad_get_plan(const conv_wgrad_desc_t* desc, conv_wgrad_plan_t* plan);

/*
 * Enqueue the weight gradient on `stream` (a hipStream_t; NULL = the null
 * stream of the current device) and return without synchronising.
 *   x, dy     : device pointers, layouts above, 16-byte aligned
 *   dw        : device pointer, fp32 [K][R][S][Cg], 16-byte aligned; overwritten
 *               (every element written exactly once; no accumulate)
 *   workspace : device pointer of at least conv_wgrad_workspace_size bytes,
 *               16-byte aligned; may be NULL when that size is 0.  Its content on
 *               entry is irrelevant.  The caller owns every buffer; the library
 *               never allocates or frees device memory.
 * Buffers must not overlap.  Concurrent calls on different streams need
 * different workspaces.
 */
conv_wgrad_status_t conv_wgrad(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                               float* dw, void* workspace, void* stream);

/* As conv_wgrad, also checking that ws_bytes covers the workspace the plan needs
 * (CONV_WGRAD_ERR_WORKSPACE otherwise). */
conv_wgrad_status_t conv_wgrad_ex(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                  float* dw, void* workspace, size_t ws_bytes, void* stream);

/*
 * Profiling variant of conv_wgrad: identical work on `stream`, and the caller's
 * HIP events (hipEvent_t, created by the caller; either may be NULL) take the
 * start and end timestamps of the stage-1 kernel's own dispatch (the stage-1
 * launch goes through hipExtLaunchKernel with them), so the caller can time
 * that kernel alone, without the launch gaps around it; the slab reduce, when
 * launched, is not included.  The events are only recorded, never
 * synchronised or destroyed.
 */
conv_wgrad_status_t conv_wgrad_timed(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                     float* dw, void* workspace, size_t ws_bytes, void* stream,
                                     void* stage1_begin, void* stage1_end);

/*
 * Weight gradient and bias gradient in one pass over dy.  The bias gradient of
 * a convolution is the sum of the output gradient over every output pixel
 * (rocm-libraries PR #11188, section Motivation, checks bias.grad beside
 * weight.grad of nn.Conv2d):
 *   db[k] = sum over n, ho, wo of dy[n][ho][wo][k]
 *   db        : device pointer, fp32 [K], 16-byte aligned; overwritten
 * The stage-1 kernels add up the dy values they already stage, per slice;
 * db is folded with the slabs in the same fixed order as dw (fp32 adds), so
 * the result is bit-identical from run to run at a fixed split, and dw is
 * bit-identical to what conv_wgrad_ex writes for the same desc.  The other
 * arguments, the workspace size and the errors are those of conv_wgrad_ex
 * (NULL_ARG also for a NULL db, MISALIGNED for a misaligned one).
 */
conv_wgrad_status_t conv_wgrad_bias(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                    float* dw, float* db, void* workspace, size_t ws_bytes,
                                    void* stream);

/* Profiling variant of conv_wgrad_bias, with stage-1 events as in conv_wgrad_timed. */
conv_wgrad_status_t conv_wgrad_bias_timed(const conv_wgrad_desc_t* desc, const void* x,
                                          const void* dy, float* dw, float* db, void* workspace,
                                          size_t ws_bytes, void* stream, void* stage1_begin,
                                          void* stage1_end);

/*
 * Extended problem descriptor: per-axis geometry, an arithmetic mode for fp32
 * inputs and the width fold.  conv_wgrad_desc_t is this with equal axes,
 * math = CONV_WGRAD_MATH_EXACT and fold_width = -1.
 *
 * Per-axis geometry (the column padding pad_w beside the row padding of
 * rocm-libraries PR #14393's embedded depthwise-dgrad PR #14386, section
 * "Per-axis padding"; stride and dilation the same way):
 *   dW[k, r, s, c] = sum_{n, ho, wo} dY[n, ho, wo, k]
 *       * X[n, ho*stride_h + r*dil_h - pad_h, wo*stride_w + s*dil_w - pad_w, g(k)*Cg + c]
 *   Ho = (H + 2*pad_h - dil_h*(R-1) - 1) / stride_h + 1,
 *   Wo = (W + 2*pad_w - dil_w*(S-1) - 1) / stride_w + 1.
 *   pad_h, pad_w >= 0; stride_h, stride_w, dil_h, dil_w >= 1 (BAD_SHAPE otherwise).
 *
 * math (fp32 inputs; ignored for bf16 / fp16, which always use their own MFMA):
 *   CONV_WGRAD_MATH_EXACT  (0): fp32 products on f32 MFMA (the default).
 *   CONV_WGRAD_MATH_BF16X3 (1): BF16x3 emulation, the form the pages give for
 *       fp32 ("TF32") matrix work on gfx950 (rocm-libraries PR #14393,
 *       timeline, the TF32 entry: native XF32 on gfx942, BF16x3 on gfx950):
 *       each fp32 value v = hi + lo with hi = bf16(v), lo = bf16(v - hi), and
 *       a*b ~ a_hi*b_hi + a_hi*b_lo + a_lo*b_hi on bf16 MFMA with fp32
 *       accumulation.  Each product carries a relative error of at most about
 *       3 * 2^-16 (the dropped a_lo*b_lo term and the two splits' residuals),
 *       so the normalised error is bounded by ~4.6e-5 in the worst case and is
 *       ~1e-7 for inputs of random sign.  It is a permission, never a silent
 *       downgrade of other shapes: the plan uses it only where a BF16x3 kernel
 *       covers the shape (plan variant CONV_WGRAD_VARIANT_DENSE_BF16X3 or
 *       CONV_WGRAD_VARIANT_DENSE_BF16X3_TAPS) and the exact fp32 path
 *       elsewhere.  Any other value is BAD_DTYPE.
 * fold_width (rocm-libraries PR #14393, commit bodies, the fold_width
 * paragraph: f adjacent W positions folded into the channels when f divides
 * the filter width, the W stride, the input width and the W padding; the
 * identity holds in every direction, so it is a view of the same tensors):
 *   -1: fold by the largest such f when the shape gains from it (input
 *       channels per group not a multiple of 4, a multiple after folding);
 *    0 or 1: never fold;  f >= 2: fold by f (BAD_SHAPE if f does not divide
 *       S, stride_w, W and pad_w, or if dil_w != 1 or groups != 1).
 *   Folding changes only the kernel and the summation order, never the
 *   layouts: X [N][H][W][C] is read as [N][H][W/f][f*C], dY is unchanged, and
 *   dW [K][R][S][Cg] is written as [K][R][S/f][f*Cg] -- the same bytes.
 */
typedef struct conv_wgrad_desc2 {
  int64_t N, C, H, W, K, R, S;
  int64_t pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
  int64_t groups;
  int32_t dtype;       /* conv_wgrad_dtype_t of x and dy */
  int32_t split_k;     /* as in conv_wgrad_desc_t */
  int32_t math;        /* CONV_WGRAD_MATH_* */
  int32_t fold_width;  /* -1 auto, 0 / 1 off, f >= 2 fold by f */
} conv_wgrad_desc2_t;

#define CONV_WGRAD_MATH_EXACT 0
#define CONV_WGRAD_MATH_BF16X3 1

/* conv_wgrad_plan_t::variant of the BF16x3 dense kernels: the row kernel
 * (one filter row per tile) and the all-taps kernel (3 x 3 filters, output
 * rows of at most 61 pixels). */
#define CONV_WGRAD_VARIANT_DENSE_BF16X3 4
#define CONV_WGRAD_VARIANT_DENSE_BF16X3_TAPS 6

/* The plan of an extended descriptor: the base plan (of the problem the kernels
 * run, i.e. after a width fold) and what was applied. */
typedef struct conv_wgrad_plan2 {
  conv_wgrad_plan_t base;
  int32_t math;        /* CONV_WGRAD_MATH_* the kernels use */
  int32_t fold_width;  /* applied fold (1 = none) */
} conv_wgrad_plan2_t;

/*
 * conv_wgrad_workspace_size for an extended descriptor: the workspace bytes
 * conv_wgrad2 needs (0 when the plan has one slice).  Pure host function;
 * errors: NULL_ARG (desc or bytes NULL), BAD_SHAPE, BAD_DTYPE (also a math
 * value outside CONV_WGRAD_MATH_*), BAD_SPLIT, UNSUPPORTED.
 */
conv_wgrad_status_t conv_wgrad2_workspace_size(const conv_wgrad_desc2_t* desc, size_t* bytes);

/* conv_wgrad_get_plan for an extended descriptor (same validation and errors). */
conv_wgrad_status_t conv_wgrad2_get_plan(const conv_wgrad_desc2_t* desc, conv_wgrad_plan2_t* plan);

/*
 * The weight gradient (and, when db is not NULL, the bias gradient db[k] =
 * sum of dy over n, ho, wo) for an extended descriptor, enqueued on `stream`.
 * Layouts, ownership, workspace rules (at least conv_wgrad2_workspace_size
 * bytes, WORKSPACE otherwise; NULL allowed when that is 0), alignment,
 * determinism at a fixed split and errors are those of conv_wgrad_bias; dw
 * and db are overwritten.
 */
conv_wgrad_status_t conv_wgrad2(const conv_wgrad_desc2_t* desc, const void* x, const void* dy,
                                float* dw, float* db, void* workspace, size_t ws_bytes, void* stream);

/* Profiling variant of conv_wgrad2, with stage-1 events as in conv_wgrad_timed. */
conv_wgrad_status_t conv_wgrad2_timed(const conv_wgrad_desc2_t* desc, const void* x, const void* dy,
                                      float* dw, float* db, void* workspace, size_t ws_bytes,
                                      void* stream, void* stage1_begin, void* stage1_end);

/* Profiling variant of conv_wgrad2 that times the whole call on the GPU: the
 * caller's events (hipEvent_t, either may be NULL) take the start timestamp of
 * the call's first kernel (stage 1) and the end timestamp of its last kernel
 * (the slab fold, or stage 1 with one slice), through hipExtLaunchKernel, so
 * hipEventElapsedTime gives stage 1 + fold + the gap between them without any
 * marker of its own.  Only recorded, never synchronised or destroyed. */
conv_wgrad_status_t conv_wgrad2_call_timed(const conv_wgrad_desc2_t* desc, const void* x, const void* dy,
                                           float* dw, float* db, void* workspace, size_t ws_bytes,
                                           void* stream, void* call_begin, void* call_end);

/*
 * Forward convolution and data gradient on the same implicit-GEMM, split-K
 * slab and fold machinery (rocm-libraries PR #14393 "split-K forward
 * implicit-GEMM convolution on gfx1250": sections Summary, "Two-stage
 * split-K" -- every workgroup stores an fp32 partial tile into its slab, a
 * second kernel folds the slabs, no workspace clearing, deterministic -- and
 * "Auto-deduced degree (split_k = -1)", whose policy is refitted here for 256
 * CUs: split only a grid under 4 workgroups per CU (1024) over a reduction at
 * least 512 deep, by the smallest power of two that brings the grid to 8
 * workgroups per CU (2048), at most 32, with at least two 32-entry reduction
 * tiles per slice).
 *
 *   forward: y[n][ho][wo][k] = sum_{r,s,c} x[n][ho*stride_h + r*dil_h - pad_h]
 *                                            [wo*stride_w + s*dil_w - pad_w][g(k)*Cg + c]
 *                                          * w[k][r][s][c]
 *   dgrad:   dx[n][h][w][g*Cg + c] = sum over k of group g and r, s with
 *              ho*stride_h = h + pad_h - r*dil_h, wo*stride_w = w + pad_w - s*dil_w
 *              (exactly, 0 <= ho < Ho, 0 <= wo < Wo) of dy[n][ho][wo][k] * w[k][r][s][c]
 *
 * The descriptor is conv_wgrad_desc2_t (per-axis geometry, groups, dtype,
 * split_k, fold_width; math is read as in conv_wgrad2 and only the exact path
 * exists for these directions).  Layouts: x [N][H][W][C] and dy [N][Ho][Wo][K]
 * and the filter w [K][R][S][Cg] in desc->dtype; y [N][Ho][Wo][K] and dx
 * [N][H][W][C] are fp32 (fp32 accumulation for every dtype), overwritten.
 * Workspace, alignment (16 bytes), ownership, determinism at a fixed split and
 * errors are those of conv_wgrad_ex; the workspace holds ks_count slabs of the
 * whole output.
 */
#define CONV_DIRECTION_WGRAD 0
#define CONV_DIRECTION_FWD 1
#define CONV_DIRECTION_DGRAD 2

/* Plan of a direction (CONV_DIRECTION_*; WGRAD gives conv_wgrad2_get_plan's).
 * For FWD / DGRAD: base.L is the output pixel count, base.E the output
 * elements, base.unit_rows 32 reduction entries, base.variant 20 / 21.
 * Unknown direction: BAD_DTYPE.  Pure host function. */
conv_wgrad_status_t conv_igemm_get_plan(const conv_wgrad_desc2_t* desc, int32_t direction,
                                        conv_wgrad_plan2_t* plan);

/* Workspace bytes of conv_fwd (direction FWD) or conv_dgrad (DGRAD). */
conv_wgrad_status_t conv_igemm_workspace_size(const conv_wgrad_desc2_t* desc, int32_t direction,
                                              size_t* bytes);

/* Forward convolution: y (fp32) from x and w, enqueued on stream. */
conv_wgrad_status_t conv_fwd(const conv_wgrad_desc2_t* desc, const void* x, const void* w, float* y,
                             void* workspace, size_t ws_bytes, void* stream);

/* Data gradient: dx (fp32) from dy and w, enqueued on stream. */
conv_wgrad_status_t conv_dgrad(const conv_wgrad_desc2_t* desc, const void* dy, const void* w, float* dx,
                               void* workspace, size_t ws_bytes, void* stream);

/* Profiling variant of conv_fwd (direction FWD: src = x, out = y) and
 * conv_dgrad (DGRAD: src = dy, out = dx) that times the whole call on the
 * GPU as conv_wgrad2_call_timed does: call_begin takes the start timestamp of
 * the implicit GEMM's dispatch, call_end the end timestamp of the call's last
 * kernel (either may be NULL; only recorded).  Another direction: BAD_DTYPE. */
conv_wgrad_status_t conv_igemm_call_timed(const conv_wgrad_desc2_t* desc, int32_t direction,
                                          const void* src, const void* w, float* out, void* workspace,
                                          size_t ws_bytes, void* stream, void* call_begin,
                                          void* call_end);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): conv_wgrad_bias
 * without the workspace argument.  The slabs live in a library-owned device
 * array of CONV_WGRAD_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held until the
 * process ends; its device address is looked up (hipGetSymbolAddress) on the
 * first call on each device, with that device current.  No call allocates or
 * frees memory (no hipMalloc / hipFree, no allocating library routine).
 *   db : NULL for the weight gradient only (dw then equals conv_wgrad's), or
 *        an fp32 [K] buffer for the bias gradient as in conv_wgrad_bias
 * The other arguments, the results and the errors are those of conv_wgrad_bias,
 * plus CONV_WGRAD_ERR_WORKSPACE when conv_wgrad_workspace_size(desc) exceeds
 * CONV_WGRAD_NOALLOC_SCRATCH_BYTES (pin a smaller split_k to fit) and
 * CONV_WGRAD_ERR_HIP when the address lookup fails; errors are returned
 * before anything is enqueued.  The current device must be the stream's.
 * Every call on one GPU shares that GPU's array (nothing in it needs clearing:
 * each slab element is written before the fold reads it), so calls that
 * overlap in time on one GPU (other streams, other host threads) race.
 */
#define CONV_WGRAD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
conv_wgrad_status_t conv_wgrad_noalloc(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                       float* dw, float* db, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV_WGRAD_H_ */
