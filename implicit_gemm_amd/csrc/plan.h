// Host-side problem canonicalisation and execution planning.
//
// Pure integer code: no HIP call, no floating point.  Every ceiling division
// is the exact integer form (a + b - 1) / b on non-negative 64-bit values; the
// truncating "ceil of an integer quotient" idiom is what let one dispatch
// address more than ~4 GB in rocm-libraries PR #11188 (section Technical
// Details).
#pragma once

#include <stdint.h>

#include "../../include/conv_wgrad.h"

namespace cw {

// Kernel variants (conv_wgrad_plan_t::variant).
enum Variant : int32_t {
  kDenseLds = 0,      // dense implicit GEMM, LDS-staged tiles, f32 MFMA 16x16x4 (any geometry)
  kDenseRows = 1,     // dense implicit GEMM over output-row units, per-filter-row tiles
  kDense1x1 = 2,      // 1x1 stride-1 unpadded fp32: rows streamed into MFMA registers
  kDense16Rows = 3,   // 16-bit dense, stride 1, dilation 1: row units on 16x16x32 bf16/fp16 MFMA
  kDense16RowsX3 = 4, // fp32 dense by BF16x3 emulation on the 16-bit row kernel (math = BF16X3)
  kDense16Taps = 5,   // 16-bit dense 3x3, stride 1, short rows: all taps per tile, packed row units
  kDense16TapsX3 = 6, // fp32 dense 3x3 by BF16x3 on the all-taps kernel (math = BF16X3)
  kDirectElem = 10,   // direct small-group kernel, one dW element per lane
  kGrouped16 = 11,    // 16-bit small groups: block-diagonal 16x16x32 MFMA, transposed LDS reads
  kDepthwise = 12,    // 16-bit depthwise: batched 4x4x4 MFMA, 64 channels per workgroup
  kGrouped16Rows = 13,  // 16-bit small groups, 1x1 / 3x3, Wo <= 32: row-streaming 16x16x32 MFMA
  kFwdIgemm = 20,     // forward convolution: implicit GEMM over (r, s, c), split-K slabs
  kDgradIgemm = 21,   // data gradient: implicit GEMM over (r, s, k), split-K slabs
};

struct Problem {
  int64_t N, C, H, W, K, R, S, groups;
  // Per-axis geometry: rows (h) and columns (w).
  int64_t pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
  // The row values, for the kernels the planner gives only problems whose
  // two axes agree (uniform).
  int64_t pad, stride, dil;
  bool uniform;
  int32_t math;          // CONV_WGRAD_MATH_*
  int32_t fold;          // width fold applied (1 = none): C, W, S, stride_w, pad_w are the folded ones
  int32_t dtype;
  int32_t esize;         // bytes per x / dy element
  int64_t Ho, Wo, Cg, Kg;
  int64_t L;             // N * Ho * Wo
  int64_t cols;          // R * S * Cg (GEMM N extent per group)
  int64_t E;             // K * R * S * Cg
  int64_t x_img, dy_img; // elements per image of x and dy
  uint64_t x_bytes, dy_bytes, dw_bytes;
};

struct Plan {
  conv_wgrad_plan_t pub;
  Problem p;
  // Dense path tiling.
  int32_t bm, bn, bk;      // tile of output channels, tile of GEMM columns, rows per unit
  int64_t m_tiles, n_tiles;
  int32_t vec_a, vec_b;    // elements per vector load of dy / x (1 or 4)
  // Row-unit dense kernel.
  int32_t sb, wt, xspan;   // taps per tile, output pixels per unit, staged X pixels per unit
  int64_t c_tiles, s_blocks, wchunks;
  int32_t bv;              // 1x1 kernel: input channels per lane
  int32_t ru, xrows;       // grouped16, 16-bit and fp32 packed rows: output rows per unit; staged X rows
  int32_t qa, qb;          // fp32 packed rows: dY and X pixel slots between a unit's rows
  // Depthwise: staged X row length (elements), LDS bytes, column of dY element 0.
  int32_t dw_xl, dw_lds, dw_off;
  // Depthwise: slice s covers output rows [dw_starts[s], dw_starts[s + 1])
  // when dw_balanced (slices balanced by staging steps), else uniform runs of
  // units_per_slice rows.
  static constexpr int kDwMaxSlices = 256;
  int32_t dw_balanced;
  int32_t dw_starts[kDwMaxSlices + 1];
  // Direct path: lanes per workgroup.  Row-unit dense kernel: 256 (two
  // workgroups per CU, each stages and computes its own units) or 512 (one
  // workgroup per CU in two ping-pong halves).
  int32_t threads;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A slab holds the weight-gradient partial in elements [0, E) and the
// bias-gradient partial (K elements) from this 16-byte aligned offset on.
inline int64_t db_offset(const Problem& p) { return ceil_div(p.E, 4) * 4; }

// The extended descriptor of a plain one (equal axes, exact math, automatic fold).
conv_wgrad_desc2_t to_desc2(const conv_wgrad_desc_t& d);

// Validate and canonicalise desc (and apply the width fold it asks for or
// allows).  Returns CONV_WGRAD_OK or the error code.
conv_wgrad_status_t canonicalise(const conv_wgrad_desc2_t* desc, Problem* out);

// LDS bytes of the depthwise kernel for staged rows of xl columns and an R x S
// filter (0 if xl is not a supported length); defined with the kernel.
int32_t depthwise_lds_bytes(int32_t xl, int32_t R, int32_t S);

// Build the full plan (calls canonicalise).
conv_wgrad_status_t make_plan(const conv_wgrad_desc2_t* desc, Plan* out);

// Plan of the forward (CONV_DIRECTION_FWD) or data-gradient
// (CONV_DIRECTION_DGRAD) implicit GEMM of the same convolution.  In these
// plans pub.L is the output pixel count (N*Ho*Wo forward, N*H*W dgrad), pub.E
// and p.E the output elements the slab fold covers, a unit is 32 reduction
// entries (r, s, c) or (r, s, k), and tiles are 64 pixels x 64 channels.
conv_wgrad_status_t make_igemm_plan(const conv_wgrad_desc2_t* desc, int32_t direction, Plan* out);

// Split policy shared by all paths.  `units` reduction units, `tiles` output
// tiles per slice, `requested` the descriptor's split_k (-1 = auto).  Fills
// units_per_slice, ks_count, needs_reduce, grid, slab_stride and ws_bytes.
//
// Auto degree: floor(target_groups / tiles) slices (so the grid never exceeds
// target_groups), at most units / min_units, and with the slab traffic
// (each slab element written once and read once) at most the algorithmic
// bytes times traffic_mul / traffic_div.  forced_ups >= 1 fixes the units per
// slice instead (the degree follows from it).
conv_wgrad_status_t choose_split(int64_t units, int64_t tiles, int32_t requested, int64_t min_units,
                                 int64_t target_groups, int64_t traffic_div, const Problem& p,
                                 conv_wgrad_plan_t* pub, int64_t forced_ups = 0,
                                 int64_t traffic_mul = 1);

}  // namespace cw
