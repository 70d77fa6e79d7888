// Problem validation and execution planning (host, integer-only).
#include "plan.h"

#include <string.h>

namespace cw {

namespace {

// Checked a * b for non-negative operands; false on overflow.
bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  int64_t t;
  return mul_ok(a, b, &t) && mul_ok(t, c, out);
}

bool mul4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* out) {
  int64_t t;
  return mul3(a, b, c, &t) && mul_ok(t, d, out);
}

// Output extent along one axis; -1 when it would be < 1 or overflows.
int64_t extent(int64_t in, int64_t k, int64_t pad, int64_t stride, int64_t dil) {
  int64_t span_k, twice_pad, span;
  if (!mul_ok(dil, k - 1, &span_k) || !mul_ok(pad, 2, &twice_pad)) return -1;
  if (__builtin_add_overflow(in, twice_pad, &span)) return -1;
  span = span - span_k - 1;
  if (span < 0) return -1;
  return span / stride + 1;
}

constexpr int64_t kI32Max = 2147483647;
// Reduction rows stay below 2^31 with room for one rounded-up slice.
constexpr int64_t kMaxRows = kI32Max - 65536;
constexpr int64_t kDwLdsMax = 160 * 1024;  // LDS per CU
// Upper bound on the split degree (the slab fold launches one workgroup row per run).
constexpr int64_t kMaxSlices = 65536;
// Launch geometry limits: lanes per launch, the widest stage-1 workgroup, and
// the slab fold's workgroup (256 lanes folding 64 consecutive elements).
constexpr int64_t kLaunchLanes = (int64_t)1 << 32;
constexpr int64_t kMaxBlock = 512;
constexpr int64_t kFoldBlock = 256, kFoldElemsPerBlock = 64;

}  // namespace

conv_wgrad_desc2_t to_desc2(const conv_wgrad_desc_t& d) {
  conv_wgrad_desc2_t e;
  memset(&e, 0, sizeof(e));
  e.N = d.N; e.C = d.C; e.H = d.H; e.W = d.W; e.K = d.K; e.R = d.R; e.S = d.S;
  e.pad_h = e.pad_w = d.pad;
  e.stride_h = e.stride_w = d.stride;
  e.dil_h = e.dil_w = d.dilation;
  e.groups = d.groups;
  e.dtype = d.dtype;
  e.split_k = d.split_k;
  e.math = CONV_WGRAD_MATH_EXACT;
  e.fold_width = -1;
  return e;
}

namespace {

int64_t gcd64(int64_t a, int64_t b) {
  while (b != 0) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Width fold by f (the caller has checked that f divides S, stride_w, W and
// pad_w, with dil_w == 1 and one group): X [N][H][W][C] read as
// [N][H][W/f][f*C], the filter [K][R][S][C] as [K][R][S/f][f*C].  Wo, the
// tensor sizes and the dW layout do not change.
void apply_fold(Problem* o, int64_t f) {
  o->W /= f;
  o->S /= f;
  o->stride_w /= f;
  o->pad_w /= f;
  o->C *= f;
  o->fold = (int32_t)f;
}

}  // namespace

conv_wgrad_status_t canonicalise(const conv_wgrad_desc2_t* d, Problem* o) {
  if (!d || !o) return CONV_WGRAD_ERR_NULL_ARG;
  memset(o, 0, sizeof(*o));
  if (d->dtype != CONV_WGRAD_F32 && d->dtype != CONV_WGRAD_BF16 && d->dtype != CONV_WGRAD_F16)
    return CONV_WGRAD_ERR_BAD_DTYPE;
  if (d->math != CONV_WGRAD_MATH_EXACT && d->math != CONV_WGRAD_MATH_BF16X3) return CONV_WGRAD_ERR_BAD_DTYPE;
  if (d->split_k == 0 || d->split_k < -1) return CONV_WGRAD_ERR_BAD_SPLIT;
  if (d->N < 1 || d->C < 1 || d->H < 1 || d->W < 1 || d->K < 1 || d->R < 1 || d->S < 1 ||
      d->pad_h < 0 || d->pad_w < 0 || d->stride_h < 1 || d->stride_w < 1 || d->dil_h < 1 ||
      d->dil_w < 1 || d->groups < 1 || d->fold_width < -1)
    return CONV_WGRAD_ERR_BAD_SHAPE;
  if (d->C % d->groups != 0 || d->K % d->groups != 0) return CONV_WGRAD_ERR_BAD_SHAPE;
  o->N = d->N; o->C = d->C; o->H = d->H; o->W = d->W; o->K = d->K; o->R = d->R; o->S = d->S;
  o->pad_h = d->pad_h; o->pad_w = d->pad_w;
  o->stride_h = d->stride_h; o->stride_w = d->stride_w;
  o->dil_h = d->dil_h; o->dil_w = d->dil_w;
  o->groups = d->groups;
  o->dtype = d->dtype;
  o->math = d->dtype == CONV_WGRAD_F32 ? d->math : CONV_WGRAD_MATH_EXACT;
  o->fold = 1;
  o->esize = d->dtype == CONV_WGRAD_F32 ? 4 : 2;
  o->Ho = extent(d->H, d->R, d->pad_h, d->stride_h, d->dil_h);
  o->Wo = extent(d->W, d->S, d->pad_w, d->stride_w, d->dil_w);
  if (o->Ho < 1 || o->Wo < 1) return CONV_WGRAD_ERR_BAD_SHAPE;
  o->Cg = d->C / d->groups;
  o->Kg = d->K / d->groups;
  int64_t x_elems, dy_elems, t;
  if (!mul3(o->N, o->Ho, o->Wo, &o->L) || !mul3(o->R, o->S, o->Cg, &o->cols) ||
      !mul_ok(o->K, o->cols, &o->E) || !mul3(o->H, o->W, o->C, &o->x_img) ||
      !mul3(o->Ho, o->Wo, o->K, &o->dy_img) || !mul_ok(o->N, o->x_img, &x_elems) ||
      !mul_ok(o->N, o->dy_img, &dy_elems) || !mul_ok(x_elems, o->esize, &t) ||
      !mul_ok(dy_elems, o->esize, &t) || !mul_ok(o->E, 4, &t))
    return CONV_WGRAD_ERR_BAD_SHAPE;
  o->x_bytes = (uint64_t)x_elems * (uint64_t)o->esize;
  o->dy_bytes = (uint64_t)dy_elems * (uint64_t)o->esize;
  o->dw_bytes = (uint64_t)o->E * 4u;
  // Documented limits: offsets inside one image, the reduction index and the
  // dW index are 32-bit in the kernels; bases of images are 64-bit.
  if (o->x_img > kI32Max || o->dy_img > kI32Max || o->L > kMaxRows || o->E > kI32Max ||
      o->H > kI32Max / 2 || o->W > kI32Max / 2 || o->pad_h > kI32Max / 4 || o->pad_w > kI32Max / 4 ||
      o->stride_h > kI32Max / 4 || o->stride_w > kI32Max / 4 || o->dil_h > kI32Max / 4 ||
      o->dil_w > kI32Max / 4 || o->R > kI32Max / 4 || o->S > kI32Max / 4)
    return CONV_WGRAD_ERR_UNSUPPORTED;

  // Width fold (the foldable f all divide S, stride_w, W and pad_w).
  const bool foldable = o->groups == 1 && o->dil_w == 1;
  const int64_t fmax = foldable ? gcd64(gcd64(o->S, o->stride_w), gcd64(o->W, o->pad_w)) : 1;
  if (d->fold_width >= 2) {
    if (!foldable || fmax % d->fold_width != 0) return CONV_WGRAD_ERR_BAD_SHAPE;
    int64_t fc;
    if (!mul_ok(o->C, d->fold_width, &fc) || fc > kI32Max) return CONV_WGRAD_ERR_UNSUPPORTED;
    apply_fold(o, d->fold_width);
  } else if (d->fold_width == -1 && fmax >= 2 && o->Cg % 4 != 0 && (o->Cg * fmax) % 4 == 0 &&
             o->C * fmax <= kI32Max) {
    apply_fold(o, fmax);
  }
  if (o->fold > 1) {
    o->Cg = o->C;   // one group
    o->cols = o->R * o->S * o->Cg;
  }
  o->uniform = o->pad_h == o->pad_w && o->stride_h == o->stride_w && o->dil_h == o->dil_w;
  o->pad = o->pad_h;
  o->stride = o->stride_h;
  o->dil = o->dil_h;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t choose_split(int64_t units, int64_t tiles, int32_t requested, int64_t min_units,
                                 int64_t target_groups, int64_t traffic_div, const Problem& p,
                                 conv_wgrad_plan_t* pub, int64_t forced_ups, int64_t traffic_mul) {
  int64_t degree;
  if (forced_ups >= 1) {
    degree = ceil_div(units, forced_ups < units ? forced_ups : units);
  } else if (requested >= 1) {
    degree = requested;
  } else {
    degree = target_groups / tiles;
    int64_t by_depth = units / (min_units > 0 ? min_units : 1);
    if (by_depth < 1) by_depth = 1;
    if (degree > by_depth) degree = by_depth;
    uint64_t alg = p.x_bytes + p.dy_bytes + p.dw_bytes;
    uint64_t slab = (uint64_t)p.E * 8u;  // 4 bytes written + 4 bytes read per slab element
    int64_t by_traffic = (int64_t)(alg * (uint64_t)traffic_mul / ((uint64_t)traffic_div * slab));
    if (by_traffic < 1) by_traffic = 1;
    if (degree > by_traffic) degree = by_traffic;
    if (degree < 1) degree = 1;
  }
  if (degree > units) degree = units;
  if (degree > kMaxSlices) degree = kMaxSlices;
  pub->units = units;
  pub->units_per_slice = ceil_div(units, degree);
  // A forced slice length is kept as given (a later slice may be shorter).
  if (forced_ups >= 1 && pub->units_per_slice < forced_ups && forced_ups <= units)
    pub->units_per_slice = forced_ups;
  int64_t ks = ceil_div(units, pub->units_per_slice);
  if (ks > kI32Max) return CONV_WGRAD_ERR_UNSUPPORTED;
  pub->ks_count = (int32_t)ks;
  pub->needs_reduce = ks > 1 ? 1 : 0;
  pub->tiles = tiles;
  int64_t grid;
  if (!mul_ok(tiles, ks, &grid) || grid > kI32Max) return CONV_WGRAD_ERR_UNSUPPORTED;
  // A launch's lanes (workgroups x lanes per workgroup) must stay below 2^32:
  // stage 1 (at most kMaxBlock lanes per workgroup, plus the up to 7
  // workgroups the XCD-ordered grids round up by) and the slab fold.
  if ((grid + 8) * kMaxBlock >= kLaunchLanes) return CONV_WGRAD_ERR_UNSUPPORTED;
  if (ks > 1 && (ceil_div(p.E, kFoldElemsPerBlock) + ceil_div(p.K, kFoldElemsPerBlock)) * kFoldBlock >=
                    kLaunchLanes)
    return CONV_WGRAD_ERR_UNSUPPORTED;
  pub->grid = grid;
  pub->slab_stride = ceil_div(db_offset(p) + p.K, 64) * 64;   // dW partial, then db partial
  int64_t ws_elems;
  if (ks > 1) {
    if (!mul_ok(pub->slab_stride, ks, &ws_elems) || ws_elems > INT64_MAX / 4)
      return CONV_WGRAD_ERR_UNSUPPORTED;
    pub->ws_bytes = (uint64_t)ws_elems * 4u;
  } else {
    pub->ws_bytes = 0;
  }
  return CONV_WGRAD_OK;
}

namespace {

int vec_width(int64_t n) { return n % 4 == 0 ? 4 : 1; }

// Limits of the row-unit kernel's LDS tiles (see dense_rows.hip).
constexpr int kRowsMaxWt = 64, kRowsMaxXSpan = 80;

// Row-unit dense kernel: channel counts in whole quads, and a staged X
// segment of at most 80 pixels for at least 16 output pixels per unit.
bool plan_dense_rows(const Problem& p, Plan* out) {
  if (p.Kg % 4 != 0 || p.Cg % 4 != 0) return false;
  // Buffer loads address one X or dY row with 32-bit byte offsets: a lane's
  // offsets reach 64 dY pixels past the unit's first one, and X columns from
  // -pad to past the image by up to the staged span plus the filter's reach.
  if (p.W * p.C * p.esize > kI32Max / 2 || p.Wo * p.K * p.esize > kI32Max / 2) return false;
  int64_t dy_reach, x_cols, x_reach;
  if (!mul3(kRowsMaxWt, p.K, p.esize, &dy_reach) || dy_reach > kI32Max / 2) return false;
  if (!mul_ok(p.S, p.dil_w, &x_cols) || x_cols > kI32Max) return false;
  x_cols += p.W + 2 * p.pad_w + kRowsMaxXSpan;
  if (!mul3(x_cols, p.C, p.esize, &x_reach) || x_reach > kI32Max / 2) return false;
  const int64_t sb = p.S < 4 ? p.S : 4;
  int64_t wt = 0;
  for (int64_t cand = kRowsMaxWt; cand >= 16; cand -= 16) {
    if ((cand - 1) * p.stride_w + (sb - 1) * p.dil_w + 1 <= kRowsMaxXSpan) {
      wt = cand;
      break;
    }
  }
  if (wt == 0) return false;
  const int64_t wo16 = ceil_div(p.Wo, 16) * 16;
  if (wt > wo16) wt = wo16;
  out->sb = (int32_t)sb;
  out->wt = (int32_t)wt;
  out->xspan = (int32_t)((wt - 1) * p.stride_w + (sb - 1) * p.dil_w + 1);
  out->s_blocks = ceil_div(p.S, sb);
  out->c_tiles = ceil_div(p.Cg, 64);
  out->m_tiles = ceil_div(p.Kg, 64);
  out->wchunks = ceil_div(p.Wo, wt);
  // Packed rows (dense_rows.hip): four output rows of at most 14 pixels per
  // unit at unit row stride and unit column stride and dilation, each row's
  // X segment (Wo + SB - 1 pixels) within the 16 columns the loader stages.
  // A unit's rows are staged QA (dY) and QB (X) pixel slots apart, each the
  // smallest of 2, 6, 10, 14 (, 18) that holds the row (QA * 72 and QB * 72
  // are then 16 or 48 mod 64 banks); the reads one k-step past the last must
  // stay in the 64 dY and 72 X slots.
  out->ru = 1;
  out->qa = out->qb = 0;
  if (p.stride_h == 1 && p.stride_w == 1 && p.dil_w == 1 && p.Wo <= 14) {
    auto slots = [](int64_t need, int64_t cap) -> int64_t {
      for (int64_t c = 2; c <= cap; c += 4)
        if (c >= need) return c;
      return 0;
    };
    const int64_t xw = p.Wo + sb - 1;   // X pixels of a row segment
    const int64_t qa = slots(p.Wo, 14), qb = slots(xw, 18);
    if (xw <= 16 && qa > 0 && qb > 0 && 3 * qa + p.Wo <= 63 && 3 * qb + xw <= 71) {
      out->ru = 4;
      out->qa = (int32_t)qa;
      out->qb = (int32_t)qb;
    }
  }
  return true;
}

// 1x1 streaming kernel: fp32, unpadded stride-1 1x1 filter, output channels in
// whole 64-channel tiles and input channels in 16-channel lane groups.
bool plan_dense_1x1(const Problem& p, Plan* out) {
  if (p.dtype != CONV_WGRAD_F32 || p.R != 1 || p.S != 1 || p.pad_h != 0 || p.pad_w != 0 ||
      p.stride_h != 1 || p.stride_w != 1)
    return false;
  if (p.Kg % 64 != 0 || p.Cg % 16 != 0) return false;
  // A batch's buffer range (4 rows) and the lane offsets are 32-bit.
  if (p.C > (1 << 26) || p.K > (1 << 26)) return false;
  const int64_t q = p.Cg / 16;
  int32_t bv = 1;
  for (int32_t cand = 8; cand >= 1; --cand) {
    if (q % cand == 0) {
      bv = cand;
      break;
    }
  }
  out->bv = bv;
  out->m_tiles = p.Kg / 64;
  out->c_tiles = q / bv;
  return true;
}

// Block-diagonal 16-bit kernel (grouped16.hip): stride 1, equal channels per
// group dividing 16, channel count in 16-channel super-groups, at most 9 taps,
// and a staged tile of at most 8 X rows x 40 X pixels.
bool plan_grouped16(const Problem& p, Plan* out) {
  if (!p.uniform || p.dtype == CONV_WGRAD_F32 || p.stride != 1 || p.Cg != p.Kg || 16 % p.Cg != 0) return false;
  if (p.C % 16 != 0 || p.R * p.S > 9 || (p.S - 1) * p.dil + 32 > 40) return false;
  int32_t ru = 0;
  for (int32_t cand = 4; cand >= 1; cand /= 2) {
    if ((cand - 1) + (p.R - 1) * p.dil + 1 <= 8) {
      ru = cand;
      break;
    }
  }
  if (ru == 0) return false;
  out->ru = ru;
  out->xrows = (int32_t)((ru - 1) + (p.R - 1) * p.dil + 1);
  out->xspan = (int32_t)(31 + (p.S - 1) * p.dil + 1);
  out->c_tiles = ceil_div(p.C, 64);
  out->wchunks = ceil_div(p.Wo, 32);
  return true;
}

// Row-streaming grouped kernel (grouped16.hip): as the block-diagonal kernel,
// plus stride 1 or 2, no dilation, a 1x1, 3x3, 5x5 or 7x7 filter, output rows
// of at most 64 pixels at stride 1 (two MFMA k-steps) or 32 at stride 2, and
// padding below the filter size.
bool plan_grouped16_rows(const Problem& p, Plan* out) {
  if (!p.uniform || p.dtype == CONV_WGRAD_F32 || (p.stride != 1 && p.stride != 2) || p.dil != 1 || p.Cg != p.Kg ||
      16 % p.Cg != 0)
    return false;
  // Rows of up to 64 output pixels at stride 1 (two MFMA k-steps), 32 at stride 2.
  if (p.C % 16 != 0 || p.Wo > (p.stride == 1 ? 64 : 32) || p.pad >= p.S || p.pad >= p.R) return false;
  if (p.R != p.S || !(p.R == 1 || p.R == 3 || p.R == 5 || p.R == 7)) return false;
  if (p.W * p.C * 2 > kI32Max / 2 || p.Wo * p.K * 2 > kI32Max / 2) return false;
  out->c_tiles = ceil_div(p.C, 64);
  return true;
}

// 16-bit dense row kernel (dense16_rows.hip): stride 1, dilation 1, channel
// counts in whole 16-byte chunks (8 channels); units of up to 64 output pixels
// (32 when the output row is that short), up to 4 taps per tile.
bool plan_dense16_rows(const Problem& p, Plan* out) {
  // 16-bit inputs, or fp32 inputs under BF16x3 (split into two bf16 planes at staging).
  const bool x3 = p.dtype == CONV_WGRAD_F32 && p.math == CONV_WGRAD_MATH_BF16X3;
  if ((p.dtype == CONV_WGRAD_F32 && !x3) || p.stride_h != 1 || p.stride_w != 1 || p.dil_h != 1 || p.dil_w != 1)
    return false;
  if (p.C % 8 != 0 || p.K % 8 != 0 || p.Cg % 8 != 0 || p.Kg % 8 != 0) return false;
  const int64_t es = p.esize;
  if (p.W * p.C * es > kI32Max / 2 || p.Wo * p.K * es > kI32Max / 2) return false;
  // Lane offsets reach 64 dY pixels into a unit and X columns from -pad to
  // past the image by the staged 96 pixels plus the filter's reach.
  int64_t dy_reach, x_reach;
  if (!mul3(64, p.K, es, &dy_reach) || dy_reach > kI32Max / 2) return false;
  if (!mul3(p.W + 2 * p.pad_w + p.S + 96, p.C, es, &x_reach) || x_reach > kI32Max / 2) return false;
  out->sb = (int32_t)(p.S < 4 ? p.S : 4);
  out->wt = p.Wo > 32 ? 64 : 32;
  out->s_blocks = ceil_div(p.S, out->sb);
  out->c_tiles = ceil_div(p.Cg, 64);
  out->m_tiles = ceil_div(p.Kg, 64);
  out->wchunks = ceil_div(p.Wo, out->wt);
  // Short rows: units of ru output rows staged at a pitch of Wo + SB - 1
  // pixels in the 64 slots of a unit (ru >= 2).
  const int64_t pitch = p.Wo + out->sb - 1;
  out->ru = pitch <= 32 ? (int32_t)(64 / pitch) : 1;
  // A unit's rows are one buffer range each for X and dY (32-bit).
  // (Below 2^30, so the out-of-range offset the loaders use for empty slots
  // lies past every range.)
  if (out->ru > 1 && (out->ru * p.W * p.C * es > kI32Max / 2 || out->ru * p.Wo * p.K * es > kI32Max / 2))
    out->ru = 1;
  if (out->ru > 1) {
    out->wt = 64;
    out->wchunks = 1;
  }
  return true;
}

// 16-bit dense kernel with all taps per tile (dense16_taps.hip): 3 x 3
// filters, stride 1, dilation 1, channel counts in whole 8-channel chunks,
// output rows short enough that one padded row (P = Wo + 2 slots) fits a
// 64-slot unit and the unit's X rows fit 192 staged slots (P <= 63).
bool plan_dense16_taps(const Problem& p, Plan* out) {
  const bool x3 = p.dtype == CONV_WGRAD_F32 && p.math == CONV_WGRAD_MATH_BF16X3;
  if ((p.dtype == CONV_WGRAD_F32 && !x3) || p.stride_h != 1 || p.stride_w != 1 || p.dil_h != 1 || p.dil_w != 1)
    return false;
  if (p.R != 3 || p.S != 3) return false;
  if (p.C % 8 != 0 || p.K % 8 != 0 || p.Cg % 8 != 0 || p.Kg % 8 != 0) return false;
  // 16-bit groups of at most 64 x 64 channels keep the row kernel (3 x 3 C = K
  // = 64 56x56: 29.3 us there, 31.3 us here, whose one tile per slice holds
  // the whole gradient and doubles the slab bytes per workgroup).
  if (!x3 && p.Kg <= 64 && p.Cg <= 64) return false;
  const int64_t pitch = p.Wo + p.S - 1;
  const int64_t need = 64 + (p.R - 1) * pitch + p.S - 1;   // X slots the MFMAs of a unit read
  if (pitch > 64 || need > 192) return false;
  const int64_t ru = 64 / pitch;
  // Buffer ranges of a unit's dY rows and X rows, and every lane offset in
  // them, below 2^30 (the out-of-range offset the loaders use lies past them).
  const int64_t es = p.esize;
  int64_t dy_bytes, x_bytes;
  if (!mul3(ru * p.Wo, p.K, es, &dy_bytes) || dy_bytes > kI32Max / 2) return false;
  if (!mul3((ru + p.R) * p.W, p.C, es, &x_bytes) || x_bytes > kI32Max / 2) return false;
  out->ru = (int32_t)ru;
  out->sb = (int32_t)p.S;
  out->xspan = need <= 128 ? 128 : need <= 160 ? 160 : 192;
  // 16-bit: 32 output channels per tile (two workgroups fit a CU); BF16x3
  // (one workgroup per CU, 160 KB of LDS at most): 64, which halves the B
  // operand reads per MFMA of its three products.
  out->bm = x3 && p.Kg > 32 ? 64 : 32;
  out->m_tiles = ceil_div(p.Kg, out->bm);
  out->c_tiles = ceil_div(p.Cg, 64);
  return true;
}

// Depthwise 4x4x4 kernel (depthwise_mfma.hip): 16-bit, one channel per group,
// stride 1, no dilation, channels in whole 16-channel groups, filter up to
// 12 x 12 (blocks of 4 filter rows / columns: 1 or 2 each up to 8 x 8, 3 x 3
// above), rows of at most 120 columns staged as 8 mod 16 columns, padding up
// to 12.  A staged dY row holds element 0 at an even column off with
// 4 * (SB - 1) + 3 <= pad + off <= 12, so every lane's window blocks, from
// SB - 1 column steps before column 0 to one past the row, lie in the xl + 16
// staged columns.
//
// Stride 2 (filters up to 8 x 8) stages each dY row upsampled, element wo at
// column off + 2 wo with zeros between, so the column windows are those of
// stride 1 on an output row twice as long; off is then a multiple of 4 (the
// stores of a pixel pair are 8-byte aligned).  X rows advance two per output
// row.
bool plan_depthwise(const Problem& p, Plan* out) {
  if (!p.uniform || p.dtype == CONV_WGRAD_F32 || p.Cg != 1 || p.Kg != 1 || p.dil != 1) return false;
  if (p.stride != 1 && p.stride != 2) return false;
  if (p.C % 16 != 0 || p.C > (1 << 20) || p.R > 12 || p.S > 12 || p.pad > 12) return false;
  if (p.W > 120 || p.Wo > 128 || p.W * p.C * 2 > kI32Max) return false;
  int64_t xl = 8;
  while (xl < p.W) xl += 16;
  const int64_t np = xl > 64 ? 2 : 1;
  const bool blocks3 = p.R > 8 || p.S > 8;        // 3 x 3 filter blocks
  if (p.stride == 2 && blocks3) return false;
  int64_t off;
  if (p.stride == 2) {
    off = 0;
    while (p.pad + off < 7) off += 4;
  } else {
    off = ((blocks3 ? 12 : 8) - p.pad) & ~(int64_t)1;
    if (off < 0) off = 0;
  }
  const int64_t staged = p.stride * 2 * ceil_div(p.Wo, 2);   // dY columns the pixel pairs cover
  if (p.Wo > 64 * np || staged + off > xl + 16) return false;
  const int32_t lds = depthwise_lds_bytes((int32_t)xl, (int32_t)p.R, (int32_t)p.S);
  if (lds <= 0 || lds > kDwLdsMax) return false;
  out->dw_xl = (int32_t)xl;
  out->dw_lds = lds;
  out->dw_off = (int32_t)off;
  out->c_tiles = ceil_div(p.C, 64);
  return true;
}

}  // namespace

// Depthwise slices balanced by staging steps.  A slice of output rows stages,
// per image segment of len rows, stride * (len - 1) + R X rows (one step
// each); uniform runs of rows leave the slices that straddle an image
// boundary R - 1 steps longer than the others, and the longest slice sets the
// kernel's time.  For the planned slice count: the smallest largest-cost T a
// greedy fill needs at most that many slices for (binary search), that fill,
// then the slices with the most rows halved until the count is met (no slice
// cost grows).  The count, and so the grid and the workspace, are unchanged.
namespace {
void balance_depthwise(const Problem& p, Plan* out) {
  conv_wgrad_plan_t& pub = out->pub;
  const int64_t ks = pub.ks_count, rows = p.N * p.Ho;
  if (ks < 2 || ks > Plan::kDwMaxSlices || rows > (1 << 22)) return;
  int32_t* st = out->dw_starts;
  auto greedy = [&](int64_t T, bool fill) -> int64_t {
    int64_t count = 0, cost = 0;
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t add = r % p.Ho == 0 ? p.R : p.stride;   // a segment's first row stages R rows
      if (count == 0 || cost + add > T) {
        if (count >= ks) return count + 1;                   // over the count: T is too small
        if (fill) st[count] = (int32_t)r;
        ++count;
        cost = p.R;
      } else {
        cost += add;
      }
    }
    return count;
  };
  int64_t lo = p.R, hi = p.N * (p.stride * (p.Ho - 1) + p.R);
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (greedy(mid, false) <= ks) hi = mid;
    else lo = mid + 1;
  }
  int64_t count = greedy(lo, true);
  st[count] = (int32_t)rows;
  while (count < ks) {
    int64_t best = 0;
    for (int64_t i = 1; i < count; ++i)
      if (st[i + 1] - st[i] > st[best + 1] - st[best]) best = i;
    const int32_t len = st[best + 1] - st[best];
    if (len < 2) return;   // cannot happen: ks <= rows (leave the uniform slices)
    for (int64_t i = count + 1; i > best + 1; --i) st[i] = st[i - 1];
    st[best + 1] = st[best] + len / 2;
    ++count;
  }
  int32_t longest = 0;
  for (int64_t i = 0; i < ks; ++i) longest = st[i + 1] - st[i] > longest ? st[i + 1] - st[i] : longest;
  pub.units_per_slice = longest;
  out->dw_balanced = 1;
}
}  // namespace

conv_wgrad_status_t make_plan(const conv_wgrad_desc2_t* desc, Plan* out) {
  if (!desc || !out) return CONV_WGRAD_ERR_NULL_ARG;
  memset(out, 0, sizeof(*out));
  Problem& p = out->p;
  conv_wgrad_status_t st = canonicalise(desc, &p);
  if (st != CONV_WGRAD_OK) return st;
  conv_wgrad_plan_t& pub = out->pub;
  pub.Ho = p.Ho;
  pub.Wo = p.Wo;
  pub.L = p.L;
  pub.E = p.E;
  pub.x_bytes = p.x_bytes;
  pub.dy_bytes = p.dy_bytes;
  pub.dw_bytes = p.dw_bytes;
  const uint64_t big = p.x_bytes > p.dy_bytes ? p.x_bytes : p.dy_bytes;
  pub.windows_4g = (int64_t)((big + ((uint64_t)1 << 32) - 1) >> 32);

  const bool small_groups = p.groups > 1 && p.Cg <= 8 && p.Kg <= 8;
  if (small_groups && plan_depthwise(p, out)) {
    pub.path = CONV_WGRAD_PATH_DIRECT;
    pub.variant = kDepthwise;
    pub.unit_rows = p.Wo;  // a unit is one output row
    int64_t units;
    if (!mul_ok(p.N, p.Ho, &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
    // Four-wave workgroups, as many per CU as the LDS holds.
    const int64_t per_cu = kDwLdsMax / out->dw_lds;
    st = choose_split(units, out->c_tiles, desc->split_k, 8, 256 * per_cu, 4, p, &pub);
    if (st == CONV_WGRAD_OK) balance_depthwise(p, out);
    return st;
  }
  if (small_groups && plan_grouped16_rows(p, out)) {
    pub.path = CONV_WGRAD_PATH_DIRECT;
    pub.variant = kGrouped16Rows;
    pub.unit_rows = p.Wo;  // a unit is one output row
    int64_t units;
    if (!mul_ok(p.N, p.Ho, &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
    // Four-wave workgroups, about one per CU, each streaming long runs of rows.
    // Slabs may cost up to half the algorithmic bytes (the larger filters
    // have large slabs, and a half-empty device costs more).
    if (desc->split_k >= 1) return choose_split(units, out->c_tiles, desc->split_k, 8, 256, 2, p, &pub);
    // A slice that straddles two images restarts the row pipeline (and
    // re-reads R - 1 halo rows), so the automatic slice length is rounded to
    // the nearest whole number of images, or up to a divisor of an image's rows.
    conv_wgrad_plan_t probe = pub;
    st = choose_split(units, out->c_tiles, -1, 8, 256, 2, p, &probe);
    if (st != CONV_WGRAD_OK) return st;
    int64_t ups = probe.units_per_slice;
    if (ups >= p.Ho) {
      ups = (ups + p.Ho / 2) / p.Ho * p.Ho;
    } else {
      while (p.Ho % ups != 0) ++ups;
    }
    return choose_split(units, out->c_tiles, -1, 8, 256, 2, p, &pub, ups);
  }
  if (small_groups && plan_grouped16(p, out)) {
    pub.path = CONV_WGRAD_PATH_DIRECT;
    pub.variant = kGrouped16;
    pub.unit_rows = (int64_t)out->ru * 32;
    int64_t units;
    if (!mul3(p.N, ceil_div(p.Ho, out->ru), out->wchunks, &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
    // 2 (3 for the 3x3 and 1x1 fast path) workgroups per CU fit in LDS.
    return choose_split(units, out->c_tiles, desc->split_k, 2, 768, 4, p, &pub);
  }
  if (small_groups) {
    // Direct path: one dW element per lane; a unit is 64 output pixels.
    pub.path = CONV_WGRAD_PATH_DIRECT;
    pub.variant = kDirectElem;
    out->threads = 256;
    pub.unit_rows = 64;
    int64_t units = ceil_div(p.L, pub.unit_rows);
    int64_t tiles = ceil_div(p.E, out->threads);
    return choose_split(units, tiles, desc->split_k, 16, 2048, 4, p, &pub);
  }
  // Dense implicit GEMM per group.
  pub.path = CONV_WGRAD_PATH_DENSE;
  // Launch-bound problems (at most 2^20 FLOP with an automatic split: the
  // whole reduction takes a few microseconds on one workgroup) run in one
  // launch on the general kernel; a split would add a dependent fold launch
  // to a call that is nothing but launch latency.
  const bool tiny = desc->split_k < 1 && p.L <= (1 << 20) && p.E <= (1 << 20) && 2 * p.L * p.E <= (1 << 20);
  if (!tiny && plan_dense_1x1(p, out)) {
    pub.variant = kDense1x1;
    pub.unit_rows = 64;
    int64_t tiles;
    if (!mul3(p.groups, out->m_tiles, out->c_tiles, &tiles)) return CONV_WGRAD_ERR_UNSUPPORTED;
    // One-wave workgroups, about eight per CU.
    return choose_split(ceil_div(p.L, 64), tiles, desc->split_k, 4, 2048, 4, p, &pub);
  }
  if (!tiny && plan_dense16_taps(p, out)) {
    pub.variant = p.dtype == CONV_WGRAD_F32 ? kDense16TapsX3 : kDense16Taps;
    pub.unit_rows = out->ru * p.Wo;   // a unit is ru whole output rows
    int64_t units, tiles;
    if (!mul_ok(p.N, ceil_div(p.Ho, out->ru), &units) || !mul3(p.groups, out->m_tiles, out->c_tiles, &tiles))
      return CONV_WGRAD_ERR_UNSUPPORTED;
    // Measured on 3x3 shapes of 14x14 to 56x56: the call time is set by the
    // units per workgroup (a unit costs ~1 us whatever its MFMA work) and the
    // slab bytes, and is lowest at 14-16 units per slice with up to two
    // workgroups per CU (16-bit) or about 7 with one (BF16x3); slab traffic
    // up to 8x the algorithmic bytes pays off there.
    if (pub.variant == kDense16TapsX3) return choose_split(units, tiles, desc->split_k, 7, 256, 1, p, &pub, 0, 8);
    return choose_split(units, tiles, desc->split_k, 14, 512, 1, p, &pub, 0, 8);
  }
  if (!tiny && plan_dense16_rows(p, out)) {
    const bool x3 = p.dtype == CONV_WGRAD_F32;   // BF16x3 (the planner only allows it then)
    pub.variant = x3 ? kDense16RowsX3 : kDense16Rows;
    int64_t units, tiles;
    if (out->ru > 1) {
      pub.unit_rows = out->ru * p.Wo;   // a unit is ru whole output rows
      if (!mul_ok(p.N, ceil_div(p.Ho, out->ru), &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
    } else {
      pub.unit_rows = out->wt;
      if (!mul3(p.N, p.Ho, out->wchunks, &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
    }
    if (!mul4(p.groups, out->m_tiles, p.R, out->s_blocks, &tiles) ||
        !mul_ok(tiles, out->c_tiles, &tiles))
      return CONV_WGRAD_ERR_UNSUPPORTED;
    // Three 256-lane workgroups fit per CU (42 KB of LDS each), two per CU
    // are targeted.  A unit costs the same time whatever the MFMA work, so
    // slices are worth up to 4x the algorithmic bytes in slab traffic.  Units
    // of several short rows carry ~4x the MFMA work of a single short row:
    // three per CU, and slab traffic up to 8x (it overlaps the MFMAs).
    // BF16x3 holds two planes (82.5 KB of LDS): one workgroup per CU.
    if (x3) return choose_split(units, tiles, desc->split_k, 2, 256, 1, p, &pub, 0, 4);
    if (out->ru > 1) return choose_split(units, tiles, desc->split_k, 2, 768, 1, p, &pub, 0, 8);
    return choose_split(units, tiles, desc->split_k, 2, 512, 1, p, &pub, 0, 4);
  }
  // A width fold exists to give the general kernel 4-wide input-channel loads
  // (three input channels become 48 for a 16x16 patch); the row kernel would
  // take the folded problem's few-pixel output rows one unit each (a 16x16
  // stride-16 patch embedding of 224x224 images ran at 644 us folded on the
  // row kernel against 329 us unfolded on the general kernel).
  if (!tiny && p.fold == 1 && plan_dense_rows(p, out)) {
    pub.variant = kDenseRows;
    pub.unit_rows = out->wt;
    int64_t units, tiles;
    if (!mul3(p.N, p.Ho, out->wchunks, &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
    if (!mul4(p.groups, out->m_tiles, p.R, out->s_blocks, &tiles) ||
        !mul_ok(tiles, out->c_tiles, &tiles))
      return CONV_WGRAD_ERR_UNSUPPORTED;
    if (out->ru > 1) {
      // Packed rows: 256 lanes, two workgroups per CU, about 768 workgroups
      // (3x3 fp32 C=K=512 14x14 N=8, 192 tiles, cold call at 1 / 2 / 3 / 4 /
      // 8 slices: 107 / 104 / 113 / 89 / 101 us); slabs may cost up to 6x
      // the algorithmic bytes, since a deep reduction over few, short rows
      // otherwise leaves most of the CUs idle.
      pub.unit_rows = out->ru * p.Wo;
      if (!mul_ok(p.N, ceil_div(p.Ho, out->ru), &units)) return CONV_WGRAD_ERR_UNSUPPORTED;
      out->threads = 256;
      return choose_split(units, tiles, desc->split_k, 2, 768, 1, p, &pub, 0, 6);
    }
    // Two workgroup shapes (Plan::threads).  256 lanes, two workgroups per
    // CU, each staging and computing its own units: the CU interleaves the
    // two, so one's staging and barriers overlap the other's MFMAs and two
    // waves per SIMD keep the MFMA pipe fed (3x3 fp32 C=K=64 56x56 N=32: 75.6
    // -> 71.9 us), taken when the split gives at least 1.5 workgroups per CU.
    // Otherwise 512 lanes, one workgroup per CU, whose two halves ping-pong
    // (one stages while the other computes): with few units the 256-lane form
    // would leave half of each CU idle (3x3 C=K=512 14x14 N=8, 192 tiles and
    // one slice: 126 us ping-pong, 158 us with 256 lanes).  Slabs may cost up
    // to the algorithmic bytes, since this kernel is MFMA-bound on the shapes
    // it takes.
    conv_wgrad_status_t st = choose_split(units, tiles, desc->split_k, 2, 512, 1, p, &pub);
    if (st != CONV_WGRAD_OK) return st;
    if (pub.grid >= 384) {
      out->threads = 256;
      // The interleaved form (strided or dilated columns, rows wider than a
      // unit, or ceil(Wo / 4) a multiple of 4) gains from about 768
      // workgroups (3x3 fp32 C=K=64 N=32, stride 2 / dilation 2, 163 vs 256
      // slices: 91.3 vs 84.8 / 82.2 vs 79.8 us cold); the quarters form does
      // not (56x56: 78.3 vs 95.3 us).
      const bool quarters = p.stride_w == 1 && p.dil_w == 1 && out->wchunks == 1 && ((p.Wo + 3) / 4) % 4 != 0;
      if (!quarters && desc->split_k < 1) return choose_split(units, tiles, desc->split_k, 2, 768, 1, p, &pub, 0, 2);
      return CONV_WGRAD_OK;
    }
    out->threads = 512;
    return choose_split(units, tiles, desc->split_k, 2, 256, 1, p, &pub);
  }
  pub.variant = kDenseLds;
  out->bm = 64;
  out->bn = 64;
  out->bk = 32;
  out->m_tiles = ceil_div(p.Kg, out->bm);
  out->n_tiles = ceil_div(p.cols, out->bn);
  out->vec_a = vec_width(p.Kg);
  out->vec_b = vec_width(p.Cg);
  pub.unit_rows = out->bk;
  int64_t units = ceil_div(p.L, pub.unit_rows);
  int64_t tiles;
  if (!mul3(p.groups, out->m_tiles, out->n_tiles, &tiles)) return CONV_WGRAD_ERR_UNSUPPORTED;
  // About 8 workgroups per CU (the kernel's 20 KB of LDS allow it, and the
  // waves hide each other's staging and loads), slabs up to the algorithmic
  // bytes: 16x16 stride-16 patch embedding fp32 N=64 (144 tiles), 2 / 4 / 8 /
  // 16 / 24 slices: 327 / 228 / 179 / 167 / 179 us hot.
  return choose_split(units, tiles, tiny ? 1 : desc->split_k, 8, 2048, 1, p, &pub);
}

conv_wgrad_status_t make_igemm_plan(const conv_wgrad_desc2_t* desc, int32_t direction, Plan* out) {
  if (!desc || !out) return CONV_WGRAD_ERR_NULL_ARG;
  if (direction != CONV_DIRECTION_FWD && direction != CONV_DIRECTION_DGRAD) return CONV_WGRAD_ERR_BAD_DTYPE;
  memset(out, 0, sizeof(*out));
  Problem& p = out->p;
  conv_wgrad_status_t st = canonicalise(desc, &p);
  if (st != CONV_WGRAD_OK) return st;
  p.math = CONV_WGRAD_MATH_EXACT;   // no BF16x3 kernel for these directions
  const bool fwd = direction == CONV_DIRECTION_FWD;
  conv_wgrad_plan_t& pub = out->pub;
  pub.path = CONV_WGRAD_PATH_DENSE;
  pub.variant = fwd ? kFwdIgemm : kDgradIgemm;
  pub.Ho = p.Ho;
  pub.Wo = p.Wo;
  pub.x_bytes = p.x_bytes;
  pub.dy_bytes = p.dy_bytes;
  pub.dw_bytes = p.dw_bytes;   // the filter (read by these directions)
  // Output pixels, channels and the per-group reduction length.
  int64_t M, Q, E;
  if (fwd) {
    M = p.L;
    if (!mul3(p.R, p.S, p.Cg, &Q)) return CONV_WGRAD_ERR_UNSUPPORTED;
  } else {
    if (!mul3(p.N, p.H, p.W, &M)) return CONV_WGRAD_ERR_UNSUPPORTED;
    if (!mul3(p.R, p.S, p.Kg, &Q)) return CONV_WGRAD_ERR_UNSUPPORTED;
  }
  const int64_t NT = fwd ? p.K : p.C, Ng = fwd ? p.Kg : p.Cg;
  if (!mul_ok(M, NT, &E)) return CONV_WGRAD_ERR_UNSUPPORTED;
  // Pixel and reduction indices are 32-bit in the kernel; the output index is 64-bit.
  if (M > kMaxRows || Q > kI32Max - 64) return CONV_WGRAD_ERR_UNSUPPORTED;
  const uint64_t out_bytes = (uint64_t)E * 4u;
  const uint64_t big = p.x_bytes > out_bytes ? p.x_bytes : out_bytes;
  pub.windows_4g = (int64_t)((big + ((uint64_t)1 << 32) - 1) >> 32);
  pub.L = M;
  pub.E = E;
  p.E = E;   // the slab fold covers the output
  out->m_tiles = ceil_div(M, 64);
  out->n_tiles = ceil_div(Ng, 64);
  // 16-byte loads along the contiguous axis: the gathered tensor's channels
  // of a group (c forward, k dgrad); the filter along q (forward, whole rows)
  // or along c (dgrad).
  out->vec_a = (fwd ? p.Cg : p.Kg) % 4 == 0 ? 4 : 1;
  out->vec_b = fwd ? (Q % 4 == 0 ? 4 : 1) : (p.Cg % 4 == 0 ? 4 : 1);
  int64_t tiles;
  if (!mul3(p.groups, out->m_tiles, out->n_tiles, &tiles)) return CONV_WGRAD_ERR_UNSUPPORTED;
  pub.unit_rows = 32;
  const int64_t units = ceil_div(Q, 32);
  int64_t degree;
  if (desc->split_k >= 1) {
    degree = desc->split_k;
  } else {
    // Split only a grid under half of 8 workgroups per CU (the kernel keeps
    // 6-7 resident per CU) over a reduction at least 512 deep, by the
    // smallest power of two that reaches 8 workgroups per CU, at most 32, with
    // at least two reduction tiles per slice.  Measured on the 3x3 C=K=512
    // 14x14 N=8 forward (200 tiles): 1 / 2 / 4 / 8 / 16 / 32 slices took
    // 151 / 124 / 108 / 95 / 91 / 97 us.
    constexpr int64_t kThreshold = 4 * 256, kTarget = 8 * 256;
    degree = 1;
    if (tiles < kThreshold && Q >= 512) {
      while (tiles * degree < kTarget && degree * 2 <= 32 && units / (degree * 2) >= 2) degree *= 2;
    }
  }
  if (degree > units) degree = units;
  if (degree > kMaxSlices) degree = kMaxSlices;
  pub.units = units;
  pub.units_per_slice = ceil_div(units, degree);
  const int64_t ks = ceil_div(units, pub.units_per_slice);
  pub.ks_count = (int32_t)ks;
  pub.needs_reduce = ks > 1 ? 1 : 0;
  pub.tiles = tiles;
  int64_t grid;
  if (!mul_ok(tiles, ks, &grid) || grid > kI32Max || grid * 256 >= kLaunchLanes) return CONV_WGRAD_ERR_UNSUPPORTED;
  if (ks > 1 && ceil_div(E, kFoldElemsPerBlock) * kFoldBlock >= kLaunchLanes) return CONV_WGRAD_ERR_UNSUPPORTED;
  pub.grid = grid;
  pub.slab_stride = ceil_div(E, 64) * 64;
  if (ks > 1) {
    int64_t ws_elems;
    if (!mul_ok(pub.slab_stride, ks, &ws_elems) || ws_elems > INT64_MAX / 4) return CONV_WGRAD_ERR_UNSUPPORTED;
    pub.ws_bytes = (uint64_t)ws_elems * 4u;
  } else {
    pub.ws_bytes = 0;
  }
  return CONV_WGRAD_OK;
}

}  // namespace cw
