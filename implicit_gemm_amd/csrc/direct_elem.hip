// Direct weight gradient for small groups, one dW element per lane (gfx950).
//
// For grouped convolutions with at most 8 channels per group (depthwise,
// 4 and 8 channels per group: the cases of rocm-libraries PR #14157,
// "depthwise 7x7 and grouped cpg4/8 wgrad", section Technical Details) each
// dW element is a dot product over the output pixels of one slice:
//   dW[k][(r*S + s)*Cg + c] = sum_l dY[l][k] * X[n][h(ho,r)][w(wo,s)][g(k)*Cg + c]
// Lanes are ordered with k fastest, so the loads of one wave are consecutive
// channels of one pixel.  The pixel loop is uniform across the workgroup.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

struct DirectArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;
  int32_t H, W, C, K, Ho, Wo;
  int32_t R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, Cg, Kg;
  int32_t taps;  // R*S*Cg
  int32_t E;     // K*taps
  int32_t L, pix_per_slice, ks_count;
  float* dbo;    // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
};

template <typename T>
__global__ __launch_bounds__(256) void direct_elem_kernel(DirectArgs a) {
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ dy = static_cast<const T*>(a.dy);
  const int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  const int tile = bid / a.ks_count;
  const int e = tile * 256 + (int)threadIdx.x;  // tap-major: e = t*K + k
  if (e >= a.E) return;                          // no barrier in this kernel
  const int k = e % a.K, t = e / a.K;
  const int c = t % a.Cg, rs = t / a.Cg;
  const int s = rs % a.S, r = rs / a.S;
  const int ch = (k / a.Kg) * a.Cg + c;
  const int dh = r * a.dil_h - a.pad_h, dw = s * a.dil_w - a.pad_w;
  const int p_begin = slice * a.pix_per_slice;
  const int p_end = min(a.L, p_begin + a.pix_per_slice);
  const int HoWo = a.Ho * a.Wo;
  int n = p_begin / HoWo;
  int rem = p_begin - n * HoWo;
  int ho = rem / a.Wo, wo = rem - ho * a.Wo;
  // The lanes of tap column 0 (e < K) also sum dY[., k] over every pixel of
  // the slice: the bias-gradient partial of channel k.
  const bool db_lane = a.dbo != nullptr && t == 0;
  float acc = 0.f, dbacc = 0.f;
  for (int pix = p_begin; pix < p_end; ++pix) {
    const int h = ho * a.stride_h + dh, w = wo * a.stride_w + dw;
    if (h >= 0 && h < a.H && w >= 0 && w < a.W) {
      const float gy = to_f32(dy[(int64_t)pix * a.K + k]);
      const float xv = to_f32(x[(int64_t)n * a.x_img + ((int64_t)h * a.W + w) * a.C + ch]);
      acc = __builtin_fmaf(gy, xv, acc);
    }
    if (db_lane) dbacc += to_f32(dy[(int64_t)pix * a.K + k]);
    if (++wo == a.Wo) {
      wo = 0;
      if (++ho == a.Ho) { ho = 0; ++n; }
    }
  }
  a.out[(int64_t)slice * a.slab_stride + (int64_t)k * a.taps + t] = acc;
  if (db_lane) a.dbo[(int64_t)slice * a.slab_stride + k] = dbacc;
}

}  // namespace

hipError_t launch_direct(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                         hipStream_t stream) {
  const Problem& p = plan.p;
  DirectArgs a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.x_img = p.x_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.R = (int32_t)p.R; a.S = (int32_t)p.S;
  a.pad_h = (int32_t)p.pad_h; a.pad_w = (int32_t)p.pad_w;
  a.stride_h = (int32_t)p.stride_h; a.stride_w = (int32_t)p.stride_w;
  a.dil_h = (int32_t)p.dil_h; a.dil_w = (int32_t)p.dil_w;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg;
  a.taps = (int32_t)p.cols;
  a.E = (int32_t)p.E;
  a.L = (int32_t)p.L;
  a.pix_per_slice = (int32_t)(plan.pub.units_per_slice * plan.pub.unit_rows);
  a.ks_count = plan.pub.ks_count;
  a.dbo = out.db;
  const dim3 grid((unsigned)plan.pub.grid), block(256);
  switch (p.dtype) {
    case CONV_WGRAD_F32: return launch_kernel(direct_elem_kernel<float>, grid, block, a, stream);
    case CONV_WGRAD_BF16: return launch_kernel(direct_elem_kernel<Bf16>, grid, block, a, stream);
    default: return launch_kernel(direct_elem_kernel<F16>, grid, block, a, stream);
  }
}

}  // namespace cw
