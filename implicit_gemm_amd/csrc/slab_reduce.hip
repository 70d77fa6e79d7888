// Stage 2: deterministic fold of the fp32 partial slabs (gfx950).
//
// dw[e] = (((ws[0][e] + ws[1][e]) + ws[2][e]) + ... ) + ws[ks-1][e], fp32
// round-to-nearest-even adds in ascending slice order, then a plain store: no
// epilogue is applied to partial sums (the two-stage split-K of
// rocm-libraries PR #14393, sections "Two-stage split-K" and "Review
// follow-ups").  Each lane folds 4 consecutive elements with 16-byte loads.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

struct ReduceArgs {
  const float* ws;
  float* dw;
  int64_t E, slab_stride;
  int32_t ks;
};

__global__ __launch_bounds__(256) void slab_reduce_kernel(ReduceArgs a) {
  const float* __restrict__ ws = a.ws;
  float* __restrict__ dw = a.dw;
  const int64_t E = a.E, slab_stride = a.slab_stride;
  const int32_t ks = a.ks;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= E) return;
  if (i + 4 <= E) {
    float4 acc = *reinterpret_cast<const float4*>(ws + i);
    for (int32_t j = 1; j < ks; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(ws + (int64_t)j * slab_stride + i);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(dw + i) = acc;  // dw is 16-byte aligned (checked by the ABI)
  } else {
    for (int64_t e = i; e < E; ++e) {
      float acc = ws[e];
      for (int32_t j = 1; j < ks; ++j) acc += ws[(int64_t)j * slab_stride + e];
      dw[e] = acc;
    }
  }
}

}  // namespace

hipError_t launch_slab_reduce(const Plan& plan, const float* ws, float* dw, hipStream_t stream) {
  const int64_t E = plan.p.E;
  const int64_t blocks = (E + 1023) / 1024;
  ReduceArgs a{ws, dw, E, plan.pub.slab_stride, plan.pub.ks_count};
  return launch_kernel(slab_reduce_kernel, dim3((unsigned)blocks), dim3(256), a, stream);
}

}  // namespace cw
