// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace cw {

// Stage-1 output: dw itself (one slice) or the fp32 slab workspace.
struct Stage1Out {
  float* base;           // dw or workspace
  int64_t slab_stride;   // floats between slabs (0 when writing dw)
};

// Launch `kernel(args)`; returns the status of this launch only.
template <typename Args>
inline hipError_t launch_kernel(void (*kernel)(Args), dim3 grid, dim3 block, const Args& args,
                                hipStream_t stream) {
  void* params[] = {const_cast<Args*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, 0, stream);
}

hipError_t launch_dense(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                        hipStream_t stream);
hipError_t launch_dense_rows(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                             hipStream_t stream);
hipError_t launch_dense_1x1(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream);
hipError_t launch_grouped16(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream);
hipError_t launch_depthwise(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream);
hipError_t launch_direct(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                         hipStream_t stream);
hipError_t launch_slab_reduce(const Plan& plan, float* ws, float* dw, hipStream_t stream);

}  // namespace cw
