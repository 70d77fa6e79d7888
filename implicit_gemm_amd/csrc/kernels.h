// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace cw {

// Stage-1 output: dw itself (one slice) or the fp32 slab workspace.  When the
// bias gradient is requested, db points at slice 0's bias partial (db itself
// for one slice, else the slab's bias range) and the workgroups that own an
// output-channel block of a slice write its sum of dY there; slices are
// slab_stride floats apart as for the weight gradient.
struct Stage1Out {
  float* base;           // dw or workspace
  int64_t slab_stride;   // floats between slabs (0 when writing dw)
  float* db = nullptr;   // bias-gradient partial of slice 0, or nullptr
};

// Events the launches of one call on this thread record in (the dispatches'
// own timestamps, not the stream position around them); set by the timed
// entry points, consumed by launch_raw.  Stage-1 timing: begin and end on the
// first launch.  Call timing (end_on_last): begin at the start of the first
// launch, end at the end of the launch that leaves launches_left at zero.
struct Stage1Events {
  hipEvent_t begin = nullptr, end = nullptr;
  bool end_on_last = false;
  int launches_left = 0;
};
Stage1Events& stage1_events();

// Launch one kernel; with pending stage-1 events, hipExtLaunchKernel records
// them at the kernel's start and end.  Returns the status of this launch only.
hipError_t launch_raw(const void* fn, dim3 grid, dim3 block, void** params, size_t shmem,
                      hipStream_t stream);

// Launch `kernel(args)`; returns the status of this launch only.
template <typename Args>
inline hipError_t launch_kernel(void (*kernel)(Args), dim3 grid, dim3 block, const Args& args,
                                hipStream_t stream) {
  void* params[] = {const_cast<Args*>(&args)};
  return launch_raw(reinterpret_cast<const void*>(kernel), grid, block, params, 0, stream);
}

hipError_t launch_dense(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                        hipStream_t stream);
hipError_t launch_dense_rows(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                             hipStream_t stream);
hipError_t launch_dense16_rows(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                               hipStream_t stream);
hipError_t launch_dense16_taps(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                               hipStream_t stream);
hipError_t launch_dense_1x1(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream);
hipError_t launch_grouped16(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream);
hipError_t launch_depthwise(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream);
hipError_t launch_direct(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                         hipStream_t stream);
// Forward or data-gradient implicit GEMM (plan variant kFwdIgemm / kDgradIgemm):
// a_src is x (forward) or dy (dgrad), w the filter; out.base the output or slab 0.
hipError_t launch_igemm(const Plan& plan, const void* a_src, const void* w, Stage1Out out, hipStream_t stream);

// Library-owned workspace of conv_wgrad_noalloc: the device address of this
// process's copy on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = CONV_WGRAD_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// Folds the slabs into dw and, when db is not null, into db.
hipError_t launch_slab_reduce(const Plan& plan, float* ws, float* dw, float* db, hipStream_t stream);

}  // namespace cw
