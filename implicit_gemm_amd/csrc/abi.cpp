// C ABI: validation, plan cache and launch sequencing.
//
// conv_wgrad validates synchronously, looks the plan up (or builds it), then
// enqueues stage 1 and, when the plan has more than one slice, the slab
// reduce, on the caller's stream, and returns without synchronising.  The
// plan (and everything packed from it) is built once per descriptor, outside
// any timed loop (the launch-binding lesson of rocm-libraries PR #14393,
// section Benchmark).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <string>
#include <unordered_map>

#include "../../include/conv_wgrad.h"
#include "kernels.h"

#include <hip/hip_ext.h>
#include "plan.h"

namespace cw {

Stage1Events& stage1_events() {
  static thread_local Stage1Events ev;
  return ev;
}

hipError_t launch_raw(const void* fn, dim3 grid, dim3 block, void** params, size_t shmem,
                      hipStream_t stream) {
  Stage1Events& ev = stage1_events();
  if (ev.end_on_last) {
    const hipEvent_t b = ev.begin;
    const hipEvent_t e = --ev.launches_left == 0 ? ev.end : nullptr;
    ev.begin = nullptr;
    if (ev.launches_left <= 0) ev = Stage1Events{};
    if (b || e) return hipExtLaunchKernel(fn, grid, block, params, shmem, stream, b, e, 0);
    return hipLaunchKernel(fn, grid, block, params, shmem, stream);
  }
  if (ev.begin || ev.end) {
    const Stage1Events use = ev;
    ev = Stage1Events{};
    return hipExtLaunchKernel(fn, grid, block, params, shmem, stream, use.begin, use.end, 0);
  }
  return hipLaunchKernel(fn, grid, block, params, shmem, stream);
}

}  // namespace cw

namespace {

std::mutex g_mutex;
std::unordered_map<std::string, cw::Plan>* g_plans = nullptr;

conv_wgrad_status_t get_plan(const conv_wgrad_desc2_t* desc, cw::Plan* out,
                             int32_t direction = CONV_DIRECTION_WGRAD) {
  if (!desc) return CONV_WGRAD_ERR_NULL_ARG;
  std::string key(reinterpret_cast<const char*>(desc), sizeof(*desc));
  key.push_back(static_cast<char>(direction));
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_plans) {
      auto it = g_plans->find(key);
      if (it != g_plans->end()) {
        *out = it->second;
        return CONV_WGRAD_OK;
      }
    }
  }
  conv_wgrad_status_t st = direction == CONV_DIRECTION_WGRAD ? cw::make_plan(desc, out)
                                                             : cw::make_igemm_plan(desc, direction, out);
  if (st != CONV_WGRAD_OK) return st;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_plans) g_plans = new std::unordered_map<std::string, cw::Plan>();
  if (g_plans->size() > 4096) g_plans->clear();  // bound the cache; plans are cheap to rebuild
  (*g_plans)[key] = *out;
  return CONV_WGRAD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The plain descriptor as an extended one (NULL stays NULL).
struct Desc2 {
  conv_wgrad_desc2_t d;
  const conv_wgrad_desc2_t* ptr;
  explicit Desc2(const conv_wgrad_desc_t* p) : ptr(nullptr) {
    if (p) {
      d = cw::to_desc2(*p);
      ptr = &d;
    }
  }
};

// Launches of one call: stage 1, then one fold pass (two beyond 256 slabs).
int launches_of(const cw::Plan& plan) {
  return 1 + (plan.pub.needs_reduce ? (plan.pub.ks_count > 256 ? 2 : 1) : 0);
}

// Timing events for the launches of one call: the stage-1 launch takes them
// (timestamps of its own dispatch), or with `whole` the first launch takes the
// begin event and the last the end event.  The destructor clears them again
// whatever happens, so no later launch records them.
struct EventsGuard {
  EventsGuard(void* b, void* e, bool whole, int launches) {
    cw::Stage1Events& ev = cw::stage1_events();
    ev.begin = static_cast<hipEvent_t>(b);
    ev.end = static_cast<hipEvent_t>(e);
    ev.end_on_last = whole && (b || e);
    ev.launches_left = launches;
  }
  ~EventsGuard() { cw::stage1_events() = cw::Stage1Events{}; }
};

// with_db: the bias gradient is requested (db must then be a valid pointer).
conv_wgrad_status_t run(const conv_wgrad_desc2_t* desc, const void* x, const void* dy, float* dw,
                        bool with_db, float* db, void* workspace, bool check_ws, size_t ws_bytes,
                        void* stream, void* ev_begin = nullptr, void* ev_end = nullptr,
                        bool whole_call = false) {
  cw::Plan plan;
  conv_wgrad_status_t st = get_plan(desc, &plan);
  if (st != CONV_WGRAD_OK) return st;
  if (!x || !dy || !dw || (with_db && !db)) return CONV_WGRAD_ERR_NULL_ARG;
  if (plan.pub.ws_bytes > 0 && !workspace) return CONV_WGRAD_ERR_NULL_ARG;
  if (check_ws && ws_bytes < plan.pub.ws_bytes) return CONV_WGRAD_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dw) || (with_db && !aligned16(db)) ||
      (plan.pub.ws_bytes > 0 && !aligned16(workspace)))
    return CONV_WGRAD_ERR_MISALIGNED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  cw::Stage1Out out;
  if (plan.pub.needs_reduce) {
    out.base = static_cast<float*>(workspace);
    out.slab_stride = plan.pub.slab_stride;
    out.db = with_db ? out.base + cw::db_offset(plan.p) : nullptr;
  } else {
    out.base = dw;
    out.slab_stride = 0;
    out.db = with_db ? db : nullptr;
  }
  hipError_t err;
  EventsGuard guard(ev_begin, ev_end, whole_call, launches_of(plan));
  switch (plan.pub.variant) {
    case cw::kDirectElem: err = cw::launch_direct(plan, x, dy, out, s); break;
    case cw::kGrouped16:
    case cw::kGrouped16Rows: err = cw::launch_grouped16(plan, x, dy, out, s); break;
    case cw::kDepthwise: err = cw::launch_depthwise(plan, x, dy, out, s); break;
    case cw::kDenseRows: err = cw::launch_dense_rows(plan, x, dy, out, s); break;
    case cw::kDense1x1: err = cw::launch_dense_1x1(plan, x, dy, out, s); break;
    case cw::kDense16Rows:
    case cw::kDense16RowsX3: err = cw::launch_dense16_rows(plan, x, dy, out, s); break;
    case cw::kDense16Taps:
    case cw::kDense16TapsX3: err = cw::launch_dense16_taps(plan, x, dy, out, s); break;
    default: err = cw::launch_dense(plan, x, dy, out, s); break;
  }
  if (err != hipSuccess) return CONV_WGRAD_ERR_HIP;
  if (plan.pub.needs_reduce) {
    err = cw::launch_slab_reduce(plan, static_cast<float*>(workspace), dw, with_db ? db : nullptr, s);
    if (err != hipSuccess) return CONV_WGRAD_ERR_HIP;
  }
  return CONV_WGRAD_OK;
}

// Forward / data gradient: validate, stage 1 (the implicit GEMM) and, with
// several slices, the slab fold into the output, on the caller's stream.
conv_wgrad_status_t run_igemm(const conv_wgrad_desc2_t* desc, int32_t direction, const void* a_src,
                              const void* w, float* out, void* workspace, size_t ws_bytes, void* stream,
                              void* ev_begin = nullptr, void* ev_end = nullptr) {
  cw::Plan plan;
  conv_wgrad_status_t st = get_plan(desc, &plan, direction);
  if (st != CONV_WGRAD_OK) return st;
  if (!a_src || !w || !out) return CONV_WGRAD_ERR_NULL_ARG;
  if (plan.pub.ws_bytes > 0 && !workspace) return CONV_WGRAD_ERR_NULL_ARG;
  if (ws_bytes < plan.pub.ws_bytes) return CONV_WGRAD_ERR_WORKSPACE;
  if (!aligned16(a_src) || !aligned16(w) || !aligned16(out) ||
      (plan.pub.ws_bytes > 0 && !aligned16(workspace)))
    return CONV_WGRAD_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  cw::Stage1Out o;
  if (plan.pub.needs_reduce) {
    o.base = static_cast<float*>(workspace);
    o.slab_stride = plan.pub.slab_stride;
  } else {
    o.base = out;
    o.slab_stride = 0;
  }
  EventsGuard guard(ev_begin, ev_end, true, launches_of(plan));
  if (cw::launch_igemm(plan, a_src, w, o, s) != hipSuccess) return CONV_WGRAD_ERR_HIP;
  if (plan.pub.needs_reduce &&
      cw::launch_slab_reduce(plan, static_cast<float*>(workspace), out, nullptr, s) != hipSuccess)
    return CONV_WGRAD_ERR_HIP;
  return CONV_WGRAD_OK;
}

}  // namespace

extern "C" {

const char* conv_wgrad_status_string(conv_wgrad_status_t status) {
  switch (status) {
    case CONV_WGRAD_OK: return "ok";
    case CONV_WGRAD_ERR_NULL_ARG: return "null argument";
    case CONV_WGRAD_ERR_BAD_SHAPE: return "invalid shape";
    case CONV_WGRAD_ERR_BAD_DTYPE: return "invalid dtype";
    case CONV_WGRAD_ERR_BAD_SPLIT: return "invalid split_k (must be -1 or >= 1)";
    case CONV_WGRAD_ERR_UNSUPPORTED: return "unsupported problem (outside documented limits)";
    case CONV_WGRAD_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case CONV_WGRAD_ERR_WORKSPACE: return "workspace too small";
    case CONV_WGRAD_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

conv_wgrad_status_t conv_wgrad_get_plan(const conv_wgrad_desc_t* desc, conv_wgrad_plan_t* plan) {
  if (!desc || !plan) return CONV_WGRAD_ERR_NULL_ARG;
  cw::Plan p;
  conv_wgrad_status_t st = get_plan(Desc2(desc).ptr, &p);
  if (st != CONV_WGRAD_OK) return st;
  *plan = p.pub;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t conv_wgrad_workspace_size(const conv_wgrad_desc_t* desc, size_t* bytes) {
  if (!desc || !bytes) return CONV_WGRAD_ERR_NULL_ARG;
  cw::Plan p;
  conv_wgrad_status_t st = get_plan(Desc2(desc).ptr, &p);
  if (st != CONV_WGRAD_OK) return st;
  *bytes = (size_t)p.pub.ws_bytes;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t conv_wgrad(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                               float* dw, void* workspace, void* stream) {
  return run(Desc2(desc).ptr, x, dy, dw, false, nullptr, workspace, false, 0, stream);
}

conv_wgrad_status_t conv_wgrad_ex(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                  float* dw, void* workspace, size_t ws_bytes, void* stream) {
  return run(Desc2(desc).ptr, x, dy, dw, false, nullptr, workspace, true, ws_bytes, stream);
}

conv_wgrad_status_t conv_wgrad_timed(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                     float* dw, void* workspace, size_t ws_bytes, void* stream,
                                     void* stage1_begin, void* stage1_end) {
  return run(Desc2(desc).ptr, x, dy, dw, false, nullptr, workspace, true, ws_bytes, stream, stage1_begin,
             stage1_end);
}

conv_wgrad_status_t conv_wgrad_bias(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                    float* dw, float* db, void* workspace, size_t ws_bytes,
                                    void* stream) {
  return run(Desc2(desc).ptr, x, dy, dw, true, db, workspace, true, ws_bytes, stream);
}

conv_wgrad_status_t conv_wgrad_bias_timed(const conv_wgrad_desc_t* desc, const void* x,
                                          const void* dy, float* dw, float* db, void* workspace,
                                          size_t ws_bytes, void* stream, void* stage1_begin,
                                          void* stage1_end) {
  return run(Desc2(desc).ptr, x, dy, dw, true, db, workspace, true, ws_bytes, stream, stage1_begin,
             stage1_end);
}

conv_wgrad_status_t conv_wgrad_noalloc(const conv_wgrad_desc_t* desc, const void* x, const void* dy,
                                       float* dw, float* db, void* stream) {
  cw::Plan plan;
  const Desc2 d2(desc);
  conv_wgrad_status_t st = get_plan(d2.ptr, &plan);
  if (st != CONV_WGRAD_OK) return st;
  if (!x || !dy || !dw) return CONV_WGRAD_ERR_NULL_ARG;
  if (plan.pub.ws_bytes > cw::kNoallocScratchBytes) return CONV_WGRAD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.pub.ws_bytes > 0 && cw::noalloc_scratch(&ws) != hipSuccess) return CONV_WGRAD_ERR_HIP;
  return run(d2.ptr, x, dy, dw, db != nullptr, db, ws, true, cw::kNoallocScratchBytes, stream);
}

conv_wgrad_status_t conv_wgrad2_workspace_size(const conv_wgrad_desc2_t* desc, size_t* bytes) {
  if (!desc || !bytes) return CONV_WGRAD_ERR_NULL_ARG;
  cw::Plan p;
  conv_wgrad_status_t st = get_plan(desc, &p);
  if (st != CONV_WGRAD_OK) return st;
  *bytes = (size_t)p.pub.ws_bytes;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t conv_wgrad2_get_plan(const conv_wgrad_desc2_t* desc, conv_wgrad_plan2_t* plan) {
  if (!desc || !plan) return CONV_WGRAD_ERR_NULL_ARG;
  cw::Plan p;
  conv_wgrad_status_t st = get_plan(desc, &p);
  if (st != CONV_WGRAD_OK) return st;
  plan->base = p.pub;
  plan->math = p.pub.variant == CONV_WGRAD_VARIANT_DENSE_BF16X3 || p.pub.variant == CONV_WGRAD_VARIANT_DENSE_BF16X3_TAPS
                   ? CONV_WGRAD_MATH_BF16X3
                   : CONV_WGRAD_MATH_EXACT;
  plan->fold_width = p.p.fold;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t conv_wgrad2(const conv_wgrad_desc2_t* desc, const void* x, const void* dy,
                                float* dw, float* db, void* workspace, size_t ws_bytes, void* stream) {
  return run(desc, x, dy, dw, db != nullptr, db, workspace, true, ws_bytes, stream);
}

conv_wgrad_status_t conv_wgrad2_timed(const conv_wgrad_desc2_t* desc, const void* x, const void* dy,
                                      float* dw, float* db, void* workspace, size_t ws_bytes,
                                      void* stream, void* stage1_begin, void* stage1_end) {
  return run(desc, x, dy, dw, db != nullptr, db, workspace, true, ws_bytes, stream, stage1_begin,
             stage1_end);
}

conv_wgrad_status_t conv_wgrad2_call_timed(const conv_wgrad_desc2_t* desc, const void* x, const void* dy,
                                           float* dw, float* db, void* workspace, size_t ws_bytes,
                                           void* stream, void* call_begin, void* call_end) {
  return run(desc, x, dy, dw, db != nullptr, db, workspace, true, ws_bytes, stream, call_begin, call_end,
             true);
}

conv_wgrad_status_t conv_igemm_get_plan(const conv_wgrad_desc2_t* desc, int32_t direction,
                                        conv_wgrad_plan2_t* plan) {
  if (!desc || !plan) return CONV_WGRAD_ERR_NULL_ARG;
  if (direction == CONV_DIRECTION_WGRAD) return conv_wgrad2_get_plan(desc, plan);
  cw::Plan p;
  conv_wgrad_status_t st = get_plan(desc, &p, direction);
  if (st != CONV_WGRAD_OK) return st;
  plan->base = p.pub;
  plan->math = CONV_WGRAD_MATH_EXACT;
  plan->fold_width = p.p.fold;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t conv_igemm_workspace_size(const conv_wgrad_desc2_t* desc, int32_t direction,
                                              size_t* bytes) {
  if (!desc || !bytes) return CONV_WGRAD_ERR_NULL_ARG;
  if (direction == CONV_DIRECTION_WGRAD) return conv_wgrad2_workspace_size(desc, bytes);
  cw::Plan p;
  conv_wgrad_status_t st = get_plan(desc, &p, direction);
  if (st != CONV_WGRAD_OK) return st;
  *bytes = (size_t)p.pub.ws_bytes;
  return CONV_WGRAD_OK;
}

conv_wgrad_status_t conv_fwd(const conv_wgrad_desc2_t* desc, const void* x, const void* w, float* y,
                             void* workspace, size_t ws_bytes, void* stream) {
  return run_igemm(desc, CONV_DIRECTION_FWD, x, w, y, workspace, ws_bytes, stream);
}

conv_wgrad_status_t conv_dgrad(const conv_wgrad_desc2_t* desc, const void* dy, const void* w, float* dx,
                               void* workspace, size_t ws_bytes, void* stream) {
  return run_igemm(desc, CONV_DIRECTION_DGRAD, dy, w, dx, workspace, ws_bytes, stream);
}

conv_wgrad_status_t conv_igemm_call_timed(const conv_wgrad_desc2_t* desc, int32_t direction,
                                          const void* src, const void* w, float* out, void* workspace,
                                          size_t ws_bytes, void* stream, void* call_begin,
                                          void* call_end) {
  if (direction != CONV_DIRECTION_FWD && direction != CONV_DIRECTION_DGRAD) return CONV_WGRAD_ERR_BAD_DTYPE;
  return run_igemm(desc, direction, src, w, out, workspace, ws_bytes, stream, call_begin, call_end);
}

}  // extern "C"
