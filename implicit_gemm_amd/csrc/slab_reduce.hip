// Stage 2: deterministic fold of the fp32 partial slabs (gfx950).
//
// The slabs are summed with fp32 round-to-nearest-even adds in one fixed
// order and then stored; no epilogue is applied to partial sums (the
// two-stage split-K of rocm-libraries PR #14393, sections "Two-stage split-K"
// and "Review follow-ups").
//
// A slab holds the weight-gradient partial (E elements) and, from element
// db_offset on, the bias-gradient partial (K elements) when one is requested;
// both ranges are folded the same way.
//
// One fold pass sums, for every output group o, the input slabs
// [o*G, min(n, (o+1)*G)).  The group's slabs are cut into P consecutive parts
// (P = 1 for G <= 16, 4 for G <= 32, else 8); a workgroup owns 256 / P
// element chunks (4 floats each), lane (chunk, part) sums its part left to
// right with its loads in flight, and part sums are then added in ascending
// part order through LDS:
//   out = ((sum(part 0) + sum(part 1)) + sum(part 2)) + ...
// Few slabs thus take one part and 1024 elements per workgroup: a fold of a
// large output over a handful of slabs is not split into tens of thousands
// of workgroups that each read a few lines.  With at most 256 slabs a single
// pass writes dw; with more, a first pass folds runs of 32 slabs into the
// first slab of each run and a second pass folds those run sums.  The order
// depends only on the slab count, so the result is bit-identical from run to
// run.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kLanes = 256;
constexpr int kRun = 32;          // slabs per run in the first of two passes
constexpr int kMaxSinglePass = 256;


struct FoldArgs {
  const float* src;   // input slab 0
  int64_t src_step;   // floats between consecutive input slabs
  int32_t n;          // input slabs
  int32_t group;      // input slabs per output
  int64_t dst_step;   // floats between outputs
  // Two element ranges of a slab are folded: [0, E) into dst (the weight
  // gradient) and, when E2 > 0, [off2, off2 + E2) into dst2 (the bias
  // gradient).  Blocks [0, nb1) take the first range, the rest the second.
  float* dst;
  int64_t E;
  int32_t nb1;
  int64_t off2;
  int64_t E2;
  float* dst2;
};

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return float4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
}

// kParts lanes share one element chunk; kLanes / kParts chunks per workgroup.
template <int kParts>
__global__ __launch_bounds__(kLanes) void slab_fold_kernel(FoldArgs a) {
  constexpr int kChunks = kLanes / kParts;
  constexpr int kBatch = kParts == 4 ? 8 : 16;   // loads issued before their adds
  __shared__ float4 part_sum[kParts][kChunks];
  __shared__ int part_len[kParts];
  const int c = threadIdx.x % kChunks, p = threadIdx.x / kChunks;
  const bool second = (int)blockIdx.x >= a.nb1;
  const int blk = second ? (int)blockIdx.x - a.nb1 : (int)blockIdx.x;
  const int64_t E = second ? a.E2 : a.E;
  const float* const src = a.src + (second ? a.off2 : 0);
  float* const dst = second ? a.dst2 : a.dst;
  const int64_t i = ((int64_t)blk * kChunks + c) * 4;  // first element of the chunk
  const int o = blockIdx.y;
  const int first = o * a.group;
  const int len = min(a.group, a.n - first);
  const int lo = first + (int)((int64_t)p * len / kParts);
  const int hi = first + (int)((int64_t)(p + 1) * len / kParts);
  if (c == 0) part_len[p] = hi - lo;
  const bool full = i + 4 <= E;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  if (i < E && hi > lo) {
    const float* s = src + (int64_t)lo * a.src_step + i;
    const int cnt = hi - lo;
    if (full) {
      // All loads of a batch are issued before its adds (a part is usually
      // shorter than one batch, so its slabs cost one memory latency).
      for (int j0 = 0; j0 < cnt; j0 += kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          v[b] = j0 + b < cnt ? *reinterpret_cast<const float4*>(s + (int64_t)(j0 + b) * a.src_step)
                              : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (j0 + b < cnt) acc = j0 + b == 0 ? v[b] : add4(acc, v[b]);
      }
    } else {
      float t[4] = {0.f, 0.f, 0.f, 0.f};
      for (int e = 0; e < 4 && i + e < E; ++e) {
        t[e] = s[e];
        for (int j = 1; j < cnt; ++j) t[e] += s[(int64_t)j * a.src_step + e];
      }
      acc = float4{t[0], t[1], t[2], t[3]};
    }
  }
  float4 r = acc;
  if constexpr (kParts > 1) {
    part_sum[p][c] = acc;
    __syncthreads();  // every read of this group's slabs is done before the in-place store below
    if (p == 0 && i < E) {
      int q = 0;
      while (part_len[q] == 0) ++q;  // the group has >= 1 slab, so some part is non-empty
      r = part_sum[q][c];
      for (++q; q < kParts; ++q)
        if (part_len[q] > 0) r = add4(r, part_sum[q][c]);
    }
  }
  // One part: the lane's own sum is the result (it has read all its slabs).
  if (p == 0 && i < E) {
    float* d = dst + (int64_t)o * a.dst_step + i;
    if (full) {
      *reinterpret_cast<float4*>(d) = r;  // dw and the slabs are 16-byte aligned
    } else {
      const float rv[4] = {r.x, r.y, r.z, r.w};
      for (int e = 0; e < 4 && i + e < E; ++e) d[e] = rv[e];
    }
  }
}

template <int kParts>
hipError_t fold_p(FoldArgs a, int outputs, hipStream_t stream) {
  const int64_t per_block = 4 * (kLanes / kParts);
  a.nb1 = (int32_t)ceil_div(a.E, per_block);
  const int64_t nb2 = a.E2 > 0 ? ceil_div(a.E2, per_block) : 0;
  const dim3 grid((unsigned)(a.nb1 + nb2), (unsigned)outputs);
  return launch_kernel(slab_fold_kernel<kParts>, grid, dim3(kLanes), a, stream);
}

hipError_t fold(FoldArgs a, int outputs, hipStream_t stream) {
  if (a.group <= 16) return fold_p<1>(a, outputs, stream);
  if (a.group <= 32) return fold_p<4>(a, outputs, stream);
  return fold_p<8>(a, outputs, stream);
}

}  // namespace

hipError_t launch_slab_reduce(const Plan& plan, float* ws, float* dw, float* db, hipStream_t stream) {
  const int64_t E = plan.p.E, stride = plan.pub.slab_stride;
  const int64_t off2 = db_offset(plan.p), E2 = db ? plan.p.K : 0;
  const int32_t ks = plan.pub.ks_count;
  if (ks <= kMaxSinglePass)
    return fold(FoldArgs{ws, stride, ks, ks, 0, dw, E, 0, off2, E2, db}, 1, stream);
  // Pass 1: run r of kRun slabs -> slab r*kRun (each workgroup reads all of
  // its run before writing that run's first slab).
  const int32_t runs = (ks + kRun - 1) / kRun;
  hipError_t err = fold(FoldArgs{ws, stride, ks, kRun, stride * kRun, ws, E, 0, off2, E2, ws + off2},
                        runs, stream);
  if (err != hipSuccess) return err;
  return fold(FoldArgs{ws, stride * kRun, runs, runs, 0, dw, E, 0, off2, E2, db}, 1, stream);
}

}  // namespace cw
