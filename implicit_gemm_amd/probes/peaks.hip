// Achievable-peak probes (gfx950): a streaming read of a device buffer and a
// loop of independent MFMA chains.  They measure what the chip sustains on
// the two resources the weight-gradient kernels are priced against (HBM
// bandwidth, dense MFMA rate); they compute nothing of the gradient.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "probes.h"
#include "../csrc/device_common.h"

namespace cw {

namespace {

constexpr uint32_t kNever = 0x9e3779b9u;   // folded value that triggers the sink store

__device__ __forceinline__ uint32_t fold16(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Grid-stride read of n16 16-byte words; four loads per lane in flight.  The
// XOR of every word a lane read decides a store, so all loads stay live.
__global__ __launch_bounds__(256) void peak_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  const int64_t step = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * step < n16; i += 4 * step) {
    const uint4 a = src[i], b = src[i + step], c = src[i + 2 * step], d = src[i + 3 * step];
    x ^= fold16(a) ^ fold16(b) ^ fold16(c) ^ fold16(d);
  }
  for (; i < n16; i += step) x ^= fold16(src[i]);
  if (x == kNever) sink[blockIdx.x] = threadIdx.x;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// iters rounds of independent MFMA chains on register operands (f32: 8
// chains of v_mfma_f32_16x16x4_f32; 16-bit: 4 chains of the 32x32x16 form),
// then each lane stores the sum of its
// accumulators.  Each chain starts from its own value (chains that start
// equal share one register and cost a copy per round), and the operands are
// small, so the sums stay finite for any iteration count used for timing.
template <int kType>   // 0: f32, 1: bf16, 2: f16
__global__ __launch_bounds__(256) void peak_mfma_kernel(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const float va = 1.0e-3f * (float)(1 + (lane & 15)), vb = 1.0e-3f * (float)(1 + (lane >> 4));
  float s = 0.f;
  if constexpr (kType == 0) {
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{(float)c, (float)lane, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, vb, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    typedef typename std::conditional<kType == 1, bf16x8, f16x8>::type V;
    typedef typename std::conditional<kType == 1, __bf16, _Float16>::type E;
    V a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (E)va;
      b[e] = (E)vb;
    }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] = (float)(16 * c + v);
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (kType == 1)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[c][v];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

conv_wgrad_status_t launch(const void* fn, int32_t blocks, void** params, void* stream, void* begin,
                           void* end) {
  const hipError_t e = hipExtLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), params, 0,
                                          static_cast<hipStream_t>(stream),
                                          static_cast<hipEvent_t>(begin), static_cast<hipEvent_t>(end), 0);
  return e == hipSuccess ? CONV_WGRAD_OK : CONV_WGRAD_ERR_HIP;
}

}  // namespace

}  // namespace cw

extern "C" conv_wgrad_status_t cwprobe_read(const void* src, int64_t nbytes, int32_t blocks,
                                                    uint32_t* sink, void* stream, void* begin, void* end) {
  if (!src || !sink) return CONV_WGRAD_ERR_NULL_ARG;
  if (nbytes <= 0 || nbytes % 16 != 0 || blocks < 1 || blocks > 65536) return CONV_WGRAD_ERR_BAD_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return CONV_WGRAD_ERR_MISALIGNED;
  const uint4* s = static_cast<const uint4*>(src);
  int64_t n16 = nbytes / 16;
  void* params[] = {&s, &n16, &sink};
  return cw::launch(reinterpret_cast<const void*>(cw::peak_read_kernel), blocks, params, stream, begin, end);
}

extern "C" conv_wgrad_status_t cwprobe_mfma(int32_t dtype, int64_t iters, int32_t blocks, float* sink,
                                                    void* stream, void* begin, void* end) {
  if (!sink) return CONV_WGRAD_ERR_NULL_ARG;
  if (dtype != CONV_WGRAD_F32 && dtype != CONV_WGRAD_BF16 && dtype != CONV_WGRAD_F16)
    return CONV_WGRAD_ERR_BAD_DTYPE;
  if (iters < 1 || iters > INT32_MAX || blocks < 1 || blocks > 65536) return CONV_WGRAD_ERR_BAD_SHAPE;
  void* params[] = {&iters, &sink};
  const void* fn = dtype == CONV_WGRAD_F32    ? reinterpret_cast<const void*>(cw::peak_mfma_kernel<0>)
                   : dtype == CONV_WGRAD_BF16 ? reinterpret_cast<const void*>(cw::peak_mfma_kernel<1>)
                                              : reinterpret_cast<const void*>(cw::peak_mfma_kernel<2>);
  return cw::launch(fn, blocks, params, stream, begin, end);
}
