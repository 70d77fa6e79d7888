// Achievable-peak probes (gfx950): a streaming read of a device buffer, loops
// of independent MFMA chains and loops of LDS reads.  They measure what the
// chip sustains on the resources the weight-gradient kernels are priced
// against (HBM bandwidth, dense MFMA rate) or bound by (LDS operand reads);
// they compute nothing of the gradient.
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

// iters rounds of 8 independent chains of v_mfma_f32_16x16x32_bf16 (the form
// the 16-bit kernels use), as peak_mfma_kernel.
__global__ __launch_bounds__(256) void peak_mfma16_kernel(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0e-3f * (float)(1 + (lane & 15)));
    b[e] = (__bf16)(1.0e-3f * (float)(1 + (lane >> 4)));
  }
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{(float)c, (float)lane, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// LDS reads of 256-lane workgroups (32 KB of LDS each): iters rounds of 8
// reads per lane at the addressing of the 16-bit kernels' operand reads (16
// pixel rows of 64 channels at a 160-byte pitch), folded into registers.
// kMode 0: ds_read_b64_tr_b16 (the transposed 8-byte read), 1: ds_read_b64,
// 2: ds_read_b128.  Every address lies inside the 32 KB array.
template <int kMode>
__global__ __launch_bounds__(256) void peak_lds_kernel(int64_t iters, uint32_t* __restrict__ sink) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  __shared__ __attribute__((aligned(16))) unsigned short s[16384];
  for (int i = threadIdx.x; i < 16384; i += 256) s[i] = (unsigned short)(i * 7);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, gq = lane >> 4;
  const int off = (8 * gq + (j >> 2)) * 80 + 4 * (j & 3) + 16 * wave;   // < 2300
  uint32_t x0 = 0, x1 = 0, x2 = 0, x3 = 0;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int o = off + (int)((it * 8 + k) & 31) * 80;   // < 2300 + 31 * 80 + 8 < 16384
      if constexpr (kMode == 0) {
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(s + o));
        x0 ^= (uint32_t)v[0]; x1 ^= (uint32_t)v[1]; x2 ^= (uint32_t)v[2]; x3 ^= (uint32_t)v[3];
      } else if constexpr (kMode == 1) {
        const uint2 v = *reinterpret_cast<const uint2*>(s + o);
        x0 ^= v.x; x1 ^= v.y;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(s + (o & ~7));
        x0 ^= v.x; x1 ^= v.y; x2 ^= v.z; x3 ^= v.w;
      }
    }
  }
  if ((x0 ^ x1 ^ x2 ^ x3) == kNever) sink[blockIdx.x] = threadIdx.x;
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

extern "C" conv_wgrad_status_t cwprobe_mfma16(int64_t iters, int32_t blocks, float* sink, void* stream, void* begin,
                                              void* end) {
  if (!sink) return CONV_WGRAD_ERR_NULL_ARG;
  if (iters < 1 || iters > INT32_MAX || blocks < 1 || blocks > 65536) return CONV_WGRAD_ERR_BAD_SHAPE;
  void* params[] = {&iters, &sink};
  return cw::launch(reinterpret_cast<const void*>(cw::peak_mfma16_kernel), blocks, params, stream, begin, end);
}

extern "C" conv_wgrad_status_t cwprobe_lds(int32_t mode, int64_t iters, int32_t blocks, uint32_t* sink,
                                           void* stream, void* begin, void* end) {
  if (!sink) return CONV_WGRAD_ERR_NULL_ARG;
  if (mode < 0 || mode > 2 || iters < 1 || iters > INT32_MAX || blocks < 1 || blocks > 65536)
    return CONV_WGRAD_ERR_BAD_SHAPE;
  void* params[] = {&iters, &sink};
  const void* fn = mode == 0   ? reinterpret_cast<const void*>(cw::peak_lds_kernel<0>)
                   : mode == 1 ? reinterpret_cast<const void*>(cw::peak_lds_kernel<1>)
                               : reinterpret_cast<const void*>(cw::peak_lds_kernel<2>);
  return cw::launch(fn, blocks, params, stream, begin, end);
}
