// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cw {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element types of x / dy as stored in memory.
struct Bf16 { uint16_t bits; };
struct F16 { _Float16 v; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(Bf16 v) { return __uint_as_float((uint32_t)v.bits << 16); }
__device__ __forceinline__ float to_f32(F16 v) { return (float)v.v; }

// Load 4 consecutive elements (16 B for fp32, 8 B for 16-bit) from an
// address aligned to 4 elements, widened to fp32.
__device__ __forceinline__ void load4(const float* p, float out[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
__device__ __forceinline__ void load4(const Bf16* p, float out[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(v.x << 16);
  out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16);
  out[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const F16* p, float out[4]) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 v = *reinterpret_cast<const h4*>(p);
  out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
}

// Raw buffer resource over nbytes from base (gfx9: stride 0, default data
// format).  Loads at offsets >= nbytes, or negative offsets (read as large
// unsigned values, so nbytes must stay below 2^31), return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
}

// Buffer load of 4 consecutive elements at byte offset off, widened to fp32.
__device__ __forceinline__ void buf_load4(__amdgpu_buffer_rsrc_t r, int off, const float*, float out[4]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 v = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}
__device__ __forceinline__ void buf_load4(__amdgpu_buffer_rsrc_t r, int off, const Bf16*, float out[4]) {
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  out[0] = __uint_as_float(v[0] << 16);
  out[1] = __uint_as_float(v[0] & 0xffff0000u);
  out[2] = __uint_as_float(v[1] << 16);
  out[3] = __uint_as_float(v[1] & 0xffff0000u);
}
__device__ __forceinline__ void buf_load4(__amdgpu_buffer_rsrc_t r, int off, const F16*, float out[4]) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 v = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
}

// Adds the 8 16-bit values of v (8 consecutive channels as loaded) to d.
template <bool kBf16>
__device__ __forceinline__ void add8(float (&d)[8], uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kBf16) {
      d[2 * i] += __uint_as_float(w[i] << 16);
      d[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
    } else {
      d[2 * i] += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      d[2 * i + 1] += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
}

// Bias-gradient partial of a 64-channel block: thread t holds NV per-thread
// sums d[j] of channel ch0 + j for partial row `row` (ROWS rows, each channel
// covered once per row).  The rows are added in ascending order through
// `scratch` (ROWS * 64 floats of LDS) and out[c] = sum for c < nvalid.  Every
// thread of the workgroup calls it (it has barriers before and after).
template <int ROWS, int NV>
__device__ __forceinline__ void block_sum64(float* scratch, int row, int ch0, const float (&d)[NV],
                                            float* out, int nvalid) {
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NV; ++j) scratch[row * 64 + ch0 + j] = d[j];
  __syncthreads();
  const int c = (int)threadIdx.x;
  if (c < 64 && c < nvalid) {
    float r = scratch[c];
    for (int i = 1; i < ROWS; ++i) r += scratch[i * 64 + c];
    out[c] = r;
  }
  __syncthreads();
}

// Workgroup barrier that waits for this wave's LDS accesses only (not for
// its outstanding global loads); the memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace cw
