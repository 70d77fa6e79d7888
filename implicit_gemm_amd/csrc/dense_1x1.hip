// 1x1, stride-1, unpadded dense weight gradient: dW_g = dY_g^T X_g streamed
// from HBM straight into MFMA operand registers (gfx950, fp32).
//
// For a 1x1 filter the weight gradient is the product of the reshaped
// [N*H*W, K] and [N*H*W, C] matrices (the "F.linear on the reshaped tensor"
// equivalence of rocm-libraries PR #11188, section Motivation), a GEMM with a
// tiny output and a reduction of N*H*W rows: HBM-bound with an arithmetic
// intensity at the f32-MFMA ridge, so no LDS staging is used at all.
//
// One wave owns one slice of rows.  Lane (i, g) = (lane % 16, lane / 16)
// loads, for row 4*b + g of batch b, the AV consecutive output channels
// m0 + AV*i .. of dY and the BV consecutive input channels c0 + BV*i .. of X:
// 16 lanes read one whole row (256 B of dY, 384 B of X for K=64, C=96) and
// the 4 lane groups read 4 consecutive rows.  Register j of the dY load is the
// A operand of v_mfma_f32_16x16x4_f32 for output channels {m0 + AV*i + j},
// register j' of the X load the B operand for input channels
// {c0 + BV*i + j'}, so AV*BV MFMAs per 4 rows cover the whole M x N tile with
// no data movement between load and MFMA.  Loads run PF batches ahead.
// Row offsets are 64-bit (tensors may span many 4 GiB windows).
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kPf = 8;  // row batches in flight per wave

struct OneByOneArgs {
  const float* x;
  const float* dy;
  float* out;
  int64_t slab_stride;
  int32_t C, K, Cg, Kg, groups;
  int32_t m_tiles, c_tiles;
  int64_t L;            // rows
  int64_t rows_per_slice;
  int32_t ks_count;
  float* dbo;   // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
};

// One 4-row batch: lane (i, g) loads row g of the batch, AV channels of dY at
// byte offset ody and BV channels of X at byte offset ox, from buffer
// resources whose ranges end at the slice's last row (rows past it read 0).
template <int AV, int BV>
__device__ __forceinline__ void load_batch(__amdgpu_buffer_rsrc_t rdy, int ody, __amdgpu_buffer_rsrc_t rx, int ox,
                                           float (&a)[AV], float (&b)[BV]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  static_assert(AV == 4, "four output channels per lane");
  const f4 va = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rdy, ody, 0, 0));
  a[0] = va[0]; a[1] = va[1]; a[2] = va[2]; a[3] = va[3];
  int j = 0;
#pragma unroll
  for (; j + 4 <= BV; j += 4) {
    const f4 v = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rx, ox + 4 * j, 0, 0));
    b[j] = v[0]; b[j + 1] = v[1]; b[j + 2] = v[2]; b[j + 3] = v[3];
  }
  if constexpr (BV % 4 >= 2) {
    const f2 v = __builtin_bit_cast(f2, __builtin_amdgcn_raw_buffer_load_b64(rx, ox + 4 * j, 0, 0));
    b[j] = v[0]; b[j + 1] = v[1];
    j += 2;
  }
  if constexpr (BV % 2 == 1)
    b[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, ox + 4 * j, 0, 0));
}

// kDb: the bias-gradient variant (a separate instantiation keeps the extra
// registers and code out of the plain kernel's load pipeline).
template <int AV, int BV, bool kDb>
__global__ __launch_bounds__(64) void dense_1x1_kernel(OneByOneArgs a) {
  const int lane = threadIdx.x;
  const int li = lane & 15, lg = lane >> 4;
  const int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  int tile = bid / a.ks_count;
  const int ct = tile % a.c_tiles;
  tile /= a.c_tiles;
  const int mt = tile % a.m_tiles;
  const int g = tile / a.m_tiles;
  const int m0 = mt * 16 * AV, c0 = ct * 16 * BV;

  const int64_t r_begin = (int64_t)slice * a.rows_per_slice;
  const int64_t r_end = min(a.L, r_begin + a.rows_per_slice);
  // 4-row batches, rounded up to whole rings so that the loop body has no
  // branches (the load counters stay exact and the ring never drains); the
  // extra batches read zeros.
  const int64_t nb = (r_end - r_begin + 4 * kPf - 1) / (4 * kPf) * kPf;

  // Batch t reads rows r_begin + 4t .. + 3 from uniform 64-bit bases; the
  // buffer range of a batch ends at the slice's last row.
  const int cdy = g * a.Kg + m0, cx = g * a.Cg + c0;          // first channel of the tile
  const unsigned char* const dy0 = reinterpret_cast<const unsigned char*>(a.dy + r_begin * a.K + cdy);
  const unsigned char* const x0 = reinterpret_cast<const unsigned char*>(a.x + r_begin * a.C + cx);
  const int ody = (lg * a.K + AV * li) * 4, ox = (lg * a.C + BV * li) * 4;
  auto load = [&](int64_t t, float (&ra)[AV], float (&rb)[BV]) {
    const int64_t left = r_end - r_begin - 4 * t;              // rows of the slice from this batch on
    const int rows = left < 0 ? 0 : left > 4 ? 4 : (int)left;
    const __amdgpu_buffer_rsrc_t rdy =
        buf_rsrc(dy0 + 16 * t * a.K, rows > 0 ? (rows * a.K - cdy) * 4 : 0);
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x0 + 16 * t * a.C, rows > 0 ? (rows * a.C - cx) * 4 : 0);
    load_batch<AV, BV>(rdy, ody, rx, ox, ra, rb);
  };

  f32x4 acc[AV][BV];
#pragma unroll
  for (int i = 0; i < AV; ++i)
#pragma unroll
    for (int j = 0; j < BV; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Bias gradient: the first input-channel tile of each (group, output-channel
  // tile) adds up the dY values it feeds to the MFMAs (rows past the slice
  // load as zero); lane (i, g) sums rows = g mod 4 for channels m0 + AV*i ...
  const bool want_db = kDb && ct == 0;
  float dbp[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) dbp[i] = 0.f;

  // The prologue issues the ring in the order the loop consumes it (pinned by
  // scheduling barriers), so the wait at the loop head is for one batch only.
  float ra[kPf][AV], rb[kPf][BV];
#pragma unroll
  for (int p = 0; p < kPf; ++p) {
    load(p, ra[p], rb[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t b = 0; b < nb; b += kPf) {
#pragma unroll
    for (int p = 0; p < kPf; ++p) {
#pragma unroll
      for (int i = 0; i < AV; ++i)
#pragma unroll
        for (int j = 0; j < BV; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[p][i], rb[p][j], acc[i][j], 0, 0, 0);
      if constexpr (kDb) {
#pragma unroll
        for (int i = 0; i < AV; ++i) dbp[i] += ra[p][i];
      }
      load(b + p + kPf, ra[p], rb[p]);
    }
  }

  if (want_db) {
    // Lanes i, i + 16, i + 32, i + 48 hold the same channels: a fixed pairwise tree.
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      float v = dbp[i];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      dbp[i] = v;
    }
    if (lg == 0) {
      float* o = a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0 + AV * li;
#pragma unroll
      for (int i = 0; i < AV; ++i) o[i] = dbp[i];
    }
  }

  // acc[i][j][v] is dW[m0 + AV*(4*lg + v) + i][c0 + BV*li + j].
  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int64_t cols = a.Cg;
#pragma unroll
  for (int i = 0; i < AV; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + AV * (4 * lg + v) + i;
      float* o = out + ((int64_t)g * a.Kg + m) * cols + c0 + BV * li;
#pragma unroll
      for (int j = 0; j < BV; ++j) o[j] = acc[i][j][v];
    }
}

template <int AV, int BV>
hipError_t launch_ab(const OneByOneArgs& args, int64_t grid, hipStream_t stream) {
  if (args.dbo)
    return launch_kernel(dense_1x1_kernel<AV, BV, true>, dim3((unsigned)grid), dim3(64), args, stream);
  return launch_kernel(dense_1x1_kernel<AV, BV, false>, dim3((unsigned)grid), dim3(64), args, stream);
}

}  // namespace

hipError_t launch_dense_1x1(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream) {
  const Problem& p = plan.p;
  OneByOneArgs a;
  a.x = static_cast<const float*>(x);
  a.dy = static_cast<const float*>(dy);
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.C = (int32_t)p.C; a.K = (int32_t)p.K; a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg;
  a.groups = (int32_t)p.groups;
  a.m_tiles = (int32_t)plan.m_tiles;
  a.c_tiles = (int32_t)plan.c_tiles;
  a.L = p.L;
  a.rows_per_slice = plan.pub.units_per_slice * plan.pub.unit_rows;
  a.ks_count = plan.pub.ks_count;
  a.dbo = out.db;
  const int64_t grid = plan.pub.grid;
  switch (plan.bv) {
    case 1: return launch_ab<4, 1>(a, grid, stream);
    case 2: return launch_ab<4, 2>(a, grid, stream);
    case 3: return launch_ab<4, 3>(a, grid, stream);
    case 4: return launch_ab<4, 4>(a, grid, stream);
    case 5: return launch_ab<4, 5>(a, grid, stream);
    case 6: return launch_ab<4, 6>(a, grid, stream);
    case 7: return launch_ab<4, 7>(a, grid, stream);
    default: return launch_ab<4, 8>(a, grid, stream);
  }
}

}  // namespace cw
