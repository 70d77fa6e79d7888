// Dense implicit-GEMM weight gradient over output-row units (gfx950, f32 MFMA).
//
// Same GEMM as the general dense kernel (per group: M = Kg, N = R*S*Cg,
// reduction over output pixels), organised so that every staged element is
// reused by all the taps of one filter row:
//
//   * a reduction unit is a run of up to `wt` consecutive output pixels of one
//     output row (n, ho);
//   * a workgroup tile is (group, 64 output channels, filter row r, SB
//     consecutive taps s, 64 input channels), so its B operand for tap s is
//     the staged X row segment shifted by s*dil pixels -- an LDS address
//     offset, not another load;
//   * the unit's dY rows [wt][64] and X segment [xspan][64] are staged once in
//     LDS (widened to fp32), double-buffered so the global loads of unit u+1
//     overlap the MFMA work of unit u, with one barrier per unit;
//   * wave w owns input channels 16w..16w+15 of the tile and all 64 output
//     channels: 4*SB independent v_mfma_f32_16x16x4_f32 accumulators, fed by
//     4 + SB LDS reads per 4 reduction rows.
//
// Rows of the LDS tiles are 80 floats apart (16 mod 32 and 16 mod 64 banks),
// so the 4 pixel rows a wave reads per MFMA fall in disjoint bank groups.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kPitch = 80;      // floats per staged pixel row (64 channels + pad)
constexpr int kMaxWt = 64;      // output pixels per unit
constexpr int kMaxXSpan = 80;   // staged X pixels per unit

struct RowsArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;  // H*W*C
  int32_t H, W, C, K, Ho, Wo;
  int32_t R, S, pad, stride, dil;
  int32_t Cg, Kg, cols;
  int32_t m_tiles, c_tiles, s_blocks;
  int32_t wt, wchunks, xspan;
  int32_t units, units_per_slice, ks_count;
};

template <typename T, int SB>
__global__ __launch_bounds__(256, 1) void dense_rows_kernel(RowsArgs a) {
  extern __shared__ float smem[];
  constexpr int kBuf = (kMaxWt + kMaxXSpan) * kPitch;  // floats per buffer
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ dy = static_cast<const T*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  int tile = bid / a.ks_count;
  const int ct = tile % a.c_tiles;
  tile /= a.c_tiles;
  const int sb = tile % a.s_blocks;
  tile /= a.s_blocks;
  const int r = tile % a.R;
  tile /= a.R;
  const int mt = tile % a.m_tiles;
  const int g = tile / a.m_tiles;
  const int m0 = mt * 64, c0 = ct * 64, s0 = sb * SB;

  const int u_begin = slice * a.units_per_slice;
  const int u_end = min(a.units, u_begin + a.units_per_slice);

  // Loader role: pixel rows p0 + 16*i, channel quad q (4 channels).
  const int q = tid & 15, p0 = tid >> 4;
  const bool a_ok = m0 + 4 * q < a.Kg;   // Kg % 4 == 0: the quad is all in or all out
  const bool b_ok = c0 + 4 * q < a.Cg;
  const int64_t dy_col = (int64_t)g * a.Kg + m0 + 4 * q;
  const int64_t x_col = (int64_t)g * a.Cg + c0 + 4 * q;
  const int dh = r * a.dil - a.pad;
  const int xw_off = s0 * a.dil - a.pad;

  float ra[kMaxWt / 16][4];
  float rb[kMaxXSpan / 16][4];
  int npix_next = 0;

  auto load_unit = [&](int u) {
    const int wc = u % a.wchunks;
    const int t = u / a.wchunks;
    const int ho = t % a.Ho, n = t / a.Ho;
    const int wo0 = wc * a.wt;
    const int npix = min(a.wt, a.Wo - wo0);
    npix_next = npix;
    const T* dyp = dy + ((int64_t)(n * a.Ho + ho) * a.Wo + wo0) * a.K + dy_col;
#pragma unroll
    for (int i = 0; i < kMaxWt / 16; ++i) {
      const int p = p0 + 16 * i;
      if (a_ok && p < npix) {
        load4(dyp + (int64_t)p * a.K, ra[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[i][e] = 0.f;
      }
    }
    const int h = ho * a.stride + dh;
    const bool row_ok = b_ok && h >= 0 && h < a.H;
    const int w0 = wo0 * a.stride + xw_off;
    const T* xp = x + (int64_t)n * a.x_img + ((int64_t)h * a.W) * a.C + x_col;
#pragma unroll
    for (int i = 0; i < kMaxXSpan / 16; ++i) {
      const int p = p0 + 16 * i;
      const int w = w0 + p;
      if (row_ok && p < a.xspan && w >= 0 && w < a.W) {
        load4(xp + (int64_t)w * a.C, rb[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[i][e] = 0.f;
      }
    }
  };

  auto store_unit = [&](float* buf) {
#pragma unroll
    for (int i = 0; i < kMaxWt / 16; ++i)
      *reinterpret_cast<float4*>(&buf[(p0 + 16 * i) * kPitch + 4 * q]) =
          float4{ra[i][0], ra[i][1], ra[i][2], ra[i][3]};
    float* xb = buf + kMaxWt * kPitch;
#pragma unroll
    for (int i = 0; i < kMaxXSpan / 16; ++i)
      *reinterpret_cast<float4*>(&xb[(p0 + 16 * i) * kPitch + 4 * q]) =
          float4{rb[i][0], rb[i][1], rb[i][2], rb[i][3]};
  };

  f32x4 acc[4][SB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < SB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int a_lane = lg * kPitch + li;                  // + 4*kstep rows, + 16*mt
  const int b_lane = lg * a.stride * kPitch + 16 * wave + li;
  const int b_kstep = 4 * a.stride * kPitch;
  const int b_tap = a.dil * kPitch;

  load_unit(u_begin);
  int buf_id = 0;
  for (int u = u_begin; u < u_end; ++u) {
    float* buf = smem + buf_id * kBuf;
    const int npix = npix_next;
    store_unit(buf);
    __syncthreads();
    if (u + 1 < u_end) load_unit(u + 1);
    const float* A = buf + a_lane;
    const float* B = buf + kMaxWt * kPitch + b_lane;
    const int nk = (npix + 3) >> 2;
    // Fragments of k-step k+1 are read while the MFMAs of k-step k run.
    float fa[4], fb[SB];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = A[16 * i];
#pragma unroll
    for (int s = 0; s < SB; ++s) fb[s] = B[s * b_tap];
    for (int k = 0; k < nk; ++k) {
      const int kn = k + 1 < nk ? k + 1 : k;
      float na[4], nb[SB];
#pragma unroll
      for (int i = 0; i < 4; ++i) na[i] = A[4 * kn * kPitch + 16 * i];
#pragma unroll
      for (int s = 0; s < SB; ++s) nb[s] = B[kn * b_kstep + s * b_tap];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < SB; ++s)
          acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[s], acc[i][s], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = na[i];
#pragma unroll
      for (int s = 0; s < SB; ++s) fb[s] = nb[s];
    }
    buf_id ^= 1;
  }

  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int c = c0 + 16 * wave + li;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * i + 4 * lg + v;
        const int sa = s0 + s;
        if (m < a.Kg && c < a.Cg && sa < a.S)
          out[((int64_t)g * a.Kg + m) * a.cols + (r * a.S + sa) * a.Cg + c] = acc[i][s][v];
      }
}

template <typename T, int SB>
hipError_t launch_sb(const RowsArgs& args, int64_t grid, hipStream_t stream) {
  constexpr size_t kLds = 2 * (kMaxWt + kMaxXSpan) * kPitch * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(dense_rows_kernel<T, SB>);
  // More than 64 KB of dynamic LDS must be enabled per kernel (once).
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  void* params[] = {const_cast<RowsArgs*>(&args)};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), params, kLds, stream);
}

template <typename T>
hipError_t launch_t(const Plan& plan, const RowsArgs& args, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  switch (plan.sb) {
    case 1: return launch_sb<T, 1>(args, grid, stream);
    case 2: return launch_sb<T, 2>(args, grid, stream);
    case 3: return launch_sb<T, 3>(args, grid, stream);
    default: return launch_sb<T, 4>(args, grid, stream);
  }
}

}  // namespace

hipError_t launch_dense_rows(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                             hipStream_t stream) {
  const Problem& p = plan.p;
  RowsArgs a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.x_img = p.x_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.R = (int32_t)p.R; a.S = (int32_t)p.S; a.pad = (int32_t)p.pad;
  a.stride = (int32_t)p.stride; a.dil = (int32_t)p.dil;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg; a.cols = (int32_t)p.cols;
  a.m_tiles = (int32_t)plan.m_tiles;
  a.c_tiles = (int32_t)plan.c_tiles;
  a.s_blocks = (int32_t)plan.s_blocks;
  a.wt = plan.wt;
  a.wchunks = (int32_t)plan.wchunks;
  a.xspan = plan.xspan;
  a.units = (int32_t)plan.pub.units;
  a.units_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  switch (p.dtype) {
    case CONV_WGRAD_F32: return launch_t<float>(plan, a, stream);
    case CONV_WGRAD_BF16: return launch_t<Bf16>(plan, a, stream);
    default: return launch_t<F16>(plan, a, stream);
  }
}

}  // namespace cw
