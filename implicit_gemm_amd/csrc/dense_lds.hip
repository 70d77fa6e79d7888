// Dense implicit-GEMM weight gradient, general geometry (gfx950).
//
// Per group g the weight gradient is a GEMM (rocm-libraries PR #14157 names
// the family conv_implicit_gemm_wgrad; PR #11188 section Motivation gives the
// 1x1 case as dY^T X):
//   M = Kg output channels, N = R*S*Cg columns (r, s, c), reduction over the
//   L = N*Ho*Wo output pixels l = (n, ho, wo):
//   dW[g*Kg + m][(r*S + s)*Cg + c] += dY[l][g*Kg + m] * X[n][h(ho,r)][w(wo,s)][g*Cg + c]
// The B operand is im2col(X), gathered on the fly with zero fill for pixels
// outside the image; it is never materialised in memory.
//
// Tiling: a workgroup (4 waves) owns a 64 x 64 output tile and one slice of
// reduction rows.  Each step stages 32 rows of dY and of im2col(X) in LDS as
// fp32, then each wave runs 2 x 2 v_mfma_f32_16x16x4_f32 per 4 rows on its
// 32 x 32 quarter.  Global loads of the next step are issued before the MFMA
// work of the current one.  16-bit inputs are widened to fp32 when staged
// (exact), so every dtype accumulates in fp32 on the f32 MFMA.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kBM = 64, kBN = 64, kBK = 32;
constexpr int kLdA = kBM + 16, kLdB = kBN + 16;  // row pitch = 16 (mod 32) floats: conflict-free reads

struct DenseArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;  // H*W*C
  int32_t H, W, C, K, Ho, Wo;
  int32_t R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
  int32_t Cg, Kg, cols;
  int32_t m_tiles, n_tiles;
  int32_t L, rows_per_slice, ks_count;
  float* dbo;   // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
};

// One thread's view of 4 consecutive GEMM columns (fixed for the whole kernel).
struct ColInfo {
  int dh[4], dw[4], ch[4];
  bool valid[4];
};

template <typename T, int VA, int VB>
__global__ __launch_bounds__(256) void dense_lds_kernel(DenseArgs a) {
  __shared__ float sA[kBK * kLdA];
  __shared__ float sB[kBK * kLdB];
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ dy = static_cast<const T*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  int tile = bid / a.ks_count;
  const int nt = tile % a.n_tiles;
  tile /= a.n_tiles;
  const int mt = tile % a.m_tiles;
  const int g = tile / a.m_tiles;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int l_begin = slice * a.rows_per_slice;
  const int l_end = min(a.L, l_begin + a.rows_per_slice);

  // Loader role: rows row0 and row0 + 16 of each 32-row step, columns 4*c4 .. 4*c4+3.
  const int c4 = tid & 15, row0 = tid >> 4;
  const int a_col = m0 + 4 * c4;
  ColInfo ci;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = n0 + 4 * c4 + e;
    ci.valid[e] = j < a.cols;
    const int jj = ci.valid[e] ? j : 0;
    const int c = jj % a.Cg, rs = jj / a.Cg;
    const int s = rs % a.S, r = rs / a.S;
    ci.dh[e] = r * a.dil_h - a.pad_h;
    ci.dw[e] = s * a.dil_w - a.pad_w;
    ci.ch[e] = g * a.Cg + c;
  }
  const int HoWo = a.Ho * a.Wo;
  // Pixel cursors of the thread's two rows: the steps visit l0 = l_begin,
  // l_begin + 32, ... in order, so (n, ho, wo) advance by 32 pixels per step
  // with carries instead of two divisions per row and step.
  int cn[2], cho[2], cwo[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int l = l_begin + row0 + 16 * it;
    cn[it] = l / HoWo;
    const int rem = l - cn[it] * HoWo;
    cho[it] = rem / a.Wo;
    cwo[it] = rem - cho[it] * a.Wo;
  }

  float ra[2][4], rb[2][4];
  auto load_step = [&](int l0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int l = l0 + row0 + 16 * it;
      const bool lv = l < l_end;
      const int n_c = cn[it], ho_c = cho[it], wo_c = cwo[it];
      cwo[it] += kBK;
      while (cwo[it] >= a.Wo) {
        cwo[it] -= a.Wo;
        if (++cho[it] == a.Ho) {
          cho[it] = 0;
          ++cn[it];
        }
      }
      // dY row l, output channels a_col .. a_col+3 of group g.
      const T* dyp = dy + (int64_t)l * a.K + (int64_t)g * a.Kg + a_col;
      if (VA == 4) {
        if (lv && a_col < a.Kg) {
          load4(dyp, ra[it]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) ra[it][e] = 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[it][e] = (lv && a_col + e < a.Kg) ? to_f32(dyp[e]) : 0.f;
      }
      // im2col(X) row l, columns n0 + 4*c4 .. +3.
      const int n = lv ? n_c : 0;
      const int ho = lv ? ho_c : 0, wo = lv ? wo_c : 0;
      const T* xn = x + (int64_t)n * a.x_img;
      if (VB == 4) {
        const int h = ho * a.stride_h + ci.dh[0], w = wo * a.stride_w + ci.dw[0];
        if (lv && ci.valid[0] && h >= 0 && h < a.H && w >= 0 && w < a.W) {
          load4(xn + ((int64_t)h * a.W + w) * a.C + ci.ch[0], rb[it]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) rb[it][e] = 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int h = ho * a.stride_h + ci.dh[e], w = wo * a.stride_w + ci.dw[e];
          rb[it][e] = (lv && ci.valid[e] && h >= 0 && h < a.H && w >= 0 && w < a.W)
                          ? to_f32(xn[((int64_t)h * a.W + w) * a.C + ci.ch[e]])
                          : 0.f;
        }
      }
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  // Bias gradient: the first column tile of each (group, output-channel
  // tile) adds up the dY rows it stages (rows past the slice load as zero).
  const bool want_db = a.dbo != nullptr && nt == 0;
  float dbp[4] = {0.f, 0.f, 0.f, 0.f};

  load_step(l_begin);
  for (int l0 = l_begin; l0 < l_end; l0 += kBK) {
    __syncthreads();  // previous step's MFMA reads of LDS are done
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row = row0 + 16 * it;
      if (want_db) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dbp[e] += ra[it][e];
      }
      *reinterpret_cast<float4*>(&sA[row * kLdA + 4 * c4]) =
          float4{ra[it][0], ra[it][1], ra[it][2], ra[it][3]};
      *reinterpret_cast<float4*>(&sB[row * kLdB + 4 * c4]) =
          float4{rb[it][0], rb[it][1], rb[it][2], rb[it][3]};
    }
    __syncthreads();
    if (l0 + kBK < l_end) load_step(l0 + kBK);  // overlap the next step's loads with MFMA
    // The operands of k-step kk + 1 are read before the MFMAs of kk issue
    // (two register sets), so each read has the previous step's MFMAs to
    // arrive instead of being waited for right before its own.
    float fa[2][2], fb[2][2];
    auto read_k = [&](int kk, float (&ra_)[2], float (&rb_)[2]) {
      const int rrow = 4 * kk + lg;
      ra_[0] = sA[rrow * kLdA + wm * 32 + li];
      ra_[1] = sA[rrow * kLdA + wm * 32 + 16 + li];
      rb_[0] = sB[rrow * kLdB + wn * 32 + li];
      rb_[1] = sB[rrow * kLdB + wn * 32 + 16 + li];
      __builtin_amdgcn_sched_barrier(0);
    };
    read_k(0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < kBK / 4; ++kk) {
      if (kk + 1 < kBK / 4) read_k(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      const float(&a)[2] = fa[kk & 1];
      const float(&b)[2] = fb[kk & 1];
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[1], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[0], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc[1][1], 0, 0, 0);
    }
  }

  if (want_db)   // 16 loader rows per channel quad
    block_sum64<16, 4>(sA, row0, 4 * c4, dbp,
                       a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0,
                       min(kBM, a.Kg - m0));

  // Each output element of this tile is written once, to dw or to slab `slice`.
  float* out = a.out + (int64_t)slice * a.slab_stride;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 32 + mi * 16 + 4 * lg + v;
        const int j = n0 + wn * 32 + ni * 16 + li;
        if (m < a.Kg && j < a.cols) out[((int64_t)g * a.Kg + m) * a.cols + j] = acc[mi][ni][v];
      }
}

template <typename T, int VA, int VB>
hipError_t launch_t(const DenseArgs& args, int64_t grid, hipStream_t stream) {
  return launch_kernel(dense_lds_kernel<T, VA, VB>, dim3((unsigned)grid), dim3(256), args, stream);
}

template <typename T>
hipError_t launch_vec(const Plan& plan, const DenseArgs& args, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  if (plan.vec_a == 4 && plan.vec_b == 4) return launch_t<T, 4, 4>(args, grid, stream);
  if (plan.vec_a == 4) return launch_t<T, 4, 1>(args, grid, stream);
  if (plan.vec_b == 4) return launch_t<T, 1, 4>(args, grid, stream);
  return launch_t<T, 1, 1>(args, grid, stream);
}

}  // namespace

hipError_t launch_dense(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                        hipStream_t stream) {
  const Problem& p = plan.p;
  DenseArgs a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.dbo = out.db;
  a.x_img = p.x_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.R = (int32_t)p.R; a.S = (int32_t)p.S;
  a.pad_h = (int32_t)p.pad_h; a.pad_w = (int32_t)p.pad_w;
  a.stride_h = (int32_t)p.stride_h; a.stride_w = (int32_t)p.stride_w;
  a.dil_h = (int32_t)p.dil_h; a.dil_w = (int32_t)p.dil_w;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg; a.cols = (int32_t)p.cols;
  a.m_tiles = (int32_t)plan.m_tiles; a.n_tiles = (int32_t)plan.n_tiles;
  a.L = (int32_t)p.L;
  a.rows_per_slice = (int32_t)(plan.pub.units_per_slice * plan.pub.unit_rows);
  a.ks_count = plan.pub.ks_count;
  switch (p.dtype) {
    case CONV_WGRAD_F32: return launch_vec<float>(plan, a, stream);
    case CONV_WGRAD_BF16: return launch_vec<Bf16>(plan, a, stream);
    default: return launch_vec<F16>(plan, a, stream);
  }
}

}  // namespace cw
