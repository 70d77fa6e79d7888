// Forward and data-gradient convolution as implicit GEMMs on the split-K
// slab machinery of the weight gradient (gfx950).
//
// rocm-libraries PR #14393 ("split-K forward implicit-GEMM convolution on
// gfx1250", sections Summary and "Two-stage split-K") adds split-K to the
// forward implicit GEMM: layers with few output pixels and a deep reduction
// leave too few workgroups, so the reduction is cut into slices, each writing
// an fp32 partial tile into its own slab, and a second kernel folds the slabs
// in a fixed order.  Here the same planner rules, slabs and fold serve both
// directions; per group g:
//
//   forward:  Y[m][g*Kg + n]  = sum_q A[m][q] * B[q][n]
//             m = output pixel (img, ho, wo), n < Kg, q = (r, s, c), c fastest;
//             A = Xpad[img][ho*stride_h + r*dil_h - pad_h][wo*stride_w + s*dil_w - pad_w][g*Cg + c],
//             B = W[g*Kg + n][r][s][c]  (contiguous along q for fixed n)
//   dgrad:    dX[m][g*Cg + n] = sum_q A[m][q] * B[q][n]
//             m = input pixel (img, h, w), n < Cg, q = (r, s, k), k fastest;
//             A = dY[img][ho][wo][g*Kg + k] with ho*stride_h = h + pad_h - r*dil_h
//                 (and the same for wo) exactly and inside the output, else 0,
//             B = W[g*Kg + k][r][s][n]  (contiguous along n for fixed q)
//
// A and B are gathered on the fly (never materialised).  Tiling: a 256-lane
// workgroup owns a 64 x 64 output tile and one slice of the reduction;
// every step stages 32 reduction entries of A and B in LDS as fp32 (16-bit
// inputs widened exactly), and each wave runs 2 x 2 v_mfma_f32_16x16x4_f32
// per 4 entries on its 32 x 32 quarter; the next step's global loads are
// issued before the current step's MFMAs.  Loads are 16-byte vectors along
// the contiguous axis when the channel counts allow it.  The dgrad A gather
// visits every (r, s) of a pixel; at stride > 1 most of them are holes that
// load zero (the work a stride-aware decomposition would skip).
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kBM = 64, kBN = 64, kBK = 32;
constexpr int kLdQ = kBK + 4;    // [row][q] layouts: 36 floats per row
constexpr int kLdN = kBN + 16;   // [q][n] layout (dgrad B): 80 floats per row

struct IgemmArgs {
  const void* a_src;     // x (forward) or dy (dgrad)
  const void* w;         // filter [K][R][S][Cg]
  float* out;            // y / dx, or slab 0
  int64_t slab_stride;   // floats between slabs (0 when writing the output)
  int64_t a_img;         // elements per image of the gathered tensor
  int32_t H, W, C, K, Ho, Wo;
  int32_t R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
  int32_t Cg, Kg;
  int32_t M;             // output pixels: N*Ho*Wo (forward) or N*H*W (dgrad)
  int32_t Ng;            // output channels per group (Kg or Cg)
  int32_t NT;            // output channels (K or C)
  int32_t Q;             // reduction length per group: R*S*Cg or R*S*Kg
  int32_t m_tiles, n_tiles, q_per_slice, ks_count;
};

template <typename T, bool kFwd, int VA, int VB>
__global__ __launch_bounds__(256) void igemm_kernel(IgemmArgs a) {
  __shared__ float sA[kBM * kLdQ];
  __shared__ float sB[kFwd ? kBN * kLdQ : kBK * kLdN];
  const T* __restrict__ src = static_cast<const T*>(a.a_src);
  const T* __restrict__ wt = static_cast<const T*>(a.w);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  int tile = bid / a.ks_count;
  const int nt = tile % a.n_tiles;
  tile /= a.n_tiles;
  const int mt = tile % a.m_tiles;
  const int g = tile / a.m_tiles;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int q_begin = slice * a.q_per_slice;
  const int q_end = min(a.Q, q_begin + a.q_per_slice);

  // A loader: rows ml and ml + 32 of the tile, reduction entries 4*q4 .. 4*q4+3.
  const int ml = tid >> 3, q4 = tid & 7;
  // Pixel coordinates of the two rows (fixed for the kernel).
  int img[2], py[2], px[2];
  bool mv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + ml + 32 * i;
    mv[i] = m < a.M;
    const int mm = mv[i] ? m : 0;
    const int hw = kFwd ? a.Ho * a.Wo : a.H * a.W;
    const int wdt = kFwd ? a.Wo : a.W;
    img[i] = mm / hw;
    const int rem = mm - img[i] * hw;
    py[i] = rem / wdt;
    px[i] = rem - py[i] * wdt;
  }
  // The channels a reduction entry q of group g reads in the gathered tensor,
  // and the filter tap it belongs to.
  const int ch_per = kFwd ? a.Cg : a.Kg;
  const int ch_base = g * ch_per;
  const int stride_src = kFwd ? a.C : a.K;     // elements per pixel of the gathered tensor

  float ra[2][4], rb[2][4];

  // Source offset (within the image) of A[row i][q .. q+3] for tap (r, s), or -1.
  auto a_offset = [&](int i, int r, int s, int ch) -> int {
    if (!mv[i]) return -1;
    if constexpr (kFwd) {
      const int h = py[i] * a.stride_h + r * a.dil_h - a.pad_h;
      const int w = px[i] * a.stride_w + s * a.dil_w - a.pad_w;
      if (h < 0 || h >= a.H || w < 0 || w >= a.W) return -1;
      return (h * a.W + w) * stride_src + ch_base + ch;
    } else {
      const int hn = py[i] + a.pad_h - r * a.dil_h;
      const int wn = px[i] + a.pad_w - s * a.dil_w;
      if (hn < 0 || wn < 0) return -1;
      // Unit strides (a workgroup-uniform test) skip the two divisions.
      int ho = hn, wo = wn;
      if (a.stride_h != 1 || a.stride_w != 1) {
        ho = hn / a.stride_h;
        wo = wn / a.stride_w;
        if (ho * a.stride_h != hn || wo * a.stride_w != wn) return -1;
      }
      if (ho >= a.Ho || wo >= a.Wo) return -1;
      return (ho * a.Wo + wo) * stride_src + ch_base + ch;
    }
  };

  // Reduction cursors: the steps visit q0 = q_begin, q_begin + 32, ... in
  // order, so the (channel, tap) of a thread's entries advance by 32 channels
  // per step with carries instead of two divisions per step (the VALU work of
  // the divisions does not overlap the MFMAs).
  // A (VA == 4): entry q_begin + 4*q4 as (ca, sa, ra_) = (channel, s, r).
  int ca = 0, sa = 0, ra_ = 0;
  if (VA == 4) {
    const int q = q_begin + 4 * q4;
    ca = q % ch_per;
    const int rs = q / ch_per;
    sa = rs % a.S;
    ra_ = rs / a.S;
  }
  // dgrad B: entries q_begin + ql + 16*i as (k, r*S + s).
  int kb[2] = {0, 0}, rsb[2] = {0, 0};
  if constexpr (!kFwd) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = q_begin + (tid >> 4) + 16 * i;
      kb[i] = q % a.Kg;
      rsb[i] = q / a.Kg;
    }
  }

  auto load_step = [&](int q0) {
    // A: entries q .. q + 3 of the two rows.
    const int q = q0 + 4 * q4;
    if (VA == 4) {
      // ch_per % 4 == 0: the four entries share one tap.
      const bool qv = q < q_end;
      const int ch = ca, s = sa, r = ra_;
      ca += kBK;
      while (ca >= ch_per) {
        ca -= ch_per;
        if (++sa == a.S) {
          sa = 0;
          ++ra_;
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int off = qv ? a_offset(i, r, s, ch) : -1;
        if (off >= 0) {
          load4(src + (int64_t)img[i] * a.a_img + off, ra[i]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) ra[i][e] = 0.f;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qe = q + e;
        const bool qv = qe < q_end;
        const int qq = qv ? qe : 0;
        const int ch = qq % ch_per, rs = qq / ch_per;
        const int s = rs % a.S, r = rs / a.S;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int off = qv ? a_offset(i, r, s, ch) : -1;
          ra[i][e] = off >= 0 ? to_f32(src[(int64_t)img[i] * a.a_img + off]) : 0.f;
        }
      }
    }
    // B.
    if constexpr (kFwd) {
      // Rows n (filter k = g*Kg + n0 + nl (+32)), entries q .. q + 3: contiguous in W.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = n0 + ml + 32 * i;
        const T* wr = wt + (int64_t)(g * a.Kg + n) * a.Q;
        if (VB == 4) {
          if (n < a.Kg && q < q_end) {
            load4(wr + q, rb[i]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) rb[i][e] = 0.f;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) rb[i][e] = (n < a.Kg && q + e < q_end) ? to_f32(wr[q + e]) : 0.f;
        }
      }
    } else {
      // Entries ql and ql + 16 of the step, channels n0 + 4*n4 .. +3: contiguous in W.
      const int ql = tid >> 4, n4 = tid & 15;
      const int n = n0 + 4 * n4;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int qe = q0 + ql + 16 * i;
        const bool qv = qe < q_end;
        const int k = kb[i], rs = rsb[i];     // q = (r, s, k): W[g*Kg + k][r][s][.]
        kb[i] += kBK;
        while (kb[i] >= a.Kg) {
          kb[i] -= a.Kg;
          ++rsb[i];
        }
        const T* wr = wt + ((int64_t)(g * a.Kg + (qv ? k : 0)) * a.R * a.S + (qv ? rs : 0)) * a.Cg;
        if (VB == 4) {
          if (qv && n < a.Cg) {
            load4(wr + n, rb[i]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) rb[i][e] = 0.f;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) rb[i][e] = (qv && n + e < a.Cg) ? to_f32(wr[n + e]) : 0.f;
        }
      }
    }
  };

  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<float4*>(&sA[(ml + 32 * i) * kLdQ + 4 * q4]) =
          float4{ra[i][0], ra[i][1], ra[i][2], ra[i][3]};
    if constexpr (kFwd) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<float4*>(&sB[(ml + 32 * i) * kLdQ + 4 * q4]) =
            float4{rb[i][0], rb[i][1], rb[i][2], rb[i][3]};
    } else {
      const int ql = tid >> 4, n4 = tid & 15;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<float4*>(&sB[(ql + 16 * i) * kLdN + 4 * n4]) =
            float4{rb[i][0], rb[i][1], rb[i][2], rb[i][3]};
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  if (q_begin < q_end) load_step(q_begin);
  for (int q0 = q_begin; q0 < q_end; q0 += kBK) {
    __syncthreads();   // the previous step's MFMA reads are done
    store_step();
    __syncthreads();
    if (q0 + kBK < q_end) load_step(q0 + kBK);   // overlap the next step's loads with the MFMAs
#pragma unroll
    for (int kk = 0; kk < kBK / 4; ++kk) {
      const int qc = 4 * kk + lg;
      const float a0 = sA[(wm * 32 + li) * kLdQ + qc];
      const float a1 = sA[(wm * 32 + 16 + li) * kLdQ + qc];
      float b0, b1;
      if constexpr (kFwd) {
        b0 = sB[(wn * 32 + li) * kLdQ + qc];
        b1 = sB[(wn * 32 + 16 + li) * kLdQ + qc];
      } else {
        b0 = sB[qc * kLdN + wn * 32 + li];
        b1 = sB[qc * kLdN + wn * 32 + 16 + li];
      }
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  }

  // acc[mi][ni][v]: row m = m0 + 32 wm + 16 mi + 4 lg + v, column n = n0 + 32 wn + 16 ni + li.
  float* out = a.out + (int64_t)slice * a.slab_stride;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 32 + mi * 16 + 4 * lg + v;
        const int n = n0 + wn * 32 + ni * 16 + li;
        if (m < a.M && n < a.Ng) out[(int64_t)m * a.NT + (int64_t)g * a.Ng + n] = acc[mi][ni][v];
      }
}

template <typename T, bool kFwd>
hipError_t launch_dir(const Plan& plan, const IgemmArgs& args, hipStream_t stream) {
  const dim3 grid((unsigned)plan.pub.grid), block(256);
  if (plan.vec_a == 4 && plan.vec_b == 4) return launch_kernel(igemm_kernel<T, kFwd, 4, 4>, grid, block, args, stream);
  if (plan.vec_a == 4) return launch_kernel(igemm_kernel<T, kFwd, 4, 1>, grid, block, args, stream);
  if (plan.vec_b == 4) return launch_kernel(igemm_kernel<T, kFwd, 1, 4>, grid, block, args, stream);
  return launch_kernel(igemm_kernel<T, kFwd, 1, 1>, grid, block, args, stream);
}

template <bool kFwd>
hipError_t launch_t(const Plan& plan, const IgemmArgs& args, hipStream_t stream) {
  switch (plan.p.dtype) {
    case CONV_WGRAD_F32: return launch_dir<float, kFwd>(plan, args, stream);
    case CONV_WGRAD_BF16: return launch_dir<Bf16, kFwd>(plan, args, stream);
    default: return launch_dir<F16, kFwd>(plan, args, stream);
  }
}

}  // namespace

hipError_t launch_igemm(const Plan& plan, const void* a_src, const void* w, Stage1Out out, hipStream_t stream) {
  const Problem& p = plan.p;
  const bool fwd = plan.pub.variant == kFwdIgemm;
  IgemmArgs a;
  a.a_src = a_src;
  a.w = w;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.a_img = fwd ? p.x_img : p.dy_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.R = (int32_t)p.R; a.S = (int32_t)p.S;
  a.pad_h = (int32_t)p.pad_h; a.pad_w = (int32_t)p.pad_w;
  a.stride_h = (int32_t)p.stride_h; a.stride_w = (int32_t)p.stride_w;
  a.dil_h = (int32_t)p.dil_h; a.dil_w = (int32_t)p.dil_w;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg;
  a.M = (int32_t)plan.pub.L;
  a.Ng = (int32_t)(fwd ? p.Kg : p.Cg);
  a.NT = (int32_t)(fwd ? p.K : p.C);
  a.Q = (int32_t)(fwd ? p.R * p.S * p.Cg : p.R * p.S * p.Kg);
  a.m_tiles = (int32_t)plan.m_tiles;
  a.n_tiles = (int32_t)plan.n_tiles;
  a.q_per_slice = (int32_t)(plan.pub.units_per_slice * plan.pub.unit_rows);
  a.ks_count = plan.pub.ks_count;
  return fwd ? launch_t<true>(plan, a, stream) : launch_t<false>(plan, a, stream);
}

}  // namespace cw
