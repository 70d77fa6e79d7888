// Depthwise weight gradient on batched 4x4x4 MFMA (gfx950, bf16 / fp16 in, fp32 out).
//
// For one channel c the depthwise weight gradient is a 2-D correlation,
//   dW[c][r][s] = sum_{ho} sum_{w} X[ho + r - pad][w][c] * dY[ho][w - s + pad][c]
// (X zero outside the image, dY zero outside [0, Wo)).  Following the batched
// 4x4x4 MFMA organisation of rocm-libraries PR #14157 ("depthwise 7x7 and
// grouped cpg4/8 wgrad on batched mfma 4x4x4", Technical Details), one
// v_mfma_f32_4x4x4_16b instruction computes 16 independent 4 x 4 x 4 products,
// here one per channel: block b = channel, M = 4 filter rows r, N = 4 filter
// columns s, K = 4 input columns w.  2 x 2 instructions (RB x SB) cover a
// filter of up to 8 x 8.
//
//   A_b[i][k] = X[ho - pad + 4*rb + i][w0 + k]        (4 consecutive columns of one row)
//   B_b[k][j] = dY[ho][w0 + k - (4*sb + j) + pad]     (a shifted dY row segment)
//
// Each one-wave workgroup owns 16 channels and a slice of output rows.  Rows
// are staged in LDS per channel with columns contiguous, so A is one aligned
// 8-byte read.  B starts at a column that depends on the lane's j; every dY row
// is stored twice, the second copy shifted by one element, so each lane reads
// its window dword-aligned from one of the two copies.  The B operand of
// s-block 1 at column step w0 equals the s-block-0 operand of step w0 - 4, so
// it is carried in registers.  X rows live in an 8-row ring (a row is loaded
// once per slice); the NHWC -> per-channel transpose happens in registers
// (v_perm_b32) between the global load and the LDS store, and rows are
// prefetched four steps ahead.  The wave never waits on another wave.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kChW = 16;     // channels per wave (MFMA blocks)
constexpr int kRing = 8;     // X rows held
constexpr int kOff = 8;      // leading zero columns of a staged dY row
constexpr int kPf = 4;       // steps prefetched ahead

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

struct DwArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img, dy_img;   // elements per image
  int32_t H, W, C, Ho, Wo, R, S, pad;
  int32_t xl, dl;          // staged row lengths (elements) of X and dY
  int32_t x_slot;          // bytes between X ring slots
  int32_t rows, rows_per_slice, ks_count;  // rows = N * Ho
  int32_t quads;           // ceil(C / 64): channel quads of four 16-channel groups
  int32_t lds_bytes;
};

template <bool kBf16>
__device__ __forceinline__ f32x4 mfma4(s16x4 a, s16x4 b, f32x4 c) {
  if constexpr (kBf16)
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, a),
                                              __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// 4 pixels x 8 channels of one row, as loaded (pixel-major).
struct Item {
  uint4 p[4];
};

__device__ __forceinline__ void fetch(const unsigned short* base, int64_t row_off, int n_pix,
                                      int cstride, int pg, bool active, Item& it) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int w = 4 * pg + q;
    it.p[q] = uint4{0u, 0u, 0u, 0u};
    if (active && w < n_pix)
      it.p[q] = *reinterpret_cast<const uint4*>(base + row_off + (int64_t)w * cstride);
  }
}

__device__ __forceinline__ uint32_t word(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Channel cc of the item: pixels (0,1) and (2,3) packed as two dwords.
__device__ __forceinline__ void channel_pair(const Item& it, int cc, uint32_t& lo, uint32_t& hi) {
  const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
  lo = __builtin_amdgcn_perm(word(it.p[1], cc >> 1), word(it.p[0], cc >> 1), sel);
  hi = __builtin_amdgcn_perm(word(it.p[3], cc >> 1), word(it.p[2], cc >> 1), sel);
}

template <bool kBf16, int RB, int SB>
__global__ __launch_bounds__(64) void depthwise_mfma_kernel(DwArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const unsigned short* __restrict__ x = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ dy = static_cast<const unsigned short*>(a.dy);
  const int lane = threadIdx.x;
  // Workgroups are dispatched to the 8 XCDs round-robin (block i on XCD i % 8).
  // The four 16-channel groups that share a 128-byte pixel segment of X and dY
  // are given block ids 8 apart (same XCD, adjacent in dispatch order), so the
  // lines one group fetches are served from that XCD's L2 to the other three.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, jq = bid >> 3;
  const int work = (jq >> 2) * 8 + xcd;          // (slice, channel quad) pair
  if (work >= a.ks_count * a.quads) return;
  const int slice = work % a.ks_count;
  const int group = (work / a.ks_count) * 4 + (jq & 3);
  if (group * kChW >= a.C) return;
  const int c0 = group * kChW;
  const int r_begin = slice * a.rows_per_slice;
  const int r_end = min(a.rows, r_begin + a.rows_per_slice);

  unsigned char* xring = lds;
  unsigned char* dyrow = lds + kRing * a.x_slot;              // copy 0; copy 1 follows
  const int dy_copy = kChW * a.dl * 2;                         // bytes per copy
  for (int i = lane * 16; i < a.lds_bytes; i += 64 * 16)
    *reinterpret_cast<uint4*>(lds + i) = uint4{0u, 0u, 0u, 0u};

  // Loader role: pixel group pg (pixels 4pg..4pg+3), channel half hh (8 channels).
  const int pg = lane >> 1, hh = lane & 1;
  const bool x_act = 4 * pg < a.xl;
  const bool dy_act = 4 * pg < a.Wo + 4;
  const unsigned short* xb = x + c0 + 8 * hh;
  const unsigned short* dyb = dy + c0 + 8 * hh;

  auto x_slot_of = [&](int h) { return ((h % kRing) + kRing) % kRing; };
  auto fetch_x = [&](int n, int h, Item& it) {
    const bool ok = x_act && h >= 0 && h < a.H;
    fetch(xb, (int64_t)n * a.x_img + (int64_t)h * a.W * a.C, a.W, a.C, pg, ok, it);
  };
  auto fetch_dy = [&](int n, int ho, Item& it) {
    fetch(dyb, (int64_t)n * a.dy_img + (int64_t)ho * a.Wo * a.C, a.Wo, a.C, pg, dy_act, it);
  };
  auto store_x = [&](int slot, const Item& it) {
    if (!x_act) return;
    unsigned char* base = xring + slot * a.x_slot + (8 * hh) * a.xl * 2 + 8 * pg;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      uint32_t lo, hi;
      channel_pair(it, cc, lo, hi);
      *reinterpret_cast<uint2*>(base + cc * a.xl * 2) = uint2{lo, hi};
    }
  };
  auto store_dy = [&](const Item& it) {
    if (!dy_act) return;
    // copy 0: element e at column e + kOff; copy 1: element e at column e + kOff + 1.
    unsigned char* b0 = dyrow + (8 * hh) * a.dl * 2 + (4 * pg + kOff) * 2;
    unsigned char* b1 = b0 + dy_copy + 2;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      uint32_t lo, hi;
      channel_pair(it, cc, lo, hi);
      *reinterpret_cast<uint2*>(b0 + cc * a.dl * 2) = uint2{lo, hi};
      unsigned char* p1 = b1 + cc * a.dl * 2;
      *reinterpret_cast<unsigned short*>(p1) = (unsigned short)(lo & 0xffffu);
      *reinterpret_cast<uint32_t*>(p1 + 2) = __builtin_amdgcn_perm(hi, lo, 0x05040302u);
      *reinterpret_cast<unsigned short*>(p1 + 6) = (unsigned short)(hi >> 16);
    }
  };

  // MFMA operand addressing.  Lane = 4*b + q: block b = channel c0 + b.
  const int b = lane >> 2, q = lane & 3;
  const int a_lane = b * a.xl * 2;                 // + slot * x_slot + 2*w0
  // The B window of s-block 0 starts at dY element w0 + pad - q, stored at
  // column w0 + col0 of copy 0 (col0 = kOff + pad - q) or one column later in
  // copy 1; the lane takes the copy in which that column is even, so its two
  // dword reads are aligned.
  const int col0 = kOff + a.pad - q;
  const int b_lane = b * a.dl * 2 + ((col0 & 1) ? dy_copy + 2 * (col0 + 1) : 2 * col0);

  f32x4 acc[RB][SB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < SB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_row = [&](int ho) {
    int slot_a[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) slot_a[i] = x_slot_of(ho - a.pad + 4 * i + q) * a.x_slot + a_lane;
    const unsigned char* bp = dyrow + b_lane;
    s16x4 bprev = {0, 0, 0, 0};
    if (SB > 1) {  // window of column step -4: dY columns -4 - q + pad (zero padding)
      const uint32_t* p = reinterpret_cast<const uint32_t*>(bp - 8);
      bprev = __builtin_bit_cast(s16x4, uint2{p[0], p[1]});
    }
    // Operands of column step w0 + 4 are read while the MFMAs of step w0 run.
    auto read_a = [&](int w0, s16x4 (&fa)[RB]) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
        fa[i] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(xring + slot_a[i] + 2 * w0));
    };
    auto read_b = [&](int w0) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(bp + 2 * w0);
      return __builtin_bit_cast(s16x4, uint2{p[0], p[1]});
    };
    auto mfma_step = [&](const s16x4 (&fa)[RB], const s16x4& fb) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        acc[i][0] = mfma4<kBf16>(fa[i], fb, acc[i][0]);
        if (SB > 1) acc[i][1] = mfma4<kBf16>(fa[i], bprev, acc[i][1]);
      }
      bprev = fb;
    };
    // Two named operand sets, so the reads of one step stay in flight while
    // the other step's MFMAs issue.  xl is a multiple of 8.
    s16x4 fa0[RB], fa1[RB], fb0, fb1;
    read_a(0, fa0);
    fb0 = read_b(0);
    for (int w0 = 0; w0 < a.xl; w0 += 8) {
      read_a(w0 + 4, fa1);
      fb1 = read_b(w0 + 4);
      mfma_step(fa0, fb0);
      const int wn = w0 + 8 < a.xl ? w0 + 8 : w0;
      read_a(wn, fa0);
      fb0 = read_b(wn);
      mfma_step(fa1, fb1);
    }
  };

  // Stream the slice one image segment at a time.  Step t of a segment that
  // starts at output row ho0 brings X row ho0 - pad + t into the ring and, from
  // step R - 1 on, dY row ho = ho0 + t - (R - 1), after which the ring holds X
  // rows ho - pad .. ho - pad + R - 1 and row ho is computed.  Loads run kPf
  // steps ahead of their use.
  Item qx[kPf], qd[kPf];
  int row = r_begin;
  while (row < r_end) {
    const int n = row / a.Ho, ho0 = row % a.Ho;
    const int seg = min(r_end - row, a.Ho - ho0);
    const int steps = seg + a.R - 1;
    auto fetch_step = [&](int t, Item& ix, Item& id) {
      fetch_x(n, ho0 - a.pad + t, ix);
      if (t >= a.R - 1) fetch_dy(n, ho0 + t - (a.R - 1), id);
    };
#pragma unroll
    for (int k = 0; k < kPf; ++k)
      if (k < steps) fetch_step(k, qx[k], qd[k]);
    for (int t = 0; t < steps; t += kPf) {
#pragma unroll
      for (int k = 0; k < kPf; ++k) {
        const int tk = t + k;
        if (tk < steps) {
          store_x(x_slot_of(ho0 - a.pad + tk), qx[k]);
          const bool has_dy = tk >= a.R - 1;
          if (has_dy) store_dy(qd[k]);
          if (tk + kPf < steps) fetch_step(tk + kPf, qx[k], qd[k]);
          if (has_dy) compute_row(ho0 + tk - (a.R - 1));
        }
      }
    }
    row += seg;
  }

  // acc[rb][sb][v] = dW[c0 + b][4*rb + v][4*sb + q]
  float* out = a.out + (int64_t)slice * a.slab_stride + (int64_t)(c0 + b) * a.R * a.S;
  if (c0 + b < a.C) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * i + v, s = 4 * j + q;
          if (r < a.R && s < a.S) out[r * a.S + s] = acc[i][j][v];
        }
  }
}

template <bool kBf16, int RB, int SB>
hipError_t launch_rs(const DwArgs& args, int64_t grid, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(depthwise_mfma_kernel<kBf16, RB, SB>);
  if (args.lds_bytes > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, args.lds_bytes);
    if (e != hipSuccess) return e;
  }
  void* params[] = {const_cast<DwArgs*>(&args)};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64), params, (size_t)args.lds_bytes, stream);
}

template <bool kBf16>
hipError_t launch_b(const Plan& plan, const DwArgs& a, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  const bool r2 = a.R > 4, s2 = a.S > 4;
  if (r2 && s2) return launch_rs<kBf16, 2, 2>(a, grid, stream);
  if (r2) return launch_rs<kBf16, 2, 1>(a, grid, stream);
  if (s2) return launch_rs<kBf16, 1, 2>(a, grid, stream);
  return launch_rs<kBf16, 1, 1>(a, grid, stream);
}

}  // namespace

hipError_t launch_depthwise(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream) {
  const Problem& p = plan.p;
  DwArgs a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.x_img = p.x_img;
  a.dy_img = p.dy_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.R = (int32_t)p.R; a.S = (int32_t)p.S; a.pad = (int32_t)p.pad;
  a.xl = plan.dw_xl;
  a.dl = plan.dw_dl;
  a.x_slot = plan.dw_xslot;
  a.rows = (int32_t)(p.N * p.Ho);
  a.rows_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  a.quads = (int32_t)ceil_div(p.C, 64);
  a.lds_bytes = plan.dw_lds;
  if (p.dtype == CONV_WGRAD_BF16) return launch_b<true>(plan, a, stream);
  return launch_b<false>(plan, a, stream);
}

}  // namespace cw
