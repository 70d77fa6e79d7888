// Depthwise weight gradient on batched 4x4x4 MFMA (gfx950, bf16 / fp16 in, fp32 out).
//
// For one channel c the depthwise weight gradient is a 2-D correlation,
//   dW[c][r][s] = sum_{ho} sum_{w} X[ho + r - pad][w][c] * dY[ho][w - s + pad][c]
// (X zero outside the image, dY zero outside [0, Wo)).  Following the batched
// 4x4x4 MFMA organisation of rocm-libraries PR #14157 ("depthwise 7x7 and
// grouped cpg4/8 wgrad on batched mfma 4x4x4", Technical Details), one
// v_mfma_f32_4x4x4_16b instruction computes 16 independent 4 x 4 x 4 products,
// here one per channel: block b = channel, M = 4 filter rows r, N = 4 filter
// columns s, K = 4 input columns w.  RB x SB (up to 2 x 2) instructions cover
// a filter of up to 8 x 8.
//
//   A_b[i][k] = X[ho - pad + 4*rb + i][w0 + k]        (4 consecutive columns of one row)
//   B_b[k][j] = dY[ho][w0 + k - (4*sb + j) + pad]     (a shifted dY row segment)
//
// A workgroup of four waves owns 64 consecutive channels (one 128-byte pixel
// segment of X and dY) and a slice of output rows; wave w computes channels
// w, w + 4, ..., w + 60 of them.  Per step the workgroup loads one X row and
// one dY row with full-line 16-byte loads (8 lanes per pixel) and stages them
// in LDS per channel with columns contiguous:
//  * Raw buffer loads whose range is the valid part of the row (empty for rows
//    outside the image or the segment) supply the zero padding.
//  * A lane holds 2 pixels x 8 channels and transposes them to 8 channel
//    dwords with v_perm_b32.  Interleaving channels across waves puts the
//    8 octets of one store instruction in 8 different 32-byte bank groups.
//  * X rows live in a ring of 4 or 8 rows.  The channel pitch is 16 mod 32
//    bytes and the slot pitch 64 mod 256 bytes, so the A reads (one 16-byte
//    read gives the operands of two column steps) are free of bank conflicts.
//  * dY rows alternate between two buffers.  A lane's B window starts at a
//    column that depends on its filter column j; it is cut out of two
//    4-byte-aligned dword pairs (ds_read2_b32, starting at the window's column
//    rounded down to even) with two v_perm_b32 whose selector is per lane.
//    The B operand of s-block 1 at column step w0 equals the s-block-0
//    operand of step w0 - 4, so it is carried in registers.
// The staged row length is a template parameter: every LDS offset is an
// immediate and a row's column loop is fully unrolled.  One barrier per step
// (waiting for LDS only, so global loads stay kPf steps ahead) separates the
// staging of step t from the MFMAs of step t; the ring holds R + 1 rows and
// the dY buffers alternate, so step t + 1 can be staged while step t computes.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kThreads = 256;
constexpr int kQuadCh = 64;   // channels per workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const unsigned char lds_cu8;

struct DwArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img, dy_img;   // elements per image
  int32_t H, W, C, Ho, Wo, R, S, pad;
  int32_t stride;          // 1 or 2 (both axes)
  int32_t dy_off;          // column of dY element 0 in a staged dY row
  int32_t rows, rows_per_slice, ks_count;  // rows = N * Ho
  int32_t quads;           // ceil(C / 64)
  float* dbo;              // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
  int32_t balanced;        // slice s covers rows [starts[s], starts[s + 1]); else uniform runs
  int32_t starts[Plan::kDwMaxSlices + 1];
};

// LDS layout for staged rows of XL columns.
// Ring rows for RB row blocks: R + 1 rows (the rows of one output row plus the
// row being staged) rounded up to a power of two.
template <int RB>
constexpr int dw_ring() { return RB == 1 ? 4 : RB == 2 ? 8 : 16; }

template <int XL, int RING, int TAPS>
struct DwLayout {
  static constexpr int kCs = 2 * XL;              // bytes per X channel row
  static constexpr int kXWave = 16 * kCs;         // bytes per wave in a ring slot
  static constexpr int kSlot = 64 * kCs + 64;     // ring slot pitch (64 mod 256)
  static constexpr int kDl = XL + 16;             // dY row length (elements, 8 mod 16)
  static constexpr int kDs = 2 * kDl;             // bytes per dY channel row
  static constexpr int kDWave = 16 * kDs;
  static constexpr int kDBuf = 64 * kDs;          // bytes per dY buffer
  static constexpr int kDyBase = RING * kSlot;
  static constexpr int kOut = kQuadCh * TAPS * 4;  // output block: 64 channels x up to TAPS taps
  static constexpr int kBytes = kDyBase + 2 * kDBuf > kOut ? kDyBase + 2 * kDBuf : kOut;
};

template <bool kBf16>
__device__ __forceinline__ f32x4 mfma4(s16x4 a, s16x4 b, f32x4 c) {
  if constexpr (kBf16)
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, a),
                                              __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const unsigned char* base, int nbytes) {
  // gfx9 raw buffer: stride 0, default data format; offsets >= nbytes read 0.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0, nbytes,
                                           0x00020000);
}

// Pixels 2pp, 2pp + 1 x 8 channels per pass, as loaded (pixel-major).
template <int NP>
struct Item {
  u32x4 p[NP][2];
};

template <bool kBf16, int RB, int SB, int XL>
__global__ __launch_bounds__(kThreads) void depthwise_mfma_kernel(DwArgs a) {
  constexpr int NP = XL > 64 ? 2 : 1;   // pixel-pair passes per row
  constexpr int kPf = 2;                // steps fetched ahead (even: dY buffer parity is static)
  constexpr int RING = dw_ring<RB>();
  constexpr int NPAIRS = XL / 8;
  using L = DwLayout<XL, RING, 16 * RB * SB>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const unsigned char* __restrict__ xg = static_cast<const unsigned char*>(a.x);
  const unsigned char* __restrict__ dyg = static_cast<const unsigned char*>(a.dy);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // Work item w = (slice, channel quad), quad fastest.  Block b runs on XCD
  // b % 8 (round-robin dispatch) and XCD x takes the items
  // [x * per_xcd, (x + 1) * per_xcd), so the quads of a slice, which read
  // the same pixel records at the same time, share one L2 and reach DRAM
  // together; the grid is a multiple of 8 and the blocks past the items exit.
  const int work = a.quads * a.ks_count;
  const int per_xcd = (work + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || w >= work) return;
  const int quad = w % a.quads;
  const int slice = w / a.quads;
  const int c0 = quad * kQuadCh;
  // Slices balanced by staging steps (boundaries from the plan), else uniform.
  const int r_begin = a.balanced ? a.starts[slice] : slice * a.rows_per_slice;
  const int r_end = a.balanced ? a.starts[slice + 1] : min(a.rows, r_begin + a.rows_per_slice);

  // Zero both dY buffers once: their columns outside the dY row are never written.
  for (int i = L::kDyBase + tid * 16; i < L::kBytes; i += kThreads * 16)
    *reinterpret_cast<uint4*>(lds + i) = uint4{0u, 0u, 0u, 0u};

  // Loader role: pixel pair pp (+ 32 per pass), channel octet o of the quad.
  const int o = tid & 7, pp = tid >> 3;
  const int row_bytes_x = (a.W * a.C - c0) * 2;     // valid bytes from the quad's first channel
  const int row_bytes_dy = (a.Wo * a.C - c0) * 2;
  const int pix_bytes = a.C * 2;
  int vo[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) vo[p] = 2 * (pp + 32 * p) * pix_bytes + 16 * o;
  auto fetch = [&](__amdgpu_buffer_rsrc_t rs, Item<NP>& it) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      it.p[p][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo[p], 0, 0));
      it.p[p][1] = __builtin_bit_cast(u32x4,
                                      __builtin_amdgcn_raw_buffer_load_b128(rs, vo[p] + pix_bytes, 0, 0));
    }
  };
  // Channel cc of the octet for pixels (2pp, 2pp + 1) as one dword.
  auto chan = [](const u32x4& p0, const u32x4& p1, int cc) {
    return __builtin_amdgcn_perm(p1[cc >> 1], p0[cc >> 1], (cc & 1) ? 0x07060302u : 0x05040100u);
  };
  // Quad channel ch = 8o + cc belongs to wave ch & 3 (= cc & 3), block ch >> 2.
  unsigned char* const xw = lds + 2 * o * L::kCs + 4 * pp;
  unsigned char* const dw0 = lds + L::kDyBase + 2 * o * L::kDs + 2 * a.dy_off + 4 * pp;
  auto store_x = [&](int slot, const Item<NP>& it) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (2 * (pp + 32 * p) < XL) {
        unsigned char* d = xw + slot * L::kSlot + 128 * p;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
          *reinterpret_cast<uint32_t*>(d + (cc & 3) * L::kXWave + (cc >> 2) * L::kCs) =
              chan(it.p[p][0], it.p[p][1], cc);
      }
    }
  };
  // Stride 2 stages each dY row upsampled (element wo at column 2 wo, zeros
  // between), so that the column-step windows below are those of stride 1.
  unsigned char* const dw2 = lds + L::kDyBase + 2 * o * L::kDs + 2 * a.dy_off + 8 * pp;
  auto store_dy = [&](int buf, const Item<NP>& it) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (2 * (pp + 32 * p) < a.Wo) {
        if (a.stride == 2) {
          unsigned char* d = dw2 + buf * L::kDBuf + 256 * p;
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const uint32_t v = chan(it.p[p][0], it.p[p][1], cc);
            *reinterpret_cast<u32x2*>(d + (cc & 3) * L::kDWave + (cc >> 2) * L::kDs) =
                u32x2{v & 0xffffu, v >> 16};
          }
          continue;
        }
        unsigned char* d = dw0 + buf * L::kDBuf + 128 * p;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
          *reinterpret_cast<uint32_t*>(d + (cc & 3) * L::kDWave + (cc >> 2) * L::kDs) =
              chan(it.p[p][0], it.p[p][1], cc);
      }
    }
  };

  // MFMA operand addressing.  Lane = 4*b + q: block b = channel c0 + wave + 4b.
  const int b = lane >> 2, q = lane & 3;
  // The s-block-0 window of lane q at column step w0 starts at dY element
  // w0 + pad - q, staged at column w0 + d with d = dy_off + pad - q: it is
  // elements u..u+3 (u = d mod 2) of the dword pairs at columns w0 + 2m and
  // w0 + 2m + 4 (m = d / 2).
  const int d0 = a.dy_off + a.pad - q;
  const uint32_t bsel = (d0 & 1) ? 0x05040302u : 0x03020100u;     // u odd: shift by one element
  lds_cu8* const bq = (lds_cu8*)lds + L::kDyBase + wave * L::kDWave + b * L::kDs + 2 * (d0 & ~1);
  // Separate base registers keep the two dword-pair reads of a column-step
  // pair as separate instructions.
  lds_cu8* bq4 = bq + 8;
  asm volatile("" : "+v"(bq4));
  auto window = [&](u32x2 q0, u32x2 q1) {
    const uint32_t lo = q0.x, mid = q0.y, hi = q1.x;
    const u32x2 v{__builtin_amdgcn_perm(mid, lo, bsel), __builtin_amdgcn_perm(hi, mid, bsel)};
    return __builtin_bit_cast(s16x4, v);
  };
  const unsigned char* const xr = lds + wave * L::kXWave + b * L::kCs;

  f32x4 acc[RB][SB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < SB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One row: NPAIRS pairs of column steps, fully unrolled.
  auto compute_row = [&](int ho, int buf) {
    const unsigned char* ap[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) ap[i] = xr + ((a.stride * ho - a.pad + 4 * i + q) & (RING - 1)) * L::kSlot;
    lds_cu8* bp = bq + buf * L::kDBuf;
    lds_cu8* bp4 = bq4 + buf * L::kDBuf;
    auto blk = [](lds_cu8* ptr) { const auto* w = reinterpret_cast<__attribute__((address_space(3))) const uint32_t*>(ptr); return u32x2{w[0], w[1]}; };
    u32x2 qprev = blk(bp - 8);    // block of step -4
    u32x2 qcur = blk(bp);         // block of step 0
    s16x4 b1 = window(qprev, qcur);                           // s-block 1 of step 0
    // s-block 2 of step 0 is the s-block-0 window of step -8 (SB = 3 only).
    s16x4 b2 = SB > 2 ? window(blk(bp - 16), qprev) : b1;
    // Operands of pair pr + 1 are read before the MFMAs of pair pr; the empty
    // asm between pairs also keeps the block reads of different pairs from
    // being merged into ds_read2_b64.
    u32x4 fa[NPAIRS][RB];
    u32x2 q1[NPAIRS], q2[NPAIRS];
    auto load_pair = [&](int pr) {
#pragma unroll
      for (int i = 0; i < RB; ++i) fa[pr][i] = *reinterpret_cast<const u32x4*>(ap[i] + 16 * pr);
      q1[pr] = blk(bp4 + 16 * pr);        // block of step 8pr + 4
      q2[pr] = blk(bp + 16 * pr + 16);    // block of step 8pr + 8
    };
    load_pair(0);
#pragma unroll
    for (int pr = 0; pr < NPAIRS; ++pr) {
      if (pr + 1 < NPAIRS) load_pair(pr + 1);
      asm volatile("" ::: "memory");
      s16x4 b0 = window(qcur, q1[pr]);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const s16x4 av = __builtin_bit_cast(s16x4, u32x2{fa[pr][i].x, fa[pr][i].y});
        acc[i][0] = mfma4<kBf16>(av, b0, acc[i][0]);
        if (SB > 1) acc[i][1] = mfma4<kBf16>(av, b1, acc[i][1]);
        if (SB > 2) acc[i][2] = mfma4<kBf16>(av, b2, acc[i][2]);
      }
      b2 = b1;
      b1 = b0;
      b0 = window(q1[pr], q2[pr]);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const s16x4 av = __builtin_bit_cast(s16x4, u32x2{fa[pr][i].z, fa[pr][i].w});
        acc[i][0] = mfma4<kBf16>(av, b0, acc[i][0]);
        if (SB > 1) acc[i][1] = mfma4<kBf16>(av, b1, acc[i][1]);
        if (SB > 2) acc[i][2] = mfma4<kBf16>(av, b2, acc[i][2]);
      }
      b2 = b1;
      b1 = b0;
      qcur = q2[pr];
    }
  };

  lds_barrier();

  // Stream the slice one image segment at a time.  Step t of a segment that
  // starts at output row ho0 brings X row ho0 - pad + t into the ring and dY
  // row ho = ho0 + t - (R - 1) into dY buffer t & 1; from step R - 1 on, the
  // ring then holds X rows ho - pad .. ho - pad + R - 1 and row ho is
  // computed.  Ring rows past R - 1 that the 4 * RB operand rows include feed
  // only accumulator rows r >= R, which are never stored.  A step's staging
  // overwrites the ring slot and the dY buffer that step t - 1 did not use,
  // except for R = 8, where a second barrier guards the ring.  Every step
  // issues the same loads (rows outside the image or the segment have an
  // empty range and read 0), so the load counters are static.
  const bool guard_ring = a.R + 1 > RING;
  const bool want_db = a.dbo != nullptr;
  float dbp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // channels 8o .. 8o + 7
  Item<NP> qx[kPf], qd[kPf];
  int row = r_begin;
  while (row < r_end) {
    const int n = row / a.Ho, ho0 = row % a.Ho;
    const int seg = min(r_end - row, a.Ho - ho0);
    const int steps = a.stride * (seg - 1) + a.R;  // X rows of the segment
    const int last = ho0 + seg;                    // first output row past the segment
    const int h0 = a.stride * ho0 - a.pad;         // X row of step 0
    // Step t stages X row h0 + t and, when u = t - (R - 1) is a non-negative
    // multiple of the stride, dY row ho0 + u / stride, which it then computes.
    auto fetch_step = [&](int t, Item<NP>& ix, Item<NP>& id) {
      const int h = h0 + t;
      const bool x_in = h >= 0 && h < a.H && t < steps;
      const int64_t ex = (int64_t)n * a.x_img + (int64_t)(x_in ? h : 0) * a.W * a.C + c0;
      fetch(row_rsrc(xg + 2 * ex, x_in ? row_bytes_x : 0), ix);
      const int u = t - (a.R - 1);
      const int ho = ho0 + (a.stride == 2 ? u >> 1 : u);
      const bool d_in = u >= 0 && (u & (a.stride - 1)) == 0 && ho < last;
      const int64_t ed = (int64_t)n * a.dy_img + (int64_t)(d_in ? ho : ho0) * a.Wo * a.C + c0;
      fetch(row_rsrc(dyg + 2 * ed, d_in ? row_bytes_dy : 0), id);
    };
#pragma unroll
    for (int k = 0; k < kPf; ++k) fetch_step(k, qx[k], qd[k]);
    for (int t = 0; t < steps; t += kPf) {
#pragma unroll
      for (int k = 0; k < kPf; ++k) {
        const int tk = t + k;
        store_x((h0 + tk) & (RING - 1), qx[k]);
        store_dy(k & 1, qd[k]);
        if (want_db) {
          // Each dY row of the segment is staged by exactly one step; rows
          // outside it and pixels past the row were loaded as zero.
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            add8<kBf16>(dbp, __builtin_bit_cast(uint4, qd[k].p[p][0]));
            add8<kBf16>(dbp, __builtin_bit_cast(uint4, qd[k].p[p][1]));
          }
        }
        fetch_step(tk + kPf, qx[k], qd[k]);
        lds_barrier();
        const int u = tk - (a.R - 1);
        if (u >= 0 && (u & (a.stride - 1)) == 0 && tk < steps) {
          compute_row(ho0 + (a.stride == 2 ? u >> 1 : u), k & 1);
          if (guard_ring) lds_barrier();
        }
      }
    }
    // The next segment restarts at step 0 (buffer 0, ring slot of its first
    // row); all waves finish this segment's last row before it is overwritten.
    lds_barrier();
    row += seg;
  }

  if (want_db)   // sums of the 32 pixel-pair loaders, channels c0 .. c0 + 63 (LDS is free here)
    block_sum64<32, 8>(reinterpret_cast<float*>(lds), pp, 8 * o, dbp,
                       a.dbo + (int64_t)slice * a.slab_stride + c0, min(kQuadCh, a.C - c0));

  // acc[rb][sb][v] = dW[c0 + wave + 4b][4*rb + v][4*sb + q].  The outputs are
  // gathered in LDS in the [c][r][s] order of the output (every wave has
  // passed the last barrier above, after its last LDS access), so that the
  // workgroup writes its min(64, C - c0) channels as whole 16-byte stores.
  const int RS = a.R * a.S;
  float* s_out = reinterpret_cast<float*>(lds);
  const int cl = wave + 4 * b;
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * i + v, s = 4 * j + q;
        if (r < a.R && s < a.S) s_out[cl * RS + r * a.S + s] = acc[i][j][v];
      }
  __syncthreads();
  const int n4 = min(kQuadCh, a.C - c0) * RS / 4;   // C % 16 == 0
  float4* out = reinterpret_cast<float4*>(a.out + (int64_t)slice * a.slab_stride + (int64_t)c0 * RS);
  for (int i = tid; i < n4; i += kThreads) out[i] = reinterpret_cast<const float4*>(lds)[i];
}

template <bool kBf16, int RB, int SB, int XL>
hipError_t launch_xl(const DwArgs& args, int64_t grid, hipStream_t stream) {
  using L = DwLayout<XL, dw_ring<RB>(), 16 * RB * SB>;
  const void* fn = reinterpret_cast<const void*>(depthwise_mfma_kernel<kBf16, RB, SB, XL>);
  if (L::kBytes > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes);
    if (e != hipSuccess) return e;
  }
  void* params[] = {const_cast<DwArgs*>(&args)};
  const int64_t xcd_grid = (grid + 7) / 8 * 8;   // whole rounds over the 8 XCDs
  return launch_raw(fn, dim3((unsigned)xcd_grid), dim3(kThreads), params, (size_t)L::kBytes, stream);
}

template <bool kBf16, int RB, int SB>
hipError_t launch_rs(int xl, const DwArgs& a, int64_t grid, hipStream_t stream) {
  switch (xl) {
    case 8: return launch_xl<kBf16, RB, SB, 8>(a, grid, stream);
    case 24: return launch_xl<kBf16, RB, SB, 24>(a, grid, stream);
    case 40: return launch_xl<kBf16, RB, SB, 40>(a, grid, stream);
    case 56: return launch_xl<kBf16, RB, SB, 56>(a, grid, stream);
    case 72: return launch_xl<kBf16, RB, SB, 72>(a, grid, stream);
    case 88: return launch_xl<kBf16, RB, SB, 88>(a, grid, stream);
    case 104: return launch_xl<kBf16, RB, SB, 104>(a, grid, stream);
    case 120: return launch_xl<kBf16, RB, SB, 120>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kBf16>
hipError_t launch_b(const Plan& plan, const DwArgs& a, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  const int xl = plan.dw_xl;
  if (a.R > 8 || a.S > 8) return launch_rs<kBf16, 3, 3>(xl, a, grid, stream);
  const bool r2 = a.R > 4, s2 = a.S > 4;
  if (r2 && s2) return launch_rs<kBf16, 2, 2>(xl, a, grid, stream);
  if (r2) return launch_rs<kBf16, 2, 1>(xl, a, grid, stream);
  if (s2) return launch_rs<kBf16, 1, 2>(xl, a, grid, stream);
  return launch_rs<kBf16, 1, 1>(xl, a, grid, stream);
}

}  // namespace

// LDS bytes the depthwise kernel uses for a staged row length and filter size
// (0 if unsupported).
int32_t depthwise_lds_bytes(int32_t xl, int32_t R, int32_t S) {
  const int rb = R > 8 || S > 8 ? 3 : R > 4 ? 2 : 1;
  const int sb = R > 8 || S > 8 ? 3 : S > 4 ? 2 : 1;
  switch (xl) {
#define CW_DW_CASE(V)                                                           \
  case V:                                                                       \
    if (rb == 3) return DwLayout<V, dw_ring<3>(), 144>::kBytes;                 \
    if (rb == 2)                                                                \
      return sb == 2 ? DwLayout<V, dw_ring<2>(), 64>::kBytes                    \
                     : DwLayout<V, dw_ring<2>(), 32>::kBytes;                   \
    return sb == 2 ? DwLayout<V, dw_ring<1>(), 32>::kBytes                      \
                   : DwLayout<V, dw_ring<1>(), 16>::kBytes;
    CW_DW_CASE(8) CW_DW_CASE(24) CW_DW_CASE(40) CW_DW_CASE(56)
    CW_DW_CASE(72) CW_DW_CASE(88) CW_DW_CASE(104) CW_DW_CASE(120)
#undef CW_DW_CASE
    default: return 0;
  }
}

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
  a.stride = (int32_t)p.stride;
  a.dy_off = plan.dw_off;
  a.rows = (int32_t)(p.N * p.Ho);
  a.rows_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  a.quads = (int32_t)ceil_div(p.C, 64);
  a.dbo = out.db;
  a.balanced = plan.dw_balanced;
  if (a.balanced)
    for (int i = 0; i <= a.ks_count; ++i) a.starts[i] = plan.dw_starts[i];
  if (p.dtype == CONV_WGRAD_BF16) return launch_b<true>(plan, a, stream);
  return launch_b<false>(plan, a, stream);
}

}  // namespace cw
