// Dense implicit-GEMM weight gradient for 16-bit inputs with every filter tap
// of a tile in one workgroup (gfx950, 16x16x32 bf16 / fp16 MFMA).
//
// The GEMM of the dense kernels (per group: M = Kg output channels,
// N = R*S*Cg columns, reduction over the output pixels) at stride 1 and
// dilation 1.  A workgroup tile is (group, 32 or 64 output channels, 64
// input channels, all R x S taps), so a staged dY element feeds every tap and
// a staged X element every (r, s) that reaches it, and a unit carries R*S
// times the MFMA work of a one-tap tile for the same staging and barrier:
//
//   * a reduction unit is ru consecutive output rows of one image,
//     ru = 64 / P with P = Wo + S - 1.  dY row j of the unit fills slots
//     j*P .. j*P + Wo - 1 of a 64-slot buffer (zeros elsewhere); X row
//     ho0 - pad_h + i (i < ru + R - 1) fills slots i*P .. i*P + P - 1 with
//     columns -pad_w .. P - 1 - pad_w (zeros outside the image and past the
//     unit's rows);
//   * tap (r, s) pairs dY slot p with X slot p + r*P + s.  For a filled dY
//     slot (row j, column wo) that is X[ho0 + j - pad_h + r][wo - pad_w + s],
//     the product of the definition; an empty dY slot holds zero and meets a
//     staged (finite) or zero X slot, so it adds nothing;
//   * operands are ds_read_b64_tr_b16 transposed reads of the NHWC staging
//     (8 consecutive slots of one channel per lane).  Wave w owns input
//     channels 16w .. 16w + 15 and the tile's 16*MB output channels: per 32
//     slots MB A (dY) reads and R*S B (X) reads feed MB*R*S accumulators;
//   * two LDS buffers alternate (a unit is staged while the previous one is
//     computed, one LDS-only barrier per unit), and the global loads of the
//     next units are held in register sets, each set its own registers and
//     every load unconditional (units past the slice have empty buffer ranges).
//
// BF16x3 (fp32 inputs, math = BF16X3; rocm-libraries PR #14393, timeline, the
// TF32 entry): each fp32 value is split at staging into hi = bf16(v) and
// lo = bf16(v - hi) in two LDS planes, and a product is
// a_lo*b_hi + a_hi*b_lo + a_hi*b_hi, three bf16 MFMAs into the fp32
// accumulator; the bias gradient is then summed from the fp32 values at
// staging.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kPitchE = 80;   // 16-bit elements per staged slot (64 channels + pad)
constexpr int kSlots = 64;    // dY slots per unit (two 32-slot MFMA k-steps)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct TapsArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;   // H*W*C
  int32_t H, W, C, K, Ho, Wo, pad_h, pad_w;
  int32_t Cg, Kg, cols;
  int32_t m_tiles, c_tiles;
  int32_t ru, pitch, hblocks;   // output rows per unit, slot pitch P, ceil(Ho / ru)
  int32_t units, units_per_slice, ks_count;
  int32_t tiles, work;
  float* dbo;      // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
};

__device__ __forceinline__ s16x4 tr_read(const unsigned short* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

template <bool kBf16>
__device__ __forceinline__ f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
  if constexpr (kBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 8 fp32 values (two 16-byte loads) into 8 bf16 high parts and 8 bf16 low
// parts, round-to-nearest-even (v - hi is exact in fp32).
__device__ __forceinline__ void split8(uint4 v0, uint4 v1, uint4& hi, uint4& lo) {
  const float f[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z), __uint_as_float(v0.w),
                      __uint_as_float(v1.x), __uint_as_float(v1.y), __uint_as_float(v1.z), __uint_as_float(v1.w)};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h0 = (__bf16)f[2 * i], h1 = (__bf16)f[2 * i + 1];
    const __bf16 l0 = (__bf16)(f[2 * i] - (float)h0), l1 = (__bf16)(f[2 * i + 1] - (float)h1);
    h[i] = (uint32_t)__builtin_bit_cast(unsigned short, h0) | ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
    l[i] = (uint32_t)__builtin_bit_cast(unsigned short, l0) | ((uint32_t)__builtin_bit_cast(unsigned short, l1) << 16);
  }
  hi = uint4{h[0], h[1], h[2], h[3]};
  lo = uint4{l[0], l[1], l[2], l[3]};
}

// MB: 16-row MFMA blocks of output channels per wave (the tile has 16 * MB
// output channels).  XS: X slots staged per unit (a multiple of 32, at least
// 64 + (R-1)*P + S - 1).  kDb: also the bias gradient.  kX3: fp32 inputs by
// BF16x3 (kBf16 is then true).  kSets: register sets of unit loads in flight.
template <bool kBf16, int MB, int R, int S, int XS, bool kDb, bool kX3, int kSets>
__global__ __launch_bounds__(256) void dense16_taps_kernel(TapsArgs a) {
  constexpr int kEs = kX3 ? 4 : 2;          // bytes per input element
  constexpr int kLd = kX3 ? 2 : 1;          // 16-byte loads per 8-channel chunk
  constexpr int kPlanes = kX3 ? 2 : 1;      // hi (and lo) planes
  constexpr int kXChunks = XS / 32;         // X loader chunks per lane: XS slots x 8 chunks / 256 lanes
  constexpr int kTaps = R * S;
  constexpr int kTileM = 16 * MB;           // output channels per tile
  constexpr int kDq = 2 * MB;               // 8-channel dY chunks per slot
  constexpr int kDyChunks = kSlots * kDq / 256;   // dY loader chunks per lane
  static_assert(XS % 32 == 0 && XS >= 96, "X slots");
  static_assert(MB == 2 || MB == 4, "output-channel blocks");
  __shared__ __attribute__((aligned(16))) unsigned short s_dy[kPlanes][2][kSlots * kPitchE];
  __shared__ __attribute__((aligned(16))) unsigned short s_x[kPlanes][2][XS * kPitchE];
  const unsigned char* __restrict__ xg = static_cast<const unsigned char*>(a.x);
  const unsigned char* __restrict__ dyg = static_cast<const unsigned char*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work item w = slice * tiles + tile; XCD x (block b runs on XCD b % 8)
  // takes a contiguous run of items, so the tiles of a slice share one L2.
  const int per_xcd = (a.work + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || w >= a.work) return;
  const int slice = w / a.tiles;
  int tile = w % a.tiles;
  const int ct = tile % a.c_tiles;
  tile /= a.c_tiles;
  const int mt = tile % a.m_tiles;
  const int g = tile / a.m_tiles;
  const int m0 = mt * kTileM, c0 = ct * 64;
  const int u_begin = slice * a.units_per_slice;
  const int u_end = min(a.units, u_begin + a.units_per_slice);

  // Loader roles.  dY: slots tid / kDq + (256 / kDq) i, channels
  // 8 * (tid % kDq) .. + 7 of the tile's.  X: slots tid / 8 + 32 i, channels
  // 8 * (tid % 8) .. + 7.
  const int P = a.pitch;
  const int d_slot = tid / kDq, dq = tid % kDq;
  const int xs0 = tid >> 3, xq = tid & 7;
  // Per-lane parts of the loader offsets that are the same for every unit:
  // byte offset within the unit's rows and whether the slot's column lies
  // inside the output row (dY) or the image (X).  A load that must read zero
  // gets an offset of at least kOob, past every buffer range.
  constexpr int kOob = 0x7fffffe0;
  int d_row[kDyChunks], d_part[kDyChunks];
  bool d_colok[kDyChunks];
#pragma unroll
  for (int i = 0; i < kDyChunks; ++i) {
    const int slot = d_slot + (256 / kDq) * i;
    d_row[i] = slot / P;
    const int col = slot % P;
    d_colok[i] = col < a.Wo;
    d_part[i] = ((d_row[i] * a.Wo + col) * a.K + 8 * dq) * kEs;
  }
  int x_row[kXChunks], x_part[kXChunks];
  bool x_colok[kXChunks];
#pragma unroll
  for (int i = 0; i < kXChunks; ++i) {
    x_row[i] = (xs0 + 32 * i) / P;
    const int wc = (xs0 + 32 * i) % P - a.pad_w;
    x_colok[i] = wc >= 0 && wc < a.W;
    x_part[i] = (wc * a.C + 8 * xq) * kEs;
  }
  const unsigned x_row_bytes = (unsigned)(a.W * a.C * kEs);
  const int dy_col0 = g * a.Kg + m0;   // first output channel of the tile
  const int x_col0 = g * a.Cg + c0;    // first input channel of the tile

  struct Set {
    uint4 dy[kDyChunks][kLd], x[kXChunks][kLd];
    int nslots;   // slots up to the last filled dY slot (0 past the slice)
  };
  // The loads take the slice's units in order: the unit's (image, row block)
  // is a cursor advanced by one per load.  The offsets are selected without
  // branches, so the loads can be scheduled among the MFMAs of a unit.
  int cur_n = u_begin / a.hblocks, cur_b = u_begin % a.hblocks;
  const int n_first = cur_n, b_first = cur_b;
  auto load_unit = [&](int u, Set& st) {
    const bool live = u < u_end;
    const int n = live ? cur_n : n_first, hb = live ? cur_b : b_first;
    if (live && ++cur_b == a.hblocks) {
      cur_b = 0;
      ++cur_n;
    }
    const int ho0 = hb * a.ru;
    const int rows = live ? min(a.ru, a.Ho - ho0) : 0;
    st.nslots = rows > 0 ? (rows - 1) * P + a.Wo : 0;
    // dY rows ho0 .. ho0 + rows - 1 are contiguous; empty slots read zero.
    const unsigned char* dyp = dyg + kEs * (((int64_t)(n * a.Ho + ho0) * a.Wo) * a.K + dy_col0);
    const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dyp, rows > 0 ? (rows * a.Wo * a.K - dy_col0) * kEs : 0);
#pragma unroll
    for (int i = 0; i < kDyChunks; ++i) {
      const int doff = d_part[i] | (d_colok[i] && d_row[i] < rows ? 0 : kOob);
#pragma unroll
      for (int h = 0; h < kLd; ++h)
        st.dy[i][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, doff + 16 * h, 0, 0));
    }
    // X rows h0 .. h0 + rows + R - 2 (those inside the image), columns
    // -pad_w .. P - 1 - pad_w (those inside the image); the rest read zero.
    // Row i of a lane's slot is image row hlo + x_row[i] + (h0 - hlo).
    const int h0 = ho0 - a.pad_h;
    const int hlo = max(h0, 0), hhi = rows > 0 ? min(h0 + rows + R - 1, a.H) : hlo;
    const int rdelta = h0 - hlo, rspan = hhi - hlo;
    const unsigned char* xp = xg + kEs * ((int64_t)n * a.x_img + (int64_t)hlo * a.W * a.C + x_col0);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(xp, rspan > 0 ? (rspan * a.W * a.C - x_col0) * kEs : 0);
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      const int ri = x_row[i] + rdelta;
      const bool ok = x_colok[i] && ri >= 0 && ri < rspan;
      // Unsigned: the offset of a slot outside the rows may wrap; it is then replaced.
      const int off = (int)(((unsigned)ri * x_row_bytes + (unsigned)x_part[i]) | (ok ? 0u : (unsigned)kOob));
#pragma unroll
      for (int hh = 0; hh < kLd; ++hh)
        st.x[i][hh] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * hh, 0, 0));
    }
  };
  // BF16x3: per-thread fp32 sums of the staged dY values (8 channels at
  // 8 dq of the loader's slots), for the bias gradient.
  const bool db_x3 = kX3 && kDb && ct == 0;
  float dbp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto store_unit = [&](int buf, const Set& st) {
#pragma unroll
    for (int i = 0; i < kDyChunks; ++i) {
      const int slot = d_slot + (256 / kDq) * i;
      unsigned short* d = &s_dy[0][buf][slot * kPitchE + 8 * dq];
      if constexpr (kX3) {
        uint4 hi, lo;
        split8(st.dy[i][0], st.dy[i][kLd - 1], hi, lo);
        *reinterpret_cast<uint4*>(d) = hi;
        *reinterpret_cast<uint4*>(&s_dy[kPlanes - 1][buf][slot * kPitchE + 8 * dq]) = lo;
        if (db_x3) {
          const uint32_t v[8] = {st.dy[i][0].x, st.dy[i][0].y, st.dy[i][0].z, st.dy[i][0].w,
                                 st.dy[i][kLd - 1].x, st.dy[i][kLd - 1].y, st.dy[i][kLd - 1].z, st.dy[i][kLd - 1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) dbp[e] += __uint_as_float(v[e]);
        }
      } else {
        *reinterpret_cast<uint4*>(d) = st.dy[i][0];
      }
    }
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      unsigned short* dx = &s_x[0][buf][(xs0 + 32 * i) * kPitchE + 8 * xq];
      if constexpr (kX3) {
        uint4 hi, lo;
        split8(st.x[i][0], st.x[i][kLd - 1], hi, lo);
        *reinterpret_cast<uint4*>(dx) = hi;
        *reinterpret_cast<uint4*>(&s_x[kPlanes - 1][buf][(xs0 + 32 * i) * kPitchE + 8 * xq]) = lo;
      } else {
        *reinterpret_cast<uint4*>(dx) = st.x[i][0];
      }
    }
  };

  // Transposed-read addressing: in 16-lane group gq, lane j points at slot
  // 8 gq + j / 4 (+ 4 for the second read) and 4 channels at 4 (j % 4).
  const int j = lane & 15, gq = lane >> 4;
  const int lane_off = (8 * gq + (j >> 2)) * kPitchE + 4 * (j & 3);
  auto tr8 = [&](const unsigned short* p) {
    return __builtin_shufflevector(tr_read(p), tr_read(p + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x4 acc[MB][kTaps];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int t = 0; t < kTaps; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Bias gradient (16-bit): in the tiles of the first input-channel block,
  // wave 0 multiplies each A operand by ones (every column of the product is
  // the per-channel sum of the operand's 32 slots).
  const bool db_wave = kDb && !kX3 && ct == 0 && wave == 0;
  f32x4 acc_db[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc_db[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned short one = kBf16 ? 0x3f80 : 0x3c00;
  const s16x8 ones{(short)one, (short)one, (short)one, (short)one,
                   (short)one, (short)one, (short)one, (short)one};

  // One unit's MFMAs: per 32-slot k-step the MB A operands, then per filter
  // row r and tap s the B operand read r*P + s slots further on and its MB
  // MFMAs (with BF16x3 the two cross terms, small, before hi * hi).
  auto compute_unit = [&](int buf, int nslots) {
    const unsigned short* ad = s_dy[0][buf] + lane_off;
    const unsigned short* bx = s_x[0][buf] + lane_off + 16 * wave;
    const unsigned short* ad_lo = s_dy[kPlanes - 1][buf] + lane_off;
    const unsigned short* bx_lo = s_x[kPlanes - 1][buf] + lane_off + 16 * wave;
#pragma unroll
    for (int ks = 0; ks < kSlots / 32; ++ks) {
      // 16-bit without the bias gradient: both k-steps run for every unit
      // (empty slots and units past the slice staged zeros, whose products
      // add nothing), so the loads issued before them are scheduled among
      // the MFMAs.  The other forms skip empty k-steps: with more registers
      // live, one region would move the accumulators in and out of AGPRs.
      if ((!kX3 && !kDb) || 32 * ks < nslots) {
        s16x8 fa[MB], fa_lo[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[i] = tr8(ad + 32 * ks * kPitchE + 16 * i);
        if constexpr (kX3) {
#pragma unroll
          for (int i = 0; i < MB; ++i) fa_lo[i] = tr8(ad_lo + 32 * ks * kPitchE + 16 * i);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row_off = (32 * ks + r * P) * kPitchE;
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const s16x8 fb = tr8(bx + row_off + s * kPitchE);
            if constexpr (kX3) {
              const s16x8 fb_lo = tr8(bx_lo + row_off + s * kPitchE);
#pragma unroll
              for (int i = 0; i < MB; ++i) {
                acc[i][r * S + s] = mfma16<true>(fa_lo[i], fb, acc[i][r * S + s]);
                acc[i][r * S + s] = mfma16<true>(fa[i], fb_lo, acc[i][r * S + s]);
              }
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) acc[i][r * S + s] = mfma16<kBf16>(fa[i], fb, acc[i][r * S + s]);
          }
        }
        if constexpr (kDb && !kX3) {
          if (db_wave) {
#pragma unroll
            for (int i = 0; i < MB; ++i) acc_db[i] = mfma16<kBf16>(fa[i], ones, acc_db[i]);
          }
        }
      }
    }
  };

  // Whole rounds of kSets units; the prologue issues the sets in the order
  // the loop consumes them (pinned by scheduling barriers).
  const int rounds = (u_end - u_begin + kSets - 1) / kSets;
  Set sets[kSets];
#pragma unroll
  for (int p = 0; p < kSets; ++p) {
    load_unit(u_begin + p, sets[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int p = 0; p < kSets; ++p) {
      const int u = u_begin + it * kSets + p;
      const int buf = (it * kSets + p) & 1;
      const int nslots = sets[p].nslots;
      store_unit(buf, sets[p]);
      // The unit is staged and every wave is done with the other buffer (an
      // LDS-only barrier: earlier loads stay in flight).  The next loads into
      // this set are then issued among the unit's MFMAs.
      lds_barrier();
      load_unit(u + kSets, sets[p]);
      compute_unit(buf, nslots);
    }
  }

  // acc[i][t][v] = dW[g*Kg + m0 + 16 i + 4 gq + v][t*Cg + c0 + 16 wave + j], t = r*S + s.
  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int c = c0 + 16 * wave + j;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 16 * i + 4 * gq + v;
      if (m < a.Kg && c < a.Cg) {
        float* o = out + ((int64_t)g * a.Kg + m) * a.cols + c;
#pragma unroll
        for (int t = 0; t < kTaps; ++t) o[(int64_t)t * a.Cg] = acc[i][t][v];
      }
    }
  if constexpr (kX3 && kDb) {
    // 256 / kDq loader rows x kTileM channels of per-thread sums, added in
    // ascending row order through LDS (the staging buffers are free now).
    if (db_x3)   // workgroup-uniform; block_sum64 has its own barriers
      block_sum64<256 / kDq, 8>(reinterpret_cast<float*>(&s_x[0][0][0]), d_slot, 8 * dq, dbp,
                             a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0,
                             min(kTileM, a.Kg - m0));
  }
  if (db_wave && j == 0) {
    float* o = a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * i + 4 * gq + v;
        if (m < a.Kg) o[m] = acc_db[i][v];
      }
  }
}

template <bool kBf16, int MB, int XS, bool kX3>
hipError_t launch_xs(const TapsArgs& args, int64_t grid, hipStream_t stream) {
  const dim3 xcd_grid((unsigned)((grid + 7) / 8 * 8)), block(256);   // whole rounds over the 8 XCDs
  constexpr int kS = kX3 ? 1 : 2;
  if (args.dbo)
    return launch_kernel(dense16_taps_kernel<kBf16, MB, 3, 3, XS, true, kX3, kS>, xcd_grid, block, args, stream);
  return launch_kernel(dense16_taps_kernel<kBf16, MB, 3, 3, XS, false, kX3, kS>, xcd_grid, block, args, stream);
}

template <bool kBf16, int MB, bool kX3>
hipError_t launch_mb(const Plan& plan, const TapsArgs& args, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  switch (plan.xspan) {
    case 128: return launch_xs<kBf16, MB, 128, kX3>(args, grid, stream);
    case 160: return launch_xs<kBf16, MB, 160, kX3>(args, grid, stream);
    case 192: return launch_xs<kBf16, MB, 192, kX3>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kBf16, bool kX3>
hipError_t launch_b(const Plan& plan, const TapsArgs& args, hipStream_t stream) {
  if constexpr (kX3) {
    if (plan.bm == 64) return launch_mb<kBf16, 4, kX3>(plan, args, stream);
  }
  return launch_mb<kBf16, 2, kX3>(plan, args, stream);
}

}  // namespace

hipError_t launch_dense16_taps(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                               hipStream_t stream) {
  const Problem& p = plan.p;
  TapsArgs a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.dbo = out.db;
  a.x_img = p.x_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.pad_h = (int32_t)p.pad_h; a.pad_w = (int32_t)p.pad_w;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg; a.cols = (int32_t)p.cols;
  a.m_tiles = (int32_t)plan.m_tiles;
  a.c_tiles = (int32_t)plan.c_tiles;
  a.ru = plan.ru;
  a.pitch = (int32_t)(p.Wo + p.S - 1);
  a.hblocks = (int32_t)ceil_div(p.Ho, plan.ru);
  a.units = (int32_t)plan.pub.units;
  a.units_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  a.tiles = (int32_t)plan.pub.tiles;
  a.work = (int32_t)(plan.pub.tiles * plan.pub.ks_count);
  if (p.dtype == CONV_WGRAD_F32) return launch_b<true, true>(plan, a, stream);   // BF16x3
  if (p.dtype == CONV_WGRAD_BF16) return launch_b<true, false>(plan, a, stream);
  return launch_b<false, false>(plan, a, stream);
}

}  // namespace cw
